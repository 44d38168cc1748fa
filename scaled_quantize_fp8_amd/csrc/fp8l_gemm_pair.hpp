// Two GEMM problems in one launch: the grouped backward, in which the dX
// and dW GEMMs of a linear (both waiting only for the quantized G) share
// one grid instead of two launches on two streams.
//
// Why: at the layer's shapes neither GEMM fills the chip with one tile per
// CU (dX of a 6912 -> 1536 projection has 192 tiles of 128x128, its dW 162
// of 256x256), and each launch pays its own fixed phases (block start-up,
// first stage, epilogue store burst, block-end spread).  One grid of both
// problems' tiles keeps every CU busy while tiles remain: the hardware
// dispatches blocks in index order as CUs free up, so the launcher gives the
// problem with the longer tiles the first block range (longest first), and
// the shorter tiles fill in behind them.  Unlike two streams, the overlap
// holds inside a captured graph too.
//
// Problem P runs in launch blocks [P.blk0, P.blk0 + P.nblk); the second
// range starts at a multiple of 8 (blocks in the gap exit at once), so each
// problem's tile numbering keeps its XCD-major order (tile_coords_xcd).
// Both bodies are 512-thread, one-block-per-CU kernels on the same dynamic
// LDS (the larger of the two sizes).
#pragma once

#include "fp8l_gemm5.hpp"

namespace fp8l {

template <int LA, int LB, int FA, int FB>
struct Body4 {  // 256x256 tiles, 8 waves (gemm4)
  static constexpr int kBM = 256, kBN = 256;
  static constexpr int kLds = gemm4_lds_bytes();
  FP8L_DEV static void run(GemmArgs& g, uint8_t* smem) { gemm4_body<LA, LB, FA, FB>(g, smem); }
};

template <int LA, int LB, int FA, int FB>
struct Body5 {  // 128x128 tiles, 8 waves (gemm5)
  static constexpr int kBM = 128, kBN = 128;
  static constexpr int kLds = gemm5_lds_bytes();
  FP8L_DEV static void run(GemmArgs& g, uint8_t* smem) { gemm5_body<LA, LB, FA, FB>(g, smem); }
};

template <class A, class B>
__global__ __launch_bounds__(512, 1) void gemm_pair_kernel(GemmArgs a, GemmArgs b) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_pair[];
  const int x = blockIdx.x;
  if (x >= a.blk0 && x < a.blk0 + a.nblk)
    A::run(a, smem_pair);
  else if (x >= b.blk0 && x < b.blk0 + b.nblk)
    B::run(b, smem_pair);
}

template <class A, class B>
constexpr int pair_lds_bytes() {
  return A::kLds > B::kLds ? A::kLds : B::kLds;
}

}  // namespace fp8l
