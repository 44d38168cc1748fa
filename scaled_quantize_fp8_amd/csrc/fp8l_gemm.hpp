// FP8 GEMMs of the linear layer on gfx950 MFMA (v_mfma_f32_16x16x128_f8f6f4).
//
//   C[i, j] = sum_k A(i, k) B(j, k) / (sa sb) (+ bias[j]), bf16 out
//
// fwd:  C = Y  [M,N], A = X8 [M,K] (k contiguous),  B = W8 [N,K] (k contiguous)
// dX:   C = dX [M,K], A = G8 [M,N] (k=n contiguous), B = W8 [N,K] read crosswise
// dW:   C = dW [N,K], A = G8 [M,N] crosswise,        B = X8 [M,K] crosswise
// ([P1] entries on the crosswise-B staging of dX and the crosswise-A load of
// dW; [P3] entries on bf16 output and the forward scale reaching the
// backward; [P1]/[P4] entries on the fused bias and bias_scale.)
//
// This file holds the shared GEMM definitions (GemmArgs, layouts, bias and
// tile helpers) and gemm_kernel, the general-shape kernel: it accepts any
// sizes, strides and alignments, and runs whenever the pipelined kernel of
// fp8l_gemm3.hpp cannot (dimensions not multiples of 16, unaligned pointers
// or leading dimensions, matrices of 2 GiB and more).
//
// gemm_kernel (the pages' ldmatrix/cp.async/PRMT kernel is prior art for
// another machine): a 256-thread block owns a 128x128 C tile and walks K in
// steps of 128 (one MFMA depth).  Both operands are staged in LDS through a
// double buffer, one barrier per K step.  A k-contiguous operand tile is
// kept as [128 rows][128 bytes]; a crosswise operand tile is kept exactly as
// it lies in memory, [128 k][128 bytes], and fed to the MFMA with the LDS
// transpose read ds_read_b64_tr_b8, so no register shuffles are needed.
// 16-byte chunks are XOR-swizzled per row so both the 16-byte stores and the
// MFMA fragment reads avoid bank conflicts.  Each of the 4 waves computes a
// 64x64 quarter as 4x4 MFMA tiles with fp32 accumulators; the MFMA's A input
// is the B operand so each lane ends up with four consecutive C columns of
// one row (8-byte bf16 stores).  The epilogue multiplies by (1/sa)(1/sb),
// adds the bias in fp32 (one fma) and rounds once to bf16.
#pragma once

#include "fp8l_device.hpp"

namespace fp8l {

constexpr int kGThreads = 256;
constexpr int kBM = 128;   // C rows per block
constexpr int kBN = 128;   // C cols per block
constexpr int kBK = 128;   // contraction per step
constexpr int kTileBytes = 128 * 128;

enum { kKContig = 0, kCross = 1 };
enum { kBiasNone = 0, kBiasBF16 = 1, kBiasE4M3 = 2, kBiasE5M2 = 3 };

// The ring fold of a launch that ran in kScaleDefer mode (its blocks left
// their maxima in the ring's election groups), done by one wave of a later
// launch on the same stream: the GEMM that consumes the codes, or a one-wave
// fold launch.  ring null: nothing to fold.
struct RingFold {
  RingHdr* ring;
  float* hist;
  int32_t hist_len;  // 1..64: one window slot per lane of the folding wave
  float fmt_max;
  float* amax_out;   // optional
};

struct GemmArgs {
  const uint8_t* a;
  int64_t lda;
  const uint8_t* b;
  int64_t ldb;
  int64_t Mc, Nc, Kc;
  uint16_t* c;
  int64_t ldc;
  const float* scale_a;
  const float* scale_b;
  const void* bias;
  int32_t bias_kind;
  const float* bias_scale;
  // bias-gradient finalize (dW): db[i] = bf16(mult * sum_r ws[r][i])
  uint16_t* db;
  const float* db_ws;
  int32_t db_R;
  const float* db_scale;  // null: mult = 1; else mult = 1 / *db_scale
  // snapshot copies for pre-quantized operands (block 0 writes them)
  float* aux_scale_dst0;
  const float* aux_scale_src0;
  float* aux_amax_dst0;
  float* aux_scale_dst1;
  const float* aux_scale_src1;
  float* aux_amax_dst1;
  int32_t a_vec, b_vec, c_vec;
  int32_t tiles_m, tiles_n;
  // batched operands (grid.y = batch): slice z starts at a + z bsa, b + z bsb
  // (bytes) and c + z bsc (elements); a stride of 0 broadcasts the slice
  int64_t bsa, bsb, bsc;
  int32_t batch;  // >= 1
  // FP8 output (fp8_gemm_fp8out): codes c8 [Mc, ldc], made with the output
  // ring's scale; the launch's last block folds max |y| into that ring, or,
  // with odefer, each block only adds its max to its election group and a
  // one-wave launch after the GEMM folds the groups (ring_fold_wave).
  uint8_t* c8;
  RingHdr* oring;
  float* ohist;
  int32_t ohist_len;
  float* oscale_used;
  float* oamax;
  int32_t odefer;
  // ring folds left by the quantizes of this GEMM's operands (block 0)
  RingFold fold[2];
  // This problem's blocks within the launch: x indices blk0 .. blk0 + nblk - 1
  // (nblk 0: the whole grid).  A launch that runs two problems (the grouped
  // backward) gives each its own range; a problem's block b is launch block
  // blk0 + b, and blk0 is a multiple of 8, so b and the launch block sit on
  // the same XCD (workgroups are dealt round-robin over the 8 XCDs).
  int32_t blk0, nblk;
};

// This block's index within its problem, and the problem's block count (x).
FP8L_DEV int prob_block(const GemmArgs& g) { return (int)blockIdx.x - g.blk0; }
FP8L_DEV int prob_nblk(const GemmArgs& g) { return g.nblk ? g.nblk : (int)gridDim.x; }

// The fold of one ring by one full wave: take the 64 group maxima (leaving
// zeros), fold the launch amax into hist[idx], advance idx, publish
// S(window max), mark the ring seeded, write amax_out.  The quantize launch
// ran before this kernel on the same stream and has completed, so every
// group max is in place; nothing else touches the ring while this kernel
// runs.  The loads and the atomic exchange are waited for here.
FP8L_DEV void ring_fold_wave(const RingFold& f) {
  const int lane = threadIdx.x & 63;
  const uint32_t gm = atom_xchg(&f.ring->group[lane].amax, 0u);
  const uint32_t H = (uint32_t)f.hist_len;
  const uint32_t hv = (uint32_t)lane < H ? __float_as_uint(f.hist[lane]) : 0u;
  const uint32_t idx = f.ring->idx % H;  // in range even for a corrupted header
  const float prev = f.ring->scale;
  const uint32_t amax = wave_max_u32(gm);
  const uint32_t m = wave_max_u32((uint32_t)lane == idx ? amax : hv);
  if (lane == 0) {
    f.hist[idx] = __uint_as_float(amax);
    f.ring->idx = idx + 1 == H ? 0u : idx + 1;
    f.ring->scale = scale_from_amax(__uint_as_float(m), f.fmt_max, prev);
    f.ring->seeded = 1u;
    if (f.amax_out) *f.amax_out = __uint_as_float(amax);
  }
}

// Block (0, 0)'s wave 0 folds the rings: one device round trip on one wave
// of one block.  The pipelined kernels do it after their K loop (side_work),
// the general kernel at its start.
FP8L_DEV void ring_folds(const GemmArgs& g) {
  if (prob_block(g) != 0 || blockIdx.y != 0 || (threadIdx.x >> 6) != 0) return;
  if (g.fold[0].ring) ring_fold_wave(g.fold[0]);
  if (g.fold[1].ring) ring_fold_wave(g.fold[1]);
}

// Move the operand pointers to this block's batch slice (blockIdx.y).
FP8L_DEV void batch_slice(GemmArgs& g) {
  const int64_t z = blockIdx.y;
  g.a += z * g.bsa;
  g.b += z * g.bsb;
  g.c += z * g.bsc;
}

// Swizzle of the 16-byte chunk index within a 128-byte LDS row.
// k-contiguous tiles (row = C row): 16 consecutive rows read the same logical
// chunk in one ds_read_b128; rows r and r^8 land in different halves.
FP8L_DEV int swz_k(int r) { return (r ^ (r >> 3)) & 7; }
// crosswise tiles (row = k): a ds_read_b64_tr_b8 lane group reads 8
// consecutive k rows of one chunk, and groups 0/1 sit 32 rows apart.
FP8L_DEV int swz_x(int kk) { return ((kk >> 1) & 3) | (((kk >> 5) & 1) << 2); }

// One 16-byte chunk of an operand tile: outer index o (tile row), inner
// byte offset in (16 bytes).  Out-of-range bytes read as zero.
FP8L_DEV uint4 load_chunk(const uint8_t* p, int64_t ld, int64_t o, int64_t olim, int64_t in,
                          int64_t inlim, int vec) {
  uint4 r = make_uint4(0, 0, 0, 0);
  if (o >= olim || in >= inlim) return r;
  const uint8_t* q = p + o * ld + in;
  if (vec && in + 16 <= inlim) return *reinterpret_cast<const uint4*>(q);
  uint32_t w[4] = {0, 0, 0, 0};
  for (int j = 0; j < 16; ++j)
    if (in + j < inlim) w[j >> 2] |= (uint32_t)q[j] << (8 * (j & 3));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Load this thread's 4 chunks of an operand tile (128 tile rows x 128
// bytes).  Thread t owns chunk t&7 of tile rows (t>>3) + 32*i.
// k-contiguous: tile row = C index (rbase + r), bytes = k0 + 16c.
// crosswise:    tile row = k0 + r,            bytes = rbase + 16c.
template <int L>
FP8L_DEV void load_tile(const uint8_t* p, int64_t ld, int64_t rbase, int64_t rlim, int64_t k0,
                        int64_t klim, int vec, uint4 v[4]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 3) + 32 * i;
    if constexpr (L == kKContig)
      v[i] = load_chunk(p, ld, rbase + r, rlim, k0 + 16 * c, klim, vec);
    else
      v[i] = load_chunk(p, ld, k0 + r, klim, rbase + 16 * c, rlim, vec);
  }
}

template <int L>
FP8L_DEV void store_tile(uint8_t* s, const uint4 v[4]) {
  const int t = threadIdx.x;
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 3) + 32 * i;
    const int pc = (L == kKContig) ? (c ^ swz_k(r)) : (c ^ swz_x(r));
    *reinterpret_cast<uint4*>(s + r * 128 + pc * 16) = v[i];
  }
}

// MFMA input fragment (16 tile-indices x 128 k) for lane l: index f0 + (l&15),
// k = 32*(l>>4) + byte.
template <int L>
FP8L_DEV v8i load_frag(const uint8_t* s, int f0) {
  const int l = threadIdx.x & 63;
  v8i out;
  if constexpr (L == kKContig) {
    const int r = f0 + (l & 15);
    const int g = l >> 4;
    const uint4 lo = *reinterpret_cast<const uint4*>(s + r * 128 + (((2 * g) ^ swz_k(r)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(s + r * 128 + (((2 * g + 1) ^ swz_k(r)) << 4));
    out[0] = lo.x; out[1] = lo.y; out[2] = lo.z; out[3] = lo.w;
    out[4] = hi.x; out[5] = hi.y; out[6] = hi.z; out[7] = hi.w;
  } else {
    // ds_read_b64_tr_b8: within each 16-lane group, lane 8h+i receives byte
    // i of the 8-byte rows addressed by lanes 2j+h (j = 0..7).  Lane 2j+h
    // therefore addresses k row (k0 + j), columns f0 + 8h.. of the tile.
    const int q = l >> 4, sidx = l & 15;
    const int cc = f0 >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kk = 32 * q + 8 * t + (sidx >> 1);
      const uint8_t* addr = s + kk * 128 + ((cc ^ swz_x(kk)) << 4) + ((sidx & 1) << 3);
      v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)((__attribute__((address_space(3))) uint8_t*)addr));
      out[2 * t] = r.x;
      out[2 * t + 1] = r.y;
    }
  }
  return out;
}

FP8L_DEV float bias_at(const GemmArgs& g, int64_t j, float inv_bs) {
  if (g.bias_kind == kBiasBF16)
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(g.bias)[j]);
  const uint32_t code = reinterpret_cast<const uint8_t*>(g.bias)[j];
  return fp8_to_f32_rt(code, g.bias_kind == kBiasE4M3 ? kE4M3 : kE5M2) * inv_bs;
}

// Tile order: groups of 8 tile-rows walk the tile-columns so the blocks
// resident together share A rows and B columns in L2.
// Bias-gradient finalize, db[i] = bf16(mult * sum_r ws[r][i]), shared by all
// blocks of the launch: 16 lanes per entry, lane q adding partial rows q,
// q + 16, ...; the 16 sums meet in a fixed xor tree, so the result does not
// depend on the launch shape.  Every thread of the block calls it (the
// shuffles need whole 16-lane groups; the loop's trip count is uniform).
// NT: threads per block.  A lane loads four of its partial rows at a time
// and adds them in row order, so the sum is the plain sequential one.
template <int NT>
FP8L_DEV void db_finalize(const GemmArgs& g) {
  const int tid = threadIdx.x;
  const int64_t nblk = (int64_t)prob_nblk(g) * gridDim.y;
  const int64_t b = (int64_t)blockIdx.y * prob_nblk(g) + prob_block(g);
  constexpr int per = NT / 16;  // entries per block and pass
  const int q = tid & 15;
  for (int64_t i = b * per + tid / 16; i - tid / 16 < g.Mc; i += nblk * per) {
    float s = 0.0f;
    if (i < g.Mc) {
      const float* col = g.db_ws + i;
      const int64_t st = g.Mc;
      int r = q;
      for (; r + 48 < g.db_R; r += 64) {
        const float v0 = col[(int64_t)r * st], v1 = col[(int64_t)(r + 16) * st];
        const float v2 = col[(int64_t)(r + 32) * st], v3 = col[(int64_t)(r + 48) * st];
        s += v0;
        s += v1;
        s += v2;
        s += v3;
      }
      for (; r < g.db_R; r += 16) s += col[(int64_t)r * st];
    }
    s += __shfl_xor(s, 1, 16);
    s += __shfl_xor(s, 2, 16);
    s += __shfl_xor(s, 4, 16);
    s += __shfl_xor(s, 8, 16);
    if (q == 0 && i < g.Mc) {
      if (g.db_scale) s *= 1.0f / *g.db_scale;
      g.db[i] = (uint16_t)f32_to_bf16(s);
    }
  }
}

// Tile of linear index pid: pids walk down groups of G tile rows, column by
// column, so that a run of consecutive pids (one XCD's share, see
// tile_coords_xcd) covers a block G rows tall.  G = 4 gives the 2048 x 1536
// outputs of the 128x128 kernels 4 x 6 blocks per XCD, 10 operand panels
// where G = 8 gives 8 x 3, 11 panels; measured, it is 0.5-1% faster over the
// layer's GEMMs.
FP8L_DEV void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int group = pid / per_group;
  const int first = group * G;
  const int gm = min(tiles_m - first, G);
  const int in_group = pid - group * per_group;
  tm = first + in_group % gm;
  tn = in_group / gm;
}

template <int LA, int LB, int FA, int FB>
__global__ __launch_bounds__(kGThreads, 2) void gemm_kernel(GemmArgs g) {
  batch_slice(g);
  ring_folds(g);
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][2][kTileBytes];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  int tm, tn;
  tile_coords(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t i0 = (int64_t)tm * kBM;
  const int64_t j0 = (int64_t)tn * kBN;

  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    if (g.aux_scale_dst0) *g.aux_scale_dst0 = *g.aux_scale_src0;
    if (g.aux_amax_dst0) *g.aux_amax_dst0 = 0.0f;
    if (g.aux_scale_dst1) *g.aux_scale_dst1 = *g.aux_scale_src1;
    if (g.aux_amax_dst1) *g.aux_amax_dst1 = 0.0f;
  }

  if (g.db) db_finalize<kGThreads>(g);

  const int wm = wave >> 1, wn = wave & 1;
  v4f acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = (int)((g.Kc + kBK - 1) / kBK);
  uint4 ra[4], rb[4];
  if (nk > 0) {
    load_tile<LA>(g.a, g.lda, i0, g.Mc, 0, g.Kc, g.a_vec, ra);
    load_tile<LB>(g.b, g.ldb, j0, g.Nc, 0, g.Kc, g.b_vec, rb);
    store_tile<LA>(smem[0][0], ra);
    store_tile<LB>(smem[0][1], rb);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k1 = (int64_t)(kt + 1) * kBK;
      load_tile<LA>(g.a, g.lda, i0, g.Mc, k1, g.Kc, g.a_vec, ra);
      load_tile<LB>(g.b, g.ldb, j0, g.Nc, k1, g.Kc, g.b_vec, rb);
    }
    v8i fa[4], fb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) fa[f] = load_frag<LA>(smem[cur][0], wm * 64 + 16 * f);
#pragma unroll
    for (int f = 0; f < 4; ++f) fb[f] = load_frag<LB>(smem[cur][1], wn * 64 + 16 * f);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[b], fa[a], acc[a][b], FB, FA,
                                                                      0, 0, 0, 0);
    if (more) {
      store_tile<LA>(smem[cur ^ 1][0], ra);
      store_tile<LB>(smem[cur ^ 1][1], rb);
    }
    __syncthreads();
  }

  // epilogue: lane holds C[i0 + wm*64 + 16a + (lane&15)][j0 + wn*64 + 16b + 4*(lane>>4) + t]
  const float dq = (1.0f / *g.scale_a) * (1.0f / *g.scale_b);
  const float inv_bs =
      (g.bias_kind == kBiasE4M3 || g.bias_kind == kBiasE5M2) ? 1.0f / *g.bias_scale : 1.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t j = j0 + wn * 64 + 16 * b + 4 * (lane >> 4);
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (g.bias_kind != kBiasNone) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (j + t < g.Nc) bias[t] = bias_at(g, j + t, inv_bs);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t i = i0 + wm * 64 + 16 * a + (lane & 15);
      if (i >= g.Mc) continue;
      uint32_t h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) h[t] = f32_to_bf16(__builtin_fmaf(acc[a][b][t], dq, bias[t]));
      uint16_t* dst = g.c + i * g.ldc + j;
      if (g.c_vec && j + 4 <= g.Nc) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (j + t < g.Nc) dst[t] = (uint16_t)h[t];
      }
    }
  }
}

}  // namespace fp8l
