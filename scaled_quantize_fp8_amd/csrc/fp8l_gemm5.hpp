// 128x128 FP8 GEMM with two waves per SIMD, for outputs with few tiles;
// same contract and operand layouts as gemm3_kernel (fp8l_gemm3.hpp), whose
// staging it shares.
//
// Where it is used: an output of 2048 x 1536 (the forward of a 6912 -> 1536
// projection, the dX of the 1536 -> 6912 ones) has 192 tiles of 128x128,
// fewer than the CUs, so each CU holds one block.  gemm3's 128x128 block has
// 4 waves, one per SIMD, and its K loop drains the MFMA pipe at every
// barrier and LDS wait (about 800 cycles per 256 cycles of MFMA work there).
// Here the block has 8 waves (64x32 each, two per SIMD), and one LDS stage
// holds 128 bytes of K as two 64-byte sub-steps in gemm3's layout, so each
// barrier is followed by 4 MFMAs per wave (8 per SIMD) instead of 2.
//
// Per stage each wave reads, for both sub-steps, its A fragment pair and its
// B fragment for the next stage (double-buffered in registers), each read
// block carrying one MFMA of the current stage; 4 DMA loads per wave refill
// the stage freed by the barrier, one after each read block.
#pragma once

#include "fp8l_gemm4.hpp"

namespace fp8l {

// One fragment (tile index f) of operand Op, read without MFMAs.
template <typename Op>
FP8L_DEV void read1(const uint8_t* s, int f, v8i& n0) {
  uint32_t a[8];
  Op::frag_addrs(s, f, a);  // the first fragment of the pair at f
  if constexpr (Op::kLayout == kKContig) {
    v4i r0, r1;
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1)
        : "v"(a[0]), "v"(a[1])
        : "memory");
    n0 = v8i{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  } else {
    v2i r0, r1, r2, r3;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4\n\t"
        "ds_read_b64_tr_b8 %1, %5\n\t"
        "ds_read_b64_tr_b8 %2, %6\n\t"
        "ds_read_b64_tr_b8 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
    n0 = v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
  }
}

template <int LA, int LB, int FA, int FB>
__global__ __launch_bounds__(512, 1) void gemm5_kernel(GemmArgs g) {
  batch_slice(g);
  constexpr int BM = 128, BN = 128, WGM = 2, WGN = 4, NW = WGM * WGN;
  using OA = Op3<LA, BM, NW>;  // one 64-byte sub-step: 8 KB, one DMA load per wave
  using OB = Op3<LB, BN, NW>;
  static_assert(OA::kPerWave == 1 && OB::kPerWave == 1, "one load per operand per sub-step");
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // 64 x 32 per wave
  static_assert(WTM == 64 && WTN == 32, "schedule below is written for 2 x 1 fragments");
  constexpr int kSub = OA::kBytes + OB::kBytes;  // 16 KB: A then B of one sub-step
  constexpr int kStage = 2 * kSub;               // 128 bytes of K
  constexpr int kDma = 4;                        // loads per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem5[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_coords_xcd(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;

  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    if (g.aux_scale_dst0) *g.aux_scale_dst0 = *g.aux_scale_src0;
    if (g.aux_amax_dst0) *g.aux_amax_dst0 = 0.0f;
    if (g.aux_scale_dst1) *g.aux_scale_dst1 = *g.aux_scale_src1;
    if (g.aux_amax_dst1) *g.aux_amax_dst1 = 0.0f;
  }
  if (g.db && tn == 0 && tid < BM) {
    const int64_t i = i0 + tid;
    if (i < g.Mc) {
      float s = 0.0f;
      for (int r = 0; r < g.db_R; ++r) s += g.db_ws[(int64_t)r * g.Mc + i];
      if (g.db_scale) s *= 1.0f / *g.db_scale;
      g.db[i] = (uint16_t)f32_to_bf16(s);
    }
  }
  const float dq = (1.0f / *g.scale_a) * (1.0f / *g.scale_b);
  const float inv_bs =
      (g.bias_kind == kBiasE4M3 || g.bias_kind == kBiasE5M2) ? 1.0f / *g.bias_scale : 1.0f;
  wait_vm<0>();  // nothing above may count against vmcnt in the loop

  const int64_t a_rows = (LA == kKContig) ? g.Mc : g.Kc;
  const int64_t b_rows = (LB == kKContig) ? g.Nc : g.Kc;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, (uint32_t)(a_rows * g.lda));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, (uint32_t)(b_rows * g.ldb));
  OA oa;
  OB ob;
  oa.init(g.lda, i0, g.Mc, g.Kc);
  ob.init(g.ldb, j0, g.Nc, g.Kc);

  const int wm = wave / WGN, wn = wave % WGN;
  const int ra0 = wm * WTM, rb0 = wn * WTN;
  v16f acc[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[a][e] = 0.0f;

  // ns stages of 128 bytes of K, padded to even; sub-steps past K land as
  // zeros, and the last stage's reads of a successor are never used
  const int ns = (int)(((g.Kc + 2 * kBK3 - 1) / (2 * kBK3) + 1) & ~1);
  auto stage_buf = [&](int st) { return smem5 + (st % kStages3) * kStage; };
  // DMA load j (0..3) of stage st: A sub0, B sub0, A sub1, B sub1
  auto load = [&](int st, auto j_tag) {
    constexpr int j = decltype(j_tag)::value;
    uint8_t* const b = stage_buf(st) + (j >> 1) * kSub;
    if constexpr ((j & 1) == 0)
      oa.template issue_one<0>(ra, b, 2 * st + (j >> 1));
    else
      ob.template issue_one<0>(rb, b + OA::kBytes, 2 * st + (j >> 1));
  };

  // fragments [parity][sub-step]
  v8i fa[2][2][2], fb[2][2];
  auto slot = [&](int a, int par, int sub) {
    return MfmaSlot{&acc[a], &fb[par][sub], &fa[par][sub][a]};
  };

  for (int s = 0; s < kStages3 && s < ns; ++s) {
    load(s, std::integral_constant<int, 0>{});
    load(s, std::integral_constant<int, 1>{});
    load(s, std::integral_constant<int, 2>{});
    load(s, std::integral_constant<int, 3>{});
  }
  if (ns > 0) {
    const int later = min(3, ns - 1);
    if (later >= 3) wait_vm<3 * kDma>();
    else if (later == 2) wait_vm<2 * kDma>();
    else if (later == 1) wait_vm<kDma>();
    else wait_vm<0>();
    barrier_only();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const uint8_t* b = stage_buf(0) + sub * kSub;
      OA::read2(b, ra0, fa[0][sub][0], fa[0][sub][1]);
      read1<OB>(b + OA::kBytes, rb0, fb[0][sub]);
    }
  }

  // Stage st: fa/fb[CUR] hold its fragments; the blocks read stage st+1's
  // into [NXT] while issuing stage st's four MFMAs.
  auto stage_body = [&](int st, auto cur_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr int NXT = CUR ^ 1;
    {
      const int later = min(2, ns - 2 - st);
      if (later >= 2) wait_vm<2 * kDma>();
      else if (later == 1) wait_vm<kDma>();
      else wait_vm<0>();
    }
    barrier_only();  // stage st+1 visible to all; stage st's buffer is free
    const bool refill = st + kStages3 < ns;
    const uint8_t* const nb = stage_buf(st + 1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      {
        const MfmaSlot m[4] = {slot(0, CUR, sub), slot(0, CUR, sub), slot(0, CUR, sub),
                               slot(0, CUR, sub)};
        OA::template read2_fused<FA, FB, 1>(nb + sub * kSub, ra0, fa[NXT][sub][0], fa[NXT][sub][1],
                                            m);
      }
      if (refill) {
        if (sub == 0) load(st + kStages3, std::integral_constant<int, 0>{});
        else load(st + kStages3, std::integral_constant<int, 2>{});
      }
      {
        const MfmaSlot m[4] = {slot(1, CUR, sub), slot(1, CUR, sub), slot(1, CUR, sub),
                               slot(1, CUR, sub)};
        read1_fused<OB, FA, FB, 1>(nb + sub * kSub + OA::kBytes, rb0, fb[NXT][sub], m);
      }
      if (refill) {
        if (sub == 0) load(st + kStages3, std::integral_constant<int, 1>{});
        else load(st + kStages3, std::integral_constant<int, 3>{});
      }
    }
  };
  for (int st = 0; st < ns; st += 2) {
    stage_body(st, std::integral_constant<int, 0>{});
    stage_body(st + 1, std::integral_constant<int, 1>{});
  }

  // Epilogue as in gemm3_kernel.
  constexpr int RS = BN * 2 + 16;
  mfma_drain();
  barrier_only();
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int jl = rb0 + 8 * grp + 4 * (lane >> 5);
    const int64_t j = j0 + jl;
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (g.bias_kind != kBiasNone) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (j + t < g.Nc) bias[t] = bias_at(g, j + t, inv_bs);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int il = ra0 + 32 * a + (lane & 31);
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(acc[a][4 * grp + t], dq, bias[t]);
      *reinterpret_cast<uint2*>(smem5 + il * RS + jl * 2) =
          make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
    }
  }
  lds_barrier();
  constexpr int kChunksPerRow = BN / 8;
  const int64_t rows_left = g.Mc - i0, cols_left = g.Nc - j0;
#pragma unroll 4
  for (int q = tid; q < BM * kChunksPerRow; q += 64 * NW) {
    const int r = q / kChunksPerRow, ch = q % kChunksPerRow;
    if (r < rows_left && 8 * ch < cols_left)
      __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(smem5 + r * RS + ch * 16),
                                  reinterpret_cast<v4u*>(g.c + (i0 + r) * g.ldc + j0 + 8 * ch));
  }
}

constexpr int gemm5_lds_bytes() {
  return kStages3 * 2 * 256 * kBK3 > 128 * (128 * 2 + 16) ? kStages3 * 2 * 256 * kBK3
                                                          : 128 * (128 * 2 + 16);
}

}  // namespace fp8l
