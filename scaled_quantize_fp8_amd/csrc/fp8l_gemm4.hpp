// 256x256 FP8 GEMM with two waves per SIMD; same contract and operand
// layouts as gemm3_kernel (fp8l_gemm3.hpp), whose staging it shares.
//
// Why a second 256x256 kernel: on gfx950 an MFMA issue holds its wave until
// the matrix pipe accepts it, so a wave can queue at most one MFMA ahead.
// With one wave per SIMD (gemm3's 256x256 tile, 128x128 per wave) every
// barrier, DMA issue and LDS wait of that wave drains the pipe.  Here 8 waves
// (2 per SIMD) each own a 128x64 quarter-column, so one wave's MFMAs cover
// the other's memory work.  That needs at most 256 registers per wave: the
// 128 accumulators live in AGPRs, and the fragments take 64 VGPRs by
// single-buffering A (each A fragment is refilled with the next step's data
// right after the last MFMA that reads it) and double-buffering only B.
//
// Per K step (64 bytes) each wave issues 8 MFMAs (4 A fragments x 2 B
// fragments) and 4 DMA loads; the LDS ring is the 4-deep ring of gemm3.
// The next step's first two MFMAs are issued in the step's last read block,
// ahead of the barrier.  For the last step that means one step past K: its
// DMA is issued like any other and lands as zeros (every offset lies past K),
// so those MFMAs add exact zeros.
#pragma once

#include "fp8l_gemm3.hpp"

namespace fp8l {

// LDS: the operand ring or the staged output tile, then the bias of the
// block's 256 columns (BiasStage).
constexpr int kGemm4BiasOff =
    kStages3 * 512 * kBK3 > 256 * (256 * 2 + 16) ? kStages3 * 512 * kBK3 : 256 * (256 * 2 + 16);

// The kernel's work for one block, on the dynamic LDS at smem4 (also run by
// the grouped launch of fp8l_gemm_pair.hpp).
template <int LA, int LB, int FA, int FB, int EPI = kEpiBF16, int OF = kE4M3>
FP8L_DEV void gemm4_body(GemmArgs& g, uint8_t* smem4) {
  batch_slice(g);
  constexpr int BM = 256, BN = 256, WGM = 2, WGN = 4, NW = WGM * WGN;
  using OA = Op3<LA, BM, NW>;
  using OB = Op3<LB, BN, NW>;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // 128 x 64 per wave
  constexpr int FM = WTM / 32, FN = WTN / 32;    // 4 x 2 MFMA tiles
  static_assert(FM == 4 && FN == 2, "schedule below is written for 4 x 2");
  constexpr int kStep = OA::kBytes + OB::kBytes;
  constexpr int kDma = OA::kPerWave + OB::kPerWave;  // 2 + 2
  static_assert(kDma == 4, "one DMA load after each of the four read groups");

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_coords_xcd(prob_block(g), g.tiles_m, g.tiles_n, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  uint8_t* const sbias = smem4 + kGemm4BiasOff;  // BiasStage area


  const int64_t a_rows = (LA == kKContig) ? g.Mc : g.Kc;
  const int64_t b_rows = (LB == kKContig) ? g.Nc : g.Kc;
  const uint32_t a_bytes = (uint32_t)(a_rows * g.lda), b_bytes = (uint32_t)(b_rows * g.ldb);
  OA oa;
  OB ob;
  oa.init(g.lda, i0, g.Mc, g.Kc);
  ob.init(g.ldb, j0, g.Nc, g.Kc);
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // uniform wave index

  const int wm = wave / WGN, wn = wave % WGN;
  const int ra0 = wm * WTM, rb0 = wn * WTN;  // this wave's first A row / B column in the tile
  FragBase<OA, FM> fra;
  FragBase<OB, FN> frb;
  fra.init(smem4, ra0);
  frb.init(smem4 + OA::kBytes, rb0);
  v16f acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // nk K steps (padded to even); steps 0 .. nk are loaded, step nk being
  // all zeros (see the header comment)
  const int nk = (int)(((g.Kc + kBK3 - 1) / kBK3 + 1) & ~1);
  auto step_buf = [&](int kt) { return smem4 + (kt % kStages3) * kStep; };
  auto issue_step = [&](int kt) {
    const __amdgpu_buffer_rsrc_t ra_k = oa.step_rsrc(g.a, a_bytes, kt);
    const __amdgpu_buffer_rsrc_t rb_k = ob.step_rsrc(g.b, b_bytes, kt);
    static_for<OA::kPerWave>([&](auto i) {
      oa.template issue_step<decltype(i)::value>(ra_k, step_buf(kt), kt, wv);
    });
    static_for<OB::kPerWave>([&](auto i) {
      ob.template issue_step<decltype(i)::value>(rb_k, step_buf(kt) + OA::kBytes, kt, wv);
    });
  };

  v8i fa[FM], fb[2][FN];
  auto slot = [&](int a, int b, int buf) { return MfmaSlot{&acc[a][b], &fb[buf][b], &fa[a]}; };

  // prologue: DMA steps 0..3, read step 0, issue its first two MFMAs
  BiasStage<BN>::load(g, j0, sbias, wv);  // ahead of the stages (see BiasStage)
  const EpiScales es = load_scales(g);
  const float s_out = out_scale<EPI, OF>(g);
  for (int s = 0; s < kStages3 && s <= nk; ++s) issue_step(s);
  if (nk > 0) {
    const int later = min(3, nk);  // steps 1..min(3, nk) may still be in flight
    if (later >= 3) wait_vm<3 * kDma>();
    else if (later == 2) wait_vm<2 * kDma>();
    else wait_vm<kDma>();
    barrier_only();
#pragma unroll
    for (int f = 0; f < FM; f += 2) OA::read2(step_buf(0), ra0 + 32 * f, fa[f], fa[f + 1]);
    OB::read2(step_buf(0) + OA::kBytes, rb0, fb[0][0], fb[0][1]);
    const MfmaSlot m[4] = {slot(0, 0, 0), slot(0, 1, 0), slot(0, 0, 0), slot(0, 0, 0)};
    mfma_only<FA, FB, 2>(m);
  }

  // Step kt: on entry MFMAs (a0, *) of step kt are issued; fa holds step kt's
  // A fragments, fb[CUR] its B fragments.
  // FAST: the refill of this step (step kt+4) lies wholly inside K, so its
  // loads take the whole-operand resources with the advance as scalar
  // offset (issue_full), the refill is unconditional and the wait count is
  // fixed; the last steps take the general form (partial step, the zero
  // step past K, no refill).
  const __amdgpu_buffer_rsrc_t ra_all = make_rsrc(g.a, a_bytes);
  const __amdgpu_buffer_rsrc_t rb_all = make_rsrc(g.b, b_bytes);
  auto kstep_body = [&](int kt, auto cur_tag, auto fast_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr int NXT = CUR ^ 1;
    constexpr bool FAST = decltype(fast_tag)::value;
    if constexpr (FAST) {
      wait_vm<2 * kDma>();
    } else {
      // step kt+1 landed: later steps kt+2 .. min(kt+3, nk) may be in flight
      const int later = min(2, nk - kt - 1);
      if (later >= 2) wait_vm<2 * kDma>();
      else if (later == 1) wait_vm<kDma>();
      else wait_vm<0>();
    }
    barrier_only();  // step kt+1 visible to all; step kt's buffer is free
    const bool refill = FAST || kt + kStages3 <= nk;
    const int kf = kt + kStages3;
    uint8_t* const sf = step_buf(kf);
    auto load = [&](auto j_tag) {
      constexpr int j = decltype(j_tag)::value;
      if constexpr (FAST) {
        if constexpr (j < OA::kPerWave)
          oa.template issue_full<j>(ra_all, sf, (uint32_t)kf * oa.kstep, wv);
        else
          ob.template issue_full<j - OA::kPerWave>(rb_all, sf + OA::kBytes, (uint32_t)kf * ob.kstep, wv);
      } else if (refill) {
        const __amdgpu_buffer_rsrc_t ra_k = oa.step_rsrc(g.a, a_bytes, kf);
        const __amdgpu_buffer_rsrc_t rb_k = ob.step_rsrc(g.b, b_bytes, kf);
        if constexpr (j < OA::kPerWave)
          oa.template issue_step<j>(ra_k, sf, kf, wv);
        else
          ob.template issue_step<j - OA::kPerWave>(rb_k, sf + OA::kBytes, kf, wv);
      }
    };
    // this step's fragment addresses: the stage-0 lane addresses plus the
    // byte offset of step kt+1's stage
    const uint32_t d = (uint32_t)(((kt + 1) % kStages3) * kStep);
    auto readA = [&](auto i_tag, v8i& dst, const MfmaSlot (&m)[4], auto nm_tag) {
      constexpr int i = decltype(i_tag)::value, NM = decltype(nm_tag)::value;
      if constexpr (LA == kKContig)
        kc1o<FA, FB, NM, 2048 * i>(fra.a[0] + d, fra.a[1] + d, dst, m);
      else
        x1o<FA, FB, NM, 8 * BM>(fra.a[i] + d, dst, m);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    {  // fa[0] <- step kt+1; MFMAs (a1, *)
      const MfmaSlot m[4] = {slot(1, 0, CUR), slot(1, 1, CUR), slot(1, 0, CUR), slot(1, 0, CUR)};
      readA(I0{}, fa[0], m, I2{});
    }
    load(I0{});
    {  // fa[1] <- step kt+1; MFMAs (a2, *)
      const MfmaSlot m[4] = {slot(2, 0, CUR), slot(2, 1, CUR), slot(2, 0, CUR), slot(2, 0, CUR)};
      readA(I1{}, fa[1], m, I2{});
    }
    load(I1{});
    {  // fa[2] <- step kt+1; MFMA (a3, b0)
      const MfmaSlot m[4] = {slot(3, 0, CUR), slot(3, 0, CUR), slot(3, 0, CUR), slot(3, 0, CUR)};
      readA(I2{}, fa[2], m, I1{});
    }
    load(I2{});
    {  // fb[NXT] <- step kt+1; MFMA (a3, b1)
      const MfmaSlot m[4] = {slot(3, 1, CUR), slot(3, 1, CUR), slot(3, 1, CUR), slot(3, 1, CUR)};
      if constexpr (LB == kKContig)
        kc2o<FA, FB, 1>(frb.a[0] + d, frb.a[1] + d, fb[NXT][0], fb[NXT][1], m);
      else
        x2o<FA, FB, 1, 8 * BN>(frb.a[0] + d, frb.a[1] + d, fb[NXT][0], fb[NXT][1], m);
    }
    load(I3{});
    {  // fa[3] <- step kt+1; MFMAs (a0, *) of step kt+1
      const MfmaSlot m[4] = {slot(0, 0, NXT), slot(0, 1, NXT), slot(0, 0, NXT), slot(0, 0, NXT)};
      readA(I3{}, fa[3], m, I2{});
    }
  };
  // steps whose refill (step kt+4) ends at or before K: kt + 4 < nf, with
  // nf the number of whole 64-byte K steps; an even count, as the loop
  // below takes two steps per iteration
  const int nf = (int)(g.Kc / kBK3);
  const int kfast = max(0, min(nk, nf - kStages3)) & ~1;
  int kt = 0;
  for (; kt < kfast; kt += 2) {
    kstep_body(kt, std::integral_constant<int, 0>{}, std::true_type{});
    kstep_body(kt + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  for (; kt < nk; kt += 2) {
    kstep_body(kt, std::integral_constant<int, 0>{}, std::false_type{});
    kstep_body(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
  }
  wait_vm<0>();  // the DMA of step nk (zeros) must not land in the staging area

  // Epilogue as in gemm3_kernel: scale, bias, one packed RNE to bf16, staged
  // through LDS (rows padded by 16 bytes) and stored as whole rows.
  constexpr int RS = BN * 2 + 16;
  mfma_drain();
  side_work<64 * NW>(g);  // after the drain: its VALU work may reuse fragment registers
  const float dq = es.dq(), inv_bs = es.inv_bs();
  barrier_only();
  if constexpr (EPI != kEpiBF16) {
    fp8_out_epilogue<BM, BN, WTM, WTN, EPI, OF, 64 * NW>(g, acc, dq, inv_bs, s_out, sbias, smem4,
                                                         i0, j0, wm, wn);
    return;
  }
#pragma unroll
  for (int b = 0; b < FN; ++b) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int jl = rb0 + 32 * b + 8 * grp + 4 * (lane >> 5);
      float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (g.bias_kind != kBiasNone) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bias[t] = BiasStage<BN>::get(g, sbias, j0, jl + t, inv_bs);
      }
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int il = ra0 + 32 * a + (lane & 31);
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(acc[a][b][4 * grp + t], dq, bias[t]);
        *reinterpret_cast<uint2*>(smem4 + il * RS + jl * 2) =
            make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
      }
    }
  }
  lds_barrier();
  constexpr int kChunksPerRow = BN / 8;
  const int64_t rows_left = g.Mc - i0, cols_left = g.Nc - j0;
#pragma unroll 4
  for (int q = tid; q < BM * kChunksPerRow; q += 64 * NW) {
    const int r = q / kChunksPerRow, ch = q % kChunksPerRow;
    if (r < rows_left && 8 * ch < cols_left)
      __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(smem4 + r * RS + ch * 16),
                                  reinterpret_cast<v4u*>(g.c + (i0 + r) * g.ldc + j0 + 8 * ch));
  }
}

template <int LA, int LB, int FA, int FB, int EPI = kEpiBF16, int OF = kE4M3>
__global__ __launch_bounds__(512, 1) void gemm4_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem4[];
  gemm4_body<LA, LB, FA, FB, EPI, OF>(g, smem4);
}

constexpr int gemm4_lds_bytes() { return kGemm4BiasOff + BiasStage<256>::kBytes; }

}  // namespace fp8l
