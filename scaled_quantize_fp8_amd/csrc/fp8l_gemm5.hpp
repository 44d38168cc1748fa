// 128x128 FP8 GEMM with two waves per SIMD, for outputs with few tiles;
// same contract and operand layouts as gemm3_kernel (fp8l_gemm3.hpp), whose
// fragment reads it shares.
//
// Where it is used: an output of 2048 x 1536 (the forward of a 6912 -> 1536
// projection, the dX of the 1536 -> 6912 ones) has 192 tiles of 128x128,
// fewer than the CUs, so each CU holds one block.  gemm3's 128x128 block has
// 4 waves, one per SIMD, and its K loop drains the MFMA pipe at every
// barrier and LDS wait.  Here the block has 8 waves, two per SIMD, and one
// LDS stage holds 128 bytes of K as two 64-byte sub-steps.
//
// What bounds the loop is the CU's LDS port (about 128 bytes per clock),
// which carries both the DMA writes of the stages and the fragment reads.
// A 32x32x64 MFMA keeps a SIMD busy for 16 clocks of the CU's 4 SIMDs, i.e.
// the CU retires one every 16 clocks, against 2 KB of LDS traffic in that
// time.  Eight waves of 64x32 would read 3 KB of fragments per MFMA; here
// each wave owns a 64x64 quadrant of C for one of the two sub-steps of
// every stage (4 quadrants x 2 K halves), which reads 2 KB per MFMA, and
// the two K halves of a quadrant are added through LDS after the loop.
//
// Per stage each wave reads its A fragment pair and its B fragment pair for
// the next stage (double-buffered in registers), each read block carrying
// two MFMAs of the current stage; 4 DMA loads per wave refill the stage
// freed by the barrier, two after each read block.
#pragma once

#include "fp8l_gemm4.hpp"

namespace fp8l {

// One operand staged 128 bytes of K at a time (two 64-byte sub-steps), R
// rows or columns of C, NW waves; same interface for both layouts:
//   kBytes        LDS bytes per stage
//   kLoads        DMA instructions per wave per stage
//   sub(x, s)     base of sub-step s inside the stage region x
//   frag_addrs    lane addresses of a fragment pair in a sub-step
//   pair_base     the two address registers read_at takes for that pair
//   read_at       the pair's reads at those addresses plus a stage offset,
//                 fused with NM MFMAs
//   load<J>       DMA instruction J of stage st into the stage region
//   load_full<J>  the same for a stage that lies wholly inside K, through
//                 the resource over the whole operand (see Op3::issue_full)
template <int L, int R, int NW>
struct Stage128;

// k-contiguous: each DMA instruction fetches 8 rows x 128 bytes (whole
// 128-byte lines; half-line rows measured about a quarter slower per CU on
// this access path).  1 KB block b holds rows 8b .. 8b+7: sub-step 0's 64
// bytes of them, then sub-step 1's, each row's 4 chunks permuted by swz64.
// A row's address modulo 256 is that of gemm3's 64-byte-row layout, so the
// fragment reads meet the same banks.  Lane i of an instruction carries
// sub-step i >> 5, row (i >> 2) & 7 of its block, slot i & 3.
template <int R, int NW>
struct Stage128<kKContig, R, NW> {
  static constexpr int kLayout = kKContig;
  static constexpr int kBytes = R * 2 * kBK3;
  static constexpr int kLoads = kBytes / 1024 / NW;
  static_assert(kLoads >= 1 && (kBytes / 1024) % NW == 0, "tile / wave split");

  uint32_t base[kLoads];  // byte offset of this lane's chunk at stage 0
  int32_t inner[kLoads];  // its position along K inside a stage
  int32_t klim;

  FP8L_DEV void init(int64_t ld, int64_t rbase, int64_t /*rlim: rows past it lie past the buffer*/,
                     int64_t klim_) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row = (wave * kLoads + i) * 8 + ((lane >> 2) & 7);
      const int c = (lane & 3) ^ swz64(row);
      inner[i] = 64 * (lane >> 5) + 16 * c;
      base[i] = (uint32_t)((rbase + row) * ld + inner[i]);
    }
    klim = (int32_t)klim_;  // K < 2^31 on this path
  }

  template <int J>
  FP8L_DEV void load(__amdgpu_buffer_rsrc_t rs, uint8_t* x, int st, int wave) const {
    const int k0 = st * 2 * kBK3;
    const uint32_t off = k0 + inner[J] < klim ? base[J] + (uint32_t)k0 : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(x + (wave * kLoads + J) * 1024), 16, off, 0,
        0, 0);
  }

  template <int J>
  FP8L_DEV void load_full(__amdgpu_buffer_rsrc_t rs, uint8_t* x, int st, int wave) const {
    const uint32_t voff = base[J];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(x + (wave * kLoads + J) * 1024), 16, voff,
        (uint32_t)st * (2 * kBK3), 0, 0);
  }

  FP8L_DEV static const uint8_t* sub(const uint8_t* x, int s) { return x + 512 * s; }

  FP8L_DEV static uint32_t row_off(int r) { return ((r >> 3) << 10) + ((r & 7) << 6); }

  // as Op3::frag_addrs (k-contiguous) with this stage's row placement
  FP8L_DEV static void frag_addrs(const uint8_t* s, int f0, uint32_t a[8]) {
    const int l = threadIdx.x & 63;
    const uint32_t sb = lds_off(s);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int r = f0 + 32 * f + (l & 31);
      const int c0 = 2 * (l >> 5);
      a[2 * f + 0] = sb + row_off(r) + ((c0 ^ swz64(r)) << 4);
      a[2 * f + 1] = sb + row_off(r) + (((c0 + 1) ^ swz64(r)) << 4);
    }
  }

  // the two chunk addresses of fragment f0; fragment f0 + 32 lies 4096
  // bytes further (4 blocks of 8 rows, same swizzle)
  FP8L_DEV static void pair_base(const uint8_t* s, int f0, uint32_t b[2]) {
    uint32_t a[8];
    frag_addrs(s, f0, a);
    b[0] = a[0];
    b[1] = a[1];
  }

  template <int FA, int FB, int NM>
  FP8L_DEV static void read_at(const uint32_t b[2], uint32_t d, v8i& n0, v8i& n1,
                               const MfmaSlot (&m)[4]) {
    kc2o<FA, FB, NM, 4096>(b[0] + d, b[1] + d, n0, n1, m);
  }

  FP8L_DEV static void read2(const uint8_t* s, int f0, v8i& x0, v8i& x1) {
    uint32_t a[8];
    frag_addrs(s, f0, a);
    lds_read_kc2(a[0], a[1], a[2], a[3], x0, x1);
  }
};

// Crosswise: gemm3's sub-step planes (64 k rows x R bytes, whole lines
// already), one after the other.
template <int R, int NW>
struct Stage128<kCross, R, NW> : Op3<kCross, R, NW> {
  using Base = Op3<kCross, R, NW>;
  static constexpr int kBytes = 2 * Base::kBytes;
  static constexpr int kLoads = 2 * Base::kPerWave;
  static_assert(Base::kPerWave == 1, "one load per sub-step");

  FP8L_DEV void init(int64_t ld, int64_t rbase, int64_t rlim, int64_t klim) {
    Base::init(ld, rbase, rlim, klim);
  }

  template <int J>
  FP8L_DEV void load(__amdgpu_buffer_rsrc_t rs, uint8_t* x, int st, int) const {
    this->template issue_one<0>(rs, x + J * Base::kBytes, 2 * st + J);
  }

  template <int J>
  FP8L_DEV void load_full(__amdgpu_buffer_rsrc_t rs, uint8_t* x, int st, int wave) const {
    this->template issue_full<0>(rs, x + J * Base::kBytes, (uint32_t)(2 * st + J) * this->kstep,
                                 wave);
  }

  FP8L_DEV static const uint8_t* sub(const uint8_t* x, int s) { return x + Base::kBytes * s; }

  // one base per fragment (f0 and f0 + 32); a fragment's four transpose
  // reads lie 8 R bytes apart
  FP8L_DEV static void pair_base(const uint8_t* s, int f0, uint32_t b[2]) {
    uint32_t a[8];
    Base::frag_addrs(s, f0, a);
    b[0] = a[0];
    b[1] = a[4];
  }

  template <int FA, int FB, int NM>
  FP8L_DEV static void read_at(const uint32_t b[2], uint32_t d, v8i& n0, v8i& n1,
                               const MfmaSlot (&m)[4]) {
    x2o<FA, FB, NM, 8 * R>(b[0] + d, b[1] + d, n0, n1, m);
  }
};

// LDS: the operand ring (the output staging and the K-half exchange reuse
// it), then the bias of the block's 128 columns (BiasStage).
constexpr int kGemm5BiasOff = kStages3 * 2 * 256 * kBK3 > 128 * (128 * 2 + 16)
                                  ? kStages3 * 2 * 256 * kBK3
                                  : 128 * (128 * 2 + 16);

// The kernel's work for one block, on the dynamic LDS at smem5 (also run by
// the grouped launch of fp8l_gemm_pair.hpp).
template <int LA, int LB, int FA, int FB>
FP8L_DEV void gemm5_body(GemmArgs& g, uint8_t* smem5) {
  batch_slice(g);
  constexpr int BM = 128, BN = 128, NW = 8;
  using OA = Stage128<LA, BM, NW>;  // 16 KB per stage, two DMA loads per wave
  using OB = Stage128<LB, BN, NW>;
  static_assert(OA::kLoads == 2 && OB::kLoads == 2, "two loads per operand per stage");
  constexpr int kStage = OA::kBytes + OB::kBytes;  // 128 bytes of K: A then B
  constexpr int kDma = 4;                          // loads per wave per stage

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_coords_xcd(prob_block(g), g.tiles_m, g.tiles_n, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  uint8_t* const sbias = smem5 + kGemm5BiasOff;  // BiasStage area


  const int64_t a_rows = (LA == kKContig) ? g.Mc : g.Kc;
  const int64_t b_rows = (LB == kKContig) ? g.Nc : g.Kc;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, (uint32_t)(a_rows * g.lda));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, (uint32_t)(b_rows * g.ldb));
  OA oa;
  OB ob;
  oa.init(g.lda, i0, g.Mc, g.Kc);
  ob.init(g.ldb, j0, g.Nc, g.Kc);
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // uniform wave index

  // wave = 4 kq + quad: output quadrant quad (64 x 64), K sub-step kq of
  // every stage
  const int quad = wave & 3, kq = wave >> 2;
  const int ra0 = (quad >> 1) * 64, rb0 = (quad & 1) * 64;
  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // ns stages of 128 bytes of K, padded to even; sub-steps past K land as
  // zeros, and the last stage's reads of a successor are never used
  const int ns = (int)(((g.Kc + 2 * kBK3 - 1) / (2 * kBK3) + 1) & ~1);
  auto stage_buf = [&](int st) { return smem5 + (st % kStages3) * kStage; };
  // DMA load j (0..3) of stage st: A 0, B 0, A 1, B 1
  auto load = [&](int st, auto j_tag) {
    constexpr int j = decltype(j_tag)::value;
    uint8_t* const b = stage_buf(st);
    if constexpr ((j & 1) == 0)
      oa.template load<(j >> 1)>(ra, b, st, wv);
    else
      ob.template load<(j >> 1)>(rb, b + OA::kBytes, st, wv);
  };
  auto load_full = [&](int st, auto j_tag) {
    constexpr int j = decltype(j_tag)::value;
    uint8_t* const b = stage_buf(st);
    if constexpr ((j & 1) == 0)
      oa.template load_full<(j >> 1)>(ra, b, st, wv);
    else
      ob.template load_full<(j >> 1)>(rb, b + OA::kBytes, st, wv);
  };
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;

  // fragments [parity][index]
  v8i fa[2][2], fb[2][2];
  auto slot = [&](int a, int b, int par) { return MfmaSlot{&acc[a][b], &fb[par][b], &fa[par][a]}; };

  BiasStage<BN>::load(g, j0, sbias, wv);  // ahead of the stages (see BiasStage)
  const EpiScales es = load_scales(g);
  for (int s = 0; s < kStages3 && s < ns; ++s) {
    load(s, J0{});
    load(s, J1{});
    load(s, J2{});
    load(s, J3{});
  }
  if (ns > 0) {
    const int later = min(3, ns - 1);
    if (later >= 3) wait_vm<3 * kDma>();
    else if (later == 2) wait_vm<2 * kDma>();
    else if (later == 1) wait_vm<kDma>();
    else wait_vm<0>();
    barrier_only();
    OA::read2(OA::sub(stage_buf(0), kq), ra0, fa[0][0], fa[0][1]);
    OB::read2(OB::sub(stage_buf(0) + OA::kBytes, kq), rb0, fb[0][0], fb[0][1]);
  }

  // this wave's fragment address registers in stage 0 (sub-step kq); a
  // stage adds its byte offset
  uint32_t pa[2], pb[2];
  OA::pair_base(OA::sub(smem5, kq), ra0, pa);
  OB::pair_base(OB::sub(smem5 + OA::kBytes, kq), rb0, pb);

  // Stage st: fa/fb[CUR] hold its fragments; two read blocks fetch stage
  // st+1's into [NXT], each carrying two of stage st's four MFMAs.
  // FAST: the refill (stage st+4) lies wholly inside K, so it is
  // unconditional, takes load_full and the wait count is fixed; the last
  // stages take the general form (partial stage, zero stages, no refill).
  auto stage_body = [&](int st, auto cur_tag, auto fast_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr int NXT = CUR ^ 1;
    constexpr bool FAST = decltype(fast_tag)::value;
    if constexpr (FAST) {
      wait_vm<2 * kDma>();
    } else {
      const int later = min(2, ns - 2 - st);
      if (later >= 2) wait_vm<2 * kDma>();
      else if (later == 1) wait_vm<kDma>();
      else wait_vm<0>();
    }
    barrier_only();  // stage st+1 visible to all; stage st's buffer is free
    const bool refill = FAST || st + kStages3 < ns;
    const uint32_t d = (uint32_t)(((st + 1) % kStages3) * kStage);
    auto refill2 = [&](auto j0_tag, auto j1_tag) {
      if constexpr (FAST) {
        load_full(st + kStages3, j0_tag);
        load_full(st + kStages3, j1_tag);
      } else if (refill) {
        load(st + kStages3, j0_tag);
        load(st + kStages3, j1_tag);
      }
    };
    {
      const MfmaSlot m[4] = {slot(0, 0, CUR), slot(0, 1, CUR), slot(0, 0, CUR), slot(0, 0, CUR)};
      OA::template read_at<FA, FB, 2>(pa, d, fa[NXT][0], fa[NXT][1], m);
    }
    refill2(J0{}, J1{});
    {
      const MfmaSlot m[4] = {slot(1, 0, CUR), slot(1, 1, CUR), slot(1, 0, CUR), slot(1, 0, CUR)};
      OB::template read_at<FA, FB, 2>(pb, d, fb[NXT][0], fb[NXT][1], m);
    }
    refill2(J2{}, J3{});
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using Fast = std::true_type;
  using Slow = std::false_type;
  // stages whose refill ends at or before K (stage = 128 bytes of K)
  const int nfull = (int)(g.Kc / (2 * kBK3));
  const int sfast = max(0, min(ns, nfull - kStages3)) & ~1;
  int st = 0;
  for (; st < sfast; st += 2) {
    stage_body(st, C0{}, Fast{});
    stage_body(st + 1, C1{}, Fast{});
  }
  for (; st < ns; st += 2) {
    stage_body(st, C0{}, Slow{});
    stage_body(st + 1, C1{}, Slow{});
  }

  // The two K halves of a quadrant meet in LDS: wave kq keeps fragment row
  // a = kq of its quadrant and hands row 1 - kq to its partner (4 KB per
  // fragment, lane-contiguous 16-byte pieces), then adds what it receives.
  // The exchange area lies past the output staging area, so the staging
  // writes below need no barrier after the exchange reads.
  constexpr int RS = BN * 2 + 16;
  constexpr int kXchg = 36864;  // >= BM * RS, 1 KB aligned
  static_assert(kXchg >= BM * RS && kXchg + 16 * 4096 <= 4 * 32768, "LDS split");
  mfma_drain();
  side_work<64 * NW>(g);  // after the drain: its VALU work may reuse fragment registers
  const float dq = es.dq(), inv_bs = es.inv_bs();
  barrier_only();  // every wave's last stage reads are done
  auto xslot = [&](int a, int b, int g4) {
    return smem5 + kXchg + ((quad * 2 + a) * 2 + b) * 4096 + g4 * 1024 + lane * 16;
  };
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (a == kq) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<v4f*>(xslot(a, b, g4)) =
            v4f{acc[a][b][4 * g4], acc[a][b][4 * g4 + 1], acc[a][b][4 * g4 + 2], acc[a][b][4 * g4 + 3]};
  }
  lds_barrier();
  v16f own[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const v4f p = *reinterpret_cast<const v4f*>(xslot(kq, b, g4));
#pragma unroll
      for (int t = 0; t < 4; ++t)
        own[b][4 * g4 + t] = (kq == 0 ? acc[0][b][4 * g4 + t] : acc[1][b][4 * g4 + t]) + p[t];
    }

  // Epilogue as in gemm3_kernel, for fragment row kq of the quadrant.
  const int il = ra0 + 32 * kq + (lane & 31);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int jl = rb0 + 32 * b + 8 * grp + 4 * (lane >> 5);
      float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (g.bias_kind != kBiasNone) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bias[t] = BiasStage<BN>::get(g, sbias, j0, jl + t, inv_bs);
      }
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(own[b][4 * grp + t], dq, bias[t]);
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

template <int LA, int LB, int FA, int FB>
__global__ __launch_bounds__(512, 1) void gemm5_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem5[];
  gemm5_body<LA, LB, FA, FB>(g, smem5);
}

constexpr int gemm5_lds_bytes() { return kGemm5BiasOff + BiasStage<128>::kBytes; }

}  // namespace fp8l
