// Fast-path FP8 GEMM for gfx950 (dimensions multiples of 16, matrices below
// 2 GiB): same contract as gemm_kernel in fp8l_gemm.hpp,
//
//   C[i, j] = sum_k A(i, k) B(j, k) / (sa sb) (+ bias[j]), bf16 out,
//
// with the fwd / dX / dW operand layouts described there.
//
// Design for CDNA4:
//  * Block tile BM x BN computed by a WGM x WGN grid of waves: 256x256 by 8
//    waves (two per SIMD, 128x64 each, so one wave multiplies while the other
//    waits on LDS), 256x128 and 128x128 by 4 waves.  Each wave owns its
//    quarter/eighth as 32x32 tiles of v_mfma_f32_32x32x64_f8f6f4 with fp32
//    accumulators (AGPRs).
//  * K advances 128 bytes per LDS stage (two MFMA k-steps).  LDS holds two
//    stages (dynamic shared memory, up to 128 KB).  The next stage is fetched
//    into registers with buffer loads while the current one is multiplied,
//    then written to the other LDS buffer; one barrier per stage, which waits
//    only for the LDS writes (never for the loads in flight).
//  * Buffer loads return zero past the end of the matrix, and a K chunk
//    beyond the contraction length is redirected past the end, so ragged
//    tails need no branches and contribute exact zeros.
//  * k-contiguous operand tiles sit in LDS as [rows][128 B]; crosswise
//    operand tiles (dX's W, both operands of dW) sit as they lie in memory,
//    [128 k][rows], and are fed to the MFMA with ds_read_b64_tr_b8.  16-byte
//    chunks are XOR-swizzled per row against LDS bank conflicts.
//  * Blocks are renumbered so that consecutive tile indices land on the same
//    XCD (workgroups are dealt round-robin over the 8 XCDs), then walked in
//    groups of 8 tile rows, so tiles sharing operand rows share an L2.
//  * Epilogue: (1/sa)(1/sb), bias in one fp32 fma, one RNE to bf16; each lane
//    holds 4 consecutive columns per store (8 bytes).
#pragma once

#include "fp8l_gemm.hpp"

namespace fp8l {

constexpr int kBK2 = 128;

typedef float v16f __attribute__((ext_vector_type(16)));

FP8L_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

FP8L_DEV uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// LDS write completion, then a workgroup barrier.  Loads still in flight are
// not waited for; the memory clobber keeps the compiler from moving LDS
// accesses across it.
FP8L_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Chunk swizzles.  k-contiguous tiles ([rows][128 B]): 32 consecutive rows
// read one logical chunk; rows r and r^8 fall in different bank halves.
// Crosswise tiles ([128 k][R bytes]): the two 16-lane groups serviced
// together by one ds_read_b64_tr_b8 read chunks cc and cc+1 (cc even) of the
// same 8 consecutive k rows; the swizzle keeps bit 0 of the chunk index, so
// the two groups land on disjoint slots and each group's 8 rows on distinct
// ones.
template <int ROWB>
FP8L_DEV int swz_cross(int kk) {
  if constexpr (ROWB >= 256)
    return (kk & 7) << 1;          // 8 rows of 256 B: 16 distinct 16-B slots
  else
    return ((kk >> 1) & 3) << 1;   // 128-B rows pair up within a 256-B bank row
}

// Per-operand tile geometry.  R = tile extent along C (rows of A or columns
// of B), NT = threads per block.  Thread t owns kNL 16-byte chunks per stage.
template <int L, int R, int NT>
struct Tile2 {
  static constexpr int kBytes = R * kBK2;
  static constexpr int kNL = kBytes / 16 / NT;
  // k-contiguous: chunk t&7 of rows (t>>3) + (NT/8) i
  // crosswise:    chunk t % (R/16) of k rows t / (R/16) + (NT / (R/16)) i
  static constexpr int kCpr = (L == kKContig) ? 8 : R / 16;   // chunks per LDS row
  static constexpr int kRowsPerPass = NT / kCpr;
  static_assert(kNL >= 1, "tile too small for the block");

  // Per-thread state: byte offset of each chunk at k = 0, and the chunk's
  // position along the contiguous dimension (for the edge mask).
  uint32_t base[kNL];
  int32_t inner[kNL];
  int64_t inlim;
  uint32_t kstep;  // byte step of one stage along k

  FP8L_DEV void init(int64_t ld, int64_t rbase, int64_t rlim, int64_t klim) {
    const int t = threadIdx.x;
    const int c = t % kCpr;
#pragma unroll
    for (int i = 0; i < kNL; ++i) {
      const int r = t / kCpr + kRowsPerPass * i;
      if constexpr (L == kKContig) {
        base[i] = (uint32_t)((rbase + r) * ld + 16 * c);
        inner[i] = 16 * c;              // + k0
      } else {
        base[i] = (uint32_t)((int64_t)r * ld + rbase + 16 * c);
        inner[i] = (int32_t)(rbase + 16 * c);
      }
    }
    inlim = (L == kKContig) ? klim : rlim;
    kstep = (L == kKContig) ? (uint32_t)kBK2 : (uint32_t)(kBK2 * ld);
  }
  // Rows past the matrix end land past num_records; a chunk past the
  // contiguous extent is sent there explicitly.
  FP8L_DEV void load(__amdgpu_buffer_rsrc_t rs, int kt, uint4 v[kNL]) const {
    const uint32_t koff = (uint32_t)kt * kstep;
    const int64_t k0 = (int64_t)kt * kBK2;
#pragma unroll
    for (int i = 0; i < kNL; ++i) {
      const int64_t in = (L == kKContig) ? k0 + inner[i] : (int64_t)inner[i];
      const uint32_t off = in < inlim ? base[i] + koff : 0x80000000u;
      v[i] = buf_load16(rs, off);
    }
  }
  FP8L_DEV static void store(uint8_t* s, const uint4 v[kNL]) {
    const int t = threadIdx.x;
    const int c = t % kCpr;
#pragma unroll
    for (int i = 0; i < kNL; ++i) {
      const int r = t / kCpr + kRowsPerPass * i;
      const int pc = (L == kKContig) ? (c ^ swz_k(r)) : (c ^ swz_cross<R>(r));
      *reinterpret_cast<uint4*>(s + r * (kCpr * 16) + pc * 16) = v[i];
    }
  }
  // 32x32x64 MFMA input for lane l: tile index f0 + (l & 31), k bytes
  // 64*ks + 32*(l>>5) + [0, 32).
  FP8L_DEV static v8i frag(const uint8_t* s, int f0, int ks) {
    const int l = threadIdx.x & 63;
    v8i out;
    if constexpr (L == kKContig) {
      const int r = f0 + (l & 31);
      const int c0 = 4 * ks + 2 * (l >> 5);
      const uint4 lo = *reinterpret_cast<const uint4*>(s + r * 128 + ((c0 ^ swz_k(r)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(s + r * 128 + (((c0 + 1) ^ swz_k(r)) << 4));
      out[0] = lo.x; out[1] = lo.y; out[2] = lo.z; out[3] = lo.w;
      out[4] = hi.x; out[5] = hi.y; out[6] = hi.z; out[7] = hi.w;
    } else {
      // transpose read: in each 16-lane group, lane 8h+i gets byte i of the
      // 8-byte rows addressed by lanes 2j+h; group q covers tile indices
      // f0 + 16 (q & 1) + [0, 16) and k rows 64 ks + 32 (q >> 1) + 8 t + j.
      const int q = l >> 4, sidx = l & 15;
      const int cc = (f0 >> 4) + (q & 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kk = 64 * ks + 32 * (q >> 1) + 8 * t + (sidx >> 1);
        const uint8_t* addr = s + kk * R + ((cc ^ swz_cross<R>(kk)) << 4) + ((sidx & 1) << 3);
        const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)((__attribute__((address_space(3))) uint8_t*)addr));
        out[2 * t] = r.x;
        out[2 * t + 1] = r.y;
      }
    }
    return out;
  }
};

// Renumber blocks so consecutive tile ids share an XCD (round-robin dealing
// over 8 XCDs), then group 8 tile rows.
FP8L_DEV void tile_coords_xcd(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nb = tiles_m * tiles_n;
  const int q = nb / 8, r = nb % 8;
  const int x = b % 8, i = b / 8;
  const int pid = x * q + min(x, r) + i;
  tile_coords(pid, tiles_m, tiles_n, tm, tn);
}

template <int BM, int BN, int WGM, int WGN, int LA, int LB, int FA, int FB>
__global__ __launch_bounds__(64 * WGM * WGN, (64 * WGM * WGN == 256 && BM * BN <= 128 * 128) ? 2 : 1)
void gemm2_kernel(GemmArgs g) {
  constexpr int NT = 64 * WGM * WGN;
  using TA = Tile2<LA, BM, NT>;
  using TB = Tile2<LB, BN, NT>;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 MFMA tiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem2[];
  constexpr int kStage = TA::kBytes + TB::kBytes;  // stage s: A at s*kStage, B after it

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_coords_xcd(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;

  if (blockIdx.x == 0 && tid == 0) {
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

  // operand extents in bytes (rows x leading dimension)
  const int64_t a_rows = (LA == kKContig) ? g.Mc : g.Kc;
  const int64_t b_rows = (LB == kKContig) ? g.Nc : g.Kc;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, (uint32_t)(a_rows * g.lda));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, (uint32_t)(b_rows * g.ldb));
  TA ta;
  TB tb;
  ta.init(g.lda, i0, g.Mc, g.Kc);
  tb.init(g.ldb, j0, g.Nc, g.Kc);

  const int wm = wave / WGN, wn = wave % WGN;
  v16f acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const int nk = (int)((g.Kc + kBK2 - 1) / kBK2);
  uint4 va[TA::kNL], vb[TB::kNL];
  if (nk > 0) {
    ta.load(ra, 0, va);
    tb.load(rb, 0, vb);
    TA::store(smem2, va);
    TB::store(smem2 + TA::kBytes, vb);
  }
  lds_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      ta.load(ra, kt + 1, va);
      tb.load(rb, kt + 1, vb);
    }
    const uint8_t* sa = smem2 + cur * kStage;
    const uint8_t* sb = sa + TA::kBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i fa[FM], fb[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) fa[f] = TA::frag(sa, wm * WTM + 32 * f, ks);
#pragma unroll
      for (int f = 0; f < FN; ++f) fb[f] = TB::frag(sb, wn * WTN + 32 * f, ks);
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[b], fa[a], acc[a][b], FB,
                                                                       FA, 0, 0, 0, 0);
    }
    if (more) {
      TA::store(smem2 + (cur ^ 1) * kStage, va);
      TB::store(smem2 + (cur ^ 1) * kStage + TA::kBytes, vb);
    }
    lds_barrier();
  }

  // epilogue: lane holds, for reg e, C[i0 + wm*WTM + 32a + (lane & 31)]
  //   [j0 + wn*WTN + 32b + 8(e>>2) + 4(lane>>5) + (e&3)]
  const float dq = (1.0f / *g.scale_a) * (1.0f / *g.scale_b);
  const float inv_bs =
      (g.bias_kind == kBiasE4M3 || g.bias_kind == kBiasE5M2) ? 1.0f / *g.bias_scale : 1.0f;
#pragma unroll
  for (int b = 0; b < FN; ++b) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int64_t j = j0 + wn * WTN + 32 * b + 8 * grp + 4 * (lane >> 5);
      float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (g.bias_kind != kBiasNone) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (j + t < g.Nc) bias[t] = bias_at(g, j + t, inv_bs);
      }
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int64_t i = i0 + wm * WTM + 32 * a + (lane & 31);
        if (i >= g.Mc) continue;
        uint32_t h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          h[t] = f32_to_bf16(__builtin_fmaf(acc[a][b][4 * grp + t], dq, bias[t]));
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
}

template <int BM, int BN>
constexpr int gemm2_lds_bytes() {
  return 2 * (BM + BN) * kBK2;
}

}  // namespace fp8l
