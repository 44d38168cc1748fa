// Pipelined FP8 GEMM for gfx950 (dimensions multiples of 16, matrices below
// 2 GiB); same contract as gemm_kernel in fp8l_gemm.hpp:
//
//   C[i, j] = sum_k A(i, k) B(j, k) / (sa sb) (+ bias[j]), bf16 out.
//
// Why this shape of pipeline: on MI355X an operand fetch that misses L2
// takes thousands of cycles, far more than one K step of MFMA work, so the
// K loop must keep several steps of operands in flight.  Register staging
// cannot (each step in flight costs a register set), so operands go from
// HBM/L2 straight into LDS with buffer_load_dwordx4 ... lds (DMA: each lane
// writes its 16 bytes at base + 16 * lane, and an offset past the buffer's
// end writes zeros, which is how row and K tails become exact zeros).
//
//  * K advances 64 bytes per step (one v_mfma_f32_32x32x64_f8f6f4 depth).
//    LDS holds 4 steps; the DMA for step k+4 is issued while step k is being
//    multiplied, so each step's operands have 3 steps of MFMA time to land.
//  * Fragments are double-buffered in registers: during step k the waves
//    multiply step k's fragments while reading step k+1's from LDS.  One
//    barrier per step (it also retires the LDS buffer step k+4 refills).
//  * LDS reads are inline asm (ds_read_b128, ds_read_b64_tr_b8) that wait
//    for their own results: the compiler cannot see them, so it does not
//    drain the DMA queue before them; vmcnt is managed explicitly.
//  * k-contiguous tiles sit in LDS as [rows][64 B]; crosswise tiles (dX's W,
//    both operands of dW) as they lie in memory, [64 k][rows], read through
//    the LDS transpose ds_read_b64_tr_b8.  16-byte chunks are XOR-swizzled
//    against bank conflicts on both the DMA writes and the fragment reads.
//  * Block tile BM x BN by a WGM x WGN grid of waves, each wave a grid of
//    32x32 MFMA tiles; tiles renumbered XCD-major (tile_coords_xcd).
//  * Epilogue: (1/sa)(1/sb), bias in one fp32 fma, one RNE to bf16, staged
//    through LDS and written back as whole rows.
#pragma once

#include <type_traits>

#include "fp8l_gemm.hpp"
#include "fp8l_quantize.hpp"

namespace fp8l {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer resource over [p, p + bytes): raw buffer loads past the end return
// zeros (flags 0x00020000: the gfx9-family resource word 3).
FP8L_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS write completion, then a workgroup barrier.  Loads still in flight are
// not waited for; the memory clobber keeps the compiler from moving LDS
// accesses across it.
FP8L_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Chunk swizzle of crosswise tiles ([64 k][ROWB bytes]): the two 16-lane
// groups serviced together by one ds_read_b64_tr_b8 read chunks cc and cc+1
// (cc even) of the same 8 consecutive k rows; the swizzle keeps bit 0 of
// the chunk index, so the two groups land on disjoint slots and each
// group's 8 rows on distinct ones.
template <int ROWB>
FP8L_DEV int swz_cross(int kk) {
  if constexpr (ROWB >= 256)
    return (kk & 7) << 1;          // 8 rows of 256 B: 16 distinct 16-B slots
  else
    return ((kk >> 1) & 3) << 1;   // 128-B rows pair up within a 256-B bank row
}

// Workgroups are dealt round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Renumber so that each XCD gets a contiguous range of tile indices,
// then walk them in groups of tile rows (tile_coords), so that tiles sharing
// operand rows or columns share one XCD's L2.
FP8L_DEV void tile_coords_xcd(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nb = tiles_m * tiles_n;
  const int q = nb / 8, r = nb % 8;
  const int x = b % 8, i = b / 8;
  const int pid = x * q + min(x, r) + i;
  tile_coords(pid, tiles_m, tiles_n, tm, tn);
}

constexpr int kBK3 = 64;
constexpr int kStages3 = 4;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

FP8L_DEV uint32_t lds_off(const uint8_t* p) { return (uint32_t)(uintptr_t)(const lds_u8*)p; }

// k-contiguous rows of 64 B (4 chunks): 16 consecutive rows reading one
// logical chunk hit 16 distinct 16-byte slots of a 256-byte bank row, and 8
// consecutive rows 8 distinct slots of a 128-byte one.
FP8L_DEV int swz64(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// ---- LDS fragment reads (inline asm; each block waits for its own data)

FP8L_DEV void lds_read_kc2(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, v8i& f0, v8i& f1) {
  v4i r0, r1, r2, r3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
  f0 = v8i{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  f1 = v8i{r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w};
}

FP8L_DEV void lds_read_x2(const uint32_t a[8], v8i& f0, v8i& f1) {
  v2i r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b8 %0, %8\n\t"
      "ds_read_b64_tr_b8 %1, %9\n\t"
      "ds_read_b64_tr_b8 %2, %10\n\t"
      "ds_read_b64_tr_b8 %3, %11\n\t"
      "ds_read_b64_tr_b8 %4, %12\n\t"
      "ds_read_b64_tr_b8 %5, %13\n\t"
      "ds_read_b64_tr_b8 %6, %14\n\t"
      "ds_read_b64_tr_b8 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
  f0 = v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
  f1 = v8i{r4.x, r4.y, r5.x, r5.y, r6.x, r6.y, r7.x, r7.y};
}

// MFMAs of the current K step issued inside the same asm block as the LDS
// reads of the next step's fragments, so the read latency overlaps MFMA
// execution while the block still waits for its own data.  Operand roles as
// in the builtin form: vdst/srcC = accumulator (AGPRs), srcA = fragment of B
// (C columns, format FB via cbsz), srcB = fragment of A (C rows, FA via
// blgp).  The compiler does not see these MFMAs, so the blocks carry their
// own hazard padding and kernels drain before any VALU read of an
// accumulator.  Mfma<NM> bundles the NM (1..4) accumulator updates a block
// issues; unused slots alias slot 0 and are never named in the asm.
struct MfmaSlot {
  v16f* c;
  const v8i* b;
  const v8i* x;
};

#define FP8L_MF(i) \
  "v_mfma_f32_32x32x64_f8f6f4 %[c" #i "], %[b" #i "], %[x" #i "], %[c" #i "] cbsz:%[fb] blgp:%[fa]\n\t"
#define FP8L_MF1 FP8L_MF(0)
#define FP8L_MF2 FP8L_MF1 FP8L_MF(1)
#define FP8L_MF3 FP8L_MF2 FP8L_MF(2)
#define FP8L_MF4 FP8L_MF3 FP8L_MF(3)
#define FP8L_CO(i) [c##i] "+a"(*m[i].c)
#define FP8L_CO1 FP8L_CO(0)
#define FP8L_CO2 FP8L_CO1, FP8L_CO(1)
#define FP8L_CO3 FP8L_CO2, FP8L_CO(2)
#define FP8L_CO4 FP8L_CO3, FP8L_CO(3)
#define FP8L_CI(i) [b##i] "v"(*m[i].b), [x##i] "v"(*m[i].x)
#define FP8L_CI1 FP8L_CI(0)
#define FP8L_CI2 FP8L_CI1, FP8L_CI(1)
#define FP8L_CI3 FP8L_CI2, FP8L_CI(2)
#define FP8L_CI4 FP8L_CI3, FP8L_CI(3)
#define FP8L_FMT [fb] "n"(FB), [fa] "n"(FA)

template <int FA, int FB, int NM>
FP8L_DEV void mfma_only(const MfmaSlot (&m)[4]) {
  // s_nop 1: operands may have just been written by VALU
#define FP8L_ONLY(n) \
  asm volatile("s_nop 1\n\t" FP8L_MF##n "" : FP8L_CO##n : FP8L_CI##n, FP8L_FMT)
  if constexpr (NM == 1) FP8L_ONLY(1);
  else if constexpr (NM == 2) FP8L_ONLY(2);
  else if constexpr (NM == 3) FP8L_ONLY(3);
  else FP8L_ONLY(4);
#undef FP8L_ONLY
}

// VALU reads of MFMA results need wait states the compiler cannot insert
// for asm MFMAs (a 16-pass MFMA needs 18); pad generously.
FP8L_DEV void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

// Calls f(integral_constant<int, i>) for i = 0 .. N-1 (compile-time indices,
// so register arrays indexed by them stay in registers).
template <int N, int I = 0, typename F>
FP8L_DEV void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Explicit waits on the DMA queue (vmcnt) and the LDS barrier.
template <int N>
FP8L_DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
FP8L_DEV void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// The epilogue's scales, loaded ahead of the first DMA stages (older than
// every stage load, they leave the loop's in-order vmcnt waits exact) and
// first used in the epilogue: the reciprocals are taken there
// (EpiScales::dq/inv_bs), so no use of them makes the prologue wait.
struct EpiScales {
  float sa, sb, bs;  // scale_a, scale_b, bias_scale for an FP8 bias (else 1)
  FP8L_DEV float dq() const { return (1.0f / sa) * (1.0f / sb); }
  FP8L_DEV float inv_bs() const { return 1.0f / bs; }
};

FP8L_DEV EpiScales load_scales(const GemmArgs& g) {
  EpiScales e;
  e.sa = *g.scale_a;
  e.sb = *g.scale_b;
  e.bs = (g.bias_kind == kBiasE4M3 || g.bias_kind == kBiasE5M2) ? *g.bias_scale : 1.0f;
  return e;
}

// Work beside the tile: block 0's snapshot copies for pre-quantized
// operands and ring folds, and the bias-gradient finalize (shared by all
// blocks; one thread per entry walking all rows, in the first tile column's
// blocks only, made those blocks the launch's last by many microseconds).
// Kernels call it after the K loop and the MFMA drain, when no operand DMA
// is in flight: a wait for these loads then waits for nothing else (in the
// prologue the first such wait held every stage in flight; the ring folds
// there delayed block 0's first stage by a device round trip and measured
// ~0.5 us slower per GEMM).  NT: threads per block.
template <int NT>
FP8L_DEV void side_work(const GemmArgs& g) {
  if (prob_block(g) == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    if (g.aux_scale_dst0) *g.aux_scale_dst0 = *g.aux_scale_src0;
    if (g.aux_amax_dst0) *g.aux_amax_dst0 = 0.0f;
    if (g.aux_scale_dst1) *g.aux_scale_dst1 = *g.aux_scale_src1;
    if (g.aux_amax_dst1) *g.aux_amax_dst1 = 0.0f;
  }
  if (g.db) db_finalize<NT>(g);
  ring_folds(g);
}

// Bias of the block's BN output columns, staged in LDS for the epilogue so
// that it does not wait a memory latency for them.  Wave 0 fetches the raw
// codes (bf16 or fp8 bytes) with one DMA load issued before any operand
// stage: loads complete in issue order, so the prologue's wait for the
// first stage covers it, and no register holds the codes (a register
// destination would make the compiler wait for it, and so for every stage
// in flight, at its first use).  Lane l carries bytes [16 l, 16 l + 16) of
// the block's columns; lanes past the bias read zeros, so the area is
// kBytes = 1 KB.  The DMA path needs every 16-byte piece wholly inside or
// wholly outside the bias (N times the code size a multiple of 16);
// otherwise, and without bias, the epilogue reads the bias from memory as
// before (bias_at).  get() decodes as bias_at does, bit for bit.
template <int BN>
struct BiasStage {
  static constexpr int kBytes = 1024;
  static_assert(2 * BN <= kBytes, "bias codes of the block in one DMA load");
  FP8L_DEV static int code_bytes(const GemmArgs& g) { return g.bias_kind == kBiasBF16 ? 2 : 1; }
  FP8L_DEV static bool staged(const GemmArgs& g) {
    return g.bias_kind != kBiasNone && (g.Nc * code_bytes(g)) % 16 == 0;
  }
  // wave: this wave's index (uniform)
  FP8L_DEV static void load(const GemmArgs& g, int64_t j0, uint8_t* sb, int wave) {
    if (wave != 0 || !staged(g)) return;
    const int eb = code_bytes(g);
    const uint32_t bytes = (uint32_t)(g.Nc * eb);
    const uint32_t first = (uint32_t)(j0 * eb);
    const int lane = threadIdx.x & 63;
    const uint32_t off = first + 16u * lane;
    const uint32_t voff = (16 * lane < BN * eb && off < bytes) ? off : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(g.bias, bytes),
                                             (__attribute__((address_space(3))) void*)sb, 16,
                                             voff, 0, 0, 0);
  }
  // bias of block column jl (the value bias_at gives for column j0 + jl)
  FP8L_DEV static float get(const GemmArgs& g, const uint8_t* sb, int64_t j0, int jl,
                            float inv_bs) {
    if (!staged(g)) return j0 + jl < g.Nc ? bias_at(g, j0 + jl, inv_bs) : 0.0f;
    if (g.bias_kind == kBiasBF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(sb)[jl]);
    return fp8_to_f32_rt(sb[jl], g.bias_kind == kBiasE4M3 ? kE4M3 : kE5M2) * inv_bs;
  }
};

// One operand of the pipelined kernel.  R: tile extent along C; NW: waves.
template <int L, int R, int NW>
struct Op3 {
  static constexpr int kBytes = R * kBK3;          // one K step
  static constexpr int kBlocks = kBytes / 1024;    // 1 KB DMA blocks per step
  static constexpr int kPerWave = kBlocks / NW;    // DMA instructions per wave per step
  static_assert(kPerWave >= 1 && kBlocks % NW == 0, "tile / wave split");
  static constexpr int kCpr = (L == kKContig) ? 4 : R / 16;  // 16-byte chunks per LDS row
  static constexpr int kLayout = L;

  uint32_t base[kPerWave];  // byte offset of this lane's chunk at step 0
  int32_t inner[kPerWave];  // position along the contiguous dimension (edge mask)
  int64_t inlim;
  uint32_t kstep;           // bytes per K step

  FP8L_DEV static int swz(int row) {
    if constexpr (L == kKContig) return swz64(row);
    else return swz_cross<R>(row);
  }

  FP8L_DEV void init(int64_t ld, int64_t rbase, int64_t rlim, int64_t klim) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;
      const int row = blk * (1024 / (kCpr * 16)) + lane / kCpr;  // LDS row of this lane
      const int c = (lane % kCpr) ^ swz(row);                    // logical chunk it holds
      if constexpr (L == kKContig) {
        base[i] = (uint32_t)((rbase + row) * ld + 16 * c);
        inner[i] = 16 * c;
      } else {
        base[i] = (uint32_t)((int64_t)row * ld + rbase + 16 * c);
        inner[i] = (int32_t)(rbase + 16 * c);
      }
    }
    inlim = (L == kKContig) ? klim : rlim;
    kstep = (L == kKContig) ? (uint32_t)kBK3 : (uint32_t)(kBK3 * ld);
    if constexpr (L != kKContig) {
      // columns past the edge: an offset past every resource (loop-invariant)
#pragma unroll
      for (int i = 0; i < kPerWave; ++i)
        if ((int64_t)inner[i] >= inlim) base[i] = 0x80000000u;
    }
  }

  // DMA instruction I of a K step that lies wholly inside K, through the
  // resource over the whole operand: the lane's fixed offset, and the step's
  // advance soff (uniform) as the instruction's scalar offset.  The range
  // check sees only the lane's offset, which is enough here: rows past the
  // operand's last one and columns past its edge (whose offsets init set to
  // 2^31) have offsets past the range and read zeros, and every other byte
  // the step reads lies inside the operand because the step ends at or
  // before K.  Against issue_step this drops the per-step resource and the
  // per-lane K test and select.
  template <int I>
  FP8L_DEV void issue_full(__amdgpu_buffer_rsrc_t rs, uint8_t* s, uint32_t soff, int wave) const {
    const uint32_t voff = base[I];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(s + (wave * kPerWave + I) * 1024), 16, voff,
        soff, 0, 0);
  }

  // DMA instruction i of K step kt into the step buffer at s.
  template <int I>
  FP8L_DEV void issue_one(__amdgpu_buffer_rsrc_t rs, uint8_t* s, int kt) const {
    const int wave = threadIdx.x >> 6;
    const int64_t in = (L == kKContig) ? (int64_t)kt * kBK3 + inner[I] : (int64_t)inner[I];
    const uint32_t off = in < inlim ? base[I] + (uint32_t)kt * kstep : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(s + (wave * kPerWave + I) * 1024), 16, off, 0,
        0, 0);
  }

  // DMA instruction I of K step kt through a buffer resource advanced to
  // the step (rs_kt: base moved by kt * kstep bytes, record count reduced by
  // as much and clamped at zero; see step_rsrc), so the per-lane offset is
  // loop-invariant and the range check still sees every byte.  Only a K step
  // that reaches past the end of a k-contiguous operand needs per-lane
  // selects (those bytes lie inside the buffer, in the next row).  wave: this
  // wave's index, uniform, so the LDS address stays scalar.
  template <int I>
  FP8L_DEV void issue_step(__amdgpu_buffer_rsrc_t rs_kt, uint8_t* s, int kt, int wave) const {
    uint32_t voff;
    if constexpr (L == kKContig) {
      // K < 2^31 on this path (the resource's byte count is 32-bit)
      const int k0 = kt * kBK3, klim = (int)inlim;
      const int full = __builtin_amdgcn_readfirstlane(k0 + kBK3 <= klim ? 1 : 0);
      voff = (full || k0 + inner[I] < klim) ? base[I] : 0x80000000u;
    } else {
      voff = (int64_t)inner[I] < inlim ? base[I] : 0x80000000u;  // columns past the edge
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs_kt, (__attribute__((address_space(3))) void*)(s + (wave * kPerWave + I) * 1024), 16, voff,
        0, 0, 0);
  }

  // Resource over the operand advanced to K step kt (uniform arithmetic).
  // (readfirstlane: the values are uniform, and saying so keeps the resource
  // in scalar registers instead of a per-lane loop around each load)
  FP8L_DEV __amdgpu_buffer_rsrc_t step_rsrc(const uint8_t* p, uint32_t bytes, int kt) const {
    const uint32_t adv = __builtin_amdgcn_readfirstlane((uint32_t)kt * kstep);
    const uint32_t n = __builtin_amdgcn_readfirstlane(adv < bytes ? bytes - adv : 0u);
    return make_rsrc(p + adv, n);
  }

  // DMA of K step kt into the step buffer at s (wave-uniform).
  FP8L_DEV void issue(__amdgpu_buffer_rsrc_t rs, uint8_t* s, int kt) const {
    const int wave = threadIdx.x >> 6;
    const uint32_t koff = (uint32_t)kt * kstep;
    const int64_t k0 = (int64_t)kt * kBK3;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int64_t in = (L == kKContig) ? k0 + inner[i] : (int64_t)inner[i];
      const uint32_t off = in < inlim ? base[i] + koff : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(s + (wave * kPerWave + i) * 1024), 16, off,
          0, 0, 0);
    }
  }

  // LDS addresses of the reads that build two 32x32x64 fragments for tile
  // indices f0 and f0 + 32 (lane l: index f0 + (l & 31), k bytes
  // 32 (l >> 5) + [0, 32)).  k-contiguous: 2 reads per fragment; crosswise:
  // 4 transpose reads per fragment (in each 16-lane group, lane 8h+i gets
  // byte i of the 8-byte rows addressed by lanes 2j+h).
  FP8L_DEV static void frag_addrs(const uint8_t* s, int f0, uint32_t a[8]) {
    const int l = threadIdx.x & 63;
    const uint32_t sb = lds_off(s);
    if constexpr (L == kKContig) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int r = f0 + 32 * f + (l & 31);
        const int c0 = 2 * (l >> 5);
        a[2 * f + 0] = sb + r * 64 + ((c0 ^ swz64(r)) << 4);
        a[2 * f + 1] = sb + r * 64 + (((c0 + 1) ^ swz64(r)) << 4);
      }
    } else {
      const int q = l >> 4, sidx = l & 15;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int cc = ((f0 + 32 * f) >> 4) + (q & 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kk = 32 * (q >> 1) + 8 * t + (sidx >> 1);
          a[4 * f + t] = sb + kk * R + ((cc ^ swz_cross<R>(kk)) << 4) + ((sidx & 1) << 3);
        }
      }
    }
  }

  FP8L_DEV static void read2(const uint8_t* s, int f0, v8i& x0, v8i& x1) {
    uint32_t a[8];
    frag_addrs(s, f0, a);
    if constexpr (L == kKContig)
      lds_read_kc2(a[0], a[1], a[2], a[3], x0, x1);
    else
      lds_read_x2(a, x0, x1);
  }
};

// Fragment reads addressed with the instruction's immediate offset, so a
// step needs one or two address registers per operand.  A k-contiguous
// fragment 32 rows further lies exactly 2048 bytes further (the chunk
// swizzle repeats every 4 rows); the four 8-row reads of a crosswise
// fragment lie 8 R bytes apart (the swizzle repeats every 8 k rows).
#define FP8L_RKC(r, a, o) "ds_read_b128 %[" #r "], %[" #a "] offset:%[" #o "]\n\t"
#define FP8L_RX(r, a, o) "ds_read_b64_tr_b8 %[" #r "], %[" #a "] offset:%[" #o "]\n\t"

// k-contiguous fragment at offset OFF from the lane addresses a0, a1
template <int FA, int FB, int NM, int OFF>
FP8L_DEV void kc1o(uint32_t a0, uint32_t a1, v8i& n0, const MfmaSlot (&m)[4]) {
  v4i r0, r1;
#define FP8L_KC1O(n)                                                                      \
  asm volatile(FP8L_RKC(r0, a0, o0) FP8L_RKC(r1, a1, o0) FP8L_MF##n "s_waitcnt lgkmcnt(0)" \
               : [r0] "=&v"(r0), [r1] "=&v"(r1), FP8L_CO##n                                \
               : [a0] "v"(a0), [a1] "v"(a1), [o0] "n"(OFF), FP8L_CI##n, FP8L_FMT           \
               : "memory")
  if constexpr (NM == 1) FP8L_KC1O(1);
  else if constexpr (NM == 2) FP8L_KC1O(2);
  else if constexpr (NM == 3) FP8L_KC1O(3);
  else FP8L_KC1O(4);
#undef FP8L_KC1O
  n0 = v8i{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
}

// k-contiguous fragment pair at offsets O0 and O0 + D1
template <int FA, int FB, int NM, int D1 = 2048, int O0 = 0>
FP8L_DEV void kc2o(uint32_t a0, uint32_t a1, v8i& n0, v8i& n1, const MfmaSlot (&m)[4]) {
  v4i r0, r1, r2, r3;
#define FP8L_KC2O(n)                                                                           \
  asm volatile(FP8L_RKC(r0, a0, o0) FP8L_RKC(r1, a1, o0) FP8L_RKC(r2, a0, o1)                  \
                   FP8L_RKC(r3, a1, o1) FP8L_MF##n "s_waitcnt lgkmcnt(0)"                      \
               : [r0] "=&v"(r0), [r1] "=&v"(r1), [r2] "=&v"(r2), [r3] "=&v"(r3), FP8L_CO##n     \
               : [a0] "v"(a0), [a1] "v"(a1), [o0] "n"(O0), [o1] "n"(O0 + D1), FP8L_CI##n,    \
                 FP8L_FMT                                                                      \
               : "memory")
  if constexpr (NM == 1) FP8L_KC2O(1);
  else if constexpr (NM == 2) FP8L_KC2O(2);
  else if constexpr (NM == 3) FP8L_KC2O(3);
  else FP8L_KC2O(4);
#undef FP8L_KC2O
  n0 = v8i{r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
  n1 = v8i{r2.x, r2.y, r2.z, r2.w, r3.x, r3.y, r3.z, r3.w};
}

// crosswise fragment from base b: reads at b + t * DT, t = 0..3
template <int FA, int FB, int NM, int DT>
FP8L_DEV void x1o(uint32_t b, v8i& n0, const MfmaSlot (&m)[4]) {
  v2i r0, r1, r2, r3;
#define FP8L_X1O(n)                                                                            \
  asm volatile(FP8L_RX(r0, p0, o0) FP8L_RX(r1, p0, o1) FP8L_RX(r2, p0, o2) FP8L_RX(r3, p0, o3) \
                   FP8L_MF##n "s_waitcnt lgkmcnt(0)"                                           \
               : [r0] "=&v"(r0), [r1] "=&v"(r1), [r2] "=&v"(r2), [r3] "=&v"(r3), FP8L_CO##n     \
               : [p0] "v"(b), [o0] "n"(0), [o1] "n"(DT), [o2] "n"(2 * DT), [o3] "n"(3 * DT),     \
                 FP8L_CI##n, FP8L_FMT                                                          \
               : "memory")
  if constexpr (NM == 1) FP8L_X1O(1);
  else if constexpr (NM == 2) FP8L_X1O(2);
  else if constexpr (NM == 3) FP8L_X1O(3);
  else FP8L_X1O(4);
#undef FP8L_X1O
  n0 = v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
}

// crosswise fragment pair from bases b0, b1
template <int FA, int FB, int NM, int DT>
FP8L_DEV void x2o(uint32_t b0, uint32_t b1, v8i& n0, v8i& n1, const MfmaSlot (&m)[4]) {
  v2i r0, r1, r2, r3, r4, r5, r6, r7;
#define FP8L_X2O(n)                                                                             \
  asm volatile(FP8L_RX(r0, p0, o0) FP8L_RX(r1, p0, o1) FP8L_RX(r2, p0, o2) FP8L_RX(r3, p0, o3)  \
                   FP8L_RX(r4, p1, o0) FP8L_RX(r5, p1, o1) FP8L_RX(r6, p1, o2)                  \
                       FP8L_RX(r7, p1, o3) FP8L_MF##n "s_waitcnt lgkmcnt(0)"                    \
               : [r0] "=&v"(r0), [r1] "=&v"(r1), [r2] "=&v"(r2), [r3] "=&v"(r3), [r4] "=&v"(r4), \
                 [r5] "=&v"(r5), [r6] "=&v"(r6), [r7] "=&v"(r7), FP8L_CO##n                     \
               : [p0] "v"(b0), [p1] "v"(b1), [o0] "n"(0), [o1] "n"(DT), [o2] "n"(2 * DT),        \
                 [o3] "n"(3 * DT), FP8L_CI##n, FP8L_FMT                                         \
               : "memory")
  if constexpr (NM == 1) FP8L_X2O(1);
  else if constexpr (NM == 2) FP8L_X2O(2);
  else if constexpr (NM == 3) FP8L_X2O(3);
  else FP8L_X2O(4);
#undef FP8L_X2O
  n0 = v8i{r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
  n1 = v8i{r4.x, r4.y, r5.x, r5.y, r6.x, r6.y, r7.x, r7.y};
}

// Lane address registers of one operand's fragments in the stage-0 buffer
// (add a stage's byte offset to use them for that stage).  k-contiguous:
// the two chunk addresses of fragment f0 (fragment f0 + 32 i is at offset
// 2048 i).  Crosswise: one base per fragment f0 + 32 i, i < NF.
template <typename Op, int NF>
struct FragBase {
  uint32_t a[(Op::kLayout == kKContig) ? 2 : NF];
  FP8L_DEV void init(const uint8_t* s0, int f0) {
    uint32_t t[8];
    if constexpr (Op::kLayout == kKContig) {
      Op::frag_addrs(s0, f0, t);
      a[0] = t[0];
      a[1] = t[1];
    } else {
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        Op::frag_addrs(s0, f0 + 32 * i, t);
        a[i] = t[0];
      }
    }
  }
};

// LDS: the operand ring, or the staged output tile if that is larger, then
// the bias of the block's BN columns (BiasStage).
template <int BM, int BN>
constexpr int gemm3_bias_off() {
  return kStages3 * (BM + BN) * kBK3 > BM * (BN * 2 + 16) ? kStages3 * (BM + BN) * kBK3
                                                         : BM * (BN * 2 + 16);
}

template <int BM, int BN, int WGM, int WGN>
constexpr int gemm3_lds_bytes() {
  return gemm3_bias_off<BM, BN>() + BiasStage<BN>::kBytes;
}

// Epilogue of gemm3_kernel: bf16 output, or the FP8-output GEMM's passes
// (codes with the ring's scale, codes with the scale of a seeding amax pass,
// or that amax pass alone).
enum { kEpiBF16 = 0, kEpiFp8Ring = 1, kEpiFp8Seed = 2, kEpiAmax = 3 };

// FP8-output epilogue (fp8_gemm_fp8out).  y = acc (1/sa)(1/sb) + bias in
// fp32, the value the bf16 epilogue rounds; then q = enc(fl32(y s)) with the
// output ring's scale s, the quantize kernels' conversion (RNE, saturating,
// NaN to 0x7F | sign).  Codes are staged in LDS (rows padded by 16 bytes)
// and stored as 16-byte row pieces (the ragged end of a row byte by byte).
// max |y| over the block's outputs inside M x N goes to the launch's
// last-block election, which folds it into the output ring as a quantize
// launch does (with g.odefer, to the block's election group only, for the
// fold launch that follows the GEMM); kEpiAmax computes and elects max |y| only, leaving it for
// the converting pass of a seeding call.  acc: the block's accumulators in
// the pipelined kernels' fragment layout; s: the output scale (out_scale);
// sbias: the BiasStage area; NT: threads per block.
// Scale of the FP8-output epilogue: the ring's, or (seeding) S of the max
// the amax pass left in the header.  Kernels read it at their start, with
// the other scales, so the epilogue does not wait for it; the previous
// launch on the stream, which wrote it, has completed by then.
template <int EPI, int OF>
FP8L_DEV float out_scale(const GemmArgs& g) {
  if constexpr (EPI == kEpiFp8Ring) {
    return g.oring->scale;
  } else if constexpr (EPI == kEpiFp8Seed) {
    const float m = __uint_as_float(
        __hip_atomic_load(&g.oring->top_amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return scale_from_amax(m, FmtTraits<OF>::kMax, g.oring->scale);
  } else {
    return 0.0f;
  }
}

template <int BM, int BN, int WTM, int WTN, int EPI, int OF, int NT, int FM, int FN>
FP8L_DEV void fp8_out_epilogue(const GemmArgs& g, const v16f (&acc)[FM][FN], float dq,
                               float inv_bs, float s, const uint8_t* sbias, uint8_t* smem,
                               int64_t i0, int64_t j0, int wm, int wn) {
  constexpr int RSB = BN + 16;  // LDS bytes per staged row of codes
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t bid = blockIdx.y * prob_nblk(g) + prob_block(g), total = prob_nblk(g) * gridDim.y;
  const int64_t rows_left = g.Mc - i0, cols_left = g.Nc - j0;
  // a tile inside M x N needs no per-element mask on its max
  const bool interior = rows_left >= BM && cols_left >= BN;
  uint32_t mx = 0;
#pragma unroll
  for (int b = 0; b < FN; ++b) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int jl = wn * WTN + 32 * b + 8 * grp + 4 * (lane >> 5);
      float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (g.bias_kind != kBiasNone) {
#pragma unroll
        for (int t = 0; t < 4; ++t) bias[t] = BiasStage<BN>::get(g, sbias, j0, jl + t, inv_bs);
      }
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int il = wm * WTM + 32 * a + (lane & 31);
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(acc[a][b][4 * grp + t], dq, bias[t]);
        // max |v| bits of the four (above the infinity's bits: a NaN among them)
        const uint32_t m4 = max(max(absbits(v[0]), absbits(v[1])), max(absbits(v[2]), absbits(v[3])));
        if (interior) {
          mx = max(mx, m4);
        } else if (il < rows_left) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (jl + t < cols_left) mx = max(mx, absbits(v[t]));
        }
        if constexpr (EPI != kEpiAmax)
          *reinterpret_cast<uint32_t*>(smem + il * RSB + jl) = quant4_m<OF>(v, s, m4);
      }
    }
  }
  if constexpr (EPI == kEpiAmax) {
    amax_pass_finish<NT>(g.oring, mx, bid, total);
  } else {
    lds_barrier();
    constexpr int kChunks = BN / 16;
#pragma unroll 2
    for (int q = tid; q < BM * kChunks; q += NT) {
      const int r = q / kChunks, ch = q % kChunks;
      if (r < rows_left && 16 * ch < cols_left) {
        uint8_t* dst = g.c8 + (i0 + r) * g.ldc + j0 + 16 * ch;
        const uint8_t* src = smem + r * RSB + 16 * ch;
        if (16 * ch + 16 <= cols_left) {
          __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(src),
                                      reinterpret_cast<v4u*>(dst));
        } else {
          for (int k = 0; k < cols_left - 16 * ch; ++k) dst[k] = src[k];
        }
      }
    }
    QArgs qa = {};
    qa.ring = g.oring;
    qa.hist = g.ohist;
    qa.hist_len = g.ohist_len;
    qa.scale_used = g.oscale_used;
    qa.amax_out = g.oamax;
    if (EPI == kEpiFp8Ring && g.odefer)
      finish_launch<OF, kScaleDefer, NT>(qa, mx, s, bid, total);
    else
      finish_launch<OF, EPI == kEpiFp8Seed ? kScaleSeed : kScaleRing, NT>(qa, mx, s, bid, total);
  }
}

template <int BM, int BN, int WGM, int WGN, int LA, int LB, int FA, int FB, int EPI = kEpiBF16,
          int OF = kE4M3>
__global__ __launch_bounds__(64 * WGM * WGN, (BM * BN <= 128 * 128) ? 2 : 1)
void gemm3_kernel(GemmArgs g) {
  batch_slice(g);
  constexpr int NW = WGM * WGN;
  using OA = Op3<LA, BM, NW>;
  using OB = Op3<LB, BN, NW>;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 MFMA tiles per wave
  static_assert(FM % 2 == 0 && FN % 2 == 0, "fragments are read in pairs");
  constexpr int kStep = OA::kBytes + OB::kBytes;  // LDS bytes per K step
  constexpr int kDma = OA::kPerWave + OB::kPerWave;  // DMA instructions per wave per step
  extern __shared__ __attribute__((aligned(16))) uint8_t smem3[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_coords_xcd(prob_block(g), g.tiles_m, g.tiles_n, tm, tn);
  const int64_t i0 = (int64_t)tm * BM, j0 = (int64_t)tn * BN;
  uint8_t* const sbias = smem3 + gemm3_bias_off<BM, BN>();  // BiasStage area


  const int64_t a_rows = (LA == kKContig) ? g.Mc : g.Kc;
  const int64_t b_rows = (LB == kKContig) ? g.Nc : g.Kc;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(g.a, (uint32_t)(a_rows * g.lda));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(g.b, (uint32_t)(b_rows * g.ldb));
  OA oa;
  OB ob;
  oa.init(g.lda, i0, g.Mc, g.Kc);
  ob.init(g.ldb, j0, g.Nc, g.Kc);
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // uniform wave index

  const int wm = wave / WGN, wn = wave % WGN;
  v16f acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const int nk = (int)(((g.Kc + kBK3 - 1) / kBK3 + 1) & ~1);  // K steps, padded to even
  auto step_buf = [&](int kt) { return smem3 + (kt % kStages3) * kStep; };

  // prologue: DMA steps 0..3, then step 0's fragments
  BiasStage<BN>::load(g, j0, sbias, wv);  // ahead of the stages (see BiasStage)
  const EpiScales es = load_scales(g);
  const float s_out = out_scale<EPI, OF>(g);
  for (int s = 0; s < kStages3 && s < nk; ++s) {
    oa.issue(ra, step_buf(s), s);
    ob.issue(rb, step_buf(s) + OA::kBytes, s);
  }
  v8i fa[2][FM], fb[2][FN];
  if (nk > 0) {
    // step 0 landed: at most min(3, nk - 1) later steps still in flight
    const int later = min(3, nk - 1);
    if (later >= 3) wait_vm<3 * kDma>();
    else if (later == 2) wait_vm<2 * kDma>();
    else if (later == 1) wait_vm<kDma>();
    else wait_vm<0>();
    barrier_only();
#pragma unroll
    for (int f = 0; f < FM; f += 2) OA::read2(step_buf(0), wm * WTM + 32 * f, fa[0][f], fa[0][f + 1]);
#pragma unroll
    for (int f = 0; f < FN; f += 2)
      OB::read2(step_buf(0) + OA::kBytes, wn * WTN + 32 * f, fb[0][f], fb[0][f + 1]);
  }

  // One K step.  CUR holds step kt's fragments; the other set receives
  // step kt+1's.  Two MFMAs go ahead of the barrier; the rest are spread
  // over the asm blocks that read the next fragments (one block per
  // fragment pair), in row-major (a, b) order.
  constexpr int kGroups = FM / 2 + FN / 2;
  constexpr int kRest = FM * FN - 2;
  static_assert(kRest >= kGroups && kRest <= 4 * kGroups, "MFMA split");
  auto slot = [&](int CUR, int e) {
    const int a = e / FN, b = e % FN;
    return MfmaSlot{&acc[a][b], &fb[CUR][b], &fa[CUR][a]};
  };
  // fragment address registers in the step-0 buffer (a step adds its
  // buffer's byte offset)
  FragBase<OA, FM> fra;
  FragBase<OB, FN> frb;
  fra.init(smem3, wm * WTM);
  frb.init(smem3 + OA::kBytes, wn * WTN);
  // FAST: the refill of this step (step kt+4) lies wholly inside K, so it
  // is unconditional, goes through the whole-operand resources with the
  // advance as scalar offset (Op3::issue_full) and the wait count is fixed;
  // the last steps take the general form.
  auto kstep_body = [&](int kt, auto cur_tag, auto fast_tag) {
    constexpr int CUR = decltype(cur_tag)::value;
    constexpr int NXT = CUR ^ 1;
    constexpr bool FAST = decltype(fast_tag)::value;
    {
      const MfmaSlot m[4] = {slot(CUR, 0), slot(CUR, 1), slot(CUR, 0), slot(CUR, 0)};
      mfma_only<FA, FB, 2>(m);
    }
    if constexpr (FAST) {
      wait_vm<2 * kDma>();
    } else {
      // step kt+1 landed: at most min(2, nk-2-kt) later steps in flight
      const int later = min(2, nk - 2 - kt);
      if (later >= 2) wait_vm<2 * kDma>();
      else if (later == 1) wait_vm<kDma>();
      else wait_vm<0>();
    }
    barrier_only();  // step kt+1 visible to all; step kt's buffer is free
    // The DMA of step kt+4 (into the buffer just freed) is spread over the
    // groups: each load instruction occupies the wave until the load path
    // accepts it, and issued between groups it overlaps the MFMAs already
    // in flight instead of stalling them all at once.
    const bool refill = FAST || kt + kStages3 < nk;
    const int kf = kt + kStages3;
    uint8_t* const sf = step_buf(kf);
    const uint32_t d = (uint32_t)(((kt + 1) % kStages3) * kStep);
    static_for<kGroups>([&](auto gi_tag) {
      constexpr int gi = decltype(gi_tag)::value;
      // group gi issues entries [e0, e0 + n) of the MFMA list and the DMA
      // loads j with j * kGroups / kDma == gi
      constexpr int n = kRest / kGroups + (gi < kRest % kGroups ? 1 : 0);
      constexpr int e0 = 2 + gi * (kRest / kGroups) + (gi < kRest % kGroups ? gi : kRest % kGroups);
      constexpr int j0 = (gi * kDma + kGroups - 1) / kGroups;
      constexpr int j1 = ((gi + 1) * kDma + kGroups - 1) / kGroups;
      constexpr int nl = j1 - j0;                  // loads of this group
      constexpr int nt = nl < n - 1 ? nl : n - 1;  // loads placed between MFMAs
      auto load = [&](auto j_tag) {
        constexpr int j = decltype(j_tag)::value;
        if constexpr (FAST) {
          if constexpr (j < OA::kPerWave)
            oa.template issue_full<j>(ra, sf, (uint32_t)kf * oa.kstep, wv);
          else
            ob.template issue_full<j - OA::kPerWave>(rb, sf + OA::kBytes, (uint32_t)kf * ob.kstep, wv);
        } else if (refill) {
          if constexpr (j < OA::kPerWave)
            oa.template issue_one<j>(ra, sf, kf);
          else
            ob.template issue_one<j - OA::kPerWave>(rb, sf + OA::kBytes, kf);
        }
      };
      // loads that find no MFMA to follow go first
      static_for<nl - nt>([&](auto t) { load(std::integral_constant<int, j0 + decltype(t)::value>{}); });
      {
        constexpr int nf = n - nt;  // MFMAs inside the read block
        const MfmaSlot m[4] = {slot(CUR, e0), slot(CUR, nf > 1 ? e0 + 1 : e0),
                               slot(CUR, nf > 2 ? e0 + 2 : e0), slot(CUR, nf > 3 ? e0 + 3 : e0)};
        // fragments 2h, 2h+1 of the operand (64 h rows/columns further)
        auto read_pair = [&](const auto& fr, auto lay_tag, auto rows_tag, v8i& n0, v8i& n1,
                             auto h_tag) {
          constexpr int lay = decltype(lay_tag)::value, R = decltype(rows_tag)::value;
          constexpr int h = decltype(h_tag)::value;
          if constexpr (lay == kKContig)
            kc2o<FA, FB, nf, 2048, 4096 * h>(fr.a[0] + d, fr.a[1] + d, n0, n1, m);
          else
            x2o<FA, FB, nf, 8 * R>(fr.a[2 * h] + d, fr.a[2 * h + 1] + d, n0, n1, m);
        };
        if constexpr (gi < FM / 2)
          read_pair(fra, std::integral_constant<int, LA>{}, std::integral_constant<int, BM>{},
                    fa[NXT][2 * gi], fa[NXT][2 * gi + 1], std::integral_constant<int, gi>{});
        else
          read_pair(frb, std::integral_constant<int, LB>{}, std::integral_constant<int, BN>{},
                    fb[NXT][2 * (gi - FM / 2)], fb[NXT][2 * (gi - FM / 2) + 1],
                    std::integral_constant<int, gi - FM / 2>{});
      }
      // then each remaining load right after an MFMA issue, in its shadow
      static_for<nt>([&](auto t) {
        constexpr int tt = decltype(t)::value;
        load(std::integral_constant<int, j0 + (nl - nt) + tt>{});
        const MfmaSlot m1[4] = {slot(CUR, e0 + n - nt + tt), slot(CUR, 0), slot(CUR, 0),
                                slot(CUR, 0)};
        mfma_only<FA, FB, 1>(m1);
      });
    });
  };

  // The step count is padded to even so the loop body is one unrolled pair
  // with a single register assignment: the padded step's DMA lies past K and
  // lands as exact zeros (+0 products leave every sum unchanged), and the
  // last step's reads of a successor fetch a stale buffer that is never used.
  const int nfull = (int)(g.Kc / kBK3);  // K steps that end at or before K
  const int kfast = max(0, min(nk, nfull - kStages3)) & ~1;
  int kt = 0;
  for (; kt < kfast; kt += 2) {
    kstep_body(kt, std::integral_constant<int, 0>{}, std::true_type{});
    kstep_body(kt + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  for (; kt < nk; kt += 2) {
    kstep_body(kt, std::integral_constant<int, 0>{}, std::false_type{});
    kstep_body(kt + 1, std::integral_constant<int, 1>{}, std::false_type{});
  }

  // Epilogue.  Each lane's accumulators hold 4 consecutive columns per
  // register group, spread over 32 rows; storing them straight to global
  // memory writes 16-byte pieces of many cache lines and ran at a fraction
  // of HBM write bandwidth.  Instead the finished bf16 tile is staged in LDS
  // (rows padded by 16 bytes, so the 32 rows of one store land on distinct
  // banks) and written back as whole rows, 16 bytes per lane.
  // lane holds, for reg e: row wm*WTM + 32a + (lane & 31),
  //   column wn*WTN + 32b + 8(e>>2) + 4(lane>>5) + (e&3) of the block tile
  constexpr int RS = BN * 2 + 16;  // LDS bytes per staged row
  mfma_drain();                    // accumulators are read by VALU below
  side_work<64 * WGM * WGN>(g);    // after the drain: it may reuse fragment registers
  barrier_only();                  // every wave is done reading operand tiles
  const float dq = es.dq(), inv_bs = es.inv_bs();
  if constexpr (EPI != kEpiBF16) {
    fp8_out_epilogue<BM, BN, WTM, WTN, EPI, OF, 64 * WGM * WGN>(g, acc, dq, inv_bs, s_out, sbias,
                                                                smem3, i0, j0, wm, wn);
    return;
  }
#pragma unroll
  for (int b = 0; b < FN; ++b) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int jl = wn * WTN + 32 * b + 8 * grp + 4 * (lane >> 5);
      float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (g.bias_kind != kBiasNone) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bias[t] = BiasStage<BN>::get(g, sbias, j0, jl + t, inv_bs);
      }
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const int il = wm * WTM + 32 * a + (lane & 31);
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = __builtin_fmaf(acc[a][b][4 * grp + t], dq, bias[t]);
        *reinterpret_cast<uint2*>(smem3 + il * RS + jl * 2) =
            make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
      }
    }
  }
  lds_barrier();
  constexpr int kChunksPerRow = BN / 8;  // 16-byte chunks of bf16
  const int64_t rows_left = g.Mc - i0, cols_left = g.Nc - j0;
#pragma unroll 4
  for (int q = tid; q < BM * kChunksPerRow; q += 64 * WGM * WGN) {
    const int r = q / kChunksPerRow, ch = q % kChunksPerRow;
    if (r < rows_left && 8 * ch < cols_left)
      __builtin_nontemporal_store(*reinterpret_cast<const v4u*>(smem3 + r * RS + ch * 16),
                                  reinterpret_cast<v4u*>(g.c + (i0 + r) * g.ldc + j0 + 8 * ch));
  }
}

}  // namespace fp8l
