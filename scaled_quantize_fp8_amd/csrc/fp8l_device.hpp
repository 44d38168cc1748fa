// Device helpers shared by the quantize and GEMM kernels (gfx950 / CDNA4).
//
// Sources cited in this library (AstrAI commit-log pages):
//   [P1] commit 2eeac02d, page tests/extension
//   [P2] commit 2eeac02d, page csrc
//   [P3] commit 057c0d33, page astrai/extension/ops
//   [P4] commit 4019ddac, page astrai
//   [OCP] OCP 8-bit Floating Point Specification (OFP8) rev 1.0
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8l {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define FP8L_DEV __device__ __forceinline__

enum { kE4M3 = 0, kE5M2 = 1 };
enum { kInF32 = 0, kInF16 = 1, kInBF16 = 2 };

// Largest finite magnitude of each OCP format [OCP]: E4M3 S.1111.110 = 448,
// E5M2 S.11110.11 = 57344.
template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<kE4M3> {
  static constexpr float kMax = 448.0f;
};
template <>
struct FmtTraits<kE5M2> {
  static constexpr float kMax = 57344.0f;
};

// Ring buffer in device memory: a 128-byte header, 64 election groups of
// 128 bytes (each on its own cache line so the blocks of different groups
// never contend for one address), then float hist[H].
constexpr int kGroups = 64;
struct RingGroup {
  uint32_t count;      // blocks of this group that finished (0 between launches)
  uint32_t pad0[15];
  uint32_t amax;       // max |x| bits over those blocks (0 between launches)
  uint32_t pad1[15];
};
struct RingHdr {
  float scale;         // scale the next quantize uses
  uint32_t top_count;  // groups that finished (0 between launches)
  uint32_t top_amax;   // max |x| bits over finished groups (0 between launches,
                       // except between the two passes of a seeding quantize)
  uint32_t idx;        // next hist slot
  uint32_t hist_len;
  uint32_t seeded;
  uint32_t reserved[26];
  RingGroup group[kGroups];
};
static_assert(sizeof(RingGroup) == 128, "one election group per 128-byte line");
static_assert(sizeof(RingHdr) == 128 + 64 * 128, "ring header layout");

// ---------------------------------------------------------------- scale

// S(m) = fmt_max / m, IEEE fp32 division (correctly rounded: the library is
// built without fast-math), or prev when m is 0, NaN, inf or the quotient
// overflows.  The plainest reading of "scale = fmt_max / amax" with a zero
// margin.
FP8L_DEV float scale_from_amax(float m, float fmt_max, float prev) {
  if (m > 0.0f && m <= 3.402823466e38f) {
    float r = fmt_max / m;
    if (r <= 3.402823466e38f) return r;
  }
  return prev;
}

// ---------------------------------------------------------------- conversion

// Four fp32 values -> four codes (byte i = value i).  The hardware
// conversion rounds to nearest even with OCP encodings; it turns overflow
// into NaN / inf, so values are first clamped to +-max with v_med3_f32
// (saturation; inf clamps too).  NaN inputs are fixed up by the caller.
template <int FMT>
FP8L_DEV uint32_t cvt4(float a, float b, float c, float d) {
  constexpr float M = FmtTraits<FMT>::kMax;
  a = __builtin_amdgcn_fmed3f(a, -M, M);
  b = __builtin_amdgcn_fmed3f(b, -M, M);
  c = __builtin_amdgcn_fmed3f(c, -M, M);
  d = __builtin_amdgcn_fmed3f(d, -M, M);
  int w;
  if constexpr (FMT == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// Byte SEL of a packed word, decoded to fp32 (exact).
template <int FMT, int SEL = 0>
FP8L_DEV float fp8_to_f32(uint32_t word) {
  if constexpr (FMT == kE4M3)
    return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
  else
    return __builtin_amdgcn_cvt_f32_bf8((int)word, SEL);
}

FP8L_DEV float fp8_to_f32_rt(uint32_t code, int fmt) {
  return fmt == kE4M3 ? __builtin_amdgcn_cvt_f32_fp8((int)code, 0)
                      : __builtin_amdgcn_cvt_f32_bf8((int)code, 0);
}

FP8L_DEV float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
FP8L_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bf16 (a in the low half) with one v_cvt_pk_bf16_f32.
// On gfx950, in the kernels' default FP mode, this instruction gives the
// same bits as f32_to_bf16 above for every one of the 2^32 float inputs
// (round to nearest even, NaN kept quiet, subnormals kept); checked
// exhaustively on the device.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
FP8L_DEV uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ---------------------------------------------------------------- reductions

// Max of non-negative float bit patterns across a wave of 64 lanes: DPP row
// shuffles within each row of 16 lanes, then readlane across the 4 rows.
// Unsigned order of non-negative floats is their numeric order (NaN above
// inf), so the max propagates NaN.
FP8L_DEV uint32_t wave_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2] and [2,3,0,1]: xor 1, xor 2 inside each quad
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  // row_ror:4 and row_ror:8 combine the four quads of a row
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false));
  uint32_t r0 = __builtin_amdgcn_readlane(v, 0);
  uint32_t r1 = __builtin_amdgcn_readlane(v, 16);
  uint32_t r2 = __builtin_amdgcn_readlane(v, 32);
  uint32_t r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Device-scope atomics are all relaxed read-modify-writes: they are
// performed at the device's point of coherence, so no L2 write-back or
// invalidate (what an agent-scope release/acquire costs on a multi-XCD
// part) is ever needed; ordering between two of them in one thread is
// enforced by waiting for the first to return.
FP8L_DEV uint32_t atom_max(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
FP8L_DEV uint32_t atom_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
FP8L_DEV uint32_t atom_xchg(uint32_t* p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
FP8L_DEV uint32_t atom_read(uint32_t* p) {
  return __hip_atomic_fetch_max(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
FP8L_DEV void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace fp8l
