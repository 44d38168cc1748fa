// Per-tensor FP8 quantize for gfx950: amax over the input values, a
// saturating RNE conversion, and the delayed-scaling ring finalize in the
// launch's last block ([P1] entry on finalizing scale rings inside the
// quantize kernels; [P4] entry on the atomic ticket and fences; [P3] entries
// on the quantize templated on bf16/fp16/fp32 input and on fp32-domain amax).
//
// Work decomposition: every thread converts 16 consecutive elements per
// step (two or four 16-byte loads, one 16-byte store); blocks of 256 threads
// stride over the tensor.  The block's amax is reduced with DPP row shuffles
// and readlane, then one atomic max per block goes to the accumulator.  With
// a ring, an agent-scope atomic ticket elects the last block, which folds
// amax into hist[idx], takes the window max, publishes the next scale and
// resets the accumulator and ticket for the next launch -- no extra launch.
//
// The column-sum variant walks a [rows, cols] tensor by column strips and
// row chunks and also writes fp32 partial column sums (the bias gradient of
// [P4], summed over the values as given).
#pragma once

#include "fp8l_device.hpp"

namespace fp8l {

enum { kScaleRing = 0, kScaleSeed = 1, kScaleDyn = 2 };

constexpr int kQThreads = 256;
constexpr int kQVec = 16;               // elements per thread per step
constexpr int kColStrip = 256;          // columns per block in the column-sum variant
constexpr int kColRowsPerChunk = 32;    // rows per block (one workspace row) in that variant

struct QArgs {
  const void* x;
  uint8_t* q;
  int64_t n;          // flat element count
  int64_t rows, cols; // column-sum variant: x is [rows, cols]
  RingHdr* ring;
  float* hist;
  int32_t hist_len;
  float* scale_used;
  float* amax_out;    // dynamic: complete amax from the amax pass; ring: optional output
  float* colsum;      // [ceil(rows / kColRowsPerChunk)][cols] partial sums or null
  int32_t vec_ok;     // x, q 16-byte aligned (and cols % 16 == 0 for the column variant)
};

template <int IN>
struct InTraits;
template <>
struct InTraits<kInF32> { static constexpr int kBytes = 4; };
template <>
struct InTraits<kInF16> { static constexpr int kBytes = 2; };
template <>
struct InTraits<kInBF16> { static constexpr int kBytes = 2; };

template <int IN>
FP8L_DEV float load1(const void* x, int64_t e) {
  if constexpr (IN == kInF32) {
    return reinterpret_cast<const float*>(x)[e];
  } else if constexpr (IN == kInF16) {
    return (float)reinterpret_cast<const _Float16*>(x)[e];
  } else {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[e]);
  }
}

// 16 elements starting at element e (16-byte aligned, all in range).
template <int IN>
FP8L_DEV void load16(const void* x, int64_t e, float v[16]) {
  if constexpr (IN == kInF32) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 u = p[j];
      v[4 * j + 0] = __uint_as_float(u.x);
      v[4 * j + 1] = __uint_as_float(u.y);
      v[4 * j + 2] = __uint_as_float(u.z);
      v[4 * j + 3] = __uint_as_float(u.w);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + e);
    uint4 u0 = p[0], u1 = p[1];
    uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (IN == kInBF16) {
        v[2 * j + 0] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        h2 h = __builtin_bit_cast(h2, w[j]);
        v[2 * j + 0] = (float)h.x;
        v[2 * j + 1] = (float)h.y;
      }
    }
  }
}

// Max of |v| bits over a thread's elements.
FP8L_DEV uint32_t absbits(float f) { return __float_as_uint(f) & 0x7fffffffu; }

// Quantize 16 values with scale s into four packed words; NaN inputs become
// 0x7F | sign (the med3 clamp would otherwise turn them into +-max).
template <int FMT>
FP8L_DEV void quant16(const float v[16], float s, uint32_t nan_seen, uint32_t w[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = cvt4<FMT>(v[4 * j] * s, v[4 * j + 1] * s, v[4 * j + 2] * s, v[4 * j + 3] * s);
  if (nan_seen) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (absbits(v[i]) > 0x7f800000u) {
        uint32_t code = 0x7fu | ((__float_as_uint(v[i]) >> 24) & 0x80u);
        w[i >> 2] = (w[i >> 2] & ~(0xffu << (8 * (i & 3)))) | (code << (8 * (i & 3)));
      }
    }
  }
}

// Convert the (up to 16) elements [e, e + cnt) one at a time (ragged or
// unaligned chunks).  Returns the max |x| bits.
template <int IN, int FMT>
FP8L_DEV uint32_t quant_scalar(const void* x, uint8_t* q, int64_t e, int cnt, float s, float* vals) {
  float v[16];
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[i] = i < cnt ? load1<IN>(x, e + i) : 0.0f;
    mx = max(mx, absbits(v[i]));
  }
  uint32_t w[4];
  quant16<FMT>(v, s, mx > 0x7f800000u, w);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < cnt) q[e + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    if (vals) vals[i] = v[i];
  }
  return mx;
}

// Block-wide max of non-negative float bits (all 256 threads participate).
FP8L_DEV uint32_t block_max_u32(uint32_t v, uint32_t* sh4) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh4[wave] = v;
  __syncthreads();
  uint32_t r = max(max(sh4[0], sh4[1]), max(sh4[2], sh4[3]));
  __syncthreads();
  return r;
}

// Scale the launch quantizes with.
template <int FMT, int SMODE>
FP8L_DEV float launch_scale(const QArgs& a) {
  constexpr float M = FmtTraits<FMT>::kMax;
  if constexpr (SMODE == kScaleRing) {
    return a.ring->scale;
  } else if constexpr (SMODE == kScaleSeed) {
    float m = __uint_as_float(atomic_load_agent(&a.ring->amax_acc));
    return scale_from_amax(m, M, a.ring->scale);
  } else {
    float m = __uint_as_float(atomic_load_agent(reinterpret_cast<const uint32_t*>(a.amax_out)));
    return scale_from_amax(m, M, 1.0f);
  }
}

// Ring epilogue: elect the last block; it folds amax into the window and
// publishes the next scale.  s is the scale this launch used (the snapshot
// written to scale_used).
template <int FMT, int SMODE>
FP8L_DEV void ring_epilogue(const QArgs& a, uint32_t block_mx, float s, uint32_t* sh4) {
  __shared__ int sh_last;
  const int tid = threadIdx.x;
  if (tid == 0) {
    if (SMODE == kScaleRing && block_mx != 0)
      __hip_atomic_fetch_max(&a.ring->amax_acc, block_mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t total = gridDim.x * gridDim.y;
    uint32_t t = __hip_atomic_fetch_add(&a.ring->counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = (t == total - 1);
  }
  __syncthreads();
  if (!sh_last) return;
  const uint32_t amax_bits = atomic_load_agent(&a.ring->amax_acc);
  const int H = a.hist_len;
  const uint32_t idx = a.ring->idx % (uint32_t)H;  // in range even for a corrupted header
  uint32_t m = 0;
  for (int j = tid; j < H; j += kQThreads)
    m = max(m, (uint32_t)j == idx ? amax_bits : __float_as_uint(a.hist[j]));
  m = block_max_u32(m, sh4);
  if (tid == 0) {
    a.hist[idx] = __uint_as_float(amax_bits);
    a.ring->idx = (idx + 1 == (uint32_t)H) ? 0u : idx + 1;
    a.ring->scale = scale_from_amax(__uint_as_float(m), FmtTraits<FMT>::kMax, s);
    a.ring->seeded = 1u;
    a.ring->amax_acc = 0u;
    a.ring->counter = 0u;
    *a.scale_used = s;
    if (a.amax_out) *a.amax_out = __uint_as_float(amax_bits);
  }
}

// Flat quantize: SMODE chooses where the scale comes from (ring slot, seed
// from the completed amax pass, or dynamic).
template <int IN, int FMT, int SMODE>
__global__ __launch_bounds__(kQThreads) void quantize_flat_kernel(QArgs a) {
  __shared__ uint32_t sh4[4];
  const float s = launch_scale<FMT, SMODE>(a);
  const int64_t nch = (a.n + kQVec - 1) / kQVec;
  const int64_t stride = (int64_t)gridDim.x * kQThreads;
  uint32_t mx = 0;
  for (int64_t c = (int64_t)blockIdx.x * kQThreads + threadIdx.x; c < nch; c += stride) {
    const int64_t e = c * kQVec;
    if (a.vec_ok && e + kQVec <= a.n) {
      float v[16];
      load16<IN>(a.x, e, v);
      uint32_t lm = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) lm = max(lm, absbits(v[i]));
      uint32_t w[4];
      quant16<FMT>(v, s, lm > 0x7f800000u, w);
      *reinterpret_cast<uint4*>(a.q + e) = make_uint4(w[0], w[1], w[2], w[3]);
      mx = max(mx, lm);
    } else {
      const int cnt = (int)min<int64_t>(kQVec, a.n - e);
      mx = max(mx, quant_scalar<IN, FMT>(a.x, a.q, e, cnt, s, nullptr));
    }
  }
  if constexpr (SMODE == kScaleDyn) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.scale_used = s;
  } else {
    const uint32_t bm = block_max_u32(mx, sh4);
    ring_epilogue<FMT, SMODE>(a, bm, s, sh4);
  }
}

// Column-sum quantize over x [rows, cols]: block (bx, by) covers columns
// [bx*256, +256) and rows [by*32, +32); 16 threads across (16 columns
// each) by 16 threads down.  Writes colsum[by][col] = sum of its rows.
template <int IN, int FMT, int SMODE>
__global__ __launch_bounds__(kQThreads) void quantize_colsum_kernel(QArgs a) {
  __shared__ uint32_t sh4[4];
  __shared__ float shsum[16][kColStrip + 1];
  const float s = launch_scale<FMT, SMODE>(a);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kColStrip + tx * kQVec;
  const int64_t r0 = (int64_t)blockIdx.y * kColRowsPerChunk;
  const int64_t r1 = min<int64_t>(r0 + kColRowsPerChunk, a.rows);
  float cs[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) cs[i] = 0.0f;
  uint32_t mx = 0;
  if (c0 < a.cols) {
    const int cnt = (int)min<int64_t>(kQVec, a.cols - c0);
    for (int64_t r = r0 + ty; r < r1; r += 16) {
      const int64_t e = r * a.cols + c0;
      float v[16];
      if (a.vec_ok && cnt == kQVec) {
        load16<IN>(a.x, e, v);
        uint32_t lm = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) lm = max(lm, absbits(v[i]));
        uint32_t w[4];
        quant16<FMT>(v, s, lm > 0x7f800000u, w);
        *reinterpret_cast<uint4*>(a.q + e) = make_uint4(w[0], w[1], w[2], w[3]);
        mx = max(mx, lm);
      } else {
        mx = max(mx, quant_scalar<IN, FMT>(a.x, a.q, e, cnt, s, v));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) cs[i] += v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) shsum[ty][tx * 16 + i] = cs[i];
  __syncthreads();
  {
    const int col = threadIdx.x;  // 0..255
    const int64_t gc = (int64_t)blockIdx.x * kColStrip + col;
    float t = 0.0f;
#pragma unroll
    for (int y = 0; y < 16; ++y) t += shsum[y][col];
    if (gc < a.cols) a.colsum[(int64_t)blockIdx.y * a.cols + gc] = t;
  }
  if constexpr (SMODE == kScaleDyn) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.scale_used = s;
  } else {
    const uint32_t bm = block_max_u32(mx, sh4);
    ring_epilogue<FMT, SMODE>(a, bm, s, sh4);
  }
}

// amax pass (seed and dynamic paths): atomic max of |x| bits into target,
// which must hold 0 (or a smaller value) on entry.
template <int IN>
__global__ __launch_bounds__(kQThreads) void amax_kernel(const void* x, int64_t n, int vec_ok,
                                                        uint32_t* target) {
  __shared__ uint32_t sh4[4];
  const int64_t nch = (n + kQVec - 1) / kQVec;
  const int64_t stride = (int64_t)gridDim.x * kQThreads;
  uint32_t mx = 0;
  for (int64_t c = (int64_t)blockIdx.x * kQThreads + threadIdx.x; c < nch; c += stride) {
    const int64_t e = c * kQVec;
    if (vec_ok && e + kQVec <= n) {
      float v[16];
      load16<IN>(x, e, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = max(mx, absbits(v[i]));
    } else {
      const int cnt = (int)min<int64_t>(kQVec, n - e);
      for (int i = 0; i < cnt; ++i) mx = max(mx, absbits(load1<IN>(x, e + i)));
    }
  }
  const uint32_t bm = block_max_u32(mx, sh4);
  if (threadIdx.x == 0 && bm != 0)
    __hip_atomic_fetch_max(target, bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Column sums of pre-quantized codes g8 [rows, cols] (decoded values; the
// caller's epilogue multiplies by 1/sg): same decomposition as the
// column-sum quantize.
template <int FMT>
__global__ __launch_bounds__(kQThreads) void colsum_fp8_kernel(const uint8_t* g8, int64_t rows,
                                                              int64_t cols, float* colsum) {
  __shared__ float shsum[16][kColStrip + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * kColStrip + tx * kQVec;
  const int64_t r0 = (int64_t)blockIdx.y * kColRowsPerChunk;
  const int64_t r1 = min<int64_t>(r0 + kColRowsPerChunk, rows);
  float cs[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) cs[i] = 0.0f;
  if (c0 < cols) {
    const int cnt = (int)min<int64_t>(kQVec, cols - c0);
    for (int64_t r = r0 + ty; r < r1; r += 16) {
      const uint8_t* p = g8 + r * cols + c0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < cnt) cs[i] += fp8_to_f32<FMT>(p[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) shsum[ty][tx * 16 + i] = cs[i];
  __syncthreads();
  const int col = threadIdx.x;
  const int64_t gc = (int64_t)blockIdx.x * kColStrip + col;
  float t = 0.0f;
#pragma unroll
  for (int y = 0; y < 16; ++y) t += shsum[y][col];
  if (gc < cols) colsum[(int64_t)blockIdx.y * cols + gc] = t;
}

// Ring reset (one block).
__global__ void ring_init_kernel(RingHdr* h, float* hist, int H) {
  for (int j = threadIdx.x; j < H; j += blockDim.x) hist[j] = 0.0f;
  if (threadIdx.x == 0) {
    h->scale = 1.0f;
    h->amax_acc = 0u;
    h->counter = 0u;
    h->idx = 0u;
    h->hist_len = (uint32_t)H;
    h->seeded = 0u;
    for (int i = 0; i < 10; ++i) h->reserved[i] = 0u;
  }
}

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

}  // namespace fp8l
