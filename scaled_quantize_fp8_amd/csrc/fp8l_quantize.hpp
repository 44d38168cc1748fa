// Per-tensor FP8 quantize for gfx950: amax over the input values, a
// saturating RNE conversion, and the delayed-scaling ring finalize ([P1]
// entry on finalizing scale rings inside the quantize kernels; [P4] entry on
// the atomic ticket; [P3] entries on the quantize templated on bf16/fp16/fp32
// input and on fp32-domain amax).  The finalize runs in the launch's last
// block (Ring, Seed below), or one wave of a later launch folds the maxima
// the blocks left in the ring's election groups (Defer: the GEMM that
// consumes the codes, or a one-wave launch after a standalone quantize).
//
// Memory access: a wave converts 1024 consecutive elements per step; each of
// its load instructions covers 1 KB of contiguous input (16 bytes per lane)
// and each store a contiguous run of codes.  Blocks of 4 waves stride over
// the tensor.
//
// Last-block election without contention: a single counter hit by thousands
// of blocks serializes at roughly 11 ns per device atomic on MI355X, and an
// agent-scope acquire/release around it writes back and invalidates the L2.
// Instead the blocks are split into 64 groups, each with its own cache line
// holding a counter and a running max.  A block folds its max into its group
// and takes a group ticket; the group's last block takes a header ticket;
// the last header ticket is the launch's last block, which collects the 64
// group maxima in one parallel round of atomics, folds amax into hist[idx],
// takes the window max, publishes the next scale and leaves every counter
// and max at zero.  The launch's last block waits on four dependent device
// atomics after its data (max, group ticket, header ticket, collection).
//
// The column-sum variant walks G [rows, cols] by column strips and row
// chunks and also writes fp32 partial column sums (the bias gradient of
// [P4], summed over the values as given).
#pragma once

#include "fp8l_device.hpp"
#include "fp8linear.h"

namespace fp8l {

// Scale modes of a converting launch: the ring's scale with the ring fold
// in the last block (Ring); the seed from the amax pass, then the fold
// (Seed); dynamic, from the amax pass (Dyn); the ring's scale with the fold
// left to a later launch on the stream (Defer: each block only folds its max
// into its election group; see finish_launch and RingFold).
enum { kScaleRing = 0, kScaleSeed = 1, kScaleDyn = 2, kScaleDefer = 3 };

constexpr int kQThreads = 256;
constexpr int kWaveChunk = 1024;            // elements per wave per step (flat kernel)
constexpr int kBlockChunk = 4 * kWaveChunk;
constexpr int kColStrip = 256;              // columns per block (column-sum kernel)
constexpr int kColRowsPerChunk = 32;        // rows per block = one workspace row

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
  int32_t vec_ok;     // x, q 16-byte aligned (and cols % 8 == 0 for the column variant)
  uint8_t* qt;        // transposed variant: [cols, rows] codes or null (q may be null)
  int32_t qt_vec;     // qt 16-byte aligned and rows % 16 == 0
};

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

// 8 consecutive elements starting at element e (16-byte aligned for 2-byte
// types, 32-byte for fp32).
template <int IN>
FP8L_DEV void load8(const void* x, int64_t e, float v[8]) {
  if constexpr (IN == kInF32) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + e);
    const uint4 a = p[0], b = p[1];
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + e);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (IN == kInBF16) {
        v[2 * j + 0] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 h = __builtin_bit_cast(h2, w[j]);
        v[2 * j + 0] = (float)h.x;
        v[2 * j + 1] = (float)h.y;
      }
    }
  }
}

FP8L_DEV uint32_t absbits(float f) { return __float_as_uint(f) & 0x7fffffffu; }

// Quantize 8 values with scale s into two packed words; NaN inputs become
// 0x7F | sign (the med3 clamp would otherwise turn them into +-max).
template <int FMT>
FP8L_DEV uint2 quant8(const float v[8], float s, uint32_t lane_max) {
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    w[j] = cvt4<FMT>(v[4 * j] * s, v[4 * j + 1] * s, v[4 * j + 2] * s, v[4 * j + 3] * s);
  if (lane_max > 0x7f800000u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (absbits(v[i]) > 0x7f800000u) {
        const uint32_t code = 0x7fu | ((__float_as_uint(v[i]) >> 24) & 0x80u);
        w[i >> 2] = (w[i >> 2] & ~(0xffu << (8 * (i & 3)))) | (code << (8 * (i & 3)));
      }
    }
  }
  return make_uint2(w[0], w[1]);
}

// Quantize 4 values with scale s into one packed word, NaN as in quant8.
template <int FMT>
FP8L_DEV uint32_t quant4(const float v[4], float s) {
  uint32_t w = cvt4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (absbits(v[i]) > 0x7f800000u) {
      const uint32_t code = 0x7fu | ((__float_as_uint(v[i]) >> 24) & 0x80u);
      w = (w & ~(0xffu << (8 * i))) | (code << (8 * i));
    }
  }
  return w;
}

// quant4 when m4, the max of the four |v| bits, is known: the NaN repair
// runs only when one of them is a NaN.
template <int FMT>
FP8L_DEV uint32_t quant4_m(const float v[4], float s, uint32_t m4) {
  if (m4 > 0x7f800000u) return quant4<FMT>(v, s);
  return cvt4<FMT>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
}

// Elements [e, e + cnt), cnt <= 8, one at a time (ragged or unaligned).
// vals receives the values (0 past cnt).  Returns the max |x| bits.
template <int IN, int FMT>
FP8L_DEV uint32_t quant_scalar8(const void* x, uint8_t* q, int64_t e, int cnt, float s,
                                float vals[8]) {
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    vals[i] = i < cnt ? load1<IN>(x, e + i) : 0.0f;
    mx = max(mx, absbits(vals[i]));
  }
  const uint2 w = quant8<FMT>(vals, s, mx);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < cnt) q[e + i] = (uint8_t)((i < 4 ? w.x : w.y) >> (8 * (i & 3)));
  return mx;
}

// Block-wide max of non-negative float bits (all NT threads participate;
// sh holds one word per wave).
template <int NT = kQThreads>
FP8L_DEV uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
  static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = sh[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) r = max(r, sh[w]);
  __syncthreads();
  return r;
}

// Two-level last-block election.  Group level (thread 0): fold bm (this
// block's max |x| bits) into the block's group max, then take a group
// ticket; true in the group's last block, which resets the group counter.
// The group max stays in place for the launch's last block to collect.
FP8L_DEV bool elect_group(RingHdr* h, uint32_t bid, uint32_t total, uint32_t bm) {
  const uint32_t G = total < (uint32_t)kGroups ? total : (uint32_t)kGroups;
  const uint32_t g = bid % G;
  const uint32_t gsize = (total - g + G - 1) / G;
  RingGroup* grp = &h->group[g];
  if (bm) atom_max(&grp->amax, bm);
  wait_vmem();  // the max is performed before the ticket is taken
  if (atom_add(&grp->count, 1u) != gsize - 1) return false;
  atom_xchg(&grp->count, 0u);
  return true;
}

// Top level (thread 0 of a group's last block): true in the launch's last
// block, which resets the top counter.
FP8L_DEV bool elect_top(RingHdr* h, uint32_t total) {
  const uint32_t G = total < (uint32_t)kGroups ? total : (uint32_t)kGroups;
  if (atom_add(&h->top_count, 1u) != G - 1) return false;
  atom_xchg(&h->top_count, 0u);
  return true;
}

// The launch max, in the launch's last block (every thread calls it): one
// lane per group takes its max and leaves 0 behind, all in one round trip.
// Every group's max was performed before its last block's group ticket,
// and that ticket before the top ticket that made this block the last.
// consume: also take (and clear) the header max that the amax pass of a
// seeding quantize leaves for the converting launch.
template <int NT = kQThreads>
FP8L_DEV uint32_t gather_amax(RingHdr* h, uint32_t total, bool consume, uint32_t* sh) {
  const uint32_t G = total < (uint32_t)kGroups ? total : (uint32_t)kGroups;
  static_assert(kGroups < NT, "one lane per group plus one");
  uint32_t m = 0;
  if (threadIdx.x < G) m = atom_xchg(&h->group[threadIdx.x].amax, 0u);
  else if (consume && threadIdx.x == G) m = atom_xchg(&h->top_amax, 0u);
  return block_max_u32<NT>(m, sh);
}

// End of an amax pass (the first pass of a seeding quantize, or of a
// seeding FP8-output GEMM): the launch's last block leaves max |x| in the
// ring header's top_amax, the counters back at zero, for the converting
// launch that follows.  mx: this thread's max |x| bits; NT: threads per
// block.
template <int NT = kQThreads>
FP8L_DEV void amax_pass_finish(RingHdr* h, uint32_t mx, uint32_t bid, uint32_t total) {
  __shared__ uint32_t sh[NT / 64];
  __shared__ uint32_t sh_flag;
  const uint32_t bm = block_max_u32<NT>(mx, sh);
  if (threadIdx.x == 0)
    sh_flag = (elect_group(h, bid, total, bm) && elect_top(h, total)) ? 1u : 0u;
  __syncthreads();
  if (!sh_flag) return;
  const uint32_t amax_bits = gather_amax<NT>(h, total, false, sh);
  if (threadIdx.x == 0) atom_xchg(&h->top_amax, amax_bits);
}

// Scale the launch quantizes with.
template <int FMT, int SMODE>
FP8L_DEV float launch_scale(const QArgs& a) {
  constexpr float M = FmtTraits<FMT>::kMax;
  if constexpr (SMODE == kScaleRing || SMODE == kScaleDefer) {
    return a.ring->scale;
  } else if constexpr (SMODE == kScaleSeed) {
    // amax left in the header by the amax pass that ran just before
    const float m = __uint_as_float(__hip_atomic_load(&a.ring->top_amax, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
    return scale_from_amax(m, M, a.ring->scale);
  } else {
    const float m = __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(a.amax_out),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return scale_from_amax(m, M, 1.0f);
  }
}

// End of a converting launch: dynamic -> block 0 writes scale_used; ring ->
// elect the last block, which folds amax into the window and publishes the
// next scale.  s is the scale this launch used (the snapshot in scale_used).
// NT: threads per block.
template <int FMT, int SMODE, int NT = kQThreads>
FP8L_DEV void finish_launch(const QArgs& a, uint32_t mx, float s, uint32_t bid, uint32_t total) {
  __shared__ uint32_t sh4[NT / 64];
  __shared__ uint32_t sh_flag;
  if constexpr (SMODE == kScaleDyn) {
    if (bid == 0 && threadIdx.x == 0) *a.scale_used = s;
    return;
  } else if constexpr (SMODE == kScaleDefer) {
    // No election: the block's max goes into its group (no return value
    // is awaited, so nothing here waits on a device round trip), and the
    // launch that consumes the codes folds the groups into the ring when
    // it starts (RingFold).  Block 0 writes the scale snapshot.
    const uint32_t bm = block_max_u32<NT>(mx, sh4);
    if (threadIdx.x == 0) {
      if (bid == 0) *a.scale_used = s;
      const uint32_t G = total < (uint32_t)kGroups ? total : (uint32_t)kGroups;
      if (bm) atom_max(&a.ring->group[bid % G].amax, bm);
    }
    return;
  } else {
    const uint32_t bm = block_max_u32<NT>(mx, sh4);
    if (threadIdx.x == 0) sh_flag = elect_group(a.ring, bid, total, bm) ? 1u : 0u;
    __syncthreads();
    if (!sh_flag) return;
    // A group winner may be the launch's last block: load the window and its
    // index now, in parallel with the top-level election.  Only the last
    // block writes them, and only after it has won, so what a winner reads
    // here is the state the previous launch left.
    const int H = a.hist_len;
    uint32_t hv[FP8_RING_MAX_HIST / NT];
#pragma unroll
    for (int k = 0; k < FP8_RING_MAX_HIST / NT; ++k) {
      const int j = threadIdx.x + k * NT;
      hv[k] = j < H ? __float_as_uint(a.hist[j]) : 0u;
    }
    const uint32_t idx = a.ring->idx % (uint32_t)H;  // in range even for a corrupted header
    __syncthreads();  // every thread has read sh_flag before it is reused
    if (threadIdx.x == 0) sh_flag = elect_top(a.ring, total) ? 1u : 0u;
    __syncthreads();
    if (!sh_flag) return;
    const uint32_t amax_bits = gather_amax<NT>(a.ring, total, true, sh4);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < FP8_RING_MAX_HIST / NT; ++k) {
      const int j = threadIdx.x + k * NT;
      if (j < H) m = max(m, (uint32_t)j == idx ? amax_bits : hv[k]);
    }
    m = block_max_u32<NT>(m, sh4);
    if (threadIdx.x == 0) {
      a.hist[idx] = __uint_as_float(amax_bits);
      a.ring->idx = (idx + 1 == (uint32_t)H) ? 0u : idx + 1;
      a.ring->scale = scale_from_amax(__uint_as_float(m), FmtTraits<FMT>::kMax, s);
      a.ring->seeded = 1u;
      *a.scale_used = s;
      if (a.amax_out) *a.amax_out = __uint_as_float(amax_bits);
    }
  }
}

// Flat quantize.  Lane l of a wave handles elements [c + 8l, +8) and
// [c + 512 + 8l, +8) of each 1024-element wave chunk c.  bid / nblk: this
// block's index among the nblk blocks working on the tensor.
template <int IN, int FMT, int SMODE>
FP8L_DEV void quantize_flat_body(const QArgs& a, uint32_t bid, uint32_t nblk) {
  const float s = launch_scale<FMT, SMODE>(a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mx = 0;
  for (int64_t base = (int64_t)bid * kBlockChunk + wave * kWaveChunk; base < a.n;
       base += (int64_t)nblk * kBlockChunk) {
    const int64_t e0 = base + 8 * lane, e1 = base + 512 + 8 * lane;
    if (a.vec_ok && base + kWaveChunk <= a.n) {
      float v0[8], v1[8];
      load8<IN>(a.x, e0, v0);
      load8<IN>(a.x, e1, v1);
      uint32_t m0 = 0, m1 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        m0 = max(m0, absbits(v0[i]));
        m1 = max(m1, absbits(v1[i]));
      }
      *reinterpret_cast<uint2*>(a.q + e0) = quant8<FMT>(v0, s, m0);
      *reinterpret_cast<uint2*>(a.q + e1) = quant8<FMT>(v1, s, m1);
      mx = max(mx, max(m0, m1));
    } else {
      float v[8];
      if (e0 < a.n)
        mx = max(mx, quant_scalar8<IN, FMT>(a.x, a.q, e0, (int)min<int64_t>(8, a.n - e0), s, v));
      if (e1 < a.n)
        mx = max(mx, quant_scalar8<IN, FMT>(a.x, a.q, e1, (int)min<int64_t>(8, a.n - e1), s, v));
    }
  }
  finish_launch<FMT, SMODE>(a, mx, s, bid, nblk);
}

template <int IN, int FMT, int SMODE>
__global__ __launch_bounds__(kQThreads) void quantize_flat_kernel(QArgs a) {
  quantize_flat_body<IN, FMT, SMODE>(a, blockIdx.x, gridDim.x);
}

// Two tensors of one input type and format, each with its own seeded ring,
// in one launch: blocks [0, nblk0) quantize a0, the rest a1.  The forward of
// a linear layer quantizes X and W this way, so that one tensor's fixed
// latency (first loads, the election chain) overlaps the other's.
template <int IN, int FMT, int SMODE>
__global__ __launch_bounds__(kQThreads) void quantize_flat2_kernel(QArgs a0, QArgs a1,
                                                                   uint32_t nblk0) {
  if (blockIdx.x < nblk0)
    quantize_flat_body<IN, FMT, SMODE>(a0, blockIdx.x, nblk0);
  else
    quantize_flat_body<IN, FMT, SMODE>(a1, blockIdx.x - nblk0, gridDim.x - nblk0);
}

// Quantize x [rows, cols] into q [rows, cols] and/or its transpose
// qt [cols, rows] ([P4] entry on the transposed and dual quantize layouts):
// qt[c][r] = q[r][c], same codes, same amax and ring finalize as the flat
// kernel.  Tiles of 64 x 64: each thread converts 16 consecutive elements of
// one row (stored to q directly), the tile's codes pass through LDS, and each
// thread then writes 16 consecutive codes of one qt row.
constexpr int kTT = 64;

template <int IN, int FMT, int SMODE>
__global__ __launch_bounds__(kQThreads) void quantize_t_kernel(QArgs a) {
  __shared__ uint8_t tile[kTT][kTT + 4];  // rows 68 bytes apart
  const float s = launch_scale<FMT, SMODE>(a);
  const int t = threadIdx.x;
  const int lr = t >> 2, lc = (t & 3) * 16;  // load: row lr, columns lc .. lc + 15
  const int tc = t >> 2, tr = (t & 3) * 16;  // store: qt row tc, rows tr .. tr + 15
  const int64_t tiles_c = (a.cols + kTT - 1) / kTT;
  const int64_t ntiles = ((a.rows + kTT - 1) / kTT) * tiles_c;
  uint32_t mx = 0;
  for (int64_t ti = blockIdx.x; ti < ntiles; ti += gridDim.x) {
    const int64_t r0 = (ti / tiles_c) * kTT, c0 = (ti % tiles_c) * kTT;
    const int64_t r = r0 + lr, c = c0 + lc;
    float v[16];
    uint32_t m0 = 0, m1 = 0;
    const bool full = a.vec_ok && r < a.rows && c + 16 <= a.cols;
    if (full) {
      load8<IN>(a.x, r * a.cols + c, v);
      load8<IN>(a.x, r * a.cols + c + 8, v + 8);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = (r < a.rows && c + i < a.cols) ? load1<IN>(a.x, r * a.cols + c + i) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m0 = max(m0, absbits(v[i]));
      m1 = max(m1, absbits(v[8 + i]));
    }
    const uint2 w0 = quant8<FMT>(v, s, m0), w1 = quant8<FMT>(v + 8, s, m1);
    mx = max(mx, max(m0, m1));
    const uint32_t w[4] = {w0.x, w0.y, w1.x, w1.y};
    if (a.q) {
      if (full) {
        *reinterpret_cast<uint2*>(a.q + r * a.cols + c) = w0;
        *reinterpret_cast<uint2*>(a.q + r * a.cols + c + 8) = w1;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (r < a.rows && c + i < a.cols)
            a.q[r * a.cols + c + i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(&tile[lr][lc + 4 * j]) = w[j];
    __syncthreads();
    if (a.qt && c0 + tc < a.cols) {
      uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i >> 2] |= (uint32_t)tile[tr + i][tc] << (8 * (i & 3));
      uint8_t* dst = a.qt + (c0 + tc) * a.rows + r0 + tr;
      if (a.qt_vec && r0 + tr + 16 <= a.rows) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (r0 + tr + i < a.rows) dst[i] = (uint8_t)(o[i >> 2] >> (8 * (i & 3)));
      }
    }
    __syncthreads();  // the next tile reuses the LDS tile
  }
  finish_launch<FMT, SMODE>(a, mx, s, blockIdx.x, gridDim.x);
}

// Column-sum quantize over x [rows, cols]: block (bx, by) covers columns
// [bx*256, +256) and rows [by*32, +32).  32 threads across (8 columns each,
// one 16-byte load of bf16) by 8 threads down; each thread walks 4 rows.
// Writes colsum[by][col] = sum over the block's rows (fixed order).
template <int IN, int FMT, int SMODE>
__global__ __launch_bounds__(kQThreads) void quantize_colsum_kernel(QArgs a) {
  __shared__ float shsum[8][kColStrip + 1];
  const float s = launch_scale<FMT, SMODE>(a);
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * kColStrip + tx * 8;
  const int64_t r0 = (int64_t)blockIdx.y * kColRowsPerChunk;
  const int64_t r1 = min<int64_t>(r0 + kColRowsPerChunk, a.rows);
  float cs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cs[i] = 0.0f;
  uint32_t mx = 0;
  if (c0 < a.cols) {
    const int cnt = (int)min<int64_t>(8, a.cols - c0);
    if (a.vec_ok && cnt == 8 && r0 + kColRowsPerChunk <= a.rows) {
      float v[4][8];
#pragma unroll
      for (int k = 0; k < 4; ++k) load8<IN>(a.x, (r0 + ty + 8 * k) * a.cols + c0, v[k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t lm = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          lm = max(lm, absbits(v[k][i]));
          cs[i] += v[k][i];
        }
        *reinterpret_cast<uint2*>(a.q + (r0 + ty + 8 * k) * a.cols + c0) = quant8<FMT>(v[k], s, lm);
        mx = max(mx, lm);
      }
    } else {
      for (int64_t r = r0 + ty; r < r1; r += 8) {
        float v[8];
        mx = max(mx, quant_scalar8<IN, FMT>(a.x, a.q, r * a.cols + c0, cnt, s, v));
#pragma unroll
        for (int i = 0; i < 8; ++i) cs[i] += v[i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) shsum[ty][tx * 8 + i] = cs[i];
  __syncthreads();
  {
    const int col = threadIdx.x;  // 0..255
    const int64_t gc = (int64_t)blockIdx.x * kColStrip + col;
    float t = 0.0f;
#pragma unroll
    for (int y = 0; y < 8; ++y) t += shsum[y][col];
    if (gc < a.cols) a.colsum[(int64_t)blockIdx.y * a.cols + gc] = t;
  }
  finish_launch<FMT, SMODE>(a, mx, s, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
}

// Max |x| bits of this thread's share of a flat tensor (amax passes).
template <int IN>
FP8L_DEV uint32_t flat_absmax(const void* x, int64_t n, int vec_ok) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t mx = 0;
  for (int64_t base = (int64_t)blockIdx.x * kBlockChunk + wave * kWaveChunk; base < n;
       base += (int64_t)gridDim.x * kBlockChunk) {
    const int64_t e0 = base + 8 * lane, e1 = base + 512 + 8 * lane;
    if (vec_ok && base + kWaveChunk <= n) {
      float v0[8], v1[8];
      load8<IN>(x, e0, v0);
      load8<IN>(x, e1, v1);
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = max(mx, max(absbits(v0[i]), absbits(v1[i])));
    } else {
      for (int i = 0; i < 8; ++i) {
        if (e0 + i < n) mx = max(mx, absbits(load1<IN>(x, e0 + i)));
        if (e1 + i < n) mx = max(mx, absbits(load1<IN>(x, e1 + i)));
      }
    }
  }
  return mx;
}

// amax pass of a seeding quantize: leaves max |x| in the ring header's
// top_amax (counters back at zero) for the converting launch that follows.
template <int IN>
__global__ __launch_bounds__(kQThreads) void amax_ring_kernel(const void* x, int64_t n, int vec_ok,
                                                             RingHdr* h) {
  amax_pass_finish(h, flat_absmax<IN>(x, n, vec_ok), blockIdx.x, gridDim.x);
}

// amax pass of a dynamic quantize: one device atomic max per block into
// target (zeroed by the preceding launch).  The launcher keeps this grid at
// one block per CU, so the atomics stay few.
template <int IN>
__global__ __launch_bounds__(kQThreads) void amax_dyn_kernel(const void* x, int64_t n, int vec_ok,
                                                            uint32_t* target) {
  __shared__ uint32_t sh4[4];
  const uint32_t bm = block_max_u32(flat_absmax<IN>(x, n, vec_ok), sh4);
  if (threadIdx.x == 0 && bm != 0) atom_max(target, bm);
}

// Column sums of pre-quantized codes g8 [rows, cols] (decoded values; the
// GEMM epilogue multiplies by 1/sg): same decomposition as the column-sum
// quantize.
template <int FMT>
__global__ __launch_bounds__(kQThreads) void colsum_fp8_kernel(const uint8_t* g8, int64_t rows,
                                                              int64_t cols, float* colsum) {
  __shared__ float shsum[8][kColStrip + 1];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * kColStrip + tx * 8;
  const int64_t r0 = (int64_t)blockIdx.y * kColRowsPerChunk;
  const int64_t r1 = min<int64_t>(r0 + kColRowsPerChunk, rows);
  float cs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) cs[i] = 0.0f;
  if (c0 < cols) {
    const int cnt = (int)min<int64_t>(8, cols - c0);
    for (int64_t r = r0 + ty; r < r1; r += 8) {
      const uint8_t* p = g8 + r * cols + c0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < cnt) cs[i] += fp8_to_f32<FMT>(p[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) shsum[ty][tx * 8 + i] = cs[i];
  __syncthreads();
  const int col = threadIdx.x;
  const int64_t gc = (int64_t)blockIdx.x * kColStrip + col;
  float t = 0.0f;
#pragma unroll
  for (int y = 0; y < 8; ++y) t += shsum[y][col];
  if (gc < cols) colsum[(int64_t)blockIdx.y * cols + gc] = t;
}

// Ring reset (one block): scale 1, idx 0, hist 0, every counter and max 0.
__global__ void ring_init_kernel(RingHdr* h, float* hist, int H) {
  for (int j = threadIdx.x; j < H; j += blockDim.x) hist[j] = 0.0f;
  uint32_t* w = reinterpret_cast<uint32_t*>(h);
  for (int j = threadIdx.x; j < (int)(sizeof(RingHdr) / 4); j += blockDim.x) w[j] = 0u;
  __syncthreads();
  if (threadIdx.x == 0) {
    h->scale = 1.0f;
    h->hist_len = (uint32_t)H;
  }
}

__global__ void zero_u32_kernel(uint32_t* p) { *p = 0u; }

}  // namespace fp8l
