// C ABI of libfp8linear.so: argument validation, then launches on the
// caller's streams.  No device allocation, no host synchronization (the
// two-stream backward creates one event per device on first use).
//
// The four entry points follow the two-primitive API of [P3] (quantize, and
// a GEMM that consumes quantized operands and their scales) with the
// optional per-operand rings of [P1] and the pre-quantized operands of
// [P1]/[P3].  Every check below runs before the first launch, so an error
// status means nothing was enqueued.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/fp8linear.h"
#include "fp8l_device.hpp"
#include "fp8l_gemm.hpp"
#include "fp8l_gemm5.hpp"
#include "fp8l_gemm_pair.hpp"
#include "fp8l_quantize.hpp"

namespace fp8l {
namespace {

// Per-device host caches are atomics: library calls may come from several
// host threads, and two first calls on one device may both fill an entry
// (with the same value).
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Raise a kernel's dynamic LDS limit to lds bytes, once per device (the
// flag is published after the attribute is set, so a thread that sees it
// launches after the setting).
void set_lds_limit(const void* kernel, int lds, std::atomic<bool> (&done)[64]) {
  int dev = 0;
  const bool known = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  if (known && done[dev].load(std::memory_order_acquire)) return;
  (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (known) done[dev].store(true, std::memory_order_release);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool is_hp(int32_t dt) { return dt == FP8_DT_F32 || dt == FP8_DT_F16 || dt == FP8_DT_BF16; }
bool is_f8(int32_t dt) { return dt == FP8_DT_E4M3 || dt == FP8_DT_E5M2; }
bool valid_fmt(int32_t f) { return f == FP8_E4M3 || f == FP8_E5M2; }
int32_t fmt_dtype(int32_t f) { return f == FP8_E4M3 ? FP8_DT_E4M3 : FP8_DT_E5M2; }
int dtype_fmt(int32_t dt) { return dt == FP8_DT_E4M3 ? kE4M3 : kE5M2; }
bool is_fp8_dtype(int32_t dt) { return dt == FP8_DT_E4M3 || dt == FP8_DT_E5M2; }

// a * b fits in int64 (a, b >= 0)
bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / 4 / a; }

int check_ring(const fp8_ring_t* r) {
  if (!r) return FP8_OK;
  if (!r->dev) return FP8_ERR_NULL;
  if (r->hist_len < 1 || r->hist_len > FP8_RING_MAX_HIST) return FP8_ERR_RING;
  if (((uintptr_t)r->dev & 255u) != 0) return FP8_ERR_RING;
  return FP8_OK;
}

// a scale output must not be the ring's own scale slot
int check_alias(const fp8_ring_t* r, const float* scale_out) {
  if (r && scale_out && (const void*)scale_out >= r->dev &&
      (const char*)scale_out < (const char*)r->dev + sizeof(RingHdr))
    return FP8_ERR_RING;
  return FP8_OK;
}

// True while the stream is being captured into a graph.  A query that fails
// counts as not capturing (a launch on such a stream fails on its own).
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive;
}

// A ring's first use seeds it with an extra amax pass, decided on the host
// from ring->seeded.  Captured into a graph, that pass and the seeding
// conversion would run again on every replay (dynamic scaling, while the
// host flag says seeded), so an unseeded ring is refused under capture.
int check_seed_capture(const fp8_ring_t* r, hipStream_t st) {
  return (r && !r->seeded && capturing(st)) ? FP8_ERR_RING : FP8_OK;
}

// Checks for one quantize (shared by the four entry points).
int check_quant(const void* x, int32_t in_dtype, int64_t n, int32_t fmt, const uint8_t* q,
                const fp8_ring_t* ring, const float* scale_used, const float* amax_out,
                hipStream_t stream) {
  if (n < 0) return FP8_ERR_SHAPE;
  if (!is_hp(in_dtype) || !valid_fmt(fmt)) return FP8_ERR_DTYPE;
  if (n > 0 && (!x || !q)) return FP8_ERR_NULL;
  if (!scale_used) return FP8_ERR_NULL;
  if (!ring && !amax_out) return FP8_ERR_NULL;
  int st = check_ring(ring);
  if (st) return st;
  if ((st = check_alias(ring, scale_used))) return st;
  return check_seed_capture(ring, stream);
}

// 2-D shape of a quantize: the column-sum variant (ws != null) or the
// transposed/dual variant (tkernel: q and/or qt).
struct ColsumSpec {
  int64_t rows, cols;
  float* ws;
  uint8_t* qt = nullptr;
  bool tkernel = false;
};

int64_t flat_blocks(int64_t n, int64_t cap) {
  int64_t blocks = (n + kBlockChunk - 1) / kBlockChunk;
  return blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
}

template <int IN, int FMT, int SMODE>
void launch_convert(const QArgs& a, const ColsumSpec* cs, hipStream_t st) {
  if (cs && cs->tkernel) {
    const int64_t tiles = ((cs->rows + kTT - 1) / kTT) * ((cs->cols + kTT - 1) / kTT);
    const int64_t cap = (int64_t)cu_count() * 8;
    const int64_t blocks = tiles < 1 ? 1 : (tiles > cap ? cap : tiles);
    hipLaunchKernelGGL((quantize_t_kernel<IN, FMT, SMODE>), dim3((unsigned)blocks), dim3(kQThreads),
                       0, st, a);
  } else if (cs && cs->rows > 0 && cs->cols > 0) {
    dim3 grid((unsigned)((cs->cols + kColStrip - 1) / kColStrip),
              (unsigned)((cs->rows + kColRowsPerChunk - 1) / kColRowsPerChunk));
    hipLaunchKernelGGL((quantize_colsum_kernel<IN, FMT, SMODE>), grid, dim3(kQThreads), 0, st, a);
  } else {
    const int64_t blocks = flat_blocks(a.n, (int64_t)cu_count() * 8);
    hipLaunchKernelGGL((quantize_flat_kernel<IN, FMT, SMODE>), dim3((unsigned)blocks),
                       dim3(kQThreads), 0, st, a);
  }
}

template <int IN, int FMT>
void enqueue_quant_t(const void* x, int64_t n, uint8_t* q, fp8_ring_t* ring, float* scale_used,
                     float* amax_out, const ColsumSpec* cs, hipStream_t st, bool defer) {
  QArgs a = {};
  a.x = x;
  a.q = q;
  a.n = n;
  a.scale_used = scale_used;
  a.amax_out = amax_out;
  a.vec_ok = aligned16(x) && aligned16(q);
  if (cs) {
    a.rows = cs->rows;
    a.cols = cs->cols;
    a.colsum = cs->ws;
    a.vec_ok = a.vec_ok && (cs->cols % 8 == 0);
    a.qt = cs->qt;
    a.qt_vec = cs->qt && aligned16(cs->qt) && cs->rows % 16 == 0;
  }
  const int vec_x = aligned16(x);
  if (ring) {
    a.ring = reinterpret_cast<RingHdr*>(ring->dev);
    a.hist = reinterpret_cast<float*>(reinterpret_cast<char*>(ring->dev) + sizeof(RingHdr));
    a.hist_len = ring->hist_len;
    if (ring->seeded && defer) {
      launch_convert<IN, FMT, kScaleDefer>(a, cs, st);  // the consuming GEMM folds
    } else if (ring->seeded) {
      launch_convert<IN, FMT, kScaleRing>(a, cs, st);
    } else {
      // first use: the amax pass leaves max |x| in the ring header, the
      // converting launch seeds the scale from it, converts and folds.
      const int64_t blocks = flat_blocks(n, (int64_t)cu_count() * 8);
      hipLaunchKernelGGL((amax_ring_kernel<IN>), dim3((unsigned)blocks), dim3(kQThreads), 0, st, x,
                         n, vec_x, a.ring);
      launch_convert<IN, FMT, kScaleSeed>(a, cs, st);
      ring->seeded = 1;
    }
  } else {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, st, reinterpret_cast<uint32_t*>(amax_out));
    const int64_t blocks = flat_blocks(n, (int64_t)cu_count());
    hipLaunchKernelGGL((amax_dyn_kernel<IN>), dim3((unsigned)blocks), dim3(kQThreads), 0, st, x, n,
                       vec_x, reinterpret_cast<uint32_t*>(amax_out));
    launch_convert<IN, FMT, kScaleDyn>(a, cs, st);
  }
}

// X and W of a forward in one launch (same input type, both rings seeded).
template <int IN, int FMT>
void enqueue_quant2_t(const void* x0, int64_t n0, uint8_t* q0, fp8_ring_t* r0, float* su0,
                      float* am0, const void* x1, int64_t n1, uint8_t* q1, fp8_ring_t* r1,
                      float* su1, float* am1, hipStream_t st, bool defer) {
  auto args = [](const void* x, int64_t n, uint8_t* q, fp8_ring_t* r, float* su, float* am) {
    QArgs a = {};
    a.x = x;
    a.q = q;
    a.n = n;
    a.scale_used = su;
    a.amax_out = am;
    a.vec_ok = aligned16(x) && aligned16(q);
    a.ring = reinterpret_cast<RingHdr*>(r->dev);
    a.hist = reinterpret_cast<float*>(reinterpret_cast<char*>(r->dev) + sizeof(RingHdr));
    a.hist_len = r->hist_len;
    return a;
  };
  const QArgs a0 = args(x0, n0, q0, r0, su0, am0), a1 = args(x1, n1, q1, r1, su1, am1);
  const int64_t cap = (int64_t)cu_count() * 8;
  int64_t b0 = flat_blocks(n0, cap), b1 = flat_blocks(n1, cap);
  if (b0 + b1 > cap) {  // share the cap in proportion to the sizes
    b0 = (int64_t)((double)cap * (double)n0 / (double)(n0 + n1));
    b0 = b0 < 1 ? 1 : (b0 > cap - 1 ? cap - 1 : b0);
    b1 = cap - b0;
  }
  if (defer)
    hipLaunchKernelGGL((quantize_flat2_kernel<IN, FMT, kScaleDefer>), dim3((unsigned)(b0 + b1)),
                       dim3(kQThreads), 0, st, a0, a1, (uint32_t)b0);
  else
    hipLaunchKernelGGL((quantize_flat2_kernel<IN, FMT, kScaleRing>), dim3((unsigned)(b0 + b1)),
                       dim3(kQThreads), 0, st, a0, a1, (uint32_t)b0);
}

template <int IN>
void enqueue_quant2_in(int32_t fmt, const void* x0, int64_t n0, uint8_t* q0, fp8_ring_t* r0,
                       float* su0, float* am0, const void* x1, int64_t n1, uint8_t* q1,
                       fp8_ring_t* r1, float* su1, float* am1, hipStream_t st, bool defer) {
  if (fmt == FP8_E4M3)
    enqueue_quant2_t<IN, kE4M3>(x0, n0, q0, r0, su0, am0, x1, n1, q1, r1, su1, am1, st, defer);
  else
    enqueue_quant2_t<IN, kE5M2>(x0, n0, q0, r0, su0, am0, x1, n1, q1, r1, su1, am1, st, defer);
}

template <int IN>
void enqueue_quant_in(const void* x, int64_t n, int32_t fmt, uint8_t* q, fp8_ring_t* ring,
                      float* scale_used, float* amax_out, const ColsumSpec* cs, hipStream_t st,
                      bool defer) {
  if (fmt == FP8_E4M3)
    enqueue_quant_t<IN, kE4M3>(x, n, q, ring, scale_used, amax_out, cs, st, defer);
  else
    enqueue_quant_t<IN, kE5M2>(x, n, q, ring, scale_used, amax_out, cs, st, defer);
}

// A quantize through this ring may leave its fold to the GEMM that consumes
// the codes: the ring is seeded (one converting launch, no seeding pass) and
// its window fits the one wave that folds it.
bool can_defer(const fp8_ring_t* r) { return r && r->seeded && r->hist_len <= 64; }

// The fold the consuming GEMM does for a deferred quantize through r.
RingFold fold_of(const fp8_ring_t* r, int32_t fmt, float* amax_out) {
  RingFold f = {};
  f.ring = reinterpret_cast<RingHdr*>(r->dev);
  f.hist = reinterpret_cast<float*>(reinterpret_cast<char*>(r->dev) + sizeof(RingHdr));
  f.hist_len = r->hist_len;
  f.fmt_max = fmt == FP8_E4M3 ? FmtTraits<kE4M3>::kMax : FmtTraits<kE5M2>::kMax;
  f.amax_out = amax_out;
  return f;
}

// The fold of a ring whose groups a deferring launch filled, as a launch of
// its own (one wave): for codes that no GEMM of the same call consumes (a
// standalone quantize, the FP8-output GEMM's output), so that no block of
// the converting launch waits on an election.
__global__ __launch_bounds__(64) void ring_fold_kernel(RingFold f) { ring_fold_wave(f); }
__global__ __launch_bounds__(64) void ring_fold2_kernel(RingFold f0, RingFold f1) {
  ring_fold_wave(f0);
  ring_fold_wave(f1);
}

// One quantize.  may_defer: the caller launches a GEMM on the codes next,
// on the same stream, which folds the ring when this returns true.
bool enqueue_quant(const void* x, int32_t in_dtype, int64_t n, int32_t fmt, uint8_t* q,
                   fp8_ring_t* ring, float* scale_used, float* amax_out, const ColsumSpec* cs,
                   hipStream_t st, bool may_defer = false) {
  const bool defer = may_defer && can_defer(ring);
  // no consuming GEMM to hand the fold to: a one-wave launch folds it
  const bool fold_after = !may_defer && can_defer(ring);
  const bool groups_only = defer || fold_after;
  if (in_dtype == FP8_DT_F32)
    enqueue_quant_in<kInF32>(x, n, fmt, q, ring, scale_used, amax_out, cs, st, groups_only);
  else if (in_dtype == FP8_DT_F16)
    enqueue_quant_in<kInF16>(x, n, fmt, q, ring, scale_used, amax_out, cs, st, groups_only);
  else
    enqueue_quant_in<kInBF16>(x, n, fmt, q, ring, scale_used, amax_out, cs, st, groups_only);
  if (fold_after)
    hipLaunchKernelGGL(ring_fold_kernel, dim3(1), dim3(64), 0, st, fold_of(ring, fmt, amax_out));
  return defer;
}

// Two quantizes: one launch when the input types match and both rings are
// seeded (the steady state of delayed scaling), else one after the other.
// may_defer as enqueue_quant; *d0 / *d1 say which folds were left.
void enqueue_quant_pair(const void* x0, int32_t dt0, int64_t n0, uint8_t* q0, fp8_ring_t* r0,
                        float* su0, float* am0, const void* x1, int32_t dt1, int64_t n1,
                        uint8_t* q1, fp8_ring_t* r1, float* su1, float* am1, int32_t fmt,
                        hipStream_t st, bool may_defer = false, bool* d0 = nullptr,
                        bool* d1 = nullptr) {
  const bool one = dt0 == dt1 && r0 && r1 && r0->seeded && r1->seeded && n0 > 0 && n1 > 0;
  bool f0 = false, f1 = false;
  if (!one) {
    f0 = enqueue_quant(x0, dt0, n0, fmt, q0, r0, su0, am0, nullptr, st, may_defer);
    f1 = enqueue_quant(x1, dt1, n1, fmt, q1, r1, su1, am1, nullptr, st, may_defer);
  } else {
    const bool both = can_defer(r0) && can_defer(r1);
    f0 = f1 = may_defer && both;
    const bool fold_after = !may_defer && both;  // as in enqueue_quant
    const bool groups_only = f0 || fold_after;
    if (dt0 == FP8_DT_F32)
      enqueue_quant2_in<kInF32>(fmt, x0, n0, q0, r0, su0, am0, x1, n1, q1, r1, su1, am1, st,
                                groups_only);
    else if (dt0 == FP8_DT_F16)
      enqueue_quant2_in<kInF16>(fmt, x0, n0, q0, r0, su0, am0, x1, n1, q1, r1, su1, am1, st,
                                groups_only);
    else
      enqueue_quant2_in<kInBF16>(fmt, x0, n0, q0, r0, su0, am0, x1, n1, q1, r1, su1, am1, st,
                                 groups_only);
    if (fold_after)
      hipLaunchKernelGGL(ring_fold2_kernel, dim3(1), dim3(64), 0, st, fold_of(r0, fmt, am0),
                         fold_of(r1, fmt, am1));
  }
  if (d0) *d0 = f0;
  if (d1) *d1 = f1;
}

template <int LA, int LB, int FA, int FB>
void launch_gemm_t(GemmArgs& g, hipStream_t st) {
  hipLaunchKernelGGL((gemm_kernel<LA, LB, FA, FB>),
                     dim3((unsigned)(g.tiles_m * g.tiles_n), (unsigned)g.batch), dim3(kGThreads), 0,
                     st, g);
}

template <int BM, int BN, int WGM, int WGN, int LA, int LB, int FA, int FB, int EPI = kEpiBF16,
          int OF = kE4M3>
void launch_gemm3_t(GemmArgs& g, hipStream_t st) {
  constexpr int lds = gemm3_lds_bytes<BM, BN, WGM, WGN>();
  static std::atomic<bool> lds_set[64];
  set_lds_limit((const void*)gemm3_kernel<BM, BN, WGM, WGN, LA, LB, FA, FB, EPI, OF>, lds,
                lds_set);
  g.tiles_m = (int32_t)((g.Mc + BM - 1) / BM);
  g.tiles_n = (int32_t)((g.Nc + BN - 1) / BN);
  if (g.tiles_m < 1) g.tiles_m = 1;
  if (g.tiles_n < 1) g.tiles_n = 1;
  hipLaunchKernelGGL((gemm3_kernel<BM, BN, WGM, WGN, LA, LB, FA, FB, EPI, OF>),
                     dim3((unsigned)(g.tiles_m * g.tiles_n), (unsigned)g.batch), dim3(64 * WGM * WGN),
                     lds, st, g);
}

enum { kTileAuto = 0, kTile256x256, kTile256x128, kTile128x128, kTileV1, kTile256x256w8, kTile128x128w8 };

// FP8L_TILE forces a tile configuration (for sweeps and tests): 256x256,
// 256x128, 128x128 or v1 (the general register-staged kernel).  Read at
// every launch so one process can compare configurations.
int forced_tile() {
  const char* e = getenv("FP8L_TILE");
  if (!e) return kTileAuto;
  if (!strcmp(e, "256x256")) return kTile256x256;
  if (!strcmp(e, "256x128")) return kTile256x128;
  if (!strcmp(e, "128x128")) return kTile128x128;
  if (!strcmp(e, "v1")) return kTileV1;
  if (!strcmp(e, "256x256w8")) return kTile256x256w8;
  if (!strcmp(e, "128x128w8")) return kTile128x128w8;
  return kTileAuto;
}

// Tile choice (measured crossovers on the layer shapes; tiles counted over
// all batch slices).  Larger tiles move fewer operand bytes per MFMA but
// leave CUs idle when the output has few tiles, and one tile per CU cannot
// overlap its epilogue with another loop.
//  * 128x128, 4 waves, two blocks per CU (gemm3): when K <= 1024 and the
//    tiles fit one round at two blocks per CU.  With a short K loop the
//    fixed phases (first stage, epilogue burst) weigh most, and the second
//    block on each CU overlaps them (2048 x 4096 x 1024: 16.1 us against
//    19.4 on 256x256; 4608 x 1536 x 512: 8.6 against 10.1 on 256x128).
//  * 256x256, 8 waves (gemm4): when its tiles fill at least half the CUs.
//  * 128x128, 8 waves (gemm5): when the 128x128 tiles fit one per CU; the
//    block's 8 waves give each SIMD two waves.
//  * 256x128, 4 waves (gemm3): when more 128x128 tiles than CUs but the
//    256x128 tiles fit one per CU (the 4608 x 1536 weight gradient at
//    K = 2048: 18.7 us against 21.3 us for two 128x128 blocks per CU).
//  * 128x128, 4 waves, two blocks per CU (gemm3): otherwise.
int choose_tile(int64_t Mc, int64_t Nc, int64_t Kc, int64_t batch) {
  const int64_t cus = cu_count();
  const int64_t tiles256 = batch * ((Mc + 255) / 256) * ((Nc + 255) / 256);
  const int64_t tiles128 = batch * ((Mc + 127) / 128) * ((Nc + 127) / 128);
  const int64_t tiles256x128 = batch * ((Mc + 255) / 256) * ((Nc + 127) / 128);
  if (Kc <= 1024 && tiles128 <= 2 * cus) return kTile128x128;
  if (2 * tiles256 >= cus) return kTile256x256w8;
  if (tiles128 <= cus) return kTile128x128w8;
  return tiles256x128 <= cus ? kTile256x128 : kTile128x128;
}

template <int BM, int BN, int WGM, int WGN, int LA, int LB>
void launch_gemm3_f(GemmArgs& g, int fa, int fb, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) launch_gemm3_t<BM, BN, WGM, WGN, LA, LB, kE4M3, kE4M3>(g, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_gemm3_t<BM, BN, WGM, WGN, LA, LB, kE4M3, kE5M2>(g, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_gemm3_t<BM, BN, WGM, WGN, LA, LB, kE5M2, kE4M3>(g, st);
  else launch_gemm3_t<BM, BN, WGM, WGN, LA, LB, kE5M2, kE5M2>(g, st);
}



template <int LA, int LB, int FA, int FB, int EPI = kEpiBF16, int OF = kE4M3>
void launch_gemm4_t(GemmArgs& g, hipStream_t st) {
  constexpr int lds = gemm4_lds_bytes();
  static std::atomic<bool> lds_set[64];
  set_lds_limit((const void*)gemm4_kernel<LA, LB, FA, FB, EPI, OF>, lds, lds_set);
  g.tiles_m = (int32_t)((g.Mc + 255) / 256);
  g.tiles_n = (int32_t)((g.Nc + 255) / 256);
  if (g.tiles_m < 1) g.tiles_m = 1;
  if (g.tiles_n < 1) g.tiles_n = 1;
  hipLaunchKernelGGL((gemm4_kernel<LA, LB, FA, FB, EPI, OF>),
                     dim3((unsigned)(g.tiles_m * g.tiles_n), (unsigned)g.batch), dim3(512), lds, st,
                     g);
}

template <int LA, int LB>
void launch_gemm4_f(GemmArgs& g, int fa, int fb, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) launch_gemm4_t<LA, LB, kE4M3, kE4M3>(g, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_gemm4_t<LA, LB, kE4M3, kE5M2>(g, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_gemm4_t<LA, LB, kE5M2, kE4M3>(g, st);
  else launch_gemm4_t<LA, LB, kE5M2, kE5M2>(g, st);
}

// The FP8-output GEMM runs with one of the fp8 epilogues on the 256x256
// 8-wave kernel when its tiles fill at least half the CUs (the bf16 rule),
// else on gemm3's 128x128 block (4 waves, two blocks per CU).
template <int FA, int FB, int EPI, int OF>
void launch_fp8out_t(GemmArgs& g, hipStream_t st) {
  const int64_t tiles256 = ((g.Mc + 255) / 256) * ((g.Nc + 255) / 256);
  if (2 * tiles256 >= cu_count())
    launch_gemm4_t<kKContig, kKContig, FA, FB, EPI, OF>(g, st);
  else
    launch_gemm3_t<128, 128, 2, 2, kKContig, kKContig, FA, FB, EPI, OF>(g, st);
}

template <int EPI, int OF>
void launch_fp8out(GemmArgs& g, int fa, int fb, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) launch_fp8out_t<kE4M3, kE4M3, EPI, OF>(g, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_fp8out_t<kE4M3, kE5M2, EPI, OF>(g, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_fp8out_t<kE5M2, kE4M3, EPI, OF>(g, st);
  else launch_fp8out_t<kE5M2, kE5M2, EPI, OF>(g, st);
}

template <int LA, int LB, int FA, int FB>
void launch_gemm5_t(GemmArgs& g, hipStream_t st) {
  constexpr int lds = gemm5_lds_bytes();
  static std::atomic<bool> lds_set[64];
  set_lds_limit((const void*)gemm5_kernel<LA, LB, FA, FB>, lds, lds_set);
  g.tiles_m = (int32_t)((g.Mc + 127) / 128);
  g.tiles_n = (int32_t)((g.Nc + 127) / 128);
  if (g.tiles_m < 1) g.tiles_m = 1;
  if (g.tiles_n < 1) g.tiles_n = 1;
  hipLaunchKernelGGL((gemm5_kernel<LA, LB, FA, FB>),
                     dim3((unsigned)(g.tiles_m * g.tiles_n), (unsigned)g.batch), dim3(512), lds, st,
                     g);
}

template <int LA, int LB>
void launch_gemm5_f(GemmArgs& g, int fa, int fb, hipStream_t st) {
  if (fa == kE4M3 && fb == kE4M3) launch_gemm5_t<LA, LB, kE4M3, kE4M3>(g, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_gemm5_t<LA, LB, kE4M3, kE5M2>(g, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_gemm5_t<LA, LB, kE5M2, kE4M3>(g, st);
  else launch_gemm5_t<LA, LB, kE5M2, kE5M2>(g, st);
}

// The fast kernel needs 16-byte chunks that never straddle a matrix edge and
// byte offsets that fit a buffer descriptor.
template <int LA, int LB>
bool fast_path_ok(const GemmArgs& g) {
  const int64_t a_rows = (LA == kKContig) ? g.Mc : g.Kc;
  const int64_t b_rows = (LB == kKContig) ? g.Nc : g.Kc;
  const int64_t a_inner = (LA == kKContig) ? g.Kc : g.Mc;
  const int64_t b_inner = (LB == kKContig) ? g.Kc : g.Nc;
  // a tile may hang up to 256 rows past the last one; its offsets must stay
  // below 2^32 so they read as out of range instead of wrapping
  return aligned16(g.a) && aligned16(g.b) && aligned16(g.c) && g.ldc % 8 == 0 && g.Nc % 8 == 0 &&
         g.bsa % 16 == 0 && g.bsb % 16 == 0 && g.bsc % 8 == 0 &&
         g.lda % 16 == 0 && g.ldb % 16 == 0 &&
         a_inner % 16 == 0 && b_inner % 16 == 0 && (a_rows + 256) * g.lda < (1LL << 31) &&
         (b_rows + 256) * g.ldb < (1LL << 31);
}

template <int LA, int LB>
void launch_gemm_l(GemmArgs& g, int fa, int fb, hipStream_t st) {
  int tile = forced_tile();
  if (!fast_path_ok<LA, LB>(g)) tile = kTileV1;
  if (tile == kTileAuto) tile = choose_tile(g.Mc, g.Nc, g.Kc, g.batch);
  switch (tile) {
    case kTile256x256: launch_gemm3_f<256, 256, 2, 2, LA, LB>(g, fa, fb, st); return;
    case kTile256x128: launch_gemm3_f<256, 128, 2, 2, LA, LB>(g, fa, fb, st); return;
    case kTile128x128: launch_gemm3_f<128, 128, 2, 2, LA, LB>(g, fa, fb, st); return;
    case kTile256x256w8: launch_gemm4_f<LA, LB>(g, fa, fb, st); return;
    case kTile128x128w8: launch_gemm5_f<LA, LB>(g, fa, fb, st); return;
    default: break;
  }
  if (fa == kE4M3 && fb == kE4M3) launch_gemm_t<LA, LB, kE4M3, kE4M3>(g, st);
  else if (fa == kE4M3 && fb == kE5M2) launch_gemm_t<LA, LB, kE4M3, kE5M2>(g, st);
  else if (fa == kE5M2 && fb == kE4M3) launch_gemm_t<LA, LB, kE5M2, kE4M3>(g, st);
  else launch_gemm_t<LA, LB, kE5M2, kE5M2>(g, st);
}

// The grouped backward (fp8l_gemm_pair.hpp): dX (A = G8 k-contiguous, B =
// W8 crosswise) and dW (both crosswise) in one launch, each problem on the
// 8-wave kernel its own launch would take (256x256 or 128x128).  The
// problem whose tiles take longer (tile area times K) gets the first block
// range.
template <class BX, class BW>
void launch_pair_t(GemmArgs& dx, GemmArgs& dw, hipStream_t st) {
  constexpr int lds = pair_lds_bytes<BX, BW>();
  static std::atomic<bool> lds_set[64];
  set_lds_limit((const void*)gemm_pair_kernel<BX, BW>, lds, lds_set);
  auto tiles = [](GemmArgs& g, int bm, int bn) {
    g.tiles_m = (int32_t)((g.Mc + bm - 1) / bm);
    g.tiles_n = (int32_t)((g.Nc + bn - 1) / bn);
    if (g.tiles_m < 1) g.tiles_m = 1;
    if (g.tiles_n < 1) g.tiles_n = 1;
    return g.tiles_m * g.tiles_n;
  };
  const int nx = tiles(dx, BX::kBM, BX::kBN), nw = tiles(dw, BW::kBM, BW::kBN);
  const double work_x = (double)BX::kBM * BX::kBN * (double)dx.Kc;
  const double work_w = (double)BW::kBM * BW::kBN * (double)dw.Kc;
  GemmArgs& first = work_x >= work_w ? dx : dw;
  GemmArgs& second = work_x >= work_w ? dw : dx;
  first.blk0 = 0;
  first.nblk = work_x >= work_w ? nx : nw;
  second.blk0 = (first.nblk + 7) & ~7;
  second.nblk = work_x >= work_w ? nw : nx;
  hipLaunchKernelGGL((gemm_pair_kernel<BX, BW>), dim3((unsigned)(second.blk0 + second.nblk)),
                     dim3(512), lds, st, dx, dw);
}

// Grouped launch when both problems would take an 8-wave kernel on their
// own (so the grouped results are the two launches' bits), with the
// standard recipe's formats (G in e5m2, W8 and X8 in e4m3) and no tile
// forced; false: the caller launches them one by one.
bool launch_pair(GemmArgs& dx, GemmArgs& dw, int fmt_g, int fmt_w, int fmt_x, hipStream_t st) {
  if (fmt_g != kE5M2 || fmt_w != kE4M3 || fmt_x != kE4M3 || forced_tile() != kTileAuto) return false;
  if (dx.batch != 1 || dw.batch != 1) return false;
  if (!fast_path_ok<kKContig, kCross>(dx) || !fast_path_ok<kCross, kCross>(dw)) return false;
  const int tx = choose_tile(dx.Mc, dx.Nc, dx.Kc, 1), tw = choose_tile(dw.Mc, dw.Nc, dw.Kc, 1);
  const bool eight = [](int t) { return t == kTile256x256w8 || t == kTile128x128w8; }(tx) &&
                     (tw == kTile256x256w8 || tw == kTile128x128w8);
  if (!eight) return false;
  const bool big_x = tx == kTile256x256w8;
  const bool big_w = tw == kTile256x256w8;
  using X4 = Body4<kKContig, kCross, kE5M2, kE4M3>;
  using X5 = Body5<kKContig, kCross, kE5M2, kE4M3>;
  using W4 = Body4<kCross, kCross, kE5M2, kE4M3>;
  using W5 = Body5<kCross, kCross, kE5M2, kE4M3>;
  if (big_x && big_w) launch_pair_t<X4, W4>(dx, dw, st);
  else if (big_x) launch_pair_t<X4, W5>(dx, dw, st);
  else if (big_w) launch_pair_t<X5, W4>(dx, dw, st);
  else launch_pair_t<X5, W5>(dx, dw, st);
  return true;
}

void finish_gemm_args(GemmArgs& g) {
  const int64_t tm = (g.Mc + kBM - 1) / kBM, tn = (g.Nc + kBN - 1) / kBN;
  g.tiles_m = (int32_t)(tm < 1 ? 1 : tm);
  g.tiles_n = (int32_t)(tn < 1 ? 1 : tn);
  if (g.batch < 1) g.batch = 1;
  g.a_vec = aligned16(g.a) && g.lda % 16 == 0 && g.bsa % 16 == 0;
  g.b_vec = aligned16(g.b) && g.ldb % 16 == 0 && g.bsb % 16 == 0;
  g.c_vec = ((uintptr_t)g.c & 7u) == 0 && g.ldc % 4 == 0 && g.bsc % 4 == 0;
}

int hip_status() { return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_HIP; }

}  // namespace

// Library-owned device memory of fp8_linear_bwd_dw_noalloc: the db column
// partials, FP8_NOALLOC_WS_MAX bytes, one copy per GPU for the life of the
// process.  Host code never uses the array's name as an address (on the host
// it is only a stand-in); it uses the address hipGetSymbolAddress returns on
// each device, kept in scratch_dev.
__device__ __align__(256) float scratch[FP8_NOALLOC_WS_MAX / 4];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64];

// Device address of this GPU's scratch array (the current device's), looked
// up once per device with that device current.  nullptr if the lookup fails.
float* scratch_dev() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_dev[dev] = p;
  }
  return reinterpret_cast<float*>(g_scratch_dev[dev]);
}
}  // namespace
}  // namespace fp8l

using namespace fp8l;

extern "C" {

int fp8_abi_version(void) { return FP8_ABI_VERSION; }

#ifndef FP8L_SOURCE_HASH
#define FP8L_SOURCE_HASH "unknown"
#endif
const char* fp8_source_hash(void) { return FP8L_SOURCE_HASH; }

const char* fp8_status_str(int status) {
  switch (status) {
    case FP8_OK: return "ok";
    case FP8_ERR_NULL: return "a required pointer is NULL";
    case FP8_ERR_SHAPE: return "invalid size (negative or overflowing)";
    case FP8_ERR_DTYPE: return "invalid or mismatched dtype/format";
    case FP8_ERR_RING: return "invalid scale ring (hist_len, alignment or aliasing)";
    case FP8_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t fp8_ring_bytes(int32_t hist_len) {
  if (hist_len < 1 || hist_len > FP8_RING_MAX_HIST) return 0;
  return sizeof(RingHdr) + 4u * (size_t)hist_len;
}

size_t fp8_db_workspace_bytes(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return 0;
  const int64_t R = (M + kColRowsPerChunk - 1) / kColRowsPerChunk;
  return (size_t)(4 * R * N);
}

int fp8_ring_init(fp8_ring_t* ring, void* dev, int32_t hist_len, hipStream_t stream) {
  if (!ring || !dev) return FP8_ERR_NULL;
  if (hist_len < 1 || hist_len > FP8_RING_MAX_HIST || ((uintptr_t)dev & 255u)) return FP8_ERR_RING;
  hipLaunchKernelGGL(ring_init_kernel, dim3(1), dim3(256), 0, stream, reinterpret_cast<RingHdr*>(dev),
                     reinterpret_cast<float*>(reinterpret_cast<char*>(dev) + sizeof(RingHdr)),
                     (int)hist_len);
  const int st = hip_status();
  if (st) return st;
  ring->dev = dev;
  ring->hist_len = hist_len;
  ring->seeded = 0;
  return FP8_OK;
}

int fp8_quantize_pair(const void* x0, int32_t dtype0, int64_t n0, uint8_t* q0, fp8_ring_t* ring0,
                      float* scale_used0, float* amax_out0, const void* x1, int32_t dtype1,
                      int64_t n1, uint8_t* q1, fp8_ring_t* ring1, float* scale_used1,
                      float* amax_out1, int32_t fmt, hipStream_t stream) {
  int st = check_quant(x0, dtype0, n0, fmt, q0, ring0, scale_used0, amax_out0, stream);
  if (st) return st;
  st = check_quant(x1, dtype1, n1, fmt, q1, ring1, scale_used1, amax_out1, stream);
  if (st) return st;
  if (!mul_ok(n0, 4) || !mul_ok(n1, 4)) return FP8_ERR_SHAPE;
  if (ring0 && ring0 == ring1) return FP8_ERR_RING;
  enqueue_quant_pair(x0, dtype0, n0, q0, ring0, scale_used0, amax_out0, x1, dtype1, n1, q1, ring1,
                     scale_used1, amax_out1, fmt, stream);
  return hip_status();
}

int fp8_quantize_2d(const void* x, int32_t in_dtype, int64_t rows, int64_t cols, int32_t fmt,
                    int32_t layout, uint8_t* q, uint8_t* qt, fp8_ring_t* ring, float* scale_used,
                    float* amax_out, hipStream_t stream) {
  if (rows < 0 || cols < 0 || !mul_ok(rows, cols)) return FP8_ERR_SHAPE;
  if (layout != FP8_QUANT_ROWS && layout != FP8_QUANT_TRANSPOSED && layout != FP8_QUANT_DUAL)
    return FP8_ERR_DTYPE;
  const int64_t n = rows * cols;
  if (!mul_ok(n, 4)) return FP8_ERR_SHAPE;
  const bool want_q = layout != FP8_QUANT_TRANSPOSED, want_qt = layout != FP8_QUANT_ROWS;
  if (n > 0 && ((want_q && !q) || (want_qt && !qt))) return FP8_ERR_NULL;
  // the rest as fp8_quantize (q stands for whichever output is given)
  int st = check_quant(x, in_dtype, n, fmt, want_q ? q : qt, ring, scale_used, amax_out, stream);
  if (st) return st;
  if (layout == FP8_QUANT_ROWS) {
    enqueue_quant(x, in_dtype, n, fmt, q, ring, scale_used, amax_out, nullptr, stream);
  } else {
    ColsumSpec cs;
    cs.rows = rows;
    cs.cols = cols;
    cs.ws = nullptr;
    cs.qt = qt;
    cs.tkernel = true;
    enqueue_quant(x, in_dtype, n, fmt, want_q ? q : nullptr, ring, scale_used, amax_out, &cs,
                  stream);
  }
  return hip_status();
}

int fp8_quantize(const void* x, int32_t in_dtype, int64_t n, int32_t fmt, uint8_t* q,
                 fp8_ring_t* ring, float* scale_used, float* amax_out, hipStream_t stream) {
  int st = check_quant(x, in_dtype, n, fmt, q, ring, scale_used, amax_out, stream);
  if (st) return st;
  if (!mul_ok(n, 4)) return FP8_ERR_SHAPE;
  enqueue_quant(x, in_dtype, n, fmt, q, ring, scale_used, amax_out, nullptr, stream);
  return hip_status();
}

int fp8_linear_fwd(int64_t M, int64_t N, int64_t K, fp8_operand_t x, fp8_operand_t w,
                   fp8_operand_t bias, int32_t fmt, fp8_ring_t* ring_x, fp8_ring_t* ring_w,
                   void* y, uint8_t* x8_out, uint8_t* w8_out, float* sx_used, float* sw_used,
                   float* amax_x, float* amax_w, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return FP8_ERR_SHAPE;
  if (!valid_fmt(fmt)) return FP8_ERR_DTYPE;
  const int32_t f8dt = fmt_dtype(fmt);
  int st;
  // X
  if (is_hp(x.dtype)) {
    st = check_quant(x.data, x.dtype, M * K, fmt, x8_out, ring_x, sx_used, amax_x, stream);
    if (st) return st;
  } else if (x.dtype == f8dt) {
    if ((M * K > 0 && !x.data) || !x.scale) return FP8_ERR_NULL;
  } else {
    return FP8_ERR_DTYPE;
  }
  // W
  if (is_hp(w.dtype)) {
    st = check_quant(w.data, w.dtype, N * K, fmt, w8_out, ring_w, sw_used, amax_w, stream);
    if (st) return st;
  } else if (w.dtype == f8dt) {
    if ((N * K > 0 && !w.data) || !w.scale) return FP8_ERR_NULL;
  } else {
    return FP8_ERR_DTYPE;
  }
  if (ring_x && ring_x == ring_w) return FP8_ERR_RING;
  // bias
  int bias_kind = kBiasNone;
  if (bias.data) {
    if (bias.dtype == FP8_DT_BF16) bias_kind = kBiasBF16;
    else if (bias.dtype == FP8_DT_E4M3) bias_kind = kBiasE4M3;
    else if (bias.dtype == FP8_DT_E5M2) bias_kind = kBiasE5M2;
    else return FP8_ERR_DTYPE;
    if (bias_kind != kBiasBF16 && !bias.scale) return FP8_ERR_NULL;
  }
  if (M * N > 0 && !y) return FP8_ERR_NULL;

  // The quantizes leave their ring folds to the GEMM below (same stream),
  // which folds them in its first block before any operand load.
  GemmArgs g = {};
  bool fold_x = false, fold_w = false;
  if (is_hp(x.dtype) && is_hp(w.dtype))
    enqueue_quant_pair(x.data, x.dtype, M * K, x8_out, ring_x, sx_used, amax_x, w.data, w.dtype,
                       N * K, w8_out, ring_w, sw_used, amax_w, fmt, stream, true, &fold_x, &fold_w);
  const bool pair = is_hp(x.dtype) && is_hp(w.dtype);
  if (is_hp(x.dtype)) {
    if (!pair)
      fold_x = enqueue_quant(x.data, x.dtype, M * K, fmt, x8_out, ring_x, sx_used, amax_x, nullptr,
                             stream, true);
    g.a = x8_out;
    g.scale_a = sx_used;
  } else {
    g.a = reinterpret_cast<const uint8_t*>(x.data);
    g.scale_a = x.scale;
    g.aux_scale_dst0 = sx_used;
    g.aux_scale_src0 = x.scale;
    g.aux_amax_dst0 = amax_x;
  }
  if (is_hp(w.dtype)) {
    if (!pair)
      fold_w = enqueue_quant(w.data, w.dtype, N * K, fmt, w8_out, ring_w, sw_used, amax_w, nullptr,
                             stream, true);
    g.b = w8_out;
    g.scale_b = sw_used;
  } else {
    g.b = reinterpret_cast<const uint8_t*>(w.data);
    g.scale_b = w.scale;
    g.aux_scale_dst1 = sw_used;
    g.aux_scale_src1 = w.scale;
    g.aux_amax_dst1 = amax_w;
  }
  g.lda = K;
  g.ldb = K;
  g.Mc = M;
  g.Nc = N;
  g.Kc = K;
  g.c = reinterpret_cast<uint16_t*>(y);
  g.ldc = N;
  g.bias = bias.data;
  g.bias_kind = bias_kind;
  g.bias_scale = bias.scale;
  if (fold_x) g.fold[0] = fold_of(ring_x, fmt, amax_x);
  if (fold_w) g.fold[1] = fold_of(ring_w, fmt, amax_w);
  finish_gemm_args(g);
  launch_gemm_l<kKContig, kKContig>(g, fmt, fmt, stream);
  return hip_status();
}

// Shared front half of the two backward entry points: validate g and
// enqueue its quantize if it is high precision.  Outputs the fp8 pointer
// and scale pointer the GEMM uses.
// fold: when not null, the quantize may leave its ring fold to the GEMM the
// caller launches next on the same stream, and *fold receives that fold
// (ring null if the quantize folded in its own launch).
static int bwd_prepare(int64_t M, int64_t N, fp8_operand_t g, int32_t fmt_g, fp8_ring_t* ring_g,
                       uint8_t* g8_out, float* sg_used, float* amax_g, bool validate_only,
                       const ColsumSpec* cs, hipStream_t stream, const uint8_t** g8,
                       const float** sg, bool* pre, RingFold* fold = nullptr) {
  if (!valid_fmt(fmt_g)) return FP8_ERR_DTYPE;
  if (is_hp(g.dtype)) {
    if (validate_only)
      return check_quant(g.data, g.dtype, M * N, fmt_g, g8_out, ring_g, sg_used, amax_g, stream);
    if (enqueue_quant(g.data, g.dtype, M * N, fmt_g, g8_out, ring_g, sg_used, amax_g, cs, stream,
                      fold != nullptr))
      *fold = fold_of(ring_g, fmt_g, amax_g);
    *g8 = g8_out;
    *sg = sg_used;
    *pre = false;
  } else if (g.dtype == fmt_dtype(fmt_g)) {
    if (validate_only) return ((M * N > 0 && !g.data) || !g.scale) ? FP8_ERR_NULL : FP8_OK;
    *g8 = reinterpret_cast<const uint8_t*>(g.data);
    *sg = g.scale;
    *pre = true;
  } else {
    return FP8_ERR_DTYPE;
  }
  return FP8_OK;
}

// The dX GEMM of a backward: dX = G8 W8 / (sg sw).  pre: g was given
// pre-quantized, so this launch's block 0 also snapshots its scale into
// sg_used and clears amax_g.
static GemmArgs dx_gemm_args(int64_t M, int64_t N, int64_t K, const uint8_t* g8, const float* sg,
                             fp8_operand_t w8, void* dx, bool pre, const float* g_scale,
                             float* sg_used, float* amax_g, const RingFold& fold) {
  GemmArgs a = {};
  a.fold[0] = fold;
  a.a = g8;  // [M, N], contraction n contiguous
  a.lda = N;
  a.b = reinterpret_cast<const uint8_t*>(w8.data);  // [N, K] read crosswise
  a.ldb = K;
  a.Mc = M;
  a.Nc = K;
  a.Kc = N;
  a.c = reinterpret_cast<uint16_t*>(dx);
  a.ldc = K;
  a.scale_a = sg;
  a.scale_b = w8.scale;
  if (pre) {
    a.aux_scale_dst0 = sg_used;
    a.aux_scale_src0 = g_scale;
    a.aux_amax_dst0 = amax_g;
  }
  finish_gemm_args(a);
  return a;
}

static void enqueue_dx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* g8, const float* sg,
                            int32_t fmt_g, fp8_operand_t w8, void* dx, bool pre, const float* g_scale,
                            float* sg_used, float* amax_g, hipStream_t stream,
                            const RingFold& fold = RingFold{}) {
  GemmArgs a = dx_gemm_args(M, N, K, g8, sg, w8, dx, pre, g_scale, sg_used, amax_g, fold);
  launch_gemm_l<kKContig, kCross>(a, fmt_g, dtype_fmt(w8.dtype), stream);
}

// The column partials of a pre-quantized g for db (dec(g8) / sg is summed
// by the finalize); a high-precision g gets them from its quantize.
static void enqueue_db_colsum_pre(int64_t M, int64_t N, const uint8_t* g8, int32_t fmt_g,
                                  float* db_ws, hipStream_t stream) {
  if (N <= 0) return;
  dim3 grid((unsigned)((N + kColStrip - 1) / kColStrip),
            (unsigned)((M + kColRowsPerChunk - 1) / kColRowsPerChunk));
  if (fmt_g == FP8_E4M3)
    hipLaunchKernelGGL(colsum_fp8_kernel<kE4M3>, grid, dim3(kQThreads), 0, stream, g8, M, N, db_ws);
  else
    hipLaunchKernelGGL(colsum_fp8_kernel<kE5M2>, grid, dim3(kQThreads), 0, stream, g8, M, N, db_ws);
}

// The dW GEMM of a backward: dW = G8^T X8 / (sg sx), and db from the column
// partials in db_ws.  aux: snapshot a pre-quantized g's scale (see
// enqueue_dx_gemm).
static GemmArgs dw_gemm_args(int64_t M, int64_t N, int64_t K, const uint8_t* g8, const float* sg,
                             fp8_operand_t x8, void* dw, void* db, float* db_ws, bool pre, bool aux,
                             const float* g_scale, float* sg_used, float* amax_g,
                             const RingFold& fold) {
  GemmArgs a = {};
  a.fold[0] = fold;
  a.a = g8;  // G8 [M, N] as A(i = n, k = m): crosswise
  a.lda = N;
  a.b = reinterpret_cast<const uint8_t*>(x8.data);  // X8 [M, K] as B(j = k, k = m): crosswise
  a.ldb = K;
  a.Mc = N;
  a.Nc = K;
  a.Kc = M;
  a.c = reinterpret_cast<uint16_t*>(dw);
  a.ldc = K;
  a.scale_a = sg;
  a.scale_b = x8.scale;
  if (db) {
    a.db = reinterpret_cast<uint16_t*>(db);
    a.db_ws = db_ws;
    a.db_R = (int32_t)((M + kColRowsPerChunk - 1) / kColRowsPerChunk);
    a.db_scale = pre ? sg : nullptr;
  }
  if (pre && aux) {
    a.aux_scale_dst0 = sg_used;
    a.aux_scale_src0 = g_scale;
    a.aux_amax_dst0 = amax_g;
  }
  finish_gemm_args(a);
  return a;
}

static void enqueue_dw_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* g8, const float* sg,
                            int32_t fmt_g, fp8_operand_t x8, void* dw, void* db, float* db_ws,
                            bool pre, bool aux, const float* g_scale, float* sg_used,
                            float* amax_g, hipStream_t stream, const RingFold& fold = RingFold{}) {
  GemmArgs a = dw_gemm_args(M, N, K, g8, sg, x8, dw, db, db_ws, pre, aux, g_scale, sg_used, amax_g,
                            fold);
  launch_gemm_l<kCross, kCross>(a, fmt_g, dtype_fmt(x8.dtype), stream);
}

static int check_dx_operands(int64_t M, int64_t N, int64_t K, fp8_operand_t w8, const void* dx) {
  if (!is_f8(w8.dtype)) return FP8_ERR_DTYPE;
  if ((N * K > 0 && !w8.data) || !w8.scale) return FP8_ERR_NULL;
  if (M * K > 0 && !dx) return FP8_ERR_NULL;
  return FP8_OK;
}

static int check_dw_operands(int64_t M, int64_t N, int64_t K, fp8_operand_t x8, const void* dw,
                             const void* db, const float* db_ws) {
  if (!is_f8(x8.dtype)) return FP8_ERR_DTYPE;
  if ((M * K > 0 && !x8.data) || !x8.scale) return FP8_ERR_NULL;
  if (N * K > 0 && !dw) return FP8_ERR_NULL;
  if (db && M > 0 && !db_ws) return FP8_ERR_NULL;
  return FP8_OK;
}

// One event per device for the fork of fp8_linear_bwd, created on first
// use.  Record and wait happen under one lock, so a wait always refers to
// the record made just before it by the same call.
static std::mutex g_fork_mu;
static hipEvent_t g_fork_ev[64];

static int fork_after(hipStream_t from, hipStream_t to) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FP8_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_fork_mu);
  if (!g_fork_ev[dev] && hipEventCreateWithFlags(&g_fork_ev[dev], hipEventDisableTiming) != hipSuccess) {
    g_fork_ev[dev] = nullptr;
    return FP8_ERR_HIP;
  }
  if (hipEventRecord(g_fork_ev[dev], from) != hipSuccess) return FP8_ERR_HIP;
  if (hipStreamWaitEvent(to, g_fork_ev[dev], 0) != hipSuccess) return FP8_ERR_HIP;
  return FP8_OK;
}

int fp8_linear_bwd_dx(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                      fp8_ring_t* ring_g, fp8_operand_t w8, void* dx, uint8_t* g8_out,
                      float* sg_used, float* amax_g, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return FP8_ERR_SHAPE;
  const uint8_t* g8 = nullptr;
  const float* sg = nullptr;
  bool pre = false;
  int st = bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, true, nullptr, stream, &g8,
                       &sg, &pre);
  if (st) return st;
  if ((st = check_dx_operands(M, N, K, w8, dx))) return st;
  RingFold fold = {};
  bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, false, nullptr, stream, &g8, &sg, &pre,
              &fold);
  enqueue_dx_gemm(M, N, K, g8, sg, fmt_g, w8, dx, pre, g.scale, sg_used, amax_g, stream, fold);
  return hip_status();
}

int fp8_linear_bwd_dw(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                      fp8_ring_t* ring_g, fp8_operand_t x8, void* dw, void* db, float* db_ws,
                      uint8_t* g8_out, float* sg_used, float* amax_g, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return FP8_ERR_SHAPE;
  const uint8_t* g8 = nullptr;
  const float* sg = nullptr;
  bool pre = false;
  int st = bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, true, nullptr, stream, &g8,
                       &sg, &pre);
  if (st) return st;
  if ((st = check_dw_operands(M, N, K, x8, dw, db, db_ws))) return st;

  ColsumSpec cs = {M, N, db_ws};
  const bool want_db = db != nullptr && M > 0;
  RingFold fold = {};
  bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, false, want_db ? &cs : nullptr,
              stream, &g8, &sg, &pre, &fold);
  if (want_db && pre) enqueue_db_colsum_pre(M, N, g8, fmt_g, db_ws, stream);
  enqueue_dw_gemm(M, N, K, g8, sg, fmt_g, x8, dw, db, db_ws, pre, true, g.scale, sg_used, amax_g,
                  stream, fold);
  return hip_status();
}

int fp8_linear_bwd_dw_noalloc(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                              fp8_ring_t* ring_g, fp8_operand_t x8, void* dw, void* db,
                              uint8_t* g8_out, float* sg_used, float* amax_g, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return FP8_ERR_SHAPE;
  const bool want_db = db != nullptr && M > 0;
  if (want_db && fp8_db_workspace_bytes(M, N) > (size_t)FP8_NOALLOC_WS_MAX) return FP8_ERR_SHAPE;
  const uint8_t* g8 = nullptr;
  const float* sg = nullptr;
  bool pre = false;
  int st = bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, true, nullptr, stream, &g8,
                       &sg, &pre);
  if (st) return st;
  float* ws = nullptr;
  if (want_db && !(ws = scratch_dev())) return FP8_ERR_HIP;
  if ((st = check_dw_operands(M, N, K, x8, dw, db, ws))) return st;
  // from here on exactly fp8_linear_bwd_dw with ws as its workspace
  ColsumSpec cs = {M, N, ws};
  RingFold fold = {};
  bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, false, want_db ? &cs : nullptr,
              stream, &g8, &sg, &pre, &fold);
  if (want_db && pre) enqueue_db_colsum_pre(M, N, g8, fmt_g, ws, stream);
  enqueue_dw_gemm(M, N, K, g8, sg, fmt_g, x8, dw, db, ws, pre, true, g.scale, sg_used, amax_g,
                  stream, fold);
  return hip_status();
}

int fp8_linear_bwd(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                   fp8_ring_t* ring_g, fp8_operand_t x8, fp8_operand_t w8, void* dx, void* dw,
                   void* db, float* db_ws, uint8_t* g8_out, float* sg_used, float* amax_g,
                   hipStream_t stream, hipStream_t stream_dw) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return FP8_ERR_SHAPE;
  const uint8_t* g8 = nullptr;
  const float* sg = nullptr;
  bool pre = false;
  int st = bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, true, nullptr, stream, &g8,
                       &sg, &pre);
  if (st) return st;
  if ((st = check_dx_operands(M, N, K, w8, dx))) return st;
  if ((st = check_dw_operands(M, N, K, x8, dw, db, db_ws))) return st;

  ColsumSpec cs = {M, N, db_ws};
  const bool want_db = db != nullptr && M > 0;
  RingFold fold = {};  // left to the dX GEMM, which runs on stream after the quantize
  bwd_prepare(M, N, g, fmt_g, ring_g, g8_out, sg_used, amax_g, false, want_db ? &cs : nullptr,
              stream, &g8, &sg, &pre, &fold);
  if (want_db && pre) enqueue_db_colsum_pre(M, N, g8, fmt_g, db_ws, stream);
  if ((st = hip_status())) return st;
  if (stream_dw == stream) {
    // one stream: both GEMMs in one grouped launch where they qualify
    GemmArgs ax = dx_gemm_args(M, N, K, g8, sg, w8, dx, pre, g.scale, sg_used, amax_g, fold);
    GemmArgs aw = dw_gemm_args(M, N, K, g8, sg, x8, dw, db, db_ws, pre, false, g.scale, sg_used,
                               amax_g, RingFold{});
    if (launch_pair(ax, aw, fmt_g, dtype_fmt(w8.dtype), dtype_fmt(x8.dtype), stream))
      return hip_status();
  }
  if (stream_dw != stream && (st = fork_after(stream, stream_dw))) return st;
  // the dX GEMM snapshots a pre-quantized g's scale; the dW GEMM reads
  // g's own scale, so the two streams touch no common output.  dX is
  // enqueued first: a captured graph's replay dispatches ready nodes in
  // capture order, and the dX GEMM, which the next layer's backward waits
  // for, should take the CUs before the dW GEMM fills what it leaves (as
  // the eager streams do by themselves)
  enqueue_dx_gemm(M, N, K, g8, sg, fmt_g, w8, dx, pre, g.scale, sg_used, amax_g, stream, fold);
  enqueue_dw_gemm(M, N, K, g8, sg, fmt_g, x8, dw, db, db_ws, pre, false, g.scale, sg_used, amax_g,
                  stream_dw);
  return hip_status();
}

}  // extern "C"

int fp8_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, fp8_operand_t a, int32_t layout_a,
             int64_t lda, int64_t stride_a, fp8_operand_t b, int32_t layout_b, int64_t ldb,
             int64_t stride_b, fp8_operand_t bias, void* c, int64_t ldc, int64_t stride_c,
             hipStream_t stream) {
  if (batch < 0 || M < 0 || N < 0 || K < 0 || stride_a < 0 || stride_b < 0 || stride_c < 0)
    return FP8_ERR_SHAPE;
  if (batch > 65535) return FP8_ERR_SHAPE;
  if (!is_fp8_dtype(a.dtype) || !is_fp8_dtype(b.dtype)) return FP8_ERR_DTYPE;
  if ((layout_a != FP8_K_CONTIG && layout_a != FP8_K_STRIDED) ||
      (layout_b != FP8_K_CONTIG && layout_b != FP8_K_STRIDED))
    return FP8_ERR_DTYPE;
  int bias_kind = kBiasNone;
  if (bias.data) {
    if (bias.dtype == FP8_DT_BF16) bias_kind = kBiasBF16;
    else if (bias.dtype == FP8_DT_E4M3) bias_kind = kBiasE4M3;
    else if (bias.dtype == FP8_DT_E5M2) bias_kind = kBiasE5M2;
    else return FP8_ERR_DTYPE;
    if (bias_kind != kBiasBF16 && !bias.scale) return FP8_ERR_NULL;
  }
  if (!a.scale || !b.scale) return FP8_ERR_NULL;
  if (batch == 0 || M == 0 || N == 0) return FP8_OK;
  // leading dimensions, slice extents and non-overlapping output slices
  const int64_t a_rows = layout_a == FP8_K_CONTIG ? M : K, a_inner = layout_a == FP8_K_CONTIG ? K : M;
  const int64_t b_rows = layout_b == FP8_K_CONTIG ? N : K, b_inner = layout_b == FP8_K_CONTIG ? K : N;
  if (lda < a_inner || ldb < b_inner || ldc < N) return FP8_ERR_SHAPE;
  if (!mul_ok(a_rows, lda) || !mul_ok(b_rows, ldb) || !mul_ok(M, ldc) || !mul_ok(batch, stride_a) ||
      !mul_ok(batch, stride_b) || !mul_ok(batch, stride_c))
    return FP8_ERR_SHAPE;
  if (batch > 1 && stride_c < (M - 1) * ldc + N) return FP8_ERR_SHAPE;
  if (K > 0 && (!a.data || !b.data)) return FP8_ERR_NULL;
  if (!c) return FP8_ERR_NULL;

  GemmArgs g = {};
  g.a = reinterpret_cast<const uint8_t*>(a.data);
  g.lda = lda;
  g.b = reinterpret_cast<const uint8_t*>(b.data);
  g.ldb = ldb;
  g.Mc = M;
  g.Nc = N;
  g.Kc = K;
  g.c = reinterpret_cast<uint16_t*>(c);
  g.ldc = ldc;
  g.scale_a = a.scale;
  g.scale_b = b.scale;
  g.bias = bias.data;
  g.bias_kind = bias_kind;
  g.bias_scale = bias.scale;
  g.bsa = stride_a;
  g.bsb = stride_b;
  g.bsc = stride_c;
  g.batch = (int32_t)batch;
  finish_gemm_args(g);
  const int fa = dtype_fmt(a.dtype), fb = dtype_fmt(b.dtype);
  if (layout_a == FP8_K_CONTIG && layout_b == FP8_K_CONTIG)
    launch_gemm_l<kKContig, kKContig>(g, fa, fb, stream);
  else if (layout_a == FP8_K_CONTIG)
    launch_gemm_l<kKContig, kCross>(g, fa, fb, stream);
  else if (layout_b == FP8_K_CONTIG)
    launch_gemm_l<kCross, kKContig>(g, fa, fb, stream);
  else
    launch_gemm_l<kCross, kCross>(g, fa, fb, stream);
  return hip_status();
}

int fp8_gemm_fp8out(int64_t M, int64_t N, int64_t K, fp8_operand_t a, fp8_operand_t b,
                    fp8_operand_t bias, int32_t fmt_out, fp8_ring_t* ring_out, uint8_t* c8,
                    float* scale_used, float* amax_out, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0) return FP8_ERR_SHAPE;
  if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return FP8_ERR_SHAPE;
  if (!is_fp8_dtype(a.dtype) || !is_fp8_dtype(b.dtype) || !valid_fmt(fmt_out)) return FP8_ERR_DTYPE;
  int bias_kind = kBiasNone;
  if (bias.data) {
    if (bias.dtype == FP8_DT_BF16) bias_kind = kBiasBF16;
    else if (bias.dtype == FP8_DT_E4M3) bias_kind = kBiasE4M3;
    else if (bias.dtype == FP8_DT_E5M2) bias_kind = kBiasE5M2;
    else return FP8_ERR_DTYPE;
    if (bias_kind != kBiasBF16 && !bias.scale) return FP8_ERR_NULL;
  }
  if (!a.scale || !b.scale || !scale_used || !ring_out) return FP8_ERR_NULL;
  int st = check_ring(ring_out);
  if (st) return st;
  if (check_alias(ring_out, scale_used) || check_alias(ring_out, amax_out)) return FP8_ERR_RING;
  if ((st = check_seed_capture(ring_out, stream))) return st;
  if (M == 0 || N == 0) return FP8_OK;
  if (K > 0 && (!a.data || !b.data)) return FP8_ERR_NULL;
  if (!c8) return FP8_ERR_NULL;
  // the one kernel this runs on: 16-byte operand and code pieces that never
  // straddle a row end, byte offsets that fit a buffer descriptor
  if (K % 16 != 0 || N % 16 != 0 || !aligned16(a.data) || !aligned16(b.data) || !aligned16(c8) ||
      (M + 256) * K >= (1LL << 31) || (N + 256) * K >= (1LL << 31))
    return FP8_ERR_SHAPE;

  GemmArgs g = {};
  g.a = reinterpret_cast<const uint8_t*>(a.data);
  g.lda = K;
  g.b = reinterpret_cast<const uint8_t*>(b.data);
  g.ldb = K;
  g.Mc = M;
  g.Nc = N;
  g.Kc = K;
  g.ldc = N;
  g.scale_a = a.scale;
  g.scale_b = b.scale;
  g.bias = bias.data;
  g.bias_kind = bias_kind;
  g.bias_scale = bias.scale;
  g.batch = 1;
  g.c8 = c8;
  g.oring = reinterpret_cast<RingHdr*>(ring_out->dev);
  g.ohist = reinterpret_cast<float*>(reinterpret_cast<char*>(ring_out->dev) + sizeof(RingHdr));
  g.ohist_len = ring_out->hist_len;
  g.oscale_used = scale_used;
  g.oamax = amax_out;
  finish_gemm_args(g);
  const int fa = dtype_fmt(a.dtype), fb = dtype_fmt(b.dtype);
  const bool e4 = fmt_out == FP8_E4M3;
  if (!ring_out->seeded) {
    // seeding call: an amax pass leaves max |y| in the ring header, then the
    // converting pass quantizes with S(max |y|) and folds it into the window
    launch_fp8out<kEpiAmax, kE4M3>(g, fa, fb, stream);
    if (e4) launch_fp8out<kEpiFp8Seed, kE4M3>(g, fa, fb, stream);
    else launch_fp8out<kEpiFp8Seed, kE5M2>(g, fa, fb, stream);
    ring_out->seeded = 1;
  } else {
    // steady state: the blocks end without an election and a one-wave
    // launch folds the ring after the GEMM (a window longer than one wave
    // keeps the last-block fold)
    g.odefer = can_defer(ring_out) ? 1 : 0;
    if (e4) launch_fp8out<kEpiFp8Ring, kE4M3>(g, fa, fb, stream);
    else launch_fp8out<kEpiFp8Ring, kE5M2>(g, fa, fb, stream);
    if (g.odefer)
      hipLaunchKernelGGL(ring_fold_kernel, dim3(1), dim3(64), 0, stream,
                         fold_of(ring_out, fmt_out, amax_out));
  }
  return hip_status();
}
