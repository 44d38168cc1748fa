/*
 * fp8linear.h -- C ABI of the MI355X (gfx950) FP8 linear-layer hot path.
 *
 * One library, libfp8linear.so, hand-written HIP for CDNA4.  Four entry
 * points do the work of one FP8 linear layer in training (fp8_linear_bwd
 * below runs the two backward ones from one quantized G on two streams):
 *
 *   fp8_quantize        per-tensor quantize with on-device amax and the
 *                       delayed-scaling ring finalize in the same launch
 *   fp8_linear_fwd      quantize X and W (unless pre-quantized), then
 *                       Y = X8 W8^T / (sx sw) + bias
 *   fp8_linear_bwd_dx   quantize G (unless pre-quantized), then
 *                       dX = G8 W8 / (sg sw)
 *   fp8_linear_bwd_dw   quantize G (unless pre-quantized), then
 *                       dW = G8^T X8 / (sg sx) and optionally db = sum_m G
 *
 * Sources (AstrAI commit-log pages, cited by commit and page path):
 *   [P1] commit 2eeac02d, page tests/extension
 *   [P2] commit 2eeac02d, page csrc
 *   [P3] commit 057c0d33, page astrai/extension/ops
 *   [P4] commit 4019ddac, page astrai
 *   [P5] commit 3e57cc80, page astrai/extension/fp8.py
 *   [OCP] OCP 8-bit Floating Point Specification (OFP8) rev 1.0
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Matrices are row-major and contiguous: X [M,K], W [N,K], Y [M,N],
 *   G [M,N], dX [M,K], dW [N,K], bias/db [N].  M = tokens, K = in features,
 *   N = out features.  Any M, N, K >= 0 is computed correctly (ragged tails
 *   are guarded); the fast paths want multiples of 128 and 16-byte aligned
 *   buffers.
 * - Every pointer except the fp8_ring_t / fp8_operand_t structs themselves
 *   is a DEVICE pointer.  The caller allocates and owns every buffer; the
 *   library never allocates, frees or synchronizes, and enqueues all work on
 *   the given stream (fp8_linear_bwd: on its two streams, ordered by one
 *   HIP event per device that the library keeps).  A NULL optional pointer
 *   means "absent" ([P2] entry on null defaults for optional pointer
 *   members).
 * - Outputs must not alias inputs.  Scale outputs must not alias a ring's
 *   own scale slot (the snapshot rule of [P3]: the GEMM dequantizes with the
 *   scale the quantize used, not with the one the ring publishes next).
 * - Validation completes before anything is enqueued: on any error status
 *   nothing runs and nothing is modified (ring->seeded included).
 * - Errors: FP8_OK = 0; otherwise one of fp8_status_t.  FP8_ERR_HIP means a
 *   launch failed after validation (hipGetLastError); work enqueued before
 *   the failing launch may have run.
 */
#ifndef FP8LINEAR_H
#define FP8LINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8_ABI_VERSION 5
#define FP8_RING_MAX_HIST 1024

typedef enum {
  FP8_OK = 0,
  FP8_ERR_NULL = 1,   /* a required pointer is NULL */
  FP8_ERR_SHAPE = 2,  /* a size is negative or a byte count overflows int64 */
  FP8_ERR_DTYPE = 3,  /* unknown format/dtype enum, or an fp8 operand whose
                         format does not match the call's format ([P3] entry
                         validating the fmt enum; [P1] pre-quantized operands
                         must match fmt) */
  FP8_ERR_RING = 4,   /* ring hist_len outside [1, 1024], dev NULL or not
                         256-byte aligned, a scale output aliasing it, or an
                         unseeded ring used on a stream under graph capture */
  FP8_ERR_HIP = 5     /* a kernel launch failed */
} fp8_status_t;

/* Formats: OCP E4M3 (max 448, no inf) and E5M2 (max 57344) [OCP]. */
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format_t;

/* Element types of tensors crossing the boundary. */
typedef enum {
  FP8_DT_F32 = 0,
  FP8_DT_F16 = 1,
  FP8_DT_BF16 = 2,
  FP8_DT_E4M3 = 3,
  FP8_DT_E5M2 = 4
} fp8_dtype_t;

/*
 * An operand that is either high precision (F32/F16/BF16: the call
 * quantizes it) or already quantized (E4M3/E5M2 matching the call's format:
 * the call skips its quantize, [P3] entry on g/x/w arriving bf16 or
 * pre-quantized).  scale: device float, the QUANTIZATION multiplier s of a
 * pre-quantized operand (q ~ x * s; the GEMM multiplies by 1/s); required
 * iff dtype is fp8, ignored otherwise.
 */
typedef struct {
  const void* data;
  int32_t dtype;
  const float* scale;
} fp8_operand_t;

/*
 * Delayed-scaling state of one operand ([P1] entries on finalizing scale
 * rings in the quantize kernel and on one ring per operand; [P3] entry on
 * the scale snapshot).  Host struct owned by the caller.
 *   dev       device buffer of fp8_ring_bytes(hist_len) bytes, 256-byte
 *             aligned: a 128-byte header {float scale; u32 top_count;
 *             u32 top_amax; u32 idx; u32 hist_len; u32 seeded; ...}, 64
 *             election groups of 128 bytes {u32 count; ...; u32 amax; ...}
 *             that collect a launch's block maxima for the fold (all zero
 *             between calls), then float hist[hist_len].
 *   hist_len  H, 1..1024.
 *   seeded    host mirror, 0 until the first quantize through the ring has
 *             been enqueued.  That first quantize seeds the scale from its
 *             own amax (two passes over the input); later ones run one pass
 *             with the scale published by the previous step.
 * Byte-copying dev plus seeded resumes the scale sequence exactly.  A ring
 * must not be used by two calls that may run concurrently.
 * Graph capture: whether a call seeds is decided on the host when it is
 * issued, so a ring must be seeded (one call through it enqueued) before any
 * call on it is captured; a call that would seed a ring on a capturing
 * stream returns FP8_ERR_RING with nothing enqueued.
 */
typedef struct {
  void* dev;
  int32_t hist_len;
  int32_t seeded;
} fp8_ring_t;

/* Library ABI version (FP8_ABI_VERSION). */
int fp8_abi_version(void);

/* Identity of the sources the library was built from: the SHA-256 (hex) of
 * its HIP sources and this header, fixed at build time ("unknown" when the
 * build did not supply it).  Static string, never NULL. */
const char* fp8_source_hash(void);

/* Static description of a status code. */
const char* fp8_status_str(int status);

/* Bytes of a ring's device buffer: 8320 + 4 * hist_len (0 if out of range). */
size_t fp8_ring_bytes(int32_t hist_len);

/*
 * Bind dev to ring and enqueue its reset: scale = 1, hist = 0, idx = 0,
 * every election counter and max = 0; sets ring->hist_len and
 * ring->seeded = 0.
 * Errors: FP8_ERR_NULL (ring or dev NULL), FP8_ERR_RING (hist_len out of
 * range, dev misaligned), FP8_ERR_HIP.
 */
int fp8_ring_init(fp8_ring_t* ring, void* dev, int32_t hist_len, hipStream_t stream);

/*
 * Per-tensor quantize ([P3] entries on the quantize primitive templated on
 * bf16/fp16/fp32 input and on fp32-domain amax; [P1] entry on the ring
 * finalize in the kernel's last block; [P4] entry on the atomic ticket).
 *
 *   x          device, n elements of in_dtype (F32, F16 or BF16).
 *   n          element count, >= 0 (n = 0 folds amax = 0 into the ring).
 *   fmt        FP8_E4M3 or FP8_E5M2.
 *   q          device, n bytes out: q_i = enc_fmt(fl32(x_i * s_used)),
 *              round-to-nearest-even, saturating to +-max; NaN -> 0x7F|sign.
 *   ring       NULL: dynamic scaling, s_used = fmt_max / amax(x) (two
 *              passes).  Otherwise delayed scaling: s_used = the ring's
 *              current scale (seeded from amax(x) on the ring's first use);
 *              then amax(x) is folded into hist[idx], idx advanced and
 *              fmt_max / max(hist) published as the next scale (kept
 *              unchanged if that max is 0 or not finite).  The fold runs in
 *              a one-wave launch after the converting launch when the ring
 *              is seeded and H <= 64 (the converting blocks only leave their
 *              maxima in the election groups), otherwise in the converting
 *              launch's last block, elected by atomic tickets; the results
 *              are the same bits either way.
 *   scale_used device float out, required: the s the bytes were made with.
 *   amax_out   device float out: max |x_i| over the input values.
 *              Required when ring is NULL (it is also the accumulator),
 *              optional otherwise.
 */
int fp8_quantize(const void* x, int32_t in_dtype, int64_t n, int32_t fmt, uint8_t* q,
                 fp8_ring_t* ring, float* scale_used, float* amax_out, hipStream_t stream);

/* Output orientation of fp8_quantize_2d ([P4] entry on splitting the quantize
 * into transposed and dual variants with a layout enum). */
typedef enum {
  FP8_QUANT_ROWS = 0,        /* q [rows, cols] only (as fp8_quantize) */
  FP8_QUANT_TRANSPOSED = 1,  /* qt [cols, rows] only */
  FP8_QUANT_DUAL = 2         /* both */
} fp8_quant_layout_t;

/*
 * Per-tensor quantize of a row-major x [rows, cols] with transposed and dual
 * outputs ([P4] entry on the quantize bindings split into transposed and
 * dual variants, tested for byte equality between orientations): the codes,
 * scale, amax and ring update are exactly those of fp8_quantize on the same
 * rows * cols elements; q receives them row-major, qt transposed,
 * qt[c * rows + r] = q[r * cols + c].  A transposed copy of X8 or G8 lets
 * fp8_gemm run the weight gradient with both operands k-contiguous.
 *
 *   layout   FP8_QUANT_ROWS, FP8_QUANT_TRANSPOSED or FP8_QUANT_DUAL.
 *   q        device [rows, cols] bytes out; required unless TRANSPOSED.
 *   qt       device [cols, rows] bytes out; required unless ROWS.
 *   x, in_dtype, fmt, ring, scale_used, amax_out: as fp8_quantize.
 * Errors: as fp8_quantize; FP8_ERR_DTYPE for an unknown layout.
 */
int fp8_quantize_2d(const void* x, int32_t in_dtype, int64_t rows, int64_t cols, int32_t fmt,
                    int32_t layout, uint8_t* q, uint8_t* qt, fp8_ring_t* ring, float* scale_used,
                    float* amax_out, hipStream_t stream);

/*
 * Two per-tensor quantizes in one call, each exactly as fp8_quantize with
 * its own input, output, ring, scale_used and amax_out, in one format.  When
 * both inputs have the same dtype and both rings are seeded, the two are one
 * kernel launch (a linear layer's X and W: the fixed latency of one tensor's
 * loads and ring finalize overlaps the other's); otherwise they are enqueued
 * one after the other.  fp8_linear_fwd uses the same path for a high-precision
 * X and W ([P1] entry on finalizing scale rings inside the quantize kernels
 * with no extra launches per linear layer).
 *
 *   x0, dtype0, n0, q0, ring0, scale_used0, amax_out0   first tensor
 *   x1, dtype1, n1, q1, ring1, scale_used1, amax_out1   second tensor
 *   fmt                                                 format of both
 * Errors: as fp8_quantize for either tensor; FP8_ERR_RING if both rings are
 * the same ring.  Nothing is enqueued on error.
 */
int fp8_quantize_pair(const void* x0, int32_t dtype0, int64_t n0, uint8_t* q0, fp8_ring_t* ring0,
                      float* scale_used0, float* amax_out0, const void* x1, int32_t dtype1,
                      int64_t n1, uint8_t* q1, fp8_ring_t* ring1, float* scale_used1,
                      float* amax_out1, int32_t fmt, hipStream_t stream);

/*
 * Forward of one FP8 linear layer ([P1] entries on optional ring arguments,
 * pre-quantized w8 with amax_w = 0, and the bias fused into the epilogue
 * with bias_scale; [P4] entry on the bias added in fp32 before the single
 * bf16 rounding; [P3] entry on bf16 output).
 *
 *   x        [M,K]: F32/F16/BF16 (quantized here with ring_x into x8_out)
 *            or fp8 of format fmt with its scale.
 *   w        [N,K]: same choices, ring_w, w8_out.
 *   bias     [N]: data NULL = no bias; BF16 values; or fp8 codes (E4M3 or
 *            E5M2) with scale = bias_scale, contributing dec(b8)/bias_scale.
 *   fmt      format of X8 and W8.
 *   y        [M,N] bf16 out: RNE_bf16(sum_k x8 w8 / (sx sw) + bias), with
 *            fp32 accumulation.
 *   x8_out   [M,K] bytes out, required when x is high precision (keep it
 *            with sx_used for the backward: [P3] entry on the forward's
 *            scale reaching the backward).  w8_out likewise for w.
 *   sx_used  device float out: the scale X8 was made with; required when x
 *            is high precision, optional (copied from x.scale) otherwise.
 *            sw_used likewise.
 *   amax_x   device float out, max |x|; required when x is high precision
 *            and ring_x is NULL (dynamic), else optional; 0 is written for a
 *            pre-quantized operand.  amax_w likewise.
 */
int fp8_linear_fwd(int64_t M, int64_t N, int64_t K, fp8_operand_t x, fp8_operand_t w,
                   fp8_operand_t bias, int32_t fmt, fp8_ring_t* ring_x, fp8_ring_t* ring_w,
                   void* y, uint8_t* x8_out, uint8_t* w8_out, float* sx_used, float* sw_used,
                   float* amax_x, float* amax_w, hipStream_t stream);

/*
 * Input gradient ([P3] entries on bf16 grad outputs and on the forward's
 * scale reused by the backward; [P2] entry on the crosswise-B operand).
 *
 *   g        [M,N]: F32/F16/BF16 (quantized here with ring_g into g8_out in
 *            format fmt_g) or fp8 of format fmt_g with its scale.
 *   w8       [N,K] fp8 (E4M3 or E5M2) with its scale (sw_used of the
 *            forward).
 *   dx       [M,K] bf16 out: RNE_bf16(sum_n g8 w8 / (sg sw)).
 *   g8_out, sg_used, amax_g: as x8_out / sx_used / amax_x of the forward.
 */
int fp8_linear_bwd_dx(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                      fp8_ring_t* ring_g, fp8_operand_t w8, void* dx, uint8_t* g8_out,
                      float* sg_used, float* amax_g, hipStream_t stream);

/*
 * Bytes of the fp32 workspace fp8_linear_bwd_dw needs for db:
 * 4 * N * ceil(M / 32).
 */
size_t fp8_db_workspace_bytes(int64_t M, int64_t N);

/*
 * Weight and bias gradients ([P4] entry on computing the bias column sum
 * only when the bias needs a gradient; [P3] entry on a pre-quantized g being
 * dequantized before that sum; [P1] entry on crosswise A and B operands).
 *
 *   g        [M,N] as in fp8_linear_bwd_dx.
 *   x8       [M,K] fp8 (E4M3 or E5M2) with its scale (sx_used of the
 *            forward).
 *   dw       [N,K] bf16 out: RNE_bf16(sum_m g8 x8 / (sg sx)).
 *   db       [N] bf16 out or NULL.  When g is high precision, db sums the
 *            g values as given; when g is pre-quantized, it sums
 *            dec(g8)/sg.  fp32 accumulation, one bf16 rounding.
 *   db_ws    device fp32 workspace of fp8_db_workspace_bytes(M, N) bytes,
 *            required iff db is not NULL and M > 0; contents on entry are
 *            ignored.
 *   g8_out, sg_used, amax_g: as in fp8_linear_bwd_dx.
 *
 * Calling order within one backward: call fp8_linear_bwd_dw with the
 * high-precision g first (one quantize, one ring fold, db from g itself),
 * then fp8_linear_bwd_dx with g = {g8_out, fp8 dtype, sg_used}.
 */
int fp8_linear_bwd_dw(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                      fp8_ring_t* ring_g, fp8_operand_t x8, void* dw, void* db, float* db_ws,
                      uint8_t* g8_out, float* sg_used, float* amax_g, hipStream_t stream);

/* Bytes of the device array fp8_linear_bwd_dw_noalloc keeps per GPU. */
#define FP8_NOALLOC_WS_MAX (8 << 20)

/*
 * fp8_linear_bwd_dw for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and kernels without db_ws.  The
 * db column partials live in a static device array of FP8_NOALLOC_WS_MAX
 * bytes (8 MiB) that the library holds on each GPU it runs on until the
 * process ends; this entry point calls no hipMalloc, hipFree or allocating
 * routine.  The array's device address is looked up once per GPU on the
 * first call there (hipGetSymbolAddress, with that GPU current); the stream
 * must belong to the current device.
 *
 *   all arguments   as fp8_linear_bwd_dw.
 * The partials a call writes are all read by that call, so the array needs
 * no clearing; every call on one GPU shares it, so two calls that may
 * overlap on one GPU (two streams, or two host threads) race on it and must
 * be ordered by the caller.
 * Errors: as fp8_linear_bwd_dw; FP8_ERR_SHAPE when db is wanted and
 * fp8_db_workspace_bytes(M, N) exceeds FP8_NOALLOC_WS_MAX; FP8_ERR_HIP when
 * the array's address cannot be looked up (nothing is enqueued then).
 */
int fp8_linear_bwd_dw_noalloc(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                              fp8_ring_t* ring_g, fp8_operand_t x8, void* dw, void* db,
                              uint8_t* g8_out, float* sg_used, float* amax_g, hipStream_t stream);

/*
 * Both gradients of one linear from one quantized G, the weight gradient on
 * a second stream ([P3] entries on the backward's bf16 grad outputs and on
 * the forward's scales reused there; [P4] entry on the bias column sum).
 * The results are those of fp8_linear_bwd_dw(g, ...) followed by
 * fp8_linear_bwd_dx(g8, ...), bit for bit; only the streams differ:
 *
 *   on stream:     the quantize of g (with db's column partials when db is
 *                  wanted), then the dX GEMM;
 *   on stream_dw:  after the quantize (an event recorded on stream and
 *                  waited on by stream_dw), the dW GEMM and db.
 *
 * The dX chain of a backward (the critical path: dX feeds the layer below)
 * then never waits for a dW GEMM, which fills the CUs the dX work leaves
 * idle.  stream_dw == stream runs everything on stream, the dX and dW GEMMs
 * as one grouped launch (both problems' tiles in one grid, the longer tiles
 * first) when G8 is e5m2, W8 and X8 are e4m3 and each GEMM alone would run
 * on one of the 8-wave tiled kernels; otherwise one after the other.  The
 * results are the same bits either way.
 *
 *   g, ring_g, g8_out, sg_used, amax_g: as in fp8_linear_bwd_dw.
 *   x8, dw, db, db_ws: as in fp8_linear_bwd_dw (dw, db written on stream_dw;
 *            db_ws read there).
 *   w8, dx:  as in fp8_linear_bwd_dx (dx written on stream).
 *
 * The dW GEMM, running on stream_dw, reads g8_out (or a pre-quantized g),
 * sg_used, x8 with its scale and db_ws whenever stream_dw reaches it.  The
 * caller orders later uses of dw and db, and any rewrite of those inputs
 * (say g8_out or db_ws reused by the next layer's backward on stream),
 * after stream_dw, for example with an event recorded on stream_dw; under
 * graph capture it joins stream_dw back to the capturing stream before the
 * capture ends.  The library keeps one event per device for the fork
 * (created on first use, held until the process ends); record and wait run
 * under one lock, so calls from several host threads stay correct.
 * Errors as for the other entry points; FP8_ERR_HIP also covers a failed
 * event record or wait.
 */
int fp8_linear_bwd(int64_t M, int64_t N, int64_t K, fp8_operand_t g, int32_t fmt_g,
                   fp8_ring_t* ring_g, fp8_operand_t x8, fp8_operand_t w8, void* dx, void* dw,
                   void* db, float* db_ws, uint8_t* g8_out, float* sg_used, float* amax_g,
                   hipStream_t stream, hipStream_t stream_dw);

/* Storage of a GEMM operand, with its contraction index k ([P4] entry on 3D
 * operands and transposed views folding into the layout tag):
 *   FP8_K_CONTIG   element (r, k) at p[r * ld + k]  (rows of k-contiguous codes)
 *   FP8_K_STRIDED  element (r, k) at p[k * ld + r]  (the transposed view of such
 *                  rows; read through the LDS transpose, no copy) */
typedef enum { FP8_K_CONTIG = 0, FP8_K_STRIDED = 1 } fp8_layout_t;

/*
 * Batched FP8 GEMM on pre-quantized operands ([P4] entry on the fp8 matmul
 * accepting 3D operands: batch slices by stride, size-1 batches broadcast
 * with stride 0, transposed views as a layout tag; [P4] entry on the bias
 * added in fp32 before the single bf16 rounding).  For z < batch:
 *
 *   C_z[i, j] = RNE_bf16( sum_k A_z(i, k) B_z(j, k) / (sa sb) + bias[j] ),
 *
 * fp32 accumulation, i < M, j < N, k < K.
 *
 *   a         fp8 codes (E4M3 or E5M2) with their device scale sa; A_z is the
 *             M x K operand at a.data + z * stride_a in layout layout_a with
 *             leading dimension lda (>= K for FP8_K_CONTIG, >= M otherwise).
 *   b         likewise, N x K, with layout_b, ldb, stride_b and scale sb.
 *   stride_a, stride_b   elements between batch slices; 0 broadcasts one
 *             slice to every z.
 *   bias      [N]: data NULL = none; BF16; or fp8 codes with scale =
 *             bias_scale (dec(b8)/bias_scale).  The same for every slice.
 *   c         bf16 out: C_z at c + z * stride_c, leading dimension ldc >= N;
 *             when batch > 1, stride_c >= (M - 1) * ldc + N (slices must not
 *             overlap).
 * Errors: FP8_ERR_SHAPE (a negative size, a leading dimension or stride too
 * small, a byte count overflowing int64, batch > 65535), FP8_ERR_DTYPE (a
 * non-fp8 operand, an unknown layout, a bad bias dtype), FP8_ERR_NULL (a
 * missing pointer or scale).  Nothing is enqueued on error.
 */
int fp8_gemm(int64_t batch, int64_t M, int64_t N, int64_t K, fp8_operand_t a, int32_t layout_a,
             int64_t lda, int64_t stride_a, fp8_operand_t b, int32_t layout_b, int64_t ldb,
             int64_t stride_b, fp8_operand_t bias, void* c, int64_t ldc, int64_t stride_c,
             hipStream_t stream);

/*
 * FP8-in / FP8-out GEMM ([P1] entry on the custom op for an FP8-in/FP8-out
 * GEMM on pre-quantized operands; [P1] entry on the fp8 bias dequantized
 * after the operand scaling and before any output quantization; [P3] entry
 * on dropping the fp8-output template parameter, after which every other
 * GEMM here writes bf16).  The forward layout, pre-quantized:
 *
 *   y[i, j] = sum_k A(i, k) B(j, k) / (sa sb) + bias[j]        (fp32)
 *   c8[i, j] = enc_fmt_out( fl32( y[i, j] * s_out ) )
 *
 * y is the fp32 value the bf16-output GEMMs round to bf16 (fp32
 * accumulation, one fma with the bias); enc is the quantize's conversion
 * (round to nearest even, saturating, NaN -> 0x7F | sign).  s_out comes from
 * the output's delayed-scaling ring exactly as fp8_quantize takes it: the
 * ring's current scale, or, on the ring's first use, S(max |y|) from an
 * extra amax pass over the same GEMM.  max |y| (over the M x N outputs) is
 * then folded into hist[idx], idx advanced and fmt_max / max(hist)
 * published as the next scale, as a quantize launch does: in the steady
 * state of a window of at most 64 entries by a one-wave launch that follows
 * the GEMM on the same stream (the GEMM's blocks only leave their maxima in
 * the ring's election groups), otherwise by the GEMM's last block.
 *
 *   a, b       fp8 codes (E4M3 or E5M2) with device scales: A [M,K] and
 *              B [N,K], both k-contiguous (rows of K codes).
 *   bias       [N]: data NULL = none; BF16; or fp8 codes with scale =
 *              bias_scale (dec(b8)/bias_scale).
 *   fmt_out    FP8_E4M3 or FP8_E5M2: the format of c8.
 *   ring_out   required: the output's scale ring (fp8_ring_init).
 *   c8         device [M,N] bytes out, 16-byte aligned.
 *   scale_used device float out, required: the s_out the codes were made
 *              with (dequantize c8 by 1/s_out).
 *   amax_out   device float out or NULL: max |y|.
 * Shapes: K and N multiples of 16, a, b and c8 16-byte aligned (one tiled
 * kernel runs it), else FP8_ERR_SHAPE; any M.  M or N = 0 does nothing.
 * Errors: as fp8_gemm, plus FP8_ERR_RING for an invalid ring or a
 * scale_used / amax_out inside the ring header.
 */
int fp8_gemm_fp8out(int64_t M, int64_t N, int64_t K, fp8_operand_t a, fp8_operand_t b,
                    fp8_operand_t bias, int32_t fmt_out, fp8_ring_t* ring_out, uint8_t* c8,
                    float* scale_used, float* amax_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8LINEAR_H */
