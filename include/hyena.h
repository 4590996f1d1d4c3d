/*
 * hyena.h -- C ABI of the MI355X (gfx950) Hyena order-N forward library.
 *
 * The operator (Hyena Hierarchy explainer, abeam-guide-lp.pages.dev, section
 * "Hyena 演算子の形"; paper digest, irregular6612.github.io, section
 * "방법 (Method)", framework figure):
 *
 *     z_1 = v,   z_{n+1} = x_n * (h_n conv z_n)  (n = 1..N),   y = z_{N+1}
 *
 * where "*" is the elementwise product and "conv" the causal long
 * convolution c[t] = sum_{k<=t} h[k] z[t-k] over the full length L
 * (homemade-llm "02. 3つの Hyena 演算子", section 4, causal FIR equation).
 * The convolution is evaluated by FFT with zero padding to at least 2L
 * (jisaku.com glossary "Hyena（ハイエナ）", section "計算効率"; gist.science
 * HyenaND summary, section "手法: HyenaND", boundary handling).  The filters
 * are generated implicitly as Window(t) * FFN(t/L, sin, cos) (jisaku.com
 * glossary, section "暗黙的畳み込みフィルタ").
 *
 * Conventions shared by every call:
 *   - Device pointers point to memory of the current HIP device; the caller
 *     allocates and frees all of it.  The library never allocates device
 *     memory and is reentrant; the only state it keeps across calls is the
 *     resident-workgroup count of a kernel, looked up once.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns; results are ready after the stream syncs.
 *     No call allocates, clears memory or synchronises, so the calls can be
 *     captured into a HIP graph and replayed.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and returned as a status; nothing is written in that case.  A failed
 *     kernel launch returns HYENA_ERR_HIP.  Device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses this ABI.
 *   - Activations v, x_n and y are contiguous [B][D][L] arrays (time
 *     fastest) in the I/O dtype; device pointers must be 16-byte aligned.
 *   - Test hook: the environment variable HYENA_FORCE_PATH ("single" or
 *     "fourstep") and HYENA_FOURSTEP_N1 (a power of two) override the
 *     planner.  Both the spectrum and the forward read them at each call,
 *     so set them identically for both.
 */
#ifndef HYENA_MI355X_H
#define HYENA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HYENA_OK = 0,
  HYENA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  HYENA_ERR_SHAPE = 2,       /* a size is <= 0 or out of the supported range     */
  HYENA_ERR_UNSUPPORTED = 3, /* a valid request the library does not implement   */
  HYENA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned          */
  HYENA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
  HYENA_ERR_ALIAS = 6,       /* the output overlaps an input                     */
  HYENA_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed       */
} hyena_status;

typedef enum { HYENA_FP32 = 0, HYENA_BF16 = 1 } hyena_dtype;

typedef enum { HYENA_PATH_SINGLE = 1, HYENA_PATH_FOURSTEP = 2 } hyena_path;

/* Limits of the library. */
#define HYENA_MAX_ORDER 8          /* N in 1..8                                 */
#define HYENA_MAX_L (1LL << 22)    /* L in 1..2^22                              */
#define HYENA_MAX_FREQ 16          /* K in 0..16 (positional features 1+2K)     */

/*
 * Implicit filter generator weights (jisaku.com glossary, section
 * "暗黙的畳み込みフィルタ"; paper digest figure, HyenaFilter node).  All device
 * pointers, fp32, row-major [out][in]:
 *   W1 [H][1+2K], b1 [H]; W2 [H][H], b2 [H]; W3 [N*D][H], b3 [N*D]; alpha [D].
 * b1, b2, b3 may be NULL (zero bias).  H must be one of 8, 16, 32, 64, 128.
 */
typedef struct {
  int32_t D;      /* channels                                   */
  int32_t N;      /* order (number of filters per channel)      */
  int32_t K;      /* sin/cos frequencies; feature dim is 1+2K   */
  int32_t H;      /* FFN hidden width                           */
  const float* W1;
  const float* b1;
  const float* W2;
  const float* b2;
  const float* W3;
  const float* b3;
  const float* alpha;
} hyena_filter_params;

/* Planner result for a sequence length (host only, no GPU needed). */
typedef struct {
  int64_t L;            /* sequence length                                          */
  int64_t M;            /* real FFT length of a zero-padded row, M >= 2L; each row   */
                        /* is transformed as a complex signal of N = M/2 points     */
  int32_t path;         /* hyena_path                                               */
  int32_t n1;           /* four-step: column FFT length, n1*n2 = N (0 single path)  */
  int32_t n2;           /* four-step: row FFT length (0 on the single path)         */
  int32_t reserved;
  int64_t spec_stride;  /* complex64 elements per (n, d) filter in the spectrum     */
} hyena_plan_info;

/* Fill *out with the plan the library uses for length L.
 * Errors: NULL out -> HYENA_ERR_NULL; L outside 1..HYENA_MAX_L -> HYENA_ERR_SHAPE. */
hyena_status hyena_plan(int64_t L, hyena_plan_info* out);

/*
 * hyena_filter_gen: h[n][d][t] = exp(-alpha_d * t / L) * o_{n*D+d}(t),
 *   o(t) = W3 sin(W2 sin(W1 e(t) + b1) + b2) + b3,
 *   e(t) = [t/L, sin(2 pi k t/L) (k=1..K), cos(2 pi k t/L) (k=1..K)].
 * Output h: device fp32 [N][D][L], written completely.
 * Errors: NULL p/h/weights -> NULL; bad D, N, K, H or L -> SHAPE / UNSUPPORTED.
 */
hyena_status hyena_filter_gen(const hyena_filter_params* p, int64_t L, float* h, void* stream);

/* Bytes of the spectrum buffer for (D, N, L): N*D*spec_stride*8. -1 on bad sizes. */
int64_t hyena_spectrum_bytes(int32_t D, int32_t N, int64_t L);

/* Bytes of scratch hyena_filter_spectrum needs (0 on the single path). -1 on bad sizes. */
int64_t hyena_spectrum_workspace_bytes(int32_t D, int32_t N, int64_t L);

/*
 * hyena_filter_spectrum: the DFT of each filter zero-padded to M points
 * (first step of the FFT convolution applied to h; jisaku.com glossary,
 * section "計算効率"), computed once and reused for any batch.
 * In: h, device fp32 [N][D][L].  Out: spec, device, hyena_spectrum_bytes()
 * bytes, in a library-defined order and scale (read it back in natural order
 * with hyena_spectrum_export).  workspace: device scratch of at least
 * hyena_spectrum_workspace_bytes() bytes (may be NULL when that is 0).
 * Errors: NULL -> NULL; sizes -> SHAPE; alignment -> ALIGN; small workspace
 * -> WORKSPACE; spec overlapping h -> ALIAS.
 */
hyena_status hyena_filter_spectrum(const float* h, int32_t D, int32_t N, int64_t L, void* spec,
                                   void* workspace, int64_t workspace_bytes, void* stream);

/* Natural-order copy of the spectrum: out[n][d][k][re,im] = sum_{t<L} h[n][d][t]
 * exp(-2 pi i k t / M) for k = 0..M/2 (device fp32, N*D*(M/2+1)*2 floats).  For tests. */
hyena_status hyena_spectrum_export(const void* spec, int32_t D, int32_t N, int64_t L, float* out,
                                   void* stream);

/* Bytes of scratch hyena_forward needs for this shape (0 on the single path). -1 on bad sizes. */
int64_t hyena_forward_workspace_bytes(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io);

/*
 * hyena_forward: y = z_{N+1} of the order-N recurrence above.
 *   v        device [B][D][L], I/O dtype
 *   x        HOST array of N device pointers, each [B][D][L], I/O dtype
 *   spec     the spectrum hyena_filter_spectrum wrote for the same (D, N, L)
 *   y        device [B][D][L], I/O dtype; must not overlap v, any x_n or spec
 *   io       HYENA_FP32, or HYENA_BF16 (bf16 loads widened exactly, all
 *            arithmetic fp32, y rounded to nearest even; on the four-step
 *            path (long rows, see hyena_plan) with N <= 2 the transform
 *            between its passes is also kept as bf16 pairs, rounded to
 *            nearest even: half the intermediate traffic and workspace)
 *   workspace device scratch of hyena_forward_workspace_bytes() bytes
 * Errors: NULL -> NULL; sizes -> SHAPE; N > HYENA_MAX_ORDER -> UNSUPPORTED;
 * alignment -> ALIGN; workspace -> WORKSPACE; y overlapping an input -> ALIAS.
 */
hyena_status hyena_forward(const void* v, const void* const* x, const void* spec, void* y,
                           int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io,
                           void* workspace, int64_t workspace_bytes, void* stream);

/*
 * hyena_forward_static: hyena_forward for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, checks, kernels and results as
 * hyena_forward (linear mode), without the workspace: the four-step
 * intermediate lives in one static device buffer of the library,
 * HYENA_STATIC_SCRATCH_BYTES (128 MiB) per GPU, held from the library's load
 * until the process ends; pass groups are sized to it (at most 256 rows of
 * 512 KiB for L = 64K, 16 rows of 8 MiB for L = 1M).  The buffer needs no
 * clearing: each pass group writes its intermediate before reading it.  The
 * call allocates nothing (no hipMalloc, no hipFree); its first call on a
 * device looks the buffer's address up there, once.  All calls on one GPU
 * share that buffer: calls that may overlap in time on one GPU (different
 * streams, threads) race and must be serialised by the caller, e.g. by
 * issuing them on one stream.
 * Errors as hyena_forward; WORKSPACE if one row's intermediate (8 * M / 2
 * bytes) exceeded the buffer, which no supported L reaches (L = 2^22 needs
 * 32 MiB); HIP if the buffer's address cannot be obtained.
 */
#define HYENA_STATIC_SCRATCH_BYTES (128LL << 20)
hyena_status hyena_forward_static(const void* v, const void* const* x, const void* spec, void* y,
                                  int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io, void* stream);

/*
 * Other filter families (homemade-llm "02. 3つの Hyena 演算子", section 3).
 *
 * hyena_filter_gen_li -- Hyena-LI: each filter is a sum of S real
 * exponentials, h[f][t] = sum_s R[f][s] * lambda[f][s]^t for t = 0..L-1
 * (0^0 = 1), f = n*D + d.  R, lambda: device fp32 [N*D][S]; h: device fp32
 * [N][D][L] (feed it to hyena_filter_spectrum like the FFN filters).
 * Errors: NULL -> NULL; D, N, L or S (1..64) out of range -> SHAPE.
 */
hyena_status hyena_filter_gen_li(const float* R, const float* lambda, int32_t D, int32_t N, int32_t S, int64_t L,
                                 float* h, void* stream);

/* hyena_filter_gen_mr -- Hyena-MR: explicit filters of Lh taps damped per
 * channel, h[n][d][t] = hhat[n][d][t] * exp(-alpha[d] * t), t < Lh.  hhat,
 * h: device fp32 [N][D][Lh]; alpha: [D].  Errors as above. */
hyena_status hyena_filter_gen_mr(const float* hhat, const float* alpha, int32_t D, int32_t N, int32_t Lh,
                                 float* h, void* stream);

/* hyena_forward_fir -- the order-N recurrence with explicit short filters
 * (Hyena-SE, or Hyena-MR after hyena_filter_gen_mr): h device fp32
 * [N][D][Lh], Lh in 1..HYENA_MAX_FIR, each convolution evaluated directly
 * (c[t] = sum_{k<Lh, k<=t} h[k] z[t-k]; no FFT, no spectrum, no workspace).
 * Other arguments and errors as hyena_forward. */
#define HYENA_MAX_FIR 256
hyena_status hyena_forward_fir(const void* v, const void* const* x, const float* h, int32_t Lh, void* y,
                               int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io, void* stream);

/*
 * Backward of the recurrence (chain rule through the operator above; the
 * pages state no gradient formulas): for a scalar loss with dloss/dy = gy,
 *   gx_n = g_{n+1} * c_n,   gc_n = g_{n+1} * x_n,
 *   g_n[s] = sum_{t>=s} h_n[t-s] gc_n[t]        (adjoint of the causal conv),
 *   gh_n[k] = sum_b sum_{t>=k} gc_n[t] z_n[t-k]  (summed over the batch),
 * with c_n = h_n conv z_n, g_{N+1} = gy and gv = g_1.  The forward
 * intermediates are recomputed from v, x and the spectrum.
 *   gy, gv    device [B][D][L], I/O dtype;   gx  HOST array of N device
 *   pointers [B][D][L], I/O dtype;  gh  device fp32 [N][D][L].
 * L <= 8192 runs in one launch, one workgroup per channel; longer rows (up
 * to the forward's limit) express every convolution of the chain through
 * the forward's four-step causal convolution and a row reversal, with the
 * forward's c_n kept in the workspace (about (N + 1) * B * D * L * 4 bytes, N + 2 rows with B > 1,
 * plus per-row spectra; a spectrum built on the single path is rewritten
 * into the four-step layout there).  Errors as hyena_forward, plus ALIAS for an output overlapping an
 * input or another output.  hyena_backward_ex takes the convolution mode (see the circular mode below):
 * for circular rows (periodic convolution, c[t] = sum_k h[k] z[(t - k) mod L]) the adjoint and the
 * filter gradient are circular correlations; the one-launch kernel serves L <= 16384, longer rows the
 * four-step pipeline with the periodic reversal t -> -t mod L.
 */
int64_t hyena_backward_workspace_bytes(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io);

hyena_status hyena_backward(const void* v, const void* const* x, const void* spec, const void* gy, void* gv,
                            void* const* gx, float* gh, int64_t B, int32_t D, int32_t N, int64_t L,
                            hyena_dtype io, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The block around the operator (paper digest, irregular6612.github.io,
 * section "방법 (Method)", framework figure: one projection of width (N+1)D
 * yields v and the gates; homemade-llm "02. 3つの Hyena 演算子", section 2:
 * every projected stream is featurised by a short convolution and the result
 * is mapped back by a dense matrix; Hyena Hierarchy explainer section
 * "計算方法": these projections are the D in O(NDL(log L + D))).
 *
 *   Z[b][t][c]  = sum_k u[b][t][k] W_in[c][k] + b_in[c]        c < (N+1)D
 *   S[b][c][t]  = sum_{j<T, j<=t} w_short[c][j] Z[b][t-j][c]    (causal, depthwise)
 *   v = S[:, 0:D],  x_n = S[:, nD:(n+1)D]                       ([B][D][L] each)
 *   y = hyena_forward(v, x, spec)
 *   out[b][t][e] = sum_d W_out[e][d] y[b][d][t] + b_out[e]      ([B][L][D])
 *
 * Device pointers; W_in, W_out and the activations u, out are in the I/O
 * dtype (bf16: fp32 accumulation on the matrix cores, stored values rounded
 * to nearest even), biases and short filters fp32.  b_in / b_out may be NULL.
 */
#define HYENA_MAX_SHORT 16         /* T in 1..16                                */

typedef struct {
  int32_t D;             /* width                                             */
  int32_t N;             /* order                                             */
  int32_t T;             /* short-filter taps                                 */
  int32_t reserved;      /* 0                                                 */
  const void* W_in;      /* [(N+1)*D][D], I/O dtype                           */
  const float* b_in;     /* [(N+1)*D] or NULL                                 */
  const float* w_short;  /* [(N+1)*D][T]                                      */
  const void* W_out;     /* [D][D], I/O dtype                                 */
  const float* b_out;    /* [D] or NULL                                       */
} hyena_block_params;

/* In-projection + short convolution: u [B][L][D] -> streams[0] = v,
 * streams[n] = x_n (HOST array of N+1 device pointers, each [B][D][L], I/O
 * dtype).  Uses W_in, b_in, w_short.  Errors: NULL -> NULL; sizes (incl. T
 * outside 1..HYENA_MAX_SHORT) -> SHAPE; alignment -> ALIGN; a stream
 * overlapping u or W_in -> ALIAS. */
hyena_status hyena_in_projection(const void* u, const hyena_block_params* p, void* const* streams,
                                 int64_t B, int64_t L, hyena_dtype io, void* stream);

/* Output projection: y [B][D][L] -> out [B][L][D] (I/O dtype).  Uses W_out,
 * b_out.  Errors as above; out overlapping y or W_out -> ALIAS. */
hyena_status hyena_out_projection(const void* y, const hyena_block_params* p, void* out, int64_t B,
                                  int64_t L, hyena_dtype io, void* stream);

/* Scratch of hyena_block_forward: v, x_1..x_N and y ([B][D][L] each, I/O
 * dtype, 256-byte aligned) plus the forward's own workspace.  -1 on bad sizes. */
int64_t hyena_block_workspace_bytes(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io);

/* The whole block: u [B][L][D] -> out [B][L][D] with the spectrum of the
 * block's filters (hyena_filter_spectrum for (D, N, L)).  workspace: at least
 * hyena_block_workspace_bytes() bytes.  Errors as the three calls it runs,
 * plus WORKSPACE for a small workspace and ALIAS for out overlapping u. */
hyena_status hyena_block_forward(const void* u, const hyena_block_params* p, const void* spec, void* out,
                                 int64_t B, int64_t L, hyena_dtype io, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/*
 * Circular mode (gist.science HyenaND summary, section "手法: HyenaND",
 * boundary handling: periodic systems use circular convolution, other data
 * the zero-padded linear one).  c[t] = sum_{k<L} h[k] z[(t-k) mod L]: the
 * FFT length is M = L with no padding, so L must be a power of two >= 128
 * (HYENA_ERR_UNSUPPORTED otherwise).  The _ex calls take the mode; the calls
 * without the suffix are HYENA_CONV_LINEAR.  A spectrum is valid only for
 * the mode it was built with.
 */
typedef enum { HYENA_CONV_LINEAR = 0, HYENA_CONV_CIRCULAR = 1 } hyena_conv_mode;

hyena_status hyena_plan_ex(int64_t L, hyena_conv_mode mode, hyena_plan_info* out);
int64_t hyena_spectrum_bytes_ex(int32_t D, int32_t N, int64_t L, hyena_conv_mode mode);
int64_t hyena_spectrum_workspace_bytes_ex(int32_t D, int32_t N, int64_t L, hyena_conv_mode mode);
hyena_status hyena_filter_spectrum_ex(const float* h, int32_t D, int32_t N, int64_t L, hyena_conv_mode mode,
                                      void* spec, void* workspace, int64_t workspace_bytes, void* stream);
hyena_status hyena_spectrum_export_ex(const void* spec, int32_t D, int32_t N, int64_t L, hyena_conv_mode mode,
                                      float* out, void* stream);
int64_t hyena_forward_workspace_bytes_ex(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io,
                                         hyena_conv_mode mode);
hyena_status hyena_forward_ex(const void* v, const void* const* x, const void* spec, void* y, int64_t B,
                              int32_t D, int32_t N, int64_t L, hyena_dtype io, hyena_conv_mode mode,
                              void* workspace, int64_t workspace_bytes, void* stream);
int64_t hyena_backward_workspace_bytes_ex(int64_t B, int32_t D, int32_t N, int64_t L, hyena_dtype io,
                                          hyena_conv_mode mode);
hyena_status hyena_backward_ex(const void* v, const void* const* x, const void* spec, const void* gy, void* gv,
                               void* const* gx, float* gh, int64_t B, int32_t D, int32_t N, int64_t L,
                               hyena_dtype io, hyena_conv_mode mode, void* workspace, int64_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * Convolutions on 2-D and 3-D grids (gist.science HyenaND summary, "手法:
 * HyenaND": native N-D long convolution evaluated through the N-D FFT, with
 * circular boundaries for periodic systems and every axis zero-padded to
 * twice its size for images and volumes; "実装: nSubQ": the FFT, the
 * spectral product and the inverse FFT fused with the intermediate on chip).
 *
 * Grid of k = ndim in {2, 3} axes with sides dims[0..k-1] (row-major, the
 * last axis contiguous).  The same order-N recurrence as hyena_forward,
 * z_1 = v, z_{n+1} = x_n * (K_n conv z_n), y = z_{N+1}, with
 *   non-circular: c[t] = sum over grid points s of K[t - s] z[s]; the kernel
 *                 holds one value per offset o with |o_a| < dims[a], stored
 *                 row-major with extent 2*dims[a]-1 and index o_a+dims[a]-1
 *                 (a causal kernel is zero at negative offsets);
 *   circular:     c[t] = sum_s K[(t - s) mod dims] z[s]; the kernel has the
 *                 grid's shape.
 * Supported: the FFT grid is a cube of side P, a power of two with, per
 * dimension count, 16 <= P <= 1024 (2-D) or 8 <= P <= 128 (3-D).  Non-circular
 * grids take the smallest such P >= 2*max(dims)-1 (so sides up to 512 in
 * 2-D and 64 in 3-D); circular grids need every side equal to one such P.
 * Other shapes return HYENA_ERR_UNSUPPORTED (a side outside 1..4096: SHAPE).
 * Up to P = 128 (2-D) or 32 (3-D) one workgroup holds a grid for all orders
 * and no workspace is used; larger grids run as passes over the first axis
 * and over rows (2-D) or planes (3-D) through a workspace of
 * hyena_nd_workspace_bytes (at least one grid, P^k/2 complex64 values; a
 * smaller one than returned means more, smaller pass groups).
 *
 * hyena_nd_plan: writes P.
 * hyena_nd_spectrum_bytes: bytes of the spectrum of `rows` kernels (-1 for
 *   an invalid or unsupported shape).  The layout is private.
 * hyena_nd_filter_spectrum: kernel [rows][extent] fp32 (device) -> spec
 *   (device, hyena_nd_spectrum_bytes).  Row r is the kernel n*D + d for the
 *   shared form, (b*N + n)*D + d for per-sample kernels (the summary's
 *   input-dependent kernels, one per sample).
 * hyena_nd_workspace_bytes: workspace for `rows` grids (kernel rows for the
 *   spectrum, B*D for the forward); 0 on the single-pass shapes, -1 for an
 *   invalid or unsupported shape.
 * hyena_nd_forward: v, each x[n] (host array of N device pointers) and y are
 *   [B][D][dims...] in `io`; spec from hyena_nd_filter_spectrum with N*D
 *   rows (per_sample = 0) or B*N*D rows (per_sample = 1).  1 <= N <= 8.
 *   Pointers 16-byte aligned (HYENA_ERR_ALIGN); y and the workspace must not
 *   overlap v, any x[n], spec or each other (HYENA_ERR_ALIAS); a missing or
 *   too small workspace where one is needed is HYENA_ERR_WORKSPACE.  No
 *   allocation; the work is enqueued on `stream`.
 * ---------------------------------------------------------------------- */
hyena_status hyena_nd_plan(int32_t ndim, const int64_t* dims, int32_t circular, int64_t* padded_side);
int64_t hyena_nd_spectrum_bytes(int32_t rows, int32_t ndim, const int64_t* dims, int32_t circular);
int64_t hyena_nd_workspace_bytes(int64_t rows, int32_t ndim, const int64_t* dims, int32_t circular);
hyena_status hyena_nd_filter_spectrum(const float* kernel, int32_t rows, int32_t ndim, const int64_t* dims,
                                      int32_t circular, void* spec, void* workspace, int64_t workspace_bytes,
                                      void* stream);
hyena_status hyena_nd_forward(const void* v, const void* const* x, const void* spec, void* y, int64_t B,
                              int32_t D, int32_t N, int32_t ndim, const int64_t* dims, int32_t circular,
                              int32_t per_sample, hyena_dtype io, void* workspace, int64_t workspace_bytes,
                              void* stream);

/* Static description of a status code. */
const char* hyena_status_str(hyena_status s);

#ifdef __cplusplus
}
#endif

#endif /* HYENA_MI355X_H */
