/*
 * gconv.h -- C ABI of libgconv.so, a grouped-convolution forward engine for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  Grouped convolution as the neon issue "Grouped convolutions"
 * defines it (thestew42's first reply): the C input channels, the Cout filters
 * and the Cout output channels are split into `groups` groups that are not
 * connected to each other.  Group k reads input channels [k*C/g, (k+1)*C/g) and
 * writes output channels [k*Cout/g, (k+1)*Cout/g) (the "usual" group-contiguous
 * output order in ibmua's reply on the same issue).  Each output is the
 * cross-correlation F.conv2d computes in the discuss.pytorch.org thread "F.conv2d
 * runs x15 slower in mixed-precision/half-precision mode" (the poster's script:
 * F.conv2d(input, weight, padding=3 // 2, groups=4)):
 *
 *   y[n,o,oh,ow] = bias[o] + sum_{ci<C/g, kh<KH, kw<KW}
 *                  x[n, (o/(Cout/g))*(C/g)+ci, oh*sh-ph+kh*dh, ow*sw-pw+kw*dw] * w[o,ci,kh,kw]
 *
 * with x read as zero outside [0,H)x[0,W).  The second layout is the depthwise
 * 1-D convolution of speechbrain issue #2733 (Conformer convolution module,
 * groups equal to the channel count, tensor laid out (batch, steps, channels)):
 *
 *   y[b,t,c] = bias[c] + sum_{k<K} x[b, t*s-p+k*d, c] * w[c,0,k]
 *
 * Arithmetic.  fp32 tensors are multiplied and accumulated in fp32.  fp16 and
 * bf16 tensors are multiplied exactly and accumulated in fp32 (matrix cores or
 * fp32 FMA); the bias is added to the fp32 accumulator and the result is rounded
 * once to the tensor dtype, round-to-nearest-even.
 *
 * Conventions shared by every entry point:
 *  - Pointers x, w, bias, y are DEVICE pointers owned by the caller, contiguous
 *    in the stated layout, all of the one dtype `dtype`.  y must not overlap
 *    x, w or bias.  bias may be NULL (no bias).
 *  - Shape arrays and stride/pad/dilation arrays are HOST pointers.
 *      NCHW: x_shape = {N,C,H,W}, w_shape = {Cout, C/groups, KH, KW},
 *            stride/pad/dilation = {h, w} (2 ints each), y = {N,Cout,OH,OW}.
 *      NTC : x_shape = {B,T,C}, w_shape = {C,1,K}, groups must equal C,
 *            stride/pad/dilation = 1 int each, y = {B,To,C}.
 *      NHWC: the NCHW convolution over channels-last tensors (the NHWC memory
 *            format the discuss.pytorch.org thread turns to for the fp16 grouped
 *            conv): x_shape = {N,H,W,C}, w_shape = {Cout, KH, KW, C/groups}
 *            (channels_last weight order), stride/pad/dilation = {h, w},
 *            y = {N,OH,OW,Cout}.  The implicit-GEMM route runs fp16/bf16 with C/g a
 *            multiple of 16, Cout/g a multiple of 4, the grouped output order, x
 *            and w 16-byte and y 8-byte aligned (its 16-byte fragment loads need
 *            whole, aligned 8-channel runs of x and w); otherwise
 *            GCONV_ERR_UNSUPPORTED when forced.
 *    Output length per axis: floor((L + 2p - d*(K-1) - 1)/s) + 1.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without synchronising.
 *  - The library keeps no state between calls apart from a thread-local error
 *    string, the route cache of gconv_autotune (empty unless it is called) and
 *    the device scratch array of gconv_dw1d_bwd_filter_noalloc (static device
 *    memory, one copy per GPU).  It allocates no device memory and is safe to
 *    call from several host threads at once (gconv_dw1d_bwd_filter_noalloc
 *    calls that overlap on one GPU excepted).
 *  - Errors: argument and shape errors are detected on the host before anything
 *    is enqueued, and leave y untouched.  A zero-sized batch (N == 0 or B == 0)
 *    is valid and enqueues nothing; x and y may then be NULL.  No C++ exception
 *    crosses this boundary.
 */
#ifndef GCONV_H
#define GCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GCONV_OK = 0,
    GCONV_ERR_INVALID_ARG = 1,  /* NULL pointer, bad enum, size/stride/dilation < 1, pad < 0  */
    GCONV_ERR_SHAPE = 2,        /* C or Cout not divisible by groups, weight shape mismatch,
                                   or an output length below 1                               */
    GCONV_ERR_UNSUPPORTED = 3,  /* a valid convolution this library does not run, e.g. NTC
                                   with groups != C, or a forced route that cannot run it   */
    GCONV_ERR_LAUNCH = 4        /* the HIP runtime reported an error when launching         */
} gconv_status_t;

typedef enum {
    GCONV_LAYOUT_NCHW = 0,      /* conv2d, x [N,C,H,W]                                      */
    GCONV_LAYOUT_NTC = 1,       /* depthwise conv1d, x [B,T,C] = (batch, steps, channels)   */
    GCONV_LAYOUT_NHWC = 2       /* conv2d over channels-last tensors, x [N,H,W,C]          */
} gconv_layout_t;

typedef enum { GCONV_F32 = 0, GCONV_F16 = 1, GCONV_BF16 = 2 } gconv_dtype_t;

/* Which kernel family runs a call.  The option of choosing the route follows
 * functorch issue #365 "Optimize convolution batching rule performance", where
 * the maintainers agree on a user option selecting the group-convolution route. */
typedef enum {
    GCONV_ROUTE_AUTO = 0,       /* chosen per shape by gconv_select_route (a route recorded
                                   by gconv_autotune, else the static heuristic)            */
    GCONV_ROUTE_DIRECT = 1,     /* direct convolution on the vector ALUs: LDS halo tiles,
                                   group index folded into the grid (NCHW), or the
                                   (batch, steps, channels) sliding-window kernel (NTC)     */
    GCONV_ROUTE_IGEMM = 2       /* implicit GEMM per group on the matrix cores, im2col
                                   never materialised (NCHW: tiles built in LDS; NHWC:
                                   fragments read straight from x and w)                  */
    /* NHWC: the direct route is a channels-on-lanes tile kernel for depthwise layers
       and a coalesced one-thread-per-output kernel otherwise; the implicit-GEMM route
       loads its fragments straight from the channels-last tensors. */
} gconv_route_t;

/* Output shape of a convolution.  y_shape receives 4 (NCHW, NHWC) or 3 (NTC) values.
 * Each spatial or time axis has floor((L + 2p - d(K-1) - 1) / s) + 1 outputs: the
 * length torch.nn.functional.conv2d gives the layer timed by the poster's script in
 * the discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
 * half-precision mode" (3x3, padding 3//2: same size), and nn.Conv1d the 'same'
 * padded depthwise conv of speechbrain issue #2733 (K = 31, padding 15).  Channels:
 * Cout (NCHW, NHWC) or C (NTC).
 * Returns GCONV_OK, GCONV_ERR_INVALID_ARG (null pointer, non-positive size, groups
 * not dividing C and Cout, w not [Cout, C/g, ...]) or GCONV_ERR_SHAPE (an axis with
 * fewer than one output); no device work. */
gconv_status_t gconv_out_shape(const int64_t *x_shape, const int64_t *w_shape,
                               const int32_t *stride, const int32_t *pad,
                               const int32_t *dilation, int32_t groups,
                               gconv_layout_t layout, int64_t *y_shape);

/* The route GCONV_ROUTE_AUTO takes for this geometry and dtype (written to
 * *route; never GCONV_ROUTE_AUTO).  A route recorded by gconv_autotune for this
 * geometry comes first.  Otherwise NCHW and NHWC layers with enough reduction depth
 * and filters per group (C/g*KH*KW >= 64 and Cout/g >= 16) whose implicit-GEMM plan
 * exists take GCONV_ROUTE_IGEMM: the discuss.pytorch.org thread "F.conv2d runs x15
 * slower in mixed-precision/half-precision mode" traces the slow fp16 grouped conv to
 * grouped convs not reaching the tensor cores, so these run per group on the matrix
 * cores.  Smaller groups, where a matrix tile would be mostly padding, and every NTC
 * call take GCONV_ROUTE_DIRECT, the kernels with the group index in the launch grid
 * (neon issue "Grouped convolutions", the reply proposing to offset the pointers by
 * blockIdx times the group stride).  Same validation and return codes as
 * gconv_out_shape; no device work. */
gconv_status_t gconv_select_route(const int64_t *x_shape, const int64_t *w_shape,
                                  const int32_t *stride, const int32_t *pad,
                                  const int32_t *dilation, int32_t groups,
                                  gconv_layout_t layout, gconv_dtype_t dtype,
                                  gconv_route_t *route);

/* Grouped convolution forward, route chosen per shape (GCONV_ROUTE_AUTO). */
gconv_status_t gconv_fwd(const void *x, const int64_t *x_shape,
                         const void *w, const int64_t *w_shape,
                         const void *bias, void *y,
                         const int32_t *stride, const int32_t *pad, const int32_t *dilation,
                         int32_t groups, gconv_layout_t layout, gconv_dtype_t dtype,
                         void *hip_stream);

/* gconv_fwd with the route forced by the caller.  GCONV_ROUTE_IGEMM on NTC, or
 * on a geometry the implicit-GEMM kernels do not cover, returns
 * GCONV_ERR_UNSUPPORTED without enqueuing anything. */
gconv_status_t gconv_fwd_route(const void *x, const int64_t *x_shape,
                               const void *w, const int64_t *w_shape,
                               const void *bias, void *y,
                               const int32_t *stride, const int32_t *pad, const int32_t *dilation,
                               int32_t groups, gconv_layout_t layout, gconv_dtype_t dtype,
                               gconv_route_t route, void *hip_stream);

/* ---- backward of the depthwise 1-D convolution over (batch, steps, channels) --
 *
 * speechbrain issue #2733 ("Investigate custom Triton kernels for depthwise-
 * separable convolutions in Conformer"), its author's follow-up comments: the
 * backward pass of the (batch, steps, channels) depthwise conv.  For the forward
 *     y[b][t][c] = bias[c] + sum_k x[b][t*s - p + k*d][c] * w[c][0][k]
 * (gconv_fwd with layout GCONV_LAYOUT_NTC, groups = C) and an upstream gradient
 * dy[b][t][c] of y's shape [B][To][C], the gradients are
 *     dx[b][i][c] = sum over (t, k) with t*s - p + k*d == i of dy[b][t][c] * w[c][0][k]
 *     dw[c][0][k] = sum over (b, t), 0 <= t*s - p + k*d < T, of dy[b][t][c] * x[b][t*s-p+k*d][c]
 *     db[c]       = sum over (b, t) of dy[b][t][c]
 * Shapes are the forward call's: x_shape = {B, T, C}, w_shape = {C, 1, K};
 * stride, pad and dilation each point to one int32.  All tensors are contiguous
 * device buffers of `dtype`, owned by the caller; accumulation is fp32 and each
 * result is rounded once to `dtype`.  Validation errors (the forward's, plus
 * the overlaps named below) return before anything is enqueued and leave the
 * outputs untouched; work is asynchronous on hip_stream and deterministic (no
 * atomics). */

/* Input gradient dx [B][T][C] from dy [B][To][C] and w [C][1][K].  dx must not
 * overlap dy or w.  B = 0: GCONV_OK, nothing enqueued (dy, dx may be NULL). */
gconv_status_t gconv_dw1d_bwd_data(const void *dy, const int64_t *x_shape,
                                   const void *w, const int64_t *w_shape, void *dx,
                                   const int32_t *stride, const int32_t *pad,
                                   const int32_t *dilation, gconv_dtype_t dtype,
                                   void *hip_stream);

/* Bytes of device workspace gconv_dw1d_bwd_filter needs for this geometry
 * (fp32 per-tile partial sums; 0 for B = 0).  GCONV_ERR_UNSUPPORTED for filter
 * lengths above 64.  No device work. */
gconv_status_t gconv_dw1d_bwd_filter_workspace(const int64_t *x_shape, const int64_t *w_shape,
                                               const int32_t *stride, const int32_t *pad,
                                               const int32_t *dilation, gconv_dtype_t dtype,
                                               size_t *bytes);

/* Filter gradient dw [C][1][K] and, if db is not NULL, bias gradient db [C], from
 * x [B][T][C] and dy [B][To][C].  workspace: caller-owned device memory of at
 * least gconv_dw1d_bwd_filter_workspace bytes (any alignment of 4 bytes or
 * more), overwritten; fewer bytes is GCONV_ERR_INVALID_ARG.  dw, db, workspace,
 * x and dy must not overlap.  B = 0 writes zeros to dw and db. */
gconv_status_t gconv_dw1d_bwd_filter(const void *x, const int64_t *x_shape, const void *dy,
                                     const int64_t *w_shape, void *dw, void *db,
                                     const int32_t *stride, const int32_t *pad,
                                     const int32_t *dilation, gconv_dtype_t dtype,
                                     void *workspace, size_t workspace_bytes, void *hip_stream);

/* gconv_dw1d_bwd_filter for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the per-tile partial sums go to a scratch array the library holds in device
 * memory, GCONV_DW1D_BWD_FILTER_SCRATCH_BYTES bytes per GPU, kept until the
 * process ends (its device address is looked up once per device, on the first
 * call there).  The call allocates nothing.  Arguments, results and errors are
 * those of gconv_dw1d_bwd_filter without the workspace; a geometry whose
 * gconv_dw1d_bwd_filter_workspace exceeds the scratch size is
 * GCONV_ERR_UNSUPPORTED, checked before anything is enqueued.  Every call on one
 * GPU uses that GPU's one array: calls whose work overlaps in time on the same
 * GPU (other streams, other host threads) race and give wrong results; order
 * them on one stream.  The array holds the last call's partial sums; nothing in
 * it needs clearing (each call writes every entry it reads). */
#define GCONV_DW1D_BWD_FILTER_SCRATCH_BYTES (16u << 20)
gconv_status_t gconv_dw1d_bwd_filter_noalloc(const void *x, const int64_t *x_shape, const void *dy,
                                             const int64_t *w_shape, void *dw, void *db,
                                             const int32_t *stride, const int32_t *pad,
                                             const int32_t *dilation, gconv_dtype_t dtype,
                                             void *hip_stream);

/* Order of the output channels.  The neon issue "Grouped convolutions" (ibmua's
 * reply on output ordering) names two: the usual group-contiguous order
 * 111122223333 (filter j of group k at channel k*Cout/g + j) and the interleaved
 * order 123412341234 (filter j of group k at channel j*g + k).  Only the output
 * channel index changes; w and bias stay indexed by filter o = k*Cout/g + j. */
typedef enum {
    GCONV_ORDER_GROUPED = 0,
    GCONV_ORDER_INTERLEAVED = 1
} gconv_out_order_t;

/* gconv_fwd with the route and the output-channel order chosen by the caller
 * (GCONV_ROUTE_AUTO and GCONV_ORDER_GROUPED give gconv_fwd).  The orders coincide
 * when there is one group or one filter per group (NTC always).  Same arguments,
 * conventions and errors as gconv_fwd_route; an unknown order is
 * GCONV_ERR_INVALID_ARG. */
gconv_status_t gconv_fwd_ex(const void *x, const int64_t *x_shape,
                            const void *w, const int64_t *w_shape,
                            const void *bias, void *y,
                            const int32_t *stride, const int32_t *pad, const int32_t *dilation,
                            int32_t groups, gconv_layout_t layout, gconv_dtype_t dtype,
                            gconv_route_t route, gconv_out_order_t order, void *hip_stream);

/* Per-shape route tuning.  The discuss.pytorch.org thread "F.conv2d runs x15
 * slower in mixed-precision/half-precision mode" suggests
 * torch.backends.cudnn.benchmark (time the candidate algorithms once per shape,
 * keep the fastest), and the neon issue "Grouped convolutions" describes neon
 * compiling kernel variants, timing them and keeping the fastest.
 *
 * gconv_autotune runs the call once per route that can run it (GCONV_ROUTE_DIRECT,
 * GCONV_ROUTE_IGEMM) untimed, then `reps` (>= 1) times between two HIP events on
 * hip_stream, and records the route with the shortest time for this geometry
 * (layout, dtype, shapes, stride, padding, dilation, groups) in a process-wide
 * cache.  Later GCONV_ROUTE_AUTO calls and gconv_select_route of the same
 * geometry take the recorded route (when it can run the call: the implicit-GEMM
 * route also depends on pointer alignment).  The arguments are those of
 * gconv_fwd; y is overwritten and holds the chosen route's result on return.
 * Unlike every other entry point this one SYNCHRONISES hip_stream (to read the
 * events).  *best receives the chosen route.  Errors as gconv_fwd;
 * GCONV_ERR_UNSUPPORTED if no route runs the call.  The cache is guarded by a
 * mutex; it holds host memory only and lives until gconv_autotune_clear or the
 * end of the process. */
gconv_status_t gconv_autotune(const void *x, const int64_t *x_shape,
                              const void *w, const int64_t *w_shape,
                              const void *bias, void *y,
                              const int32_t *stride, const int32_t *pad, const int32_t *dilation,
                              int32_t groups, gconv_layout_t layout, gconv_dtype_t dtype,
                              int32_t reps, void *hip_stream, gconv_route_t *best);

/* Forgets every route gconv_autotune recorded. */
void gconv_autotune_clear(void);

/* Name of the kernel the last successful gconv_fwd / gconv_fwd_route / gconv_fwd_ex /
 * gconv_dw1d_bwd_data / gconv_dw1d_bwd_filter call on this host thread launched
 * (the first of two for the filter gradient; "" before the first call or after
 * an empty batch).  The string has static storage. */
const char *gconv_last_kernel(void);

/* Fixed English text for a status code.  Static storage.  (The status codes and the
 * error text are this library's own conventions; the pages define none.) */
const char *gconv_status_string(gconv_status_t status);

/* Detail of the last non-OK status returned on this host thread ("" if none).
 * Thread-local storage, valid until the next call on the same thread. */
const char *gconv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GCONV_H */
