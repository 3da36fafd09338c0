/*
 * dcn_core.h -- C ABI of the MI355X (gfx950) deformable sampling core used by
 * DCNv3 and DCNv4.
 *
 * Pages cited (title, site):
 *   [FB]  "没有CUDA内核也能跑：InternImage-G的DCNv3纯PyTorch回退实现逐行解读"
 *         (the DCNv3 pure-PyTorch fallback read line by line), trdm.cn
 *   [V4]  "DCNv4高效实践指南：掌握可变形卷积的3倍速度提升技术"
 *         (DCNv4 practice guide), seekfood.cn
 *   [A100] "告别DCNv3的卡顿：实测DCNv4在A100上3倍提速…", framerc.cn
 *   [FII] FlashInternImage image-classification guide, m.nxbn.cn
 *
 * The operation ([FB] section 4, steps 1-5; the DCNv4 variant drops the
 * softmax, [V4] core-architecture section, [A100] section 1):
 *
 *   out[n,ho,wo,g*Cg+c] = sum_{i<K, j<K} m[n,ho,wo,g,p] * B(in[n,:,:,g*Cg+c], x_p, y_p)
 *
 *   p   = i*K + j            i = kernel column (x), j = kernel row (y)
 *   c0  = floor(dilation*(K-1)/2)
 *   x_p = fmaf(offset_scale, dx, fmaf(offset_scale, (float)(i*dilation - c0), (float)(wo*stride - pad + c0)))
 *   y_p = fmaf(offset_scale, dy, fmaf(offset_scale, (float)(j*dilation - c0), (float)(ho*stride - pad + c0)))
 *         -- formed in binary32 in exactly this order (the inner fmaf is
 *         exact when offset_scale is 1); these are pixel
 *         coordinates in the UNPADDED map (the zero padding of step 1 is
 *         virtual: everything outside [0,H) x [0,W) reads as zero)
 *   B   = bilinear interpolation from the four pixels around (x_p, y_p);
 *         corners outside the map contribute zero; a sample with no corner
 *         on the map (or a NaN/Inf coordinate) contributes nothing
 *   m   = softmax over the P = K*K points of each (pixel, group) when
 *         softmax_flag != 0 (DCNv3, [FB] section 3 item 3), else the raw
 *         mask (DCNv4)
 *
 * Weights, softmax and accumulation are binary32 for every dtype; half
 * precision inputs are widened exactly and the result is rounded once (to
 * nearest even) to the output dtype.
 *
 * Tensor layout (all dense, row-major, channels last, one dtype for all):
 *   input   (N, H,  W,  G*Cg)        channel = g*Cg + c
 *   offset  (N, Ho, Wo, G, P, 2)     last axis = (dx, dy) in pixels
 *   mask    (N, Ho, Wo, G, P)        logits (softmax_flag) or raw weights
 *   output  (N, Ho, Wo, G*Cg)
 *   Ho = dcn_core_out_size(H, K, stride, pad, dilation), Wo likewise.
 * Gradients have the shape and dtype of their primal.
 *
 * Ownership and threading: every pointer is a device pointer owned by the
 * caller.  The library allocates no memory, keeps no state between calls,
 * and is safe to call from several host threads.  Calls are asynchronous on
 * `stream` (a hipStream_t passed as void*; NULL = the default stream) and
 * never synchronise; a kernel fault surfaces at the caller's next
 * synchronising call.
 *
 * Errors: arguments are validated on the host before any HIP call; a
 * rejected call launches nothing and touches no buffer.
 */
#ifndef DCN_CORE_H
#define DCN_CORE_H

#ifdef __cplusplus
extern "C" {
#endif

enum dcn_dtype { DCN_F32 = 0, DCN_F16 = 1, DCN_BF16 = 2 };

enum dcn_status {
    DCN_OK = 0,
    DCN_ERR_INVALID_ARG = 1,  /* bad size, geometry, dtype or null pointer */
    DCN_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement */
    DCN_ERR_HIP = 3,          /* the HIP runtime reported an error at launch */
    DCN_ERR_SCRATCH_LIMIT = 4 /* dcn_core_backward_static: larger than its static scratch */
};

/* Output extent along one axis of a K-tap sampling grid with the given
 * stride, zero padding and dilation: floor((in + 2*pad - dilation*(K-1) - 1)
 * / stride) + 1 ([FB] section 4 step 1 takes H_out, W_out from the offset
 * tensor and notes that stride 2 halves them).  Returns a value <= 0 when the
 * arguments are invalid (in, K, stride, dilation < 1; pad < 0) or the grid
 * does not fit. */
int dcn_core_out_size(int in, int K, int stride, int pad, int dilation);

/* Forward sampling core (definition above).
 *   input, offset, mask: device pointers, read only; output: device pointer,
 *   overwritten.  N >= 0 (N == 0 is a no-op and then the pointers may be
 *   NULL); H, W, G, Cg, K, stride, dilation >= 1; pad >= 0; the output grid
 *   must be non-empty.  offset_scale is any finite float; softmax_flag is 0
 *   (raw mask) or 1 (softmax); dtype is a dcn_dtype.
 * Returns DCN_OK, DCN_ERR_INVALID_ARG, DCN_ERR_UNSUPPORTED (one image of
 * any tensor holds 2^31 elements or more, or K > 16), or DCN_ERR_HIP. */
int dcn_core_forward(const void* input, const void* offset, const void* mask, void* output,
                     int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                     int dilation, float offset_scale, int softmax_flag, int dtype,
                     void* stream);

/* Backward of the forward above for an upstream gradient grad_output
 * (N, Ho, Wo, G*Cg).  Writes:
 *   grad_input  (N, H, W, G*Cg): for each input pixel, the sum of
 *               m_p * w * grad_output over every valid corner of every sample
 *               that lands on it.  The sum is formed in an order that is not
 *               fixed (adds into on-chip memory and, for corners far from
 *               their sample's base, float atomics), so its last bits can
 *               vary from run to run;
 *   grad_offset (N, Ho, Wo, G, P, 2): offset_scale * m_p * sum_c g_c * dB/dx
 *               (and dB/dy), the derivative of the bilinear read taken from
 *               the right where floor() jumps;
 *   grad_mask   (N, Ho, Wo, G, P): sum_c g_c * B_p for a raw mask, or the
 *               softmax Jacobian applied to it, m_p * (gm_p - sum_q m_q gm_q),
 *               when softmax_flag is set (gradient w.r.t. the logits).
 * Samples that contribute nothing to the forward get zero gradients.  The
 * three outputs are overwritten, never accumulated into.  The pages print
 * no gradient formulas; these are the derivatives of the definition.
 * Same arguments and errors as dcn_core_forward.  The arithmetic is binary32
 * for every dtype and each gradient is rounded once to the dtype.  This call
 * takes no workspace, so it serves binary32 only: a half-precision grad_input
 * is summed in a binary32 workspace, which dcn_core_backward_ws takes from
 * the caller (DCN_ERR_UNSUPPORTED here for fp16 and bf16). */
int dcn_core_backward(const void* input, const void* offset, const void* mask,
                      const void* grad_output, void* grad_input, void* grad_offset,
                      void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                      int pad, int dilation, float offset_scale, int softmax_flag, int dtype,
                      void* stream);

/* Options of the _ex entry points, OR-ed into `flags`. */
enum dcn_flags {
    /* softmax over each (pixel, group)'s points (DCNv3); absent: raw mask (DCNv4) */
    DCN_FLAG_SOFTMAX = 1,
    /* leave out the centre tap of an odd K: P = K*K - 1 points, the remaining
     * taps keep their order p = i*K + j with the centre index skipped ([FB]
     * section 4 step 3 subtracts remove_center from the point count; the
     * DCNv4 module takes the same switch, [V4] programming-interface section).
     * K must be odd and >= 3. */
    DCN_FLAG_REMOVE_CENTER = 2,
    /* DCNv4's single offset-and-weight tensor ([A100] section 1 passes one
     * tensor carrying both to the DCNv4 core): `offset` is
     * (N, Ho, Wo, G, 3P), each (pixel, group) record holding its 2P offsets
     * as (dx, dy) pairs in point order, then its P mask values; `mask` (and
     * grad_mask) must be NULL and grad_offset receives the gradient in the
     * same record layout.  The record order is not printed on the pages; this
     * is the layout the library defines.  The tensor must start on a 4-byte
     * boundary. */
    DCN_FLAG_PACKED = 4
};

/* dcn_core_forward with options: `flags` is an OR of dcn_flags (any other
 * bit is DCN_ERR_INVALID_ARG); P = K*K, or K*K - 1 with
 * DCN_FLAG_REMOVE_CENTER, in every tensor shape above.  Otherwise the same
 * arguments, definition and errors as dcn_core_forward, which equals this
 * call with flags = softmax_flag. */
int dcn_core_forward_ex(const void* input, const void* offset, const void* mask, void* output,
                        int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                        int dilation, float offset_scale, int flags, int dtype, void* stream);

/* dcn_core_backward with options (flags as for dcn_core_forward_ex).  With
 * DCN_FLAG_PACKED, offset and grad_offset are packed records and mask and
 * grad_mask are NULL; the gradient of each mask value lands in its record's
 * tail.  Same support limits and errors as dcn_core_backward. */
int dcn_core_backward_ex(const void* input, const void* offset, const void* mask,
                         const void* grad_output, void* grad_input, void* grad_offset,
                         void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                         int pad, int dilation, float offset_scale, int flags, int dtype,
                         void* stream);

/* Bytes of device workspace dcn_core_backward_ws needs for this call: 0 when
 * the call runs without one (binary32 or an empty batch), else N*H*W*G*Cg*4
 * (one binary32 accumulator per grad_input element: every half-precision
 * call).  The pointers are the ones the call will use.  Returns minus a
 * dcn_status for invalid arguments. */
long long dcn_core_backward_workspace_size(const void* input, const void* grad_output, const void* grad_input,
                                           int N, int H, int W, int G, int Cg, int K, int stride, int pad,
                                           int dilation, float offset_scale, int flags, int dtype);

/* dcn_core_backward_ex with a caller-owned device workspace (workspace_bytes
 * of it, at least what dcn_core_backward_workspace_size returns, 16-byte
 * aligned; NULL and 0 when none is needed): the half-precision backward
 * (mixed-precision training is the pages' main use of the core, and [FII]
 * section 5.3 traces its NaN and loss trouble to half-precision numerics,
 * so no sum is kept in a half type).  The workspace holds a
 * binary32 image of grad_input: every contribution to a grad_input element
 * is summed in binary32 (on-chip per input tile for corners near their
 * sample's base, binary32 atomics into the workspace for the rest) and the
 * element is rounded once to the dtype.  The workspace is overwritten; its
 * contents after the call are unspecified.  Half precision runs on every
 * shape whose channels per group split into a power-of-two number of lanes.
 * Binary32 calls ignore the workspace and behave as dcn_core_backward_ex.
 * Returns DCN_ERR_INVALID_ARG for a workspace that is too small or
 * misaligned, DCN_ERR_UNSUPPORTED if one is needed and none is given or if
 * the group width does not split. */
int dcn_core_backward_ws(const void* input, const void* offset, const void* mask,
                         const void* grad_output, void* grad_input, void* grad_offset,
                         void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                         int pad, int dilation, float offset_scale, int flags, int dtype,
                         void* workspace, long long workspace_bytes, void* stream);

/* Size in bytes of dcn_core_backward_static's static scratch. */
#define DCN_STATIC_SCRATCH_BYTES (64ll << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * dcn_core_backward_ws with the library's own static device array as the
 * binary32 workspace, so the caller passes only inputs and outputs.  The
 * array is DCN_STATIC_SCRATCH_BYTES (64 MiB: a half-precision call with
 * N*H*W*G*Cg up to 16,777,216 elements); each GPU holds its own
 * copy from the library's first use of it on that device (the device current
 * when the call is made, which must be the stream's) until the process ends.
 * The call allocates and frees nothing.  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (each call clears what it
 * needs with a kernel on `stream`): calls that overlap on one GPU -- on two
 * streams, or from two host threads -- race and give wrong gradients; calls
 * on different GPUs do not.  Binary32 calls and N == 0 use no scratch and
 * behave as dcn_core_backward_ex.  Same arguments, results and errors as
 * dcn_core_backward_ws, plus DCN_ERR_SCRATCH_LIMIT for a call that needs
 * more than the array. */
int dcn_core_backward_static(const void* input, const void* offset, const void* mask,
                             const void* grad_output, void* grad_input, void* grad_offset,
                             void* grad_mask, int N, int H, int W, int G, int Cg, int K, int stride,
                             int pad, int dilation, float offset_scale, int flags, int dtype,
                             void* stream);

/* dcn_core_forward_ex followed by the DCNv4 layer's centre-feature gate
 * (dcn_center_gate_forward) in one pass, for the layer's geometry: odd K,
 * stride 1, pad = dilation * (K - 1) / 2 (so Ho = H, Wo = W and output
 * pixel (h, w) is centred on input pixel (h, w)) and a raw mask
 * (DCN_FLAG_SOFTMAX is DCN_ERR_UNSUPPORTED).  gate_logits is (N, H, W, G) in
 * the dtype (2-byte aligned for half types); with y the sampled result and
 * s = 1 / (1 + exp(-gate_logits[n, h, w, g])):
 *
 *   output[n, h, w, g*Cg + c] = y * (1 - s) + input[n, h, w, g*Cg + c] * s
 *
 * computed in binary32 from the unrounded y and rounded once.  core_output,
 * if not NULL (16-byte aligned), receives y rounded to the dtype (what the
 * gate's backward needs).  Only shapes the tiled kernel serves are taken
 * (see dcn_core_backward for the tiled shapes); others return
 * DCN_ERR_UNSUPPORTED, and a caller then runs dcn_core_forward_ex and
 * dcn_center_gate_forward.  Other arguments and errors as
 * dcn_core_forward_ex. */
int dcn_core_forward_gated(const void* input, const void* offset, const void* mask, const void* gate_logits,
                           void* output, void* core_output, int N, int H, int W, int G, int Cg, int K,
                           int stride, int pad, int dilation, float offset_scale, int flags, int dtype,
                           void* stream);

/* Centre-feature gate of the DCNv4 layer ([FB] section 3: an optional sigmoid
 * gate blends the centre pixel's projected features with the sampling
 * result).  For M pixels of G groups of Cg channels:
 *
 *   output[m, g*Cg+c] = y[m, g*Cg+c] * (1 - s) + v[m, g*Cg+c] * s,
 *   s = 1 / (1 + exp(-z[m, g]))
 *
 * y (the core's output), v (the layer's projected input) and output are
 * (M, G*Cg); z is (M, G); one dtype for all, binary32 arithmetic, one
 * rounding per stored value.  output may be the same buffer as y or v.
 * M >= 0 (M == 0 is a no-op; then the pointers may be NULL), G, Cg >= 1.
 * Returns DCN_OK, DCN_ERR_INVALID_ARG (bad size or dtype, a NULL or
 * misaligned pointer), DCN_ERR_UNSUPPORTED (a row of 2^30 bytes or more, or
 * 2^40 or more (pixel, group) rows) or DCN_ERR_HIP. */
int dcn_center_gate_forward(const void* y, const void* v, const void* z, void* output, long long M,
                            int G, int Cg, int dtype, void* stream);

/* Backward of the gate for grad_output (M, G*Cg): grad_y = grad_output *
 * (1 - s), grad_v = grad_output * s (each overwritten, shape of y), and
 * grad_z[m, g] = s (1 - s) * sum_c grad_output * (v - y) (overwritten, shape
 * of z).  grad_y or grad_v may be the same buffer as grad_output.  Same sizes
 * and errors as dcn_center_gate_forward. */
int dcn_center_gate_backward(const void* y, const void* v, const void* z, const void* grad_output,
                             void* grad_y, void* grad_v, void* grad_z, long long M, int G, int Cg,
                             int dtype, void* stream);

/* A projection of the DCNv4 layer ([FB] section 3: the module's input and
 * output projections and the fully connected offset/mask layer; [A100]
 * section 1 merges the latter into one):
 *
 *   y[m, n] = sum_k x[m, k] * w[n, k] + bias[n]
 *
 * x (M, K), w (N, K) and y (M, N) are dense row-major in one dtype; bias (N)
 * may be NULL (no bias).  Products and sums are binary32 (half-precision
 * products are exact), y is rounded once.  M >= 0 (M == 0 is a no-op),
 * N, K >= 1.  Returns DCN_OK, DCN_ERR_INVALID_ARG (bad size or dtype, a NULL
 * or misaligned pointer), DCN_ERR_UNSUPPORTED (K not a multiple of 4, x, w
 * or y not 16-byte aligned, or K > 636 in binary32 / 1208 in half
 * precision, whose 64 rows of w would not fit in on-chip memory) or
 * DCN_ERR_HIP.  A caller falls back to another GEMM on DCN_ERR_UNSUPPORTED. */
int dcn_linear_forward(const void* x, const void* w, const void* bias, void* y, long long M, int N, int K,
                       int dtype, void* stream);

/* Weight and bias gradients of a projection (the same layer as
 * dcn_linear_forward), for g (M, O), the gradient of the projection's output,
 * and x (M, I), its input, dense row-major in dtype:
 *
 *   dw[o, i] = sum_m g[m, o] * x[m, i]      (O, I) row-major, in out_dtype
 *   db[o]    = sum_m g[m, o]                (O) in out_dtype, skipped if db is NULL
 *
 * Products and sums are binary32 (half-precision products are exact); the
 * rows are summed in chunks whose binary32 partials are added in a fixed
 * order, so a call gives the same bits on every run.  Each sum is rounded
 * once to out_dtype (DCN_F32 keeps it; DCN_F16 / DCN_BF16 round to nearest
 * even, the parameters' own type in a half-precision layer).  The partials
 * live in a caller-owned device workspace of at least
 * dcn_linear_weight_grad_workspace_size(M, O, I) bytes, 16-byte aligned
 * (overwritten; contents afterwards unspecified).  dw and db are overwritten,
 * also for M == 0 (zeros; g, x and workspace may then be NULL).  M >= 0,
 * O, I >= 1.  Returns DCN_OK, DCN_ERR_INVALID_ARG (bad size, dtype or
 * out_dtype, a NULL or misaligned pointer, a workspace too small),
 * DCN_ERR_UNSUPPORTED (O * I of 2^40 or more, or a size the chunking cannot
 * index) or DCN_ERR_HIP. */
int dcn_linear_weight_grad(const void* g, const void* x, void* dw, void* db, long long M, int O, int I,
                           int dtype, int out_dtype, void* workspace, long long workspace_bytes, void* stream);

/* Workspace bytes dcn_linear_weight_grad needs (0 for M == 0), or minus a
 * dcn_status for invalid sizes. */
long long dcn_linear_weight_grad_workspace_size(long long M, int O, int I);

/* Static, human-readable name of a dcn_status value. */
const char* dcn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DCN_CORE_H */
