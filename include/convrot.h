/*
 * convrot.h -- C ABI of libconvrot.so, the INT8 ConvRot linear layer for
 * AMD MI355X (gfx950).
 *
 * What the layer computes (page "int8 Compute", InvokeAI docs, opening
 * section): the weight is stored as int8 codes with one scale for the whole
 * tensor, coded after a rotation; each call applies that same rotation to its
 * activation, codes it as int8 with one scale per token, and multiplies the
 * two code tensors on the integer matrix units.
 * The rotation is group-wise (same page, "What stays on the default path":
 * groups of 256 in every published build; the synthetic workloads here also
 * use 128) and is applied block after block along K (page "Explanation of
 * INT8 ConvRot", "What is INT8 ConvRot?").  Outputs are bf16 (same page
 * "int8 Compute", "What stays on the default path": BF16/FP16 compute).
 *
 * Definitions used by every entry point (the readings of what the pages
 * leave open):
 *   R   = blockdiag(H_g / sqrt(g)) along K, H_g the Sylvester Hadamard matrix
 *         (H[i][j] = (-1)^popcount(i & j)); applied in fp32 as the radix-2
 *         butterfly with half-span h = 1, 2, ..., g/2 ((a, b) -> (a+b, a-b)),
 *         then one multiply by the float nearest to 1/sqrt(g).
 *   s_w = max |W R| / 127 over the whole weight;   Wq = rne(W R / s_w)
 *   s_x = max_k |x_m R| / 127 per token m;         q_x = rne(x_m R / s_x)
 *         (IEEE fp32 division, round half to even, clamp to [-127, 127];
 *          an all-zero token or weight gets scale 0 and codes 0)
 *   acc = q_x . Wq^T in int32 (exact)
 *   y   = bf16_rne(fmaf((float)acc, s_x[m] * s_w, bias[n]))   (bias 0 if NULL)
 * Repeated calls give the same bytes, whatever the slicing of the tokens or
 * the tile shape (page "int8 Compute": both paths repeat their results
 * exactly, and a streamed model's image equals the resident one's).
 *
 * Conventions for every entry point
 *   - All tensors are row-major and contiguous; bf16 values are raw 16-bit
 *     patterns.  Every pointer argument except `stream` (and the host pointer
 *     noted at convrot_last_error) is a DEVICE pointer on the current HIP
 *     device.  The caller owns every buffer; the library never allocates,
 *     frees or keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every launch is asynchronous on that stream; no entry point waits for
 *     the device, except the check that convrot_linear_guarded runs on its
 *     first call per layer shape and token bucket.  Outputs are valid once
 *     the stream has reached the call.
 *   - Argument errors are found before any launch and return a negative
 *     status without touching the device; convrot_last_error() then holds a
 *     message.  A failed launch returns CONVROT_EHIP.  Faults inside a kernel
 *     surface at the caller's next synchronisation and are not recoverable.
 *   - Group sizes: 128 or 256 (else CONVROT_EUNSUPPORTED).  K must be a
 *     multiple of the group and at most 131072 (so 127*127*K < 2^31).
 *     M = 0 is a valid empty batch (nothing is launched); N >= 1.
 *   - x, xq, wq, y and workspace must be 16-byte aligned (CONVROT_EALIGN).
 *   - No entry point falls back to another implementation: an unsupported
 *     request is an error.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVROT_ABI_VERSION 1

enum convrot_status {
    CONVROT_OK = 0,
    CONVROT_EINVAL = -1,        /* bad size, NULL pointer, K % group != 0, ... */
    CONVROT_EUNSUPPORTED = -2,  /* group not in {128, 256}, unknown dtype     */
    CONVROT_EALIGN = -3,        /* a pointer is not 16-byte aligned           */
    CONVROT_EWORKSPACE = -4,    /* workspace missing or too small             */
    CONVROT_EHIP = -5           /* a HIP launch or query failed               */
};

enum convrot_dtype { CONVROT_F32 = 0, CONVROT_BF16 = 1, CONVROT_F16 = 2 };

/* Weight scale granularity of the _ex entry points: one scale for the whole
 * weight (int8_tensorwise) or one per output channel (row n of W). */
enum convrot_scale_mode { CONVROT_SCALE_TENSOR = 0, CONVROT_SCALE_ROW = 1 };

/* CONVROT_ABI_VERSION of the built library. */
int convrot_abi_version(void);

/* Message of the last failed call on this thread (host pointer to static,
 * thread-local storage; "" if none).  Valid until the next call. */
const char *convrot_last_error(void);

/* ---------------------------------------------------------------- weights */

/* Workspace bytes convrot_prepare_weight needs (a few bytes for the global
 * absmax; the same for every shape). */
size_t convrot_prepare_weight_workspace(int64_t N, int64_t K);

/* Offline weight preparation (page "int8 Compute": builds ship the weight
 * already rotated and int8_tensorwise quantized; this makes such a build
 * from a float weight).
 *   w           [N, K] weight, fp32 (w_dtype CONVROT_F32) or bf16 (CONVROT_BF16),
 *               PyTorch nn.Linear layout (out x in, K contiguous).
 *   wq_out      [N, K] int8 codes of W R.
 *   w_scale_out one float on the device: s_w.
 *   workspace   >= convrot_prepare_weight_workspace(N, K) bytes, device.
 * Two passes over w (rotate + global absmax, then rotate + quantize). */
int convrot_prepare_weight(const void *w, int w_dtype, int64_t N, int64_t K, int group,
                           int8_t *wq_out, float *w_scale_out,
                           void *workspace, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- forward */

/* Workspace bytes convrot_linear needs: codes and scales of one slice of
 * min(M, 2N) tokens (page "int8 Compute", "Memory": the activation is coded
 * a slice at a time, no slice taller than two output widths, which keeps the
 * working memory within the 2*N*K bytes an unpacked bf16 weight takes). */
size_t convrot_linear_workspace(int64_t M, int64_t K, int64_t N);

/* The whole layer: y = dequant(rotate_quant(x) . Wq^T) + bias.
 *   x_bf16    [M, K] bf16 activation.
 *   wq        [N, K] int8 and w_scale (one float, device) from
 *             convrot_prepare_weight with the same group.
 *   bias_bf16 [N] bf16 or NULL.
 *   y_bf16    [M, N] bf16 output (must not overlap the inputs).
 *   workspace ws_bytes of device scratch.  Tokens are processed in slices of
 *             S = min(M, 2N, ws_bytes / (K + 4) rounded down to a multiple
 *             of 16 (or M if smaller)) rows; a workspace too small for one
 *             slice of min(M, 2N, 16) rows is CONVROT_EWORKSPACE.
 *             The result does not depend on S.
 * Per slice: one rotate+quant launch, then one GEMM+epilogue launch. */
int convrot_linear(const void *x_bf16, int64_t M, int64_t K,
                   const int8_t *wq, const float *w_scale, int64_t N, int group,
                   const void *bias_bf16, void *y_bf16,
                   void *workspace, size_t ws_bytes, void *stream);

/* convrot_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without a workspace.  The codes and scales of a slice
 * live in a library-owned device array of CONVROT_NOALLOC_SCRATCH_BYTES
 * (32 MiB) per GPU, allocated when the library's code object is loaded on
 * that GPU and held until the process ends; its address is looked up once
 * per device.  The call allocates nothing and runs the same kernels as
 * convrot_linear with that array as its workspace, so its slices hold
 * S = min(M, 2N, CONVROT_NOALLOC_SCRATCH_BYTES / (K + 4) rounded down to a
 * multiple of 16) tokens and the bytes written equal convrot_linear's.
 * Errors are those of convrot_linear; a K whose minimum slice would not fit
 * the array is CONVROT_EWORKSPACE (no K <= 131072 reaches it).  Calls on one
 * GPU share its array: calls on one stream are ordered, but calls whose work
 * overlaps on the GPU (different streams, or several host threads) race on
 * it and must be serialised by the caller.  Nothing in the array needs to
 * start at zero: every byte a slice reads, that slice has written. */
#define CONVROT_NOALLOC_SCRATCH_BYTES (32u << 20)
int convrot_linear_noalloc(const void *x_bf16, int64_t M, int64_t K,
                           const int8_t *wq, const float *w_scale, int64_t N, int group,
                           const void *bias_bf16, void *y_bf16, void *stream);

/* ---------------------------------------------------------------- stages
 * The same kernels convrot_linear launches, exposed one by one. */

/* Rotate + per-token quantization: xq [M, K] int8, x_scale [M] fp32. */
int convrot_rotate_quant(const void *x_bf16, int64_t M, int64_t K, int group,
                         int8_t *xq, float *x_scale, void *stream);

/* Raw int32 products acc [M, N] = xq . wq^T (xq [M, K], wq [N, K] int8).
 * Runs the GEMM main loop of convrot_gemm_dequant with an int32 store in
 * place of the epilogue.  K a multiple of 128, at most 131072. */
int convrot_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                     int32_t *acc, void *stream);

/* GEMM + fused epilogue: y [M, N] bf16 = bf16_rne(fmaf((float)(xq . wq^T),
 * x_scale[m] * w_scale[0], bias[n])).  x_scale [M] and w_scale [1] are
 * device fp32; bias_bf16 [N] or NULL.  K a multiple of 128, at most 131072. */
int convrot_gemm_dequant(const int8_t *xq, const float *x_scale,
                         const int8_t *wq, const float *w_scale,
                         const void *bias_bf16, void *y_bf16,
                         int64_t M, int64_t N, int64_t K, void *stream);

/* ---------------------------------------------------------------- variants
 * The layer in FP16 (page "int8 Compute", "What stays on the default path":
 * compute is offered in BF16 or FP16) and with one weight scale per output
 * channel (page "Explanation of INT8 ConvRot", format table: row-wise
 * scaling).  Same kernels and the same definitions as above, except:
 *   - io_dtype / x_dtype CONVROT_F16: the activation, the bias and the output
 *     are IEEE binary16 bit patterns; fp16 -> fp32 widening is exact and the
 *     output is fp16_rne(fmaf(...)), with overflow to infinity;
 *   - scale_mode CONVROT_SCALE_ROW: s_w holds N scales, each row of W R is
 *     quantized like a token (s_w[n] = max_k |(W R)[n][k]| / 127), and the
 *     epilogue uses alpha = s_x[m] * s_w[n] (one fp32 product).
 * io_dtype / x_dtype: CONVROT_BF16 or CONVROT_F16, else
 * CONVROT_EUNSUPPORTED; scale_mode: CONVROT_SCALE_TENSOR or CONVROT_SCALE_ROW,
 * else CONVROT_EUNSUPPORTED.  Every other rule is that of the entry point
 * without _ex. */

/* convrot_prepare_weight with w_dtype CONVROT_F32, CONVROT_BF16 or
 * CONVROT_F16 and a scale mode; w_scale_out has 1 (tensor) or N (row)
 * floats.  The workspace is that of convrot_prepare_weight (row mode leaves
 * it untouched). */
int convrot_prepare_weight_ex(const void *w, int w_dtype, int64_t N, int64_t K, int group,
                              int scale_mode, int8_t *wq_out, float *w_scale_out,
                              void *workspace, size_t ws_bytes, void *stream);

/* convrot_rotate_quant for a bf16 or fp16 activation. */
int convrot_rotate_quant_ex(const void *x, int x_dtype, int64_t M, int64_t K, int group,
                            int8_t *xq, float *x_scale, void *stream);

/* convrot_gemm_dequant with a scale mode (w_scale: 1 or N floats) and bf16
 * or fp16 bias (nullable) and output. */
int convrot_gemm_dequant_ex(const int8_t *xq, const float *x_scale, const int8_t *wq,
                            const float *w_scale, int scale_mode, const void *bias, void *y,
                            int io_dtype, int64_t M, int64_t N, int64_t K, void *stream);

/* convrot_linear with bf16 or fp16 activation, bias and output, and a scale
 * mode.  Same workspace (convrot_linear_workspace) and slicing. */
int convrot_linear_ex(const void *x, int io_dtype, int64_t M, int64_t K, const int8_t *wq,
                      const float *w_scale, int scale_mode, int64_t N, int group,
                      const void *bias, void *y, void *workspace, size_t ws_bytes,
                      void *stream);

/* ---------------------------------------------------------------- streamed weights
 * Page "int8 Compute", "Partially loaded models": when a layer's weight lives
 * in host memory, the int8 codes (half the size of an unpacked bf16 weight)
 * cross to the GPU on every step and the layer runs as it would with the
 * weight resident, with no change in the result's bits.  convrot_linear_streamed runs a sequence of layers
 * whose int8 weights live in pinned host memory: each weight is copied into
 * one of two device slots on `copy_stream` while the previous layer computes
 * on `stream`, and each layer then runs exactly as convrot_linear on its slot
 * (same kernels, same bits).  A slot is refilled only after the layer that
 * used it two steps earlier has finished; the first copy waits for the work
 * already queued on `stream`.  The layers run in order on `stream`; when
 * `stream` reaches the end of the call every output is complete and nothing
 * of the call is left on `copy_stream`.  Copies overlap compute only when
 * both streams are created streams: HIP's null stream (NULL) orders itself
 * against the other streams, which serialises copy and compute (the results
 * are the same). */
typedef struct convrot_stream_layer {
    const void   *x;         /* device, bf16 [M, K] */
    int64_t       M, K, N;
    const int8_t *wq_host;   /* HOST, pinned (hipHostMalloc or torch pin_memory), int8 [N, K],
                                as written by convrot_prepare_weight */
    const float  *w_scale;   /* device, 1 float */
    int           group;     /* 128 or 256 */
    const void   *bias;      /* device, bf16 [N], or NULL */
    void         *y;         /* device, bf16 [M, N] */
} convrot_stream_layer;

/* Bytes one weight slot needs: the largest N*K of the layers, rounded up to
 * 256.  0 if n_layers < 1 or layers is NULL. */
size_t convrot_stream_slot_bytes(const convrot_stream_layer *layers, int n_layers);

/* layers: host array of n_layers >= 0 descriptors (read during the call only).
 * slots: device, 2 * slot_bytes, 16-byte aligned, slot_bytes >= every N*K.
 * workspace / ws_bytes: as for convrot_linear, enough for every layer (the
 * layers run one after another on `stream` and share it).
 * Every layer is checked before anything is queued: the convrot_linear rules
 * (CONVROT_EINVAL, CONVROT_EUNSUPPORTED, CONVROT_EALIGN, CONVROT_EWORKSPACE),
 * a slot too small (CONVROT_EWORKSPACE) and a weight that is not pinned host
 * memory (CONVROT_EINVAL); nothing is queued then.  HIP errors while queueing
 * return CONVROT_EHIP (work queued so far stays queued). */
int convrot_linear_streamed(const convrot_stream_layer *layers, int n_layers,
                            void *slots, size_t slot_bytes, void *workspace, size_t ws_bytes,
                            void *copy_stream, void *stream);

/* ---------------------------------------------------------------- default path and guarded layer
 * Page "int8 Compute" (InvokeAI docs):
 *   - "What stays on the default path": layers outside the int8 path keep
 *     unpacking their weights per forward.  Here the default path of a
 *     rotated int8 weight is: dequantize each row (s * q in fp32, s the
 *     tensor scale or the row's), rotate it back by R (R is symmetric and
 *     orthogonal, so R^-1 = R: the same fp32 butterfly and multiply as
 *     above), round to the compute dtype (bf16 or fp16, RNE); the layer is
 *     then y = rnd(x . Wu^T + bias), the product in the compute dtype with an
 *     fp32 accumulator on the bf16/fp16 matrix cores.  The activation is not
 *     rotated or quantized.
 *   - "When something goes wrong": a new combination of layer shape and
 *     batch-size bucket is verified once against the default path; on a
 *     disagreement or a kernel error a single warning is written and the
 *     device stays on the default path for the rest of the process.
 *   - "Memory": the default path reserves the unpacked weight (2*N*K bytes);
 *     the check keeps 256 rows of the layer's output from each path.
 *   - "Enabling": a line is logged once per GPU when the int8 path is first
 *     used on it.
 */

/* Bytes of workspace convrot_default_linear needs: the unpacked weight,
 * 2*N*K rounded up to 256.  0 for a bad size. */
size_t convrot_default_workspace(int64_t K, int64_t N);

/* Unpack a rotated int8 weight (as written by convrot_prepare_weight[_ex]):
 * wu[n][k] = rnd((W_n R)[k]) of the dequantized row W_n = s * wq[n], rnd =
 * bf16 (out_dtype CONVROT_BF16) or fp16 (CONVROT_F16).  wq: int8 [N, K];
 * w_scale: 1 float (CONVROT_SCALE_TENSOR) or N (CONVROT_SCALE_ROW); wu: 16-bit
 * [N, K].  Same checks as convrot_prepare_weight_ex (group, K, N, alignment of
 * wq and wu, dtype and scale mode). */
int convrot_unpack_weight(const int8_t *wq, const float *w_scale, int scale_mode, int64_t N, int64_t K,
                          int group, int out_dtype, void *wu, void *stream);

/* The default path for a whole batch: unpack the weight into the workspace
 * (convrot_default_workspace bytes), then y = rnd(x . Wu^T + bias).  Arguments
 * as convrot_linear_ex (x, bias and y in io_dtype); the same checks.  The
 * product accumulates in fp32 on the matrix cores in an order that depends
 * on the tile the shape takes (batches of at most 16 tokens with many
 * channels split K over four waves), so y agrees with the exact value within
 * one output ulp plus the fp32 bound of a K-term sum; a given shape repeats
 * its bytes from call to call. */
int convrot_default_linear(const void *x, int io_dtype, int64_t M, int64_t K, const int8_t *wq,
                           const float *w_scale, int scale_mode, int64_t N, int group,
                           const void *bias, void *y, void *workspace, size_t ws_bytes,
                           void *stream);

/* Bytes of workspace convrot_linear_guarded needs: enough for
 * convrot_linear_ex and for the check (the unpacked weight, 256 gathered
 * activation rows, 256 default-path output rows and the per-row sums). */
size_t convrot_guarded_workspace(int64_t M, int64_t K, int64_t N);

/* The int8 layer (convrot_linear_ex), guarded.  Per device (the current HIP
 * device), the library keeps: the set of (N, K, group, io dtype, scale mode,
 * token bucket) already checked, where the token bucket is M rounded up to a
 * power of two, and a sticky fallback flag.
 *   - Fallback set: the call runs convrot_default_linear.
 *   - Else the int8 layer runs.  If its launch fails, the fallback is set
 *     (one warning) and the call reruns on the default path.
 *   - On the first call for a bucket the default path is also run on
 *     R = min(M, 256) rows spread evenly over the batch (row_i =
 *     i * (M - 1) / (R - 1)), and the call waits for the stream to compare
 *     them: the int8 result matches when no value of its R rows is
 *     non-finite where the default path's is not (or the reverse) -- the
 *     same infinity on both, an output past the io type's range, agrees and
 *     is left out of the norms -- and
 *     ||y_int8 - y_default||_F / ||y_default||_F <= tol over those rows
 *     (tol = 0.1 unless configured; the int8 layer differs from the default
 *     path by its activation quantization).  A match marks the bucket
 *     checked; a mismatch sets the fallback (one warning) and recomputes
 *     the whole output on the default path.
 * Argument errors return as for convrot_linear_ex and change no state.  A
 * checking call cannot be captured into a graph: it returns
 * CONVROT_EUNSUPPORTED if `stream` is capturing (run one call per bucket
 * first).  Calls that need no check add no synchronisation.  Concurrent
 * calls are safe; the state is guarded by a lock. */
int convrot_linear_guarded(const void *x, int io_dtype, int64_t M, int64_t K, const int8_t *wq,
                           const float *w_scale, int scale_mode, int64_t N, int group,
                           const void *bias, void *y, void *workspace, size_t ws_bytes,
                           void *stream);

/* Guard state of one device, for logs and tests. */
typedef struct convrot_guard_info {
    int     fallback;       /* 1: this device runs the default path */
    int64_t checked;        /* buckets checked and matched */
    int64_t checks_run;     /* checks run (matched or not) */
    double  last_error;     /* relative error of the latest check; -1 if none */
    char    message[256];   /* the latest log line for this device, "" if none */
} convrot_guard_info;

/* Host pointer info.  CONVROT_EINVAL for a NULL pointer or a negative device. */
int convrot_guard_query(int device, convrot_guard_info *info);

/* Forget the state of one device (checked buckets, fallback, pending
 * injection).  CONVROT_EINVAL for a negative device. */
int convrot_guard_reset(int device);

/* Match tolerance (finite, > 0) and whether log lines also go to stderr
 * (they are always kept in convrot_guard_info.message).  Applies to every
 * device.  CONVROT_EINVAL for a bad tolerance. */
int convrot_guard_configure(double tol, int log_to_stderr);

/* Fault injection from the host, for tests of the guard: arms one fault on
 * a device, consumed by the next convrot_linear_guarded call there that runs
 * the int8 layer.  CONVROT_FAULT_MISMATCH makes that call's check see the
 * int8 rows negated (and runs the check even if the bucket was checked);
 * CONVROT_FAULT_KERNEL makes the int8 launch report a failure.  Nothing is
 * done to the GPU.  CONVROT_EINVAL for an unknown fault or a negative
 * device. */
enum convrot_fault { CONVROT_FAULT_NONE = 0, CONVROT_FAULT_MISMATCH = 1, CONVROT_FAULT_KERNEL = 2 };
int convrot_guard_inject(int device, int fault);

/* ---------------------------------------------------------------- measurement aid
 * Not a step of the layer and defined by no page: it exists so that a
 * benchmark can state the rate the matrix cores sustain on this machine,
 * under its power limit, for given operand bytes.
 *
 * Runs `blocks` workgroups of twelve waves (three per SIMD).  Every lane
 * loads four 16-byte fragments from a and four from b (a_bytes / 16 and
 * b_bytes / 16 fragments are cycled through), then issues iters x 16
 * independent v_mfma_i32_16x16x64_i8 from registers, and writes one int32
 * checksum to out[blocks * 768].  Integer ops per call:
 * blocks * 12 * iters * 16 * 32768.  a, b and out are 16-byte aligned device
 * buffers owned by the caller; asynchronous on `stream`.
 * Errors: NULL buffer, buffers under 16 bytes, blocks outside [1, 2^20] or
 * iters < 1 -> CONVROT_EINVAL; misalignment -> CONVROT_EALIGN; launch error
 * -> CONVROT_EHIP. */
int convrot_probe_mfma_i8(const int8_t *a, int64_t a_bytes, const int8_t *b, int64_t b_bytes,
                          int blocks, int iters, int32_t *out, void *stream);

/* A second measurement aid, also defined by no page: the traffic of
 * rotate + quant without its arithmetic, so that a benchmark can state what
 * this machine's HBM sustains for exactly that traffic.  Reads n 16-bit
 * values from x_16 and writes the high byte of each to q[n] (q[i] =
 * x_16[i] >> 8), 16-byte loads and 8-byte stores, grid-stride over at most
 * 2048 workgroups.  x_16 and q are 16-byte aligned device buffers owned by
 * the caller; asynchronous on `stream`; n = 0 is a no-op.
 * Errors: n negative or not a multiple of 8, NULL buffer (n > 0) ->
 * CONVROT_EINVAL; misalignment -> CONVROT_EALIGN; launch error ->
 * CONVROT_EHIP. */
int convrot_probe_stream(const void *x_16, int64_t n, int8_t *q, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
