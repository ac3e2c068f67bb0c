/*
 * ptb.h -- C ABI of libptb: one Parallel Transformer Block (PTB) layer,
 * forward and backward, on one AMD Instinct MI355X (gfx950).
 *
 * The layer (MegaScale reading notes, "MegaScale: ByteDance 如何在 12,288 块
 * GPU 上实现 55% MFU 的大规模 LLM 训练", section 1.1, eq (4)):
 *
 *     a = LN(x)                       LayerNorm with gamma, beta, eps
 *     y = x + Attn(a) W_o + GeLU(a W_fc1) W_fc2
 *     Attn: causal sliding-window attention per head (same notes, section 1.1,
 *           eq (5)-(6)): query i sees the `window` most recent tokens, itself
 *           included (keys j with 0 <= i - j < window); softmax scale
 *           1/sqrt(head_dim); q, k, v are column blocks of a W_qkv.
 *     MLP:  Y = GeLU(X A) B with exact-erf GeLU, no biases (Megatron-LM
 *           tensor-parallel explainer, section 2.1).
 *
 * Both branches read the same LayerNorm output.  The backward recomputes the
 * attention probabilities from the saved log-sum-exp instead of storing them
 * (selective recompute of the core attention: MegaScale notes, section 1.3;
 * Megatron tuning post "显存与性能调优", recompute section).
 *
 * Tensors.  Every tensor argument is a DEVICE pointer to bfloat16 values
 * (stored as raw 16-bit words), row-major and contiguous, 16-byte aligned.
 * T = batch*seq tokens, token t = batch_index*seq + position.
 * h = hidden, h_l = heads*head_dim, f = ffn.
 *     x, y, dy, dx  [T, h]
 *     ln_gamma, ln_beta, d_ln_gamma, d_ln_beta  [h]
 *     w_qkv  [h, 3*h_l]   columns [Q heads | K heads | V heads]; head j's
 *                         head_dim columns are contiguous inside each block
 *     w_o    [h_l, h]     rows in the same head order
 *     w_fc1  [h, f]       ([h, 2f] for the SwiGLU variant, see ptb_dims.mlp)
 *     w_fc2  [f, h]
 * Gradients have the shape of what they differentiate.  Arithmetic is bf16
 * operands with fp32 accumulation; LayerNorm statistics and the attention
 * log-sum-exp are fp32.
 *
 * Ownership and lifetime.  The caller allocates and owns every buffer,
 * including `saved` (ptb_saved_bytes) and `workspace` (ptb_workspace_bytes).
 * The library allocates nothing.  Its only mutable global state is a
 * per-device cache of the compute-unit count (set once, with the same value,
 * by whichever call comes first) and, for the one allocation-free call
 * (ptb_lamb_step_noalloc), the per-device address of its static scratch
 * array; each calling thread also keeps, in thread-local storage, the
 * attention chunk lengths it computed for its last four shapes (the same
 * value a fresh computation gives).  Calls on different streams with
 * different buffers (workspace included) may run concurrently.  `saved` is written by ptb_forward and read by ptb_backward;
 * it must stay untouched in between.  `workspace` is scratch for the duration
 * of one call: its contents need no initialisation and are not kept.
 * Outputs are overwritten, never accumulated into.
 *
 * Asynchrony.  `stream` is a hipStream_t (NULL = the default stream).  Calls
 * only enqueue kernels on it and never synchronise; a fault inside a kernel
 * surfaces at the caller's next synchronisation of that stream.
 *
 * Errors.  Every entry point returns PTB_OK (0) or a negative PTB_ERR_* code.
 * All argument checks are done on the host before the first HIP call, so an
 * invalid call enqueues nothing.  PTB_ERR_HIP reports a failed kernel launch
 * (hipGetLastError after a launch).  No C++ exception crosses this boundary.
 */
#ifndef PTB_H_
#define PTB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PTB_ABI_VERSION 11

enum ptb_status {
  PTB_OK = 0,
  PTB_ERR_NULL = -1,      /* a required pointer is NULL                         */
  PTB_ERR_DIMS = -2,      /* a size is < 1, not a multiple of 64 where required,
                             or too large (see ptb_validate_dims)               */
  PTB_ERR_HEAD_DIM = -3,  /* head_dim is not 64 or 128                          */
  PTB_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned                   */
  PTB_ERR_WINDOW = -5,    /* window < 1                                         */
  PTB_ERR_EPS = -6,       /* ln_eps is not a finite positive number             */
  PTB_ERR_HIP = -7,       /* a kernel launch failed                             */
  PTB_ERR_ARG = -8,       /* invalid layer variant (norm, mlp), optimizer
                             hyper-parameters or tensor list                    */
  PTB_ERR_SCRATCH = -9    /* an allocation-free call needs more scratch than
                             the library's static buffer holds                 */
};

typedef struct ptb_dims {
  int32_t batch;     /* b >= 1                                                */
  int32_t seq;       /* s >= 1                                                */
  int32_t hidden;    /* h: multiple of 64, 64 <= h <= 16384                   */
  int32_t heads;     /* n >= 1 (heads of this GPU's share)                    */
  int32_t head_dim;  /* d: 64 or 128                                          */
  int32_t ffn;       /* f: multiple of 64, >= 64                              */
  int32_t window;    /* w >= 1; w >= seq is full causal attention             */
  float ln_eps;      /* LayerNorm epsilon, added to the variance, > 0         */
  int32_t norm;      /* PTB_NORM_LAYERNORM (0) or PTB_NORM_RMSNORM (1)         */
  int32_t mlp;       /* PTB_MLP_GELU (0) or PTB_MLP_SWIGLU (1)                 */
  float dropout_p;          /* dropout rate, 0 <= p < 1; 0 = no dropout        */
  uint32_t dropout_layer;   /* this layer's index (< 2^31): picks its masks    */
  uint64_t dropout_seed;    /* generator key                                   */
} ptb_dims;

/* Dropout (MegaScale notes, section 1.3: dropout fused into the layer, its
 * activations kept for backward).  With dropout_p = p > 0 the block's branch
 * output is dropped before the residual add:
 *   parallel block  y  = x  + D0 * (Attn(a) W_o + MLP(a))
 *   serial block    x1 = x  + D0 * Attn(a1) W_o,   y = x1 + D1 * MLP(a2)
 * where D_b is 0 for a dropped element and 1/(1 - p) (fp32) for a kept one.
 * Element e = t h + c of the [T, h] branch output is kept iff word e & 3 of
 * Philox-4x32-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2,
 * 3", SC'11) of the counter (e >> 2, 2 dropout_layer + b, 0, 0) under the key
 * (dropout_seed mod 2^32, dropout_seed >> 32) is >= floor(p 2^32).  The mask
 * is never stored: the forward's [O ; FC2] epilogue applies it, and the
 * backward regenerates it from the same key (the "kept" activation is the
 * key); pass the same dims to both.  ptb_dropout_mask writes the mask itself.
 * The FP8 calls take p = 0 only (PTB_ERR_ARG otherwise).  A zero-initialised
 * ptb_dims has no dropout. */

/* Layer variants (MegaScale notes, section 1.3: the fused RMSNorm and SwiGLU
 * kernels of MegaScale's own model; the default is the layer above).
 *   PTB_NORM_RMSNORM: a = gamma * x / sqrt(mean(x^2) + ln_eps); ln_beta is
 *     ignored (it must still be a valid pointer) and d_ln_beta is written as
 *     zeros; the stashed row mean (PTB_SAVED_MU) is 0.
 *   PTB_MLP_SWIGLU: MLP(a) = (silu(a W1) * (a W3)) W2, silu(u) = u sigmoid(u),
 *     no biases.  W1 and W3 [h, f] travel as one w_fc1 [h, 2f] whose columns
 *     are 32-wide blocks alternating W1 and W3: block 2j holds W1 columns
 *     32j .. 32j+31 and block 2j+1 the same columns of W3; dw_fc1 has the same
 *     layout, w_fc2 stays [f, h]; PTB_SAVED_U holds [a W1 | a W3] in that
 *     layout ([T, 2f]) and PTB_SAVED_G silu(a W1) * (a W3) [T, f]. */
enum ptb_norm_kind { PTB_NORM_LAYERNORM = 0, PTB_NORM_RMSNORM = 1 };
enum ptb_mlp_kind { PTB_MLP_GELU = 0, PTB_MLP_SWIGLU = 1 };

/* Version of this ABI (PTB_ABI_VERSION). */
int32_t ptb_abi_version(void);

/* Static description of a status code.  Never NULL. */
const char* ptb_status_string(int32_t status);

/* Check `dims` alone.  Besides the per-field rules above, every tensor of the
 * layer must hold fewer than 2^30 elements (T*(3*h_l+f), h*(3*h_l+f), ...),
 * i.e. stay below 2 GiB. */
int32_t ptb_validate_dims(const ptb_dims* dims);

/* Bytes of the forward->backward stash of one layer (`saved`). */
int32_t ptb_saved_bytes(const ptb_dims* dims, size_t* bytes);

/* Bytes of scratch (`workspace`) that ptb_forward and ptb_backward need:
 * fp32 partial sums of matrix-product tiles that are split over several
 * workgroups, their arrival counters, the forward's fp16 copy of the q, k
 * columns of W_qkv, and the backward's intermediate gradients (dc, dZ, da,
 * the LayerNorm column partials). */
int32_t ptb_workspace_bytes(const ptb_dims* dims, size_t* bytes);

/* Byte offsets inside `saved` of what ptb_forward stores there, for
 * inspection by tests and tools (the backward needs no caller help):
 *   PTB_SAVED_A    a = LN(x)                 bf16 [T, h]
 *   PTB_SAVED_MU   row mean of x             fp32 [T]
 *   PTB_SAVED_RSTD 1/sqrt(var + eps)         fp32 [T]
 *   PTB_SAVED_QKV  a W_qkv                   bf16 [T, 3*h_l]
 *   PTB_SAVED_U    a W_fc1 (pre-activation)  bf16 [T, f] ([T, 2f] for SwiGLU)
 *   PTB_SAVED_G    GeLU(u)                   bf16 [T, f]
 *   PTB_SAVED_C    attention output          bf16 [T, h_l] (head-major cols)
 *   PTB_SAVED_LSE  base-2 log-sum-exp of the logits scaled by log2(e)/sqrt(d)
 *                                            fp32 [b, n, s]
 *   PTB_SAVED_A16  fp16 copy of LN(x)         fp16 [T, h]
 *   PTB_SAVED_QK16 the q and k columns of qkv in fp16: a16 W_q|k with fp16
 *                  operands and fp32 sums    fp16 [T, 2*h_l]
 * The logits q.k/sqrt(d) are one fp16 product of these q and k (10 mantissa
 * bits instead of bf16's 7): with the large logits of wide layers a bf16
 * rounding of LN(x), q or k shifts every logit by a few thousandths, which
 * the softmax turns into a comparable relative error of the attention output
 * and of the q, k gradients.  fp16 has a narrower range than bf16: q, k and
 * LN(x) are saturated at +-65504 (far outside what a LayerNorm output and
 * 0.02-scale weights produce), and weights below 2^-14 in magnitude enter the
 * q, k product as fp16 subnormals (absolute error <= 2^-25).
 * `offsets` must have room for PTB_SAVED_COUNT entries. */
enum ptb_saved_slot {
  PTB_SAVED_A = 0, PTB_SAVED_MU, PTB_SAVED_RSTD, PTB_SAVED_QKV, PTB_SAVED_U,
  PTB_SAVED_G, PTB_SAVED_C, PTB_SAVED_LSE, PTB_SAVED_A16, PTB_SAVED_QK16,
  PTB_SAVED_COUNT
};
int32_t ptb_saved_layout(const ptb_dims* dims, size_t* offsets);

/* Forward of one layer (MegaScale notes, section 1.1, eq (4)):
 *   y = x + Attn(LN(x)) + MLP(LN(x)).
 * Writes y [T, h] and fills `saved` (ptb_saved_bytes(dims) bytes);
 * `workspace` holds ptb_workspace_bytes(dims) bytes of scratch. */
int32_t ptb_forward(const ptb_dims* dims,
                    const void* x,
                    const void* ln_gamma, const void* ln_beta,
                    const void* w_qkv, const void* w_o,
                    const void* w_fc1, const void* w_fc2,
                    void* y, void* saved, void* workspace, void* stream);

/* Backward of one layer (the gradient of eq (4), MegaScale notes, section
 * 1.1) for upstream gradient dy [T, h], reading the `saved` of the matching
 * ptb_forward and the same x and weights.  The attention probabilities are
 * recomputed from the saved log-sum-exp, never stored (selective recompute
 * of the core attention, same notes, section 1.3).  Writes dx (which
 * includes the residual path dy), d_ln_gamma, d_ln_beta and the four weight
 * gradients.  `workspace` holds ptb_workspace_bytes(dims) bytes of scratch. */
int32_t ptb_backward(const ptb_dims* dims,
                     const void* dy, const void* x,
                     const void* ln_gamma,
                     const void* w_qkv, const void* w_o,
                     const void* w_fc1, const void* w_fc2,
                     const void* saved,
                     void* dx, void* d_ln_gamma, void* d_ln_beta,
                     void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2,
                     void* workspace, void* stream);

/* Dropout mask of `n` elements (e = 0 .. n-1) of one generator stream, as the
 * layer draws it: mask[e] = 1 if element e is kept, 0 if dropped (device
 * bytes, caller-owned).  stream = 2 * layer (+ 1 for the serial block's MLP
 * branch).  PTB_ERR_ARG unless 0 <= p < 1 and 0 <= n < 2^32 - 4. */
int32_t ptb_dropout_mask(uint64_t seed, uint32_t stream, float p, int64_t n, void* mask,
                         void* stream_handle);

/* Stage timing.  The same calls with an array of hipEvent_t handles
 * (`stage_events`, 2 per stage, NULL entries skipped): event 2*i is recorded on
 * `stream` right before stage i is enqueued and event 2*i+1 right after it, so
 * hipEventElapsedTime(events[2i], events[2i+1]) is the device time of stage i.
 * The events are created and owned by the caller.  Stages:
 *   forward  (PTB_FWD_STAGES = 5): 0 LayerNorm, 1 fp16 copy of the q, k
 *            columns of W_qkv, 2 [QKV | FC1] GEMM + GeLU, 3 attention,
 *            4 [O ; FC2] GEMM + residual;
 *   backward (PTB_BWD_STAGES = 6): 0 dgrad [O ; FC2] + GeLU' (under dropout
 *            preceded by the regenerated mask applied to dy), 1 attention
 *            backward (3 kernels), 2 wgrad [O ; FC2], 3 dgrad [QKV | FC1],
 *            4 wgrad [QKV | FC1], 5 LayerNorm backward (2 kernels).
 * Each GEMM stage is exactly one kernel launch.  Each call also clears the
 * tile counters in `workspace`: the forward inside stage 0's LayerNorm
 * launch, the backward with one small kernel ahead of stage 0. */
#define PTB_FWD_STAGES 5
#define PTB_BWD_STAGES 6
int32_t ptb_forward_timed(const ptb_dims* dims,
                          const void* x,
                          const void* ln_gamma, const void* ln_beta,
                          const void* w_qkv, const void* w_o,
                          const void* w_fc1, const void* w_fc2,
                          void* y, void* saved, void* workspace, void* stream,
                          void* const* stage_events);
int32_t ptb_backward_timed(const ptb_dims* dims,
                           const void* dy, const void* x,
                           const void* ln_gamma,
                           const void* w_qkv, const void* w_o,
                           const void* w_fc1, const void* w_fc2,
                           const void* saved,
                           void* dx, void* d_ln_gamma, void* d_ln_beta,
                           void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2,
                           void* workspace, void* stream,
                           void* const* stage_events);

/* ------------------------------------------------------------------------
 * Serial (standard) block, for comparison with the parallel one: the same
 * notes, section 1.1, eq (3), built from the same kernels.  The notes print
 * eq (3) with x alone in the outer sum, y = x + MLP(LN(x + Attn(LN(x)))), but
 * describe the parallel block, eq (4), as this standard block with LN(x) in
 * place of LN(x + Attn(LN(x))) as the MLP's input and nothing else changed;
 * eq (4) keeps Attn(LN(x)) in the outer sum, so the standard block is read
 * with it there too, and with two LayerNorms of their own gamma and beta:
 *     a1 = LN1(x);  x1 = x + Attn(a1) W_o;  a2 = LN2(x1)
 *     y  = x1 + GeLU(a2 W_fc1) W_fc2
 * Attention, GeLU, dims, layouts, weights, ownership, asynchrony and errors
 * are exactly as for ptb_forward / ptb_backward; ln1_* are the parameters of
 * the first LayerNorm (the one ptb_forward calls ln_*), ln2_* [h] those of the
 * second.  The QKV, O, FC1 and FC2 products are separate launches, and the
 * MLP waits for the attention output.  `saved` and `workspace` have their own
 * sizes (ptb_serial_saved_bytes, ptb_serial_workspace_bytes).
 * ------------------------------------------------------------------------ */

/* What ptb_serial_forward stores in `saved` (byte offsets from
 * ptb_serial_saved_layout; `offsets` must have room for
 * PTB_SERIAL_SAVED_COUNT entries):
 *   A1, MU1, RSTD1, A1_16   LN1(x) as for the parallel block (PTB_SAVED_A ...)
 *   QKV, QK16, C, LSE       as PTB_SAVED_QKV, _QK16, _C, _LSE
 *   X1                      x + Attn(a1) W_o          bf16 [T, h]
 *   A2, MU2, RSTD2          LN2(x1) and its row statistics
 *   U, G                    a2 W_fc1 and GeLU of it   bf16 [T, f] */
enum ptb_serial_saved_slot {
  PTB_SERIAL_A1 = 0, PTB_SERIAL_MU1, PTB_SERIAL_RSTD1, PTB_SERIAL_A1_16,
  PTB_SERIAL_QKV, PTB_SERIAL_QK16, PTB_SERIAL_C, PTB_SERIAL_LSE,
  PTB_SERIAL_X1, PTB_SERIAL_A2, PTB_SERIAL_MU2, PTB_SERIAL_RSTD2,
  PTB_SERIAL_U, PTB_SERIAL_G,
  PTB_SERIAL_SAVED_COUNT
};
int32_t ptb_serial_saved_bytes(const ptb_dims* dims, size_t* bytes);
int32_t ptb_serial_workspace_bytes(const ptb_dims* dims, size_t* bytes);
int32_t ptb_serial_saved_layout(const ptb_dims* dims, size_t* offsets);

/* Forward of one serial block: writes y [T, h] and fills `saved`. */
int32_t ptb_serial_forward(const ptb_dims* dims,
                           const void* x,
                           const void* ln1_gamma, const void* ln1_beta,
                           const void* ln2_gamma, const void* ln2_beta,
                           const void* w_qkv, const void* w_o,
                           const void* w_fc1, const void* w_fc2,
                           void* y, void* saved, void* workspace, void* stream);

/* Backward of one serial block for upstream gradient dy [T, h], reading the
 * `saved` of the matching ptb_serial_forward and the same x and weights.
 * Writes dx (residual paths included), the gradients of both LayerNorms'
 * gamma and beta, and the four weight gradients. */
int32_t ptb_serial_backward(const ptb_dims* dims,
                            const void* dy, const void* x,
                            const void* ln1_gamma, const void* ln2_gamma,
                            const void* w_qkv, const void* w_o,
                            const void* w_fc1, const void* w_fc2,
                            const void* saved,
                            void* dx,
                            void* d_ln1_gamma, void* d_ln1_beta,
                            void* d_ln2_gamma, void* d_ln2_beta,
                            void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2,
                            void* workspace, void* stream);

/* Stage timing as for ptb_forward_timed.  Stages:
 *   forward  (PTB_SERIAL_FWD_STAGES = 8): 0 LN1, 1 fp16 copy of W_q|k,
 *            2 QKV GEMM, 3 attention, 4 O GEMM + residual, 5 LN2,
 *            6 FC1 GEMM + GeLU, 7 FC2 GEMM + residual;
 *   backward (PTB_SERIAL_BWD_STAGES = 11): 0 dgrad FC2 + GeLU', 1 wgrad FC2,
 *            2 dgrad FC1, 3 wgrad FC1, 4 LN2 backward (+ dy), 5 dgrad O
 *            (stages 0 and 5 under dropout preceded by the masks),
 *            6 wgrad O, 7 attention backward, 8 dgrad QKV, 9 wgrad QKV,
 *            10 LN1 backward (+ dx1). */
#define PTB_SERIAL_FWD_STAGES 8
#define PTB_SERIAL_BWD_STAGES 11
int32_t ptb_serial_forward_timed(const ptb_dims* dims,
                                 const void* x,
                                 const void* ln1_gamma, const void* ln1_beta,
                                 const void* ln2_gamma, const void* ln2_beta,
                                 const void* w_qkv, const void* w_o,
                                 const void* w_fc1, const void* w_fc2,
                                 void* y, void* saved, void* workspace, void* stream,
                                 void* const* stage_events);
int32_t ptb_serial_backward_timed(const ptb_dims* dims,
                                  const void* dy, const void* x,
                                  const void* ln1_gamma, const void* ln2_gamma,
                                  const void* w_qkv, const void* w_o,
                                  const void* w_fc1, const void* w_fc2,
                                  const void* saved,
                                  void* dx,
                                  void* d_ln1_gamma, void* d_ln1_beta,
                                  void* d_ln2_gamma, void* d_ln2_beta,
                                  void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2,
                                  void* workspace, void* stream,
                                  void* const* stage_events);

/* ------------------------------------------------------------------------
 * LAMB optimizer step (the same notes, section 1.1, eq (7)) over a list of
 * parameter tensors, each its own "layer" for the trust ratio:
 *     m <- beta1 m + (1 - beta1) g,      v <- beta2 v + (1 - beta2) g^2
 *     r  = (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps)
 *     theta <- theta - lr * (||theta|| / ||r||) * r
 * with the norms taken over the whole tensor (theta before the update) and a
 * trust ratio of 1 when either norm is zero.  Eq (7) gives the trust ratio's
 * denominator as ||m/sqrt(v) + eps||; it is read as the norm of the same
 * direction r that the step applies.  No weight decay.  theta, m, v are the
 * fp32 master weights and moments (mixed precision: Megatron tuning post,
 * mixed-precision section), updated in place; the gradient is the bf16
 * output of ptb_backward; `weight` receives bf16(theta) for the next forward
 * (it may be the tensor the gradient belongs to, never the gradient itself).
 * ------------------------------------------------------------------------ */
#define PTB_LAMB_MAX_TENSORS 32

typedef struct ptb_lamb_hyper {
  float lr;      /* learning rate eta, finite                          */
  float beta1;   /* 0 <= beta1 < 1                                     */
  float beta2;   /* 0 <= beta2 < 1                                     */
  float eps;     /* > 0                                                */
  int32_t step;  /* t >= 1: bias corrections 1 - beta^t                */
} ptb_lamb_hyper;

typedef struct ptb_lamb_tensor {
  float* theta;       /* device fp32 [numel], in/out                  */
  float* m;           /* device fp32 [numel], in/out (zero at step 1)  */
  float* v;           /* device fp32 [numel], in/out (zero at step 1)  */
  const void* grad;   /* device bf16 [numel]                           */
  void* weight;       /* device bf16 [numel], out: bf16(theta)         */
  int64_t numel;      /* >= 8, a multiple of 8; < 2^31                 */
} ptb_lamb_tensor;

/* Scratch bytes of one ptb_lamb_step over `tensors` (host array of n). */
int32_t ptb_lamb_workspace_bytes(const ptb_lamb_tensor* tensors, int32_t n, size_t* bytes);

/* One LAMB step over n (1..PTB_LAMB_MAX_TENSORS) tensors, enqueued on
 * `stream`: three kernels (moments and partial norms; norms; update).
 * `tensors` and `hyper` are host memory, read before the call returns.
 * `norms` (device fp32 [n][2], caller-owned) receives ||theta|| (before the
 * update) and ||r|| of each tensor; their ratio is the trust ratio applied.
 * Every device pointer must be non-NULL and 16-byte aligned, tensors must not
 * overlap.  PTB_ERR_ARG for an invalid list or hyper-parameters,
 * PTB_ERR_NULL / PTB_ERR_ALIGN as for the layer calls.  The result is
 * deterministic (fixed reduction order). */
int32_t ptb_lamb_step(const ptb_lamb_hyper* hyper, const ptb_lamb_tensor* tensors, int32_t n,
                      float* norms, void* workspace, void* stream);

/* The same step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight training loops, harnesses that forbid hipMalloc.
 * It takes no workspace: its scratch (two fp64 partial sums per 16384
 * elements of each tensor) lives in a static device array of
 * PTB_LAMB_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds
 * from the first such call until the process ends (its address is looked up
 * once per device).  It calls no allocating routine.  Calls whose
 * ptb_lamb_workspace_bytes exceed that size return PTB_ERR_SCRATCH (the
 * limit is 262144 such blocks, 4.29e9 elements per call); every other check
 * and result is exactly ptb_lamb_step's, with the same kernels.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, no ordering between them) race and must not be issued. */
#define PTB_LAMB_NOALLOC_SCRATCH_BYTES (4u << 20)
int32_t ptb_lamb_step_noalloc(const ptb_lamb_hyper* hyper, const ptb_lamb_tensor* tensors,
                              int32_t n, float* norms, void* stream);

/* ------------------------------------------------------------------------
 * FP8 GEMM variant of the parallel block (Megatron-LM tuning post,
 * mixed-precision section): the four GEMM parts, forward [QKV | FC1] and
 * [O ; FC2] and their dgrad and wgrad products, run on 8-bit float operands
 * with fp32 accumulation; LayerNorm, attention, GeLU, the residual sums and
 * every stored tensor stay bf16/fp32.
 *   formats   E4M3 (OCP; largest 448) for the forward operands and the
 *             weights, E5M2 (largest 57344) for the gradient operands dy and
 *             dZ = [dqkv | du]; the weight gradients take the saved
 *             activations in E4M3;
 *   scaling   current scaling, one scale per GEMM operand, a concatenated
 *             operand ([W_qkv | W_fc1], [W_o ; W_fc2], [c | g], dZ) being one
 *             tensor: s = FMAX / amax (fp32 division; s = 1 for an all-zero
 *             tensor), code = round-to-nearest-even(clamp(x s, -FMAX, FMAX))
 *             with x s one fp32 multiply, and the product's fp32 sums are
 *             multiplied by (1/sA)(1/sB) before the epilogue
 *             (PTB_FP8_CURRENT); or block scaling, mxfp8 as the OCP
 *             Microscaling Formats v1.0 define it (PTB_FP8_MX): blocks of 32
 *             values along each product's contraction dimension, one E8M0
 *             scale 2^X per block with X = floor(log2 amax_block) - emax
 *             (emax 8 for E4M3, 15 for E5M2; X = 0 for an all-zero block),
 *             code = RNE(clamp(x 2^-X, -FMAX, FMAX)); the matrix cores apply
 *             the block scales.  A tensor that feeds two products is
 *             quantized once per orientation.
 * dims as for ptb_forward; norm LayerNorm or RMSNorm, mlp GeLU only
 * (PTB_ERR_ARG for SwiGLU).  Any b, s, h, f allowed by ptb_validate_dims:
 * the FP8 copies pad their contiguous dimension with zero codes to a
 * multiple of 128.  Inputs, outputs and ownership are as for the bf16 calls.
 * `saved` (ptb_fp8_saved_bytes) holds the parallel block's slots at the
 * offsets ptb_saved_layout gives (A16 is not written), followed by the
 * transposed E4M3 copies of a and [c | g] and their amax or block scales, which the forward
 * casts for the weight gradients;
 * the calls are asynchronous on `stream` and return PTB_ERR_HIP if a launch
 * fails.  stage_events: NULL, or 2 hipEvent_t per stage (start, end; NULL
 * entries skipped) recorded around each stage as for ptb_forward_timed.
 * ------------------------------------------------------------------------ */
#define PTB_FP8_FWD_STAGES 6
#define PTB_FP8_BWD_STAGES 8

/* Every FP8 call takes the scaling recipe; PTB_ERR_ARG for another value.
 * Buffers sized, cast or saved under one recipe are read under the same. */
enum ptb_fp8_recipe { PTB_FP8_CURRENT = 0, PTB_FP8_MX = 1 };

/* Bytes of the FP8 weight buffer (amax of W1 = [W_qkv | W_fc1] and
 * W2 = [W_o ; W_fc2] or the block scales of each copy, and W1^T, W1, W2^T
 * and W2 in E4M3), of the FP8 layer's stash and of its workspace. */
int32_t ptb_fp8_weights_bytes(const ptb_dims* dims, int32_t recipe, size_t* bytes);
int32_t ptb_fp8_saved_bytes(const ptb_dims* dims, int32_t recipe, size_t* bytes);
int32_t ptb_fp8_workspace_bytes(const ptb_dims* dims, int32_t recipe, size_t* bytes);

/* Byte offsets of the parts of the FP8 weight buffer (`offsets` has room
 * for PTB_FP8_WEIGHT_PARTS entries):
 *   AMAX   fp32 [2]: amax of W1, amax of W2
 *   W1T    E4M3 [N1][pad128(h)]   W1^T, N1 = 3 n d + f
 *   W1     E4M3 [h][pad128(N1)]   W1
 *   W2T    E4M3 [h][pad128(K2)]   W2^T, K2 = n d + f
 *   W2     E4M3 [K2][pad128(h)]   W2
 *   W1T_S, W1_S, W2T_S, W2_S  PTB_FP8_MX only: the block scales of each
 *          copy, pad128(k)/128 x pad128(rows) x 4 bytes for a copy of `rows`
 *          rows and contraction extent k, one E8M0 code per row and k-block
 *          of 32 values, in the order the matrix cores' lanes consume them:
 *          with r = 128 g + 32 i + l (i < 4, l < 32), the code of row r's
 *          k-block 4 j + b (b < 4) is byte
 *            4 (j pad128(rows) + 128 g) + 16 l + 8 (b & 1) + 4 (b >> 1) + i
 * pad128(v) / pad64(v) round up to a multiple of 128 / 64; padding codes
 * are zero, padding blocks and rows have scale code 127.  Parts a recipe
 * does not use (AMAX under PTB_FP8_MX, the scales under PTB_FP8_CURRENT)
 * get offset SIZE_MAX. */
enum ptb_fp8_weight_part {
  PTB_FP8_AMAX = 0, PTB_FP8_W1T, PTB_FP8_W1, PTB_FP8_W2T, PTB_FP8_W2,
  PTB_FP8_W1T_S, PTB_FP8_W1_S, PTB_FP8_W2T_S, PTB_FP8_W2_S,
  PTB_FP8_WEIGHT_PARTS
};
int32_t ptb_fp8_weights_layout(const ptb_dims* dims, int32_t recipe, size_t* offsets);

/* The current-scaling cast on its own, for any bf16 matrix x [rows][cols]
 * (device, row-major, cols a multiple of 8, rows * cols < 2^30):
 * *amax = max |x| (device fp32), s = FMAX / *amax, and the codes of x s in
 * `format` (PTB_FP8_E4M3 or PTB_FP8_E5M2) written row-wise to
 * q [rows][pad64(cols)] and/or transposed to qt [cols][pad64(rows)]
 * (either may be NULL; padding codes are zero).  The same kernels as the
 * layer's casts.  Pointers 16-byte aligned. */
enum ptb_fp8_format { PTB_FP8_E4M3 = 0, PTB_FP8_E5M2 = 1 };
int32_t ptb_fp8_quantize(const void* x, int32_t rows, int32_t cols, int32_t format, float* amax,
                         void* q, void* qt, void* stream);

/* The block-scaled (PTB_FP8_MX) cast on its own, for the same x: codes
 * row-wise to q [rows][pad128(cols)] with scales q_scales
 * (pad128(cols)/128 x pad128(rows) x 4 bytes, blocks along each row),
 * and/or transposed to qt [cols][pad128(rows)] with qt_scales
 * (pad128(rows)/128 x pad128(cols) x 4 bytes, blocks along each column of
 * x); byte order as for the weight buffer's scale parts.  A copy is written when
 * both its pointers are non-NULL.  The same kernel as the layer's casts. */
int32_t ptb_fp8_quantize_mx(const void* x, int32_t rows, int32_t cols, int32_t format, void* q,
                            void* q_scales, void* qt, void* qt_scales, void* stream);

/* Casts the four bf16 weights (as for ptb_forward) into `fp8_weights`
 * (device, caller-owned, ptb_fp8_weights_bytes), both orientations of each
 * concatenated weight on one current scale.  Call it after every change of
 * the weights (once per optimizer step); forward and backward read it. */
int32_t ptb_fp8_cast_weights(const ptb_dims* dims, int32_t recipe, const void* w_qkv,
                             const void* w_o, const void* w_fc1, const void* w_fc2,
                             void* fp8_weights, void* stream);

/* Forward: y [T, h] and `saved`.  Stages: 0 LayerNorm, 1 cast a (row-wise
 * and transposed), 2 [QKV | FC1] FP8 product + GeLU, 3 attention, 4 cast
 * [c | g] (both ways), 5 [O ; FC2] FP8 product + residual. */
int32_t ptb_fp8_forward(const ptb_dims* dims, int32_t recipe, const void* x,
                        const void* ln_gamma, const void* ln_beta, const void* fp8_weights,
                        void* y, void* saved, void* workspace, void* stream,
                        void* const* stage_events);

/* Backward for upstream gradient dy [T, h] from the `saved` of the matching
 * ptb_fp8_forward (same x, same fp8_weights); writes what ptb_backward
 * writes.  It reads the forward's FP8 copies of a and [c | g] from `saved`
 * and casts the gradient operands itself; it does not depend on the
 * forward's workspace contents.  Stages: 0 cast dy (both ways), 1 dgrad
 * [O ; FC2] + GeLU', 2 attention backward, 3 wgrad [O ; FC2], 4 cast dZ (both
 * ways), 5 dgrad [QKV | FC1], 6 wgrad [QKV | FC1], 7 LayerNorm backward
 * (+ dy). */
int32_t ptb_fp8_backward(const ptb_dims* dims, int32_t recipe, const void* dy,
                         const void* x, const void* ln_gamma, const void* fp8_weights,
                         const void* saved, void* dx, void* d_ln_gamma, void* d_ln_beta,
                         void* dw_qkv, void* dw_o, void* dw_fc1, void* dw_fc2, void* workspace,
                         void* stream, void* const* stage_events);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* PTB_H_ */
