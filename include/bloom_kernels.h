/*
 * bloom_kernels.h -- C ABI of the BLOOM fused kernels and BF16Optimizer step
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed comes from four pages on how BLOOM-176B was trained with
 * Megatron-DeepSpeed:
 *   [overview]  "BLOOM 176B 训练技术概览"
 *   [ru]        "Как обучали BLOOM: технологии Megatron и DeepSpeed для 176-миллиардной модели"
 *   [3d]        "企业官网建设流程全解析" (its body covers BLOOM's 3-D parallelism,
 *               ZeRO, BF16 and fused kernels despite the title)
 *   [mini]      "单机多卡实战：Megatron-DeepSpeed训练类BLOOM模型全流程解析"
 * Each entry point below names the section it implements.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are raw DEVICE pointers to caller-owned memory (e.g. allocated by
 *   PyTorch).  The library never allocates, frees or synchronises; a call only
 *   validates its arguments and enqueues kernels on `stream` (NULL = the
 *   default stream).  Outputs are complete once the stream reaches that point.
 *   (bloom_layernorm_bwd_noalloc is the one entry point with memory of its
 *   own: a static device array, see there.)
 * - bf16 values are raw bfloat16 bit patterns (`bloom_bf16`).  All arithmetic
 *   is FP32 (FP64 for the gradient-norm sum); bf16 outputs are rounded to
 *   nearest, ties to even.
 * - Matrices are row-major and contiguous.  Every array pointer must be
 *   16-byte aligned, and row widths (hidden, cols, seq) must be multiples of 8
 *   so that every row starts on a 16-byte boundary.
 * - Outputs must not overlap inputs (no in-place operation) unless stated.
 * - Validation happens before anything is enqueued: on any error the function
 *   returns a non-zero status, enqueues nothing, and bloom_last_error() holds a
 *   message (thread-local).  A launch failure reported by the HIP runtime
 *   returns BLOOM_ERR_HIP; faults inside a kernel surface at the caller's next
 *   synchronisation.  Empty inputs (rows == 0, n == 0, batch*heads == 0) return
 *   BLOOM_OK and enqueue nothing.
 * - Results are bitwise deterministic run to run on one device type: every
 *   reduction has a fixed order that depends only on the shape.
 */
#ifndef BLOOM_KERNELS_H
#define BLOOM_KERNELS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t bloom_bf16; /* raw bfloat16 bits */

typedef enum {
  BLOOM_OK = 0,
  BLOOM_ERR_NULL = 1,      /* a required pointer is NULL */
  BLOOM_ERR_SHAPE = 2,     /* a size is negative, too large, or not a multiple of 8 */
  BLOOM_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  BLOOM_ERR_WORKSPACE = 4, /* workspace missing or smaller than the *_workspace_size query */
  BLOOM_ERR_HPARAM = 5,    /* a scalar argument is out of range */
  BLOOM_ERR_HIP = 6        /* the HIP runtime reported an error */
} bloom_status;

/* Version of this ABI (incremented on any signature change). */
int bloom_abi_version(void);
/* Static text for a status code. */
const char* bloom_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char* bloom_last_error(void);

/* Largest supported row width of the LayerNorm and bias-GeLU kernels, and
 * largest softmax sequence length. */
#define BLOOM_MAX_HIDDEN 65536
#define BLOOM_MAX_SEQ 16384
#define BLOOM_MAX_HEADS 256
#define BLOOM_MAX_ACCUM_BATCH 16

/* ---------------------------------------------------------------------------
 * LayerNorm forward.  [overview] "融合 CUDA 核" (the fused LayerNorm kernel)
 * and "架构微调" (the embedding LayerNorm after the word embedding: same call
 * on embedding rows); [3d] 4.3.
 *   per row:  mu = sum(x)/H,  var = sum((x-mu)^2)/H,  r = 1/sqrt(var+eps),
 *             y = (x-mu)*r*gamma + beta
 * x, y    [rows, hidden] bf16;  gamma, beta [hidden] bf16;
 * mean, rstd [rows] fp32 (saved for the backward).
 * hidden: 8 .. BLOOM_MAX_HIDDEN, multiple of 8.  eps > 0.
 */
bloom_status bloom_layernorm_fwd(const bloom_bf16* x, const bloom_bf16* gamma,
                                 const bloom_bf16* beta, bloom_bf16* y, float* mean,
                                 float* rstd, int64_t rows, int64_t hidden, float eps,
                                 hipStream_t stream);

/* Bytes of workspace bloom_layernorm_bwd needs for its column partial sums. */
size_t bloom_layernorm_bwd_workspace_size(int64_t rows, int64_t hidden);

/* LayerNorm backward.  [overview] "融合 CUDA 核".
 *   x_hat = (x-mean)*rstd,  g = dy*gamma,
 *   dx     = rstd * (g - mean_row(g) - x_hat * mean_row(g*x_hat))
 *   dgamma = sum_rows(dy * x_hat),   dbeta = sum_rows(dy)
 * dy, x, dx [rows, hidden] bf16; gamma [hidden] bf16; mean, rstd [rows] fp32
 * from bloom_layernorm_fwd; dgamma, dbeta [hidden] bf16 (written, not added
 * to).  workspace: device memory of at least
 * bloom_layernorm_bwd_workspace_size(rows, hidden) bytes, 16-byte aligned,
 * owned by the caller; its contents on entry do not matter.
 */
bloom_status bloom_layernorm_bwd(const bloom_bf16* dy, const bloom_bf16* x,
                                 const bloom_bf16* gamma, const float* mean,
                                 const float* rstd, bloom_bf16* dx, bloom_bf16* dgamma,
                                 bloom_bf16* dbeta, void* workspace, size_t workspace_bytes,
                                 int64_t rows, int64_t hidden, hipStream_t stream);

/* Size of the static device scratch of bloom_layernorm_bwd_noalloc (32 MiB
 * per device). */
#define BLOOM_NOALLOC_SCRATCH_BYTES (32u << 20)

/* bloom_layernorm_bwd for callers that cannot allocate memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results (bit for bit) as bloom_layernorm_bwd,
 * without the workspace: the column partial sums go to a static device array
 * of BLOOM_NOALLOC_SCRATCH_BYTES that each device holds from the library's
 * load until the process ends.  The call allocates nothing.
 *   - rows, hidden whose bloom_layernorm_bwd_workspace_size exceeds
 *     BLOOM_NOALLOC_SCRATCH_BYTES -> BLOOM_ERR_WORKSPACE (with 256 compute
 *     units: any rows at hidden <= 16384; BLOOM-176B's 14336 needs 28 MiB);
 *   - `stream` must belong to the current device, else BLOOM_ERR_HPARAM;
 *   - the first call on a device looks the array's device address up
 *     (hipGetSymbolAddress) and keeps it; a failure -> BLOOM_ERR_HIP.
 * Every call on one device shares the one array and leaves its contents
 * behind (nothing in it needs to start at zero).  Calls that overlap on one
 * device -- on different streams, or from different threads -- race on it
 * and must not be issued. */
bloom_status bloom_layernorm_bwd_noalloc(const bloom_bf16* dy, const bloom_bf16* x,
                                         const bloom_bf16* gamma, const float* mean,
                                         const float* rstd, bloom_bf16* dx, bloom_bf16* dgamma,
                                         bloom_bf16* dbeta, int64_t rows, int64_t hidden,
                                         hipStream_t stream);

/* LayerNorm fused with the residual connection, forward.  [3d] 4.3 (a fused
 * LayerNorm + residual kernel, printed there as a stub); the LayerNorm is the
 * one of bloom_layernorm_fwd.  BLOOM's blocks are pre-LN, so the sum is also
 * the residual stream the next block adds to, and it is written out:
 *   h = x + residual, added in FP32 and rounded once to bf16 (for bf16
 *       inputs this is the exact sum rounded to nearest even)
 *   y = LayerNorm(h), bit for bit what bloom_layernorm_fwd returns for h.
 * x, residual, h, y [rows, hidden] bf16; gamma, beta [hidden] bf16;
 * mean, rstd [rows] fp32 of h.  h must not overlap x or residual.
 */
bloom_status bloom_layernorm_residual_fwd(const bloom_bf16* x, const bloom_bf16* residual,
                                          const bloom_bf16* gamma, const bloom_bf16* beta,
                                          bloom_bf16* h, bloom_bf16* y, float* mean, float* rstd,
                                          int64_t rows, int64_t hidden, float eps,
                                          hipStream_t stream);

/* Backward of bloom_layernorm_residual_fwd.  [3d] 4.3.
 *   dh = dLN(dy; h) + dres, summed in FP32 and rounded once, where dLN is
 *        the dx of bloom_layernorm_bwd with x = h and dres is the gradient
 *        reaching h through the residual stream; dh is the gradient of both
 *        x and residual
 *   dgamma, dbeta as bloom_layernorm_bwd on h.
 * dy, dres, h, dh [rows, hidden] bf16; gamma [hidden]; mean, rstd [rows] fp32
 * from the forward; workspace as for bloom_layernorm_bwd (same size query).
 */
bloom_status bloom_layernorm_residual_bwd(const bloom_bf16* dy, const bloom_bf16* dres,
                                          const bloom_bf16* h, const bloom_bf16* gamma,
                                          const float* mean, const float* rstd, bloom_bf16* dh,
                                          bloom_bf16* dgamma, bloom_bf16* dbeta, void* workspace,
                                          size_t workspace_bytes, int64_t rows, int64_t hidden,
                                          hipStream_t stream);

/* ---------------------------------------------------------------------------
 * ALiBi slopes (host only, no device work).  [overview] "架构微调" (ALiBi
 * replaces position embeddings) and "资源" (the ALiBi paper, arXiv:2108.12409,
 * whose rule this is): n heads, n a power of two -> head h (1-based) has
 * slope 2^(-8h/n); otherwise the c = 2^floor(log2 n) slopes of that rule
 * followed by the 1st, 3rd, 5th, ... slopes of the rule for 2c, n-c of them.
 * Computed in FP64, rounded once to FP32.  Writes the slopes of heads
 * head_offset .. head_offset+heads-1 to out_host (HOST memory, `heads` floats).
 */
bloom_status bloom_alibi_slopes(int32_t total_heads, int32_t head_offset, int32_t heads,
                                float* out_host);

/* Scale + ALiBi bias + causal mask + softmax, forward.  [overview] "融合 CUDA
 * 核" (the combined scale/mask/softmax kernel) with the ALiBi bias of
 * "架构微调"; [3d] 4.3 (trained at 2048, run at 8192).
 * For every (b, h, query i) row of the [batch, heads, seq, seq] scores:
 *   z_j = scale*s_ij - slope_h*(i-j)  (j <= i),   y_j = softmax_j(z)   (j <= i),
 *   y_j = +0 for j > i.   Score entries with j > i are never read.
 * slope_h is head (head_offset + h) of a model with total_heads heads (the
 * tensor-parallel rank's slice).  seq: 8 .. BLOOM_MAX_SEQ, multiple of 8;
 * heads <= BLOOM_MAX_HEADS; scale finite.
 */
bloom_status bloom_alibi_softmax_fwd(const bloom_bf16* scores, bloom_bf16* probs,
                                     int64_t batch, int32_t heads, int64_t seq,
                                     int32_t head_offset, int32_t total_heads, float scale,
                                     hipStream_t stream);

/* Backward of bloom_alibi_softmax_fwd with respect to the raw scores:
 *   ds_j = scale * y_j * (dy_j - sum_{k<=i} y_k dy_k)   (j <= i),  +0 for j > i.
 * probs = the forward output y, dprobs = dy, dscores = ds, all
 * [batch, heads, seq, seq] bf16.  Entries with j > i are never read.
 */
bloom_status bloom_alibi_softmax_bwd(const bloom_bf16* probs, const bloom_bf16* dprobs,
                                     bloom_bf16* dscores, int64_t batch, int32_t heads,
                                     int64_t seq, float scale, hipStream_t stream);

/* Fused causal attention with the ALiBi bias, forward, flash-style: the
 * L x L scores are never written.  [overview] "架构微调" (ALiBi in place of
 * position embeddings) and "融合 CUDA 核" (the fused scale + mask + softmax,
 * here applied between Q K^T and V); [3d] 4.3 (trained at 2048 tokens,
 * extrapolated to 8192).
 *   z_ij  = scale*(q_i . k_j) - slope_h*(i - j) for keys j <= i; j > i masked
 *   o_i   = sum_j softmax_j(z_i) v_j   (P rounded to bf16 for the product,
 *           FP32 accumulation)
 *   lse_i = ln sum_{j<=i} exp(z_ij)     (FP32; what a backward needs)
 * q, k, v, o [batch, heads, seq, head_dim] bf16 row-major; lse [batch, heads,
 * seq] fp32.  head_dim 32, 64 or 128; seq a multiple of 8, <=
 * BLOOM_MAX_SEQ; slopes as for bloom_alibi_softmax_fwd (heads [head_offset,
 * head_offset+heads) of a total_heads model).  scale > 0 (at least 1e-30;
 * 1/sqrt(head_dim) in BLOOM), else BLOOM_ERR_HPARAM.  o must not overlap
 * q, k, v.
 */
bloom_status bloom_alibi_attention_fwd(const bloom_bf16* q, const bloom_bf16* k, const bloom_bf16* v,
                                       bloom_bf16* o, float* lse, int64_t batch, int32_t heads,
                                       int64_t seq, int32_t head_dim, int32_t head_offset,
                                       int32_t total_heads, float scale, hipStream_t stream);

/* Fused causal attention with the ALiBi bias, backward: the gradients of
 * bloom_alibi_attention_fwd's o with respect to q, k and v for an upstream
 * gradient dout, without the L x L matrices (same passages as the forward;
 * training runs every fused kernel backward too):
 *   p_ij  = exp(scale*(q_i . k_j) - slope_h*(i - j) - lse_i)  (j <= i, else 0)
 *   dp_ij = dout_i . v_j,  D_i = sum_j p_ij dp_ij (FP32),
 *   ds_ij = p_ij * (dp_ij - D_i)
 *   dq_i  = scale * sum_j ds_ij k_j,  dk_j = scale * sum_i ds_ij q_i,
 *   dv_j  = sum_i p_ij dout_i
 * q, k, v, dout, dq, dk, dv [batch, heads, seq, head_dim] bf16 row-major;
 * lse [batch, heads, seq] fp32 as written by the forward (natural log); the
 * forward's o is not needed (D is summed from p and dp, not as dout . o).
 * Shapes, slopes and scale as for bloom_alibi_attention_fwd.  p enters the
 * dv product as bf16; ds enters the dq and dk products as two bf16 parts
 * (about 16 significant bits, since those sums can cancel); products
 * accumulate in FP32.
 * Deterministic: each output element is written by one workgroup.  The
 * caller-owned device workspace (16-byte aligned, at least
 * bloom_alibi_attention_bwd_workspace_size bytes; its contents are not
 * needed between calls) holds D.  dq, dk, dv must not overlap the inputs or
 * each other.  BLOOM_ERR_WORKSPACE if the workspace is NULL or too small.
 */
size_t bloom_alibi_attention_bwd_workspace_size(int64_t batch, int32_t heads, int64_t seq);
bloom_status bloom_alibi_attention_bwd(const bloom_bf16* q, const bloom_bf16* k, const bloom_bf16* v,
                                       const bloom_bf16* dout, const float* lse,
                                       bloom_bf16* dq, bloom_bf16* dk, bloom_bf16* dv, int64_t batch,
                                       int32_t heads, int64_t seq, int32_t head_dim, int32_t head_offset,
                                       int32_t total_heads, float scale, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * bias + GeLU forward.  [overview] "融合 CUDA 核" (bias + GeLU fusion); the
 * MLP's GeLU(XA) of [3d] 2.1.  tanh form (Hendrycks and Gimpel,
 * arXiv:1606.08415):  u = x + bias (FP32),
 *   y = u/2 * (1 + tanh(sqrt(2/pi) * (u + 0.044715 u^3)))
 * x, y [rows, cols] bf16; bias [cols] bf16.  cols: 8 .. BLOOM_MAX_HIDDEN,
 * multiple of 8.
 */
bloom_status bloom_bias_gelu_fwd(const bloom_bf16* x, const bloom_bf16* bias, bloom_bf16* y,
                                 int64_t rows, int64_t cols, hipStream_t stream);

/* Bytes of workspace bloom_bias_gelu_bwd needs for its column partial sums. */
size_t bloom_bias_gelu_bwd_workspace_size(int64_t rows, int64_t cols);

/* bias + GeLU backward:  dx = dy * gelu'(x + bias),  dbias = sum_rows(dx)
 * (dbias sums the unrounded FP32 dx).  dy, x, dx [rows, cols] bf16; bias,
 * dbias [cols] bf16 (dbias written, not added to).  workspace as for
 * bloom_layernorm_bwd, sized by bloom_bias_gelu_bwd_workspace_size.
 */
bloom_status bloom_bias_gelu_bwd(const bloom_bf16* dy, const bloom_bf16* x,
                                 const bloom_bf16* bias, bloom_bf16* dx, bloom_bf16* dbias,
                                 void* workspace, size_t workspace_bytes, int64_t rows,
                                 int64_t cols, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * BF16Optimizer, stage 1: FP32 gradient accumulation across pipeline
 * micro-batches.  [overview] "BF16 优化器"; 32 accumulation steps in [3d] 3.3.
 *   first_microbatch != 0:  grad_acc[i] = float(grad[i])
 *   first_microbatch == 0:  grad_acc[i] = grad_acc[i] + float(grad[i])  (one FP32 add)
 * grad_acc [n] fp32 (read-modify-write), grad [n] bf16.  Any n >= 0.
 */
bloom_status bloom_bf16_grad_accumulate(float* grad_acc, const bloom_bf16* grad, int64_t n,
                                        int32_t first_microbatch, hipStream_t stream);

/* Hyperparameters of bloom_bf16_adamw_step, as FP64; the library derives every
 * FP32 kernel constant from them in FP64 and rounds each once. */
typedef struct {
  double lr;            /* >= 0; [3d] 3.3 and [mini] 3 use 6e-5 */
  double beta1;         /* in [0, 1) */
  double beta2;         /* in [0, 1) */
  double eps;           /* > 0 */
  double weight_decay;  /* >= 0; [3d] 3.3 and [mini] 3 use 0.01 */
  double max_grad_norm; /* > 0; [3d] 4.3 and [mini] 3 use 1.0 */
  int64_t step;         /* t >= 1 of this update (bias correction 1 - beta^t) */
  int32_t sumsq_in_workspace; /* 1: the workspace already holds the norm's partial
                                 sums, written by bloom_bf16_grad_accumulate_sumsq
                                 for this n and grad_acc, and the step skips its own
                                 read of grad_acc for the norm; 0: the step computes them */
  int32_t reserved;     /* must be 0 */
} bloom_adamw_hparams;

/* Stage 1 for the last micro-batch: the same accumulation as
 * bloom_bf16_grad_accumulate, and in the same pass the FP64 partial sums of
 * grad_acc^2 that the norm of bloom_bf16_adamw_step needs, written into
 * `workspace` (sized by bloom_bf16_adamw_workspace_size(n)).  Pass that
 * workspace to bloom_bf16_adamw_step with hp->sumsq_in_workspace = 1 and leave
 * grad_acc unchanged in between; the step then reads grad_acc once instead of
 * twice.  The norm is bit-identical to the one the step computes by itself. */
bloom_status bloom_bf16_grad_accumulate_sumsq(float* grad_acc, const bloom_bf16* grad, int64_t n,
                                              int32_t first_microbatch, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream);

/* Stage 1 over several micro-batches in one pass.  [overview] "BF16 优化器"
 * (FP32 accumulation across micro-batches); [3d] 3.3 (32 accumulation steps).
 * grad_acc accumulates grads[0], grads[1], ..., grads[count-1] in that order,
 * each with one FP32 add exactly as bloom_bf16_grad_accumulate does (the
 * result is bit-identical to `count` such calls), while grad_acc is read and
 * written once instead of `count` times: for callers that keep several
 * micro-batch gradients of the shard resident.
 *   first_microbatch != 0: grads[0] starts the accumulation (grad_acc is only
 *   written).
 * grads: host array of `count` device pointers, 1 <= count <=
 * BLOOM_MAX_ACCUM_BATCH, each [n] bf16 and 16-byte aligned (the array itself
 * is read during the call only).  workspace: NULL, or a workspace of at least
 * bloom_bf16_adamw_workspace_size(n) bytes, into which the norm's partial sums
 * of the final grad_acc^2 are written as bloom_bf16_grad_accumulate_sumsq
 * does (then pass hp->sumsq_in_workspace = 1 to the step).  Errors: count out
 * of range or n out of range -> BLOOM_ERR_SHAPE; a NULL array or pointer ->
 * BLOOM_ERR_NULL; misaligned -> BLOOM_ERR_ALIGN; a short workspace ->
 * BLOOM_ERR_WORKSPACE. */
bloom_status bloom_bf16_grad_accumulate_many(float* grad_acc, const bloom_bf16* const* grads, int32_t count,
                                             int64_t n, int32_t first_microbatch, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace bloom_bf16_adamw_step needs (norm partials and the
 * clip coefficient). */
size_t bloom_bf16_adamw_workspace_size(int64_t n);

/* BF16Optimizer, stages 2-5, in one call: global L2 norm of the accumulated
 * gradient (FP64 sum), clip coefficient, AdamW on the FP32 master weights and
 * moments, and the bf16 parameter copy.  [overview] "BF16 优化器"; [3d] 1 (FP32
 * master, momentum and variance), 3.3 (AdamW, lr, weight decay), 4.3 (global
 * norm clipped at 1.0); [mini] 3.
 *   N = sqrt(sum acc^2);  c = max_grad_norm/N if N > max_grad_norm else 1
 *   g = c*acc;  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2
 *   master -= lr * ( (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps) + weight_decay*master )
 *   param_bf16 = round-to-nearest-even(master)
 * master, exp_avg, exp_avg_sq [n] fp32 (updated in place); grad_acc [n] fp32
 * (read only); param_bf16 [n] bf16 (written).  grad_norm_out: optional device
 * pointer to one float that receives N (NULL to skip).  A NaN norm leaves
 * c = 1; an infinite norm gives c = 0.  The norm and c never leave the device.
 * workspace: device memory of bloom_bf16_adamw_workspace_size(n) bytes.
 */
bloom_status bloom_bf16_adamw_step(float* master, float* exp_avg, float* exp_avg_sq,
                                   bloom_bf16* param_bf16, const float* grad_acc, int64_t n,
                                   const bloom_adamw_hparams* hp, float* grad_norm_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One contiguous range of the flat optimizer buffers with its own weight
 * decay: the optimizer group splitting of [overview] "工程挑战" (for example,
 * no decay on biases and LayerNorm weights). */
typedef struct {
  int64_t offset;      /* first element; a multiple of 8 */
  int64_t length;      /* elements, >= 1 */
  double weight_decay; /* finite, >= 0 */
} bloom_adamw_segment;

/* bloom_bf16_adamw_step with per-segment weight decay.  The norm and the clip
 * coefficient are global over all n elements, exactly as in
 * bloom_bf16_adamw_step; the update of the elements of segment s uses
 * segments[s].weight_decay in place of hp->weight_decay (which is ignored).
 * segments: host array of num_segments >= 1 entries in increasing offset
 * order that tile [0, n) exactly (the first starts at 0, each starts where
 * the previous ends, the last ends at n).  Other arguments, the workspace
 * and hp->sumsq_in_workspace are as for bloom_bf16_adamw_step.  One segment
 * {0, n, wd} gives bit for bit the result of bloom_bf16_adamw_step with
 * hp->weight_decay = wd.
 */
bloom_status bloom_bf16_adamw_step_segments(float* master, float* exp_avg, float* exp_avg_sq,
                                            bloom_bf16* param_bf16, const float* grad_acc, int64_t n,
                                            const bloom_adamw_hparams* hp,
                                            const bloom_adamw_segment* segments,
                                            int32_t num_segments, float* grad_norm_out,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream);

/* Learning rate for optimizer step `step` (1-based), host only.  [mini] 3
 * (lr 6e-5, min_lr 1e-6, cosine decay, 500 warmup iterations, 100000
 * iterations):
 *   step <= warmup_steps:  max_lr * step / warmup_steps
 *   step >= decay_steps:   min_lr
 *   otherwise:             min_lr + (max_lr - min_lr) * (1 + cos(pi * q)) / 2,
 *                          q = (step - warmup_steps) / (decay_steps - warmup_steps)
 * Requires step >= 1, 0 <= min_lr <= max_lr (finite) and
 * 0 <= warmup_steps < decay_steps; writes *lr_out (FP64).
 */
bloom_status bloom_lr_warmup_cosine(int64_t step, double max_lr, double min_lr, int64_t warmup_steps,
                                    int64_t decay_steps, double* lr_out);

#ifdef __cplusplus
}
#endif

#endif /* BLOOM_KERNELS_H */
