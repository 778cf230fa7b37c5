/*
 * slt.h - C ABI of the MI355X (gfx950) training-step library for a small
 * bias-free decoder: token embedding, per block norm / RoPE causal attention
 * (MHA or GQA) / MLP, final norm, untied lm_head, cross-entropy, the
 * hand-written backward and AdamW.
 *
 * Sources (page title, section):
 *   Hephaistos, "Architecture at a glance": the Llama block
 *     x + Attn(RMSNorm(x)), then x + SwiGLU(RMSNorm(x)); RoPE on q and k;
 *     causal attention with a stable softmax; SwiGLU (silu(x W1) * x W3) W2;
 *     untied lm_head; AdamW with decoupled decay and bias correction.
 *   Hephaistos, "Design notes": one flat parameter buffer and one activation
 *     arena, each tensor addressed by (offset, length); the forward caches
 *     what the backward needs; the backward is a reverse walk.
 *   strata, capability tables: the matmul family A.B, A.B^T, A^T.B; backward
 *     rules for matmul, LayerNorm, RMSNorm, GELU, SiLU, embedding,
 *     cross-entropy and causal attention taking n_head and n_kv_head
 *     independently with optional RoPE; the compile-time planner of parameter
 *     and memory sizes with static validation.
 *   Transformer in Rust, "CodeGen: Parallel Sub-Block Design": one LayerNorm
 *     feeds attention and a GELU MLP whose outputs join the residual in one
 *     add; "Key Features": RoPE on even-odd pairs; "Model Configurations":
 *     rotary_dim 32 of head dim 64.
 *   randyGPT, "Training (Metal GPU path)": cross-entropy over all positions,
 *     AdamW moments resident on the device.
 *
 * Conventions for every call:
 *   - Matrices are row-major; weights are [out, in], so a projection is
 *     y = x W^T.
 *   - "bf16" storage is the upper 16 bits of an IEEE binary32 (uint16_t in
 *     this header); rounding to it is to nearest, ties to even.
 *   - Device pointers point to memory the caller allocated and owns; the
 *     library allocates no device memory.  Its only device state is, per
 *     device, one second stream (default priority, non-blocking) and six
 *     events that the three backward calls create on their first use and
 *     keep until the process ends; every other call uses only the caller's
 *     stream.
 *   - Calls taking a stream only enqueue work on it (a hipStream_t passed as
 *     void*; NULL is the null stream) and return without synchronising.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Return value: SLT_OK, or an error code after which nothing was enqueued
 *     (argument errors are found on the host before any launch) - except
 *     SLT_EHIP, which reports a failed launch.  slt_last_error() gives a
 *     message for the calling thread.
 *   - Gradients are written, not accumulated.
 */
#ifndef SLT_H
#define SLT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLT_OK = 0,
  SLT_EINVAL = 1,        /* bad argument, shape or configuration           */
  SLT_EUNSUPPORTED = 2,  /* valid but not supported combination            */
  SLT_EHIP = 3           /* a HIP runtime call or kernel launch failed      */
} slt_status;

typedef enum { SLT_F32 = 0, SLT_BF16 = 1 } slt_dtype;
typedef enum { SLT_ROPE_HALF = 0, SLT_ROPE_PAIRS = 1 } slt_rope_mode;
typedef enum { SLT_BLOCK_LLAMA = 0, SLT_BLOCK_PARALLEL = 1 } slt_block;
typedef enum { SLT_NORM_L2 = 0, SLT_NORM_LINF = 1 } slt_norm_kind;

/* Model and workload shape.  d = C / H is the head dimension. */
typedef struct {
  int32_t V, C, H, Hkv, L, T, B, F, R; /* vocab, width, heads, kv heads, layers,
                                          sequence, batch, MLP width, rotary dims */
  int32_t rope_mode;  /* slt_rope_mode: HALF pairs (j, j+R/2); PAIRS (2j, 2j+1) */
  int32_t block;      /* slt_block: LLAMA (RMSNorm, SwiGLU) or PARALLEL (LayerNorm, GELU) */
  int32_t act;        /* slt_dtype of activations and of the compute copy of weights */
  float eps;          /* norm epsilon, added inside the square root (1e-5)          */
  float rope_base;    /* RoPE base (10000)                                           */
  float dropout;      /* inverted-dropout probability p, 0 <= p < 1 (0: off); applied by
                         the training forward (slt_forward_loss) to the embedding output,
                         to each block's attention weights (after the softmax
                         normalisation), and to its attention-projection and MLP outputs
                         (the parallel block's one combined output) before the residual
                         add, kept values scaled by float(1/(1-p)) (Hephaistos,
                         "Architecture at a glance"; randyGPT, "Architecture Details").
                         Element e of a site's tensor is kept iff word e mod 4 of
                         Philox-4x32-10(counter (e/4 mod 2^32, e/4 div 2^32, site, layer),
                         key (seed mod 2^32, seed div 2^32)) is at least floor(p 2^32);
                         sites 0 = embedding, 1 = attention projection, 2 = MLP, with
                         e = row*C + column of the [B*T, C] output, and 3 = attention
                         weights, with e = ((b*H + h)*T + i)*T + j for query i, key j of
                         head h of sequence b.  slt_backward regenerates the same masks;
                         slt_forward_cached applies none. */
  uint64_t dropout_seed; /* key of the mask generator; change it per step for fresh masks */
} slt_config;

/* One tensor of the flat parameter buffer.  rows/cols describe a matrix
 * [rows, cols]; vectors have rows = 1.  decay is 1 when weight decay applies. */
typedef struct {
  char name[40];
  int64_t offset;   /* in elements */
  int64_t numel;
  int64_t rows, cols;
  int32_t decay;
} slt_tensor;

/* Thread-local message describing the last error of the calling thread. */
const char* slt_last_error(void);

/* Library version string. */
const char* slt_version(void);

/* ------------------------------------------------------------------------
 * Planning (host only; strata, the compile-time planner with static
 * validation)
 * ---------------------------------------------------------------------- */

/* Checks a configuration: all sizes positive, C = H*d, H a multiple of Hkv,
 * R even and R <= d, rope_mode/block/act valid, C <= 4096, 0 <= dropout < 1.
 * SLT_EINVAL with a message otherwise. */
slt_status slt_validate(const slt_config* cfg);

/* Parameter layout (Hephaistos, "Design notes": flat buffer, (offset, len)).
 * Order: wte [V,C]; per layer (LLAMA) attn_norm [C], qkvw [(H+2Hkv)d, C],
 * w_o [C, Hd], mlp_norm [C], w1 [F,C], w3 [F,C], w2 [C,F]; (PARALLEL) ln_g [C],
 * ln_b [C], qkvw, fc_in [F,C], w_out [C, Hd+F] = [W_o | W_fc2]; then norm_f [C]
 * (LLAMA) or lnf_g, lnf_b [C] (PARALLEL); lm_head [V,C].  Layer tensors are
 * named "h<l>.<name>".  out may be NULL (only counts); otherwise it receives
 * min(cap, n) entries.  *n_tensors and *n_params are always set. */
slt_status slt_param_layout(const slt_config* cfg, slt_tensor* out, int32_t cap,
                            int32_t* n_tensors, int64_t* n_params);

/* Bytes of the activation arena (kept from forward to backward) and of the
 * scratch area (used inside one call) that the step calls need.  Both are
 * caller-allocated device memory, 256-byte aligned. */
slt_status slt_workspace_bytes(const slt_config* cfg, int64_t* act_bytes, int64_t* scratch_bytes);

/* Philox-4x32-10 counter-based generator (Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011), host side; the
 * device copy draws the normals of slt_model_init.  out = philox(ctr, key). */
void slt_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* ------------------------------------------------------------------------
 * Whole-step calls
 * ---------------------------------------------------------------------- */

/* Initialises the fp32 master parameters on the device: matrices
 * N(0, std^2) (output projections w_o, w2, w_out times out_scale), gains 1,
 * LayerNorm shifts 0.  Normal draws are Box-Muller on Philox-4x32-10
 * counters keyed by seed, so the result depends only on (seed, index). */
slt_status slt_model_init(const slt_config* cfg, uint64_t seed, float std, float out_scale,
                          float* master, void* stream);

/* bf16 compute copy of fp32 values: dst[i] = bf16(src[i]), n elements. */
slt_status slt_cast_bf16(const float* src, uint16_t* dst, int64_t n, void* stream);

/* Forward pass and mean cross-entropy over the B*T positions.
 * params: the compute copy of the flat parameters in cfg->act (fp32 master for
 *   F32 configs, its bf16 copy for BF16 configs), layout of slt_param_layout.
 * tokens: int32 [B, T+1] on the device; inputs are columns 0..T-1 and the
 *   next-token targets columns 1..T; every id must lie in [0, V).
 * acts: activation arena, scratch: scratch area (slt_workspace_bytes).
 * loss: device float, receives the mean loss.
 * On return the arena holds what slt_backward reads, including the logit
 * gradient, which overwrites the logits in place. */
slt_status slt_forward_loss(const slt_config* cfg, const void* params, const int32_t* tokens,
                            void* acts, void* scratch, float* loss, void* stream);

/* Backward pass after slt_forward_loss with the same params/tokens/acts.
 * grads: fp32 flat buffer in the parameter layout, every element written.
 * Besides `stream`, the call enqueues work on a second stream the library
 * creates for the current device on first use (each layer's weight
 * gradients, the norm-gain column sums, the token sort of the embedding
 * gradient), ordered by events both ways: work enqueued on `stream` after
 * the call runs after all of it, and the call's reads of acts/scratch/tokens
 * happen after what `stream` held before it.  Several host threads may call
 * it for one device; their enqueues take turns.  Results do not depend on
 * the overlap (the same kernels in the same order). */
slt_status slt_backward(const slt_config* cfg, const void* params, const int32_t* tokens,
                        void* acts, void* scratch, float* grads, void* stream);

/* slt_backward followed by the AdamW update of slt_adamw_step (no gradient
 * scale), fused: each layer's parameters are updated as soon as its
 * gradients are final, on the library's second stream while the walk goes
 * through the layers below (the final norm and lm_head after the last
 * layer's weight gradients, the embedding table last).  grads, master,
 * shadow (bf16 configurations; NULL for fp32), m, v and decay_mask (or
 * NULL) are the buffers of slt_adamw_step over the whole layout, with the
 * same alignment; t, lr, beta1, beta2, eps, wd as there.  Results equal
 * slt_backward then slt_adamw_step bit for bit.  For clipped steps (the
 * factor needs the whole gradient) use the separate calls. */
slt_status slt_backward_adamw(const slt_config* cfg, const void* params, const int32_t* tokens,
                              void* acts, void* scratch, float* grads, float* master,
                              uint16_t* shadow, float* m, float* v, int64_t t, float lr, float beta1,
                              float beta2, float eps, float wd, const uint8_t* decay_mask,
                              void* stream);

/* Gradient accumulation over micro-batches (Transformer in Rust,
 * "Configuration" and "Features": forward passes per optimizer step): the
 * same backward, but grads += scale * (gradient of this micro-batch's mean
 * loss) instead of overwriting.  With S micro-batches of equal size and
 * scale = 1/S, starting from zeroed grads, the result is the gradient of the
 * mean loss over all S micro-batches -- the full batch's gradient, up to the
 * summation order.  Activation gradients are not scaled; only the writes of
 * parameter gradients are.  loss / loss_sum (device fp32 scalars, both given
 * or both NULL): *loss_sum += scale * *loss, on the device, with loss the
 * micro-batch's mean loss that slt_forward_loss wrote -- from a zeroed
 * loss_sum, the mean loss over the micro-batches. */
slt_status slt_backward_accumulate(const slt_config* cfg, const void* params, const int32_t* tokens,
                                   void* acts, void* scratch, float* grads, float scale, const float* loss,
                                   float* loss_sum, void* stream);

/* Key/value-cache forward (randyGPT, "Features": the prompt is run once and
 * each further token costs one single-token forward; Transformer in Rust,
 * "CodeGen Inference Pipeline": prefill fills the cache and every generated
 * token appends its keys and values; strata, model table: the cache holds
 * pre-rotated keys, and the cached decoder equals the full forward).
 *
 * slt_kv_cache_bytes: bytes of the cache for B sequences of up to Tmax
 * positions, and of the workspace one slt_forward_cached call of Tq new
 * tokens per sequence needs (a workspace sized for (B, Tq) serves every call
 * with smaller B or Tq).  Host only; cfg->T and cfg->B are not used.
 *
 * slt_forward_cached: runs tokens [B, Tq] (row stride ld_tokens, ids in
 * [0, V)) at positions pos0 .. pos0+Tq-1 of each sequence, pos0 being the
 * number of positions already in the cache (pos0 = 0 starts a sequence and
 * fills the RoPE table kept in the cache; the caller supplies pos0, the
 * library keeps no length).  Each layer writes the new rows' rotated keys and
 * values into the cache and attends each query to cached positions
 * 0 .. its own; prompts of 16 or more tokens at pos0 = 0 use the training
 * forward's attention kernel.  Logits: [B*Tq, V] (row stride ld_logits) of
 * every new row, or [B, V] of the last row of each sequence when last_only
 * != 0, in cfg->act.  params: compute copy as for slt_forward_loss.
 * cache: caller-owned device memory of slt_kv_cache_bytes(Tmax) bytes, per
 * layer K then V [B, Hkv, Tmax, d] in cfg->act, then the RoPE table;
 * positions >= pos0+Tq are neither read nor written.  workspace: 256-byte
 * aligned, contents not kept.  SLT_EINVAL when pos0 + Tq > Tmax or a size is
 * non-positive; SLT_EUNSUPPORTED for head dimensions above 64. */
slt_status slt_kv_cache_bytes(const slt_config* cfg, int32_t B, int32_t Tq, int32_t Tmax,
                              int64_t* cache_bytes, int64_t* workspace_bytes);
slt_status slt_forward_cached(const slt_config* cfg, const void* params, const int32_t* tokens, int32_t B,
                              int32_t Tq, int64_t ld_tokens, int32_t pos0, void* cache, int32_t Tmax,
                              void* workspace, int32_t last_only, void* logits, int64_t ld_logits,
                              void* stream);

/* AdamW on n flat fp32 elements at step t >= 1 (Hephaistos, "Architecture at a
 * glance"; strata, "AdamW (decoupled decay, bias-corrected)"):
 *   g = s grads;  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   theta -= lr (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd theta)
 * with wd applied where decay_mask[i] != 0 (all elements when decay_mask is
 * NULL).  s = *grad_scale, a device fp32 scalar such as the factor written by
 * slt_clip_grad_norm, or 1 when grad_scale is NULL.  When shadow is not NULL
 * it receives bf16(theta).  master, m, v are updated in place; grads is not
 * modified.  Buffers 16-byte aligned (shadow 8, decay_mask 4). */
slt_status slt_adamw_step(int64_t n, float* master, uint16_t* shadow, const float* grads,
                          float* m, float* v, int64_t t, float lr, float beta1, float beta2,
                          float eps, float wd, const uint8_t* decay_mask, const float* grad_scale,
                          void* stream);

/* Global gradient norm and clipping factor (MicroGPT in Rust, "Gradient
 * Clipping"; Transformer in Rust, "Features": clipping by global norm;
 * randyGPT, "Training (Metal GPU path)": the L-infinity variant).  Over the n
 * fp32 values of grads (the flat gradient buffer): kind SLT_NORM_L2 gives
 * sqrt(sum g^2), SLT_NORM_LINF gives max |g|; the sums are formed in float64
 * in a fixed order (bitwise reproducible).  Writes, to device memory, *norm
 * (if not NULL) and *scale = max_norm / norm when norm > max_norm, else 1
 * (if not NULL) -- the factor slt_adamw_step's grad_scale applies.  No host
 * synchronisation.  workspace: slt_clip_workspace_bytes() bytes of device
 * memory, 16-byte aligned, scratch for the call.  grads 16-byte aligned. */
int64_t slt_clip_workspace_bytes(void);
slt_status slt_clip_grad_norm(int64_t n, const float* grads, int32_t kind, float max_norm, float* norm,
                              float* scale, void* workspace, void* stream);

/* ------------------------------------------------------------------------
 * Per-op calls.  dtype is the storage type of the activation operands
 * (SLT_F32 or SLT_BF16); statistics, weight gradients and losses are fp32.
 * ---------------------------------------------------------------------- */

/* GEMM of the matmul family (strata, "A.B, A.B^T, A^T.B"):
 *   C[m, n] = sum_k A(m, k) B(n, k)  (+ R[m, n] when R is not NULL)
 * A(m, k) = A[m*lda + k] if a_kmajor else A[k*lda + m];
 * B(n, k) = B[n*ldb + k] if b_kmajor else B[k*ldb + n].
 * A and B have type in_dtype; C and R have type out_dtype (R may equal C).
 * So y = x W^T is (a_kmajor=1, b_kmajor=1), dX = dY W is (1, 0) and
 * dW = dY^T X is (0, 0).  workspace (fp32, workspace_bytes) lets the library
 * split K across workgroups with a fixed-order reduction; NULL disables it. */
slt_status slt_gemm(int32_t M, int32_t N, int32_t K,
                    const void* A, int64_t lda, int32_t a_kmajor,
                    const void* B, int64_t ldb, int32_t b_kmajor,
                    void* C, int64_t ldc, const void* R, int64_t ldr,
                    int32_t in_dtype, int32_t out_dtype,
                    void* workspace, int64_t workspace_bytes, void* stream);

/* Grouped weight gradients (the matmul family's A^T.B form, several
 * products in one launch; Hephaistos, "Design notes": the backward walk
 * produces each layer's weight gradients from cached activations).  Product
 * i computes, in fp32,
 *   C_i[m, n] = alpha_i sum_k A_i[k*lda_i + m] B_i[k*ldb_i + n]  (+ C_i when accumulate_i)
 * with bf16 operands whose rows are the K tokens (dW = dY^T X).  All products
 * share K.  Requirements (else SLT_EUNSUPPORTED, nothing enqueued): bf16
 * operands, K a positive multiple of 32, M_i and N_i multiples of 8 (>= 8),
 * lda/ldb multiples of 8, ldc a multiple of 4, A/B/C 16-byte aligned,
 * 1 <= n <= 6.  workspace (fp32 partials, may be NULL) lets the library split
 * K over the products' tiles with a fixed-order reduction (deterministic).
 * items is host memory, read before the call returns. */
typedef struct {
  int32_t M, N;
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  float* C; int64_t ldc;
  float alpha;
  int32_t accumulate;
} slt_gemm_group_item;
slt_status slt_gemm_dw_group(const slt_gemm_group_item* items, int32_t n, int32_t K, void* workspace,
                             int64_t workspace_bytes, void* stream);

/* MLP input projection with SwiGLU (Hephaistos, "Architecture at a glance":
 * (silu(x W1) * x W3) W2):
 *   ab[M, 2F] = x[M, C] [W1; W3]^T   (a in columns 0..F-1, b in F..2F-1)
 *   h[M, F]   = silu(a) * b          (from a and b as stored, i.e. rounded)
 * w13: [2F, C] (w1 then w3, as in the parameter layout); row strides C, 2F,
 * F.  Large bf16 shapes run as one launch (the GEMM epilogue writes a, b and
 * h), others as the GEMM and the element kernel; the results are the same
 * either way. */
slt_status slt_mlp_swiglu_fwd(int32_t M, int32_t F, int32_t C, const void* x, const void* w13, void* ab, void* h,
                              int32_t dtype, void* stream);

/* Projection whose trailing columns feed GELU (Transformer in Rust, "CodeGen:
 * Parallel Sub-Block Design": one LayerNorm output feeds attention and the
 * GELU MLP, so [q | k | v | fc_in] is one product):
 *   y[M, N] = x[M, K] w[N, K]^T        (row stride ldy)
 *   u[M, N - col0] = gelu(y[:, col0:])  (tanh form, from y as stored; row
 *                                        stride ldu) */
slt_status slt_proj_gelu_fwd(int32_t M, int32_t N, int32_t K, const void* x, const void* w, void* y, int64_t ldy,
                             int32_t col0, void* u, int64_t ldu, int32_t dtype, void* stream);

/* QKV projection with RoPE in its epilogue (Hephaistos, "Architecture at a
 * glance": RoPE on q and k; Transformer in Rust, "Key Features"):
 *   y[M, N] = x[M, K] w[N, K]^T   (row stride ldy)
 * where columns [0, H d) are the query heads and [H d, (H + Hkv) d) the key
 * heads of d dims: their first R dims are rotated as slt_rope_fwd does, with
 * row m at position m % T, in fp32 before the one rounding to dtype.  The
 * remaining columns (values, and any further projection) are the plain
 * product.  This is the training forward's QKV step: the stored q and k are
 * the rotated ones. */
slt_status slt_qkv_rope_fwd(int32_t M, int32_t N, int32_t K, const void* x, const void* w, void* y, int64_t ldy,
                            int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t R, int32_t rope_mode, const float* cs,
                            int32_t dtype, void* stream);

/* Its backward into the projection outputs:
 *   dh = dy[M, C] W2[C, F]  -> dh_workspace [M, F] in dtype (row stride F)
 *   da, db from a, b (ab, row stride 2F) and dh  ->  dab[M, 2F] = [da | db]
 * w2: [C, F].  All pointers non-NULL. */
slt_status slt_mlp_swiglu_bwd(int32_t M, int32_t F, int32_t C, const void* dy, const void* w2, const void* ab,
                              void* dab, void* dh_workspace, int32_t dtype, void* stream);

/* x[b*T + t, :] = wte[tokens[b*ld_tokens + t], :] for t < T. */
slt_status slt_embedding_fwd(const int32_t* tokens, int32_t B, int32_t T, int64_t ld_tokens,
                             const void* wte, void* x, int32_t V, int32_t C, int32_t dtype,
                             void* stream);

/* dwte[v, :] = sum of dx[i, :] over positions i whose id is v, summed in
 * increasing position order (deterministic); rows of absent ids are 0.
 * workspace: at least slt_embedding_bwd_workspace(B*T, V) bytes. */
int64_t slt_embedding_bwd_workspace(int64_t N, int32_t V);
slt_status slt_embedding_bwd(const int32_t* tokens, int32_t B, int32_t T, int64_t ld_tokens,
                             const void* dx, float* dwte, int32_t V, int32_t C, int32_t dtype,
                             void* workspace, void* stream);

/* RMSNorm (Hephaistos, "Architecture at a glance"; MicroGPT in Rust,
 * "RMSNorm"): r = (mean_c x^2 + eps)^-1/2, y = x r g.  x, y: [rows, C];
 * g: [C] in dtype; rstd: fp32 [rows]. */
slt_status slt_rmsnorm_fwd(const void* x, const void* g, void* y, float* rstd,
                           int32_t rows, int32_t C, float eps, int32_t dtype, void* stream);

/* RMSNorm backward: dx = dres + r (dy g - xh mean(dy g xh)) with xh = x r;
 * dg = sum_rows dy xh (fp32, fixed-order two-stage reduction).  dres may be
 * NULL (treated as 0) and may equal dx.  workspace: at least
 * slt_norm_bwd_workspace(rows, C) bytes. */
int64_t slt_norm_bwd_workspace(int32_t rows, int32_t C);
slt_status slt_rmsnorm_bwd(const void* x, const void* g, const float* rstd, const void* dy,
                           const void* dres, void* dx, float* dg, int32_t rows, int32_t C,
                           int32_t dtype, void* workspace, void* stream);

/* LayerNorm (strata, GPT-2 reference; Transformer in Rust, "CodeGen: Parallel
 * Sub-Block Design"): mu = mean x, r = (mean (x-mu)^2 + eps)^-1/2,
 * y = (x - mu) r gamma + beta; mean, rstd fp32 [rows]. */
slt_status slt_layernorm_fwd(const void* x, const void* gamma, const void* beta, void* y,
                             float* mean, float* rstd, int32_t rows, int32_t C, float eps,
                             int32_t dtype, void* stream);

/* LayerNorm backward: dx = dres + r (dxh - mean dxh - xh mean(dxh xh)),
 * dxh = dy gamma; dgamma = sum dy xh, dbeta = sum dy (fp32). */
slt_status slt_layernorm_bwd(const void* x, const void* gamma, const float* mean,
                             const float* rstd, const void* dy, const void* dres, void* dx,
                             float* dgamma, float* dbeta, int32_t rows, int32_t C, int32_t dtype,
                             void* workspace, void* stream);

/* RoPE table: cs[t*R + 2j] = cos(t theta_j), cs[t*R + 2j + 1] = sin(t theta_j),
 * theta_j = base^(-2j/R), angles in float64 then rounded to fp32; fp32
 * [T, R] on the device. */
slt_status slt_rope_table(int32_t T, int32_t R, float base, float* cs, void* stream);

/* RoPE (Hephaistos, "Architecture at a glance": rotary embedding of q and
 * k; Transformer in Rust, "Key Features": even-odd pairs, "Model
 * Configurations": rotary dims 32 of 64).  Row r = b*T + t (position t) of x
 * holds nheads heads of d dims (head h at x + r*ldx + h*d); each pair (u, w)
 * of its first R dims -- (j, j + R/2) for SLT_ROPE_HALF, (2j, 2j+1) for
 * SLT_ROPE_PAIRS, j < R/2 -- becomes (u c - w s, u s + w c) with (c, s) =
 * cs[t*R + 2j], cs[t*R + 2j + 1] (the table of slt_rope_table), computed in
 * fp32 and rounded once to dtype.  Dims >= R are copied.  y may equal x
 * (then ldy = ldx).  slt_rope_bwd applies the transposed rotation (angle
 * -t theta_j): the gradient with respect to the un-rotated input. */
slt_status slt_rope_fwd(const void* x, int64_t ldx, void* y, int64_t ldy, int32_t B, int32_t T, int32_t nheads,
                        int32_t d, int32_t R, int32_t rope_mode, const float* cs, int32_t dtype, void* stream);
slt_status slt_rope_bwd(const void* dy, int64_t lddy, void* dx, int64_t lddx, int32_t B, int32_t T, int32_t nheads,
                        int32_t d, int32_t R, int32_t rope_mode, const float* cs, int32_t dtype, void* stream);

/* Causal attention forward, RoPE applied to q and k as they are loaded
 * (Hephaistos, "Architecture at a glance"; strata, flash-style attention with
 * online softmax and no T x T scores).  Head h of token b*T+t reads
 * q[(b*T+t)*ldq + h*d ...], k and v of KV head h*Hkv/H likewise with ldk/ldv,
 * and writes o[(b*T+t)*ldo + h*d ...].  lse: fp32 [B, H, T], the natural log
 * of the softmax denominator of each query row (scores scaled by 1/sqrt(d)).
 * o_res (may be NULL): dense [B*T, H*d] in dtype, receives o - round(o), the
 * part of the output its storage type dropped; the backward uses it.
 * cs: the RoPE table of slt_rope_table for (T, R); R = 0 disables RoPE.
 * bf16: the rotated q and k are rounded once to bf16 before the products (as
 * the training step stores them).  workspace: slt_attention_fwd_workspace(...)
 * bytes of device memory owned by the caller (16-byte aligned; NULL allowed
 * when that size is 0), scratch for the call only: bf16 operands with d a
 * multiple of 16 (d <= 64) and R > 0 are rotated once into it (slt_rope_fwd)
 * before the tiled kernel runs. */
int64_t slt_attention_fwd_workspace(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d,
                                    int32_t dtype);
slt_status slt_attention_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                             void* o_res, int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                             int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t R,
                             int32_t rope_mode, const float* cs, int32_t dtype, void* workspace,
                             void* stream);

/* Causal attention backward (recomputing probabilities from lse): writes dq
 * (of the un-rotated q), dk (un-rotated k; summed over the query heads of each
 * KV head) and dv with the same addressing as q, k, v.  o_res: the residual
 * written by the forward, or NULL.  workspace: at least
 * slt_attention_bwd_workspace(B, T, H, Hkv, d, dtype) bytes of caller-owned,
 * 16-byte aligned device memory (per-row D = dO.O, and for bf16 the rotated
 * q/k copies, rounded once as in the forward), scratch for the call only. */
int64_t slt_attention_bwd_workspace(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d,
                                    int32_t dtype);
slt_status slt_attention_bwd(const void* q, const void* k, const void* v, const void* o,
                             const void* o_res, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int64_t lddo,
                             int64_t lddq, int64_t lddk, int64_t lddv,
                             int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t d, int32_t R,
                             int32_t rope_mode, const float* cs, int32_t dtype, void* workspace,
                             void* stream);

/* SwiGLU (Hephaistos, "Architecture at a glance"): h = silu(a) * b on
 * [rows, F] operands with row strides lda, ldb, ldh. */
slt_status slt_swiglu_fwd(const void* a, const void* b, void* h, int32_t rows, int32_t F,
                          int64_t lda, int64_t ldb, int64_t ldh, int32_t dtype, void* stream);

/* da = dh b sigmoid(a) (1 + a (1 - sigmoid(a))), db = dh silu(a). */
slt_status slt_swiglu_bwd(const void* a, const void* b, const void* dh, void* da, void* db,
                          int32_t rows, int32_t F, int64_t lda, int64_t ldb, int64_t lddh,
                          int64_t ldda, int64_t lddb, int32_t dtype, void* stream);

/* GELU, tanh form: u = a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))). */
slt_status slt_gelu_fwd(const void* a, void* u, int32_t rows, int32_t F, int64_t lda,
                        int64_t ldu, int32_t dtype, void* stream);
slt_status slt_gelu_bwd(const void* a, const void* du, void* da, int32_t rows, int32_t F,
                        int64_t lda, int64_t lddu, int64_t ldda, int32_t dtype, void* stream);

/* Fused softmax cross-entropy over rows of logits z [rows, V] (row stride ldz)
 * with int32 targets (targets[i * ld_targets_row + col] addressing of
 * slt_forward_loss: row i = b*T + t reads tokens[b*ld_tokens + t + 1]).
 * loss (device fp32) = mean_i (lse_i - z[i, y_i]); z is overwritten with
 * dz = (softmax(z_i) - onehot(y_i)) / rows.  lse (fp32 [rows]) may be NULL.
 * workspace: at least 4*rows bytes (per-row losses, summed in fixed order). */
slt_status slt_softmax_xent(void* z, int64_t ldz, const int32_t* tokens, int32_t B, int32_t T,
                            int64_t ld_tokens, int32_t V, float* loss, float* lse, int32_t dtype,
                            void* workspace, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): slt_softmax_xent
 * with its per-row loss scratch in a static device array of the library
 * instead of a workspace argument -- same kernels, same results bit for bit.
 * At most 1048576 rows (B*T); larger inputs return SLT_EINVAL before any
 * launch.  Calls no hipMalloc/hipFree: the array (4 MiB) lives on every
 * device the library runs on until the process ends, and its address is
 * looked up once per device on the first call there.  Every call on a device
 * shares that device's array, so calls that overlap on one GPU (two streams
 * at once) race; calls in one stream order are safe.  Other arguments as
 * slt_softmax_xent. */
slt_status slt_softmax_xent_noalloc(void* z, int64_t ldz, const int32_t* tokens, int32_t B, int32_t T,
                                    int64_t ld_tokens, int32_t V, float* loss, float* lse, int32_t dtype,
                                    void* stream);

/* ------------------------------------------------------------------------
 * Machine bounds (strata, benchmark methodology: kernels are reported as a
 * fraction of a measured machine bound)
 * ---------------------------------------------------------------------- */

/* Launch timing by class, for measurement.  slt_timing(1) makes the
 * whole-step calls bracket every launch of five classes with a pair of HIP
 * events on the stream that launch runs on (the caller's stream, or the
 * backward's second stream for the weight gradients): 0 = forward
 * projections (the QKV, output, MLP and lm_head products, their epilogues
 * included), 1 = activation gradients dX = dY W, 2 = weight gradients
 * dW = dY^T X (a grouped launch with its split-K reduction counted as one),
 * 3 = attention forward, 4 = attention backward (dQ then dK / dV as one).
 * Element-wise, norm, loss and optimizer kernels are not bracketed.  The
 * events add gaps between launches, so timed runs keep it off (the default);
 * results do not depend on it.  slt_timing_read waits for the recorded pairs
 * and writes, for classes 0 .. nclass-1, the summed milliseconds ms[i] and
 * the number of launches launches[i] since the previous read, then forgets
 * them.  Host-global state shared by all threads and devices; SLT_EINVAL for
 * NULL outputs, SLT_EHIP if an event could not be read (the pairs are
 * forgotten either way). */
slt_status slt_timing(int32_t on);
slt_status slt_timing_read(double* ms, int64_t* launches, int32_t nclass);

/* dst = src over `bytes` bytes (a multiple of 16; both 16-byte aligned, not
 * overlapping) with 16-byte loads and stores: the read + write rate a
 * streaming kernel reaches on this GPU.  variant selects the launch shape
 * (0: 4 words per thread per iteration on 8192 blocks; 1: 8 words on 4096
 * blocks; 2: one pass over the buffer, 4 words per thread; these three with
 * non-temporal loads and stores; 3: as 2 with ordinary ones; 4: as 2 with
 * 1024-thread workgroups); the best of them is the measured bound.  SLT_EINVAL for another variant, a size that
 * is not a multiple of 16 or a NULL / misaligned pointer. */
slt_status slt_stream_copy(const void* src, void* dst, int64_t bytes, int32_t variant, void* stream);

/* `blocks` workgroups of 4 waves, each wave running `iters` rounds of
 * independent MFMAs on register operands: variant 0 = 8 chains of
 * v_mfma_f32_16x16x32_bf16, 1 = 8 chains of v_mfma_f32_32x32x16_bf16, 2 = 16
 * chains of v_mfma_f32_16x16x32_bf16.  out receives 256 * blocks floats (so
 * the work is not dead).  slt_mfma_loop_flops (host only) gives the FLOPs
 * one call performs. */
int64_t slt_mfma_loop_flops(int32_t blocks, int32_t iters, int32_t variant);
slt_status slt_mfma_loop(int32_t blocks, int32_t iters, int32_t variant, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SLT_H */
