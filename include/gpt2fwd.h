/*
 * gpt2fwd.h - C ABI of the MI355X (gfx950) GPT-2 forward-pass library.
 *
 * One entry per step of the forward pass, following the per-kernel split of
 * "ECE408 Final Project - GPT-2, Milestone 1" (Code Submission and Grading,
 * kernel table: Encoder, LayerNorm, MatMul, Attention including Softmax,
 * Residual, GELU), plus the vocabulary softmax of the classifier (llm.c
 * discussion "State of the Union [April 22, 2024]", kernel summaries:
 * fused_classifier_kernel3), the whole forward, and a KV-cache decode step
 * (optdl2025 projects, "Understanding and Improving GPT-2 Implementations in
 * NanoGPT": KV caching for autoregressive prediction).
 *
 * Ownership (as the ECE408 page fixes for its xxxx_forward() host functions,
 * Milestone Requirements): the caller allocates, fills and frees every buffer.
 * The library never allocates, frees or copies device memory, and never
 * synchronises. Every pointer argument is a DEVICE pointer unless marked
 * "host". Work is enqueued on `stream` (a hipStream_t; NULL = the default
 * stream) and the call returns once it is enqueued; results are valid after
 * the caller synchronises that stream.
 *
 * Errors: every entry returns an int status (GPT2_OK = 0 or a negative
 * GPT2_ERR_*). Arguments are validated before any launch, so a failed call
 * enqueues nothing. A launch failure returns GPT2_ERR_HIP and records the HIP
 * error code for gpt2_last_hip_error() (per host thread). No entry prints,
 * aborts or throws. A zero-sized problem returns GPT2_OK and launches nothing.
 *
 * Layout: row-major, contiguous. Every device pointer must be 16-byte aligned.
 * dtype (GPT2_F32 or GPT2_BF16) applies to weights and activations alike;
 * LayerNorm statistics are always fp32 and all accumulation is fp32.
 * bf16 results are rounded to nearest even. Outputs may alias inputs only
 * where stated.
 */
#ifndef GPT2FWD_H
#define GPT2FWD_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GPT2_F32 = 0, GPT2_BF16 = 1 };

enum {
    GPT2_OK = 0,
    GPT2_ERR_INVALID_ARGUMENT = -1,   /* NULL pointer, negative size, C % NH != 0, ... */
    GPT2_ERR_UNSUPPORTED = -2,        /* valid but not handled: head size, alignment, width */
    GPT2_ERR_HIP = -3,                /* a launch failed; see gpt2_last_hip_error() */
    GPT2_ERR_WORKSPACE_TOO_SMALL = -4
};

/* Token + position embedding (ECE408 Milestone 1 kernel table: Encoder).
 *   out[b,t,:] = wte[tokens[b,t],:] + wpe[t,:]
 * out [B,T,C]; tokens int32 [B,T] (values must lie in [0, rows of wte): not
 * checked on the device); wte [*,C]; wpe [>=T,C]. C % 8 == 0,
 * B*T <= INT32_MAX (else GPT2_ERR_UNSUPPORTED).
 * To embed a single position p for every sequence (decode), pass T = 1 and
 * wpe + p*C. */
int encoder_forward(void* out, const int32_t* tokens, const void* wte, const void* wpe,
                    int B, int T, int C, int dtype, void* stream);

/* LayerNorm over the last dimension (ECE408 kernel table: LayerNorm):
 *   mu = mean(x), var = mean((x-mu)^2), rstd = 1/sqrt(var+eps),
 *   out = (x-mu)*rstd*gamma + beta.
 * inp, out [N,C]; gamma, beta [C]; mean, rstd fp32 [N], nullable.
 * 8 <= C <= 4096, C % 8 == 0. out must not alias inp. */
int layernorm_forward(void* out, float* mean, float* rstd, const void* inp,
                      const void* gamma, const void* beta, int N, int C, float eps,
                      int dtype, void* stream);

/* Linear layer (ECE408 kernel table: MatMul):
 *   out[n,o] = sum_c inp[n,c] * weight[o,c] + bias[o]
 * inp [N,C]; weight [OC,C] (out_features x in_features); bias [OC], nullable;
 * out [N,OC], must not alias inp/weight. C % 8 == 0, OC % 8 == 0. */
int matmul_forward(void* out, const void* inp, const void* weight, const void* bias,
                   int N, int C, int OC, int dtype, void* stream);

/* Name of the GEMM kernel configuration matmul_forward launches for this
 * problem (host call), e.g. "gemm_f32_64x128_p3": dtype, output tile, and
 * "_p3" for the three-stage load-to-LDS pipeline or "_r" for the
 * register-staged kernel; so profiles can be attributed to shapes. The string
 * lives in thread-local storage until this thread's next call. Returns
 * "invalid" for negative sizes or an unknown dtype. */
const char* matmul_kernel_config(int N, int C, int OC, int dtype);

/* Causal multi-head self-attention with its softmax fused (ECE408 kernel
 * table: Attention including Softmax; the tiled online-softmax algorithm of
 * the optdl2025 project "Understand FlashAttention (I)", computing only the
 * lower triangle as the llm.c "big stones" list proposes).
 * qkv [B,T,3C] = [q | k | v], head h at columns h*hs..(h+1)*hs-1 of each third,
 * hs = C/NH in {16, 32, 64, 128}; out [B,T,C] with the same head order.
 *   out_t = sum_{j<=t} softmax_j(q_t.k_j / sqrt(hs)) v_j */
int attention_forward(void* out, const void* qkv, int B, int T, int C, int NH,
                      int dtype, void* stream);

/* GELU, tanh form (ECE408 kernel table: GELU):
 *   out = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
 * n elements; out may alias inp. */
int gelu_forward(void* out, const void* inp, int64_t n, int dtype, void* stream);

/* Residual add (ECE408 kernel table: Residual): out = a + b, n elements.
 * out may alias a or b. */
int residual_forward(void* out, const void* a, const void* b, int64_t n, int dtype,
                     void* stream);

/* Softmax over the vocabulary (forward half of llm.c's
 * fused_classifier_kernel3): logits, probs [N,Vp]; the first V columns are
 * real tokens, columns V..Vp-1 are padding and receive probability 0.
 * V <= Vp <= 131072, Vp % 8 == 0. probs must not alias logits. */
int softmax_forward(void* probs, const void* logits, int N, int V, int Vp, int dtype,
                    void* stream);

/* Softmax with cross-entropy, the whole forward of llm.c's
 * fused_classifier_kernel3 in one pass over the logits:
 *   losses[n] = log(sum_{v<V} exp(l[n,v] - m_n)) + m_n - l[n, targets[n]]  (fp32, [N])
 *   probs [N,Vp] as softmax_forward, or NULL to skip writing them;
 *   mean_loss (one fp32, nullable) = the mean of the N losses, summed in a
 *   fixed order.
 * targets int32 [N] must lie in [0, V) (not checked on the device). */
int crossentropy_forward(float* losses, float* mean_loss, void* probs, const void* logits,
                         const int32_t* targets, int N, int V, int Vp, int dtype, void* stream);

/* The vocabulary projection and softmax with the row statistics taken in the
 * GEMM epilogue (the fused classifier of llm.c "State of the Union [April 22,
 * 2024]", kernel summaries: fused_classifier_kernel3; the kernel-fusion item
 * of its "big stones" list). gpt2_forward does not use this pair: on MI355X
 * the epilogue's exponentials (one per logit, on the vector units while the
 * matrix cores wait) cost more than the softmax saves, since softmax_forward
 * already reads the logits once and writes the probabilities once.
 *
 * matmul_logits_stats_forward: logits [N,Vp] = inp [N,C] . wte[Vp,C]^T (no
 * bias), as matmul_forward, and
 *   stats[n][g] = (m, s),  m = max of the stored logits[n, v],
 *                          s = sum of exp(logits[n, v] - m)
 * over the columns v < V of group g = v / 128 (fp32 pairs, stats
 * [N, ceil(Vp/128), 2]; a group with no column below V holds (-inf, 0)).
 * Needs C % 32 == 0 (fp32) or C % 64 == 0 (bf16), else GPT2_ERR_UNSUPPORTED.
 *
 * softmax_stats_forward: probs [N,Vp] as softmax_forward, from the logits and
 * the stats above: M = max_g m_g, S = sum_g s_g exp(m_g - M),
 * probs[n,v] = exp(l_v - M) / S for v < V, 0 for V <= v < Vp. One read of the
 * logits and one write of the probabilities. probs must not alias logits;
 * Vp <= 131072. */
int matmul_logits_stats_forward(void* logits, float* stats, const void* inp, const void* wte, int N, int C,
                                int V, int Vp, int dtype, void* stream);
int softmax_stats_forward(void* probs, const void* logits, const float* stats, int N, int V, int Vp,
                          int dtype, void* stream);

/* ---------------------------------------------------------------- model */
typedef struct {
    int L;        /* layers */
    int C;        /* channels */
    int NH;       /* heads; C/NH in {16,32,64,128} */
    int V;        /* vocabulary */
    int Vp;       /* padded vocabulary (rows of wte), Vp >= V, Vp % 8 == 0 */
    int maxT;     /* rows of wpe */
    int dtype;    /* GPT2_F32 or GPT2_BF16 */
    float ln_eps; /* LayerNorm epsilon, 1e-5 for GPT-2 */
} gpt2_config;

/* Elements in the flat parameter buffer (host call):
 * Vp*C + maxT*C + L*(12*C*C + 13*C) + 2*C, stored as
 * wte[Vp,C] wpe[maxT,C] ln1_g[L,C] ln1_b[L,C] qkv_w[L,3C,C] qkv_b[L,3C]
 * attproj_w[L,C,C] attproj_b[L,C] ln2_g[L,C] ln2_b[L,C] fc_w[L,4C,C] fc_b[L,4C]
 * fcproj_w[L,C,4C] fcproj_b[L,C] lnf_g[C] lnf_b[C]. Rows V..Vp-1 of wte should
 * be zero. Returns -1 for an invalid config. */
int64_t gpt2_param_count(const gpt2_config* cfg /* host */);

/* Bytes of workspace gpt2_forward needs for B sequences of T tokens (host
 * call); -1 for an invalid config. */
int64_t gpt2_workspace_bytes(const gpt2_config* cfg /* host */, int B, int T);

/* The whole forward: pre-LayerNorm GPT-2 blocks, final LayerNorm, logits
 * against the tied token embedding (no bias), vocabulary softmax.
 * tokens int32 [B,T] (T <= maxT); params: the flat buffer above; logits
 * [B,T,Vp]; probs [B,T,Vp] or NULL to skip the softmax. */
int gpt2_forward(void* logits, void* probs, const int32_t* tokens, const void* params,
                 const gpt2_config* cfg /* host */, int B, int T, void* workspace,
                 int64_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- decode */
/* Bytes of workspace attention_decode_forward needs (host call). */
int64_t attention_decode_workspace_bytes(int B, int C, int NH, int maxT);

/* One query per sequence against a KV cache (optdl2025 NanoGPT project: KV
 * caching). qkv_new [B,3C] holds this step's q,k,v; kcache, vcache
 * [B,NH,maxT,hs] for one layer. Writes k,v of qkv_new at position pos, then
 * out[b, head h] = sum_{j<=pos} softmax_j(q.k_j/sqrt(hs)) v_j. 0 <= pos < maxT.
 * Cache slot pos is never read before it is written. */
int attention_decode_forward(void* out, const void* qkv_new, void* kcache, void* vcache,
                             int B, int pos, int maxT, int C, int NH, int dtype,
                             void* workspace, int64_t workspace_bytes, void* stream);

/* Decode-step building blocks. gpt2_decode_step on B <= 32 sequences runs
 * each layer as: matmul_forward (qkv) -> attention_decode_forward ->
 * matmul_splitk_forward (attproj) -> residual_layernorm_forward (ln2) ->
 * matmul_gelu_forward (fc, below) -> matmul_splitk_forward (fcproj) ->
 * residual_layernorm_forward (ln1 of the next layer, or lnf), i.e. the block
 * of the forward with the residual adds and the GELU fused into neighbours.
 *
 * Split-k linear layer without bias, for N <= 32 rows:
 *   part[s][n][o] = sum over c in k-range s of inp[n,c] * weight[o,c]
 * with the C columns cut into `splits` consecutive ranges of whole 128-byte
 * chunks (a range may be empty, giving zeros). part fp32 [splits,N,OC];
 * inp [N,C]; weight [OC,C]. 1 <= splits <= 8, C % 8 == 0, OC % 8 == 0;
 * N > 32 returns GPT2_ERR_UNSUPPORTED. */
int matmul_splitk_forward(float* part, const void* inp, const void* weight, int N, int C, int OC,
                          int splits, int dtype, void* stream);

/* The split count gpt2_decode_step uses for a C -> OC projection (host
 * call): enough workgroups to cover the chip, >= 2 chunks each; 1..8. */
int matmul_splitk_count(int C, int OC, int dtype);

/* Linear layer with the next step of a block fused into its epilogue (the
 * "kernel fusion" item of llm.c "State of the Union", big stones):
 *   matmul_gelu_forward:     out[n,o] = gelu(y[n,o])             (fc + GELU)
 *   matmul_residual_forward: out[n,o] = res[n,o] + y[n,o]        (attproj/fcproj + residual)
 * with y = sum_c inp[n,c] * weight[o,c] + bias[o] rounded to the dtype first,
 * so the result is bit-identical to matmul_forward followed by gelu_forward
 * or residual_forward. Shapes and rules as matmul_forward (bias nullable);
 * res [N,OC] may be out itself (x += ...); out must not alias inp or weight. One launch. */
int matmul_gelu_forward(void* out, const void* inp, const void* weight, const void* bias,
                        int N, int C, int OC, int dtype, void* stream);
int matmul_residual_forward(void* out, const void* inp, const void* weight, const void* bias,
                            const void* res, int N, int C, int OC, int dtype, void* stream);

/* Residual add of a split-k projection, then LayerNorm:
 *   x[n,:] <- x[n,:] + (bias + sum_{s<splits} part[s][n][:])   (in place;
 *            the partial sums are added in split order, in fp32)
 *   out[n,:] = LayerNorm(x[n,:]; gamma, beta, eps)      (of the stored x)
 * x, out [N,C] (distinct); part fp32 [splits,N,C]; bias, gamma, beta [C].
 * 1 <= splits <= 8; C as layernorm_forward. */
int residual_layernorm_forward(void* out, void* x, const float* part, int splits,
                               const void* bias, const void* gamma, const void* beta,
                               int N, int C, float eps, int dtype, void* stream);

/* Bytes of workspace gpt2_decode_step needs (host call); -1 if invalid. */
int64_t gpt2_decode_workspace_bytes(const gpt2_config* cfg /* host */, int B);

/* One autoregressive step for B sequences, each with one new token at
 * position pos: tokens int32 [B]; kcache, vcache [L,B,NH,maxT,hs] (updated at
 * pos); logits [B,Vp]; probs [B,Vp] or NULL. */
int gpt2_decode_step(void* logits, void* probs, const int32_t* tokens, int pos,
                     void* kcache, void* vcache, const void* params,
                     const gpt2_config* cfg /* host */, int B, void* workspace,
                     int64_t workspace_bytes, void* stream);

/* gpt2_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc). The step's scratch lives in a device
 * array of GPT2_DECODE_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; the call itself allocates nothing. Arguments as
 * gpt2_decode_step. Returns GPT2_ERR_WORKSPACE_TOO_SMALL (before any launch)
 * when gpt2_decode_workspace_bytes(cfg, B) exceeds GPT2_DECODE_SCRATCH_BYTES
 * (GPT-2 small needs ~2.8 MB at B = 32, GPT-2 medium ~3.7 MB). Every call on one
 * GPU shares that GPU's array: calls that may overlap on one device (other
 * streams, other host threads) race and must be serialised by the caller. */
#define GPT2_DECODE_SCRATCH_BYTES (8 << 20)
int gpt2_decode_step_noalloc(void* logits, void* probs, const int32_t* tokens, int pos,
                             void* kcache, void* vcache, const void* params,
                             const gpt2_config* cfg /* host */, int B, void* stream);

/* ------------------------------------------------------------ generation */
/* Greedy choice (the next-token step of autoregressive prediction, optdl2025
 * NanoGPT project): tokens[n] = argmax over v < V of logits[n, v], the lowest
 * index among equal maxima; logits [N,Vp], Vp % 8 == 0. */
int argmax_forward(int32_t* tokens, const void* logits, int N, int V, int Vp, int dtype, void* stream);

/* Prefill for KV-cached generation: the blocks of gpt2_forward over the prompt
 * tokens int32 [B,T] (1 <= T <= maxT), storing every layer's keys and values
 * at positions 0..T-1 of kcache, vcache [L,B,NH,maxT,hs]; then logits [B,Vp]
 * (and probs [B,Vp] or NULL) of the LAST position of each sequence. The
 * workspace is gpt2_workspace_bytes(cfg, B, T). */
int gpt2_prefill(void* logits, void* probs, const int32_t* tokens, void* kcache, void* vcache,
                 const void* params, const gpt2_config* cfg /* host */, int B, int T,
                 void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace gpt2_generate needs (host call); -1 if invalid. */
int64_t gpt2_generate_workspace_bytes(const gpt2_config* cfg /* host */, int B, int T);

/* Greedy generation of n_new tokens per sequence: gpt2_prefill of the prompt
 * [B,T], argmax_forward of its last logits -> token 0, then for i = 1..n_new-1
 * one gpt2_decode_step at position T+i-1 on token i-1 and argmax -> token i.
 * Everything is enqueued on the stream at once (no host round trip per
 * token). out_tokens int32 [B,n_new]; caches as gpt2_prefill, positions
 * 0..T+n_new-2 are written. Requires T + n_new - 1 <= maxT. */
int gpt2_generate(int32_t* out_tokens, const int32_t* prompt, int n_new, void* kcache, void* vcache,
                  const void* params, const gpt2_config* cfg /* host */, int B, int T,
                  void* workspace, int64_t workspace_bytes, void* stream);

/* ============================================================== backward
 * The training step's backward, one entry per forward step (the backward
 * kernels of llm.c's training step, "State of the Union [April 22, 2024]",
 * kernel summaries; the attention backward is the one asked for in the
 * optdl2025 project "Understand FlashAttention (II)"). Gradients have the
 * dtype and layout of the tensors they belong to; every reduction is done in
 * fp32 in a fixed order (bitwise reproducible). Scratch comes from the
 * caller's workspace, sized by the matching *_workspace_size call (host;
 * negative on invalid arguments). */

/* Fused classifier, backward half (llm.c fused_classifier_kernel3): for the
 * loss sum_n dloss * loss_n,
 *   dlogits[n,v] = dloss * (softmax(l_n)[v] - [v == targets[n]])  for v < V,
 *   dlogits[n,v] = 0                                             for V <= v < Vp,
 * and, from the same pass, losses [N] and mean_loss as crossentropy_forward
 * (both nullable; mean_loss needs losses). dlogits may be logits (in place).
 * For the mean loss pass dloss = 1/N. */
int crossentropy_backward(void* dlogits, float* losses, float* mean_loss, const void* logits,
                          const int32_t* targets, float dloss, int N, int V, int Vp, int dtype,
                          void* stream);

/* GELU backward: dinp = dout * g'(inp) with g the tanh-form GELU of
 * gelu_forward; n elements; dinp may be dout, not inp. */
int gelu_backward(void* dinp, const void* inp, const void* dout, int64_t n, int dtype, void* stream);

/* LayerNorm backward for y = (x - mean) * rstd * gamma + beta over rows of C,
 * with mean, rstd the fp32 statistics layernorm_forward saved:
 *   dinp  = [dres +] rstd * (g - mean_c(g) - xh * mean_c(g * xh)),  g = dout * gamma,
 *           xh = (x - mean) * rstd;
 *   dgamma = sum_n dout * xh,  dbeta = sum_n dout   (each [C], nullable, overwritten).
 * dres (nullable) is added: the residual stream's gradient flowing past the
 * LayerNorm; it may be dinp. dinp must not alias dout or inp. C % 8 == 0,
 * C <= 2048 (fp32) / 4096 (bf16). */
int64_t layernorm_backward_workspace_size(int N, int C);
int layernorm_backward(void* dinp, void* dgamma, void* dbeta, const void* dres, const void* dout,
                       const void* inp, const void* gamma, const float* mean, const float* rstd, int N, int C,
                       int dtype, void* workspace, int64_t workspace_bytes, void* stream);

/* Linear backward for out = inp [N,C] . weight[OC,C]^T + bias, given dout [N,OC]:
 *   dinp [N,C] = dout . weight,  dweight [OC,C] = dout^T . inp,  dbias [OC] = sum_n dout
 * each nullable (skipped) and overwritten; inp is needed for dweight, weight
 * for dinp. C % 8 == 0, OC % 8 == 0. */
int64_t matmul_backward_workspace_size(int N, int C, int OC, int dtype);
int matmul_backward(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                    const void* weight, int N, int C, int OC, int dtype, void* workspace,
                    int64_t workspace_bytes, void* stream);

/* attention_forward that also writes lse [B,NH,T] (fp32): the natural
 * log-sum-exp of each query's causal scaled scores, ln sum_{j<=t} exp(S_tj),
 * which attention_backward uses to rebuild the probabilities. */
int attention_forward_lse(void* out, float* lse, const void* qkv, int B, int T, int C, int NH, int dtype,
                          void* stream);

/* Attention backward: dqkv [B,T,3C] (packed like qkv, overwritten) of the
 * causal attention given dout [B,T,C] and the forward's qkv, out and lse:
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowsum(dO o O)),
 *   dQ = dS K / sqrt(hs),  dK = dS^T Q / sqrt(hs),   P = exp(S - lse).
 * hs = C/NH in {16, 32, 64}. dqkv must not alias an input. */
int64_t attention_backward_workspace_size(int B, int T, int C, int NH);
int attention_backward(void* dqkv, const void* dout, const void* qkv, const void* out, const float* lse,
                       int B, int T, int C, int NH, int dtype, void* workspace, int64_t workspace_bytes,
                       void* stream);

/* Embedding backward, accumulating:
 *   dwte[tokens[b,t], :] += dout[b,t,:]   (each row summed over its positions in ascending order)
 *   dwpe[t, :] += sum_b dout[b,t,:]
 * either output may be NULL. tokens int32 [B,T] in [0, Vp) (not checked on
 * the device). C % 8 == 0, C <= 4096 (fp32) / 8192 (bf16). */
int encoder_backward(void* dwte, void* dwpe, const void* dout, const int32_t* tokens, int B, int T, int C,
                     int dtype, void* stream);

/* ------------------------------------------------------- training step
 * gpt2_train_forward runs the forward (encoder, blocks, lnf, logits) keeping
 * every activation the backward needs in acts (gpt2_train_acts_bytes), then
 * the fused classifier: per-row losses against targets int32 [B,T] (losses
 * fp32 [B*T], nullable), their mean (mean_loss fp32 [1], nullable) and, over
 * the logits inside acts, the gradient of the mean loss with respect to them.
 * gpt2_backward then writes the gradient of that mean loss with respect to
 * every parameter into grads (the flat parameter layout, overwritten), using
 * acts and the workspace (gpt2_train_workspace_bytes). Head size 16, 32 or 64.
 * The optimizer is not part of this library. */
int64_t gpt2_train_acts_bytes(const gpt2_config* cfg /* host */, int B, int T);
int64_t gpt2_train_workspace_bytes(const gpt2_config* cfg /* host */, int B, int T);
int gpt2_train_forward(float* losses, float* mean_loss, const int32_t* tokens, const int32_t* targets,
                       const void* params, const gpt2_config* cfg /* host */, int B, int T, void* acts,
                       int64_t acts_bytes, void* stream);
int gpt2_backward(void* grads, const int32_t* tokens, const void* params, const gpt2_config* cfg /* host */,
                  int B, int T, void* acts, int64_t acts_bytes, void* workspace, int64_t workspace_bytes,
                  void* stream);

/* ---------------------------------------------------------------- status */
const char* gpt2_status_string(int status);  /* static string, never NULL */
int gpt2_last_hip_error(void);               /* hipError_t of this thread's last failure */

#ifdef __cplusplus
}
#endif
#endif
