/*
 * oracle.h - plain, slow, single-threaded CPU GPT-2 forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists to check the GPU library.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it. It shares no code, header, table or helper with the GPU library
 * and neither one includes or links the other.
 *
 * Precision: every tensor passed from one step to the next is fp32; inside a
 * step, each dot product and reduction accumulates in double and is rounded to
 * fp32 once. tanh and exp are libm's, in double.
 *
 * Layouts (all row-major, contiguous):
 *   tokens  int32 [B,T]
 *   qkv     [B,T,3C] = [q | k | v]; head h occupies columns h*hs..(h+1)*hs-1
 *           of each third (hs = C/NH)
 *   linear weights [OC,C]: out = inp * W^T + bias
 *   params  one flat fp32 buffer:
 *           wte[Vp,C] wpe[maxT,C] ln1_g[L,C] ln1_b[L,C] qkv_w[L,3C,C] qkv_b[L,3C]
 *           attproj_w[L,C,C] attproj_b[L,C] ln2_g[L,C] ln2_b[L,C] fc_w[L,4C,C]
 *           fc_b[L,4C] fcproj_w[L,C,4C] fcproj_b[L,C] lnf_g[C] lnf_b[C]
 *   kv cache [L,B,NH,maxT,hs]
 *
 * Parity status: every function below (forward and backward) is pinned by the CPU test suite
 * (closed forms, identities, brute force, a library GPT-2) except the full-size
 * logits of the 124M/350M workloads, which the pages print no values for.
 */
#ifndef GPT2_ORACLE_H
#define GPT2_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

void oracle_encoder(float* out, const int32_t* tokens, const float* wte, const float* wpe,
                    int B, int T, int C);
void oracle_layernorm(float* out, float* mean, float* rstd, const float* inp,
                      const float* gamma, const float* beta, int N, int C, double eps);
void oracle_matmul(float* out, const float* inp, const float* weight, const float* bias,
                   int N, int C, int OC);
void oracle_attention(float* out, const float* qkv, int B, int T, int C, int NH);
void oracle_gelu(float* out, const float* inp, int64_t n);
void oracle_residual(float* out, const float* a, const float* b, int64_t n);
void oracle_softmax(float* probs, const float* logits, int N, int V, int Vp);
void oracle_crossentropy(float* losses, const float* logits, const int32_t* targets, int N, int V, int Vp);

int64_t oracle_param_count(int L, int C, int maxT, int Vp);
/* Floats in the capture buffer of oracle_forward: N*C*(2 + 18*L), N = B*T.
 * Order: encoder out [N,C]; per layer: ln1 [N,C], qkv [N,3C], attention [N,C],
 * attproj [N,C], residual1 [N,C], ln2 [N,C], fc [N,4C], gelu [N,4C],
 * fcproj [N,C], residual2 [N,C]; then lnf [N,C]. */
int64_t oracle_capture_count(int L, int C, int B, int T);

/* Returns 0 on success, nonzero on a bad argument or allocation failure.
 * probs and capture may be NULL. logits/probs are [B,T,Vp]. */
int oracle_forward(float* logits, float* probs, const int32_t* tokens, const float* params,
                   int L, int C, int NH, int V, int Vp, int maxT, double eps,
                   int B, int T, float* capture);

/* One decode step: tokens [B] at position pos (0 <= pos < maxT). For every
 * layer, writes the new key and value rows into kcache/vcache at pos, then
 * attends over positions 0..pos. logits/probs are [B,Vp]. */
int oracle_decode_step(float* logits, float* probs, const int32_t* tokens, int pos,
                       float* kcache, float* vcache, const float* params,
                       int L, int C, int NH, int V, int Vp, int maxT, double eps, int B);

/* ------------------------------------------------------------------ backward
 * Outputs are overwritten unless stated; optional outputs may be NULL. */
void oracle_crossentropy_backward(float* dlogits, const float* logits, const int32_t* targets,
                                  double dloss, int N, int V, int Vp);
void oracle_matmul_backward(float* dinp, float* dweight, float* dbias, const float* dout,
                            const float* inp, const float* weight, int N, int C, int OC);
void oracle_layernorm_backward(float* dinp, float* dgamma, float* dbeta, const float* dout,
                               const float* inp, const float* gamma, int N, int C, double eps);
void oracle_gelu_backward(float* dinp, const float* inp, const float* dout, int64_t n);
/* lse [B,NH,T] */
void oracle_attention_lse(float* lse, const float* qkv, int B, int T, int C, int NH);
void oracle_attention_backward(float* dqkv, const float* dout, const float* qkv, int B, int T, int C,
                               int NH);
/* accumulates into dwte [Vp,C] and dwpe [maxT,C] (dwpe may be NULL) */
void oracle_encoder_backward(float* dwte, float* dwpe, const float* dout, const int32_t* tokens,
                             int B, int T, int C);
/* grads: flat buffer in the parameter layout (overwritten); loss may be NULL. */
int oracle_backward(float* grads, float* loss, const int32_t* tokens, const int32_t* targets,
                    const float* params, int L, int C, int NH, int V, int Vp, int maxT, double eps,
                    int B, int T);

#ifdef __cplusplus
}
#endif
#endif
