/*
 * oracle.c - plain, slow, single-threaded CPU GPT-2 forward pass.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h). Nothing in the GPU library uses
 * this file, and nothing here is taken from the GPU library.
 *
 * The steps follow the per-kernel decomposition of the forward pass in
 * "ECE408 Final Project - GPT-2, Milestone 1" (Code Submission and Grading,
 * kernel table: Encoder, LayerNorm, MatMul, Attention including Softmax,
 * Residual, GELU). The pages name the steps but do not write out their
 * mathematics; each function states the standard GPT-2 definition it uses.
 * Attention is the standard algorithm that materialises the score and
 * probability matrices ("Algorithm 0" in the optdl2025 project
 * "Understand FlashAttention (I)"), which gives the same exact result as the
 * tiled online-softmax algorithm the GPU uses.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (no reassociation, no FMA
 * contraction), so every operation is the IEEE operation written here.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Token + position embedding: out[b,t,:] = wte[tokens[b,t],:] + wpe[t,:],
 * one fp32 addition per element.
 * (ECE408 Milestone 1, kernel table: Encoder.) */
void oracle_encoder(float* out, const int32_t* tokens, const float* wte, const float* wpe,
                    int B, int T, int C) {
    for (int b = 0; b < B; b++)
        for (int t = 0; t < T; t++) {
            const float* e = wte + (int64_t)tokens[b * T + t] * C;
            const float* p = wpe + (int64_t)t * C;
            float* o = out + ((int64_t)b * T + t) * C;
            for (int c = 0; c < C; c++) o[c] = e[c] + p[c];
        }
}

/* LayerNorm over the last dimension, biased variance, eps inside the root:
 *   mu = (1/C) sum x,  var = (1/C) sum (x - mu)^2,  rstd = 1/sqrt(var + eps),
 *   y = (x - mu) * rstd * gamma + beta.
 * mean and rstd (nullable) receive the fp32-rounded statistics.
 * (ECE408 Milestone 1, kernel table: LayerNorm.) */
void oracle_layernorm(float* out, float* mean, float* rstd, const float* inp,
                      const float* gamma, const float* beta, int N, int C, double eps) {
    for (int n = 0; n < N; n++) {
        const float* x = inp + (int64_t)n * C;
        double s = 0.0;
        for (int c = 0; c < C; c++) s += (double)x[c];
        double mu = s / C;
        double v = 0.0;
        for (int c = 0; c < C; c++) {
            double d = (double)x[c] - mu;
            v += d * d;
        }
        v /= C;
        double r = 1.0 / sqrt(v + eps);
        float* y = out + (int64_t)n * C;
        for (int c = 0; c < C; c++)
            y[c] = (float)(((double)x[c] - mu) * r * (double)gamma[c] + (double)beta[c]);
        if (mean) mean[n] = (float)mu;
        if (rstd) rstd[n] = (float)r;
    }
}

/* Linear layer: out[n,o] = sum_c inp[n,c] * W[o,c] + bias[o] (bias nullable),
 * the dot product accumulated in double.
 * (ECE408 Milestone 1, kernel table: MatMul; the optdl2025 project "A study on
 * GPU for matrix-matrix products" describes the same product, one output entry
 * per inner product.) */
void oracle_matmul(float* out, const float* inp, const float* weight, const float* bias,
                   int N, int C, int OC) {
    for (int n = 0; n < N; n++) {
        const float* a = inp + (int64_t)n * C;
        for (int o = 0; o < OC; o++) {
            const float* w = weight + (int64_t)o * C;
            double acc = bias ? (double)bias[o] : 0.0;
            for (int c = 0; c < C; c++) acc += (double)a[c] * (double)w[c];
            out[(int64_t)n * OC + o] = (float)acc;
        }
    }
}

/* Causal multi-head self-attention over a packed qkv tensor.
 * For batch b, head h, query t:
 *   S[t][j] = q_t . k_j / sqrt(hs)          for j <= t
 *   P[t][.] = softmax over j <= t of S[t][.] (row max subtracted first)
 *   y_t     = sum_{j<=t} P[t][j] v_j
 * Keys after t are excluded (they contribute exactly 0). S and P are
 * materialised in full, as in the standard algorithm ("Algorithm 0" of the
 * optdl2025 project "Understand FlashAttention (I)"). q, k and v come from one
 * packed projection and heads are contiguous column slices of each third (the
 * optdl2025 NanoGPT project: one projection for queries, keys and values;
 * head splitting). (ECE408 Milestone 1, kernel table: Attention including
 * Softmax.) */
void oracle_attention(float* out, const float* qkv, int B, int T, int C, int NH) {
    int hs = C / NH;
    double scale = 1.0 / sqrt((double)hs);
    double* S = (double*)malloc(sizeof(double) * (size_t)T * (size_t)T);
    if (!S) return;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++) {
            /* scores and the masked softmax, row by row */
            for (int t = 0; t < T; t++) {
                const float* q = qkv + ((int64_t)b * T + t) * 3 * C + h * hs;
                double* row = S + (int64_t)t * T;
                double mx = -INFINITY;
                for (int j = 0; j <= t; j++) {
                    const float* k = qkv + ((int64_t)b * T + j) * 3 * C + C + h * hs;
                    double d = 0.0;
                    for (int e = 0; e < hs; e++) d += (double)q[e] * (double)k[e];
                    row[j] = d * scale;
                    if (row[j] > mx) mx = row[j];
                }
                double sum = 0.0;
                for (int j = 0; j <= t; j++) {
                    row[j] = exp(row[j] - mx);
                    sum += row[j];
                }
                for (int j = 0; j <= t; j++) row[j] /= sum;
                for (int j = t + 1; j < T; j++) row[j] = 0.0;
            }
            /* y = P V */
            for (int t = 0; t < T; t++) {
                const double* row = S + (int64_t)t * T;
                float* y = out + ((int64_t)b * T + t) * C + h * hs;
                for (int e = 0; e < hs; e++) {
                    double acc = 0.0;
                    for (int j = 0; j <= t; j++) {
                        const float* v = qkv + ((int64_t)b * T + j) * 3 * C + 2 * C + h * hs;
                        acc += row[j] * (double)v[e];
                    }
                    y[e] = (float)acc;
                }
            }
        }
    free(S);
}

/* GELU, tanh form: g(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))).
 * (ECE408 Milestone 1, kernel table: GELU.) */
void oracle_gelu(float* out, const float* inp, int64_t n) {
    const double k = sqrt(2.0 / M_PI);
    for (int64_t i = 0; i < n; i++) {
        double x = (double)inp[i];
        out[i] = (float)(0.5 * x * (1.0 + tanh(k * (x + 0.044715 * x * x * x))));
    }
}

/* Residual connection: out = a + b, one fp32 addition per element.
 * (ECE408 Milestone 1, kernel table: Residual.) */
void oracle_residual(float* out, const float* a, const float* b, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = a[i] + b[i];
}

/* Softmax over the vocabulary of each row of a [N,Vp] logits tensor: only the
 * first V columns are real tokens; columns V..Vp-1 are padding and get
 * probability exactly 0.
 *   m = max_{v<V} l_v,  p_v = exp(l_v - m) / sum_{u<V} exp(l_u - m).
 * (The forward half of the llm.c classifier, "State of the Union [April 22,
 * 2024]", kernel summaries: fused_classifier_kernel3.) */
void oracle_softmax(float* probs, const float* logits, int N, int V, int Vp) {
    for (int n = 0; n < N; n++) {
        const float* l = logits + (int64_t)n * Vp;
        float* p = probs + (int64_t)n * Vp;
        double mx = -INFINITY;
        for (int v = 0; v < V; v++)
            if ((double)l[v] > mx) mx = (double)l[v];
        double sum = 0.0;
        for (int v = 0; v < V; v++) sum += exp((double)l[v] - mx);
        for (int v = 0; v < V; v++) p[v] = (float)(exp((double)l[v] - mx) / sum);
        for (int v = V; v < Vp; v++) p[v] = 0.0f;
    }
}

/* Cross-entropy of each row against its target token t_n (0 <= t_n < V):
 *   loss_n = -log softmax(l_n)[t_n] = log(sum_{v<V} exp(l_v - m)) + m - l_{t_n},
 * the log-sum-exp form (no probability is rounded before the log). The loss
 * half of the llm.c classifier (fused_classifier_kernel3). */
void oracle_crossentropy(float* losses, const float* logits, const int32_t* targets, int N, int V, int Vp) {
    for (int n = 0; n < N; n++) {
        const float* l = logits + (int64_t)n * Vp;
        double mx = -INFINITY;
        for (int v = 0; v < V; v++)
            if ((double)l[v] > mx) mx = (double)l[v];
        double sum = 0.0;
        for (int v = 0; v < V; v++) sum += exp((double)l[v] - mx);
        losses[n] = (float)(log(sum) + mx - (double)l[targets[n]]);
    }
}

int64_t oracle_param_count(int L, int C, int maxT, int Vp) {
    int64_t c = C;
    return (int64_t)Vp * c + (int64_t)maxT * c + (int64_t)L * (12 * c * c + 13 * c) + 2 * c;
}

int64_t oracle_capture_count(int L, int C, int B, int T) {
    return (int64_t)B * T * C * (2 + 18 * (int64_t)L);
}

/* Pointers into the flat parameter buffer for layer l. */
typedef struct {
    const float *wte, *wpe, *ln1_g, *ln1_b, *qkv_w, *qkv_b, *attproj_w, *attproj_b;
    const float *ln2_g, *ln2_b, *fc_w, *fc_b, *fcproj_w, *fcproj_b, *lnf_g, *lnf_b;
} layer_params;

static layer_params params_at(const float* p, int L, int C, int maxT, int Vp, int l) {
    int64_t c = C;
    layer_params r;
    const float* q = p;
    r.wte = q;                q += (int64_t)Vp * c;
    r.wpe = q;                q += (int64_t)maxT * c;
    const float* ln1_g = q;   q += L * c;
    const float* ln1_b = q;   q += L * c;
    const float* qkv_w = q;   q += L * 3 * c * c;
    const float* qkv_b = q;   q += L * 3 * c;
    const float* ap_w = q;    q += L * c * c;
    const float* ap_b = q;    q += L * c;
    const float* ln2_g = q;   q += L * c;
    const float* ln2_b = q;   q += L * c;
    const float* fc_w = q;    q += L * 4 * c * c;
    const float* fc_b = q;    q += L * 4 * c;
    const float* fp_w = q;    q += L * 4 * c * c;
    const float* fp_b = q;    q += L * c;
    r.lnf_g = q;              q += c;
    r.lnf_b = q;
    r.ln1_g = ln1_g + l * c;            r.ln1_b = ln1_b + l * c;
    r.qkv_w = qkv_w + l * 3 * c * c;    r.qkv_b = qkv_b + l * 3 * c;
    r.attproj_w = ap_w + l * c * c;     r.attproj_b = ap_b + l * c;
    r.ln2_g = ln2_g + l * c;            r.ln2_b = ln2_b + l * c;
    r.fc_w = fc_w + l * 4 * c * c;      r.fc_b = fc_b + l * 4 * c;
    r.fcproj_w = fp_w + l * 4 * c * c;  r.fcproj_b = fp_b + l * c;
    return r;
}

static float* cap(float* capture, int64_t* off, const float* src, int64_t n) {
    if (capture) {
        memcpy(capture + *off, src, sizeof(float) * (size_t)n);
        *off += n;
    }
    return capture;
}

/* The GPT-2 forward pass: pre-LayerNorm blocks
 *   x <- x + attproj(attention(ln1(x)))
 *   x <- x + fcproj(gelu(fc(ln2(x))))
 * then a final LayerNorm, logits against the (tied) token embedding, no bias,
 * and the vocabulary softmax. Composition of the steps listed in ECE408
 * Milestone 1 (kernel table) in GPT-2's order; the llm.c summary ("State of the
 * Union", step breakdown) splits the same pass into encoder, forward blocks and
 * classifier. */
int oracle_forward(float* logits, float* probs, const int32_t* tokens, const float* params,
                   int L, int C, int NH, int V, int Vp, int maxT, double eps,
                   int B, int T, float* capture) {
    if (!logits || !tokens || !params || L < 0 || C <= 0 || NH <= 0 || C % NH ||
        V <= 0 || Vp < V || T <= 0 || T > maxT || B <= 0)
        return 1;
    int64_t N = (int64_t)B * T, c = C;
    float* x = (float*)malloc(sizeof(float) * N * c);
    float* a = (float*)malloc(sizeof(float) * N * c);
    float* qkv = (float*)malloc(sizeof(float) * N * 3 * c);
    float* y = (float*)malloc(sizeof(float) * N * c);
    float* f = (float*)malloc(sizeof(float) * N * 4 * c);
    float* g = (float*)malloc(sizeof(float) * N * 4 * c);
    if (!x || !a || !qkv || !y || !f || !g) {
        free(x); free(a); free(qkv); free(y); free(f); free(g);
        return 2;
    }
    int64_t off = 0;
    layer_params p0 = params_at(params, L, C, maxT, Vp, 0);
    oracle_encoder(x, tokens, p0.wte, p0.wpe, B, T, C);
    cap(capture, &off, x, N * c);
    for (int l = 0; l < L; l++) {
        layer_params p = params_at(params, L, C, maxT, Vp, l);
        oracle_layernorm(a, NULL, NULL, x, p.ln1_g, p.ln1_b, (int)N, C, eps);
        cap(capture, &off, a, N * c);
        oracle_matmul(qkv, a, p.qkv_w, p.qkv_b, (int)N, C, 3 * C);
        cap(capture, &off, qkv, N * 3 * c);
        oracle_attention(y, qkv, B, T, C, NH);
        cap(capture, &off, y, N * c);
        oracle_matmul(a, y, p.attproj_w, p.attproj_b, (int)N, C, C);
        cap(capture, &off, a, N * c);
        oracle_residual(x, x, a, N * c);
        cap(capture, &off, x, N * c);
        oracle_layernorm(a, NULL, NULL, x, p.ln2_g, p.ln2_b, (int)N, C, eps);
        cap(capture, &off, a, N * c);
        oracle_matmul(f, a, p.fc_w, p.fc_b, (int)N, C, 4 * C);
        cap(capture, &off, f, N * 4 * c);
        oracle_gelu(g, f, N * 4 * c);
        cap(capture, &off, g, N * 4 * c);
        oracle_matmul(a, g, p.fcproj_w, p.fcproj_b, (int)N, 4 * C, C);
        cap(capture, &off, a, N * c);
        oracle_residual(x, x, a, N * c);
        cap(capture, &off, x, N * c);
    }
    oracle_layernorm(a, NULL, NULL, x, p0.lnf_g, p0.lnf_b, (int)N, C, eps);
    cap(capture, &off, a, N * c);
    oracle_matmul(logits, a, p0.wte, NULL, (int)N, C, Vp);
    if (probs) oracle_softmax(probs, logits, (int)N, V, Vp);
    free(x); free(a); free(qkv); free(y); free(f); free(g);
    return 0;
}

/* Attention of one new query per sequence over a key/value cache that already
 * holds this step's key and value at pos (the optdl2025 NanoGPT project, KV
 * caching for autoregressive prediction). Same definition as oracle_attention
 * restricted to the last row: keys 0..pos. */
static void decode_attention(float* out, const float* qkv, const float* kc, const float* vc,
                             int B, int pos, int maxT, int C, int NH) {
    int hs = C / NH;
    double scale = 1.0 / sqrt((double)hs);
    double* s = (double*)malloc(sizeof(double) * (size_t)(pos + 1));
    if (!s) return;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++) {
            const float* q = qkv + (int64_t)b * 3 * C + h * hs;
            const float* K = kc + (((int64_t)b * NH + h) * maxT) * hs;
            const float* Vv = vc + (((int64_t)b * NH + h) * maxT) * hs;
            double mx = -INFINITY;
            for (int j = 0; j <= pos; j++) {
                double d = 0.0;
                for (int e = 0; e < hs; e++) d += (double)q[e] * (double)K[(int64_t)j * hs + e];
                s[j] = d * scale;
                if (s[j] > mx) mx = s[j];
            }
            double sum = 0.0;
            for (int j = 0; j <= pos; j++) {
                s[j] = exp(s[j] - mx);
                sum += s[j];
            }
            float* y = out + (int64_t)b * C + h * hs;
            for (int e = 0; e < hs; e++) {
                double acc = 0.0;
                for (int j = 0; j <= pos; j++) acc += (s[j] / sum) * (double)Vv[(int64_t)j * hs + e];
                y[e] = (float)acc;
            }
        }
    free(s);
}

int oracle_decode_step(float* logits, float* probs, const int32_t* tokens, int pos,
                       float* kcache, float* vcache, const float* params,
                       int L, int C, int NH, int V, int Vp, int maxT, double eps, int B) {
    if (!logits || !tokens || !params || !kcache || !vcache || L < 0 || C <= 0 || NH <= 0 ||
        C % NH || V <= 0 || Vp < V || pos < 0 || pos >= maxT || B <= 0)
        return 1;
    int64_t c = C;
    int hs = C / NH;
    float* x = (float*)malloc(sizeof(float) * B * c);
    float* a = (float*)malloc(sizeof(float) * B * c);
    float* qkv = (float*)malloc(sizeof(float) * B * 3 * c);
    float* y = (float*)malloc(sizeof(float) * B * c);
    float* f = (float*)malloc(sizeof(float) * B * 4 * c);
    float* g = (float*)malloc(sizeof(float) * B * 4 * c);
    if (!x || !a || !qkv || !y || !f || !g) {
        free(x); free(a); free(qkv); free(y); free(f); free(g);
        return 2;
    }
    layer_params p0 = params_at(params, L, C, maxT, Vp, 0);
    /* position embedding row pos for every sequence */
    for (int b = 0; b < B; b++)
        for (int e = 0; e < C; e++)
            x[(int64_t)b * C + e] = p0.wte[(int64_t)tokens[b] * C + e] + p0.wpe[(int64_t)pos * C + e];
    int64_t layer_stride = (int64_t)B * NH * maxT * hs;
    for (int l = 0; l < L; l++) {
        layer_params p = params_at(params, L, C, maxT, Vp, l);
        float* kc = kcache + l * layer_stride;
        float* vc = vcache + l * layer_stride;
        oracle_layernorm(a, NULL, NULL, x, p.ln1_g, p.ln1_b, B, C, eps);
        oracle_matmul(qkv, a, p.qkv_w, p.qkv_b, B, C, 3 * C);
        for (int b = 0; b < B; b++)
            for (int h = 0; h < NH; h++)
                for (int e = 0; e < hs; e++) {
                    int64_t dst = (((int64_t)b * NH + h) * maxT + pos) * hs + e;
                    kc[dst] = qkv[(int64_t)b * 3 * C + C + h * hs + e];
                    vc[dst] = qkv[(int64_t)b * 3 * C + 2 * C + h * hs + e];
                }
        decode_attention(y, qkv, kc, vc, B, pos, maxT, C, NH);
        oracle_matmul(a, y, p.attproj_w, p.attproj_b, B, C, C);
        oracle_residual(x, x, a, B * c);
        oracle_layernorm(a, NULL, NULL, x, p.ln2_g, p.ln2_b, B, C, eps);
        oracle_matmul(f, a, p.fc_w, p.fc_b, B, C, 4 * C);
        oracle_gelu(g, f, B * 4 * c);
        oracle_matmul(a, g, p.fcproj_w, p.fcproj_b, B, 4 * C, C);
        oracle_residual(x, x, a, B * c);
    }
    oracle_layernorm(a, NULL, NULL, x, p0.lnf_g, p0.lnf_b, B, C, eps);
    oracle_matmul(logits, a, p0.wte, NULL, B, C, Vp);
    if (probs) oracle_softmax(probs, logits, B, V, Vp);
    free(x); free(a); free(qkv); free(y); free(f); free(g);
    return 0;
}

/* ===================================================================== backward
 * Gradients of the same steps (the backward kernels of the llm.c training step,
 * "State of the Union [April 22, 2024]", kernel summaries; attention after
 * "Understand FlashAttention (II)", which asks for the backward of the standard
 * algorithm). Each sum or dot product accumulates in double and every output
 * is rounded to fp32 once. The derivations are the standard calculus of each
 * forward definition above; the CPU test suite checks them against float64
 * automatic differentiation of library operations and against central finite
 * differences.
 */

/* Cross-entropy backward fused with the softmax (the backward half of the llm.c
 * classifier): for the loss sum_n dloss * loss_n,
 *   dlogits[n,v] = dloss * (p_v - [v == t_n])   for v < V,
 * with p the softmax over the V real columns, and 0 in the padding columns. */
void oracle_crossentropy_backward(float* dlogits, const float* logits, const int32_t* targets,
                                  double dloss, int N, int V, int Vp) {
    for (int n = 0; n < N; n++) {
        const float* l = logits + (int64_t)n * Vp;
        float* d = dlogits + (int64_t)n * Vp;
        double mx = -INFINITY;
        for (int v = 0; v < V; v++)
            if ((double)l[v] > mx) mx = (double)l[v];
        double sum = 0.0;
        for (int v = 0; v < V; v++) sum += exp((double)l[v] - mx);
        for (int v = 0; v < V; v++) {
            double p = exp((double)l[v] - mx) / sum;
            d[v] = (float)(dloss * (p - (v == targets[n] ? 1.0 : 0.0)));
        }
        for (int v = V; v < Vp; v++) d[v] = 0.0f;
    }
}

/* Linear backward, for out = inp W^T + b and the incoming gradient dout [N,OC]:
 *   dinp[n,c] = sum_o dout[n,o] W[o,c],   dW[o,c] = sum_n dout[n,o] inp[n,c],
 *   db[o] = sum_n dout[n,o].
 * Each output is optional (NULL) and overwritten. */
void oracle_matmul_backward(float* dinp, float* dweight, float* dbias, const float* dout,
                            const float* inp, const float* weight, int N, int C, int OC) {
    if (dinp)
        for (int n = 0; n < N; n++)
            for (int c = 0; c < C; c++) {
                double acc = 0.0;
                for (int o = 0; o < OC; o++)
                    acc += (double)dout[(int64_t)n * OC + o] * (double)weight[(int64_t)o * C + c];
                dinp[(int64_t)n * C + c] = (float)acc;
            }
    if (dweight)
        for (int o = 0; o < OC; o++)
            for (int c = 0; c < C; c++) {
                double acc = 0.0;
                for (int n = 0; n < N; n++)
                    acc += (double)dout[(int64_t)n * OC + o] * (double)inp[(int64_t)n * C + c];
                dweight[(int64_t)o * C + c] = (float)acc;
            }
    if (dbias)
        for (int o = 0; o < OC; o++) {
            double acc = 0.0;
            for (int n = 0; n < N; n++) acc += (double)dout[(int64_t)n * OC + o];
            dbias[o] = (float)acc;
        }
}

/* LayerNorm backward. With xh = (x - mu) rstd (mu, rstd recomputed from x in
 * double exactly as oracle_layernorm defines them), y = xh gamma + beta, and
 * g = dy gamma:
 *   dx = rstd (g - mean_c(g) - xh mean_c(g xh)),
 *   dgamma[c] = sum_n dy xh,   dbeta[c] = sum_n dy.
 * (dx follows from d rstd / dx = -rstd^3 (x - mu) / C and d mu / dx = 1/C.)
 * dinp is overwritten; dgamma and dbeta (optional) are overwritten. */
void oracle_layernorm_backward(float* dinp, float* dgamma, float* dbeta, const float* dout,
                               const float* inp, const float* gamma, int N, int C, double eps) {
    double* xh = (double*)malloc(sizeof(double) * (size_t)N * (size_t)C);
    if (!xh) return;
    for (int n = 0; n < N; n++) {
        const float* x = inp + (int64_t)n * C;
        const float* dy = dout + (int64_t)n * C;
        double s = 0.0;
        for (int c = 0; c < C; c++) s += (double)x[c];
        double mu = s / C, v = 0.0;
        for (int c = 0; c < C; c++) v += ((double)x[c] - mu) * ((double)x[c] - mu);
        double r = 1.0 / sqrt(v / C + eps);
        double mg = 0.0, mgx = 0.0;
        for (int c = 0; c < C; c++) {
            double h = ((double)x[c] - mu) * r;
            xh[(int64_t)n * C + c] = h;
            double g = (double)dy[c] * (double)gamma[c];
            mg += g;
            mgx += g * h;
        }
        mg /= C;
        mgx /= C;
        for (int c = 0; c < C; c++) {
            double h = xh[(int64_t)n * C + c];
            double g = (double)dy[c] * (double)gamma[c];
            dinp[(int64_t)n * C + c] = (float)(r * (g - mg - h * mgx));
        }
    }
    for (int c = 0; c < C; c++) {
        double sg = 0.0, sb = 0.0;
        for (int n = 0; n < N; n++) {
            double dy = (double)dout[(int64_t)n * C + c];
            sg += dy * xh[(int64_t)n * C + c];
            sb += dy;
        }
        if (dgamma) dgamma[c] = (float)sg;
        if (dbeta) dbeta[c] = (float)sb;
    }
    free(xh);
}

/* GELU backward: with u = sqrt(2/pi) (x + 0.044715 x^3),
 *   g'(x) = (1 + tanh u)/2 + (x/2)(1 - tanh^2 u) sqrt(2/pi)(1 + 3*0.044715 x^2),
 *   dinp = dout g'(x). */
void oracle_gelu_backward(float* dinp, const float* inp, const float* dout, int64_t n) {
    const double k = sqrt(2.0 / M_PI);
    for (int64_t i = 0; i < n; i++) {
        double x = (double)inp[i];
        double t = tanh(k * (x + 0.044715 * x * x * x));
        double d = 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * k * (1.0 + 3.0 * 0.044715 * x * x);
        dinp[i] = (float)((double)dout[i] * d);
    }
}

/* The natural log-sum-exp of every causal score row, lse[b,h,t] =
 * log sum_{j<=t} exp(S[t][j]) with S as in oracle_attention: what a tiled
 * (FlashAttention) forward keeps per query row so its backward can rebuild P
 * as exp(S - lse). */
void oracle_attention_lse(float* lse, const float* qkv, int B, int T, int C, int NH) {
    int hs = C / NH;
    double scale = 1.0 / sqrt((double)hs);
    double* s = (double*)malloc(sizeof(double) * (size_t)T);
    if (!s) return;
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++)
            for (int t = 0; t < T; t++) {
                const float* q = qkv + ((int64_t)b * T + t) * 3 * C + h * hs;
                double mx = -INFINITY;
                for (int j = 0; j <= t; j++) {
                    const float* k = qkv + ((int64_t)b * T + j) * 3 * C + C + h * hs;
                    double d = 0.0;
                    for (int e = 0; e < hs; e++) d += (double)q[e] * (double)k[e];
                    s[j] = d * scale;
                    if (s[j] > mx) mx = s[j];
                }
                double sum = 0.0;
                for (int j = 0; j <= t; j++) sum += exp(s[j] - mx);
                lse[((int64_t)b * NH + h) * T + t] = (float)(mx + log(sum));
            }
    free(s);
}

/* Attention backward, the backward of the standard algorithm (materialised S
 * and P, "Understand FlashAttention (II)"). Per batch b and head h, with
 * S = Q K^T / sqrt(hs) over j <= t, P = row softmax of S, O = P V and the
 * incoming dO:
 *   dV = P^T dO,   dP = dO V^T,   dS[t][j] = P[t][j] (dP[t][j] - sum_j' P[t][j'] dP[t][j']),
 *   dQ = dS K / sqrt(hs),   dK = dS^T Q / sqrt(hs).
 * dqkv [B,T,3C] has the packed layout of qkv and is overwritten. */
void oracle_attention_backward(float* dqkv, const float* dout, const float* qkv, int B, int T, int C,
                               int NH) {
    int hs = C / NH;
    double scale = 1.0 / sqrt((double)hs);
    double* P = (double*)malloc(sizeof(double) * (size_t)T * (size_t)T);
    double* dS = (double*)malloc(sizeof(double) * (size_t)T * (size_t)T);
    if (!P || !dS) {
        free(P); free(dS);
        return;
    }
#define Q_(t, e) ((double)qkv[((int64_t)b * T + (t)) * 3 * C + h * hs + (e)])
#define K_(t, e) ((double)qkv[((int64_t)b * T + (t)) * 3 * C + C + h * hs + (e)])
#define V_(t, e) ((double)qkv[((int64_t)b * T + (t)) * 3 * C + 2 * C + h * hs + (e)])
#define DO_(t, e) ((double)dout[((int64_t)b * T + (t)) * C + h * hs + (e)])
    for (int b = 0; b < B; b++)
        for (int h = 0; h < NH; h++) {
            for (int t = 0; t < T; t++) {
                double* p = P + (int64_t)t * T;
                double mx = -INFINITY;
                for (int j = 0; j <= t; j++) {
                    double d = 0.0;
                    for (int e = 0; e < hs; e++) d += Q_(t, e) * K_(j, e);
                    p[j] = d * scale;
                    if (p[j] > mx) mx = p[j];
                }
                double sum = 0.0;
                for (int j = 0; j <= t; j++) {
                    p[j] = exp(p[j] - mx);
                    sum += p[j];
                }
                for (int j = 0; j <= t; j++) p[j] /= sum;
                /* dP row and dS row */
                double* ds = dS + (int64_t)t * T;
                double dot = 0.0;
                for (int j = 0; j <= t; j++) {
                    double d = 0.0;
                    for (int e = 0; e < hs; e++) d += DO_(t, e) * V_(j, e);
                    ds[j] = d; /* dP for now */
                    dot += p[j] * d;
                }
                for (int j = 0; j <= t; j++) ds[j] = p[j] * (ds[j] - dot);
            }
            for (int t = 0; t < T; t++) {
                float* dq = dqkv + ((int64_t)b * T + t) * 3 * C + h * hs;
                float* dk = dq + C;
                float* dv = dq + 2 * C;
                for (int e = 0; e < hs; e++) {
                    double aq = 0.0, ak = 0.0, av = 0.0;
                    for (int j = 0; j <= t; j++) aq += dS[(int64_t)t * T + j] * K_(j, e);
                    for (int i = t; i < T; i++) {
                        ak += dS[(int64_t)i * T + t] * Q_(i, e);
                        av += P[(int64_t)i * T + t] * DO_(i, e);
                    }
                    dq[e] = (float)(aq * scale);
                    dk[e] = (float)(ak * scale);
                    dv[e] = (float)av;
                }
            }
        }
#undef Q_
#undef K_
#undef V_
#undef DO_
    free(P);
    free(dS);
}

/* Encoder backward, accumulating: for every vocabulary row v that occurs,
 * dwte[v,:] += sum over positions (b,t) with tokens[b,t] == v of dout[b,t,:];
 * dwpe[t,:] += sum_b dout[b,t,:]. Each sum is taken in double and added to the
 * existing fp32 value once. (The token embedding is tied to the logits
 * weight, so its gradient collects both uses.) */
void oracle_encoder_backward(float* dwte, float* dwpe, const float* dout, const int32_t* tokens,
                             int B, int T, int C) {
    int N = B * T;
    for (int n = 0; n < N; n++) {
        int v = tokens[n];
        int first = 1;
        for (int m = 0; m < n; m++)
            if (tokens[m] == v) { first = 0; break; }
        if (!first) continue;
        for (int c = 0; c < C; c++) {
            double acc = 0.0;
            for (int m = n; m < N; m++)
                if (tokens[m] == v) acc += (double)dout[(int64_t)m * C + c];
            dwte[(int64_t)v * C + c] = (float)((double)dwte[(int64_t)v * C + c] + acc);
        }
    }
    if (dwpe)
        for (int t = 0; t < T; t++)
            for (int c = 0; c < C; c++) {
                double acc = 0.0;
                for (int b = 0; b < B; b++) acc += (double)dout[((int64_t)b * T + t) * C + c];
                dwpe[(int64_t)t * C + c] = (float)((double)dwpe[(int64_t)t * C + c] + acc);
            }
}

/* Gradient of the mean cross-entropy loss L = (1/N) sum_n loss_n (N = B*T,
 * targets [B,T]) with respect to every parameter, in the flat parameter
 * layout. Runs the steps of oracle_forward keeping every intermediate, then
 * the backward steps above in reverse order; the residual stream's gradient
 * is the sum of the gradient passed straight through and the branch's. *loss
 * (optional) receives L. Returns 0 on success. */
int oracle_backward(float* grads, float* loss, const int32_t* tokens, const int32_t* targets,
                    const float* params, int L, int C, int NH, int V, int Vp, int maxT, double eps,
                    int B, int T) {
    if (!grads || !tokens || !targets || !params || L < 0 || C <= 0 || NH <= 0 || C % NH ||
        V <= 0 || Vp < V || T <= 0 || T > maxT || B <= 0)
        return 1;
    int64_t N = (int64_t)B * T, c = C;
    /* per layer: x_in, ln1, qkv, att, res1, ln2, fc, gelu  (= 1+1+3+1+1+1+4+4 = 16 C per row) */
    int64_t per_layer = N * c * 16;
    float* acts = (float*)malloc(sizeof(float) * (size_t)(per_layer * L + 3 * N * c));
    float* logits = (float*)malloc(sizeof(float) * (size_t)(N * Vp));
    float* d1 = (float*)malloc(sizeof(float) * (size_t)(N * 4 * c));
    float* d2 = (float*)malloc(sizeof(float) * (size_t)(N * 4 * c));
    float* dres = (float*)malloc(sizeof(float) * (size_t)(N * c));
    float* tmp = (float*)malloc(sizeof(float) * (size_t)(N * c));
    if (!acts || !logits || !d1 || !d2 || !dres || !tmp) {
        free(acts); free(logits); free(d1); free(d2); free(dres); free(tmp);
        return 2;
    }
    memset(grads, 0, sizeof(float) * (size_t)oracle_param_count(L, C, maxT, Vp));
    /* forward, keeping everything */
    layer_params p0 = params_at(params, L, C, maxT, Vp, 0);
    float* x0 = acts + per_layer * L;      /* encoder output */
    float* xf = x0 + N * c;                /* final residual stream */
    float* lnf = xf + N * c;
    oracle_encoder(x0, tokens, p0.wte, p0.wpe, B, T, C);
    const float* xin = x0;
    for (int l = 0; l < L; l++) {
        layer_params p = params_at(params, L, C, maxT, Vp, l);
        float* A = acts + per_layer * l;
        float *x = A, *ln1 = x + N * c, *qkv = ln1 + N * c, *att = qkv + 3 * N * c;
        float *res1 = att + N * c, *ln2 = res1 + N * c, *fc = ln2 + N * c, *ge = fc + 4 * N * c;
        memcpy(x, xin, sizeof(float) * (size_t)(N * c));
        oracle_layernorm(ln1, NULL, NULL, x, p.ln1_g, p.ln1_b, (int)N, C, eps);
        oracle_matmul(qkv, ln1, p.qkv_w, p.qkv_b, (int)N, C, 3 * C);
        oracle_attention(att, qkv, B, T, C, NH);
        oracle_matmul(tmp, att, p.attproj_w, p.attproj_b, (int)N, C, C);
        oracle_residual(res1, x, tmp, N * c);
        oracle_layernorm(ln2, NULL, NULL, res1, p.ln2_g, p.ln2_b, (int)N, C, eps);
        oracle_matmul(fc, ln2, p.fc_w, p.fc_b, (int)N, C, 4 * C);
        oracle_gelu(ge, fc, N * 4 * c);
        oracle_matmul(tmp, ge, p.fcproj_w, p.fcproj_b, (int)N, 4 * C, C);
        float* xo = (l + 1 < L) ? acts + per_layer * (l + 1) : xf;
        oracle_residual(xo, res1, tmp, N * c);
        xin = xo;
    }
    if (L == 0) memcpy(xf, x0, sizeof(float) * (size_t)(N * c));
    oracle_layernorm(lnf, NULL, NULL, xf, p0.lnf_g, p0.lnf_b, (int)N, C, eps);
    oracle_matmul(logits, lnf, p0.wte, NULL, (int)N, C, Vp);
    if (loss) {
        float* ls = (float*)malloc(sizeof(float) * (size_t)N);
        if (ls) {
            oracle_crossentropy(ls, logits, targets, (int)N, V, Vp);
            double s = 0.0;
            for (int64_t n = 0; n < N; n++) s += (double)ls[n];
            *loss = (float)(s / (double)N);
            free(ls);
        }
    }
    /* backward */
    layer_params g0 = params_at(grads, L, C, maxT, Vp, 0);
    float* dwte = (float*)g0.wte;
    float* dwpe = (float*)g0.wpe;
    oracle_crossentropy_backward(logits, logits, targets, 1.0 / (double)N, (int)N, V, Vp);
    oracle_matmul_backward(tmp, dwte, NULL, logits, lnf, p0.wte, (int)N, C, Vp);
    oracle_layernorm_backward(dres, (float*)g0.lnf_g, (float*)g0.lnf_b, tmp, xf, p0.lnf_g, (int)N, C, eps);
    for (int l = L - 1; l >= 0; l--) {
        layer_params p = params_at(params, L, C, maxT, Vp, l);
        layer_params g = params_at(grads, L, C, maxT, Vp, l);
        float* A = acts + per_layer * l;
        float *x = A, *ln1 = x + N * c, *qkv = ln1 + N * c, *att = qkv + 3 * N * c;
        float *res1 = att + N * c, *ln2 = res1 + N * c, *fc = ln2 + N * c, *ge = fc + 4 * N * c;
        /* x_out = res1 + fcproj(gelu(fc(ln2(res1)))) */
        oracle_matmul_backward(d1, (float*)g.fcproj_w, (float*)g.fcproj_b, dres, ge, p.fcproj_w, (int)N, 4 * C, C);
        oracle_gelu_backward(d1, fc, d1, N * 4 * c);
        oracle_matmul_backward(tmp, (float*)g.fc_w, (float*)g.fc_b, d1, ln2, p.fc_w, (int)N, C, 4 * C);
        oracle_layernorm_backward(d2, (float*)g.ln2_g, (float*)g.ln2_b, tmp, res1, p.ln2_g, (int)N, C, eps);
        oracle_residual(dres, dres, d2, N * c);
        /* res1 = x + attproj(attention(qkv(ln1(x)))) */
        oracle_matmul_backward(tmp, (float*)g.attproj_w, (float*)g.attproj_b, dres, att, p.attproj_w, (int)N, C, C);
        oracle_attention_backward(d1, tmp, qkv, B, T, C, NH);
        oracle_matmul_backward(tmp, (float*)g.qkv_w, (float*)g.qkv_b, d1, ln1, p.qkv_w, (int)N, C, 3 * C);
        oracle_layernorm_backward(d2, (float*)g.ln1_g, (float*)g.ln1_b, tmp, x, p.ln1_g, (int)N, C, eps);
        oracle_residual(dres, dres, d2, N * c);
    }
    oracle_encoder_backward(dwte, dwpe, dres, tokens, B, T, C);
    free(acts); free(logits); free(d1); free(d2); free(dres); free(tmp);
    return 0;
}
