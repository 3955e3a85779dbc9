// Training step: a forward that keeps every activation its backward needs,
// the fused classifier (losses and the logit gradient in one pass over the
// logits), and the backward through every layer to the gradient of each
// parameter. The decomposition is that of the llm.c training step ("State of
// the Union [April 22, 2024]": encoder, forward blocks, classifier, backward
// blocks; the optimizer is not part of this library).
//
// Backward, per block in reverse order, with dres the gradient of the
// residual stream after the block:
//   fcproj: dW, db, d(gelu out) = dres . W     gelu: d(fc out) = d(gelu out) g'(fc out)
//   fc:     dW, db, d(ln2 out)                 ln2:  dres += LayerNorm backward
//   attproj: dW, db, d(att out)                attention: d(qkv)
//   qkv:    dW, db, d(ln1 out)                 ln1:  dres += LayerNorm backward
// and finally the embedding: d(wte) += the scatter of dres (d(wte) already
// holds the logits' weight gradient: the embedding is tied), d(wpe).
#include <algorithm>

#include "common.h"
#include "model.h"

namespace gpt2 {

int launch_encoder(void*, const int32_t*, const void*, const void*, int, int, int, int, hipStream_t);
int launch_layernorm(void*, float*, float*, const void*, const void*, const void*, int, int, float, int, hipStream_t);
int launch_matmul(void*, const void*, const void*, const void*, int, int, int, int, hipStream_t);
int launch_matmul_epi(void*, const void*, const void*, const void*, const void*, int, int, int, int, int,
                      hipStream_t);
int launch_matmul_gelu2(void*, void*, const void*, const void*, const void*, int, int, int, int, hipStream_t);
int launch_attention(void*, const void*, int, int, int, int, int, hipStream_t, float*);
int launch_gelu(void*, const void*, int64_t, int, hipStream_t);
int launch_crossentropy_backward(void*, float*, float*, const void*, const int32_t*, float, int, int, int, int,
                                 hipStream_t);
int launch_matmul_backward(void*, void*, void*, const void*, const void*, const void*, int, int, int, int, void*,
                           hipStream_t, const void* gelu_in);
int64_t matmul_backward_workspace_bytes(int N, int C, int OC, int dtype);
int launch_layernorm_backward(void*, void*, void*, const void*, const void*, const void*, const void*, const float*,
                              const float*, int, int, int, void*, hipStream_t);
int64_t layernorm_backward_workspace_bytes(int N, int C);
int launch_attention_backward(void*, const void*, const void*, const void*, const float*, int, int, int, int, int,
                              void*, hipStream_t);
int64_t attention_backward_workspace_bytes(int B, int T, int NH);
bool attention_backward_head_size_ok(int hs);
int launch_encoder_backward(void*, void*, const void*, const int32_t*, int, int, int, int, hipStream_t);
void launch_zero(void*, int64_t, hipStream_t);

// Activations of one block (element type T unless noted).
struct LayerActs {
    char *x, *ln1, *qkv, *att, *res1, *ln2, *fch, *fchg;  // x: the block's input (residual stream)
    float *ln1_mean, *ln1_rstd, *ln2_mean, *ln2_rstd, *lse;  // lse [B,NH,T]
};
// The activation buffer, walked in a fixed order: L blocks, then the final
// residual stream, lnf output and statistics, the logits (replaced by their
// gradient) and the per-row losses.
struct ActsLayout {
    int64_t layer_bytes, xf, lnf, lnf_mean, lnf_rstd, logits, losses, total;
    int64_t o_x, o_ln1, o_qkv, o_att, o_res1, o_ln2, o_fch, o_fchg, o_m1, o_r1, o_m2, o_r2, o_lse;
};

static ActsLayout acts_layout(const gpt2_config& c, int B, int T) {
    const int64_t N = (int64_t)B * T, C = c.C, es = elem_size(c.dtype);
    ActsLayout a;
    int64_t o = 0;
    auto take = [&](int64_t bytes) { int64_t r = o; o += align256(bytes); return r; };
    a.o_x = take(N * C * es);
    a.o_ln1 = take(N * C * es);
    a.o_qkv = take(N * 3 * C * es);
    a.o_att = take(N * C * es);
    a.o_res1 = take(N * C * es);
    a.o_ln2 = take(N * C * es);
    a.o_fch = take(N * 4 * C * es);
    a.o_fchg = take(N * 4 * C * es);
    a.o_m1 = take(N * 4);
    a.o_r1 = take(N * 4);
    a.o_m2 = take(N * 4);
    a.o_r2 = take(N * 4);
    a.o_lse = take(N * c.NH * 4);
    a.layer_bytes = o;
    o = a.layer_bytes * c.L;
    a.xf = take(N * C * es);
    a.lnf = take(N * C * es);
    a.lnf_mean = take(N * 4);
    a.lnf_rstd = take(N * 4);
    a.logits = take(N * c.Vp * es);
    a.losses = take(N * 4);
    a.total = o;
    return a;
}

static LayerActs layer_acts(char* base, const ActsLayout& a, int l) {
    char* p = base + a.layer_bytes * l;
    LayerActs r;
    r.x = p + a.o_x;
    r.ln1 = p + a.o_ln1;
    r.qkv = p + a.o_qkv;
    r.att = p + a.o_att;
    r.res1 = p + a.o_res1;
    r.ln2 = p + a.o_ln2;
    r.fch = p + a.o_fch;
    r.fchg = p + a.o_fchg;
    r.ln1_mean = (float*)(p + a.o_m1);
    r.ln1_rstd = (float*)(p + a.o_r1);
    r.ln2_mean = (float*)(p + a.o_m2);
    r.ln2_rstd = (float*)(p + a.o_r2);
    r.lse = (float*)(p + a.o_lse);
    return r;
}

// Backward scratch: dres [N,C], d4 [N,4C], dC [N,C], dqkv [N,3C], then the
// largest workspace any backward step asks for.
struct TrainWs {
    char *dres, *d4, *dC, *dqkv, *step;
    int64_t step_bytes, total;
};

static TrainWs train_ws(char* base, const gpt2_config& c, int B, int T) {
    const int64_t N = (int64_t)B * T, C = c.C, es = elem_size(c.dtype);
    TrainWs w;
    int64_t o = 0;
    auto take = [&](int64_t bytes) { char* r = base ? base + o : nullptr; o += align256(bytes); return r; };
    w.dres = take(N * C * es);
    w.d4 = take(N * 4 * C * es);
    w.dC = take(N * C * es);
    w.dqkv = take(N * 3 * C * es);
    const int n = (int)N, Ci = (int)C;
    int64_t s = matmul_backward_workspace_bytes(n, Ci, c.Vp, c.dtype);
    const int shapes[4][2] = {{Ci, 3 * Ci}, {Ci, Ci}, {Ci, 4 * Ci}, {4 * Ci, Ci}};
    for (auto& sh : shapes) s = std::max(s, matmul_backward_workspace_bytes(n, sh[0], sh[1], c.dtype));
    s = std::max(s, layernorm_backward_workspace_bytes(n, Ci));
    s = std::max(s, attention_backward_workspace_bytes(B, T, c.NH));
    w.step_bytes = s;
    w.step = take(s);
    w.total = o;
    return w;
}

static bool train_supported(const gpt2_config* c) {
    const int V = c->dtype == GPT2_BF16 ? 8 : 4;
    return config_supported(c) && attention_backward_head_size_ok(c->C / c->NH) && c->C / V <= 8 * 64;
}

}  // namespace gpt2

using namespace gpt2;

#define CHECK(call)                     \
    do {                                \
        int rc_ = (call);               \
        if (rc_ != GPT2_OK) return rc_; \
    } while (0)

extern "C" int64_t gpt2_train_acts_bytes(const gpt2_config* cfg, int B, int T) {
    if (!config_ok(cfg) || B < 0 || T < 0) return -1;
    return acts_layout(*cfg, B, T).total;
}

extern "C" int64_t gpt2_train_workspace_bytes(const gpt2_config* cfg, int B, int T) {
    if (!config_ok(cfg) || B < 0 || T < 0) return -1;
    return train_ws(nullptr, *cfg, B, T).total;
}

extern "C" int gpt2_train_forward(float* losses, float* mean_loss, const int32_t* tokens, const int32_t* targets,
                                  const void* params, const gpt2_config* cfg, int B, int T, void* acts,
                                  int64_t acts_bytes, void* stream) {
    if (!config_ok(cfg) || B < 0 || T < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!tokens || !targets || !params || !acts || T > cfg->maxT) return GPT2_ERR_INVALID_ARGUMENT;
    if (!train_supported(cfg) || !aligned16(params) || !aligned16(acts)) return GPT2_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)B * T;
    if (N > INT32_MAX / 4) return GPT2_ERR_UNSUPPORTED;
    const ActsLayout al = acts_layout(*cfg, B, T);
    if (acts_bytes < al.total) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    const ParamOffsets po = param_offsets(*cfg);
    const int C = cfg->C, L = cfg->L, dt = cfg->dtype, es = elem_size(dt), n = (int)N;
    const int64_t C64 = C;
    const char* P = (const char*)params;
    auto at = [&](int64_t off) { return (const void*)(P + off * es); };
    char* A = (char*)acts;
    hipStream_t s = (hipStream_t)stream;

    CHECK(launch_encoder(layer_acts(A, al, 0).x, tokens, at(po.wte), at(po.wpe), B, T, C, dt, s));
    for (int l = 0; l < L; l++) {
        const LayerActs a = layer_acts(A, al, l);
        char* xnext = l + 1 < L ? layer_acts(A, al, l + 1).x : A + al.xf;
        CHECK(launch_layernorm(a.ln1, a.ln1_mean, a.ln1_rstd, a.x, at(po.ln1_g + l * C64), at(po.ln1_b + l * C64), n,
                               C, cfg->ln_eps, dt, s));
        CHECK(launch_matmul(a.qkv, a.ln1, at(po.qkv_w + l * 3 * C64 * C64), at(po.qkv_b + l * 3 * C64), n, C, 3 * C,
                            dt, s));
        CHECK(launch_attention(a.att, a.qkv, B, T, C, cfg->NH, dt, s, a.lse));
        CHECK(launch_matmul_epi(a.res1, a.att, at(po.ap_w + l * C64 * C64), at(po.ap_b + l * C64), a.x, n, C, C,
                                EPI_BIAS_RESIDUAL, dt, s));
        CHECK(launch_layernorm(a.ln2, a.ln2_mean, a.ln2_rstd, a.res1, at(po.ln2_g + l * C64), at(po.ln2_b + l * C64),
                               n, C, cfg->ln_eps, dt, s));
        // the pre-activation is kept for GELU's backward, the activation for
        // fcproj's: both from the product's epilogue where its tile allows
        const int rg = launch_matmul_gelu2(a.fch, a.fchg, a.ln2, at(po.fc_w + l * 4 * C64 * C64),
                                           at(po.fc_b + l * 4 * C64), n, C, 4 * C, dt, s);
        if (rg == GPT2_ERR_UNSUPPORTED) {
            CHECK(launch_matmul(a.fch, a.ln2, at(po.fc_w + l * 4 * C64 * C64), at(po.fc_b + l * 4 * C64), n, C,
                                4 * C, dt, s));
            CHECK(launch_gelu(a.fchg, a.fch, N * 4 * C64, dt, s));
        } else {
            CHECK(rg);
        }
        CHECK(launch_matmul_epi(xnext, a.fchg, at(po.fp_w + l * 4 * C64 * C64), at(po.fp_b + l * C64), a.res1, n,
                                4 * C, C, EPI_BIAS_RESIDUAL, dt, s));
    }
    CHECK(launch_layernorm(A + al.lnf, (float*)(A + al.lnf_mean), (float*)(A + al.lnf_rstd), A + al.xf, at(po.lnf_g),
                           at(po.lnf_b), n, C, cfg->ln_eps, dt, s));
    CHECK(launch_matmul(A + al.logits, A + al.lnf, at(po.wte), nullptr, n, C, cfg->Vp, dt, s));
    // losses, their mean, and d(mean loss)/d(logits) over the logits in place
    float* ls = losses ? losses : (float*)(A + al.losses);
    return launch_crossentropy_backward(A + al.logits, ls, mean_loss, A + al.logits, targets, 1.0f / (float)N, n,
                                        cfg->V, cfg->Vp, dt, s);
}

extern "C" int gpt2_backward(void* grads, const int32_t* tokens, const void* params, const gpt2_config* cfg, int B,
                             int T, void* acts, int64_t acts_bytes, void* workspace, int64_t workspace_bytes,
                             void* stream) {
    if (!config_ok(cfg) || B < 0 || T < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!grads || !tokens || !params || !acts || !workspace || T > cfg->maxT) return GPT2_ERR_INVALID_ARGUMENT;
    if (!train_supported(cfg) || !aligned16(grads) || !aligned16(params) || !aligned16(acts) ||
        !aligned16(workspace))
        return GPT2_ERR_UNSUPPORTED;
    if (grads == params) return GPT2_ERR_INVALID_ARGUMENT;
    const int64_t N = (int64_t)B * T;
    if (N > INT32_MAX / 4) return GPT2_ERR_UNSUPPORTED;
    const ActsLayout al = acts_layout(*cfg, B, T);
    if (acts_bytes < al.total) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    const TrainWs w = train_ws((char*)workspace, *cfg, B, T);
    if (workspace_bytes < w.total) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    const ParamOffsets po = param_offsets(*cfg);
    const int C = cfg->C, L = cfg->L, dt = cfg->dtype, es = elem_size(dt), n = (int)N;
    const int64_t C64 = C;
    const char* P = (const char*)params;
    char* G = (char*)grads;
    auto at = [&](int64_t off) { return (const void*)(P + off * es); };
    auto gat = [&](int64_t off) { return (void*)(G + off * es); };
    char* A = (char*)acts;
    hipStream_t s = (hipStream_t)stream;

    // only d(wpe) rows < T receive anything
    launch_zero(gat(po.wpe), (int64_t)cfg->maxT * C * es, s);
    // classifier: d(lnf out) and the logits' part of d(wte)
    CHECK(launch_matmul_backward(w.dC, gat(po.wte), nullptr, A + al.logits, A + al.lnf, at(po.wte), n, C, cfg->Vp, dt,
                                 w.step, s, nullptr));
    CHECK(launch_layernorm_backward(w.dres, gat(po.lnf_g), gat(po.lnf_b), nullptr, w.dC, A + al.xf, at(po.lnf_g),
                                    (const float*)(A + al.lnf_mean), (const float*)(A + al.lnf_rstd), n, C, dt, w.step,
                                    s));
    for (int l = L - 1; l >= 0; l--) {
        const LayerActs a = layer_acts(A, al, l);
        // d(fc pre-activation) straight from the product: the GELU backward
        // is the input gradient's epilogue
        CHECK(launch_matmul_backward(w.d4, gat(po.fp_w + l * 4 * C64 * C64), gat(po.fp_b + l * C64), w.dres, a.fchg,
                                     at(po.fp_w + l * 4 * C64 * C64), n, 4 * C, C, dt, w.step, s, a.fch));
        CHECK(launch_matmul_backward(w.dC, gat(po.fc_w + l * 4 * C64 * C64), gat(po.fc_b + l * 4 * C64), w.d4, a.ln2,
                                     at(po.fc_w + l * 4 * C64 * C64), n, C, 4 * C, dt, w.step, s, nullptr));
        CHECK(launch_layernorm_backward(w.dres, gat(po.ln2_g + l * C64), gat(po.ln2_b + l * C64), w.dres, w.dC, a.res1,
                                        at(po.ln2_g + l * C64), a.ln2_mean, a.ln2_rstd, n, C, dt, w.step, s));
        CHECK(launch_matmul_backward(w.dC, gat(po.ap_w + l * C64 * C64), gat(po.ap_b + l * C64), w.dres, a.att,
                                     at(po.ap_w + l * C64 * C64), n, C, C, dt, w.step, s, nullptr));
        CHECK(launch_attention_backward(w.dqkv, w.dC, a.qkv, a.att, a.lse, B, T, C, cfg->NH, dt, w.step, s));
        CHECK(launch_matmul_backward(w.dC, gat(po.qkv_w + l * 3 * C64 * C64), gat(po.qkv_b + l * 3 * C64), w.dqkv,
                                     a.ln1, at(po.qkv_w + l * 3 * C64 * C64), n, C, 3 * C, dt, w.step, s, nullptr));
        CHECK(launch_layernorm_backward(w.dres, gat(po.ln1_g + l * C64), gat(po.ln1_b + l * C64), w.dres, w.dC, a.x,
                                        at(po.ln1_g + l * C64), a.ln1_mean, a.ln1_rstd, n, C, dt, w.step, s));
    }
    return launch_encoder_backward(gat(po.wte), gat(po.wpe), w.dres, tokens, B, T, C, dt, s);
}
