// Model-level helpers shared by the forward/decode entries and the training
// entries: the flat parameter layout and the configuration checks.
#pragma once
#include "common.h"

namespace gpt2 {

bool attention_head_size_ok(int hs);

// Element offsets into the flat parameter buffer.
struct ParamOffsets {
    int64_t wte, wpe, ln1_g, ln1_b, qkv_w, qkv_b, ap_w, ap_b, ln2_g, ln2_b, fc_w, fc_b, fp_w, fp_b,
        lnf_g, lnf_b, total;
};

inline ParamOffsets param_offsets(const gpt2_config& c) {
    const int64_t C = c.C, L = c.L;
    ParamOffsets o;
    int64_t p = 0;
    o.wte = p;   p += (int64_t)c.Vp * C;
    o.wpe = p;   p += (int64_t)c.maxT * C;
    o.ln1_g = p; p += L * C;
    o.ln1_b = p; p += L * C;
    o.qkv_w = p; p += L * 3 * C * C;
    o.qkv_b = p; p += L * 3 * C;
    o.ap_w = p;  p += L * C * C;
    o.ap_b = p;  p += L * C;
    o.ln2_g = p; p += L * C;
    o.ln2_b = p; p += L * C;
    o.fc_w = p;  p += L * 4 * C * C;
    o.fc_b = p;  p += L * 4 * C;
    o.fp_w = p;  p += L * 4 * C * C;
    o.fp_b = p;  p += L * C;
    o.lnf_g = p; p += C;
    o.lnf_b = p; p += C;
    o.total = p;
    return o;
}

inline bool config_ok(const gpt2_config* c) {
    return c && c->L >= 1 && c->C > 0 && c->NH > 0 && c->C % c->NH == 0 && c->V > 0 &&
           c->Vp >= c->V && c->maxT > 0 && valid_dtype(c->dtype) && c->ln_eps >= 0.f;
}
inline bool config_supported(const gpt2_config* c) {
    return c->C % 8 == 0 && c->C <= 4096 && c->Vp % 8 == 0 && c->Vp <= 131072 &&
           attention_head_size_ok(c->C / c->NH);
}

inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

}  // namespace gpt2
