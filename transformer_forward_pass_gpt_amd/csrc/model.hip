// The whole forward pass and the KV-cache decode step, composed from the
// per-step launchers on one stream, plus the status plumbing of the C ABI.
//
// Block order (GPT-2, pre-LayerNorm):
//   x <- x + attproj(attention(ln1(x)))
//   x <- x + fcproj(gelu(fc(ln2(x))))
// then lnf, logits against the tied token embedding, vocabulary softmax.
// The steps are those of ECE408 Final Project - GPT-2, Milestone 1 (kernel
// table); llm.c "State of the Union [April 22, 2024]" (step breakdown) splits
// the same pass into encoder, forward blocks and classifier. GELU and the two
// residual adds run in the epilogues of the fc, attproj and fcproj GEMMs
// (the kernel-fusion item of the llm.c "big stones" list), bit-identical to
// the separate kernels: 7L + 4 launches.
#include <mutex>

#include "common.h"
#include "model.h"

namespace gpt2 {

static thread_local int g_last_hip_error = 0;
void set_last_hip_error(int e) { g_last_hip_error = e; }
int launch_status() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return GPT2_ERR_HIP;
    }
    return GPT2_OK;
}

int launch_encoder(void*, const int32_t*, const void*, const void*, int, int, int, int, hipStream_t);
int launch_layernorm(void*, float*, float*, const void*, const void*, const void*, int, int, float,
                     int, hipStream_t);
int launch_softmax(void*, const void*, int, int, int, int, hipStream_t);
int launch_matmul(void*, const void*, const void*, const void*, int, int, int, int, hipStream_t);
int launch_matmul_epi(void*, const void*, const void*, const void*, const void*, int, int, int, int, int,
                      hipStream_t);
int launch_attention(void*, const void*, int, int, int, int, int, hipStream_t, float*);
int launch_attention_decode(void*, const void*, void*, void*, int, int, int, int, int, int, float*,
                            hipStream_t, int* nsplit_out);
int decode_attention_splits(int pos, int hs, int dtype);
int64_t decode_workspace_bytes(int B, int C, int NH, int maxT);
bool attention_head_size_ok(int hs);
int launch_skinny_gemm(void*, float*, const void*, const void*, const void*, int, int, int, int, int, int,
                       hipStream_t);
int launch_skinny_gemm_acomb(float* part, const float* apart, int asplits, int hs, const void* weight, int M, int K,
                             int N, int splits, int dtype, hipStream_t s);
int skinny_acomb_max_splits();
int launch_kv_store(void*, void*, const void*, int, int, int, int, int, int, hipStream_t);
int launch_argmax(int32_t*, int32_t*, int, const void*, int, int, int, int, hipStream_t);
int launch_layernorm_rows(void*, const void*, int64_t, const void*, const void*, int, int, float, int, hipStream_t);
int launch_residual_layernorm(void*, void*, const float*, int, const void*, const void*, const void*, int, int,
                              float, int, hipStream_t);

int skinny_split_count(int K, int N, int es);

// Decode steps on at most kSkinnyRows sequences run the projections as skinny
// GEMMs; attproj and fcproj split k over up to kMaxSplits workgroups per
// column tile and leave fp32 partial sums for the fused residual+LayerNorm.
static constexpr int kSkinnyRows = 32;
static constexpr int kMaxSplits = 8;

// fp32 partials of the decode step: the attention's key chunks, and (skinny
// path) the split-k projections. They are separate: the attproj product
// reads the first while it writes the second.
static int64_t decode_apart_bytes(int B, int C, int NH, int maxT) { return decode_workspace_bytes(B, C, NH, maxT); }
static int64_t decode_part_bytes(int B, int C) { return B <= kSkinnyRows ? (int64_t)kMaxSplits * B * C * 4 : 0; }

// Workspace: residual stream x [N,C], LayerNorm output [N,C], qkv [N,3C],
// attention output [N,C], MLP hidden [N,4C], the attention's partials and
// the projections' partials.
struct Workspace {
    char *x, *ln, *qkv, *att, *fc;
    float *apart, *part;
    int64_t bytes;
};
static Workspace carve(char* base, int64_t N, int64_t C, int es, int64_t apart_bytes, int64_t part_bytes) {
    Workspace w;
    int64_t o = 0;
    auto take = [&](int64_t n) { char* p = base ? base + o : nullptr; o += align256(n); return p; };
    w.x = take(N * C * es);
    w.ln = take(N * C * es);
    w.qkv = take(N * 3 * C * es);
    w.att = take(N * C * es);
    w.fc = take(N * 4 * C * es);
    w.apart = (float*)take(apart_bytes);
    w.part = (float*)take(part_bytes);
    w.bytes = o;
    return w;
}
static Workspace decode_carve(char* base, int B, int C, int NH, int maxT, int es) {
    return carve(base, B, C, es, decode_apart_bytes(B, C, NH, maxT), decode_part_bytes(B, C));
}

}  // namespace gpt2

using namespace gpt2;

#define CHECK(call)                       \
    do {                                  \
        int rc_ = (call);                 \
        if (rc_ != GPT2_OK) return rc_;   \
    } while (0)

extern "C" const char* gpt2_status_string(int status) {
    switch (status) {
        case GPT2_OK: return "ok";
        case GPT2_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GPT2_ERR_UNSUPPORTED: return "unsupported shape, head size, width or alignment";
        case GPT2_ERR_HIP: return "HIP launch error (see gpt2_last_hip_error)";
        case GPT2_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        default: return "unknown status";
    }
}

extern "C" int gpt2_last_hip_error(void) { return g_last_hip_error; }

extern "C" int64_t gpt2_param_count(const gpt2_config* cfg) {
    if (!config_ok(cfg)) return -1;
    return param_offsets(*cfg).total;
}

extern "C" int64_t gpt2_workspace_bytes(const gpt2_config* cfg, int B, int T) {
    if (!config_ok(cfg) || B < 0 || T < 0) return -1;
    return carve(nullptr, (int64_t)B * T, cfg->C, elem_size(cfg->dtype), 0, 0).bytes;
}

// Embedding and the L blocks over B x T tokens; the residual stream ends in
// w.x. With kcache/vcache ([L,B,NH,kv_maxT,hs]) the keys and values of every
// layer are also stored at positions 0..T-1 (prefill).
static int run_blocks(const Workspace& w, const int32_t* tokens, const char* P, const ParamOffsets& po,
                      const gpt2_config& cf, int B, int T, void* kcache, void* vcache, int kv_maxT, hipStream_t s) {
    const gpt2_config* cfg = &cf;
    const int C = cfg->C, L = cfg->L, dt = cfg->dtype, es = elem_size(dt);
    auto at = [&](int64_t off) { return (const void*)(P + off * es); };
    const int n = B * T;
    const int64_t C64 = C;
    const int64_t layer_elems = (int64_t)B * cfg->NH * kv_maxT * (C / cfg->NH);
    CHECK(launch_encoder(w.x, tokens, at(po.wte), at(po.wpe), B, T, C, dt, s));
    for (int l = 0; l < L; l++) {
        CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.ln1_g + l * C64),
                               at(po.ln1_b + l * C64), n, C, cfg->ln_eps, dt, s));
        CHECK(launch_matmul(w.qkv, w.ln, at(po.qkv_w + l * 3 * C64 * C64), at(po.qkv_b + l * 3 * C64),
                            n, C, 3 * C, dt, s));
        if (kcache)
            CHECK(launch_kv_store((char*)kcache + l * layer_elems * es, (char*)vcache + l * layer_elems * es, w.qkv,
                                  B, T, C, cfg->NH, kv_maxT, dt, s));
        CHECK(launch_attention(w.att, w.qkv, B, T, C, cfg->NH, dt, s, nullptr));
        // x += attproj(att), the residual add in the GEMM epilogue
        CHECK(launch_matmul_epi(w.x, w.att, at(po.ap_w + l * C64 * C64), at(po.ap_b + l * C64), w.x, n, C, C,
                                EPI_BIAS_RESIDUAL, dt, s));
        CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.ln2_g + l * C64),
                               at(po.ln2_b + l * C64), n, C, cfg->ln_eps, dt, s));
        // fc = gelu(fc(ln)), GELU in the GEMM epilogue
        CHECK(launch_matmul_epi(w.fc, w.ln, at(po.fc_w + l * 4 * C64 * C64), at(po.fc_b + l * 4 * C64), nullptr,
                                n, C, 4 * C, EPI_BIAS_GELU, dt, s));
        // x += fcproj(fc)
        CHECK(launch_matmul_epi(w.x, w.fc, at(po.fp_w + l * 4 * C64 * C64), at(po.fp_b + l * C64), w.x, n,
                                4 * C, C, EPI_BIAS_RESIDUAL, dt, s));
    }
    return GPT2_OK;
}

extern "C" int gpt2_forward(void* logits, void* probs, const int32_t* tokens, const void* params,
                            const gpt2_config* cfg, int B, int T, void* workspace,
                            int64_t workspace_bytes, void* stream) {
    if (!config_ok(cfg) || B < 0 || T < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!logits || !tokens || !params || !workspace || T > cfg->maxT) return GPT2_ERR_INVALID_ARGUMENT;
    if (!config_supported(cfg) || !aligned16(logits) || !aligned16(params) ||
        !aligned16(workspace) || (probs && !aligned16(probs)))
        return GPT2_ERR_UNSUPPORTED;
    if (probs == logits) return GPT2_ERR_INVALID_ARGUMENT;
    const int64_t N = (int64_t)B * T;
    const int C = cfg->C, L = cfg->L, dt = cfg->dtype, es = elem_size(dt);
    if (N > INT32_MAX / 4) return GPT2_ERR_UNSUPPORTED;
    Workspace w = carve((char*)workspace, N, C, es, 0, 0);
    if (workspace_bytes < w.bytes) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    const ParamOffsets po = param_offsets(*cfg);
    const char* P = (const char*)params;
    auto at = [&](int64_t off) { return (const void*)(P + off * es); };
    hipStream_t s = (hipStream_t)stream;
    const int n = (int)N;

    CHECK(run_blocks(w, tokens, P, po, *cfg, B, T, nullptr, nullptr, 0, s));
    CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.lnf_g), at(po.lnf_b), n, C,
                           cfg->ln_eps, dt, s));
    // The vocabulary softmax holds each row in registers, so it reads the
    // logits once and writes the probabilities once. The variant with row
    // statistics from the GEMM epilogue (matmul_logits_stats_forward) was
    // measured slower: its exponentials run on the vector units while the
    // matrix cores idle.
    CHECK(launch_matmul(logits, w.ln, at(po.wte), nullptr, n, C, cfg->Vp, dt, s));
    if (probs) CHECK(launch_softmax(probs, logits, n, cfg->V, cfg->Vp, dt, s));
    return GPT2_OK;
}

extern "C" int64_t gpt2_decode_workspace_bytes(const gpt2_config* cfg, int B) {
    if (!config_ok(cfg) || B < 0) return -1;
    return decode_carve(nullptr, B, cfg->C, cfg->NH, cfg->maxT, elem_size(cfg->dtype))
        .bytes;
}

// One decode step for B sequences at position pos (arguments validated).
static int decode_step_impl(void* logits, void* probs, const int32_t* tokens, int pos, void* kcache, void* vcache,
                            const void* params, const gpt2_config* cfg, int B, const Workspace& w, hipStream_t s) {
    const int C = cfg->C, L = cfg->L, NH = cfg->NH, dt = cfg->dtype, es = elem_size(dt);
    const ParamOffsets po = param_offsets(*cfg);
    const char* P = (const char*)params;
    auto at = [&](int64_t off) { return (const void*)(P + off * es); };
    const int64_t C64 = C;
    const int64_t layer_elems = (int64_t)B * NH * cfg->maxT * (C / NH);

    CHECK(launch_encoder(w.x, tokens, at(po.wte), at(po.wpe + (int64_t)pos * C64), B, 1, C, dt, s));
    if (B <= kSkinnyRows && C % 8 == 0) {
        // Skinny path: per layer qkv, attention (2 launches), attproj, residual+ln2,
        // fc+GELU, fcproj, residual+ln1 of the next layer (or lnf).
        const int s_ap = skinny_split_count(C, C, es), s_fp = skinny_split_count(4 * C, C, es);
        CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.ln1_g), at(po.ln1_b), B, C, cfg->ln_eps,
                               dt, s));
        for (int l = 0; l < L; l++) {
            CHECK(launch_skinny_gemm(w.qkv, nullptr, w.ln, at(po.qkv_w + l * 3 * C64 * C64),
                                     at(po.qkv_b + l * 3 * C64), B, C, 3 * C, 1, EPI_BIAS, dt, s));
            // an attention split in two (or up to the merge's limit) leaves
            // its partials to the attproj product, which merges them as it
            // loads its A operand (no combine launch)
            int nsp = 1;
            const bool defer = decode_attention_splits(pos, C / NH, dt) <= skinny_acomb_max_splits();
            CHECK(launch_attention_decode(w.att, w.qkv, (char*)kcache + l * layer_elems * es,
                                          (char*)vcache + l * layer_elems * es, B, pos, cfg->maxT, C, NH,
                                          dt, w.apart, s, defer ? &nsp : nullptr));
            if (nsp > 1)
                CHECK(launch_skinny_gemm_acomb(w.part, w.apart, nsp, C / NH, at(po.ap_w + l * C64 * C64), B, C, C,
                                               s_ap, dt, s));
            else
                CHECK(launch_skinny_gemm(nullptr, w.part, w.att, at(po.ap_w + l * C64 * C64), nullptr, B, C, C,
                                         s_ap, EPI_BIAS, dt, s));
            CHECK(launch_residual_layernorm(w.ln, w.x, w.part, s_ap, at(po.ap_b + l * C64),
                                            at(po.ln2_g + l * C64), at(po.ln2_b + l * C64), B, C,
                                            cfg->ln_eps, dt, s));
            CHECK(launch_skinny_gemm(w.fc, nullptr, w.ln, at(po.fc_w + l * 4 * C64 * C64),
                                     at(po.fc_b + l * 4 * C64), B, C, 4 * C, 1, EPI_BIAS_GELU, dt, s));
            CHECK(launch_skinny_gemm(nullptr, w.part, w.fc, at(po.fp_w + l * 4 * C64 * C64), nullptr, B,
                                     4 * C, C, s_fp, EPI_BIAS, dt, s));
            const bool last = l == L - 1;
            CHECK(launch_residual_layernorm(w.ln, w.x, w.part, s_fp, at(po.fp_b + l * C64),
                                            at(last ? po.lnf_g : po.ln1_g + (l + 1) * C64),
                                            at(last ? po.lnf_b : po.ln1_b + (l + 1) * C64), B, C,
                                            cfg->ln_eps, dt, s));
        }
        CHECK(launch_matmul(logits, w.ln, at(po.wte), nullptr, B, C, cfg->Vp, dt, s));
        if (probs) CHECK(launch_softmax(probs, logits, B, cfg->V, cfg->Vp, dt, s));
        return GPT2_OK;
    }
    for (int l = 0; l < L; l++) {
        CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.ln1_g + l * C64),
                               at(po.ln1_b + l * C64), B, C, cfg->ln_eps, dt, s));
        CHECK(launch_matmul(w.qkv, w.ln, at(po.qkv_w + l * 3 * C64 * C64), at(po.qkv_b + l * 3 * C64),
                            B, C, 3 * C, dt, s));
        CHECK(launch_attention_decode(w.att, w.qkv, (char*)kcache + l * layer_elems * es,
                                      (char*)vcache + l * layer_elems * es, B, pos, cfg->maxT, C, NH,
                                      dt, w.apart, s, nullptr));
        CHECK(launch_matmul_epi(w.x, w.att, at(po.ap_w + l * C64 * C64), at(po.ap_b + l * C64), w.x, B, C, C,
                                EPI_BIAS_RESIDUAL, dt, s));
        CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.ln2_g + l * C64),
                               at(po.ln2_b + l * C64), B, C, cfg->ln_eps, dt, s));
        CHECK(launch_matmul_epi(w.fc, w.ln, at(po.fc_w + l * 4 * C64 * C64), at(po.fc_b + l * 4 * C64), nullptr,
                                B, C, 4 * C, EPI_BIAS_GELU, dt, s));
        CHECK(launch_matmul_epi(w.x, w.fc, at(po.fp_w + l * 4 * C64 * C64), at(po.fp_b + l * C64), w.x, B,
                                4 * C, C, EPI_BIAS_RESIDUAL, dt, s));
    }
    CHECK(launch_layernorm(w.ln, nullptr, nullptr, w.x, at(po.lnf_g), at(po.lnf_b), B, C,
                           cfg->ln_eps, dt, s));
    CHECK(launch_matmul(logits, w.ln, at(po.wte), nullptr, B, C, cfg->Vp, dt, s));
    if (probs) CHECK(launch_softmax(probs, logits, B, cfg->V, cfg->Vp, dt, s));
    return GPT2_OK;
}

extern "C" int gpt2_decode_step(void* logits, void* probs, const int32_t* tokens, int pos,
                                void* kcache, void* vcache, const void* params,
                                const gpt2_config* cfg, int B, void* workspace,
                                int64_t workspace_bytes, void* stream) {
    if (!config_ok(cfg) || B < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (B == 0) return GPT2_OK;
    if (!logits || !tokens || !params || !kcache || !vcache || !workspace || pos < 0 ||
        pos >= cfg->maxT)
        return GPT2_ERR_INVALID_ARGUMENT;
    if (!config_supported(cfg) || !aligned16(logits) || !aligned16(params) || !aligned16(kcache) ||
        !aligned16(vcache) || !aligned16(workspace) || (probs && !aligned16(probs)))
        return GPT2_ERR_UNSUPPORTED;
    if (probs == logits) return GPT2_ERR_INVALID_ARGUMENT;
    const int C = cfg->C, NH = cfg->NH, es = elem_size(cfg->dtype);
    Workspace w = decode_carve((char*)workspace, B, C, NH, cfg->maxT, es);
    if (workspace_bytes < w.bytes) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    return decode_step_impl(logits, probs, tokens, pos, kcache, vcache, params, cfg, B, w, (hipStream_t)stream);
}

// ------------------------------------------------------------ decode without allocation
// The decode step's workspace (residual stream, LayerNorm output, qkv,
// attention output, MLP hidden and the fp32 partials of the attention chunks
// and the split-k projections) in a file-scope device array instead of a
// caller buffer. Every GPU the library runs on holds its own copy until the
// process ends. Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[GPT2_DECODE_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (resolved on the first call
// made with the device current), or nullptr with the HIP error recorded.
static void* scratch_address() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        set_last_hip_error(e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            set_last_hip_error(e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol);
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

extern "C" int gpt2_decode_step_noalloc(void* logits, void* probs, const int32_t* tokens, int pos,
                                        void* kcache, void* vcache, const void* params,
                                        const gpt2_config* cfg, int B, void* stream) {
    if (!config_ok(cfg) || B < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (B == 0) return GPT2_OK;
    if (!logits || !tokens || !params || !kcache || !vcache || pos < 0 || pos >= cfg->maxT)
        return GPT2_ERR_INVALID_ARGUMENT;
    if (!config_supported(cfg) || !aligned16(logits) || !aligned16(params) || !aligned16(kcache) ||
        !aligned16(vcache) || (probs && !aligned16(probs)))
        return GPT2_ERR_UNSUPPORTED;
    if (probs == logits) return GPT2_ERR_INVALID_ARGUMENT;
    const int C = cfg->C, NH = cfg->NH, es = elem_size(cfg->dtype);
    const int64_t need = decode_carve(nullptr, B, C, NH, cfg->maxT, es).bytes;
    if (need > (int64_t)GPT2_DECODE_SCRATCH_BYTES) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    void* base = scratch_address();
    if (!base) return GPT2_ERR_HIP;
    // Nothing in the carve has to start at zero: every kernel of the step
    // writes each scratch element before any kernel reads it.
    const Workspace w = decode_carve((char*)base, B, C, NH, cfg->maxT, es);
    return decode_step_impl(logits, probs, tokens, pos, kcache, vcache, params, cfg, B, w, (hipStream_t)stream);
}

// ------------------------------------------------------------ generation
// Prefill: the blocks over the prompt, storing every layer's keys and values
// in the caches, then the logits (and probabilities) of the last position of
// each sequence only.
static int prefill_impl(void* logits, void* probs, const int32_t* tokens, void* kcache, void* vcache,
                        const char* P, const gpt2_config* cfg, int B, int T, const Workspace& w, hipStream_t s) {
    const int C = cfg->C, dt = cfg->dtype, es = elem_size(dt);
    const ParamOffsets po = param_offsets(*cfg);
    auto at = [&](int64_t off) { return (const void*)(P + off * es); };
    CHECK(run_blocks(w, tokens, P, po, *cfg, B, T, kcache, vcache, cfg->maxT, s));
    CHECK(launch_layernorm_rows(w.ln, w.x + (int64_t)(T - 1) * C * es, (int64_t)T * C, at(po.lnf_g), at(po.lnf_b),
                                B, C, cfg->ln_eps, dt, s));
    CHECK(launch_matmul(logits, w.ln, at(po.wte), nullptr, B, C, cfg->Vp, dt, s));
    if (probs) CHECK(launch_softmax(probs, logits, B, cfg->V, cfg->Vp, dt, s));
    return GPT2_OK;
}

static bool prefill_args_ok(const gpt2_config* cfg, int B, int T) {
    return config_ok(cfg) && B >= 0 && T >= 1 && T <= cfg->maxT && (int64_t)B * T <= INT32_MAX / 4;
}

extern "C" int gpt2_prefill(void* logits, void* probs, const int32_t* tokens, void* kcache, void* vcache,
                            const void* params, const gpt2_config* cfg, int B, int T, void* workspace,
                            int64_t workspace_bytes, void* stream) {
    if (!prefill_args_ok(cfg, B, T)) return GPT2_ERR_INVALID_ARGUMENT;
    if (B == 0) return GPT2_OK;
    if (!logits || !tokens || !kcache || !vcache || !params || !workspace || probs == logits)
        return GPT2_ERR_INVALID_ARGUMENT;
    if (!config_supported(cfg) || !aligned16(logits) || !aligned16(params) || !aligned16(kcache) ||
        !aligned16(vcache) || !aligned16(workspace) || (probs && !aligned16(probs)))
        return GPT2_ERR_UNSUPPORTED;
    const Workspace w = carve((char*)workspace, (int64_t)B * T, cfg->C, elem_size(cfg->dtype), 0, 0);
    if (workspace_bytes < w.bytes) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    return prefill_impl(logits, probs, tokens, kcache, vcache, (const char*)params, cfg, B, T, w,
                        (hipStream_t)stream);
}

// Generation workspace: the larger of the prefill and decode carves (they are
// used one after the other), then the last logits [B,Vp] and the token ids [B].
struct GenLayout {
    int64_t logits_off, tok_off, bytes;
};
static GenLayout gen_layout(const gpt2_config* cfg, int B, int T) {
    const int C = cfg->C, es = elem_size(cfg->dtype);
    const int64_t pre = carve(nullptr, (int64_t)B * T, C, es, 0, 0).bytes;
    const int64_t dec = decode_carve(nullptr, B, C, cfg->NH, cfg->maxT, es).bytes;
    GenLayout g;
    g.logits_off = align256(pre > dec ? pre : dec);
    g.tok_off = g.logits_off + align256((int64_t)B * cfg->Vp * es);
    g.bytes = g.tok_off + align256((int64_t)B * 4);
    return g;
}

extern "C" int64_t gpt2_generate_workspace_bytes(const gpt2_config* cfg, int B, int T) {
    if (!prefill_args_ok(cfg, B, T)) return -1;
    return gen_layout(cfg, B, T).bytes;
}

extern "C" int gpt2_generate(int32_t* out_tokens, const int32_t* prompt, int n_new, void* kcache, void* vcache,
                             const void* params, const gpt2_config* cfg, int B, int T, void* workspace,
                             int64_t workspace_bytes, void* stream) {
    if (!prefill_args_ok(cfg, B, T) || n_new < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (B == 0 || n_new == 0) return GPT2_OK;
    // token i > 0 comes from the decode step at position T + i - 1 < maxT
    if ((int64_t)T + n_new - 1 > cfg->maxT) return GPT2_ERR_INVALID_ARGUMENT;
    if (!out_tokens || !prompt || !kcache || !vcache || !params || !workspace) return GPT2_ERR_INVALID_ARGUMENT;
    if (!config_supported(cfg) || !aligned16(params) || !aligned16(kcache) || !aligned16(vcache) ||
        !aligned16(workspace))
        return GPT2_ERR_UNSUPPORTED;
    const GenLayout g = gen_layout(cfg, B, T);
    if (workspace_bytes < g.bytes) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    char* base = (char*)workspace;
    const int C = cfg->C, es = elem_size(cfg->dtype);
    const Workspace wp = carve(base, (int64_t)B * T, C, es, 0, 0);
    const Workspace wd = decode_carve(base, B, C, cfg->NH, cfg->maxT, es);
    void* logits = base + g.logits_off;
    int32_t* tok = (int32_t*)(base + g.tok_off);
    hipStream_t s = (hipStream_t)stream;
    CHECK(prefill_impl(logits, nullptr, prompt, kcache, vcache, (const char*)params, cfg, B, T, wp, s));
    CHECK(launch_argmax(tok, out_tokens, n_new, logits, B, cfg->V, cfg->Vp, cfg->dtype, s));
    for (int i = 1; i < n_new; i++) {
        CHECK(decode_step_impl(logits, nullptr, tok, T + i - 1, kcache, vcache, params, cfg, B, wd, s));
        CHECK(launch_argmax(tok, out_tokens + i, n_new, logits, B, cfg->V, cfg->Vp, cfg->dtype, s));
    }
    return GPT2_OK;
}
