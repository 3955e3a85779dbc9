// HBM-streaming kernels: token+position embedding, residual add, tanh-GELU.
// Each thread moves 16-byte vectors in a grid-stride loop, so every wavefront
// issues fully coalesced 1 KiB requests; arithmetic is fp32 and bf16 results
// are rounded to nearest even.
#include "common.h"

namespace gpt2 {

static constexpr int kThreads = 256;

static unsigned stream_grid(int64_t nvec) {
    // 256 CUs x 8 resident workgroups keeps enough requests in flight; the
    // grid-stride loop covers the rest.
    int64_t g = (nvec + kThreads - 1) / kThreads;
    if (g > 2048) g = 2048;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// out[b,t,:] = wte[tokens[b,t],:] + wpe[t,:]
// (ECE408 Final Project - GPT-2, Milestone 1, kernel table: Encoder.)
// One wavefront per row n = b*T + t: the token id is one scalar load shared
// by the wave, and the lanes stride over the row's 16-byte vectors, kEncU
// per lane per batch. The position rows do not depend on the token, so their
// loads are issued before the token arrives; every load of a batch is in
// flight before the first add (indices clamped into the row; the clamped
// duplicates are not stored).
static constexpr int kEncU = 4;
static constexpr int kEncRows = kThreads / 64;  // rows per workgroup

template <typename T>
__global__ __launch_bounds__(kThreads) void encoder_kernel(T* __restrict__ out,
                                                           const int32_t* __restrict__ tokens,
                                                           const T* __restrict__ wte,
                                                           const T* __restrict__ wpe, int N, int T_, int C) {
    constexpr int V = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int n = __builtin_amdgcn_readfirstlane(blockIdx.x * kEncRows + (threadIdx.x >> 6));
    if (n >= N) return;  // wave-uniform
    const int t = n % T_;
    const int cv = C / V;
    const T* p = wpe + (int64_t)t * C;
    T* o = out + (int64_t)n * C;
    const T* e = nullptr;
    for (int base = 0; base < cv; base += 64 * kEncU) {
        float a[kEncU][V], b[kEncU][V];
#pragma unroll
        for (int u = 0; u < kEncU; u++) load_vec(p + min(base + lane + 64 * u, cv - 1) * V, b[u]);
        if (base == 0) e = wte + (int64_t)__builtin_amdgcn_readfirstlane(tokens[n]) * C;
#pragma unroll
        for (int u = 0; u < kEncU; u++) load_vec(e + min(base + lane + 64 * u, cv - 1) * V, a[u]);
#pragma unroll
        for (int u = 0; u < kEncU; u++) {
            const int idx = base + lane + 64 * u;
            if (idx < cv) {
#pragma unroll
                for (int j = 0; j < V; j++) a[u][j] += b[u][j];
                store_vec(o + idx * V, a[u]);
            }
        }
    }
}

// out = a + b  (ECE408 Milestone 1, kernel table: Residual.)
template <typename T>
__global__ __launch_bounds__(kThreads) void residual_kernel(T* out, const T* a, const T* b,
                                                            int64_t n) {
    constexpr int V = Vec<T>::N;
    const int64_t nvec = n / V;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nvec; i += stride) {
        float x[V], y[V];
        load_vec(a + i * V, x);
        load_vec(b + i * V, y);
#pragma unroll
        for (int j = 0; j < V; j++) x[j] += y[j];
        store_vec(out + i * V, x);
    }
    for (int64_t i = nvec * V + blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n; i += stride)
        store_scalar(out + i, load_scalar(a + i) + load_scalar(b + i));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void gelu_kernel(T* out, const T* inp, int64_t n) {
    constexpr int V = Vec<T>::N;
    const int64_t nvec = n / V;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < nvec; i += stride) {
        float x[V];
        load_vec(inp + i * V, x);
#pragma unroll
        for (int j = 0; j < V; j++) x[j] = gelu_tanh(x[j]);
        store_vec(out + i * V, x);
    }
    for (int64_t i = nvec * V + blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n; i += stride)
        store_scalar(out + i, gelu_tanh(load_scalar(inp + i)));
}

int launch_encoder(void* out, const int32_t* tokens, const void* wte, const void* wpe, int B,
                   int T, int C, int dtype, hipStream_t s) {
    const int N = B * T;
    const unsigned grid = (unsigned)((N + kEncRows - 1) / kEncRows);
    if (dtype == GPT2_BF16)
        encoder_kernel<bf16><<<grid, kThreads, 0, s>>>((bf16*)out, tokens, (const bf16*)wte, (const bf16*)wpe,
                                                       N, T, C);
    else
        encoder_kernel<float><<<grid, kThreads, 0, s>>>((float*)out, tokens, (const float*)wte,
                                                        (const float*)wpe, N, T, C);
    return launch_status();
}

int launch_residual(void* out, const void* a, const void* b, int64_t n, int dtype,
                    hipStream_t s) {
    int64_t nvec = n / (dtype == GPT2_BF16 ? 8 : 4) + 1;
    if (dtype == GPT2_BF16)
        residual_kernel<bf16><<<stream_grid(nvec), kThreads, 0, s>>>((bf16*)out, (const bf16*)a,
                                                                    (const bf16*)b, n);
    else
        residual_kernel<float><<<stream_grid(nvec), kThreads, 0, s>>>(
            (float*)out, (const float*)a, (const float*)b, n);
    return launch_status();
}

int launch_gelu(void* out, const void* inp, int64_t n, int dtype, hipStream_t s) {
    int64_t nvec = n / (dtype == GPT2_BF16 ? 8 : 4) + 1;
    if (dtype == GPT2_BF16)
        gelu_kernel<bf16><<<stream_grid(nvec), kThreads, 0, s>>>((bf16*)out, (const bf16*)inp, n);
    else
        gelu_kernel<float><<<stream_grid(nvec), kThreads, 0, s>>>((float*)out, (const float*)inp, n);
    return launch_status();
}

}  // namespace gpt2

// ------------------------------------------------------------------ C ABI
using namespace gpt2;

extern "C" int encoder_forward(void* out, const int32_t* tokens, const void* wte, const void* wpe,
                               int B, int T, int C, int dtype, void* stream) {
    if (!valid_dtype(dtype) || B < 0 || T < 0 || C < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T * C == 0) return GPT2_OK;
    if (!out || !tokens || !wte || !wpe) return GPT2_ERR_INVALID_ARGUMENT;
    if (C % 8 || !aligned16(out) || !aligned16(wte) || !aligned16(wpe)) return GPT2_ERR_UNSUPPORTED;
    if ((int64_t)B * T > INT32_MAX) return GPT2_ERR_UNSUPPORTED;  // rows are indexed in 32 bits
    return launch_encoder(out, tokens, wte, wpe, B, T, C, dtype, (hipStream_t)stream);
}

extern "C" int residual_forward(void* out, const void* a, const void* b, int64_t n, int dtype,
                                void* stream) {
    if (!valid_dtype(dtype) || n < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (n == 0) return GPT2_OK;
    if (!out || !a || !b) return GPT2_ERR_INVALID_ARGUMENT;
    if (!aligned16(out) || !aligned16(a) || !aligned16(b)) return GPT2_ERR_UNSUPPORTED;
    return launch_residual(out, a, b, n, dtype, (hipStream_t)stream);
}

extern "C" int gelu_forward(void* out, const void* inp, int64_t n, int dtype, void* stream) {
    if (!valid_dtype(dtype) || n < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (n == 0) return GPT2_OK;
    if (!out || !inp) return GPT2_ERR_INVALID_ARGUMENT;
    if (!aligned16(out) || !aligned16(inp)) return GPT2_ERR_UNSUPPORTED;
    return launch_gelu(out, inp, n, dtype, (hipStream_t)stream);
}
