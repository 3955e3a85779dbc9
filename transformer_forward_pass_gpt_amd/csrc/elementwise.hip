// HBM-streaming kernels: token+position embedding, residual add, tanh-GELU.
// Threads move 16-byte vectors, so every wavefront issues fully coalesced
// 1 KiB requests; arithmetic is fp32 and bf16 results are rounded to nearest
// even.
#include "common.h"

namespace gpt2 {

static constexpr int kThreads = 256;

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

// Residual add and GELU stream their tensors once. Each thread owns kStreamU
// 16-byte vectors kThreads apart and issues all of their loads before the
// first use (indices clamped into the tensor; the duplicates are not
// stored), so a workgroup keeps kStreamU KiB per wavefront in flight: with
// HBM latency in the microseconds, one load per thread at a time leaves the
// memory system idle. The grid covers the tensor once; the n % V trailing
// elements (bf16: up to 7) go to the first threads of the last workgroup.
static constexpr int kStreamU = 4;

static unsigned stream_blocks(int64_t n, int v) {
    const int64_t nvec = n / v;
    const int64_t g = (nvec + (int64_t)kThreads * kStreamU - 1) / ((int64_t)kThreads * kStreamU);
    return (unsigned)(g < 1 ? 1 : g);
}

// out = a + b  (ECE408 Milestone 1, kernel table: Residual.)
template <typename T>
__global__ __launch_bounds__(kThreads) void residual_kernel(T* out, const T* a, const T* b, int64_t n) {
    constexpr int V = Vec<T>::N;
    const int64_t nvec = n / V;
    const int64_t i0 = (int64_t)blockIdx.x * kThreads * kStreamU + threadIdx.x;
    if (nvec > 0) {
        float x[kStreamU][V], y[kStreamU][V];
#pragma unroll
        for (int u = 0; u < kStreamU; u++) {
            const int64_t i = min(i0 + u * kThreads, nvec - 1);
            load_vec(a + i * V, x[u]);
            load_vec(b + i * V, y[u]);
        }
#pragma unroll
        for (int u = 0; u < kStreamU; u++) {
            const int64_t i = i0 + u * kThreads;
            if (i < nvec) {
#pragma unroll
                for (int j = 0; j < V; j++) x[u][j] += y[u][j];
                store_vec(out + i * V, x[u]);
            }
        }
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - nvec * V) {
        const int64_t i = nvec * V + threadIdx.x;
        store_scalar(out + i, load_scalar(a + i) + load_scalar(b + i));
    }
}

// out = gelu(inp), tanh form  (ECE408 Milestone 1, kernel table: GELU.)
template <typename T>
__global__ __launch_bounds__(kThreads) void gelu_kernel(T* out, const T* inp, int64_t n) {
    constexpr int V = Vec<T>::N;
    const int64_t nvec = n / V;
    const int64_t i0 = (int64_t)blockIdx.x * kThreads * kStreamU + threadIdx.x;
    if (nvec > 0) {
        float x[kStreamU][V];
#pragma unroll
        for (int u = 0; u < kStreamU; u++) load_vec(inp + min(i0 + u * kThreads, nvec - 1) * V, x[u]);
#pragma unroll
        for (int u = 0; u < kStreamU; u++) {
            const int64_t i = i0 + u * kThreads;
            if (i < nvec) {
#pragma unroll
                for (int j = 0; j < V; j++) x[u][j] = gelu_tanh(x[u][j]);
                store_vec(out + i * V, x[u]);
            }
        }
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x < n - nvec * V) {
        const int64_t i = nvec * V + threadIdx.x;
        store_scalar(out + i, gelu_tanh(load_scalar(inp + i)));
    }
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
    if (dtype == GPT2_BF16)
        residual_kernel<bf16><<<stream_blocks(n, 8), kThreads, 0, s>>>((bf16*)out, (const bf16*)a,
                                                                       (const bf16*)b, n);
    else
        residual_kernel<float><<<stream_blocks(n, 4), kThreads, 0, s>>>((float*)out, (const float*)a,
                                                                        (const float*)b, n);
    return launch_status();
}

int launch_gelu(void* out, const void* inp, int64_t n, int dtype, hipStream_t s) {
    if (dtype == GPT2_BF16)
        gelu_kernel<bf16><<<stream_blocks(n, 8), kThreads, 0, s>>>((bf16*)out, (const bf16*)inp, n);
    else
        gelu_kernel<float><<<stream_blocks(n, 4), kThreads, 0, s>>>((float*)out, (const float*)inp, n);
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
