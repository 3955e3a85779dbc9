// Row kernels: LayerNorm (one wavefront per row, the row held in registers)
// and the vocabulary softmax (one workgroup per row, the row held in
// registers). Each reads its input once and writes its output once; the
// statistics are reduced with cross-lane shuffles in fp32.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace gpt2 {

// ------------------------------------------------------------------ LayerNorm
// mu = mean(x), var = mean((x-mu)^2), rstd = 1/sqrt(var+eps),
// y = (x-mu)*rstd*gamma + beta.  Two passes over the registers, so the
// variance is the centred sum of squares, not E[x^2]-mu^2.
// (ECE408 Final Project - GPT-2, Milestone 1, kernel table: LayerNorm;
// llm.c "State of the Union [April 22, 2024]", kernel summaries:
// layernorm_forward_kernel3.)
//
// RES (decode step): the row is first updated in place as
// x <- x + (bias + sum_s part[s]), the split-k partial sums of the preceding
// projection added in split order; LayerNorm then runs on the stored
// (rounded) row, as it would after a separate residual add.
static constexpr int kMaxResSplits = 8;

// Sum over the 64 lanes of a wavefront, the same value in every lane, on
// DPP lane moves instead of LDS-routed shuffles: lane^1 and lane^2 within each
// quad, then the half-row and row mirrors (8 and 16 lanes), then the four
// 16-lane rows read out and added in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_move<0x141>(x);  // row_half_mirror
    x += dpp_move<0x140>(x);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}

template <typename T, int VPL, bool RES>
__global__ __launch_bounds__(256) void layernorm_kernel(T* __restrict__ out, float* __restrict__ mean,
                                                        float* __restrict__ rstd, T* __restrict__ inp,
                                                        const T* __restrict__ gamma,
                                                        const T* __restrict__ beta, int N, int C,
                                                        float eps, const float* __restrict__ part,
                                                        int splits, const T* __restrict__ bias, int64_t ldx) {
    constexpr int V = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= N) return;  // wave-uniform
    T* x = inp + (int64_t)row * ldx;  // input rows ldx apart (C, or T*C to take one position per sequence)
    const int cv = C / V;
    float v[VPL][V], g[VPL][V], bt[VPL][V];
    float s = 0.f;
    // Loads are unconditional (vector index clamped to the row), so every
    // load of the row, and of gamma and beta, is in flight before the first use.
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int idx = min(lane + i * 64, cv - 1);
        load_vec(x + idx * V, v[i]);
        load_vec(gamma + idx * V, g[i]);
        load_vec(beta + idx * V, bt[i]);
    }
    if constexpr (RES) {
        // x <- x + (bias + partials in split order); unused splits read a
        // clamped split and are selected to zero
        float4 q[VPL][kMaxResSplits][V / 4];
        float d[VPL][V];
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int idx = min(lane + i * 64, cv - 1);
            load_vec(bias + idx * V, d[i]);
#pragma unroll
            for (int sp = 0; sp < kMaxResSplits; sp++) {
                const float* p = part + ((int64_t)min(sp, splits - 1) * N + row) * C + idx * V;
#pragma unroll
                for (int j = 0; j < V / 4; j++) q[i][sp][j] = *reinterpret_cast<const float4*>(p + 4 * j);
            }
        }
#pragma unroll
        for (int i = 0; i < VPL; i++) {
#pragma unroll
            for (int sp = 0; sp < kMaxResSplits; sp++) {
                const bool on = sp < splits;
#pragma unroll
                for (int j = 0; j < V / 4; j++) {
                    d[i][4 * j] += on ? q[i][sp][j].x : 0.f;
                    d[i][4 * j + 1] += on ? q[i][sp][j].y : 0.f;
                    d[i][4 * j + 2] += on ? q[i][sp][j].z : 0.f;
                    d[i][4 * j + 3] += on ? q[i][sp][j].w : 0.f;
                }
            }
            // LayerNorm continues from the stored (rounded) row
#pragma unroll
            for (int j = 0; j < V; j++) v[i][j] = storage_round(x, v[i][j] + d[i][j]);
            if (lane + i * 64 < cv) store_vec(x + (lane + i * 64) * V, v[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        if (lane + i * 64 >= cv) {
#pragma unroll
            for (int j = 0; j < V; j++) v[i][j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < V; j++) s += v[i][j];
    }
    s = wave_sum_dpp(s);
    const float mu = s / (float)C;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        if (lane + i * 64 < cv) {
#pragma unroll
            for (int j = 0; j < V; j++) {
                float d = v[i][j] - mu;
                ss += d * d;
            }
        }
    }
    ss = wave_sum_dpp(ss);
    const float r = 1.0f / sqrtf(ss / (float)C + eps);
    T* y = out + (int64_t)row * C;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        int idx = lane + i * 64;
        if (idx < cv) {
#pragma unroll
            for (int j = 0; j < V; j++) v[i][j] = (v[i][j] - mu) * r * g[i][j] + bt[i][j];
            store_vec(y + idx * V, v[i]);
        }
    }
    if (lane == 0) {
        if (mean) mean[row] = mu;
        if (rstd) rstd[row] = r;
    }
}

// Sum over each half-wave (lanes 0-31, 32-63), the half's value in its lanes:
// the same DPP steps, then the two 16-lane rows of the half added.
__device__ __forceinline__ float half_sum_dpp(float x) {
    x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_move<0x141>(x);  // row_half_mirror
    x += dpp_move<0x140>(x);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
}

// LayerNorm of rows of exactly 32*VPL vectors, two rows per wavefront (lanes
// 0-31 row 2w, lanes 32-63 row 2w+1), so no lane idles where a row has an odd
// number of 32-vector groups (bf16 C = 768: 96 vectors, 3 per lane). The
// statistics are the same two-pass sums, reduced per half-wave. A missing
// second row (odd N) loads the first row's addresses and stores nothing.
template <typename T, int VPL>
__global__ __launch_bounds__(256) void layernorm2_kernel(T* __restrict__ out, float* __restrict__ mean,
                                                         float* __restrict__ rstd, const T* __restrict__ inp,
                                                         const T* __restrict__ gamma, const T* __restrict__ beta,
                                                         int N, int C, float eps, int64_t ldx) {
    constexpr int V = Vec<T>::N;
    const int hl = threadIdx.x & 31;
    const int row0 = 2 * (blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    if (row0 >= N) return;  // wave-uniform
    const int row = row0 + ((threadIdx.x >> 5) & 1);
    const bool valid = row < N;
    const T* x = inp + (int64_t)(valid ? row : row0) * ldx;
    float v[VPL][V], g[VPL][V], bt[VPL][V];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        const int idx = hl + i * 32;
        load_vec(x + idx * V, v[i]);
        load_vec(gamma + idx * V, g[i]);
        load_vec(beta + idx * V, bt[i]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++)
#pragma unroll
        for (int j = 0; j < V; j++) s += v[i][j];
    s = half_sum_dpp(s);
    const float mu = s / (float)C;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; i++)
#pragma unroll
        for (int j = 0; j < V; j++) {
            const float d = v[i][j] - mu;
            ss += d * d;
        }
    ss = half_sum_dpp(ss);
    const float r = 1.0f / sqrtf(ss / (float)C + eps);
    if (!valid) return;
    T* y = out + (int64_t)row * C;
#pragma unroll
    for (int i = 0; i < VPL; i++) {
#pragma unroll
        for (int j = 0; j < V; j++) v[i][j] = (v[i][j] - mu) * r * g[i][j] + bt[i][j];
        store_vec(y + (hl + i * 32) * V, v[i]);
    }
    if (hl == 0) {
        if (mean) mean[row] = mu;
        if (rstd) rstd[row] = r;
    }
}

template <typename T, bool RES>
static void launch_ln_t(T* out, float* mean, float* rstd, T* inp, const T* g, const T* b, int N, int C,
                        float eps, const float* part, int splits, const T* bias, hipStream_t s, int64_t ldx = 0) {
    if (ldx == 0) ldx = C;
    const int cv = C / Vec<T>::N;
    if (!RES && cv % 64 == 32 && cv <= 160) {  // 1, 3 or 5 groups of 32 vectors: two rows per wavefront
        const dim3 grid2((N + 7) / 8), block2(256);
#define LN2_LAUNCH(P) \
    layernorm2_kernel<T, P><<<grid2, block2, 0, s>>>(out, mean, rstd, inp, g, b, N, C, eps, ldx)
        if (cv == 32) LN2_LAUNCH(1);
        else if (cv == 96) LN2_LAUNCH(3);
        else LN2_LAUNCH(5);
#undef LN2_LAUNCH
        return;
    }
    const int vpl = (cv + 63) / 64;
    // RES runs on decode-sized batches: one row per workgroup spreads them over CUs
    const int rows = RES ? 1 : 4;
    const dim3 grid((N + rows - 1) / rows), block(64 * rows);
#define LN_LAUNCH(P) \
    layernorm_kernel<T, P, RES><<<grid, block, 0, s>>>(out, mean, rstd, inp, g, b, N, C, eps, part, splits, bias, \
                                                       ldx)
    if (vpl <= 1) LN_LAUNCH(1);
    else if (vpl <= 2) LN_LAUNCH(2);
    else if (vpl <= 3) LN_LAUNCH(3);
    else if (vpl <= 4) LN_LAUNCH(4);
    else if (vpl <= 8) LN_LAUNCH(8);
    else LN_LAUNCH(16);
#undef LN_LAUNCH
}

int launch_layernorm(void* out, float* mean, float* rstd, const void* inp, const void* gamma,
                     const void* beta, int N, int C, float eps, int dtype, hipStream_t s) {
    // the input is only read on this path
    if (dtype == GPT2_BF16)
        launch_ln_t<bf16, false>((bf16*)out, mean, rstd, (bf16*)inp, (const bf16*)gamma, (const bf16*)beta, N,
                                 C, eps, nullptr, 0, nullptr, s);
    else
        launch_ln_t<float, false>((float*)out, mean, rstd, (float*)inp, (const float*)gamma,
                                  (const float*)beta, N, C, eps, nullptr, 0, nullptr, s);
    return launch_status();
}

// LayerNorm of N rows taken ldx elements apart (out rows are contiguous).
int launch_layernorm_rows(void* out, const void* inp, int64_t ldx, const void* gamma, const void* beta, int N,
                          int C, float eps, int dtype, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_ln_t<bf16, false>((bf16*)out, nullptr, nullptr, (bf16*)inp, (const bf16*)gamma, (const bf16*)beta,
                                 N, C, eps, nullptr, 0, nullptr, s, ldx);
    else
        launch_ln_t<float, false>((float*)out, nullptr, nullptr, (float*)inp, (const float*)gamma,
                                  (const float*)beta, N, C, eps, nullptr, 0, nullptr, s, ldx);
    return launch_status();
}

// x <- x + bias + sum_s part[s][N][C] (in place), then out = LayerNorm(x).
int launch_residual_layernorm(void* out, void* x, const float* part, int splits, const void* bias,
                              const void* gamma, const void* beta, int N, int C, float eps, int dtype,
                              hipStream_t s) {
    if (splits < 1 || splits > kMaxResSplits) return GPT2_ERR_INVALID_ARGUMENT;
    if (dtype == GPT2_BF16)
        launch_ln_t<bf16, true>((bf16*)out, nullptr, nullptr, (bf16*)x, (const bf16*)gamma, (const bf16*)beta,
                                N, C, eps, part, splits, (const bf16*)bias, s);
    else
        launch_ln_t<float, true>((float*)out, nullptr, nullptr, (float*)x, (const float*)gamma,
                                 (const float*)beta, N, C, eps, part, splits, (const float*)bias, s);
    return launch_status();
}

// ------------------------------------------------------------ vocab softmax
// probs[v] = exp(l_v - m) / sum_{u<V} exp(l_u - m) for v < V, 0 for v >= V,
// m = max_{u<V} l_u. One workgroup of up to 1024 threads per row; each
// thread keeps PT 16-byte vectors of the row in registers between the max,
// the sum and the write, so HBM sees one read and one write per element.
// PACKED: the vectors stay as loaded (bf16: two values per register) and each
// pass widens them again, the exponential is evaluated again for the store:
// a bf16 row of GPT-2's vocabulary then needs 52 instead of 95 registers, so
// two 1024-thread workgroups share a CU and one row's loads overlap the
// other's reductions and stores. Worth it when there are rows for every CU
// twice over; otherwise the widened copies stay live (shorter chains).
// Both forms compute the same values in the same order.
// (llm.c "State of the Union", kernel summaries: the softmax half of
// fused_classifier_kernel3.)
template <int NW>
__device__ __forceinline__ float block_max(float x, float* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    x = wave_max(x);
    if (lane == 0) sh[w] = x;
    __syncthreads();
    x = lane < NW ? sh[lane] : -INFINITY;
    x = wave_max(x);
    __syncthreads();
    return x;
}
template <int NW>
__device__ __forceinline__ float block_sum(float x, float* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    x = wave_sum(x);
    if (lane == 0) sh[w] = x;
    __syncthreads();
    x = lane < NW ? sh[lane] : 0.f;
    x = wave_sum(x);
    __syncthreads();
    return x;
}

// With targets and losses (the loss half of fused_classifier_kernel3, llm.c
// "State of the Union", kernel summaries) the same pass also writes the
// cross-entropy of each row, loss = log(sum_{v<V} e^{l_v - m}) + m - l_target,
// from the max and sum it already holds; probs may then be NULL.
// BWD (the backward half of that classifier): probs receives instead the
// gradient of sum_n dscale * loss_n with respect to the logits,
// dscale * (p_v - [v == target]), 0 in the padding columns. It may overwrite
// the logits in place: every element of the row (and the target's logit) is
// read before the first barrier, and every write comes after it.
template <typename T, int PT, int NT, bool BWD = false, bool PACKED = false>
__global__ __launch_bounds__(NT) void softmax_kernel(T* probs, const T* logits, int V, int Vp,
                                                     const int32_t* __restrict__ targets,
                                                     float* __restrict__ losses, float dscale) {
    constexpr int VE = Vec<T>::N;
    constexpr int NW = NT / 64;
    __shared__ float sh[NW];
    const int64_t row = blockIdx.x;
    const T* x = logits + row * Vp;
    T* y = probs + row * Vp;
    const int cv = Vp / VE;
    const int tg = targets ? targets[row] : 0;
    const float lt = targets ? load_scalar(x + tg) : 0.f;
    // The row is read once and the probabilities written once, so both go
    // past the caches (non-temporal), leaving them to the operands of the
    // kernels around this one.
    // Every load of the row is issued before the first use: indices past the
    // row are clamped to its last vector and masked, not branched around
    // (a load inside a divergent branch would be waited for at the branch's end).
    if constexpr (PACKED) {
        u32x4 raw[PT];
#pragma unroll
        for (int i = 0; i < PT; i++)
            raw[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(x + min((int)threadIdx.x + i * NT, cv - 1) * VE));
        // An empty asm that may rewrite the vectors keeps the compiler from
        // carrying widened copies (or exponentials) from one pass to the next.
        auto opaque = [&]() {
#pragma unroll
            for (int i = 0; i < PT; i++) asm volatile("" : "+v"(raw[i]));
        };
        // Elements at or past V (padding columns, or a clamped vector past the
        // row) become -inf once, so the passes below need no masks.
#pragma unroll
        for (int i = 0; i < PT; i++) {
            const int idx = threadIdx.x + i * NT;
            const int nv = idx < cv ? V - idx * VE : 0;  // valid elements of vector i (when < VE)
            if constexpr (VE == 8) {
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    const uint32_t lo = 2 * w < nv ? raw[i][w] & 0xffffu : 0xff80u;
                    const uint32_t hi = 2 * w + 1 < nv ? raw[i][w] >> 16 : 0xff80u;
                    raw[i][w] = lo | (hi << 16);
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; w++) raw[i][w] = w < nv ? raw[i][w] : 0xff800000u;  // -inf
            }
        }
        opaque();
        auto elem = [&](int i, int j) -> float {
            if constexpr (VE == 8) return bf16_to_f32((raw[i][j >> 1] >> (16 * (j & 1))) & 0xffffu);
            else return __uint_as_float(raw[i][j]);
        };
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < PT; i++)
#pragma unroll
            for (int j = 0; j < VE; j++) m = fmaxf(m, elem(i, j));
        m = block_max<NW>(m, sh);
        opaque();
        // e^{l - m} = 2^{(l - m) log2 e} on the hardware base-2 exponential; the
        // difference is formed first, so the argument's rounding error scales with
        // |l - m| (tiny probabilities), not with |l|.
        const float L2E = 1.4426950408889634f;
        auto ex = [&](int i, int j) { return __builtin_amdgcn_exp2f((elem(i, j) - m) * L2E); };  // 2^-inf = 0
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < PT; i++)
#pragma unroll
            for (int j = 0; j < VE; j++) s += ex(i, j);
        s = block_sum<NW>(s, sh);
        if (losses && threadIdx.x == 0) losses[row] = logf(s) + m - lt;
        if (!probs) return;
        const float inv = 1.0f / s;
        opaque();
#pragma unroll
        for (int i = 0; i < PT; i++) {
            const int idx = threadIdx.x + i * NT;
            if (idx < cv) {
                float v[VE];
#pragma unroll
                for (int j = 0; j < VE; j++) {
                    if constexpr (BWD)
                        v[j] = (ex(i, j) * inv - (idx * VE + j == tg ? 1.f : 0.f)) * dscale;
                    else
                        v[j] = ex(i, j) * inv;
                }
                store_vec_nt(y + idx * VE, v);
            }
        }
    } else {
        float v[PT][VE];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < PT; i++) {
            const u32x4 raw = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(x + min((int)threadIdx.x + i * NT, cv - 1) * VE));
            unpack_vec<T>(raw, v[i]);
        }
#pragma unroll
        for (int i = 0; i < PT; i++) {
            const int idx = threadIdx.x + i * NT;
#pragma unroll
            for (int j = 0; j < VE; j++) {
                if (idx >= cv || idx * VE + j >= V) v[i][j] = -INFINITY;
                m = fmaxf(m, v[i][j]);
            }
        }
        m = block_max<NW>(m, sh);
        // e^{l - m} = 2^{(l - m) log2 e} on the hardware base-2 exponential; the
        // difference is formed first, so the argument's rounding error scales with
        // |l - m| (tiny probabilities), not with |l|.
        const float L2E = 1.4426950408889634f;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < PT; i++)
#pragma unroll
            for (int j = 0; j < VE; j++) {
                v[i][j] = __builtin_amdgcn_exp2f((v[i][j] - m) * L2E);  // 2^-inf = 0 for padding
                s += v[i][j];
            }
        s = block_sum<NW>(s, sh);
        if (losses && threadIdx.x == 0) losses[row] = logf(s) + m - lt;
        if (!probs) return;
        const float inv = 1.0f / s;
#pragma unroll
        for (int i = 0; i < PT; i++) {
            int idx = threadIdx.x + i * NT;
            if (idx < cv) {
#pragma unroll
                for (int j = 0; j < VE; j++) {
                    if constexpr (BWD)
                        v[i][j] = (v[i][j] * inv - (idx * VE + j == tg ? 1.f : 0.f)) * dscale;
                    else
                        v[i][j] *= inv;
                }
                store_vec_nt(y + idx * VE, v[i]);
            }
        }
    }
}

// Mean of n fp32 values in one workgroup, in a fixed order (deterministic).
__global__ __launch_bounds__(1024) void mean_kernel(float* __restrict__ out, const float* __restrict__ x, int n) {
    __shared__ float sh[16];
    float a = 0.f;
    for (int i = threadIdx.x; i < n; i += 1024) a += x[i];
    a = block_sum<16>(a, sh);
    if (threadIdx.x == 0) *out = a / (float)n;
}

template <typename T, bool BWD = false>
static void launch_softmax_t(T* probs, const T* logits, int N, int V, int Vp, hipStream_t s,
                             const int32_t* targets = nullptr, float* losses = nullptr, float dscale = 0.f) {
    const int cv = Vp / Vec<T>::N;
    dim3 grid(N);
#define SM_LAUNCH(P, NT) \
    softmax_kernel<T, P, NT, BWD><<<grid, NT, 0, s>>>(probs, logits, V, Vp, targets, losses, dscale)
    if (cv <= 256) {
        SM_LAUNCH(1, 256);
        return;
    }
    const int pt = (cv + 1023) / 1024;
    if constexpr (std::is_same<T, bf16>::value) {
        if (pt == 7 && N >= 512) {  // GPT-2's vocabulary, many rows
            softmax_kernel<T, 7, 1024, BWD, true><<<grid, 1024, 0, s>>>(probs, logits, V, Vp, targets, losses,
                                                                          dscale);
            return;
        }
    }
    if (pt <= 1) SM_LAUNCH(1, 1024);
    else if (pt <= 2) SM_LAUNCH(2, 1024);
    else if (pt <= 4) SM_LAUNCH(4, 1024);
    else if (pt <= 7) SM_LAUNCH(7, 1024);
    else if (pt <= 13) SM_LAUNCH(13, 1024);
    else if (pt <= 16) SM_LAUNCH(16, 1024);
    else SM_LAUNCH(32, 1024);
#undef SM_LAUNCH
}

// One-pass vocabulary softmax from the row statistics the logits GEMM wrote
// (EPI_STATS: per group g of kStatCols columns, m_g = max and s_g = sum of
// e^{l - m_g} over the group's columns < V): M = max_g m_g,
// S = sum_g s_g e^{m_g - M}, probs_v = e^{l_v - M} / S for v < V and 0 for
// V <= v < Vp. As softmax_kernel, one workgroup per row holds the row in
// registers (every load issued at once), but the max and the sum need no
// reduction over the row: wavefront 0 combines the groups (fixed order: by
// lane, then a fixed shuffle tree) while the loads are in flight, and one
// barrier hands M and 1/S to the others.
template <typename T, int PT, int NT>
__global__ __launch_bounds__(NT) void softmax_stats_kernel(T* __restrict__ probs, const T* __restrict__ logits,
                                                           const float* __restrict__ stats, int V, int Vp, int ngrp) {
    constexpr int VE = Vec<T>::N;
    __shared__ float sh[2];
    const int64_t row = blockIdx.x;
    const T* x = logits + row * Vp;
    T* y = probs + row * Vp;
    const int cv = Vp / VE;
    float v[PT][VE];
#pragma unroll
    for (int i = 0; i < PT; i++) load_vec(x + min((int)threadIdx.x + i * NT, cv - 1) * VE, v[i]);
    const float L2E = 1.4426950408889634f;
    if (threadIdx.x < 64) {
        const float* st = stats + row * ngrp * 2;
        const int lane = threadIdx.x;
        float m = -INFINITY;
        for (int g = lane; g < ngrp; g += 64) m = fmaxf(m, st[2 * g]);
        m = wave_max(m);
        float sum = 0.f;
        for (int g = lane; g < ngrp; g += 64) sum += st[2 * g + 1] * __builtin_amdgcn_exp2f((st[2 * g] - m) * L2E);
        sum = wave_sum(sum);
        if (lane == 0) {
            sh[0] = m;
            sh[1] = 1.0f / sum;
        }
    }
    __syncthreads();
    const float m = sh[0], inv = sh[1];
#pragma unroll
    for (int i = 0; i < PT; i++) {
        const int idx = threadIdx.x + i * NT;
        if (idx < cv) {
#pragma unroll
            for (int j = 0; j < VE; j++)
                v[i][j] = idx * VE + j < V ? __builtin_amdgcn_exp2f((v[i][j] - m) * L2E) * inv : 0.f;
            store_vec(y + idx * VE, v[i]);
        }
    }
}

int launch_softmax_stats(void* probs, const void* logits, const float* stats, int N, int V, int Vp, int dtype,
                         hipStream_t s) {
    const int ngrp = (Vp + kStatCols - 1) / kStatCols;
    const int cv = Vp / (dtype == GPT2_BF16 ? 8 : 4);
    const dim3 grid(N);
#define SMS_LAUNCH(P, NT)                                                                                          \
    do {                                                                                                           \
        if (dtype == GPT2_BF16)                                                                                    \
            softmax_stats_kernel<bf16, P, NT><<<grid, NT, 0, s>>>((bf16*)probs, (const bf16*)logits, stats, V, Vp, \
                                                                  ngrp);                                           \
        else                                                                                                       \
            softmax_stats_kernel<float, P, NT><<<grid, NT, 0, s>>>((float*)probs, (const float*)logits, stats, V,  \
                                                                   Vp, ngrp);                                      \
    } while (0)
    if (cv <= 256) SMS_LAUNCH(1, 256);
    else if (cv <= 1024) SMS_LAUNCH(1, 1024);
    else if (cv <= 2048) SMS_LAUNCH(2, 1024);
    else if (cv <= 4096) SMS_LAUNCH(4, 1024);
    else if (cv <= 7168) SMS_LAUNCH(7, 1024);
    else if (cv <= 13312) SMS_LAUNCH(13, 1024);
    else if (cv <= 16384) SMS_LAUNCH(16, 1024);
    else SMS_LAUNCH(32, 1024);
#undef SMS_LAUNCH
    return launch_status();
}

// Softmax (probs nullable) with per-row cross-entropy, and the mean loss.
int launch_softmax_loss(void* probs, float* losses, float* mean, const void* logits, const int32_t* targets, int N,
                        int V, int Vp, int dtype, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_softmax_t<bf16>((bf16*)probs, (const bf16*)logits, N, V, Vp, s, targets, losses);
    else
        launch_softmax_t<float>((float*)probs, (const float*)logits, N, V, Vp, s, targets, losses);
    if (mean) mean_kernel<<<1, 1024, 0, s>>>(mean, losses, N);
    return launch_status();
}

// dlogits = dscale * (softmax - onehot(target)) (may overwrite logits), with
// the per-row losses and their mean (both nullable).
int launch_crossentropy_backward(void* dlogits, float* losses, float* mean, const void* logits,
                                 const int32_t* targets, float dscale, int N, int V, int Vp, int dtype,
                                 hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_softmax_t<bf16, true>((bf16*)dlogits, (const bf16*)logits, N, V, Vp, s, targets, losses, dscale);
    else
        launch_softmax_t<float, true>((float*)dlogits, (const float*)logits, N, V, Vp, s, targets, losses,
                                      dscale);
    if (mean && losses) mean_kernel<<<1, 1024, 0, s>>>(mean, losses, N);
    return launch_status();
}

int launch_softmax(void* probs, const void* logits, int N, int V, int Vp, int dtype,
                   hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_softmax_t<bf16>((bf16*)probs, (const bf16*)logits, N, V, Vp, s);
    else
        launch_softmax_t<float>((float*)probs, (const float*)logits, N, V, Vp, s);
    return launch_status();
}

// --------------------------------------------------------------- argmax
// Greedy next-token choice: tok[n] = argmax over v < V of logits[n, v], the
// lowest index among equal maxima; also written to out[n * out_stride] when
// out is given. One 256-thread workgroup per row; each thread keeps its best
// (value, index) over its 16-byte vectors of the row, then wavefront shuffles
// and LDS reduce with the same tie rule, so the result does not depend on the
// order. Vp % 8 == 0 (16-byte rows).
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) {
        bv = v;
        bi = i;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void argmax_kernel(int32_t* __restrict__ tok, int32_t* __restrict__ out,
                                                     int out_stride, const T* __restrict__ logits, int V, int Vp) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int VE = Vec<T>::N, U = 8;
    const T* l = logits + (int64_t)row * Vp;
    const int cv = Vp / VE;
    float bv = -INFINITY;
    int bi = V;  // beats nothing: every real index is lower
    // U 16-byte vectors per thread in flight (indices clamped, values masked)
    for (int base = 0; base < cv; base += 256 * U) {
        float x[U][VE];
#pragma unroll
        for (int u = 0; u < U; u++) load_vec(l + min(base + u * 256 + tid, cv - 1) * VE, x[u]);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int vi = base + u * 256 + tid;
#pragma unroll
            for (int j = 0; j < VE; j++)
                if (vi < cv && vi * VE + j < V) better(bv, bi, x[u][j], vi * VE + j);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        better(bv, bi, ov, oi);
    }
    if (lane == 0) {
        sv[w] = bv;
        si[w] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int i = 1; i < 4; i++) better(bv, bi, sv[i], si[i]);
        tok[row] = bi;
        if (out) out[(int64_t)row * out_stride] = bi;
    }
}

int launch_argmax(int32_t* tok, int32_t* out, int out_stride, const void* logits, int N, int V, int Vp, int dtype,
                  hipStream_t s) {
    if (dtype == GPT2_BF16)
        argmax_kernel<bf16><<<N, 256, 0, s>>>(tok, out, out_stride, (const bf16*)logits, V, Vp);
    else
        argmax_kernel<float><<<N, 256, 0, s>>>(tok, out, out_stride, (const float*)logits, V, Vp);
    return launch_status();
}

}  // namespace gpt2

// ------------------------------------------------------------------ C ABI
using namespace gpt2;

extern "C" int layernorm_forward(void* out, float* mean, float* rstd, const void* inp,
                                 const void* gamma, const void* beta, int N, int C, float eps,
                                 int dtype, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || C < 0 || !(eps >= 0.f)) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!out || !inp || !gamma || !beta || C == 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (C % 8 || C > 4096 || !aligned16(out) || !aligned16(inp) || !aligned16(gamma) ||
        !aligned16(beta))
        return GPT2_ERR_UNSUPPORTED;
    if (out == inp) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_layernorm(out, mean, rstd, inp, gamma, beta, N, C, eps, dtype,
                            (hipStream_t)stream);
}

extern "C" int residual_layernorm_forward(void* out, void* x, const float* part, int splits, const void* bias,
                                          const void* gamma, const void* beta, int N, int C, float eps,
                                          int dtype, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || C < 0 || !(eps >= 0.f) || splits < 1 || splits > kMaxResSplits)
        return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!out || !x || !part || !bias || !gamma || !beta || C == 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (C % 8 || C > 4096 || !aligned16(out) || !aligned16(x) || !aligned16(part) || !aligned16(bias) ||
        !aligned16(gamma) || !aligned16(beta))
        return GPT2_ERR_UNSUPPORTED;
    if (out == x) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_residual_layernorm(out, x, part, splits, bias, gamma, beta, N, C, eps, dtype,
                                     (hipStream_t)stream);
}

extern "C" int argmax_forward(int32_t* tokens, const void* logits, int N, int V, int Vp, int dtype, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || V < 0 || Vp < V) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!tokens || !logits || V == 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (Vp % 8 || !aligned16(logits)) return GPT2_ERR_UNSUPPORTED;
    return launch_argmax(tokens, nullptr, 0, logits, N, V, Vp, dtype, (hipStream_t)stream);
}

extern "C" int crossentropy_forward(float* losses, float* mean_loss, void* probs, const void* logits,
                                    const int32_t* targets, int N, int V, int Vp, int dtype, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || V < 0 || Vp < V) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!losses || !logits || !targets || V == 0 || probs == logits) return GPT2_ERR_INVALID_ARGUMENT;
    if (Vp % 8 || Vp > 131072 || !aligned16(logits) || (probs && !aligned16(probs))) return GPT2_ERR_UNSUPPORTED;
    return launch_softmax_loss(probs, losses, mean_loss, logits, targets, N, V, Vp, dtype, (hipStream_t)stream);
}

extern "C" int softmax_stats_forward(void* probs, const void* logits, const float* stats, int N, int V, int Vp,
                                     int dtype, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || V < 1 || V > Vp) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!probs || !logits || !stats || probs == logits) return GPT2_ERR_INVALID_ARGUMENT;
    if (Vp % 8 || Vp > 131072 || !aligned16(probs) || !aligned16(logits) || !aligned16(stats))
        return GPT2_ERR_UNSUPPORTED;
    return launch_softmax_stats(probs, logits, stats, N, V, Vp, dtype, (hipStream_t)stream);
}

extern "C" int softmax_forward(void* probs, const void* logits, int N, int V, int Vp, int dtype,
                               void* stream) {
    if (!valid_dtype(dtype) || N < 0 || V < 0 || Vp < V) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!probs || !logits || V == 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (Vp % 8 || Vp > 131072 || !aligned16(probs) || !aligned16(logits))
        return GPT2_ERR_UNSUPPORTED;
    if (probs == logits) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_softmax(probs, logits, N, V, Vp, dtype, (hipStream_t)stream);
}

extern "C" int crossentropy_backward(void* dlogits, float* losses, float* mean_loss, const void* logits,
                                     const int32_t* targets, float dloss, int N, int V, int Vp, int dtype,
                                     void* stream) {
    if (!valid_dtype(dtype) || N < 0 || V < 0 || Vp < V) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!dlogits || !logits || !targets || V == 0 || (mean_loss && !losses)) return GPT2_ERR_INVALID_ARGUMENT;
    if (Vp % 8 || Vp > 131072 || !aligned16(logits) || !aligned16(dlogits)) return GPT2_ERR_UNSUPPORTED;
    return launch_crossentropy_backward(dlogits, losses, mean_loss, logits, targets, dloss, N, V, Vp, dtype,
                                        (hipStream_t)stream);
}
