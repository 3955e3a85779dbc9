// Linear layer on the gfx950 matrix cores:
//   out[n,o] = sum_c inp[n,c] * W[o,c] + bias[o]
// (ECE408 Final Project - GPT-2, Milestone 1, kernel table: MatMul; the
// optdl2025 project "A study on GPU for matrix-matrix products" motivates
// staging operand tiles in on-chip shared memory.)
//
// Both operands are K-contiguous, which is the layout the MFMA operand
// fragments want: every lane reads one 16-byte run of k from one row.
// Tiles of A and W are staged through LDS (double-buffered, one barrier per
// k-tile), each wavefront owns a TM x TN grid of 32x32 accumulator tiles.
//   fp32: v_mfma_f32_32x32x2_f32  (4 instructions per 16-byte fragment)
//   bf16: v_mfma_f32_32x32x16_bf16 (1 instruction per 16-byte fragment)
// The k order inside a 16-byte fragment is the same for A and W, so the
// contraction is exact whatever slot each k lands in.
#include "common.h"

namespace gpt2 {

template <typename T> struct Mfma32;
template <> struct Mfma32<float> {
    static __device__ __forceinline__ void run(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
        for (int e = 0; e < 4; e++)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]),
                                                      acc, 0, 0, 0);
    }
};
template <> struct Mfma32<bf16> {
    static __device__ __forceinline__ void run(f32x16& acc, const u32x4& a, const u32x4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

// WM x WN wavefronts, each owning TM x TN 32x32 tiles; BK = k per LDS tile.
template <typename T, int WM, int WN, int TM, int TN, int BK>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(T* __restrict__ out, const T* __restrict__ A,
                                                           const T* __restrict__ W,
                                                           const T* __restrict__ bias, int M, int N,
                                                           int K) {
    constexpr int NT = WM * WN * 64;
    constexpr int VE = Vec<T>::N;
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    constexpr int LDK = BK + VE;  // 16-byte pad per LDS row: conflict-free 16-byte reads
    constexpr int KV = BK / VE;   // 16-byte vectors per tile row
    constexpr int LA = BM * KV / NT, LB = BN * KV / NT;
    static_assert((BM * KV) % NT == 0 && (BN * KV) % NT == 0, "tile/thread mismatch");
    static_assert(BK % (2 * VE) == 0, "BK must hold whole fragments");
    __shared__ __attribute__((aligned(16))) T As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int h = lane >> 5, r32 = lane & 31;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    u32x4 ra[LA], rb[LB];
    auto gload = [&](int k0) {
#pragma unroll
        for (int r = 0; r < LA; r++) {
            int li = tid + r * NT, row = li / KV, kv = li % KV;
            int gm = m0 + row, k = k0 + kv * VE;
            ra[r] = (gm < M && k < K) ? *reinterpret_cast<const u32x4*>(A + (int64_t)gm * K + k) : zero;
        }
#pragma unroll
        for (int r = 0; r < LB; r++) {
            int li = tid + r * NT, row = li / KV, kv = li % KV;
            int gn = n0 + row, k = k0 + kv * VE;
            rb[r] = (gn < N && k < K) ? *reinterpret_cast<const u32x4*>(W + (int64_t)gn * K + k) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int r = 0; r < LA; r++) {
            int li = tid + r * NT, row = li / KV, kv = li % KV;
            *reinterpret_cast<u32x4*>(&As[buf][row * LDK + kv * VE]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < LB; r++) {
            int li = tid + r * NT, row = li / KV, kv = li % KV;
            *reinterpret_cast<u32x4*>(&Bs[buf][row * LDK + kv * VE]) = rb[r];
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = f32x16{};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kc = 0; kc < BK / (2 * VE); kc++) {
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                fa[i] = *reinterpret_cast<const u32x4*>(
                    &As[cur][(wm * TM * 32 + i * 32 + r32) * LDK + kc * 2 * VE + h * VE]);
#pragma unroll
            for (int j = 0; j < TN; j++)
                fb[j] = *reinterpret_cast<const u32x4*>(
                    &Bs[cur][(wn * TN * 32 + j * 32 + r32) * LDK + kc * 2 * VE + h * VE]);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) Mfma32<T>::run(acc[i][j], fa[i], fb[j]);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // 32x32 accumulator layout: register v of lane (h, r32) holds
    // row 8*(v/4) + 4*h + v%4, column r32.
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int col = n0 + wn * TN * 32 + j * 32 + r32;
        if (col >= N) continue;
        const float bv = bias ? load_scalar(bias + col) : 0.f;
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int row = m0 + wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                if (row < M) store_scalar(out + (int64_t)row * N + col, acc[i][j][v] + bv);
            }
        }
    }
}

template <typename T, int WM, int WN, int TM, int TN, int BK>
static void launch_cfg(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                       hipStream_t s) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
    gemm_kernel<T, WM, WN, TM, TN, BK><<<grid, WM * WN * 64, 0, s>>>(out, A, W, bias, M, N, K);
}

template <typename T>
static void launch_gemm_t(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                          hipStream_t s) {
    constexpr int BK = Vec<T>::N * 8;  // 128 bytes of k per row per LDS tile
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (M <= 32)
        launch_cfg<T, 1, 2, 1, 1, BK>(out, A, W, bias, M, N, K, s);
    else if (tiles(128, 128) >= 512)
        launch_cfg<T, 2, 2, 2, 2, BK>(out, A, W, bias, M, N, K, s);
    else if (tiles(64, 128) >= 256)
        launch_cfg<T, 2, 2, 1, 2, BK>(out, A, W, bias, M, N, K, s);
    else
        launch_cfg<T, 2, 2, 1, 1, BK>(out, A, W, bias, M, N, K, s);
}

int launch_matmul(void* out, const void* inp, const void* weight, const void* bias, int N, int C,
                  int OC, int dtype, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_gemm_t<bf16>((bf16*)out, (const bf16*)inp, (const bf16*)weight, (const bf16*)bias, N,
                            OC, C, s);
    else
        launch_gemm_t<float>((float*)out, (const float*)inp, (const float*)weight,
                             (const float*)bias, N, OC, C, s);
    return launch_status();
}

}  // namespace gpt2

using namespace gpt2;

extern "C" int matmul_forward(void* out, const void* inp, const void* weight, const void* bias,
                              int N, int C, int OC, int dtype, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || C < 0 || OC < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)N * OC == 0) return GPT2_OK;
    if (!out || !inp || !weight || C == 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (C % 8 || OC % 8 || !aligned16(out) || !aligned16(inp) || !aligned16(weight))
        return GPT2_ERR_UNSUPPORTED;
    if (out == inp || out == weight) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_matmul(out, inp, weight, bias, N, C, OC, dtype, (hipStream_t)stream);
}
