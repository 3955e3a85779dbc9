// MFMA GEMM kernel template for the linear layers:
//   out[m,n] = sum_k A[m,k] * W[n,k] + bias[n]
// (ECE408 Final Project - GPT-2, Milestone 1, kernel table: MatMul; the
// optdl2025 project "A study on GPU for matrix-matrix products" motivates
// staging operand tiles in on-chip shared memory.)
//
// Both operands are K-contiguous, which is the layout the MFMA operand
// fragments want: every lane reads one 16-byte run of k from one row.
// Tiles of A and W are staged through LDS (double-buffered, one barrier per
// k-tile); each wavefront owns a TM x TN grid of 32x32 accumulator tiles.
//   fp32: v_mfma_f32_32x32x2_f32  (4 instructions per 16-byte fragment)
//   bf16: v_mfma_f32_32x32x16_bf16 (1 instruction per 16-byte fragment)
// The k order inside a 16-byte fragment is the same for A and W, so the
// contraction is exact whatever slot each k lands in.
//
// Tile order: the 1-D grid is first regrouped so each of the 8 XCDs (which
// receive workgroups round-robin) owns a contiguous range of tiles, and that
// range is walked in groups of `group_m` row tiles, so the A rows and W
// columns a CU needs are shared with its XCD neighbours through that XCD's L2.
#pragma once
#include "common.h"

namespace gpt2 {

// One 16-byte fragment pair holds STEPS MFMA k-steps: step e of a fragment
// pair is one MFMA instruction.
template <typename T> struct Mfma32;
template <> struct Mfma32<float> {
    static constexpr int STEPS = 4;
    static __device__ __forceinline__ void step(f32x16& acc, const u32x4& a, const u32x4& b, int e) {
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc,
                                                  0, 0, 0);
    }
};
template <> struct Mfma32<bf16> {
    static constexpr int STEPS = 1;
    static __device__ __forceinline__ void step(f32x16& acc, const u32x4& a, const u32x4& b, int) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

static constexpr int kNumXcd = 8;

// Workgroup i runs on XCD i % 8. Map it to a logical tile index so that XCD x
// owns the contiguous logical range assigned to it. A bijection on [0, n).
__device__ __forceinline__ int xcd_contiguous(int i, int n) {
    const int q = n / kNumXcd, r = n % kNumXcd;
    const int x = i % kNumXcd, local = i / kNumXcd;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

// WM x WN wavefronts, each owning TM x TN 32x32 tiles; BK = k per LDS tile.
template <typename T, int WM, int WN, int TM, int TN, int BK, bool ILV = true>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(T* __restrict__ out, const T* __restrict__ A,
                                                           const T* __restrict__ W,
                                                           const T* __restrict__ bias, int M, int N,
                                                           int K, int group_m, int remap) {
    constexpr int NT = WM * WN * 64;
    constexpr int VE = Vec<T>::N;
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    constexpr int LDK = BK + VE;  // 16-byte pad per LDS row: conflict-free 16-byte reads
    constexpr int KV = BK / VE;   // 16-byte vectors per tile row
    constexpr int LA = (BM * KV + NT - 1) / NT, LB = (BN * KV + NT - 1) / NT;
    static_assert(BK % (2 * VE) == 0, "BK must hold whole fragments");
    __shared__ __attribute__((aligned(16))) T As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) T Bs[2][BN * LDK];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int h = lane >> 5, r32 = lane & 31;

    // tile coordinates
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int nwg = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if (remap) pid = xcd_contiguous(pid, nwg);
    const int per_group = group_m * tiles_n;
    const int g = pid / per_group, first_m = g * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in_g = pid - g * per_group;
    const int m0 = (first_m + in_g % gsz) * BM, n0 = (in_g / gsz) * BN;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    u32x4 ra[LA], rb[LB];
    auto gload = [&](int k0) {
#pragma unroll
        for (int r = 0; r < LA; r++) {
            const int li = tid + r * NT, row = li / KV, kv = li % KV;
            const int gm = m0 + row, k = k0 + kv * VE;
            ra[r] = (li < BM * KV && gm < M && k < K)
                        ? *reinterpret_cast<const u32x4*>(A + (int64_t)gm * K + k) : zero;
        }
#pragma unroll
        for (int r = 0; r < LB; r++) {
            const int li = tid + r * NT, row = li / KV, kv = li % KV;
            const int gn = n0 + row, k = k0 + kv * VE;
            rb[r] = (li < BN * KV && gn < N && k < K)
                        ? *reinterpret_cast<const u32x4*>(W + (int64_t)gn * K + k) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int r = 0; r < LA; r++) {
            const int li = tid + r * NT, row = li / KV, kv = li % KV;
            if (li < BM * KV) *reinterpret_cast<u32x4*>(&As[buf][row * LDK + kv * VE]) = ra[r];
        }
#pragma unroll
        for (int r = 0; r < LB; r++) {
            const int li = tid + r * NT, row = li / KV, kv = li % KV;
            if (li < BN * KV) *reinterpret_cast<u32x4*>(&Bs[buf][row * LDK + kv * VE]) = rb[r];
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
            // ILV: step e of every tile before step e+1, so back-to-back
            // MFMAs never chain on one accumulator
            if constexpr (ILV) {
#pragma unroll
                for (int e = 0; e < Mfma32<T>::STEPS; e++)
#pragma unroll
                    for (int i = 0; i < TM; i++)
#pragma unroll
                        for (int j = 0; j < TN; j++) Mfma32<T>::step(acc[i][j], fa[i], fb[j], e);
            } else {
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
#pragma unroll
                        for (int e = 0; e < Mfma32<T>::STEPS; e++)
                            Mfma32<T>::step(acc[i][j], fa[i], fb[j], e);
            }
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

// ---------------------------------------------------------------------------
// Pipelined variant: operand tiles are copied HBM/L2 -> LDS directly by the
// gfx950 load-to-LDS instruction (global_load_lds_dwordx4: each lane's 16
// bytes land at M0 + 16*lane), through S = 3 LDS stages, so two k-tiles of
// loads are always in flight behind the MFMAs and no VGPRs are spent on
// staging. Rows are stored unpadded (BK elements = 8 x 16-byte chunks); the
// chunk holding logical k-chunk c of row r sits at slot c ^ (r % 8), which
// keeps the 16-byte fragment reads of 8 consecutive rows on distinct banks.
// The copies are issued from inline assembly so the compiler does not track
// them: its wait-count pass would otherwise drain every outstanding load
// before some LDS reads. All ordering is explicit instead: vmcnt waits for
// this wave's own copies, then a bare s_barrier (a __syncthreads fence would
// also wait for the copies still in flight for later tiles). Every copy is
// complete before the loop exits. Requires K % BK == 0; rows past M or N read
// a clamped (valid) row whose results are never stored.
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Copy 16 bytes per lane from global memory to LDS: lane i's bytes land at
// lds + 16*i (lds is wave-uniform; it goes to M0).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void* src, lds_void_ptr lds) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0v), "v"(src)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt simm16 on gfx9: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

template <typename T, int WM, int WN, int TM, int TN, int BK>
__global__ __launch_bounds__(WM* WN * 64) void gemm_lds3_kernel(T* __restrict__ out, const T* __restrict__ A,
                                                                const T* __restrict__ W,
                                                                const T* __restrict__ bias, int M, int N,
                                                                int K, int group_m, int remap) {
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int VE = Vec<T>::N;
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    constexpr int CH = BK / VE;  // 16-byte chunks per tile row
    static_assert(CH == 8, "swizzle assumes 8 chunks (128 bytes) per tile row");
    constexpr int LA = BM * CH / 64 / NW, LB = BN * CH / 64 / NW;  // DMA instructions per wave
    static_assert(LA * 64 * NW == BM * CH && LB * 64 * NW == BN * CH, "tile/wave mismatch");
    constexpr int LPW = LA + LB;
    __shared__ __attribute__((aligned(16))) T sA0[BM * BK];
    __shared__ __attribute__((aligned(16))) T sB0[BN * BK];
    __shared__ __attribute__((aligned(16))) T sA1[BM * BK];
    __shared__ __attribute__((aligned(16))) T sB1[BN * BK];
    __shared__ __attribute__((aligned(16))) T sA2[BM * BK];
    __shared__ __attribute__((aligned(16))) T sB2[BN * BK];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;
    const int h = lane >> 5, r32 = lane & 31;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int nwg = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if (remap) pid = xcd_contiguous(pid, nwg);
    const int per_group = group_m * tiles_n;
    const int g = pid / per_group, first_m = g * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in_g = pid - g * per_group;
    const int m0 = (first_m + in_g % gsz) * BM, n0 = (in_g / gsz) * BN;

    // Per-lane source offsets (element index at k = 0) for this wave's DMA
    // instructions; chunk q of the tile = row q/8, slot q%8.
    int64_t offA[LA], offB[LB];
#pragma unroll
    for (int j = 0; j < LA; j++) {
        const int q = (wid * LA + j) * 64 + lane, row = q >> 3, lc = (q & 7) ^ (row & 7);
        offA[j] = (int64_t)min(m0 + row, M - 1) * K + lc * VE;
    }
#pragma unroll
    for (int j = 0; j < LB; j++) {
        const int q = (wid * LB + j) * 64 + lane, row = q >> 3, lc = (q & 7) ^ (row & 7);
        offB[j] = (int64_t)min(n0 + row, N - 1) * K + lc * VE;
    }
    auto issue = [&](T* sA, T* sB, int k0) {
#pragma unroll
        for (int j = 0; j < LA; j++)
            copy16_to_lds(A + offA[j] + k0, (lds_void_ptr)(sA + (wid * LA + j) * 64 * VE));
#pragma unroll
        for (int j = 0; j < LB; j++)
            copy16_to_lds(W + offB[j] + k0, (lds_void_ptr)(sB + (wid * LB + j) * 64 * VE));
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = f32x16{};

    auto compute = [&](const T* sA, const T* sB) {
#pragma unroll
        for (int kc = 0; kc < CH / 2; kc++) {
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int row = wm * TM * 32 + i * 32 + r32;
                fa[i] = *reinterpret_cast<const u32x4*>(&sA[row * BK + (((2 * kc + h) ^ (row & 7)) * VE)]);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int row = wn * TN * 32 + j * 32 + r32;
                fb[j] = *reinterpret_cast<const u32x4*>(&sB[row * BK + (((2 * kc + h) ^ (row & 7)) * VE)]);
            }
#pragma unroll
            for (int e = 0; e < Mfma32<T>::STEPS; e++)
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++) Mfma32<T>::step(acc[i][j], fa[i], fb[j], e);
        }
    };

    const int nk = K / BK;
    issue(sA0, sB0, 0);
    if (nk > 1) issue(sA1, sB1, BK);
    // One k-tile per step: wait for this tile's loads (the next tile's may
    // stay in flight), barrier, launch the tile two ahead into the stage the
    // previous step just finished reading, compute.
#define GEMM_LDS3_STEP(SA, SB, SA2, SB2, T_)            \
    {                                                      \
        const int t = (T_);                                \
        if (t + 1 < nk) wait_vmcnt<LPW>();                 \
        else wait_vmcnt<0>();                              \
        __builtin_amdgcn_s_barrier();                      \
        if (t + 2 < nk) issue(SA2, SB2, (t + 2) * BK);     \
        compute(SA, SB);                                   \
    }
    int kt = 0;
    for (; kt + 3 <= nk; kt += 3) {
        GEMM_LDS3_STEP(sA0, sB0, sA2, sB2, kt)
        GEMM_LDS3_STEP(sA1, sB1, sA0, sB0, kt + 1)
        GEMM_LDS3_STEP(sA2, sB2, sA1, sB1, kt + 2)
    }
    if (kt < nk) GEMM_LDS3_STEP(sA0, sB0, sA2, sB2, kt)
    if (kt + 1 < nk) GEMM_LDS3_STEP(sA1, sB1, sA0, sB0, kt + 1)
#undef GEMM_LDS3_STEP

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

template <typename T, int WM, int WN, int TM, int TN>
static void launch_gemm_lds3(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                             int group_m, int remap, hipStream_t s) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32, BK = Vec<T>::N * 8;
    const int nwg = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_lds3_kernel<T, WM, WN, TM, TN, BK><<<nwg, WM * WN * 64, 0, s>>>(out, A, W, bias, M, N, K,
                                                                         group_m, remap);
}

template <typename T, int WM, int WN, int TM, int TN, int BK, bool ILV = true>
static void launch_gemm_cfg(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                            int group_m, int remap, hipStream_t s) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    const int nwg = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_kernel<T, WM, WN, TM, TN, BK, ILV><<<nwg, WM * WN * 64, 0, s>>>(out, A, W, bias, M, N, K,
                                                                          group_m, remap);
}

}  // namespace gpt2
