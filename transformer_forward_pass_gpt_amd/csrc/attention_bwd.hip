// Backward of causal multi-head attention on the gfx950 matrix cores.
//
// Method: the backward of the tiled forward (derived in the optdl2025 project
// "Understand FlashAttention (II)" from "Algorithm 1" of FlashAttention): the
// probabilities are rebuilt from the scores and the saved per-row
// log-sum-exp, P = exp(S - lse), so no T x T matrix ever reaches HBM. With
// D_q = sum_d dO[q,d] O[q,d] (= sum_j P[q,j] dP[q,j]):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dK = dS^T Q / sqrt(hs),
//   dQ = dS K / sqrt(hs).
// Two kernels, so every output has exactly one writer and a fixed summation
// order (no atomics): one walks, per 64-key tile, the query tiles at or after
// it and accumulates dK and dV; the other walks, per 64-query tile, the key
// tiles up to it and accumulates dQ (recomputing S and dP). Key tiles above
// the diagonal are never visited.
//
// fp32 runs every product on v_mfma_f32_32x32x2_f32; bf16 on
// v_mfma_f32_32x32x16_bf16 with its own operand layouts (below).
//
// Register layouts (32x32 MFMA: lane (h, r32) supplies A[r32][k-slot h] and
// B[k-slot h][r32]; accumulator register v holds row 8*(v/4) + 4*h + v%4,
// column r32):
//  - head-dim contractions (S, dP) use k-slot h of step i <-> head dim
//    (HS/2)*h + i, so a lane's operand is one contiguous run of its row;
//  - the query (key) contractions of dV, dK (dQ) take the probabilities
//    straight from the accumulator of S (S^T): step v pairs slot h with
//    row 8*(v/4) + 4*h + v%4, and the other operand is read from LDS at that
//    row, column r32.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace gpt2 {

static constexpr int kAB = 64;  // queries / keys per tile

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Widen one 16-byte vector of T into VE consecutive floats of LDS.
__device__ __forceinline__ void put_f32(float* dst, const u32x4& v, const float*) {
    *reinterpret_cast<u32x4*>(dst) = v;
}
__device__ __forceinline__ void put_f32(float* dst, const u32x4& v, const bf16*) {
    float f[8];
    unpack_vec<bf16>(v, f);
    *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// A lane's HS/2 contiguous elements of one head row, as fp32 registers
// (zeros for rows past the sequence).
template <typename T, int KH>
__device__ __forceinline__ void load_half_row(float (&f)[KH], const T* p, bool ok) {
    constexpr int VE = Vec<T>::N;
#pragma unroll
    for (int i = 0; i < KH / VE; i++) {
        float t[VE];
        if (ok) load_vec(p + i * VE, t);
#pragma unroll
        for (int j = 0; j < VE; j++) f[i * VE + j] = ok ? t[j] : 0.f;
    }
}

// Four consecutive head dims of one row, scaled, stored to T.
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    u32x2 pk = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2*>(p) = pk;
}

// D[b,h,t] = sum_d dO[b,t,h*HS+d] O[b,t,h*HS+d]; one thread per (b,t,h).
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(float* __restrict__ D, const T* __restrict__ dout,
                                                           const T* __restrict__ out, int B, int Tn, int C, int NH) {
    constexpr int VE = Vec<T>::N;
    const int64_t i = blockIdx.x * 256LL + threadIdx.x;
    if (i >= (int64_t)B * Tn * NH) return;
    const int hd = (int)(i % NH);
    const int64_t bt = i / NH;
    const int b = (int)(bt / Tn), t = (int)(bt % Tn);
    const T* o = out + bt * C + hd * HS;
    const T* d = dout + bt * C + hd * HS;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < HS; c += VE) {
        float x[VE], y[VE];
        load_vec(o + c, x);
        load_vec(d + c, y);
#pragma unroll
        for (int j = 0; j < VE; j++) s += x[j] * y[j];
    }
    D[((int64_t)b * NH + hd) * Tn + t] = s;
}

// ------------------------------------------------------------------ dK, dV
// Workgroup (b*NH + h, key tile kb), 4 wavefronts: wave (kc, par) owns keys
// kb*64 + 32*kc .. +31 and, of every 64-query tile, the 32 queries 32*par..;
// the two parities' dK, dV are added through LDS at the end (par 0 + par 1).
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(T* __restrict__ dqkv, const T* __restrict__ qkv,
                                                           const T* __restrict__ dout, const float* __restrict__ lse,
                                                           const float* __restrict__ Dg, int Tn, int C, int NH,
                                                           float sl2, float scale) {
    constexpr int VE = Vec<T>::N;
    constexpr int KH = HS / 2;             // head-dim contraction steps
    constexpr int DT = (HS + 31) / 32;     // 32-row tiles of dK^T, dV^T
    constexpr int LD = HS + 4;             // fp32 LDS row stride
    constexpr int TILE = kAB * LD;
    constexpr int BUF = 2 * TILE + 2 * kAB;  // Q, dO, lse2, D
    constexpr int RV = HS / VE;              // 16-byte vectors per head row
    constexpr int NV = (kAB * RV + 255) / 256;
    static_assert(KH % VE == 0, "head size");
    __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int kc = wid & 1, par = wid >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int kb = blockIdx.y;  // dispatched in order: tile 0 (the longest walk) first
    const int k0 = kb * kAB + kc * 32, key = k0 + r32;
    const int64_t rs = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tn * rs;
    const T* dbase = dout + (int64_t)b * Tn * C + hd * HS;
    const float* lrow = lse + (int64_t)bh * Tn;
    const float* drow = Dg + (int64_t)bh * Tn;
    const float L2E = 1.4426950408889634f;

    // this lane's key row as the B operand of S = Q K^T and dP = dO V^T
    float kf[KH], vf[KH];
    load_half_row<T, KH>(kf, base + (int64_t)min(key, Tn - 1) * rs + C + hd * HS + KH * h, key < Tn);
    load_half_row<T, KH>(vf, base + (int64_t)min(key, Tn - 1) * rs + 2 * C + hd * HS + KH * h, key < Tn);

    u32x4 rq[NV], rd[NV];
    float rl = 0.f, rD = 0.f;
    auto gload = [&](int qt) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int li = tid + i * 256, r = li / RV, cv = li % RV, q = min(qt * kAB + r, Tn - 1);
            rq[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)q * rs + hd * HS + cv * VE);
            rd[i] = *reinterpret_cast<const u32x4*>(dbase + (int64_t)q * C + cv * VE);
        }
        const int q = min(qt * kAB + (tid & 63), Tn - 1);
        rl = lrow[q];
        rD = drow[q];
    };
    auto sstore = [&](int buf, int qt) {
        float* sQ = smem + buf * BUF;
        float* sO = sQ + TILE;
        float* sL = sO + TILE;
        float* sD = sL + kAB;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int li = tid + i * 256, r = li / RV, cv = li % RV;
            if (li < kAB * RV) {
                const bool ok = qt * kAB + r < Tn;
                const u32x4 z = {0u, 0u, 0u, 0u};
                put_f32(sQ + r * LD + cv * VE, ok ? rq[i] : z, (const T*)nullptr);
                put_f32(sO + r * LD + cv * VE, ok ? rd[i] : z, (const T*)nullptr);
            }
        }
        if (tid < 64) {
            const bool ok = qt * kAB + tid < Tn;
            sL[tid] = ok ? rl * L2E : 0.f;
            sD[tid] = ok ? rD : 0.f;
        }
    };

    f32x16 dv[DT], dk[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) dv[dt] = dk[dt] = f32x16{};

    auto compute = [&](int buf, int qt) {
        const float* sQ = smem + buf * BUF;
        const float* sO = sQ + TILE;
        const float* sL = sO + TILE;
        const float* sD = sL + kAB;
        const int qb = qt * kAB + par * 32;  // this wave's queries qb .. qb+31
        if (qb + 31 < k0) return;           // every query precedes every key: P = 0
        f32x16 s = f32x16{}, dp = f32x16{};
        const float* qrow = sQ + (par * 32 + r32) * LD + KH * h;
        const float* orow = sO + (par * 32 + r32) * LD + KH * h;
#pragma unroll
        for (int i = 0; i < KH; i += 4) {
            const float4 qa = *reinterpret_cast<const float4*>(qrow + i);
            const float4 oa = *reinterpret_cast<const float4*>(orow + i);
            s = mfma_f32(qa.x, kf[i], s);
            dp = mfma_f32(oa.x, vf[i], dp);
            s = mfma_f32(qa.y, kf[i + 1], s);
            dp = mfma_f32(oa.y, vf[i + 1], dp);
            s = mfma_f32(qa.z, kf[i + 2], s);
            dp = mfma_f32(oa.z, vf[i + 2], dp);
            s = mfma_f32(qa.w, kf[i + 3], s);
            dp = mfma_f32(oa.w, vf[i + 3], dp);
        }
        // P and dS; register v: query qb + m, m = 8*(v/4) + 4h + v%4; key k0 + r32
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3), q = qb + m;
            const bool on = key <= q && q < Tn;
            const float p = on ? __builtin_amdgcn_exp2f(s[v] * sl2 - sL[par * 32 + m]) : 0.f;
            s[v] = p;
            dp[v] = p * (dp[v] - sD[par * 32 + m]);
        }
        // dV^T += dO^T P, dK^T += Q^T dS: A = (dO | Q)[query m][head dim dt*32 + r32]
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = par * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const int d = dt * 32 + r32;
                const float ao = d < HS ? sO[m * LD + min(d, HS - 1)] : 0.f;
                const float aq = d < HS ? sQ[m * LD + min(d, HS - 1)] : 0.f;
                dv[dt] = mfma_f32(ao, s[v], dv[dt]);
                dk[dt] = mfma_f32(aq, dp[v], dk[dt]);
            }
        }
    };

    const int nqt = (Tn + kAB - 1) / kAB;
    gload(kb);
    sstore(0, kb);
    __syncthreads();
    for (int qt = kb; qt < nqt; qt++) {
        const int cur = (qt - kb) & 1;
        if (qt + 1 < nqt) gload(qt + 1);
        compute(cur, qt);
        if (qt + 1 < nqt) sstore(cur ^ 1, qt + 1);
        __syncthreads();
    }

    // parity merge (par 1 -> LDS -> par 0), then dK (scaled) and dV
    float* mg = smem + kc * (2 * DT * 16 * 64);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                mg[((2 * dt) * 16 + v) * 64 + lane] = dv[dt][v];
                mg[((2 * dt + 1) * 16 + v) * 64 + lane] = dk[dt][v];
            }
    }
    __syncthreads();
    if (par == 1 || key >= Tn) return;
    T* drow_k = dqkv + ((int64_t)b * Tn + key) * rs + C + hd * HS;
    T* drow_v = drow_k + C;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            if (d0 < HS) {
                float x[4], y[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int v = 4 * g + e;
                    x[e] = dv[dt][v] + mg[((2 * dt) * 16 + v) * 64 + lane];
                    y[e] = (dk[dt][v] + mg[((2 * dt + 1) * 16 + v) * 64 + lane]) * scale;
                }
                store4(drow_v + d0, x[0], x[1], x[2], x[3]);
                store4(drow_k + d0, y[0], y[1], y[2], y[3]);
            }
        }
}

// --------------------------------------------------------------------- dQ
// Workgroup (b*NH + h, query tile), 4 wavefronts: wave (qc, par) owns queries
// qt*64 + 32*qc .. +31 and, of every 64-key tile, the 32 keys 32*par..; the
// parities' dQ are added through LDS at the end.
template <typename T, int HS>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(T* __restrict__ dqkv, const T* __restrict__ qkv,
                                                          const T* __restrict__ dout, const float* __restrict__ lse,
                                                          const float* __restrict__ Dg, int Tn, int C, int NH,
                                                          float sl2, float scale) {
    constexpr int VE = Vec<T>::N;
    constexpr int KH = HS / 2;
    constexpr int DT = (HS + 31) / 32;
    constexpr int LD = HS + 4;
    constexpr int TILE = kAB * LD;
    constexpr int BUF = 2 * TILE;  // K, V
    constexpr int RV = HS / VE;
    constexpr int NV = (kAB * RV + 255) / 256;
    __shared__ __attribute__((aligned(16))) float smem[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int qc = wid & 1, par = wid >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int qt = gridDim.y - 1 - blockIdx.y;  // the last (longest) query tiles first
    const int qw = qt * kAB + qc * 32, q = qw + r32;
    const int64_t rs = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tn * rs;
    const float L2E = 1.4426950408889634f;

    float qf[KH], df[KH];
    load_half_row<T, KH>(qf, base + (int64_t)min(q, Tn - 1) * rs + hd * HS + KH * h, q < Tn);
    load_half_row<T, KH>(df, dout + ((int64_t)b * Tn + min(q, Tn - 1)) * C + hd * HS + KH * h, q < Tn);
    const float l2 = q < Tn ? lse[(int64_t)bh * Tn + q] * L2E : 0.f;
    const float Dq = q < Tn ? Dg[(int64_t)bh * Tn + q] : 0.f;

    u32x4 rk[NV], rv[NV];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int li = tid + i * 256, r = li / RV, cv = li % RV, k = min(kt * kAB + r, Tn - 1);
            rk[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)k * rs + C + hd * HS + cv * VE);
            rv[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)k * rs + 2 * C + hd * HS + cv * VE);
        }
    };
    auto sstore = [&](int buf, int kt) {
        float* sK = smem + buf * BUF;
        float* sV = sK + TILE;
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int li = tid + i * 256, r = li / RV, cv = li % RV;
            if (li < kAB * RV) {
                const bool ok = kt * kAB + r < Tn;
                const u32x4 z = {0u, 0u, 0u, 0u};
                put_f32(sK + r * LD + cv * VE, ok ? rk[i] : z, (const T*)nullptr);
                put_f32(sV + r * LD + cv * VE, ok ? rv[i] : z, (const T*)nullptr);
            }
        }
    };

    f32x16 dq[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) dq[dt] = f32x16{};

    auto compute = [&](int buf, int kt) {
        const float* sK = smem + buf * BUF;
        const float* sV = sK + TILE;
        const int kbse = kt * kAB + par * 32;  // this wave's keys kbse .. kbse+31
        if (kbse > qw + 31) return;            // every key follows every query
        f32x16 s = f32x16{}, dp = f32x16{};
        const float* krow = sK + (par * 32 + r32) * LD + KH * h;
        const float* vrow = sV + (par * 32 + r32) * LD + KH * h;
#pragma unroll
        for (int i = 0; i < KH; i += 4) {
            const float4 ka = *reinterpret_cast<const float4*>(krow + i);
            const float4 va = *reinterpret_cast<const float4*>(vrow + i);
            s = mfma_f32(ka.x, qf[i], s);
            dp = mfma_f32(va.x, df[i], dp);
            s = mfma_f32(ka.y, qf[i + 1], s);
            dp = mfma_f32(va.y, df[i + 1], dp);
            s = mfma_f32(ka.z, qf[i + 2], s);
            dp = mfma_f32(va.z, df[i + 2], dp);
            s = mfma_f32(ka.w, qf[i + 3], s);
            dp = mfma_f32(va.w, df[i + 3], dp);
        }
        // S^T register v: key kbse + m, m = 8*(v/4) + 4h + v%4; query q
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            const bool on = kbse + m <= q && q < Tn;
            const float p = on ? __builtin_amdgcn_exp2f(s[v] * sl2 - l2) : 0.f;
            dp[v] = p * (dp[v] - Dq);
        }
        // dQ^T += K^T dS^T: A = K[key m][head dim dt*32 + r32]
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = par * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const int d = dt * 32 + r32;
                const float a = d < HS ? sK[m * LD + min(d, HS - 1)] : 0.f;
                dq[dt] = mfma_f32(a, dp[v], dq[dt]);
            }
        }
    };

    const int nkt = qt + 1;
    gload(0);
    sstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        compute(cur, kt);
        if (kt + 1 < nkt) sstore(cur ^ 1, kt + 1);
        __syncthreads();
    }

    float* mg = smem + qc * (DT * 16 * 64);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mg[(dt * 16 + v) * 64 + lane] = dq[dt][v];
    }
    __syncthreads();
    if (par == 1 || q >= Tn) return;
    T* drow = dqkv + ((int64_t)b * Tn + q) * rs + hd * HS;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            if (d0 < HS) {
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int v = 4 * g + e;
                    x[e] = (dq[dt][v] + mg[(dt * 16 + v) * 64 + lane]) * scale;
                }
                store4(drow + d0, x[0], x[1], x[2], x[3]);
            }
        }
}

// ------------------------------------------------------------------ bf16
// The same two walks on v_mfma_f32_32x32x16_bf16 (lane (h, r32) supplies
// A[r32][8h..8h+7] and B[8h..8h+7][r32]). Operand tiles stay bf16 in LDS:
//  - head-dim contractions (S, dP): step i covers head dims 16i..16i+15, a
//    lane's 8 values are one 16-byte run of a row-major tile row;
//  - the query (key) contractions take P and dS from the accumulator: step j
//    covers accumulator registers 8j..8j+7, i.e. rows 16j + 8(u/4) + 4h + u%4
//    for the lane's slots u = 0..7. The other operand is kept TRANSPOSED in
//    LDS ([head dim][row]) with bits 2 and 3 of the row index swapped inside
//    each 16, which puts exactly those 8 rows in slots 16j + 8h .. +7: one
//    16-byte read. P and dS are rounded to bf16 for these products, as the
//    forward rounds P before P.V.
__device__ __forceinline__ int bwd_slot(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// accumulator registers 8j..8j+7 of one lane, as 8 bf16 (the B operand above)
__device__ __forceinline__ u32x4 pack8(const f32x16& x, int j) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; e++) r[e] = pack_bf16x2(x[8 * j + 2 * e], x[8 * j + 2 * e + 1]);
    return r;
}

// Staging of one 64-row tile of a head (rows r0 .. r0+63 of a [rows, ld]
// tensor, head columns col .. col+HS-1): thread item (quad kq, chunk cv)
// holds rows 4kq..4kq+3 x 8 head dims; it writes them row-major (rows of
// LDR) and, when tr is given, transposed with permuted slots (rows of LDT).
template <int HS>
struct QuadTile {
    static constexpr int LDR = HS + 8, LDT = kAB + 8;
    static constexpr int ITEMS = 16 * (HS / 8);  // quads x chunks
    u32x4 v[4];
    __device__ __forceinline__ void load(const bf16* base, int64_t ld, int r0, int Tn, int item) {
        const int kq = item & 15, cv = item >> 4;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = r0 + 4 * kq + e;
            const u32x4 x = *reinterpret_cast<const u32x4*>(base + (int64_t)min(r, Tn - 1) * ld + cv * 8);
            v[e] = r < Tn ? x : z;
        }
    }
    __device__ __forceinline__ void store(bf16* row, bf16* tr, int item) const {
        const int kq = item & 15, cv = item >> 4;
#pragma unroll
        for (int e = 0; e < 4; e++) *reinterpret_cast<u32x4*>(row + (4 * kq + e) * LDR + cv * 8) = v[e];
        if (tr) {
            const int slot = bwd_slot(4 * kq);
#pragma unroll
            for (int d = 0; d < 8; d++) {
                const int w = d >> 1, sh = 16 * (d & 1);
                const uint32_t a0 = (v[0][w] >> sh) & 0xffffu, a1 = (v[1][w] >> sh) & 0xffffu;
                const uint32_t a2 = (v[2][w] >> sh) & 0xffffu, a3 = (v[3][w] >> sh) & 0xffffu;
                const u32x2 col = {a0 | (a1 << 16), a2 | (a3 << 16)};
                *reinterpret_cast<u32x2*>(tr + (cv * 8 + d) * LDT + slot) = col;
            }
        }
    }
};

// dK, dV (bf16): workgroup and wave roles as attn_bwd_dkv_kernel.
template <int HS>
__global__ __launch_bounds__(256) void attn_bwd_dkv_bf16_kernel(bf16* __restrict__ dqkv, const bf16* __restrict__ qkv,
                                                                const bf16* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                const float* __restrict__ Dg, int Tn, int C, int NH,
                                                                float sl2, float scale) {
    using QT = QuadTile<HS>;
    constexpr int LDR = QT::LDR, LDT = QT::LDT;
    constexpr int KS = HS / 16;          // 16-deep head-dim steps
    constexpr int DT = (HS + 31) / 32;   // 32-row tiles of dK^T, dV^T
    constexpr int RT = kAB * LDR, TT = HS * LDT;
    constexpr int BUF = 2 * RT + 2 * TT + 4 * kAB;  // Qr, Or, Qt, Ot (bf16) + lse2, D (fp32 = 2 bf16 each)
    static_assert(HS % 16 == 0, "head size");
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int kc = wid & 1, par = wid >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int kb = blockIdx.y;
    const int k0 = kb * kAB + kc * 32, key = k0 + r32;
    const int64_t rs = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * Tn * rs;
    const bf16* dbase = dout + (int64_t)b * Tn * C + hd * HS;
    const float* lrow = lse + (int64_t)bh * Tn;
    const float* drow = Dg + (int64_t)bh * Tn;
    const float L2E = 1.4426950408889634f;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    // this lane's key and value row: B operands of S = Q K^T and dP = dO V^T
    u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int i = 0; i < KS; i++) {
        const bf16* kr = base + (int64_t)min(key, Tn - 1) * rs + C + hd * HS + 16 * i + 8 * h;
        const u32x4 a = *reinterpret_cast<const u32x4*>(kr);
        const u32x4 c = *reinterpret_cast<const u32x4*>(kr + C);
        kf[i] = key < Tn ? a : z4;
        vf[i] = key < Tn ? c : z4;
    }

    // staging: threads 0..127 the Q tile, 128..255 the dO tile
    const int which = tid >> 7, item = tid & 127;
    const bool stager = item < QT::ITEMS;
    QT st;
    float rl = 0.f, rD = 0.f;
    const bf16* src = which ? dbase : base + hd * HS;
    const int64_t ld = which ? (int64_t)C : rs;
    auto gload = [&](int qt) {
        // unconditional (idle items reload item 0): no load behind a branch
        st.load(src, ld, qt * kAB, Tn, stager ? item : 0);
        const int q = min(qt * kAB + (tid & 63), Tn - 1);
        rl = lrow[q];
        rD = drow[q];
    };
    auto sstore = [&](int buf, int qt) {
        bf16* b0 = smem + buf * BUF;
        if (stager) st.store(b0 + which * RT, b0 + 2 * RT + which * TT, item);
        float* sL = reinterpret_cast<float*>(b0 + 2 * RT + 2 * TT);
        if (tid < 64) {
            const bool ok = qt * kAB + tid < Tn;
            sL[tid] = ok ? rl * L2E : 0.f;
            sL[kAB + tid] = ok ? rD : 0.f;
        }
    };

    f32x16 dv[DT], dk[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) dv[dt] = dk[dt] = f32x16{};

    auto compute = [&](int buf, int qt) {
        const bf16* sQr = smem + buf * BUF;
        const bf16* sOr = sQr + RT;
        const bf16* sQt = sQr + 2 * RT;
        const bf16* sOt = sQt + TT;
        const float* sL = reinterpret_cast<const float*>(sQr + 2 * RT + 2 * TT);
        const float* sD = sL + kAB;
        const int qb = qt * kAB + par * 32;
        if (qb + 31 < k0) return;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int i = 0; i < KS; i++) {
            const u32x4 qa = *reinterpret_cast<const u32x4*>(sQr + (par * 32 + r32) * LDR + 16 * i + 8 * h);
            const u32x4 oa = *reinterpret_cast<const u32x4*>(sOr + (par * 32 + r32) * LDR + 16 * i + 8 * h);
            s = mfma_bf16(qa, kf[i], s);
            dp = mfma_bf16(oa, vf[i], dp);
        }
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3), q = qb + m;
            const bool on = key <= q && q < Tn;
            const float p = on ? __builtin_amdgcn_exp2f(s[v] * sl2 - sL[par * 32 + m]) : 0.f;
            s[v] = p;
            dp[v] = p * (dp[v] - sD[par * 32 + m]);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const u32x4 pb = pack8(s, j), sb = pack8(dp, j);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const int d = dt * 32 + r32;
                const int off = min(d, HS - 1) * LDT + par * 32 + 16 * j + 8 * h;
                const u32x4 ao = *reinterpret_cast<const u32x4*>(sOt + off);
                const u32x4 aq = *reinterpret_cast<const u32x4*>(sQt + off);
                dv[dt] = mfma_bf16(d < HS ? ao : z4, pb, dv[dt]);
                dk[dt] = mfma_bf16(d < HS ? aq : z4, sb, dk[dt]);
            }
        }
    };

    const int nqt = (Tn + kAB - 1) / kAB;
    gload(kb);
    sstore(0, kb);
    __syncthreads();
    for (int qt = kb; qt < nqt; qt++) {
        const int cur = (qt - kb) & 1;
        if (qt + 1 < nqt) gload(qt + 1);
        compute(cur, qt);
        if (qt + 1 < nqt) sstore(cur ^ 1, qt + 1);
        __syncthreads();
    }

    float* mg = reinterpret_cast<float*>(smem) + kc * (2 * DT * 16 * 64);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                mg[((2 * dt) * 16 + v) * 64 + lane] = dv[dt][v];
                mg[((2 * dt + 1) * 16 + v) * 64 + lane] = dk[dt][v];
            }
    }
    __syncthreads();
    if (par == 1 || key >= Tn) return;
    bf16* drow_k = dqkv + ((int64_t)b * Tn + key) * rs + C + hd * HS;
    bf16* drow_v = drow_k + C;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            if (d0 < HS) {
                float x[4], y[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int v = 4 * g + e;
                    x[e] = dv[dt][v] + mg[((2 * dt) * 16 + v) * 64 + lane];
                    y[e] = (dk[dt][v] + mg[((2 * dt + 1) * 16 + v) * 64 + lane]) * scale;
                }
                store4(drow_v + d0, x[0], x[1], x[2], x[3]);
                store4(drow_k + d0, y[0], y[1], y[2], y[3]);
            }
        }
}

// dQ (bf16): workgroup and wave roles as attn_bwd_dq_kernel.
template <int HS>
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_kernel(bf16* __restrict__ dqkv, const bf16* __restrict__ qkv,
                                                               const bf16* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ Dg, int Tn, int C, int NH,
                                                               float sl2, float scale) {
    using QT = QuadTile<HS>;
    constexpr int LDR = QT::LDR, LDT = QT::LDT;
    constexpr int KS = HS / 16;
    constexpr int DT = (HS + 31) / 32;
    constexpr int RT = kAB * LDR, TT = HS * LDT;
    constexpr int BUF = 2 * RT + TT;  // Kr, Vr, Kt
    constexpr int MERGE = 2 * DT * 16 * 64 * 2;  // bf16 units of the fp32 parity merge
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * BUF > MERGE ? 2 * BUF : MERGE];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int qc = wid & 1, par = wid >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int qt = gridDim.y - 1 - blockIdx.y;
    const int qw = qt * kAB + qc * 32, q = qw + r32;
    const int64_t rs = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * Tn * rs;
    const float L2E = 1.4426950408889634f;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    u32x4 qf[KS], df[KS];
#pragma unroll
    for (int i = 0; i < KS; i++) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base + (int64_t)min(q, Tn - 1) * rs + hd * HS + 16 * i + 8 * h);
        const u32x4 c = *reinterpret_cast<const u32x4*>(dout + ((int64_t)b * Tn + min(q, Tn - 1)) * C + hd * HS +
                                                        16 * i + 8 * h);
        qf[i] = q < Tn ? a : z4;
        df[i] = q < Tn ? c : z4;
    }
    const float l2 = q < Tn ? lse[(int64_t)bh * Tn + q] * L2E : 0.f;
    const float Dq = q < Tn ? Dg[(int64_t)bh * Tn + q] : 0.f;

    // staging: threads 0..127 the K tile (row-major and transposed), 128..255 the V tile
    const int which = tid >> 7, item = tid & 127;
    const bool stager = item < QT::ITEMS;
    QT st;
    auto gload = [&](int kt) { st.load(base + (1 + which) * C + hd * HS, rs, kt * kAB, Tn, stager ? item : 0); };
    auto sstore = [&](int buf) {
        bf16* b0 = smem + buf * BUF;
        if (stager) st.store(b0 + which * RT, which == 0 ? b0 + 2 * RT : nullptr, item);
    };

    f32x16 dq[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) dq[dt] = f32x16{};

    auto compute = [&](int buf, int kt) {
        const bf16* sKr = smem + buf * BUF;
        const bf16* sVr = sKr + RT;
        const bf16* sKt = sKr + 2 * RT;
        const int kbse = kt * kAB + par * 32;
        if (kbse > qw + 31) return;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int i = 0; i < KS; i++) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(sKr + (par * 32 + r32) * LDR + 16 * i + 8 * h);
            const u32x4 va = *reinterpret_cast<const u32x4*>(sVr + (par * 32 + r32) * LDR + 16 * i + 8 * h);
            s = mfma_bf16(ka, qf[i], s);
            dp = mfma_bf16(va, df[i], dp);
        }
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            const bool on = kbse + m <= q && q < Tn;
            const float p = on ? __builtin_amdgcn_exp2f(s[v] * sl2 - l2) : 0.f;
            dp[v] = p * (dp[v] - Dq);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const u32x4 sb = pack8(dp, j);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const int d = dt * 32 + r32;
                const u32x4 a =
                    *reinterpret_cast<const u32x4*>(sKt + min(d, HS - 1) * LDT + par * 32 + 16 * j + 8 * h);
                dq[dt] = mfma_bf16(d < HS ? a : z4, sb, dq[dt]);
            }
        }
    };

    const int nkt = qt + 1;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nkt; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        compute(cur, kt);
        if (kt + 1 < nkt) sstore(cur ^ 1);
        __syncthreads();
    }

    float* mg = reinterpret_cast<float*>(smem) + qc * (DT * 16 * 64);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mg[(dt * 16 + v) * 64 + lane] = dq[dt][v];
    }
    __syncthreads();
    if (par == 1 || q >= Tn) return;
    bf16* drow = dqkv + ((int64_t)b * Tn + q) * rs + hd * HS;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            if (d0 < HS) {
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int v = 4 * g + e;
                    x[e] = (dq[dt][v] + mg[(dt * 16 + v) * 64 + lane]) * scale;
                }
                store4(drow + d0, x[0], x[1], x[2], x[3]);
            }
        }
}

// ---------------------------------------------------------- bf16, hs = 64
// The same two walks at head size 64 (GPT-2 small and medium) with the
// forward kernel's operand machinery: every 64-row operand tile goes from
// HBM/L2 to LDS by load-to-LDS copies (no VGPR staging), twice, in two chunk
// permutations of its 128-byte rows: for the row reads of the head-dim
// contractions (S, dP: slot = chunk ^ ((row/2) % 8), conflict-free 16-row
// fragment reads), and for the transposing reads (ds_read_b64_tr_b16) that
// give the query / key contractions their transposed operand (slot = chunk ^
// 4*((row/2) % 2)): in each 16-lane group lane 4j+q addresses 4 head dims of
// row j, lane i receives head dim i of rows 0..3, so two reads give a lane the
// 8 rows 16j' + 4h + 0..3 and 16j' + 8 + 4h + 0..3 that pack8 takes from the
// accumulator. Two stages: tile t+1 lands while tile t is multiplied. Rows
// past the sequence copy its last row (finite; their P and dS are 0).
namespace bwd64 {
constexpr int HS = 64, TILE = kAB * HS;  // one 64 x 64 bf16 operand tile
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

// Per-lane copy offsets (elements, inside the head's row) of the two 8-row
// copy instructions of wave wid: rows 16 wid + 8i + lane/8, LDS slot lane % 8.
struct CopyRows {
    int row[2], offr[2], offt[2];
    __device__ __forceinline__ CopyRows(int wid, int lane) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            row[i] = 16 * wid + 8 * i + (lane >> 3);
            offr[i] = ((lane & 7) ^ ((row[i] >> 1) & 7)) * 8;
            offt[i] = ((lane & 7) ^ (4 * ((row[i] >> 1) & 1))) * 8;
        }
    }
};

// Copy rows r0 .. r0+63 of a [rows, ld] tensor's head columns (src points at
// the head's first column) into the row-read tile tr and, if tt, the
// transposing-read tile tt; rows clamped to the sequence.
__device__ __forceinline__ void copy_tile(const CopyRows& cr, const bf16* src, int64_t ld, int r0, int Tn, int wid,
                                          bf16* tr, bf16* tt) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const bf16* rp = src + (int64_t)min(r0 + cr.row[i], Tn - 1) * ld;
        copy16_to_lds(rp + cr.offr[i], (lds_void_ptr)(tr + (16 * wid + 8 * i) * HS));
        if (tt) copy16_to_lds(rp + cr.offt[i], (lds_void_ptr)(tt + (16 * wid + 8 * i) * HS));
    }
}

// Row-read fragment: row `row` (a multiple of 16 plus r32) of a row-read tile,
// head dims 16i + 8h .. +7.
__device__ __forceinline__ u32x4 row_frag(const bf16* t, int row, int i, int h) {
    return *reinterpret_cast<const u32x4*>(t + row * HS + ((2 * i + h) ^ ((row >> 1) & 7)) * 8);
}

// Transposed fragment of a transposing-read tile: A[head dim 32 dt + r32][k-slot]
// with k-slots = rows r0 + 16j' pattern above (r0 a multiple of 16).
struct TrRead {
    int vbase[2];
    __device__ __forceinline__ TrRead(int lane) {
        const int h = lane >> 5, r32 = lane & 31;
        const int gj = (lane & 15) >> 2, gq = lane & 3;
        const int vy = (gj >> 1) & 1, vx = 2 * (r32 >> 4) + (gq >> 1);
#pragma unroll
        for (int dt = 0; dt < 2; dt++) vbase[dt] = (4 * h + gj) * HS + (4 * (dt ^ vy) + vx) * 8 + (gq & 1) * 4;
    }
    __device__ __forceinline__ u32x4 operator()(const bf16* t, int r0, int dt) const {
        const lds_v4s_ptr p = (lds_v4s_ptr)t;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p + (vbase[dt] + r0 * HS) / 4);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p + (vbase[dt] + (r0 + 8) * HS) / 4);
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
};
}  // namespace bwd64

// dK, dV (bf16, hs 64): workgroup and wave roles as attn_bwd_dkv_kernel.
__global__ __launch_bounds__(256) void attn_bwd_dkv_bf16_d64_kernel(bf16* __restrict__ dqkv,
                                                                    const bf16* __restrict__ qkv,
                                                                    const bf16* __restrict__ dout,
                                                                    const float* __restrict__ lse,
                                                                    const float* __restrict__ Dg, int Tn, int C,
                                                                    int NH, float sl2, float scale) {
    using namespace bwd64;
    constexpr int DT = 2;
    constexpr int STAGE = 4 * TILE + 4 * kAB;  // Q, Q^T-read, dO, dO^T-read tiles; lse2, D (fp32 = 2 bf16 each)
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kc = wid & 1, par = wid >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int kb = blockIdx.y;
    const int k0 = kb * kAB + kc * 32, key = k0 + r32;
    const int64_t rs = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * Tn * rs;
    const bf16* qsrc = base + hd * HS;
    const bf16* dsrc = dout + (int64_t)b * Tn * C + hd * HS;
    const float* lrow = lse + (int64_t)bh * Tn;
    const float* drow = Dg + (int64_t)bh * Tn;
    const float L2E = 1.4426950408889634f;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    // this lane's key and value row: B operands of S = Q K^T and dP = dO V^T
    u32x4 kf[4], vf[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const bf16* kr = base + (int64_t)min(key, Tn - 1) * rs + C + hd * HS + 16 * i + 8 * h;
        const u32x4 a = *reinterpret_cast<const u32x4*>(kr);
        const u32x4 c = *reinterpret_cast<const u32x4*>(kr + C);
        kf[i] = key < Tn ? a : z4;
        vf[i] = key < Tn ? c : z4;
    }

    const CopyRows cr(wid, lane);
    const TrRead trr(lane);
    float rl = 0.f, rD = 0.f;
    auto issue = [&](int st, int qt) {
        bf16* s0 = smem + st * STAGE;
        copy_tile(cr, qsrc, rs, qt * kAB, Tn, wid, s0, s0 + TILE);
        copy_tile(cr, dsrc, C, qt * kAB, Tn, wid, s0 + 2 * TILE, s0 + 3 * TILE);
        if (tid < kAB) {  // after the copies: the compiler's wait for these never counts them
            const int q = min(qt * kAB + tid, Tn - 1);
            rl = lrow[q];
            rD = drow[q];
        }
    };
    auto put_stats = [&](int st, int qt) {
        float* sL = reinterpret_cast<float*>(smem + st * STAGE + 4 * TILE);
        if (tid < kAB) {
            const bool ok = qt * kAB + tid < Tn;
            sL[tid] = ok ? rl * L2E : 0.f;
            sL[kAB + tid] = ok ? rD : 0.f;
        }
    };

    f32x16 dv[DT], dk[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) dv[dt] = dk[dt] = f32x16{};

    auto compute = [&](int st, int qt) {
        const bf16* sQ = smem + st * STAGE;
        const bf16* sQt = sQ + TILE;
        const bf16* sO = sQ + 2 * TILE;
        const bf16* sOt = sQ + 3 * TILE;
        const float* sL = reinterpret_cast<const float*>(sQ + 4 * TILE);
        const float* sD = sL + kAB;
        const int qb = qt * kAB + par * 32;
        if (qb + 31 < k0) return;  // every query precedes every key: P = 0
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            s = mfma_bf16(row_frag(sQ, par * 32 + r32, i, h), kf[i], s);
            dp = mfma_bf16(row_frag(sO, par * 32 + r32, i, h), vf[i], dp);
        }
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3), q = qb + m;
            const bool on = key <= q && q < Tn;
            const float p = on ? __builtin_amdgcn_exp2f(s[v] * sl2 - sL[par * 32 + m]) : 0.f;
            s[v] = p;
            dp[v] = p * (dp[v] - sD[par * 32 + m]);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const u32x4 pb = pack8(s, j), sb = pack8(dp, j);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                dv[dt] = mfma_bf16(trr(sOt, par * 32 + 16 * j, dt), pb, dv[dt]);
                dk[dt] = mfma_bf16(trr(sQt, par * 32 + 16 * j, dt), sb, dk[dt]);
            }
        }
    };

    const int nqt = (Tn + kAB - 1) / kAB;
    issue(0, kb);
    put_stats(0, kb);
    for (int qt = kb; qt < nqt; qt++) {
        const int st = (qt - kb) & 1;
        // this wave's copies of tile qt have landed (and its reads of the
        // other stage are done); after the barrier every wave's have
        wait_vmcnt_lds<0>();
        __builtin_amdgcn_s_barrier();
        if (qt + 1 < nqt) issue(st ^ 1, qt + 1);
        compute(st, qt);
        if (qt + 1 < nqt) put_stats(st ^ 1, qt + 1);
    }
    wait_vmcnt_lds<0>();
    __builtin_amdgcn_s_barrier();  // every wave is done with the stages before the merge reuses them

    float* mg = reinterpret_cast<float*>(smem) + kc * (2 * DT * 16 * 64);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                mg[((2 * dt) * 16 + v) * 64 + lane] = dv[dt][v];
                mg[((2 * dt + 1) * 16 + v) * 64 + lane] = dk[dt][v];
            }
    }
    __syncthreads();
    if (par == 1 || key >= Tn) return;
    bf16* drow_k = dqkv + ((int64_t)b * Tn + key) * rs + C + hd * HS;
    bf16* drow_v = drow_k + C;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            float x[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int v = 4 * g + e;
                x[e] = dv[dt][v] + mg[((2 * dt) * 16 + v) * 64 + lane];
                y[e] = (dk[dt][v] + mg[((2 * dt + 1) * 16 + v) * 64 + lane]) * scale;
            }
            store4(drow_v + d0, x[0], x[1], x[2], x[3]);
            store4(drow_k + d0, y[0], y[1], y[2], y[3]);
        }
}

// dQ (bf16, hs 64): workgroup and wave roles as attn_bwd_dq_kernel.
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16_d64_kernel(bf16* __restrict__ dqkv,
                                                                   const bf16* __restrict__ qkv,
                                                                   const bf16* __restrict__ dout,
                                                                   const float* __restrict__ lse,
                                                                   const float* __restrict__ Dg, int Tn, int C,
                                                                   int NH, float sl2, float scale) {
    using namespace bwd64;
    constexpr int DT = 2;
    constexpr int STAGE = 3 * TILE;  // K, K^T-read, V tiles
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qc = wid & 1, par = wid >> 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int qt = gridDim.y - 1 - blockIdx.y;  // the last (longest) query tiles first
    const int qw = qt * kAB + qc * 32, q = qw + r32;
    const int64_t rs = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * Tn * rs;
    const float L2E = 1.4426950408889634f;
    const u32x4 z4 = {0u, 0u, 0u, 0u};

    u32x4 qf[4], df[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base + (int64_t)min(q, Tn - 1) * rs + hd * HS + 16 * i + 8 * h);
        const u32x4 c = *reinterpret_cast<const u32x4*>(dout + ((int64_t)b * Tn + min(q, Tn - 1)) * C + hd * HS +
                                                        16 * i + 8 * h);
        qf[i] = q < Tn ? a : z4;
        df[i] = q < Tn ? c : z4;
    }
    const float l2 = q < Tn ? lse[(int64_t)bh * Tn + q] * L2E : 0.f;
    const float Dq = q < Tn ? Dg[(int64_t)bh * Tn + q] : 0.f;

    const CopyRows cr(wid, lane);
    const TrRead trr(lane);
    auto issue = [&](int st, int kt) {
        bf16* s0 = smem + st * STAGE;
        copy_tile(cr, base + C + hd * HS, rs, kt * kAB, Tn, wid, s0, s0 + TILE);
        copy_tile(cr, base + 2 * C + hd * HS, rs, kt * kAB, Tn, wid, s0 + 2 * TILE, nullptr);
    };

    f32x16 dq[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) dq[dt] = f32x16{};

    auto compute = [&](int st, int kt) {
        const bf16* sK = smem + st * STAGE;
        const bf16* sKt = sK + TILE;
        const bf16* sV = sK + 2 * TILE;
        const int kbse = kt * kAB + par * 32;
        if (kbse > qw + 31) return;  // every key follows every query
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            s = mfma_bf16(row_frag(sK, par * 32 + r32, i, h), qf[i], s);
            dp = mfma_bf16(row_frag(sV, par * 32 + r32, i, h), df[i], dp);
        }
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int m = 8 * (v >> 2) + 4 * h + (v & 3);
            const bool on = kbse + m <= q && q < Tn;
            const float p = on ? __builtin_amdgcn_exp2f(s[v] * sl2 - l2) : 0.f;
            dp[v] = p * (dp[v] - Dq);
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const u32x4 sb = pack8(dp, j);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) dq[dt] = mfma_bf16(trr(sKt, par * 32 + 16 * j, dt), sb, dq[dt]);
        }
    };

    const int nkt = qt + 1;
    issue(0, 0);
    for (int kt = 0; kt < nkt; kt++) {
        const int st = kt & 1;
        wait_vmcnt_lds<0>();
        __builtin_amdgcn_s_barrier();
        if (kt + 1 < nkt) issue(st ^ 1, kt + 1);
        compute(st, kt);
    }
    wait_vmcnt_lds<0>();
    __builtin_amdgcn_s_barrier();

    float* mg = reinterpret_cast<float*>(smem) + qc * (DT * 16 * 64);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mg[(dt * 16 + v) * 64 + lane] = dq[dt][v];
    }
    __syncthreads();
    if (par == 1 || q >= Tn) return;
    bf16* drow = dqkv + ((int64_t)b * Tn + q) * rs + hd * HS;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int v = 4 * g + e;
                x[e] = (dq[dt][v] + mg[(dt * 16 + v) * 64 + lane]) * scale;
            }
            store4(drow + d0, x[0], x[1], x[2], x[3]);
        }
}

int64_t attention_backward_workspace_bytes(int B, int T, int NH) { return ((int64_t)B * NH * T * 4 + 255) & ~255LL; }

template <typename T, int HS>
static void launch_attn_bwd_hs(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse, float* D, int B,
                               int Tn, int C, int NH, hipStream_t s) {
    const float scale = 1.0f / sqrtf((float)HS);
    const float sl2 = 1.4426950408889634f * scale;
    const int64_t rows = (int64_t)B * Tn * NH;
    attn_bwd_dot_kernel<T, HS><<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(D, dout, out, B, Tn, C, NH);
    const dim3 grid(B * NH, (Tn + kAB - 1) / kAB);
    if constexpr (std::is_same<T, bf16>::value) {
        if constexpr (HS == 64) {
            attn_bwd_dkv_bf16_d64_kernel<<<grid, 256, 0, s>>>(dqkv, qkv, dout, lse, D, Tn, C, NH, sl2, scale);
            attn_bwd_dq_bf16_d64_kernel<<<grid, 256, 0, s>>>(dqkv, qkv, dout, lse, D, Tn, C, NH, sl2, scale);
        } else {
            attn_bwd_dkv_bf16_kernel<HS><<<grid, 256, 0, s>>>(dqkv, qkv, dout, lse, D, Tn, C, NH, sl2, scale);
            attn_bwd_dq_bf16_kernel<HS><<<grid, 256, 0, s>>>(dqkv, qkv, dout, lse, D, Tn, C, NH, sl2, scale);
        }
    } else {
        attn_bwd_dkv_kernel<T, HS><<<grid, 256, 0, s>>>(dqkv, qkv, dout, lse, D, Tn, C, NH, sl2, scale);
        attn_bwd_dq_kernel<T, HS><<<grid, 256, 0, s>>>(dqkv, qkv, dout, lse, D, Tn, C, NH, sl2, scale);
    }
}

template <typename T>
static void launch_attn_bwd_t(T* dqkv, const T* dout, const T* qkv, const T* out, const float* lse, float* D, int B,
                              int Tn, int C, int NH, hipStream_t s) {
    switch (C / NH) {
        case 16: launch_attn_bwd_hs<T, 16>(dqkv, dout, qkv, out, lse, D, B, Tn, C, NH, s); break;
        case 32: launch_attn_bwd_hs<T, 32>(dqkv, dout, qkv, out, lse, D, B, Tn, C, NH, s); break;
        default: launch_attn_bwd_hs<T, 64>(dqkv, dout, qkv, out, lse, D, B, Tn, C, NH, s); break;
    }
}

bool attention_backward_head_size_ok(int hs) { return hs == 16 || hs == 32 || hs == 64; }

// dqkv [B,T,3C] from dout [B,T,C], the forward's qkv, out and lse [B,NH,T];
// ws: D [B,NH,T] fp32.
int launch_attention_backward(void* dqkv, const void* dout, const void* qkv, const void* out, const float* lse,
                              int B, int T, int C, int NH, int dtype, void* ws, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_attn_bwd_t<bf16>((bf16*)dqkv, (const bf16*)dout, (const bf16*)qkv, (const bf16*)out, lse, (float*)ws,
                                B, T, C, NH, s);
    else
        launch_attn_bwd_t<float>((float*)dqkv, (const float*)dout, (const float*)qkv, (const float*)out, lse,
                                 (float*)ws, B, T, C, NH, s);
    return launch_status();
}

}  // namespace gpt2

using namespace gpt2;

extern "C" int64_t attention_backward_workspace_size(int B, int T, int C, int NH) {
    if (B < 0 || T < 0 || C <= 0 || NH <= 0 || C % NH) return GPT2_ERR_INVALID_ARGUMENT;
    return attention_backward_workspace_bytes(B, T, NH);
}

extern "C" int attention_backward(void* dqkv, const void* dout, const void* qkv, const void* out, const float* lse,
                                  int B, int T, int C, int NH, int dtype, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
    if (!valid_dtype(dtype) || B < 0 || T < 0 || C < 0 || NH <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!dqkv || !dout || !qkv || !out || !lse || !workspace || C == 0 || C % NH) return GPT2_ERR_INVALID_ARGUMENT;
    if (dqkv == qkv || dqkv == dout || dqkv == out) return GPT2_ERR_INVALID_ARGUMENT;
    if (!attention_backward_head_size_ok(C / NH) || !aligned16(dqkv) || !aligned16(dout) || !aligned16(qkv) ||
        !aligned16(out))
        return GPT2_ERR_UNSUPPORTED;
    if (workspace_bytes < attention_backward_workspace_bytes(B, T, NH)) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    return launch_attention_backward(dqkv, dout, qkv, out, lse, B, T, C, NH, dtype, workspace, (hipStream_t)stream);
}
