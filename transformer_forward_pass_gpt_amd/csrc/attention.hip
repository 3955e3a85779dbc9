// Causal multi-head self-attention, softmax fused, on the gfx950 matrix cores.
//
// Method: the tiled, exact online-softmax forward ("Algorithm 1" of
// FlashAttention, the optdl2025 project "Understand FlashAttention (I)"):
// scores and probabilities are never written to HBM; each query keeps a
// running max m and normaliser l and its output is rescaled as key blocks
// arrive. Key blocks above the diagonal are never loaded or multiplied (the
// "only doing lower triangular matmuls" item of llm.c's "State of the Union
// [April 22, 2024]", big stones list). Heads are read straight out of the
// packed qkv tensor and written straight into [B,T,C] (no permute/unpermute
// pass; optdl2025 NanoGPT project: one projection for q, k, v and head
// splitting).
//
// Mapping to 64-wide wavefronts: each wavefront owns 32 queries and computes
// the TRANSPOSED score tile S^T = K Q^T with 32x32 MFMA tiles. In the 32x32
// accumulator layout a lane owns one column (= one query) and 16 rows
// (= keys), the other half-wave owning the other 16 keys of that query. So
//  - the row max / row sum of the softmax is a per-lane loop plus ONE
//    cross-half shuffle, and
//  - the probabilities are already where the next product O^T = V^T P^T wants
//    its B operand: no data movement between the two products.
// The output O^T is likewise per-lane per-query, so the online rescale is a
// per-lane scalar multiply.
#include <math.h>

#include <type_traits>

#include <algorithm>

#include "common.h"

namespace gpt2 {

template <typename T> struct MfmaS;  // one 16-byte fragment of the contraction
template <> struct MfmaS<float> {
    static __device__ __forceinline__ void run(f32x16& acc, const u32x4& a, const u32x4& b) {
#pragma unroll
        for (int e = 0; e < 4; e++)
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]),
                                                      acc, 0, 0, 0);
    }
};
template <> struct MfmaS<bf16> {
    static __device__ __forceinline__ void run(f32x16& acc, const u32x4& a, const u32x4& b) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
};

// Lane l combined with lane l^32 (the other half-wave holds the other 16 keys
// of the same query), on gfx950's half-wave swap instead of an LDS-routed
// shuffle. max and + are commutative, so the value is the shuffle's exactly.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

static constexpr float kLazyMax = 8.0f;  // running-max slack, log2 units (probabilities < 256)
static constexpr int kBKV = 64;  // keys per LDS block

// V is kept TRANSPOSED in LDS (Vt[d][key]) so that the k-slots of the P.V
// product (which run over keys) are contiguous in LDS for every operand.
// bf16: within each group of 16 keys, bits 2 and 3 of the key index are
// swapped, which makes the 8 keys one half-wave feeds into one
// v_mfma_f32_32x32x16_bf16 k-step (keys 16ks+4h+{0..3} and 16ks+8+4h+{0..3})
// land in 8 consecutive slots: one 16-byte LDS read per operand.
__device__ __forceinline__ int vt_slot_bf16(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Workgroup: 8 wavefronts = 4 query chunks of 32 x 2 key parities. Wave
// (c, p) owns queries q0 + 32c .. +31 and the key blocks 2i + p, so the two
// waves of a query chunk split its key range; their partial (o, m, l) merge
// through LDS at the end, in a fixed order. Each iteration stages two key
// blocks (the even and the odd one); when two iterations' worth fits in LDS
// the next pair is loaded while the current one is computed.
// WPE: minimum wavefronts per SIMD the registers must allow (0: none).
// QC: 32-query chunks per workgroup (4: 8 wavefronts, 128 queries, the two
// staged block pairs double-buffered when they fit; 2: 4 wavefronts, 64
// queries, one staged pair with the next pair's loads held in registers while
// the current one is multiplied, so two workgroups share a CU).
template <typename T, int HS, int WPE = 0, int QC = 4>
__global__ __launch_bounds__(128 * QC, WPE) void attention_kernel(T* __restrict__ out, const T* __restrict__ qkv,
                                                             int Tn, int C, int NH, float sl2,
                                                             float* __restrict__ lse) {
    constexpr bool F32 = std::is_same<T, float>::value;
    constexpr int VE = Vec<T>::N;
    constexpr int DT = (HS + 31) / 32;  // 32-row tiles of O^T (head dim padded to 32)
    constexpr int HSP = DT * 32;
    constexpr int KCH = HS / (2 * VE);  // 16-byte fragments along the head dim
    static_assert(HS % (2 * VE) == 0, "head size must hold whole fragments");
    constexpr int LDK = HS + VE;    // K block [kBKV][HS], 16-byte row pad
    constexpr int LDV = kBKV + VE;  // V^T block [HSP][kBKV], 16-byte row pad
    constexpr int KSZ = kBKV * LDK, VSZ = HSP * LDV;  // elements per block
    constexpr int PAIR = 2 * (KSZ + VSZ);             // one iteration: even + odd block
    constexpr int NT = 128 * QC, BQ = 32 * QC;        // threads, queries per workgroup
    constexpr bool DB = QC == 4 && 2 * PAIR * (int)sizeof(T) <= 160 * 1024;  // double-buffered
    constexpr bool PF = QC == 2;  // single-buffered, next pair prefetched into registers
    constexpr int NBUF = DB ? 2 : 1;
    constexpr int RV = HS / VE;                                  // 16-byte vectors per key row
    constexpr int NKV = (2 * kBKV * RV + NT - 1) / NT;           // K vectors per thread
    constexpr int NVS = (2 * kBKV / 4 * RV + NT - 1) / NT;       // V 4-key sub-blocks per thread
    constexpr int MERGE = QC * 64 * (DT * 16 + 2);               // floats for the parity merge
    static_assert(MERGE * 4 <= NBUF * PAIR * (int)sizeof(T), "merge area");
    __shared__ __attribute__((aligned(16))) T smem[NBUF * PAIR];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int qc = wid % QC, par = wid / QC;
    const int h = lane >> 5, r32 = lane & 31;
    // Workgroups are dispatched in linear order (x fastest): all (batch, head)
    // pairs of the last, longest query block first, then the next, so the
    // causal triangle's long rows never end up in the tail.
    const int qb = gridDim.y - 1 - blockIdx.y;
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int q0 = qb * BQ, qw = q0 + qc * 32;
    const int64_t rs = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * Tn * rs;
    const int qoff = hd * HS, koff = C + hd * HS, voff = 2 * C + hd * HS;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto Kblk = [&](int buf, int p) { return smem + buf * PAIR + p * KSZ; };
    auto Vblk = [&](int buf, int p) { return smem + buf * PAIR + 2 * KSZ + p * VSZ; };

    // Padded head rows of V^T (HS < 32) are never loaded: zero them once.
    if (HS < HSP) {
        for (int i = tid; i < NBUF * 2 * (HSP - HS) * LDV; i += NT) {
            const int blk = i / ((HSP - HS) * LDV), j = i % ((HSP - HS) * LDV);
            T* vb = Vblk(blk >> 1, blk & 1) + HS * LDV + j;
            if constexpr (F32) *vb = 0.f;
            else vb->bits = 0;
        }
    }

    // Q fragments: the B operand of S^T = K Q^T. Lane (h, r32) holds query
    // qw + r32, head dims kc*2*VE + h*VE .. +VE-1.
    u32x4 qf[KCH];
    {
        const int q = qw + r32;
#pragma unroll
        for (int kc = 0; kc < KCH; kc++)
            qf[kc] = q < Tn ? *reinterpret_cast<const u32x4*>(base + q * rs + qoff + kc * 2 * VE + h * VE)
                            : zero;
    }

    // ---- staging of a block pair: global -> registers -> LDS
    u32x4 rk[NKV], rv[NVS][4];
    auto gload = [&](int k0) {  // keys k0 .. k0 + 127
#pragma unroll
        for (int i = 0; i < NKV; i++) {
            const int li = tid + i * NT, r = li / RV, cv = li % RV, key = k0 + r;
            rk[i] = (li < 2 * kBKV * RV && key < Tn)
                        ? *reinterpret_cast<const u32x4*>(base + key * rs + koff + cv * VE) : zero;
        }
        // V sub-block li: keys 4kq..4kq+3, head dims cv*VE..; consecutive lanes
        // take consecutive key quads, so the 16 lanes of one LDS write cycle
        // fill one contiguous run of a V^T row (no bank conflicts).
#pragma unroll
        for (int i = 0; i < NVS; i++) {
            const int li = tid + i * NT, rest = li >> 4;
            const int kq = (rest / RV) * 16 + (li & 15), cv = rest % RV;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int key = k0 + 4 * kq + e;
                rv[i][e] = (li < 2 * kBKV / 4 * RV && key < Tn)
                               ? *reinterpret_cast<const u32x4*>(base + key * rs + voff + cv * VE) : zero;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NKV; i++) {
            const int li = tid + i * NT, r = li / RV, cv = li % RV;
            if (li < 2 * kBKV * RV)
                *reinterpret_cast<u32x4*>(&Kblk(buf, r / kBKV)[(r % kBKV) * LDK + cv * VE]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < NVS; i++) {
            const int li = tid + i * NT, rest = li >> 4;
            const int kq = (rest / RV) * 16 + (li & 15), cv = rest % RV;
            if (li < 2 * kBKV / 4 * RV) {
                T* vb = Vblk(buf, (4 * kq) / kBKV);
                const int kl = (4 * kq) % kBKV;
                // 4 keys x VE head dims -> VE rows of V^T, 4 consecutive slots each
                if constexpr (F32) {
#pragma unroll
                    for (int d = 0; d < 4; d++) {
                        const u32x4 col = {rv[i][0][d], rv[i][1][d], rv[i][2][d], rv[i][3][d]};
                        *reinterpret_cast<u32x4*>(&vb[(cv * 4 + d) * LDV + kl]) = col;
                    }
                } else {
                    const int slot = vt_slot_bf16(kl);
#pragma unroll
                    for (int d = 0; d < 8; d++) {
                        const int w = d >> 1, sh = 16 * (d & 1);
                        const uint32_t k0v = (rv[i][0][w] >> sh) & 0xffffu, k1v = (rv[i][1][w] >> sh) & 0xffffu;
                        const uint32_t k2v = (rv[i][2][w] >> sh) & 0xffffu, k3v = (rv[i][3][w] >> sh) & 0xffffu;
                        const u32x2 col = {k0v | (k1v << 16), k2v | (k3v << 16)};
                        *reinterpret_cast<u32x2*>(&vb[(cv * 8 + d) * LDV + slot]) = col;
                    }
                }
            }
        }
    };

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;  // for query qw + r32, in log2 units

    // One key block (keys k0..k0+63) for this wave's 32 queries.
    auto block = [&](const T* Ks, const T* Vt, int k0) {
        // S^T tiles: keys k0 + kt*32 + (8*(v/4) + 4*h + v%4), query qw + r32.
        // The two key tiles' MFMAs alternate, so neither chain waits on itself.
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kc = 0; kc < KCH; kc++) {
            const u32x4 ka0 = *reinterpret_cast<const u32x4*>(&Ks[r32 * LDK + kc * 2 * VE + h * VE]);
            const u32x4 ka1 = *reinterpret_cast<const u32x4*>(&Ks[(32 + r32) * LDK + kc * 2 * VE + h * VE]);
            if constexpr (F32) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    s[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ka0[e]), __uint_as_float(qf[kc][e]),
                                                               s[0], 0, 0, 0);
                    s[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ka1[e]), __uint_as_float(qf[kc][e]),
                                                               s[1], 0, 0, 0);
                }
            } else {
                MfmaS<T>::run(s[0], ka0, qf[kc]);
                MfmaS<T>::run(s[1], ka1, qf[kc]);
            }
        }
        const int q = qw + r32;
        float mx = -INFINITY;
        if (k0 + kBKV - 1 > qw) {  // diagonal block: mask keys after the query
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int key = k0 + kt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    if (key > q) s[kt][v] = -INFINITY;
                }
        }
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mx = fmaxf(mx, s[kt][v]);
        mx = halves_max(mx);
        // The reference max m_run moves only when a block's max exceeds it by
        // more than kLazyMax (log2 units), so probabilities stay below
        // 2^kLazyMax and most blocks skip rescaling o. o and l always share
        // one reference, so o / l is unchanged. The decision is per query (a
        // multiply by exactly 1 elsewhere), so each query's result depends on
        // its own scores only; the wave-wide test only skips no-op multiplies.
        // mx is finite: a processed block always holds key k0 <= every query.
        const float mb = mx * sl2;
        const bool grow = mb > m_run + kLazyMax;
        const float m_new = grow ? mb : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kt][v], sl2, -m_new));
                s[kt][v] = p;
                ls += p;
            }
        ls = halves_sum(ls);
        l_run = l_run * alpha + ls;
        m_run = m_new;
        if (__any(grow)) {
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int v = 0; v < 16; v++) o[dt][v] *= alpha;
        }

        // O^T += V^T P^T. The k slots of both operands name the same keys.
        if constexpr (F32) {
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int g = 0; g < 4; g++)
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        // keys kt*32 + 8g + 4h + e, e = 0..3
                        const u32x4 va = *reinterpret_cast<const u32x4*>(
                            &Vt[(dt * 32 + r32) * LDV + kt * 32 + 8 * g + 4 * h]);
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(va[e]), s[kt][4 * g + e],
                                                                        o[dt], 0, 0, 0);
                    }
        } else {
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    // slot (h, e): key 16ks + 4h + e (e<4), 16ks + 8 + 4h + e-4 (e>=4)
                    u32x4 pb;
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        pb[e] = pack_bf16x2(s[kt][8 * ks + 2 * e], s[kt][8 * ks + 2 * e + 1]);
#pragma unroll
                    for (int dt = 0; dt < DT; dt++) {
                        const u32x4 va = *reinterpret_cast<const u32x4*>(
                            &Vt[(dt * 32 + r32) * LDV + kt * 32 + 16 * ks + 8 * h]);
                        MfmaS<T>::run(o[dt], va, pb);
                    }
                }
        }
    };

    const int kend = min(Tn, q0 + BQ);
    const int nkb = (kend + kBKV - 1) / kBKV;  // key blocks this workgroup needs
    const int npair = (nkb + 1) / 2;
    auto compute_pair = [&](int buf, int i) {
        const int kb = 2 * i + par, k0 = kb * kBKV;
        if (kb < nkb && k0 <= qw + 31) block(Kblk(buf, par), Vblk(buf, par), k0);
    };
    if constexpr (DB) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int i = 0; i < npair; i++) {
            const int cur = i & 1;
            if (i + 1 < npair) gload((i + 1) * 2 * kBKV);
            compute_pair(cur, i);
            if (i + 1 < npair) sstore(cur ^ 1);
            __syncthreads();
        }
    } else if constexpr (PF) {
        gload(0);
        sstore(0);
        __syncthreads();
        for (int i = 0; i < npair; i++) {
            if (i + 1 < npair) gload((i + 1) * 2 * kBKV);
            compute_pair(0, i);
            __syncthreads();
            if (i + 1 < npair) {
                sstore(0);
                __syncthreads();
            }
        }
    } else {
        for (int i = 0; i < npair; i++) {
            gload(i * 2 * kBKV);
            sstore(0);
            __syncthreads();
            compute_pair(0, i);
            __syncthreads();
        }
    }

    // Merge the two parities of each query chunk (fixed order: even + odd).
    float* mg = reinterpret_cast<float*>(smem) + qc * 64 * (DT * 16 + 2);
    if (par == 1) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mg[(dt * 16 + v) * 64 + lane] = o[dt][v];
        mg[(DT * 16) * 64 + lane] = m_run;
        mg[(DT * 16 + 1) * 64 + lane] = l_run;
    }
    __syncthreads();
    if (par == 1) return;
    const float m1 = mg[(DT * 16) * 64 + lane], l1 = mg[(DT * 16 + 1) * 64 + lane];
    const float m = fmaxf(m_run, m1);  // m_run is finite: the even half holds key block 0
    const float a0 = __builtin_amdgcn_exp2f(m_run - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
    const float lsum = l_run * a0 + l1 * a1;
    const float inv = 1.0f / lsum;

    // O^T register v of lane (h, r32): head dim dt*32 + 8*(v/4) + 4*h + v%4,
    // query qw + r32. Four consecutive head dims per store.
    const int q = qw + r32;
    // lse (optional): the natural log-sum-exp of the query's scaled scores,
    // ln sum_j e^{S_j} = (m + log2 l) ln 2 in the base-2 units used above.
    if (lse && h == 0 && q < Tn) lse[(int64_t)bh * Tn + q] = (m + __log2f(lsum)) * 0.6931471805599453f;
    if (q < Tn) {
        T* orow = out + ((int64_t)b * Tn + q) * C + hd * HS;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int d0 = dt * 32 + 8 * g + 4 * h;
                if (d0 < HS) {
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        x[e] = (o[dt][4 * g + e] * a0 + mg[(dt * 16 + 4 * g + e) * 64 + lane] * a1) * inv;
                    if constexpr (F32) {
                        *reinterpret_cast<float4*>(orow + d0) = make_float4(x[0], x[1], x[2], x[3]);
                    } else {
                        u32x2 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                        *reinterpret_cast<u32x2*>(orow + d0) = pk;
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// bf16, head size 64 (GPT-2 small and medium). The same online-softmax
// algorithm, arranged so the vector units do little beyond the softmax:
//  - K and V blocks (64 keys) go from HBM/L2 straight to LDS with the
//    load-to-LDS copies (no VGPR staging, no transposing stores), through a
//    two-stage ring: block j+1 is in flight while block j is multiplied. A
//    key row is 128 bytes = 8 chunks of 16; rows are stored with their chunks
//    permuted (K: slot = chunk ^ ((row/2) % 8), conflict-free for the 16-row
//    fragment reads; V: slot = chunk ^ 4*((row/2) % 2), conflict-free for the
//    transposing reads below), the copies fetching the permuted global
//    chunks instead. Copy and read addresses are per-lane constants plus
//    wave-uniform or immediate offsets.
//  - The V^T operand of O^T += V^T P^T is read with gfx950's transposing LDS
//    read (ds_read_b64_tr_b16): in each 16-lane group, lane 4j+q addresses
//    4 head dims (4q..4q+3 past the group's base) of key j, and lane i
//    receives head dim i of keys 0..3. Two reads give a lane the 8 keys its
//    half of the P^T accumulator holds (16ks+4h+0..3 and 16ks+8+4h+0..3),
//    so V needs no reordering.
//  - A block's K fragments are all read before its score products, and its
//    V^T fragments right after them, so their LDS latency overlaps the
//    matrix work and the softmax instead of stalling each product.
// Workgroup: 4 wavefronts x 32 queries (128 queries), each walking all key
// blocks of the workgroup's causal range; 32 KiB of LDS, <= 168 VGPRs: 3
// workgroups per CU.
static constexpr int kAttnD64Waves = 4;

__global__ __launch_bounds__(64 * kAttnD64Waves, 3) void attention_bf16_d64_kernel(
    bf16* __restrict__ out, const bf16* __restrict__ qkv, int Tn, int C, int NH, float sl2,
    float* __restrict__ lse) {
    constexpr int HS = 64, KB = 64;  // head size, keys per block
    constexpr int BLK = KB * HS;     // elements of one K or V block (8 KiB)
    constexpr int STAGE = 2 * BLK;   // K block then V block
    constexpr int BQ = 32 * kAttnD64Waves;
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, r32 = lane & 31;
    const int qb = gridDim.y - 1 - blockIdx.y;  // longest query blocks first
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH;
    const int q0 = qb * BQ, qw = q0 + wid * 32;
    const int64_t rs = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * Tn * rs;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    u32x4 qf[4];  // B operand of S^T = K Q^T: query qw + r32, head dims 16kc + 8h .. +7
    {
        const int q = qw + r32;
#pragma unroll
        for (int kc = 0; kc < 4; kc++)
            qf[kc] = q < Tn ? *reinterpret_cast<const u32x4*>(base + (int64_t)q * rs + hd * HS + kc * 16 + h * 8)
                            : zero;
    }

    // Copies: wave w moves key rows 16w .. 16w+15 of the K and of the V block
    // (two 8-row instructions each); lane l takes row 8i + l/8, LDS slot l % 8,
    // i.e. global chunk slot ^ swizzle(row). Element offsets inside the
    // sequence (T * 3C < 2^31) for block 0; block j adds j*64 rows. Rows past
    // the sequence read its last key (finite, and masked).
    const int crow0 = 16 * wid + (lane >> 3), cslot = lane & 7;
    int kp[2], vp[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int row = crow0 + 8 * i;
        kp[i] = row * (int)rs + C + hd * HS + (cslot ^ ((row >> 1) & 7)) * 8;
        vp[i] = row * (int)rs + 2 * C + hd * HS + (cslot ^ (4 * ((row >> 1) & 1))) * 8;
    }
    auto issue = [&](int stage, int j) {
        bf16* st = smem + stage * STAGE;
        const int k0 = j * KB;
        const bool full = k0 + KB <= Tn;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int row = crow0 + 8 * i;
            const int radd = (full ? k0 : min(k0 + row, Tn - 1) - row) * (int)rs;
            copy16_to_lds(base + kp[i] + radd, (lds_void_ptr)(st + (16 * wid + 8 * i) * HS));
            copy16_to_lds(base + vp[i] + radd, (lds_void_ptr)(st + BLK + (16 * wid + 8 * i) * HS));
        }
    };

    // K fragment reads: row r32 (+32), chunk (2kc + h) ^ swizzle = 2kc ^ kx
    const int kx = h ^ ((r32 >> 1) & 7), krow = r32 * HS;
    // Transposing-read base of this lane: lane 4gj+gq of its 16-lane group
    // addresses key 4h + gj (+ a compile-time key offset), head dims
    // gdim + 4gq (+ 32dt); key bit 1 is gj's bit 1, so the V swizzle of the
    // chunk is a per-lane constant.
    const int gj = (lane & 15) >> 2, gq = lane & 3;
    const int vy = (gj >> 1) & 1, vx = 2 * (r32 >> 4) + (gq >> 1);
    int vbase[2];
#pragma unroll
    for (int dt = 0; dt < 2; dt++) vbase[dt] = (4 * h + gj) * HS + (4 * (dt ^ vy) + vx) * 8 + (gq & 1) * 4;

    f32x16 o[2] = {f32x16{}, f32x16{}};  // O^T tiles: head dims 0..31 and 32..63
    float m_run = -INFINITY;             // reference max of query qw + r32, log2 units
    float l_part = 0.f;                  // this lane's share of the normaliser (its 16 keys per tile)

    auto block = [&](const bf16* Ks, const bf16* Vs, int k0) {
        // every K fragment of the block first, then the score products; the
        // compiler's MFMA/memory interleaving strategy 1 for the block
        __builtin_amdgcn_iglp_opt(1);
        u32x4 ka[4][2];
#pragma unroll
        for (int kc = 0; kc < 4; kc++) {
            const int ko = krow + ((2 * kc) ^ kx) * 8;
            ka[kc][0] = *reinterpret_cast<const u32x4*>(&Ks[ko]);
            ka[kc][1] = *reinterpret_cast<const u32x4*>(&Ks[ko + 32 * HS]);
        }
        f32x16 sc[2];
        // Issue priority for the score products and the V^T reads after them:
        // of the wavefronts sharing a SIMD (other workgroups'), one entering
        // its products goes ahead of those in their softmax, so matrix and
        // vector work overlap more.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kc = 0; kc < 4; kc++)
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
                sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[kc][kt]),
                                                                __builtin_bit_cast(bf16x8, qf[kc]),
                                                                kc ? sc[kt] : f32x16{}, 0, 0, 0);
        // the V^T fragments of the whole block, read while the softmax runs
        const lds_v4s_ptr vt = (lds_v4s_ptr)Vs;
        u32x4 va[2][2][2];
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int dt = 0; dt < 2; dt++) {
                    const int kofs = (kt * 32 + 16 * ks) * HS;  // compile-time element offset
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vt + (vbase[dt] + kofs) / 4);
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vt + (vbase[dt] + kofs + 8 * HS) / 4);
                    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                    va[kt][ks][dt] = u32x4{l2[0], l2[1], h2[0], h2[1]};
                }
        __builtin_amdgcn_s_setprio(0);
        const int q = qw + r32;
        if (k0 + KB - 1 > qw) {  // diagonal block: keys after the query are -inf
#pragma unroll
            for (int kt = 0; kt < 2; kt++)
#pragma unroll
                for (int v = 0; v < 16; v++)
                    if (k0 + kt * 32 + 8 * (v >> 2) + 4 * h + (v & 3) > q) sc[kt][v] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int v = 0; v < 16; v++) mx = fmaxf(mx, sc[kt][v]);
        mx = halves_max(mx);
        const float mb = mx * sl2;
        const bool grow = mb > m_run + kLazyMax;
        const float m_new = grow ? mb : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        m_run = m_new;
        l_part *= alpha;
        if (__any(grow)) {
#pragma unroll
            for (int dt = 0; dt < 2; dt++)
#pragma unroll
                for (int v = 0; v < 16; v++) o[dt][v] *= alpha;
        }
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                u32x4 pbk;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * ks + 2 * e], sl2, -m_new));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kt][8 * ks + 2 * e + 1], sl2, -m_new));
                    l_part += p0 + p1;
                    pbk[e] = pack_bf16x2(p0, p1);
                }
#pragma unroll
                for (int dt = 0; dt < 2; dt++)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[kt][ks][dt]),
                                                                   __builtin_bit_cast(bf16x8, pbk), o[dt], 0, 0, 0);
            }
    };

    const int kend = min(Tn, q0 + BQ);
    const int nkb = (kend + KB - 1) / KB;
    issue(0, 0);
    for (int j = 0; j < nkb; j++) {
        // this wave's copies of block j have landed and its LDS reads of
        // block j-1 are done; after the barrier every wave's are
        wait_vmcnt_lds<0>();
        __builtin_amdgcn_s_barrier();
        if (j + 1 < nkb) issue((j + 1) & 1, j + 1);
        const int k0 = j * KB;
        if (k0 <= qw + 31) block(smem + (j & 1) * STAGE, smem + (j & 1) * STAGE + BLK, k0);
    }

    const float l_run = halves_sum(l_part);  // both halves' keys
    const int q = qw + r32;
    if (q >= Tn) return;
    const float inv = 1.0f / l_run;
    if (lse && h == 0) lse[(int64_t)bh * Tn + q] = (m_run + __log2f(l_run)) * 0.6931471805599453f;
    bf16* orow = out + ((int64_t)b * Tn + q) * C + hd * HS;
#pragma unroll
    for (int dt = 0; dt < 2; dt++)
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int d0 = dt * 32 + 8 * g + 4 * h;
            u32x2 pk = {pack_bf16x2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv),
                        pack_bf16x2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + d0) = pk;
        }
}

// Launch shape: fp32 asks the register allocator for as many wavefronts per
// SIMD as its accumulators allow (3 up to head size 32; 2 from 64, where the
// kernel needs more than the 168 VGPRs of 3); bf16 (head sizes other than
// 64, which have their own kernel) runs double-buffered.
template <typename T, int HS>
static void launch_attn_hs(T* out, const T* qkv, int B, int Tn, int C, int NH, hipStream_t s, float* lse) {
    const float sl2 = 1.4426950408889634f / sqrtf((float)HS);  // log2(e)/sqrt(hs)
    dim3 grid(B * NH, (Tn + 127) / 128);
    if constexpr (std::is_same<T, float>::value) {
        if constexpr (HS == 64) {
            if ((int)(grid.x * grid.y) <= kNumCUs) {
                // Fewer 128-query workgroups than CUs: 64-query workgroups,
                // two per CU, reach every CU and halve the longest one's work.
                grid.y = (Tn + 63) / 64;
                attention_kernel<T, HS, 2, 2><<<grid, 256, 0, s>>>(out, qkv, Tn, C, NH, sl2, lse);
                return;
            }
        }
        attention_kernel<T, HS, (HS >= 64 ? 2 : 3)><<<grid, 512, 0, s>>>(out, qkv, Tn, C, NH, sl2, lse);
    } else {
        attention_kernel<T, HS><<<grid, 512, 0, s>>>(out, qkv, Tn, C, NH, sl2, lse);
    }
}

template <typename T>
static void launch_attn_t(T* out, const T* qkv, int B, int Tn, int C, int NH, hipStream_t s, float* lse) {
    if constexpr (std::is_same<T, bf16>::value) {
        if (C / NH == 64) {
            const float sl2 = 1.4426950408889634f / 8.0f;  // log2(e)/sqrt(64)
            dim3 grid(B * NH, (Tn + 32 * kAttnD64Waves - 1) / (32 * kAttnD64Waves));
            attention_bf16_d64_kernel<<<grid, 64 * kAttnD64Waves, 0, s>>>(out, qkv, Tn, C, NH, sl2, lse);
            return;
        }
    }
    switch (C / NH) {
        case 16: launch_attn_hs<T, 16>(out, qkv, B, Tn, C, NH, s, lse); break;
        case 32: launch_attn_hs<T, 32>(out, qkv, B, Tn, C, NH, s, lse); break;
        case 64:
            if constexpr (std::is_same<T, float>::value) launch_attn_hs<T, 64>(out, qkv, B, Tn, C, NH, s, lse);
            break;
        default: launch_attn_hs<T, 128>(out, qkv, B, Tn, C, NH, s, lse); break;
    }
}

// lse (nullable): [B,NH,T] fp32, the log-sum-exp of every query row.
int launch_attention(void* out, const void* qkv, int B, int T, int C, int NH, int dtype,
                     hipStream_t s, float* lse) {
    if (dtype == GPT2_BF16)
        launch_attn_t<bf16>((bf16*)out, (const bf16*)qkv, B, T, C, NH, s, lse);
    else
        launch_attn_t<float>((float*)out, (const float*)qkv, B, T, C, NH, s, lse);
    return launch_status();
}

bool attention_head_size_ok(int hs) { return hs == 16 || hs == 32 || hs == 64 || hs == 128; }

// ------------------------------------------------------------- cache store
// Prefill: the keys and values of positions 0..T-1 (the k and v thirds of
// qkv [B,T,3C]) into one layer's caches [B,NH,maxT,hs], the layout the decode
// step reads. One 16-byte vector per thread, grid-stride.
template <typename T>
__global__ __launch_bounds__(256) void kv_store_kernel(T* __restrict__ kc, T* __restrict__ vc,
                                                       const T* __restrict__ qkv, int B, int Tn, int C, int NH,
                                                       int maxT, int64_t nvec) {
    constexpr int VE = Vec<T>::N;
    const int hs = C / NH, cv = C / VE;
    for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / (2 * cv);  // b*T + t
        const int rem = (int)(i - row * 2 * cv), which = rem / cv, c = (rem % cv) * VE;
        const int b = (int)(row / Tn), t = (int)(row % Tn), h = c / hs, d = c % hs;
        const u32x4 v = *reinterpret_cast<const u32x4*>(qkv + row * 3 * C + (1 + which) * C + c);
        T* dst = (which ? vc : kc) + (((int64_t)b * NH + h) * maxT + t) * hs + d;
        *reinterpret_cast<u32x4*>(dst) = v;
    }
}

int launch_kv_store(void* kc, void* vc, const void* qkv, int B, int Tn, int C, int NH, int maxT, int dtype,
                    hipStream_t s) {
    const int64_t nvec = (int64_t)B * Tn * 2 * C / (dtype == GPT2_BF16 ? 8 : 4);
    const unsigned grid = (unsigned)std::min<int64_t>((nvec + 255) / 256, 2048);
    if (dtype == GPT2_BF16)
        kv_store_kernel<bf16><<<grid, 256, 0, s>>>((bf16*)kc, (bf16*)vc, (const bf16*)qkv, B, Tn, C, NH, maxT, nvec);
    else
        kv_store_kernel<float><<<grid, 256, 0, s>>>((float*)kc, (float*)vc, (const float*)qkv, B, Tn, C, NH, maxT,
                                                    nvec);
    return launch_status();
}

// ------------------------------------------------------------------ decode
// One new query per sequence against a KV cache (optdl2025 NanoGPT project:
// KV caching for autoregressive prediction). The keys 0..pos of each
// (sequence, head) are cut into chunks of decode_chunk<T, HS> keys, one
// 512-thread workgroup per chunk. Each thread owns a 16-byte slice of
// kDecPasses key rows and the matching value rows and issues all of those
// loads before the first use, so a workgroup waits on memory once. Scores
// stay in registers: the TPK threads of a key row end the dot product with
// the same value, the chunk's max and sum-of-exponentials are block
// reductions, and the weighted value rows are summed across key groups by
// shuffles and then across wavefronts through LDS in a fixed order. A chunk
// that covers every key writes the normalised output; otherwise it leaves an
// unnormalised partial (o, m, l) that decode_combine_kernel merges in chunk
// order, so the result does not depend on scheduling.
static constexpr int kDecThreads = 512;
static constexpr int kDecPasses = 8;
static constexpr int kDecMinChunk = 64;  // smallest chunk a launch may use (bounds the workspace)

template <typename T, int HS, int NT = kDecThreads, int NP = kDecPasses>
constexpr int decode_chunk() {
    return NP * NT / (HS / Vec<T>::N);
}

template <typename T, int HS, int NT = kDecThreads, int NP = kDecPasses>
__global__ __launch_bounds__(NT) void decode_attn_kernel(T* __restrict__ out, float* __restrict__ part,
                                                                  const T* __restrict__ qkv_new,
                                                                  T* __restrict__ kc, T* __restrict__ vc,
                                                                  int pos, int maxT, int C, int NH, float sl2) {
    constexpr int VE = Vec<T>::N;
    constexpr int TPK = HS / VE;             // threads per key row
    constexpr int KPP = NT / TPK;   // key rows per pass
    constexpr int CHUNK = KPP * NP;
    constexpr int NW = NT / 64;
    static_assert(HS % VE == 0 && 64 % TPK == 0, "head size");
    __shared__ float red[NW * HS];
    __shared__ float shm[NW], shl[NW];

    const int split = blockIdx.x, nsplit = gridDim.x, bh = blockIdx.y;
    const int b = bh / NH, hd = bh % NH;
    const int j0 = split * CHUNK, j1 = min(j0 + CHUNK, pos + 1);  // j0 <= pos: the grid covers 0..pos
    const int tid = threadIdx.x, sub = tid % TPK, kg = tid / TPK;
    const int lane = tid & 63, w = tid >> 6;
    const T* qrow = qkv_new + (int64_t)b * 3 * C;
    const T* knew = qrow + C + hd * HS + sub * VE;
    const T* vnew = qrow + 2 * C + hd * HS + sub * VE;
    T* K = kc + (int64_t)bh * maxT * HS + sub * VE;
    T* Vc = vc + (int64_t)bh * maxT * HS + sub * VE;

    if (pos >= j0 && pos < j1 && tid < TPK) {  // this step's k, v into the cache
        *reinterpret_cast<u32x4*>(K + (int64_t)pos * HS) = *reinterpret_cast<const u32x4*>(knew);
        *reinterpret_cast<u32x4*>(Vc + (int64_t)pos * HS) = *reinterpret_cast<const u32x4*>(vnew);
    }
    // every load first: key row j (the new one from qkv_new, never from the
    // cache slot being written); rows past the chunk read row j0 and are masked.
    // The cache is read once per step, so its lines are marked non-temporal:
    // they do not displace the weights the step's projections read again.
    u32x4 kr[NP], vr[NP];
#pragma unroll
    for (int p = 0; p < NP; p++) {
        const int j = j0 + kg + p * KPP;
        const int jc = j < j1 ? j : j0;
        kr[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(jc == pos ? knew : K + (int64_t)jc * HS));
        vr[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(jc == pos ? vnew : Vc + (int64_t)jc * HS));
    }
    float q[VE];
    load_vec(qrow + hd * HS + sub * VE, q);
    float sc[NP];
    float mx = -INFINITY;
#pragma unroll
    for (int p = 0; p < NP; p++) {
        float k[VE];
        unpack_vec<T>(kr[p], k);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < VE; e++) d += q[e] * k[e];
#pragma unroll
        for (int o = TPK / 2; o > 0; o >>= 1) d += __shfl_xor(d, o, 64);
        sc[p] = j0 + kg + p * KPP < j1 ? d * sl2 : -INFINITY;
        mx = fmaxf(mx, sc[p]);
    }
    mx = wave_max(mx);
    if (lane == 0) shm[w] = mx;
    __syncthreads();
    mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; i++) mx = fmaxf(mx, shm[i]);  // finite: key j0 is valid
    float ls = 0.f, acc[VE];
#pragma unroll
    for (int e = 0; e < VE; e++) acc[e] = 0.f;
#pragma unroll
    for (int p = 0; p < NP; p++) {
        const float pw = exp2f(sc[p] - mx);  // 0 for masked rows
        ls += pw;
        float v[VE];
        unpack_vec<T>(vr[p], v);
#pragma unroll
        for (int e = 0; e < VE; e++) acc[e] += pw * v[e];
    }
    // key groups of a wavefront: lanes that differ in the bits above TPK
#pragma unroll
    for (int o = TPK; o < 64; o <<= 1) {
        ls += __shfl_xor(ls, o, 64);
#pragma unroll
        for (int e = 0; e < VE; e++) acc[e] += __shfl_xor(acc[e], o, 64);
    }
    if (lane < TPK) {
#pragma unroll
        for (int e = 0; e < VE; e++) red[w * HS + sub * VE + e] = acc[e];
        if (lane == 0) shl[w] = ls;  // the wave's key groups, each key once
    }
    __syncthreads();
    if (tid < HS) {
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int i = 0; i < NW; i++) {
            o += red[i * HS + tid];
            l += shl[i];
        }
        if (nsplit == 1) {
            store_scalar(out + (int64_t)b * C + hd * HS + tid, o / l);
        } else {
            float* pp = part + ((int64_t)bh * nsplit + split) * (HS + 2);
            pp[tid] = o;
            if (tid == 0) {
                pp[HS] = mx;
                pp[HS + 1] = l;
            }
        }
    }
}

template <typename T, int HS>
__global__ __launch_bounds__(HS) void decode_combine_kernel(T* __restrict__ out,
                                                            const float* __restrict__ part,
                                                            int nsplit, int C, int NH) {
    const int bh = blockIdx.x, b = bh / NH, hd = bh % NH, d = threadIdx.x;
    const float* pp = part + (int64_t)bh * nsplit * (HS + 2);
    float M = -INFINITY;
    for (int s = 0; s < nsplit; s++) M = fmaxf(M, pp[s * (HS + 2) + HS]);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < nsplit; s++) {
        const float m = pp[s * (HS + 2) + HS];
        const float wgt = m == -INFINITY ? 0.f : exp2f(m - M);
        L += pp[s * (HS + 2) + HS + 1] * wgt;
        o += pp[s * (HS + 2) + d] * wgt;
    }
    store_scalar(out + (int64_t)b * C + hd * HS + d, o / L);
}

int64_t decode_workspace_bytes(int B, int C, int NH, int maxT) {
    const int hs = C / NH;
    const int64_t nsplit = (maxT + kDecMinChunk - 1) / kDecMinChunk;
    return (int64_t)B * NH * nsplit * (hs + 2) * 4;
}

template <typename T, int HS>
static int launch_decode_hs(T* out, const T* qkv_new, T* kc, T* vc, int B, int pos, int maxT,
                            int C, int NH, float* part, hipStream_t s, bool combine) {
    constexpr int CHUNK = decode_chunk<T, HS>();
    static_assert(CHUNK >= kDecMinChunk, "workspace bound");
    const float sl2 = 1.4426950408889634f / sqrtf((float)HS);
    const int nsplit = (pos + 1 + CHUNK - 1) / CHUNK;
    decode_attn_kernel<T, HS><<<dim3(nsplit, B * NH), kDecThreads, 0, s>>>(out, part, qkv_new, kc, vc, pos,
                                                                           maxT, C, NH, sl2);
    if (nsplit > 1 && combine) decode_combine_kernel<T, HS><<<B * NH, HS, 0, s>>>(out, part, nsplit, C, NH);
    return nsplit;
}

template <typename T>
static int launch_decode_t(T* out, const T* qkv_new, T* kc, T* vc, int B, int pos, int maxT,
                           int C, int NH, float* part, hipStream_t s, bool combine) {
    switch (C / NH) {
        case 16: return launch_decode_hs<T, 16>(out, qkv_new, kc, vc, B, pos, maxT, C, NH, part, s, combine);
        case 32: return launch_decode_hs<T, 32>(out, qkv_new, kc, vc, B, pos, maxT, C, NH, part, s, combine);
        case 64: return launch_decode_hs<T, 64>(out, qkv_new, kc, vc, B, pos, maxT, C, NH, part, s, combine);
        default: return launch_decode_hs<T, 128>(out, qkv_new, kc, vc, B, pos, maxT, C, NH, part, s, combine);
    }
}

// Key chunks of a decode attention at position pos (the grid's x extent).
template <typename T, int HS>
static int decode_splits_hs(int pos) {
    constexpr int CHUNK = decode_chunk<T, HS>();
    return (pos + 1 + CHUNK - 1) / CHUNK;
}
template <typename T>
static int decode_splits_t(int pos, int hs) {
    switch (hs) {
        case 16: return decode_splits_hs<T, 16>(pos);
        case 32: return decode_splits_hs<T, 32>(pos);
        case 64: return decode_splits_hs<T, 64>(pos);
        default: return decode_splits_hs<T, 128>(pos);
    }
}
int decode_attention_splits(int pos, int hs, int dtype) {
    return dtype == GPT2_BF16 ? decode_splits_t<bf16>(pos, hs) : decode_splits_t<float>(pos, hs);
}

// nsplit_out (nullable): when given, a split attention (more than one chunk
// of keys) leaves its fp32 partials in `part` for the consumer to merge
// (launch_skinny_gemm_acomb) instead of launching the combine, and
// *nsplit_out receives the chunk count (1: `out` was written).
int launch_attention_decode(void* out, const void* qkv_new, void* kcache, void* vcache, int B,
                            int pos, int maxT, int C, int NH, int dtype, float* part,
                            hipStream_t s, int* nsplit_out) {
    const bool combine = nsplit_out == nullptr;
    int ns;
    if (dtype == GPT2_BF16)
        ns = launch_decode_t<bf16>((bf16*)out, (const bf16*)qkv_new, (bf16*)kcache, (bf16*)vcache, B,
                                   pos, maxT, C, NH, part, s, combine);
    else
        ns = launch_decode_t<float>((float*)out, (const float*)qkv_new, (float*)kcache, (float*)vcache,
                                    B, pos, maxT, C, NH, part, s, combine);
    if (nsplit_out) *nsplit_out = ns;
    return launch_status();
}

}  // namespace gpt2

using namespace gpt2;

extern "C" int attention_forward(void* out, const void* qkv, int B, int T, int C, int NH,
                                 int dtype, void* stream) {
    if (!valid_dtype(dtype) || B < 0 || T < 0 || C < 0 || NH <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!out || !qkv || C == 0 || C % NH) return GPT2_ERR_INVALID_ARGUMENT;
    if (!attention_head_size_ok(C / NH) || !aligned16(out) || !aligned16(qkv))
        return GPT2_ERR_UNSUPPORTED;
    if (out == qkv) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_attention(out, qkv, B, T, C, NH, dtype, (hipStream_t)stream, nullptr);
}

extern "C" int attention_forward_lse(void* out, float* lse, const void* qkv, int B, int T, int C, int NH,
                                     int dtype, void* stream) {
    if (!valid_dtype(dtype) || B < 0 || T < 0 || C < 0 || NH <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!out || !lse || !qkv || C == 0 || C % NH) return GPT2_ERR_INVALID_ARGUMENT;
    if (!attention_head_size_ok(C / NH) || !aligned16(out) || !aligned16(qkv)) return GPT2_ERR_UNSUPPORTED;
    if (out == qkv) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_attention(out, qkv, B, T, C, NH, dtype, (hipStream_t)stream, lse);
}

extern "C" int64_t attention_decode_workspace_bytes(int B, int C, int NH, int maxT) {
    if (B < 0 || C <= 0 || NH <= 0 || C % NH || maxT <= 0) return -1;
    return decode_workspace_bytes(B, C, NH, maxT);
}

extern "C" int attention_decode_forward(void* out, const void* qkv_new, void* kcache, void* vcache,
                                        int B, int pos, int maxT, int C, int NH, int dtype,
                                        void* workspace, int64_t workspace_bytes, void* stream) {
    if (!valid_dtype(dtype) || B < 0 || C < 0 || NH <= 0 || maxT <= 0 || pos < 0 || pos >= maxT)
        return GPT2_ERR_INVALID_ARGUMENT;
    if (B == 0) return GPT2_OK;
    if (!out || !qkv_new || !kcache || !vcache || !workspace || C == 0 || C % NH)
        return GPT2_ERR_INVALID_ARGUMENT;
    if (!attention_head_size_ok(C / NH) || !aligned16(out) || !aligned16(qkv_new) ||
        !aligned16(kcache) || !aligned16(vcache) || !aligned16(workspace))
        return GPT2_ERR_UNSUPPORTED;
    if (workspace_bytes < decode_workspace_bytes(B, C, NH, maxT)) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    return launch_attention_decode(out, qkv_new, kcache, vcache, B, pos, maxT, C, NH, dtype,
                                   (float*)workspace, (hipStream_t)stream, nullptr);
}
