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
#include <type_traits>

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
// EPI and res as for gemm_pipe_kernel.
template <typename T, int WM, int WN, int TM, int TN, int BK, bool ILV = true, int EPI = EPI_BIAS>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(T* out, const T* __restrict__ A,
                                                           const T* __restrict__ W,
                                                           const T* __restrict__ bias, const T* res, int M,
                                                           int N, int K, int group_m, int remap) {
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
                // residual (GELU input) read with the row clamped, outside the bounds branch
                const float r = EPI == EPI_BIAS_RESIDUAL || EPI == EPI_DGELU
                                    ? load_scalar(res + (int64_t)min(row, M - 1) * N + col)
                                    : 0.f;
                if (row < M) {
                    float y = acc[i][j][v] + bv;
                    if constexpr (EPI == EPI_BIAS_GELU) y = gelu_tanh(storage_round(out, y));
                    if constexpr (EPI == EPI_BIAS_RESIDUAL) y = storage_round(out, y) + r;
                    if constexpr (EPI == EPI_DGELU) y = storage_round(out, y) * gelu_tanh_grad(r);
                    store_scalar(out + (int64_t)row * N + col, y);
                }
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
// chunk holding logical k-chunk c of row r sits at slot c ^ ((r / 2) % 8).
// LDS serves a 16-byte read for 16 lanes at a time from 64 four-byte banks
// (256 bytes): with 128-byte rows, rows r and r+1 fall in the two halves, and
// the swizzle gives the 8 rows of each parity 8 different 16-byte slots, so
// the 16 rows a fragment read touches hit every bank exactly once.
// The copies are issued from inline assembly so the compiler does not track
// them: its wait-count pass would otherwise drain every outstanding load
// before some LDS reads. All ordering is explicit instead: vmcnt waits for
// this wave's own copies, then a bare s_barrier (a __syncthreads fence would
// also wait for the copies still in flight for later tiles). Every copy is
// complete before the loop exits. Requires K % BK == 0; rows past M or N read
// a clamped (valid) row whose results are never stored. The copy and wait
// helpers (copy16_to_lds, wait_vmcnt_lds) are in common.h.

// SCHED: 0 = compiler order; 1, 2 = the backend's iglp strategies 0 and 1;
// 3 = scheduling groups: after the first k-chunk's fragment reads, every MFMA
// is followed by one fragment read; 4 = hard fences: each segment issues the
// fragment reads of k-chunk kc+1, then the MFMAs of chunk kc, whose operands
// were read one segment earlier (so no MFMA waits on a fresh LDS read).
// WPE: minimum wavefronts per SIMD the register allocation must allow (0: no
// constraint); 2 workgroups of 8 wavefronts per CU need WPE = 4. DIRECT:
// store the output straight from the accumulators (no LDS staging), which
// keeps the LDS footprint at the stages alone.
// EPI: the epilogue (common.h); res [M,N] is the residual of
// EPI_BIAS_RESIDUAL or the GELU input of EPI_DGELU and may be `out` itself
// (each element is read and then written by the same thread).
// SPLITK: workgroup row blockIdx.y multiplies the k-range [y*K, (y+1)*K) and
// writes its product to out + y*split_out; A and W rows are then lda and ldb
// elements long (without SPLITK they are K long and lda, ldb, split_out are
// unused).
// TO: the output type; fp32 products of bf16 operands (split-k partial sums
// that a later fp32 sum reduces) take the plain epilogue or EPI_ASUM only.
// TA / TB: the operand is stored k-major, A as [K][M] (row stride lda), W as
// [K][N] (row stride ldb): out = A^T-stored . W^T-stored without a transpose
// pass. Its tile is copied as BK rows of BM (BN) elements.
//  - fp32: a lane gathers its 4 k-steps with 4 scalar LDS reads; the two lane
//    halves of one read take k-rows 4 apart (k = 8kc + 4h + e), so k-rows
//    with bit 2 set are rotated by 8 chunks (32 banks) and the two halves use
//    disjoint banks.
//  - bf16: transposing reads (ds_read_b64_tr_b16). In each 16-lane group,
//    lane 4j+q addresses k-row j and 4 columns; lane i receives column i of
//    the 4 k-rows. Read r of k-step kc addresses k-rows 16kc + 8h + 4r + j,
//    so a lane gets k = 16kc + 8h + 0..7 of its column, the same k order as
//    a row-major fragment (the two operand forms mix). Chunk c of k-row k is
//    stored in slot c ^ 4(k % 4): the 4 k-rows one lane half reads land in 4
//    different 64-byte bank quarters (BM, BN multiples of 128).
template <typename T, int WM, int WN, int TM, int TN, int RB, int S, int SCHED, int WPE = 0, bool DIRECT = false,
          int EPI = EPI_BIAS, bool SPLITK = false, bool TA = false, bool TB = false, typename TO = T>
__global__ __launch_bounds__(WM* WN * 64, WPE) void gemm_pipe_kernel(TO* out, const T* __restrict__ A,
                                                                const T* __restrict__ W,
                                                                const T* __restrict__ bias, const TO* res, int M,
                                                                int N, int K, int group_m, int remap, int lda,
                                                                int ldb, int64_t split_out,
                                                                float* __restrict__ stats, int vlim,
                                                                TO* __restrict__ out2) {
    // RB: bytes of k per tile row (64 or 128); S: LDS stages (S-1 tiles in flight;
    // S = 2 is plain double buffering: tile t+1 loads while tile t is multiplied)
    constexpr int NW = WM * WN;
    constexpr int VE = Vec<T>::N;
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    constexpr int BK = RB / (int)sizeof(T);  // k elements per tile
    constexpr int CH = RB / 16;              // 16-byte chunks per tile row
    constexpr int RP = 256 / RB;             // rows sharing one 256-byte bank line
    static_assert(CH == 4 || CH == 8, "64- or 128-byte tile rows");
    static_assert(S >= 2 && S <= 6, "stages");
    constexpr int LA = BM * CH / 64 / NW, LB = BN * CH / 64 / NW;  // copies per wave per tile
    static_assert(LA * 64 * NW == BM * CH && LB * 64 * NW == BN * CH, "tile/wave mismatch");
    constexpr int LPW = LA + LB;
    constexpr bool KBF = std::is_same<T, bf16>::value;  // k-major bf16: transposing reads
    constexpr int CMA = BM * (int)sizeof(T) / 16, CMB = BN * (int)sizeof(T) / 16;  // chunks per k-row
    constexpr int ROTA = 8, ROTB = 8;
    static_assert(!(TA || TB) || (CMA >= 16 && CMB >= 16), "k-major tiles need >= 16 chunks per k-row");
    static_assert(!KBF || ((!TA || CMA % 16 == 0) && (!TB || CMB % 16 == 0)), "bf16 k-major: BM, BN % 128 == 0");
    static_assert(LPW * (S - 2) < 64, "vmcnt range");
    constexpr int STAGE = (BM + BN) * BK;  // elements per stage (A tile then W tile)
    constexpr int VO = Vec<TO>::N;          // output elements per 16-byte vector
    static_assert(std::is_same<TO, T>::value || EPI == EPI_BIAS || EPI == EPI_ASUM,
                  "wider output: plain products only");
    static_assert(EPI != EPI_ASUM || TA, "A sums: k-major A only");
    constexpr int LDO = BN + VO;           // row stride of the output tile in the epilogue
    // stage the output tile through LDS when it fits in 160 KiB
    constexpr bool STAGED = !DIRECT && BM * LDO * (int)sizeof(TO) <= 160 * 1024;
    constexpr int SOUT = BM * LDO * (int)sizeof(TO) / (int)sizeof(T);  // staged tile, in T elements
    constexpr int SMEM = (STAGED && SOUT > S * STAGE) ? SOUT : S * STAGE;
    __shared__ __attribute__((aligned(16))) T smem[SMEM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;
    const int h = lane >> 5, r32 = lane & 31;
    if constexpr (SPLITK) {
        A += (int64_t)blockIdx.y * K * (TA ? lda : 1);
        W += (int64_t)blockIdx.y * K * (TB ? ldb : 1);
        out += (int64_t)blockIdx.y * split_out;
    }
    const int lda_ = SPLITK || TA ? lda : K, ldb_ = SPLITK || TB ? ldb : K;

    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int nwg = tiles_m * tiles_n;
    int pid = blockIdx.x;
    if (remap) pid = xcd_contiguous(pid, nwg);
    const int per_group = group_m * tiles_n;
    const int g = pid / per_group, first_m = g * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int in_g = pid - g * per_group;
    const int m0 = (first_m + in_g % gsz) * BM, n0 = (in_g / gsz) * BN;

    // Chunk q of a tile = row q / CH, slot q % CH; the slot holds logical
    // k-chunk slot ^ ((row / RP) % CH).
    // k-major operands: chunk q = k-row q / CM, slot q % CM holding the chunk
    // of m (n) elements (slot - ROT*((row>>2)&1)) mod CM (fp32) or
    // slot ^ 4(row % 4) (bf16); columns past M (N) read a clamped (valid)
    // chunk whose results are never stored.
    int64_t offA[LA], offB[LB];
#pragma unroll
    for (int j = 0; j < LA; j++) {
        const int q = (wid * LA + j) * 64 + lane;
        if constexpr (TA) {
            const int row = q / CMA;
            const int c = KBF ? (q % CMA) ^ (4 * (row & 3)) : (q % CMA + CMA - ROTA * ((row >> 2) & 1)) % CMA;
            offA[j] = (int64_t)row * lda_ + min(m0 + c * VE, M - VE);
        } else {
            const int row = q / CH, lc = (q % CH) ^ ((row / RP) % CH);
            offA[j] = (int64_t)min(m0 + row, M - 1) * lda_ + lc * VE;
        }
    }
#pragma unroll
    for (int j = 0; j < LB; j++) {
        const int q = (wid * LB + j) * 64 + lane;
        if constexpr (TB) {
            const int row = q / CMB;
            const int c = KBF ? (q % CMB) ^ (4 * (row & 3)) : (q % CMB + CMB - ROTB * ((row >> 2) & 1)) % CMB;
            offB[j] = (int64_t)row * ldb_ + min(n0 + c * VE, N - VE);
        } else {
            const int row = q / CH, lc = (q % CH) ^ ((row / RP) % CH);
            offB[j] = (int64_t)min(n0 + row, N - 1) * ldb_ + lc * VE;
        }
    }
    auto issue = [&](int stage, int k0) {
        T* sA = smem + stage * STAGE;
        T* sB = sA + BM * BK;
        const int64_t ka = TA ? (int64_t)k0 * lda_ : k0, kb = TB ? (int64_t)k0 * ldb_ : k0;
#pragma unroll
        for (int j = 0; j < LA; j++)
            copy16_to_lds(A + offA[j] + ka, (lds_void_ptr)(sA + (wid * LA + j) * 64 * VE));
#pragma unroll
        for (int j = 0; j < LB; j++)
            copy16_to_lds(W + offB[j] + kb, (lds_void_ptr)(sB + (wid * LB + j) * 64 * VE));
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) acc[i][j] = f32x16{};

    // fp32: a k-major tile element (k, m) sits at k*BM + slot*VE + m%VE with
    // slot = (m/VE + ROT*((k>>2)&1)) mod CM. A fragment's step e is k = 8kc +
    // 4h + e, whose bit 2 is h: the slot of a lane's column is a per-lane
    // constant, so every read is that lane offset plus a compile-time one.
    // bf16: the transposing read's address for k-step 0, read 0: k-row 8h + j
    // (j = lane/4 % 4), columns c0 + 16(lane/16 % 2) + 4(lane % 4) .. +3 of the
    // lane's 32-column tile c0; slot (column/8) ^ 4j since k-row % 4 = j.
    const int tj = (lane >> 2) & 3, tq = lane & 3, tg = (lane >> 4) & 1;
    auto kcol = [&](int c0, int LD) {
        return (8 * h + tj) * LD + (((c0 >> 3) + 2 * tg + (tq >> 1)) ^ (4 * tj)) * 8 + 4 * (tq & 1);
    };
    int colA[TM], colB[TN];
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int m = wm * TM * 32 + i * 32 + r32;
        colA[i] = !TA   ? 0
                  : KBF ? kcol(wm * TM * 32 + i * 32, BM)
                        : 4 * h * BM + ((m / VE + ROTA * h) % CMA) * VE + m % VE;
    }
#pragma unroll
    for (int j = 0; j < TN; j++) {
        const int n = wn * TN * 32 + j * 32 + r32;
        colB[j] = !TB   ? 0
                  : KBF ? kcol(wn * TN * 32 + j * 32, BN)
                        : 4 * h * BN + ((n / VE + ROTB * h) % CMB) * VE + n % VE;
    }
    // bf16 k-step kc of a k-major tile with LD columns: the two transposing
    // reads of k-rows 16kc + 8h + j and 16kc + 8h + 4 + j
    auto tr_frag = [&](const T* t, int col, int kc, int LD) {
        typedef short v4s __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;
        const lds_v4s_ptr p = (lds_v4s_ptr)t;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p + (col + 16 * kc * LD) / 4);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p + (col + (16 * kc + 4) * LD) / 4);
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
    };
    auto load_frags = [&](const T* sA, const T* sB, int kc, u32x4 (&fa)[TM], u32x4 (&fb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int row = wm * TM * 32 + i * 32 + r32;
            if constexpr (TA && KBF) {
                fa[i] = tr_frag(sA, colA[i], kc, BM);
            } else if constexpr (TA) {
                // fp32: element index = 32-bit word index
                const uint32_t* w = reinterpret_cast<const uint32_t*>(sA) + colA[i] + 8 * kc * BM;
#pragma unroll
                for (int e = 0; e < VE; e++) fa[i][e] = w[e * BM];
            } else {
                fa[i] = *reinterpret_cast<const u32x4*>(&sA[row * BK + (((2 * kc + h) ^ ((row / RP) % CH)) * VE)]);
            }
        }
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int row = wn * TN * 32 + j * 32 + r32;
            if constexpr (TB && KBF) {
                fb[j] = tr_frag(sB, colB[j], kc, BN);
            } else if constexpr (TB) {
                const uint32_t* w = reinterpret_cast<const uint32_t*>(sB) + colB[j] + 8 * kc * BN;
#pragma unroll
                for (int e = 0; e < VE; e++) fb[j][e] = w[e * BN];
            } else {
                fb[j] = *reinterpret_cast<const u32x4*>(&sB[row * BK + (((2 * kc + h) ^ ((row / RP) % CH)) * VE)]);
            }
        }
    };
    // EPI_ASUM: the waves of tile column 0 with wn == 0 (each A row once) add
    // up their A fragments: lane (h, r32) sums its k of row r32 (bf16:
    // 16kc + 8h .. +7; fp32: 8kc + 4h .. +3) of each of its TM row tiles; the
    // two halves are combined at the end.
    float asum[TM];
#pragma unroll
    for (int i = 0; i < TM; i++) asum[i] = 0.f;
    const bool asum_on = EPI == EPI_ASUM && n0 == 0 && wn == 0;
    auto compute = [&](const int stage) {
        const T* sA = smem + stage * STAGE;
        const T* sB = sA + BM * BK;
        u32x4 fa[2][TM], fb[2][TN];
        load_frags(sA, sB, 0, fa[0], fb[0]);
        if constexpr (SCHED == 1) __builtin_amdgcn_iglp_opt(0);
        if constexpr (SCHED == 2) __builtin_amdgcn_iglp_opt(1);
#pragma unroll
        for (int kc = 0; kc < CH / 2; kc++) {
            if constexpr (SCHED == 4) __builtin_amdgcn_sched_barrier(0);
            if (kc + 1 < CH / 2) load_frags(sA, sB, kc + 1, fa[(kc + 1) & 1], fb[(kc + 1) & 1]);
            if constexpr (SCHED == 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < Mfma32<T>::STEPS; e++)
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int j = 0; j < TN; j++)
                        Mfma32<T>::step(acc[i][j], fa[kc & 1][i], fb[kc & 1][j], e);
            if constexpr (EPI == EPI_ASUM) {
                if (asum_on) {
#pragma unroll
                    for (int i = 0; i < TM; i++) {
                        float t = 0.f;
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const uint32_t x = fa[kc & 1][i][e];
                            if constexpr (KBF) t += __uint_as_float(x << 16) + __uint_as_float(x & 0xffff0000u);
                            else t += __uint_as_float(x);
                        }
                        asum[i] += t;
                    }
                }
            }
        }
    };

    const int nk = K / BK;
#pragma unroll
    for (int t = 0; t < S - 1; t++)
        if (t < nk) issue(t, t * BK);
    // One k-tile per step: wait until only the later tiles' copies may still
    // be in flight (and this wave's LDS reads are done), barrier, launch the
    // tile S-1 ahead into the stage the previous step finished reading,
    // compute. Steps are unrolled S at a time so every stage offset is a
    // compile-time constant.
    auto step = [&](auto stage_c, int t) {
        constexpr int st = decltype(stage_c)::value;
        if (t + S - 2 < nk) {
            wait_vmcnt_lds<(S - 2) * LPW>();
        } else {
            const int ahead = nk - 1 - t;  // < S - 2 here
            if constexpr (S - 2 > 3) { if (ahead == 3) wait_vmcnt_lds<3 * LPW>(); }
            if constexpr (S - 2 > 2) { if (ahead == 2) wait_vmcnt_lds<2 * LPW>(); }
            if (ahead == 1) wait_vmcnt_lds<LPW>();
            if (ahead <= 0) wait_vmcnt_lds<0>();
        }
        __builtin_amdgcn_s_barrier();
        if (t + S - 1 < nk) issue((st + S - 1) % S, (t + S - 1) * BK);
        compute(st);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    int kt = 0;
    for (; kt + S <= nk; kt += S) {
        step(I0{}, kt);
        step(I1{}, kt + 1);
        if constexpr (S > 2) step(I2{}, kt + 2);
        if constexpr (S > 3) step(I3{}, kt + 3);
        if constexpr (S > 4) step(I4{}, kt + 4);
        if constexpr (S > 5) step(I5{}, kt + 5);
    }
    if (kt < nk) step(I0{}, kt);
    if (kt + 1 < nk) step(I1{}, kt + 1);
    if constexpr (S > 3) { if (kt + 2 < nk) step(I2{}, kt + 2); }
    if constexpr (S > 4) { if (kt + 3 < nk) step(I3{}, kt + 3); }
    if constexpr (S > 5) { if (kt + 4 < nk) step(I4{}, kt + 4); }

    if constexpr (EPI == EPI_ASUM) {
        if (asum_on) {
            float* dst = stats + (SPLITK ? (int64_t)blockIdx.y * M : 0);
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const float v = asum[i] + __shfl_xor(asum[i], 32, 64);
                const int m = m0 + wm * TM * 32 + i * 32 + r32;
                if (h == 0 && m < M) dst[m] = v;
            }
        }
    }

    // Epilogue through LDS: every copy has landed (the last step waited for
    // vmcnt 0); once all waves are past this barrier the stage memory is
    // free. Each wave adds the bias, rounds to T and writes its tiles into a
    // row-major [BM][BN] tile (rows padded by 16 bytes); the workgroup then
    // stores whole 16-byte row chunks, so a wavefront writes 1 KiB of
    // contiguous rows per instruction instead of 2- or 4-byte scattered
    // elements.
    if constexpr (STAGED) {
        __builtin_amdgcn_s_barrier();
        TO* so = reinterpret_cast<TO*>(smem);
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int cl = wn * TN * 32 + j * 32 + r32;
            const float bv = (bias && n0 + cl < N) ? load_scalar(bias + n0 + cl) : 0.f;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int rl = wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    float y = acc[i][j][v] + bv;
                    if constexpr (EPI == EPI_BIAS_GELU) y = gelu_tanh(storage_round(so, y));
                    store_scalar(&so[rl * LDO + cl], y);
                }
        }
        __builtin_amdgcn_s_waitcnt((0xF) | (7 << 4) | (0x0 << 8) | (3 << 14));  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        constexpr int CPR = BN / VO;  // 16-byte chunks per tile row
        if constexpr (EPI == EPI_BIAS_RESIDUAL || EPI == EPI_DGELU) {
            // every residual (GELU input) chunk of this thread is loaded
            // before the first use (rows and columns clamped into the matrix;
            // out-of-range chunks are then not stored), so the loads overlap
            constexpr int NCH = (BM * CPR + NW * 64 - 1) / (NW * 64);
            u32x4 rv[NCH];
#pragma unroll
            for (int j = 0; j < NCH; j++) {
                const int c = min(tid + j * NW * 64, BM * CPR - 1);
                const int row = min(m0 + c / CPR, M - 1), col = min(n0 + (c % CPR) * VO, N - VO);
                rv[j] = *reinterpret_cast<const u32x4*>(res + (int64_t)row * N + col);
            }
#pragma unroll
            for (int j = 0; j < NCH; j++) {
                const int c = tid + j * NW * 64;
                const int rl = c / CPR, cv = c % CPR;
                const int row = m0 + rl, col = n0 + cv * VO;
                if (c < BM * CPR && row < M && col < N) {
                    float a[VO], r[VO];
                    unpack_vec<TO>(*reinterpret_cast<const u32x4*>(&so[rl * LDO + cv * VO]), a);
                    unpack_vec<TO>(rv[j], r);
#pragma unroll
                    for (int e = 0; e < VO; e++) {
                        if constexpr (EPI == EPI_DGELU) a[e] *= gelu_tanh_grad(r[e]);
                        else a[e] += r[e];
                    }
                    store_vec(out + (int64_t)row * N + col, a);
                }
            }
        } else if constexpr (EPI == EPI_STATS) {
            // the stored tile, then one thread per (row, column group): the
            // max of the group's stored values of columns < vlim from LDS,
            // then the sum of e^{y - max} (hardware base-2 exponential of the
            // scaled difference) in a second pass. Consecutive lanes take
            // consecutive rows: 528-byte rows put them on distinct banks.
            static_assert(BN % kStatCols == 0, "stats groups must tile the output tile");
            constexpr int NG = BN / kStatCols, GCH = kStatCols / VO;
            const int ngrp = (N + kStatCols - 1) / kStatCols;
            const float L2E = 1.4426950408889634f;
#pragma unroll 4
            for (int c = tid; c < BM * CPR; c += NW * 64) {
                const int rl = c / CPR, cv = c % CPR;
                const int row = m0 + rl, col = n0 + cv * VO;
                if (row < M && col < N)
                    *reinterpret_cast<u32x4*>(out + (int64_t)row * N + col) =
                        *reinterpret_cast<const u32x4*>(&so[rl * LDO + cv * VO]);
            }
            for (int p = tid; p < BM * NG; p += NW * 64) {
                const int rl = p % BM, gi = p / BM;
                const int row = m0 + rl, c0 = n0 + gi * kStatCols, grp = c0 / kStatCols;
                const TO* src = &so[rl * LDO + gi * kStatCols];
                float mx = -INFINITY;
#pragma unroll 4
                for (int j = 0; j < GCH; j++) {
                    float y[VO];
                    unpack_vec<TO>(*reinterpret_cast<const u32x4*>(src + j * VO), y);
#pragma unroll
                    for (int e = 0; e < VO; e++)
                        if (c0 + j * VO + e < vlim) mx = fmaxf(mx, y[e]);
                }
                float sm = 0.f;
                if (mx != -INFINITY) {
#pragma unroll 4
                    for (int j = 0; j < GCH; j++) {
                        float y[VO];
                        unpack_vec<TO>(*reinterpret_cast<const u32x4*>(src + j * VO), y);
#pragma unroll
                        for (int e = 0; e < VO; e++)
                            sm += c0 + j * VO + e < vlim ? __builtin_amdgcn_exp2f((y[e] - mx) * L2E) : 0.f;
                    }
                }
                if (row < M && grp < ngrp) {
                    float* st = stats + ((int64_t)row * ngrp + grp) * 2;
                    st[0] = mx;
                    st[1] = sm;
                }
            }
        } else {
#pragma unroll 4
            for (int c = tid; c < BM * CPR; c += NW * 64) {
                const int rl = c / CPR, cv = c % CPR;
                const int row = m0 + rl, col = n0 + cv * VO;
                if (row < M && col < N) {
                    const u32x4 y = *reinterpret_cast<const u32x4*>(&so[rl * LDO + cv * VO]);
                    if constexpr (EPI == EPI_BIAS_NT)
                        __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(out + (int64_t)row * N + col));
                    else
                        *reinterpret_cast<u32x4*>(out + (int64_t)row * N + col) = y;
                    if constexpr (EPI == EPI_BIAS_GELU2) {
                        float a[VO];
                        unpack_vec<TO>(y, a);
#pragma unroll
                        for (int e = 0; e < VO; e++) a[e] = gelu_tanh(a[e]);
                        store_vec(out2 + (int64_t)row * N + col, a);
                    }
                }
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int col = n0 + wn * TN * 32 + j * 32 + r32;
            if (col >= N) continue;
            const float bv = bias ? load_scalar(bias + col) : 0.f;
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int row = m0 + wm * TM * 32 + i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    const float r = EPI == EPI_BIAS_RESIDUAL || EPI == EPI_DGELU
                                        ? load_scalar(res + (int64_t)min(row, M - 1) * N + col)
                                        : 0.f;
                    if (row < M) {
                        float y = acc[i][j][v] + bv;
                        if constexpr (EPI == EPI_BIAS_GELU) y = gelu_tanh(storage_round(out, y));
                        if constexpr (EPI == EPI_BIAS_RESIDUAL) y = storage_round(out, y) + r;
                        if constexpr (EPI == EPI_DGELU) y = storage_round(out, y) * gelu_tanh_grad(r);
                        store_scalar(out + (int64_t)row * N + col, y);
                        if constexpr (EPI == EPI_BIAS_GELU2)
                            store_scalar(out2 + (int64_t)row * N + col, gelu_tanh(storage_round(out, y)));
                    }
                }
        }
    }
}

template <typename T, int WM, int WN, int TM, int TN, int RB, int S, int SCHED, int WPE = 0, bool DIRECT = false>
static void launch_gemm_pipe(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                             int group_m, int remap, hipStream_t s, int epi = EPI_BIAS, const T* res = nullptr,
                             int lda = 0, int splits = 1, int64_t split_out = 0, float* stats = nullptr,
                             int vlim = 0, T* out2 = nullptr) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    const int nwg = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(nwg, splits);
    if (lda == 0) lda = K;
#define GEMM_PIPE_LAUNCH(E)                                                                              \
    gemm_pipe_kernel<T, WM, WN, TM, TN, RB, S, SCHED, WPE, DIRECT, E><<<grid, WM * WN * 64, 0, s>>>( \
        out, A, W, bias, res, M, N, K, group_m, remap, lda, lda, split_out, stats, vlim, out2)
    if (splits > 1 || lda != K) {
        gemm_pipe_kernel<T, WM, WN, TM, TN, RB, S, SCHED, WPE, DIRECT, EPI_BIAS, true>
            <<<grid, WM * WN * 64, 0, s>>>(out, A, W, bias, res, M, N, K, group_m, remap, lda, lda, split_out,
                                           nullptr, 0, static_cast<T*>(nullptr));
        return;
    }
    if constexpr (BN % kStatCols == 0) {
        if (epi == EPI_STATS) {
            GEMM_PIPE_LAUNCH(EPI_STATS);
            return;
        }
    }
    if (epi == EPI_BIAS_GELU) GEMM_PIPE_LAUNCH(EPI_BIAS_GELU);
    else if (epi == EPI_BIAS_RESIDUAL) GEMM_PIPE_LAUNCH(EPI_BIAS_RESIDUAL);
    else if (epi == EPI_DGELU) GEMM_PIPE_LAUNCH(EPI_DGELU);
    else if (epi == EPI_BIAS_GELU2) GEMM_PIPE_LAUNCH(EPI_BIAS_GELU2);
    else if (epi == EPI_BIAS_NT) GEMM_PIPE_LAUNCH(EPI_BIAS_NT);
    else GEMM_PIPE_LAUNCH(EPI_BIAS);
#undef GEMM_PIPE_LAUNCH
}

// k-major operand variants: out [M,N] (+ y*split_out per k-slice y of depth
// K) from A ([K][M] rows lda apart if TA, else [M][K]) and W ([K][N] rows ldb
// apart if TB, else [N][K]); bias only without split. TO: the output type.
template <int WM, int WN, int TM, int TN, int RB, int S, int SCHED, int WPE, bool TA, bool TB, typename T,
          typename TO, int EPI = EPI_BIAS>
static void launch_gemm_kmajor(TO* out, const T* A, const T* W, const typename std::enable_if<true, T>::type* bias,
                               int M, int N, int K, int lda, int ldb,
                               int splits, int64_t split_out, int group_m, int remap, hipStream_t s,
                               float* stats = nullptr, const TO* res = nullptr) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    const int nwg = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const dim3 grid(nwg, splits);
    gemm_pipe_kernel<T, WM, WN, TM, TN, RB, S, SCHED, WPE, false, EPI, true, TA, TB, TO>
        <<<grid, WM * WN * 64, 0, s>>>(out, A, W, bias, res, M, N, K, group_m, remap, lda, ldb, split_out, stats,
                                       0, nullptr);
}

template <typename T, int WM, int WN, int TM, int TN, int SCHED = 4>
static void launch_gemm_lds3(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                             int group_m, int remap, hipStream_t s) {
    launch_gemm_pipe<T, WM, WN, TM, TN, 128, 3, SCHED>(out, A, W, bias, M, N, K, group_m, remap, s);
}

template <typename T, int WM, int WN, int TM, int TN, int BK, bool ILV = true>
static void launch_gemm_cfg(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                            int group_m, int remap, hipStream_t s, int epi = EPI_BIAS, const T* res = nullptr) {
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    const int nwg = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
#define GEMM_CFG_LAUNCH(E) \
    gemm_kernel<T, WM, WN, TM, TN, BK, ILV, E><<<nwg, WM * WN * 64, 0, s>>>(out, A, W, bias, res, M, N, K, group_m, remap)
    if (epi == EPI_BIAS_GELU) GEMM_CFG_LAUNCH(EPI_BIAS_GELU);
    else if (epi == EPI_BIAS_RESIDUAL) GEMM_CFG_LAUNCH(EPI_BIAS_RESIDUAL);
    else if (epi == EPI_DGELU) GEMM_CFG_LAUNCH(EPI_DGELU);
    else GEMM_CFG_LAUNCH(EPI_BIAS);
#undef GEMM_CFG_LAUNCH
}

// 16x16 MFMA step: bf16 16x16x32 (one 16-byte piece per lane) or fp32
// 16x16x4 (one float of the piece per step). Lane l supplies row l%16 of its
// operand at k-group l/16; accumulator element i of lane l is row 4*(l/16)+i,
// column l%16.
template <typename T> struct Mfma16;
template <> struct Mfma16<float> {
    static constexpr int STEPS = 4;
    static __device__ __forceinline__ void step(f32x4& acc, const u32x4& a, const u32x4& b, int e) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
    }
};
template <> struct Mfma16<bf16> {
    static constexpr int STEPS = 1;
    static __device__ __forceinline__ void step(f32x4& acc, const u32x4& a, const u32x4& b, int) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      acc, 0, 0, 0);
    }
};

// Skinny GEMM for M <= 32 rows (a decode step: one row per sequence). Its
// cost is one pass over W plus fixed latency. Every operand byte arrives
// through direct-to-LDS copies in which eight consecutive lanes fetch one
// 128-byte line of a row (each copy instruction moves eight whole lines);
// each lane then reads its 16x16 MFMA pieces from LDS. Rows are stored with
// their 16-byte slots permuted by (row/2) mod 8, so the sixteen rows one
// fragment read touches fall in distinct bank groups. Piece (s, g) of a
// 128-byte chunk is slot 4s + g for both operands: one k map, so the
// contraction is unchanged. Rows past M or N read row 0 (their results are
// never stored); k past K reads a clamped address and is zeroed at use.
//
// Grid (column tiles of 32, splits): workgroup (x, y) reduces k-chunks
// [y*cps, (y+1)*cps) with cps = ceil(chunks/splits); within it each of the NW
// wavefronts takes a contiguous run, PF chunks per batch, in its own LDS
// stages (PF x 8 KiB per wave); the NW partial tiles are summed through LDS
// in wave order. With part == nullptr (then splits == 1) it writes
// out = EPI(bias + sum) (res: the residual of EPI_BIAS_RESIDUAL, may be out);
// otherwise it writes the fp32 partial sums part[y][M][N] (no bias), which
// the consumer adds in split order.
// ACOMB: A is the output of a split decode attention, given as its fp32
// partials apart[(row*NH + head)*asplits + s] = (o[hs], m, l) (NH = K/hs,
// 1 <= asplits <= kAcombMax); each lane merges its 16-byte piece of A from
// them (the arithmetic and order of decode_combine_kernel, rounded to T)
// and writes it where the load-to-LDS copy would have put it.
constexpr int kAcombMax = 2;
template <typename T, int NW, int PF, int EPI, bool ACOMB = false>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_lds_kernel(T* out, float* __restrict__ part,
                                                                  const T* __restrict__ A,
                                                                  const T* __restrict__ W,
                                                                  const T* __restrict__ bias, const T* res, int M,
                                                                  int N, int K, const float* __restrict__ apart,
                                                                  int asplits, int hs) {
    constexpr int VE = Vec<T>::N;
    constexpr int CK = 128 / (int)sizeof(T);  // k per chunk: one 128-byte line per row
    constexpr int TILE = 32 * 128;            // bytes of one 32-row chunk tile
    static_assert(NW * PF * 2 * TILE <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) char smem[NW * PF * 2 * TILE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int n0 = blockIdx.x * 32;
    const int splits = gridDim.y;
    const int nchunk = (K + CK - 1) / CK;
    const int cps = (nchunk + splits - 1) / splits;
    const int kb = min((int)blockIdx.y * cps, nchunk), ke = min(kb + cps, nchunk);
    const int per = (ke - kb + NW - 1) / NW;
    const int c_begin = min(kb + w * per, ke), c_end = min(c_begin + per, ke);

    // Copy q (0..3) of a tile: lane i fetches slot (i%8) ^ ((row/2)%8) of row
    // 8q + i/8 into LDS byte 1024q + 16i.
    const T* srcA[4];
    const T* srcW[4];
    int gsl[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int row = 8 * q + (lane >> 3);
        gsl[q] = ((lane & 7) ^ ((row >> 1) & 7)) * VE;
        srcA[q] = ACOMB ? nullptr : A + (int64_t)(row < M ? row : 0) * K;
        srcW[q] = W + (int64_t)(n0 + row < N ? n0 + row : 0) * K;
    }
    float bcol[2] = {0.f, 0.f};
    if (bias && !part) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int col = n0 + 16 * j + (lane & 15);
            const float bv = load_scalar(bias + min(col, N - 1));  // unconditional: no wait here
            bcol[j] = col < N ? bv : 0.f;
        }
    }
    char* wbase = smem + w * (PF * 2 * TILE);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = c_begin; c0 < c_end; c0 += PF) {
        wait_vmcnt_lds<0>();  // the previous batch's fragment reads are complete
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const int c = min(c0 + p, c_end - 1);
            char* st = wbase + p * 2 * TILE;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int off = min(c * CK + gsl[q], K - VE);  // K % 8 == 0: slots are whole
                if constexpr (!ACOMB) copy16_to_lds(srcA[q] + off, (lds_void_ptr)(st + q * 1024));
                copy16_to_lds(srcW[q] + off, (lds_void_ptr)(st + TILE + q * 1024));
            }
            if constexpr (ACOMB) {
                // after the W copies are in flight: row 8q + lane/8, elements
                // off .. off+VE-1 (one head, hs % VE == 0) of the merged output.
                // Every partial load of the batch is issued before the first
                // use (8-byte loads: records are hs + 2 floats, hs % 8 == 0;
                // rows past M read row 0 and are not used).
                float2 pm[4][kAcombMax], po[4][kAcombMax][VE / 2];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int row = 8 * q + (lane >> 3);
                    const int off = min(c * CK + gsl[q], K - VE);
                    const int hd = off / hs, d0 = off % hs;
                    const float* pp = apart + ((int64_t)(row < M ? row : 0) * (K / hs) + hd) * asplits * (hs + 2);
#pragma unroll
                    for (int sp = 0; sp < kAcombMax; sp++) {
                        const float* rec = pp + min(sp, asplits - 1) * (hs + 2);
                        pm[q][sp] = *reinterpret_cast<const float2*>(rec + hs);
#pragma unroll
                        for (int e = 0; e < VE / 2; e++)
                            po[q][sp][e] = *reinterpret_cast<const float2*>(rec + d0 + 2 * e);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int row = 8 * q + (lane >> 3);
                    float mx = -INFINITY;
#pragma unroll
                    for (int sp = 0; sp < kAcombMax; sp++)
                        if (sp < asplits) mx = fmaxf(mx, pm[q][sp].x);
                    float L = 0.f, o[VE];
#pragma unroll
                    for (int e = 0; e < VE; e++) o[e] = 0.f;
#pragma unroll
                    for (int sp = 0; sp < kAcombMax; sp++) {
                        if (sp < asplits) {
                            const float m = pm[q][sp].x;
                            const float wgt = m == -INFINITY ? 0.f : exp2f(m - mx);
                            L += pm[q][sp].y * wgt;
#pragma unroll
                            for (int e = 0; e < VE / 2; e++) {
                                o[2 * e] += po[q][sp][e].x * wgt;
                                o[2 * e + 1] += po[q][sp][e].y * wgt;
                            }
                        }
                    }
                    u32x4 v = zero;
                    if (row < M) {
#pragma unroll
                        for (int e = 0; e < VE; e++) o[e] = o[e] / L;
                        if constexpr (std::is_same<T, float>::value) {
#pragma unroll
                            for (int e = 0; e < 4; e++) v[e] = __float_as_uint(o[e]);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; e++) v[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
                        }
                    }
                    *reinterpret_cast<u32x4*>(st + q * 1024 + lane * 16) = v;
                }
            }
        }
        wait_vmcnt_lds<0>();
#pragma unroll
        for (int p = 0; p < PF; p++) {
            const char* st = wbase + p * 2 * TILE;
#pragma unroll
            for (int sh = 0; sh < 2; sh++) {
                const int slot = sh * 4 + g;
                const bool ok = c0 + p < c_end && (c0 + p) * CK + slot * VE < K;
                u32x4 a[2], b[2];
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const int row = 16 * i + r16;
                    const int sw = (slot ^ ((row >> 1) & 7)) * 16;
                    a[i] = *reinterpret_cast<const u32x4*>(st + row * 128 + sw);
                    b[i] = *reinterpret_cast<const u32x4*>(st + TILE + row * 128 + sw);
                    a[i] = ok ? a[i] : zero;
                    b[i] = ok ? b[i] : zero;
                }
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++)
#pragma unroll
                        for (int e = 0; e < Mfma16<T>::STEPS; e++) Mfma16<T>::step(acc[i][j], a[i], b[j], e);
            }
        }
    }
    __syncthreads();  // the reduction buffer reuses the stages
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 4; v++) red[(w * 16 + (i * 2 + j) * 4 + v) * 64 + lane] = acc[i][j][v];
    __syncthreads();
    // Entry (i, j, v) of lane l is row 16i + 4*(l/16) + v, column 16j + l%16.
#pragma unroll
    for (int idx = tid; idx < 16 * 64; idx += NW * 64) {
        const int q = idx / 64;
        const int i = q >> 3, j = (q >> 2) & 1, v = q & 3;
        const int row = 16 * i + 4 * (lane >> 4) + v, col = n0 + 16 * j + (lane & 15);
        if (row < M && col < N) {
            float x = 0.f;
            for (int ww = 0; ww < NW; ww++) x += red[(ww * 16 + q) * 64 + lane];
            if (part) {
                part[((int64_t)blockIdx.y * M + row) * N + col] = x;
            } else {
                x += bcol[j];
                if constexpr (EPI == EPI_BIAS_GELU) x = gelu_tanh(storage_round(out, x));
                if constexpr (EPI == EPI_BIAS_RESIDUAL)
                    x = storage_round(out, x) + load_scalar(res + (int64_t)row * N + col);
                if constexpr (EPI == EPI_DGELU)
                    x = storage_round(out, x) * gelu_tanh_grad(load_scalar(res + (int64_t)row * N + col));
                store_scalar(out + (int64_t)row * N + col, x);
            }
        }
    }
}

}  // namespace gpt2
