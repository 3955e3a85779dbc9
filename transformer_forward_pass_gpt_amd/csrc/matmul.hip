// Linear layer entry: out[n,o] = sum_c inp[n,c] * W[o,c] + bias[o], on the
// MFMA GEMM of gemm.h with a tile shape chosen per problem size.
#include <stdio.h>

#include <type_traits>

#include "gemm.h"

namespace gpt2 {

static constexpr int kMaxSplits = 8;  // split-k ranges of the decode projections

// Skinny (M <= 32) problems: the LDS-staged kernel, 8 wavefronts, one chunk
// per load batch (the fastest variant on every decode shape swept on MI355X).
template <typename T>
static void launch_skinny(T* out, float* part, const T* A, const T* W, const T* bias, const T* res, int M, int N,
                          int K, int splits, int epi, hipStream_t s) {
    const dim3 grid((N + 31) / 32, splits);
#define SKINNY_LAUNCH(E) \
    gemm_skinny_lds_kernel<T, 8, 1, E><<<grid, 512, 0, s>>>(out, part, A, W, bias, res, M, N, K, nullptr, 0, 0)
    if (epi == EPI_BIAS_GELU) SKINNY_LAUNCH(EPI_BIAS_GELU);
    else if (epi == EPI_BIAS_RESIDUAL) SKINNY_LAUNCH(EPI_BIAS_RESIDUAL);
    else if (epi == EPI_DGELU) SKINNY_LAUNCH(EPI_DGELU);
    else SKINNY_LAUNCH(EPI_BIAS);
#undef SKINNY_LAUNCH
}

// Tile shapes, chosen per problem from on-box sweeps (MI355X) over the GPT-2
// small and medium layer shapes. The pipelined kernel (S LDS stages filled by
// load-to-LDS copies, k-tile rows of RB bytes) runs whenever K is a whole
// number of k-tiles; otherwise the register-staged kernel with a masked k
// tail. Problems of at most 32 rows (decode) stream W with the skinny kernel.
struct PipeCfg {
    const char* name;
    int bk_bytes;  // RB: bytes of k per tile row
};
enum GemmCfg {
    S32 = 0, R64x64, R64x128, R128x96,
    P128x96_S4, P128x96_S5, P256x128_S3A, P128x128_O2, P128x288_I, P128x192_R4,  // fp32
    P128x256_O4, P128x256_R3, P256x128_G, P128x128_R4, P128x128_K3, P256x256_K2, P128x192_K2,  // bf16
    P128x192_K3, P256x192_K2,                                                                     // bf16
    G_NCFG
};
// fp32 128x288_p3: 4 wavefronts of 32x288 (nine accumulator tiles each), so GPT-2 small's qkv
// (2304 wide) is 256 tiles, one round of the CUs; three stages fill 156 KiB of LDS;
// 128x192_p4_r64: four stages of 64-byte rows.
// "_p<S>" = S-stage pipeline; "_o<n>" = registers capped so n wavefronts fit per SIMD (2 or 3
// workgroups per CU); "_k128" = 128-byte k-rows per stage (twice the default bf16 depth); "g" =
// grouped XCD-aware walk (the fp32 vocabulary tile walks columns instead). 256x256_p2_k128:
// 8 wavefronts of 128x64, two stages of 128-byte rows (the L2 sees one 128-byte request per
// row per k-tile instead of two 64-byte ones; the same bytes in flight as three 64-byte stages).
// 128x192_p2_k128: two stages of 128-byte rows in 80 KiB, so two workgroups fill a CU's LDS;
// 128x192_p3_k128: three stages (one workgroup per CU) for the 768-wide projections at 8192
// rows; 256x192_p2_k128: 8 wavefronts of 64x96, chosen where its tile count fills whole rounds.
static const PipeCfg kCfg[G_NCFG] = {
    {"skinny32", 0},          {"64x64_r", 0},          {"64x128_r", 0},         {"128x96_r", 0},
    {"128x96_p4", 128},       {"128x96_p5", 128},      {"256x128_p3", 128},     {"128x128_p4_o2", 64},
    {"128x288_p3", 128},      {"128x192_p4_r64", 64},
    {"128x256_p3_o4", 64},    {"128x256_p3_k128", 128}, {"256x128_p3g", 128},
    {"128x128_p4_k128", 128}, {"128x128_p3_k128", 128}, {"256x256_p2_k128", 128},
    {"128x192_p2_k128", 128}, {"128x192_p3_k128", 128}, {"256x192_p2_k128", 128},
};

static GemmCfg choose_pipe(int M, int N, int K, int dtype) {
    if (dtype == GPT2_F32) {
        if (N >= 16384) return P256x128_S3A;                 // vocabulary projection
        if (K >= 2048) return P128x96_S5;                    // fcproj
        if (N <= 1024) return P128x96_S4;                    // attproj
        if (N % 288 == 0) return P128x288_I;                 // qkv at GPT-2 small's width
        if (N % 192 == 0) return P128x192_R4;                // fc at GPT-2 small's width
        return N >= 3072 ? P128x128_O2 : P128x96_S5;         // fc, qkv
    }
    // bf16, chosen with operands cold in HBM, as in the forward (a pipeline
    // tuned on cache-resident operands loses 10-30% there): wide projections
    // use two resident two-stage 128x192 workgroups per CU where the width
    // allows, else 128x256 (two per CU) or two-stage 256x256 tiles; every
    // 128-byte-row tile halves the L2 requests of a 64-byte-row one.
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (N >= 16384) return P256x256_K2;                         // vocabulary projection
    if (K >= 2048) {  // fcproj (and the training step's vocabulary input gradient, K = Vp):
        // enough tiles for the 256 CUs at GPT-2 small's width
        if (M >= 8192) return N % 192 == 0 ? P128x192_K3 : P128x256_R3;
        return N <= 768 ? P128x96_S4 : P128x128_R4;
    }
    if (N <= 1024) {  // attproj
        if (M >= 8192) return N % 192 == 0 ? P128x192_K3 : P128x256_R3;
        return N <= 768 ? P128x96_S4 : P128x128_K3;
    }
    if (N % 192 == 0) {  // qkv, fc at GPT-2 small and medium widths
        if (tiles(256, 192) % 256 == 0) return P256x192_K2;     // whole rounds of the 256 CUs
        return M >= 8192 ? P128x192_R4 : P128x192_K2;
    }
    return M >= 8192 ? P128x256_O4 : P256x256_K2;               // qkv, fc
}

static GemmCfg choose_cfg(int M, int N, int K, int dtype) {
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (M > 32) {
        const GemmCfg p = choose_pipe(M, N, K, dtype);
        const int bk = kCfg[p].bk_bytes / (dtype == GPT2_BF16 ? 2 : 4);
        if (K % bk == 0) return p;
        if (tiles(128, 96) >= 1024) return R128x96;
        return tiles(64, 128) >= 256 ? R64x128 : R64x64;
    }
    return S32;
}

// out2: the second output of EPI_BIAS_GELU2 (pipelined tiles only; the
// caller checks matmul_gelu2_supported).
template <typename T>
static void launch_gemm_t(T* out, const T* A, const T* W, const T* bias, const T* res, int M, int N, int K,
                          int dtype, int epi, hipStream_t s, T* out2 = nullptr) {
    constexpr int BK = Vec<T>::N * 8;  // 128 bytes of k per row per LDS tile
    // vocabulary-wide outputs (hundreds of MB) are stored past the caches
    if (epi == EPI_BIAS && N >= 16384) epi = EPI_BIAS_NT;
    switch (choose_cfg(M, N, K, dtype)) {
        case S32: launch_skinny<T>(out, nullptr, A, W, bias, res, M, N, K, 1, epi, s); break;
        // launch_gemm_cfg<T, WM, WN, TM, TN, BK>(..., group_m, remap, s, epi, res)
        case R64x64: launch_gemm_cfg<T, 2, 2, 1, 1, BK>(out, A, W, bias, M, N, K, 4, 1, s, epi, res); break;
        case R64x128: launch_gemm_cfg<T, 2, 2, 1, 2, BK>(out, A, W, bias, M, N, K, 8, 1, s, epi, res); break;
        case R128x96: launch_gemm_cfg<T, 4, 1, 1, 3, BK>(out, A, W, bias, M, N, K, 8, 1, s, epi, res); break;
        // launch_gemm_pipe<T, WM, WN, TM, TN, RB, S, SCHED, WPE>(..., group_m, remap, s, epi, res)
#define PIPE(WM, WN, TM, TN, RB, S, SC, WPE, G, R) \
    launch_gemm_pipe<T, WM, WN, TM, TN, RB, S, SC, WPE>(out, A, W, bias, M, N, K, G, R, s, epi, res, 0, 1, 0, \
                                                        nullptr, 0, out2)
        case P128x96_S4: PIPE(4, 1, 1, 3, 128, 4, 4, 0, 8, 1); break;
        case P128x96_S5: PIPE(4, 1, 1, 3, 128, 5, 4, 0, 8, 1); break;
        case P256x128_S3A: PIPE(4, 2, 2, 2, 128, 3, 2, 0, 1, 0); break;
        case P128x128_O2: PIPE(2, 2, 2, 2, 64, 4, 2, 2, 4, 1); break;
        case P128x288_I: PIPE(4, 1, 1, 9, 128, 3, 2, 0, 8, 1); break;
        case P128x192_R4: PIPE(2, 2, 2, 3, 64, 4, 2, 0, 4, 1); break;
        default:
            if constexpr (std::is_same<T, bf16>::value) {  // the bf16-only shapes (choose_pipe)
                switch (choose_cfg(M, N, K, dtype)) {
                    case P128x256_O4: PIPE(2, 4, 2, 2, 64, 3, 2, 4, 4, 1); break;
                    case P128x256_R3: PIPE(2, 4, 2, 2, 128, 3, 2, 0, 4, 1); break;
                    case P256x128_G: PIPE(4, 2, 2, 2, 128, 3, 2, 0, 8, 1); break;
                    case P128x128_R4: PIPE(2, 2, 2, 2, 128, 4, 2, 0, 8, 1); break;
                    case P128x128_K3: PIPE(2, 2, 2, 2, 128, 3, 2, 0, 8, 1); break;
                    case P128x192_K2: PIPE(2, 2, 2, 3, 128, 2, 2, 2, 4, 1); break;
                    case P128x192_K3: PIPE(2, 2, 2, 3, 128, 3, 2, 0, 4, 1); break;
                    case P256x192_K2: PIPE(4, 2, 2, 3, 128, 2, 2, 0, 4, 1); break;
                    default:
                        if (N >= 16384 && M >= 8192)  // vocabulary, 8192+ rows: pairs of row
                            PIPE(2, 4, 4, 2, 128, 2, 2, 0, 2, 1);  // bands, XCD-contiguous ranges
                        else if (N >= 16384)  // vocabulary: column sweep within each row band
                            PIPE(2, 4, 4, 2, 128, 2, 2, 0, 1, 0);
                        else
                            PIPE(2, 4, 4, 2, 128, 2, 2, 0, 4, 1);
                        break;
                }
            }
            break;
#undef PIPE
    }
}

static thread_local char g_cfg_name[64];

const char* matmul_config_name(int N, int C, int OC, int dtype) {
    snprintf(g_cfg_name, sizeof g_cfg_name, "gemm_%s_%s", dtype == GPT2_BF16 ? "bf16" : "f32",
             kCfg[choose_cfg(N, OC, C, dtype)].name);
    return g_cfg_name;
}

// out = epi(inp W^T + bias [, res]); res (the residual of EPI_BIAS_RESIDUAL,
// the GELU input of EPI_DGELU) may alias out.
int launch_matmul_epi(void* out, const void* inp, const void* weight, const void* bias, const void* res, int N,
                      int C, int OC, int epi, int dtype, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_gemm_t<bf16>((bf16*)out, (const bf16*)inp, (const bf16*)weight, (const bf16*)bias,
                            (const bf16*)res, N, OC, C, dtype, epi, s);
    else
        launch_gemm_t<float>((float*)out, (const float*)inp, (const float*)weight, (const float*)bias,
                             (const float*)res, N, OC, C, dtype, epi, s);
    return launch_status();
}

// out = inp W^T + bias and out2 = GELU(out), both rounded to the storage
// type, in one product (EPI_BIAS_GELU2) when its tile is a pipelined one;
// GPT2_ERR_UNSUPPORTED otherwise (the caller then runs the product and
// launch_gelu).
int launch_matmul_gelu2(void* out, void* out2, const void* inp, const void* weight, const void* bias, int N, int C,
                        int OC, int dtype, hipStream_t s) {
    if (choose_cfg(N, OC, C, dtype) < P128x96_S4) return GPT2_ERR_UNSUPPORTED;  // skinny / register-staged
    if (dtype == GPT2_BF16)
        launch_gemm_t<bf16>((bf16*)out, (const bf16*)inp, (const bf16*)weight, (const bf16*)bias, nullptr, N, OC,
                            C, dtype, EPI_BIAS_GELU2, s, (bf16*)out2);
    else
        launch_gemm_t<float>((float*)out, (const float*)inp, (const float*)weight, (const float*)bias, nullptr, N,
                             OC, C, dtype, EPI_BIAS_GELU2, s, (float*)out2);
    return launch_status();
}

int launch_matmul(void* out, const void* inp, const void* weight, const void* bias, int N, int C,
                  int OC, int dtype, hipStream_t s) {
    return launch_matmul_epi(out, inp, weight, bias, nullptr, N, C, OC, EPI_BIAS, dtype, s);
}

// Vocabulary projection with row statistics (no bias): out [M,N] = A W^T and
// stats [M, ceil(N/kStatCols), 2] = (max, sum of e^{y - max}) of the stored
// y over each group's columns < vlim. Always the vocabulary tiles (fp32
// 256x128, bf16 256x256), whose rows are 32 16-byte chunks. K must be a whole
// number of 128-byte k-tiles (fp32 K % 32, bf16 K % 64).
bool matmul_stats_supported(int K, int dtype) { return K > 0 && K % (dtype == GPT2_BF16 ? 64 : 32) == 0; }

int launch_matmul_stats(void* out, float* stats, const void* inp, const void* weight, int M, int K, int N, int vlim,
                        int dtype, hipStream_t s) {
    if (!matmul_stats_supported(K, dtype)) return GPT2_ERR_UNSUPPORTED;
    if (dtype == GPT2_BF16)
        launch_gemm_pipe<bf16, 2, 4, 4, 2, 128, 2, 2, 0>((bf16*)out, (const bf16*)inp, (const bf16*)weight, nullptr,
                                                         M, N, K, 1, 0, s, EPI_STATS, nullptr, 0, 1, 0, stats, vlim);
    else
        launch_gemm_pipe<float, 4, 2, 2, 2, 128, 3, 2, 0>((float*)out, (const float*)inp, (const float*)weight,
                                                          nullptr, M, N, K, 1, 0, s, EPI_STATS, nullptr, 0, 1, 0,
                                                          stats, vlim);
    return launch_status();
}

// Split-k partial products (fp32): part[s] [M,N] = A_s W_s^T for s < splits,
// where A_s, W_s are the columns s*Kc .. s*Kc+Kc-1 of A [M, lda] and
// W [N, lda]; one launch, splits x tiles workgroups. For weight gradients,
// whose M x N output has too few tiles for the chip while K (the tokens) is
// deep. Kc % 32 == 0.
int launch_matmul_splitk_part(float* part, const float* A, const float* W, int M, int N, int Kc, int lda,
                              int splits, hipStream_t s) {
    if (Kc % 32 || splits < 1 || (int64_t)Kc * splits > lda) return GPT2_ERR_INVALID_ARGUMENT;
    launch_gemm_pipe<float, 4, 1, 1, 3, 128, 4, 4>(part, A, W, nullptr, M, N, Kc, 8, 1, s, EPI_BIAS, nullptr, lda,
                                                   splits, (int64_t)M * N);
    return launch_status();
}

// The same with bf16 operands: fp32 partial products (no rounding to bf16
// before the fp32 sum of the slices), 128x128 tiles; Kc % 64 == 0.
int launch_matmul_splitk_part(float* part, const bf16* A, const bf16* W, int M, int N, int Kc, int lda, int splits,
                              hipStream_t s) {
    if (Kc % 64 || splits < 1 || (int64_t)Kc * splits > lda) return GPT2_ERR_INVALID_ARGUMENT;
    const int nwg = ((M + 127) / 128) * ((N + 127) / 128);
    gemm_pipe_kernel<bf16, 2, 2, 2, 2, 128, 3, 2, 0, false, EPI_BIAS, true, false, false, float>
        <<<dim3(nwg, splits), 256, 0, s>>>(part, A, W, nullptr, nullptr, M, N, Kc, 8, 1, lda, lda, (int64_t)M * N,
                                           nullptr, 0, nullptr);
    return launch_status();
}

// fp32 products with k-major operands (no transpose pass): out [M,N] (slice y
// of `splits` at out + y*M*N) = sum over k of A(k, m) W(k, n), A stored
// [K][M] (rows lda apart) when ta else [M][K] (lda = K), W stored [K][N]
// (rows ldb apart) when tb else [N][K]. K (per slice) % 32 == 0; M % 4 == 0
// when ta, N % 4 == 0 when tb. gelu_in (nullable; W k-major alone, one
// slice): the EPI_DGELU epilogue with that [M,N] GELU input. asum (nullable;
// both k-major): asum[y*M + m] = the sum of A(k, m) over slice y's k-range
// (EPI_ASUM).
int launch_matmul_kmajor(float* out, const float* A, const float* W, int M, int N, int K, int lda, int ldb, bool ta,
                         bool tb, int splits, hipStream_t s, const float* gelu_in, float* asum) {
    if (K % 32 || splits < 1 || (ta && M % 4) || (tb && N % 4)) return GPT2_ERR_INVALID_ARGUMENT;
    const int64_t so = (int64_t)M * N;
    if (asum) {
        if (!ta || !tb || gelu_in) return GPT2_ERR_INVALID_ARGUMENT;
        launch_gemm_kmajor<4, 1, 1, 3, 128, 4, 4, 0, true, true, float, float, EPI_ASUM>(
            out, A, W, nullptr, M, N, K, lda, ldb, splits, so, 8, 1, s, asum);
        return launch_status();
    }
    if (gelu_in) {
        if (ta || !tb || splits != 1) return GPT2_ERR_INVALID_ARGUMENT;
        launch_gemm_kmajor<4, 1, 1, 3, 128, 4, 4, 0, false, true, float, float, EPI_DGELU>(
            out, A, W, nullptr, M, N, K, lda, ldb, 1, so, 8, 1, s, nullptr, gelu_in);
        return launch_status();
    }
    if (ta && tb)
        launch_gemm_kmajor<4, 1, 1, 3, 128, 4, 4, 0, true, true>(out, A, W, nullptr, M, N, K, lda, ldb, splits, so, 8,
                                                                1, s);
    else if (tb)
        launch_gemm_kmajor<4, 1, 1, 3, 128, 4, 4, 0, false, true>(out, A, W, nullptr, M, N, K, lda, ldb, splits, so, 8,
                                                                 1, s);
    else if (ta)
        launch_gemm_kmajor<4, 1, 1, 3, 128, 4, 4, 0, true, false>(out, A, W, nullptr, M, N, K, lda, ldb, splits, so, 8,
                                                                 1, s);
    else
        return GPT2_ERR_INVALID_ARGUMENT;
    return launch_status();
}

// bf16 weight-gradient products, both operands k-major (no transpose pass),
// fp32 accumulation: slice y of `splits` (k-range y*K .. y*K+K-1) gives
// part + y*M*N (fp32 partial sums); the bf16 overload writes out [M,N] in one
// slice. A stored [K][M] (rows lda apart), W stored [K][N] (rows ldb apart),
// out = A^T W. asum (nullable, partial-sum form only): asum[y*M + m] = the
// sum of A(k, m) over slice y's k-range (fp32), taken from the fragments the
// product reads. K (per slice) % 64 == 0, M % 8 == 0, N % 8 == 0. 128x128
// tiles, two stages in 64 KiB, so two workgroups share a CU (on MI355X this
// beat 3- and 4-stage single-resident and 128x256 / 256x128 tiles on every
// GPT-2 weight-gradient shape swept, with the split counts of the caller).
template <typename TO>
static int launch_kmajor_bf16(TO* out, const bf16* A, const bf16* W, int M, int N, int K, int lda, int ldb, bool ta,
                              bool tb, int splits, float* asum, hipStream_t s) {
    if (!ta || !tb || K % 64 || K <= 0 || splits < 1 || M % 8 || N % 8) return GPT2_ERR_INVALID_ARGUMENT;
    if constexpr (std::is_same<TO, float>::value) {
        if (asum) {
            launch_gemm_kmajor<2, 2, 2, 2, 128, 2, 2, 0, true, true, bf16, TO, EPI_ASUM>(
                out, A, W, nullptr, M, N, K, lda, ldb, splits, (int64_t)M * N, 8, 1, s, asum);
            return launch_status();
        }
    }
    launch_gemm_kmajor<2, 2, 2, 2, 128, 2, 2, 0, true, true>(out, A, W, nullptr, M, N, K, lda, ldb, splits,
                                                            (int64_t)M * N, 8, 1, s);
    return launch_status();
}

int launch_matmul_kmajor(float* part, const bf16* A, const bf16* W, int M, int N, int K, int lda, int ldb, bool ta,
                         bool tb, int splits, float* asum, hipStream_t s) {
    return launch_kmajor_bf16(part, A, W, M, N, K, lda, ldb, ta, tb, splits, asum, s);
}

int launch_matmul_kmajor(bf16* out, const bf16* A, const bf16* W, int M, int N, int K, int lda, int ldb, bool ta,
                         bool tb, int splits, hipStream_t s) {
    if (splits != 1) return GPT2_ERR_INVALID_ARGUMENT;
    return launch_kmajor_bf16(out, A, W, M, N, K, lda, ldb, ta, tb, 1, static_cast<float*>(nullptr), s);
}

// Decode-step projection of a split attention's output (at most 32 rows):
// part[y][M][N] (fp32 partial sums over `splits` k-ranges, no bias) of A W^T
// with A [M, K] the merge of the attention's fp32 partials apart (per row and
// head of size hs, asplits chunks of (o[hs], m, l)), merged while the product
// loads them: the attention's separate combine launch is not needed. K % 8 == 0,
// hs % 8 == 0, K % hs == 0, 1 <= asplits <= skinny_acomb_max_splits().
int launch_skinny_gemm_acomb(float* part, const float* apart, int asplits, int hs, const void* weight, int M, int K,
                             int N, int splits, int dtype, hipStream_t s) {
    if (M < 1 || M > 32 || K % 8 || hs < 8 || hs % 8 || K % hs || splits < 1 || asplits < 1 ||
        asplits > kAcombMax || !part || !apart)
        return GPT2_ERR_INVALID_ARGUMENT;
    const dim3 grid((N + 31) / 32, splits);
    if (dtype == GPT2_BF16)
        gemm_skinny_lds_kernel<bf16, 8, 1, EPI_BIAS, true><<<grid, 512, 0, s>>>(
            nullptr, part, nullptr, (const bf16*)weight, nullptr, nullptr, M, N, K, apart, asplits, hs);
    else
        gemm_skinny_lds_kernel<float, 8, 1, EPI_BIAS, true><<<grid, 512, 0, s>>>(
            nullptr, part, nullptr, (const float*)weight, nullptr, nullptr, M, N, K, apart, asplits, hs);
    return launch_status();
}

int skinny_acomb_max_splits() { return kAcombMax; }

// Decode-step GEMM on at most 32 rows (K % 8 == 0). part == nullptr:
// out = epi(inp W^T + bias) in one split; otherwise fp32 partial sums over
// `splits` k-ranges into part[splits][M][N], bias and epilogue left to the
// consumer (out must then be nullptr).
int launch_skinny_gemm(void* out, float* part, const void* inp, const void* weight, const void* bias, int M,
                       int K, int N, int splits, int epi, int dtype, hipStream_t s) {
    // exactly one destination: out (one split) or the partial-sum buffer
    if (M < 1 || M > 32 || K % 8 || splits < 1 || (part ? out != nullptr : (out == nullptr || splits != 1)))
        return GPT2_ERR_INVALID_ARGUMENT;
    if (dtype == GPT2_BF16)
        launch_skinny<bf16>((bf16*)out, part, (const bf16*)inp, (const bf16*)weight, (const bf16*)bias, nullptr,
                            M, N, K, splits, epi, s);
    else
        launch_skinny<float>((float*)out, part, (const float*)inp, (const float*)weight, (const float*)bias,
                             nullptr, M, N, K, splits, epi, s);
    return launch_status();
}

// Splits for a decode-step projection of K-deep rows onto N columns: enough
// workgroups to cover the chip (256 CUs), each keeping >= 2 k-chunks of 128
// bytes; at most kMaxSplits.
int skinny_split_count(int K, int N, int es) {
    const int tiles = (N + 31) / 32;
    const int chunks = (K * es + 127) / 128;
    int s = 1;
    while (s < kMaxSplits && tiles * s * 2 <= 256 && chunks >= 4 * s) s *= 2;
    return s;
}

}  // namespace gpt2

using namespace gpt2;

static int check_linear(const void* out, const void* inp, const void* weight, int N, int C, int OC, int dtype) {
    if (!valid_dtype(dtype) || N < 0 || C < 0 || OC < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)N * OC == 0) return GPT2_OK;
    if (!out || !inp || !weight || C == 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (C % 8 || OC % 8 || !aligned16(out) || !aligned16(inp) || !aligned16(weight))
        return GPT2_ERR_UNSUPPORTED;
    if (out == inp || out == weight) return GPT2_ERR_INVALID_ARGUMENT;
    return 1;  // valid, non-empty
}

extern "C" int matmul_splitk_forward(float* part, const void* inp, const void* weight, int N, int C, int OC,
                                     int splits, int dtype, void* stream) {
    if (splits < 1 || splits > kMaxSplits) return GPT2_ERR_INVALID_ARGUMENT;
    const int rc = check_linear(part, inp, weight, N, C, OC, dtype);
    if (rc <= 0) return rc;
    if (N > 32) return GPT2_ERR_UNSUPPORTED;
    return launch_skinny_gemm(nullptr, part, inp, weight, nullptr, N, C, OC, splits, EPI_BIAS, dtype,
                              (hipStream_t)stream);
}

extern "C" int matmul_splitk_count(int C, int OC, int dtype) {
    if (!valid_dtype(dtype) || C <= 0 || OC <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    return skinny_split_count(C, OC, elem_size(dtype));
}

extern "C" int matmul_gelu_forward(void* out, const void* inp, const void* weight, const void* bias, int N,
                                   int C, int OC, int dtype, void* stream) {
    const int rc = check_linear(out, inp, weight, N, C, OC, dtype);
    if (rc <= 0) return rc;
    return launch_matmul_epi(out, inp, weight, bias, nullptr, N, C, OC, EPI_BIAS_GELU, dtype, (hipStream_t)stream);
}

extern "C" int matmul_residual_forward(void* out, const void* inp, const void* weight, const void* bias,
                                       const void* res, int N, int C, int OC, int dtype, void* stream) {
    const int rc = check_linear(out, inp, weight, N, C, OC, dtype);
    if (rc <= 0) return rc;
    if (!res) return GPT2_ERR_INVALID_ARGUMENT;
    if (!aligned16(res)) return GPT2_ERR_UNSUPPORTED;
    return launch_matmul_epi(out, inp, weight, bias, res, N, C, OC, EPI_BIAS_RESIDUAL, dtype,
                             (hipStream_t)stream);
}

extern "C" int matmul_forward(void* out, const void* inp, const void* weight, const void* bias,
                              int N, int C, int OC, int dtype, void* stream) {
    const int rc = check_linear(out, inp, weight, N, C, OC, dtype);
    if (rc <= 0) return rc;
    return launch_matmul(out, inp, weight, bias, N, C, OC, dtype, (hipStream_t)stream);
}

extern "C" int matmul_logits_stats_forward(void* logits, float* stats, const void* inp, const void* wte, int N,
                                           int C, int V, int Vp, int dtype, void* stream) {
    if (V < 1 || V > Vp) return GPT2_ERR_INVALID_ARGUMENT;
    const int rc = check_linear(logits, inp, wte, N, C, Vp, dtype);
    if (rc <= 0) return rc;
    if (!stats) return GPT2_ERR_INVALID_ARGUMENT;
    if (!aligned16(stats) || !matmul_stats_supported(C, dtype)) return GPT2_ERR_UNSUPPORTED;
    return launch_matmul_stats(logits, stats, inp, wte, N, C, Vp, V, dtype, (hipStream_t)stream);
}

extern "C" const char* matmul_kernel_config(int N, int C, int OC, int dtype) {
    if (!valid_dtype(dtype) || N < 0 || C < 0 || OC < 0) return "invalid";
    return matmul_config_name(N, C, OC, dtype);
}
