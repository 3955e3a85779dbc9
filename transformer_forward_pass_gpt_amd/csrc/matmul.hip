// Linear layer entry: out[n,o] = sum_c inp[n,c] * W[o,c] + bias[o], on the
// MFMA GEMM of gemm.h with a tile shape chosen per problem size.
#include "gemm.h"

namespace gpt2 {

// Tile shapes, chosen per problem from measurements on MI355X (GPT-2 small and
// medium layer shapes): wide outputs (the vocabulary projection) take
// 128x128 tiles; deep reductions take 128x96 with 256-byte k tiles; the
// rest picks the largest tile that still gives every CU several workgroups.
enum GemmCfg { G32x64 = 0, G64x64, G64x128, G128x96, G128x96_K2, G128x128, G_NCFG };
static const char* kCfgName[2][G_NCFG] = {
    {"gemm_f32_32x64_bk32", "gemm_f32_64x64_bk32", "gemm_f32_64x128_bk32", "gemm_f32_128x96_bk32",
     "gemm_f32_128x96_bk64", "gemm_f32_128x128_bk32"},
    {"gemm_bf16_32x64_bk64", "gemm_bf16_64x64_bk64", "gemm_bf16_64x128_bk64",
     "gemm_bf16_128x96_bk64", "gemm_bf16_128x96_bk128", "gemm_bf16_128x128_bk64"}};

static GemmCfg choose_cfg(int M, int N, int K, int dtype) {
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (M <= 32) return G32x64;
    if (N >= 16384) return G128x128;
    if (dtype == GPT2_F32) {
        if (K >= 2048 && tiles(128, 96) >= 256) return G128x96_K2;
        if (tiles(128, 96) >= 1024) return G128x96;
        return G64x64;
    }
    if (tiles(128, 96) >= 512) return G128x96;
    return G64x128;
}

template <typename T>
static void launch_gemm_t(T* out, const T* A, const T* W, const T* bias, int M, int N, int K,
                          int dtype, hipStream_t s) {
    constexpr int BK = Vec<T>::N * 8;  // 128 bytes of k per row per LDS tile
    switch (choose_cfg(M, N, K, dtype)) {
        case G32x64: launch_gemm_cfg<T, 1, 2, 1, 1, BK>(out, A, W, bias, M, N, K, 1, 0, s); break;
        case G64x64: launch_gemm_cfg<T, 2, 2, 1, 1, BK>(out, A, W, bias, M, N, K, 4, 1, s); break;
        case G64x128: launch_gemm_cfg<T, 2, 2, 1, 2, BK>(out, A, W, bias, M, N, K, 8, 1, s); break;
        case G128x96: launch_gemm_cfg<T, 4, 1, 1, 3, BK>(out, A, W, bias, M, N, K, 8, 1, s); break;
        case G128x96_K2:
            launch_gemm_cfg<T, 4, 1, 1, 3, 2 * BK>(out, A, W, bias, M, N, K, 4, 1, s);
            break;
        default: launch_gemm_cfg<T, 1, 4, 4, 1, BK>(out, A, W, bias, M, N, K, 4, 1, s); break;
    }
}

const char* matmul_config_name(int N, int C, int OC, int dtype) {
    return kCfgName[dtype == GPT2_BF16 ? 1 : 0][choose_cfg(N, OC, C, dtype)];
}

int launch_matmul(void* out, const void* inp, const void* weight, const void* bias, int N, int C,
                  int OC, int dtype, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_gemm_t<bf16>((bf16*)out, (const bf16*)inp, (const bf16*)weight, (const bf16*)bias, N,
                            OC, C, dtype, s);
    else
        launch_gemm_t<float>((float*)out, (const float*)inp, (const float*)weight,
                             (const float*)bias, N, OC, C, dtype, s);
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

extern "C" const char* matmul_kernel_config(int N, int C, int OC, int dtype) {
    if (!valid_dtype(dtype) || N < 0 || C < 0 || OC < 0) return "invalid";
    return matmul_config_name(N, C, OC, dtype);
}
