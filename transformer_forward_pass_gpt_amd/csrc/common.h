// Device helpers shared by the gfx950 kernels: storage types, 16-byte vector
// loads/stores with fp32 unpacking, bf16 rounding, wavefront reductions, the
// MFMA operand types, and the host-side status plumbing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gpt2fwd.h"

namespace gpt2 {

// bf16 storage: the raw 16-bit pattern (upper half of an fp32).
struct bf16 {
    uint16_t bits;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Elements of T per 16-byte vector.
template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<bf16> { static constexpr int N = 8; };

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950: one v_cvt_pk_bf16_f32 per pair).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// 16-byte load of Vec<T>::N elements, widened to fp32.
__device__ __forceinline__ void load_vec(const float* p, float (&v)[4]) {
    float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
__device__ __forceinline__ void load_vec(const bf16* p, float (&v)[8]) {
    uint4 x = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_to_f32(x.x & 0xffffu); v[1] = bf16_to_f32(x.x >> 16);
    v[2] = bf16_to_f32(x.y & 0xffffu); v[3] = bf16_to_f32(x.y >> 16);
    v[4] = bf16_to_f32(x.z & 0xffffu); v[5] = bf16_to_f32(x.z >> 16);
    v[6] = bf16_to_f32(x.w & 0xffffu); v[7] = bf16_to_f32(x.w >> 16);
}
// A 16-byte vector already in registers, widened to fp32.
template <typename T> __device__ __forceinline__ void unpack_vec(const u32x4& x, float (&v)[Vec<T>::N]);
template <> __device__ __forceinline__ void unpack_vec<float>(const u32x4& x, float (&v)[4]) {
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = __uint_as_float(x[i]);
}
template <> __device__ __forceinline__ void unpack_vec<bf16>(const u32x4& x, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = bf16_to_f32(x[i] & 0xffffu);
        v[2 * i + 1] = bf16_to_f32(x[i] >> 16);
    }
}
__device__ __forceinline__ void store_vec(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_vec(bf16* p, const float (&v)[8]) {
    uint4 x;
    x.x = pack_bf16x2(v[0], v[1]); x.y = pack_bf16x2(v[2], v[3]);
    x.z = pack_bf16x2(v[4], v[5]); x.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = x;
}
// Non-temporal forms, for streams written once and not read again soon.
__device__ __forceinline__ void store_vec_nt(float* p, const float (&v)[4]) {
    const u32x4 x = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_vec_nt(bf16* p, const float (&v)[8]) {
    const u32x4 x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

// The value a store of v into T's storage keeps (identity for fp32).
__device__ __forceinline__ float storage_round(const float*, float v) { return v; }
__device__ __forceinline__ float storage_round(const bf16*, float v) { return bf16_to_f32(f32_to_bf16(v)); }

__device__ __forceinline__ float load_scalar(const float* p) { return *p; }
__device__ __forceinline__ float load_scalar(const bf16* p) { return bf16_to_f32(p->bits); }
__device__ __forceinline__ void store_scalar(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_scalar(bf16* p, float v) { p->bits = (uint16_t)f32_to_bf16(v); }

// GELU, tanh form: x/2 (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// Evaluated through the identity 1 + tanh(u) = 2 / (1 + e^{-2u}), so
// g(x) = x / (1 + e^{-2u}): no cancellation for u << 0, and e^{-2u} = inf
// gives the correct limit -0. The exponential is the hardware base-2 one
// (__expf) and the division a hardware reciprocal: a few ulp, a handful of
// instructions (this runs in GEMM epilogues, after the matrix work).
// (ECE408 Milestone 1, kernel table: GELU.)
__device__ __forceinline__ float gelu_tanh(float x) {
    const float k2 = -2.0f * 0.7978845608028654f;  // -2 sqrt(2/pi)
    float u = x * (1.0f + 0.044715f * x * x);
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(k2 * u));
}

// d/dx [x s(2u)] with s the logistic function, u = sqrt(2/pi)(x + 0.044715 x^3)
// (s(2u) = (1 + tanh u)/2, the forward's form):
//   g'(x) = s + x s (1 - s) 2u',  u' = sqrt(2/pi)(1 + 3 * 0.044715 x^2),
// with 1 - s = e s for e = e^{-2u}, so nothing cancels as s -> 1. u is
// clamped at -40 so e stays finite (g' is below 1e-30 there either way).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
    const float k = 0.7978845608028654f;  // sqrt(2/pi)
    const float x2 = x * x;
    const float u = fmaxf(k * x * (1.0f + 0.044715f * x2), -40.0f);
    const float e = __expf(-2.0f * u);
    const float sg = __builtin_amdgcn_rcpf(1.0f + e);
    return sg + x * (sg * sg * e) * (2.0f * k) * (1.0f + 3.0f * 0.044715f * x2);
}

// Reductions across the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

// ---- direct global -> LDS copies (gfx950 global_load_lds_dwordx4)
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

// Wait until at most N of this wave's vector-memory operations are
// outstanding AND all of its LDS operations are done (lgkmcnt 0): before the
// barrier that lets other waves overwrite a stage, this wave's reads of that
// stage must have completed, not merely been issued.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt simm16 on gfx9: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
}

}  // namespace gpt2

// ------------------------------------------------------------------ host side
namespace gpt2 {
void set_last_hip_error(int e);
// GEMM epilogues: y = acc + bias, rounded to the output type; then either
// nothing, GELU of the rounded y, or a residual r added to the rounded y
// (each rounded again), i.e. exactly what a separate GELU or residual kernel
// would compute from the stored product.
// EPI_STATS (vocabulary projection, no bias): the stored product plus, per
// row and per group of kStatCols columns, the max m and the sum of
// e^{y - m} over the group's columns below a limit V (row statistics for a
// one-pass softmax).
// EPI_ASUM (weight gradients, A stored k-major, no bias): the stored
// product plus the sum of A(k, m) over the launch's k-range for every m, i.e.
// the column sums of the stored A rows (the bias gradient of a linear layer
// is the column sum of its output gradient, which is this A), taken from the
// fragments the product already reads, written as fp32 to stats[slice * M + m]
// by the workgroups of output tile column 0.
// EPI_DGELU (the backward of a GELU whose output fed the forward product):
// y = acc + bias rounded to the output type, times g'(x) for x = res[row][col]
// (the GELU's input), rounded again: what a separate GELU backward computes
// from the stored product.
// EPI_BIAS_GELU2 (training forward): y = acc + bias rounded to the output
// type is stored in out, and GELU of that stored y, rounded, in out2: the
// pre-activation a GELU backward needs and the activation the next product
// reads, as a separate GELU kernel would compute it.
// EPI_BIAS_NT: EPI_BIAS with non-temporal stores, for outputs far larger than
// the caches (the vocabulary logits) that would otherwise displace operands.
enum Epilogue {
    EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_RESIDUAL = 2, EPI_STATS = 3, EPI_ASUM = 4, EPI_DGELU = 5,
    EPI_BIAS_GELU2 = 6, EPI_BIAS_NT = 7
};
constexpr int kStatCols = 128;
constexpr int kNumCUs = 256;  // compute units of one MI355X (8 XCDs x 32)

// Status after a launch: GPT2_OK, or GPT2_ERR_HIP with the code recorded.
int launch_status();
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_dtype(int d) { return d == GPT2_F32 || d == GPT2_BF16; }
inline int elem_size(int d) { return d == GPT2_BF16 ? 2 : 4; }
}  // namespace gpt2
