// Backward kernels of the training step, one per forward step (the backward
// kernels of the llm.c training step: gelu_backward_kernel,
// layernorm_backward_kernel2, matmul_backward_bias_kernel4,
// encoder_backward_kernel and the cuBLAS GEMMs of the linear layers; "State
// of the Union [April 22, 2024]", kernel summaries).
//
// Every reduction runs in a fixed order with fp32 partial sums written to a
// caller-provided workspace and summed by a second kernel, so results are
// bitwise reproducible (no floating-point atomics).
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"

namespace gpt2 {

int launch_matmul(void*, const void*, const void*, const void*, int, int, int, int, hipStream_t);
int launch_matmul_splitk_part(float*, const float*, const float*, int, int, int, int, int, hipStream_t);
int launch_matmul_splitk_part(float*, const bf16*, const bf16*, int, int, int, int, int, hipStream_t);
int launch_matmul_epi(void*, const void*, const void*, const void*, const void*, int, int, int, int, int,
                      hipStream_t);
int launch_matmul_kmajor(float*, const float*, const float*, int, int, int, int, int, bool, bool, int, hipStream_t,
                         const float* = nullptr, float* = nullptr);
int launch_matmul_kmajor(float*, const bf16*, const bf16*, int, int, int, int, int, bool, bool, int, float*,
                         hipStream_t);
int launch_matmul_kmajor(bf16*, const bf16*, const bf16*, int, int, int, int, int, bool, bool, int, hipStream_t);

static constexpr int kBwdThreads = 256;

static unsigned stream_grid_bwd(int64_t nvec) {
    int64_t g = (nvec + kBwdThreads - 1) / kBwdThreads;
    if (g > 2048) g = 2048;
    if (g < 1) g = 1;
    return (unsigned)g;
}

static inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

// ------------------------------------------------------------ GELU backward
// dinp = dout * g'(inp); dinp may be dout (each element is read, then written
// by the same thread).
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void gelu_backward_kernel(T* dinp, const T* inp, const T* dout, int64_t n) {
    constexpr int V = Vec<T>::N;
    const int64_t nvec = n / V;
    const int64_t stride = (int64_t)gridDim.x * kBwdThreads;
    for (int64_t i = blockIdx.x * (int64_t)kBwdThreads + threadIdx.x; i < nvec; i += stride) {
        float x[V], d[V];
        load_vec(inp + i * V, x);
        load_vec(dout + i * V, d);
#pragma unroll
        for (int j = 0; j < V; j++) d[j] *= gelu_tanh_grad(x[j]);
        store_vec(dinp + i * V, d);
    }
    for (int64_t i = nvec * V + blockIdx.x * (int64_t)kBwdThreads + threadIdx.x; i < n; i += stride)
        store_scalar(dinp + i, load_scalar(dout + i) * gelu_tanh_grad(load_scalar(inp + i)));
}

// ------------------------------------------------------- column reduction
// out[c] = sum_{r < R} part[r * C + c]: 64 columns x 16 row slices per
// workgroup (1024 threads); slice k sums rows k*q .. k*q+q-1 in ascending
// order (q = ceil(R/16)), and the 16 slice sums are added in slice order, so
// the result is a fixed function of the partials. Grid row y = 1 (when
// out2 is given) does the same for (out2, part2): two reductions of the same
// shape in one launch.
static constexpr int kColSlices = 16;

template <typename T>
__global__ __launch_bounds__(1024) void colsum_kernel(T* out, const float* __restrict__ part, int R, int C,
                                                      T* out2, const float* __restrict__ part2) {
    __shared__ float sh[kColSlices][64];
    if (blockIdx.y == 1) {  // workgroup-uniform
        out = out2;
        part = part2;
    }
    const int lane = threadIdx.x & 63, k = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const int q = (R + kColSlices - 1) / kColSlices, r0 = k * q, r1 = min(R, r0 + q);
    float s = 0.f;
    if (c < C) {
        int r = r0;
        for (; r + 8 <= r1; r += 8) {
            float a[8];
#pragma unroll
            for (int u = 0; u < 8; u++) a[u] = part[(int64_t)(r + u) * C + c];
#pragma unroll
            for (int u = 0; u < 8; u++) s += a[u];
        }
        for (; r < r1; r++) s += part[(int64_t)r * C + c];
    }
    sh[k][lane] = s;
    __syncthreads();
    if (k == 0 && c < C) {
        float t = sh[0][lane];
#pragma unroll
        for (int i = 1; i < kColSlices; i++) t += sh[i][lane];
        store_scalar(out + c, t);
    }
}

template <typename T>
static void launch_colsum(T* out, const float* part, int R, int C, hipStream_t s, T* out2 = nullptr,
                          const float* part2 = nullptr) {
    colsum_kernel<T><<<dim3((C + 63) / 64, out2 ? 2 : 1), 1024, 0, s>>>(out, part, R, C, out2, part2);
}

// First stage of the column sums of x [R, C] (fp32): part[y][c] = sum of rows
// 256y .. 256y+255 of column c, four 64-row quarters (one wavefront each, rows
// ascending) added in order. Grid (ceil(C/64), ceil(R/256)).
template <typename T>
__global__ __launch_bounds__(256) void colpart_kernel(float* __restrict__ part, const T* __restrict__ x, int R, int C) {
    __shared__ float sh[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const int r0 = blockIdx.y * 256 + w * 64, r1 = min(R, r0 + 64);
    float s = 0.f;
    if (c < C) {
        int r = r0;
        for (; r + 8 <= r1; r += 8) {
            float a[8];
#pragma unroll
            for (int u = 0; u < 8; u++) a[u] = load_scalar(x + (int64_t)(r + u) * C + c);
#pragma unroll
            for (int u = 0; u < 8; u++) s += a[u];
        }
        for (; r < r1; r++) s += load_scalar(x + (int64_t)r * C + c);
    }
    sh[w][lane] = s;
    __syncthreads();
    if (w == 0 && c < C) part[(int64_t)blockIdx.y * C + c] = ((sh[0][lane] + sh[1][lane]) + sh[2][lane]) + sh[3][lane];
}

// out[i] = sum_{s < S} part[s * n + i] (s ascending), n = M*N elements, 16
// bytes of T per thread: the split-k partial products of a weight gradient;
// then, when out2 is given, the same over the n2 elements of part2 into out2
// (the slices' bias-gradient partials), in the same launch. n, n2 % V == 0.
template <typename T>
__global__ __launch_bounds__(256) void splitsum_kernel(T* out, const float* __restrict__ part, int S, int64_t n,
                                                       T* out2, const float* __restrict__ part2, int n2) {
    constexpr int V = Vec<T>::N;
    const int64_t nvec = n / V, nall = nvec + (out2 ? n2 / V : 0);
    for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < nall; i += (int64_t)gridDim.x * 256) {
        const bool first = i < nvec;
        const float* src = first ? part + i * V : part2 + (i - nvec) * V;
        const int64_t stride = first ? n : n2;
        float a[V];
#pragma unroll
        for (int j = 0; j < V; j++) a[j] = 0.f;
        for (int sp = 0; sp < S; sp++) {
            float b[V];
            const float* p = src + (int64_t)sp * stride;
#pragma unroll
            for (int j = 0; j < V; j += 4) {
                const float4 x = *reinterpret_cast<const float4*>(p + j);
                b[j] = x.x; b[j + 1] = x.y; b[j + 2] = x.z; b[j + 3] = x.w;
            }
#pragma unroll
            for (int j = 0; j < V; j++) a[j] += b[j];
        }
        store_vec(first ? out + i * V : out2 + (i - nvec) * V, a);
    }
}

// ------------------------------------------------------ LayerNorm backward
// For y = xh * gamma + beta, xh = (x - mu) * rstd (mu and rstd as saved by
// the forward), g = dy * gamma:
//   dx = rstd * (g - mean_c(g) - xh * mean_c(g * xh))   [+ dres]
//   dgamma = sum_n dy * xh,   dbeta = sum_n dy.
// One wavefront per row (the row in registers, loads clamped and masked),
// rows strided over the grid; each workgroup sums its rows' dgamma and dbeta
// terms in registers, combines its kLnbWaves wavefronts through LDS in order
// and writes one row of partials (gpart, bpart: [gridDim.x][C]). dres may be
// dinp (read before written by the same lane).
static constexpr int kLnbWaves = 8;

template <typename T, int VPL>
__global__ __launch_bounds__(64 * kLnbWaves) void layernorm_backward_kernel(T* dinp, float* __restrict__ gpart,
                                                                 float* __restrict__ bpart, const T* dres,
                                                                 const T* __restrict__ dout,
                                                                 const T* __restrict__ inp,
                                                                 const T* __restrict__ gamma,
                                                                 const float* __restrict__ mean,
                                                                 const float* __restrict__ rstd, int N, int C) {
    constexpr int V = Vec<T>::N;
    __shared__ float sh[kLnbWaves][64 * V];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int cv = C / V;
    const float invC = 1.0f / (float)C;
    float gm[VPL][V], ag[VPL][V], ab[VPL][V];
#pragma unroll
    for (int i = 0; i < VPL; i++) {
        load_vec(gamma + min(lane + i * 64, cv - 1) * V, gm[i]);
#pragma unroll
        for (int j = 0; j < V; j++) ag[i][j] = ab[i][j] = 0.f;
    }
    // Up to two vectors per lane (PF), the loads of a wave's next row are
    // issued before its current row is computed (raw 16-byte vectors,
    // unpacked once the row is current); wider rows would need the registers
    // of a second resident workgroup or spill.
    constexpr bool PF = VPL <= 2;
    const int stride = gridDim.x * kLnbWaves;
    u32x4 px[VPL], pd[VPL], pr[VPL];
    float pmu = 0.f, prs = 0.f;
    auto fetch = [&](int row) {
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int64_t off = (int64_t)row * C + min(lane + i * 64, cv - 1) * V;
            px[i] = *reinterpret_cast<const u32x4*>(inp + off);
            pd[i] = *reinterpret_cast<const u32x4*>(dout + off);
            // unconditional (dout stands in when there is no dres), so no load waits at a branch
            pr[i] = *reinterpret_cast<const u32x4*>((dres ? dres : dout) + off);
        }
        pmu = mean[row];
        prs = rstd[row];
    };
    if (PF && blockIdx.x * kLnbWaves + w < N) fetch(blockIdx.x * kLnbWaves + w);
    for (int row = blockIdx.x * kLnbWaves + w; row < N; row += stride) {  // wave-uniform
        if (!PF) fetch(row);
        float x[VPL][V], d[VPL][V], r0[VPL][V];
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            unpack_vec<T>(px[i], x[i]);
            unpack_vec<T>(pd[i], d[i]);
            unpack_vec<T>(pr[i], r0[i]);
        }
        const float mu = pmu, rs = prs;
        if (PF && row + stride < N) fetch(row + stride);
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const bool on = lane + i * 64 < cv;
#pragma unroll
            for (int j = 0; j < V; j++) {
                const float dy = on ? d[i][j] : 0.f;
                const float xh = (x[i][j] - mu) * rs;
                const float g = dy * gm[i][j];
                a += g;
                b += g * xh;
                ag[i][j] += dy * xh;
                ab[i][j] += dy;
                x[i][j] = xh;
                d[i][j] = g;
            }
        }
        a = wave_sum(a) * invC;
        b = wave_sum(b) * invC;
#pragma unroll
        for (int i = 0; i < VPL; i++) {
            const int idx = lane + i * 64;
            if (idx < cv) {
#pragma unroll
                for (int j = 0; j < V; j++) {
                    float dx = rs * (d[i][j] - a - x[i][j] * b);
                    dx += dres ? r0[i][j] : 0.f;
                    x[i][j] = dx;
                }
                store_vec(dinp + (int64_t)row * C + idx * V, x[i]);
            }
        }
    }
    // the workgroup's partial rows, added in wavefront order
#pragma unroll
    for (int p = 0; p < 2; p++) {
        float* dst = p == 0 ? gpart : bpart;
#pragma unroll
        for (int i = 0; i < VPL; i++) {
#pragma unroll
            for (int j = 0; j < V; j++) sh[w][lane * V + j] = p == 0 ? ag[i][j] : ab[i][j];
            __syncthreads();
            for (int e = threadIdx.x; e < 64 * V; e += 64 * kLnbWaves) {
                const int c = i * 64 * V + e;
                if (c < C) {
                    float t = sh[0][e];
#pragma unroll
                    for (int k = 1; k < kLnbWaves; k++) t += sh[k][e];
                    dst[(int64_t)blockIdx.x * C + c] = t;
                }
            }
            __syncthreads();
        }
    }
}

static int ln_bwd_grid(int N) { return max(1, min((N + kLnbWaves - 1) / kLnbWaves, 512)); }

int64_t layernorm_backward_workspace_bytes(int N, int C) {
    return 2 * align256((int64_t)ln_bwd_grid(N) * C * 4);
}

// Workgroups of one instantiation resident per CU (registers and LDS decide),
// asked of the runtime once.
template <typename T, int P>
static int ln_bwd_per_cu() {
    static const int n = [] {
        int k = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&k, layernorm_backward_kernel<T, P>, 64 * kLnbWaves, 0) !=
            hipSuccess)
            k = 1;
        return max(k, 1);
    }();
    return n;
}

template <typename T>
static void launch_ln_bwd_t(T* dinp, T* dgamma, T* dbeta, const T* dres, const T* dout, const T* inp, const T* gamma,
                            const float* mean, const float* rstd, int N, int C, void* ws, hipStream_t s) {
    const int rows = ln_bwd_grid(N);  // workspace bound: at most this many partial rows
    float* gpart = (float*)ws;
    float* bpart = (float*)((char*)ws + align256((int64_t)rows * C * 4));
    const int vpl = (C / Vec<T>::N + 63) / 64;
    // One resident round of workgroups (rows strided over it, the next row's
    // loads in flight while one is computed), not a second partial round.
    int grid = rows;
#define LNB(P)                                                                                                    \
    grid = min(rows, kNumCUs * ln_bwd_per_cu<T, P>());                                                            \
    layernorm_backward_kernel<T, P><<<grid, 64 * kLnbWaves, 0, s>>>(dinp, gpart, bpart, dres, dout, inp, gamma,   \
                                                                    mean, rstd, N, C)
    if (vpl <= 1) { LNB(1); }
    else if (vpl <= 2) { LNB(2); }
    else if (vpl <= 3) { LNB(3); }
    else if (vpl <= 4) { LNB(4); }
    else { LNB(8); }
#undef LNB
    // both column sums in one launch when both are wanted
    if (dgamma && dbeta) launch_colsum<T>(dgamma, gpart, grid, C, s, dbeta, bpart);
    else if (dgamma) launch_colsum<T>(dgamma, gpart, grid, C, s);
    else if (dbeta) launch_colsum<T>(dbeta, bpart, grid, C, s);
}

// ---------------------------------------------------------------- transpose
// out[c][r] = in[r][c] for r < R and 0 for R <= r < ldo (in: [R, Cc], out:
// [Cc, ldo], ldo >= R, Cc and ldo multiples of 16 bytes' worth of T). A
// 64 x 64 tile per workgroup staged through LDS (rows padded by one word:
// both the row-wise writes and the column-wise reads are conflict-free),
// 16-byte loads and stores on both sides. colpart (nullable): one fp32 row of
// column sums per 64-row tile, colpart[tile][c] = sum of the tile's in[r][c]
// in ascending r (the bias gradient's first stage, taken from the same read).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(T* __restrict__ out, float* __restrict__ colpart,
                                                        const T* __restrict__ in, int R, int Cc, int ldo) {
    constexpr int V = Vec<T>::N;
    constexpr int VPR = 64 / V;  // 16-byte vectors per 64-element tile row
    __shared__ float tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64, tid = threadIdx.x;
    float v[(64 * VPR + 255) / 256][V];
#pragma unroll
    for (int k = 0; k < (64 * VPR + 255) / 256; k++) {
        const int q = tid + k * 256, rl = q / VPR, cl = (q % VPR) * V;
        load_vec(in + (int64_t)min(r0 + rl, R - 1) * Cc + min(c0 + cl, Cc - V), v[k]);
    }
#pragma unroll
    for (int k = 0; k < (64 * VPR + 255) / 256; k++) {
        const int q = tid + k * 256, rl = q / VPR, cl = (q % VPR) * V;
        const bool ok = r0 + rl < R && c0 + cl < Cc;
#pragma unroll
        for (int j = 0; j < V; j++) tile[rl][cl + j] = ok ? v[k][j] : 0.f;
    }
    __syncthreads();
    if (colpart && tid < 64 && c0 + tid < Cc) {
        float s = 0.f;
        for (int rl = 0; rl < 64; rl++) s += tile[rl][tid];
        colpart[(int64_t)blockIdx.y * Cc + c0 + tid] = s;
    }
#pragma unroll
    for (int k = 0; k < (64 * VPR + 255) / 256; k++) {
        const int q = tid + k * 256, cl = q / VPR, rl = (q % VPR) * V;
        if (c0 + cl < Cc && r0 + rl < ldo) {
            float o[V];
#pragma unroll
            for (int j = 0; j < V; j++) o[j] = tile[rl + j][cl];
            store_vec(out + (int64_t)(c0 + cl) * ldo + r0 + rl, o);
        }
    }
}

template <typename T>
static void launch_transpose(T* out, float* colpart, const T* in, int R, int Cc, int ldo, hipStream_t s) {
    dim3 grid((Cc + 63) / 64, (ldo + 63) / 64);
    transpose_kernel<T><<<grid, 256, 0, s>>>(out, colpart, in, R, Cc, ldo);
}

// ---------------------------------------------------------- linear backward
// For out = inp W^T + b (inp [N,C], W [OC,C]) and dout [N,OC]:
//   dinp = dout W          : contraction over OC, for which W [OC][C] is k-major
//   dW   = dout^T inp      : contraction over the N tokens, for which dout and
//                            inp are both k-major
//   db   = column sums of dout
// When the contraction is a whole number of k-tiles (fp32 32, bf16 64) the
// GEMM reads the k-major operands in place (fp32: scalar LDS gathers; bf16:
// transposing LDS reads). Otherwise the operands whose contraction index is
// their row index are transposed first (tiled, 16-byte traffic both ways),
// the token dimension zero-padded to Np, a multiple of 64, so the K loop of
// the pipelined GEMM has no tail; the bias partials then come from the dout
// transpose.
static int64_t round64(int64_t n) { return (n + 63) / 64 * 64; }

// Split-k count for the weight gradient: its OC x C output (fp32 in 128x96
// tiles, bf16 in 128x128) is often far below the chip's 256 CUs while K = Np
// is deep, so the token range is cut into up to 8 slices (each a whole number
// of k-tiles, 32 deep for fp32 and 64 for bf16, at least 256 deep) until there
// are >= 512 workgroups (fp32) or >= 256 (bf16, one 128x128 workgroup per
// CU; outputs of 128 or more tiles stay whole: two half-depth rounds take as
// long as one full one, plus the partials' traffic). The slices' products are
// fp32 partial sums in both dtypes, added in slice order by splitsum_kernel.
static int dw_splits(int N, int C, int OC, int dtype) {
    const bool f32 = dtype == GPT2_F32;
    const int64_t Np = round64(N), kt = f32 ? 32 : 64;
    const int64_t tiles = (int64_t)((OC + 127) / 128) * ((C + (f32 ? 95 : 127)) / (f32 ? 96 : 128));
    const int64_t target = f32 ? 512 : 256;
    if (!f32 && tiles >= 128) return 1;
    int s = 1;
    while (s < 8 && tiles * s < target && (Np / (2 * s)) % kt == 0 && Np / (2 * s) >= 256 && Np % (2 * s) == 0)
        s *= 2;
    return s;
}

// The k-major paths, whose k-range is the N tokens themselves: slices of N/S
// rows, each a whole number of k-tiles. fp32 (N % 32 == 0, 128x96 tiles): the
// rule above. bf16 (N % 64 == 0, 128x128 tiles, two workgroups per CU):
// slices until there are >= 384 workgroups, each slice >= 512 tokens deep
// (GPT-2 small at 8192 tokens: fc and fcproj 4 slices, qkv 4, attproj 8).
static int dw_splits_kmajor(int N, int C, int OC, int dtype) {
    const bool f32 = dtype == GPT2_F32;
    const int kt = f32 ? 32 : 64, target = f32 ? 512 : 384, depth = f32 ? 256 : 512;
    const int64_t tiles = (int64_t)((OC + 127) / 128) * ((C + (f32 ? 95 : 127)) / (f32 ? 96 : 128));
    int s = 1;
    while (s < 8 && tiles * s < target && N % (2 * s) == 0 && (N / (2 * s)) % kt == 0 && N / (2 * s) >= depth)
        s *= 2;
    return s;
}

int64_t matmul_backward_workspace_bytes(int N, int C, int OC, int dtype) {
    const int64_t es = elem_size(dtype), Np = round64(N);
    const int S = std::max(dw_splits(N, C, OC, dtype), dw_splits_kmajor(N, C, OC, dtype));
    return align256((int64_t)C * OC * es) + align256((int64_t)OC * Np * es) + align256((int64_t)C * Np * es) +
           align256(Np / 64 * OC * 4) + (S > 1 ? align256((int64_t)S * OC * C * 4) : 0);
}

template <typename T>
static int launch_matmul_bwd_t(T* dinp, T* dweight, T* dbias, const T* dout, const T* inp, const T* weight, int N,
                               int C, int OC, int dtype, void* ws, hipStream_t s, const T* gelu_in) {
    const int64_t es = sizeof(T), Np = round64(N);
    char* p = (char*)ws;
    T* wt = (T*)p;
    p += align256((int64_t)C * OC * es);
    T* doutT = (T*)p;
    p += align256((int64_t)OC * Np * es);
    T* inpT = (T*)p;
    p += align256((int64_t)C * Np * es);
    float* bpart = (float*)p;
    p += align256(Np / 64 * OC * 4);
    float* wpart = (float*)p;  // split-k partials of dweight
    int rc = GPT2_OK;
    {
        // k-major operands read in place when the contraction is a whole
        // number of k-tiles (fp32 32, bf16 64): dinp = dout . W with W as
        // stored ([OC][C] is k-major for this product; fp32 only: in bf16 the
        // transpose of W is small and the row-major tile shapes chosen per
        // problem are faster), dW = dout^T . inp with both as stored; the bias
        // from a two-stage column sum of dout
        constexpr bool f32 = std::is_same<T, float>::value;
        constexpr int kt = f32 ? 32 : 64;
        const bool km_dinp = f32 && OC % kt == 0, km_dw = N % kt == 0;
        if (dinp && km_dinp) {
            if constexpr (f32)
                rc = launch_matmul_kmajor(dinp, dout, weight, N, C, OC, OC, C, false, true, 1, s, gelu_in);
            if (rc) return rc;
        }
        if (dweight && km_dw) {
            const int Sk = dw_splits_kmajor(N, C, OC, dtype);
            // in slices: the bias partials come from the product's own reads
            // of dout (per slice, into bpart: Sk <= 8 <= N/64 rows) and are
            // summed with the weight slices
            T* db_fused = Sk > 1 ? dbias : nullptr;
            if constexpr (f32)
                rc = launch_matmul_kmajor(Sk > 1 ? wpart : dweight, dout, inp, OC, C, N / Sk, OC, C, true, true, Sk, s,
                                          nullptr, db_fused ? bpart : nullptr);
            else if (Sk > 1)
                rc = launch_matmul_kmajor(wpart, dout, inp, OC, C, N / Sk, OC, C, true, true, Sk,
                                          db_fused ? bpart : nullptr, s);
            else
                rc = launch_matmul_kmajor(dweight, dout, inp, OC, C, N, OC, C, true, true, 1, s);
            if (rc) return rc;
            if (Sk > 1) {
                const int64_t n = (int64_t)OC * C;
                splitsum_kernel<T><<<stream_grid_bwd((n + OC) / 4), 256, 0, s>>>(dweight, wpart, Sk, n, db_fused,
                                                                                 bpart, OC);
            }
            if (db_fused) dbias = nullptr;  // done
        }
        if (dbias && km_dw) {
            const int R = (N + 255) / 256;
            colpart_kernel<T><<<dim3((OC + 63) / 64, R), 256, 0, s>>>(bpart, dout, N, OC);
            launch_colsum<T>(dbias, bpart, R, OC, s);
        }
        if (km_dinp) dinp = nullptr;  // done
        if (km_dw) dweight = dbias = nullptr;
        if (!dinp && !dweight && !dbias) return launch_status();
    }
    // otherwise (a ragged contraction) the transposed operands, token range
    // zero-padded to Np
    const int S = dw_splits(N, C, OC, dtype);
    if (dinp) {
        launch_transpose<T>(wt, nullptr, weight, OC, C, OC, s);  // W^T [C, OC]
        rc = launch_matmul_epi(dinp, dout, wt, nullptr, gelu_in, N, OC, C, gelu_in ? EPI_DGELU : EPI_BIAS, dtype, s);
        if (rc) return rc;
    }
    if (dweight || dbias) launch_transpose<T>(doutT, dbias ? bpart : nullptr, dout, N, OC, (int)Np, s);
    if (dweight) {
        launch_transpose<T>(inpT, nullptr, inp, N, C, (int)Np, s);
        if (S > 1) {
            rc = launch_matmul_splitk_part(wpart, doutT, inpT, OC, C, (int)(Np / S), (int)Np, S, s);
            if (rc) return rc;
            const int64_t n = (int64_t)OC * C;
            splitsum_kernel<T><<<stream_grid_bwd(n / 4), 256, 0, s>>>(dweight, wpart, S, n, nullptr, nullptr, 0);
        } else {
            rc = launch_matmul(dweight, doutT, inpT, nullptr, OC, (int)Np, C, dtype, s);
            if (rc) return rc;
        }
    }
    if (dbias) launch_colsum<T>(dbias, bpart, (int)(Np / 64), OC, s);
    return launch_status();
}

// gelu_in (nullable, [N, C]): the input gradient comes out already through the
// backward of the GELU whose output was `inp` (dinp = (dout W) o g'(gelu_in),
// each factor rounded as the separate GELU backward rounds it).
int launch_matmul_backward(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                           const void* weight, int N, int C, int OC, int dtype, void* ws, hipStream_t s,
                           const void* gelu_in) {
    if (dtype == GPT2_BF16)
        return launch_matmul_bwd_t<bf16>((bf16*)dinp, (bf16*)dweight, (bf16*)dbias, (const bf16*)dout,
                                         (const bf16*)inp, (const bf16*)weight, N, C, OC, dtype, ws, s,
                                         (const bf16*)gelu_in);
    return launch_matmul_bwd_t<float>((float*)dinp, (float*)dweight, (float*)dbias, (const float*)dout,
                                      (const float*)inp, (const float*)weight, N, C, OC, dtype, ws, s,
                                      (const float*)gelu_in);
}

// --------------------------------------------------------- encoder backward
// dwte[v,:] += sum of dout[n,:] over the positions n holding token v, in
// ascending n: one workgroup per position; the workgroup of a token's first
// occurrence does the whole sum (finding the later occurrences 256 positions
// at a time with an ordered ballot compaction), every other workgroup exits.
// No two workgroups write the same row, so no atomics and a fixed order.
static constexpr int kEncMaxVecPerThread = 4;  // C <= 1024 * 16 bytes' worth

template <typename T>
__global__ __launch_bounds__(256) void encoder_wte_backward_kernel(T* dwte, const T* __restrict__ dout,
                                                                   const int32_t* __restrict__ tokens, int N, int C) {
    constexpr int V = Vec<T>::N;
    __shared__ int list[256];
    __shared__ int cnt[4];
    const int n = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int tok = tokens[n];
    int earlier = 0;
    for (int m = tid; m < n; m += 256) earlier |= (tokens[m] == tok);
    if (__syncthreads_or(earlier)) return;  // workgroup-uniform
    const int cv = C / V;
    float acc[kEncMaxVecPerThread][V];
#pragma unroll
    for (int k = 0; k < kEncMaxVecPerThread; k++)
#pragma unroll
        for (int j = 0; j < V; j++) acc[k][j] = 0.f;
    for (int m0 = n; m0 < N; m0 += 256) {
        const int m = m0 + tid;
        const bool hit = m < N && tokens[m] == tok;
        const unsigned long long bal = __ballot(hit);
        if (lane == 0) cnt[w] = __popcll(bal);
        __syncthreads();
        int base = 0;
        for (int i = 0; i < w; i++) base += cnt[i];
        const int total = cnt[0] + cnt[1] + cnt[2] + cnt[3];
        if (hit) list[base + __popcll(bal & ((1ull << lane) - 1ull))] = m;
        __syncthreads();
        for (int i = 0; i < total; i++) {
            const int64_t row = list[i];
#pragma unroll
            for (int k = 0; k < kEncMaxVecPerThread; k++) {
                const int cvi = tid + k * 256;
                if (cvi < cv) {
                    float d[V];
                    load_vec(dout + row * C + cvi * V, d);
#pragma unroll
                    for (int j = 0; j < V; j++) acc[k][j] += d[j];
                }
            }
        }
        __syncthreads();  // list and cnt are rewritten next round
    }
#pragma unroll
    for (int k = 0; k < kEncMaxVecPerThread; k++) {
        const int cvi = tid + k * 256;
        if (cvi < cv) {
            T* dst = dwte + (int64_t)tok * C + cvi * V;
            float o[V];
            load_vec(dst, o);
#pragma unroll
            for (int j = 0; j < V; j++) o[j] += acc[k][j];
            store_vec(dst, o);
        }
    }
}

// dwpe[t,:] += sum_b dout[b,t,:] (b ascending), one thread per 16-byte vector.
template <typename T>
__global__ __launch_bounds__(256) void encoder_wpe_backward_kernel(T* dwpe, const T* __restrict__ dout, int B, int T_,
                                                                   int C) {
    constexpr int V = Vec<T>::N;
    const int cv = C / V;
    const int64_t nvec = (int64_t)T_ * cv;
    for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < nvec; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / cv, c = (i % cv) * V;
        float acc[V], d[V];
#pragma unroll
        for (int j = 0; j < V; j++) acc[j] = 0.f;
        for (int b = 0; b < B; b++) {
            load_vec(dout + ((int64_t)b * T_ + t) * C + c, d);
#pragma unroll
            for (int j = 0; j < V; j++) acc[j] += d[j];
        }
        load_vec(dwpe + t * C + c, d);
#pragma unroll
        for (int j = 0; j < V; j++) d[j] += acc[j];
        store_vec(dwpe + t * C + c, d);
    }
}

// Zero n elements (a fill kernel rather than a memset node, so the call can
// be captured in a graph).
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t nwords) {
    for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

void launch_zero(void* p, int64_t bytes, hipStream_t s) {
    const int64_t nw = bytes / 4;
    zero_kernel<<<stream_grid_bwd(nw), 256, 0, s>>>((uint32_t*)p, nw);
}

int launch_encoder_backward(void* dwte, void* dwpe, const void* dout, const int32_t* tokens, int B, int T, int C,
                            int dtype, hipStream_t s) {
    const int N = B * T, V = dtype == GPT2_BF16 ? 8 : 4;
    if (dtype == GPT2_BF16) {
        if (dwte) encoder_wte_backward_kernel<bf16><<<N, 256, 0, s>>>((bf16*)dwte, (const bf16*)dout, tokens, N, C);
        if (dwpe)
            encoder_wpe_backward_kernel<bf16><<<stream_grid_bwd((int64_t)T * C / V), 256, 0, s>>>(
                (bf16*)dwpe, (const bf16*)dout, B, T, C);
    } else {
        if (dwte)
            encoder_wte_backward_kernel<float><<<N, 256, 0, s>>>((float*)dwte, (const float*)dout, tokens, N, C);
        if (dwpe)
            encoder_wpe_backward_kernel<float><<<stream_grid_bwd((int64_t)T * C / V), 256, 0, s>>>(
                (float*)dwpe, (const float*)dout, B, T, C);
    }
    return launch_status();
}

int launch_gelu_backward(void* dinp, const void* inp, const void* dout, int64_t n, int dtype, hipStream_t s) {
    const int64_t nvec = n / (dtype == GPT2_BF16 ? 8 : 4) + 1;
    if (dtype == GPT2_BF16)
        gelu_backward_kernel<bf16><<<stream_grid_bwd(nvec), kBwdThreads, 0, s>>>((bf16*)dinp, (const bf16*)inp,
                                                                                (const bf16*)dout, n);
    else
        gelu_backward_kernel<float><<<stream_grid_bwd(nvec), kBwdThreads, 0, s>>>((float*)dinp, (const float*)inp,
                                                                                 (const float*)dout, n);
    return launch_status();
}

int launch_layernorm_backward(void* dinp, void* dgamma, void* dbeta, const void* dres, const void* dout,
                              const void* inp, const void* gamma, const float* mean, const float* rstd, int N, int C,
                              int dtype, void* ws, hipStream_t s) {
    if (dtype == GPT2_BF16)
        launch_ln_bwd_t<bf16>((bf16*)dinp, (bf16*)dgamma, (bf16*)dbeta, (const bf16*)dres, (const bf16*)dout,
                              (const bf16*)inp, (const bf16*)gamma, mean, rstd, N, C, ws, s);
    else
        launch_ln_bwd_t<float>((float*)dinp, (float*)dgamma, (float*)dbeta, (const float*)dres, (const float*)dout,
                               (const float*)inp, (const float*)gamma, mean, rstd, N, C, ws, s);
    return launch_status();
}

}  // namespace gpt2

using namespace gpt2;

// ------------------------------------------------------------------ C ABI
extern "C" int gelu_backward(void* dinp, const void* inp, const void* dout, int64_t n, int dtype, void* stream) {
    if (!valid_dtype(dtype) || n < 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (n == 0) return GPT2_OK;
    if (!dinp || !inp || !dout || dinp == inp) return GPT2_ERR_INVALID_ARGUMENT;
    if (!aligned16(dinp) || !aligned16(inp) || !aligned16(dout)) return GPT2_ERR_UNSUPPORTED;
    return launch_gelu_backward(dinp, inp, dout, n, dtype, (hipStream_t)stream);
}

extern "C" int64_t layernorm_backward_workspace_size(int N, int C) {
    if (N < 0 || C <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    return layernorm_backward_workspace_bytes(N, C);
}

extern "C" int layernorm_backward(void* dinp, void* dgamma, void* dbeta, const void* dres, const void* dout,
                                  const void* inp, const void* gamma, const float* mean, const float* rstd, int N,
                                  int C, int dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || C <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!dinp || !dout || !inp || !gamma || !mean || !rstd || !workspace) return GPT2_ERR_INVALID_ARGUMENT;
    if (dinp == dout || dinp == inp) return GPT2_ERR_INVALID_ARGUMENT;
    const int V = dtype == GPT2_BF16 ? 8 : 4;
    if (C % 8 || C / V > 8 * 64 || !aligned16(dinp) || !aligned16(dout) || !aligned16(inp) || !aligned16(gamma) ||
        (dres && !aligned16(dres)))
        return GPT2_ERR_UNSUPPORTED;
    if (workspace_bytes < layernorm_backward_workspace_bytes(N, C)) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    return launch_layernorm_backward(dinp, dgamma, dbeta, dres, dout, inp, gamma, mean, rstd, N, C, dtype, workspace,
                                     (hipStream_t)stream);
}

extern "C" int64_t matmul_backward_workspace_size(int N, int C, int OC, int dtype) {
    if (!valid_dtype(dtype) || N < 0 || C <= 0 || OC <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    return matmul_backward_workspace_bytes(N, C, OC, dtype);
}

extern "C" int matmul_backward(void* dinp, void* dweight, void* dbias, const void* dout, const void* inp,
                               const void* weight, int N, int C, int OC, int dtype, void* workspace,
                               int64_t workspace_bytes, void* stream) {
    if (!valid_dtype(dtype) || N < 0 || C <= 0 || OC <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    if (N == 0) return GPT2_OK;
    if (!dout || (dinp && !weight) || (dweight && !inp) || !workspace) return GPT2_ERR_INVALID_ARGUMENT;
    if (!dinp && !dweight && !dbias) return GPT2_OK;
    if (C % 8 || OC % 8 || !aligned16(dout) || (dinp && !aligned16(dinp)) || (dweight && !aligned16(dweight)) ||
        (inp && !aligned16(inp)) || (weight && !aligned16(weight)) || !aligned16(workspace))
        return GPT2_ERR_UNSUPPORTED;
    if (dinp && (dinp == dout || dinp == inp || dinp == weight)) return GPT2_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < matmul_backward_workspace_bytes(N, C, OC, dtype)) return GPT2_ERR_WORKSPACE_TOO_SMALL;
    return launch_matmul_backward(dinp, dweight, dbias, dout, inp, weight, N, C, OC, dtype, workspace,
                                  (hipStream_t)stream, nullptr);
}

extern "C" int encoder_backward(void* dwte, void* dwpe, const void* dout, const int32_t* tokens, int B, int T, int C,
                                int dtype, void* stream) {
    if (!valid_dtype(dtype) || B < 0 || T < 0 || C <= 0) return GPT2_ERR_INVALID_ARGUMENT;
    if ((int64_t)B * T == 0) return GPT2_OK;
    if (!dout || !tokens || (!dwte && !dwpe)) return GPT2_ERR_INVALID_ARGUMENT;
    const int V = dtype == GPT2_BF16 ? 8 : 4;
    if (C % 8 || C / V > 256 * kEncMaxVecPerThread || !aligned16(dout) || (dwte && !aligned16(dwte)) ||
        (dwpe && !aligned16(dwpe)))
        return GPT2_ERR_UNSUPPORTED;
    return launch_encoder_backward(dwte, dwpe, dout, tokens, B, T, C, dtype, (hipStream_t)stream);
}
