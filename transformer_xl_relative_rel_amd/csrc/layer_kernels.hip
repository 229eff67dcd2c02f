// Elementwise and row kernels of the post-LN decoder layer ([SRC]
// "Transformer-XL模型 核心源码阅读笔记": PositionalEmbedding,
// PositionwiseFF.forward, RelPartialLearnableMultiHeadAttn.forward with
// pre_lnorm = False).  The projections are plain GEMMs (rocBLAS); these
// kernels are everything in between.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "internal.h"

namespace txl {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Round to nearest even (inputs are finite in this layer; NaN keeps a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// [SRC] PositionalEmbedding: row c of [K][d] is position p = K-1-c;
// columns [0, d/2) are sin(p f_t), [d/2, d) are cos(p f_t), f_t = 10000^(-2t/d).
// Thread (t, row block): f_t once in fp64, then for each row the angle p f_t
// in fp64, reduced to [-pi, pi] in fp64 (two-part 2 pi), sin and cos of the
// reduced angle in fp32 (error ~1e-7, far below the bf16 rounding of the
// stored value).
constexpr int POS_ROWS = 4;    // rows per workgroup
__global__ __launch_bounds__(256) void pos_emb_kernel(uint16_t *out, int K, int d, int clamp_len)
{
    const int half = d / 2;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= half) return;
    const double f = exp(-(2.0 * t / d) * 9.210340371976184);   // ln(10000)
    const double two_pi_hi = 6.283185307179586, two_pi_lo = 2.4492935982947064e-16;
    for (int c0 = blockIdx.y * POS_ROWS; c0 < K; c0 += gridDim.y * POS_ROWS) {
        const int c1 = min(K, c0 + POS_ROWS);
        for (int c = c0; c < c1; ++c) {
            int p = K - 1 - c;
            if (clamp_len > 0 && p > clamp_len) p = clamp_len;
            const double ang = p * f;
            const double k = rint(ang / two_pi_hi);
            const float red = (float)((ang - k * two_pi_hi) - k * two_pi_lo);
            float sv, cv;
            sincosf(red, &sv, &cv);
            out[(int64_t)c * d + t] = f32_to_bf16(sv);
            out[(int64_t)c * d + half + t] = f32_to_bf16(cv);
        }
    }
}

// y = max(x + b, 0) rounded to bf16; x [N][n] fp32, b [n] fp32 (may be NULL);
// n a multiple of 8.  Each thread moves 8 consecutive values.
__global__ __launch_bounds__(256) void bias_relu_kernel(const float *x, const float *b, uint16_t *y, int64_t N, int n)
{
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int n8 = n / 8;
    const int64_t total = N * n8;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = e / n8;
        const int col = (int)(e - row * n8) * 8;
        const f32x4v *xp = reinterpret_cast<const f32x4v *>(x + row * n + col);
        f32x4v v0 = xp[0], v1 = xp[1];
        if (b) {
            v0 += *reinterpret_cast<const f32x4v *>(b + col);
            v1 += *reinterpret_cast<const f32x4v *>(b + col + 4);
        }
        u32x4v o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float lo = k < 2 ? v0[2 * k] : v1[2 * k - 4], hi = k < 2 ? v0[2 * k + 1] : v1[2 * k - 3];
            o[k] = (uint32_t)f32_to_bf16(lo > 0.f ? lo : 0.f) | ((uint32_t)f32_to_bf16(hi > 0.f ? hi : 0.f) << 16);
        }
        *reinterpret_cast<u32x4v *>(y + row * n + col) = o;
    }
}

constexpr int LN_THREADS = 256;

// Sum over a 256-thread workgroup, the result in every thread: DPP row sums
// (lanes 1, 2 apart, then the half-row and row mirrors), the four rows of a
// wave read out by lane, then the four waves through LDS.
template <int CTRL> __device__ __forceinline__ float ln_dpp_add(float x)
{
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float block_sum(float v, float *red)
{
    v = ln_dpp_add<0xb1>(v);    // quad_perm [1, 0, 3, 2]
    v = ln_dpp_add<0x4e>(v);    // quad_perm [2, 3, 0, 1]
    v = ln_dpp_add<0x141>(v);   // row_half_mirror
    v = ln_dpp_add<0x140>(v);   // row_mirror
    const int vi = __builtin_bit_cast(int, v);
    v = (__builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 0)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 16))) +
        (__builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 32)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(vi, 48)));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// out = LN(res + add + bias) * g + beta over rows of d ([SRC] nn.LayerNorm:
// biased variance, eps).  res bf16 [N][d], add fp32 [N][d], bias fp32 [d] or
// NULL, out bf16; d a multiple of 4 and 16-byte aligned rows and vectors.
// One workgroup per row; thread t holds columns 4 t + 1024 c .. + 3 for
// chunks c, loaded before any arithmetic; two passes (mean, then the centred
// second moment) over the values held in registers.
constexpr int LN_CHUNKS = 4;   // d <= LN_THREADS * 4 * LN_CHUNKS = 4096
__global__ __launch_bounds__(LN_THREADS) void add_layer_norm_kernel(const uint16_t *res, const float *add,
                                                                    const float *bias, const float *g,
                                                                    const float *beta, uint16_t *out, int d,
                                                                    float eps)
{
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    __shared__ float red[2][LN_THREADS / 64];
    const int64_t row = blockIdx.x;
    const uint16_t *rp = res + row * d;
    const float *ap = add + row * d;
    u32x2v rv[LN_CHUNKS];
    f32x4v av[LN_CHUNKS], bv[LN_CHUNKS];
#pragma unroll
    for (int c = 0; c < LN_CHUNKS; ++c) {
        const int col = 4 * (threadIdx.x + c * LN_THREADS);
        rv[c] = u32x2v{0u, 0u};
        av[c] = bv[c] = f32x4v{0.f, 0.f, 0.f, 0.f};
        if (col < d) {
            rv[c] = *reinterpret_cast<const u32x2v *>(rp + col);
            av[c] = *reinterpret_cast<const f32x4v *>(ap + col);
            if (bias) bv[c] = *reinterpret_cast<const f32x4v *>(bias + col);
        }
    }
    f32x4v v[LN_CHUNKS];
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < LN_CHUNKS; ++c) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t w = rv[c][k >> 1];
            v[c][k] = bf16_to_f32((uint16_t)((k & 1) ? (w >> 16) : (w & 0xffffu))) + av[c][k] + bv[c][k];
        }
        s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);   // zero past d
    }
    const float mean = block_sum(s, red[0]) / d;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < LN_CHUNKS; ++c) {
        if (4 * (threadIdx.x + c * LN_THREADS) < d) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float x = v[c][k] - mean;
                q += x * x;
            }
        }
    }
    const float var = block_sum(q, red[1]) / d;
    const float inv = 1.f / sqrtf(var + eps);
    uint16_t *op = out + row * d;
#pragma unroll
    for (int c = 0; c < LN_CHUNKS; ++c) {
        const int col = 4 * (threadIdx.x + c * LN_THREADS);
        if (col < d) {
            const f32x4v gg = *reinterpret_cast<const f32x4v *>(g + col);
            const f32x4v bb = *reinterpret_cast<const f32x4v *>(beta + col);
            u32x2v o;
#pragma unroll
            for (int k = 0; k < 2; ++k)
                o[k] = (uint32_t)f32_to_bf16((v[c][2 * k] - mean) * inv * gg[2 * k] + bb[2 * k]) |
                       ((uint32_t)f32_to_bf16((v[c][2 * k + 1] - mean) * inv * gg[2 * k + 1] + bb[2 * k + 1]) << 16);
            *reinterpret_cast<u32x2v *>(op + col) = o;
        }
    }
}

int grid_for(int64_t n)
{
    int64_t b = (n + 255) / 256;
    return (int)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

int layer_norm_max_width() { return LN_THREADS * 4 * LN_CHUNKS; }

hipError_t launch_pos_emb(uint16_t *out, int K, int d, int clamp_len, hipStream_t s)
{
    if (K <= 0 || d < 2) return hipSuccess;
    const int ry = std::min((K + POS_ROWS - 1) / POS_ROWS, 65535);
    hipLaunchKernelGGL(pos_emb_kernel, dim3((unsigned)((d / 2 + 255) / 256), (unsigned)ry), dim3(256), 0, s, out, K, d,
                       clamp_len);
    return hipGetLastError();
}

hipError_t launch_bias_relu(const float *x, const float *b, uint16_t *y, int64_t N, int n, hipStream_t s)
{
    if (n % 8 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(bias_relu_kernel, dim3(grid_for(N * (n / 8))), dim3(256), 0, s, x, b, y, N, n);
    return hipGetLastError();
}

hipError_t launch_add_layer_norm(const uint16_t *res, const float *add, const float *bias, const float *g,
                                 const float *beta, uint16_t *out, int64_t N, int d, float eps, hipStream_t s)
{
    if (d > LN_THREADS * 4 * LN_CHUNKS || d % 4 || N > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(add_layer_norm_kernel, dim3((unsigned)N), dim3(LN_THREADS), 0, s, res, add, bias, g, beta,
                       out, d, eps);
    return hipGetLastError();
}

}  // namespace txl
