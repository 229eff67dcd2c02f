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

__device__ __forceinline__ float block_sum(float v, float *red)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < LN_THREADS / 64; ++i) s += red[i];
    return s;
}

// out = LN(res + add + bias) * g + beta over rows of d ([SRC] nn.LayerNorm:
// biased variance, eps).  res bf16 [N][d], add fp32 [N][d], bias fp32 [d] or
// NULL, out bf16.  One workgroup per row; two passes (mean, then the centred
// second moment) over values held in registers.
constexpr int LN_MAXV = 16;   // values per thread: d <= 4096
__global__ __launch_bounds__(LN_THREADS) void add_layer_norm_kernel(const uint16_t *res, const float *add,
                                                                    const float *bias, const float *g,
                                                                    const float *beta, uint16_t *out, int d,
                                                                    float eps)
{
    __shared__ float red[LN_THREADS / 64];
    const int64_t row = blockIdx.x;
    const uint16_t *rp = res + row * d;
    const float *ap = add + row * d;
    float v[LN_MAXV];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
        const int col = threadIdx.x + i * LN_THREADS;
        v[i] = 0.f;
        if (col < d) {
            v[i] = bf16_to_f32(rp[col]) + ap[col] + (bias ? bias[col] : 0.f);
            s += v[i];
        }
    }
    const float mean = block_sum(s, red) / d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
        const int col = threadIdx.x + i * LN_THREADS;
        if (col < d) {
            const float c = v[i] - mean;
            q += c * c;
        }
    }
    const float var = block_sum(q, red) / d;
    const float inv = 1.f / sqrtf(var + eps);
    uint16_t *op = out + row * d;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
        const int col = threadIdx.x + i * LN_THREADS;
        if (col < d) op[col] = f32_to_bf16((v[i] - mean) * inv * g[col] + beta[col]);
    }
}

int grid_for(int64_t n)
{
    int64_t b = (n + 255) / 256;
    return (int)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

int layer_norm_max_width() { return LN_THREADS * LN_MAXV; }

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
    if (d > LN_THREADS * LN_MAXV || N > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(add_layer_norm_kernel, dim3((unsigned)N), dim3(LN_THREADS), 0, s, res, add, bias, g, beta,
                       out, d, eps);
    return hipGetLastError();
}

}  // namespace txl
