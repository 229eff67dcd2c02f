// Elementwise and row kernels of the post-LN decoder layer ([SRC]
// "Transformer-XL模型 核心源码阅读笔记": PositionalEmbedding,
// PositionwiseFF.forward, RelPartialLearnableMultiHeadAttn.forward with
// pre_lnorm = False).  The projections are plain GEMMs (rocBLAS); these
// kernels are everything in between.

#include <hip/hip_runtime.h>
#include <stdint.h>

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
__global__ void pos_emb_kernel(uint16_t *out, int K, int d, int clamp_len)
{
    const int half = d / 2;
    const int64_t total = (int64_t)K * half;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(e / half), t = (int)(e - (int64_t)c * half);
        int p = K - 1 - c;
        if (clamp_len > 0 && p > clamp_len) p = clamp_len;
        const double f = exp(-(2.0 * t / d) * 9.210340371976184);   // ln(10000)
        const double ang = p * f;
        out[(int64_t)c * d + t] = f32_to_bf16((float)sin(ang));
        out[(int64_t)c * d + half + t] = f32_to_bf16((float)cos(ang));
    }
}

// y = max(x + b, 0) rounded to bf16; x [N][n] fp32, b [n] fp32 (may be NULL).
__global__ void bias_relu_kernel(const float *x, const float *b, uint16_t *y, int64_t N, int n)
{
    const int64_t total = N * n;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int col = (int)(e % n);
        float v = x[e] + (b ? b[col] : 0.f);
        y[e] = f32_to_bf16(v > 0.f ? v : 0.f);
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
    hipLaunchKernelGGL(pos_emb_kernel, dim3(grid_for((int64_t)K * (d / 2))), dim3(256), 0, s, out, K, d, clamp_len);
    return hipGetLastError();
}

hipError_t launch_bias_relu(const float *x, const float *b, uint16_t *y, int64_t N, int n, hipStream_t s)
{
    hipLaunchKernelGGL(bias_relu_kernel, dim3(grid_for(N * n)), dim3(256), 0, s, x, b, y, N, n);
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
