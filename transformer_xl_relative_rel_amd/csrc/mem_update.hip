// Memory update (Tail_M) as one coalesced copy kernel.
//
// [SRC] "Transformer-XL模型 核心源码阅读笔记", MemTransformerLM._update_mems:
// the next memory of every layer is rows [beg, end) of cat([mem; h]) along
// the sequence, end = M_cur + max(0, L - ext_len), beg = max(0, end - mem_len).
// [XL] "Transformer-XL" textbook notes, "Segment-Level Recurrence", names the
// ext_len = 0 case Tail_M.  Rows are moved as 16-byte words, so the copy is
// bit-exact for any element type.  blockIdx.y selects one of up to
// kMaxMemBuffers independent buffers (the per-layer memories of a stack).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace txl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 4;

__global__ __launch_bounds__(256) void mem_update_kernel(MemUpdateArgs a)
{
    const int buf = blockIdx.y;
    const unsigned char *mem = a.mem[buf];
    const unsigned char *hh = a.h[buf];
    unsigned char *dst = a.dst[buf];
    const int64_t per_batch = (int64_t)a.M_new * a.row_chunks;
    const int64_t total = per_batch * a.B;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < total; base += stride * kUnroll) {
        u32x4 val[kUnroll];
        unsigned char *out[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t e = base + u * stride;
            out[u] = nullptr;
            if (e < total) {
                const int b = (int)(e / per_batch);
                const int64_t rem = e - (int64_t)b * per_batch;
                const int t = (int)(rem / a.row_chunks);          // row of the new memory
                const int c = (int)(rem - (int64_t)t * a.row_chunks);
                const int src_row = a.beg + t;                      // row of cat([mem; h])
                const unsigned char *src = (src_row < a.M_cur)
                    ? mem + b * a.mem_bs + ((int64_t)src_row * a.row_chunks + c) * 16
                    : hh + b * a.h_bs + ((int64_t)(src_row - a.M_cur) * a.row_chunks + c) * 16;
                val[u] = *reinterpret_cast<const u32x4 *>(src);
                out[u] = dst + b * a.new_bs + ((int64_t)t * a.row_chunks + c) * 16;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (out[u]) *reinterpret_cast<u32x4 *>(out[u]) = val[u];
    }
}

}  // namespace

hipError_t launch_mem_update(const MemUpdateArgs &a, hipStream_t s)
{
    const int64_t total = (int64_t)a.M_new * a.row_chunks * a.B;
    if (total == 0 || a.n_buf == 0) return hipSuccess;
    int64_t blocks = (total + 256 * kUnroll - 1) / (256 * kUnroll);
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(mem_update_kernel, dim3((unsigned)blocks, (unsigned)a.n_buf), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace txl
