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
constexpr int kThreads = 256;
constexpr int kUnroll = 2;      // 16-byte words per thread

// grid: x over the 16-byte words of one batch row's new memory, y over
// (buffer, batch row).  Every load of a thread is issued before its stores.
// The stores are non-temporal (the new memory is next read a whole segment
// later); the loads are plain, so a source the previous step left in the
// last-level cache is read from there (17 buffers of [4, 512, 1024] bf16:
// 21.7 us with plain loads against 24.4 us with non-temporal ones; on copies
// of several GB, which no longer fit that cache, non-temporal loads are ~5%
// faster).
__global__ __launch_bounds__(kThreads) void mem_update_kernel(MemUpdateArgs a)
{
    const int buf = (int)blockIdx.y / a.B;
    const int b = (int)blockIdx.y - buf * a.B;
    const unsigned char *mem = a.mem[buf] ? a.mem[buf] + b * a.mem_bs : nullptr;
    const unsigned char *hh = a.h[buf] + b * a.h_bs;
    unsigned char *dst = a.dst[buf] + b * a.new_bs;
    const uint32_t per_batch = (uint32_t)a.M_new * (uint32_t)a.row_chunks;
    const uint32_t rc = (uint32_t)a.row_chunks;
    const uint32_t e0 = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    u32x4 val[kUnroll];
    // When every row of the new memory comes from one source (all of it from
    // h, as in a stack whose memory length equals the segment length, or all
    // from mem), the chunks are contiguous in that source and need no row split.
    const unsigned char *one = nullptr;
    if (a.beg >= a.M_cur) one = hh + (int64_t)(a.beg - a.M_cur) * rc * 16;
    else if (a.beg + a.M_new <= a.M_cur) one = mem + (int64_t)a.beg * rc * 16;
    if (one) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t e = e0 + u * kThreads;
            if (e < per_batch) val[u] = *reinterpret_cast<const u32x4 *>(one + (int64_t)e * 16);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t e = e0 + u * kThreads;
            if (e < per_batch) {
                const uint32_t t = e / rc;                  // row of the new memory
                const uint32_t c = e - t * rc;
                const int src_row = a.beg + (int)t;         // row of cat([mem; h])
                const unsigned char *src = (src_row < a.M_cur) ? mem + ((int64_t)src_row * rc + c) * 16
                                                               : hh + ((int64_t)(src_row - a.M_cur) * rc + c) * 16;
                val[u] = *reinterpret_cast<const u32x4 *>(src);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t e = e0 + u * kThreads;
        if (e < per_batch) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4 *>(dst + (int64_t)e * 16));
    }
}

}  // namespace

hipError_t launch_mem_update(const MemUpdateArgs &a, hipStream_t s)
{
    const int64_t per_batch = (int64_t)a.M_new * a.row_chunks;
    if (per_batch == 0 || a.n_buf == 0 || a.B == 0) return hipSuccess;
    if (per_batch >= ((int64_t)1 << 31) || (int64_t)a.n_buf * a.B > 65535) return hipErrorInvalidValue;
    const int64_t blocks = (per_batch + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    hipLaunchKernelGGL(mem_update_kernel, dim3((unsigned)blocks, (unsigned)(a.n_buf * a.B)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace txl
