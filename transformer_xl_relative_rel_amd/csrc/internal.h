// Internal launch interface between the host API (txl_api.cpp) and the HIP
// kernels.  Not installed; not part of the C ABI.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace txl {

// Keys per staged tile of the fused attention kernel and waves per workgroup.
constexpr int kBK = 64;
constexpr int kWaves = 4;

// One Tail_M update carried out by an attention launch (nchunks = 0: none).
// Work unit: 1 KB chunk `ch` of row t of batch row b of the new memory,
// numbered ((b * M_new + t) * cpr + ch); source row beg + t of [mem; h].
struct FusedCopy {
    const unsigned char *mem, *h;   // batch row 0 of each source
    unsigned char *dst;
    int64_t mem_bs, h_bs, new_bs;   // batch strides in bytes
    int M_cur, beg, M_new, B;
    int row_bytes;                  // bytes per row, a multiple of 16
    int cpr;                        // 1 KB chunks per row
    int nchunks;                    // B * M_new * cpr
    int inc_ch, inc_t, inc_b;       // chunk-number stride between a wave's chunks (the launch's
                                    // wave count) as (batch row, row, chunk) steps; set at launch
};

struct RelAttnArgs {
    const void *q, *k, *v, *r;
    const float *u, *vb;
    void *out;
    float *lse;
    float *part_o;   // unnormalised partial outputs (split path): [nsplit][B*H][L][dh] row-major, or with
                     // part_native [nsplit][B*H][ceil(L/16)][dh/16][64] 16-byte groups, group (dt, 16 g + n)
                     // holding query 16 blk + n, head columns 16 dt + 4 g .. + 3 (the bf16 kernels' MFMA
                     // result layout, so that a wave stores 1 KB contiguously per instruction)
    float *part_ml;  // [nsplit][B*H][L][2]  running max (log2 units) and denominator
    int part_native;
    int64_t qs[3], ks[3], vs[3], os[3], rs[2];
    int B, H, L, M, K;
    float c;          // scale * log2(e)
    int nqb;          // query blocks of 16 * kWaves * rb rows
    int nsplit;       // key-range splits (1 = normalise in the kernel)
    int tiles_per_split;
    int remap;        // XCD-aware workgroup order: 0 none, 1 blocks of (b, h) pairs (B*H % 8 == 0),
                      // 2 heads h = x (mod 8) of every batch row on XCD x (H % 8 == 0)
    const int *mem_valid;   // [B] valid memory rows per batch row, or NULL (all M)
    int window;             // > 0: query i sees keys j >= i + M + 1 - window
    FusedCopy cp;           // memory update done by the bf16 throughput kernel's waves
};
// The bf16 throughput kernel reads `cp` at offsetof(RelAttnArgs, cp) in its
// kernel argument segment (RelAttnArgs is its only argument).
static_assert(std::is_standard_layout<RelAttnArgs>::value && std::is_trivially_copyable<RelAttnArgs>::value,
              "kernel arguments are read by byte offset");

// First key visible to query i of batch row b: keys below it are masked.
__device__ __forceinline__ int key_lo(const RelAttnArgs &a, int b, int i)
{
    int lo = 0;
    if (a.mem_valid) {
        int mv = a.mem_valid[b];
        mv = mv < 0 ? 0 : (mv > a.M ? a.M : mv);
        lo = a.M - mv;
    }
    if (a.window > 0) {
        const int w = i + a.M + 1 - a.window;
        lo = w > lo ? w : lo;
    }
    return lo;
}

// Flat (b, h) index of the j-th pair that the XCD-aware order places on XCD x
// (workgroup w runs on XCD w % 8).  With remap 2 every batch row of a head
// runs on one XCD, so the head's r rows, which all batch rows read, are
// fetched into one L2 only; with remap 1 each XCD owns B*H/8 consecutive pairs.
__device__ __forceinline__ int xcd_pair(const RelAttnArgs &a, int x, int j)
{
    if (a.remap == 2) {
        const int hx = a.H >> 3;
        const int b = j / hx;
        return b * a.H + (j - b * hx) * 8 + x;
    }
    return x * ((a.B * a.H) >> 3) + j;
}

// rb = 16-row blocks per wave (1 or 2).  dtype: 0 = f32, 1 = bf16.
bool relattn_supported(int dtype, int dh, int rb);
hipError_t launch_relattn(const RelAttnArgs &a, int dtype, int dh, int rb, hipStream_t s);

// bf16 throughput kernel (dh = 64): workgroups per (b, h) along the queries
// (before key splits), and launch.
int relattn_bf16_groups_per_head(int L);
bool relattn_bf16_supported(int dh);
hipError_t launch_relattn_bf16(const RelAttnArgs &a, int dh, hipStream_t s);
// bf16 streaming kernel (dh = 64, no lower key bounds): nqb = query runs per
// head, one one-wave workgroup per (b*h, key split, run).
int relattn_bf16_stream_runs(int L);
hipError_t launch_relattn_bf16_stream(const RelAttnArgs &a, int dh, hipStream_t s);
// Key-range combine used by both kernels when nsplit > 1.
hipError_t launch_relattn_combine(const RelAttnArgs &a, int dtype, int dh, hipStream_t s);

// Backward of the relative attention (relattn_bwd_bf16.hip): bf16, dh = 64.
struct RelAttnBwdArgs {
    const void *q, *k, *v, *r, *out, *dout;
    const float *u, *vb, *lse;
    void *dq, *dk, *dv;
    float *dr, *du, *dvb;
    int64_t qs[3], ks[3], vs[3], os[3], rs[2];   // q/dq, k/dk, v/dv, out/dout (elements), r
    int B, H, L, M, K;
    float c;          // scale * log2(e)
    float scale;
    const int *mem_valid;
    int window;
    // workspace
    uint16_t *qu, *qv;      // [B*H][L][64] bf16: c (q + u), c (q + vb)
    float *dd, *lse2;       // [B*H][L]: rowsum(dout * out), lse * log2(e)
    uint16_t *g;            // [B*H][L][kp] bf16: dS of (i, j) at column L-1-i+j
    float *bias_part;       // [nsplit][B*H][nqblk][2][64]: per 16-query block sums of dq's two parts
    float *dq_part;         // [nsplit][B*H][L][64] fp32 partial dq of each key split (nsplit > 1)
    int kp;                 // row stride of g (K rounded up to 64)
    int nqblk;              // 16-query blocks per head
    int nsplit, tps;        // key splits of the dq kernel and key tiles per split
};

size_t relattn_bwd_workspace_bytes(int B, int H, int L, int M);
// Carves the workspace into a's workspace pointers (ws 256-byte aligned).
void relattn_bwd_carve(RelAttnBwdArgs &a, void *ws);
hipError_t launch_relattn_bwd_bf16(const RelAttnBwdArgs &a, hipStream_t s);

// Static scratch of the entry points that allocate nothing (noalloc_scratch.hip):
// its size, and its device address on the current device (taken on the
// first call there).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_buffer(void **ptr, size_t *bytes);

constexpr int kMaxMemBuffers = 64;

struct MemUpdateArgs {
    const unsigned char *mem[kMaxMemBuffers];
    const unsigned char *h[kMaxMemBuffers];
    unsigned char *dst[kMaxMemBuffers];
    int n_buf;
    int M_cur, beg, M_new, B;
    int row_chunks;                 // 16-byte chunks per row
    int64_t mem_bs, h_bs, new_bs;   // batch strides in bytes
};

hipError_t launch_mem_update(const MemUpdateArgs &a, hipStream_t s);

// Decoder-layer helpers (layer_kernels.hip).  Tensors are bf16 (uint16_t) or fp32.
int layer_norm_max_width();
hipError_t launch_pos_emb(uint16_t *out, int K, int d, int clamp_len, hipStream_t s);
hipError_t launch_bias_relu(const float *x, const float *b, uint16_t *y, int64_t N, int n, hipStream_t s);
hipError_t launch_add_layer_norm(const uint16_t *res, const float *add, const float *bias, const float *g,
                                 const float *beta, uint16_t *out, int64_t N, int d, float eps, hipStream_t s);

}  // namespace txl
