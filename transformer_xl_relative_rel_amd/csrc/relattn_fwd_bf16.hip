// Fused relative-position attention, forward, bf16 in / fp32 accumulate, for
// gfx950: the throughput path (dh = 64).
//
// Computes the same function as relattn_fwd.hip ([SRC] "Transformer-XL模型
// 核心源码阅读笔记", RelPartialLearnableMultiHeadAttn.forward; [XL]
// "Transformer-XL" textbook notes, "Relative Positional Encoding" and "Causal
// Mask With Memory"):
//   s_ij = scale * ((q_i + u) . k_j + (q_i + vb) . r[L-1-i+j]),
//   visible iff j <= i + M,  out_i = softmax_j(s_ij) . v_j.
//
// Work decomposition.  A workgroup is 8 waves (two per SIMD) and owns 256
// query rows of one (b, h); each wave owns 32 rows as two 16-query blocks.
// Keys are walked in tiles of 64.  Waves w and w + 4 share a SIMD and own
// 32-query blocks s and 7 - s, whose key ranges add up to the same length.
//
// Everything is computed transposed (keys on MFMA rows, queries on lanes):
//   T^T = R_band . (c (q + vb))^T - m   with c = scale * log2(e) folded into
//       the query operand and the running row max m of each query folded into
//       the accumulator's initial value; 16 queries need 79 consecutive r rows
//       per 64-key tile: 5 band MFMA tiles;
//   the band value of (query n, r row cc) belongs to key jj = cc + n - 15: it
//   is written to a per-wave LDS row at column cc + n + 1 and read back in key
//   order as the initial accumulator of
//   S'^T = K . (c (q + u))^T + T^T      = log2-domain score minus row max;
//   mask j <= i + M (only on tiles that cross the diagonal), p = exp2(S');
//   the running max is raised only when a score exceeds it by more than 2^8
//   (rare branch; a query's first visible tile sets it exactly);
//   P comes out of the score MFMA in the B-operand layout of
//   O^T += V^T . P^T  with V^T fragments read from row-major V through the
//   transposing LDS read; the denominator is one more MFMA against ones.
// The two blocks of a wave are software-pipelined: the softmax of block 0
// sits in one basic block with the band and content MFMAs of block 1 and the
// P.V MFMAs of block 0.
//
// LDS: double-buffered K and V tiles, a ring of r rows (a tile uses 320 rows;
// the 64 rows the next tile adds go into the free quarter), one skew buffer
// per wave.  Tiles move HBM -> LDS with direct-to-LDS loads issued one tile
// ahead; rows are 16-byte chunks with an XOR swizzle so that the 16 lanes of a
// fragment read hit distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace txl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int DH = 64;
constexpr int NW = 8;            // waves per workgroup (two per SIMD)
constexpr int RB = 2;            // 16-query blocks per wave
constexpr int BQ = NW * RB * 16; // queries per workgroup
constexpr int BK = 64;           // keys per tile
constexpr int NT = BK / 16;      // 16-key sub-tiles per tile
constexpr int NBT = NT + 1;      // band tiles per 16-query block
constexpr int NWB = NT + RB;     // band tiles per wave
constexpr int NQ = (BQ + BK - 1 + 63) / 64 + 1;   // ring quarters: those a tile uses plus one loading
constexpr int RING = 64 * NQ;    // r rows held in LDS
constexpr int SROW = 84;         // skew buffer row stride (floats)
constexpr int SKEW = 16 * SROW + 16;
constexpr int CPR = DH / 8;      // 16-byte chunks per row
constexpr int RP = 16 / CPR;     // rows per 256 bytes
constexpr int NKK = DH / 32;     // MFMA k-steps over dh
constexpr int NDT = DH / 16;     // 16-wide output tiles over dh
constexpr int TILE_CH = BK * CPR;              // chunks per K or V tile (and per ring quarter)
constexpr float LN2 = 0.69314718055994530942f;
constexpr float TAU = 8.0f;      // deferred-rescale threshold (log2 units)
static_assert(BQ + BK <= RING - 64, "ring must have a free quarter");
static_assert(TILE_CH == NW * 64, "one 16-byte chunk of each tile per thread");

// Swizzle of chunk c in row r: K and r rows (16-row b128 fragment reads), V
// rows (transposing b64 reads of 4 rows x 32 bytes).
__device__ __forceinline__ int swz_k(int r) { return ((unsigned)r / RP) & (CPR - 1); }
__device__ __forceinline__ int swz_v(int r) { return (r & 6) & (CPR - 1); }

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t x16) { return __uint_as_float(x16 << 16); }

__device__ __forceinline__ float row_max4(float x)
{
    // max over the four 16-lane groups that hold one query
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Direct HBM -> LDS load of 16 bytes per lane through a buffer resource: lane
// l of the wave writes LDS byte address lds + 16 l.  Byte offsets at or past
// the resource's size (negative ones included, as unsigned) read zeros.
// Written as inline assembly so that the compiler does not track the load:
// its own tracking of direct-to-LDS loads makes it wait for them before any
// LDS read it cannot prove disjoint, which defeats the prefetch.  The caller
// waits (s_waitcnt vmcnt(0) and a barrier) before anything reads the target.
// M0 is saved and restored around the load.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds)
        : "memory");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(LDS_AS const void *)p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

struct Tile {
    bool first;  // first tile of this key range
    const u32x4 *sk, *sv, *sr;
    float *skw;
    int kt;      // key tile index (selects the ring quarters)
    int wband;   // first row of this wave's band inside the workgroup band
    int j0, wq0, M;
};

// Per-wave state carried across key tiles.
struct State {
    bf16x8 qu[RB][NKK], qv[RB][NKK];   // c (q + u), c (q + vb): B operands, lane (g, n) = query n
    f32x4 o[RB][NDT];                   // O^T accumulators (unnormalised)
    f32x4 lsum[RB];                     // softmax denominators (all 4 entries equal)
    float mneg[RB];                     // -m: initial accumulator value of the band MFMA
    float mref[RB];                     // running max (log2 units)
    int klo[RB];                        // first visible key of this lane's query (lower bound)
};

// LOWER: some query has a lower key bound (window or memory validity), so a
// query's first visible tile need not be the first tile of the range.
template <bool MASK, bool LOWER>
__device__ __forceinline__ void tile_body(State &st, const Tile &t, int g, int n)
{
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    const int d0 = 4 * g - n;   // key offset minus query offset of this lane

    // K fragments (A operands of the content MFMA)
    auto load_k = [&](bf16x8 (&kf)[NT][NKK]) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int krow = 16 * tt + n;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                kf[tt][kk] = __builtin_bit_cast(bf16x8, t.sk[krow * CPR + ((4 * kk + g) ^ swz_k(krow))]);
        }
    };
    // V^T fragments (A operands of P.V), read through the transposing LDS read
    auto load_v = [&](bf16x8 (&vf)[NT / 2][NDT]) {
        LDS_AS char *vb = (LDS_AS char *)(LDS_AS void *)t.sv;
#pragma unroll
        for (int ch = 0; ch < NT / 2; ++ch)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                // lane (g, n) gets V[32 ch + 4 g + e][16 dt + n] (lo) and the rows 16 below (hi)
                const int row0 = 32 * ch + 4 * g + (n >> 2);
                const int chunk = 2 * dt + ((n >> 1) & 1);
                const int off0 = (row0 * CPR + (chunk ^ swz_v(row0))) * 16 + 8 * (n & 1);
                const int row1 = row0 + 16;
                const int off1 = (row1 * CPR + (chunk ^ swz_v(row1))) * 16 + 8 * (n & 1);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vb + off0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(vb + off1));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                vf[ch][dt] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
            }
    };
    bf16x8 rf[NWB][NKK];
    auto load_r = [&](int wb) {
        // workgroup band row x = wband + 16 wb + n lives in ring quarter (kt + x / 64) % NQ
        const int x0 = t.wband + 16 * wb;
        const int rrow = ((t.kt + (x0 >> 6)) % NQ) * 64 + (x0 & 63) + n;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            rf[wb][kk] = __builtin_bit_cast(bf16x8, t.sr[rrow * CPR + ((4 * kk + g) ^ swz_k(rrow))]);
    };

    f32x4 sc[RB][NT];
    bf16x8 pf[RB][NT / 2];

    // band MFMA of block rb (wave band tiles RB-1-rb .. RB-1-rb+NT) and skew into LDS
    auto stage_a = [&](int rb) {
        // all fragment reads first, then the five chains interleaved, then the skew writes
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) load_r(bt + (RB - 1) - rb);
        const f32x4 m4 = {st.mneg[rb], st.mneg[rb], st.mneg[rb], st.mneg[rb]};
        f32x4 acc[NBT];
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) acc[bt] = mfma(rf[bt + (RB - 1) - rb][0], st.qv[rb][0], m4);
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) acc[bt] = mfma(rf[bt + (RB - 1) - rb][kk], st.qv[rb][kk], acc[bt]);
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
            // band row cc = 16 bt + 4 g + v of query n -> column cc + n + 1
            float *dst = t.skw + n * (SROW + 1) + 16 * bt + 4 * g + 1;
            dst[0] = acc[bt][0];
            dst[1] = acc[bt][1];
            dst[2] = acc[bt][2];
            dst[3] = acc[bt][3];
        }
        wave_lds_sync();
    };
    // content MFMA of block rb on top of the skewed band values
    auto stage_b = [&](int rb) {
        bf16x8 kf[NT][NKK];
        load_k(kf);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 acc = *reinterpret_cast<const f32x4 *>(t.skw + n * SROW + 16 + 16 * tt + 4 * g);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) acc = mfma(kf[tt][kk], st.qu[rb][kk], acc);
            sc[rb][tt] = acc;
        }
        wave_lds_sync();
    };
    // mask, overflow check (rare rescale)
    auto stage_check = [&](int rb) {
        if constexpr (MASK) {
            const int thr = t.M + t.wq0 + 16 * rb - t.j0;   // visible iff 16 tt + v + d0 <= thr
            const int thl = LOWER ? st.klo[rb] - t.j0 - 4 * g : 0;   // and 16 tt + v >= thl
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (16 * tt + v + d0 > thr || (LOWER && 16 * tt + v < thl)) sc[rb][tt][v] = -INFINITY;
        }
        float mx = max3(sc[rb][0][0], sc[rb][0][1], sc[rb][0][2]);
        mx = max3(mx, sc[rb][0][3], sc[rb][1][0]);
        mx = max3(mx, sc[rb][1][1], sc[rb][1][2]);
        mx = max3(mx, sc[rb][1][3], sc[rb][2][0]);
        mx = max3(mx, sc[rb][2][1], sc[rb][2][2]);
        mx = max3(mx, sc[rb][2][3], sc[rb][3][0]);
        mx = max3(mx, sc[rb][3][1], sc[rb][3][2]);
        mx = fmaxf(mx, sc[rb][3][3]);
        // A query that has not seen a visible key yet takes the exact max of its
        // first visible tile; afterwards the max is only raised when a score
        // exceeds it by more than TAU.  Without lower key bounds that tile is
        // the first tile of the range; with them, a query is fresh while its
        // denominator is still empty.
        const bool fresh = LOWER ? st.lsum[rb][0] == 0.f : t.first;
        if ((!LOWER && t.first) ||
            __builtin_amdgcn_ballot_w64(mx > TAU || (LOWER && fresh && mx != -INFINITY)) != 0) {
            const float rmx = row_max4(mx);
            float dlt;
            if (fresh) dlt = (rmx == -INFINITY) ? 0.f : rmx;   // exact max of the first visible tile
            else dlt = fmaxf(rmx, 0.f);                         // only ever raised
            st.mref[rb] += dlt;
            st.mneg[rb] -= dlt;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) sc[rb][tt] -= dlt;
            const float alpha = fresh ? 1.f : __builtin_amdgcn_exp2f(-dlt);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) st.o[rb][dt] *= alpha;
            st.lsum[rb] *= alpha;
        }
    };
    // probabilities as bf16 B fragments
    auto stage_c = [&](int rb) {
#pragma unroll
        for (int ch = 0; ch < NT / 2; ++ch) {
            f32x8 p8;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                p8[v] = __builtin_amdgcn_exp2f(sc[rb][2 * ch][v]);
                p8[4 + v] = __builtin_amdgcn_exp2f(sc[rb][2 * ch + 1][v]);
            }
            pf[rb][ch] = __builtin_convertvector(p8, bf16x8);
        }
    };
    // O^T += V^T . P^T, denominator += ones . P^T
    auto stage_d = [&](int rb) {
        bf16x8 vf[NT / 2][NDT];
        load_v(vf);
#pragma unroll
        for (int ch = 0; ch < NT / 2; ++ch) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) st.o[rb][dt] = mfma(vf[ch][dt], pf[rb][ch], st.o[rb][dt]);
            st.lsum[rb] = mfma(ones, pf[rb][ch], st.lsum[rb]);
        }
    };

    stage_a(0);
    stage_b(0);
    stage_check(0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        stage_c(rb);
        if (rb + 1 < RB) {
            stage_a(rb + 1);
            stage_b(rb + 1);
        }
        stage_d(rb);
        if (rb + 1 < RB) stage_check(rb + 1);
    }
}

template <bool LOWER>
__global__ __launch_bounds__(NW * 64) void relattn_fwd_bf16_kernel(RelAttnArgs a)
{
    __shared__ __attribute__((aligned(16))) u32x4 sk[2][TILE_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sv[2][TILE_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sr[RING * CPR];
    __shared__ __attribute__((aligned(16))) float sskew[NW][SKEW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;

    // ---- which (query block, b*h, key split) this workgroup owns
    const int BH = a.B * a.H;
    const int w = blockIdx.x;
    int slot = w, xg = 0, G = BH;
    if (a.remap) { xg = w & 7; slot = w >> 3; G = BH >> 3; }
    const int per = a.nsplit;
    const int qb_rank = slot / (G * per);
    const int r2 = slot - qb_rank * G * per;
    const int bh = xg * G + r2 / per;
    const int split = r2 % per;
    const int qb = a.nqb - 1 - qb_rank;   // longest query blocks first
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L, M = a.M, K = a.K;
    const int i0 = qb * BQ;
    const int kv_end = min(i0 + BQ, L) + M;
    const int ntile = (kv_end + BK - 1) / BK;
    // keys below the first query's lower bound are hidden from the whole block
    const int kt0 = max(split * a.tiles_per_split, key_lo(a, b, i0) / BK);
    const int kt1 = min(ntile, split * a.tiles_per_split + a.tiles_per_split);

    const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + b * a.qs[0] + h * a.qs[1];
    const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + b * a.ks[0] + h * a.ks[1];
    const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.v) + b * a.vs[0] + h * a.vs[1];
    const uint16_t *rp = reinterpret_cast<const uint16_t *>(a.r) + h * a.rs[0];
    const float *up = a.u + h * DH;
    const float *wp = a.vb + h * DH;
    const int c_base = L - i0 - BQ;   // first r row of the workgroup band at tile 0
    const float c = a.c;              // scale * log2(e)

    // Wave w owns the 32 queries of block qblk; waves w and w + 4 share a SIMD
    // and own blocks s and 7 - s, whose key ranges add up to the same length.
    const int qblk = wave < NW / 2 ? wave : (3 * NW / 2 - 1) - wave;
    const int wq0 = i0 + 16 * RB * qblk;                    // first query of the wave
    const int wband = (BQ - 16 * RB) - 16 * RB * qblk;      // first row of its band in the workgroup band

    State st;
    // ---- query fragments: c (q + u) and c (q + vb), in fp32, rounded once to bf16
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int iq = wq0 + 16 * rb + n;
        const bool ok = iq < L;
        const int iqc = ok ? iq : L - 1;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(qp + (int64_t)iqc * a.qs[2] + kk * 32 + 8 * g);
            f32x8 fu, fv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = bf16_to_f32((raw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                const int col = kk * 32 + 8 * g + e;
                fu[e] = ok ? (x + up[col]) * c : 0.f;
                fv[e] = ok ? (x + wp[col]) * c : 0.f;
            }
            st.qu[rb][kk] = __builtin_convertvector(fu, bf16x8);
            st.qv[rb][kk] = __builtin_convertvector(fv, bf16x8);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) st.o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.lsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.mneg[rb] = 0.f;
        st.mref[rb] = 0.f;
        st.klo[rb] = key_lo(a, b, iqc);
    }
    const int wlo_first = key_lo(a, b, wq0);                      // smallest lower bound of the wave
    const int wlo_last = key_lo(a, b, min(wq0 + 16 * RB - 1, L - 1));   // largest

    // ---- direct loads: thread tid moves chunk tid of each tile (row tid / 8),
    // reading the chunk the XOR swizzle puts at that LDS position.  Rows outside
    // [0, K) read zeros.
    const int lrow = (unsigned)tid / CPR;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)(((int64_t)(K - 1) * a.ks[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)(((int64_t)(K - 1) * a.vs[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rp, (uint32_t)(((int64_t)(K - 1) * a.rs[1] + DH) * 2));
    const int kch = ((tid & (CPR - 1)) ^ swz_k(lrow)) * 16;
    const int vch = ((tid & (CPR - 1)) ^ swz_v(lrow)) * 16;
    const int krow_b = (int)a.ks[2] * 2, vrow_b = (int)a.vs[2] * 2, rrow_b = (int)a.rs[1] * 2;
    const uint32_t sk_base = __builtin_amdgcn_readfirstlane(lds_addr(&sk[0][wave * 64]));
    const uint32_t sv_base = __builtin_amdgcn_readfirstlane(lds_addr(&sv[0][wave * 64]));
    const uint32_t sr_base = __builtin_amdgcn_readfirstlane(lds_addr(&sr[wave * 64]));
    auto load_kv = [&](int kt) {
        const int row = kt * BK + lrow;
        const uint32_t boff = (uint32_t)(kt & 1) * (TILE_CH * 16);
        load_lds16(krs, (uint32_t)(row * krow_b + kch), sk_base + boff);
        load_lds16(vrs, (uint32_t)(row * vrow_b + vch), sv_base + boff);
    };
    // ring quarter t % NQ holds r rows c_base + 64 t .. +63 (the swizzle only
    // depends on the row within the quarter)
    auto load_r_quarter = [&](int t) {
        const int row = c_base + 64 * t + lrow;
        load_lds16(rrs, (uint32_t)(row * rrow_b + kch), sr_base + (uint32_t)(t % NQ) * (TILE_CH * 16));
    };

    if (kt0 < kt1) {
        load_kv(kt0);
#pragma unroll
        for (int q = 0; q < NQ - 1; ++q) load_r_quarter(kt0 + q);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = kt0; kt < kt1; ++kt) {
        const int j0 = kt * BK;
        if (kt + 1 < kt1) {
            load_kv(kt + 1);
            load_r_quarter(kt + NQ - 1);
        }
        if (wq0 < L && j0 <= min(wq0 + 16 * RB - 1, L - 1) + M && j0 + BK - 1 >= wlo_first) {
            Tile t;
            t.sk = sk[kt & 1];
            t.sv = sv[kt & 1];
            t.sr = sr;
            t.skw = &sskew[wave][0];
            t.kt = kt;
            t.wband = wband;
            t.j0 = j0;
            t.wq0 = wq0;
            t.M = M;
            t.first = (kt == kt0);
            if (j0 + BK - 1 > wq0 + M || j0 < wlo_last) tile_body<true, LOWER>(st, t, g, n);
            else tile_body<false, LOWER>(st, t, g, n);
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
        __syncthreads();
    }

    // ---- epilogue: lane (g, n) holds query n, head columns 16 dt + 4 g + v
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int iq = wq0 + 16 * rb + n;
        if (iq >= L) continue;
        const float l = st.lsum[rb][0];
        if (a.nsplit == 1) {
            const float inv = 1.f / l;
            uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + b * a.os[0] + h * a.os[1] + (int64_t)iq * a.os[2];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x4 yb = __builtin_convertvector(st.o[rb][dt] * inv, bf16x4);
                *reinterpret_cast<u32x2 *>(op + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, yb);
            }
            if (a.lse && g == 0) a.lse[(int64_t)bh * L + iq] = (st.mref[rb] + __log2f(l)) * LN2;
        } else {
            float *po = a.part_o + (((int64_t)split * BH + bh) * L + iq) * DH;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(po + 16 * dt + 4 * g) = st.o[rb][dt];
            if (g == 0) {
                float *pm = a.part_ml + (((int64_t)split * BH + bh) * L + iq) * 2;
                pm[0] = (l > 0.f) ? st.mref[rb] : -INFINITY;   // no visible key in this split
                pm[1] = l;
            }
        }
    }
}

}  // namespace

int relattn_bf16_rows_per_block() { return BQ; }

bool relattn_bf16_supported(int dh) { return dh == DH; }

hipError_t launch_relattn_bf16(const RelAttnArgs &a, int dh, hipStream_t s)
{
    if (dh != DH) return hipErrorInvalidValue;
    const int blocks = a.nqb * a.B * a.H * a.nsplit;
    if (a.window > 0 || a.mem_valid)
        hipLaunchKernelGGL(relattn_fwd_bf16_kernel<true>, dim3(blocks), dim3(NW * 64), 0, s, a);
    else
        hipLaunchKernelGGL(relattn_fwd_bf16_kernel<false>, dim3(blocks), dim3(NW * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_relattn_combine(a, 1, dh, s);
}

}  // namespace txl
