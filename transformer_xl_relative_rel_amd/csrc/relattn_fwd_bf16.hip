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
// Work decomposition.  The queries of one (b, h) are cut into runs of 32
// (two 16-query blocks each) and the runs are paired from both ends: pair p
// is runs p and nr-1-p, so every pair covers the same number of (query, key)
// tiles.  A workgroup owns four pairs and is 8 waves: waves w and w + 4 share
// a SIMD and take the two runs of pair w, so every SIMD and every workgroup
// carries the same work.  A wave keeps its two blocks' state in registers and
// reads each K and V fragment from LDS once per key tile for both blocks.
// Keys are walked in tiles of 64.
//
// Everything is computed transposed (keys on MFMA rows, queries on lanes):
//   T^T = R_band . (c (q + vb))^T - m   with c = scale * log2(e) folded into
//       the query operand and the running row max m of each query folded into
//       the accumulator's initial value; 16 queries need 79 consecutive r rows
//       per 64-key tile: 5 band MFMA tiles.  Along a band row the key minus the
//       query is fixed, so the causal bound j <= i + M (and the same_length
//       window) is a threshold on the band row shared by the whole block: on
//       the few tiles that need it, masked band rows start at -inf.
//   the band value of (query n, band row cc) belongs to key jj = cc + n - 15: it
//   is written to a per-wave LDS row at column cc + n + 1 and read back in key
//   order as the initial accumulator of
//   S'^T = K . (c (q + u))^T + T^T      = log2-domain score minus row max;
//   p = exp2(S'); the running max is raised only when a score exceeds it by
//   more than 2^8 (rare branch; a query's first visible tile sets it exactly);
//   P comes out of the score MFMA in the B-operand layout of
//   O^T += V^T . P^T  with V^T fragments read from row-major V through the
//   transposing LDS read; the denominator is one more MFMA against ones.
// The two blocks of a wave are software-pipelined (the band MFMAs of block 1
// next to the softmax of block 0); the other wave on the SIMD fills the gaps.
//
// LDS: double-buffered K and V tiles, two rings of r rows (one per end of the
// paired query range; a tile needs three 64-row quarters of each, a fourth
// loads ahead), one skew buffer per wave.  Tiles move HBM -> LDS with
// direct-to-LDS loads issued one tile ahead.  K and r are stored
// fragment-major: the MFMA operand fragment of 16 rows x 32 columns is one
// contiguous 1 KB block in lane order, so a fragment read is a linear read of
// 1 KB (measured ~19 cycles per wave against ~51 for a row-major tile read
// through a bank-spreading swizzle; the direct loads pick each lane's 16
// bytes from HBM, so the layout costs nothing).  V keeps row-major rows of
// 16-byte chunks with an XOR swizzle for the transposing reads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "bf16_tiles.h"
#include "internal.h"

namespace txl {
namespace {

using namespace tiles;   // vector types, DH = 64, CPR, LN2, mfma, direct-to-LDS loads, buffer resources
constexpr int BK = 64;           // keys per tile
constexpr int NT = BK / 16;      // 16-key sub-tiles per tile
constexpr int NBT = NT + 1;      // band tiles per 16-query block
constexpr int RQ = 4;            // ring quarters: three in use plus one loading
// Work split of a workgroup: XW 16-query blocks per wave (one run of 16 XW
// queries), 16 / XW waves, runs paired from both ends of a head's query range
// (waves w and w + NW / 2 take the two runs of a pair and share a SIMD), so a
// workgroup covers 128 queries at each end whatever XW.
template <int XW> struct Split {
    static constexpr int NX = XW;            // 16-query blocks per wave
    static constexpr int NW = 16 / XW;       // waves per workgroup
    static constexpr int RUNQ = 16 * XW;     // queries per run
    static constexpr int PAIRS = NW / 2;     // run pairs per workgroup
    static constexpr int NRB = NT + XW;      // band tiles per run
    static constexpr int NTHR = NW * 64;
};
// Skew buffer: row n (query n) starts at float 80 n + 4 (n / 4); it is
// written at columns 1..95 and read at columns 16..79, and consecutive rows
// start at least 80 floats apart, so no row's writes reach another row's read
// range.  One-word LDS stores are serviced 32 lanes at a time over 32 banks;
// with these starts the 32 lanes of each half of a skew store (row n, column
// c + 4 g + n, g = lane / 16) hit 32 distinct banks (starts 80 n + 12 (n / 4)
// measured two extra cycles per store).  Row starts are multiples of 4, so the
// 16-byte skew loads are aligned.
__device__ __forceinline__ int skew_row(int n) { return 80 * n + 4 * (n >> 2); }
constexpr int SKEW = 80 * 15 + 4 * 3 + 96;   // floats per wave
constexpr int NKK = DH / 32;     // MFMA k-steps over dh
constexpr int NDT = DH / 16;     // 16-wide output tiles over dh
constexpr int TILE_CH = BK * CPR;              // chunks per K or V tile (and per ring quarter)
constexpr float TAU = 8.0f;      // deferred-rescale threshold (log2 units)
static_assert(Split<2>::RUNQ * (Split<2>::PAIRS - 1) + 16 * Split<2>::NRB <= 64 * (RQ - 1) &&
              Split<1>::RUNQ * (Split<1>::PAIRS - 1) + 16 * Split<1>::NRB <= 64 * (RQ - 1),
              "a ring must hold one tile's bands in RQ - 1 quarters");

// Fragment-major K and r tiles: block (m, kk) of a 64-row tile, 1 KB at byte
// 1024 (2 m + kk), holds rows 16 m .. 16 m + 15, columns 32 kk .. 32 kk + 31;
// lane (g, n) of the block (byte 16 (16 g + n)) holds row 16 m + n, columns
// 32 kk + 8 g .. + 7 -- the A operand layout of a 16x16x32 MFMA.
constexpr int FRAG = 1024;
// Byte offset, within its 16-row block's pair of fragments, of the 16-byte
// chunk that lane l of a direct load fetches when it fills fragment kk: row
// l % 16 of the block, columns 32 kk + 8 (l / 16) .. + 7.
__device__ __forceinline__ int frag_src(int l, int kk, int row_bytes)
{
    return (l & 15) * row_bytes + 64 * kk + 16 * (l >> 4);
}
// Swizzle of chunk c in a V row (transposing b64 reads of 4 rows x 32 bytes).
__device__ __forceinline__ int swz_v(int r) { return (r & 6) & (CPR - 1); }

__device__ __forceinline__ float row_max4(float x)
{
    // max over the four 16-lane groups that hold one query
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

template <int X> using IC = std::integral_constant<int, X>;

// Query fragments of one 16-query block: qu = c (q + u), qv = c (q + vb),
// added in fp32 and rounded once to bf16 (B operands: lane (g, n) holds query
// i0 + n, head columns 32 kk + 8 g .. + 7).  u and vb of the head are loaded
// once as 16-byte buffer loads (they do not depend on the query), so every
// load is issued up front; queries at or past L get zero fragments.
struct QBias {
    f32x4 u[2][2], w[2][2];   // [kk][half]: u and vb at columns 32 kk + 8 g + 4 half .. + 3
};

__device__ __forceinline__ QBias load_qbias(const float *u_h, const float *vb_h, int g)
{
    const __amdgpu_buffer_rsrc_t urs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(u_h), 0, 64 * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(vb_h), 0, 64 * 4, 0x00020000);
    QBias qb;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint32_t off = (uint32_t)(32 * kk + 8 * g + 4 * hf) * 4;
            qb.u[kk][hf] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(urs, off, 0, 0));
            qb.w[kk][hf] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
        }
    return qb;
}

__device__ __forceinline__ void query_frags(const uint16_t *qrow, bool ok, float c, const QBias &qb, int g,
                                            bf16x8 (&qu)[2], bf16x8 (&qv)[2])
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const u32x4 raw = *reinterpret_cast<const u32x4 *>(qrow + kk * 32 + 8 * g);
        f32x8 fu, fv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xv = __uint_as_float(((raw[e >> 1] >> (16 * (e & 1))) & 0xffffu) << 16);
            fu[e] = (xv + qb.u[kk][e >> 2][e & 3]) * c;
            fv[e] = (xv + qb.w[kk][e >> 2][e & 3]) * c;
        }
        const bf16x8 zero = {};
        qu[kk] = ok ? __builtin_convertvector(fu, bf16x8) : zero;
        qv[kk] = ok ? __builtin_convertvector(fv, bf16x8) : zero;
    }
}

// Per-wave state of the query blocks of the wave's run.
template <int NX> struct State {
    bf16x8 qu[NX][NKK], qv[NX][NKK];   // c (q + u), c (q + vb): B operands, lane (g, n) = query n
    f32x4 o[NX][NDT];                   // O^T accumulators (unnormalised)
    f32x4 lsum[NX];                     // softmax denominators (all 4 entries equal)
    float mneg[NX];                     // -m: initial accumulator value of the band MFMA
    float mref[NX];                     // running max (log2 units)
};

// Per-tile, wave-uniform description of one block.
struct Blk {
    int thi;    // band rows above thi are masked (causal bound)
    int tlo;    // band rows below tlo are masked (same_length window)
    int kmem;   // keys below kmem (tile-relative) are masked (per-row memory validity)
};

// Byte offsets of this lane's part of every LDS fragment access, fixed for the
// whole key loop: the tile, the 32-row half, the sub-tile and the ring slot add
// wave-uniform amounts (immediate offsets or one scalar base per buffer).
struct LaneOff {
    int k0;         // K and r fragments: 16 * lane (fragment-major blocks)
    int v0;         // V^T: rows 4 g + n / 4 (+ 16 for the upper half, + 32 per chunk) of column block 0
                    // (column block dt: v0 ^ 32 dt)
    int sst, sld;   // skew row: store at column 4 g + n + 1, load at column 16 + 4 g (floats)
};

__device__ __forceinline__ LaneOff lane_offsets(int g, int n)
{
    LaneOff o;
    // chunk (4 kk + g) ^ swz = (g ^ swz) ^ 4 kk: k-step kk flips bit 6 of the byte offset
    o.k0 = 16 * (16 * g + n);
    // chunk (2 dt + b) ^ swz = 2 (dt ^ swz / 2) + b (swz even): column block dt flips bits 5-6
    const int row0 = 4 * g + (n >> 2);
    o.v0 = (row0 * CPR + (((n >> 1) & 1) ^ swz_v(row0))) * 16 + 8 * (n & 1);
    o.sst = skew_row(n) + 4 * g + n + 1;
    o.sld = skew_row(n) + 16 + 4 * g;
    return o;
}

struct Tile {
    const u32x4 *sk, *sv, *sr;
    float *skw;         // this wave's skew buffer
    int kt;             // key tile index (selects the ring quarters)
    int offr;           // ring row offset of the run's band tile 0
    bool first;         // first tile of the key range
};

// The tile body is split in two halves: H1 (band MFMAs, skew round trip,
// content MFMAs) reads K and the r ring, H2 (softmax and P.V) reads V, so the
// throughput kernel can meet its per-tile barrier between them.
//
// LOWER: some query has a lower key bound (window or memory validity), so a
// query's first visible tile need not be the first tile of the range.
// MASKED: some key of the run is masked on this tile (band rows or key
// columns); otherwise every band row starts at -m.
template <bool LOWER, bool MASKED, int NX>
__device__ __forceinline__ void tile_h1(State<NX> &st, const Tile &t, const Blk (&bk)[NX], int g, const LaneOff &lo,
                                        f32x4 (&sc)[NX][NT])
{
    const int k0 = lo.k0;

    // K fragments (A operands of the content MFMA), shared by the two blocks
    bf16x8 kf[NT][NKK];
    {
        const TXL_LDS_AS char *kb = lds_bytes(t.sk);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                kf[tt][kk] = *(const TXL_LDS_AS bf16x8 *)(kb + k0 + (2 * tt + kk) * FRAG);
    }
    // r fragments of one run: run band tile u holds ring rows offr + 16 u + n.
    // A 16-row band tile never straddles a 64-row quarter (offr is a multiple
    // of 32), so its quarter slot is uniform across the wave.
    constexpr int NRB = NT + NX;   // band tiles of the run
    bf16x8 rf[NRB][NKK];
    {
        const TXL_LDS_AS char *srb = lds_bytes(t.sr);
        const int offr = t.offr;
#pragma unroll
        for (int u = 0; u < NRB; ++u) {
            const int x0 = offr + 16 * u;   // wave-uniform
            const int ubase = ((t.kt + (x0 >> 6)) & (RQ - 1)) * (TILE_CH * 16) + ((x0 >> 4) & 3) * (2 * FRAG);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) rf[u][kk] = *(const TXL_LDS_AS bf16x8 *)(srb + ubase + k0 + kk * FRAG);
        }
    }

    // band MFMA of block x (run band tiles NX-1-x .. NX+3-x: later queries need lower r rows)
    auto band = [&](auto X, f32x4 (&acc)[NBT]) {
        constexpr int x = decltype(X)::value;
        constexpr int h = NX - 1 - x;
        const bf16x8 *qv = st.qv[x];
        const float m = st.mneg[x];
        f32x4 cin[NBT];
        if constexpr (MASKED) {
            // band row 16 bt + 4 g + v is visible iff tlo <= row <= thi
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 16 * bt + 4 * g + v;
                    cin[bt][v] = (row > bk[x].thi || row < bk[x].tlo) ? -INFINITY : m;
                }
        } else {
            const f32x4 m4 = {m, m, m, m};
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) cin[bt] = m4;
        }
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) acc[bt] = mfma(rf[bt + h][0], qv[0], cin[bt]);
#pragma unroll
        for (int kk = 1; kk < NKK; ++kk)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) acc[bt] = mfma(rf[bt + h][kk], qv[kk], acc[bt]);
    };
    // skew of a block's band values into the wave's LDS rows
    auto skew_store = [&](const f32x4 (&acc)[NBT]) {
        float *skw = t.skw;
        lds_order();
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt)   // band row cc = 16 bt + 4 g + v of query n -> column cc + n + 1
            lds_store4(skw + lo.sst + 16 * bt, acc[bt]);
        lds_order();
    };
    // read back block x's skewed band values (keys on rows, in key order)
    auto skew_load = [&](auto X, f32x4 (&cin)[NT]) {
        constexpr int x = decltype(X)::value;
        const float *skw = t.skw;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            cin[tt] = *reinterpret_cast<const f32x4 *>(skw + lo.sld + 16 * tt);
        lds_order();
        if (LOWER && MASKED) {
            // keys below kmem are hidden from every query of the block
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (16 * tt + 4 * g + v < bk[x].kmem) cin[tt][v] = -INFINITY;
        }
    };
    // content MFMA of block x on top of the skewed band values
    auto content = [&](auto X, const f32x4 (&cin)[NT]) {
        constexpr int x = decltype(X)::value;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 acc = cin[tt];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) acc = mfma(kf[tt][kk], st.qu[x][kk], acc);
            sc[x][tt] = acc;
        }
    };

    // Both blocks' band MFMAs first, then the two skew round trips back to
    // back (one skew buffer per wave: LDS operations of a wave complete in
    // order, so block 1's stores land after block 0's loads have read), so
    // that their latencies overlap; then the content MFMAs.
    f32x4 acc0[NBT], acc1[NBT], cin0[NT], cin1[NT];
    band(IC<0>{}, acc0);
    if constexpr (NX > 1) band(IC<1>{}, acc1);
    skew_store(acc0);
    skew_load(IC<0>{}, cin0);
    if constexpr (NX > 1) {
        skew_store(acc1);
        skew_load(IC<1>{}, cin1);
    }
    content(IC<0>{}, cin0);
    if constexpr (NX > 1) content(IC<1>{}, cin1);
}

template <bool LOWER, int NX>
__device__ __forceinline__ void tile_h2(State<NX> &st, const Tile &t, const LaneOff &lo, f32x4 (&sc)[NX][NT])
{
    // column blocks 1-3 of V^T are formed per tile from the base offset
    int v0 = lo.v0;
    asm volatile("" : "+v"(v0));
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

    // V^T fragments (A operands of P.V), read through the transposing LDS read
    bf16x8 vf[NT / 2][NDT];
    auto load_v = [&]() {
        TXL_LDS_AS char *vb = (TXL_LDS_AS char *)(TXL_LDS_AS void *)t.sv;
#pragma unroll
        for (int ch = 0; ch < NT / 2; ++ch)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                // lane (g, n) gets V[32 ch + 4 g + e][16 dt + n] (lo) and the rows 16 below (hi);
                // the swizzle of rows 32 ch + r and 32 ch + r + 16 is that of row r
                TXL_LDS_AS char *p0 = vb + (v0 ^ (32 * dt)) + ch * 32 * CPR * 16;
                const i16x4 l = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)p0);
                const i16x4 hh = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)(p0 + 16 * CPR * 16));
                const u32x2 l2 = __builtin_bit_cast(u32x2, l), h2 = __builtin_bit_cast(u32x2, hh);
                vf[ch][dt] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
            }
    };

    bf16x8 pf[NX][NT / 2];
    // overflow check (rare rescale), probabilities as bf16 B fragments
    auto softmax = [&](auto X) {
        constexpr int x = decltype(X)::value;
        float mx = max3(sc[x][0][0], sc[x][0][1], sc[x][0][2]);
        mx = max3(mx, sc[x][0][3], sc[x][1][0]);
        mx = max3(mx, sc[x][1][1], sc[x][1][2]);
        mx = max3(mx, sc[x][1][3], sc[x][2][0]);
        mx = max3(mx, sc[x][2][1], sc[x][2][2]);
        mx = max3(mx, sc[x][2][3], sc[x][3][0]);
        mx = max3(mx, sc[x][3][1], sc[x][3][2]);
        mx = fmaxf(mx, sc[x][3][3]);
        // A query that has not seen a visible key yet takes the exact max of its
        // first visible tile; afterwards the max is only raised when a score
        // exceeds it by more than TAU.  Without lower key bounds that tile is
        // the first tile of the range; with them, a query is fresh while its
        // denominator is still empty.
        const bool fresh = LOWER ? st.lsum[x][0] == 0.f : t.first;
        if ((!LOWER && t.first) ||
            __builtin_amdgcn_ballot_w64(mx > TAU || (LOWER && fresh && mx != -INFINITY)) != 0) {
            const float rmx = row_max4(mx);
            float dlt;
            if (fresh) dlt = (rmx == -INFINITY) ? 0.f : rmx;   // exact max of the first visible tile
            else dlt = fmaxf(rmx, 0.f);                         // only ever raised
            st.mref[x] += dlt;
            st.mneg[x] -= dlt;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) sc[x][tt] -= dlt;
            const float alpha = fresh ? 1.f : __builtin_amdgcn_exp2f(-dlt);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) st.o[x][dt] *= alpha;
            st.lsum[x] *= alpha;
        }
#pragma unroll
        for (int ch = 0; ch < NT / 2; ++ch) {
            f32x8 p8;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                p8[v] = __builtin_amdgcn_exp2f(sc[x][2 * ch][v]);
                p8[4 + v] = __builtin_amdgcn_exp2f(sc[x][2 * ch + 1][v]);
            }
            pf[x][ch] = __builtin_convertvector(p8, bf16x8);
        }
    };
    // O^T += V^T . P^T, denominator += ones . P^T
    auto pv = [&](auto X) {
        constexpr int x = decltype(X)::value;
#pragma unroll
        for (int ch = 0; ch < NT / 2; ++ch) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) st.o[x][dt] = mfma(vf[ch][dt], pf[x][ch], st.o[x][dt]);
            st.lsum[x] = mfma(ones, pf[x][ch], st.lsum[x]);
        }
    };

    softmax(IC<0>{});
    load_v();
    pv(IC<0>{});
    if constexpr (NX > 1) {
        softmax(IC<1>{});
        pv(IC<1>{});
    }
}

template <bool LOWER, bool MASKED, int NX>
__device__ __forceinline__ void tile_body(State<NX> &st, const Tile &t, const Blk (&bk)[NX], int g, const LaneOff &lo)
{
    f32x4 sc[NX][NT];
    tile_h1<LOWER, MASKED, NX>(st, t, bk, g, lo, sc);
    tile_h2<LOWER, NX>(st, t, lo, sc);
}

// ---------------------------------------------------------------------------
// Memory update (Tail_M) carried by the attention launch.  The copy's 1 KB
// chunks, numbered ((b M_new + t) cpr + ch) for chunk ch of row t of batch
// row b of the new memory, are dealt to the launch's waves round-robin: wave
// w of W takes chunks w, w + W, ...  A wave walks its chunks as scalar
// coordinates (b, t, ch) advanced by the host's increments with carries, so
// the key loop needs no division.  A chunk lies in one row, so its source and
// destination rows are wave-uniform buffer resources and each lane moves 16
// bytes; lanes past the row end read zeros and their writes are dropped.
typedef const __attribute__((address_space(4))) FusedCopy KFusedCopy;

// The copy's arguments, read from the kernel argument segment (the launch's
// only argument is the RelAttnArgs) through a pointer the compiler cannot
// follow, so that every use reloads them with scalar loads instead of holding
// them in scalar registers across the key loop.
__device__ __forceinline__ KFusedCopy *fused_copy_args()
{
    KFusedCopy *c = (KFusedCopy *)((const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr() +
                                   offsetof(RelAttnArgs, cp));
    asm volatile("" : "+s"(c));
    return c;
}

struct CopyPos {
    int b, t, ch;      // batch row, row of the new memory, 1 KB chunk of the row
};

__device__ __forceinline__ CopyPos copy_first(KFusedCopy *c, int w)
{
    const int cpr = c->cpr, mn = c->M_new;
    const int row = w / cpr;
    return CopyPos{row / mn, row % mn, w % cpr};
}

__device__ __forceinline__ void copy_advance(KFusedCopy *c, CopyPos &p)
{
    p.ch += c->inc_ch;
    const int c1 = p.ch >= c->cpr;
    p.ch -= c1 ? c->cpr : 0;
    p.t += c->inc_t + c1;
    const int c2 = p.t >= c->M_new;
    p.t -= c2 ? c->M_new : 0;
    p.b += c->inc_b + c2;
}

// source and destination rows of chunk p (valid for p.b < B)
__device__ __forceinline__ void copy_rows(KFusedCopy *c, const CopyPos &p, __amdgpu_buffer_rsrc_t &src,
                                          __amdgpu_buffer_rsrc_t &dst)
{
    const int sr = c->beg + p.t;                  // row of [mem; h]
    const int rb = c->row_bytes;
    const unsigned char *s = sr < c->M_cur ? c->mem + p.b * c->mem_bs + (int64_t)sr * rb
                                           : c->h + p.b * c->h_bs + (int64_t)(sr - c->M_cur) * rb;
    src = make_rsrc(s, (uint32_t)rb);
    dst = make_rsrc(c->dst + p.b * c->new_bs + (int64_t)p.t * rb, (uint32_t)rb);
}

template <bool LOWER, int XW>
__global__ __launch_bounds__(Split<XW>::NTHR) void relattn_fwd_bf16_kernel(RelAttnArgs a)
{
    using S = Split<XW>;
    constexpr int NX = S::NX, NW = S::NW, RUNQ = S::RUNQ, PAIRS = S::PAIRS;
    __shared__ __attribute__((aligned(16))) u32x4 sk[2][TILE_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sv[3][TILE_CH];   // three: a wave's H2 may run past the barrier
    __shared__ __attribute__((aligned(16))) u32x4 sr[2][RQ * TILE_CH];
    __shared__ __attribute__((aligned(16))) float sskew[NW][SKEW];
    __shared__ __attribute__((aligned(16))) u32x4 scopy[NW][64];   // one staged Tail_M chunk per wave

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;

    // ---- which (pair group, b*h, key split) this workgroup owns
    const int BH = a.B * a.H;
    const int w = blockIdx.x;
    int slot = w, xg = 0, G = BH;
    if (a.remap) { xg = w & 7; slot = w >> 3; G = BH >> 3; }
    const int per = a.nsplit;
    const int grp = slot / (G * per);
    const int r2 = slot - grp * G * per;
    const int bh = a.remap ? xcd_pair(a, xg, r2 / per) : r2 / per;
    const int split = r2 % per;
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L, M = a.M, K = a.K;

    // runs of RUNQ queries, paired from both ends
    const int nr = (L + RUNQ - 1) / RUNQ;
    const int npair = (nr + 1) / 2;
    const int p0 = PAIRS * grp;
    const int np = min(PAIRS, npair - p0);
    // ring 0 holds the band rows of runs [p0, p0 + np), ring 1 those of runs
    // [nr - p0 - np, nr - p0); ring row 0 of quarter q is r row cb + 64 q where
    // cb belongs to the last (unclamped) query of the range and key 0.
    const int ihi0 = RUNQ * (p0 + np) - 1;
    const int ihi1 = RUNQ * (nr - p0) - 1;
    const int cb0 = L - 1 - ihi0, cb1 = L - 1 - ihi1;
    const int qmax = min(ihi1, L - 1);
    const int ntile = (qmax + M + 1 + BK - 1) / BK;
    int kt0 = split * a.tiles_per_split;
    if (LOWER) kt0 = max(kt0, key_lo(a, b, RUNQ * p0) / BK);
    const int kt1 = min(ntile, split * a.tiles_per_split + a.tiles_per_split);

    // this wave's run: waves w and w + PAIRS (one SIMD) take runs p and
    // nr - 1 - p of pair p = p0 + w % PAIRS (one run if they coincide)
    const int end = wave / PAIRS;
    const int p = p0 + wave % PAIRS;
    const int run = end == 0 ? p : nr - 1 - p;
    const bool run_ok = wave % PAIRS < np && (end == 0 || nr - 1 - p > p);
    int i0[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) i0[x] = RUNQ * run + 16 * x;

    const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + b * a.qs[0] + h * a.qs[1];
    const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + b * a.ks[0] + h * a.ks[1];
    const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.v) + b * a.vs[0] + h * a.vs[1];
    const uint16_t *rp = reinterpret_cast<const uint16_t *>(a.r) + h * a.rs[0];
    const float *up = a.u + h * DH;
    const float *wp = a.vb + h * DH;
    const float c = a.c;              // scale * log2(e)

    // per-row memory validity: keys below M - mem_valid[b] are hidden from every query
    int kmem_abs = 0;
    if (LOWER && a.mem_valid) {
        int mv = a.mem_valid[b];
        mv = mv < 0 ? 0 : (mv > M ? M : mv);
        kmem_abs = M - mv;
    }

    // ---- direct loads.  Each 8 KB tile (K, V, one r ring quarter) is eight
    // 1 KB blocks, one per loading wave: K and r fragment block w (16-row
    // block w / 2, k-step w % 2; see frag_src), V rows 8 w .. 8 w + 7 with the
    // chunk the V swizzle puts at each LDS position.  With eight waves every
    // wave loads a block of each; with sixteen, waves 0-7 load K and ring 0,
    // waves 8-15 V and ring 1.  Rows outside [0, K) read zeros.
    const int lw = wave & 7;                       // block this wave loads
    const int lrow = 8 * lw + (lane >> 3);         // V row of this lane's chunk
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)(((int64_t)(K - 1) * a.ks[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)(((int64_t)(K - 1) * a.vs[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rp, (uint32_t)(((int64_t)(K - 1) * a.rs[1] + DH) * 2));
    const int krow_b = (int)a.ks[2] * 2, vrow_b = (int)a.vs[2] * 2, rrow_b = (int)a.rs[1] * 2;
    const int fsrc_k = (16 * (lw >> 1)) * krow_b + frag_src(lane, lw & 1, krow_b);
    const int fsrc_r = (16 * (lw >> 1)) * rrow_b + frag_src(lane, lw & 1, rrow_b);
    const int vsrc = lrow * vrow_b + ((lane & (CPR - 1)) ^ swz_v(lrow)) * 16;
    const uint32_t sk_base = __builtin_amdgcn_readfirstlane(lds_addr(&sk[0][lw * 64]));
    const uint32_t sv_base = __builtin_amdgcn_readfirstlane(lds_addr(&sv[0][lw * 64]));
    const uint32_t sr0_base = __builtin_amdgcn_readfirstlane(lds_addr(&sr[0][lw * 64]));
    const uint32_t sr1_base = __builtin_amdgcn_readfirstlane(lds_addr(&sr[1][lw * 64]));
    const bool load_k = NW == 8 || wave < 8;      // K and ring 0
    const bool load_v = NW == 8 || wave >= 8;     // V and ring 1
    auto load_kv = [&](int kt) {
        if (load_k) load_lds16(krs, (uint32_t)(kt * BK * krow_b + fsrc_k), sk_base + (uint32_t)(kt & 1) * (TILE_CH * 16));
        if (load_v) load_lds16(vrs, (uint32_t)(kt * BK * vrow_b + vsrc), sv_base + (uint32_t)(kt % 3) * (TILE_CH * 16));
    };
    // ring quarter q % RQ holds r rows cb + 64 q .. +63
    auto load_r_quarter = [&](int q) {
        const uint32_t qoff = (uint32_t)(q & (RQ - 1)) * (TILE_CH * 16);
        if (load_k) load_lds16(rrs, (uint32_t)((cb0 + 64 * q) * rrow_b + fsrc_r), sr0_base + qoff);
        if (load_v) load_lds16(rrs, (uint32_t)((cb1 + 64 * q) * rrow_b + fsrc_r), sr1_base + qoff);
    };

    if (kt0 < kt1) {
        load_kv(kt0);
#pragma unroll
        for (int q = 0; q < RQ - 1; ++q) load_r_quarter(kt0 + q);
    }
    State<NX> st;
    // ---- query fragments: c (q + u) and c (q + vb), in fp32, rounded once to bf16
    // (their loads go out after the first tile's, so the two latencies overlap)
    const QBias qb = load_qbias(up, wp, g);
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int iq = i0[x] + n;
        const bool ok = run_ok && iq < L;
        const int iqc = ok ? iq : 0;
        query_frags(qp + (int64_t)iqc * a.qs[2], ok, c, qb, g, st.qu[x], st.qv[x]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) st.o[x][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.lsum[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.mneg[x] = 0.f;
        st.mref[x] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const LaneOff lo = lane_offsets(g, n);
    f32x4 sc[NX][NT];   // scores of the current tile, from H1 to H2
    Tile t;
    t.sr = sr[end];
    t.skw = sskew[wave];
    t.offr = (end == 0 ? ihi0 : ihi1) - (RUNQ * run + RUNQ - 1);

    // Tiles on which the run has a visible key: [ks, ke); within them, tiles on
    // which no key of the run is masked: [us, ue).  Within the run's range one
    // of its two blocks may see nothing; its band rows start at -inf.
    int ks, ke, us = 0, ue;
    {
        const int ifirst = RUNQ * run, ilast = min(ifirst + RUNQ - 1, L - 1);
        ks = LOWER ? max(kt0, key_lo(a, b, ifirst) / BK) : kt0;
        ke = min(kt1, (ilast + M) / BK + 1);
        if (!run_ok || ifirst >= L) ke = ks;
        // causal: every key of tile kt is visible to the run's first query iff
        // 64 kt + 63 <= ifirst + M (queries past L are discarded, unmasked)
        ue = (ifirst + M + 1) / BK;
        if (LOWER) {
            // window: band rows below tlo of the run's second block; memory validity: keys below kmem_abs
            if (a.window > 0) us = max(us, (ifirst + 16 + M + 15 - a.window + BK) / BK);
            us = max(us, (kmem_abs + BK - 1) / BK);
        }
    }

    // Tail_M chunks of this wave: inside the key loop one every cstride tiles
    // (the copy steps, staggered over the workgroup's waves so that the copy's
    // traffic is spread over the loop), staged in LDS by a direct load after
    // the barrier of a copy step and written out after the next tile's wait
    // and barrier, so the copy holds no vector registers across the tile body;
    // the rest after the loop.  pos is the staged chunk while one is staged,
    // else the next to load.
    CopyPos pos{0x7fffffff, 0, 0};    // past the last batch row: no copy
    if (fused_copy_args()->nchunks > 0) pos = copy_first(fused_copy_args(), (int)blockIdx.x * NW + wave);
    bool staged = false;
    const uint32_t scopy_base = __builtin_amdgcn_readfirstlane(lds_addr(&scopy[wave][0]));
    auto lane16 = [&]() {
        uint32_t l = 16u * (uint32_t)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        asm volatile("" : "+v"(l));
        return l;
    };
    // tiles until this wave's next copy step; without a copy the countdown
    // never reaches zero inside the key loop
    int cstride = 1, ccount = 0x7fffffff;
    {
        KFusedCopy *c = fused_copy_args();
        if (c->nchunks > 0) {
            const int waves = (int)gridDim.x * NW;
            const int cpw = (c->nchunks + waves - 1) / waves;     // chunks per wave
            cstride = max(1, (kt1 - kt0) / (cpw + 1));
            ccount = wave % cstride;
        }
    }
    auto copy_out = [&]() {
        if (staged) {
            KFusedCopy *c = fused_copy_args();
            __amdgpu_buffer_rsrc_t src, dst;
            copy_rows(c, pos, src, dst);
            const uint32_t l16 = lane16();
            const u32x4 val = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(&scopy[wave][0]) + l16);
            __builtin_amdgcn_raw_buffer_store_b128(val, dst, 1024u * pos.ch + l16, 0, 0);
            copy_advance(c, pos);
            staged = false;
        }
    };

    // One key tile: stage the next tile, compute H1 of this one, wait for the
    // staged loads and meet the workgroup, then H2.  A wave's H2 of tile kt
    // runs while other waves start tile kt + 1 and its loads land: K and the
    // r ring are only read in H1, V has three buffers (tile kt + 2 loads into
    // the one tile kt - 1 used).  Taking the barrier between the halves
    // measured faster (37.0 us at B8 H16 L512 M512) than after them (38.4 us)
    // or than half of the waves taking it at each point (39.5 us).
    auto step = [&](auto ACT, auto MC, int kt) {
        constexpr bool ACTIVE = decltype(ACT)::value != 0;
        constexpr bool MASKED = decltype(MC)::value != 0;
        const int j0 = kt * BK;
        if (kt + 1 < kt1) {
            load_kv(kt + 1);
            load_r_quarter(kt + RQ - 1);
        }
        if constexpr (ACTIVE) {
            Blk bk[NX];
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                // band row cc of query n is key j0 + cc + n - 15: visible iff cc <= M + i0 - j0 + 15
                bk[x].thi = i0[x] < L ? M + i0[x] - j0 + 15 : -1;   // ragged tail: nothing visible
                bk[x].tlo = (LOWER && a.window > 0) ? i0[x] + M + 1 - a.window - j0 + 15 : -1;
                bk[x].kmem = kmem_abs - j0;
            }
            t.sk = sk[kt & 1];
            t.sv = sv[kt % 3];
            t.kt = kt;
            t.first = (kt == kt0);
            tile_h1<LOWER, MASKED, NX>(st, t, bk, g, lo, sc);
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
        __syncthreads();
        // The chunk staged in the previous copy step has landed: write it out
        // and stage the next one, whose load then has this H2 and the next H1
        // to land before the wait.
        copy_out();
        if (ccount-- == 0) {       // a copy step of this wave
            ccount = cstride - 1;
            if (pos.b < fused_copy_args()->B) {
                __amdgpu_buffer_rsrc_t src, dst;
                copy_rows(fused_copy_args(), pos, src, dst);
                load_lds16(src, 1024u * pos.ch + lane16(), scopy_base);
                staged = true;
            }
        }
        if constexpr (ACTIVE) tile_h2<LOWER, NX>(st, t, lo, sc);
    };
    // Walk the tiles in segments of one kind (active, masks needed) so that
    // each loop runs one instance of the tile body and the state stays in place.
    for (int kt = kt0; kt < kt1;) {
        const bool act = kt >= ks && kt < ke;
        const bool mk = kt < us || kt >= ue;
        int e = kt1;
        if (ks > kt) e = min(e, ks);
        if (ke > kt) e = min(e, ke);
        if (us > kt) e = min(e, us);
        if (ue > kt) e = min(e, ue);
        if (act) {
            if (mk) for (; kt < e; ++kt) step(IC<1>{}, IC<1>{}, kt);
            else for (; kt < e; ++kt) step(IC<1>{}, IC<0>{}, kt);
        } else {
            for (; kt < e; ++kt) step(IC<0>{}, IC<0>{}, kt);
        }
    }

    __builtin_amdgcn_s_waitcnt(0);   // the last staged chunk has landed
    copy_out();
    if (fused_copy_args()->nchunks > 0) {
        for (; pos.b < fused_copy_args()->B; copy_advance(fused_copy_args(), pos)) {
            __amdgpu_buffer_rsrc_t src, dst;
            copy_rows(fused_copy_args(), pos, src, dst);
            const uint32_t l16 = lane16();
            const u32x4 val = __builtin_amdgcn_raw_buffer_load_b128(src, 1024u * pos.ch + l16, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(val, dst, 1024u * pos.ch + l16, 0, 0);
        }
    }

    // ---- epilogue: lane (g, n) holds query n, head columns 16 dt + 4 g + v.
    // Lane ids made opaque here so that the epilogue's addresses are formed
    // after the key loop instead of being held (and spilled) across it.
    int ge = g, ne = n;
    asm volatile("" : "+v"(ge), "+v"(ne));
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int iq = i0[x] + ne;
        if (!run_ok || iq >= L) continue;
        const float l = st.lsum[x][0];
        if (a.nsplit == 1) {
            const float inv = 1.f / l;
            uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + b * a.os[0] + h * a.os[1] + (int64_t)iq * a.os[2];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x4 yb = __builtin_convertvector(st.o[x][dt] * inv, bf16x4);
                *reinterpret_cast<u32x2 *>(op + 16 * dt + 4 * ge) = __builtin_bit_cast(u32x2, yb);
            }
            if (a.lse && ge == 0) a.lse[(int64_t)bh * L + iq] = (st.mref[x] + __log2f(l)) * LN2;
        } else {
            // lane layout: group (dt, lane) of the query's 16-query block, 1 KB per store instruction
            float *po = a.part_o + (((int64_t)split * BH + bh) * ((L + 15) >> 4) + (i0[x] >> 4)) * (NDT * 64 * 4);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(po + (64 * dt + 16 * ge + ne) * 4) = st.o[x][dt];
            if (ge == 0) {
                float *pm = a.part_ml + (((int64_t)split * BH + bh) * L + iq) * 2;
                pm[0] = (l > 0.f) ? st.mref[x] : -INFINITY;   // no visible key in this split
                pm[1] = l;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming path: short segments against a long memory (L <= 128, so at most
// four 32-query runs per head, and many keys).  One workgroup per (b, h, key
// split) with one wave per run, one wave per SIMD; the waves share the split's
// K and V tiles and one ring of r rows in LDS, moved by direct-to-LDS loads
// of whole 128-byte rows one tile ahead, so the workgroup fetches each byte of
// its keys once (a wave that loaded its own K and r fragments straight into
// registers touched 16 rows per 1 KB load and four waves fetched the same
// tile).  The tile body is the throughput kernel's; the key splits of a head
// are merged by the split combine.
// Work split of the streaming kernel: STREAM_XW 16-query blocks per wave, one
// wave per run of 16 STREAM_XW queries, so at most SNW waves for L <= 128.
constexpr int STREAM_XW = 2;
constexpr int SNW = 128 / Split<STREAM_XW>::RUNQ;   // waves per streaming workgroup at most

__global__ __launch_bounds__(SNW * 64) void relattn_stream_bf16_kernel(RelAttnArgs a)
{
    constexpr int NX = Split<STREAM_XW>::NX, RUNQ = Split<STREAM_XW>::RUNQ;
    __shared__ __attribute__((aligned(16))) u32x4 sk[2][TILE_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sv[2][TILE_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sr[RQ * TILE_CH];
    __shared__ __attribute__((aligned(16))) float sskew[SNW][SKEW];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int nw = a.nqb;   // waves of the workgroup = runs of the head
    const int BH = a.B * a.H;
    // XCD-aware order: every key split of a head runs on one XCD (workgroup w
    // runs on XCD w % 8), so the head's K, V and r rows are fetched into one L2
    const int w = blockIdx.x;
    int bh, split;
    if (a.remap) {
        const int j = w >> 3;
        bh = xcd_pair(a, w & 7, j / a.nsplit);
        split = j % a.nsplit;
    } else {
        bh = w / a.nsplit;
        split = w - bh * a.nsplit;
    }
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L, M = a.M, K = a.K;
    const int run = wave;
    const int ifirst = RUNQ * run, ilast = min(ifirst + RUNQ - 1, L - 1);
    const int ntile = (L - 1 + M) / BK + 1;   // tiles up to the last query's bound
    const int kt0 = split * a.tiles_per_split;
    const int kt1 = min(ntile, kt0 + a.tiles_per_split);
    int i0[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) i0[x] = ifirst + 16 * x;

    const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + b * a.qs[0] + h * a.qs[1];
    const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + b * a.ks[0] + h * a.ks[1];
    const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.v) + b * a.vs[0] + h * a.vs[1];
    const uint16_t *rp = reinterpret_cast<const uint16_t *>(a.r) + h * a.rs[0];
    const float *up = a.u + h * DH;
    const float *wp = a.vb + h * DH;

    // ---- direct loads: wave w moves the 1 KB blocks w, w + nw, ... of each
    // 8 KB tile (block blk holds rows 8 blk .. 8 blk + 7, lane l row l / 8),
    // reading the chunk the XOR swizzle puts at that LDS position; the K and r
    // swizzle of row 8 blk + l / 8 only depends on the parity of blk.  Rows
    // outside [0, K) read zeros.
    const int lr = lane >> 3;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)(((int64_t)(K - 1) * a.ks[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vp, (uint32_t)(((int64_t)(K - 1) * a.vs[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rp, (uint32_t)(((int64_t)(K - 1) * a.rs[1] + DH) * 2));
    const int vch = ((lane & (CPR - 1)) ^ swz_v(lr)) * 16;
    const int krow_b = (int)a.ks[2] * 2, vrow_b = (int)a.vs[2] * 2, rrow_b = (int)a.rs[1] * 2;
    const uint32_t sk_base = __builtin_amdgcn_readfirstlane(lds_addr(&sk[0][0]));
    const uint32_t sv_base = __builtin_amdgcn_readfirstlane(lds_addr(&sv[0][0]));
    const uint32_t sr_base = __builtin_amdgcn_readfirstlane(lds_addr(&sr[0]));
    // ring quarter q % RQ holds r rows cb + 64 q .. + 63, where cb belongs to
    // the last (unclamped) query of the workgroup's runs and key 0
    const int cb = L - RUNQ * nw;
    auto load_kv = [&](int kt) {
        const uint32_t boff = (uint32_t)(kt & 1) * (TILE_CH * 16);
        for (int blk = wave; blk < TILE_CH / 64; blk += nw) {
            const int row = kt * BK + 8 * blk + lr;
            const uint32_t loff = boff + (uint32_t)blk * 1024u;
            // K: fragment block blk (16-row block blk / 2, k-step blk % 2); V: rows 8 blk .. + 7
            const int ksrc = (kt * BK + 16 * (blk >> 1)) * krow_b + frag_src(lane, blk & 1, krow_b);
            load_lds16(krs, (uint32_t)ksrc, sk_base + loff);
            load_lds16(vrs, (uint32_t)(row * vrow_b + vch), sv_base + loff);
        }
    };
    auto load_r_quarter = [&](int q) {
        const uint32_t qoff = (uint32_t)(q & (RQ - 1)) * (TILE_CH * 16);
        for (int blk = wave; blk < TILE_CH / 64; blk += nw) {
            const int rsrc = (cb + 64 * q + 16 * (blk >> 1)) * rrow_b + frag_src(lane, blk & 1, rrow_b);
            load_lds16(rrs, (uint32_t)rsrc, sr_base + qoff + (uint32_t)blk * 1024u);
        }
    };
    // the first tile's loads go out before the query fragments' (they do not
    // depend on them), so the two memory latencies overlap
    if (kt0 < kt1) {
        load_kv(kt0);
#pragma unroll
        for (int q = 0; q < RQ - 1; ++q) load_r_quarter(kt0 + q);
    }

    State<NX> st;
    const QBias qb = load_qbias(up, wp, g);
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int iq = i0[x] + n;
        const bool ok = iq < L;
        const int iqc = ok ? iq : 0;
        query_frags(qp + (int64_t)iqc * a.qs[2], ok, a.c, qb, g, st.qu[x], st.qv[x]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) st.o[x][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.lsum[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.mneg[x] = 0.f;
        st.mref[x] = 0.f;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const LaneOff lo = lane_offsets(g, n);
    Tile t;
    t.sr = sr;
    t.skw = sskew[wave];
    t.offr = RUNQ * (nw - 1 - run);   // ring row of the run's band tile 0
    // the run sees keys on tiles [kt0, ke); no key of the run is masked below ue
    const int ke = min(kt1, (ilast + M) / BK + 1);
    const int ue = (ifirst + M + 1) / BK;
    for (int kt = kt0; kt < kt1; ++kt) {
        if (kt + 1 < kt1) {
            load_kv(kt + 1);
            load_r_quarter(kt + RQ - 1);
        }
        if (kt < ke) {
            const int j0 = kt * BK;
            Blk bk[NX];
#pragma unroll
            for (int x = 0; x < NX; ++x) {
                // band row cc of query n is key j0 + cc + n - 15: visible iff cc <= M + i0 - j0 + 15
                bk[x].thi = i0[x] < L ? M + i0[x] - j0 + 15 : -1;   // ragged tail: nothing visible
                bk[x].tlo = -1;
                bk[x].kmem = 0;
            }
            t.sk = sk[kt & 1];
            t.sv = sv[kt & 1];
            t.kt = kt;
            t.first = (kt == kt0);
            if (kt >= ue) tile_body<false, true, NX>(st, t, bk, g, lo);
            else tile_body<false, false, NX>(st, t, bk, g, lo);
        }
        __builtin_amdgcn_s_waitcnt(0);   // this wave's direct loads have landed
        __syncthreads();
    }

    // ---- epilogue: lane (g, n) holds query n, head columns 16 dt + 4 g + v
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int iq = i0[x] + n;
        if (iq >= L) continue;
        const float l = st.lsum[x][0];
        if (a.nsplit == 1) {
            const float inv = 1.f / l;
            uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + b * a.os[0] + h * a.os[1] + (int64_t)iq * a.os[2];
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x4 yb = __builtin_convertvector(st.o[x][dt] * inv, bf16x4);
                *reinterpret_cast<u32x2 *>(op + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, yb);
            }
            if (a.lse && g == 0) a.lse[(int64_t)bh * L + iq] = (st.mref[x] + __log2f(l)) * LN2;
        } else {
            // a split in which the query sees no key leaves o = 0, l = 0 and writes m = -inf;
            // lane layout: group (dt, lane) of the query's 16-query block, 1 KB per store instruction
            float *po = a.part_o + (((int64_t)split * BH + bh) * ((L + 15) >> 4) + (i0[x] >> 4)) * (NDT * 64 * 4);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(po + (64 * dt + 16 * g + n) * 4) = st.o[x][dt];
            if (g == 0) {
                float *pm = a.part_ml + (((int64_t)split * BH + bh) * L + iq) * 2;
                pm[0] = (l > 0.f) ? st.mref[x] : -INFINITY;
                pm[1] = l;
            }
        }
    }
}

}  // namespace

// Work split of the throughput kernel (16-query blocks per wave).
constexpr int FWD_XW = 2;

int relattn_bf16_groups_per_head(int L)
{
    using S = Split<FWD_XW>;
    const int nr = (L + S::RUNQ - 1) / S::RUNQ;
    const int npair = (nr + 1) / 2;
    return (npair + S::PAIRS - 1) / S::PAIRS;
}

bool relattn_bf16_supported(int dh) { return dh == DH; }

int relattn_bf16_stream_runs(int L) { return (L + Split<STREAM_XW>::RUNQ - 1) / Split<STREAM_XW>::RUNQ; }

hipError_t launch_relattn_bf16_stream(const RelAttnArgs &a, int dh, hipStream_t s)
{
    if (dh != DH || a.window > 0 || a.mem_valid || a.nqb < 1 || a.nqb > SNW) return hipErrorInvalidValue;
    const int blocks = a.B * a.H * a.nsplit;   // one workgroup per (b, h, key split), one wave per run
    hipLaunchKernelGGL(relattn_stream_bf16_kernel, dim3(blocks), dim3(64 * a.nqb), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_relattn_combine(a, 1, dh, s);
}

hipError_t launch_relattn_bf16(const RelAttnArgs &args, int dh, hipStream_t s)
{
    if (dh != DH) return hipErrorInvalidValue;
    using S = Split<FWD_XW>;
    const int blocks = args.nqb * args.B * args.H * args.nsplit;
    RelAttnArgs a = args;
    if (a.cp.nchunks > 0) {
        // a wave's next chunk is the launch's wave count further on
        const int64_t waves = (int64_t)blocks * S::NW, cpb = (int64_t)a.cp.M_new * a.cp.cpr;
        const int64_t rem = waves % cpb;
        a.cp.inc_b = (int)std::min<int64_t>(waves / cpb, a.cp.B);
        a.cp.inc_t = (int)(rem / a.cp.cpr);
        a.cp.inc_ch = (int)(rem % a.cp.cpr);
    }
    if (a.window > 0 || a.mem_valid)
        hipLaunchKernelGGL((relattn_fwd_bf16_kernel<true, FWD_XW>), dim3(blocks), dim3(S::NTHR), 0, s, a);
    else
        hipLaunchKernelGGL((relattn_fwd_bf16_kernel<false, FWD_XW>), dim3(blocks), dim3(S::NTHR), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_relattn_combine(a, 1, dh, s);
}

}  // namespace txl
