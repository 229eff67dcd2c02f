// Relative-position attention, backward: bf16 in, fp32 accumulate, dh = 64,
// for gfx950.
//
// The forward ([SRC] "Transformer-XL模型 核心源码阅读笔记",
// RelPartialLearnableMultiHeadAttn.forward; [XL] "Transformer-XL" textbook
// notes, "Relative Positional Encoding" and "Causal Mask With Memory") is
//   s_ij = scale ((q_i + u) . k_j + (q_i + vb) . r[L-1-i+j]),
//   visible iff lo(b, i) <= j <= i + M,   out_i = softmax_j(s_ij) . v_j.
// The pages fix no backward; the gradients below are the chain rule on it
// ([XL] "Why Stop Gradient" only detaches the memory states of a layer
// stack: the attention still returns dk, dv for the memory keys, which a
// layer needs for its projection weights).  With dP_ij = dout_i . v_j,
// D_i = dout_i . out_i = sum_j p_ij dP_ij and dS_ij = p_ij (dP_ij - D_i):
//   dq_i = scale sum_j dS_ij (k_j + r[L-1-i+j])
//   dk_j = scale sum_i dS_ij (q_i + u),   dv_j = sum_i p_ij dout_i
//   dr_c = scale sum over b and (i, j) with L-1-i+j = c of dS_ij (q_i + vb)
//   du = sum over b, i of the k part of dq_i, dvb = the same of its r part.
//
// Kernels (one stream, in the order prep, dkv, dq, dr):
//   prep : c (q + u) and c (q + vb) rounded to bf16 exactly as the forward
//          forms its query operands (c = scale log2 e), D_i, lse in log2 units.
//   dkv  : one workgroup per 128 keys (4 waves of 32 keys), queries in steps
//          of 32, untransposed (queries on MFMA rows, keys on lanes).  The band
//          T = c (q + vb) . R^T of the step's 32 queries and the 160 r rows
//          they need (a ring of r rows in LDS, loaded a step ahead with the
//          query tiles) is shared by the workgroup through LDS; each wave reads
//          its skewed part, recomputes p and dS and accumulates
//          dv^T += dout^T . P and dk^T += (c (q + u))^T . dS (operands of
//          the step's query tiles through the transposing LDS read; P and dS
//          pass from the score MFMA's result layout to the operand layout
//          without data movement).  It also stores dS of the visible pairs as
//          G[i][L-1-i+j] (bf16) to the workspace.
//   dq   : one wave per 16 queries, 8 waves per workgroup, keys in tiles of
//          64, transposed (head columns on MFMA rows, queries on lanes).  The
//          wave's G window of a tile (16 rows x 88 columns) is staged in LDS
//          with direct loads into one buffer per wave, refilled for the next
//          tile once the wave has read it; dq^T += K^T . dS^T reads dS at key positions
//          (row i shifted by L-1-i: aligned words and a byte shift), and
//          dq^T += R_band^T . G^T reads the same rows at band positions.  Per
//          16-query sums of both parts go to the workspace for du and dvb.
//   dr   : dr[h] = sum_b G_b^T . c (q + vb)_b (one workgroup per 64 rows of r);
//          the head's first two workgroups then sum du and dvb from the
//          per-block sums in a fixed order.
// No atomics: every output element has one writer and a fixed summation
// order, so results are bitwise reproducible.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "bf16_tiles.h"
#include "internal.h"

namespace txl {
namespace {

using namespace tiles;

constexpr int BK = 64;           // keys per tile
constexpr int NT = BK / 16;      // 16-key sub-tiles per tile
constexpr int NBT = NT + 1;      // band tiles per 16-query block (79 rows)
constexpr int NKK = DH / 32;     // MFMA k-steps over dh
constexpr int NDT = DH / 16;     // 16-wide output tiles over dh
constexpr int TILE_CH = BK * CPR;
constexpr int BLK16B = 16 * CPR * 16;   // bytes of 16 tile rows



typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
template <bool B> struct BoolC { static constexpr bool value = B; };   // compile-time flag for generic lambdas
__device__ __forceinline__ float bf16_val(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Sums over groups of lanes by DPP moves on the VALU (no LDS traffic): swaps
// within quads (lane distance 1, then 2), the half-row mirror (pairs the two
// quads of each 8 lanes) and the row mirror (pairs the two halves of each 16).
// Every lane adds the same two partial sums as an xor butterfly would, so the
// results are the butterfly's bit for bit.
template <int CTRL> __device__ __forceinline__ float dpp_add(float x)
{
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum8(float x)      // lanes 8k .. 8k + 7
{
    x = dpp_add<0xb1>(x);       // quad_perm [1, 0, 3, 2]
    x = dpp_add<0x4e>(x);       // quad_perm [2, 3, 0, 1]
    return dpp_add<0x141>(x);   // row_half_mirror
}
__device__ __forceinline__ float sum16(float x)     // lanes 16k .. 16k + 15
{
    return dpp_add<0x140>(sum8(x));   // row_mirror
}

// ---------------------------------------------------------------------------
// prep: PREP_RPT groups of 32 rows per 256-thread workgroup, 8 threads (16 bytes
// each) per row; a thread issues the loads of all its rows before any arithmetic.

constexpr int PREP_RPT = 2;
constexpr int PREP_ROWS = 32 * PREP_RPT;

__global__ __launch_bounds__(256) void bwd_prep_kernel(RelAttnBwdArgs a)
{
    const int t = threadIdx.x;
    const int part = t & 7;
    const int64_t nrows = (int64_t)a.B * a.H * a.L;
    int64_t rr[PREP_RPT];
    bool ok[PREP_RPT];
    u32x4 raw[PREP_RPT], o[PREP_RPT], d[PREP_RPT];
    f32x4 u0[PREP_RPT], u1[PREP_RPT], w0[PREP_RPT], w1[PREP_RPT];
    float lse[PREP_RPT];
#pragma unroll
    for (int k = 0; k < PREP_RPT; ++k) {
        const int64_t row = (int64_t)blockIdx.x * PREP_ROWS + 32 * k + (t >> 3);
        ok[k] = row < nrows;
        rr[k] = ok[k] ? row : 0;
        const int bh = (int)(rr[k] / a.L), i = (int)(rr[k] - (int64_t)bh * a.L);
        const int b = bh / a.H, h = bh - b * a.H;
        // every load first, so that a thread waits for one memory round trip
        // (stores to qu and qv may alias out or dout as far as the compiler
        // knows, so it would not move those loads above them); rows past the
        // end read row 0 and store nothing
        const uint16_t *qp = static_cast<const uint16_t *>(a.q) + b * a.qs[0] + h * a.qs[1] + (int64_t)i * a.qs[2];
        const int64_t ooff = b * a.os[0] + h * a.os[1] + (int64_t)i * a.os[2] + 8 * part;
        raw[k] = *reinterpret_cast<const u32x4 *>(qp + 8 * part);
        o[k] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.out) + ooff);
        d[k] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.dout) + ooff);
        const f32x4 *up = reinterpret_cast<const f32x4 *>(a.u + h * DH + 8 * part);
        const f32x4 *wp = reinterpret_cast<const f32x4 *>(a.vb + h * DH + 8 * part);
        u0[k] = up[0]; u1[k] = up[1]; w0[k] = wp[0]; w1[k] = wp[1];
        lse[k] = a.lse[rr[k]];
    }
    __builtin_amdgcn_sched_barrier(0);   // no arithmetic (and so no wait) between the loads
#pragma unroll
    for (int k = 0; k < PREP_RPT; ++k) {
        f32x8 fu, fv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = bf16_val((raw[k][e >> 1] >> (16 * (e & 1))) & 0xffffu);
            fu[e] = (x + (e < 4 ? u0[k][e & 3] : u1[k][e & 3])) * a.c;     // same operation order as the forward's query operands
            fv[e] = (x + (e < 4 ? w0[k][e & 3] : w1[k][e & 3])) * a.c;
        }
        float dsum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            dsum += bf16_val((o[k][e >> 1] >> (16 * (e & 1))) & 0xffffu) * bf16_val((d[k][e >> 1] >> (16 * (e & 1))) & 0xffffu);
        if (ok[k]) {
            *reinterpret_cast<bf16x8 *>(a.qu + rr[k] * DH + 8 * part) = __builtin_convertvector(fu, bf16x8);
            *reinterpret_cast<bf16x8 *>(a.qv + rr[k] * DH + 8 * part) = __builtin_convertvector(fv, bf16x8);
        }
        dsum = sum8(dsum);
        if (ok[k] && part == 0) {
            a.dd[rr[k]] = dsum;
            a.lse2[rr[k]] = lse[k] * LOG2E;
        }
    }
}

// ---------------------------------------------------------------------------
// dq (and the bias partial sums) from the score gradients G that dkv stored

constexpr int QW = 8;               // waves per workgroup
constexpr int QROWS = 16 * QW;      // queries per workgroup
constexpr int QTHR = 64 * QW;
constexpr int QLPT = TILE_CH / QTHR;   // 16-byte loads per thread per tile
constexpr int RQ = 4;               // r ring quarters: three in use, one loading
static_assert(QLPT * QTHR == TILE_CH, "whole tiles per load round");
static_assert(QROWS - 16 + 16 * NBT <= 64 * (RQ - 1), "a tile's bands fit in three ring quarters");

// G staging: the G window of one wave and one key tile is 16 rows x GCOL
// columns starting at an 8-aligned column; row n at 16-byte chunk GRC n.  One
// buffer per wave: a tile reads its whole window first, and the next tile's
// window is loaded into the buffer after those reads have completed.
constexpr int GCOL = 88;            // band rows 0..79 plus up to 7 columns of alignment slack
constexpr int GRC = GCOL / 8;       // 16-byte chunks per staged row
constexpr int GLD = (16 * GRC + 63) / 64;   // staging loads per lane
constexpr int GBUF = GLD * 1024;    // bytes per wave

// s_waitcnt immediate that waits for every LDS operation of the wave and for
// no vector-memory or export operation
constexpr int WAIT_LGKM_ONLY = 0xF | (7 << 4) | (0 << 8) | (3 << 14);

// keep mask of one word (two bf16): element e0 and e0 + 1 kept iff their key lies in [lo, hi]
__device__ __forceinline__ uint32_t keep2(int j, int lo, int hi)
{
    return ((j >= lo && j <= hi) ? 0x0000ffffu : 0u) | ((j + 1 >= lo && j + 1 <= hi) ? 0xffff0000u : 0u);
}
// Four consecutive bf16 of a staged row starting at element e (e >= 0): three
// aligned words, shifted by one element when e is odd.
__device__ __forceinline__ u32x2 gquad(const TXL_LDS_AS char *row, int e)
{
    const TXL_LDS_AS uint32_t *w = (const TXL_LDS_AS uint32_t *)(row + (e >> 1) * 4);
    const uint32_t sh = (uint32_t)(e & 1) * 2;
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    return u32x2{__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh)};
}

// 72 KB of LDS: two workgroups (16 waves) per CU, at most 128 registers per wave.
__global__ __launch_bounds__(QTHR) __attribute__((amdgpu_waves_per_eu(4))) void bwd_dq_kernel(RelAttnBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) u32x4 sk[2][TILE_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sr[RQ][TILE_CH];
    __shared__ __attribute__((aligned(16))) char sgw[QW][GBUF];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int BH = a.B * a.H, L = a.L, M = a.M, K = a.K;
    const int nqb = (L + QROWS - 1) / QROWS;
    const int split = blockIdx.x % a.nsplit;
    const int wg = blockIdx.x / a.nsplit;
    const int qblk = nqb - 1 - wg / BH;            // the longest query blocks first
    const int bh = wg - (wg / BH) * BH;
    const int b = bh / a.H, h = bh - b * a.H;
    const int i0 = QROWS * qblk;
    const int i0w = i0 + 16 * wave;
    const int iq = i0w + n;
    const bool qok = iq < L;
    // key tiles [kt0, kt1) of this split; the wave's own queries see tiles below ntile_w
    const int kt0 = split * a.tps;
    const int kt1 = min((min(i0 + QROWS - 1, L - 1) + M) / BK + 1, kt0 + a.tps);
    const int ntile_w = i0w < L ? (min(i0w + 15, L - 1) + M) / BK + 1 : 0;
    const int ntg = min(ntile_w, kt1);              // the wave computes tiles [kt0, ntg)

    // keys j with kmem <= j <= iq + M have a stored dS (dkv skips key blocks
    // that lie wholly below the valid memory)
    int kmem_abs = 0;
    if (a.mem_valid) {
        int mv = a.mem_valid[b];
        mv = mv < 0 ? 0 : (mv > M ? M : mv);
        kmem_abs = M - mv;
    }
    const int jhi = qok ? iq + M : -1;

    // G rows of the head (the (b, h) slab; rows past L and offsets past the
    // slab read zeros).  Column L-16-i0w+j0+cc of every row is band row cc of
    // key tile j0; the staged window starts at the 8-aligned column below it.
    const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.g + (int64_t)bh * L * a.kp, (uint32_t)((int64_t)L * a.kp * 2));
    const int pcol0 = L - 16 - i0w;
    const uint32_t sg_base = __builtin_amdgcn_readfirstlane(lds_addr(&sgw[wave][0]));
    auto stage_g = [&](int kt) {
        const int cs = (pcol0 + kt * BK) & ~7;     // may be negative: those columns are masked
#pragma unroll
        for (int e = 0; e < GLD; ++e) {
            const int q = lane + 64 * e;           // chunk q: row q / GRC, chunk q % GRC
            const int row = q / GRC, chk = q - row * GRC;
            const uint32_t goff = (uint32_t)(i0w + row) * (uint32_t)a.kp * 2 + (uint32_t)((cs + 8 * chk) * 2);
            load_lds16(grs, goff, sg_base + (uint32_t)e * 1024);
        }
    };

    // direct loads: thread tid moves chunks tid + QTHR e of each 64-row tile
    // (rows tid / 8 + (QTHR / 8) e; the swizzle is the same for rows 16 apart)
    const int lrow = tid / CPR;
    const int lch = ((tid & (CPR - 1)) ^ swz(lrow)) * 16;
    const uint16_t *kp = static_cast<const uint16_t *>(a.k) + b * a.ks[0] + h * a.ks[1];
    const uint16_t *rp = static_cast<const uint16_t *>(a.r) + h * a.rs[0];
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kp, (uint32_t)(((int64_t)(K - 1) * a.ks[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rp, (uint32_t)(((int64_t)(K - 1) * a.rs[1] + DH) * 2));
    const int krow_b = (int)a.ks[2] * 2, rrow_b = (int)a.rs[1] * 2;
    const uint32_t sk_base = __builtin_amdgcn_readfirstlane(lds_addr(&sk[0][wave * 64]));
    const uint32_t sr_base = __builtin_amdgcn_readfirstlane(lds_addr(&sr[0][wave * 64]));
    // ring row x holds r row cb + x; wave w's band tile bt of key tile kt starts at
    // ring row xw + 64 kt + 16 bt (band row cc of query n <-> key cc + n - 15)
    const int cb = L - QROWS - i0;
    const int xw = QROWS - 16 - 16 * wave;
    auto load_k = [&](int kt) {
        const uint32_t boff = (uint32_t)(kt & 1) * (TILE_CH * 16);
#pragma unroll
        for (int e = 0; e < QLPT; ++e)
            load_lds16(krs, (uint32_t)((kt * BK + lrow + (QTHR / CPR) * e) * krow_b + lch),
                       sk_base + boff + (uint32_t)e * (QTHR * 16));
    };
    auto load_r_quarter = [&](int q) {
        const uint32_t qoff = (uint32_t)(q & (RQ - 1)) * (TILE_CH * 16);
#pragma unroll
        for (int e = 0; e < QLPT; ++e)
            load_lds16(rrs, (uint32_t)((cb + 64 * q + lrow + (QTHR / CPR) * e) * rrow_b + lch),
                       sr_base + qoff + (uint32_t)e * (QTHR * 16));
    };

    f32x4 dqu[NDT], dqv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqu[dt] = dqv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (kt0 < kt1) {
        load_k(kt0);
#pragma unroll
        for (int q = 0; q < RQ - 1; ++q) load_r_quarter(kt0 + q);
        if (kt0 < ntg) stage_g(kt0);
    }
    // lane parts of LDS addresses (a 16-row block's swizzle depends on the lane only)
    int trl[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) trl[dt] = tr_lane_off(dt, g, n);
    // Band rows of query n outside its own 64 keys (cc < 15 - n or cc > 78 - n)
    // belong to the neighbouring tiles: fixed keep masks for k-steps 0 and 2.
    uint32_t pm0[2][2], pm2[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < 2; ++w) pm0[hf][w] = keep2(16 * hf + 4 * g + 2 * w, 15 - n, 78 - n);
#pragma unroll
    for (int w = 0; w < 2; ++w) pm2[w] = keep2(64 + 4 * g + 2 * w, 15 - n, 78 - n);

    auto tile = [&](int kt) {
        const int j0 = kt * BK;
        const TXL_LDS_AS char *tk = lds_bytes(sk[kt & 1]);
        // this lane's staged row; element e of it is column cs + e
        const int cs = (pcol0 + j0) & ~7;
        const TXL_LDS_AS char *grow = (const TXL_LDS_AS char *)(const TXL_LDS_AS void *)&sgw[wave][0] + n * (GRC * 16);
        const int ec = (L - 1 - iq + j0) - cs;   // content: key j0 + k at element ec + k (>= 15 - n)
        const int ep = (pcol0 + j0) - cs;         // position: band row cc at element ep + cc (0..7)
        auto ring_blk = [&](int x0) {   // 16-row block of ring rows x0 .. x0 + 15 (x0 % 16 == 0)
            return lds_bytes(sr[(x0 >> 6) & (RQ - 1)]) + (x0 & 63) * (CPR * 16);
        };
        // G^T operands: content (keys 32 ch + ...) and position (band rows 32 ks + ...)
        u32x2 gcw[2][2], gpw[3][2];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            gcw[ch][0] = gquad(grow, ec + 32 * ch + 4 * g);
            gcw[ch][1] = gquad(grow, ec + 32 * ch + 16 + 4 * g);
        }
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
            gpw[ks][0] = gquad(grow, ep + 32 * ks + 4 * g);
            gpw[ks][1] = ks < 2 ? gquad(grow, ep + 32 * ks + 16 + 4 * g) : u32x2{0u, 0u};
        }
        // the window has been read: load the next tile's into the buffer
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM_ONLY);
        if (kt + 1 < ntg) stage_g(kt + 1);
        // keys outside [kmem, iq + M] have no stored dS: masked on the tiles that reach them
        const bool edge = j0 + BK - 1 > i0w + M || j0 < kmem_abs || !qok;
        // content part: dq^T += K^T . dS^T
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            u32x2 lo = gcw[ch][0], hi = gcw[ch][1];
            if (edge) {
                const int jl = j0 + 32 * ch + 4 * g;
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    lo[w] &= keep2(jl + 2 * w, kmem_abs, jhi);
                    hi[w] &= keep2(jl + 16 + 2 * w, kmem_abs, jhi);
                }
            }
            const bf16x8 gf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) dqu[dt] = mfma(col_frag_at(tk + ch * 32 * CPR * 16, trl[dt]), gf, dqu[dt]);
        }
        // position part: dq^T += R_band^T . G^T over band rows 0..79 in three
        // k-steps (band rows 32 ks + {4 g + e, 16 + 4 g + e}; rows >= 80 are zero)
#pragma unroll
        for (int ks = 0; ks < 3; ++ks) {
            u32x2 lo = gpw[ks][0], hi = gpw[ks][1];
            if (ks == 0) {
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    lo[w] &= pm0[0][w];
                    hi[w] &= pm0[1][w];
                }
            } else if (ks == 2) {
#pragma unroll
                for (int w = 0; w < 2; ++w) lo[w] &= pm2[w];
            }
            if (edge) {
                // band row cc of query n is key j0 + cc + n - 15
                const int jl = j0 + 32 * ks + 4 * g + n - 15;
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    lo[w] &= keep2(jl + 2 * w, kmem_abs, jhi);
                    hi[w] &= keep2(jl + 16 + 2 * w, kmem_abs, jhi);
                }
            }
            const bf16x8 gt = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
            const TXL_LDS_AS char *blo = ring_blk(xw + 64 * kt + 32 * ks);
            const TXL_LDS_AS char *bhi = ring_blk(xw + 64 * kt + 32 * ks + 16);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const u32x2 rlo = tr_half(blo, trl[dt]);
                const u32x2 rhi = ks < 2 ? tr_half(bhi, trl[dt]) : u32x2{0u, 0u};
                dqv[dt] = mfma(__builtin_bit_cast(bf16x8, u32x4{rlo[0], rlo[1], rhi[0], rhi[1]}), gt, dqv[dt]);
            }
        }
    };
    for (int kt = kt0; kt < kt1; ++kt) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kt + 1 < kt1) {
            load_k(kt + 1);
            load_r_quarter(kt + RQ - 1);
        }
        if (kt < ntg) tile(kt);
    }

    const float scale = a.scale;
    if (qok && a.nsplit == 1) {
        uint16_t *dqp = static_cast<uint16_t *>(a.dq) + b * a.qs[0] + h * a.qs[1] + (int64_t)iq * a.qs[2];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const bf16x4 y = __builtin_convertvector((dqu[dt] + dqv[dt]) * scale, bf16x4);
            *reinterpret_cast<u32x2 *>(dqp + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, y);
        }
    } else if (qok) {
        // this split's part of dq (zeros when none of its tiles is visible to the query)
        float *pp = a.dq_part + (((int64_t)split * BH + bh) * L + iq) * DH;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4 *>(pp + 16 * dt + 4 * g) = (dqu[dt] + dqv[dt]) * scale;
    }
    if (i0w < L) {
        // sums over the 16 queries of this wave (queries past L contribute 0)
        float *part = a.bias_part + (((int64_t)split * BH + bh) * a.nqblk + i0w / 16) * (2 * DH);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float su = sum16(dqu[dt][v] * scale), sw = sum16(dqv[dt][v] * scale);
                if (n == 0) {
                    part[16 * dt + 4 * g + v] = su;
                    part[DH + 16 * dt + 4 * g + v] = sw;
                }
            }
    }
}

// ---------------------------------------------------------------------------
// dk, dv: one workgroup per 128 keys, 4 waves of 32 keys (two 16-key
// sub-tiles), queries in steps of 32.

constexpr int KW = 4;               // waves per workgroup
constexpr int KPW = 32;             // keys per wave
constexpr int KBLK = KW * KPW;      // keys per workgroup
constexpr int QS = 32;              // queries per step
constexpr int QT_CH = QS * CPR;     // chunks per query tile
constexpr int NBC = (QS + KBLK) / 16;   // 16-column band tiles per step (r rows pw .. pw + 159)
constexpr int TS = 16 * NBC + 4;    // band row stride in floats
constexpr int RSEG = 8;             // r ring segments of QS rows: five in use, one loading
constexpr int KTHR = 64 * KW;
static_assert(QT_CH == KTHR, "one 16-byte load per thread per query tile");
static_assert((2 * NBC) % KW == 0, "band tiles split evenly over the waves");

__global__ __launch_bounds__(KTHR) void bwd_dkv_kernel(RelAttnBwdArgs a)
{
    __shared__ __attribute__((aligned(16))) u32x4 squ[2][QT_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sqv[2][QT_CH];
    __shared__ __attribute__((aligned(16))) u32x4 sdo[2][QT_CH];
    __shared__ __attribute__((aligned(16))) float sl2[2][QS];
    __shared__ __attribute__((aligned(16))) float sdd[2][QS];
    __shared__ __attribute__((aligned(16))) float tband[QS * TS];
    __shared__ __attribute__((aligned(16))) u32x4 sring[RSEG][QT_CH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int BH = a.B * a.H, L = a.L, M = a.M, K = a.K;
    const int wg = blockIdx.x;
    const int kb = wg / BH;                      // the key blocks seen by most queries first
    const int bh = wg - kb * BH;
    const int b = bh / a.H, h = bh - b * a.H;
    const int j0 = KBLK * kb;
    const int jw0 = j0 + KPW * wave;             // first key of this wave

    const uint16_t *kp = static_cast<const uint16_t *>(a.k) + b * a.ks[0] + h * a.ks[1];
    const uint16_t *vp = static_cast<const uint16_t *>(a.v) + b * a.vs[0] + h * a.vs[1];
    const bf16x8 zero8 = {};
    bf16x8 kf[2][NKK], vf[2][NKK];               // [key sub-tile][k-step]: lane key jw0 + 16 kx + n
#pragma unroll
    for (int kx = 0; kx < 2; ++kx) {
        const int j = jw0 + 16 * kx + n;
        const int jc = j < K ? j : 0;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const bf16x8 x = *reinterpret_cast<const bf16x8 *>(kp + (int64_t)jc * a.ks[2] + 32 * kk + 8 * g);
            const bf16x8 y = *reinterpret_cast<const bf16x8 *>(vp + (int64_t)jc * a.vs[2] + 32 * kk + 8 * g);
            kf[kx][kk] = j < K ? x : zero8;
            vf[kx][kk] = j < K ? y : zero8;
        }
    }
    int kmem_abs = 0;
    if (a.mem_valid) {
        int mv = a.mem_valid[b];
        mv = mv < 0 ? 0 : (mv > M ? M : mv);
        kmem_abs = M - mv;
    }
    const int win = a.window;
    const __amdgpu_buffer_rsrc_t gws = make_rsrc(a.g + (int64_t)bh * L * a.kp, (uint32_t)((int64_t)L * a.kp * 2));
    const int gstep = __builtin_amdgcn_readfirstlane(2 * (a.kp - 1));   // bytes from (i, c) to (i + 1, c - 1)
    // queries below j0 - M see no key of the block; a block entirely below the
    // valid memory is seen by nobody
    int ibeg = j0 - M > 0 ? ((j0 - M) / QS) * QS : 0;
    if (kmem_abs >= j0 + KBLK) ibeg = L;
    const int nsteps = ibeg < L ? (L - ibeg + QS - 1) / QS : 0;

    // loads of a query step: thread tid moves chunk tid of each 32-row tile
    const int lrow = tid / CPR;
    const int lch = ((tid & (CPR - 1)) ^ swz(lrow)) * 16;
    const __amdgpu_buffer_rsrc_t qurs = make_rsrc(a.qu + (int64_t)bh * L * DH, (uint32_t)L * DH * 2);
    const __amdgpu_buffer_rsrc_t qvrs = make_rsrc(a.qv + (int64_t)bh * L * DH, (uint32_t)L * DH * 2);
    const uint16_t *dop = static_cast<const uint16_t *>(a.dout) + b * a.os[0] + h * a.os[1];
    const __amdgpu_buffer_rsrc_t dors = make_rsrc(dop, (uint32_t)(((int64_t)(L - 1) * a.os[2] + DH) * 2));
    const __amdgpu_buffer_rsrc_t l2rs = make_rsrc(a.lse2 + (int64_t)bh * L, (uint32_t)L * 4);
    const __amdgpu_buffer_rsrc_t ddrs = make_rsrc(a.dd + (int64_t)bh * L, (uint32_t)L * 4);
    const int dorow_b = (int)a.os[2] * 2;
    const uint32_t squ_base = __builtin_amdgcn_readfirstlane(lds_addr(&squ[0][wave * 64]));
    const uint32_t sqv_base = __builtin_amdgcn_readfirstlane(lds_addr(&sqv[0][wave * 64]));
    const uint32_t sdo_base = __builtin_amdgcn_readfirstlane(lds_addr(&sdo[0][wave * 64]));
    const uint32_t sl2_base = __builtin_amdgcn_readfirstlane(lds_addr(&sl2[0][0]));
    const uint32_t sdd_base = __builtin_amdgcn_readfirstlane(lds_addr(&sdd[0][0]));
    auto issue = [&](int s) {
        const int i0 = ibeg + QS * s;
        const uint32_t boff = (uint32_t)(s & 1) * (QT_CH * 16);
        const int row = i0 + lrow;
        load_lds16(qurs, (uint32_t)(row * DH * 2 + lch), squ_base + boff);
        load_lds16(qvrs, (uint32_t)(row * DH * 2 + lch), sqv_base + boff);
        load_lds16(dors, (uint32_t)(row * dorow_b + lch), sdo_base + boff);
        // lse2 and D of the 32 queries: 8 lanes of 16 bytes each
        if (wave == 0 && lane < QS / 4) load_lds16(l2rs, (uint32_t)((i0 + 4 * lane) * 4), sl2_base + (uint32_t)(s & 1) * (QS * 4));
        if (wave == 1 && lane < QS / 4) load_lds16(ddrs, (uint32_t)((i0 + 4 * lane) * 4), sdd_base + (uint32_t)(s & 1) * (QS * 4));
    };

    // r rows of the band: step s needs rows pw_s .. pw_s + 16 NBC - 1 with
    // pw_s = L - QS - i0_s + j0, which moves down by QS per step.  Ring segment
    // sgm (slot sgm % RSEG) holds rows pwl + QS sgm .. + QS - 1, pwl being pw of
    // the last step; step s uses segments nsteps-1-s .. nsteps+3-s and loads
    // segment nsteps-2-s for the next step.  Rows outside [0, K) read zeros.
    const uint16_t *rp = static_cast<const uint16_t *>(a.r) + h * a.rs[0];
    const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rp, (uint32_t)(((int64_t)(K - 1) * a.rs[1] + DH) * 2));
    const int rrow_b = (int)a.rs[1] * 2;
    const int pwl = L - QS - (ibeg + QS * (nsteps - 1)) + j0;
    const uint32_t sring_base = __builtin_amdgcn_readfirstlane(lds_addr(&sring[0][wave * 64]));
    auto load_seg = [&](int sgm) {
        load_lds16(rrs, (uint32_t)((pwl + QS * sgm + lrow) * rrow_b + lch),
                   sring_base + (uint32_t)(sgm & (RSEG - 1)) * (QT_CH * 16));
    };

    f32x4 dkt[2][NDT], dvt[2][NDT];
#pragma unroll
    for (int kx = 0; kx < 2; ++kx)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) dkt[kx][dt] = dvt[kx][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nsteps > 0) {
        issue(0);
#pragma unroll
        for (int sg5 = 0; sg5 < NBC / 2; ++sg5) load_seg(nsteps - 1 + sg5);
    }
    // band tiles of this wave: query rows 16 s2 .. +15, band columns 16 pt .. +15
    constexpr int TPW = 2 * NBC / KW;     // band tiles per wave
    const int s2 = (TPW * wave) / NBC;
    const int pt0 = (TPW * wave) % NBC;
    // lane parts of LDS addresses (a 16-row block's swizzle depends on the lane only)
    const int rlo0 = row_lane_off(0, g, n), rlo1 = row_lane_off(1, g, n);
    int trl[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) trl[dt] = tr_lane_off(dt, g, n);
    const bool kmask = jw0 < kmem_abs;                  // keys below the valid memory in this wave
    const int glane = (4 * g * (a.kp - 1) + n) * 2;      // lane part of a G element's byte offset
    for (int s = 0; s < nsteps; ++s) {
        const int i0 = ibeg + QS * s;
        const int buf = s & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (s + 1 < nsteps) {
            issue(s + 1);
            load_seg(nsteps - 2 - s);
        }
        const TXL_LDS_AS char *tqu = lds_bytes(squ[buf]);
        const TXL_LDS_AS char *tqv = lds_bytes(sqv[buf]);
        const TXL_LDS_AS char *tdo = lds_bytes(sdo[buf]);
        // T[i][c] = c (q_i + vb) . r[pw + c] - lse2_i for the step's queries,
        // with pw the r row of (last query, first key); masked entries -inf.
        // Each phase has an unmasked instance for the steps (and waves) that
        // need no mask, chosen by a wave-uniform branch.
        const int pw = L - 1 - (i0 + QS - 1) + j0;
        // The band tiles come out transposed (band columns 4g..4g+3 of query n in
        // lane (g, n)), so each lane writes its four columns with one 16-byte store.
        auto band = [&](auto mtag) {
            constexpr bool MASKED = decltype(mtag)::value;
            const bf16x8 qa0 = row_frag_at(tqv + s2 * BLK16B, rlo0);
            const bf16x8 qa1 = row_frag_at(tqv + s2 * BLK16B, rlo1);
            float nl = -sl2[buf][16 * s2 + n];
            if (MASKED && i0 + 16 * s2 + n >= L) nl = -INFINITY;
            bf16x8 rb[TPW][2];
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int pt = pt0 + u;
                const TXL_LDS_AS char *seg =
                    lds_bytes(sring[(nsteps - 1 - s + (pt >> 1)) & (RSEG - 1)]) + (pt & 1) * BLK16B;
                rb[u][0] = row_frag_at(seg, rlo0);
                rb[u][1] = row_frag_at(seg, rlo1);
            }
            f32x4 acc[TPW];
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                f32x4 cin = f32x4{nl, nl, nl, nl};
                if (MASKED) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int pc = pw + 16 * (pt0 + u) + 4 * g + v;      // r row of element v
                        if (pc > K - 1 || (win > 0 && pc < K - win)) cin[v] = -INFINITY;
                    }
                }
                acc[u] = mfma(rb[u][0], qa0, cin);
                acc[u] = mfma(rb[u][1], qa1, acc[u]);
            }
#pragma unroll
            for (int u = 0; u < TPW; ++u)
                *reinterpret_cast<f32x4 *>(&tband[(16 * s2 + n) * TS + 16 * (pt0 + u) + 4 * g]) = acc[u];
        };
        // masking needed: rows past L, r rows past K-1 (causal) or below K - window
        const bool qmask = i0 + QS > L;
        const bool cmask = pw + 16 * (pt0 + TPW) - 1 > K - 1 || (win > 0 && pw + 16 * pt0 < K - win);
        if (qmask || cmask) band(BoolC<true>{}); else band(BoolC<false>{});
        __syncthreads();
        // scores, probabilities and dS of this wave's 32 keys; dS of the
        // visible pairs (i < L, j <= i + M) to G[i][L-1-i+j] for dq and dr
        // (masked pairs inside the step store zeros).  Element (i, L-1-i+j)
        // sits at byte 2 (i (kp - 1) + L - 1 + j) of the (b, h) slab.
        const int gstep_i0 = __builtin_amdgcn_readfirstlane((i0 * (a.kp - 1) + L - 1 + jw0) * 2);
        bf16x8 pb[2], gb[2];
        auto scores = [&](auto mtag) {
            constexpr bool MASKED = decltype(mtag)::value;
            bf16x8 qa[2][NKK], da[2][NKK];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                qa[x][0] = row_frag_at(tqu + x * BLK16B, rlo0);
                qa[x][1] = row_frag_at(tqu + x * BLK16B, rlo1);
                da[x][0] = row_frag_at(tdo + x * BLK16B, rlo0);
                da[x][1] = row_frag_at(tdo + x * BLK16B, rlo1);
            }
            f32x4 p[2][2], gs[2][2];                 // [query sub-tile][key sub-tile]
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                f32x4 nd;
#pragma unroll
                for (int v = 0; v < 4; ++v) nd[v] = -sdd[buf][16 * x + 4 * g + v];
#pragma unroll
                for (int kx = 0; kx < 2; ++kx) {
                    f32x4 cin;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int r = 16 * x + 4 * g + v;
                        cin[v] = tband[r * TS + KPW * wave + 16 * kx + n - r + QS - 1];
                    }
                    if (MASKED && jw0 + 16 * kx + n < kmem_abs) cin = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                    f32x4 sc = mfma(qa[x][0], kf[kx][0], cin);
                    sc = mfma(qa[x][1], kf[kx][1], sc);
                    f32x4 dp = mfma(da[x][0], vf[kx][0], nd);
                    dp = mfma(da[x][1], vf[kx][1], dp);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        p[x][kx][v] = __builtin_amdgcn_exp2f(sc[v]);
                        gs[x][kx][v] = p[x][kx][v] * dp[v];
                    }
                }
            }
#pragma unroll
            for (int kx = 0; kx < 2; ++kx) {
                pb[kx] = pack8(p[0][kx], p[1][kx]);
                gb[kx] = pack8(gs[0][kx], gs[1][kx]);
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int kx = 0; kx < 2; ++kx)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint16_t bits = __builtin_bit_cast(u16x8, gb[kx])[4 * x + v];
                        if (MASKED) {
                            // one lane offset per (x, kx), the row step v in the
                            // scalar offset; invisible pairs go past the slab
                            const int ib = i0 + 16 * x + 4 * g, j = jw0 + 16 * kx + n;
                            const uint32_t vo = (uint32_t)(ib * (a.kp - 1) + L - 1 + j) * 2;
                            const uint32_t off = ib + v >= L || j > ib + v + M ? 0x80000000u : vo;
                            __builtin_amdgcn_raw_buffer_store_b16(bits, gws, (int)off, v * gstep, 0);
                        } else {
                            // lane part in the vector offset, step, row and key
                            // sub-tile parts uniform
                            __builtin_amdgcn_raw_buffer_store_b16(bits, gws, glane + 32 * kx,
                                                                  gstep_i0 + (16 * x + v) * gstep, 0);
                        }
                    }
        };
        const bool gfull = jw0 + KPW - 1 <= i0 + M && i0 + QS <= L;
        if (kmask || !gfull) scores(BoolC<true>{}); else scores(BoolC<false>{});
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const bf16x8 dot = col_frag_at(tdo, trl[dt]);
            const bf16x8 qut = col_frag_at(tqu, trl[dt]);
#pragma unroll
            for (int kx = 0; kx < 2; ++kx) {
                dvt[kx][dt] = mfma(dot, pb[kx], dvt[kx][dt]);
                dkt[kx][dt] = mfma(qut, gb[kx], dkt[kx][dt]);
            }
        }
    }

#pragma unroll
    for (int kx = 0; kx < 2; ++kx) {
        const int j = jw0 + 16 * kx + n;
        if (j >= K) continue;
        uint16_t *dkp = static_cast<uint16_t *>(a.dk) + b * a.ks[0] + h * a.ks[1] + (int64_t)j * a.ks[2];
        uint16_t *dvp = static_cast<uint16_t *>(a.dv) + b * a.vs[0] + h * a.vs[1] + (int64_t)j * a.vs[2];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            // dk = scale sum dS (q + u) = (scale / c) sum dS c (q + u) = ln 2 sum dS qu
            const bf16x4 yk = __builtin_convertvector(dkt[kx][dt] * LN2, bf16x4);
            const bf16x4 yv = __builtin_convertvector(dvt[kx][dt], bf16x4);
            *reinterpret_cast<u32x2 *>(dkp + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, yk);
            *reinterpret_cast<u32x2 *>(dvp + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, yv);
        }
    }
}

// ---------------------------------------------------------------------------
// dr: one workgroup per 64 rows of r, 16 waves: wave w takes rows
// 16 (w % 4) .. + 15 of the tile for the batch rows b = w / 4 (mod 4); the
// four batch groups stage their own 64-query steps, prefetched two steps ahead
// in registers, and their sums are added in group order at the end.

// du, dvb (which = 0, 1) of head h from the per-16-query sums dq stored: 16
// waves each summing every 16th block of every (split, batch row), then the 16
// wave sums in wave order.  Called by a whole 16-wave workgroup.
__device__ __forceinline__ void bias_sums(const RelAttnBwdArgs &a, int h, int which, float (&red)[16][DH])
{
    const int t = threadIdx.x, wave = t >> 6, d = t & 63;
    float s = 0.f;
    for (int sb = 0; sb < a.nsplit * a.B; ++sb) {       // (split, b) in order; blocks k = wave (mod 16)
        const int sp = sb / a.B, b = sb - sp * a.B;
        const float *pp = a.bias_part + ((int64_t)sp * a.B * a.H + b * a.H + h) * a.nqblk * (2 * DH) + which * DH + d;
#pragma unroll 2
        for (int k = wave; k < a.nqblk; k += 16) s += pp[(int64_t)k * 2 * DH];
    }
    red[wave][d] = s;
    __syncthreads();
    if (wave == 0) {
        float tot = 0.f;
        for (int w = 0; w < 16; ++w) tot += red[w][d];
        (which ? a.dvb : a.du)[h * DH + d] = tot;
    }
}

constexpr int RW = 16;
constexpr int RG = 4;               // batch groups
constexpr int RQS = 64;             // queries per step

__global__ __launch_bounds__(64 * RW) void bwd_dr_kernel(RelAttnBwdArgs a)
{
    // two staging buffers per batch group, so that one barrier per step suffices;
    // the batch groups' sums meet in the G buffers after the loop
    __shared__ __attribute__((aligned(16))) u32x4 sg[2][RG][RQS * CPR];
    __shared__ __attribute__((aligned(16))) u32x4 sq[2][RG][RQS * CPR];
    __shared__ float bred[16][DH];
    static_assert(sizeof(sg) >= (RG - 1) * 4 * NDT * 64 * sizeof(f32x4), "the group sums fit in the G buffers");
    TXL_LDS_AS f32x4 *red = (TXL_LDS_AS f32x4 *)(TXL_LDS_AS void *)&sg[0][0][0];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int psub = wave & 3, bg = wave >> 2;
    const int L = a.L, K = a.K;
    const int nkb = (K + BK - 1) / BK;
    // Workgroup w runs on XCD w mod 8.  With H a multiple of 8 every column
    // block of head h runs on XCD h mod 8, so the head's qv rows, which all its
    // blocks read, are fetched into one L2.
    int h, kbi;
    if ((a.H & 7) == 0) {
        const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
        const int hh = slot / nkb;
        kbi = slot - hh * nkb;
        h = hh * 8 + x;
    } else {
        h = blockIdx.x / nkb;
        kbi = blockIdx.x - h * nkb;
    }
    const int p0 = BK * kbi;
    const int tg = psub * 64 + lane;              // thread within the batch group
    const int lrow = tg / CPR, lpos = tg & (CPR - 1);   // rows lrow and lrow + 32 of a step
    const int lc0 = lpos ^ swz(lrow), lc1 = lpos ^ swz(lrow + 32);
    // rows i with a column >= L-1-i in [p0, p0 + 63]
    const int ilo = L - 1 - (p0 + BK - 1) > 0 ? ((L - 1 - (p0 + BK - 1)) / QS) * QS : 0;
    const int nch = (L - ilo + RQS - 1) / RQS;
    const int nsteps = ((a.B + RG - 1) / RG) * nch;   // same count for every group

    // A fetch only issues loads; the mask of never-written columns (below
    // L-1-i + kmem: keys before the first valid one; at or past K: keys past
    // i + M) is computed from the indices
    // and applied when the data is written to LDS, so the loads stay in flight.
    struct Fetch {
        u32x4 g[2], q[2];
        u32x4 keep[2];    // per 32-bit word: bits of the bf16 columns to keep
    };
    auto fetch_row = [&](int b, int i, int lc, u32x4 &gr, u32x4 &qr, u32x4 &keep) {
        gr = u32x4{0u, 0u, 0u, 0u};
        qr = u32x4{0u, 0u, 0u, 0u};
        keep = u32x4{0u, 0u, 0u, 0u};
        if (b < a.B && i < L) {
            const int64_t bh = (int64_t)b * a.H + h;
            gr = *reinterpret_cast<const u32x4 *>(a.g + (bh * L + i) * a.kp + p0 + 8 * lc);
            qr = *reinterpret_cast<const u32x4 *>(a.qv + (bh * L + i) * DH + 8 * lc);
            // keys below the valid memory were not stored when their whole key block is hidden
            int kmem = 0;
            if (a.mem_valid) {
                int mv = a.mem_valid[b];
                mv = mv < 0 ? 0 : (mv > a.M ? a.M : mv);
                kmem = a.M - mv;
            }
            const int cmin = L - 1 - i + kmem;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = p0 + 8 * lc + e;
                if (col >= cmin && col < K) keep[e >> 1] |= (e & 1) ? 0xffff0000u : 0x0000ffffu;
            }
        }
    };
    auto fetch = [&](int t, Fetch &f) {
        const int b = bg + RG * (t / nch);
        const int i = ilo + RQS * (t % nch) + lrow;
        fetch_row(b, i, lc0, f.g[0], f.q[0], f.keep[0]);
        fetch_row(b, i + 32, lc1, f.g[1], f.q[1], f.keep[1]);
    };

    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int trg = tr_lane_off(psub, g, n);
    int trl[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) trl[dt] = tr_lane_off(dt, g, n);
    // two steps in flight: registers hold steps t + 1 and t + 2 while step t is computed
    Fetch fa, fb;
    if (nsteps > 0) fetch(0, fa);
    if (nsteps > 1) fetch(1, fb);
    // Step t stages into buffer t & 1, which step t - 2 read: every wave
    // finished that before the barrier of step t - 1, which this wave has passed.
    auto step = [&](int t, Fetch &f, int sb) {
        sg[sb][bg][lrow * CPR + lpos] = f.g[0] & f.keep[0];
        sq[sb][bg][lrow * CPR + lpos] = f.q[0];
        sg[sb][bg][(lrow + 32) * CPR + lpos] = f.g[1] & f.keep[1];
        sq[sb][bg][(lrow + 32) * CPR + lpos] = f.q[1];
        __syncthreads();
        if (t + 2 < nsteps) fetch(t + 2, f);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const TXL_LDS_AS char *tgb = lds_bytes(sg[sb][bg]) + half * 2 * BLK16B;
            const TXL_LDS_AS char *tqb = lds_bytes(sq[sb][bg]) + half * 2 * BLK16B;
            const bf16x8 ga = col_frag_at(tgb, trg);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) acc[dt] = mfma(ga, col_frag_at(tqb, trl[dt]), acc[dt]);
        }
    };
    for (int t = 0; t < nsteps; t += 2) {
        step(t, fa, 0);
        if (t + 1 < nsteps) step(t + 1, fb, 1);
    }
    __syncthreads();   // every wave's last reads of the staging buffers are done
    if (bg > 0) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) red[((bg - 1) * 4 * NDT + psub * NDT + dt) * 64 + lane] = acc[dt];
    }
    __syncthreads();
    if (bg == 0) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            f32x4 sum = acc[dt];
#pragma unroll
            for (int k = 0; k < RG - 1; ++k) sum += red[(k * 4 * NDT + psub * NDT + dt) * 64 + lane];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int p = p0 + 16 * psub + 4 * g + v;
                // dr = scale sum dS (q + vb) = ln 2 sum dS c (q + vb)
                if (p < K) a.dr[((int64_t)h * K + p) * DH + 16 * dt + n] = sum[v] * LN2;
            }
        }
    }
    // du and dvb of the head on its first two column blocks, which have the
    // fewest steps (the per-16-query sums were stored by dq, launched before)
    if (kbi < 2) bias_sums(a, h, kbi, bred);
    if (nkb == 1) {
        __syncthreads();
        bias_sums(a, h, 1, bred);
    }
}

// dq of split key ranges: the fp32 parts added in split order, rounded to bf16.
// 16 threads per row (4 columns each), 16 rows per workgroup.
__global__ __launch_bounds__(256) void bwd_dq_combine_kernel(RelAttnBwdArgs a)
{
    const int64_t rows = (int64_t)a.B * a.H * a.L;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c4 = (threadIdx.x & 15) * 4;
    if (row >= rows) return;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.nsplit; ++sp) s += *reinterpret_cast<const f32x4 *>(a.dq_part + (sp * rows + row) * DH + c4);
    const int bh = (int)(row / a.L), i = (int)(row - (int64_t)bh * a.L);
    const int b = bh / a.H, h = bh - b * a.H;
    uint16_t *dqp = static_cast<uint16_t *>(a.dq) + b * a.qs[0] + h * a.qs[1] + (int64_t)i * a.qs[2] + c4;
    *reinterpret_cast<u32x2 *>(dqp) = __builtin_bit_cast(u32x2, __builtin_convertvector(s, bf16x4));
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Row stride of the stored score gradients: stored columns stay below K; the
// dq kernel's operand loads reach column K + 70 (tiles past a query's last
// visible key, masked), rounded up to 64.
int g_row_stride(int K) { return ((K + 78 + BK - 1) / BK) * BK; }

// Key splits of the dq kernel: at least 256 workgroups (one per CU; the
// kernel's 72 KB of LDS allow two), each split at least one key tile.
void dq_split_plan(int B, int H, int L, int M, int &nsplit, int &tps)
{
    const int nqb = (L + QROWS - 1) / QROWS;
    const int ntile = (L - 1 + M) / BK + 1;
    const int64_t base = (int64_t)B * H * nqb;
    int s = base >= 256 ? 1 : (int)std::min<int64_t>(ntile, (256 + base - 1) / base);
    if (s < 1) s = 1;
    tps = (ntile + s - 1) / s;
    nsplit = (ntile + tps - 1) / tps;
}

struct BwdLayout {
    size_t qu, qv, dd, lse2, part, dqp, g, total;
    int nsplit, tps;
};

BwdLayout bwd_layout(int B, int H, int L, int M)
{
    const size_t rows = (size_t)B * H * L;
    const int K = M + L;
    const size_t kp = (size_t)g_row_stride(K);
    const size_t nqblk = (size_t)(L + 15) / 16;
    BwdLayout l{};
    dq_split_plan(B, H, L, M, l.nsplit, l.tps);
    size_t off = 0;
    l.qu = off; off += round256(rows * DH * 2);
    l.qv = off; off += round256(rows * DH * 2);
    l.dd = off; off += round256(rows * 4);
    l.lse2 = off; off += round256(rows * 4);
    l.part = off; off += round256((size_t)l.nsplit * B * H * nqblk * 2 * DH * 4);
    l.dqp = off; off += l.nsplit > 1 ? round256((size_t)l.nsplit * rows * DH * 4) : 0;
    l.g = off; off += round256(rows * kp * 2);
    l.total = off;
    return l;
}

}  // namespace

size_t relattn_bwd_workspace_bytes(int B, int H, int L, int M) { return bwd_layout(B, H, L, M).total; }

void relattn_bwd_carve(RelAttnBwdArgs &a, void *ws)
{
    const BwdLayout l = bwd_layout(a.B, a.H, a.L, a.M);
    char *base = static_cast<char *>(ws);
    a.qu = reinterpret_cast<uint16_t *>(base + l.qu);
    a.qv = reinterpret_cast<uint16_t *>(base + l.qv);
    a.dd = reinterpret_cast<float *>(base + l.dd);
    a.lse2 = reinterpret_cast<float *>(base + l.lse2);
    a.bias_part = reinterpret_cast<float *>(base + l.part);
    a.dq_part = l.nsplit > 1 ? reinterpret_cast<float *>(base + l.dqp) : nullptr;
    a.nsplit = l.nsplit;
    a.tps = l.tps;
    a.g = reinterpret_cast<uint16_t *>(base + l.g);
    a.kp = g_row_stride(a.K);
    a.nqblk = (a.L + 15) / 16;
}

hipError_t launch_relattn_bwd_bf16(const RelAttnBwdArgs &a, hipStream_t s)
{
    const int64_t rows = (int64_t)a.B * a.H * a.L;
    const int BH = a.B * a.H;
    hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((rows + PREP_ROWS - 1) / PREP_ROWS)), dim3(256), 0, s, a);
    // dkv stores the score gradients G that dq and dr read
    hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)(BH * ((a.K + KBLK - 1) / KBLK))), dim3(KTHR), 0, s, a);
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)(BH * ((a.L + QROWS - 1) / QROWS) * a.nsplit)), dim3(QTHR), 0, s, a);
    if (a.nsplit > 1)
        hipLaunchKernelGGL(bwd_dq_combine_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(bwd_dr_kernel, dim3((unsigned)(a.H * ((a.K + BK - 1) / BK))), dim3(64 * RW), 0, s, a);
    return hipGetLastError();
}

}  // namespace txl
