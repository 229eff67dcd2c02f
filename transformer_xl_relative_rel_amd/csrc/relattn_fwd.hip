// Fused segment-recurrent relative-position attention, forward, for gfx950.
//
// What it computes ([SRC] = "Transformer-XL模型 核心源码阅读笔记",
// RelPartialLearnableMultiHeadAttn.forward; [XL] = "Transformer-XL" textbook
// notes, sections "Relative Positional Encoding" and "Causal Mask With
// Memory"): for query i of the current segment and key j of [memory; segment]
//   s_ij = scale * ((q_i + u) . k_j + (q_i + vb) . r[L-1-i+j]),
//   visible iff j <= i + M,  out_i = softmax_j(s_ij) . v_j.
// The pages form the position term for every (i, r-row) and realign it with a
// pad/reshape/slice "rel_shift"; here the needed r rows are indexed directly.
//
// Work decomposition.  A workgroup owns BQ = 16 * kWaves * RB query rows of
// one (b, h) and walks the visible keys in tiles of kBK = 64.  Each wave owns
// RB blocks of 16 queries.  Everything is computed transposed (keys on MFMA
// rows, queries on MFMA columns = lanes), so that the probabilities come out of
// the score MFMA already in the B-operand layout of the P.V MFMA:
//   T^T = R_band . Qv^T    (band MFMA: 16 queries need kBK + 15 consecutive
//                            r rows per key tile)
//   skew T^T through LDS so that the value for (query n, key j) lands in the
//   accumulator slot of key j; that is the initial C of
//   S^T = K . Qu^T + BD^T  (content MFMA)
//   mask in registers, online softmax (exp2 with scale*log2(e) folded in),
//   O^T += V^T . P^T, and the softmax denominator as one more MFMA against a
//   row of ones.
// Tiles of K, V (transposed for bf16) and the r band are staged in LDS and
// prefetched into registers one tile ahead.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace txl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = kBK;
constexpr int NW = kWaves;
constexpr int NT = BK / 16;     // 16-key sub-tiles per key tile
constexpr int NBT = NT + 1;     // 16-row band tiles per 16-query block
constexpr float LN2 = 0.69314718055994530942f;

template <bool BF> struct Elem;
template <> struct Elem<true> { using T = uint16_t; static constexpr int KSTEP = 32; };
template <> struct Elem<false> { using T = float; static constexpr int KSTEP = 4; };

// LDS layout of one workgroup.  Row strides are padded so the 16 rows read
// by one MFMA fragment start in different banks.
template <bool BF, int DH, int RB>
struct Smem {
    using T = typename Elem<BF>::T;
    static constexpr int BQ = NW * RB * 16;
    static constexpr int RROWS = BQ + BK;                 // staged band rows (BQ + BK - 1 used)
    static constexpr int KRS = DH + (BF ? 8 : 4);         // K and r row stride, elements
    static constexpr int VROWS = BF ? DH : BK;            // bf16: V^T [DH][BK]; f32: V [BK][DH]
    static constexpr int VRS = BF ? (BK + 8) : (DH + 4);
    static constexpr int SROW = BK + 36;                  // skew row stride, floats
    T ks[BK * KRS];
    T vs[VROWS * VRS];
    T rs[RROWS * KRS];
    float bd[NW][16 * SROW];
};

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// 16-byte vector of one staged row chunk.
struct Chunk { u32x4 d; };

template <bool BF, int DH, int RB>
struct Kernel {
    using T = typename Elem<BF>::T;
    using S = Smem<BF, DH, RB>;
    static constexpr int KS = Elem<BF>::KSTEP;
    static constexpr int NKK = DH / KS;                  // k-steps over the head width
    static constexpr int CH = 16 / sizeof(T);            // elements per 16-byte chunk
    static constexpr int K_CHUNKS = BK * DH / CH;        // chunks per K (or f32 V) tile
    static constexpr int R_CHUNKS = S::RROWS * DH / CH;  // chunks per band tile
    static constexpr int V_PAIRS = (BK / 2) * (DH / 8);  // bf16 V: (key pair, 8-column) units
    static constexpr int NKC = (K_CHUNKS + 255) / 256;
    static constexpr int NRC = (R_CHUNKS + 255) / 256;
    static constexpr int NVC = BF ? (V_PAIRS + 255) / 256 : NKC;
    using QF = typename std::conditional<BF, bf16x8, float>::type;

    // Staging registers: one key tile ahead.
    struct Stage {
        Chunk k[NKC];
        Chunk v[BF ? 2 * NVC : NKC];
        Chunk r[NRC];
    };

    __device__ static Chunk load_chunk(const T *base, int64_t row_stride, int row, int nrows, int col)
    {
        Chunk c;
        if (row >= 0 && row < nrows)
            c.d = *reinterpret_cast<const u32x4 *>(base + (int64_t)row * row_stride + col);
        else
            c.d = u32x4{0u, 0u, 0u, 0u};
        return c;
    }

    __device__ static void prefetch(Stage &st, const RelAttnArgs &a, const T *kp, const T *vp, const T *rp,
                                    int j0, int c0, int tid)
    {
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            int e = tid + 256 * s;
            int row = e / (DH / CH), col = (e % (DH / CH)) * CH;
            if (e < K_CHUNKS) st.k[s] = load_chunk(kp, a.ks[2], j0 + row, a.K, col);
        }
        if constexpr (BF) {
#pragma unroll
            for (int s = 0; s < NVC; ++s) {
                int e = tid + 256 * s;
                int col8 = e / (BK / 2), kpair = e % (BK / 2);
                if (e < V_PAIRS) {
                    st.v[2 * s] = load_chunk(vp, a.vs[2], j0 + 2 * kpair, a.K, col8 * 8);
                    st.v[2 * s + 1] = load_chunk(vp, a.vs[2], j0 + 2 * kpair + 1, a.K, col8 * 8);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < NKC; ++s) {
                int e = tid + 256 * s;
                int row = e / (DH / CH), col = (e % (DH / CH)) * CH;
                if (e < K_CHUNKS) st.v[s] = load_chunk(vp, a.vs[2], j0 + row, a.K, col);
            }
        }
#pragma unroll
        for (int s = 0; s < NRC; ++s) {
            int e = tid + 256 * s;
            int row = e / (DH / CH), col = (e % (DH / CH)) * CH;
            if (e < R_CHUNKS) st.r[s] = load_chunk(rp, a.rs[1], c0 + row, a.K, col);
        }
    }

    __device__ static void commit(const Stage &st, S &sm, int tid)
    {
#pragma unroll
        for (int s = 0; s < NKC; ++s) {
            int e = tid + 256 * s;
            int row = e / (DH / CH), col = (e % (DH / CH)) * CH;
            if (e < K_CHUNKS) *reinterpret_cast<u32x4 *>(&sm.ks[row * S::KRS + col]) = st.k[s].d;
        }
        if constexpr (BF) {
            // Transpose key pairs into V^T[dh][key]: one 32-bit word holds keys (2p, 2p+1).
#pragma unroll
            for (int s = 0; s < NVC; ++s) {
                int e = tid + 256 * s;
                int col8 = e / (BK / 2), kpair = e % (BK / 2);
                if (e < V_PAIRS) {
                    const u32x4 lo = st.v[2 * s].d, hi = st.v[2 * s + 1].d;
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        uint32_t a0 = (lo[w] & 0xffffu) | (hi[w] << 16);
                        uint32_t a1 = (lo[w] >> 16) | (hi[w] & 0xffff0000u);
                        uint32_t *dst = reinterpret_cast<uint32_t *>(&sm.vs[(col8 * 8 + 2 * w) * S::VRS + 2 * kpair]);
                        dst[0] = a0;
                        *reinterpret_cast<uint32_t *>(&sm.vs[(col8 * 8 + 2 * w + 1) * S::VRS + 2 * kpair]) = a1;
                    }
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < NKC; ++s) {
                int e = tid + 256 * s;
                int row = e / (DH / CH), col = (e % (DH / CH)) * CH;
                if (e < K_CHUNKS) *reinterpret_cast<u32x4 *>(&sm.vs[row * S::VRS + col]) = st.v[s].d;
            }
        }
#pragma unroll
        for (int s = 0; s < NRC; ++s) {
            int e = tid + 256 * s;
            int row = e / (DH / CH), col = (e % (DH / CH)) * CH;
            if (e < R_CHUNKS) *reinterpret_cast<u32x4 *>(&sm.rs[row * S::KRS + col]) = st.r[s].d;
        }
    }

    // A operand of a 16-row MFMA block whose rows are `row0 + m` of a
    // row-major LDS tile (K or the r band), k-step kk.
    __device__ static QF afrag(const T *base, int row, int kk, int g)
    {
        if constexpr (BF) {
            u32x4 x = *reinterpret_cast<const u32x4 *>(base + row * S::KRS + kk * 32 + 8 * g);
            return __builtin_bit_cast(bf16x8, x);
        } else {
            return base[row * S::KRS + kk * 4 + g];
        }
    }

    __device__ static f32x4 mfma(QF a, QF b, f32x4 c)
    {
        if constexpr (BF)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }

    __device__ static void run(const RelAttnArgs &a)
    {
        __shared__ __attribute__((aligned(16))) S sm;
        constexpr int BQ = S::BQ;
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int g = lane >> 4, n = lane & 15;

        // ---- which (query block, b*h, key split) this workgroup owns
        const int BH = a.B * a.H;
        const int w = blockIdx.x;
        int slot = w, xg = 0, G = BH;
        if (a.remap) { xg = w & 7; slot = w >> 3; G = BH >> 3; }
        const int per = a.nsplit;
        const int qb_rank = slot / (G * per);
        const int r2 = slot - qb_rank * G * per;
        const int bh = a.remap ? xcd_pair(a, xg, r2 / per) : r2 / per;
        const int split = r2 % per;
        const int qb = a.nqb - 1 - qb_rank;   // the longest query blocks start first
        const int b = bh / a.H, h = bh - b * a.H;
        const int L = a.L, M = a.M;
        const int i0 = qb * BQ;
        const int kv_end = min(i0 + BQ, L) + M;   // keys visible to some row of the block
        const int ntile = (kv_end + BK - 1) / BK;
        // keys below the first query's lower bound are hidden from the whole block
        const int kt0 = max(split * a.tiles_per_split, key_lo(a, b, i0) / BK);
        const int kt1 = min(ntile, split * a.tiles_per_split + a.tiles_per_split);

        const T *qp = reinterpret_cast<const T *>(a.q) + b * a.qs[0] + h * a.qs[1];
        const T *kp = reinterpret_cast<const T *>(a.k) + b * a.ks[0] + h * a.ks[1];
        const T *vp = reinterpret_cast<const T *>(a.v) + b * a.vs[0] + h * a.vs[1];
        const T *rp = reinterpret_cast<const T *>(a.r) + h * a.rs[0];
        const float *up = a.u + h * DH;
        const float *wp = a.vb + h * DH;

        // ---- query fragments: B operands (q + u) and (q + vb), added in fp32,
        // rounded once to the input type.  Lane (g, n) holds query n of the block.
        QF qu[RB][NKK], qv[RB][NKK];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int iq = i0 + 16 * (wave * RB + rb) + n;
            const bool ok = iq < L;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                if constexpr (BF) {
                    f32x8 fu, fv;
                    u32x4 raw = ok ? *reinterpret_cast<const u32x4 *>(qp + (int64_t)iq * a.qs[2] + kk * 32 + 8 * g)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = bf16_to_f32((uint16_t)(raw[e >> 1] >> (16 * (e & 1))));
                        int col = kk * 32 + 8 * g + e;
                        fu[e] = ok ? x + up[col] : 0.f;
                        fv[e] = ok ? x + wp[col] : 0.f;
                    }
                    qu[rb][kk] = __builtin_convertvector(fu, bf16x8);
                    qv[rb][kk] = __builtin_convertvector(fv, bf16x8);
                } else {
                    int col = kk * 4 + g;
                    float x = ok ? qp[(int64_t)iq * a.qs[2] + col] : 0.f;
                    qu[rb][kk] = ok ? x + up[col] : 0.f;
                    qv[rb][kk] = ok ? x + wp[col] : 0.f;
                }
            }
        }

        f32x4 o[RB][DH / 16], lsum[RB];
        float mrun[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int dt = 0; dt < DH / 16; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
            lsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
            mrun[rb] = -INFINITY;
        }

        // First r row of the staged band for key tile kt: L - i0 - BQ + kt*BK.
        Stage st;
        if (kt0 < kt1) prefetch(st, a, kp, vp, rp, kt0 * BK, L - i0 - BQ + kt0 * BK, tid);

        for (int kt = kt0; kt < kt1; ++kt) {
            const int j0 = kt * BK;
            __syncthreads();
            commit(st, sm, tid);
            __syncthreads();
            if (kt + 1 < kt1) prefetch(st, a, kp, vp, rp, j0 + BK, L - i0 - BQ + j0 + BK, tid);

#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int blk = wave * RB + rb;
                const int iq0 = i0 + 16 * blk;
                if (iq0 >= L) continue;                              // rows past the segment
                const int iql = min(iq0 + 15, L - 1);
                if (j0 > iql + M) continue;                           // tile fully masked
                if (j0 + BK - 1 < key_lo(a, b, iq0)) continue;        // below every row's lower bound
                // ---- position term on the band of r rows: T^T[cc][n] = r[c0 + cc] . (q_n + vb)
                const int roff = BQ - 16 * (1 + blk);
                f32x4 t[NBT];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt) {
                    t[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk)
                        t[bt] = mfma(afrag(sm.rs, roff + 16 * bt + n, kk, g), qv[rb][kk], t[bt]);
                }
                // ---- skew: band row cc of query n belongs to key jj = cc + n - 15;
                // stored at column jj + 16 of the query's row.
                float *bdw = sm.bd[wave];
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) bdw[n * S::SROW + 16 * bt + 4 * g + v + n + 1] = t[bt][v];
                wave_lds_sync();
                f32x4 sc[NT];
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
                    sc[tt] = *reinterpret_cast<const f32x4 *>(&bdw[n * S::SROW + 16 + 16 * tt + 4 * g]);
                wave_lds_sync();
                // ---- content term accumulated on top: S^T = K . (q + u)^T + BD^T
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) sc[tt] = mfma(afrag(sm.ks, 16 * tt + n, kk, g), qu[rb][kk], sc[tt]);
                // ---- mask: key j visible to query i iff key_lo(i) <= j <= i + M
                const int iq = iq0 + n;
                if (j0 + BK - 1 > iq0 + M || j0 < key_lo(a, b, iql)) {
                    const int lo = key_lo(a, b, iq);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const int j = j0 + 16 * tt + 4 * g + v;
                            if (j > iq + M || j < lo) sc[tt][v] = -INFINITY;
                        }
                }
                // ---- online softmax in base 2
                float mx = -INFINITY;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sc[tt][v]);
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mnew = fmaxf(mrun[rb], mx * a.c);
                const float mref = (mnew == -INFINITY) ? 0.f : mnew;
                const float alpha = __builtin_amdgcn_exp2f(mrun[rb] - mref);
                mrun[rb] = mnew;
#pragma unroll
                for (int dt = 0; dt < DH / 16; ++dt) o[rb][dt] *= alpha;
                lsum[rb] *= alpha;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) sc[tt][v] = __builtin_amdgcn_exp2f(fmaf(sc[tt][v], a.c, -mref));
                // ---- O^T += V^T . P^T ; denominator += ones . P^T
                if constexpr (BF) {
                    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
#pragma unroll
                    for (int ch = 0; ch < NT / 2; ++ch) {
                        f32x8 pf32 = {sc[2 * ch][0], sc[2 * ch][1], sc[2 * ch][2], sc[2 * ch][3],
                                      sc[2 * ch + 1][0], sc[2 * ch + 1][1], sc[2 * ch + 1][2], sc[2 * ch + 1][3]};
                        const bf16x8 pf = __builtin_convertvector(pf32, bf16x8);
#pragma unroll
                        for (int dt = 0; dt < DH / 16; ++dt) {
                            const T *vrow = &sm.vs[(16 * dt + n) * S::VRS + 32 * ch + 4 * g];
                            u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow);
                            u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16);
                            u32x4 x = {lo[0], lo[1], hi[0], hi[1]};
                            o[rb][dt] = mfma(__builtin_bit_cast(bf16x8, x), pf, o[rb][dt]);
                        }
                        lsum[rb] = mfma(ones, pf, lsum[rb]);
                    }
                } else {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float p = sc[tt][v];
#pragma unroll
                            for (int dt = 0; dt < DH / 16; ++dt)
                                o[rb][dt] = mfma(sm.vs[(16 * tt + 4 * g + v) * S::VRS + 16 * dt + n], p, o[rb][dt]);
                            lsum[rb] = mfma(1.f, p, lsum[rb]);
                        }
                }
            }
        }

        // ---- epilogue: lane (g, n) holds query n, head columns 16*dt + 4*g + v.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int iq = i0 + 16 * (wave * RB + rb) + n;
            if (iq >= L) continue;
            if (a.nsplit == 1) {
                const float inv = 1.f / lsum[rb][0];
                T *op = reinterpret_cast<T *>(a.out) + b * a.os[0] + h * a.os[1] + (int64_t)iq * a.os[2];
#pragma unroll
                for (int dt = 0; dt < DH / 16; ++dt) {
                    f32x4 y = o[rb][dt] * inv;
                    if constexpr (BF) {
                        bf16x4 yb = __builtin_convertvector(y, bf16x4);
                        *reinterpret_cast<u32x2 *>(op + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, yb);
                    } else {
                        *reinterpret_cast<f32x4 *>(op + 16 * dt + 4 * g) = y;
                    }
                }
                if (a.lse && g == 0) a.lse[(int64_t)bh * L + iq] = (mrun[rb] + __log2f(lsum[rb][0])) * LN2;
            } else {
                float *po = a.part_o + (((int64_t)split * BH + bh) * L + iq) * DH;
#pragma unroll
                for (int dt = 0; dt < DH / 16; ++dt) *reinterpret_cast<f32x4 *>(po + 16 * dt + 4 * g) = o[rb][dt];
                if (g == 0) {
                    float *pm = a.part_ml + (((int64_t)split * BH + bh) * L + iq) * 2;
                    pm[0] = mrun[rb];
                    pm[1] = lsum[rb][0];
                }
            }
        }
    }
};

template <bool BF, int DH, int RB>
__global__ __launch_bounds__(256) void relattn_fwd_kernel(RelAttnArgs a)
{
    Kernel<BF, DH, RB>::run(a);
}

// Combine the key-range partials of the split path in split order:
//   m* = max_s m_s,  out = sum_s 2^(m_s - m*) o_s / sum_s 2^(m_s - m*) l_s.
// One pass over the splits in chunks of CH whose loads are issued together
// (one memory latency per chunk); the running sums are rescaled when a chunk
// raises the running max.  The order is fixed, so the result is bitwise
// deterministic.  CH = 4 serves up to four splits in one chunk.
template <bool BF, int DH, int CH>
__global__ __launch_bounds__(256) void relattn_combine_kernel(RelAttnArgs a)
{
    using T = typename Elem<BF>::T;
    constexpr int TPR = DH / 4;                     // threads per query row
    constexpr int RPB = 256 / TPR;                  // query rows per workgroup
    const int BH = a.B * a.H;
    // workgroups per (b, h); with the XCD-aware order the rows of a (b, h) are
    // combined on the XCD whose L2 holds its partials (workgroup w runs on XCD
    // w % 8, as in the attention kernels)
    const int cph = (a.L + RPB - 1) / RPB;
    const int w = blockIdx.x;
    int bh, chunk;
    if (a.remap) {
        const int j = w >> 3;
        bh = xcd_pair(a, w & 7, j / cph);
        chunk = j % cph;
    } else {
        bh = w / cph;
        chunk = w - bh * cph;
    }
    const int iq = chunk * RPB + threadIdx.x / TPR;
    const int c4 = (threadIdx.x % TPR) * 4;
    if (iq >= a.L) return;
    const int64_t row = (int64_t)bh * a.L + iq;
    const int b = bh / a.H, h = bh - b * a.H;
    const int64_t sstride = (int64_t)BH * a.L;      // rows between consecutive splits
    const int64_t r0 = (int64_t)bh * a.L + iq;
    float mrun = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.nsplit; s0 += CH) {
        float ms[CH], ls[CH];
        f32x4 os[CH];
#pragma unroll
        for (int e = 0; e < CH; ++e) {
            const bool ok = s0 + e < a.nsplit;
            const int64_t base = (ok ? s0 + e : 0) * sstride + r0;
            ms[e] = ok ? a.part_ml[base * 2] : -INFINITY;
            ls[e] = ok ? a.part_ml[base * 2 + 1] : 0.f;
            int64_t oi = base * DH + c4;   // row-major
            if (DH == 64 && a.part_native) {
                // lane layout of the bf16 kernels: 16-byte group (dt, 16 g + n) of 16-query block iq / 16
                const int64_t blk = ((ok ? s0 + e : 0) * (int64_t)BH + bh) * ((a.L + 15) >> 4) + (iq >> 4);
                oi = (blk * (DH / 16 * 64) + (c4 >> 4) * 64 + ((c4 & 15) >> 2) * 16 + (iq & 15)) * 4;
            }
            os[e] = ok ? *reinterpret_cast<const f32x4 *>(a.part_o + oi) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float mnew = mrun;
#pragma unroll
        for (int e = 0; e < CH; ++e) mnew = fmaxf(mnew, ms[e]);
        if (mnew != mrun && mrun != -INFINITY) {
            const float sc = __builtin_amdgcn_exp2f(mrun - mnew);
            den *= sc;
            num *= sc;
        }
        mrun = mnew;
#pragma unroll
        for (int e = 0; e < CH; ++e) {
            const float wgt = (ms[e] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms[e] - mrun);
            den += wgt * ls[e];
            num += wgt * os[e];
        }
    }
    f32x4 y = num * (1.f / den);
    T *op = reinterpret_cast<T *>(a.out) + b * a.os[0] + h * a.os[1] + (int64_t)iq * a.os[2] + c4;
    if constexpr (BF) {
        bf16x4 yb = __builtin_convertvector(y, bf16x4);
        *reinterpret_cast<u32x2 *>(op) = __builtin_bit_cast(u32x2, yb);
    } else {
        *reinterpret_cast<f32x4 *>(op) = y;
    }
    if (a.lse && c4 == 0) a.lse[row] = (mrun + __log2f(den)) * LN2;
}

template <bool BF, int DH, int RB>
hipError_t launch_one(const RelAttnArgs &a, hipStream_t s)
{
    const int blocks = a.nqb * a.B * a.H * a.nsplit;
    hipLaunchKernelGGL((relattn_fwd_kernel<BF, DH, RB>), dim3(blocks), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    return launch_relattn_combine(a, BF ? 1 : 0, DH, s);
}

}  // namespace

template <bool BF, int DH>
void launch_combine_dh(const RelAttnArgs &a, dim3 grid, hipStream_t s)
{
    if (a.nsplit <= 4) hipLaunchKernelGGL((relattn_combine_kernel<BF, DH, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((relattn_combine_kernel<BF, DH, 16>), grid, dim3(256), 0, s, a);
}

hipError_t launch_relattn_combine(const RelAttnArgs &a, int dtype, int dh, hipStream_t s)
{
    const int rows_per_block = 256 / (dh / 4);
    const dim3 grid((unsigned)((int64_t)a.B * a.H * ((a.L + rows_per_block - 1) / rows_per_block)));
    if (dtype == 1) {
        if (dh == 32) launch_combine_dh<true, 32>(a, grid, s);
        else if (dh == 64) launch_combine_dh<true, 64>(a, grid, s);
        else if (dh == 128) launch_combine_dh<true, 128>(a, grid, s);
        else return hipErrorInvalidValue;
    } else {
        if (dh == 16) launch_combine_dh<false, 16>(a, grid, s);
        else if (dh == 32) launch_combine_dh<false, 32>(a, grid, s);
        else if (dh == 64) launch_combine_dh<false, 64>(a, grid, s);
        else return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool relattn_supported(int dtype, int dh, int rb)
{
    if (dtype == 1) return (dh == 32 || dh == 64 || dh == 128) && (rb == 1 || (rb == 2 && dh <= 64));
    if (dtype == 0) return (dh == 16 || dh == 32 || dh == 64) && rb == 1;
    return false;
}

hipError_t launch_relattn(const RelAttnArgs &a, int dtype, int dh, int rb, hipStream_t s)
{
    if (dtype == 1) {
        if (rb == 2) {
            if (dh == 32) return launch_one<true, 32, 2>(a, s);
            if (dh == 64) return launch_one<true, 64, 2>(a, s);
        } else {
            if (dh == 32) return launch_one<true, 32, 1>(a, s);
            if (dh == 64) return launch_one<true, 64, 1>(a, s);
            if (dh == 128) return launch_one<true, 128, 1>(a, s);
        }
    } else {
        if (dh == 16) return launch_one<false, 16, 1>(a, s);
        if (dh == 32) return launch_one<false, 32, 1>(a, s);
        if (dh == 64) return launch_one<false, 64, 1>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace txl
