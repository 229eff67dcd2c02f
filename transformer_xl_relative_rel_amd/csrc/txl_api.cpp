// Host side of the C ABI declared in include/txl.h: argument validation,
// launch configuration and dispatch.  Every check runs before any launch, so
// a failing call has no side effects.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "internal.h"
#include "txl.h"

namespace {

thread_local std::string g_last_error;

txl_status fail(txl_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

txl_status ok()
{
    g_last_error.clear();
    return TXL_OK;
}

size_t elem_size(int dtype) { return dtype == TXL_BF16 ? 2 : 4; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte extent [lo, hi) touched by a strided tensor with innermost width `w`.
struct Extent {
    uintptr_t lo, hi;
};

Extent extent(const void *p, const int64_t *stride, const int *count, int ndim, int64_t w, size_t es)
{
    int64_t last = 0;
    for (int d = 0; d < ndim; ++d) last += (int64_t)(count[d] - 1) * stride[d];
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + (uintptr_t)((last + w) * (int64_t)es)};
}

bool overlap(Extent a, Extent b) { return a.lo < b.hi && b.lo < a.hi; }

// Rows kept by the memory update ([SRC] MemTransformerLM._update_mems):
// end = M_cur + max(0, L - ext_len), beg = max(0, end - mem_len), M_new = end - beg.
int tail_len(int M_cur, int L, int mem_len, int ext_len)
{
    const int end = M_cur + (L - ext_len > 0 ? L - ext_len : 0);
    const int beg = end - mem_len > 0 ? end - mem_len : 0;
    return end - beg;
}

// Kernel choice and key-range split of the attention call.
struct Plan {
    int fast;    // 1: bf16 throughput kernel, 0: generic kernel
    int stream;  // 1: bf16 streaming kernel (short segment, long memory)
    int rb, nqb, nsplit, tps;
    size_t ws_bytes;
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Bytes of the partial outputs of a split plan (the bf16 kernels store them in
// their lane layout, padded to whole 16-query blocks), rounded to 256.
size_t part_o_bytes(const txl_relattn_desc &d, const Plan &p)
{
    const int Lp = p.fast ? (d.L + 15) / 16 * 16 : d.L;
    const size_t bytes = (size_t)p.nsplit * d.B * d.H * Lp * d.dh * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

Plan plan_relattn(const txl_relattn_desc &d)
{
    Plan p{};
    const int BH = d.B * d.H;
    p.rb = 1;
    {
        // the throughput kernel addresses each head's K, V and r rows with 32-bit byte offsets
        const int64_t row = std::max(std::max(d.k_stride[2], d.v_stride[2]), d.r_stride[1]);
        const int64_t span = ((int64_t)d.L + d.M + 64) * row * 2;
        p.fast = (d.dtype == TXL_BF16 && txl::relattn_bf16_supported(d.dh) && span < ((int64_t)1 << 31)) ? 1 : 0;
    }
    if (!p.fast && d.dtype == TXL_BF16 && d.dh <= 64 && (int64_t)BH * ceil_div(d.L, 16 * txl::kWaves * 2) >= 256)
        p.rb = 2;
    // Short segments against the memory (few query runs per head, no lower key
    // bounds) go to the streaming kernel: one workgroup per (b, h, key split), one wave per run.
    p.stream = (p.fast && d.L <= 128 && d.window == 0 && !d.mem_valid) ? 1 : 0;
    p.nqb = p.stream ? txl::relattn_bf16_stream_runs(d.L)
                     : (p.fast ? txl::relattn_bf16_groups_per_head(d.L) : ceil_div(d.L, 16 * txl::kWaves * p.rb));
    const int ntile = ceil_div(d.L + d.M, txl::kBK);   // tiles of the longest query block
    int nsplit = d.splits;
    if (nsplit <= 0) {
        // the throughput and streaming kernels hold one workgroup per CU, the
        // generic one two; the streaming kernel's workgroups take all runs of a head
        const int64_t base = p.stream ? (int64_t)BH : (int64_t)p.nqb * BH;
        nsplit = 1;
        if (base < 256) nsplit = (int)std::min<int64_t>(ntile, ((p.fast ? 256 : 512) + base - 1) / base);
        if (nsplit < 1) nsplit = 1;
    }
    if (nsplit > ntile) nsplit = ntile;
    p.tps = ceil_div(ntile, nsplit);
    p.nsplit = ceil_div(ntile, p.tps);
    if (p.nsplit > 1) p.ws_bytes = part_o_bytes(d, p) + (size_t)p.nsplit * BH * d.L * 2 * sizeof(float);
    return p;
}

txl_status check_desc(const txl_relattn_desc *d)
{
    if (!d) return fail(TXL_ERR_INVALID_ARG, "desc is NULL");
    if (d->B < 1 || d->H < 1 || d->L < 1 || d->M < 0 || d->dh < 1)
        return fail(TXL_ERR_INVALID_ARG, "need B, H, L, dh >= 1 and M >= 0 (got B=%d H=%d L=%d M=%d dh=%d)", d->B,
                    d->H, d->L, d->M, d->dh);
    if (d->dtype != TXL_BF16 && d->dtype != TXL_F32) return fail(TXL_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
    if ((int64_t)d->M + d->L > (1 << 30) || (int64_t)d->B * d->H > (1 << 30))
        return fail(TXL_ERR_INVALID_ARG, "sizes too large");
    if (!txl::relattn_supported(d->dtype, d->dh, 1))
        return fail(TXL_ERR_UNSUPPORTED, "dh=%d is not supported for dtype %s (bf16: 32/64/128, f32: 16/32/64)", d->dh,
                    d->dtype == TXL_BF16 ? "bf16" : "f32");
    if (!std::isfinite(d->scale)) return fail(TXL_ERR_INVALID_ARG, "scale is not finite");
    if (d->window < 0) return fail(TXL_ERR_INVALID_ARG, "window must be >= 0 (got %d)", d->window);
    if (d->mem_valid && (reinterpret_cast<uintptr_t>(d->mem_valid) & 3u))
        return fail(TXL_ERR_INVALID_ARG, "mem_valid must be 4-byte aligned");
    const size_t es = elem_size(d->dtype);
    const int64_t *strides[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
    const char *names[4] = {"q", "k", "v", "out"};
    for (int t = 0; t < 4; ++t)
        for (int a = 0; a < 3; ++a) {
            if (strides[t][a] < 0) return fail(TXL_ERR_INVALID_ARG, "%s stride %d is negative", names[t], a);
            if ((strides[t][a] * (int64_t)es) % 16 != 0)
                return fail(TXL_ERR_INVALID_ARG, "%s stride %d (%lld elements) breaks 16-byte row alignment", names[t], a,
                            (long long)strides[t][a]);
        }
    if (d->q_stride[2] < d->dh || d->k_stride[2] < d->dh || d->v_stride[2] < d->dh || d->o_stride[2] < d->dh ||
        d->r_stride[1] < d->dh)
        return fail(TXL_ERR_INVALID_ARG, "row strides must be >= dh (rows may not overlap)");
    for (int a = 0; a < 2; ++a)
        if (d->r_stride[a] < 0 || (d->r_stride[a] * (int64_t)es) % 16 != 0)
            return fail(TXL_ERR_INVALID_ARG, "r_k stride %d breaks 16-byte row alignment", a);
    return TXL_OK;
}

}  // namespace

namespace txl {
// Records the message of the calling thread's last call (shared with txl_layer.cpp).
txl_status set_error(txl_status s, const char *msg)
{
    g_last_error = msg;
    return s;
}
}  // namespace txl

extern "C" {

const char *txl_version(void) { return "0.1.0"; }

const char *txl_status_string(txl_status s)
{
    switch (s) {
    case TXL_OK: return "ok";
    case TXL_ERR_INVALID_ARG: return "invalid argument";
    case TXL_ERR_UNSUPPORTED: return "unsupported configuration";
    case TXL_ERR_ALIAS: return "output aliases an input";
    case TXL_ERR_WORKSPACE: return "workspace missing or too small";
    case TXL_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *txl_last_error(void) { return g_last_error.c_str(); }

txl_status txl_relattn_desc_init(txl_relattn_desc *d, int B, int H, int L, int M, int dh, txl_dtype dtype)
{
    if (!d) return fail(TXL_ERR_INVALID_ARG, "desc is NULL");
    std::memset(d, 0, sizeof *d);
    d->B = B; d->H = H; d->L = L; d->M = M; d->dh = dh;
    d->dtype = dtype;
    d->scale = dh > 0 ? 1.0f / std::sqrt((float)dh) : 0.f;
    d->splits = 0;
    const int64_t K = (int64_t)M + L;
    d->q_stride[0] = (int64_t)H * L * dh; d->q_stride[1] = (int64_t)L * dh; d->q_stride[2] = dh;
    d->k_stride[0] = (int64_t)H * K * dh; d->k_stride[1] = K * dh; d->k_stride[2] = dh;
    std::memcpy(d->v_stride, d->k_stride, sizeof d->k_stride);
    std::memcpy(d->o_stride, d->q_stride, sizeof d->q_stride);
    d->r_stride[0] = K * dh; d->r_stride[1] = dh;
    return ok();
}

txl_status txl_relattn_workspace_size(const txl_relattn_desc *d, size_t *bytes)
{
    txl_status s = check_desc(d);
    if (s != TXL_OK) return s;
    if (!bytes) return fail(TXL_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = plan_relattn(*d).ws_bytes;
    return ok();
}

// Every check of txl_relattn_fwd, then its launch arguments and plan; `ext`
// receives the byte extents of q, k, v, r_k, mem_valid (inputs, 0-4), out,
// lse and the workspace (outputs, 5-7), empty where absent, for the fused
// call's alias checks.
static txl_status fwd_prepare(const txl_relattn_desc *d, const void *q, const void *k, const void *v, const void *r_k,
                              const float *u, const float *vb, void *out, float *lse, void *workspace,
                              size_t workspace_bytes, txl::RelAttnArgs &a, Plan &p, Extent (&ext)[8])
{
    txl_status s = check_desc(d);
    if (s != TXL_OK) return s;
    if (!q || !k || !v || !r_k || !u || !vb || !out) return fail(TXL_ERR_INVALID_ARG, "a required pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(r_k) || !aligned16(out))
        return fail(TXL_ERR_INVALID_ARG, "q, k, v, r_k and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(vb)) & 3u)
        return fail(TXL_ERR_INVALID_ARG, "u and vb must be 4-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(TXL_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    const size_t es = elem_size(d->dtype);
    const int K = d->M + d->L;
    const int cq[3] = {d->B, d->H, d->L}, ck[3] = {d->B, d->H, K}, cr[2] = {d->H, K};
    const Extent eo = extent(out, d->o_stride, cq, 3, d->dh, es);
    const Extent ins[5] = {extent(q, d->q_stride, cq, 3, d->dh, es), extent(k, d->k_stride, ck, 3, d->dh, es),
                           extent(v, d->v_stride, ck, 3, d->dh, es), extent(r_k, d->r_stride, cr, 2, d->dh, es),
                           d->mem_valid ? Extent{reinterpret_cast<uintptr_t>(d->mem_valid),
                                                 reinterpret_cast<uintptr_t>(d->mem_valid + d->B)}
                                        : Extent{0, 0}};
    for (const Extent &e : ins)
        if (overlap(eo, e)) return fail(TXL_ERR_ALIAS, "out overlaps an input tensor");
    if (lse) {
        const Extent el{reinterpret_cast<uintptr_t>(lse),
                        reinterpret_cast<uintptr_t>(lse) + (size_t)d->B * d->H * d->L * sizeof(float)};
        if (overlap(el, eo)) return fail(TXL_ERR_ALIAS, "lse overlaps out");
        for (const Extent &e : ins)
            if (overlap(el, e)) return fail(TXL_ERR_ALIAS, "lse overlaps an input tensor");
    }
    for (Extent &e : ext) e = Extent{0, 0};
    for (int t = 0; t < 5; ++t) ext[t] = ins[t];
    ext[5] = eo;
    if (lse) ext[6] = Extent{reinterpret_cast<uintptr_t>(lse),
                             reinterpret_cast<uintptr_t>(lse) + (size_t)d->B * d->H * d->L * sizeof(float)};
    p = plan_relattn(*d);
    a = txl::RelAttnArgs{};
    a.q = q; a.k = k; a.v = v; a.r = r_k; a.u = u; a.vb = vb; a.out = out; a.lse = lse;
    if (p.nsplit > 1) {
        if (!workspace || workspace_bytes < p.ws_bytes)
            return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", p.ws_bytes,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(TXL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        a.part_o = static_cast<float *>(workspace);
        a.part_ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + part_o_bytes(*d, p));
        a.part_native = p.fast;
        const Extent ew{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + p.ws_bytes};
        ext[7] = ew;
        if (overlap(ew, eo)) return fail(TXL_ERR_ALIAS, "workspace overlaps out");
        for (const Extent &e : ins)
            if (overlap(ew, e)) return fail(TXL_ERR_ALIAS, "workspace overlaps an input tensor");
    }
    for (int t = 0; t < 3; ++t) {
        a.qs[t] = d->q_stride[t]; a.ks[t] = d->k_stride[t]; a.vs[t] = d->v_stride[t]; a.os[t] = d->o_stride[t];
    }
    a.rs[0] = d->r_stride[0]; a.rs[1] = d->r_stride[1];
    a.B = d->B; a.H = d->H; a.L = d->L; a.M = d->M; a.K = K;
    const float scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->dh);
    a.c = (float)((double)scale * 1.4426950408889634);
    a.nqb = p.nqb;
    a.nsplit = p.nsplit;
    a.tiles_per_split = p.tps;
    a.remap = (d->H % 8 == 0) ? 2 : ((d->B * d->H) % 8 == 0 ? 1 : 0);
    a.mem_valid = d->mem_valid;
    a.window = d->window;
    return TXL_OK;
}

static hipError_t fwd_launch(const txl_relattn_desc *d, const Plan &p, const txl::RelAttnArgs &a, void *stream)
{
    return p.stream ? txl::launch_relattn_bf16_stream(a, d->dh, static_cast<hipStream_t>(stream))
           : p.fast ? txl::launch_relattn_bf16(a, d->dh, static_cast<hipStream_t>(stream))
                    : txl::launch_relattn(a, d->dtype, d->dh, p.rb, static_cast<hipStream_t>(stream));
}

txl_status txl_relattn_fwd(const txl_relattn_desc *d, const void *q, const void *k, const void *v, const void *r_k,
                           const float *u, const float *vb, void *out, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    txl::RelAttnArgs a;
    Plan p;
    Extent ext[8];
    const txl_status s = fwd_prepare(d, q, k, v, r_k, u, vb, out, lse, workspace, workspace_bytes, a, p, ext);
    if (s != TXL_OK) return s;
    const hipError_t e = fwd_launch(d, p, a, stream);
    if (e != hipSuccess) return fail(TXL_ERR_HIP, "relattn launch failed: %s", hipGetErrorString(e));
    return ok();
}

txl_status txl_relattn_fwd_noalloc(const txl_relattn_desc *d, const void *q, const void *k, const void *v,
                                   const void *r_k, const float *u, const float *vb, void *out, float *lse,
                                   void *stream)
{
    // the split workspace, if the plan needs one, is the library's static scratch
    size_t need = 0;
    txl_status s = txl_relattn_workspace_size(d, &need);
    if (s != TXL_OK) return s;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    if (need > 0) {
        if (need > txl::kScratchBytes)
            return fail(TXL_ERR_WORKSPACE,
                        "this call needs %zu bytes of key-split workspace; the static scratch holds %zu "
                        "(use txl_relattn_fwd with a workspace, or fewer splits)", need, txl::kScratchBytes);
        const hipError_t e = txl::scratch_buffer(&ws, &ws_bytes);
        if (e != hipSuccess) return fail(TXL_ERR_HIP, "static scratch unavailable: %s", hipGetErrorString(e));
    }
    txl::RelAttnArgs a;
    Plan p;
    Extent ext[8];
    s = fwd_prepare(d, q, k, v, r_k, u, vb, out, lse, ws, ws_bytes, a, p, ext);
    if (s != TXL_OK) return s;
    const hipError_t e = fwd_launch(d, p, a, stream);
    if (e != hipSuccess) return fail(TXL_ERR_HIP, "relattn launch failed: %s", hipGetErrorString(e));
    return ok();
}

// The backward kernels support bf16 with dh = 64 and address one head's rows
// with 32-bit byte offsets.
static txl_status check_bwd(const txl_relattn_desc *d)
{
    txl_status s = check_desc(d);
    if (s != TXL_OK) return s;
    if (d->dtype != TXL_BF16 || d->dh != 64)
        return fail(TXL_ERR_UNSUPPORTED, "the backward supports bf16 with dh = 64 (got %s, dh=%d)",
                    d->dtype == TXL_BF16 ? "bf16" : "f32", d->dh);
    const int64_t K = (int64_t)d->L + d->M;
    const int64_t row = std::max(std::max(d->k_stride[2], d->v_stride[2]), d->r_stride[1]);
    if ((K + 64) * row * 2 >= ((int64_t)1 << 31) || ((int64_t)d->L + 32) * d->o_stride[2] * 2 >= ((int64_t)1 << 31))
        return fail(TXL_ERR_UNSUPPORTED, "one head's rows span 2 GiB or more");
    // one head's stored score gradients (L rows of the workspace's G rows)
    const int64_t kp = ((K + 78 + 63) / 64) * 64;
    if ((int64_t)d->L * kp * 2 >= ((int64_t)1 << 31))
        return fail(TXL_ERR_UNSUPPORTED, "one head's score gradients span 2 GiB or more");
    return TXL_OK;
}

txl_status txl_relattn_bwd_workspace_size(const txl_relattn_desc *d, size_t *bytes)
{
    txl_status s = check_bwd(d);
    if (s != TXL_OK) return s;
    if (!bytes) return fail(TXL_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = txl::relattn_bwd_workspace_bytes(d->B, d->H, d->L, d->M);
    return ok();
}

txl_status txl_relattn_bwd(const txl_relattn_desc *d, const void *q, const void *k, const void *v, const void *r_k,
                           const float *u, const float *vb, const void *out, const float *lse, const void *dout,
                           void *dq, void *dk, void *dv, float *dr, float *du, float *dvb, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    txl_status s = check_bwd(d);
    if (s != TXL_OK) return s;
    if (!q || !k || !v || !r_k || !u || !vb || !out || !lse || !dout || !dq || !dk || !dv || !dr || !du || !dvb)
        return fail(TXL_ERR_INVALID_ARG, "a required pointer is NULL");
    const void *a16[] = {q, k, v, r_k, out, dout, dq, dk, dv, dr};
    for (const void *p : a16)
        if (!aligned16(p)) return fail(TXL_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(vb) | reinterpret_cast<uintptr_t>(lse) |
         reinterpret_cast<uintptr_t>(du) | reinterpret_cast<uintptr_t>(dvb)) & 3u)
        return fail(TXL_ERR_INVALID_ARG, "u, vb, lse, du and dvb must be 4-byte aligned");
    const size_t need = txl::relattn_bwd_workspace_bytes(d->B, d->H, d->L, d->M);
    if (!workspace || workspace_bytes < need)
        return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(TXL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const int K = d->M + d->L;
    const int cq[3] = {d->B, d->H, d->L}, ck[3] = {d->B, d->H, K}, cr[2] = {d->H, K};
    const uintptr_t hd = (uintptr_t)d->H * d->dh * sizeof(float);
    auto flat = [](const void *p, size_t bytes) {
        return Extent{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes};
    };
    const Extent ins[9] = {extent(q, d->q_stride, cq, 3, d->dh, 2), extent(k, d->k_stride, ck, 3, d->dh, 2),
                           extent(v, d->v_stride, ck, 3, d->dh, 2), extent(r_k, d->r_stride, cr, 2, d->dh, 2),
                           extent(out, d->o_stride, cq, 3, d->dh, 2), extent(dout, d->o_stride, cq, 3, d->dh, 2),
                           flat(lse, (size_t)d->B * d->H * d->L * sizeof(float)), flat(u, hd), flat(vb, hd)};
    const Extent outs[7] = {extent(dq, d->q_stride, cq, 3, d->dh, 2), extent(dk, d->k_stride, ck, 3, d->dh, 2),
                            extent(dv, d->v_stride, ck, 3, d->dh, 2),
                            flat(dr, (size_t)d->H * K * d->dh * sizeof(float)), flat(du, hd), flat(dvb, hd),
                            flat(workspace, need)};
    for (int o = 0; o < 7; ++o) {
        for (const Extent &e : ins)
            if (overlap(outs[o], e)) return fail(TXL_ERR_ALIAS, "an output or the workspace overlaps an input");
        for (int o2 = 0; o2 < o; ++o2)
            if (overlap(outs[o], outs[o2])) return fail(TXL_ERR_ALIAS, "two outputs (or the workspace) overlap");
    }
    txl::RelAttnBwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.r = r_k; a.out = out; a.dout = dout;
    a.u = u; a.vb = vb; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dr = dr; a.du = du; a.dvb = dvb;
    for (int t = 0; t < 3; ++t) {
        a.qs[t] = d->q_stride[t]; a.ks[t] = d->k_stride[t]; a.vs[t] = d->v_stride[t]; a.os[t] = d->o_stride[t];
    }
    a.rs[0] = d->r_stride[0]; a.rs[1] = d->r_stride[1];
    a.B = d->B; a.H = d->H; a.L = d->L; a.M = d->M; a.K = K;
    a.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->dh);
    a.c = (float)((double)a.scale * 1.4426950408889634);
    a.mem_valid = d->mem_valid;
    a.window = d->window;
    txl::relattn_bwd_carve(a, workspace);
    hipError_t e = txl::launch_relattn_bwd_bf16(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(TXL_ERR_HIP, "relattn backward launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Every check of txl_mem_update(_batched), then its launch arguments.
static txl_status mem_update_prepare(int n_buf, const void *const *mem, int M_cur, const void *const *h, int L,
                                     void *const *new_mem, int mem_len, int ext_len, int B, int d, int dtype,
                                     int64_t mem_bs, int64_t h_bs, int64_t new_bs, txl::MemUpdateArgs &a)
{
    if (n_buf < 1 || n_buf > txl::kMaxMemBuffers)
        return fail(TXL_ERR_INVALID_ARG, "n_buf must be in [1, %d] (got %d)", txl::kMaxMemBuffers, n_buf);
    if (M_cur < 0 || L < 0 || mem_len < 0 || ext_len < 0 || B < 1 || d < 1)
        return fail(TXL_ERR_INVALID_ARG, "need M_cur, L, mem_len, ext_len >= 0 and B, d >= 1");
    if (dtype != TXL_BF16 && dtype != TXL_F32) return fail(TXL_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    const size_t es = elem_size(dtype);
    const size_t row = (size_t)d * es;
    if (row % 16 != 0) return fail(TXL_ERR_INVALID_ARG, "a row of d=%d elements is not a multiple of 16 bytes", d);
    const int mnew = tail_len(M_cur, L, mem_len, ext_len);
    const int beg = M_cur + (L - ext_len > 0 ? L - ext_len : 0) - mnew;
    if ((int64_t)mnew * (int64_t)(row / 16) >= ((int64_t)1 << 31) || (int64_t)n_buf * B > 65535)
        return fail(TXL_ERR_UNSUPPORTED, "one batch row of the new memory must hold < 2^31 16-byte words and "
                    "n_buf * B must be <= 65535");
    if (mem_bs < 0 || h_bs < 0 || new_bs < 0) return fail(TXL_ERR_INVALID_ARG, "negative batch stride");
    if ((mem_bs * (int64_t)es) % 16 || (h_bs * (int64_t)es) % 16 || (new_bs * (int64_t)es) % 16)
        return fail(TXL_ERR_INVALID_ARG, "batch strides must keep 16-byte alignment");
    if ((B > 1 && M_cur > 0 && mem_bs < (int64_t)M_cur * d) || (B > 1 && L > 0 && h_bs < (int64_t)L * d) ||
        (B > 1 && mnew > 0 && new_bs < (int64_t)mnew * d))
        return fail(TXL_ERR_INVALID_ARG, "batch stride smaller than one batch row");
    a = txl::MemUpdateArgs{};
    for (int i = 0; i < n_buf; ++i) {
        if (M_cur > 0 && !mem[i]) return fail(TXL_ERR_INVALID_ARG, "mem[%d] is NULL with M_cur=%d", i, M_cur);
        if (L > 0 && !h[i]) return fail(TXL_ERR_INVALID_ARG, "h[%d] is NULL", i);
        if (mnew > 0 && !new_mem[i]) return fail(TXL_ERR_INVALID_ARG, "new_mem[%d] is NULL", i);
        if ((M_cur > 0 && !aligned16(mem[i])) || (L > 0 && !aligned16(h[i])) || (mnew > 0 && !aligned16(new_mem[i])))
            return fail(TXL_ERR_INVALID_ARG, "buffer %d is not 16-byte aligned", i);
        if (mnew > 0) {
            const int cn[2] = {B, mnew};
            const int64_t sn[2] = {new_bs, d};
            const Extent en = extent(new_mem[i], sn, cn, 2, d, es);
            for (int j = 0; j < n_buf; ++j) {
                if (M_cur > 0) {
                    const int cm[2] = {B, M_cur};
                    const int64_t sm[2] = {mem_bs, d};
                    if (overlap(en, extent(mem[j], sm, cm, 2, d, es)))
                        return fail(TXL_ERR_ALIAS, "new_mem[%d] overlaps mem[%d]; the update is out of place", i, j);
                }
                if (L > 0) {
                    const int ch[2] = {B, L};
                    const int64_t sh[2] = {h_bs, d};
                    if (overlap(en, extent(h[j], sh, ch, 2, d, es)))
                        return fail(TXL_ERR_ALIAS, "new_mem[%d] overlaps h[%d]", i, j);
                }
                if (j != i && new_mem[j] && overlap(en, extent(new_mem[j], sn, cn, 2, d, es)))
                    return fail(TXL_ERR_ALIAS, "new_mem[%d] overlaps new_mem[%d]", i, j);
            }
        }
        a.mem[i] = static_cast<const unsigned char *>(mem ? mem[i] : nullptr);
        a.h[i] = static_cast<const unsigned char *>(h[i]);
        a.dst[i] = static_cast<unsigned char *>(new_mem[i]);
    }
    a.n_buf = n_buf;
    a.M_cur = M_cur; a.beg = beg; a.M_new = mnew; a.B = B;
    a.row_chunks = (int)(row / 16);
    a.mem_bs = mem_bs * (int64_t)es; a.h_bs = h_bs * (int64_t)es; a.new_bs = new_bs * (int64_t)es;
    return TXL_OK;
}

static txl_status mem_update_common(int n_buf, const void *const *mem, int M_cur, const void *const *h, int L,
                                    void *const *new_mem, int mem_len, int ext_len, int B, int d, int dtype,
                                    int64_t mem_bs, int64_t h_bs, int64_t new_bs, int *M_new, void *stream)
{
    txl::MemUpdateArgs a;
    const txl_status s = mem_update_prepare(n_buf, mem, M_cur, h, L, new_mem, mem_len, ext_len, B, d, dtype, mem_bs,
                                            h_bs, new_bs, a);
    if (s != TXL_OK) return s;
    if (M_new) *M_new = a.M_new;
    hipError_t e = txl::launch_mem_update(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(TXL_ERR_HIP, "mem_update launch failed: %s", hipGetErrorString(e));
    return ok();
}

txl_status txl_mem_update_len(int M_cur, int L, int mem_len, int ext_len, int *M_new)
{
    if (M_cur < 0 || L < 0 || mem_len < 0 || ext_len < 0)
        return fail(TXL_ERR_INVALID_ARG, "need M_cur, L, mem_len, ext_len >= 0");
    if (!M_new) return fail(TXL_ERR_INVALID_ARG, "M_new is NULL");
    *M_new = tail_len(M_cur, L, mem_len, ext_len);
    return ok();
}

txl_status txl_mem_update(const void *mem, int M_cur, const void *h, int L, void *new_mem, int mem_len, int ext_len,
                          int B, int d, int dtype, int64_t mem_bs, int64_t h_bs, int64_t new_bs, int *M_new,
                          void *stream)
{
    return mem_update_common(1, &mem, M_cur, &h, L, &new_mem, mem_len, ext_len, B, d, dtype, mem_bs, h_bs, new_bs,
                             M_new, stream);
}

txl_status txl_mem_update_batched(int n_buf, const void *const *mem, int M_cur, const void *const *h, int L,
                                  void *const *new_mem, int mem_len, int ext_len, int B, int d, int dtype,
                                  int64_t mem_bs, int64_t h_bs, int64_t new_bs, int *M_new, void *stream)
{
    if ((M_cur > 0 && !mem) || !h || !new_mem)
        return fail(TXL_ERR_INVALID_ARG, "pointer arrays must not be NULL");
    return mem_update_common(n_buf, mem, M_cur, h, L, new_mem, mem_len, ext_len, B, d, dtype, mem_bs, h_bs, new_bs,
                             M_new, stream);
}

txl_status txl_relattn_fwd_mem_update(const txl_relattn_desc *d, const void *q, const void *k, const void *v,
                                      const void *r_k, const float *u, const float *vb, void *out, float *lse,
                                      void *workspace, size_t workspace_bytes, const void *mem, int M_cur,
                                      const void *h, int L_h, void *new_mem, int mem_len, int ext_len, int B_m,
                                      int d_model, int dtype_m, int64_t mem_bs, int64_t h_bs, int64_t new_bs,
                                      int *M_new, void *stream)
{
    txl::RelAttnArgs a;
    Plan p;
    Extent ext[8];
    txl_status s = fwd_prepare(d, q, k, v, r_k, u, vb, out, lse, workspace, workspace_bytes, a, p, ext);
    if (s != TXL_OK) return s;
    txl::MemUpdateArgs m;
    s = mem_update_prepare(1, &mem, M_cur, &h, L_h, &new_mem, mem_len, ext_len, B_m, d_model, dtype_m, mem_bs, h_bs,
                           new_bs, m);
    if (s != TXL_OK) return s;
    // the two run concurrently: the copy's output must not meet anything the
    // attention reads or writes, nor its inputs anything the attention writes
    const size_t es = elem_size(dtype_m);
    const Extent uvb[2] = {{reinterpret_cast<uintptr_t>(u), reinterpret_cast<uintptr_t>(u) + (size_t)d->H * d->dh * 4},
                           {reinterpret_cast<uintptr_t>(vb), reinterpret_cast<uintptr_t>(vb) + (size_t)d->H * d->dh * 4}};
    if (m.M_new > 0) {
        const int cn[2] = {B_m, m.M_new};
        const int64_t sn[2] = {new_bs, d_model};
        const Extent en = extent(new_mem, sn, cn, 2, d_model, es);
        for (const Extent &e : ext)
            if (overlap(en, e)) return fail(TXL_ERR_ALIAS, "new_mem overlaps a tensor of the attention call");
        for (const Extent &e : uvb)
            if (overlap(en, e)) return fail(TXL_ERR_ALIAS, "new_mem overlaps u or vb");
    }
    for (int t = 5; t < 8; ++t) {   // out, lse, workspace
        if (M_cur > 0) {
            const int cm[2] = {B_m, M_cur};
            const int64_t sm[2] = {mem_bs, d_model};
            if (overlap(ext[t], extent(mem, sm, cm, 2, d_model, es)))
                return fail(TXL_ERR_ALIAS, "mem overlaps an output or the workspace of the attention call");
        }
        if (L_h > 0) {
            const int ch[2] = {B_m, L_h};
            const int64_t sh[2] = {h_bs, d_model};
            if (overlap(ext[t], extent(h, sh, ch, 2, d_model, es)))
                return fail(TXL_ERR_ALIAS, "h overlaps an output or the workspace of the attention call");
        }
    }
    const bool fused = p.fast && !p.stream;   // the throughput kernel's waves carry the copy
    if (fused) {
        txl::FusedCopy &c = a.cp;
        c.mem = m.mem[0]; c.h = m.h[0]; c.dst = m.dst[0];
        c.mem_bs = m.mem_bs; c.h_bs = m.h_bs; c.new_bs = m.new_bs;
        c.M_cur = m.M_cur; c.beg = m.beg; c.M_new = m.M_new; c.B = m.B;
        if (m.row_chunks > 0x7fffffff / 16) return fail(TXL_ERR_UNSUPPORTED, "a memory row must be < 2 GiB");
        c.row_bytes = m.row_chunks * 16;
        c.cpr = (c.row_bytes + 1023) / 1024;
        const int64_t nch = (int64_t)m.B * m.M_new * c.cpr;
        if (nch >= ((int64_t)1 << 31)) return fail(TXL_ERR_UNSUPPORTED, "the new memory must hold < 2^31 1 KB chunks");
        c.nchunks = (int)nch;
    }
    // every check has passed: nothing below returns before the launches
    if (M_new) *M_new = m.M_new;
    hipError_t e;
    if (fused) {
        e = fwd_launch(d, p, a, stream);
    } else {
        e = fwd_launch(d, p, a, stream);
        if (e == hipSuccess) e = txl::launch_mem_update(m, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return fail(TXL_ERR_HIP, "relattn + mem_update launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
