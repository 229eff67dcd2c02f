// Host side of txl_layer_fwd (include/txl.h): argument checks, workspace
// carving, and the sequence of launches of one post-LN decoder layer
// ([SRC] "Transformer-XL模型 核心源码阅读笔记": RelPartialLearnableDecoderLayer,
// RelPartialLearnableMultiHeadAttn.forward, PositionwiseFF.forward).
//
// The five projections are plain bf16 GEMMs with fp32 accumulation, run by
// rocBLAS (row-major Y = X W^T as the column-major product W^T-op X).  The
// relative attention runs on strided views of one [B][K][3*H*dh] buffer that
// holds q (current rows only), k and v, and writes the merged heads
// [B][L][H*dh] directly.

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"
#include "txl.h"

namespace txl {
// Shared with txl_api.cpp: record a failure message for txl_last_error().
txl_status set_error(txl_status s, const char *msg);
}

namespace {

txl_status fail(txl_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    return txl::set_error(s, buf);
}

// Row-major Y[n][m] (+)= X[n][k] W[m][k]^T for `batch` independent problems.
rocblas_status gemm_xwt(rocblas_handle h, int m, int n, int k, const void *W, int ldw, const void *X, int ldx,
                        int64_t sx, void *Y, rocblas_datatype ytype, int ldy, int64_t sy, int batch)
{
    const float one = 1.f, zero = 0.f;
    return rocblas_gemm_strided_batched_ex(h, rocblas_operation_transpose, rocblas_operation_none, m, n, k, &one, W,
                                           rocblas_datatype_bf16_r, ldw, 0, X, rocblas_datatype_bf16_r, ldx, sx, &zero,
                                           Y, ytype, ldy, sy, Y, ytype, ldy, sy, batch, rocblas_datatype_f32_r,
                                           rocblas_gemm_algo_standard, 0, 0);
}

struct LayerWs {
    size_t pe, r, qkv, attn, a, x, f1, f1b, f2, attn_ws, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout; attn_ws is the attention's own (split) workspace.
bool layer_ws(const txl_layer_desc &d, int M_cur, LayerWs &w, txl_relattn_desc *ad)
{
    const int64_t B = d.B, L = d.L, K = (int64_t)M_cur + d.L, D = d.d_model, HD = (int64_t)d.n_head * d.d_head;
    const int64_t DI = d.d_inner;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    w.pe = take(K * D * 2);
    w.r = take(K * HD * 2);
    w.qkv = take(B * K * 3 * HD * 2);
    w.attn = take(B * L * HD * 2);
    w.a = take(B * L * D * 4);
    w.x = take(B * L * D * 2);
    w.f1 = take(B * L * DI * 4);
    w.f1b = take(B * L * DI * 2);
    w.f2 = w.a;   // o_net output is dead once LN1 has run
    size_t aws = 0;
    if (ad) {
        if (txl_relattn_workspace_size(ad, &aws) != TXL_OK) return false;
    }
    w.attn_ws = take(aws);
    w.total = off;
    return true;
}

// Attention descriptor for views into the qkv buffer [B][K][3 HD] and the
// merged-heads output [B][L][HD].
void attn_desc(const txl_layer_desc &d, int M_cur, txl_relattn_desc &a)
{
    const int64_t K = (int64_t)M_cur + d.L, HD = (int64_t)d.n_head * d.d_head;
    txl_relattn_desc_init(&a, d.B, d.n_head, d.L, M_cur, d.d_head, TXL_BF16);
    const int64_t row = 3 * HD;
    a.q_stride[0] = K * row; a.q_stride[1] = d.d_head; a.q_stride[2] = row;
    std::memcpy(a.k_stride, a.q_stride, sizeof a.q_stride);
    std::memcpy(a.v_stride, a.q_stride, sizeof a.q_stride);
    a.o_stride[0] = (int64_t)d.L * HD; a.o_stride[1] = d.d_head; a.o_stride[2] = HD;
    a.r_stride[0] = d.d_head; a.r_stride[1] = HD;
    a.window = d.same_length;
    a.mem_valid = d.mem_valid;
}

txl_status check_layer(const txl_layer_desc *d, int M_cur)
{
    if (!d) return fail(TXL_ERR_INVALID_ARG, "desc is NULL");
    if (d->B < 1 || d->L < 1 || M_cur < 0 || d->d_model < 2 || d->n_head < 1 || d->d_head < 1 || d->d_inner < 1)
        return fail(TXL_ERR_INVALID_ARG, "need B, L, d_model, n_head, d_head, d_inner >= 1 and M_cur >= 0");
    const int64_t HD = (int64_t)d->n_head * d->d_head;
    if (d->d_model % 8 || HD % 8 || d->d_inner % 8)
        return fail(TXL_ERR_INVALID_ARG, "d_model, n_head*d_head and d_inner must be multiples of 8");
    if (d->d_model > txl::layer_norm_max_width())
        return fail(TXL_ERR_UNSUPPORTED, "d_model=%d exceeds %d", d->d_model, txl::layer_norm_max_width());
    if (d->clamp_len < 0 || d->same_length < 0)
        return fail(TXL_ERR_INVALID_ARG, "clamp_len and same_length must be >= 0");
    if (d->d_head != 32 && d->d_head != 64 && d->d_head != 128)
        return fail(TXL_ERR_UNSUPPORTED, "d_head=%d (bf16 attention supports 32, 64, 128)", d->d_head);
    const int64_t K = (int64_t)M_cur + d->L;
    if (K * 3 * HD > 0x7fffffffLL || (int64_t)d->B * d->L * d->d_inner > 0x7fffffffLL || K > (1 << 24))
        return fail(TXL_ERR_UNSUPPORTED, "sizes exceed 32-bit GEMM indexing");
    return TXL_OK;
}

struct Range {
    uintptr_t lo, hi;
};
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range rng(const void *p, size_t bytes)
{
    return {reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + bytes};
}

}  // namespace

// The context of txl_layer_fwd: one rocBLAS handle, made on `device`.
struct txl_context_s {
    int device;
    rocblas_handle blas;
};

extern "C" {

txl_status txl_context_create(txl_context *ctx)
{
    if (!ctx) return fail(TXL_ERR_INVALID_ARG, "ctx is NULL");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(TXL_ERR_HIP, "hipGetDevice failed");
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return fail(TXL_ERR_HIP, "rocblas_create_handle failed");
    txl_context c = new (std::nothrow) txl_context_s{dev, h};
    if (!c) {
        rocblas_destroy_handle(h);
        return fail(TXL_ERR_HIP, "out of host memory");
    }
    *ctx = c;
    return txl::set_error(TXL_OK, "");
}

txl_status txl_context_destroy(txl_context ctx)
{
    if (!ctx) return txl::set_error(TXL_OK, "");
    const rocblas_status bs = rocblas_destroy_handle(ctx->blas);
    delete ctx;
    if (bs != rocblas_status_success) return fail(TXL_ERR_HIP, "rocblas_destroy_handle failed");
    return txl::set_error(TXL_OK, "");
}

txl_status txl_layer_workspace_size(const txl_layer_desc *d, int M_cur, size_t *bytes)
{
    txl_status s = check_layer(d, M_cur);
    if (s != TXL_OK) return s;
    if (!bytes) return fail(TXL_ERR_INVALID_ARG, "bytes is NULL");
    txl_relattn_desc ad;
    attn_desc(*d, M_cur, ad);
    LayerWs w;
    if (!layer_ws(*d, M_cur, w, &ad)) return TXL_ERR_INVALID_ARG;
    *bytes = w.total;
    return txl::set_error(TXL_OK, "");
}

txl_status txl_layer_fwd(txl_context ctx, const txl_layer_desc *d, const txl_layer_weights *w, const void *h_in,
                         const void *mem, int M_cur, const float *u, const float *vb, void *h_out, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    if (!ctx) return fail(TXL_ERR_INVALID_ARG, "ctx is NULL (create one with txl_context_create)");
    txl_status s = check_layer(d, M_cur);
    if (s != TXL_OK) return s;
    if (!w || !w->W_qkv || !w->W_r || !w->W_o || !w->ln1_g || !w->ln1_b || !w->W1 || !w->W2 || !w->ln2_g ||
        !w->ln2_b)
        return fail(TXL_ERR_INVALID_ARG, "a required weight pointer is NULL");
    if (!h_in || !h_out || !u || !vb || (M_cur > 0 && !mem))
        return fail(TXL_ERR_INVALID_ARG, "a required tensor pointer is NULL");
    const void *mats[] = {w->W_qkv, w->W_r, w->W_o, w->W1, w->W2, h_in, h_out, mem};
    for (const void *p : mats)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u))
            return fail(TXL_ERR_INVALID_ARG, "matrices and activations must be 16-byte aligned");
    const float *vecs[] = {w->ln1_g, w->ln1_b, w->b1, w->b2, w->ln2_g, w->ln2_b};
    for (const float *p : vecs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u))
            return fail(TXL_ERR_INVALID_ARG, "LayerNorm and bias vectors must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(u) | reinterpret_cast<uintptr_t>(vb)) & 3u)
        return fail(TXL_ERR_INVALID_ARG, "u and vb must be 4-byte aligned");

    txl_relattn_desc ad;
    attn_desc(*d, M_cur, ad);
    LayerWs lw;
    if (!layer_ws(*d, M_cur, lw, &ad)) return fail(TXL_ERR_INVALID_ARG, "attention shape rejected: %s", txl_last_error());
    if (!workspace || workspace_bytes < lw.total)
        return fail(TXL_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", lw.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(TXL_ERR_WORKSPACE, "workspace must be 256-byte aligned");

    const int B = d->B, L = d->L, D = d->d_model, H = d->n_head, dh = d->d_head, DI = d->d_inner;
    const int HD = H * dh, K = M_cur + L;
    const size_t act = (size_t)B * L * D * 2;
    const Range out_r = rng(h_out, act);
    const Range ins[] = {rng(h_in, act), rng(mem, M_cur > 0 ? (size_t)B * M_cur * D * 2 : 0),
                         rng(w->W_qkv, (size_t)3 * HD * D * 2), rng(w->W_r, (size_t)HD * D * 2),
                         rng(w->W_o, (size_t)D * HD * 2), rng(w->W1, (size_t)DI * D * 2), rng(w->W2, (size_t)D * DI * 2),
                         rng(workspace, lw.total)};
    for (const Range &r : ins)
        if (r.hi > r.lo && overlaps(out_r, r)) return fail(TXL_ERR_ALIAS, "h_out overlaps an input, a weight or the workspace");
    const Range ws_r = rng(workspace, lw.total);
    for (int i = 0; i < 7; ++i)
        if (ins[i].hi > ins[i].lo && overlaps(ws_r, ins[i])) return fail(TXL_ERR_ALIAS, "the workspace overlaps an input");

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(TXL_ERR_HIP, "hipGetDevice failed");
    if (dev != ctx->device)
        return fail(TXL_ERR_INVALID_ARG, "ctx was created on device %d, the current device is %d", ctx->device, dev);
    rocblas_handle bh = ctx->blas;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (rocblas_set_stream(bh, st) != rocblas_status_success) return fail(TXL_ERR_HIP, "rocblas_set_stream failed");

    char *ws = static_cast<char *>(workspace);
    uint16_t *pe = reinterpret_cast<uint16_t *>(ws + lw.pe);
    uint16_t *rk = reinterpret_cast<uint16_t *>(ws + lw.r);
    uint16_t *qkv = reinterpret_cast<uint16_t *>(ws + lw.qkv);
    uint16_t *attn = reinterpret_cast<uint16_t *>(ws + lw.attn);
    float *a = reinterpret_cast<float *>(ws + lw.a);
    uint16_t *x = reinterpret_cast<uint16_t *>(ws + lw.x);
    float *f1 = reinterpret_cast<float *>(ws + lw.f1);
    uint16_t *f1b = reinterpret_cast<uint16_t *>(ws + lw.f1b);
    float *f2 = reinterpret_cast<float *>(ws + lw.f2);
    const float eps = d->ln_eps > 0.f ? d->ln_eps : 1e-5f;
    const uint16_t *Wqkv = static_cast<const uint16_t *>(w->W_qkv);

    hipError_t he;
    rocblas_status bs;
#define TXL_HIP(call)                                                                                 \
    if ((he = (call)) != hipSuccess) return fail(TXL_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(he))
#define TXL_BLAS(call)                                                                                \
    if ((bs = (call)) != rocblas_status_success) return fail(TXL_ERR_HIP, "%s failed: %s", #call, rocblas_status_to_string(bs))

    // r_k = pos W_r^T  [K][HD]
    TXL_HIP(txl::launch_pos_emb(pe, K, D, d->clamp_len, st));
    TXL_BLAS(gemm_xwt(bh, HD, K, D, w->W_r, D, pe, D, 0, rk, rocblas_datatype_bf16_r, HD, 0, 1));
    // [q; k; v] of the current rows, [k; v] of the memory rows, into qkv[b][row][3 HD]
    TXL_BLAS(gemm_xwt(bh, 3 * HD, L, D, Wqkv, D, h_in, D, (int64_t)L * D, qkv + (size_t)M_cur * 3 * HD,
                      rocblas_datatype_bf16_r, 3 * HD, (int64_t)K * 3 * HD, B));
    if (M_cur > 0)
        TXL_BLAS(gemm_xwt(bh, 2 * HD, M_cur, D, Wqkv + (size_t)HD * D, D, mem, D, (int64_t)M_cur * D, qkv + HD,
                          rocblas_datatype_bf16_r, 3 * HD, (int64_t)K * 3 * HD, B));
    // relative attention over strided views, heads merged into attn [B][L][HD]
    {
        txl_status as = txl_relattn_fwd(&ad, qkv + (size_t)M_cur * 3 * HD, qkv + HD, qkv + 2 * HD, rk, u, vb, attn,
                                        nullptr, lw.attn_ws ? ws + lw.attn_ws : nullptr,
                                        lw.total - lw.attn_ws, stream);
        if (as != TXL_OK) return as;
    }
    // x = LN1(h + attn W_o^T)
    TXL_BLAS(gemm_xwt(bh, D, B * L, HD, w->W_o, HD, attn, HD, 0, a, rocblas_datatype_f32_r, D, 0, 1));
    TXL_HIP(txl::launch_add_layer_norm(static_cast<const uint16_t *>(h_in), a, nullptr, w->ln1_g, w->ln1_b, x,
                                       (int64_t)B * L, D, eps, st));
    // out = LN2(x + W2 relu(W1 x + b1) + b2)
    TXL_BLAS(gemm_xwt(bh, DI, B * L, D, w->W1, D, x, D, 0, f1, rocblas_datatype_f32_r, DI, 0, 1));
    TXL_HIP(txl::launch_bias_relu(f1, w->b1, f1b, (int64_t)B * L, DI, st));
    TXL_BLAS(gemm_xwt(bh, D, B * L, DI, w->W2, DI, f1b, DI, 0, f2, rocblas_datatype_f32_r, D, 0, 1));
    TXL_HIP(txl::launch_add_layer_norm(x, f2, w->b2, w->ln2_g, w->ln2_b, static_cast<uint16_t *>(h_out),
                                       (int64_t)B * L, D, eps, st));
#undef TXL_HIP
#undef TXL_BLAS
    return txl::set_error(TXL_OK, "");
}

}  // extern "C"
