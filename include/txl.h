/*
 * txl.h -- C ABI of the MI355X (gfx950) Transformer-XL relative-attention
 * library, libtxl.so.
 *
 * Sources (web pages; cited by title and section / class):
 *   [SRC] "Transformer-XL模型 核心源码阅读笔记" (source-reading notes,
 *         blog.csdn.net/ACM_hades/article/details/104742528)
 *   [XL]  "Transformer-XL" (textbook notes, zty624.github.io, DL notebooks,
 *         ch4_transformer/xl)
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or retains them.  Work is enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL = the null stream) and is
 *     asynchronous: a call returning TXL_OK has validated its arguments and
 *     launched; faults inside kernels surface at the caller's next
 *     synchronisation of that stream.
 *   - Every argument check runs on the host before any launch.  A call that
 *     returns an error has launched nothing and written nothing.
 *   - txl_last_error() returns a thread-local message describing the last
 *     failure on the calling thread.
 *   - Strides are in ELEMENTS.  The innermost (feature) axis is always
 *     contiguous.  Base pointers and every non-innermost stride must keep
 *     16-byte alignment of each row.
 *   - Floating-point tensors are TXL_BF16 (bfloat16) or TXL_F32.  Accumulation
 *     is fp32 in every kernel; u, vb and lse are always fp32.
 *   - Identical inputs give bitwise-identical outputs (no atomics, fixed
 *     reduction orders).
 */
#ifndef TXL_H
#define TXL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TXL_OK = 0,
    TXL_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad stride/alignment        */
    TXL_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. an unsupported dh)   */
    TXL_ERR_ALIAS = 3,       /* an output overlaps an input that must stay intact    */
    TXL_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned           */
    TXL_ERR_HIP = 5          /* a HIP runtime call failed; see txl_last_error()      */
} txl_status;

typedef enum { TXL_F32 = 0, TXL_BF16 = 1 } txl_dtype;

/* Library version string, e.g. "0.1.0". */
const char *txl_version(void);
/* Static description of a status code. */
const char *txl_status_string(txl_status s);
/* Thread-local message of the last failing call on this thread ("" if none). */
const char *txl_last_error(void);

/* ------------------------------------------------------------------------ */
/* Relative attention forward                                               */
/* ------------------------------------------------------------------------ */

/* Shapes: B batch rows, H heads, L queries (current segment), M memory rows,
 * K = M + L keys, dh = head width.
 *   q     [B][H][L][dh]   strides q_stride  = {b, h, row}
 *   k, v  [B][H][K][dh]   strides k_stride, v_stride
 *   out   [B][H][L][dh]   strides o_stride
 *   r_k   [H][K][dh]      strides r_stride  = {h, row}; row c holds the
 *                         projected encoding of relative position K-1-c
 *                         ([SRC] MemTransformerLM._forward orders positions
 *                         K-1 .. 0)
 *   u, vb [H][dh] fp32 contiguous: r_w_bias and r_r_bias
 *   lse   [B][H][L] fp32 contiguous, optional (NULL = not written)
 * q, k, v, r_k and out all have `dtype`. */
typedef struct {
    int B, H, L, M, dh;
    int dtype;            /* txl_dtype */
    float scale;          /* <= 0 selects 1/sqrt(dh) ([SRC] RelMultiHeadAttn) */
    int splits;           /* key-range splits: 0 = automatic, 1 = none, n > 1 = n */
    int64_t q_stride[3];
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
    int64_t r_stride[2];
    /* Optional lower bounds on the visible keys (both off after
     * txl_relattn_desc_init):
     *   window > 0: query i sees only keys j >= i + M + 1 - window, the
     *     `window` positions ending at itself.  With window = mem_len this is
     *     the same_length mask of [SRC] MemTransformerLM._forward
     *     (triu(1 + mlen) + tril(-mask_shift_len)).  window < 0 is invalid.
     *   mem_valid != NULL: DEVICE array [B] of ints; batch row b sees only the
     *     newest mem_valid[b] memory rows, i.e. keys j >= M - mem_valid[b]
     *     (a per-row memory reset at a document boundary, [XL] "Batched
     *     Streams"; the oldest rows hold another document).  Values are
     *     clamped to [0, M] on the device. */
    const int *mem_valid;
    int window;
} txl_relattn_desc;

/* Fills `desc` for densely packed tensors of the shapes above (splits = 0,
 * scale = 1/sqrt(dh)).  Returns TXL_ERR_INVALID_ARG for a NULL desc. */
txl_status txl_relattn_desc_init(txl_relattn_desc *desc, int B, int H, int L, int M, int dh,
                                 txl_dtype dtype);

/* Bytes of device workspace txl_relattn_fwd needs for `desc` (0 when the
 * key range is not split).  *bytes is written on success. */
txl_status txl_relattn_workspace_size(const txl_relattn_desc *desc, size_t *bytes);

/* Segment-recurrent relative-position attention, forward.
 *
 * For each (b, h) and query i in [0, L), with keys j in [0, K) at positions
 * j - M ([XL] "Batched Tensor Contract"; "Causal Mask With Memory"):
 *   visible(i, j)  <=>  lo(b, i) <= j <= i + M   (causal current segment)
 *   lo(b, i) = max(M - mem_valid[b] (if given), i + M + 1 - window (if > 0), 0)
 *   s_ij = scale * ( (q_i + u) . k_j  +  (q_i + vb) . r_k[L-1-i+j] )
 *   out_i = sum_j softmax_j(s_ij) v_j          over visible j
 *   lse_i = log sum_j exp(s_ij)                over visible j
 * This is [SRC] RelPartialLearnableMultiHeadAttn.forward from the score
 * einsums to attn_vec (AC + rel_shift(BD), scale, masked_fill(-inf),
 * softmax over keys, P.V) with the rel_shift done as direct distance
 * indexing; [XL] "Relative Positional Encoding" gives the four-term form.
 *
 * dtype TXL_BF16: dh in {32, 64, 128}; TXL_F32: dh in {16, 32, 64}.
 * L >= 1, M >= 0, B, H >= 1.  Workspace: at least
 * txl_relattn_workspace_size() bytes, 256-byte aligned (may be NULL when
 * that size is 0).  `out` must not overlap q, k, v or r_k (TXL_ERR_ALIAS). */
txl_status txl_relattn_fwd(const txl_relattn_desc *desc, const void *q, const void *k, const void *v,
                           const void *r_k, const float *u, const float *vb, void *out, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/* txl_relattn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results (bitwise), with no workspace
 * argument.  When the plan splits the key range, the partial outputs go to
 * the library's static device scratch of 32 MiB (TXL_NOALLOC_SCRATCH_BYTES),
 * one per device, held until the process ends; its address is looked up on
 * the first call on each device.  This entry point calls no hipMalloc,
 * hipFree or allocating library routine.  A call whose split workspace
 * (txl_relattn_workspace_size) exceeds the scratch returns TXL_ERR_WORKSPACE
 * and launches nothing.  All calls on one device share that scratch: calls
 * that may overlap in time on one device (different streams, or threads
 * without ordering) race and must be serialised by the caller. */
#define TXL_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
txl_status txl_relattn_fwd_noalloc(const txl_relattn_desc *desc, const void *q, const void *k, const void *v,
                                   const void *r_k, const float *u, const float *vb, void *out, float *lse,
                                   void *stream);

/* ------------------------------------------------------------------------ */
/* Relative attention backward                                              */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace txl_relattn_bwd needs for `desc` (always > 0:
 * the prepared query operands, row constants and one bf16 [B][H][L][K']
 * buffer of score gradients, K' = K + 78 rounded up to 64).  *bytes is written on
 * success; the same errors as txl_relattn_bwd for an unsupported desc. */
txl_status txl_relattn_bwd_workspace_size(const txl_relattn_desc *desc, size_t *bytes);

/* Gradients of txl_relattn_fwd with respect to all of its inputs.
 *
 * The pages define the forward only ([SRC] RelPartialLearnableMultiHeadAttn
 * .forward); these are its derivatives by the chain rule.  With the visible
 * set, s_ij and p_ij = softmax_j(s_ij) of txl_relattn_fwd, the upstream
 * gradient dout_i of out_i, dP_ij = dout_i . v_j and
 * dS_ij = p_ij (dP_ij - sum_k p_ik dP_ik):
 *   dq_i = scale sum_j dS_ij (k_j + r_k[L-1-i+j])
 *   dk_j = scale sum_i dS_ij (q_i + u)          dv_j = sum_i p_ij dout_i
 *   dr_k[c] = scale sum_{b, i, j: L-1-i+j = c} dS_ij (q_i + vb)
 *   du = scale sum_{b,i,j} dS_ij k_j           dvb = scale sum_{b,i,j} dS_ij r_k[L-1-i+j]
 * Masked pairs carry no gradient.  Memory keys (j < M) get dk and dv like the
 * others: [XL] "Why Stop Gradient" detaches the cached memory states of a
 * layer stack, which is the caller's business (it drops these rows when it
 * propagates to the memory, and keeps them for the projection weights).
 *
 * Inputs: desc, q, k, v, r_k, u, vb exactly as passed to txl_relattn_fwd
 * (same masks: window, mem_valid); out and lse (required) as it returned
 * them; dout [B][H][L][dh] with desc->o_stride.  p is recomputed from lse.
 * Outputs (caller-owned, fully overwritten):
 *   dq [B][H][L][dh] with desc->q_stride, dk and dv [B][H][K][dh] with
 *   desc->k_stride and desc->v_stride, all of `dtype`;
 *   dr [H][K][dh] fp32 contiguous, du and dvb [H][dh] fp32 contiguous.
 * Supported: dtype TXL_BF16 with dh = 64 (else TXL_ERR_UNSUPPORTED), one
 * head's rows and one head's score gradients (L x K' bf16) each within
 * 2 GiB.  Workspace: txl_relattn_bwd_workspace_size()
 * bytes, 256-byte aligned.  No output may overlap an input, another output or
 * the workspace (TXL_ERR_ALIAS).  Results are bitwise reproducible (fixed
 * summation orders, no atomics).  desc->splits is ignored. */
txl_status txl_relattn_bwd(const txl_relattn_desc *desc, const void *q, const void *k, const void *v,
                           const void *r_k, const float *u, const float *vb, const void *out, const float *lse,
                           const void *dout, void *dq, void *dk, void *dv, float *dr, float *du, float *dvb,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Memory update (Tail_M)                                                   */
/* ------------------------------------------------------------------------ */

/* new_mem = cat([mem; h], seq)[beg:end] with end = M_cur + max(0, L - ext_len)
 * and beg = max(0, end - mem_len), per batch row ([SRC]
 * MemTransformerLM._update_mems; with ext_len = 0 this is [XL] Tail_M:
 * the last mem_len rows of [mem; h]).  A bit-exact copy.
 *   mem     [B][M_cur][d]  batch stride mem_bs (rows contiguous, row = d)
 *   h       [B][L][d]      batch stride h_bs
 *   new_mem [B][M_new][d]  batch stride new_bs, M_new = end - beg
 * `mem` may be NULL iff M_cur == 0.  new_mem must not overlap mem or h
 * (TXL_ERR_ALIAS): the update is out of place, so callers double-buffer.
 * *M_new (host pointer, may be NULL) receives end - beg.
 * dtype: TXL_BF16 or TXL_F32; d * element size must be a multiple of 16 bytes. */
txl_status txl_mem_update(const void *mem, int M_cur, const void *h, int L, void *new_mem, int mem_len,
                          int ext_len, int B, int d, int dtype, int64_t mem_bs, int64_t h_bs,
                          int64_t new_bs, int *M_new, void *stream);

/* The length M_new = end - beg of the update above for these sizes, without
 * launching anything, so that a caller can size new_mem before the call.
 * Returns TXL_ERR_INVALID_ARG for a negative size or a NULL M_new. */
txl_status txl_mem_update_len(int M_cur, int L, int mem_len, int ext_len, int *M_new);

/* The same update for n_buf independent buffers in ONE launch (the N+1
 * per-layer memories of a layer stack, [XL] "Segment-Level Recurrence").
 * mem, h and new_mem are HOST arrays of n_buf device pointers; all buffers
 * share the scalar arguments.  1 <= n_buf <= 64. */
txl_status txl_mem_update_batched(int n_buf, const void *const *mem, int M_cur, const void *const *h,
                                  int L, void *const *new_mem, int mem_len, int ext_len, int B, int d,
                                  int dtype, int64_t mem_bs, int64_t h_bs, int64_t new_bs, int *M_new,
                                  void *stream);

/* txl_relattn_fwd and one txl_mem_update in a single call: the attention of
 * a layer's segment and the Tail_M update of the same layer's memory ([XL]
 * "Segment-Level Recurrence": the next segment's memory is the last mem_len
 * rows of [mem; h]).  The two results are exactly those of the two calls
 * (the copy is bit-exact and independent of the attention); the arguments
 * and every check are theirs: desc .. workspace_bytes as txl_relattn_fwd,
 * mem .. M_new as txl_mem_update (B_m batch rows of d_model elements of
 * dtype_m).  Because the two run concurrently, new_mem must not overlap q,
 * k, v, r_k, u, vb, desc->mem_valid, out, lse or the workspace, and mem and
 * h must not overlap out, lse or the workspace (TXL_ERR_ALIAS).  *M_new is
 * written only when the call succeeds.  With the bf16
 * throughput kernel (bf16, dh = 64, not the short-segment streaming case)
 * the attention kernel's own waves do the copy, 1 KB chunks spread over its
 * key loop, so the copy rides on HBM bandwidth the attention leaves unused;
 * otherwise the call launches the attention and then the copy kernel on
 * `stream`. */
txl_status txl_relattn_fwd_mem_update(const txl_relattn_desc *desc, const void *q, const void *k, const void *v,
                                      const void *r_k, const float *u, const float *vb, void *out, float *lse,
                                      void *workspace, size_t workspace_bytes, const void *mem, int M_cur,
                                      const void *h, int L_h, void *new_mem, int mem_len, int ext_len, int B_m,
                                      int d_model, int dtype_m, int64_t mem_bs, int64_t h_bs, int64_t new_bs,
                                      int *M_new, void *stream);

/* ------------------------------------------------------------------------ */
/* Decoder layer (relative attention + post-LayerNorm position-wise FF)     */
/* ------------------------------------------------------------------------ */

/* Library context of the decoder layer: the rocBLAS handle its projections
 * run on, bound to the device that is current when the context is created.
 * Creating one allocates (rocBLAS reserves device memory for its handle), so
 * callers create it once, outside timed or captured regions, and destroy it
 * when done; the library keeps no hidden per-thread state.  A context may be
 * used by one thread at a time (txl_layer_fwd sets its stream per call). */
typedef struct txl_context_s *txl_context;

/* Creates a context on the current device; *ctx receives it.  TXL_ERR_HIP if
 * rocBLAS cannot create its handle. */
txl_status txl_context_create(txl_context *ctx);
/* Destroys a context made by txl_context_create (NULL is a no-op).  Work
 * already enqueued with it is not waited for; the caller synchronises first. */
txl_status txl_context_destroy(txl_context ctx);

/* One RelPartialLearnableDecoderLayer forward with pre_lnorm = False and
 * identity dropout ([SRC] RelPartialLearnableMultiHeadAttn.forward,
 * PositionwiseFF.forward, MemTransformerLM._forward), for B batch rows of a
 * segment of L tokens with M_cur rows of memory (K = M_cur + L):
 *   pos    = sinusoid of positions K-1 .. 0      ([SRC] PositionalEmbedding:
 *            sin in the first d/2 columns, cos in the rest, 10000^(-2t/d))
 *   r_k    = pos W_r^T                            [K][H*dh]
 *   q      = h W_q^T,  [k; v] = [mem; h] [W_k; W_v]^T   (W_qkv = [W_q; W_k; W_v])
 *   attn   = txl_relattn_fwd over the H heads (rectangular mem + causal mask)
 *   x      = LN1(h + attn W_o^T)
 *   out    = LN2(x + W2 relu(W1 x + b1) + b2)
 * LayerNorm uses the biased variance and eps ([SRC] nn.LayerNorm(d_model)).
 *
 * Tensors (device, caller-owned, dense, 16-byte aligned):
 *   h_in, h_out [B][L][d] bf16;  mem [B][M_cur][d] bf16 (NULL iff M_cur == 0)
 *   weights: bf16 matrices in nn.Linear [out][in] layout, fp32 vectors.
 *   u, vb [H][dh] fp32 (r_w_bias, r_r_bias).
 * Sizes: d, H*dh and d_inner multiples of 8; d even and <= 4096; dh in
 * {32, 64, 128}.  h_out must not overlap any input, weight or the workspace
 * (TXL_ERR_ALIAS).  Workspace: txl_layer_workspace_size() bytes, 256-byte
 * aligned.  Intermediates are rounded to bf16 where they feed a GEMM or the
 * attention kernel and kept in fp32 where they feed a LayerNorm. */
typedef struct {
    int B, L, d_model, n_head, d_head, d_inner;
    float ln_eps;      /* <= 0 selects 1e-5 */
    /* Options of [SRC] MemTransformerLM (all 0 / NULL = off):
     *   clamp_len > 0: position values above clamp_len use the encoding of
     *     clamp_len ([SRC] _forward: pos_seq.clamp_(max=clamp_len));
     *   same_length > 0: the same_length mask with mem_len = same_length, i.e.
     *     query i sees keys j >= i + M_cur + 1 - same_length (txl_relattn_desc
     *     window);
     *   mem_valid: DEVICE [B] ints, row b keeps only its newest mem_valid[b]
     *     memory rows (per-row reset, txl_relattn_desc mem_valid). */
    int clamp_len;
    int same_length;
    const int *mem_valid;
} txl_layer_desc;

typedef struct {
    const void *W_qkv;                  /* [3*H*dh][d]  bf16 */
    const void *W_r;                    /* [H*dh][d]    bf16 */
    const void *W_o;                    /* [d][H*dh]    bf16 */
    const float *ln1_g, *ln1_b;         /* [d]          fp32 */
    const void *W1;                     /* [d_inner][d] bf16 */
    const float *b1;                    /* [d_inner]    fp32 (NULL = zero) */
    const void *W2;                     /* [d][d_inner] bf16 */
    const float *b2;                    /* [d]          fp32 (NULL = zero) */
    const float *ln2_g, *ln2_b;         /* [d]          fp32 */
} txl_layer_weights;

/* Workspace bytes of txl_layer_fwd for `desc` and M_cur memory rows. */
txl_status txl_layer_workspace_size(const txl_layer_desc *desc, int M_cur, size_t *bytes);

/* `ctx` (from txl_context_create, on the device of the tensors) supplies the
 * rocBLAS handle; NULL returns TXL_ERR_INVALID_ARG. */
txl_status txl_layer_fwd(txl_context ctx, const txl_layer_desc *desc, const txl_layer_weights *w,
                         const void *h_in, const void *mem, int M_cur, const float *u, const float *vb,
                         void *h_out, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TXL_H */
