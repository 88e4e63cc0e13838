/*
 * fa_fwd.h -- C ABI of the attention forward of the MI355X (gfx950) library:
 * the output O and the per-row log-sum-exp that the backward (fa_bwd.h)
 * consumes, computed without forming the Sq x Sk score matrix (the online
 * softmax of the Triton FA2 teaching page's forward kernel: running maximum,
 * rescaled partial output and sum, one division at the end).
 *
 * One kernel is enqueued on the caller's stream: one workgroup per 256 query
 * rows of one head streams the visible 64-key tiles of its KV head.
 *
 * Conventions are those of fa_bwd.h: device pointers, strides in elements,
 * caller-owned buffers, no allocation, asynchronous on `stream` (a
 * hipStream_t as void*, NULL = default stream), host-only validation before
 * any launch with the status codes of fa_bwd.h and the reason in
 * fa_bwd_last_error().
 */
#ifndef FA_FWD_H
#define FA_FWD_H

#include "fa_bwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Arguments of one forward call.  Shapes, layouts, strides, GQA head mapping,
 * the causal rule and the local window, packed variable-length inputs and
 * the LSE layout are
 * exactly those of fa_bwd_args (fa_bwd.h), so the outputs of a forward call
 * are valid `out` / `lse` inputs of a backward call on the same q, k, v:
 *   dense : q, out (batch, seqlen_q, num_heads, head_dim); k, v (batch,
 *           seqlen_k, num_heads_k, head_dim); lse (batch, num_heads,
 *           seqlen_q) fp32;
 *   packed: q, out (total_q, num_heads, head_dim); k, v (total_k,
 *           num_heads_k, head_dim); lse (batch, num_heads, seqlen_q) with
 *           batch = number of sequences and seqlen_q the maximum length.
 * Every stride but the head_dim one a multiple of 8 elements, every base
 * pointer 16-byte aligned (lse 4-byte aligned), head_dim a multiple of 8 and
 * <= 256 (padded tile widths 64, 96, 128, 192, 256) and the row strides of k and v below 2^24 elements (a 64-key tile
 * is addressed with 32-bit offsets) -- FA_ERR_UNSUPPORTED otherwise -- and
 * dtype bf16 or fp16 (inputs and out share it).
 *
 * Results:
 *   - out = softmax(softmax_scale * Q K^T + mask) V in `dtype` over the valid
 *     rows and the first head_dim columns (other memory is not written);
 *   - lse = the natural-log log-sum-exp of the scaled scores of each row;
 *   - a row with no visible key (causal with len_q > len_k, or len_k = 0)
 *     gets out = 0 and lse = -inf.
 * out and lse must not alias q, k, v or each other.  Repeated calls give
 * bit-identical results (fixed-order sums).
 */
typedef struct fa_fwd_args {
    int32_t dtype;                 /* fa_dtype: FA_DTYPE_BF16 or FA_DTYPE_F16 */
    int32_t batch;                 /* dense: B; packed: number of sequences */
    int32_t seqlen_q, seqlen_k;    /* dense: Sq, Sk; packed: maximum lengths */
    int32_t num_heads, num_heads_k, head_dim;
    const int32_t *cu_seqlens_q;   /* device; NULL for dense */
    const int32_t *cu_seqlens_k;   /* device; NULL for dense */
    int64_t total_q, total_k;      /* packed: cu_seqlens_q/k[batch] (host copies) */

    const void *q, *k, *v;         /* inputs, 16-bit elements of `dtype` */
    void *out;                     /* output, elements of `dtype` */
    float *lse;                    /* fp32 output, natural log */

    int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
    int64_t lse_stride[2];

    float softmax_scale;
    int32_t causal;                /* 0 or 1 */
    int32_t local_window;          /* local window as in fa_bwd_args */
    int32_t window_size_left;
    int32_t window_size_right;
    float softcap;                 /* soft-capped scores as in fa_bwd_args; 0: none */
    float dropout_p;               /* dropout as in fa_bwd_args; 0: none */
    uint64_t philox_seed;
    uint64_t philox_offset;
    /* Optional (dropout_p > 0): device buffer of dropout_keep_out_bytes >=
     * fa_fwd_keep_bytes() bytes, 4-byte aligned (FA_ERR_INVALID_ARG
     * otherwise), that receives the keep bits the call draws, for the
     * backward's dropout_keep: uint32[keep_words][num_heads][rows] with
     * keep_words = 2 * ceil(seqlen_k / 64) (the maximum length when packed),
     * rows and row index as in fa_bwd.h's workspace layout, bit x of word w
     * of a row the keep bit of key 32 w + x of its sequence.  Only the words
     * of the 64-key tiles that a 256-row query tile visits are written (128
     * rows above head_dim 128); the backward reads no others and uses a bit
     * only where its pair is visible.  The buffer holds one bit per (row,
     * key) pair of every head: it grows with seqlen_q * seqlen_k.  NULL:
     * nothing is written.  Ignored when dropout_p = 0. */
    uint32_t *dropout_keep_out;
    size_t dropout_keep_out_bytes;
} fa_fwd_args;

/* Bytes of the keep words of a dropout call (see dropout_keep_out): 0 when
 * dropout_p = 0 or the arguments are otherwise invalid. */
size_t fa_fwd_keep_bytes(const fa_fwd_args *args);

/* FA_OK if fa_fwd would accept `args`; otherwise the error it would return. */
fa_status fa_fwd_validate(const fa_fwd_args *args);

/* Enqueue the forward on `stream`.  Returns FA_OK or an fa_status code. */
fa_status fa_fwd(const fa_fwd_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_FWD_H */
