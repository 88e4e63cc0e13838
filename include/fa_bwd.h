/*
 * fa_bwd.h -- C ABI of the MI355X (gfx950) FlashAttention-2 backward library.
 *
 * Given Q, K, V, the forward output O, the upstream gradient dO and the
 * forward's per-row log-sum-exp, the library computes dQ, dK and dV of
 *     O = softmax(scale * Q K^T + causal mask) V
 * without ever forming the Sq x Sk score matrix: it recomputes each score tile
 * from Q, K and the saved LSE (sm90 backward kernel page, mma_one_m_block:
 * the scores, P = exp(S - LSE), dP = dO V^T, dS = P (dP - rowsum(dO * O)),
 * then dV += P^T dO, dQ = dS K, dK += dS^T Q).
 *
 * Work is enqueued on the caller's HIP stream as two or three kernels:
 *   - preprocess : rowsum(dO * O) per query row and head (the softmax_d /
 *                  dsoftmax_sum buffer of the backward call-trace page,
 *                  set_params_dgrad) and the LSE converted to base 2;
 *   - main       : one workgroup per 128-key tile of one KV head; it keeps
 *                  the K/V tile and its dK/dV accumulators on chip, loops
 *                  over every query head of the KV head's group (the GQA
 *                  reduction of the GQA/MQA page's backward section happens
 *                  in registers) and over the visible 64-row query tiles;
 *   - dQ, in one of two ways (fa_bwd_args.dq_accumulate):
 *      0 (default) dq  : one workgroup per 256 query rows (128 at head_dim
 *                        > 128) of one head loops
 *                        over the visible key tiles and forms dQ = scale *
 *                        dS K directly (dS recomputed; no atomics; the way
 *                        the Triton FA2 teaching page's dQ kernel works).
 *                        It also forms the preprocess's two row vectors, so
 *                        the sequence is dq, then main;
 *      1 accumulate    : the main kernel adds each tile's dQ partial into an
 *                        fp32 accumulator (hardware atomics, or a fixed
 *                        order when deterministic = 1), which the preprocess
 *                        clears, and dq_convert forms dQ = scale * acc
 *                        rounded to the element type (head_dim <= 128
 *                        only; above, FA_ERR_UNSUPPORTED)
 *                        (the dq_accum buffer and its reduction step on the
 *                        backward call-trace page); the sequence is
 *                        preprocess, main, dq_convert.
 *   On MI355X the fp32 atomic rate of the L2 bounds mode 1 at large sizes;
 *   mode 0 does three extra products per tile pair instead and is faster.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers; all strides are in ELEMENTS.
 *   - The caller owns every buffer, the workspace included.  The library
 *     allocates nothing and keeps no state apart from a thread-local error
 *     string.  Inputs are never written.
 *   - Calls return as soon as the work is enqueued (asynchronous, like the
 *     current-stream launch on the backward call-trace page).  `stream` is a
 *     hipStream_t passed as void*; NULL means the default stream.
 *   - Validation happens entirely on the host before any launch: on error
 *     nothing is enqueued, the status code says which class of error, and
 *     fa_bwd_last_error() says why.
 *   - Device-side contents (cu_seqlens values) cannot be validated on the
 *     host; the caller guarantees them (see fa_bwd_args).
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_BWD_ABI_VERSION 10

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1, /* null pointer, bad size, H % Hk != 0, bad stride */
    FA_ERR_UNSUPPORTED = 2, /* dtype other than bf16 / fp16, head_dim > 256 or not a multiple of 8 */
    FA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than fa_bwd_workspace_size() */
    FA_ERR_HIP = 4          /* a HIP launch or attribute call failed */
} fa_status;

typedef enum {
    FA_DTYPE_BF16 = 0,
    FA_DTYPE_F16 = 1
} fa_dtype;

/*
 * Arguments of one backward call.  The field order follows the backward
 * call-trace page's mha_bwd / _flash_attn_backward argument list:
 * (dout, q, k, v, out, softmax_lse, dq, dk, dv, softmax_scale, causal,
 *  cu_seqlens_q/k, deterministic).
 *
 * Shapes and layouts (bshd = batch, seq, head, dim), as on the backward
 * call-trace page's mha_bwd:
 *   dense  (cu_seqlens_q == cu_seqlens_k == NULL):
 *     q, out, dout, dq : (batch, seqlen_q, num_heads,   head_dim)
 *     k, v, dk, dv     : (batch, seqlen_k, num_heads_k, head_dim)
 *     lse              : (batch, num_heads, seqlen_q) fp32
 *   packed variable length (both cu_seqlens given; Triton FA2 teaching page,
 *   flash_attn_varlen_func and the backward kernels' varlen branch):
 *     q, out, dout, dq : (total_q, num_heads,   head_dim)
 *     k, v, dk, dv     : (total_k, num_heads_k, head_dim)
 *     lse              : (batch, num_heads, seqlen_q) fp32, where batch is the
 *                        number of sequences and seqlen_q the maximum query
 *                        length; sequence s uses lse[s, h, 0 : len_q(s)]
 *     cu_seqlens_q/k   : device int32[batch + 1], cu[0] = 0, non-decreasing,
 *                        cu_seqlens_q[batch] == total_q (and k likewise);
 *                        every len_q(s) <= seqlen_q and len_k(s) <= seqlen_k.
 * Strides: x_stride[0] = batch stride (ignored for packed inputs),
 *          x_stride[1] = row (token) stride, x_stride[2] = head stride;
 *          the head_dim stride must be 1.  All three must be multiples of 8
 *          elements and every base pointer 16-byte aligned (128-bit rows, as
 *          the sm90 backward page's __call__ requires of its strides).
 *          The row strides of q and dout must lie in [head_dim, 2^24):
 *          rows may not overlap (FA_ERR_INVALID_ARG) and a 64-row query
 *          tile must be addressable with 32-bit offsets (FA_ERR_UNSUPPORTED);
 *          the row strides of k and v must be below 2^24 for the same
 *          reason (FA_ERR_UNSUPPORTED).
 *          lse_stride[0] = batch/sequence stride, lse_stride[1] = head stride,
 *          row stride 1.
 *
 * Semantics:
 *   - Scores are S = softmax_scale * Q K^T.  Query head h reads KV head
 *     h / (num_heads / num_heads_k) (GQA/MQA page, KV head mapping).
 *   - causal = 1 masks key j for query i unless j <= i + len_k - len_q
 *     (bottom-right aligned, GQA/MQA page, causal block bound).
 *   - Local (sliding-window) attention, mha_bwd's window_size_left / _right
 *     on the backward call-trace page, with local_window = 1 (0 leaves the
 *     sizes unread, so a zero-filled struct has no window): key j is
 *     visible to query i only if
 *     i + len_k - len_q - window_size_left <= j (when window_size_left >= 0)
 *     and j <= i + len_k - len_q + window_size_right (when
 *     window_size_right >= 0); negative sizes leave that side unbounded.
 *     causal = 1 is the right size 0 (a positive right size with causal = 1
 *     is FA_ERR_INVALID_ARG).  Sizes above 2^29 act as 2^29 (which reaches
 *     every key: seqlen_q and seqlen_k above 2^29 are FA_ERR_UNSUPPORTED).
 *   - softcap = c > 0 (mha_bwd's softcap on the backward call-trace page,
 *     read as the usual logit soft-capping): every scaled score x =
 *     softmax_scale * q.k becomes c * tanh(x / c) before the softmax, and lse
 *     must be the forward's log-sum-exp of those capped scores; the gradients
 *     pass the cap by the chain rule (factor 1 - tanh^2).  0 switches it off;
 *     a negative or non-finite value is FA_ERR_INVALID_ARG.
 *   - dropout_p = p > 0 (mha_bwd's p_dropout and rng_state, the backward
 *     call-trace page; the keep test of the Triton FA2 teaching page's
 *     dropout_mask, read so that kept values scaled by 1 / (1 - p) keep the
 *     expectation): element (i, j) of query head h of sequence b is kept iff
 *     word j % 4 of Philox4x32-10 (Salmon et al., SC 2011) at counter
 *     (j / 4, i, b * num_heads + h, philox_offset mod 2^32) with key
 *     (philox_seed mod 2^32, (philox_seed / 2^32) xor (philox_offset /
 *     2^32)) is >= floor(p * 2^32); i, j are the sequence-local row and key.
 *     The forward's O is sum_j P_ij Z_ij / (1 - p) V_j (its lse ignores
 *     dropout); the backward must be called with the forward's p, seed and
 *     offset.  p outside [0, 1) or non-finite is FA_ERR_INVALID_ARG.  Rows that see no key behave as under the
 *     causal rule (dq = 0, and they add nothing to dk / dv).
 *   - lse is the NATURAL-log log-sum-exp of the scaled scores of each row,
 *     -inf for a row with no visible key (its dQ is then 0).
 *   - dq, dk, dv are fully overwritten over their valid rows and the first
 *     head_dim columns; dk/dv of keys no query can see are written as 0.
 *     They must not alias any input or the workspace.
 *   - head_dim padding: head_dim must be a multiple of 8 and <= 256; kernels
 *     run at a padded tile width of 64, 96, 128, 192 or 256 with zero-filled
 *     loads and masked stores (above 128 the key-tile kernel takes 64 keys
 *     per workgroup, two waves per 32 keys splitting the query rows of S
 *     and dP and the head dim of dK/dV) (sm90 backward page, __init__: head
 *     dim rounded up to
 *     the tile multiple; backward call-trace page, dout padding step).
 *   - Reproducibility: with dq_accumulate = 0 every output is a fixed-order
 *     sum, so repeated calls give bit-identical dq, dk, dv whatever
 *     `deterministic` says.  With dq_accumulate = 1, deterministic = 1 adds
 *     the dQ partials in a fixed order (per query tile, in descending
 *     key-tile order) and is bit-reproducible too; deterministic = 0 uses
 *     unordered fp32 atomics, so dq may differ in the last bits between
 *     calls (dk and dv never do).
 *   - Empty inputs: batch == 0 enqueues nothing.  A sequence with no query
 *     rows gets dk = dv = 0 for its keys; one with no keys gets dq = 0.
 *     Pointers of tensors with no elements may be NULL.
 */
typedef struct fa_bwd_args {
    int32_t dtype;                 /* fa_dtype: FA_DTYPE_BF16 or FA_DTYPE_F16 */
    int32_t batch;                 /* dense: B; packed: number of sequences */
    int32_t seqlen_q, seqlen_k;    /* dense: Sq, Sk; packed: maximum lengths */
    int32_t num_heads, num_heads_k, head_dim;
    const int32_t *cu_seqlens_q;   /* device; NULL for dense */
    const int32_t *cu_seqlens_k;   /* device; NULL for dense */
    int64_t total_q, total_k;      /* packed: cu_seqlens_q/k[batch] (host copies) */

    const void *dout, *q, *k, *v, *out;  /* 16-bit elements of `dtype` */
    const float *lse;                    /* fp32, natural log */
    void *dq, *dk, *dv;                  /* outputs, elements of `dtype` */

    int64_t do_stride[3], q_stride[3], k_stride[3], v_stride[3], o_stride[3];
    int64_t dq_stride[3], dk_stride[3], dv_stride[3];
    int64_t lse_stride[2];

    float softmax_scale;           /* the caller passes it (usually 1/sqrt(head_dim)) */
    int32_t causal;                /* 0 or 1 */
    int32_t local_window;          /* 0: no window (sizes ignored); 1: the sizes apply */
    int32_t window_size_left;      /* local window (see Semantics); < 0: unbounded */
    int32_t window_size_right;     /* < 0: unbounded; with causal = 1 only < 0 or 0 */
    float softcap;                 /* > 0: soft-capped scores (see Semantics); 0: none */
    float dropout_p;               /* dropout probability in [0, 1); 0: none */
    uint64_t philox_seed;          /* the forward's rng state (see Semantics) */
    uint64_t philox_offset;
    int32_t deterministic;         /* 0 or 1 (see Reproducibility) */
    int32_t dq_accumulate;         /* 0: separate dQ pass (default); 1: fp32 accumulator */

    void *workspace;               /* device, 256-byte aligned, caller-owned */
    size_t workspace_bytes;
    /* Largest keep region (see the workspace layout) the call may use; 0: 4 GiB.
     * The region is one bit per (query row, key) pair of every head, so it
     * grows with seqlen_q * seqlen_k; above the bound the main step draws the
     * keep bits itself instead (same bits, same results, slower). */
    size_t dropout_keep_max_bytes;
    /* Optional (dropout_p > 0, dq_accumulate = 0): the keep words a forward
     * call with the same shapes, p, seed and offset wrote (fa_fwd_args
     * dropout_keep_out: the layout of the workspace's keep region, 4-byte
     * aligned, at least fa_fwd_keep_bytes() bytes, stated in
     * dropout_keep_bytes; FA_ERR_INVALID_ARG otherwise).  The dQ and
     * key-tile steps then read the bits instead of drawing them
     * (bit-identical results, no keep region in the workspace).  Contents
     * are not checked: words of another call give wrong gradients.  NULL:
     * the steps draw the bits.  Ignored when dropout_p = 0 or dq_accumulate
     * = 1 (the fused step draws them). */
    const uint32_t *dropout_keep;
    size_t dropout_keep_bytes;
} fa_bwd_args;

/*
 * Workspace layout (byte offsets from `workspace`, each 256-byte aligned).
 * rows = batch * seqlen_q (dense) or total_q (packed); row index of query i
 * of sequence s is s * seqlen_q + i (dense) or cu_seqlens_q[s] + i (packed).
 *   lse2   : float[num_heads][rows]   LSE * log2(e), +inf for rows with no key
 *   rowdot : float[num_heads][rows]   sum_d dO * O (fp32 accumulation)
 *   dq_acc : float[num_heads][rows][head_dim_pad]  unscaled fp32 dQ sums
 *            (dq_accumulate = 1 only; zero bytes otherwise)
 *   turns  : int32[batch][num_heads][ceil(seqlen_q / 64)] ordering counters
 *            (dq_accumulate = 1 only)
 *   flags  : int32[4]  flags[0] != 0 if an ordered wait gave up (should
 *                      never happen; dq is then not bit-reproducible).  The
 *                      call still returns FA_OK (the wait is on the device):
 *                      a caller that relies on deterministic = 1 with
 *                      dq_accumulate = 1 reads flags[0] after the call.
 *   keep   : uint32[keep_words][num_heads][rows]  dropout keep bits (dropout_p
 *            > 0, dq_accumulate = 0, no dropout_keep words given and at most
 *            dropout_keep_max_bytes only; zero bytes and keep_words = 0
 *            otherwise): bit x of
 *            word w of a row is the keep bit of key 32 w + x of its sequence;
 *            keep_words = 2 * ceil(seqlen_k / 64) (max_seqlen_k when packed).
 *            Written by the dq step for every key tile a row's query tile
 *            visits (words of keys a row cannot see may hold anything), read
 *            by the main step instead of drawing the bits again.
 */
typedef struct fa_bwd_ws_layout {
    int64_t rows;
    int32_t head_dim_pad;
    int32_t q_tile;                /* 64: rows per query tile */
    int32_t k_tile;                /* 128: keys per workgroup */
    size_t off_lse2, off_rowdot, off_dq_acc, off_turns, off_flags, off_keep;
    int32_t keep_words;            /* 0 when there is no keep region */
    size_t total_bytes;
} fa_bwd_ws_layout;

/* Bytes of workspace the call needs; 0 if the arguments are invalid (host
 * only, touches no device memory). */
size_t fa_bwd_workspace_size(const fa_bwd_args *a);

/* Fills *out with the workspace layout of these arguments.  Host only. */
fa_status fa_bwd_workspace_layout(const fa_bwd_args *a, fa_bwd_ws_layout *out);

/* Checks every host-visible argument (pointers, sizes, strides, alignment,
 * workspace size).  Host only: no GPU access, nothing enqueued. */
fa_status fa_bwd_validate(const fa_bwd_args *a);

/* The whole backward, enqueued on `stream`: dq then main (dq_accumulate = 0;
 * the dq step also writes lse2 / rowdot, so no preprocess step is needed), or
 * preprocess, main, dq_convert (dq_accumulate = 1). */
fa_status fa_bwd(const fa_bwd_args *a, void *stream);

/* The steps one at a time, on one stream, in the order above (each
 * validates like fa_bwd).  Used to time and test the kernels separately.
 * fa_bwd_preprocess writes lse2 / rowdot (and, with dq_accumulate = 1, clears
 * the accumulator); fa_bwd_dq writes the same lse2 / rowdot values (bit for
 * bit) itself and needs nothing before it; fa_bwd_main needs a completed
 * fa_bwd_preprocess or fa_bwd_dq on the same workspace (with dropout_p > 0 and
 * dq_accumulate = 0, a completed fa_bwd_dq: it writes the keep bits that
 * fa_bwd_main reads); fa_bwd_dq_convert
 * needs a completed fa_bwd_main.  fa_bwd_dq requires dq_accumulate = 0 and
 * fa_bwd_dq_convert dq_accumulate = 1 (FA_ERR_INVALID_ARG otherwise). */
fa_status fa_bwd_preprocess(const fa_bwd_args *a, void *stream);
fa_status fa_bwd_main(const fa_bwd_args *a, void *stream);
fa_status fa_bwd_dq(const fa_bwd_args *a, void *stream);
fa_status fa_bwd_dq_convert(const fa_bwd_args *a, void *stream);

/* Debug read of D = rowsum(dO * O), the per-row term of dS = P (dP - D)
 * (the softmax_d that the backward call-trace page's _flash_attn_backward
 * returns, filled by the dsoftmax_sum step of set_params_dgrad): enqueues
 * the preprocess step only (exactly fa_bwd_preprocess: the workspace's lse2 /
 * rowdot are written, and with dq_accumulate = 1 the accumulator cleared)
 * and also writes each row's D into D_out.
 *   D_out : DEVICE float buffer with the layout and strides of `lse`
 *           (D_out + b * lse_stride[0] + h * lse_stride[1] + i for query row
 *           i of sequence / batch b and head h), caller-owned, 4-byte
 *           aligned; entries of packed rows past a sequence's length are not
 *           written.  It must not alias any input, output or the workspace.
 *   D is sum_d dO_id * O_id in fp32 (exact 16-bit products, fixed order),
 *   bit-identical to the value the backward's kernels use; it is computed
 *   for every row, including rows whose LSE is -inf (their O is 0).
 * Validation as fa_bwd (a workspace is required), plus D_out non-NULL when
 * there are query rows (FA_ERR_INVALID_ARG). */
fa_status fa_bwd_debug_rowsum(const fa_bwd_args *a, float *D_out, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the whole
 * backward as fa_bwd enqueues it, with `workspace` / `workspace_bytes`
 * ignored and a scratch array owned by the library used instead.  No
 * allocation happens on any call.
 *   - The scratch array holds FA_BWD_NOALLOC_MAX_WORKSPACE bytes on every GPU
 *     the library runs on, from library load to process end; a call whose
 *     fa_bwd_workspace_size (computed without a dropout keep region) is larger
 *     returns FA_ERR_WORKSPACE before touching the GPU.
 *   - With dropout, the key-tile step draws the keep bits itself instead of
 *     reading them from a keep region (same bits, bit-identical results).
 *   - All calls on one GPU share its scratch array: calls that can overlap
 *     on one GPU (different streams or threads, no ordering between them)
 *     race and give wrong results.  Calls ordered on one stream are safe:
 *     each call writes or clears the scratch it reads.
 *   - Other arguments, semantics and errors as fa_bwd; FA_ERR_HIP also if
 *     the scratch array's device address cannot be obtained. */
#define FA_BWD_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
fa_status fa_bwd_noalloc(const fa_bwd_args *a, void *stream);

/* Reason of the last non-FA_OK status on this thread ("" if none). */
const char *fa_bwd_last_error(void);

/* FA_BWD_ABI_VERSION of the built library. */
int32_t fa_bwd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
