// fa_api.cpp -- host side of the C ABI in include/fa_bwd.h and
// include/fa_fwd.h: argument validation (all on the host, before any launch),
// the backward's workspace layout and launch sequence, and the forward's
// launch, on the caller's stream.
//
// Checks follow the validations listed on the Triton FA2 teaching page
// (AttentionMetadata.validate_inputs: null pointers, head-count divisibility,
// head dim <= 256, contiguous last dim) and the sm90 backward page
// (_check_type: 16-bit input dtype, fp32 LSE / accumulators; __call__: every
// stride but the last a multiple of 128 bits).
#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <string>

#include "../../include/fa_bwd.h"
#include "../../include/fa_fwd.h"
#include "fa_internal.h"

namespace {

thread_local std::string g_last_error;

fa_status fail(fa_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Sequence lengths and window sizes stay below 2^29 so that row + offset +
// window sums fit in 32-bit integers in the kernels (a window of 2^29 or
// more reaches past every key of such a sequence).
constexpr int kMaxSeqlen = 1 << 29;

void set_softcap(fa::Params &p, float c)
{
    const double log2e = 1.4426950408889634;
    p.softcap = c;
    // (clamped: for a cap so small that the factor leaves the fp32 range,
    // tanh is +-1 for every nonzero score either way, and 0 * FLT_MAX = 0)
    p.cap_in = c > 0.f ? (float)std::min(2.0 * std::fabs((double)p.scale) * log2e / (double)c,
                                         (double)FLT_MAX)
                       : 0.f;
    if (p.scale < 0.f)
        p.cap_in = -p.cap_in;
    p.cap_out = c > 0.f ? (float)((double)c * log2e) : 0.f;
}

void set_dropout(fa::Params &p, float drop_p, uint64_t seed, uint64_t offset)
{
    p.drop_p = drop_p;
    p.drop_inv = drop_p > 0.f ? (float)(1.0 / (1.0 - (double)drop_p)) : 1.f;
    p.drop_thr = (uint32_t)std::floor((double)drop_p * 4294967296.0);
    p.drop_k0 = (uint32_t)seed;
    p.drop_k1 = (uint32_t)(seed >> 32) ^ (uint32_t)(offset >> 32);
    p.drop_c3 = (uint32_t)offset;
}

void set_window(fa::Params &p, int causal, int left, int right)
{
    p.win_l = left < 0 ? -1 : std::min(left, kMaxSeqlen);
    p.win_r = causal ? 0 : (right < 0 ? -1 : std::min(right, kMaxSeqlen));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int pad_head_dim(int d)
{
    if (d <= 64)
        return 64;
    if (d <= 96)
        return 96;
    if (d <= 128)
        return 128;
    if (d <= 192)
        return 192;
    if (d <= 256)
        return 256;
    return 0;
}

struct Plan {
    fa::Params p;
    fa_bwd_ws_layout ws;
    int dpad;
};

fa_status check_strides(const char *name, const int64_t s[3], bool varlen)
{
    for (int i = varlen ? 1 : 0; i < 3; ++i)
        if (s[i] % 8 != 0)
            return fail(FA_ERR_INVALID_ARG,
                        "%s stride[%d] = %lld is not a multiple of 8 elements (16 bytes)", name,
                        i, (long long)s[i]);
    return FA_OK;
}

// Keep words of a dropout call: 2 * ceil(seqlen_k / 64) per row of every head.
size_t keep_words_bytes(int32_t seqlen_k, int32_t heads, int64_t rows)
{
    if (seqlen_k <= 0 || heads <= 0 || rows <= 0)
        return 0;
    return 2 * (size_t)((seqlen_k + 63) / 64) * (size_t)heads * (size_t)rows * sizeof(uint32_t);
}

// The caller's keep words (forward output / backward input): 4-byte aligned,
// large enough, and one word's rows of all heads addressable with 31-bit
// byte offsets (the kernels' per-lane load and store offsets).
fa_status check_keep_words(const char *name, const void *ptr, size_t bytes, int32_t seqlen_k,
                           int32_t heads, int64_t rows)
{
    if (!aligned(ptr, 4))
        return fail(FA_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
    const size_t need = keep_words_bytes(seqlen_k, heads, rows);
    if (bytes < need)
        return fail(FA_ERR_INVALID_ARG, "%s has %zu bytes, needs %zu", name, bytes, need);
    if ((uint64_t)heads * (uint64_t)rows * 4u + 1024u >= (uint64_t(1) << 31))
        return fail(FA_ERR_UNSUPPORTED, "%s: num_heads * rows >= 2^29 is not supported", name);
    return FA_OK;
}

// Validates everything that can be checked on the host and fills the plan.
// need_ws: also require a large-enough workspace.
fa_status make_plan(const fa_bwd_args *a, Plan *pl, bool need_ws)
{
    if (!a)
        return fail(FA_ERR_INVALID_ARG, "args is NULL");
    if (a->dtype != FA_DTYPE_BF16 && a->dtype != FA_DTYPE_F16)
        return fail(FA_ERR_UNSUPPORTED, "dtype %d unsupported (bf16 or fp16)", a->dtype);
    if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0)
        return fail(FA_ERR_INVALID_ARG, "negative batch or sequence length");
    if (a->seqlen_q > kMaxSeqlen || a->seqlen_k > kMaxSeqlen)
        return fail(FA_ERR_UNSUPPORTED, "sequence length above 2^29");
    if (a->num_heads <= 0 || a->num_heads_k <= 0 || a->head_dim <= 0)
        return fail(FA_ERR_INVALID_ARG, "num_heads, num_heads_k and head_dim must be positive");
    if (a->num_heads % a->num_heads_k != 0)
        return fail(FA_ERR_INVALID_ARG, "num_heads (%d) is not a multiple of num_heads_k (%d)",
                    a->num_heads, a->num_heads_k);
    if (a->head_dim > 256)
        return fail(FA_ERR_UNSUPPORTED, "head_dim %d > 256", a->head_dim);
    if (a->head_dim % 8 != 0)
        return fail(FA_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 8 (pad it first)",
                    a->head_dim);
    const int dpad = pad_head_dim(a->head_dim);
    if (!dpad)
        return fail(FA_ERR_UNSUPPORTED, "head_dim %d is not built", a->head_dim);
    const bool varlen = a->cu_seqlens_q || a->cu_seqlens_k;
    if (varlen && !(a->cu_seqlens_q && a->cu_seqlens_k))
        return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be given together");
    if (varlen && (a->total_q < 0 || a->total_k < 0))
        return fail(FA_ERR_INVALID_ARG, "negative total_q / total_k");
    // Tensors with no elements may be NULL (an empty torch tensor has no
    // storage); every other tensor pointer must be set.
    const int64_t nq = varlen ? a->total_q : (int64_t)a->batch * a->seqlen_q;
    const int64_t nk = varlen ? a->total_k : (int64_t)a->batch * a->seqlen_k;
    if (nq > 0 && (!a->dout || !a->q || !a->out || !a->lse || !a->dq))
        return fail(FA_ERR_INVALID_ARG, "a query-side tensor pointer is NULL");
    if (nk > 0 && (!a->k || !a->v || !a->dk || !a->dv))
        return fail(FA_ERR_INVALID_ARG, "a key-side tensor pointer is NULL");
    const void *ptrs[] = {a->dout, a->q, a->k, a->v, a->out, a->dq, a->dk, a->dv};
    const char *names[] = {"dout", "q", "k", "v", "out", "dq", "dk", "dv"};
    for (int i = 0; i < 8; ++i)
        if (!aligned(ptrs[i], 16))
            return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    if (!aligned(a->lse, 4))
        return fail(FA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
    fa_status st;
    if ((st = check_strides("dout", a->do_stride, varlen)) ||
        (st = check_strides("q", a->q_stride, varlen)) ||
        (st = check_strides("k", a->k_stride, varlen)) ||
        (st = check_strides("v", a->v_stride, varlen)) ||
        (st = check_strides("out", a->o_stride, varlen)) ||
        (st = check_strides("dq", a->dq_stride, varlen)) ||
        (st = check_strides("dk", a->dk_stride, varlen)) ||
        (st = check_strides("dv", a->dv_stride, varlen)))
        return st;
    // The main kernel addresses a 64-row query tile with 32-bit offsets and
    // bounds its loads at the end of the tile's last valid row, which needs
    // rows that do not overlap.
    if (a->q_stride[1] < a->head_dim || a->do_stride[1] < a->head_dim)
        return fail(FA_ERR_INVALID_ARG, "q / dout row stride is smaller than head_dim");
    if (a->q_stride[1] >= (int64_t(1) << 24) || a->do_stride[1] >= (int64_t(1) << 24))
        return fail(FA_ERR_UNSUPPORTED, "q / dout row stride >= 2^24 elements is not supported");
    // The dQ kernel addresses a 64-key tile with 32-bit byte offsets too.
    if (a->k_stride[1] >= (int64_t(1) << 24) || a->v_stride[1] >= (int64_t(1) << 24))
        return fail(FA_ERR_UNSUPPORTED, "k / v row stride >= 2^24 elements is not supported");
    if (a->softmax_scale != a->softmax_scale || std::isinf(a->softmax_scale))
        return fail(FA_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (!(a->softcap >= 0.f) || std::isinf(a->softcap))
        return fail(FA_ERR_INVALID_ARG, "softcap must be finite and >= 0");
    if (!(a->dropout_p >= 0.f && a->dropout_p < 1.f))
        return fail(FA_ERR_INVALID_ARG, "dropout_p must lie in [0, 1)");
    if ((a->causal != 0 && a->causal != 1) || (a->deterministic != 0 && a->deterministic != 1) ||
        (a->dq_accumulate != 0 && a->dq_accumulate != 1))
        return fail(FA_ERR_INVALID_ARG, "causal, deterministic and dq_accumulate must be 0 or 1");
    if (a->dq_accumulate && a->head_dim > 128)
        return fail(FA_ERR_UNSUPPORTED,
                    "dq_accumulate = 1 is built for head_dim <= 128 only (the default dQ pass "
                    "covers head_dim %d)", a->head_dim);
    if (a->local_window != 0 && a->local_window != 1)
        return fail(FA_ERR_INVALID_ARG, "local_window must be 0 or 1");
    if (a->local_window && a->causal && a->window_size_right > 0)
        return fail(FA_ERR_INVALID_ARG, "causal = 1 with window_size_right = %d > 0",
                    a->window_size_right);
    const int64_t nq_rows = varlen ? a->total_q : (int64_t)a->batch * a->seqlen_q;
    const bool keep_given = a->dropout_keep && a->dropout_p > 0.f && !a->dq_accumulate;
    if (keep_given && (st = check_keep_words("dropout_keep", a->dropout_keep, a->dropout_keep_bytes,
                                             a->seqlen_k, a->num_heads, nq_rows)))
        return st;

    fa::Params &p = pl->p;
    std::memset(&p, 0, sizeof p);
    p.q = (const uint16_t *)a->q;
    p.k = (const uint16_t *)a->k;
    p.v = (const uint16_t *)a->v;
    p.o = (const uint16_t *)a->out;
    p.dout = (const uint16_t *)a->dout;
    p.lse = a->lse;
    p.dq = (uint16_t *)a->dq;
    p.dk = (uint16_t *)a->dk;
    p.dv = (uint16_t *)a->dv;
    p.cu_q = a->cu_seqlens_q;
    p.cu_k = a->cu_seqlens_k;
#define STR(dst, src) p.dst##_sb = a->src[0], p.dst##_ss = a->src[1], p.dst##_sh = a->src[2]
    STR(q, q_stride);
    STR(k, k_stride);
    STR(v, v_stride);
    STR(o, o_stride);
    STR(do, do_stride);
    STR(dq, dq_stride);
    STR(dk, dk_stride);
    STR(dv, dv_stride);
#undef STR
    p.lse_sb = a->lse_stride[0];
    p.lse_sh = a->lse_stride[1];
    p.batch = a->batch;
    p.H = a->num_heads;
    p.Hk = a->num_heads_k;
    p.G = a->num_heads / a->num_heads_k;
    p.D = a->head_dim;
    p.Sq = a->seqlen_q;
    p.Sk = a->seqlen_k;
    p.varlen = varlen ? 1 : 0;
    p.rows = varlen ? a->total_q : (int64_t)a->batch * a->seqlen_q;
    p.mtiles = (a->seqlen_q + fa::kQTile - 1) / fa::kQTile;
    p.ntiles = (a->seqlen_k + fa::kKTile - 1) / fa::kKTile;
    p.scale = a->softmax_scale;
    p.scale_log2 = (float)((double)a->softmax_scale * 1.4426950408889634);
    set_softcap(p, a->softcap);
    set_dropout(p, a->dropout_p, a->philox_seed, a->philox_offset);
    p.causal = a->causal;
    set_window(p, a->causal, a->local_window ? a->window_size_left : -1,
               a->local_window ? a->window_size_right : -1);
    p.deterministic = a->deterministic;
    p.fused_dq = a->dq_accumulate;
    p.f16 = a->dtype == FA_DTYPE_F16;

    // Workspace layout.
    fa_bwd_ws_layout &ws = pl->ws;
    std::memset(&ws, 0, sizeof ws);
    ws.rows = p.rows;
    ws.head_dim_pad = dpad;
    ws.q_tile = fa::kQTile;
    ws.k_tile = fa::kKTile;
    size_t off = 0;
    const size_t hr = (size_t)p.H * (size_t)p.rows;
    ws.off_lse2 = off;
    off = align256(off + hr * sizeof(float));
    ws.off_rowdot = off;
    off = align256(off + hr * sizeof(float));
    // The fp32 dQ accumulator and the turn counters exist in accumulate
    // mode only (zero bytes otherwise).
    ws.off_dq_acc = off;
    if (p.fused_dq)
        off = align256(off + hr * (size_t)dpad * sizeof(float));
    ws.off_turns = off;
    if (p.fused_dq)
        off = align256(off + (size_t)p.batch * p.H * p.mtiles * sizeof(int32_t));
    ws.off_flags = off;
    off = align256(off + 4 * sizeof(int32_t));
    // Dropout keep bits, written by the dQ pass for the key-tile kernel (the
    // accumulate mode's key-tile kernel draws them itself).
    // One bit per (row, key) pair: bounded (default 4 GiB), else the
    // key-tile kernel draws the bits itself.
    ws.off_keep = off;
    if (p.drop_p > 0.f && !p.fused_dq && !keep_given) {
        const size_t kw = 2 * (size_t)((p.Sk + 63) / 64);
        const size_t bytes = kw * hr * sizeof(uint32_t);
        const size_t cap = a->dropout_keep_max_bytes ? a->dropout_keep_max_bytes : (size_t)4 << 30;
        if (bytes <= cap) {
            ws.keep_words = (int32_t)kw;
            off = align256(off + bytes);
        }
    }
    ws.total_bytes = off;
    pl->dpad = dpad;

    if (need_ws) {
        if (!a->workspace)
            return fail(FA_ERR_WORKSPACE, "workspace is NULL");
        if (!aligned(a->workspace, 256))
            return fail(FA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
        if (a->workspace_bytes < ws.total_bytes)
            return fail(FA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu",
                        a->workspace_bytes, ws.total_bytes);
        char *base = (char *)a->workspace;
        p.lse2 = (float *)(base + ws.off_lse2);
        p.rowdot = (float *)(base + ws.off_rowdot);
        p.dq_acc = p.fused_dq ? (float *)(base + ws.off_dq_acc) : nullptr;
        p.turns = p.fused_dq ? (int *)(base + ws.off_turns) : nullptr;
        p.flags = (int *)(base + ws.off_flags);
        p.keep = ws.keep_words ? (uint32_t *)(base + ws.off_keep) : nullptr;
    }
    if (keep_given) {
        p.keep = const_cast<uint32_t *>(a->dropout_keep);   // read only (keep_given)
        p.keep_given = 1;
    }
    g_last_error.clear();
    return FA_OK;
}

fa_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return FA_OK;
}

enum Step { kPre = 1, kMain = 2, kConv = 4, kDq = 8 };

// rowsum_out: debug copy of the row sums (preprocess step only), or null.
fa_status run(const fa_bwd_args *a, void *stream, int steps, float *rowsum_out = nullptr)
{
    Plan pl;
    fa_status st = make_plan(a, &pl, true);
    if (st)
        return st;
    hipStream_t s = (hipStream_t)stream;
    pl.p.rowsum_out = rowsum_out;
    const fa::Params &p = pl.p;
    const bool has_rows = p.batch > 0 && p.Sq > 0 && p.rows > 0;
    const bool has_keys = p.batch > 0 && p.ntiles > 0;
    if ((steps & kConv) && !p.fused_dq)
        return fail(FA_ERR_INVALID_ARG, "dq_convert needs dq_accumulate = 1");
    if ((steps & kDq) && p.fused_dq)
        return fail(FA_ERR_INVALID_ARG, "the separate dQ pass needs dq_accumulate = 0");
    if ((steps & kPre) && has_rows)
        if ((st = hip_status(fa::launch_preprocess(p, pl.dpad, s), "preprocess launch")))
            return st;
    // The separate dQ pass writes lse2 / rowdot itself, so it runs before
    // the key-tile kernel that reads them.
    if ((steps & kDq) && has_rows)
        if ((st = hip_status(fa::launch_dq(p, pl.dpad, s), "dq launch")))
            return st;
    if ((steps & kMain) && has_keys)
        if ((st = hip_status(fa::launch_main(p, pl.dpad, s), "main launch")))
            return st;
    if ((steps & kConv) && has_rows)
        if ((st = hip_status(fa::launch_convert(p, pl.dpad, s), "dq_convert launch")))
            return st;
    return FA_OK;
}

// Forward: the same checks on the subset of tensors it touches.
fa_status make_fwd_plan(const fa_fwd_args *a, fa::Params *pp, int *dpad_out)
{
    if (!a)
        return fail(FA_ERR_INVALID_ARG, "args is NULL");
    if (a->dtype != FA_DTYPE_BF16 && a->dtype != FA_DTYPE_F16)
        return fail(FA_ERR_UNSUPPORTED, "dtype %d unsupported (bf16 or fp16)", a->dtype);
    if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0)
        return fail(FA_ERR_INVALID_ARG, "negative batch or sequence length");
    if (a->seqlen_q > kMaxSeqlen || a->seqlen_k > kMaxSeqlen)
        return fail(FA_ERR_UNSUPPORTED, "sequence length above 2^29");
    if (a->num_heads <= 0 || a->num_heads_k <= 0 || a->head_dim <= 0)
        return fail(FA_ERR_INVALID_ARG, "num_heads, num_heads_k and head_dim must be positive");
    if (a->num_heads % a->num_heads_k != 0)
        return fail(FA_ERR_INVALID_ARG, "num_heads (%d) is not a multiple of num_heads_k (%d)",
                    a->num_heads, a->num_heads_k);
    if (a->head_dim > 256)
        return fail(FA_ERR_UNSUPPORTED, "head_dim %d > 256", a->head_dim);
    if (a->head_dim % 8 != 0)
        return fail(FA_ERR_UNSUPPORTED, "head_dim %d is not a multiple of 8 (pad it first)",
                    a->head_dim);
    const int dpad = pad_head_dim(a->head_dim);
    if (!dpad)
        return fail(FA_ERR_UNSUPPORTED, "head_dim %d is not built", a->head_dim);
    const bool varlen = a->cu_seqlens_q || a->cu_seqlens_k;
    if (varlen && !(a->cu_seqlens_q && a->cu_seqlens_k))
        return fail(FA_ERR_INVALID_ARG, "cu_seqlens_q and cu_seqlens_k must be given together");
    if (varlen && (a->total_q < 0 || a->total_k < 0))
        return fail(FA_ERR_INVALID_ARG, "negative total_q / total_k");
    const int64_t nq = varlen ? a->total_q : (int64_t)a->batch * a->seqlen_q;
    const int64_t nk = varlen ? a->total_k : (int64_t)a->batch * a->seqlen_k;
    if (nq > 0 && (!a->q || !a->out || !a->lse))
        return fail(FA_ERR_INVALID_ARG, "a query-side tensor pointer is NULL");
    if (nk > 0 && (!a->k || !a->v))
        return fail(FA_ERR_INVALID_ARG, "a key-side tensor pointer is NULL");
    const void *ptrs[] = {a->q, a->k, a->v, a->out};
    const char *names[] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i)
        if (!aligned(ptrs[i], 16))
            return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    if (!aligned(a->lse, 4))
        return fail(FA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
    fa_status st;
    if ((st = check_strides("q", a->q_stride, varlen)) ||
        (st = check_strides("k", a->k_stride, varlen)) ||
        (st = check_strides("v", a->v_stride, varlen)) ||
        (st = check_strides("out", a->o_stride, varlen)))
        return st;
    // A 64-key tile is addressed with 32-bit byte offsets.
    if (a->k_stride[1] >= (int64_t(1) << 24) || a->v_stride[1] >= (int64_t(1) << 24))
        return fail(FA_ERR_UNSUPPORTED, "k / v row stride >= 2^24 elements is not supported");
    if (a->softmax_scale != a->softmax_scale || std::isinf(a->softmax_scale))
        return fail(FA_ERR_INVALID_ARG, "softmax_scale is not finite");
    if (!(a->softcap >= 0.f) || std::isinf(a->softcap))
        return fail(FA_ERR_INVALID_ARG, "softcap must be finite and >= 0");
    if (!(a->dropout_p >= 0.f && a->dropout_p < 1.f))
        return fail(FA_ERR_INVALID_ARG, "dropout_p must lie in [0, 1)");
    if (a->causal != 0 && a->causal != 1)
        return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1");
    if (a->local_window != 0 && a->local_window != 1)
        return fail(FA_ERR_INVALID_ARG, "local_window must be 0 or 1");
    if (a->local_window && a->causal && a->window_size_right > 0)
        return fail(FA_ERR_INVALID_ARG, "causal = 1 with window_size_right = %d > 0",
                    a->window_size_right);
    const bool keep_out = a->dropout_keep_out && a->dropout_p > 0.f;
    if (keep_out && (st = check_keep_words("dropout_keep_out", a->dropout_keep_out,
                                           a->dropout_keep_out_bytes, a->seqlen_k, a->num_heads, nq)))
        return st;

    fa::Params &p = *pp;
    std::memset(&p, 0, sizeof p);
    p.q = (const uint16_t *)a->q;
    p.k = (const uint16_t *)a->k;
    p.v = (const uint16_t *)a->v;
    p.o_w = (uint16_t *)a->out;
    p.lse_w = a->lse;
    p.cu_q = a->cu_seqlens_q;
    p.cu_k = a->cu_seqlens_k;
#define STR(dst, src) p.dst##_sb = a->src[0], p.dst##_ss = a->src[1], p.dst##_sh = a->src[2]
    STR(q, q_stride);
    STR(k, k_stride);
    STR(v, v_stride);
    STR(o, o_stride);
#undef STR
    p.lse_sb = a->lse_stride[0];
    p.lse_sh = a->lse_stride[1];
    p.batch = a->batch;
    p.H = a->num_heads;
    p.Hk = a->num_heads_k;
    p.G = a->num_heads / a->num_heads_k;
    p.D = a->head_dim;
    p.Sq = a->seqlen_q;
    p.Sk = a->seqlen_k;
    p.varlen = varlen ? 1 : 0;
    p.rows = nq;
    p.scale = a->softmax_scale;
    p.scale_log2 = (float)((double)a->softmax_scale * 1.4426950408889634);
    set_softcap(p, a->softcap);
    set_dropout(p, a->dropout_p, a->philox_seed, a->philox_offset);
    p.causal = a->causal;
    set_window(p, a->causal, a->local_window ? a->window_size_left : -1,
               a->local_window ? a->window_size_right : -1);
    p.f16 = a->dtype == FA_DTYPE_F16;
    p.keep = keep_out ? a->dropout_keep_out : nullptr;
    *dpad_out = dpad;
    g_last_error.clear();
    return FA_OK;
}

}  // namespace

namespace fa {

// Sets the thread's last-error message for the entry points defined in other
// translation units.
int report_error(int status, const char *msg)
{
    return fail((fa_status)status, "%s", msg);
}

}  // namespace fa

extern "C" {

size_t fa_fwd_keep_bytes(const fa_fwd_args *a)
{
    if (!a || !(a->dropout_p > 0.f))
        return 0;
    fa_fwd_args b = *a;
    b.dropout_keep_out = nullptr;   // validate the rest
    fa::Params p;
    int dpad;
    if (make_fwd_plan(&b, &p, &dpad))
        return 0;
    return keep_words_bytes(a->seqlen_k, a->num_heads, p.rows);
}

fa_status fa_fwd_validate(const fa_fwd_args *a)
{
    fa::Params p;
    int dpad;
    return make_fwd_plan(a, &p, &dpad);
}

fa_status fa_fwd(const fa_fwd_args *a, void *stream)
{
    fa::Params p;
    int dpad;
    fa_status st = make_fwd_plan(a, &p, &dpad);
    if (st)
        return st;
    if (p.batch > 0 && p.Sq > 0 && p.rows > 0)
        return hip_status(fa::launch_fwd(p, dpad, (hipStream_t)stream), "forward launch");
    return FA_OK;
}


size_t fa_bwd_workspace_size(const fa_bwd_args *a)
{
    Plan pl;
    if (make_plan(a, &pl, false))
        return 0;
    return pl.ws.total_bytes;
}

fa_status fa_bwd_workspace_layout(const fa_bwd_args *a, fa_bwd_ws_layout *out)
{
    if (!out)
        return fail(FA_ERR_INVALID_ARG, "out is NULL");
    Plan pl;
    fa_status st = make_plan(a, &pl, false);
    if (st)
        return st;
    *out = pl.ws;
    return FA_OK;
}

fa_status fa_bwd_validate(const fa_bwd_args *a)
{
    Plan pl;
    return make_plan(a, &pl, true);
}

fa_status fa_bwd(const fa_bwd_args *a, void *stream)
{
    if (!a)
        return fail(FA_ERR_INVALID_ARG, "args is NULL");
    return run(a, stream, a->dq_accumulate ? kPre | kMain | kConv : kDq | kMain);
}
fa_status fa_bwd_preprocess(const fa_bwd_args *a, void *stream) { return run(a, stream, kPre); }

fa_status fa_bwd_debug_rowsum(const fa_bwd_args *a, float *D_out, void *stream)
{
    if (!a)
        return fail(FA_ERR_INVALID_ARG, "args is NULL");
    const bool varlen = a->cu_seqlens_q || a->cu_seqlens_k;
    const int64_t nq = varlen ? a->total_q : (int64_t)a->batch * a->seqlen_q;
    if (nq > 0 && !D_out)
        return fail(FA_ERR_INVALID_ARG, "D_out is NULL");
    if (!aligned(D_out, 4))
        return fail(FA_ERR_INVALID_ARG, "D_out is not 4-byte aligned");
    return run(a, stream, kPre, D_out);
}
fa_status fa_bwd_main(const fa_bwd_args *a, void *stream) { return run(a, stream, kMain); }
fa_status fa_bwd_dq_convert(const fa_bwd_args *a, void *stream) { return run(a, stream, kConv); }
fa_status fa_bwd_dq(const fa_bwd_args *a, void *stream) { return run(a, stream, kDq); }

const char *fa_bwd_last_error(void) { return g_last_error.c_str(); }

int32_t fa_bwd_abi_version(void) { return FA_BWD_ABI_VERSION; }

}  // extern "C"
