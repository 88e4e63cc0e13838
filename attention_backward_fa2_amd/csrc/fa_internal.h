// fa_internal.h -- parameters and device helpers shared by the gfx950 kernels
// of the attention backward and their host launcher.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Tile sizes of the main kernel.  One workgroup owns kKTile keys of one KV
// head; it streams query tiles of kQTile rows.  Four wave64s, each owning 32
// of the keys.
constexpr int kQTile = 64;
constexpr int kKTile = 128;
constexpr int kThreads = 256;

// Rows per workgroup of the preprocess and dq_convert kernels (16 lanes per
// row, 16 rows per 256-thread workgroup).
constexpr int kRowsPerBlock = 16;

// Bound on the iterations of an ordered (deterministic) wait.  A wait that
// runs out sets flags[0] and proceeds, so every wave always exits.
constexpr int kSpinLimit = 1 << 24;

// Everything a kernel needs, passed by value.  Strides are in elements:
// *_sb batch, *_ss row (token), *_sh head.  For packed inputs the batch
// stride is unused and the row index is cu_seqlens[s] + i.
struct Params {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    float *lse2, *rowdot, *dq_acc;
    int *turns, *flags;
    const int *cu_q, *cu_k;
    uint16_t *o_w;      // forward: O (output)
    float *lse_w;       // forward: LSE (output, natural log)

    int64_t q_sb, q_ss, q_sh;
    int64_t k_sb, k_ss, k_sh;
    int64_t v_sb, v_ss, v_sh;
    int64_t o_sb, o_ss, o_sh;
    int64_t do_sb, do_ss, do_sh;
    int64_t dq_sb, dq_ss, dq_sh;
    int64_t dk_sb, dk_ss, dk_sh;
    int64_t dv_sb, dv_ss, dv_sh;
    int64_t lse_sb, lse_sh;

    int64_t rows;       // workspace rows (batch*Sq dense, total_q packed)
    int batch, H, Hk, G, D;
    int Sq, Sk;         // dense lengths, or the maxima for packed input
    int mtiles;         // ceil(Sq / kQTile)
    int ntiles;         // ceil(Sk / kKTile)
    float scale;        // softmax scale
    float scale_log2;   // softmax scale * log2(e)
    int causal, deterministic, varlen;
    // Visible keys of query row i: i + off - win_l .. i + off + win_r
    // (off = Lk - Lq; a negative size leaves that side unbounded; causal is
    // win_r = 0).
    int win_l, win_r;
    // Soft cap c > 0 of the scaled scores (0: none): with s the raw product
    // q.k, tanh(s * scale / c) = 1 - 2 / (exp2(s * cap_in) + 1) and the capped
    // score in base 2 is tanh * cap_out.
    float softcap, cap_in, cap_out;
    // Dropout (drop_p > 0): an element is kept iff its Philox word is >=
    // drop_thr; kept values are scaled by drop_inv = 1 / (1 - p).  Key
    // (drop_k0, drop_k1), last counter word drop_c3.
    float drop_p, drop_inv;
    uint32_t drop_thr, drop_k0, drop_k1, drop_c3;
    // Keep bits of the separate-dQ backward with dropout: word w of row r of
    // head h (keys 32 w .. 32 w + 31 of the row's sequence, bit x for key
    // 32 w + x) at keep[(w * H + h) * rows + r]; written by the dQ kernel
    // (keep_given = 0) or by the forward (the caller's words, keep_given =
    // 1: the dQ kernel reads them), read by the key-tile kernel.  In the
    // forward: where it writes them.  Null otherwise.
    uint32_t *keep;
    int keep_given;
    // Debug copy of rowdot in the lse layout (same batch / head strides,
    // row stride 1), written by the preprocess kernel when not null.
    float *rowsum_out;
    int fused_dq;       // 1: dQ partials added into dq_acc by the key-tile kernel
    int f16;            // 1: fp16 elements, 0: bf16
};

// Lengths and first rows of sequence b.
struct SeqInfo {
    int Lq, Lk;
    int64_t tok_q, tok_k;   // first token row (packed) -- 0 for dense
    int64_t ws_row;         // workspace row of query 0
};

__device__ inline SeqInfo seq_info(const Params &p, int b)
{
    SeqInfo s;
    if (p.varlen) {
        const int q0 = p.cu_q[b], q1 = p.cu_q[b + 1];
        const int k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
        s.Lq = q1 - q0;
        s.Lk = k1 - k0;
        s.tok_q = q0;
        s.tok_k = k0;
        s.ws_row = q0;
    } else {
        s.Lq = p.Sq;
        s.Lk = p.Sk;
        s.tok_q = 0;
        s.tok_k = 0;
        s.ws_row = (int64_t)b * p.Sq;
    }
    return s;
}

// Element offset of row `i` of sequence `b` in a tensor with the given
// batch / row strides.
__device__ inline int64_t row_offset(const Params &p, int b, int64_t tok0, int64_t i,
                                     int64_t sb, int64_t ss)
{
    return p.varlen ? (tok0 + i) * ss : (int64_t)b * sb + i * ss;
}

// Inputs and outputs hold 16-bit elements, bf16 or fp16 (F16: the template
// flag every kernel carries); they travel as their bit patterns.
// fp32 -> element, round to nearest even (hardware converts on gfx950).
template <bool F16>
__device__ inline uint16_t f2elem(float x)
{
    if constexpr (F16)
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// element -> fp32 (exact)
template <bool F16>
__device__ inline float elem2f(uint16_t x)
{
    if constexpr (F16)
        return (float)__builtin_bit_cast(_Float16, x);
    else
        return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// Host-side launchers (one translation unit each).
hipError_t launch_preprocess(const Params &p, int dpad, hipStream_t st);
hipError_t launch_main(const Params &p, int dpad, hipStream_t st);
hipError_t launch_convert(const Params &p, int dpad, hipStream_t st);
hipError_t launch_dq(const Params &p, int dpad, hipStream_t st);
hipError_t launch_fwd(const Params &p, int dpad, hipStream_t st);

}  // namespace fa
