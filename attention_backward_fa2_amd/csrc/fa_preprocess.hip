// fa_preprocess.hip -- first step of the attention backward on gfx950.
//
// Per query row i and head h:
//   rowdot[h][row] = sum_d dO_id * O_id   (fp32 accumulation of exact
//                    bf16 x bf16 products) -- the row sum that replaces the
//                    softmax-Jacobian term: backward call-trace page,
//                    set_params_dgrad (dsoftmax_sum = row sum of dout * out);
//                    sm90 backward page, mma_one_m_block pointwise step 2
//                    (dS = P (dP - dPsum)).
//   lse2[h][row]   = LSE_i * log2(e), or +inf when LSE_i = -inf (a row with
//                    no visible key), so that exp2(S*scale*log2e - lse2) is
//                    exactly 0 there instead of NaN.  The base-2 form is the
//                    exp2 with folded log2(e) of the sm90 backward page
//                    (mma_one_m_block pointwise step 1).
//   accumulate mode only: dq_acc[h][row][:] = 0, and (ordered adds) the
//                    turn counter of the row's query tile = 0.
//   debug copy (rowsum_out set): rowdot also written in the lse layout (the
//                    softmax_d the backward call-trace page's
//                    _flash_attn_backward returns for inspection).
//
// HBM-bound: reads O and dO once (2 * 2 * D bytes per row and head), writes
// 8 bytes (+ 4 * D_pad in accumulate mode).  16 lanes per row; each lane owns
// 16-byte chunks.
#include "fa_internal.h"

namespace fa {

template <int DP, bool F16>
__global__ void __launch_bounds__(kThreads) fa_bwd_preprocess_kernel(Params p)
{
    const int b = blockIdx.z, h = blockIdx.y;
    const SeqInfo si = seq_info(p, b);
    const int i = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 4)
        p.flags[threadIdx.x] = 0;
    if (blockIdx.x * kRowsPerBlock >= si.Lq)
        return;
    const bool valid = i < si.Lq;

    float acc = 0.f;
    if (valid) {
        const uint16_t *orow = p.o + row_offset(p, b, si.tok_q, i, p.o_sb, p.o_ss) + h * p.o_sh;
        const uint16_t *drow =
            p.dout + row_offset(p, b, si.tok_q, i, p.do_sb, p.do_ss) + h * p.do_sh;
        for (int ch = c; ch * 8 < p.D; ch += 16) {
            const uint4 ov = *reinterpret_cast<const uint4 *>(orow + ch * 8);
            const uint4 dv = *reinterpret_cast<const uint4 *>(drow + ch * 8);
            const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
            const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc += elem2f<F16>((uint16_t)(ow[t] & 0xffff)) * elem2f<F16>((uint16_t)(dw[t] & 0xffff));
                acc += elem2f<F16>((uint16_t)(ow[t] >> 16)) * elem2f<F16>((uint16_t)(dw[t] >> 16));
            }
        }
    }
    // Fixed-order butterfly over the 16 lanes of the row.
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
        acc += __shfl_xor(acc, off, 16);

    if (!valid)
        return;
    const int64_t wr = (int64_t)h * p.rows + si.ws_row + i;
    if (c == 0) {
        const float lse = p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + i];
        p.rowdot[wr] = acc;
        if (p.rowsum_out)
            p.rowsum_out[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + i] = acc;
        p.lse2[wr] = (lse == -INFINITY) ? INFINITY : lse * 1.4426950408889634f;
        if (p.fused_dq && p.deterministic && (i % kQTile) == 0)
            p.turns[((int64_t)b * p.H + h) * p.mtiles + i / kQTile] = 0;
    }
    // Accumulate mode (head_dim <= 128 only): clear this row of the fp32 dQ
    // accumulator, DP / 16 floats per lane.
    if constexpr (DP <= 128) {
        if (!p.fused_dq)
            return;
        constexpr int PER = DP / 16;
        float *dst = p.dq_acc + wr * DP + c * PER;
        if constexpr (PER % 4 == 0) {
#pragma unroll
            for (int t = 0; t < PER; t += 4)
                *reinterpret_cast<float4 *>(dst + t) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
#pragma unroll
            for (int t = 0; t < PER; t += 2)
                *reinterpret_cast<float2 *>(dst + t) = make_float2(0.f, 0.f);
        }
    }
}

hipError_t launch_preprocess(const Params &p, int dpad, hipStream_t st)
{
    const dim3 grid((p.Sq + kRowsPerBlock - 1) / kRowsPerBlock, p.H, p.batch);
    const dim3 block(kThreads);
#define FA_PRE_CASE(D)                                                                    \
    case D:                                                                               \
        if (p.f16)                                                                        \
            hipLaunchKernelGGL((fa_bwd_preprocess_kernel<D, true>), grid, block, 0, st, p);  \
        else                                                                              \
            hipLaunchKernelGGL((fa_bwd_preprocess_kernel<D, false>), grid, block, 0, st, p); \
        break;
    switch (dpad) {
        FA_PRE_CASE(64)
        FA_PRE_CASE(96)
        FA_PRE_CASE(128)
        FA_PRE_CASE(192)
        FA_PRE_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef FA_PRE_CASE
    return hipGetLastError();
}

}  // namespace fa
