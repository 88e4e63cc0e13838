// fa_convert.hip -- last step of the attention backward on gfx950:
//   dQ[row][h][d] = bf16_rne(scale * dq_acc[h][row][d])   for d < head_dim.
// The main kernel leaves dQ unscaled in fp32 (as the sm90 backward page's
// dQaccum_store writes the raw accumulator); the softmax scale is applied
// here once, as the Triton FA2 teaching page's dQ kernel multiplies dq by
// sm_scale at the end.  HBM-bound: 4 * D_pad bytes read, 2 * D bytes written
// per row and head; 16 lanes per row, 8 columns per lane.
#include "fa_internal.h"

namespace fa {

template <int DP, bool F16>
__global__ void __launch_bounds__(kThreads) fa_bwd_convert_kernel(Params p)
{
    const int b = blockIdx.z, h = blockIdx.y;
    const SeqInfo si = seq_info(p, b);
    const int i = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (i >= si.Lq || c * 8 >= p.D)
        return;
    const int64_t wr = (int64_t)h * p.rows + si.ws_row + i;
    const float *src = p.dq_acc + wr * DP + c * 8;
    const float4 a = *reinterpret_cast<const float4 *>(src);
    const float4 bq = *reinterpret_cast<const float4 *>(src + 4);
    const float s = p.scale;
    uint4 out;
    out.x = (uint32_t)f2elem<F16>(a.x * s) | ((uint32_t)f2elem<F16>(a.y * s) << 16);
    out.y = (uint32_t)f2elem<F16>(a.z * s) | ((uint32_t)f2elem<F16>(a.w * s) << 16);
    out.z = (uint32_t)f2elem<F16>(bq.x * s) | ((uint32_t)f2elem<F16>(bq.y * s) << 16);
    out.w = (uint32_t)f2elem<F16>(bq.z * s) | ((uint32_t)f2elem<F16>(bq.w * s) << 16);
    uint16_t *dst = p.dq + row_offset(p, b, si.tok_q, i, p.dq_sb, p.dq_ss) + h * p.dq_sh + c * 8;
    *reinterpret_cast<uint4 *>(dst) = out;
}

hipError_t launch_convert(const Params &p, int dpad, hipStream_t st)
{
    const dim3 grid((p.Sq + kRowsPerBlock - 1) / kRowsPerBlock, p.H, p.batch);
    const dim3 block(kThreads);
    switch (dpad) {
    case 64:
        if (p.f16)
            hipLaunchKernelGGL((fa_bwd_convert_kernel<64, true>), grid, block, 0, st, p);
        else
            hipLaunchKernelGGL((fa_bwd_convert_kernel<64, false>), grid, block, 0, st, p);
        break;
    case 96:
        if (p.f16)
            hipLaunchKernelGGL((fa_bwd_convert_kernel<96, true>), grid, block, 0, st, p);
        else
            hipLaunchKernelGGL((fa_bwd_convert_kernel<96, false>), grid, block, 0, st, p);
        break;
    case 128:
        if (p.f16)
            hipLaunchKernelGGL((fa_bwd_convert_kernel<128, true>), grid, block, 0, st, p);
        else
            hipLaunchKernelGGL((fa_bwd_convert_kernel<128, false>), grid, block, 0, st, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
