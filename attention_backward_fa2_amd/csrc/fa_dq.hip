// fa_dq.hip -- query-stationary dQ kernel of the attention backward on
// gfx950 (the default way dQ is formed).
//
// dQ_i = scale * sum_j dS_ij K_j with dS = P (dP - rowdot) recomputed per
// tile (the Triton FA2 teaching page's backward dQ kernel computes dQ the
// same way: one program per query block looping over key blocks, P and dS
// recomputed, dq scaled by sm_scale at the end; the products themselves are
// the sm90 backward page's mma_one_m_block steps 1, 2 and 6).  Computing dQ
// here instead of adding dQ partials from every key tile of the key-tile
// kernel costs three extra products per tile pair but needs no atomics (the
// fp32 atomic rate of the L2 would otherwise bound the whole backward), no
// fp32 accumulator and no convert pass, and the result is bit-reproducible.
//
// One workgroup (4 wave64s) owns 128 query rows of one query head; wave w
// owns rows 32w .. 32w+31, whose Q and dO rows stay in registers as the B
// operands of
//     S^T  = K Q^T        dP^T = V dO^T        (64 keys x 32 rows per wave)
// for each 64-key tile streamed through double-buffered LDS.  The
// accumulator of S^T holds one query row and 16 keys per lane, so dS (in
// bf16) is directly the A operand of dQ = dS K with the key index permuted
// as described in fa_mfma.h; K then enters as a B operand through
// transposing LDS reads.  dQ (32 x D per wave) accumulates in registers over
// all key tiles and is scaled and stored once.
//
// LDS (D_pad = 128): K and V tiles, double buffered: 4 x 18 KB = 72 KB.
#include "fa_mfma.h"

namespace fa {

constexpr int kDqRows = 128;    // query rows per workgroup
constexpr int kDqKeys = 64;     // keys per streamed tile

template <int DP>
struct __attribute__((aligned(16))) DqSmem {
    static constexpr int RK = DP + 16;   // pitch of the K / V tiles (elements)
    uint16_t k[2][kDqKeys * RK];
    uint16_t v[2][kDqKeys * RK];
};

template <int DP>
__global__ void __launch_bounds__(kThreads, 1) fa_bwd_dq_kernel(Params p)
{
    constexpr int KS = DP / 16;                  // k-steps over the head dim
    constexpr int DB = DP / 32;                  // 32-wide head-dim blocks
    constexpr int RK = DqSmem<DP>::RK;
    constexpr int CPR = DP / 8;                  // 16-byte chunks per row
    constexpr int NCH = kDqKeys * CPR / kThreads;   // chunks per thread per tile
    static_assert(kDqKeys * CPR % kThreads == 0, "tile load must divide evenly");
    __shared__ DqSmem<DP> sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

    // Workgroup -> (query tile, batch, KV head, head in group).  Under the
    // causal mask the last query tiles see the most keys, so they come
    // first; the (batch, KV head) index is the fastest, which keeps the
    // heads sharing a K/V tile on one XCD of the round-robin dispatch when
    // batch * Hk is a multiple of the XCD count.
    const int nbg = p.batch * p.Hk;
    const int nqt = (p.Sq + kDqRows - 1) / kDqRows;
    const int lin = blockIdx.x;
    const int bg = lin % nbg;
    const int hh = (lin / nbg) % p.G;
    const int mt = nqt - 1 - lin / (nbg * p.G);
    const int hk = bg % p.Hk, b = bg / p.Hk;
    const int h = hk * p.G + hh;

    const SeqInfo si = seq_info(p, b);
    const int q0 = mt * kDqRows;
    if (q0 >= si.Lq)
        return;
    const int Lq = si.Lq, Lk = si.Lk;
    const int off = Lk - Lq;
    const int qrow = q0 + 32 * w + l32;          // this lane's query row
    const bool qok = qrow < Lq;

    // ---- Q and dO rows of the lane (B operands), lse2 / rowdot ----
    bf16x8 qf[KS], of[KS];
    {
        const int qr = qok ? qrow : Lq - 1;
        const uint16_t *qp = p.q + row_offset(p, b, si.tok_q, qr, p.q_sb, p.q_ss) + h * p.q_sh;
        const uint16_t *dp_ =
            p.dout + row_offset(p, b, si.tok_q, qr, p.do_sb, p.do_ss) + h * p.do_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * g2;
            u32x4 a = 0, c = 0;
            if (qok && d0 < p.D) {
                a = *reinterpret_cast<const u32x4 *>(qp + d0);
                c = *reinterpret_cast<const u32x4 *>(dp_ + d0);
            }
            qf[ks] = __builtin_bit_cast(bf16x8, a);
            of[ks] = __builtin_bit_cast(bf16x8, c);
        }
    }
    float l2 = INFINITY, rd = 0.f;
    if (qok) {
        const int64_t wr = (int64_t)h * p.rows + si.ws_row + qrow;
        l2 = p.lse2[wr];
        rd = p.rowdot[wr];
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        zero(acc[db]);

    // Key tiles visible to some row of this query tile.
    const int q_last = min(q0 + kDqRows, Lq) - 1;
    int nkt = (Lk + kDqKeys - 1) / kDqKeys;
    if (p.causal)
        nkt = min(nkt, max(0, (q_last + off + kDqKeys) / kDqKeys));

    if (nkt > 0) {
        // Prefetch registers for one K/V tile (clamped rows, masked at
        // staging -- see the key-tile kernel for why).
        u32x4 pk[NCH], pv[NCH];
        int kv_valid = kDqKeys;
        auto prefetch = [&](int t) {
            const int n0 = t * kDqKeys;
            kv_valid = min(kDqKeys, Lk - n0);
            const uint16_t *kb = p.k + hk * p.k_sh + row_offset(p, b, si.tok_k, n0, p.k_sb, p.k_ss);
            const uint16_t *vb = p.v + hk * p.v_sh + row_offset(p, b, si.tok_k, n0, p.v_sb, p.v_ss);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int idx = tid + c * kThreads;
                const int r = min(idx / CPR, kv_valid - 1);
                const int col = (idx % CPR) * 8 < p.D ? (idx % CPR) * 8 : 0;
                pk[c] = *reinterpret_cast<const u32x4 *>(kb + r * (int)p.k_ss + col);
                pv[c] = *reinterpret_cast<const u32x4 *>(vb + r * (int)p.v_ss + col);
            }
        };
        auto stage = [&](int buf) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int idx = tid + c * kThreads;
                const uint32_t keep =
                    (idx / CPR < kv_valid && (idx % CPR) * 8 < p.D) ? ~0u : 0u;
                const int o = (idx / CPR) * RK + (idx % CPR) * 8;
                *reinterpret_cast<u32x4 *>(&sm.k[buf][o]) = pk[c] & keep;
                *reinterpret_cast<u32x4 *>(&sm.v[buf][o]) = pv[c] & keep;
            }
        };

        prefetch(0);
        stage(0);
        __syncthreads();

        for (int t = 0; t < nkt; ++t) {
            const int buf = t & 1;
            const int n0 = t * kDqKeys;
            if (t + 1 < nkt)
                prefetch(t + 1);
            const uint16_t *sk = sm.k[buf];
            const uint16_t *sv = sm.v[buf];

            // ---- S^T = K Q^T, dP^T = V dO^T (64 keys x 32 rows per wave) ----
            f32x16 st[2], dpt[2];
            const f32x16 z = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int o = (32 * mb + l32) * RK + 16 * ks + 8 * g2;
                    st[mb] = mfma32(lds16(sk + o), qf[ks], ks == 0 ? z : st[mb]);
                    dpt[mb] = mfma32(lds16(sv + o), of[ks], ks == 0 ? z : dpt[mb]);
                }
            }
            pipeline_reads<4 * KS, 1, 8>();

            // ---- P, dS; bf16 dS as A operands of dQ = dS K ----
            // key of accumulator element r of block mb: n0 + 32 mb + 8 (r/4)
            // + 4 g2 + r%4; visible iff key < Lk and (causal) key <= qrow + off.
            const bool need_mask =
                (n0 + kDqKeys > Lk) || (p.causal && (n0 + kDqKeys - 1 > q0 + off));
            const int klim = p.causal ? min(Lk - 1, qrow + off) : Lk - 1;
            bf16x4 dh[8];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 dv;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int r = 4 * r4 + t;
                        float e = __builtin_amdgcn_exp2f(st[mb][r] * p.scale_log2 - l2);
                        if (need_mask) {
                            const int key = n0 + 32 * mb + 8 * r4 + 4 * g2 + t;
                            e = key <= klim ? e : 0.f;
                        }
                        dv[t] = e * (dpt[mb][r] - rd);
                    }
                    dh[4 * mb + r4] = to_bf16(dv);
                }
            }
            bf16x8 dsa[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                dsa[kk] = concat(dh[2 * kk], dh[2 * kk + 1]);

            // ---- dQ += dS K  (k = 64 keys; K read transposed) ----
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r0 = 16 * kk + 4 * g2, r1 = r0 + 8;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[db] = mfma32(dsa[kk], frag_tr(sk, RK, r0, r1, 32 * db, lane), acc[db]);
            }
            pipeline_reads<4 * DB, 2, 8>();

            if (t + 1 < nkt)
                stage(buf ^ 1);
            __syncthreads();   // next tile staged; buffer buf free for t + 2
        }
    }

    // ---- dQ = scale * acc -> bf16.  Accumulator: column d = 32 db + l32,
    //      rows 8 (r/4) + 4 g2 + r%4 of the wave's 32 query rows. ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 32 * db + l32;
        if (d < p.D) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = q0 + 32 * w + 8 * (r >> 2) + 4 * g2 + (r & 3);
                if (qr < Lq)
                    p.dq[row_offset(p, b, si.tok_q, qr, p.dq_sb, p.dq_ss) + h * p.dq_sh + d] =
                        f2bf(acc[db][r] * p.scale);
            }
        }
    }
}

hipError_t launch_dq(const Params &p, int dpad, hipStream_t st)
{
    const int nqt = (p.Sq + kDqRows - 1) / kDqRows;
    const dim3 grid((unsigned)nqt * p.H * p.batch);
    const dim3 block(kThreads);
    switch (dpad) {
    case 64:
        hipLaunchKernelGGL(fa_bwd_dq_kernel<64>, grid, block, 0, st, p);
        break;
    case 96:
        hipLaunchKernelGGL(fa_bwd_dq_kernel<96>, grid, block, 0, st, p);
        break;
    case 128:
        hipLaunchKernelGGL(fa_bwd_dq_kernel<128>, grid, block, 0, st, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
