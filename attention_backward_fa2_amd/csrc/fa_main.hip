// fa_main.hip -- the hot loop of the attention backward on gfx950 (CDNA4).
//
// One workgroup (4 wave64s) owns a tile of kKTile = 128 keys of one KV head
// (KV-tile-stationary order of the sm90 backward page: grid over key blocks,
// K and V loaded once, query tiles streamed).  It loops over every query head
// of the KV head's group and, for each, over the 64-row query tiles that can
// see at least one of its keys (causal block bound with the seqlen_k -
// seqlen_q offset of the GQA/MQA page).  Per query tile it runs the five
// products of the sm90 backward page's mma_one_m_block on bf16 MFMA with fp32
// accumulation:
//     S  = Q K^T            dP = dO V^T
//     P  = exp2(S * scale * log2e - lse2)      (0 where masked)
//     dS = P * (dP - rowdot)
//     dV += P^T dO          dK += dS^T Q       (registers, whole group)
//     dQ_partial = dS K  -> fp32 adds into the dQ accumulator
// dK and dV accumulate over all query heads of the group in registers, which
// is the GQA reduction of dK/dV (GQA/MQA page, backward section; backward
// call-trace page, sum over the head group) done without atomics.  dK gets
// the softmax scale once at the end (sm90 backward page, epilogue scaling).
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Per lane l (l32 = l % 32, g2 = l / 32):
//   A (32 x 16, M x K): row l32, k = 8*g2 + t (t = 0..7, one 16-byte vector)
//   B (16 x 32, K x N): col l32, k = 8*g2 + t
//   C (32 x 32):        col l32, row 8*(r/4) + 4*g2 + r%4 for r = 0..15
// Each wave owns keys 32w .. 32w+31 of the tile.  With keys as the N index of
// S and dP, the accumulator of P (and dS) holds one key and 16 query rows per
// lane, which is exactly a B operand for dV^T = dO^T P and dK^T = Q^T dS
// with the query index (the contraction index) permuted within each group
// of 16: MFMA k-slot 8*g2 + t  <->  query 4*g2 + t (t < 4) or 8 + 4*g2 + t-4.
// The A operands dO^T and Q^T are read from transposed LDS copies stored in
// that same permuted order, so each is one 16-byte LDS read.  dQ = dS K
// needs dS with keys as the contraction index, so dS goes through LDS.
//
// LDS (D_pad = 128): Q, dO row-major 2 x 17 KB, Q^T, dO^T 2 x 18 KB, dS
// 17 KB, K^T 34 KB, two 256-byte row vectors: 121.5 KB per workgroup, one
// workgroup per CU.  Rows are padded by 16 bytes so that the 16-byte reads
// of 16 consecutive rows fall in distinct banks.
#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int DP>
struct Smem {
    static constexpr int RQ = DP + 8;       // row stride of q / dO (elements)
    static constexpr int RT = kQTile + 8;   // row stride of q^T / dO^T
    static constexpr int RS = kKTile + 8;   // row stride of dS / K^T
    uint16_t q[kQTile * RQ];
    uint16_t dO[kQTile * RQ];
    uint16_t qt[DP * RT];
    uint16_t dOt[DP * RT];
    uint16_t ds[kQTile * RS];
    uint16_t kt[DP * RS];
    float lse2[kQTile];
    float rowdot[kQTile];
};

// Slot of query row q (0..63) in the transposed copies: within each group of
// 16 rows the two middle groups of 4 swap places, so that k-slots
// 8*g2 .. 8*g2+7 of an MFMA step hold rows {4*g2..4*g2+3, 8+4*g2..8+4*g2+3}.
__device__ inline int qslot(int q)
{
    const int a = (q >> 2) & 3;
    const int na = ((a & 1) << 1) | (a >> 1);
    return (q & ~12) | (na << 2);
}

__device__ inline bf16x8 lds16(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

template <int DP>
__device__ inline void load_q_tile(const Params &p, Smem<DP> &sm, const uint16_t *qbase,
                                   const uint16_t *dobase, int rows_valid, int tid)
{
    constexpr int CPR = DP / 8;             // 16-byte chunks per row
    constexpr int NCH = kQTile * CPR;
    static_assert(NCH % kThreads == 0, "tile load must divide evenly");
#pragma unroll
    for (int it = 0; it < NCH / kThreads; ++it) {
        const int c = tid + it * kThreads;
        const int r = c / CPR, cc = c % CPR;
        uint4 vq = make_uint4(0, 0, 0, 0), vd = make_uint4(0, 0, 0, 0);
        if (r < rows_valid && cc * 8 < p.D) {
            vq = *reinterpret_cast<const uint4 *>(qbase + r * p.q_ss + cc * 8);
            vd = *reinterpret_cast<const uint4 *>(dobase + r * p.do_ss + cc * 8);
        }
        *reinterpret_cast<uint4 *>(&sm.q[r * Smem<DP>::RQ + cc * 8]) = vq;
        *reinterpret_cast<uint4 *>(&sm.dO[r * Smem<DP>::RQ + cc * 8]) = vd;
        const int slot = qslot(r);
        const uint32_t wq[4] = {vq.x, vq.y, vq.z, vq.w};
        const uint32_t wd[4] = {vd.x, vd.y, vd.z, vd.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int d = cc * 8 + 2 * t;
            sm.qt[d * Smem<DP>::RT + slot] = (uint16_t)(wq[t] & 0xffff);
            sm.qt[(d + 1) * Smem<DP>::RT + slot] = (uint16_t)(wq[t] >> 16);
            sm.dOt[d * Smem<DP>::RT + slot] = (uint16_t)(wd[t] & 0xffff);
            sm.dOt[(d + 1) * Smem<DP>::RT + slot] = (uint16_t)(wd[t] >> 16);
        }
    }
}

template <int DP>
__global__ void __launch_bounds__(kThreads, 1) fa_bwd_main_kernel(Params p)
{
    constexpr int KS = DP / 16;       // MFMA k-steps over the head dim
    constexpr int DB = DP / 32;       // 32-wide blocks of the head dim
    constexpr int RQ = Smem<DP>::RQ, RT = Smem<DP>::RT, RS = Smem<DP>::RS;
    __shared__ Smem<DP> sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

    // Workgroup -> (batch, KV head, key tile).  Within one (batch, KV head)
    // the key tiles run in descending order along the linear id, so that in
    // ordered mode every workgroup waits only on one with a lower id.
    const int nt = p.ntiles;
    const int lin = blockIdx.x;
    const int j = nt - 1 - (lin % nt);
    const int bg = lin / nt;
    const int hk = bg % p.Hk, b = bg / p.Hk;

    const SeqInfo si = seq_info(p, b);
    const int n0 = j * kKTile;
    if (n0 >= si.Lk)
        return;
    const int Lq = si.Lq, Lk = si.Lk;
    const int off = Lk - Lq;                // bottom-right causal offset
    const int key_local = w * 32 + l32;
    const int key = n0 + key_local;

    // ---- K, V fragments of this wave's 32 keys (B operands of S and dP) ----
    bf16x8 kf[KS], vf[KS];
    {
        const uint16_t *krow = p.k + row_offset(p, b, si.tok_k, key, p.k_sb, p.k_ss) + hk * p.k_sh;
        const uint16_t *vrow = p.v + row_offset(p, b, si.tok_k, key, p.v_sb, p.v_ss) + hk * p.v_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * g2;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (key < Lk && d0 < p.D) {
                kv = *reinterpret_cast<const uint4 *>(krow + d0);
                vv = *reinterpret_cast<const uint4 *>(vrow + d0);
            }
            kf[ks] = __builtin_bit_cast(bf16x8, kv);
            vf[ks] = __builtin_bit_cast(bf16x8, vv);
            // K^T in LDS for dQ = dS K (B operand: col d, 8 consecutive keys).
            const uint32_t wk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sm.kt[(d0 + 2 * t) * RS + key_local] = (uint16_t)(wk[t] & 0xffff);
                sm.kt[(d0 + 2 * t + 1) * RS + key_local] = (uint16_t)(wk[t] >> 16);
            }
        }
    }

    f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk_acc[db][r] = 0.f;
            dv_acc[db][r] = 0.f;
        }
    }

    const int first_q = p.causal ? max(0, n0 - off) : 0;
    if (first_q < Lq) {
        const int m_begin = first_q / kQTile;
        const int m_end = (Lq + kQTile - 1) / kQTile;
        const int nt_b = (Lk + kKTile - 1) / kKTile;
        for (int hh = 0; hh < p.G; ++hh) {
            const int h = hk * p.G + hh;
            const uint16_t *qhead = p.q + h * p.q_sh;
            const uint16_t *dohead = p.dout + h * p.do_sh;
            const int64_t wsbase = (int64_t)h * p.rows + si.ws_row;
            for (int m = m_begin; m < m_end; ++m) {
                const int q0 = m * kQTile;
                const int rows_valid = min(kQTile, Lq - q0);

                __syncthreads();   // previous tile fully consumed
                load_q_tile<DP>(p, sm,
                                qhead + row_offset(p, b, si.tok_q, q0, p.q_sb, p.q_ss),
                                dohead + row_offset(p, b, si.tok_q, q0, p.do_sb, p.do_ss),
                                rows_valid, tid);
                if (tid < kQTile) {
                    float l2 = INFINITY, rd = 0.f;
                    if (tid < rows_valid) {
                        l2 = p.lse2[wsbase + q0 + tid];
                        rd = p.rowdot[wsbase + q0 + tid];
                    }
                    sm.lse2[tid] = l2;
                    sm.rowdot[tid] = rd;
                }
                __syncthreads();

                // ---- S = Q K^T and dP = dO V^T (64 queries x 32 keys per wave) ----
                f32x16 s[2], dp[2];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        s[mb][r] = 0.f;
                        dp[mb][r] = 0.f;
                    }
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        const int row = (32 * mb + l32) * RQ + 16 * ks + 8 * g2;
                        s[mb] = mfma32(lds16(&sm.q[row]), kf[ks], s[mb]);
                        dp[mb] = mfma32(lds16(&sm.dO[row]), vf[ks], dp[mb]);
                    }
                }

                // ---- P, dS (fp32), masked; bf16 copies as MFMA B operands ----
                const bool need_mask =
                    (n0 + kKTile > Lk) || (p.causal && (n0 + kKTile - 1 > q0 + off));
                bf16x8 pb[4], dsb[4];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qi = 32 * mb + 8 * (r >> 2) + 4 * g2 + (r & 3);
                        float pv = __builtin_amdgcn_exp2f(s[mb][r] * p.scale_log2 - sm.lse2[qi]);
                        if (need_mask &&
                            (key >= Lk || (p.causal && key > q0 + qi + off)))
                            pv = 0.f;
                        const float dsv = pv * (dp[mb][r] - sm.rowdot[qi]);
                        const uint16_t pbits = f2bf(pv), dbits = f2bf(dsv);
                        pb[2 * mb + (r >> 3)][r & 7] = __builtin_bit_cast(__bf16, pbits);
                        dsb[2 * mb + (r >> 3)][r & 7] = __builtin_bit_cast(__bf16, dbits);
                        sm.ds[qi * RS + key_local] = dbits;
                    }
                }

                // ---- dV^T += dO^T P,  dK^T += Q^T dS  (k = 64 queries) ----
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int row = (32 * db + l32) * RT + 16 * kk + 8 * g2;
                        dv_acc[db] = mfma32(lds16(&sm.dOt[row]), pb[kk], dv_acc[db]);
                        dk_acc[db] = mfma32(lds16(&sm.qt[row]), dsb[kk], dk_acc[db]);
                    }
                }
                __syncthreads();   // dS of all four waves in LDS

                // ---- dQ partial = dS K: 2*DB blocks of 32x32 spread over 4 waves ----
                constexpr int NBLK = 2 * DB;
                constexpr int PERW = (NBLK + 3) / 4;
                f32x16 qacc[PERW];
#pragma unroll
                for (int u = 0; u < PERW; ++u) {
                    const int blk = w + 4 * u;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        qacc[u][r] = 0.f;
                    if (blk < NBLK) {
                        const int mb = blk & 1, db = blk >> 1;
#pragma unroll
                        for (int ks = 0; ks < kKTile / 16; ++ks) {
                            const bf16x8 a = lds16(&sm.ds[(32 * mb + l32) * RS + 16 * ks + 8 * g2]);
                            const bf16x8 bb = lds16(&sm.kt[(32 * db + l32) * RS + 16 * ks + 8 * g2]);
                            qacc[u] = mfma32(a, bb, qacc[u]);
                        }
                    }
                }

                int *turn = nullptr;
                if (p.deterministic) {
                    // Rank of this key tile among the tiles adding into query
                    // tile m, highest key tile first.
                    int jmax = nt_b - 1;
                    if (p.causal) {
                        const int lim = min(q0 + kQTile, Lq) + off;
                        jmax = min(jmax, (lim + kKTile - 1) / kKTile - 1);
                    }
                    const int rank = jmax - j;
                    turn = p.turns + ((int64_t)b * p.H + h) * p.mtiles + m;
                    if (tid == 0) {
                        int spins = 0;
                        while (__hip_atomic_load(turn, __ATOMIC_ACQUIRE,
                                                 __HIP_MEMORY_SCOPE_AGENT) != rank) {
                            __builtin_amdgcn_s_sleep(2);
                            if (++spins > kSpinLimit) {
                                __hip_atomic_fetch_or(p.flags, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                                break;
                            }
                        }
                    }
                    __syncthreads();
                }
#pragma unroll
                for (int u = 0; u < PERW; ++u) {
                    const int blk = w + 4 * u;
                    if (blk < NBLK) {
                        const int mb = blk & 1, db = blk >> 1;
                        const int d = 32 * db + l32;
                        if (d < p.D) {
                            float *dst = p.dq_acc + (wsbase + q0) * DP + d;
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int qi = 32 * mb + 8 * (r >> 2) + 4 * g2 + (r & 3);
                                if (qi < rows_valid)
                                    unsafeAtomicAdd(dst + (int64_t)qi * DP, qacc[u][r]);
                            }
                        }
                    }
                }
                if (p.deterministic) {
                    __threadfence();
                    __syncthreads();
                    if (tid == 0)
                        __hip_atomic_fetch_add(turn, 1, __ATOMIC_RELEASE,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }

    // ---- epilogue: dK = scale * acc, dV = acc, bf16, keys < Lk, d < D ----
    if (key < Lk) {
        uint16_t *dkrow = p.dk + row_offset(p, b, si.tok_k, key, p.dk_sb, p.dk_ss) + hk * p.dk_sh;
        uint16_t *dvrow = p.dv + row_offset(p, b, si.tok_k, key, p.dv_sb, p.dv_ss) + hk * p.dv_sh;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = 32 * db + 8 * r4 + 4 * g2;
                if (d < p.D) {
                    u16x4 kq, vq;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        kq[t] = f2bf(dk_acc[db][4 * r4 + t] * p.scale);
                        vq[t] = f2bf(dv_acc[db][4 * r4 + t]);
                    }
                    *reinterpret_cast<u16x4 *>(dkrow + d) = kq;
                    *reinterpret_cast<u16x4 *>(dvrow + d) = vq;
                }
            }
        }
    }
}

hipError_t launch_main(const Params &p, int dpad, hipStream_t st)
{
    const dim3 grid((unsigned)p.ntiles * p.Hk * p.batch);
    const dim3 block(kThreads);
    switch (dpad) {
    case 64:
        hipLaunchKernelGGL(fa_bwd_main_kernel<64>, grid, block, 0, st, p);
        break;
    case 96:
        hipLaunchKernelGGL(fa_bwd_main_kernel<96>, grid, block, 0, st, p);
        break;
    case 128:
        hipLaunchKernelGGL(fa_bwd_main_kernel<128>, grid, block, 0, st, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fa
