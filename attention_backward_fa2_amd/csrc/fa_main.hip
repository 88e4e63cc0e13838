// fa_main.hip -- KV-stationary tile kernel of the attention backward on
// gfx950 (CDNA4): dK and dV, and in the fused mode also the dQ partials.
//
// One workgroup (4 wave64s) owns a tile of kKTile = 128 keys of one KV head
// (KV-tile-stationary order of the sm90 backward page: grid over key blocks,
// K and V loaded once, query tiles streamed).  It loops over every query head
// of the KV head's group and, for each, over the 64-row query tiles that can
// see at least one of its keys (causal block bound with the seqlen_k -
// seqlen_q offset of the GQA/MQA page).  Per query tile it runs the products
// of the sm90 backward page's mma_one_m_block on bf16 MFMA with fp32
// accumulation:
//     S  = Q K^T            dP = dO V^T
//     P  = exp2(S * scale * log2e - lse2)      (0 where masked)
//     dS = P * (dP - rowdot)
//     dV += P^T dO          dK += dS^T Q       (registers, whole group)
//   fused mode only:
//     dQ_partial = dS K  -> fp32 adds into the dQ accumulator
// dK and dV accumulate over all query heads of the group in registers, which
// is the GQA reduction of dK/dV (GQA/MQA page, backward section; backward
// call-trace page, sum over the head group) done without atomics.  dK gets
// the softmax scale once at the end (sm90 backward page, epilogue scaling).
//
// Each wave owns keys 32w .. 32w+31 of the tile; their K and V rows stay in
// registers as the B operands of S and dP.  With keys as the N index, the
// accumulators of P and dS are directly the B operands of dV^T = dO^T P and
// dK^T = Q^T dS (query index permuted as described in fa_mfma.h); dO^T and
// Q^T come from the row-major tiles through transposing LDS reads.  In fused
// mode dS^T goes through LDS for dQ = dS K.
//
// LDS (D_pad = 128): Q and dO row-major, double buffered (4 x 18 KB), row
// vectors 1 KB: 73 KB; fused mode adds dS^T double buffered (2 x 20 KB) and
// K row-major (36 KB): 149 KB.  One workgroup per CU.  Row pitches are
// D + 16 elements (dS^T: 64 + 16) so that both the 16-byte row reads and the
// transposing reads hit distinct banks.
//
// Pipelining: the next query tile is loaded from global memory into
// registers while the current one is computed and written to the other LDS
// buffer before any dQ atomic of the current tile is issued.  One workgroup
// barrier per tile: every LDS buffer written in tile t was last read before
// the barrier of tile t-1.
#include <climits>
#include <type_traits>

#include "fa_mfma.h"

namespace fa {

template <int DP>
struct __attribute__((aligned(16))) TileSmem {
    static constexpr int RQ = DP + 16;       // pitch of q / dO / k (elements)
    static constexpr int RD = kQTile + 16;   // pitch of dS^T
    uint16_t q[2][kQTile * RQ];
    uint16_t dO[2][kQTile * RQ];
    float lse2[2][kQTile];
    float rowdot[2][kQTile];
};

template <int DP>
struct __attribute__((aligned(16))) FusedSmem : TileSmem<DP> {
    uint16_t dsT[2][kKTile * TileSmem<DP>::RD];
    uint16_t k[kKTile * TileSmem<DP>::RQ];
};

// P = exp2(S*scale*log2e - lse2) and dS = P (dP - rowdot) for one wave's
// 64 x 32 tile; bf16 copies in MFMA B-operand order and (fused mode) the
// lane's dS^T row to LDS.  MASK: query row qi (0..63 in the tile) sees this
// lane's key iff keyok && qi >= lim.
template <bool MASK, bool WRITE_DS>
__device__ inline void pointwise(const f32x16 (&s)[2], const f32x16 (&dp)[2], bf16x8 (&pb)[4],
                                 bf16x8 (&dsb)[4], uint16_t *dsT_row, const float *l2s,
                                 const float *rds, float scale_log2, int g2, int lim, bool keyok)
{
    // Accumulator rows 4*r4 .. 4*r4+3 of block mb are tile rows qi0 .. qi0+3
    // and elements 4*(r4&1) .. +3 of operand 2*mb + r4/2.
    bf16x4 ph[8], dh[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int qi0 = 32 * mb + 8 * r4 + 4 * g2;
            const f32x4 l2v = *reinterpret_cast<const f32x4 *>(l2s + qi0);
            const f32x4 rdv = *reinterpret_cast<const f32x4 *>(rds + qi0);
            f32x4 pv, dv;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float e = __builtin_amdgcn_exp2f(s[mb][4 * r4 + t] * scale_log2 - l2v[t]);
                if constexpr (MASK)
                    e = (keyok && qi0 + t >= lim) ? e : 0.f;
                pv[t] = e;
                dv[t] = e * (dp[mb][4 * r4 + t] - rdv[t]);
            }
            ph[4 * mb + r4] = to_bf16(pv);
            dh[4 * mb + r4] = to_bf16(dv);
            if constexpr (WRITE_DS)
                *reinterpret_cast<bf16x4 *>(dsT_row + qi0) = dh[4 * mb + r4];
        }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        pb[kk] = concat(ph[2 * kk], ph[2 * kk + 1]);
        dsb[kk] = concat(dh[2 * kk], dh[2 * kk + 1]);
    }
}

// Fused mode: dQ partial of one query tile = dS K over this workgroup's 128
// keys, added into the fp32 accumulator -- unordered hardware atomics, or
// (ordered mode) in descending key-tile order behind a per-(batch, head,
// query tile) turn counter.
template <int DP>
__device__ inline void dq_partial(const Params &p, FusedSmem<DP> &sm, int buf, int w, int lane,
                                  int l32, int g2, int tid, int b, int h, int m, int j, int q0,
                                  int rows_valid, int Lq, int off, int nt_b, int64_t ws_row)
{
    constexpr int DB = DP / 32;
    constexpr int RQ = TileSmem<DP>::RQ, RD = TileSmem<DP>::RD;
    const int64_t wsbase = (int64_t)h * p.rows + ws_row;
                // ---- dQ partial = dS K: 2*DB blocks of 32x32 spread over 4 waves.
                //      DB = 4: wave w owns head-dim block w for both query blocks
                //      (one K fragment feeds two MFMAs); DB = 2: one block per
                //      wave; DB = 3: blocks w and w + 4 of (query block, head-dim
                //      block) = (blk / 3, blk % 3). ----
                constexpr int NBLK = 2 * DB;
                constexpr int PERW = (NBLK + 3) / 4;
                f32x16 qacc[PERW];
    #pragma unroll
                for (int u = 0; u < PERW; ++u)
    #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        qacc[u][r] = 0.f;
                auto qblk_mb = [&](int u) { return DB == 4 ? u : (DB == 2 ? (w >> 1) : (w + 4 * u) / 3); };
                auto qblk_db = [&](int u) { return DB == 4 ? w : (DB == 2 ? (w & 1) : (w + 4 * u) % 3); };
                if constexpr (DB == 4) {
    #pragma unroll
                    for (int ks = 0; ks < kKTile / 16; ++ks) {
                        const int r0 = 16 * ks + 8 * g2, r1 = r0 + 4;
                        const bf16x8 bk = frag_tr(sm.k, RQ, r0, r1, 32 * w, lane);
    #pragma unroll
                        for (int u = 0; u < 2; ++u)
                            qacc[u] = mfma32(frag_tr(sm.dsT[buf], RD, r0, r1, 32 * u, lane), bk, qacc[u]);
                    }
                    pipeline_reads<16, 3, 12>();
                } else if constexpr (DB == 2) {
    #pragma unroll
                    for (int ks = 0; ks < kKTile / 16; ++ks) {
                        const int r0 = 16 * ks + 8 * g2, r1 = r0 + 4;
                        qacc[0] = mfma32(frag_tr(sm.dsT[buf], RD, r0, r1, 32 * qblk_mb(0), lane),
                                         frag_tr(sm.k, RQ, r0, r1, 32 * qblk_db(0), lane), qacc[0]);
                    }
                    pipeline_reads<8, 4, 12>();
                } else {
    #pragma unroll
                    for (int u = 0; u < PERW; ++u) {
                        if (w + 4 * u < NBLK) {
    #pragma unroll
                            for (int ks = 0; ks < kKTile / 16; ++ks) {
                                const int r0 = 16 * ks + 8 * g2, r1 = r0 + 4;
                                qacc[u] = mfma32(frag_tr(sm.dsT[buf], RD, r0, r1, 32 * qblk_mb(u), lane),
                                                 frag_tr(sm.k, RQ, r0, r1, 32 * qblk_db(u), lane),
                                                 qacc[u]);
                            }
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
                        while (__hip_atomic_load(turn, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) !=
                               rank) {
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
                // fp32 adds of the partial: one 128-byte row segment per
                // (lane half, accumulator row); unconditional on full tiles.
    #pragma unroll
                for (int u = 0; u < PERW; ++u) {
                    if (w + 4 * u < NBLK) {
                        const int d = 32 * qblk_db(u) + l32;
                        float *dst = p.dq_acc + (wsbase + q0 + 32 * qblk_mb(u) + 4 * g2) * DP + d;
                        if (d < p.D) {
                            if (rows_valid == kQTile) {
    #pragma unroll
                                for (int r = 0; r < 16; ++r)
                                    unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * DP, qacc[u][r]);
                            } else {
                                const int lim_r = rows_valid - 32 * qblk_mb(u) - 4 * g2;
    #pragma unroll
                                for (int r = 0; r < 16; ++r)
                                    if (8 * (r >> 2) + (r & 3) < lim_r)
                                        unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * DP, qacc[u][r]);
                            }
                        }
                    }
                }
                if (p.deterministic) {
                    __threadfence();
                    __syncthreads();
                    if (tid == 0)
                        __hip_atomic_fetch_add(turn, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
}

template <int DP, bool FUSED>
__global__ void __launch_bounds__(kThreads, 1) fa_bwd_main_kernel(Params p)
{
    constexpr int KS = DP / 16;       // MFMA k-steps over the head dim
    constexpr int DB = DP / 32;       // 32-wide blocks of the head dim
    constexpr int RQ = TileSmem<DP>::RQ, RD = TileSmem<DP>::RD;
    constexpr int CPR = DP / 8;       // 16-byte chunks per tile row
    constexpr int NCH = kQTile * CPR / kThreads;   // chunks per thread per tile
    static_assert(kQTile * CPR % kThreads == 0, "tile load must divide evenly");
    using Smem = std::conditional_t<FUSED, FusedSmem<DP>, TileSmem<DP>>;
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

    // Workgroup -> (batch, KV head, key tile).
    //  - default: longest work first.  Key tile 0 sees the most query tiles
    //    under the causal mask, so all workgroups of key tile 0 (every batch
    //    and KV head) come first, then key tile 1, ...; the (batch, KV head)
    //    index is the fast one, which keeps one (batch, KV head) on one XCD
    //    of the round-robin dispatch when batch * Hk is a multiple of the
    //    XCD count.
    //  - ordered dQ adds: within one (batch, KV head) the key tiles run in
    //    descending order along the linear id, so every workgroup waits only
    //    on one with a lower id (which the in-order dispatch has already
    //    placed on a CU).
    const int nt = p.ntiles;
    const int nbg = p.batch * p.Hk;
    const int lin = blockIdx.x;
    int j, bg;
    if (FUSED && p.deterministic) {
        j = nt - 1 - (lin % nt);
        bg = lin / nt;
    } else {
        j = lin / nbg;
        bg = lin % nbg;
    }
    const int hk = bg % p.Hk, b = bg / p.Hk;

    const SeqInfo si = seq_info(p, b);
    const int n0 = j * kKTile;
    if (n0 >= si.Lk)
        return;
    const int Lq = si.Lq, Lk = si.Lk;
    const int off = Lk - Lq;                // bottom-right causal offset
    const int key_local = w * 32 + l32;
    const int key = n0 + key_local;

    // ---- K, V rows of this wave's 32 keys: B operands of S and dP; in
    //      fused mode the K tile also goes to LDS for dQ = dS K. ----
    bf16x8 kf[KS], vf[KS];
    {
        const uint16_t *krow = p.k + row_offset(p, b, si.tok_k, key, p.k_sb, p.k_ss) + hk * p.k_sh;
        const uint16_t *vrow = p.v + row_offset(p, b, si.tok_k, key, p.v_sb, p.v_ss) + hk * p.v_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * g2;
            u32x4 kv = 0, vv = 0;
            if (key < Lk && d0 < p.D) {
                kv = *reinterpret_cast<const u32x4 *>(krow + d0);
                vv = *reinterpret_cast<const u32x4 *>(vrow + d0);
            }
            kf[ks] = __builtin_bit_cast(bf16x8, kv);
            vf[ks] = __builtin_bit_cast(bf16x8, vv);
            if constexpr (FUSED)
                *reinterpret_cast<u32x4 *>(&sm.k[key_local * RQ + d0]) = kv;
        }
    }

    f32x16 dk_acc[DB], dv_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        zero(dk_acc[db]);
        zero(dv_acc[db]);
    }

    const int first_q = p.causal ? max(0, n0 - off) : 0;
    if (first_q < Lq) {
        const int m_begin = first_q / kQTile;
        const int m_end = (Lq + kQTile - 1) / kQTile;
        const int nm = m_end - m_begin;
        const int total = p.G * nm;
        const int nt_b = (Lk + kKTile - 1) / kKTile;
        // Prefetch registers for one query tile: NCH 16-byte chunks of Q
        // and of dO per thread, plus one lse2 / rowdot value pair.  Chunk c
        // of this thread is tile row (tid + c*256) / CPR, 16-byte column
        // (tid + c*256) % CPR.  Loads always use an in-bounds (clamped)
        // address; the zero fill of rows past the sequence end and of
        // columns past head_dim is applied when staging, so issuing a
        // prefetch never has to wait for older memory traffic.
        u32x4 pq[NCH], pd[NCH];
        float pl2 = INFINITY, prd = 0.f;
        int rv_next = kQTile;             // valid rows of the prefetched tile
        auto prefetch = [&](int it) {
            const int hh = it / nm, m = m_begin + it % nm;
            const int h = hk * p.G + hh;
            const int q0 = m * kQTile;
            rv_next = min(kQTile, Lq - q0);
            const uint16_t *qb =
                p.q + h * p.q_sh + row_offset(p, b, si.tok_q, q0, p.q_sb, p.q_ss);
            const uint16_t *db =
                p.dout + h * p.do_sh + row_offset(p, b, si.tok_q, q0, p.do_sb, p.do_ss);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int idx = tid + c * kThreads;
                const int r = min(idx / CPR, rv_next - 1);
                const int col = (idx % CPR) * 8 < p.D ? (idx % CPR) * 8 : 0;
                pq[c] = *reinterpret_cast<const u32x4 *>(qb + r * (int)p.q_ss + col);
                pd[c] = *reinterpret_cast<const u32x4 *>(db + r * (int)p.do_ss + col);
            }
            const int lr = min(tid & (kQTile - 1), rv_next - 1);
            const int64_t wr = (int64_t)h * p.rows + si.ws_row + q0 + lr;
            pl2 = p.lse2[wr];
            prd = p.rowdot[wr];
        };
        auto stage = [&](int buf) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int idx = tid + c * kThreads;
                const uint32_t keep = (idx / CPR < rv_next && (idx % CPR) * 8 < p.D) ? ~0u : 0u;
                const int o = (idx / CPR) * RQ + (idx % CPR) * 8;
                *reinterpret_cast<u32x4 *>(&sm.q[buf][o]) = pq[c] & keep;
                *reinterpret_cast<u32x4 *>(&sm.dO[buf][o]) = pd[c] & keep;
            }
            if (tid < kQTile) {
                const bool ok = tid < rv_next;
                sm.lse2[buf][tid] = ok ? pl2 : INFINITY;
                sm.rowdot[buf][tid] = ok ? prd : 0.f;
            }
        };

        prefetch(0);
        stage(0);
        __syncthreads();

        for (int it = 0; it < total; ++it) {
            const int buf = it & 1;
            const int hh = it / nm, m = m_begin + it % nm;
            const int h = hk * p.G + hh;
            const int q0 = m * kQTile;
            const int rows_valid = min(kQTile, Lq - q0);
            if (it + 1 < total)
                prefetch(it + 1);
            const uint16_t *sq = sm.q[buf];
            const uint16_t *sdo = sm.dO[buf];

            // ---- S = Q K^T and dP = dO V^T (64 queries x 32 keys per wave) ----
            f32x16 s[2], dp[2];
            const f32x16 z = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int o = (32 * mb + l32) * RQ + 16 * ks + 8 * g2;
                    s[mb] = mfma32(lds16(sq + o), kf[ks], ks == 0 ? z : s[mb]);
                    dp[mb] = mfma32(lds16(sdo + o), vf[ks], ks == 0 ? z : dp[mb]);
                }
            }
            pipeline_reads<4 * KS, 1, 8>();

            // ---- P, dS (fp32), masked only on diagonal / tail tiles ----
            const bool need_mask =
                (n0 + kKTile > Lk) || (p.causal && (n0 + kKTile - 1 > q0 + off));
            bf16x8 pb[4], dsb[4];
            uint16_t *dsrow = nullptr;
            if constexpr (FUSED)
                dsrow = &sm.dsT[buf][key_local * RD];
            if (need_mask) {
                // causal: key visible to tile row qi iff key <= q0 + qi + off
                const int lim = p.causal ? key - q0 - off : INT_MIN;
                pointwise<true, FUSED>(s, dp, pb, dsb, dsrow, sm.lse2[buf], sm.rowdot[buf],
                                       p.scale_log2, g2, lim, key < Lk);
            } else {
                pointwise<false, FUSED>(s, dp, pb, dsb, dsrow, sm.lse2[buf], sm.rowdot[buf],
                                        p.scale_log2, g2, 0, true);
            }

            // ---- dV^T += dO^T P,  dK^T += Q^T dS  (k = 64 queries) ----
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r0 = 16 * kk + 4 * g2, r1 = r0 + 8;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dv_acc[db] = mfma32(frag_tr(sdo, RQ, r0, r1, 32 * db, lane), pb[kk], dv_acc[db]);
                    dk_acc[db] = mfma32(frag_tr(sq, RQ, r0, r1, 32 * db, lane), dsb[kk], dk_acc[db]);
                }
            }
            pipeline_reads<8 * DB, 2, 8>();

            // Stage the prefetched next tile now, before this tile's dQ
            // atomics are issued, so waiting for its loads never waits for
            // the atomics.  Buffer buf^1 was last read before the previous
            // barrier.
            if (it + 1 < total)
                stage(buf ^ 1);
            __syncthreads();   // next tile staged (fused: dS^T[buf] complete)

            if constexpr (FUSED)
                dq_partial<DP>(p, sm, buf, w, lane, l32, g2, tid, b, h, m, j, q0, rows_valid, Lq,
                               off, nt_b, si.ws_row);
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
#define FA_LAUNCH_MAIN(D)                                                              \
    if (p.fused_dq)                                                                    \
        hipLaunchKernelGGL((fa_bwd_main_kernel<D, true>), grid, block, 0, st, p);      \
    else                                                                               \
        hipLaunchKernelGGL((fa_bwd_main_kernel<D, false>), grid, block, 0, st, p);
    switch (dpad) {
    case 64:
        FA_LAUNCH_MAIN(64);
        break;
    case 96:
        FA_LAUNCH_MAIN(96);
        break;
    case 128:
        FA_LAUNCH_MAIN(128);
        break;
    default:
        return hipErrorInvalidValue;
    }
#undef FA_LAUNCH_MAIN
    return hipGetLastError();
}

}  // namespace fa
