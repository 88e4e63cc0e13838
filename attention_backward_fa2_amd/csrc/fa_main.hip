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
// LDS (D_pad = 128): Q and dO tiles, double buffered (4 x 16 KB) in the
// swizzled unpadded layout of fa_mfma.h, plus lse2 / rowdot (1 KB): 65 KB;
// fused mode adds dS^T double buffered (2 x 20 KB) and K row-major (36 KB,
// pitch D + 16): 141 KB.  One workgroup per CU.
//
// Pipelining: the next query tile is loaded by buffer loads that write LDS
// directly (no staging registers, zero fill of tail rows / padded columns
// by the buffer bound) while the current one is computed; one workgroup
// barrier per tile, after the wave's loads have landed.  Within a tile the
// products are ordered so that the MFMA pipe always has independent work
// while the vector ALU computes P and dS: S and dP of query rows 0-31, then
// rows 32-63 alongside the pointwise math of rows 0-31, then the dV / dK
// k-steps over rows 0-31 alongside the pointwise math of rows 32-63, then
// the k-steps over rows 32-63.
#include <climits>
#include <type_traits>

#include "fa_mfma.h"

namespace fa {

template <int V>
using IC = std::integral_constant<int, V>;

// Query-side tile geometry in LDS.
template <int DP>
struct QTile {
    static constexpr int PCH = DP <= 64 ? 8 : 16;   // 16-byte chunks per LDS row
    static constexpr int PB = 16 * PCH;             // row pitch (bytes)
    static constexpr int BYTES = kQTile * PB;
    static constexpr int NLOAD = BYTES / 1024;      // 1 KB wave loads per tile
    static constexpr int PERW = NLOAD / 4;          // ... per wave
    static constexpr int RPL = 1024 / PB;           // rows per wave load
};

template <int DP>
struct __attribute__((aligned(16))) TileSmem {
    uint8_t q[2][QTile<DP>::BYTES];
    uint8_t dO[2][QTile<DP>::BYTES];
    float lse2[2][kQTile];
    float rowdot[2][kQTile];
};

template <int DP>
struct __attribute__((aligned(16))) FusedSmem : TileSmem<DP> {
    static constexpr int RQ = DP + 16;       // pitch of k (elements)
    static constexpr int RD = kQTile + 16;   // pitch of dS^T
    uint16_t dsT[2][kKTile * RD];
    uint16_t k[kKTile * RQ];
};

// P = exp2(S*scale*log2e - lse2) and dS = P (dP - rowdot) for query rows
// 32*mb .. 32*mb+31 of the tile (one accumulator block per product), as
// bf16 B operands pb[0..1] / dsb[0..1] of the k-steps over those rows, and
// (fused mode) the lane's dS^T row segment to LDS.  MASK: tile row qi sees
// this lane's key iff keyok && qi >= lim.
template <bool MASK, bool WRITE_DS>
__device__ inline void pointwise_half(const f32x16 &s, const f32x16 &dp, bf16x8 *pb, bf16x8 *dsb,
                                      uint16_t *dsT_row, const float *l2s, const float *rds,
                                      float scale_log2, int g2, int mb, int lim, bool keyok)
{
    // Accumulator rows 4*r4 .. 4*r4+3 are tile rows qi0 .. qi0+3 and
    // elements 4*(r4&1) .. +3 of operand r4/2.
    bf16x4 ph[4], dh[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        const int qi0 = 32 * mb + 8 * r4 + 4 * g2;
        const f32x4 l2v = *reinterpret_cast<const f32x4 *>(l2s + qi0);
        const f32x4 rdv = *reinterpret_cast<const f32x4 *>(rds + qi0);
        f32x4 pv, dv;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float e = __builtin_amdgcn_exp2f(s[4 * r4 + t] * scale_log2 - l2v[t]);
            if constexpr (MASK)
                e = (keyok && qi0 + t >= lim) ? e : 0.f;
            pv[t] = e;
            dv[t] = e * (dp[4 * r4 + t] - rdv[t]);
        }
        ph[r4] = to_bf16(pv);
        dh[r4] = to_bf16(dv);
        if constexpr (WRITE_DS)
            *reinterpret_cast<bf16x4 *>(dsT_row + qi0) = dh[r4];
    }
    pb[0] = concat(ph[0], ph[1]);
    pb[1] = concat(ph[2], ph[3]);
    dsb[0] = concat(dh[0], dh[1]);
    dsb[1] = concat(dh[2], dh[3]);
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
    constexpr int RQ = FusedSmem<DP>::RQ, RD = FusedSmem<DP>::RD;
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
    using L = QTile<DP>;
    using Smem = std::conditional_t<FUSED, FusedSmem<DP>, TileSmem<DP>>;
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

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
                *reinterpret_cast<u32x4 *>(&sm.k[key_local * FusedSmem<DP>::RQ + d0]) = kv;
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

        // Global byte offset of the 16-byte chunk each lane loads for wave
        // load i of this wave: LDS row pr, LDS chunk lane % PCH, which holds
        // tile chunk c = (lane % PCH) ^ swz(pr).  Chunks past head_dim (and
        // the unused chunks of a padded row) load zeros.
        uint32_t voq[L::PERW], vod[L::PERW];
#pragma unroll
        for (int i = 0; i < L::PERW; ++i) {
            const int pr = (w * L::PERW + i) * L::RPL + lane / L::PCH;
            const int c = (lane % L::PCH) ^ swz(pr);
            const bool ok = c * 8 < p.D;
            voq[i] = ok ? (uint32_t)(pr * (int)p.q_ss * 2 + c * 16) : kOutOfRange;
            vod[i] = ok ? (uint32_t)(pr * (int)p.do_ss * 2 + c * 16) : kOutOfRange;
        }
        // LDS byte offsets (within a tile) of this lane's operand reads:
        //  gq[k4]: 16-byte read of row l32, tile chunk 2*ks + g2 (ks % 4 = k4;
        //          + 128 bytes per 4 k-steps, + 32 rows per query block);
        //  tq[x]:  transposing read of rows 4*g2 + rr (+ 16 per k-step, + 8
        //          for the second half), tile chunk 4*x + 2*h16 + b1 (+ 128
        //          bytes per two head-dim blocks), 8-byte half c16 & 1.
        int gq[4], tq[2];
        {
            const int sw = swz(l32);
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4)
                gq[k4] = l32 * L::PB + (((2 * k4 + g2) ^ sw) << 4);
            const int c16 = lane & 15, rr = c16 >> 2, h16 = (lane >> 4) & 1, b1 = (c16 >> 1) & 1;
#pragma unroll
            for (int x = 0; x < 2; ++x)
                tq[x] = (4 * g2 + rr) * L::PB + (((4 * x + 2 * h16 + b1) ^ (2 * rr + g2)) << 4) +
                        (c16 & 1) * 8;
        }

        // Query tile of step `it`: heads of the group in turn; within a head
        // the last query tile first, so the workgroups of one (batch, KV
        // head) running side by side on an XCD read the same tile at about
        // the same time (L2 reuse).  Ordered dQ adds keep the ascending
        // order, in which no workgroup waits on its first tile.
        const bool ascending = FUSED && p.deterministic;
        auto tile_m = [&](int it) {
            const int r = it % nm;
            return ascending ? m_begin + r : m_end - 1 - r;
        };

        // Issue the loads of query tile `it` into LDS buffer BF.
        auto issue = [&](int it, auto bufc) {
            constexpr int BF = decltype(bufc)::value;
            const int hh = it / nm, m = tile_m(it);
            const int h = hk * p.G + hh;
            const int q0 = m * kQTile;
            const int rv = min(kQTile, Lq - q0);
            const uint16_t *qb = p.q + h * p.q_sh + row_offset(p, b, si.tok_q, q0, p.q_sb, p.q_ss);
            const uint16_t *db =
                p.dout + h * p.do_sh + row_offset(p, b, si.tok_q, q0, p.do_sb, p.do_ss);
            const auto rq = make_rsrc(qb, (uint32_t)((rv - 1) * (int)p.q_ss * 2 + p.D * 2));
            const auto rd = make_rsrc(db, (uint32_t)((rv - 1) * (int)p.do_ss * 2 + p.D * 2));
#pragma unroll
            for (int i = 0; i < L::PERW; ++i) {
                const int ld = (w * L::PERW + i) * 1024;
                load16_to_lds(rq, sm.q[BF] + ld, voq[i]);
                load16_to_lds(rd, sm.dO[BF] + ld, vod[i]);
            }
            if (w < 2) {
                const float *src = (w == 0 ? p.lse2 : p.rowdot) + (int64_t)h * p.rows + si.ws_row + q0;
                load4_to_lds(make_rsrc(src, (uint32_t)rv * 4), w == 0 ? sm.lse2[BF] : sm.rowdot[BF],
                               (uint32_t)lane * 4);
            }
        };

        // One query tile from LDS buffer BF; MASKED: causal / tail masking.
        auto body = [&](int it, auto bufc, auto maskc) {
            constexpr int BF = decltype(bufc)::value;
            constexpr bool MASKED = decltype(maskc)::value != 0;
            const int q0 = tile_m(it) * kQTile;
            const uint8_t *sq = sm.q[BF];
            const uint8_t *sdo = sm.dO[BF];
            const int lim = MASKED && p.causal ? key - q0 - off : INT_MIN;
            const bool keyok = key < Lk;
            uint16_t *dsrow = nullptr;
            if constexpr (FUSED)
                dsrow = &sm.dsT[BF][key_local * FusedSmem<DP>::RD];

            // S = Q K^T and dP = dO V^T, query rows 0-31 then 32-63.
            f32x16 s[2], dp[2];
            const f32x16 z = {};
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int o = gq[ks & 3] + 32 * mb * L::PB + 128 * (ks >> 2);
                    s[mb] = mfma32(lds16b(sq + o), kf[ks], ks == 0 ? z : s[mb]);
                    dp[mb] = mfma32(lds16b(sdo + o), vf[ks], ks == 0 ? z : dp[mb]);
                }
            }
            bf16x8 pb[4], dsb[4];
            pointwise_half<MASKED, FUSED>(s[0], dp[0], pb, dsb, dsrow, sm.lse2[BF], sm.rowdot[BF],
                                          p.scale_log2, g2, 0, lim, keyok);
            // dV^T += dO^T P, dK^T += Q^T dS over k-steps kk (16 query rows each).
            auto g35 = [&](int kk) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int o0 = tq[db & 1] + 16 * kk * L::PB + 128 * (db >> 1);
                    const int o1 = o0 + 8 * L::PB;
                    dv_acc[db] = mfma32(tr_pair(sdo + o0, sdo + o1), pb[kk], dv_acc[db]);
                    dk_acc[db] = mfma32(tr_pair(sq + o0, sq + o1), dsb[kk], dk_acc[db]);
                }
            };
            g35(0);
            g35(1);
            pointwise_half<MASKED, FUSED>(s[1], dp[1], pb + 2, dsb + 2, dsrow, sm.lse2[BF],
                                          sm.rowdot[BF], p.scale_log2, g2, 1, lim, keyok);
            g35(2);
            g35(3);

            // Instruction order: reads run ahead of the MFMAs that use them;
            // the pointwise math of each half fills the gaps between the
            // MFMAs of the next product block.
            constexpr int NB = 2 * KS;       // MFMAs per query block of S / dP
            constexpr int NG = 4 * DB;       // MFMAs per two k-steps of dV / dK
            sched<kSchedDsRead, 6>();
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                sched<kSchedMfma, 1>();
                sched<kSchedDsRead, 1>();
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                sched<kSchedMfma, 1>();
                sched<kSchedDsRead, 1>();
                sched<kSchedValu, 5>();
            }
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                sched<kSchedMfma, 1>();
                sched<kSchedDsRead, 2>();
                sched<kSchedValu, 5>();
            }
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                sched<kSchedMfma, 1>();
                sched<kSchedDsRead, 2>();
            }
        };

        // One pipeline step: loads of the next tile, this tile, barrier.
        auto step = [&](int it, auto bufc) {
            constexpr int BF = decltype(bufc)::value;
            if (it + 1 < total)
                issue(it + 1, IC<1 - BF>{});
            const int m = tile_m(it);
            const int q0 = m * kQTile;
            const bool need_mask =
                (n0 + kKTile > Lk) || (p.causal && (n0 + kKTile - 1 > q0 + off));
            if (need_mask)
                body(it, bufc, IC<1>{});
            else
                body(it, bufc, IC<0>{});
            wait_loads();
            __syncthreads();   // next tile in LDS; buffer BF free (fused: dS^T[BF] complete)
            if constexpr (FUSED) {
                const int h = hk * p.G + it / nm;
                const int rows_valid = min(kQTile, Lq - q0);
                dq_partial<DP>(p, sm, BF, w, lane, l32, g2, tid, b, h, m, j, q0, rows_valid, Lq,
                               off, nt_b, si.ws_row);
            }
        };

        issue(0, IC<0>{});
        wait_loads();
        __syncthreads();
        for (int it = 0; it < total; it += 2) {
            step(it, IC<0>{});
            if (it + 1 < total)
                step(it + 1, IC<1>{});
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
