// fa_main.hip -- KV-stationary tile kernel of the attention backward on
// gfx950 (CDNA4): dK and dV, and in the fused mode also the dQ partials.
//
// One workgroup (4 wave64s) owns a tile of kKTile = 128 keys of one KV head
// (64 at head dims above 128, see BIG below)
// (KV-tile-stationary order of the sm90 backward page: grid over key blocks,
// K and V loaded once, query tiles streamed).  It loops over every query head
// of the KV head's group and, for each, over the 64-row query tiles that can
// see at least one of its keys (causal block bound with the seqlen_k -
// seqlen_q offset of the GQA/MQA page; with a local window of mha_bwd's
// window_size_left / _right on the backward call-trace page, the query
// rows whose window meets the tile).  Per query tile it runs the products
// of the sm90 backward page's mma_one_m_block on bf16 MFMA with fp32
// accumulation:
//     S  = Q K^T            dP = dO V^T
//     P  = exp2(S * scale * log2e - lse2)      (0 where masked)
//     dS = P * (dP - rowdot)   (the dP product starts from rowdot, with -V)
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
#include "fa_philox.h"

#ifndef FA_TU_SOFTCAP
#define FA_TU_SOFTCAP 0
#endif
#ifndef FA_TU_DROPOUT
#define FA_TU_DROPOUT 0
#endif

namespace fa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One query tile in LDS: Q and dO in the swizzled layout, lse2, rowdot.
template <int DP>
struct __attribute__((aligned(16))) QBuf {
    uint8_t q[Tile64<DP>::BYTES];
    uint8_t dO[Tile64<DP>::BYTES];
    float lse2[kQTile];
    float rowdot[kQTile];
};

// With dropout in the separate-dQ mode a tile also carries each wave's keep
// words: the word of the wave's 32 keys for each of the 64 rows.
template <int DP>
struct __attribute__((aligned(16))) QBufKeep : QBuf<DP> {
    uint32_t keep[kThreads / 64][kQTile];
};

template <int DP, int NBUF, bool KEEP = false>
struct __attribute__((aligned(16))) TileSmem {
    std::conditional_t<KEEP, QBufKeep<DP>, QBuf<DP>> buf[NBUF];
};

// Head dims above 128: the P and dS operands each wave hands to the other
// wave of its pair, [wave][P, dS][k-step of the wave's query block][lane],
// 16 bytes each.
template <int DP, int NBUF, bool KEEP>
struct __attribute__((aligned(16))) PairSmem : TileSmem<DP, NBUF, KEEP> {
    uint8_t xch[kThreads / 64][2][2][64 * 16];
};

template <int DP>
struct __attribute__((aligned(16))) FusedSmem : TileSmem<DP, 2> {
    static constexpr int RQ = DP + 16;       // pitch of k (elements)
    static constexpr int RD = kQTile + 16;   // pitch of dS^T
    uint16_t dsT[2][kKTile * RD];
    uint16_t k[kKTile * RQ];
};

// Fused mode: dQ partial of one query tile = dS K over this workgroup's 128
// keys, added into the fp32 accumulator -- unordered hardware atomics, or
// (ordered mode) in descending key-tile order behind a per-(batch, head,
// query tile) turn counter.
template <int DP, bool F16>
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
                        const e16x8 bk = frag_tr(sm.k, RQ, r0, r1, 32 * w, lane);
    #pragma unroll
                        for (int u = 0; u < 2; ++u)
                            qacc[u] = mfma32<F16>(frag_tr(sm.dsT[buf], RD, r0, r1, 32 * u, lane), bk, qacc[u]);
                    }
                    pipeline_reads<16, 3, 12>();
                } else if constexpr (DB == 2) {
    #pragma unroll
                    for (int ks = 0; ks < kKTile / 16; ++ks) {
                        const int r0 = 16 * ks + 8 * g2, r1 = r0 + 4;
                        qacc[0] = mfma32<F16>(frag_tr(sm.dsT[buf], RD, r0, r1, 32 * qblk_mb(0), lane),
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
                                qacc[u] = mfma32<F16>(frag_tr(sm.dsT[buf], RD, r0, r1, 32 * qblk_mb(u), lane),
                                                 frag_tr(sm.k, RQ, r0, r1, 32 * qblk_db(u), lane),
                                                 qacc[u]);
                            }
                        }
                    }
                }

                int *turn = nullptr;
                if (p.deterministic) {
                    // Rank of this key tile among the tiles adding into query
                    // tile m, highest key tile first (the last row of the tile
                    // sees keys up to lim, which this key tile reaches).
                    int jmax = nt_b - 1;
                    if (p.win_r >= 0) {
                        const int lim = min(q0 + kQTile, Lq) - 1 + off + p.win_r;
                        jmax = min(jmax, lim / kKTile);
                    }
                    const int rank = jmax - j;
                    turn = p.turns + ((int64_t)b * p.H + h) * p.mtiles + m;
                    // Wait while the turn is below this tile's rank (a late
                    // add of a workgroup that gave up can push the counter
                    // past a rank, which must then not wait forever).  The
                    // polls are relaxed: this workgroup reads nothing the
                    // lower ranks wrote, it only adds into the accumulator
                    // with atomics, which are never served from a stale
                    // cache line, so an acquire (an invalidation of the XCD's
                    // L2 per poll) would protect nothing.
                    if (tid == 0) {
                        int spins = 0;
                        while (__hip_atomic_load(turn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
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
                    // The next rank may add once every wave's adds are done:
                    // each wave waits for its atomics to complete, then the
                    // turn moves on.  (No release fence: the accumulator is
                    // written by atomics only, which are performed at the
                    // device's coherence point, so a write-back of the XCD's
                    // L2 would publish nothing; it cost a factor of ~4 here.)
                    wait_loads<0>();
                    __syncthreads();
                    if (tid == 0)
                        __hip_atomic_fetch_add(turn, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
}

// LOCAL: a left window bounds the visible keys from below (win_l >= 0);
// otherwise win_l < 0 and only the upper bound is masked.  SOFTCAP: scores
// soft-capped (softcap > 0).  DROP: dropout replayed from the forward's rng
// state (drop_p > 0), 1: the keep bits drawn here, 2: read from the words
// the dQ kernel wrote.
template <int DP, bool FUSED, bool F16, bool LOCAL, bool SOFTCAP, int DROP>
__global__ void __launch_bounds__(kThreads, 1) fa_bwd_main_kernel(Params p)
{
    constexpr int KS = DP / 16;       // MFMA k-steps over the head dim
    constexpr int DB = DP / 32;       // 32-wide blocks of the head dim
    using L = Tile64<DP>;
    // Head dims above 128: a wave's dK and dV accumulators over the whole
    // head dim and its K, V operands would need more than a SIMD's 512
    // registers, so each pair of waves shares 32 keys (64 keys per
    // workgroup) and splits the work: wave w & 1 of a pair computes S, dP,
    // P and dS of query block w & 1 (rows 32 (w & 1) .. +31) of each tile
    // over the whole head dim, the two waves trade their P and dS operands
    // through LDS, and each accumulates dK and dV of its half of the head
    // dim over all 64 rows.  The fused dQ modes are not built for them.
    constexpr bool BIG = DP > 128;
    static_assert(!(BIG && FUSED), "fused dQ for head dims above 128");
    constexpr int KT = BIG ? 64 : kKTile;    // keys per workgroup
    constexpr int DBL = BIG ? DB / 2 : DB;   // dK / dV head-dim blocks of a wave
    // Query-tile buffers in flight: three (loads run two tiles ahead) unless
    // the fused mode's dS^T and K tiles, or tiles of more than 128 columns,
    // leave LDS room for only two; then each tile loads the next one at its
    // start and waits for it at its end.
    constexpr bool TWO = FUSED || BIG;
    constexpr int NBUF = TWO ? 2 : 3;
    // Dropout keep bits: drawn here in the fused mode, else read from the
    // words the dQ kernel (which runs first) wrote.
    constexpr bool KEEP = DROP == 2;
    static_assert(!(KEEP && FUSED), "the fused modes draw the keep bits");
    using Smem = std::conditional_t<
        FUSED, FusedSmem<DP>,
        std::conditional_t<BIG, PairSmem<DP, NBUF, KEEP>, TileSmem<DP, NBUF, KEEP>>>;
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;
    const int kgrp = BIG ? w >> 1 : w;               // the wave's 32 keys
    const int dbo = BIG ? (w & 1) * DBL : 0;         // first dK / dV head-dim block

    // Workgroup -> (batch, KV head, key tile).
    //  - default: longest work first.  Key tile 0 sees the most query tiles
    //    under the causal mask, so within the (batch, KV head) groups an XCD
    //    runs side by side, key tile 0 comes first, then key tile 1, ...
    //    (xcd_group_order: one (batch, KV head) stays on one XCD when batch *
    //    Hk is a multiple of the XCD count, and the workgroups running on
    //    an XCD together share few groups' Q / dO streams).
    //  - ordered dQ adds: within one (batch, KV head) the key tiles run in
    //    descending order along the linear id, so every workgroup waits only
    //    on one with a lower id (which the in-order dispatch has already
    //    placed on a CU).
    const int nt = BIG ? (p.Sk + KT - 1) / KT : p.ntiles;
    const int nbg = p.batch * p.Hk;
    const int lin = blockIdx.x;
    int j, bg;
    if (FUSED && p.deterministic) {
        j = nt - 1 - (lin % nt);
        bg = lin / nt;
    } else {
        xcd_group_order(lin, nbg, nt, j, bg);
    }
    const int hk = bg % p.Hk, b = bg / p.Hk;

    const SeqInfo si = seq_info(p, b);
    const int n0 = j * KT;
    if (n0 >= si.Lk)
        return;
    const int Lq = si.Lq, Lk = si.Lk;
    const int off = Lk - Lq;                // bottom-right alignment offset
    const int key_local = kgrp * 32 + l32;
    const int key = n0 + key_local;

    // ---- K, V rows of this wave's 32 keys: B operands of S and dP; in
    //      fused mode the K tile also goes to LDS for dQ = dS K. ----
    e16x8 kf[KS], vf[KS];
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
            kf[ks] = __builtin_bit_cast(e16x8, kv);
            // -V: the dP product then starts from rowdot and yields
            // rowdot - dP (sign flips are exact in bf16)
            vf[ks] = __builtin_bit_cast(e16x8, vv ^ 0x80008000u);
            if constexpr (FUSED)
                *reinterpret_cast<u32x4 *>(&sm.k[key_local * FusedSmem<DP>::RQ + d0]) = kv;
        }
        // Land them before the tile loop: the loop's own loads are not
        // tracked by the compiler, so a wait for these inside the loop
        // would also wait for the query-tile prefetch.
        wait_loads<0>();
    }

    f32x16 dk_acc[DBL], dv_acc[DBL];
#pragma unroll
    for (int db = 0; db < DBL; ++db) {
        zero(dk_acc[db]);
        zero(dv_acc[db]);
    }

    // Query rows first_q .. last_q see some key of this tile (query row i
    // sees keys i + off - win_l .. i + off + win_r).
    const int first_q = p.win_r >= 0 ? max(0, n0 - off - p.win_r) : 0;
    const int last_q =
        LOCAL ? min(Lq - 1, min(Lk - 1, n0 + KT - 1) - off + p.win_l) : Lq - 1;
    if (first_q <= last_q) {
        const int m_begin = first_q / kQTile;
        const int m_end = last_q / kQTile + 1;
        const int nm = m_end - m_begin;
        const int total = p.G * nm;
        const int nt_b = (Lk + KT - 1) / KT;

        // Tile loads: waves 0 and 1 load the Q tile, waves 2 and 3 the dO
        // tile (half a tile, 2 PERW wave loads, each), so that every wave
        // moves one row pointer and forms one descriptor per tile.  Global
        // byte offset of the 16-byte chunk each lane loads for wave load i
        // of this wave: LDS row pr, LDS chunk lane % PCH, which holds tile
        // chunk c = (lane % PCH) ^ swz(pr).  Chunks past head_dim (and the
        // unused chunks of a padded row) load zeros.
        constexpr int MLD = 2 * L::PERW;        // Q or dO wave loads of a wave
        const bool dow = w >= 2;                // (wave-uniform)
        const int mss = dow ? (int)p.do_ss : (int)p.q_ss;
        const int64_t msh = dow ? p.do_sh : p.q_sh;
        // LDS byte offset of the wave's first load in a tile buffer (Q then
        // dO in the buffer)
        const int mlds = (dow ? L::BYTES : 0) + (w & 1) * MLD * 1024;
        uint32_t vom[MLD];
#pragma unroll
        for (int i = 0; i < MLD; ++i) {
            const int pr = ((w & 1) * MLD + i) * L::RPL + lane / L::PCH;
            const int c = (lane % L::PCH) ^ swz<L::PCH>(pr);
            const bool ok = c * 8 < p.D;
            vom[i] = ok ? (uint32_t)(pr * mss * 2 + c * 16) : kOutOfRange;
        }

        // LDS byte offsets of this lane's operand reads in the current
        // buffer (the swizzle reaches every bit of the chunk index, so there
        // is one offset per k-step / head-dim block; dO is BYTES further):
        //  gq[ks]:    16-byte read of Q row l32, tile chunk 2*ks + g2 (+ 32
        //             rows per query block);
        //  tq[db][h]: transposing read of rows 4*g2 + rr + 8*h (+ 16 rows per
        //             k-step), tile chunk 4*db + 2*h16 + b1, 8-byte half
        //             c16 & 1;
        //  rv0:       lse2 / rowdot of row 4*g2.
        // All move to the next buffer (cyclically) after each tile.
        using Buf = std::conditional_t<KEEP, QBufKeep<DP>, QBuf<DP>>;
        constexpr int BUFB = (int)sizeof(Buf);
        int gq[KS], tq[DBL][2], rv0, kv0 = 0;
        {
            const int sw = swz<L::PCH>(l32);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gq[ks] = l32 * L::PB + (((2 * ks + g2) ^ sw) << 4);
            const int c16 = lane & 15, rr = c16 >> 2, h16 = (lane >> 4) & 1, b1 = (c16 >> 1) & 1;
#pragma unroll
            for (int db = 0; db < DBL; ++db)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int row = 4 * g2 + rr + 8 * hf;
                    tq[db][hf] = row * L::PB +
                                 (((4 * (dbo + db) + 2 * h16 + b1) ^ swz<L::PCH>(row)) << 4) +
                                 (c16 & 1) * 8;
                }
            rv0 = 2 * L::BYTES + 16 * g2;
            if constexpr (KEEP)   // keep word of row 4*g2 of the wave's rows
                kv0 = (int)sizeof(QBuf<DP>) + w * 4 * kQTile + 16 * g2;
        }
        // Head dims above 128: the wave's own query block mbr enters the
        // 16-byte reads, the row vectors and keep words, and the
        // transposing reads of its own two k-steps (tq); tqp reads the two
        // k-steps of the other wave's block.
        const int mbr = BIG ? (w & 1) : 0;
        int tqp[DBL][2];
        if constexpr (BIG) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gq[ks] += 32 * mbr * L::PB;
#pragma unroll
            for (int db = 0; db < DBL; ++db)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    tqp[db][hf] = tq[db][hf] + 32 * (1 - mbr) * L::PB;
                    tq[db][hf] += 32 * mbr * L::PB;
                }
            rv0 += 128 * mbr;
            kv0 += 128 * mbr;
        }
        const uint8_t *lds = reinterpret_cast<const uint8_t *>(&sm.buf[0]);

        // Order of the query tiles: the last query tile first, and at each
        // query tile the heads of the group in turn.  Every key tile starts
        // at the same (last) query tile and moves down one tile per G steps,
        // so the workgroups of one (batch, KV head) running side by side on
        // an XCD read the same Q / dO tiles at about the same time (L2
        // reuse), however many tiles each sees.  (Head by head, workgroups
        // that see fewer tiles would move on to the next head early and the
        // group would read up to G heads at once.)  Ordered dQ adds go up
        // from the first query tile instead, in which order no workgroup
        // waits on its first tile unless a right window reaches into the
        // next key tile.  dK and dV sum in the same order in every mode
        // except the ordered one.
        const bool ascending = FUSED && p.deterministic;

        // Loads of the query tiles into LDS, strictly in the order they are
        // computed: issue(bf) loads the next tile into buffer bf.  Past the
        // last tile the loads are issued with an empty bound (no memory
        // access, zeros written) so that the tile loop has no branch.  The
        // tile's row pointers advance incrementally (scalar registers): the
        // next head at the same query tile, and after the last head the
        // first head one query tile further.
        const int q0_first = (ascending ? m_begin : m_end - 1) * kQTile;
        const int dq0 = ascending ? kQTile : -kQTile;
        const int h0 = hk * p.G;
        // the wave's tensor (Q or dO) at the group's first head
        const uint16_t *nm_head =
            dow ? p.dout + row_offset(p, b, si.tok_q, q0_first, p.do_sb, p.do_ss) + h0 * p.do_sh
                : p.q + row_offset(p, b, si.tok_q, q0_first, p.q_sb, p.q_ss) + h0 * p.q_sh;
        // lse2 (even waves) / rowdot (odd waves), see below
        const float *nr_head = ((w & 1) ? p.rowdot : p.lse2) + si.ws_row + (int64_t)h0 * p.rows + q0_first;
        const uint16_t *nm_ptr = nm_head;
        const float *nr_ptr = nr_head;
        // The keep words of the wave's 32 keys (word (n0 + 32 kgrp) / 32)
        // sit a fixed distance from the row vectors of the same (head, row)
        // (both arrays are [.][head][row] of 4-byte values in the workspace).
        int64_t kdelta = 0;
        if constexpr (KEEP) {
            const int kwi = (n0 >> 5) + kgrp;
            kdelta = reinterpret_cast<const char *>(p.keep + (int64_t)kwi * p.H * p.rows) -
                     reinterpret_cast<const char *>((w & 1) ? p.rowdot : p.lse2);
        }
        int n_r = 0, n_q0 = q0_first, n_left = total;
        const int64_t step_m = (int64_t)dq0 * mss;
        // Buffer descriptors of the next tile (bounded by its valid rows),
        // formed in parts (the wave's Q or dO, row vectors) that can sit in
        // different MFMA slots.
        u32x4_rsrc rm_n, rr_n, rk_n;
        int n_rv = 0;
        auto prep_part = [&](auto pc) {
            constexpr int part = decltype(pc)::value;
            if constexpr (part == 0) {
                keep_scalar_here(n_left, n_q0, nm_ptr);
                n_rv = n_left > 0 ? min(kQTile, Lq - n_q0) : 0;
                const uint32_t nb = n_rv ? (uint32_t)((n_rv - 1) * mss * 2 + p.D * 2) : 0u;
                rm_n = make_rsrc(nm_ptr, nb);
                keep_scalar_here(rm_n, n_rv);
            } else if constexpr (part == 1) {
                // (the second tensor's part: the other waves')
            } else {
                keep_scalar_here(n_rv, nr_ptr);
                rr_n = make_rsrc(nr_ptr, (uint32_t)n_rv * 4);
                keep_scalar_here(rr_n);
                if constexpr (KEEP) {
                    rk_n = make_rsrc(reinterpret_cast<const char *>(nr_ptr) + kdelta,
                                     (uint32_t)n_rv * 4);
                    keep_scalar_here(rk_n);
                }
            }
        };
        // Loads per wave per tile (each Q / dO wave load, lse2 / rowdot, and
        // the keep words).
        constexpr int LPT = MLD + 1 + (KEEP ? 1 : 0);
        // Load j of the next tile into buffer bf.
        auto issue_one = [&](auto jc, int bf) {
            constexpr int j = decltype(jc)::value;
            Buf &qbuf = sm.buf[bf];
            if constexpr (j < MLD) {
                load16_to_lds(rm_n, reinterpret_cast<uint8_t *>(&qbuf) + mlds + j * 1024, vom[j]);
            } else if constexpr (j == MLD) {
                // lse2 (even waves) / rowdot (odd waves): the two waves of a
                // kind write the same values.
                load4_to_lds(rr_n, (w & 1) ? qbuf.rowdot : qbuf.lse2, (uint32_t)lane * 4);
            } else if constexpr (KEEP) {
                load4_to_lds(rk_n, qbuf.keep[w], (uint32_t)lane * 4);
            }
        };
        // Move the row pointers on to the tile after (branch-free selects),
        // in three parts like the descriptors.
        int n_wrap = 0;
        // (nm_head, nr_head: the group's first head at the current
        // query tile.)
        auto advance_part = [&](auto pc) {
            constexpr int part = decltype(pc)::value;
            if constexpr (part == 0) {
                keep_scalar_here(n_left, n_r, n_q0);
                --n_left;
                n_wrap = __builtin_amdgcn_readfirstlane(n_r == p.G - 1 ? 1 : 0);   // scalar
                n_r = n_wrap ? 0 : n_r + 1;
                n_q0 = n_wrap ? n_q0 + dq0 : n_q0;
                keep_scalar_here(n_left, n_r, n_q0, n_wrap);
            } else if constexpr (part == 1) {
                keep_scalar_here(n_wrap, nm_head, nm_ptr);
                nm_head = n_wrap ? nm_head + step_m : nm_head;
                nm_ptr = n_wrap ? nm_head : nm_ptr + msh;
                keep_scalar_here(nm_head, nm_ptr);
            } else {
                keep_scalar_here(n_wrap, nr_head, nr_ptr);
                nr_head = n_wrap ? nr_head + dq0 : nr_head;
                nr_ptr = n_wrap ? nr_head : nr_ptr + p.rows;
                keep_scalar_here(nr_head, nr_ptr);
            }
        };
        // Advance and prepare parts in order: three of each.
        auto setup_part = [&](auto pc) {
            constexpr int part = decltype(pc)::value;
            if constexpr (part < 3)
                advance_part(IC<part>{});
            else
                prep_part(IC<part - 3>{});
        };
        // All loads of the next tile at once, then prepare the one after.
        auto issue = [&](int bf) {
            static_for<LPT>([&](auto jc) { issue_one(jc, bf); });
            static_for<6>([&](auto pc) { setup_part(pc); });
        };

        static_for<3>([&](auto pc) { prep_part(pc); });
#pragma unroll
        for (int t = 0; t < NBUF - 1; ++t)
            issue(t);
        wait_loads<LPT * (NBUF - 2)>();
        __syncthreads();

        // ---- Each query tile as NSLOT MFMA slots, issued in this order: ----
        //   S, dP  of rows 0-31 (k-steps over D)      slots 0 .. NB-1
        //   S, dP  of rows 32-63                      NB .. 2NB-1       + P, dS of rows 0-31
        //   dV, dK over rows 0-31 (k-steps 0, 1)      2NB .. 2NB+NG-1   + P, dS of rows 32-63
        //   dV, dK over rows 32-63 (k-steps 2, 3)     2NB+NG .. NSLOT-1
        // Each slot issues the LDS operand read of the slot RA ahead, its
        // MFMA and a share of the vector work; a scheduling fence after
        // every slot keeps this order.  Without the fused dQ, the reads run
        // ahead across the tile boundary, and the wait for the next tile's
        // loads, the workgroup barrier, the loads of the tile after next and
        // their scalar set-up sit early in the tile, in the shadow of the S /
        // dP products, which leave most issue slots free (with three buffers,
        // a buffer refilled after the barrier of tile t held tile t-1, which
        // every wave has finished by then).
        constexpr int NB = 2 * KS;            // S / dP MFMAs per query block
        constexpr int NG = 4 * DBL;           // dV / dK MFMAs per two k-steps
        constexpr int NSLOT = 2 * NB + 2 * NG;
        constexpr int RA = 8;                 // read-ahead distance (slots)
        // Pointwise slots (below): block 0 over NB .. P0E-1, block 1 over
        // P0E .. P1E-1.  Element 7 of a block must be packed before its
        // first dV / dK k-step (2NB, 2NB + NG), element 15 before its second
        // (2NB + NG/2, 2NB + 3NG/2), and block 1 starts after its S / dP.
        constexpr int P0E = 2 * NB + NG / 8;
        constexpr int P1E = 2 * NB + 3 * NG / 2 - NG / 8;
        static_assert(P0E >= 2 * NB && P0E <= 2 * NB + NG / 2 - 1 &&
                          NB + 7 * (P0E - NB) / 16 < 2 * NB - 1 &&
                          P0E + 7 * (P1E - P0E) / 16 < 2 * NB + NG - 1 && P1E <= 2 * NB + 3 * NG / 2 - 1,
                      "pointwise slots");
        // Non-fused (three buffers): the barrier early in the tile, where the
        // S / dP products leave the issue slots idle; the loads of the tile
        // after next and the scalar set-up of the one after that in the
        // following slots; the 16-byte read offsets and the row-vector
        // offset move to the next buffer at MOV, after the tile's last such
        // read and before the next tile's first, followed by the next
        // tile's rowdot reads.
        constexpr int BAR = 0;                 // barrier slot (slots 2 and 5 measured slower)
        constexpr int NLD = LPT;               // load slots (one load each)
        constexpr int SU0 = BAR + 1 + NLD;     // first of six set-up slots
        constexpr int MOV = NSLOT - RA - 6;    // read offsets to the next buffer
        // The ring of in-flight operands continues across tiles, so its
        // length must divide the slot count.
        static_assert(NB >= 8 && NG >= 8 && NSLOT % RA == 0, "slot plan");
        static_assert(SU0 + 6 <= MOV && MOV >= 2 * NB && MOV + 5 <= NSLOT - RA, "slot events");

        // A operand of slot i of a tile (offsets of the tile's buffer).
        auto op_read = [&](auto ic) -> e16x8 {
            constexpr int i = decltype(ic)::value;
            if constexpr (i < 2 * NB) {
                constexpr int mb = i / NB, jj = i % NB, ks = jj >> 1;
                return lds16b(lds + gq[ks] + 32 * mb * L::PB + ((jj & 1) ? L::BYTES : 0));
            } else {
                constexpr int jj = (i - 2 * NB) % NG, kk = 2 * ((i - 2 * NB) / NG) + jj / (2 * DBL);
                constexpr int db = (jj % (2 * DBL)) >> 1;
                constexpr int base = (jj & 1) ? 0 : L::BYTES;   // even: dO^T (dV), odd: Q^T (dK)
                return tr_pair(lds + base + tq[db][0] + 16 * kk * L::PB,
                               lds + base + tq[db][1] + 16 * kk * L::PB);
            }
        };
        // Head dims above 128, slots of a tile: S of the wave's query block
        // (KS k-steps), dP (KS), then dV and dK over the block's two k-steps
        // (2 DBL each), then dV and dK over the other block's two k-steps.
        constexpr int VO = 2 * KS, KO = VO + 2 * DBL, VP = KO + 2 * DBL, KP = VP + 2 * DBL;
        constexpr int NSB = KP + 2 * DBL;
        auto op_read_big = [&](auto ic) -> e16x8 {
            constexpr int i = decltype(ic)::value;
            if constexpr (i < KS) {
                return lds16b(lds + gq[i]);
            } else if constexpr (i < VO) {
                return lds16b(lds + gq[i - KS] + L::BYTES);
            } else {
                constexpr int u = i - VO, grp = u / (2 * DBL), kl = (u % (2 * DBL)) / DBL, db = u % DBL;
                constexpr int base = (grp & 1) ? 0 : L::BYTES;   // dV: dO^T, dK: Q^T
                const int(&t)[DBL][2] = grp < 2 ? tq : tqp;
                return tr_pair(lds + base + t[db][0] + 16 * kl * L::PB,
                               lds + base + t[db][1] + 16 * kl * L::PB);
            }
        };
        auto op_first = [&](auto ic) -> e16x8 {
            if constexpr (BIG)
                return op_read_big(ic);
            else
                return op_read(ic);
        };
        // dK / dV stay in accumulation registers for the whole loop
        // (without these pins the allocator parks some of them in ordinary
        // registers during the S / dP products and copies them back every
        // tile).
        auto pin_acc = [&]() {
#pragma unroll
            for (int db = 0; db < DBL; ++db)
                asm volatile("" : "+a"(dk_acc[db]), "+a"(dv_acc[db]));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));
        };

        e16x8 ring[RA];
        static_for<RA>([&](auto ic) { ring[decltype(ic)::value] = op_first(ic); });
        // rowdot of the rows of query block mb (accumulator layout: element
        // 4*r4 + t is row 32*mb + 8*r4 + 4*g2 + t): the initial value of the
        // dP accumulator.  Block 0 of the next tile is read once its buffer
        // is published, block 1 at the start of its own tile.
        f32x16 rdc[2];
        auto read_rowdot = [&](int mb, int r4) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(lds + rv0 + 4 * kQTile + 128 * mb + 32 * r4);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                rdc[mb][4 * r4 + t] = v[t];
        };
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
            read_rowdot(0, r4);

        int cur = 0;
        // One query tile, with (IC<1>) or without (IC<0>) the element mask
        // (the same slots otherwise).
        auto tile = [&](int it, int m, int hh, auto maskc) {
            if constexpr (TWO)
                issue(cur ^ 1);
            const int q0 = m * kQTile;
            // This lane's key is visible to tile rows 4*g2 + (32*mb + 8*r4 +
            // t) with limv <= 32*mb + 8*r4 + t <= limu: none past the key
            // end; else rows with key <= q0 + row + off + win_r and key >=
            // q0 + row + off - win_l.
            const int limv =
                key >= Lk ? INT_MAX : (p.win_r >= 0 ? key - q0 - off - p.win_r - 4 * g2 : INT_MIN);
            const int limu = LOCAL ? key - q0 - off + p.win_l - 4 * g2 : INT_MAX;
            uint16_t *dsrow = nullptr;
            if constexpr (FUSED)
                dsrow = &sm.dsT[cur][key_local * FusedSmem<DP>::RD + 4 * g2];
            const float *l2s = reinterpret_cast<const float *>(lds + rv0);
            // offset step to the next tile's buffer
            const int delta = cur == NBUF - 1 ? -(NBUF - 1) * BUFB : BUFB;

            f32x16 s[2], dp[2];
            // dropout keep bits of the tile drawn here (Philox): bit 16*mb +
            // 4*t + r4 for the lane's key and row 32*mb + 8*r4 + 4*g2 + t
            uint32_t kw = 0;
            // keep words (KEEP): word t of kq[mb][r4] is row 32*mb + 8*r4 +
            // 4*g2 + t, and its bit l32 this lane's key
            u32x4 kq[2][4];
            e16x8 pb[4], dsb[4];
            e16x4 ph[4], dh[4];
            f32x4 l2v[4], l2w[4];   // lse2 of the lane's rows, blocks 0 and 1
            f32x4 pv, dv;

            // element e (0..15) of query block mb: exp, mask, dS; packs a
            // 4-row group into bf16 after its last element.
            auto pw_elem = [&](auto mbc, auto ec) {
                constexpr int mb = decltype(mbc)::value, e = decltype(ec)::value;
                constexpr int r4 = e >> 2, t = e & 3;
                constexpr int qc = 32 * mb + 8 * r4;
                float x, cg = 1.f;
                if constexpr (SOFTCAP) {
                    // capped score tanh * c (base 2); dS picks up 1 - tanh^2
                    const float th = cap_tanh(s[mb][e], p.cap_in);
                    x = __builtin_amdgcn_exp2f(fmaf(th, p.cap_out, -(mb ? l2w : l2v)[r4][t]));
                    cg = fmaf(-th, th, 1.f);
                } else {
                    x = __builtin_amdgcn_exp2f(s[mb][e] * p.scale_log2 - (mb ? l2w : l2v)[r4][t]);
                }
                if constexpr (decltype(maskc)::value)
                    x = qc + t >= limv && (!LOCAL || qc + t <= limu) ? x : 0.f;
                // dp holds rowdot - dP; with dropout dV takes P M and
                // dS = P (M dP - rowdot), M = keep / (1 - p)
                float d, pm = x;
                if constexpr (DROP) {
                    const float zi = KEEP ? keep_mult(kq[mb][r4][t], l32, p.drop_inv)
                                          : keep_mult(kw, 16 * mb + 4 * t + r4, p.drop_inv);
                    const float rd_ = rdc[mb][e];
                    d = x * cg * fmaf(zi, rd_ - dp[mb][e], -rd_);
                    pm = x * zi;
                } else {
                    d = SOFTCAP ? x * cg * -dp[mb][e] : x * -dp[mb][e];
                }
                keep_here(pm);
                keep_here(d);
                pv[t] = pm;
                dv[t] = d;
                if constexpr (t == 3) {
                    ph[r4] = to_elem<F16>(pv);
                    dh[r4] = to_elem<F16>(dv);
                    if constexpr (FUSED)
                        *reinterpret_cast<e16x4 *>(dsrow + qc) = dh[r4];
                    if constexpr ((r4 & 1) != 0) {
                        pb[2 * mb + (r4 >> 1)] = concat(ph[r4 - 1], ph[r4]);
                        dsb[2 * mb + (r4 >> 1)] = concat(dh[r4 - 1], dh[r4]);
                    }
                }
            };

            // One Philox call per (block, 4-row group): lane a of each lane
            // quad (four consecutive keys) draws row 4*g2 + a of the group
            // for the quad's four keys; the quad then trades the nibbles so
            // that every lane holds its own key's bits for the four rows.
            auto drop_call = [&](auto cc) {
                constexpr int c = decltype(cc)::value, mb = c >> 2, r4 = c & 3;
                const int a = l32 & 3;
                const uint32_t row = (uint32_t)(q0 + 32 * (mb + mbr) + 8 * r4 + 4 * g2 + a);
                const uint32_t c2 = (uint32_t)(b * p.H + hk * p.G + hh);
                const int nib = (int)keep_nibble((uint32_t)key >> 2, row, c2, p);
                // quad broadcasts of lanes 0..3 (quad_perm [t, t, t, t])
                const uint32_t q0n = (uint32_t)__builtin_amdgcn_mov_dpp(nib, 0x00, 0xF, 0xF, false);
                const uint32_t q1n = (uint32_t)__builtin_amdgcn_mov_dpp(nib, 0x55, 0xF, 0xF, false);
                const uint32_t q2n = (uint32_t)__builtin_amdgcn_mov_dpp(nib, 0xAA, 0xF, 0xF, false);
                const uint32_t q3n = (uint32_t)__builtin_amdgcn_mov_dpp(nib, 0xFF, 0xF, 0xF, false);
                const uint32_t all16 = q0n | (q1n << 4) | (q2n << 8) | (q3n << 12);
                // bit 4t: row t of the group, this lane's key
                kw |= ((all16 >> a) & 0x1111u) << (16 * mb + r4);
            };

            pin_acc();
            if constexpr (BIG) {
                // Rows of the wave's block: 32 mbr + 8 r4 + 4 g2 + t.
                const int limv_b =
                    key >= Lk ? INT_MAX
                              : (p.win_r >= 0 ? key - q0 - off - p.win_r - 4 * g2 - 32 * mbr : INT_MIN);
                const int limu_b = LOCAL ? key - q0 - off + p.win_l - 4 * g2 - 32 * mbr : INT_MAX;
                e16x8 pbo[2], dso[2], pbx[2], dsx[2];
                float cgv[SOFTCAP ? 16 : 1];
                uint8_t *xw = &sm.xch[w][0][0][16 * lane];
                const uint8_t *xr = &sm.xch[w ^ 1][0][0][16 * lane];
                // P of element e (kept in s for dS), packed by k-step.
                auto pw_p = [&](auto ec) {
                    constexpr int e = decltype(ec)::value, r4 = e >> 2, t = e & 3, qc = 8 * r4;
                    float x;
                    if constexpr (SOFTCAP) {
                        const float th = cap_tanh(s[0][e], p.cap_in);
                        x = __builtin_amdgcn_exp2f(fmaf(th, p.cap_out, -l2v[r4][t]));
                        cgv[SOFTCAP ? e : 0] = fmaf(-th, th, 1.f);
                    } else {
                        x = __builtin_amdgcn_exp2f(s[0][e] * p.scale_log2 - l2v[r4][t]);
                    }
                    if constexpr (decltype(maskc)::value)
                        x = qc + t >= limv_b && (!LOCAL || qc + t <= limu_b) ? x : 0.f;
                    // (without dropout P itself is pinned: pinning a copy
                    // would cost a register move per element)
                    float pm = x;
                    if constexpr (DROP) {
                        pm = x * (KEEP ? keep_mult(kq[0][r4][t], l32, p.drop_inv)
                                       : keep_mult(kw, 4 * t + r4, p.drop_inv));
                        keep_here(pm);
                    } else {
                        keep_here(x);
                        pm = x;
                    }
                    s[0][e] = x;
                    pv[t] = pm;
                    if constexpr (t == 3) {
                        ph[r4] = to_elem<F16>(pv);
                        if constexpr ((r4 & 1) != 0)
                            pbo[r4 >> 1] = concat(ph[r4 - 1], ph[r4]);
                    }
                };
                // dS of element e (dp holds rowdot - dP).
                auto pw_ds = [&](auto ec) {
                    constexpr int e = decltype(ec)::value, r4 = e >> 2, t = e & 3;
                    const float x = s[0][e];
                    const float cg = SOFTCAP ? cgv[SOFTCAP ? e : 0] : 1.f;
                    float d;
                    if constexpr (DROP) {
                        const float zi = KEEP ? keep_mult(kq[0][r4][t], l32, p.drop_inv)
                                              : keep_mult(kw, 4 * t + r4, p.drop_inv);
                        const float rd_ = rdc[0][e];
                        d = x * cg * fmaf(zi, rd_ - dp[0][e], -rd_);
                    } else {
                        d = SOFTCAP ? x * cg * -dp[0][e] : x * -dp[0][e];
                    }
                    keep_here(d);
                    dv[t] = d;
                    if constexpr (t == 3) {
                        dh[r4] = to_elem<F16>(dv);
                        if constexpr ((r4 & 1) != 0)
                            dso[r4 >> 1] = concat(dh[r4 - 1], dh[r4]);
                    }
                };
                static_for<NSB>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    const e16x8 a = ring[i % RA];
                    if constexpr ((i & 1) == 0 && i + 1 < NSB)   // paired waits, as below
                        asm volatile("" ::"v"(ring[(i + 1) % RA]));
                    if constexpr (i + RA < NSB)
                        ring[i % RA] = op_read_big(IC<i + RA>{});
                    // keep bits of the block's rows (words or Philox) over
                    // the S slots; the row vectors before the first P
                    if constexpr (KEEP && i < KS)
                        static_for<4>([&](auto rc) {
                            constexpr int r4 = decltype(rc)::value;
                            if constexpr (i == r4 * KS / 4)
                                kq[0][r4] = *reinterpret_cast<const u32x4 *>(lds + kv0 + 32 * r4);
                        });
                    if constexpr (DROP && !KEEP && i < KS)
                        static_for<4>([&](auto rc) {
                            constexpr int r4 = decltype(rc)::value;
                            if constexpr (i == r4 * KS / 4)
                                drop_call(IC<r4>{});
                        });
                    if constexpr (i >= 4 && i < 8)
                        l2v[i - 4] = *reinterpret_cast<const f32x4 *>(l2s + 8 * (i - 4));
                    if constexpr (i < KS) {
                        if constexpr (i == 0)
                            mfma32_vz<F16>(s[0], a, kf[0]);
                        else
                            mfma32_vacc<F16>(s[0], a, kf[i]);
                    } else if constexpr (i < VO) {
                        constexpr int ks = i - KS;
                        if constexpr (ks == 0)   // from rowdot, without a copy
                            mfma32_vc<F16>(dp[0], a, vf[0], rdc[0]);
                        else
                            mfma32_vacc<F16>(dp[0], a, vf[ks]);
                    } else {
                        constexpr int u = i - VO, grp = u / (2 * DBL), kl = (u % (2 * DBL)) / DBL, db = u % DBL;
                        if constexpr (grp == 0) {
                            dv_acc[db] = mfma32<F16>(a, pbo[kl], dv_acc[db]);
                            keep_here_acc(dv_acc[db]);
                        } else if constexpr (grp == 1) {
                            dk_acc[db] = mfma32<F16>(a, dso[kl], dk_acc[db]);
                            keep_here_acc(dk_acc[db]);
                        } else if constexpr (grp == 2) {
                            dv_acc[db] = mfma32<F16>(a, pbx[kl], dv_acc[db]);
                            keep_here_acc(dv_acc[db]);
                        } else {
                            dk_acc[db] = mfma32<F16>(a, dsx[kl], dk_acc[db]);
                            keep_here_acc(dk_acc[db]);
                        }
                    }
                    // P over the dP slots, dS over the own dV slots
                    if constexpr (i >= KS && i < VO) {
                        constexpr int u = i - KS;
                        if constexpr (u == 0)
                            mfma_settle(s[0]);
                        static_for<16 * (u + 1) / KS - 16 * u / KS>(
                            [&](auto ec) { pw_p(IC<16 * u / KS + decltype(ec)::value>{}); });
                    }
                    if constexpr (i >= VO && i < KO) {
                        constexpr int u = i - VO;
                        if constexpr (u == 0) {
                            mfma_settle(dp[0]);
                            *reinterpret_cast<e16x8 *>(xw) = pbo[0];
                            *reinterpret_cast<e16x8 *>(xw + 1024) = pbo[1];
                        }
                        static_for<16 * (u + 1) / (2 * DBL) - 16 * u / (2 * DBL)>(
                            [&](auto ec) { pw_ds(IC<16 * u / (2 * DBL) + decltype(ec)::value>{}); });
                    }
                    if constexpr (i == KO) {
                        *reinterpret_cast<e16x8 *>(xw + 2048) = dso[0];
                        *reinterpret_cast<e16x8 *>(xw + 3072) = dso[1];
                    }
                    if constexpr (i == KO + 1) {
                        // Trade with the other wave of the pair once both
                        // have written (only LDS operations are waited for:
                        // the next tile's loads stay in flight).  Its
                        // operands are read for its k-steps' products,
                        // which come 2 DBL - 1 slots later; the area is
                        // written again only after the tile's closing
                        // barrier.
                        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                        __builtin_amdgcn_s_barrier();
                        asm volatile("" ::: "memory");
                        pbx[0] = *reinterpret_cast<const e16x8 *>(xr);
                        pbx[1] = *reinterpret_cast<const e16x8 *>(xr + 1024);
                        dsx[0] = *reinterpret_cast<const e16x8 *>(xr + 2048);
                        dsx[1] = *reinterpret_cast<const e16x8 *>(xr + 3072);
                    }
                    if constexpr (i == KS || i == VO)
                        pin_acc();
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else
            static_for<NSLOT>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const e16x8 a = ring[i % RA];
                // One operand wait per two slots: an even slot also waits
                // for the next slot's read (issued RA - 1 slots ago), so the
                // odd slot issues no wait of its own.
                if constexpr ((i & 1) == 0 && i + 1 < NSLOT)
                    asm volatile("" ::"v"(ring[(i + 1) % RA]));
                if constexpr (i + RA < NSLOT)
                    ring[i % RA] = op_read(IC<i + RA>{});
                else if constexpr (!TWO)
                    ring[i % RA] = op_read(IC<i + RA - NSLOT>{});   // next tile
                // Keep words (separate-dQ mode): the four rows of group
                // (block, r4) read from LDS where the Philox call would be;
                // the pointwise math takes this lane's key bit of each.
                if constexpr (KEEP && i < 2 * NB)
                    static_for<4>([&](auto rc) {
                        constexpr int r4 = decltype(rc)::value, mb = i / NB;
                        if constexpr ((i % NB) == r4 * NB / 4)
                            kq[mb][r4] = *reinterpret_cast<const u32x4 *>(lds + kv0 + 4 * (32 * mb + 8 * r4));
                    });
                // Philox calls: block 0's over its S / dP slots, block 1's
                // over the next NB slots (before each block's P and dS)
                if constexpr (DROP && !KEEP && i < 2 * NB)
                    static_for<4>([&](auto rc) {
                        constexpr int r4 = decltype(rc)::value;
                        if constexpr ((i % NB) == r4 * NB / 4)
                            drop_call(IC<4 * (i / NB) + r4>{});
                    });
                // row vectors of block 0, read during the slots before its
                // pointwise work starts
                if constexpr (i >= NB / 2 && i < NB / 2 + 4) {
                    constexpr int r4 = i - NB / 2;
                    l2v[r4] = *reinterpret_cast<const f32x4 *>(l2s + 8 * r4);
                }
                // rowdot of block 1, needed by its first dP step
                if constexpr (i < 4)
                    read_rowdot(1, i);
                if constexpr (i < 2 * NB) {
                    constexpr int mb = i / NB, jj = i % NB, ks = jj >> 1;
                    if constexpr ((jj & 1) != 0) {
                        // dp = rowdot - dO V^T (vf holds -V)
                        if constexpr (ks == 0) {
                            dp[mb] = rdc[mb];   // a vector copy: FRESH waits for it
                            mfma32_vacc<F16, true>(dp[mb], a, vf[ks]);
                        } else {
                            mfma32_vacc<F16>(dp[mb], a, vf[ks]);
                        }
                    } else if constexpr (ks == 0) {
                        mfma32_vz<F16>(s[mb], a, kf[ks]);
                    } else {
                        mfma32_vacc<F16>(s[mb], a, kf[ks]);
                    }
                } else {
                    constexpr int jj = (i - 2 * NB) % NG;
                    constexpr int kk = 2 * ((i - 2 * NB) / NG) + jj / (2 * DBL);
                    constexpr int db = (jj % (2 * DBL)) >> 1;
                    if constexpr ((jj & 1) != 0) {
                        dk_acc[db] = mfma32<F16>(a, dsb[kk], dk_acc[db]);
                        keep_here_acc(dk_acc[db]);
                    } else {
                        dv_acc[db] = mfma32<F16>(a, pb[kk], dv_acc[db]);
                        keep_here_acc(dv_acc[db]);
                    }
                }
                // vector work: the 16 elements of P, dS of block 0 spread over
                // slots NB .. P0E-1 and those of block 1 over P0E .. P1E-1
                // (the row vectors of block 1 are read in four slots of
                // block 1's S / dP).  The dV / dK k-step kk takes
                // elements 8 (kk % 2) .. +7 of block kk / 2, so block 0 may
                // run into the first dV / dK slots and block 1 into the last
                // ones, which evens out the vector work per MFMA.
                if constexpr (i >= NB + NB / 2 && i < NB + NB / 2 + 4) {
                    constexpr int r4 = i - (NB + NB / 2);
                    l2w[r4] = *reinterpret_cast<const f32x4 *>(l2s + 32 + 8 * r4);
                }
                if constexpr (i >= NB && i < P0E) {
                    constexpr int u = i - NB, n = P0E - NB;
                    if constexpr (u == 0)
                        mfma_settle(s[0], dp[0]);
                    static_for<16 * (u + 1) / n - 16 * u / n>(
                        [&](auto ec) { pw_elem(IC<0>{}, IC<16 * u / n + decltype(ec)::value>{}); });
                }
                if constexpr (i >= P0E && i < P1E) {
                    constexpr int u = i - P0E, n = P1E - P0E;
                    if constexpr (u == 0)
                        mfma_settle(s[1], dp[1]);
                    static_for<16 * (u + 1) / n - 16 * u / n>(
                        [&](auto ec) { pw_elem(IC<1>{}, IC<16 * u / n + decltype(ec)::value>{}); });
                }
                if constexpr (i == NB || i == 2 * NB)
                    pin_acc();
                if constexpr (!TWO && i == BAR) {
                    // Every wave has finished with the buffer of the last
                    // tile, and the only loads in flight are the next tile's
                    // (issued one tile ago): wait for them, then publish.
                    // (A bare barrier: the LDS reads in flight read this
                    // tile's buffer, which no load issued after the barrier
                    // touches.)
                    wait_loads<0>();
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
                // The loads of the tile after next, one per slot after the
                // barrier (two per slot measured 0.7% slower at head dim
                // 128, one every other slot slower still), into the buffer
                // of the last tile; then the pointers and descriptors of the
                // tile after that (the scalar work spread over slots in the
                // MFMAs' shadow).
                if constexpr (!TWO && i > BAR && i <= BAR + NLD) {
                    const int bf = cur == 0 ? NBUF - 1 : cur - 1;
                    issue_one(IC<i - BAR - 1>{}, bf);
                }
                if constexpr (!TWO && i >= SU0 && i < SU0 + 6)
                    setup_part(IC<i - SU0>{});
                if constexpr (!TWO && i == MOV) {
                    // the 16-byte operand reads, row-vector and keep-word
                    // reads of this tile are all issued
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        gq[ks] += delta;
                    rv0 += delta;
                    kv0 += delta;
                }
                if constexpr (!TWO && i > MOV && i <= MOV + 4)
                    read_rowdot(0, i - MOV - 1);   // next tile (published at this tile's barrier)
                if constexpr (!TWO && i == NSLOT - RA - 1) {
                    // last transposing read of this tile issued
#pragma unroll
                    for (int db = 0; db < DBL; ++db) {
                        tq[db][0] += delta;
                        tq[db][1] += delta;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            pin_acc();

            if constexpr (TWO) {
                // Next tile's buffer.
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    gq[ks] += delta;
#pragma unroll
                for (int db = 0; db < DBL; ++db) {
                    tq[db][0] += delta;
                    tq[db][1] += delta;
                    if constexpr (BIG) {
                        tqp[db][0] += delta;
                        tqp[db][1] += delta;
                    }
                }
                rv0 += delta;
                kv0 += delta;
                wait_loads<0>();
                __syncthreads();   // next tile in LDS; dS^T[cur] complete
                if constexpr (FUSED) {
                    const int h = hk * p.G + hh;
                    const int rows_valid = min(kQTile, Lq - q0);
                    dq_partial<DP, F16>(p, sm, cur, w, lane, l32, g2, tid, b, h, m, j, q0,
                                        rows_valid, Lq, off, nt_b, si.ws_row);
                }
                static_for<RA>([&](auto ic) { ring[decltype(ic)::value] = op_first(ic); });
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    read_rowdot(0, r4);
            }
            cur = cur == NBUF - 1 ? 0 : cur + 1;
        };
        if constexpr (FUSED) {
            const int dm = ascending ? 1 : -1;
            int m = ascending ? m_begin : m_end - 1, hh = 0;
            for (int it = 0; it < total; ++it) {
                tile(it, m, hh, IC<1>{});
                const int wrap = hh == p.G - 1;
                hh = wrap ? 0 : hh + 1;
                m += wrap ? dm : 0;
            }
        } else {
            // The wave's keys kw0 .. kw_last are visible to every row of the
            // query tiles mf_lo .. mf_hi (none if a key is past the end):
            // rows >= kw_last - off - win_r and rows <= kw0 - off + win_l.
            // In the descending order those come after nh masked tiles and
            // before the masked rest; each query tile is visited for the G
            // heads in turn.  (Three loops: one masked loop entered from both
            // edges makes the register allocator spill.)
            const int kw0 = n0 + 32 * kgrp, kw_last = kw0 + 31;
            int nh = 0, nu = 0;
            if (kw_last < Lk) {
                const int need = kw_last - off - p.win_r;
                const int mf_lo = max(m_begin, p.win_r < 0 || need <= 0 ? 0 : (need + kQTile - 1) / kQTile);
                const int top = kw0 - off + p.win_l - (kQTile - 1);   // last row of tile m <= top + 63
                const int mf_hi =
                    !LOCAL ? m_end - 1 : min(m_end - 1, top >= 0 ? top / kQTile : -1);
                if (mf_lo <= mf_hi) {
                    nh = m_end - 1 - mf_hi;
                    nu = mf_hi - mf_lo + 1;
                }
            }
            const int it_h = nh * p.G, it_u = it_h + nu * p.G;
            int it = 0, m = m_end - 1, hh = 0;
            auto next = [&]() {
                ++it;
                const int wrap = hh == p.G - 1;
                hh = wrap ? 0 : hh + 1;
                m -= wrap;
            };
            if constexpr (LOCAL)
                for (; it < it_h; next())
                    tile(it, m, hh, IC<1>{});
            for (; it < it_u; next())
                tile(it, m, hh, IC<0>{});
            for (; it < total; next())
                tile(it, m, hh, IC<1>{});
        }
        // The last iterations issued loads past the final tile (empty bound,
        // zeros into LDS); let them land before the workgroup's LDS is
        // released.
        wait_loads<0>();
    }

    // ---- epilogue: dK = scale * acc, dV = acc, 16-bit, keys < Lk, d < D.
    //      Accumulator of head-dim block db: column 32 (dbo + db) + 8 r4 +
    //      4 g2 + t of the lane's key.  Per pair of 8-column groups the lane
    //      halves trade their 8-byte pieces (both halves hold the same key),
    //      so each lane stores 16 bytes: columns 16 q + 8 g2 .. +7 of the
    //      pair q. ----
    {
        uint16_t *dkrow = p.dk + row_offset(p, b, si.tok_k, key < Lk ? key : 0, p.dk_sb, p.dk_ss) + hk * p.dk_sh;
        uint16_t *dvrow = p.dv + row_offset(p, b, si.tok_k, key < Lk ? key : 0, p.dv_sb, p.dv_ss) + hk * p.dv_sh;
        auto store16 = [&](uint16_t *row, const f32x16 &acc, float sc, int db) {
            u32x2 pc[4];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    v[t] = acc[4 * r4 + t] * sc;
                pc[r4] = __builtin_bit_cast(u32x2, to_elem<F16>(v));
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // lanes 32-63 of pc[2q] <-> lanes 0-31 of pc[2q+1]
                const auto s0 = __builtin_amdgcn_permlane32_swap(pc[2 * q][0], pc[2 * q + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(pc[2 * q][1], pc[2 * q + 1][1], false, false);
                const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
                const int d = 32 * (dbo + db) + 16 * q + 8 * g2;
                if (key < Lk && d < p.D)
                    *reinterpret_cast<u32x4 *>(row + d) = out;
            }
        };
#pragma unroll
        for (int db = 0; db < DBL; ++db) {
            store16(dkrow, dk_acc[db], p.scale, db);
            store16(dvrow, dv_acc[db], 1.f, db);
        }
    }
}

// Dropout mode of the key-tile kernel: 0 none, 1 draws the keep bits (fused
// modes, or no keep words in the workspace), 2 reads the dQ pass's words.
template <int D, bool FU, bool H16, bool LOCAL, bool SOFTCAP, bool DROP>
static void launch_main_k(const Params &p, dim3 grid, hipStream_t st)
{
    const dim3 block(kThreads);
    if constexpr (!DROP)
        hipLaunchKernelGGL((fa_bwd_main_kernel<D, FU, H16, LOCAL, SOFTCAP, 0>), grid, block, 0, st, p);
    else if constexpr (FU)
        hipLaunchKernelGGL((fa_bwd_main_kernel<D, FU, H16, LOCAL, SOFTCAP, 1>), grid, block, 0, st, p);
    else if (p.keep)
        hipLaunchKernelGGL((fa_bwd_main_kernel<D, FU, H16, LOCAL, SOFTCAP, 2>), grid, block, 0, st, p);
    else
        hipLaunchKernelGGL((fa_bwd_main_kernel<D, FU, H16, LOCAL, SOFTCAP, 1>), grid, block, 0, st, p);
}

template <bool LOCAL, bool SOFTCAP, bool DROP>
static hipError_t launch_main_t(const Params &p, int dpad, hipStream_t st)
{
    const dim3 grid((unsigned)p.ntiles * p.Hk * p.batch);
    // head dims above 128: 64 keys per workgroup
    const dim3 grid_big((unsigned)((p.Sk + 63) / 64) * p.Hk * p.batch);
#define FA_LAUNCH_MAIN(D, FU, H16) launch_main_k<D, FU, H16, LOCAL, SOFTCAP, DROP>(p, grid, st)
#define FA_LAUNCH_MAIN_BIG(D)                                                   \
    if (p.fused_dq)                                                             \
        return hipErrorInvalidValue;                                            \
    else if (p.f16)                                                             \
        launch_main_k<D, false, true, LOCAL, SOFTCAP, DROP>(p, grid_big, st);    \
    else                                                                        \
        launch_main_k<D, false, false, LOCAL, SOFTCAP, DROP>(p, grid_big, st);
#define FA_LAUNCH_MAIN_D(D)                                                     \
    if (p.fused_dq && p.f16)                                                    \
        FA_LAUNCH_MAIN(D, true, true);                                          \
    else if (p.fused_dq)                                                        \
        FA_LAUNCH_MAIN(D, true, false);                                         \
    else if (p.f16)                                                             \
        FA_LAUNCH_MAIN(D, false, true);                                         \
    else                                                                        \
        FA_LAUNCH_MAIN(D, false, false);
    switch (dpad) {
    case 64:
        FA_LAUNCH_MAIN_D(64);
        break;
    case 96:
        FA_LAUNCH_MAIN_D(96);
        break;
    case 128:
        FA_LAUNCH_MAIN_D(128);
        break;
    case 192:
        FA_LAUNCH_MAIN_BIG(192);
        break;
    case 256:
        FA_LAUNCH_MAIN_BIG(256);
        break;
    default:
        return hipErrorInvalidValue;
    }
#undef FA_LAUNCH_MAIN_BIG
#undef FA_LAUNCH_MAIN_D
#undef FA_LAUNCH_MAIN
    return hipGetLastError();
}

// The (softcap, dropout) variants build in four translation units
// (fa_main_softcap.hip, fa_main_dropout.hip and fa_main_softcap_dropout.hip
// include this file with FA_TU_SOFTCAP / FA_TU_DROPOUT set), so that they
// compile in parallel.
template <bool SOFTCAP, bool DROP>
hipError_t launch_main_v(const Params &p, int dpad, hipStream_t st)
{
    return p.win_l >= 0 ? launch_main_t<true, SOFTCAP, DROP>(p, dpad, st)
                        : launch_main_t<false, SOFTCAP, DROP>(p, dpad, st);
}

#if FA_TU_SOFTCAP || FA_TU_DROPOUT
template hipError_t launch_main_v<FA_TU_SOFTCAP != 0, FA_TU_DROPOUT != 0>(const Params &, int,
                                                                          hipStream_t);
#else
extern template hipError_t launch_main_v<true, false>(const Params &, int, hipStream_t);
extern template hipError_t launch_main_v<false, true>(const Params &, int, hipStream_t);
extern template hipError_t launch_main_v<true, true>(const Params &, int, hipStream_t);

hipError_t launch_main(const Params &p, int dpad, hipStream_t st)
{
    const bool sc = p.softcap > 0.f, dr = p.drop_p > 0.f;
    if (dr)
        return sc ? launch_main_v<true, true>(p, dpad, st) : launch_main_v<false, true>(p, dpad, st);
    return sc ? launch_main_v<true, false>(p, dpad, st) : launch_main_v<false, false>(p, dpad, st);
}
#endif

}  // namespace fa
