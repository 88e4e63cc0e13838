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
// Each wave owns keys 32w .. 32w+31 of the tile; their K and V rows stay in
// registers as the B operands of S and dP.  With keys as the N index, the
// accumulator of P (and dS) holds one key and 16 query rows per lane, which
// is directly a B operand of dV^T = dO^T P and dK^T = Q^T dS once the query
// (contraction) index is permuted within each group of 16:
//   k-slot 8*g2 + t  <->  query 4*g2 + t (t < 4) or 8 + 4*g2 + t - 4.
// Operands whose contraction index runs down the rows of a row-major LDS
// tile (dO^T, Q^T, and both operands of dQ = dS K) are read with the gfx950
// transposing LDS read ds_read_b64_tr_b16: within each 16-lane group the 16
// 8-byte reads form a 4 x 16 block (lanes 4r..4r+3 read row r) and lane c
// receives column c.  Two such reads give one 8-element operand, and the row
// base of each read implements the permutation above.  No transposed copies
// are stored.
//
// LDS (D_pad = 128): Q and dO row-major, double buffered (4 x 18 KB), dS^T
// double buffered (2 x 20 KB), K 36 KB, row vectors 1 KB: 149 KB, one
// workgroup per CU.  Row
// pitches are D + 16 elements (dS^T: 64 + 16) so that both the 16-byte row
// reads and the transposing reads hit distinct banks.
//
// Pipelining: the next query tile is loaded from global memory into
// registers while the current one is computed and written to the other LDS
// buffer before the dQ atomics of the current tile are issued.  One
// workgroup barrier per tile: every LDS buffer written in tile t was last
// read before the barrier of tile t-1.
#include <climits>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int DP>
struct __attribute__((aligned(16))) Smem {
    static constexpr int RQ = DP + 16;       // pitch of q / dO / k (elements)
    static constexpr int RD = kQTile + 16;   // pitch of dS^T
    uint16_t q[2][kQTile * RQ];
    uint16_t dO[2][kQTile * RQ];
    uint16_t dsT[2][kKTile * RD];
    uint16_t k[kKTile * RQ];
    float lse2[2][kQTile];
    float rowdot[2][kQTile];
};

__device__ inline bf16x8 lds16(const uint16_t *p)
{
    return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ inline i16x4 lds_tr(const uint16_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)((lds_u16 *)p));
}

// MFMA operand fragment from a row-major LDS matrix whose rows run along the
// contraction index: the lane receives column c0 + l32 at rows r0 .. r0+3
// (elements 0..3) and r1 .. r1+3 (elements 4..7).  r0 and r1 may depend on
// g2 only.
__device__ inline bf16x8 frag_tr(const uint16_t *base, int pitch, int r0, int r1, int c0,
                                 int lane)
{
    const int c16 = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (c16 & 3);
    const int rr = c16 >> 2;
    const i16x4 lo = lds_tr(base + (r0 + rr) * pitch + col);
    const i16x4 hi = lds_tr(base + (r1 + rr) * pitch + col);
    const i16x4 v8[2] = {lo, hi};
    return __builtin_bit_cast(bf16x8, v8);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Asks the scheduler to issue `ahead` LDS reads first and then alternate one
// MFMA with `per` reads, so each MFMA's operands were requested several
// MFMAs earlier (one wave per SIMD: the wave itself must hide LDS latency).
template <int N_MFMA, int PER, int AHEAD>
__device__ inline void pipeline_reads()
{
    constexpr int NR = N_MFMA * PER;
    static_assert(AHEAD <= NR && AHEAD % PER == 0, "bad pipeline shape");
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < N_MFMA - AHEAD / PER; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PER, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, AHEAD / PER, 0);
}

// P = exp2(S*scale*log2e - lse2) and dS = P (dP - rowdot) for one wave's
// 64 x 32 tile; bf16 copies in MFMA B-operand order, dS^T row to LDS.
// MASK: query row qi (0..63 in the tile) sees this lane's key iff
// keyok && qi >= lim.
template <bool MASK>
__device__ inline void pointwise(const f32x16 (&s)[2], const f32x16 (&dp)[2], bf16x8 (&pb)[4],
                                 bf16x8 (&dsb)[4], uint16_t *dsT_row, const float *l2s,
                                 const float *rds, float scale_log2, int g2, int lim, bool keyok)
{
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int qi0 = 32 * mb + 8 * r4 + 4 * g2;
            const float4 l2v = *reinterpret_cast<const float4 *>(l2s + qi0);
            const float4 rdv = *reinterpret_cast<const float4 *>(rds + qi0);
            const float l2a[4] = {l2v.x, l2v.y, l2v.z, l2v.w};
            const float rda[4] = {rdv.x, rdv.y, rdv.z, rdv.w};
            u16x4 dsv4;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 4 * r4 + t;
                float pv = __builtin_amdgcn_exp2f(s[mb][r] * scale_log2 - l2a[t]);
                if constexpr (MASK)
                    pv = (keyok && qi0 + t >= lim) ? pv : 0.f;
                const float dsv = pv * (dp[mb][r] - rda[t]);
                const uint16_t pbits = f2bf(pv), dbits = f2bf(dsv);
                pb[2 * mb + (r >> 3)][r & 7] = __builtin_bit_cast(__bf16, pbits);
                dsb[2 * mb + (r >> 3)][r & 7] = __builtin_bit_cast(__bf16, dbits);
                dsv4[t] = dbits;
            }
            *reinterpret_cast<u16x4 *>(dsT_row + qi0) = dsv4;
        }
    }
}

template <int DP>
__global__ void __launch_bounds__(kThreads, 1) fa_bwd_main_kernel(Params p)
{
    constexpr int KS = DP / 16;       // MFMA k-steps over the head dim
    constexpr int DB = DP / 32;       // 32-wide blocks of the head dim
    constexpr int RQ = Smem<DP>::RQ, RD = Smem<DP>::RD;
    constexpr int CPR = DP / 8;       // 16-byte chunks per tile row
    constexpr int NCH = kQTile * CPR / kThreads;   // chunks per thread per tile
    static_assert(kQTile * CPR % kThreads == 0, "tile load must divide evenly");
    __shared__ Smem<DP> sm;

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

    // Workgroup -> (batch, KV head, key tile).
    //  - atomic mode: longest work first.  Key tile 0 sees the most query
    //    tiles under the causal mask, so all workgroups of key tile 0 (every
    //    batch and KV head) come first, then key tile 1, ...; the
    //    (batch, KV head) index is the fast one, which keeps one
    //    (batch, KV head) on one XCD of the round-robin dispatch when
    //    batch * Hk is a multiple of the XCD count.
    //  - ordered mode: within one (batch, KV head) the key tiles run in
    //    descending order along the linear id, so every workgroup waits only
    //    on one with a lower id (which the in-order dispatch has already
    //    placed on a CU).
    const int nt = p.ntiles;
    const int nbg = p.batch * p.Hk;
    const int lin = blockIdx.x;
    int j, bg;
    if (p.deterministic) {
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

    // ---- K, V rows of this wave's 32 keys: B operands of S and dP; the K
    //      tile also goes to LDS row-major for dQ = dS K. ----
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
            *reinterpret_cast<uint4 *>(&sm.k[key_local * RQ + d0]) = kv;
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
            const int64_t wsbase = (int64_t)h * p.rows + si.ws_row;
            if (it + 1 < total)
                prefetch(it + 1);
            const uint16_t *sq = sm.q[buf];
            const uint16_t *sdo = sm.dO[buf];

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
                    const int o = (32 * mb + l32) * RQ + 16 * ks + 8 * g2;
                    s[mb] = mfma32(lds16(sq + o), kf[ks], s[mb]);
                    dp[mb] = mfma32(lds16(sdo + o), vf[ks], dp[mb]);
                }
            }
            pipeline_reads<4 * KS, 1, 8>();

            // ---- P, dS (fp32), masked only on diagonal / tail tiles ----
            const bool need_mask =
                (n0 + kKTile > Lk) || (p.causal && (n0 + kKTile - 1 > q0 + off));
            bf16x8 pb[4], dsb[4];
            if (need_mask) {
                // causal: key visible to tile row qi iff key <= q0 + qi + off
                const int lim = p.causal ? key - q0 - off : INT_MIN;
                pointwise<true>(s, dp, pb, dsb, &sm.dsT[buf][key_local * RD], sm.lse2[buf],
                                sm.rowdot[buf], p.scale_log2, g2, lim, key < Lk);
            } else {
                pointwise<false>(s, dp, pb, dsb, &sm.dsT[buf][key_local * RD], sm.lse2[buf],
                                 sm.rowdot[buf], p.scale_log2, g2, 0, true);
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
            __syncthreads();   // dS^T[buf] complete; next tile staged

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
