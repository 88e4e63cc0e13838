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
// One workgroup (8 wave64s, two per SIMD) owns 256 query rows of one query
// head, or under a left window the same 256 / HPW rows of HPW query heads
// that share a KV head (HPW = 4 for groups of four); each wave owns 32 rows
// of one head, whose Q and dO rows stay in registers as the B operands of
//     S^T  = K Q^T        dP^T = V (-dO)^T + rowdot   (64 keys x 32 rows per wave)
// for each 64-key tile.  The accumulator of S^T holds one query row and 16
// keys per lane, so lse2 and rowdot are one register each, and dS (16-bit)
// is directly the B operand of dQ^T = K^T dS^T with the key index permuted
// as described in fa_mfma.h; K^T enters as the A operand through
// transposing LDS reads.  dQ^T (D x 32 rows per wave) accumulates in
// registers over all key tiles and is scaled and stored once: its
// accumulator holds one row and runs of four head-dim columns per lane, so
// the stores are 16 bytes per lane after one exchange between the lane
// halves (a dQ = dS K accumulator would hold one column and sixteen rows
// per lane: 2-byte stores, eight times as many).  In the default mode this kernel
// also forms lse2 and rowdot (written to the workspace for the key-tile
// kernel, which runs after it).
//
// K and V tiles are loaded by buffer loads straight into the swizzled LDS
// layout of fa_mfma.h (zero fill of keys past the end and of padded
// head-dim columns by the buffer bound), three buffers deep.  Each key tile
// runs as a fixed sequence of MFMA slots (the same scheme as the key-tile
// kernel): S^T, dP^T of keys 0-31, of keys 32-63 alongside the pointwise
// math of keys 0-31, the dQ k-steps over keys 0-31 alongside the pointwise
// math of keys 32-63, the dQ k-steps over keys 32-63.  Operand reads run a
// fixed number of slots ahead, across tile boundaries; the wait for the next
// tile, the workgroup barrier and the loads of the tile after next sit early
// in the tile, where the S^T / dP^T products leave the issue slots idle.
//
// LDS (D_pad = 128): 3 x (K, V) x 16 KB = 96 KB.
#include <algorithm>
#include <type_traits>

#include "fa_mfma.h"
#include "fa_philox.h"

#ifndef FA_TU_DROPOUT
#define FA_TU_DROPOUT 0
#endif

namespace fa {

constexpr int kDqKeys = 64;                 // keys per streamed tile

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Workgroup shape by padded head dim: up to 128, eight waves (two per SIMD,
// 256 rows) and three K/V buffers; at 192 and 256 a wave's Q, dO and dQ
// fragments need all 512 registers of a SIMD, so four waves (128 rows), and
// three 64-key K/V buffers would not fit the LDS, so two.  SMALL (head dim
// 64 only, for grids of few workgroups): four waves of 128 rows with two
// workgroups per CU (48 KB of LDS each), the same two waves per SIMD at
// half the granularity, so that the causal mask's uneven query tiles
// spread over twice as many workgroups.
template <int DP, bool SMALL = false>
struct DqShape {
    static constexpr bool BIG = DP > 128;
    static_assert(!SMALL || DP == 64, "the small shape is built for head dim 64");
    static constexpr int WAVES = BIG || SMALL ? 4 : 8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS = 32 * WAVES;     // query rows per workgroup
    static constexpr int NBUF = BIG ? 2 : 3;
    static constexpr int PER_CU = SMALL ? 2 : 1;   // workgroups per CU (launch bound)
};

template <int DP>
struct __attribute__((aligned(16))) KVBuf {
    uint8_t k[Tile64<DP>::BYTES];
    uint8_t v[Tile64<DP>::BYTES];
};

// Dropout from the caller's keep words: a tile also carries each wave's two
// words of the tile's keys for its 32 rows (lane l of the wave's load: word
// l / 32 of row l % 32).
template <int DP, bool SMALL>
struct __attribute__((aligned(16))) KVBufKeep : KVBuf<DP> {
    uint32_t keep[DqShape<DP, SMALL>::WAVES][64];
};

template <int DP, bool KW, bool SMALL>
struct __attribute__((aligned(16))) DqSmem {
    std::conditional_t<KW, KVBufKeep<DP, SMALL>, KVBuf<DP>> buf[DqShape<DP, SMALL>::NBUF];
};

// LOCAL: a left window bounds the visible keys from below (win_l >= 0);
// otherwise win_l < 0 and only the upper bound (causal / right window / key
// end) is masked.  SOFTCAP: scores soft-capped (softcap > 0).  DROP:
// dropout (drop_p > 0) replayed from the forward's rng state (1: the keep
// bits drawn here, and written for the key-tile kernel when p.keep is set)
// or read from the words the forward wrote (2, p.keep).
template <int DP, bool F16, bool LOCAL, bool SOFTCAP, int DROP, bool SMALL = false>
__global__ void __launch_bounds__((DqShape<DP, SMALL>::THREADS), (DqShape<DP, SMALL>::PER_CU))
    fa_bwd_dq_kernel(Params p)
{
    using Shape = DqShape<DP, SMALL>;
    constexpr bool DRAW = DROP == 1, READW = DROP == 2;
    constexpr int KS = DP / 16;                  // k-steps over the head dim
    constexpr int DB = DP / 32;                  // 32-wide head-dim blocks
    constexpr int NBUF = Shape::NBUF;
    constexpr bool BIG = Shape::BIG;
    constexpr int WAVES = Shape::WAVES;
    using L = Tile64<DP>;
    constexpr int PERW = L::NLOAD / WAVES;       // 1 KB wave loads per tensor per wave
    static_assert(PERW >= 1 && L::NLOAD % WAVES == 0, "tile load split");
    __shared__ DqSmem<DP, READW, SMALL> sm;
    using Buf = std::remove_reference_t<decltype(sm.buf[0])>;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

    // Workgroup -> (query tile, batch, KV head, heads).  Under a left
    // window the workgroup's waves cover HPW query heads of one KV head's
    // group (the largest power of two dividing the group size, at most the
    // wave count) and, for each, the same RW = 32 * WAVES / HPW query rows:
    // all heads of a group read the same K/V tiles, so the workgroup's key
    // range is the window band of RW rows rather than of all its 32 * WAVES
    // rows, with fewer tiles that only some waves see (256-key window at the
    // 4096-row GQA shape: this kernel 0.144 -> 0.130 ms).  Without one (HPW =
    // 1) the band is the whole causal prefix either way and one head's 32 *
    // WAVES consecutive rows measured as fast or faster.  Under the causal
    // mask the last query tiles see the most keys, so they come first
    // within the (batch, KV head) groups an XCD runs side by side
    // (xcd_group_order: the heads and query tiles that share a K/V stream
    // stay on one XCD when batch * Hk is a multiple of the XCD count).
    const int hpw = LOCAL ? min(p.G & -p.G, WAVES) : 1;   // heads per workgroup
    const int wph = WAVES / hpw;                 // waves per head
    const int rw = 32 * wph;                     // query rows per head
    const int ngrp = p.G / hpw;                  // head sets per group
    const int nbg = p.batch * p.Hk;
    const int nqt = (p.Sq + rw - 1) / rw;
    const int lin = blockIdx.x;
    int u, bg;   // u = (last query tile - mt) * ngrp + head set
    xcd_group_order(lin, nbg, nqt * ngrp, u, bg);
    const int mt = nqt - 1 - u / ngrp;
    const int hk = bg % p.Hk, b = bg / p.Hk;
    // the wave's query head and first row (wave-uniform)
    const int h = hk * p.G + (u % ngrp) * hpw + w / wph;

    if (lin == 0 && tid < 4)
        p.flags[tid] = 0;   // the workspace flags (this pass never raises one)
    const SeqInfo si = seq_info(p, b);
    const int q0 = mt * rw;
    if (q0 >= si.Lq)
        return;
    const int Lq = si.Lq, Lk = si.Lk;
    const int off = Lk - Lq;
    const int r0w = q0 + 32 * (w % wph);
    const int qrow = r0w + l32;                  // this lane's query row
    const bool qok = qrow < Lq;
    const uint32_t drop_c2 = (uint32_t)(b * p.H + h);   // Philox counter word 2

    // Key tiles t_lo .. nkt-1 hold the keys visible to some row of this
    // query tile (rows q0 .. q_last see keys k_lo .. k_hi at most).
    const int q_last = min(q0 + rw, Lq) - 1;
    const int k_lo = LOCAL ? max(0, q0 + off - p.win_l) : 0;
    const int k_hi = p.win_r >= 0 ? min(Lk - 1, q_last + off + p.win_r) : Lk - 1;
    const int t_lo = k_lo / kDqKeys;
    const int nkt = k_hi >= k_lo ? k_hi / kDqKeys + 1 : t_lo;
    // Without a left window: the lane's row sees keys <= klim.
    const int klim = qok ? (p.win_r >= 0 ? min(Lk - 1, qrow + off + p.win_r) : Lk - 1) : -1;

    // Global byte offsets of the 16-byte chunk each lane loads for wave
    // load i (LDS row pr holds tile chunk (lane % PCH) ^ swz(pr)), held in
    // registers across the loop (at head dims above 128 too: forming them
    // per load from the lane index took about 17 vector instructions per
    // load pair, a quarter of the loop).
    uint32_t vok[PERW], vov[PERW];
    auto load_off = [&](int i, int ln, int ss) -> uint32_t {
        const int pr = (w * PERW + i) * L::RPL + ln / L::PCH;
        const int c = (ln % L::PCH) ^ swz<L::PCH>(pr);
        return c * 8 < p.D ? (uint32_t)(pr * ss * 2 + c * 16) : kOutOfRange;
    };
#pragma unroll
    for (int i = 0; i < PERW; ++i) {
        vok[i] = load_off(i, lane, (int)p.k_ss);
        vov[i] = load_off(i, lane, (int)p.v_ss);
    }
    // Issue the loads of the next key tile into buffer bf (tiles are loaded
    // strictly in order; past the last tile: empty bound, zeros, no memory
    // access).  The tile's row pointers advance by one tile per call, in
    // scalar registers kept at the call's place in the instruction stream.
    const uint16_t *k_next = p.k + hk * p.k_sh + row_offset(p, b, si.tok_k, 0, p.k_sb, p.k_ss);
    const uint16_t *v_next = p.v + hk * p.v_sh + row_offset(p, b, si.tok_k, 0, p.v_sb, p.v_ss);
    int n_next = t_lo * kDqKeys, n_left = nkt - t_lo;
    const int64_t kstep = (int64_t)kDqKeys * p.k_ss, vstep = (int64_t)kDqKeys * p.v_ss;
    k_next += t_lo * kstep;
    v_next += t_lo * vstep;
    // Caller's keep words (READW): words 2t, 2t + 1 of the wave's first row,
    // H * rows words apart; two words further per tile.
    const uint32_t *w_next = nullptr;
    const uint32_t hr4 = READW ? (uint32_t)(p.H * p.rows * 4) : 0u;
    const int64_t wstep = 2 * (int64_t)p.H * p.rows;
    if constexpr (READW)
        w_next = p.keep + ((int64_t)(2 * t_lo) * p.H + h) * p.rows + si.ws_row + r0w;
    // Load part j (0 .. 2 PERW - 1) of the next tile: part 0 forms the
    // descriptors (and loads the keep words), part j issues wave load j (K,
    // V alternating).  In the tile loop the parts go one per slot.
    u32x4_rsrc rk, rv;
    auto issue_part = [&](int bf, auto jc) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j == 0) {
            if constexpr (!Shape::BIG)   // (at 256 the pins leave no legal register class)
                keep_scalar_here(n_next, n_left, k_next, v_next);
            const int kv = n_left > 0 ? min(kDqKeys, Lk - n_next) : 0;
            const uint32_t nk = kv ? (uint32_t)((kv - 1) * (int)p.k_ss * 2 + p.D * 2) : 0u;
            const uint32_t nv = kv ? (uint32_t)((kv - 1) * (int)p.v_ss * 2 + p.D * 2) : 0u;
            rk = make_rsrc(k_next, nk);
            rv = make_rsrc(v_next, nv);
            if constexpr (READW) {
                // lane l: word l / 32 of row l % 32 (rows past the end: zeros)
                const u32x4_rsrc rw = make_rsrc(w_next, kv ? hr4 + 128u : 0u);
                w_next += wstep;
                const int ln = lane_here();
                const uint32_t vw = r0w + (ln & 31) < Lq
                                        ? (uint32_t)(ln >> 5) * hr4 + (uint32_t)(ln & 31) * 4u
                                        : kOutOfRange;
                load4_to_lds(rw, sm.buf[bf].keep[w], vw);
            }
            n_next += kDqKeys;
            --n_left;
            k_next += kstep;
            v_next += vstep;
            if constexpr (!Shape::BIG)
                keep_scalar_here(n_next, n_left, k_next, v_next);
        }
        Buf &kb = sm.buf[bf];
        constexpr int i = j >> 1;
        const int ld = (w * PERW + i) * 1024;
        if constexpr ((j & 1) != 0)
            load16_to_lds(rv, kb.v + ld, vov[i]);
        else
            load16_to_lds(rk, kb.k + ld, vok[i]);
    };
    // All loads of the next tile into buffer bf.
    auto issue = [&](int bf) {
        static_for<2 * PERW>([&](auto jc) { issue_part(bf, jc); });
    };
    // The first key tiles (two with three buffers, one with two) are in
    // flight while the row vectors below are formed.
    if (nkt > t_lo) {
        issue(0);
        if constexpr (NBUF == 3)
            issue(1);
    }

    // ---- Q and dO rows of the lane (B operands), lse2 / rowdot ----
    e16x8 qf[KS], of[KS];
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
            qf[ks] = __builtin_bit_cast(e16x8, a);
            of[ks] = __builtin_bit_cast(e16x8, c);
        }
    }
    // ---- lse2 and rowdot of the lane's row, written for the key-tile kernel
    //      (which runs after this one).  rowdot = sum_d dO * O with the same
    //      operations in the same order as the preprocess kernel, whose lane
    //      c (of 16 per row) keeps one running sum over chunks c, c + 16, ...
    //      of the row (16 bytes each, summed left to right) before a
    //      butterfly over the 16 lanes (partners c^8, c^4, c^2, c^1).  Chunk
    //      j = 2*ks + g2 lives in lane half g2 and belongs to preprocess lane
    //      j % 16 = 2*(ks % 8) + g2, so cs[ks % 8] carries that lane's sum;
    //      the first three butterfly steps are in-lane and the last one pairs
    //      the two lane halves.  The results are bit-identical. ----
    float l2 = INFINITY, rd = 0.f;
    {
        float cs[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            cs[c] = 0.f;
        if (qok) {
            const uint16_t *orow = p.o + row_offset(p, b, si.tok_q, qrow, p.o_sb, p.o_ss) + h * p.o_sh;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int d0 = 16 * ks + 8 * g2;
                if (d0 < p.D) {
                    const uint4 ov = *reinterpret_cast<const uint4 *>(orow + d0);
                    const u32x4 dw = __builtin_bit_cast(u32x4, of[ks]);
                    const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
                    float acc = cs[ks & 7];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        acc += elem2f<F16>((uint16_t)(ow[t] & 0xffff)) * elem2f<F16>((uint16_t)(dw[t] & 0xffff));
                        acc += elem2f<F16>((uint16_t)(ow[t] >> 16)) * elem2f<F16>((uint16_t)(dw[t] >> 16));
                    }
                    cs[ks & 7] = acc;
                }
            }
        }
        float a4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            a4[c] = cs[c] + cs[c ^ 4];
        const float a2_0 = a4[0] + a4[2], a2_1 = a4[1] + a4[3];
        const float half = a2_0 + a2_1;
        const float sum = half + __shfl_xor(half, 32);
        if (qok) {
            const float lse = p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow];
            l2 = (lse == -INFINITY) ? INFINITY : lse * 1.4426950408889634f;
            rd = sum;
            if (g2 == 0) {
                const int64_t wr = (int64_t)h * p.rows + si.ws_row + qrow;
                p.lse2[wr] = l2;
                p.rowdot[wr] = rd;
            }
        }
    }
    wait_loads();   // land them and the first key tiles before the tile loop

    // -dO as the dP operand and rowdot as its initial value: the product
    // then yields rowdot - dP (sign flips are exact in bf16).
    f32x16 rdt;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        of[ks] = __builtin_bit_cast(e16x8, __builtin_bit_cast(u32x4, of[ks]) ^ 0x80008000u);
    if constexpr (Shape::BIG) {
        // Q and -dO rows live in accumulation registers (operands of the
        // inline S^T / dP^T products)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            asm volatile("" : "+a"(qf[ks]), "+a"(of[ks]));
    }
#pragma unroll
    for (int e = 0; e < 16; ++e)
        rdt[e] = rd;

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        zero(acc[db]);


    if (nkt > t_lo) {
        // LDS byte offsets of this lane's operand reads in the current
        // buffer (V is BYTES further):
        //  gq[ks]:    16-byte read of K / V row l32, tile chunk 2*ks + g2 (+ 32
        //             rows per key block);
        //  tq[db][h]: transposing read of K rows 4*g2 + rr + 8*h (+ 16 rows per
        //             k-step), tile chunk 4*db + 2*h16 + b1, 8-byte half c16 & 1.
        constexpr int BUFB = (int)sizeof(Buf);
        int gq[KS], tq[DB][2];
        {
            const int sw = swz<L::PCH>(l32);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gq[ks] = l32 * L::PB + (((2 * ks + g2) ^ sw) << 4);
            const int c16 = lane & 15, rr = c16 >> 2, h16 = (lane >> 4) & 1, b1 = (c16 >> 1) & 1;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int row = 4 * g2 + rr + 8 * hf;
                    tq[db][hf] = row * L::PB +
                                 (((4 * db + 2 * h16 + b1) ^ swz<L::PCH>(row)) << 4) + (c16 & 1) * 8;
                }
        }
        const uint8_t *lds = reinterpret_cast<const uint8_t *>(&sm.buf[0]);


        // ---- Each key tile as NSLOT MFMA slots, issued in this order: ----
        //   S^T, dP^T of keys 0-31 (k-steps over D)   slots 0 .. NB-1
        //   S^T, dP^T of keys 32-63                   NB .. 2NB-1        + dS of keys 0-31
        //   dQ k-steps over keys 0-31                 2NB .. 2NB+NQ-1    + dS of keys 32-63
        //   dQ k-steps over keys 32-63                2NB+NQ .. NSLOT-1
        constexpr int NB = 2 * KS;
        constexpr int NQ = 2 * DB;
        constexpr int NSLOT = 2 * NB + 2 * NQ;
        constexpr int RA = 4;                        // read-ahead (divides NSLOT)
        // the barrier and the loads of the tile after next early in the
        // tile, where the S^T / dP^T products leave the issue slots idle
        // (when the keep bits are drawn, the Philox calls fill that phase
        // and the load set-up there makes the allocator spill: then in the
        // dQ phase, with the keep words stored right after the barrier's
        // wait); the 16-byte read offsets move at MOV, after the tile's last
        // such read
        constexpr int BAR =
            !DRAW ? 2 : (2 * NB + NQ / 2 < NSLOT - RA ? 2 * NB + NQ / 2 : NSLOT - RA - 1);
        constexpr int MOV = 2 * NB;
        constexpr int KST = NBUF == 3 && DRAW ? BAR + 1 : 2 * NB;   // keep-word store slot
        static_assert(NSLOT % RA == 0, "ring length must divide the slot count");
        static_assert((DRAW ? BAR >= 2 * NB - RA && BAR + RA < NSLOT : BAR + 1 < NB) &&
                          MOV >= 2 * NB - RA && MOV + RA < NSLOT && KST >= 2 * NB,
                      "slot events");
        constexpr int LPT = 2 * PERW;             // loads per wave per tile
        static_assert(NBUF != 3 || BAR + LPT < NSLOT, "load slots");

        auto op_read = [&](auto ic) -> e16x8 {
            constexpr int i = decltype(ic)::value;
            if constexpr (i < 2 * NB) {
                constexpr int mb = i / NB, jj = i % NB, ks = jj >> 1;
                return lds16b(lds + gq[ks] + 32 * mb * L::PB + ((jj & 1) ? L::BYTES : 0));
            } else {
                constexpr int jj = i - 2 * NB, kk = jj / DB, db = jj % DB;
                return tr_pair(lds + tq[db][0] + 16 * kk * L::PB, lds + tq[db][1] + 16 * kk * L::PB);
            }
        };
        __syncthreads();
        e16x8 ring[RA];
        static_for<RA>([&](auto ic) { ring[decltype(ic)::value] = op_read(ic); });

        // Smallest last visible key over the wave's rows (-1 if any row is
        // past the end) and largest first visible key: key tiles wholly
        // between the two are visible to every row of the wave and need no
        // mask.  They are the tiles f_lo .. f_hi-1 (none if f_lo >= f_hi).
        const int kmin_w =
            r0w + 31 < Lq ? (p.win_r >= 0 ? min(Lk - 1, r0w + off + p.win_r) : Lk - 1) : -1;
        const int kfirst_w = LOCAL ? r0w + 31 + off - p.win_l : 0;
        const int f_lo = max(t_lo, kfirst_w <= 0 ? 0 : (kfirst_w + kDqKeys - 1) / kDqKeys);
        const int f_hi = min(nkt, max(0, (kmin_w + 1) / kDqKeys));

        int cur = 0;
        // One key tile, with (IC<1>) or without (IC<0>) the element mask (the
        // same slots otherwise).
        auto tile = [&](int t, auto maskc) {
            // two buffers: the next tile's loads go into the buffer every
            // wave finished with before the barrier that ended the last tile
            if constexpr (NBUF == 2)
                issue(__builtin_amdgcn_readfirstlane(cur ^ 1));   // (scalar: an LDS base)
            const int n0 = t * kDqKeys;
            // Masked tiles: element (32*mb + 8*r4 + t) of the lane's keys (+
            // 4*g2) is kept iff it is <= kthr and (LOCAL) >= kthr_lo (the
            // lane's row sees keys row + off - win_l .. row + off + win_r,
            // none past the key end, none if the row is past the end).  With
            // a left window both are formed per tile from the lane index:
            // every register of the wave is taken.
            int kthr = 0, kthr_lo = 0;
            if constexpr (!LOCAL) {
                kthr = klim - n0 - 4 * g2;
            } else if constexpr (decltype(maskc)::value != 0) {
                const int ln = lane_here();
                const int row = r0w + (ln & 31), kg = n0 + 4 * (ln >> 5);
                const int hi = p.win_r >= 0 ? min(Lk - 1, row + off + p.win_r) : Lk - 1;
                kthr = row < Lq ? hi - kg : -1;
                kthr_lo = row + off - p.win_l - kg;
            }
            const int delta = cur == NBUF - 1 ? -(NBUF - 1) * BUFB : BUFB;

            f32x16 st[2], dpt[2];
            const f32x16 z = {};
            // dropout keep bits of the tile: bit 16*mb + 4*r4 + tt for the
            // lane's row and key 32*mb + 8*r4 + 4*g2 + tt
            uint32_t kw = 0, kwr0 = 0, kwr1 = 0;
            e16x4 dh[4];
            e16x8 dsa[4];
            f32x4 dv;

            auto pw_elem = [&](auto mbc, auto ec) {
                constexpr int mb = decltype(mbc)::value, e = decltype(ec)::value;
                constexpr int r4 = e >> 2, tt = e & 3;
                float x, cg = 1.f;
                if constexpr (SOFTCAP) {
                    // capped score tanh * c (base 2); dS picks up 1 - tanh^2
                    const float th = cap_tanh(st[mb][e], p.cap_in);
                    x = __builtin_amdgcn_exp2f(fmaf(th, p.cap_out, -l2));
                    cg = fmaf(-th, th, 1.f);
                } else {
                    x = __builtin_amdgcn_exp2f(st[mb][e] * p.scale_log2 - l2);
                }
                if constexpr (decltype(maskc)::value) {
                    constexpr int ke = 32 * mb + 8 * r4 + tt;
                    x = ke <= kthr && (!LOCAL || ke >= kthr_lo) ? x : 0.f;
                }
                // dpt holds rowdot - dP; with dropout dS = P (M dP - rowdot)
                float d;
                if constexpr (DROP) {
                    const float zi = keep_mult(kw, 16 * mb + 4 * r4 + tt, p.drop_inv);
                    const float rd_ = rdt[e];
                    d = x * cg * fmaf(zi, rd_ - dpt[mb][e], -rd_);
                } else {
                    d = SOFTCAP ? x * cg * -dpt[mb][e] : x * -dpt[mb][e];
                }
                keep_here(d);
                dv[tt] = d;
                if constexpr (tt == 3) {
                    dh[r4] = to_elem<F16>(dv);
                    if constexpr ((r4 & 1) != 0)
                        dsa[2 * mb + (r4 >> 1)] = concat(dh[r4 - 1], dh[r4]);
                }
            };

            // one Philox call: keys 4 (8*mb + 2*r4 + g2) .. +3 of the lane's
            // row (row and half from the lane index: no register holds
            // them across the loop)
            auto drop_call = [&](auto cc) {
                constexpr int c = decltype(cc)::value, mb = c >> 2, r4 = c & 3;
                const int ln = lane_here();
                const uint32_t c0 = (uint32_t)(n0 >> 2) + 8 * mb + 2 * r4 + (ln >> 5);
                const uint32_t row = (uint32_t)(r0w + (ln & 31));
                kw |= keep_nibble<false>(c0, row, drop_c2, p) << (16 * mb + 4 * r4);
            };

            // The tile's keep bits for the key-tile kernel: lane half g
            // writes the word of keys 32*g .. 32*g+31 (word 2t + g) of its
            // row, nibble 2*r4 + g2 of it from lane half g2 (one exchange
            // between the halves).
            auto keep_store = [&]() {
                const uint32_t other = (uint32_t)__shfl_xor((int)kw, 32);
                const int ln = lane_here();
                const int g = ln >> 5;
                const uint32_t n_lo = g ? other >> 16 : kw & 0xFFFFu;   // half 0's nibbles
                const uint32_t n_hi = g ? kw >> 16 : other & 0xFFFFu;   // half 1's nibbles
                const uint32_t word = spread_nibbles(n_lo) | (spread_nibbles(n_hi) << 4);
                const int row = r0w + (ln & 31);
                if (row < Lq)
                    p.keep[((int64_t)(2 * t + g) * p.H + h) * p.rows + si.ws_row + row] = word;
            };

            static_for<NSLOT>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const e16x8 a = ring[i % RA];
                // Above 128 (one wave per SIMD): one operand wait per two
                // slots, an even slot also waiting for the next slot's read.
                // (With two waves per SIMD the other wave covers the waits.)
                if constexpr (BIG && (i & 1) == 0 && i + 1 < NSLOT)
                    asm volatile("" ::"v"(ring[(i + 1) % RA]));
                if constexpr (i + RA < NSLOT)
                    ring[i % RA] = op_read(IC<i + RA>{});
                else if constexpr (NBUF == 3)
                    ring[i % RA] = op_read(IC<i + RA - NSLOT>{});   // next tile
                // after the tile's last Philox call
                if constexpr (DRAW && i == KST)
                    if (p.keep)   // (no keep words when they would be too large)
                        keep_store();
                // Caller's words: the lane's row's two words of the tile
                // (slot 0), its half's nibbles of each into kw (slot 2;
                // nibble 2 r4 + g2 of word mb is kw's nibble 4 mb + r4).
                if constexpr (READW && i == 0) {
                    const uint32_t *wl = reinterpret_cast<const uint32_t *>(
                                             lds + cur * BUFB + (int)sizeof(KVBuf<DP>)) +
                                         64 * w + (lane_here() & 31);
                    kwr0 = wl[0];
                    kwr1 = wl[32];
                }
                if constexpr (READW && i == 2) {
                    const uint32_t sh = 4u * (uint32_t)(lane_here() >> 5);
                    kw = gather_nibbles(kwr0 >> sh) | (gather_nibbles(kwr1 >> sh) << 16);
                }
                // Philox calls: block 0's over its S^T / dP^T slots, block 1's
                // over the next NB slots (before each block's dS)
                if constexpr (DRAW && i < 2 * NB)
                    static_for<4>([&](auto rc) {
                        constexpr int r4 = decltype(rc)::value;
                        if constexpr ((i % NB) == r4 * NB / 4)
                            drop_call(IC<4 * (i / NB) + r4>{});
                    });
                if constexpr (i < 2 * NB && BIG) {
                    // above 128 the kernel needs more than 256 registers, so
                    // the compiler's MFMAs use accumulation registers: S^T and
                    // dP^T as inline MFMAs in ordinary registers instead (Q and
                    // dO operands in accumulation registers), as the key-tile
                    // kernel does
                    constexpr int mb = i / NB, jj = i % NB, ks = jj >> 1;
                    if constexpr ((jj & 1) != 0) {
                        if constexpr (ks == 0)   // from rowdot, without a copy
                            mfma32_vc<F16>(dpt[mb], a, of[ks], rdt);
                        else
                            mfma32_vacc<F16>(dpt[mb], a, of[ks]);
                    } else if constexpr (ks == 0) {
                        mfma32_vz<F16>(st[mb], a, qf[ks]);
                    } else {
                        mfma32_vacc<F16>(st[mb], a, qf[ks]);
                    }
                } else if constexpr (i < 2 * NB) {
                    constexpr int mb = i / NB, jj = i % NB, ks = jj >> 1;
                    if constexpr ((jj & 1) != 0) {
                        dpt[mb] = mfma32<F16>(a, of[ks], ks == 0 ? rdt : dpt[mb]);
                        keep_here(dpt[mb]);
                    } else {
                        st[mb] = mfma32<F16>(a, qf[ks], ks == 0 ? z : st[mb]);
                        keep_here(st[mb]);
                    }
                } else {
                    constexpr int jj = i - 2 * NB, kk = jj / DB, db = jj % DB;
                    acc[db] = mfma32<F16>(a, dsa[kk], acc[db]);   // dQ^T
                    if constexpr (BIG)
                        keep_here_acc(acc[db]);
                    else
                        keep_here(acc[db]);
                }
                // inline MFMA results: 12 wait states before the first read
                if constexpr (BIG && i == NB)
                    mfma_settle(st[0], dpt[0]);
                if constexpr (BIG && i == 2 * NB)
                    mfma_settle(st[1], dpt[1]);
                // dS of keys 0-31 over slots NB .. 2NB-1, of keys 32-63 over
                // 2NB .. 2NB+NQ-1 (16 elements each)
                if constexpr (i >= NB && i < 2 * NB) {
                    constexpr int u = i - NB;
                    static_for<16 * (u + 1) / NB - 16 * u / NB>(
                        [&](auto ec) { pw_elem(IC<0>{}, IC<16 * u / NB + decltype(ec)::value>{}); });
                }
                if constexpr (i >= 2 * NB && i < 2 * NB + NQ) {
                    constexpr int u = i - 2 * NB;
                    static_for<16 * (u + 1) / NQ - 16 * u / NQ>(
                        [&](auto ec) { pw_elem(IC<1>{}, IC<16 * u / NQ + decltype(ec)::value>{}); });
                }
                if constexpr (NBUF == 3 && i == BAR) {
                    // every wave has finished with the last tile's buffer and
                    // the only loads in flight are the next tile's (issued one
                    // tile ago); a bare barrier (reads in flight touch this
                    // tile's buffer only)
                    wait_loads<0>();
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                }
                // the loads of the tile after next, one per slot (all in one
                // slot measured 0.2-0.5% slower)
                if constexpr (NBUF == 3 && i > BAR && i <= BAR + 2 * PERW)
                    issue_part(cur == 0 ? NBUF - 1 : cur - 1, IC<i - BAR - 1>{});
                if constexpr (NBUF == 3 && i == MOV) {
                    // every 16-byte read of this tile is issued: move them on
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        gq[ks] += delta;
                }
                if constexpr (NBUF == 3 && i == NSLOT - RA - 1) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        tq[db][0] += delta;
                        tq[db][1] += delta;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (NBUF == 2) {
                // the next tile: its loads landed and every wave is done
                // with this buffer; reads restart from the other one
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    gq[ks] += delta;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    tq[db][0] += delta;
                    tq[db][1] += delta;
                }
                wait_loads<0>();
                __syncthreads();
                static_for<RA>([&](auto ic) { ring[decltype(ic)::value] = op_read(ic); });
            }
            cur = cur == NBUF - 1 ? 0 : cur + 1;
        };
        // A key tile none of the wave's rows sees (under the causal mask the
        // tiles right of the diagonal of its rows, under a window also those
        // left of it): only the tile's shared work -- the barrier that
        // publishes the next tile, the wave's share of the loads, the read
        // offsets moved to the next buffer, the operand reads of the next
        // tile's first slots -- and none of its products, so the other wave
        // on the SIMD has the matrix unit to itself.
        auto skip = [&]() {
            const int delta = cur == NBUF - 1 ? -(NBUF - 1) * BUFB : BUFB;
            if constexpr (NBUF == 2)
                issue(__builtin_amdgcn_readfirstlane(cur ^ 1));
            else {
                wait_loads<0>();
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                issue(cur == 0 ? NBUF - 1 : cur - 1);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gq[ks] += delta;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                tq[db][0] += delta;
                tq[db][1] += delta;
            }
            if constexpr (NBUF == 2) {
                wait_loads<0>();
                __syncthreads();
            }
            static_for<RA>([&](auto ic) { ring[decltype(ic)::value] = op_read(ic); });
            cur = cur == NBUF - 1 ? 0 : cur + 1;
        };
        // Key tiles the wave's rows see: tv_lo .. tv_end-1 (none if the wave
        // has no row: all skipped).  Skipped t_lo .. tv_lo-1, masked tv_lo ..
        // f_lo-1, unmasked f_lo .. f_hi-1, masked f_hi .. tv_end-1, skipped
        // tv_end .. nkt-1 (separate loops: one masked loop entered twice
        // makes the register allocator spill).
        const int rl_w = min(r0w + 31, Lq - 1);   // the wave's last row
        int tv_lo = t_lo, tv_end = t_lo;
        if (r0w < Lq) {
            const int kv_lo = LOCAL ? max(0, r0w + off - p.win_l) : 0;
            const int kv_hi = p.win_r >= 0 ? min(Lk - 1, rl_w + off + p.win_r) : Lk - 1;
            if (kv_hi >= kv_lo) {
                tv_lo = max(t_lo, kv_lo / kDqKeys);
                tv_end = max(tv_lo, min(nkt, kv_hi / kDqKeys + 1));
            }
        }
        int t = t_lo;
        const int m_end = f_lo < f_hi ? f_lo : tv_lo;
        const int u_end = f_lo < f_hi ? f_hi : tv_lo;
        if constexpr (LOCAL) {
            for (; t < tv_lo; ++t)
                skip();
            for (; t < m_end; ++t)
                tile(t, IC<1>{});
        }
        for (; t < u_end; ++t)
            tile(t, IC<0>{});
        for (; t < tv_end; ++t)
            tile(t, IC<1>{});
        for (; t < nkt; ++t)
            skip();
        // loads issued past the last tile must land before LDS is released
        wait_loads<0>();
    }

    // ---- dQ = scale * acc -> elements.  Accumulator of head-dim block db:
    //      column 32 db + 8 (r/4) + 4 g2 + r%4 of the lane's row l32 (lane
    //      index formed again: no register holds it across the loop).  Per
    //      pair of 8-column groups (j0 = 2 q, j1 = 2 q + 1) the halves
    //      trade their 8-byte pieces so that half 0 holds columns 8 j0 ..
    //      8 j0 + 7 and half 1 columns 8 j1 .. 8 j1 + 7: one 16-byte store
    //      per lane and pair (columns past head_dim, a multiple of 8, and
    //      rows past the end are not written). ----
    const int ln = lane_here();
    const int orow = r0w + (ln & 31), half = ln >> 5;
    uint16_t *dqrow =
        p.dq + row_offset(p, b, si.tok_q, orow < Lq ? orow : 0, p.dq_sb, p.dq_ss) + h * p.dq_sh;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        u32x2 pc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[i] = acc[db][4 * j + i] * p.scale;
            pc[j] = __builtin_bit_cast(u32x2, to_elem<F16>(v));
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            // lanes 32-63 of pc[2q] <-> lanes 0-31 of pc[2q+1]
            const auto s0 = __builtin_amdgcn_permlane32_swap(pc[2 * q][0], pc[2 * q + 1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(pc[2 * q][1], pc[2 * q + 1][1], false, false);
            const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
            const int col = 32 * db + 16 * q + 8 * half;
            if (orow < Lq && col < p.D)
                *reinterpret_cast<u32x4 *>(dqrow + col) = out;
        }
    }
}

// Workgroups of a shape: per batch and KV head, the head sets of its group
// times the query tiles of the rows per head (the mapping at the top of the
// kernel).
template <int DP, bool SMALL, bool LOCAL>
static int64_t dq_workgroups(const Params &p)
{
    constexpr int WAVES = DqShape<DP, SMALL>::WAVES;
    const int hpw = LOCAL ? std::min(p.G & -p.G, WAVES) : 1;
    const int rw = 32 * (WAVES / hpw);
    return (int64_t)((p.Sq + rw - 1) / rw) * (p.G / hpw) * p.Hk * p.batch;
}

template <int DP, bool F16, bool LOCAL, bool SOFTCAP, int DROP, bool SMALL>
static void launch_dq_s(const Params &p, hipStream_t st)
{
    using S = DqShape<DP, SMALL>;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<DP, F16, LOCAL, SOFTCAP, DROP, SMALL>),
                       dim3((unsigned)dq_workgroups<DP, SMALL, LOCAL>(p)), dim3(S::THREADS), 0, st, p);
}

// MI355X compute units: the small shape is taken at head dim 64 when the
// standard grid has fewer than two workgroups per CU.
constexpr int kCus = 256;

template <int DP, bool F16, bool LOCAL, bool SOFTCAP, int DROP>
static void launch_dq_d(const Params &p, hipStream_t st)
{
    if constexpr (DP == 64) {
        if (dq_workgroups<64, false, false>(p) < 2 * kCus) {
            launch_dq_s<DP, F16, LOCAL, SOFTCAP, DROP, true>(p, st);
            return;
        }
    }
    launch_dq_s<DP, F16, LOCAL, SOFTCAP, DROP, false>(p, st);
}

template <bool LOCAL, bool SOFTCAP, int DROP>
static hipError_t launch_dq_t(const Params &p, int dpad, hipStream_t st)
{
#define FA_DQ_CASE(D)                                                 \
    case D:                                                           \
        if (p.f16)                                                    \
            launch_dq_d<D, true, LOCAL, SOFTCAP, DROP>(p, st);        \
        else                                                          \
            launch_dq_d<D, false, LOCAL, SOFTCAP, DROP>(p, st);       \
        break;
    switch (dpad) {
        FA_DQ_CASE(64)
        FA_DQ_CASE(96)
        FA_DQ_CASE(128)
        FA_DQ_CASE(192)
        FA_DQ_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef FA_DQ_CASE
    return hipGetLastError();
}

// The dropout instantiations build in a translation unit of their own
// (fa_dq_dropout.hip and fa_dq_keep.hip include this file with
// FA_TU_DROPOUT = 1 and 2), so that the
// two halves compile in parallel.
template <int DROP>
hipError_t launch_dq_v(const Params &p, int dpad, hipStream_t st)
{
    if (p.softcap > 0.f)
        return p.win_l >= 0 ? launch_dq_t<true, true, DROP>(p, dpad, st)
                            : launch_dq_t<false, true, DROP>(p, dpad, st);
    return p.win_l >= 0 ? launch_dq_t<true, false, DROP>(p, dpad, st)
                        : launch_dq_t<false, false, DROP>(p, dpad, st);
}

#if FA_TU_DROPOUT
template hipError_t launch_dq_v<FA_TU_DROPOUT>(const Params &, int, hipStream_t);
#else
extern template hipError_t launch_dq_v<1>(const Params &, int, hipStream_t);
extern template hipError_t launch_dq_v<2>(const Params &, int, hipStream_t);

hipError_t launch_dq(const Params &p, int dpad, hipStream_t st)
{
    if (!(p.drop_p > 0.f))
        return launch_dq_v<0>(p, dpad, st);
    return p.keep_given ? launch_dq_v<2>(p, dpad, st) : launch_dq_v<1>(p, dpad, st);
}
#endif

}  // namespace fa
