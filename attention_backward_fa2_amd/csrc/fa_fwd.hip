// fa_fwd.hip -- query-stationary attention forward on gfx950 (CDNA4): the
// output O and the per-row log-sum-exp that the backward consumes.
//
// For each query row i the forward computes the softmax of the scaled scores
// over the visible keys and O_i = sum_j P_ij V_j, keeping only a running
// maximum, a running sum and the unnormalised output while it streams key
// tiles (the online softmax of the Triton FA2 teaching page's forward inner
// loop: per key block the block maximum, exponentials of the shifted scores
// in base 2, the partial output and sum rescaled by exp2(old max - new max),
// one division by the sum at the end; its outer kernel stores max + log2(sum)
// for the backward).  Unlike that page, Q is not pre-scaled and rounded to
// bf16: the scale enters in fp32, and the stored LSE is the natural log the
// backward's interface expects.
//
// Layout of the work (the same as the query-stationary dQ kernel): one
// workgroup of 8 wave64s (two per SIMD) owns 256 query rows of one head;
// wave w owns rows 32w .. 32w+31, whose Q rows stay in registers as the B
// operand of S^T = K Q^T over 64-key tiles.  The accumulator of S^T holds
// one query row and 16 keys per lane, so the running maximum and sum are
// one register each (the two lane halves hold the two halves of a block's
// keys and combine with one cross-half exchange), and P (bf16) is directly
// the B operand of O^T += V^T P^T, with V^T read through transposing LDS
// reads; the accumulator of O^T again holds one query row per lane, so the
// rescale factor is lane-local.
//
// The rescale is lazy: the running maximum only moves (and O^T and the sum
// are rescaled) when some row of the wave sees a tile maximum more than
// 2^8 above it, so P stays below 256 and the exponentials stay exact in
// fp32; the final division by the sum makes the result independent of which
// maximum was used.
//
// K and V tiles arrive by buffer loads straight into the swizzled LDS layout
// of fa_mfma.h, three buffers deep; the tile body is a fixed sequence of
// MFMA slots: S^T of keys 0-31, S^T of keys 32-63 (with the maximum of keys
// 0-31), then the O^T k-steps, with P of keys 0-31 formed before them and P
// of keys 32-63 alongside the first half.
#include "fa_mfma.h"
#include "fa_philox.h"

#ifndef FA_TU_DROPOUT
#define FA_TU_DROPOUT 0
#endif

namespace fa {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kFwdKeys = 64;                 // keys per streamed tile

// Workgroup shape by padded head dim (as for the dQ kernel): up to 128,
// eight waves (two per SIMD, 256 rows) and three K/V buffers; at 192 and
// 256, four waves (128 rows) and two buffers.
template <int DP>
struct FwdShape {
    static constexpr bool BIG = DP > 128;
    static constexpr int WAVES = BIG ? 4 : 8;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS = 32 * WAVES;
    static constexpr int NBUF = BIG ? 2 : 3;
};

template <int DP>
struct __attribute__((aligned(16))) FwdKV {
    uint8_t k[Tile64<DP>::BYTES];
    uint8_t v[Tile64<DP>::BYTES];
};

template <int DP>
struct __attribute__((aligned(16))) FwdSmem {
    FwdKV<DP> buf[FwdShape<DP>::NBUF];
};

// LOCAL: a left window bounds the visible keys from below (win_l >= 0);
// otherwise win_l < 0 and only the upper bound is masked.  SOFTCAP: scores
// soft-capped (softcap > 0).  DROP: dropout on P for O (drop_p > 0).
template <int DP, bool F16, bool LOCAL, bool SOFTCAP, bool DROP>
__global__ void __launch_bounds__(FwdShape<DP>::THREADS, 1) fa_fwd_kernel(Params p)
{
    constexpr int KS = DP / 16;                  // k-steps over the head dim
    constexpr int DB = DP / 32;                  // 32-wide head-dim blocks
    constexpr bool BIG = FwdShape<DP>::BIG;
    constexpr int NBUF = FwdShape<DP>::NBUF;
    constexpr int WAVES = FwdShape<DP>::WAVES;
    constexpr int ROWS = FwdShape<DP>::ROWS;
    using L = Tile64<DP>;
    constexpr int PERW = L::NLOAD / WAVES;       // 1 KB wave loads per tensor per wave
    static_assert(PERW >= 1 && L::NLOAD % WAVES == 0, "tile load split");
    __shared__ FwdSmem<DP> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;

    // Workgroup -> (query tile, batch, KV head, head in group), longest
    // (last query tile under the causal mask) first within the (batch, KV
    // head) groups an XCD runs side by side (xcd_group_order).
    const int nbg = p.batch * p.Hk;
    const int nqt = (p.Sq + ROWS - 1) / ROWS;
    const int lin = blockIdx.x;
    int u, bg;   // u = (last query tile - mt) * G + hh
    xcd_group_order(lin, nbg, nqt * p.G, u, bg);
    const int hh = u % p.G;
    const int mt = nqt - 1 - u / p.G;
    const int hk = bg % p.Hk, b = bg / p.Hk;
    const int h = hk * p.G + hh;

    const SeqInfo si = seq_info(p, b);
    const int q0 = mt * ROWS;
    if (q0 >= si.Lq)
        return;
    const int Lq = si.Lq, Lk = si.Lk;
    const int off = Lk - Lq;                     // bottom-right alignment offset
    const int qrow = q0 + 32 * w + l32;          // this lane's query row
    const bool qok = qrow < Lq;
    const uint32_t drop_c2 = (uint32_t)(b * p.H + h);   // Philox counter word 2

    // Key tiles t_lo .. nkt-1 hold the keys visible to some row of this
    // query tile (rows q0 .. q_last see keys k_lo .. k_hi at most).
    const int q_last = min(q0 + ROWS, Lq) - 1;
    const int k_lo = LOCAL ? max(0, q0 + off - p.win_l) : 0;
    const int k_hi = p.win_r >= 0 ? min(Lk - 1, q_last + off + p.win_r) : Lk - 1;
    const int t_lo = k_lo / kFwdKeys;
    const int nkt = k_hi >= k_lo ? k_hi / kFwdKeys + 1 : t_lo;
    // Visible keys of this lane's row: kfirst <= key <= klim.
    const int klim = qok ? (p.win_r >= 0 ? min(Lk - 1, qrow + off + p.win_r) : Lk - 1) : -1;
    const int kfirst = LOCAL ? qrow + off - p.win_l : 0;

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
    // Loads of the next key tile into buffer bf (tiles strictly in order;
    // past the last tile: empty bound, zeros, no memory access).
    const uint16_t *k_next = p.k + hk * p.k_sh + row_offset(p, b, si.tok_k, 0, p.k_sb, p.k_ss);
    const uint16_t *v_next = p.v + hk * p.v_sh + row_offset(p, b, si.tok_k, 0, p.v_sb, p.v_ss);
    int n_next = t_lo * kFwdKeys, n_left = nkt - t_lo;
    const int64_t kstep = (int64_t)kFwdKeys * p.k_ss, vstep = (int64_t)kFwdKeys * p.v_ss;
    k_next += t_lo * kstep;
    v_next += t_lo * vstep;
    auto issue = [&](int bf) {
        if constexpr (!BIG)   // (at 256 the pins leave no legal register class)
            keep_scalar_here(n_next, n_left, k_next, v_next);
        const int kv = n_left > 0 ? min(kFwdKeys, Lk - n_next) : 0;
        const uint32_t nk = kv ? (uint32_t)((kv - 1) * (int)p.k_ss * 2 + p.D * 2) : 0u;
        const uint32_t nv = kv ? (uint32_t)((kv - 1) * (int)p.v_ss * 2 + p.D * 2) : 0u;
        const auto rk = make_rsrc(k_next, nk);
        const auto rv = make_rsrc(v_next, nv);
        n_next += kFwdKeys;
        --n_left;
        k_next += kstep;
        v_next += vstep;
        if constexpr (!BIG)   // (at 256 the pins leave no legal register class)
            keep_scalar_here(n_next, n_left, k_next, v_next);
        FwdKV<DP> &kb = sm.buf[bf];
#pragma unroll
        for (int i = 0; i < PERW; ++i) {
            const int ld = (w * PERW + i) * 1024;
            load16_to_lds(rk, kb.k + ld, vok[i]);
            load16_to_lds(rv, kb.v + ld, vov[i]);
        }
    };
    if (nkt > t_lo) {
        issue(0);
        if constexpr (NBUF == 3)
            issue(1);
    }

    // ---- Q rows of the lane (B operand of S^T) ----
    e16x8 qf[KS];
    {
        const int qr = qok ? qrow : Lq - 1;
        const uint16_t *qp = p.q + row_offset(p, b, si.tok_q, qr, p.q_sb, p.q_ss) + h * p.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * g2;
            u32x4 a = 0;
            if (qok && d0 < p.D)
                a = *reinterpret_cast<const u32x4 *>(qp + d0);
            qf[ks] = __builtin_bit_cast(e16x8, a);
        }
        if constexpr (BIG) {
            // Q rows live in accumulation registers (operands of the inline
            // S^T products)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                asm volatile("" : "+a"(qf[ks]));
        }
    }
    wait_loads();   // land them and the first key tiles before the tile loop

    f32x16 acc[DB];                 // O^T: column = the lane's row, rows = d
#pragma unroll
    for (int db = 0; db < DB; ++db)
        zero(acc[db]);
    // Running maximum of S * scale * log2(e) (base-2 units) and the lane's
    // part of the running sum of P (the lane half g2 sums its half of the
    // keys; the halves are added at the end).
    float mrun = -INFINITY, lsum = 0.f;

    if (nkt > t_lo) {
        // LDS byte offsets of this lane's operand reads in the current
        // buffer: gq[ks] the 16-byte read of K row l32, tile chunk
        // 2*ks + g2 (+ 32 rows per key block); tq[db][h] the transposing
        // read of V rows 4*g2 + rr + 8*h (+ 16 rows per k-step), tile chunk
        // 4*db + 2*h16 + b1, 8-byte half c16 & 1 (V is BYTES after K).
        constexpr int BUFB = (int)sizeof(FwdKV<DP>);
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
                    tq[db][hf] = L::BYTES + row * L::PB +
                                 (((4 * db + 2 * h16 + b1) ^ swz<L::PCH>(row)) << 4) + (c16 & 1) * 8;
                }
        }
        const uint8_t *lds = reinterpret_cast<const uint8_t *>(&sm.buf[0]);

        // ---- Each key tile as NSLOT MFMA slots: ----
        //   S^T of keys 0-31 (k-steps over D)        slots 0 .. NB-1
        //   S^T of keys 32-63                        NB .. 2NB-1      + maximum of keys 0-31
        //   (tile maximum, lazy rescale, P of keys 0-31 at the end of slot 2NB-1)
        //   O^T k-steps over keys 0-31               2NB .. 2NB+2DB-1 + P of keys 32-63
        //   O^T k-steps over keys 32-63              2NB+2DB .. NSLOT-1
        constexpr int NB = KS;
        constexpr int NO = 4 * DB;
        constexpr int NSLOT = 2 * NB + NO;
        constexpr int RA = 4;                        // read-ahead (divides NSLOT)
        constexpr int BAR = (2 * NB + NO / 2 < NSLOT - RA) ? 2 * NB + NO / 2 : NSLOT - RA - 1;
        static_assert(NSLOT % RA == 0, "ring length must divide the slot count");
        static_assert(BAR >= 2 * NB - RA && BAR + RA < NSLOT, "barrier slot");

        auto op_read = [&](auto ic) -> e16x8 {
            constexpr int i = decltype(ic)::value;
            if constexpr (i < 2 * NB) {
                constexpr int mb = i / NB, ks = i % NB;
                return lds16b(lds + gq[ks] + 32 * mb * L::PB);
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
        const int r0w = q0 + 32 * w;
        const int kmin_w =
            r0w + 31 < Lq ? (p.win_r >= 0 ? min(Lk - 1, r0w + off + p.win_r) : Lk - 1) : -1;
        const int kfirst_w = LOCAL ? r0w + 31 + off - p.win_l : 0;
        const int f_lo = max(t_lo, kfirst_w <= 0 ? 0 : (kfirst_w + kFwdKeys - 1) / kFwdKeys);
        const int f_hi = min(nkt, max(0, (kmin_w + 1) / kFwdKeys));
        const float c2 = p.scale_log2;

        int cur = 0;
        auto tile = [&](int t, auto maskc) {
            constexpr bool MASK = decltype(maskc)::value != 0;
            // two buffers: the next tile's loads go into the buffer every
            // wave finished with before the barrier that ended the last tile
            if constexpr (NBUF == 2)
                issue(__builtin_amdgcn_readfirstlane(cur ^ 1));   // (scalar: an LDS base)
            const int n0 = t * kFwdKeys;
            // element (32*mb + 8*r4 + tt) of the lane's keys (+ 4*g2) is
            // visible iff it is <= kthr and (LOCAL) >= kthr_lo
            const int kthr = klim - n0 - 4 * g2;
            const int kthr_lo = kfirst - n0 - 4 * g2;
            const int delta = cur == NBUF - 1 ? -(NBUF - 1) * BUFB : BUFB;

            f32x16 st[2];
            const f32x16 z = {};
            // dropout keep bits of the tile: bit 16*mb + 4*r4 + tt for the
            // lane's row and key 32*mb + 8*r4 + 4*g2 + tt
            uint32_t kw = 0;
            float mx0 = -INFINITY, mx1 = -INFINITY;   // raw-score maxima of the two blocks
            float mu = 0.f;                           // maximum used for P (base 2)
            e16x4 ph[4];
            e16x8 pb[4];
            f32x4 pv;

            auto visible = [&](auto mbc, auto ec) -> bool {
                constexpr int mb = decltype(mbc)::value, e = decltype(ec)::value;
                constexpr int ke = 32 * mb + 8 * (e >> 2) + (e & 3);
                if constexpr (MASK)
                    return ke <= kthr && (!LOCAL || ke >= kthr_lo);
                else
                    return true;
            };
            // elements e, e+1 of block mb into its maximum (one three-input max)
            auto max_pair = [&](auto mbc, auto ec) {
                constexpr int mb = decltype(mbc)::value, e = decltype(ec)::value;
                if constexpr (SOFTCAP) {
                    // scores become the capped ones in base 2, tanh * c
                    st[mb][e] = cap_tanh(st[mb][e], p.cap_in) * p.cap_out;
                    st[mb][e + 1] = cap_tanh(st[mb][e + 1], p.cap_in) * p.cap_out;
                }
                const float s0 = visible(mbc, ec) ? st[mb][e] : -INFINITY;
                const float s1 = visible(mbc, IC<e + 1>{}) ? st[mb][e + 1] : -INFINITY;
                float &m = mb == 0 ? mx0 : mx1;
                m = fmaxf(m, fmaxf(s0, s1));
                keep_here(m);
            };
            auto p_elem = [&](auto mbc, auto ec) {
                constexpr int mb = decltype(mbc)::value, e = decltype(ec)::value;
                constexpr int r4 = e >> 2, tt = e & 3;
                float x = __builtin_amdgcn_exp2f((SOFTCAP ? st[mb][e] : st[mb][e] * c2) - mu);
                if constexpr (MASK)
                    x = visible(mbc, ec) ? x : 0.f;
                keep_here(x);
                lsum += x;   // the normaliser ignores dropout
                if constexpr (DROP)
                    pv[tt] = x * keep_mult(kw, 16 * mb + 4 * r4 + tt, p.drop_inv);
                else
                    pv[tt] = x;
                if constexpr (tt == 3) {
                    ph[r4] = to_elem<F16>(pv);
                    if constexpr ((r4 & 1) != 0)
                        pb[2 * mb + (r4 >> 1)] = concat(ph[r4 - 1], ph[r4]);
                }
            };

            // one Philox call: keys 4 (8*mb + 2*r4 + g2) .. +3 of the lane's row
            auto drop_call = [&](auto cc) {
                constexpr int c = decltype(cc)::value, mb = c >> 2, r4 = c & 3;
                const uint32_t c0 = (uint32_t)(n0 >> 2) + 8 * mb + 2 * r4 + g2;
                kw |= keep_nibble(c0, (uint32_t)qrow, drop_c2, p) << (16 * mb + 4 * r4);
            };
            // The tile's keep bits for the backward (p.keep, the caller's
            // buffer): lane half g writes the word of keys 32*g .. 32*g+31
            // (word 2t + g) of its row, nibble 2*r4 + g2 of it from lane half
            // g2 (one exchange between the halves).
            auto keep_store = [&]() {
                const uint32_t other = (uint32_t)__shfl_xor((int)kw, 32);
                const uint32_t n_lo = g2 ? other >> 16 : kw & 0xFFFFu;   // half 0's nibbles
                const uint32_t n_hi = g2 ? kw >> 16 : other & 0xFFFFu;   // half 1's nibbles
                const uint32_t word = spread_nibbles(n_lo) | (spread_nibbles(n_hi) << 4);
                if (qok)
                    p.keep[((int64_t)(2 * t + g2) * p.H + h) * p.rows + si.ws_row + qrow] = word;
            };

            static_for<NSLOT>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                const e16x8 a = ring[i % RA];
                // the eight Philox calls of the tile over the S^T slots,
                // before the first P
                if constexpr (DROP && i < 2 * NB - 1)
                    static_for<8>([&](auto cc) {
                        if constexpr (decltype(cc)::value * (2 * NB - 1) / 8 == i)
                            drop_call(cc);
                    });
                if constexpr (DROP && i == 2 * NB)
                    if (p.keep)
                        keep_store();
                if constexpr (i + RA < NSLOT)
                    ring[i % RA] = op_read(IC<i + RA>{});
                else if constexpr (NBUF == 3)
                    ring[i % RA] = op_read(IC<i + RA - NSLOT>{});   // next tile
                if constexpr (i < 2 * NB && BIG) {
                    // above 128 the kernel needs more than 256 registers, so
                    // the compiler's MFMAs use accumulation registers: S^T as
                    // inline MFMAs in ordinary registers instead (Q operand in
                    // accumulation registers), as the key-tile kernel does
                    constexpr int mb = i / NB, ks = i % NB;
                    if constexpr (ks == 0)
                        mfma32_vz<F16>(st[mb], a, qf[ks]);
                    else
                        mfma32_vacc<F16>(st[mb], a, qf[ks]);
                } else if constexpr (i < 2 * NB) {
                    constexpr int mb = i / NB, ks = i % NB;
                    st[mb] = mfma32<F16>(a, qf[ks], ks == 0 ? z : st[mb]);
                    keep_here(st[mb]);
                } else {
                    constexpr int jj = i - 2 * NB, kk = jj / DB, db = jj % DB;
                    acc[db] = mfma32<F16>(a, pb[kk], acc[db]);
                    if constexpr (BIG)
                        keep_here_acc(acc[db]);
                    else
                        keep_here(acc[db]);
                }
                // inline MFMA results: 12 wait states before the first read
                if constexpr (BIG && i == NB)
                    mfma_settle(st[0]);
                if constexpr (BIG && i == 2 * NB - 1)
                    mfma_settle(st[1]);
                // maximum of keys 0-31 over the S^T slots of keys 32-63
                if constexpr (i >= NB && i < 2 * NB) {
                    constexpr int u = i - NB;
                    static_for<8 * (u + 1) / NB - 8 * u / NB>(
                        [&](auto ec) { max_pair(IC<0>{}, IC<2 * (8 * u / NB + decltype(ec)::value)>{}); });
                }
                if constexpr (i == 2 * NB - 1) {
                    // tile maximum of the row (both blocks, both lane halves)
                    static_for<8>([&](auto ec) { max_pair(IC<1>{}, IC<2 * decltype(ec)::value>{}); });
                    float mt = fmaxf(mx0, mx1);
                    mt = fmaxf(mt, __shfl_xor(mt, 32));
                    // -inf if no key of the tile is visible
                    const float mt2 = SOFTCAP ? mt : mt * c2;
                    // Lazy rescale: move the running maximum only if some row
                    // of the wave would see P above 2^8 otherwise.
                    const bool need = mt2 > mrun + 8.f;
                    if (__builtin_amdgcn_ballot_w64(need) != 0) {
                        const float mnew = fmaxf(mrun, mt2);
                        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
                        mrun = mnew;
                        lsum *= alpha;
#pragma unroll
                        for (int db = 0; db < DB; ++db)
                            acc[db] *= alpha;
                    }
                    mu = mrun == -INFINITY ? 0.f : mrun;
                    static_for<16>([&](auto ec) { p_elem(IC<0>{}, ec); });
                }
                // P of keys 32-63 over the O^T slots of keys 0-31
                if constexpr (i >= 2 * NB && i < 2 * NB + 2 * DB) {
                    constexpr int u = i - 2 * NB;
                    static_for<16 * (u + 1) / (2 * DB) - 16 * u / (2 * DB)>(
                        [&](auto ec) { p_elem(IC<1>{}, IC<16 * u / (2 * DB) + decltype(ec)::value>{}); });
                }
                if constexpr (NBUF == 3 && i == BAR) {
                    // every 16-byte read of this tile is issued: move them on
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        gq[ks] += delta;
                    // the only loads in flight are the next tile's; a bare
                    // barrier (reads in flight touch this tile's buffer only)
                    wait_loads<0>();
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    issue(cur == 0 ? NBUF - 1 : cur - 1);
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
        // A key tile none of the wave's rows sees: only the tile's shared
        // work (the barrier that publishes the next tile, the wave's share of
        // the loads, the read offsets moved to the next buffer, the operand
        // reads of the next tile's first slots); the running maximum and sum
        // are unchanged, and the other wave on the SIMD has the matrix unit
        // to itself.
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
        // has no row).  Skipped t_lo .. tv_lo-1, masked tv_lo .. f_lo-1,
        // unmasked f_lo .. f_hi-1, masked f_hi .. tv_end-1, skipped tv_end ..
        // nkt-1 (separate loops: one masked loop entered twice makes the
        // register allocator spill).  The dQ kernel skips the same tiles of
        // the same rows, and the key-tile kernel uses a keep bit only where
        // its pair is visible, so no kernel uses a keep word this call
        // leaves unwritten.
        const int rl_w = min(r0w + 31, Lq - 1);   // the wave's last row
        int tv_lo = t_lo, tv_end = t_lo;
        if (r0w < Lq) {
            const int kv_lo = LOCAL ? max(0, r0w + off - p.win_l) : 0;
            const int kv_hi = p.win_r >= 0 ? min(Lk - 1, rl_w + off + p.win_r) : Lk - 1;
            if (kv_hi >= kv_lo) {
                tv_lo = max(t_lo, kv_lo / kFwdKeys);
                tv_end = max(tv_lo, min(nkt, kv_hi / kFwdKeys + 1));
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

    // ---- O = O^T / sum, LSE = (max + log2(sum)) * ln 2 (natural log of the
    //      scaled scores); rows without a visible key: O = 0, LSE = -inf. ----
    const float l = lsum + __shfl_xor(lsum, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // O^T accumulator of block db: column 32 db + 8 j + 4 g2 + tt of the
    // lane's row; per pair of 8-column groups the lane halves (same row)
    // trade their 8-byte pieces, so each lane stores 16 bytes.
    {
        uint16_t *orow = p.o_w + row_offset(p, b, si.tok_q, qok ? qrow : 0, p.o_sb, p.o_ss) + h * p.o_sh;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            u32x2 pc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x4 o4;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    o4[tt] = acc[db][4 * j + tt] * inv;
                pc[j] = __builtin_bit_cast(u32x2, to_elem<F16>(o4));
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // lanes 32-63 of pc[2q] <-> lanes 0-31 of pc[2q+1]
                const auto s0 = __builtin_amdgcn_permlane32_swap(pc[2 * q][0], pc[2 * q + 1][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(pc[2 * q][1], pc[2 * q + 1][1], false, false);
                const u32x4 out = {s0[0], s1[0], s0[1], s1[1]};
                const int d = 32 * db + 16 * q + 8 * g2;
                if (qok && d < p.D)
                    *reinterpret_cast<u32x4 *>(orow + d) = out;
            }
        }
    }
    if (qok) {
        if (g2 == 0)
            p.lse_w[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + qrow] =
                l > 0.f ? (mrun + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -INFINITY;
    }
}

template <int DP, bool F16, bool LOCAL, bool SOFTCAP, bool DROP>
static void launch_fwd_d(const Params &p, hipStream_t st)
{
    const int nqt = (p.Sq + FwdShape<DP>::ROWS - 1) / FwdShape<DP>::ROWS;
    hipLaunchKernelGGL((fa_fwd_kernel<DP, F16, LOCAL, SOFTCAP, DROP>),
                       dim3((unsigned)nqt * p.H * p.batch), dim3(FwdShape<DP>::THREADS), 0, st, p);
}

template <bool LOCAL, bool SOFTCAP, bool DROP>
static hipError_t launch_fwd_t(const Params &p, int dpad, hipStream_t st)
{
#define FA_FWD_CASE(D)                                                \
    case D:                                                           \
        if (p.f16)                                                    \
            launch_fwd_d<D, true, LOCAL, SOFTCAP, DROP>(p, st);       \
        else                                                          \
            launch_fwd_d<D, false, LOCAL, SOFTCAP, DROP>(p, st);      \
        break;
    switch (dpad) {
        FA_FWD_CASE(64)
        FA_FWD_CASE(96)
        FA_FWD_CASE(128)
        FA_FWD_CASE(192)
        FA_FWD_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef FA_FWD_CASE
    return hipGetLastError();
}

// The dropout instantiations build in a translation unit of their own
// (fa_fwd_dropout.hip includes this file with FA_TU_DROPOUT = 1), so that
// the two halves compile in parallel.
template <bool DROP>
hipError_t launch_fwd_v(const Params &p, int dpad, hipStream_t st)
{
    if (p.softcap > 0.f)
        return p.win_l >= 0 ? launch_fwd_t<true, true, DROP>(p, dpad, st)
                            : launch_fwd_t<false, true, DROP>(p, dpad, st);
    return p.win_l >= 0 ? launch_fwd_t<true, false, DROP>(p, dpad, st)
                        : launch_fwd_t<false, false, DROP>(p, dpad, st);
}

#if FA_TU_DROPOUT
template hipError_t launch_fwd_v<true>(const Params &, int, hipStream_t);
#else
extern template hipError_t launch_fwd_v<true>(const Params &, int, hipStream_t);

hipError_t launch_fwd(const Params &p, int dpad, hipStream_t st)
{
    return p.drop_p > 0.f ? launch_fwd_v<true>(p, dpad, st) : launch_fwd_v<false>(p, dpad, st);
}
#endif

}  // namespace fa
