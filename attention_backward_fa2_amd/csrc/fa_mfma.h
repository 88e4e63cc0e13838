// fa_mfma.h -- gfx950 MFMA and LDS operand helpers shared by the two
// tile kernels of the attention backward.
//
// MFMA: v_mfma_f32_32x32x16_bf16 / _f16 (same lane layouts).  Per lane l
// (l32 = l % 32, g2 = l / 32):
//   A (32 x 16, M x K): row l32, k = 8*g2 + t (t = 0..7, one 16-byte vector)
//   B (16 x 32, K x N): col l32, k = 8*g2 + t
//   C (32 x 32):        col l32, row 8*(r/4) + 4*g2 + r%4 for r = 0..15
// A and B have the same lane layout, so an accumulator that holds one
// column and 16 rows per lane is directly an A or B operand of a product
// that contracts over those rows, provided the other operand lists the
// contraction index in the same (permuted) order:
//   k-slot 8*g2 + t  <->  row 4*g2 + t (t < 4) or 8 + 4*g2 + t - 4
// within each group of 16 rows (rows 16h .. 16h + 15 are accumulator
// elements 8h .. 8h + 7 of the lane).
//
// Operands whose contraction index runs down the rows of a row-major LDS
// tile are read with ds_read_b64_tr_b16: within each 16-lane group the 16
// 8-byte reads form a 4 x 16 block (lanes 4r .. 4r+3 read row r) and lane c
// receives column c.  Two such reads give one 8-element operand; the row
// base of each read implements the permutation above.  ds_read_b128 is used
// wherever the operand is contiguous in LDS (one instruction instead of two).
#pragma once

#include <type_traits>
#include <utility>

#include "fa_internal.h"

namespace fa {

// Operand containers: eight / four 16-bit elements, bf16 or fp16 bit
// patterns (the MFMA wrappers and converts below take the element type as a
// template flag).
typedef __bf16 e16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 e16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

template <bool F16>
__device__ inline f32x16 mfma32(e16x8 a, e16x8 b, f32x16 c)
{
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product as inline assembly: accumulator in ordinary registers,
// B operand in accumulation registers (A in ordinary ones).  The compiler
// gives every MFMA of a kernel one register form; a kernel whose long-lived
// accumulators must live in accumulation registers would otherwise get its
// short-lived products there as well, and each element would need a copy
// before the vector math can read it.  These are not MFMAs to the compiler,
// so the caller covers the hazards it would otherwise cover (gfx950,
// 32x32x16: a vector read of the result needs 12 wait states after the last
// product -- mfma_settle(); an accumulation chain needs none; no operand may
// come from a vector instruction of the two preceding wait states -- the
// callers feed A straight from LDS reads, and an accumulator just written by
// vector instructions (a copied initial value) goes through mfma32_vacc
// with FRESH, which waits those two states first).
template <bool F16>
__device__ inline void mfma32_vz(f32x16 &d, e16x8 a, e16x8 b)   // d = A B
{
    if constexpr (F16)
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}

template <bool F16, bool FRESH = false>
__device__ inline void mfma32_vacc(f32x16 &d, e16x8 a, e16x8 b)   // d += A B
{
    if constexpr (F16 && FRESH)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
    else if constexpr (F16)
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
    else if constexpr (FRESH)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// d = A B + c into ordinary registers, c from other registers (the initial
// value several products share); the two wait states cover a c just
// written by vector instructions.
template <bool F16>
__device__ inline void mfma32_vc(f32x16 &d, e16x8 a, e16x8 b, const f32x16 &c)
{
    if constexpr (F16)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %3"
                     : "=&v"(d) : "v"(a), "a"(b), "v"(c));
    else
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
                     : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}

// 12 wait states, ordered after the last product into s and t and before
// any read of them.
__device__ inline void mfma_settle(f32x16 &s, f32x16 &t)
{
    asm volatile("s_nop 11" : "+v"(s), "+v"(t));
}

// The same for one product (passing one value twice to mfma_settle would make
// the compiler copy it first).
__device__ inline void mfma_settle(f32x16 &s)
{
    asm volatile("s_nop 11" : "+v"(s));
}

// Keeps the computation of x at this point of the instruction stream.  The
// compiler's basic-block scheduler places pure arithmetic next to its first
// use, across the scheduling fences that separate the MFMA slots; an empty
// volatile statement that takes x as an operand ties it to the slot.
__device__ inline void keep_here(float &x)
{
    asm volatile("" : "+v"(x));
}

// The same for an MFMA result (ordinary / accumulation registers): keeps the
// product in its slot.
__device__ inline void keep_here(f32x16 &x)
{
    asm volatile("" : "+v"(x));
}

__device__ inline void keep_here_acc(f32x16 &x)
{
    asm volatile("" : "+a"(x));
}

// The same for wave-uniform values in scalar registers: placed before a
// computation, it keeps the computation from being hoisted above this point;
// placed after, from being sunk below it.
template <class T>
__device__ inline void keep_scalar_one(T &x)
{
    asm volatile("" : "+s"(x));
}

template <class... T>
__device__ inline void keep_scalar_here(T &...x)
{
    (keep_scalar_one(x), ...);
}

// tanh(s * scale / c) of a raw score product s, with cap_in = 2 scale
// log2(e) / c: 1 - 2 / (exp2(s * cap_in) + 1) (the exp2 overflows to +inf for
// large scores, giving 1, and underflows to 0 for very negative ones, giving
// -1).  Two transcendental and two ordinary VALU operations.
__device__ inline float cap_tanh(float s, float cap_in)
{
    const float e = __builtin_amdgcn_exp2f(s * cap_in);
    return fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f);
}

// The lane index, formed where this is called: a volatile statement is
// neither hoisted out of a loop nor merged with another, so values derived
// from it take no register across the loop.
__device__ inline int lane_here()
{
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// fp32 -> element (round to nearest even) of four values: two packed
// hardware converts.
template <bool F16>
__device__ inline e16x4 to_elem(f32x4 x)
{
    if constexpr (F16)
        return __builtin_bit_cast(e16x4, __builtin_convertvector(x, f16x4));
    else
        return __builtin_convertvector(x, e16x4);
}

__device__ inline e16x8 concat(e16x4 lo, e16x4 hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline void zero(f32x16 &c)
{
#pragma unroll
    for (int r = 0; r < 16; ++r)
        c[r] = 0.f;
}

__device__ inline e16x8 lds16(const uint16_t *p)
{
    return *reinterpret_cast<const e16x8 *>(p);
}

__device__ inline i16x4 lds_tr(const uint16_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)((lds_u16 *)p));
}

// MFMA operand from a row-major LDS matrix whose rows run along the
// contraction index: the lane receives column c0 + l32 at rows r0 .. r0+3
// (elements 0..3) and r1 .. r1+3 (elements 4..7).  r0 and r1 may depend on
// g2 only.
__device__ inline e16x8 frag_tr(const uint16_t *base, int pitch, int r0, int r1, int c0,
                                 int lane)
{
    const int c16 = lane & 15;
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (c16 & 3);
    const int rr = c16 >> 2;
    const i16x4 lo = lds_tr(base + (r0 + rr) * pitch + col);
    const i16x4 hi = lds_tr(base + (r1 + rr) * pitch + col);
    const i16x4 v8[2] = {lo, hi};
    return __builtin_bit_cast(e16x8, v8);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

// ---- Buffer loads straight into LDS ----
// A raw buffer resource covers `bytes` bytes from `base`; loads at offsets at
// or past that bound return zeros without touching memory, which is how tile
// rows past the end of a sequence and columns past head_dim are zero-filled.
// Each wave load of W bytes per lane writes 64 * W contiguous bytes of LDS
// (lane l at lds + l * W), so a tile's LDS layout is chosen through the
// global offset each lane loads from.
//
// The loads are written as inline assembly: the compiler then does not
// track them, and does not make LDS reads that it cannot prove disjoint from
// them (the transposing reads) wait for them.  Their completion is awaited
// explicitly with wait_loads() before the workgroup barrier that publishes
// the buffer; compiler-issued memory waits only become stricter through
// them.
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4_rsrc __attribute__((ext_vector_type(4)));
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, 32-bit elements
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline u32x4_rsrc make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4_rsrc r;
    r[0] = (uint32_t)a;
    r[1] = (uint32_t)(a >> 32) & 0xffffu;    // stride 0, no swizzle
    r[2] = bytes;
    r[3] = kRsrcWord3;
    return r;
}

__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void *)p);
}

// The descriptor operand may have just been written by a vector instruction
// (the compiler restores spilled scalar registers with v_readlane), and a
// buffer instruction must not read such a register within five wait states;
// the compiler covers that hazard for its own loads but cannot see into these
// statements, so each waits the five states itself.
__device__ inline void load16_to_lds(u32x4_rsrc r, void *lds, uint32_t voffset)
{
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(r),
                 "{m0}"(lds_addr(lds))
                 : "memory");
}

__device__ inline void load4_to_lds(u32x4_rsrc r, void *lds, uint32_t voffset)
{
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voffset), "s"(r),
                 "{m0}"(lds_addr(lds))
                 : "memory");
}

// Wait until at most N of the memory loads this wave issued (including loads
// into LDS) are still in flight; they complete in issue order.
template <int N = 0>
__device__ inline void wait_loads()
{
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);   // vmcnt(N); expcnt, lgkmcnt unchanged
}

// ---- Swizzled row-major tiles in LDS ----
// Rows of 16-byte chunks with no padding; chunk c of row r is stored at
// chunk position c ^ swz<PCH>(r) (PCH = chunks per row, 8, 16 or 32).  The LDS
// serves 256 bytes (64 banks) per clock: a 16-byte read by 16 lanes or an
// 8-byte read by 32 lanes.  The swizzle makes both conflict-free for the
// operand reads of the tile kernels:
//  - 16 consecutive rows read at one chunk (row-major operand reads): swz
//    is a bijection on r % 16 (PCH = 16) or, for the 8 rows of one parity
//    that share a 256-byte bank line, on r / 2 % 8 (PCH = 8);
//  - transposing reads, 4 consecutive rows (aligned) x 4 consecutive
//    chunks (aligned) per 32 lanes: swz differs in bits 2-3 between rows
//    of one bank line, so the 16 chunks land in distinct bank groups.
template <int PCH>
__device__ __host__ constexpr int swz(int r)
{
    // PCH = 32 (512-byte rows, two bank lines each): the PCH = 16 swizzle
    // within each half of the row keeps both read patterns conflict-free
    return PCH >= 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

__device__ inline e16x8 lds16b(const uint8_t *p)
{
    return *reinterpret_cast<const e16x8 *>(p);
}

// Transposing operand read from two byte addresses (see frag_tr).
__device__ inline e16x8 tr_pair(const uint8_t *p0, const uint8_t *p1)
{
    const i16x4 v8[2] = {lds_tr(reinterpret_cast<const uint16_t *>(p0)),
                         lds_tr(reinterpret_cast<const uint16_t *>(p1))};
    return __builtin_bit_cast(e16x8, v8);
}

template <int MASK, int N>
__device__ inline void sched()
{
    __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}

// Asks the scheduler to issue AHEAD LDS reads first and then alternate one
// MFMA with PER reads, so each MFMA's operands were requested several MFMAs
// earlier (one wave per SIMD: the wave itself must hide LDS latency).
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

template <int V>
using IC = std::integral_constant<int, V>;

template <typename F, int... I>
__device__ inline void static_for_impl(F &f, std::integer_sequence<int, I...>)
{
    (f(IC<I>{}), ...);
}

// f(IC<0>), f(IC<1>), ..., f(IC<N-1>), fully unrolled.
template <int N, typename F>
__device__ inline void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Geometry of a 64-row tile of head-dim DP in the swizzled LDS layout
// (64 query rows in the key-tile kernel, 64 keys in the query-tile kernel).
template <int DP>
struct Tile64 {
    static constexpr int PCH = DP <= 64 ? 8 : (DP <= 128 ? 16 : 32);   // 16-byte chunks per row
    static constexpr int PB = 16 * PCH;             // row pitch (bytes)
    static constexpr int BYTES = 64 * PB;
    static constexpr int NLOAD = BYTES / 1024;      // 1 KB wave loads per tile
    static constexpr int PERW = NLOAD / 4;          // ... per wave
    static constexpr int RPL = 1024 / PB;           // rows per wave load
};

// ---- Workgroup order across the XCDs ----
// The dispatcher hands consecutive workgroups to the eight XCDs in turn, and
// each XCD has its own L2.  A grid of nbg (batch, KV head) groups times
// n_inner work items per group (key tiles, or query tiles x heads, heaviest
// first) is ordered so that a group stays on one XCD (when nbg is a
// multiple of 8) and the XCD runs the items of a few groups side by side,
// which then read the same K/V or Q/dO tiles: each XCD takes its groups gs
// at a time (gs * n_inner about 64 workgroups, two rounds of its 32 CUs),
// items of the gs groups interleaved, heaviest first.  With two groups per
// XCD and 32 items (the B=2, Hk=8, 4096-key case) this is the plain order
// "item-major, group fastest".  lin -> (item u, group bg).
constexpr int kXcds = 8;
__device__ inline void xcd_group_order(int lin, int nbg, int n_inner, int &u, int &bg)
{
    if (nbg % kXcds != 0) {
        u = lin / nbg;
        bg = lin % nbg;
        return;
    }
    const int nb = nbg / kXcds;                 // groups per XCD
    int gs = n_inner >= 64 ? 1 : 64 / n_inner;  // groups side by side
    gs = gs < nb ? gs : nb;
    while (nb % gs != 0)
        --gs;
    const int x = lin % kXcds, s = lin / kXcds;
    const int span = gs * n_inner;
    const int r = s % span;
    u = r / gs;
    bg = x + kXcds * ((s / span) * gs + r % gs);
}

}  // namespace fa
