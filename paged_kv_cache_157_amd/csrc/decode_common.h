// decode_common.h -- the parts shared by the two decode kernels: decode.hip
// (one KV head per work-group) and decode_hg.h (four KV heads per
// work-group, one per wave).
//
// What both compute ("Lecture 33" §2.3): for every sequence i and query head
// h, out[i,h] = softmax(scale * q[i,h] K^T) V over the sequence's tokens,
// whose K/V rows are read in place from scattered physical blocks through
// the block table (logical block t/16, offset t%16, §2.2 walk-through).  The
// pages name a streaming (online) softmax and no more; the recurrence used is
// the standard one: running maximum, running sum, rescaled accumulator,
// followed by a log-sum-exp merge of partial results.
//
// Shared here:
//   * the lane geometry of a 16-token block (DecodeCfg, row_token) and the
//     cross-lane reductions of scores, sums and accumulators;
//   * the per-lane dot product of one 16-byte K chunk with q and the
//     widening of one V piece, for every cache type;
//   * the start-up scan that cuts the flat item list (sequence, head, block
//     or partition) into per-work-group ranges;
//   * the slot range of a (sequence, head) pair's partial records and the
//     log-sum-exp merge of those records into the output;
//   * counted waits, the LDS-only barrier and the issue-priority schedule.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace dec {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Lane geometry of one 16-token block of one KV head.  K is read in 16-byte
// chunks; V in pieces of VB bytes (16, or 8 so that an fp8 V piece widens to
// as many elements as a bf16 one).
template <int CDT, int D, int G, int VB = 16>
struct DecodeCfg {
    static constexpr int EB = Storage<CDT>::bytes;
    static constexpr int E = 16 / EB;            // cache elements per 16-byte K chunk
    static constexpr int NC = D / E;             // K chunks in one token row of one head
    static constexpr int LPT = G <= 4 ? 4 : 8;   // QK lanes per token
    static constexpr int GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
    static constexpr int CPL = NC / LPT;         // K chunks per lane and token
    static constexpr int ROUNDS = LPT / 4;       // QK passes per 16-token block
    static constexpr int TRN = 4 / ROUNDS;       // tokens per row per QK pass
    static constexpr int VPB = VB;               // bytes of one V piece
    static constexpr int EV = VB / EB;           // cache elements per V piece
    static constexpr int NCV = D / EV;           // V pieces in one token row of one head
    static constexpr int VTPR = 16 / NCV;        // tokens per row per V pass
    static constexpr int VPASS = 4 / VTPR;       // V passes per block
    using VT = std::conditional_t<VB == 16, u32x4, u32x2>;
    // q dwords per (head slot, K chunk): bf16 pairs matching the chunk, or fp32
    static constexpr int QW = CDT == DT_FP8 ? 8 : 4;
    static_assert(CPL >= 1 && NC <= 16 && NC >= 4, "unsupported chunk geometry");
    static_assert(NCV <= 16 && NCV >= 4, "unsupported V geometry");
    static_assert(G >= 1 && G <= 8, "GQA group must be 1..8");
};

// Token (0..15 within the block) held in "row" r at index k (0..3).  QK lanes
// of row r handle exactly the tokens that the V lanes of row r accumulate, so
// the running maximum of a row never has to leave it.
template <int LPT>
__host__ __device__ constexpr int row_token(int r, int k)
{
    if constexpr (LPT == 4)
        return 4 * r + k;
    else
        return 2 * r + (k & 1) + 8 * (k >> 1);
}

// The tokens of a lane's later QK rounds (V passes) lie a fixed number of
// token rows after those of its first: row_token(r, k0 + d) = row_token(r, k0)
// + row_token(0, d) for every row r and first index k0 the geometry uses, so
// one lane offset plus a scalar offset per round (pass) addresses them all.
template <int LPT, int STEP, int NSTEP, int K0S>
constexpr bool rows_shift_evenly()
{
    for (int r = 0; r < 4; ++r)
        for (int k0 = 0; k0 < K0S; ++k0)
            for (int n = 0; n < NSTEP; ++n)
                if (row_token<LPT>(r, k0 + n * STEP) != row_token<LPT>(r, k0) + row_token<LPT>(0, n * STEP))
                    return false;
    return true;
}

// Reduce-scatter of GP partial sums over the LPT lanes of one token.  On
// entry slot s of a lane holds the partial sum of head (s ^ mask); on exit
// x[0] holds the complete sum of head `mask`.
template <int LPT, int GP>
__device__ __forceinline__ float reduce_scatter(float (&x)[GP])
{
    if constexpr (LPT == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            x[k] += dpp<DPP_HALF_MIRROR>(x[k + 4]);
#pragma unroll
        for (int k = 0; k < 2; ++k)
            x[k] += dpp<DPP_QP_X1>(x[k + 2]);
        x[0] += dpp<DPP_QP_X2>(x[1]);
    } else if constexpr (GP == 4) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            x[k] += dpp<DPP_QP_X1>(x[k + 2]);
        x[0] += dpp<DPP_QP_X2>(x[1]);
    } else if constexpr (GP == 2) {
        x[0] += dpp<DPP_QP_X1>(x[1]);
        x[0] += dpp<DPP_QP_X2>(x[0]);
    } else {
        x[0] += dpp<DPP_QP_X1>(x[0]);
        x[0] += dpp<DPP_QP_X2>(x[0]);
    }
    return x[0];
}

// Head handled by a lane after reduce_scatter, and whether the lane is the
// single owner of that (token, head) value (others hold copies).
template <int LPT, int GP>
__device__ __forceinline__ int head_mask(int lane)
{
    const int b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1;
    if constexpr (LPT == 8)
        return 4 * b2 + 2 * (b0 ^ b2) + (b1 ^ b2);
    else if constexpr (GP == 4)
        return 2 * b0 + b1;
    else if constexpr (GP == 2)
        return b0;
    else
        return 0;
}
template <int LPT, int GP>
__device__ __forceinline__ bool mask_owner(int lane)
{
    if constexpr (LPT == 8 || GP == 4)
        return true;
    else if constexpr (GP == 2)
        return ((lane >> 1) & 1) == 0;
    else
        return (lane & 3) == 0;
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ long long wave_sum64(long long v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += __shfl_xor(v, d);
    return v;
}

// Sum of a value over the 64 lanes that share a "column" pattern: lanes that
// differ only in the row (bits 4-5) and in the bits selected by the pattern.
// gfx950's lane swaps exchange the wave halves (rows 0-1 <-> 2-3) and
// neighbouring rows in registers: swapping a value with itself leaves
// {v(l), v(l ^ 32)} (then {v(l), v(l ^ 16)}) in the two results of every
// lane l.
__device__ __forceinline__ float sum_rows(float v)
{
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The wave's total of a per-(token, head) value held by the owner lanes of
// head `mask` (softmax sums): over rows and over the lanes of a row that hold
// other tokens.  Lanes with the same head mask end with the same total.
template <int LPT>
__device__ __forceinline__ float token_total(float v)
{
    v = sum_rows(v);
    if constexpr (LPT == 4)
        v += dpp<DPP_ROW_ROR4>(v);
    return v + dpp<DPP_ROW_ROR8>(v);
}

// The wave's total of an accumulator element: over rows and over the lanes of
// a row that accumulate other tokens of the same V piece (VTPR per row).
template <int VTPR>
__device__ __forceinline__ float piece_total(float v)
{
    v = sum_rows(v);
    if constexpr (VTPR == 2)
        v += dpp<DPP_ROW_ROR8>(v);
    if constexpr (VTPR == 4) {
        v += dpp<DPP_ROW_ROR4>(v);
        v += dpp<DPP_ROW_ROR8>(v);
    }
    return v;
}

// The wave totals of all G x EV accumulator elements of a lane at once,
// summed over rows by a reduce-scatter.  Swapping two *different* values
// across the wave halves gives every lane one half-partial of each, so one
// swap and one add fold the halves of two elements where sum_rows folds one;
// a second level does the same across neighbouring rows.  Afterwards register
// k of a lane in row r holds element j = r * (G * EV / 4) + k (j = h * EV + e)
// summed over the four rows, in the same order of additions as sum_rows; the
// lanes of a row that accumulate other tokens of the same V piece are then
// added as in piece_total.  A quarter of the lane swaps and adds of
// piece_total on every element.
template <int G, int EV, int VTPR>
__device__ __forceinline__ void fold_totals(const float (&acc)[G][EV], float (&out)[G * EV / 4])
{
    constexpr int V = G * EV, H = V / 2, Q = V / 4;
    static_assert(V % 4 == 0, "fold needs a multiple of 4 elements");
    // rows 0-1 end with element k, rows 2-3 with element k + H
    auto halves = [&](int k) -> float {
        const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[k / EV][k % EV]),
                                                        __float_as_uint(acc[(k + H) / EV][(k + H) % EV]),
                                                        false, false);
        return __uint_as_float(s[0]) + __uint_as_float(s[1]);
    };
#pragma unroll
    for (int k = 0; k < Q; ++k) {
        // row 0: element k, row 1: k + Q, row 2: k + 2Q, row 3: k + 3Q
        const float t0 = halves(k), t1 = halves(k + Q);
        const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(t0), __float_as_uint(t1), false, false);
        float x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
        if constexpr (VTPR == 2)
            x += dpp<DPP_ROW_ROR8>(x);
        if constexpr (VTPR == 4) {
            x += dpp<DPP_ROW_ROR4>(x);
            x += dpp<DPP_ROW_ROR8>(x);
        }
        out[k] = x;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave (32-bit): shifts within
// rows of 16, then the row totals carried over with row broadcasts.
__device__ __forceinline__ int wave_scan32(int x)
{
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
    return x;
}

// s_waitcnt vmcnt(N): the kernels count their own K/V loads (the global->LDS
// loads are not tracked by the compiler), so a wait names the number of loads
// issued after the one needed.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Work-group barrier for LDS data only: every wave's LDS accesses have
// completed (lgkmcnt), global loads may stay in flight.  Where a hand-over
// needs global memory complete, the code waits for it explicitly first.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Partial dot products of one 16-byte K chunk of a token with the matching q
// dwords of one head slot: bf16 pairs (v_dot2_f32_bf16), fp8 codes widened to
// bf16 pairs (exact), or fp32 values.
template <int CDT, int QW>
__device__ __forceinline__ float dot_chunk(const uint32_t (&q)[QW], u32x4 kc, float acc)
{
    if constexpr (CDT == DT_BF16) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            acc = dot2_bf16(q[p], kc[p], acc);
    } else if constexpr (CDT == DT_FP8) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            acc = dot2_bf16(q[2 * p], fp8x2_to_bf16x2<false>(kc[p]), acc);
            acc = dot2_bf16(q[2 * p + 1], fp8x2_to_bf16x2<true>(kc[p]), acc);
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            acc = fmaf(__uint_as_float(q[p]), __uint_as_float(kc[p]), acc);
    }
    return acc;
}

// One V piece (EV cache elements) widened to fp32, exactly.
template <int CDT, int EV, typename VT>
__device__ __forceinline__ void widen_v(const VT &vv, float (&ve)[EV])
{
    if constexpr (CDT == DT_BF16) {
#pragma unroll
        for (int k = 0; k < EV / 2; ++k) {
            ve[2 * k] = bf16_lo(vv[k]);
            ve[2 * k + 1] = bf16_hi(vv[k]);
        }
    } else if constexpr (CDT == DT_FP8) {
#pragma unroll
        for (int k = 0; k < EV / 4; ++k) {
            const f32x2 lo = fp8x2_to_f32x2<false>(vv[k]);
            const f32x2 hi = fp8x2_to_f32x2<true>(vv[k]);
            ve[4 * k] = lo[0];
            ve[4 * k + 1] = lo[1];
            ve[4 * k + 2] = hi[0];
            ve[4 * k + 3] = hi[1];
        }
    } else {
#pragma unroll
        for (int k = 0; k < EV; ++k)
            ve[k] = __uint_as_float(vv[k]);
    }
}

// Issue priority follows a wave's remaining work (3 at the start, 0 near the
// end): when two work-groups share a CU, the one that has fallen behind gets
// the instruction slots, instead of the older one by default, so both finish
// together.  The persistent grid fills every CU's first slots with the first
// half of the work-groups before the rest; the later ones lower their
// priority half a step later, which cancels the age tie-break at equal
// progress.  Only the order of issue changes, never the arithmetic.
struct IssuePriority {
    int ew, lag, done = 0, cur = -1;
    __device__ IssuePriority(int expected_blocks)
    {
        ew = expected_blocks > 0 ? expected_blocks : 1;
        lag = blockIdx.x >= gridDim.x / 2 ? ew / 2 : 0;
    }
    // before each block
    __device__ __forceinline__ void step()
    {
        const int pr = 3 - min(3, max(0, 4 * done - lag) / ew);
        ++done;
        if (pr != cur) {
            cur = pr;
            if (pr == 3)
                __builtin_amdgcn_s_setprio(3);
            else if (pr == 2)
                __builtin_amdgcn_s_setprio(2);
            else if (pr == 1)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
    }
};

// ---------------------------------------------------------------------------
// Start-up scan.  The flat item list of a call is, for each sequence in
// order, `pairs` runs (one per KV head, or per head group) of n items, n =
// that sequence's 16-token units (at most maxU) or fixed partitions of PB
// units.  A persistent grid of W work-groups takes contiguous ranges of it.
// With ALPHA > 0 and the balanced split (PB == 0), ranges are equal in
// "virtual" items: every run counts ALPHA extra items ahead of its real ones
// (what starting a segment costs), so a range that starts more segments
// holds fewer real items.  Wave 0 of each work-group runs the scan (no
// work-group barrier inside) and finds the sequences holding both ends of its
// range and the first real items at or after them.
// ---------------------------------------------------------------------------
struct Range {
    long long total;    // real items of the call
    long long total_v;  // virtual items (0: plain split)
    long long r0, r1;   // this work-group's real items [r0, r1)
    int seq;            // sequence holding item r0 (-1 when the range is empty)
    int len;            // its context length (0 when the range is empty)
    long long base;     // first item of that sequence
    long long vbase;    // its first virtual item
};

__device__ __forceinline__ int items_of(int L, int maxU, int PB)
{
    L = L < 0 ? 0 : L;
    int nb = (L + 15) >> 4;
    nb = nb > maxU ? maxU : nb;
    return PB > 0 ? (nb + PB - 1) / PB : nb;
}

template <int ALPHA>
__device__ __forceinline__ Range startup_scan(const int32_t *lens, int S, int pairs, int maxU, int PB, int lane)
{
    const long long W = gridDim.x;
    // 64 lanes' item counts fit 32 bits whenever (maxU + ALPHA) * pairs * 64
    // does: DPP scans then; otherwise shuffles on 64-bit values
    const bool narrow = (long long)(maxU + ALPHA) * pairs * 64 < (1ll << 31);
    auto scan = [&](long long v) -> long long {
        if (narrow)
            return wave_scan32((int)v);
        long long incl = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const long long t = __shfl_up(incl, d);
            if (lane >= d)
                incl += t;
        }
        return incl;
    };
    auto counts = [&](int l, long long &real, long long &virt) {
        const int n = items_of(l, maxU, PB);
        real = (long long)n * pairs;
        virt = (long long)(n > 0 ? n + ALPHA : 0) * pairs;
    };
    long long tot = 0, totv = 0;
    // up to 64 sequences with narrow counts: one load of the lengths and one
    // pair of prefix sums serve the totals and the search below
    const bool one_pass = narrow && S <= 64;
    int l0 = 0, ri0 = 0, vi0 = 0;
    long long rr0 = 0, vv0 = 0;
    if (one_pass) {
        l0 = lane < S ? lens[lane] : 0;
        counts(l0, rr0, vv0);
        ri0 = wave_scan32((int)rr0);
        vi0 = wave_scan32((int)vv0);
        tot = __builtin_amdgcn_readlane(ri0, 63);
        totv = __builtin_amdgcn_readlane(vi0, 63);
    } else {
        for (int base = 0; base < S; base += 64) {
            const int s2 = base + lane;
            long long r, v;
            counts(s2 < S ? lens[s2] : 0, r, v);
            if (narrow) {
                tot += __builtin_amdgcn_readlane(wave_scan32((int)r), 63);
                totv += __builtin_amdgcn_readlane(wave_scan32((int)v), 63);
            } else {
                tot += wave_sum64(r);
                totv += wave_sum64(v);
            }
        }
    }
    const bool virt = PB == 0 && ALPHA > 0 && totv >= (long long)(ALPHA + 2) * W;
    const long long T = virt ? totv : tot;
    // position x of the split -> (sequence, its real / virtual starts, first
    // real item at or after x)
    auto locate = [&](long long x, int &seq, int &len, long long &rbase, long long &vbase) -> long long {
        seq = -1;
        len = 0;
        rbase = tot;
        vbase = totv;
        if (x >= T)
            return tot;
        long long rc = 0, vc = 0;
        for (int base = 0; base < S; base += 64) {
            const int s2 = base + lane;
            const int l = s2 < S ? lens[s2] : 0;
            long long r, v;
            counts(l, r, v);
            const long long ri = scan(r), vi = scan(v);
            const long long ex = (virt ? vi - v : ri - r), in = virt ? vi : ri;
            const long long c0 = virt ? vc : rc;
            const unsigned long long m = __builtin_amdgcn_ballot_w64(r > 0 && c0 + ex <= x && x < c0 + in);
            if (m) {
                const int l2 = __builtin_ctzll(m);
                seq = base + l2;
                len = __shfl(l, l2);
                rbase = rc + __shfl(ri - r, l2);
                vbase = vc + __shfl(vi - v, l2);
                const int n = items_of(__shfl(l, l2), maxU, PB);
                if (!virt)
                    return x;
                const long long rel = x - vbase;
                const long long gq = rel / (n + ALPHA), xv = rel - gq * (n + ALPHA);
                return rbase + gq * n + (xv > ALPHA ? xv - ALPHA : 0);
            }
            rc += __shfl(ri, 63);
            vc += __shfl(vi, 63);
        }
        return tot;  // not reached while x < T
    };
    Range R;
    R.total = tot;
    R.total_v = virt ? totv : 0;
    long long rb1, vb1;
    int seq1, len1;
    if (one_pass) {
        // the prefix sums above, the found lane read with scalar lane reads;
        // 32-bit divisions wherever the operands fit (T * W < 2^31: every
        // position, count and quotient below is under T)
        const int n = items_of(l0, maxU, PB);
        const bool d32 = T * W < (1ll << 31);
        auto div = [&](long long num, long long den) -> long long {
            return d32 ? (long long)((unsigned)num / (unsigned)den) : num / den;
        };
        auto find = [&](long long x, int &seq, int &len, long long &rbase, long long &vbase) -> long long {
            seq = -1;
            len = 0;
            rbase = tot;
            vbase = totv;
            if (x >= T)
                return tot;
            const long long in = virt ? vi0 : ri0, ex = in - (virt ? vv0 : rr0);
            const unsigned long long m = __builtin_amdgcn_ballot_w64(rr0 > 0 && ex <= x && x < in);
            const int l2 = __builtin_ctzll(m);  // m != 0 while x < T
            seq = l2;
            len = __builtin_amdgcn_readlane(l0, l2);
            rbase = __builtin_amdgcn_readlane(ri0, l2) - __builtin_amdgcn_readlane((int)rr0, l2);
            vbase = __builtin_amdgcn_readlane(vi0, l2) - __builtin_amdgcn_readlane((int)vv0, l2);
            if (!virt)
                return x;
            const int nn = __builtin_amdgcn_readlane(n, l2);
            const long long rel = x - vbase;
            const long long gq = div(rel, nn + ALPHA), xv = rel - gq * (nn + ALPHA);
            return rbase + gq * nn + (xv > ALPHA ? xv - ALPHA : 0);
        };
        R.r0 = find(div(T * blockIdx.x, W), R.seq, R.len, R.base, R.vbase);
        R.r1 = find(div(T * (blockIdx.x + 1), W), seq1, len1, rb1, vb1);
    } else {
        R.r0 = locate(T * blockIdx.x / W, R.seq, R.len, R.base, R.vbase);
        R.r1 = locate(T * (blockIdx.x + 1) / W, seq1, len1, rb1, vb1);
    }
    return R;
}

// Partial records of the balanced split: the work-group of rank k (its index
// among the work-groups with a non-empty range) writes the records of pair p
// (sequence, KV head or head group) to slot k + p, so the slots of one pair
// are contiguous and the merge order is fixed.  With at least as many items
// as work-groups every range is non-empty (rank = index); with fewer, each
// non-empty range holds one item (rank = its first item).
__device__ __forceinline__ int partial_slot(long long a0, int pair)
{
    return (int)(a0 < (long long)blockIdx.x ? a0 : (long long)blockIdx.x) + pair;
}

// Slots [lo, hi] holding the partial records of a pair whose real items are
// [first_item, first_item + n) of the balanced split.
__device__ __forceinline__ void partial_slot_range(long long first_item, int n, const Range &R, long long first_v,
                                                   int pair, int &lo, int &hi)
{
    const long long W = gridDim.x;
    if (R.total_v > 0) {
        // work-groups whose (virtual) ranges hold the pair's real items; every
        // range holds at least one real item, so rank = index
        const long long last_v = first_v + n - 1;
        lo = (int)(((first_v + 1) * W - 1) / R.total_v) + pair;
        hi = (int)(((last_v + 1) * W - 1) / R.total_v) + pair;
    } else {
        const long long last_item = first_item + n - 1;
        const long long k_first = ((first_item + 1) * W - 1) / R.total;
        const long long k_last = ((last_item + 1) * W - 1) / R.total;
        const long long r_first = k_first < k_first * R.total / W ? k_first : k_first * R.total / W;
        const long long r_last = k_last < k_last * R.total / W ? k_last : k_last * R.total / W;
        lo = (int)r_first + pair;
        hi = (int)r_last + pair;
    }
}

// Word 3 of a raw buffer descriptor (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache policy of a device-coherent (L2-bypassing) buffer load: sc1.
constexpr int kBufferCoherent = 16;

// LDS scratch of a merge: per query head the running maximum and denominator,
// and the scale factors of one batch of partial records (and of the running
// sums).
template <int HEADS, int MBMAX>
struct MergeLds {
    float mden[HEADS], mfo[HEADS], mf[MBMAX][HEADS];
};

// Log-sum-exp merge of the np partial records [lo, lo + np) of one pair into
// its output row (HEADS query heads x D): record s holds, for each head h, the
// running maximum and sum (ml[(s * HEADS + h) * 2 + 0/1], base 2) and the
// unnormalised accumulator (acc[(s * HEADS + h) * D + c]; with FOLD_NCV > 0
// the D values of a head are in the folded order of fold_totals: position
// (d % EV) * FOLD_NCV + d / EV holds column d, EV = D / FOLD_NCV).  Records are read
// in batches of MB: every thread issues the accumulator loads of its columns
// (4 consecutive d each), the threads that own a head load the (max, sum)
// pairs and publish the batch's scale factors through LDS, then all combine:
// one memory round trip per batch.  MB = 8 where no other registers are live,
// fewer where prefetched blocks occupy them.  Records are read with
// device-coherent loads (their writers stored them the same way).  Called by
// every thread of the work-group (it holds work-group barriers); no thread may
// still be reading `m` from an earlier call (a barrier between two calls).
template <int HEADS, int D, int NT, int MB, int FOLD_NCV, int MBMAX>
__device__ __forceinline__ void merge_partials(const float *ws_ml, const float *ws_acc, int lo, int np,
                                               float *out_row, float v_scale, int tid,
                                               MergeLds<HEADS, MBMAX> &m)
{
    static_assert(MB <= MBMAX, "merge batch larger than its LDS scratch");
    constexpr int KC = (HEADS * D + 4 * NT - 1) / (4 * NT);  // 4-column chunks per thread
    // the np records of this pair; loads past them read zero
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void *)(ws_acc + (int64_t)lo * HEADS * D), (short)0,
                                                      np * HEADS * D * 4, kBufferRsrcWord3);
    float num[KC][4];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            num[kc][j] = 0.f;
    // the running maximum and sum of head `tid` stay in its thread's registers
    float hM = -INFINITY, hden = 0.f;
    for (int s0 = 0; s0 < np; s0 += MB) {
        const bool final_batch = s0 + MB >= np;
        u32x4 ac[MB][KC];
#pragma unroll
        for (int k2 = 0; k2 < MB; ++k2)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int e = 4 * tid + kc * 4 * NT;
                ac[k2][kc] = e < HEADS * D ? __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, ((s0 + k2) * HEADS * D + e) * 4, 0, kBufferCoherent)
                                           : u32x4{0u, 0u, 0u, 0u};
            }
        if (tid < HEADS) {
            f32x2 ml[MB];
#pragma unroll
            for (int k2 = 0; k2 < MB; ++k2)
                ml[k2] = s0 + k2 < np ? coherent_load2(&ws_ml[((int64_t)(lo + s0 + k2) * HEADS + tid) * 2])
                                      : f32x2{-INFINITY, 0.f};
            const float M = hM;
            float Mb = M;
#pragma unroll
            for (int k2 = 0; k2 < MB; ++k2)
                Mb = fmaxf(Mb, ml[k2][0]);
            const float fo = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
            float den = hden * fo;
#pragma unroll
            for (int k2 = 0; k2 < MB; ++k2) {
                const float f = ml[k2][0] == -INFINITY ? 0.f : fast_exp2(ml[k2][0] - Mb);
                den += f * ml[k2][1];
                m.mf[k2][tid] = f;
            }
            m.mfo[tid] = fo;
            hM = Mb;
            hden = den;
            if (final_batch)
                m.mden[tid] = den;
        }
        __syncthreads();
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const int e = 4 * tid + kc * 4 * NT;
            if (e < HEADS * D) {
                const int h = e / D;
                const float fo = m.mfo[h];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    num[kc][j] *= fo;
#pragma unroll
                for (int k2 = 0; k2 < MB; ++k2) {
                    const float f = m.mf[k2][h];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        num[kc][j] = fmaf(f, __uint_as_float(ac[k2][kc][j]), num[kc][j]);
                }
            }
        }
        if (!final_batch)
            __syncthreads();  // the scale factors of the next batch go to the same place
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int e = 4 * tid + kc * 4 * NT;
        if (e < HEADS * D) {
            const int h = e / D;
            const float inv = v_scale / m.mden[h];
            if constexpr (FOLD_NCV > 0) {
                // folded records: position q = e' * NCV + p of a head holds d = p * EV + e'
                constexpr int FEV = D / FOLD_NCV;
                const int q = e - h * D, e1 = q / FOLD_NCV, p = q - e1 * FOLD_NCV;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    out_row[h * D + (p + j) * FEV + e1] = num[kc][j] * inv;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    out_row[e + j] = num[kc][j] * inv;
            }
        }
    }
}

// Sequences with no tokens get a zero output row (work-group 0 of the grid).
template <int D, int NT>
__device__ __forceinline__ void zero_empty_rows(const int32_t *lens, float *out, int S, int Hq, int tid)
{
    if (blockIdx.x == 0) {
        for (int i = tid; i < S; i += NT)
            if (lens[i] <= 0)
                for (int e = 0; e < Hq * D; ++e)
                    out[(int64_t)i * Hq * D + e] = 0.f;
    }
}

}  // namespace dec
}  // namespace pa
