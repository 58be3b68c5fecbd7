// decode_hg.h -- decode attention by KV-head groups: the variant used when a
// model has at least two groups of four KV heads and G >= 2 (decode_hg4.hip
// instantiates it; decode.hip holds the other kernel and the choice).
//
// What is computed ("Lecture 33" §2.3): for every sequence i and query head
// h, out[i,h] = softmax(scale * q[i,h] K^T) V over the sequence's tokens,
// whose K/V rows are read in place from scattered physical blocks through
// the block table (logical block t/16, offset t%16, §2.2 walk-through).  The
// pages name a streaming (online) softmax and no more; the recurrence used
// here is the standard one: running maximum, running sum, rescaled
// accumulator, followed by a log-sum-exp merge of partial results.
//
// Work decomposition (MI355X: 256 CUs in 8 XCDs, wave64):
//   * KV heads are taken HPG (four) at a time: a "head group".  The flat
//     list of "items" is (sequence, head group, x) where x is a 16-token
//     block (balanced mode) or a fixed partition of blocks.  A persistent grid of work-groups takes
//     equal contiguous ranges of the list, so a 32k-token sequence is spread
//     over many CUs as evenly as a batch of short ones.  A run of items of one
//     (sequence, head group) inside a range is a "segment".
//   * A work-group has HPG waves, one per KV head of the group, and every
//     wave walks the same blocks: the group's heads of a token row are
//     adjacent in the cache, so the work-group reads each 16-token block as
//     one stretch, and no wave ever waits for another inside a range.  A wave
//     handles all G query heads of its KV head, so each K/V row fetched from
//     HBM is used G times from registers.
//   * A segment that covers its whole sequence writes the output directly;
//     otherwise each wave writes a partial (max, sum, unnormalised
//     accumulator) of its head; the work-group that delivers the last partial
//     of a (sequence, head group) merges them (arrival counter), so a call is
//     a single kernel launch.
//   * QK^T: a token's K row (one KV head) is read by 4 or 8 lanes with
//     16-byte loads (64 or 128 contiguous bytes per token per load).  Each
//     lane forms partial dot products for G (padded to GP) query heads with
//     v_dot2_f32_bf16, then a DPP reduce-scatter leaves lane "m" with the full
//     score of head m: log2(GP) exchange steps instead of a butterfly per head.
//   * Softmax: scores are kept in base 2.  The running maximum is shared by
//     the whole wave and is only raised when a block's maximum exceeds it by
//     more than 8 (a rare, wave-uniform branch), so steady-state blocks do one
//     exp2 per lane and no rescaling.
//   * PV: probabilities go through a 512-byte LDS buffer to the lanes holding
//     V; each lane owns one 8-element piece of V for four tokens of the block
//     and accumulates G fp32 heads with FMA.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace hg {

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

template <int CDT, int D, int G>
struct DecodeCfg {
    static constexpr int EB = Storage<CDT>::bytes;
    static constexpr int E = 16 / EB;            // cache elements per 16-byte chunk
    static constexpr int NC = D / E;             // chunks in one token row of one head
    static constexpr int LPT = G <= 4 ? 4 : 8;   // QK lanes per token
    static constexpr int GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
    static constexpr int CPL = NC / LPT;         // K chunks per lane and token
    static constexpr int ROUNDS = LPT / 4;       // QK passes per 16-token block
    static constexpr int TRN = 4 / ROUNDS;       // tokens per row per QK pass
    // V is read in pieces of VB bytes (8 for fp8, so that a lane accumulates 8
    // elements per head, as for bf16)
    static constexpr int VB = CDT == DT_FP8 ? 8 : 16;
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

// Partial results whose hand-over (arrival count, and the merge by the last
// contributor) is still pending in a work-group.  Balanced split: at most two
// (the first and the last segment of a range); fixed partitions: flushed when
// full.
constexpr int kDecodeDeferred = 4;

template <int CDT, int D, int G, int HPG>
struct DecodeSmem {
    // bytes of the q rows of one (sequence, KV head): G heads x D (fp32 q with
    // an fp32 cache, else bf16), in 1 KiB pieces (one 16-byte load per lane)
    static constexpr int QB = G * D * (CDT == DT_F32 ? 4 : 2);
    static constexpr int QV = (QB + 1023) / 1024;
    __attribute__((aligned(16))) uint8_t qbuf[HPG][QV * 1024];  // q of each wave's head
    float p[HPG][16][8];       // probabilities of the current block
    float bmax[HPG][4][8];     // row maxima (rescale path)
    float lsum[HPG][8];        // a wave's softmax sums at a segment end
    float mref[HPG][8];        // a wave's running (reference) maximum per head
    long long total;  // item count of the call (start-up scan)
    int seg_i, seg_L;
    long long seg_base;
    // pending hand-overs: first slot, slot count, counter index, output row
    int def_lo[kDecodeDeferred], def_np[kDecodeDeferred], def_pair[kDecodeDeferred];
    long long def_out[kDecodeDeferred];
    int def_last[kDecodeDeferred];
    // merge of one (sequence, head group): per query head of the group, the
    // running maximum and denominator, and the scale factors of a batch of 8
    // partials (and of the running sums)
    float mM[32], mden[32], mfo[32], mf[8][32];
};

// Word 3 of a raw buffer descriptor (32-bit data format, no swizzle).
constexpr int kBufferRsrcWord3 = 0x00020000;
// Cache policy of a device-coherent (L2-bypassing) buffer load: sc1.
constexpr int kBufferCoherent = 16;

// s_waitcnt vmcnt(N)
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int CDT, int D, int G, int HPG>
__global__ __launch_bounds__(64 * HPG, 2) void decode_hg_kernel(DecodeArgs a)
{
    using C = DecodeCfg<CDT, D, G>;
    using SM = DecodeSmem<CDT, D, G, HPG>;
    constexpr int WAVES = HPG;
    constexpr int NT = 64 * WAVES;
    constexpr int LPT = C::LPT, GP = C::GP, CPL = C::CPL, ROUNDS = C::ROUNDS;
    constexpr int E = C::E, EV = C::EV, NCV = C::NCV, VTPR = C::VTPR, VPASS = C::VPASS, QW = C::QW;
    using VT = typename C::VT;
    constexpr float TAU = 8.0f;
    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);  // the wave's head inside the group
    const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_q_heads, maxB = a.max_blocks;
    const int NHG = Hkv / HPG;  // head groups
    const int PB = a.part_blocks;
    // the kernel walks 16-token units; a table entry names 2^ts consecutive ones
    const int ts = a.tbs_log2;
    const int maxU = maxB << ts;  // units a table row addresses
    auto unit_block = [&](auto tab, int u) -> int {
        return (tab[u >> ts] << ts) + (u & ((1 << ts) - 1));
    };

    auto items_of = [&](int L) -> int {
        L = L < 0 ? 0 : L;
        int nb = (L + 15) >> 4;
        nb = nb > maxU ? maxU : nb;
        return PB > 0 ? (nb + PB - 1) / PB : nb;
    };

    // ---- total item count and the sequence holding this work-group's first
    // item: wave 0 scans the lengths 64 at a time with shuffles (no work-group
    // barrier inside); the other waves wait at the barrier below.
    if (w == 0) {
        const int l0 = lane < S ? a.context_lens[lane] : 0;
        const long long v0 = items_of(l0);
        long long cnt = wave_sum64(v0);
        for (int base = 64; base < S; base += 64) {
            const int s2 = base + lane;
            cnt += wave_sum64(s2 < S ? (long long)items_of(a.context_lens[s2]) : 0);
        }
        const long long tot = cnt * NHG;
        const long long x0 = tot * blockIdx.x / gridDim.x;
        int found = -1, fL = 0;
        long long fbase = 0, carry = 0;
        for (int base = 0; base < S; base += 64) {
            const int s2 = base + lane;
            const int l = base == 0 ? l0 : s2 < S ? a.context_lens[s2] : 0;
            const long long v = (long long)items_of(l) * NHG;
            long long incl = v;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const long long t = __shfl_up(incl, d);
                if (lane >= d)
                    incl += t;
            }
            const long long excl = incl - v;
            const unsigned long long m =
                __builtin_amdgcn_ballot_w64(v > 0 && carry + excl <= x0 && x0 < carry + incl);
            if (m) {
                const int l2 = __builtin_ctzll(m);
                found = base + l2;
                fbase = carry + __shfl(excl, l2);
                fL = __shfl(l, l2);
                break;
            }
            carry += __shfl(incl, 63);
        }
        if (lane == 0) {
            sm.total = tot;
            sm.seg_i = found;
            sm.seg_L = fL;
            sm.seg_base = fbase;
        }
    }
    __syncthreads();
    const long long total = uniform64(sm.total);
    if (blockIdx.x == 0) {  // sequences with no tokens get a zero output row
        for (int i = tid; i < S; i += NT)
            if (a.context_lens[i] <= 0)
                for (int e = 0; e < Hq * D; ++e)
                    a.out[(int64_t)i * Hq * D + e] = 0.f;
    }
    const long long a0 = total * blockIdx.x / gridDim.x;
    const long long a1 = total * (blockIdx.x + 1) / gridDim.x;
    if (a0 >= a1)
        return;
    int i = uniform(sm.seg_i);
    if (i < 0)  // unreachable while a0 < total; keeps every index in range
        return;
    long long base_i = uniform64(sm.seg_base);  // first item index of sequence i
    long long item = a0;
    const int lane_m = head_mask<LPT, GP>(lane);
    const bool lane_owner = mask_owner<LPT, GP>(lane) && lane_m < G;
    const int row = lane >> 4;

    // QK lane geometry
    const int gl = lane & (LPT - 1);
    const int tr = LPT == 8 ? (lane >> 3) & 1 : (lane >> 2) & 3;
    // V lane geometry
    const int vc = (lane & 15) % NCV;
    const int vh = (lane & 15) / NCV;

    const int64_t tok_bytes = (int64_t)Hkv * D * C::EB;
    const int64_t blk_bytes = 16 * tok_bytes;
    const unsigned nblocks_pool = (unsigned)a.num_blocks;

    // per-lane byte offsets, inside one block (KV head 0), of the first K
    // chunk this lane scores and of the first V piece it accumulates; round j
    // (pass v) adds a whole number of token rows (a scalar offset), chunk c
    // adds c * LPT * 16 bytes (an immediate)
    static_assert(rows_shift_evenly<LPT, C::TRN, ROUNDS, C::TRN>(), "K rounds");
    static_assert(rows_shift_evenly<LPT, VTPR, VPASS, VTPR>(), "V passes");
    const int koff = (int)(row_token<LPT>(row, tr) * tok_bytes) + gl * 16;
    const int voff = (int)(row_token<LPT>(row, vh) * tok_bytes) + vc * C::VB;

    const auto lens_s = scalar_view(a.context_lens);
    constexpr int QEB = CDT == DT_F32 ? 4 : 2;  // bytes per q element
    static_assert(GP * D * QEB <= SM::QV * 1024, "padded q slots stay inside the q buffer");
    // q chunk (slot s, chunk c) of this lane starts at byte
    // (qlane ^ (s * D * QEB)) + c * LPT * E * QEB: D * QEB is a power of two
    // above every chunk offset, so the XOR only changes the head
    const unsigned qlane = (unsigned)(lane_m * D * QEB + gl * E * QEB);

    // A segment: the items of one (sequence, head group) inside [item, a1).
    // Every value is wave-uniform.  Sequences without items are skipped
    // (advances si).
    struct Seg {
        int L, n_i, hg, x, seg_items, b0, b1, slot;
    };
    auto describe = [&](long long it, int &si, long long sbase, int L) -> Seg {
        Seg d;
        int n = items_of(L);
        while (n == 0) {  // cannot happen for the first segment; skip empties
            ++si;
            L = lens_s[si];
            n = items_of(L);
        }
        d.L = uniform(L > maxU * 16 ? maxU * 16 : L);
        d.n_i = uniform(n);
        const long long rel = it - sbase;
        d.hg = uniform((int)(rel / d.n_i));
        d.x = uniform((int)(rel - (long long)d.hg * d.n_i));
        const int nblk = (d.L + 15) >> 4;
        if (PB > 0) {
            d.seg_items = 1;
            d.b0 = d.x * PB;
            d.b1 = d.b0 + PB < nblk ? d.b0 + PB : nblk;
            d.slot = (int)it;
        } else {
            const long long left = a1 - it;
            d.seg_items = (int)((long long)(d.n_i - d.x) < left ? (d.n_i - d.x) : left);
            d.b0 = d.x;
            d.b1 = d.x + d.seg_items;
            // rank of this work-group among those with a non-empty range: with at
            // least as many items as work-groups every range is non-empty (rank =
            // blockIdx.x); with fewer, each non-empty range holds one item (rank =
            // a0).  Ranks keep the partial slots of one (sequence, head group)
            // contiguous.
            d.slot = (int)(a0 < (long long)blockIdx.x ? a0 : (long long)blockIdx.x) + si * NHG + d.hg;
        }
        d.b0 = uniform(d.b0);
        d.b1 = uniform(d.b1);
        return d;
    };

    // q rows of (sequence si, KV head gg): G*D*QEB contiguous bytes, loaded
    // into registers (QV 16-byte pieces per lane, zeros past the rows) and
    // stored to the wave's LDS q buffer.  For a following segment this happens
    // after the block loop: the wait then overlaps the wait for that
    // segment's first blocks (issued just before), and no registers stay
    // reserved for q during the loop.
    u32x4 qn[SM::QV];
    auto load_q = [&](int si, int gg) {
        const char *src = (const char *)a.q + ((int64_t)si * Hq + gg * G) * D * QEB;
#pragma unroll
        for (int k = 0; k < SM::QV; ++k) {
            const int off = (k * 64 + lane) * 16;
            qn[k] = off < SM::QB ? *(const u32x4 *)(src + off) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto store_q = [&]() {
#pragma unroll
        for (int k = 0; k < SM::QV; ++k)
            *(u32x4 *)&sm.qbuf[w][(k * 64 + lane) * 16] = qn[k];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };

    // K and V of one block of this wave's KV head, straight into registers:
    // two slots alternate, so the loads of block t + 2 are in flight while
    // block t + 1 is waited for
    u32x4 kr0[ROUNDS][CPL], kr1[ROUNDS][CPL];
    VT vr0[VPASS], vr1[VPASS];
    // Loads go through a buffer descriptor spanning one block (scalar base,
    // 32-bit lane offsets): no 64-bit per-lane addresses, and any offset past
    // the block reads zero.
    auto block_rsrc = [&](const char *base, int pb) {
        pb = (unsigned)pb < nblocks_pool ? pb : 0;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + (int64_t)pb * blk_bytes), (short)0,
                                                 (int)blk_bytes, kBufferRsrcWord3);
    };
    auto load_k = [&](u32x4 (&kr)[ROUNDS][CPL], const char *kbase, int pb) {
        const auto rs = block_rsrc(kbase, pb);
#pragma unroll
        for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                kr[j][c] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, koff + c * LPT * 16, (int)(row_token<LPT>(0, j * C::TRN) * tok_bytes), 0);
    };
    auto load_v = [&](VT (&vr)[VPASS], const char *vbase, int pb) {
        const auto rs = block_rsrc(vbase, pb);
#pragma unroll
        for (int v = 0; v < VPASS; ++v) {
            const int vrow = (int)(row_token<LPT>(0, v * VTPR) * tok_bytes);
            if constexpr (C::VB == 16)
                vr[v] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, vrow, 0);
            else
                vr[v] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, vrow, 0);
        }
    };
    auto head_base = [&](const void *cache, int hg) {
        return (const char *)cache + (int64_t)(hg * HPG + w) * D * C::EB;
    };

    // Issue priority follows this wave's remaining work (3 at the start, 0 near
    // the end): when two work-groups share a CU, the one that has fallen behind
    // gets the instruction slots, instead of the older one by default, so both
    // finish together.  The persistent grid fills every CU's first slots with
    // the first half of the work-groups before the rest; the later ones lower
    // their priority half a step later, which cancels the age tie-break at
    // equal progress.  Only the order of issue changes, never the arithmetic.
    const int exp_w = (int)(a1 - a0);  // blocks of this wave
    const int ew = exp_w > 0 ? exp_w : 1;
    const int lag = blockIdx.x >= gridDim.x / 2 ? ew / 2 : 0;
    int done_w = 0, cur_prio = -1;
    auto update_priority = [&]() {
        const int pr = 3 - min(3, max(0, 4 * done_w - lag) / ew);
        if (pr != cur_prio) {
            cur_prio = pr;
            if (pr == 3)
                __builtin_amdgcn_s_setprio(3);
            else if (pr == 2)
                __builtin_amdgcn_s_setprio(2);
            else if (pr == 1)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
    };

    // ---- hand-over of partial results.  The partial records of one
    // (sequence, head group) are the contiguous slot range [lo, lo + np), each
    // holding the HPG*G query heads of the group.  Each contributing
    // work-group counts its arrival once its partial stores have completed; the
    // one that completes the count merges every partial and writes the output.
    // Work-groups do this for all their pending partials at once, after their
    // last segment (or when the pending list is full), so no segment waits for
    // a memory round trip.  Partials are written and read with device-coherent
    // (L2-bypassing) accesses, so the hand-over needs no cache flush.
    constexpr int HG = HPG * G;  // query heads of a head group
    int ndef = 0;
    // MB: partials per merge batch (8 after the last segment, when no other
    // registers are live; 2 in the middle of a range, next to the prefetched
    // blocks)
    auto flush = [&](auto batch_tag) {
        constexpr int MB = decltype(batch_tag)::value;
        wait_vm<0>();  // this wave's partial stores have completed
        __syncthreads();
        if (tid < ndef)
            sm.def_last[tid] = __hip_atomic_fetch_add(&a.ws_count[sm.def_pair[tid]], 1,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                               sm.def_np[tid] - 1;
        __syncthreads();
        static_assert(HG <= 32, "merge scratch holds 32 query heads");
        constexpr int KC = (HG * D + 4 * NT - 1) / (4 * NT);  // 4-column chunks per thread
        for (int k = 0; k < ndef; ++k) {
            if (!sm.def_last[k])
                continue;
            const int lo = sm.def_lo[k], np = sm.def_np[k];
            float *out_row = a.out + sm.def_out[k];
            // the np records of this (sequence, head group); loads past them read zero
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.ws_acc + (int64_t)lo * HG * D), (short)0, np * HG * D * 4, kBufferRsrcWord3);
            float num[KC][4];
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    num[kc][j] = 0.f;
            if (tid < HG) {
                sm.mM[tid] = -INFINITY;
                sm.mden[tid] = 0.f;
            }
            __syncthreads();
            // batches of MB partials: every thread issues the accumulator loads of
            // its columns, the threads that own a head load the (max, sum)
            // pairs and publish the scale factors, then all combine: one memory
            // round trip per batch
            for (int s0 = 0; s0 < np; s0 += MB) {
                u32x4 ac[MB][KC];
#pragma unroll
                for (int k2 = 0; k2 < MB; ++k2)
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        const int e = 4 * tid + kc * 4 * NT;
                        ac[k2][kc] = e < HG * D ? __builtin_amdgcn_raw_buffer_load_b128(
                                                      rs, ((s0 + k2) * HG * D + e) * 4, 0, kBufferCoherent)
                                                : u32x4{0u, 0u, 0u, 0u};
                    }
                if (tid < HG) {
                    f32x2 ml[MB];
#pragma unroll
                    for (int k2 = 0; k2 < MB; ++k2)
                        ml[k2] = s0 + k2 < np
                                     ? coherent_load2(&a.ws_ml[((int64_t)(lo + s0 + k2) * HG + tid) * 2])
                                     : f32x2{-INFINITY, 0.f};
                    const float M = sm.mM[tid];
                    float Mb = M;
#pragma unroll
                    for (int k2 = 0; k2 < MB; ++k2)
                        Mb = fmaxf(Mb, ml[k2][0]);
                    const float fo = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
                    float den = sm.mden[tid] * fo;
#pragma unroll
                    for (int k2 = 0; k2 < MB; ++k2) {
                        const float f = ml[k2][0] == -INFINITY ? 0.f : fast_exp2(ml[k2][0] - Mb);
                        den += f * ml[k2][1];
                        sm.mf[k2][tid] = f;
                    }
                    sm.mfo[tid] = fo;
                    sm.mM[tid] = Mb;
                    sm.mden[tid] = den;
                }
                __syncthreads();
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int e = 4 * tid + kc * 4 * NT;
                    if (e < HG * D) {
                        const int h = e / D;
                        const float fo = sm.mfo[h];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            num[kc][j] *= fo;
#pragma unroll
                        for (int k2 = 0; k2 < MB; ++k2) {
                            const float f = sm.mf[k2][h];
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                num[kc][j] = fmaf(f, __uint_as_float(ac[k2][kc][j]), num[kc][j]);
                        }
                    }
                }
                __syncthreads();  // the scale factors of the next batch go to the same place
            }
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                const int e = 4 * tid + kc * 4 * NT;
                if (e < HG * D) {
                    const float inv = a.v_scale / sm.mden[e / D];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        out_row[e + j] = num[kc][j] * inv;
                }
            }
            if (tid == 0)
                a.ws_count[sm.def_pair[k]] = 0;  // leave the counter at zero for the next call
        }
        ndef = 0;
        __syncthreads();  // the pending list may be refilled
    };

    // ---- first segment: q to LDS before any K/V load is issued (the wait for
    // a load also waits for every load issued before it), then its first two
    // blocks into slots 0 and 1 (the segment's first block again in slot 1 when
    // it has only one: a null block, see below)
    Seg sg = describe(item, i, base_i, uniform(sm.seg_L));
    load_q(i, sg.hg * HPG + w);
    store_q();
    {
        const auto tab = scalar_view(a.block_tables + (int64_t)i * maxB);
        const int p0 = uniform(unit_block(tab, sg.b0));
        const int p1 = sg.b1 - sg.b0 > 1 ? uniform(unit_block(tab, sg.b0 + 1)) : p0;
        const char *kb = head_base(a.k_cache, sg.hg), *vb = head_base(a.v_cache, sg.hg);
        load_k(kr0, kb, p0);
        load_v(vr0, vb, p0);
        asm volatile("" ::: "memory");  // keep the slot order: slot 0 K, V, slot 1 K, V
        load_k(kr1, kb, p1);
        load_v(vr1, vb, p1);
    }
    for (;;) {
        const int L = sg.L, n_i = sg.n_i, hg = sg.hg, x = sg.x, seg_items = sg.seg_items;
        const int b0 = sg.b0, b1 = sg.b1, slot = sg.slot;
        const int g = hg * HPG + w;  // this wave's KV head
        const bool first = x == 0;
        const bool last = x + seg_items == n_i;
        const bool direct = first && last;
        // the following segment
        const long long item_n = item + seg_items;
        const bool has_next = item_n < a1;
        int i_n = i;
        long long base_n = base_i;
        if (last && hg == NHG - 1) {
            base_n += (long long)n_i * NHG;
            ++i_n;
        }
        Seg nx = sg;
        if (has_next)
            nx = describe(item_n, i_n, base_n, i_n == i ? L : lens_s[i_n]);
        const uint8_t *qb = &sm.qbuf[w][0];

        // ---- per-wave streaming softmax over the segment's blocks -----------
        float acc[G][EV];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EV; ++e)
                acc[h][e] = 0.f;
        if (lane < G)
            sm.mref[w][lane] = -INFINITY;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float my_mref = -INFINITY;  // sm.mref[w][lane_m]
        float lsum = 0.f;

        const auto table = scalar_view(a.block_tables + (int64_t)i * maxB);
        const char *kbase = head_base(a.k_cache, hg);
        const char *vbase = head_base(a.v_cache, hg);

        // The block a slot loads after its current one: the next block of this
        // segment, else the slot's first block of the following segment (a
        // placeholder load of this segment's first block when there is none),
        // so the following segment's loads are already in flight when this one
        // ends.
        const int p_first = uniform(unit_block(table, b0));  // this segment's first block
        const char *nkbase = kbase, *nvbase = vbase;
        int npb[2] = {p_first, p_first};
        if (has_next) {
            const auto ntab = scalar_view(a.block_tables + (int64_t)i_n * maxB);
            npb[0] = uniform(unit_block(ntab, nx.b0));
            npb[1] = nx.b1 - nx.b0 > 1 ? uniform(unit_block(ntab, nx.b0 + 1)) : npb[0];
            nkbase = head_base(a.k_cache, nx.hg);
            nvbase = head_base(a.v_cache, nx.hg);
        }

        auto step = [&](int b, u32x4 (&kr)[ROUNDS][CPL], VT (&vr)[VPASS], int pb2,
                        const char *kb2, const char *vb2) {
            update_priority();
            ++done_w;

            // -- scores of this lane's token(s) for head lane_m ------------
            const int tbase = b * 16;
            float xs[ROUNDS][GP];
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
                for (int s = 0; s < GP; ++s)
                    xs[j][s] = 0.f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
#pragma unroll
                for (int s = 0; s < GP; ++s) {
                    // q chunk of (slot s, chunk c): QW dwords, used for every round
                    uint32_t qc[QW];
                    const u32x4 *qp =
                        (const u32x4 *)(qb + (qlane ^ (unsigned)(s * D * QEB)) + c * LPT * E * QEB);
#pragma unroll
                    for (int k = 0; k < QW / 4; ++k) {
                        const u32x4 u = qp[k];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            qc[4 * k + e] = u[e];
                    }
#pragma unroll
                    for (int j = 0; j < ROUNDS; ++j) {
                        const u32x4 kc = kr[j][c];
                        if constexpr (CDT == DT_BF16) {
#pragma unroll
                            for (int p = 0; p < 4; ++p)
                                xs[j][s] = dot2_bf16(qc[p], kc[p], xs[j][s]);
                        } else if constexpr (CDT == DT_FP8) {
#pragma unroll
                            for (int p = 0; p < 4; ++p) {
                                xs[j][s] = dot2_bf16(qc[2 * p], fp8x2_to_bf16x2<false>(kc[p]), xs[j][s]);
                                xs[j][s] = dot2_bf16(qc[2 * p + 1], fp8x2_to_bf16x2<true>(kc[p]), xs[j][s]);
                            }
                        } else {
#pragma unroll
                            for (int p = 0; p < 4; ++p)
                                xs[j][s] = fmaf(__uint_as_float(qc[p]), __uint_as_float(kc[p]), xs[j][s]);
                        }
                    }
                }
            }
            float sc[ROUNDS];
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j) {
                const float s2 = reduce_scatter<LPT, GP>(xs[j]) * a.qk_scale;
                const int tt = tbase + row_token<LPT>(row, tr + j * C::TRN);
                sc[j] = tt < L ? s2 : -INFINITY;
            }
            load_k(kr, kb2, pb2);

            // -- block maximum of the row for head lane_m ------------------
            float bm = sc[0];
            if constexpr (ROUNDS == 2)
                bm = fmaxf(bm, sc[1]);
            if constexpr (LPT == 4)
                bm = fmaxf(bm, dpp<DPP_ROW_ROR4>(bm));
            bm = fmaxf(bm, dpp<DPP_ROW_ROR8>(bm));

            const bool need = lane_m < G && bm > my_mref + TAU;
            if (wave_any(need)) {
                // raise the wave's reference maximum for every head
                if (lane_owner && tr == 0)
                    sm.bmax[w][row][lane_m] = bm;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
                float my_alpha = 1.f;
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float mx = fmaxf(fmaxf(sm.bmax[w][0][h], sm.bmax[w][1][h]),
                                     fmaxf(sm.bmax[w][2][h], sm.bmax[w][3][h]));
                    const float mold = sm.mref[w][h];
                    const float mnew = fmaxf(mold, mx);
                    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mold - mnew);
#pragma unroll
                    for (int e = 0; e < EV; ++e)
                        acc[h][e] *= alpha;
                    if (h == lane_m) {
                        my_alpha = alpha;
                        my_mref = mnew;
                    }
                    if (lane == 0)
                        sm.mref[w][h] = mnew;
                }
                lsum *= my_alpha;
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                __builtin_amdgcn_wave_barrier();
            }

            // -- probabilities to LDS --------------------------------------
            const float m_use = my_mref == -INFINITY ? 0.f : my_mref;
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j) {
                const float p = fast_exp2(sc[j] - m_use);
                if (lane_owner) {
                    lsum += p;
                    sm.p[w][row_token<LPT>(row, tr + j * C::TRN)][lane_m] = p;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();

            // -- PV ----------------------------------------------------------
            if (tbase + 16 > L) {  // last block of the sequence (wave-uniform): slots past
                                   // the context may hold any bits, their p is 0
#pragma unroll
                for (int v = 0; v < VPASS; ++v)
                    if (tbase + row_token<LPT>(row, v * VTPR + vh) >= L)
                        vr[v] = VT{};
            }
#pragma unroll
            for (int v = 0; v < VPASS; ++v) {
                const int tk = row_token<LPT>(row, v * VTPR + vh);
                const VT vv = vr[v];
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    pr[h] = sm.p[w][tk][h];
                float ve[EV];
                if constexpr (CDT == DT_BF16) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        ve[2 * k] = bf16_lo(vv[k]);
                        ve[2 * k + 1] = bf16_hi(vv[k]);
                    }
                } else if constexpr (CDT == DT_FP8) {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const f32x2 lo = fp8x2_to_f32x2<false>(vv[k]);
                        const f32x2 hi = fp8x2_to_f32x2<true>(vv[k]);
                        ve[4 * k] = lo[0];
                        ve[4 * k + 1] = lo[1];
                        ve[4 * k + 2] = hi[0];
                        ve[4 * k + 3] = hi[1];
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        ve[k] = __uint_as_float(vv[k]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < EV; ++e)
                        acc[h][e] = fmaf(pr[h], ve[e], acc[h][e]);
            }
            load_v(vr, vb2, pb2);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        };
        // Blocks b0, b0 + 1 are in slots 0 and 1 when the segment starts; the
        // loop takes the rest two at a time.  Every iteration processes both
        // slots and issues the same loads in the same order (slot 0 K, V, slot
        // 1 K, V), so each wait is for exactly the block it needs: an odd
        // block count is padded with a null block (an index past the end of
        // the sequence: every score masked, V rows zeroed, nothing added), and
        // in the last iteration both slots load their block of the following
        // segment.
        {
            const int nullb = (L + 15) >> 4;
            int blk0 = b0, blk1 = b1 - b0 > 1 ? b0 + 1 : nullb;
            for (int j = b0 + 2;; j += 2) {
                const bool more = j < b1;  // uniform
                const bool more1 = j + 1 < b1;
                const int p0 = more ? uniform(unit_block(table, j)) : npb[0];
                const int p1 = more1 ? uniform(unit_block(table, j + 1)) : more ? p_first : npb[1];
                step(blk0, kr0, vr0, p0, more ? kbase : nkbase, more ? vbase : nvbase);
                step(blk1, kr1, vr1, p1, more ? kbase : nkbase, more ? vbase : nvbase);
                if (!more)
                    break;
                blk0 = j;
                blk1 = more1 ? j + 1 : nullb;
            }
        }

        // ---- this wave's totals for its head -> output or partial -----------
        // sum over rows and over the lanes of a row that hold other tokens
        float ls = lane_owner ? lsum : 0.f;
        ls = sum_rows(ls);
        if constexpr (LPT == 4)
            ls += dpp<DPP_ROW_ROR4>(ls);
        ls += dpp<DPP_ROW_ROR8>(ls);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                float t = sum_rows(acc[h][e]);
                if constexpr (VTPR == 2)
                    t += dpp<DPP_ROW_ROR8>(t);
                if constexpr (VTPR == 4) {
                    t += dpp<DPP_ROW_ROR4>(t);
                    t += dpp<DPP_ROW_ROR8>(t);
                }
                acc[h][e] = t;
            }
        if (lane < 16 && tr == 0 && lane_owner)
            sm.lsum[w][lane_m] = ls;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float Lh[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            Lh[h] = sm.lsum[w][h];
        // lanes < NCV hold piece `lane` (EV elements) of every head's row
        if (direct) {
            if (lane < NCV) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float *dst = a.out + ((int64_t)i * Hq + g * G + h) * D + lane * EV;
                    const float inv = a.v_scale / Lh[h];
#pragma unroll
                    for (int e = 0; e < EV; ++e)
                        dst[e] = acc[h][e] * inv;
                }
            }
        } else {
            const int64_t rec = (int64_t)slot * HPG + w;  // this head's partial record
            if (lane < NCV) {
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < EV; e += 2)
                        coherent_store2(&a.ws_acc[(rec * G + h) * D + lane * EV + e], acc[h][e],
                                        acc[h][e + 1]);
            }
            if (lane < G)
                coherent_store2(&a.ws_ml[(rec * G + lane) * 2], sm.mref[w][lane], sm.lsum[w][lane]);
            // this partial's slot range, kept for the hand-over
            const int pair = i * NHG + hg;
            int lo, hi;
            if (PB > 0) {
                lo = (int)(item - x);
                hi = lo + n_i - 1;
            } else {
                const long long W = gridDim.x;
                const long long first_item = base_i + (long long)hg * n_i;
                const long long last_item = first_item + n_i - 1;
                const long long k_first = ((first_item + 1) * W - 1) / total;
                const long long k_last = ((last_item + 1) * W - 1) / total;
                const long long r_first = k_first < k_first * total / W ? k_first : k_first * total / W;
                const long long r_last = k_last < k_last * total / W ? k_last : k_last * total / W;
                lo = (int)r_first + pair;
                hi = (int)r_last + pair;
            }
            if (tid == 0) {
                sm.def_lo[ndef] = lo;
                sm.def_np[ndef] = hi - lo + 1;
                sm.def_pair[ndef] = pair;
                sm.def_out[ndef] = ((int64_t)i * Hq + hg * HG) * D;
            }
            ++ndef;
            if (ndef == kDecodeDeferred && has_next)
                flush(std::integral_constant<int, 2>{});
        }

        // ---- advance ----------------------------------------------------------
        if (!has_next)
            break;
        load_q(i_n, nx.hg * HPG + w);
        store_q();
        item = item_n;
        i = i_n;
        base_i = base_n;
        sg = nx;
    }
    if (ndef > 0)
        flush(std::integral_constant<int, 8>{});
}

}  // namespace hg

// Decode kernels of head groups of four KV heads.
DecodeKernels decode_hg4_kernels(int cache_dtype, int head_dim, int group);

}  // namespace pa
