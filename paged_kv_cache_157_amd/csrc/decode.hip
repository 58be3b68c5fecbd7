// decode.hip -- single-query decode attention over a paged KV cache.
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
//   * The flat list of "items" is (sequence, KV head, x) where x is a
//     16-token block (balanced mode) or a fixed partition of blocks.  A
//     persistent grid of work-groups takes contiguous ranges of the list, so a
//     32k-token sequence is spread over many CUs as evenly as a batch of short
//     ones.  Balanced ranges are equal in "virtual" items: every (sequence, KV
//     head) counts a few extra items ahead of its blocks, so a range that
//     starts more segments holds fewer blocks.  A run of items of one (sequence, KV head) inside
//     a range is a "segment".  A segment that covers its whole sequence
//     writes the output directly; otherwise it writes a partial
//     (max, sum, unnormalised accumulator); the work-group that delivers the
//     last partial of a (sequence, KV head) merges them (arrival counter),
//     so a call is a single kernel launch.
//   * Inside a work-group the four waves take every fourth block of the
//     segment.  A wave handles all G query heads of its KV head, so each
//     K/V row fetched from HBM is used G times from registers.
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
//     V; each lane owns one 16-byte chunk of V for four tokens of the block
//     and accumulates G fp32 heads with FMA.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

#ifndef DECODE_STAGES
#define DECODE_STAGES 2  // blocks of K/V in a wave's LDS ring (the loop is written for 2)
#endif
#ifndef DECODE_SEGCOST
// Virtual items charged for each (sequence, KV head), so that a range which
// starts extra segments (each costs a hand-over) holds fewer real blocks.
// Chosen by measurement on 64-sequence GQA batches: 2-3 shortens the slowest
// work-group, more overshoots.
#define DECODE_SEGCOST 2
#endif
#ifndef DECODE_WAVES
#define DECODE_WAVES 4   // waves per work-group; they split a segment's blocks
#endif

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
    static constexpr int VTPR = 16 / NC;         // tokens per row per V pass
    static constexpr int VPASS = 4 / VTPR;       // V passes per block
    // q dwords per (head slot, K chunk): bf16 pairs matching the chunk, or fp32
    static constexpr int QW = CDT == DT_FP8 ? 8 : 4;
    static_assert(CPL >= 1 && NC <= 16 && NC >= 4, "unsupported chunk geometry");
    static_assert(G >= 1 && G <= 8, "GQA group must be 1..8");
};

// Token (0..15 within the block) held in "row" r at index k (0..3).  QK lanes
// of row r handle exactly the tokens that the V lanes of row r accumulate, so
// the running maximum of a row never has to leave it.
template <int LPT>
__device__ __forceinline__ int row_token(int r, int k)
{
    if constexpr (LPT == 4)
        return 4 * r + k;
    else
        return 2 * r + (k & 1) + 8 * (k >> 1);
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

template <int CDT, int D, int G, int NSTAGE, int WAVES>
struct DecodeSmem {
    using C = DecodeCfg<CDT, D, G>;
    static constexpr int KB = 16 * D * C::EB;  // bytes of one block of one KV head (K or V)
    // bytes of the q rows of one (sequence, KV head): G heads x D (fp32 q with
    // an fp32 cache, else bf16), rounded up to whole 1 KiB DMA instructions
    static constexpr int QB = G * D * (CDT == DT_F32 ? 4 : 2);
    static constexpr int QBR = (QB + 1023) / 1024 * 1024;
    // per-wave ring of NSTAGE blocks, K then V, filled by global->LDS DMA; at a
    // segment end the last stage holds the wave's accumulators (G x D fp32)
    __attribute__((aligned(16))) uint8_t ring[WAVES][NSTAGE][2 * KB];
    // q of the current and of the next segment (double buffer)
    __attribute__((aligned(16))) uint8_t qbuf[2][QBR];
    float p[WAVES][16][8];       // probabilities of the current block
    float bmax[WAVES][4][8];     // row maxima (rescale path)
    float msum[WAVES][2][8];     // per-wave running max and sum
    long long total;  // item count of the call (start-up scan)
    long long total_v;  // the same in virtual items (0: plain split)
    long long range0, range1;  // this work-group's items [range0, range1)
    int last;
    int seg_i;
    long long seg_base, seg_vbase;
};

// s_waitcnt vmcnt(N): the global->LDS loads of the ring are counted there and
// the compiler does not wait for them by itself.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Work-group barrier for LDS data only: every wave's LDS accesses have
// completed (lgkmcnt), global loads may stay in flight.  Where a hand-over
// needs global memory complete, the code waits for it explicitly first.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void dma16(const void *src, void *lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}

// H8: the pools hold 8-token blocks (tbs_log2 < 0; a separate instantiation, so
// that the address arithmetic of larger blocks carries no branch for it)
template <int CDT, int D, int G, int NSTAGE, int WAVES, bool H8>
__global__ __launch_bounds__(64 * WAVES) void decode_kernel(DecodeArgs a)
{
    using C = DecodeCfg<CDT, D, G>;
    using SM = DecodeSmem<CDT, D, G, NSTAGE, WAVES>;
    constexpr int NT = 64 * WAVES;
    constexpr int LPT = C::LPT, GP = C::GP, CPL = C::CPL, ROUNDS = C::ROUNDS;
    constexpr int NC = C::NC, E = C::E, VTPR = C::VTPR, VPASS = C::VPASS, QW = C::QW;
    constexpr int KB = SM::KB;
    constexpr int LPB = 2 * KB / 1024;  // DMA instructions per block (K and V)
    static_assert(ROUNDS * CPL * 1024 == KB && VPASS * 1024 == KB, "DMA layout");
    constexpr float TAU = 8.0f;
    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_q_heads, maxB = a.max_blocks;
    const int PB = a.part_blocks;
    // The kernel walks 16-token units.  With blocks of 16 or more tokens a
    // table entry names 2^ts consecutive units (ts >= 0); with 8-token blocks
    // (ts < 0) a unit is two blocks, tab[2u] and tab[2u + 1], whose rows sit
    // in two unrelated places: each lane then takes the base of the half that
    // holds its row.
    const int ts = a.tbs_log2;
    constexpr bool h8 = H8;
    const int maxU = h8 ? (maxB + 1) >> 1 : maxB << ts;  // units a table row addresses
    const int maxL = h8 ? 8 * maxB : 16 * maxU;          // tokens a table row addresses
    // physical location of unit u: {unit index, -} or {block of rows 0-7, of rows 8-15}
    struct Phys {
        int a, b;
    };
    auto unit_block = [&](auto tab, int u) -> Phys {
        if (h8) {
            const int e1 = 2 * u + 1 < maxB ? 2 * u + 1 : maxB - 1;  // rows past the table are masked
            return Phys{tab[2 * u], tab[e1]};
        }
        const int e = (tab[u >> ts] << ts) + (u & ((1 << ts) - 1));
        return Phys{e, e};
    };

    auto items_of = [&](int L) -> int {
        L = L < 0 ? 0 : L;
        int nb = (L + 15) >> 4;
        nb = nb > maxU ? maxU : nb;
        return PB > 0 ? (nb + PB - 1) / PB : nb;
    };

    // ---- this work-group's range of items.  With the balanced split the
    // ranges are equal in "virtual" items: each (sequence, KV head) counts
    // ALPHA extra items ahead of its real ones (what a segment start costs),
    // so a range that starts segments holds fewer real items.  Wave 0 scans
    // the lengths 64 at a time (no work-group barrier inside), finds the
    // sequences holding both ends of its range and the first real items at or
    // after them; the other waves wait at the barrier below.
    constexpr int ALPHA = DECODE_SEGCOST;
    if (w == 0) {
        const long long W = gridDim.x;
        // 64 lanes' item counts fit 32 bits whenever (maxU + ALPHA) * Hkv * 64
        // does: DPP scans then; otherwise shuffles on 64-bit values
        const bool narrow = (long long)(maxU + ALPHA) * Hkv * 64 < (1ll << 31);
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
            const int n = items_of(l);
            real = (long long)n * Hkv;
            virt = (long long)(n > 0 ? n + ALPHA : 0) * Hkv;
        };
        long long tot = 0, totv = 0;
        // up to 64 sequences with narrow counts: one load of the lengths and
        // one pair of prefix sums serve the totals and the search below
        const bool one_pass = narrow && S <= 64;
        int l0 = 0, ri0 = 0, vi0 = 0;
        long long rr0 = 0, vv0 = 0;
        if (one_pass) {
            l0 = lane < S ? a.context_lens[lane] : 0;
            counts(l0, rr0, vv0);
            ri0 = wave_scan32((int)rr0);
            vi0 = wave_scan32((int)vv0);
            tot = __builtin_amdgcn_readlane(ri0, 63);
            totv = __builtin_amdgcn_readlane(vi0, 63);
        } else {
            for (int base = 0; base < S; base += 64) {
                const int s2 = base + lane;
                long long r, v;
                counts(s2 < S ? a.context_lens[s2] : 0, r, v);
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
        // position x of the split -> (sequence, its real / virtual starts, first
        // real item at or after x)
        auto locate = [&](long long x, int &seq, long long &rbase, long long &vbase) -> long long {
            const long long T = virt ? totv : tot;
            seq = -1;
            rbase = tot;
            vbase = totv;
            if (x >= T)
                return tot;
            long long rc = 0, vc = 0;
            for (int base = 0; base < S; base += 64) {
                const int s2 = base + lane;
                const int l = s2 < S ? a.context_lens[s2] : 0;
                long long r, v;
                counts(l, r, v);
                const long long ri = scan(r), vi = scan(v);
                const long long ex = (virt ? vi - v : ri - r), in = virt ? vi : ri;
                const long long c0 = virt ? vc : rc;
                const unsigned long long m =
                    __builtin_amdgcn_ballot_w64(r > 0 && c0 + ex <= x && x < c0 + in);
                if (m) {
                    const int l2 = __builtin_ctzll(m);
                    seq = base + l2;
                    rbase = rc + __shfl(ri - r, l2);
                    vbase = vc + __shfl(vi - v, l2);
                    const int n = items_of(__shfl(l, l2));
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
        const long long T = virt ? totv : tot;
        int seq0, seq1;
        long long rb0, vb0, rb1, vb1;
        long long r0, r1;
        if (one_pass) {
            // the prefix sums above, the found lane read with scalar lane
            // reads; 32-bit divisions wherever the operands fit (T * W < 2^31:
            // every position, count and quotient below is under T)
            const int l = l0;
            const long long rr = rr0, vv = vv0;
            const int ri = ri0, vi = vi0;
            const int n = items_of(l);
            const bool d32 = T * W < (1ll << 31);
            auto div = [&](long long num, long long den) -> long long {
                return d32 ? (long long)((unsigned)num / (unsigned)den) : num / den;
            };
            auto find = [&](long long x, int &seq, long long &rbase, long long &vbase) -> long long {
                seq = -1;
                rbase = tot;
                vbase = totv;
                if (x >= T)
                    return tot;
                const long long in = virt ? vi : ri, ex = in - (virt ? vv : rr);
                const unsigned long long m = __builtin_amdgcn_ballot_w64(rr > 0 && ex <= x && x < in);
                const int l2 = __builtin_ctzll(m);  // m != 0 while x < T
                seq = l2;
                rbase = __builtin_amdgcn_readlane(ri, l2) - __builtin_amdgcn_readlane((int)rr, l2);
                vbase = __builtin_amdgcn_readlane(vi, l2) - __builtin_amdgcn_readlane((int)vv, l2);
                if (!virt)
                    return x;
                const int nn = __builtin_amdgcn_readlane(n, l2);
                const long long rel = x - vbase;
                const long long gq = div(rel, nn + ALPHA), xv = rel - gq * (nn + ALPHA);
                return rbase + gq * nn + (xv > ALPHA ? xv - ALPHA : 0);
            };
            r0 = find(div(T * blockIdx.x, W), seq0, rb0, vb0);
            r1 = find(div(T * (blockIdx.x + 1), W), seq1, rb1, vb1);
        } else {
            r0 = locate(T * blockIdx.x / W, seq0, rb0, vb0);
            r1 = locate(T * (blockIdx.x + 1) / W, seq1, rb1, vb1);
        }
        if (lane == 0) {
            sm.total = tot;
            sm.total_v = virt ? totv : 0;
            sm.range0 = r0;
            sm.range1 = r1;
            sm.seg_i = seq0;
            sm.seg_base = rb0;
            sm.seg_vbase = vb0;
        }
    }
    barrier_lds();
    const long long total = uniform64(sm.total);
    const long long total_v = uniform64(sm.total_v);  // > 0: virtual split
    if (blockIdx.x == 0) {  // sequences with no tokens get a zero output row
        for (int i = tid; i < S; i += NT)
            if (a.context_lens[i] <= 0)
                for (int e = 0; e < Hq * D; ++e)
                    a.out[(int64_t)i * Hq * D + e] = 0.f;
    }
    const long long a0 = uniform64(sm.range0);
    const long long a1 = uniform64(sm.range1);
    if (a0 >= a1)
        return;
    int i = uniform(sm.seg_i);
    if (i < 0)  // unreachable while a0 < total; keeps every index in range
        return;
    long long base_i = uniform64(sm.seg_base);    // first item index of sequence i
    long long vbase_i = uniform64(sm.seg_vbase);  // its first virtual item
    long long item = a0;
    const int lane_m = head_mask<LPT, GP>(lane);
    const bool lane_owner = mask_owner<LPT, GP>(lane) && lane_m < G;
    const int row = lane >> 4;

    // QK lane geometry
    const int gl = lane & (LPT - 1);
    const int tr = LPT == 8 ? (lane >> 3) & 1 : (lane >> 2) & 3;
    // V lane geometry
    const int vc = (lane & 15) % NC;
    const int vh = (lane & 15) / NC;

    const int64_t tok_bytes = (int64_t)Hkv * D * C::EB;
    const int64_t blk_bytes = 16 * tok_bytes;
    const int64_t half_bytes = 8 * tok_bytes;
    const unsigned nblocks_pool = (unsigned)a.num_blocks;  // units, or 8-token blocks
    // Base address of a lane's row, given the pool base of its KV head and the
    // lane's offset inside a 16-token unit (its row is in the upper half iff
    // off >= 8 rows: the column part of off is less than one row).  Out-of-range
    // entries read block 0 (caller precondition; keeps every access in the pool).
    auto row_addr = [&](const char *hbase, Phys p, unsigned off) -> const char * {
        if (!h8) {
            const unsigned u = (unsigned)p.a < nblocks_pool ? (unsigned)p.a : 0u;
            return hbase + (int64_t)u * blk_bytes + off;
        }
        const unsigned b0 = (unsigned)p.a < nblocks_pool ? (unsigned)p.a : 0u;
        const unsigned b1 = (unsigned)p.b < nblocks_pool ? (unsigned)p.b : 0u;
        const bool upper = off >= (unsigned)half_bytes;
        return hbase + (int64_t)(upper ? b1 : b0) * half_bytes + (upper ? off - (unsigned)half_bytes : off);
    };

    // per-lane byte offsets of the K and V chunks this lane fetches inside one
    // block (KV head 0); the DMA puts chunk (j, c) of lane l at LDS
    // (j*CPL + c)*1024 + 16*l, so every lane reads back exactly what it fetched
    unsigned koff[ROUNDS][CPL];
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            koff[j][c] = (unsigned)(row_token<LPT>(row, tr + j * C::TRN) * tok_bytes) +
                         (unsigned)((gl + c * LPT) * 16);
    unsigned voff[VPASS];
#pragma unroll
    for (int v = 0; v < VPASS; ++v)
        voff[v] = (unsigned)(row_token<LPT>(row, v * VTPR + vh) * tok_bytes) + (unsigned)(vc * 16);

    uint8_t *my_ring = &sm.ring[w][0][0];

    const auto lens_s = scalar_view(a.context_lens);
    static_assert(G * D * 4 <= 2 * KB && NSTAGE == 2, "two ring stages; accumulators fit in one");
    constexpr int QEB = CDT == DT_F32 ? 4 : 2;  // bytes per q element

    // A segment: the items of one (sequence, KV head) inside [item, a1).  Every
    // value is wave-uniform.  Sequences without items are skipped (advances si).
    struct Seg {
        int L, n_i, g, x, seg_items, b0, b1, slot;
    };
    auto describe = [&](long long it, int &si, long long sbase) -> Seg {
        Seg d;
        int L = lens_s[si];
        int n = items_of(L);
        while (n == 0) {  // cannot happen for the first segment; skip empties
            ++si;
            L = lens_s[si];
            n = items_of(L);
        }
        d.L = uniform(L > maxL ? maxL : L);
        d.n_i = uniform(n);
        const long long rel = it - sbase;
        d.g = uniform((int)(rel / d.n_i));
        d.x = uniform((int)(rel - (long long)d.g * d.n_i));
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
            // a0).  Ranks keep the partial slots of one (sequence, head) contiguous.
            d.slot = (int)(total_v > 0 || a0 >= (long long)blockIdx.x ? (long long)blockIdx.x : a0) +
                     si * Hkv + d.g;
        }
        d.b0 = uniform(d.b0);
        d.b1 = uniform(d.b1);
        return d;
    };
    // q rows of (sequence si, KV head gg) -> qbuf[buf], by wave 0
    auto issue_q = [&](int si, int gg, int buf) {
        if (w == 0) {
            const char *src = (const char *)a.q + ((int64_t)si * Hq + gg * G) * D * QEB;
#pragma unroll
            for (int k = 0; k < SM::QBR / 1024; ++k) {
                const int off = k * 1024 + lane * 16;
                dma16(src + (off < SM::QB ? off : 0), &sm.qbuf[buf][k * 1024]);
            }
        }
    };
    // first block of this wave in a segment -> ring stage 0
    auto issue_first = [&](int si, const Seg &d) -> bool {
        if (d.b0 + w >= d.b1)
            return false;
        Phys pb = unit_block(scalar_view(a.block_tables + (int64_t)si * maxB), d.b0 + w);
        pb.a = uniform(pb.a);
        pb.b = uniform(pb.b);
        const char *kh = (const char *)a.k_cache + (int64_t)d.g * D * C::EB;
        const char *vh = (const char *)a.v_cache + (int64_t)d.g * D * C::EB;
#pragma unroll
        for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                dma16(row_addr(kh, pb, koff[j][c]), my_ring + (j * CPL + c) * 1024);
#pragma unroll
        for (int v = 0; v < VPASS; ++v)
            dma16(row_addr(vh, pb, voff[v]), my_ring + KB + v * 1024);
        return true;
    };

    // Issue priority follows this wave's remaining work (3 at the start, 0 near
    // the end): when two work-groups share a CU, the one that has fallen behind
    // gets the instruction slots, instead of the older one by default, so both
    // finish together.  The persistent grid fills every CU's first slot with
    // work-groups [0, grid/2) before the second; the later ones lower their
    // priority half a step later, which cancels the age tie-break at equal
    // progress.  Only the order of issue changes, never the arithmetic.
    const int exp_w = (int)((a1 - a0 + WAVES - 1) / WAVES);  // this wave's share, blocks
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

    // the first segment's q and each wave's first block go out together;
    // wave 0 then waits for q only
    Seg sg = describe(item, i, base_i);
    issue_q(i, sg.g, 0);
    bool pre0 = issue_first(i, sg);  // this wave's first block of the segment is already in stage 0
    if (w == 0) {
        if (pre0)
            wait_vm<LPB>();
        else
            wait_vm<0>();
    }
    barrier_lds();
    int qbi = 0;  // q buffer of the current segment
    for (;;) {
        const int L = sg.L, n_i = sg.n_i, g = sg.g, x = sg.x, seg_items = sg.seg_items;
        const int b0 = sg.b0, b1 = sg.b1, slot = sg.slot;
        const bool first = x == 0;
        const bool last = x + seg_items == n_i;
        const bool direct = first && last;
        // the following segment: its q is fetched now, during this one
        const long long item_n = item + seg_items;
        const bool has_next = item_n < a1;
        int i_n = i;
        long long base_n = base_i, vbase_n = vbase_i;
        if (last && g == Hkv - 1) {
            base_n += (long long)n_i * Hkv;
            vbase_n += (long long)(n_i + ALPHA) * Hkv;
            ++i_n;
        }
        Seg nx = sg;
        if (has_next) {
            nx = describe(item_n, i_n, base_n);
            issue_q(i_n, nx.g, qbi ^ 1);
        }

        // ---- q for this (sequence, KV head), slot s = head (s ^ lane_m) ---
        uint32_t qr[GP][CPL][QW];
#pragma unroll
        for (int s = 0; s < GP; ++s) {
            const int h = s ^ lane_m;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                const int chunk = gl + c * LPT;
                if (h < G) {
                    const u32x4 *t = (const u32x4 *)&sm.qbuf[qbi][(h * D + chunk * E) * QEB];
#pragma unroll
                    for (int k = 0; k < QW / 4; ++k) {
                        const u32x4 u = t[k];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            qr[s][c][4 * k + e] = u[e];
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < QW; ++k)
                        qr[s][c][k] = 0;
                }
            }
        }

        // ---- per-wave streaming softmax over blocks b0+w, b0+w+WAVES, ... ---
        float acc[G][E];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[h][e] = 0.f;
        float mref[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            mref[h] = -INFINITY;
        float my_mref = -INFINITY;
        float lsum = 0.f;

        const auto table = scalar_view(a.block_tables + (int64_t)i * maxB);
        const char *kbase = (const char *)a.k_cache + (int64_t)g * D * C::EB;
        const char *vbase = (const char *)a.v_cache + (int64_t)g * D * C::EB;

        // blocks of this wave: b0 + w + WAVES*t, t < nb_w
        const int nb_w = b1 - b0 - w > 0 ? (b1 - b0 - w + WAVES - 1) / WAVES : 0;
        // Two ring stages per wave.  K of block t + 2 is loaded into the K half
        // of block t's stage as soon as QK(t) is done, V of block t + 2 into the
        // V half once PV(t) is done, so about 1.5 blocks stay in flight per wave.
        constexpr int NK = ROUNDS * CPL, NV = VPASS;  // DMA instructions per block (K, V)
        auto issue_k = [&](int t, Phys pb) {
            uint8_t *st = my_ring + (t & 1) * 2 * KB;
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    dma16(row_addr(kbase, pb, koff[j][c]), st + (j * CPL + c) * 1024);
        };
        auto issue_v = [&](int t, Phys pb) {
            uint8_t *st = my_ring + (t & 1) * 2 * KB;
#pragma unroll
            for (int v = 0; v < VPASS; ++v)
                dma16(row_addr(vbase, pb, voff[v]), st + KB + v * 1024);
        };
        auto unit_u = [&](int u) -> Phys {
            Phys p = unit_block(table, u);
            return Phys{uniform(p.a), uniform(p.b)};
        };
        // prologue: blocks 0 and 1 in flight (block 0 may already be on its way)
        if (nb_w > 0 && !pre0) {
            const Phys p0 = unit_u(b0 + w);
            issue_k(0, p0);
            issue_v(0, p0);
        }
        if (nb_w > 1) {
            const Phys p1 = unit_u(b0 + w + WAVES);
            issue_k(1, p1);
            issue_v(1, p1);
        }

        for (int t = 0; t < nb_w; ++t) {
            update_priority();
            ++done_w;
            const int b = b0 + w + WAVES * t;
            const bool more1 = t + 1 < nb_w, more2 = t + 2 < nb_w;  // uniform
            const Phys pb2 = more2 ? unit_u(b + 2 * WAVES) : Phys{0, 0};
            // K(t); issued after it and possibly in flight: V(t), K(t+1), V(t+1)
            if (more1)
                wait_vm<NV + NK + NV>();
            else
                wait_vm<NV>();
            const uint8_t *st = my_ring + (t & 1) * 2 * KB + lane * 16;

            // -- scores of this lane's token(s) for head lane_m ------------
            const int tbase = b * 16;
            float sc[ROUNDS];
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j) {
                float xs[GP];
#pragma unroll
                for (int s = 0; s < GP; ++s)
                    xs[s] = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const u32x4 kc = *(const u32x4 *)(st + (j * CPL + c) * 1024);
                    if constexpr (CDT == DT_BF16) {
#pragma unroll
                        for (int s = 0; s < GP; ++s)
#pragma unroll
                            for (int p = 0; p < 4; ++p)
                                xs[s] = dot2_bf16(qr[s][c][p], kc[p], xs[s]);
                    } else if constexpr (CDT == DT_FP8) {
                        uint32_t kk[8];
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            kk[2 * p] = fp8x2_to_bf16x2<false>(kc[p]);
                            kk[2 * p + 1] = fp8x2_to_bf16x2<true>(kc[p]);
                        }
#pragma unroll
                        for (int s = 0; s < GP; ++s)
#pragma unroll
                            for (int p = 0; p < 8; ++p)
                                xs[s] = dot2_bf16(qr[s][c][p], kk[p], xs[s]);
                    } else {
#pragma unroll
                        for (int s = 0; s < GP; ++s)
#pragma unroll
                            for (int p = 0; p < 4; ++p)
                                xs[s] = fmaf(__uint_as_float(qr[s][c][p]), __uint_as_float(kc[p]),
                                             xs[s]);
                    }
                }
                const float s2 = reduce_scatter<LPT, GP>(xs) * a.qk_scale;
                const int tt = tbase + row_token<LPT>(row, tr + j * C::TRN);
                sc[j] = tt < L ? s2 : -INFINITY;
            }

            // K(t) is consumed: its half of the stage takes K(t+2)
            if (more2) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue_k(t + 2, pb2);
            }

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
                    const float mnew = fmaxf(mref[h], mx);
                    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref[h] - mnew);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        acc[h][e] *= alpha;
                    if (h == lane_m) {
                        my_alpha = alpha;
                        my_mref = mnew;
                    }
                    mref[h] = mnew;
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
            // V(t); issued after it and possibly in flight: K(t+1), V(t+1), K(t+2)
            if (more2)
                wait_vm<NK + NV + NK>();
            else if (more1)
                wait_vm<NK + NV>();
            else
                wait_vm<0>();
            u32x4 vrow[VPASS];
#pragma unroll
            for (int v = 0; v < VPASS; ++v)
                vrow[v] = *(const u32x4 *)(st + KB + v * 1024);
            if (tbase + 16 > L) {  // last block of the sequence (wave-uniform): slots past
                                   // the context may hold any bits, their p is 0
#pragma unroll
                for (int v = 0; v < VPASS; ++v)
                    if (tbase + row_token<LPT>(row, v * VTPR + vh) >= L)
                        vrow[v] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int v = 0; v < VPASS; ++v) {
                const int tk = row_token<LPT>(row, v * VTPR + vh);
                const u32x4 vv = vrow[v];
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    pr[h] = sm.p[w][tk][h];
                float ve[E];
                if constexpr (CDT == DT_BF16) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        ve[2 * k] = bf16_lo(vv[k]);
                        ve[2 * k + 1] = bf16_hi(vv[k]);
                    }
                } else if constexpr (CDT == DT_FP8) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
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
                    for (int e = 0; e < E; ++e)
                        acc[h][e] = fmaf(pr[h], ve[e], acc[h][e]);
            }
            // V(t) is consumed: its half of the stage takes V(t+2)
            if (more2) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue_v(t + 2, pb2);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }

        // ---- the following segment's first block goes out now, so its load
        // overlaps this segment's hand-over below (stage 0 is free: this
        // wave's blocks are consumed; the accumulators use the last stage)
        pre0 = has_next && issue_first(i_n, nx);
        if (w == 0) {  // the next segment's q (issued before any ring load) has landed
            if (pre0)
                wait_vm<LPB>();
            else
                wait_vm<0>();
        }

        // ---- wave totals -> LDS --------------------------------------------
        // sum over rows and over the lanes of a row that hold other tokens
        float ls = lane_owner ? lsum : 0.f;
        ls = sum_rows(ls);
        if constexpr (LPT == 4)
            ls += dpp<DPP_ROW_ROR4>(ls);
        ls += dpp<DPP_ROW_ROR8>(ls);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float t = sum_rows(acc[h][e]);
                if constexpr (VTPR == 2)
                    t += dpp<DPP_ROW_ROR8>(t);
                if constexpr (VTPR == 4) {
                    t += dpp<DPP_ROW_ROR4>(t);
                    t += dpp<DPP_ROW_ROR8>(t);
                }
                acc[h][e] = t;
            }
        if (lane < NC) {
            float *accw = (float *)&sm.ring[w][NSTAGE - 1][0];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    accw[h * D + lane * E + e] = acc[h][e];
        }
        if (lane < 16 && tr == 0 && lane_owner)
            sm.msum[w][1][lane_m] = ls;
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
                sm.msum[w][0][h] = mref[h];
        }
        barrier_lds();

        // ---- merge the waves; write the output, or a partial -----------------
        // two consecutive d of one head per thread
        for (int e = 2 * tid; e < G * D; e += 2 * NT) {
            const int h = e / D, c = e - h * D;
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww)
                M = fmaxf(M, sm.msum[ww][0][h]);
            float A0 = 0.f, A1 = 0.f, Ls = 0.f;
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww) {
                const float m = sm.msum[ww][0][h];
                const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
                const float *accw = (const float *)&sm.ring[ww][NSTAGE - 1][0];
                A0 += f * accw[h * D + c];
                A1 += f * accw[h * D + c + 1];
                Ls += f * sm.msum[ww][1][h];
            }
            if (direct) {
                float *dst = a.out + ((int64_t)i * Hq + g * G + h) * D + c;
                const float inv = a.v_scale / Ls;
                dst[0] = A0 * inv;
                dst[1] = A1 * inv;
            } else {
                // partials are written and read with device-coherent (L2-bypassing)
                // accesses, so the hand-over below needs no cache flush
                coherent_store2(&a.ws_acc[((int64_t)slot * G + h) * D + c], A0, A1);
                if (c == 0)
                    coherent_store2(&a.ws_ml[((int64_t)slot * G + h) * 2], M, Ls);
            }
        }
        if (!direct) {
            // The partial slots of (i, g) are the contiguous range [lo, hi].  Count
            // arrivals; the work-group that completes the count merges every
            // partial of (i, g) and writes the output.  Ordering: every wave waits
            // for its coherent partial stores to complete before the barrier that
            // precedes the count, and the merger reads them with coherent loads
            // issued after it has seen the final count.
            const int pair = i * Hkv + g;
            int lo, hi;
            if (PB > 0) {
                lo = (int)(item - x);
                hi = lo + n_i - 1;
            } else {
                const long long W = gridDim.x;
                if (total_v > 0) {
                    // work-groups whose (virtual) ranges hold the pair's real items;
                    // every range holds at least one real item, so rank = index
                    const long long first_v = vbase_i + (long long)g * (n_i + ALPHA) + ALPHA;
                    const long long last_v = first_v + n_i - 1;
                    lo = (int)(((first_v + 1) * W - 1) / total_v) + pair;
                    hi = (int)(((last_v + 1) * W - 1) / total_v) + pair;
                } else {
                    const long long first_item = base_i + (long long)g * n_i;
                    const long long last_item = first_item + n_i - 1;
                    const long long k_first = ((first_item + 1) * W - 1) / total;
                    const long long k_last = ((last_item + 1) * W - 1) / total;
                    const long long r_first = k_first < k_first * total / W ? k_first : k_first * total / W;
                    const long long r_last = k_last < k_last * total / W ? k_last : k_last * total / W;
                    lo = (int)r_first + pair;
                    hi = (int)r_last + pair;
                }
            }
            wait_vm<0>();
            barrier_lds();
            if (tid == 0)
                sm.last = __hip_atomic_fetch_add(&a.ws_count[pair], 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == hi - lo;
            barrier_lds();
            if (sm.last) {
                // merge slots lo..hi: thread = 4 consecutive d of one head; the
                // (max, sum) and accumulator loads of up to 8 slots are issued
                // together, so a typical merge costs one memory round trip
                const int np = hi - lo + 1;
                for (int e = 4 * tid; e < G * D; e += 4 * NT) {
                    const int h = e / D;
                    float M = -INFINITY, den = 0.f;
                    float num[4] = {0.f, 0.f, 0.f, 0.f};
                    for (int s0 = 0; s0 < np; s0 += 8) {
                        f32x2 ml[8], ac[8][2];
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            if (s0 + k < np) {
                                const int64_t sl = lo + s0 + k;
                                ml[k] = coherent_load2(&a.ws_ml[(sl * G + h) * 2]);
                                ac[k][0] = coherent_load2(&a.ws_acc[sl * G * D + e]);
                                ac[k][1] = coherent_load2(&a.ws_acc[sl * G * D + e + 2]);
                            } else {
                                ml[k] = f32x2{-INFINITY, 0.f};
                                ac[k][0] = ac[k][1] = f32x2{0.f, 0.f};
                            }
                        }
                        float Mb = M;
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            Mb = fmaxf(Mb, ml[k][0]);
                        const float fo = M == -INFINITY ? 0.f : fast_exp2(M - Mb);
                        den *= fo;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            num[j] *= fo;
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            const float f = ml[k][0] == -INFINITY ? 0.f : fast_exp2(ml[k][0] - Mb);
                            den += f * ml[k][1];
                            num[0] += f * ac[k][0][0];
                            num[1] += f * ac[k][0][1];
                            num[2] += f * ac[k][1][0];
                            num[3] += f * ac[k][1][1];
                        }
                        M = Mb;
                    }
                    const float inv = a.v_scale / den;
                    float *dst = a.out + ((int64_t)i * Hq + g * G) * D + e;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        dst[j] = num[j] * inv;
                }
                if (tid == 0)
                    a.ws_count[pair] = 0;  // leave the counter at zero for the next call
            }
        }
        barrier_lds();

        // ---- advance ----------------------------------------------------------
        if (!has_next)
            break;
        item = item_n;
        i = i_n;
        base_i = base_n;
        vbase_i = vbase_n;
        sg = nx;
        qbi ^= 1;
    }
}

int decode_hpg(int num_kv_heads, int group, int tbs_log2)
{
    return num_kv_heads % 4 == 0 && num_kv_heads >= 8 && group >= 2 && tbs_log2 >= 0 ? 4 : 1;
}

int64_t decode_partial_slots(int num_seqs, int num_kv_heads, int group, int max_blocks,
                             int part_blocks, int grid, int tbs_log2)
{
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    if (part_blocks > 0)  // one record per (partition, sequence, KV head)
        return pairs * ((max_blocks + part_blocks - 1) / part_blocks);
    // balanced split: a record per (range, sequence, KV head) that a range
    // can start a segment of, times the heads of one work-group
    const int hpg = decode_hpg(num_kv_heads, group, tbs_log2);
    return ((int64_t)grid + pairs / hpg) * hpg;
}

bool decode_supported(int cache_dtype, int head_dim, int group)
{
    if (group < 1 || group > 8)
        return false;
    if (head_dim != 64 && head_dim != 128)
        return false;
    if (cache_dtype == DT_F32 && head_dim != 64)
        return false;
    if (cache_dtype == DT_FP8 && head_dim == 64 && group > 4)
        return false;
    return true;
}

template <int CDT, int D, int G>
static DecodeKernels kernels_t(bool h8)
{
    return DecodeKernels{h8 ? (const void *)decode_kernel<CDT, D, G, DECODE_STAGES, DECODE_WAVES, true>
                            : (const void *)decode_kernel<CDT, D, G, DECODE_STAGES, DECODE_WAVES, false>,
                         64 * DECODE_WAVES};
}

template <int CDT, int D>
static DecodeKernels kernels_d(int G, bool h8)
{
    switch (G) {
    case 1: return kernels_t<CDT, D, 1>(h8);
    case 2: return kernels_t<CDT, D, 2>(h8);
    case 3: return kernels_t<CDT, D, 3>(h8);
    case 4: return kernels_t<CDT, D, 4>(h8);
    case 5: return kernels_t<CDT, D, 5>(h8);
    case 6: return kernels_t<CDT, D, 6>(h8);
    case 7: return kernels_t<CDT, D, 7>(h8);
    default: return kernels_t<CDT, D, 8>(h8);
    }
}

DecodeKernels decode_kernels(int cache_dtype, int head_dim, int group, int hpg, bool h8)
{
    if (hpg == 4)
        return decode_hg4_kernels(cache_dtype, head_dim, group);
    if (cache_dtype == DT_F32)
        return kernels_d<DT_F32, 64>(group, h8);
    if (cache_dtype == DT_BF16)
        return head_dim == 64 ? kernels_d<DT_BF16, 64>(group, h8) : kernels_d<DT_BF16, 128>(group, h8);
    if (head_dim == 64) {
        switch (group) {
        case 1: return kernels_t<DT_FP8, 64, 1>(h8);
        case 2: return kernels_t<DT_FP8, 64, 2>(h8);
        case 3: return kernels_t<DT_FP8, 64, 3>(h8);
        default: return kernels_t<DT_FP8, 64, 4>(h8);
        }
    }
    return kernels_d<DT_FP8, 128>(group, h8);
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    const int G = a.num_q_heads / a.num_kv_heads;
    const DecodeKernels k = decode_kernels(a.cache_dtype, a.head_dim, G,
                                           decode_hpg(a.num_kv_heads, G, a.tbs_log2), a.tbs_log2 < 0);
    DecodeArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(k.main, dim3(a.grid), dim3(k.threads), params, 0, stream);
}

}  // namespace pa
