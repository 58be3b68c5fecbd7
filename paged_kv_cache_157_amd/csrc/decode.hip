// decode.hip -- single-query decode attention over a paged KV cache, one KV
// head per work-group at a time (decode_hg.h holds the kernel that takes four
// KV heads per work-group; this file also chooses between the two).
//
// What is computed ("Lecture 33" §2.3): for every sequence i and query head
// h, out[i,h] = softmax(scale * q[i,h] K^T) V over the sequence's tokens,
// whose K/V rows are read in place from scattered physical blocks through
// the block table (logical block t/16, offset t%16, §2.2 walk-through).  The
// lane geometry, the start-up scan, the partial-record slots and the merge are
// in decode_common.h, shared with decode_hg.h.
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
//   * Segment end: each wave sums its accumulators over the four 16-lane rows
//     with a reduce-scatter of lane swaps (fold_totals: a quarter of the swaps
//     and adds of a per-element sum) and stages them in LDS in that folded
//     order; every thread then merges four positions of the four waves and
//     writes them to the output, or to the partial record, which keeps the
//     folded order until the final merge maps it back to columns.
#include "decode_common.h"

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

template <int CDT, int D, int G, int NSTAGE, int WAVES>
struct DecodeSmem {
    using C = dec::DecodeCfg<CDT, D, G>;
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
    dec::Range range;            // this work-group's range (start-up scan)
    dec::MergeLds<G, 8> merge;   // merge of one (sequence, KV head)
    int last;
};

__device__ __forceinline__ void dma16(const void *src, void *lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, 0, 0);
}

// H8: the pools hold 8-token blocks (tbs_log2 < 0; a separate instantiation, so
// that the address arithmetic of larger blocks carries no branch for it)
template <int CDT, int D, int G, int NSTAGE, int WAVES, bool H8>
__global__ __launch_bounds__(64 * WAVES) void decode_kernel(DecodeArgs a)
{
    using C = dec::DecodeCfg<CDT, D, G>;
    using SM = DecodeSmem<CDT, D, G, NSTAGE, WAVES>;
    using dec::row_token;
    using dec::wait_vm;
    using dec::barrier_lds;
    constexpr int NT = 64 * WAVES;
    constexpr int LPT = C::LPT, GP = C::GP, CPL = C::CPL, ROUNDS = C::ROUNDS;
    constexpr int EV = C::EV, NCV = C::NCV, E = C::E, VTPR = C::VTPR, VPASS = C::VPASS, QW = C::QW;
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

    // ---- this work-group's range of items (balanced split: equal in virtual
    // items, ALPHA per (sequence, KV head)); wave 0 scans, the others wait at
    // the barrier below
    constexpr int ALPHA = DECODE_SEGCOST;
    if (w == 0) {
        const dec::Range R = dec::startup_scan<ALPHA>(a.context_lens, S, Hkv, maxU, PB, lane);
        if (lane == 0)
            sm.range = R;
    }
    barrier_lds();
    dec::Range R;
    R.total = uniform64(sm.range.total);
    R.total_v = uniform64(sm.range.total_v);  // > 0: virtual split
    dec::zero_empty_rows<D, NT>(a.context_lens, a.out, S, Hq, tid);
    const long long a0 = uniform64(sm.range.r0);
    const long long a1 = uniform64(sm.range.r1);
    if (a0 >= a1)
        return;
    int i = uniform(sm.range.seq);
    if (i < 0)  // unreachable while a0 < total; keeps every index in range
        return;
    long long base_i = uniform64(sm.range.base);    // first item index of sequence i
    long long vbase_i = uniform64(sm.range.vbase);  // its first virtual item
    long long item = a0;
    const int lane_m = dec::head_mask<LPT, GP>(lane);
    const bool lane_owner = dec::mask_owner<LPT, GP>(lane) && lane_m < G;
    const int row = lane >> 4;

    // QK lane geometry
    const int gl = lane & (LPT - 1);
    const int tr = LPT == 8 ? (lane >> 3) & 1 : (lane >> 2) & 3;
    // V lane geometry
    const int vc = (lane & 15) % NCV;
    const int vh = (lane & 15) / NCV;

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
    // (L: sequence si's length when the caller has it, else -1)
    auto describe = [&](long long it, int &si, long long sbase, int L) -> Seg {
        Seg d;
        if (L < 0)
            L = lens_s[si];
        int n = dec::items_of(L, maxU, PB);
        while (n == 0) {  // cannot happen for the first segment; skip empties
            ++si;
            L = lens_s[si];
            n = dec::items_of(L, maxU, PB);
        }
        d.L = uniform(L > maxL ? maxL : L);
        d.n_i = uniform(n);
        const long long rel = it - sbase;  // < n_i * Hkv: 32-bit division whenever it fits
        d.g = uniform(rel < (1ll << 32) ? (int)((unsigned)rel / (unsigned)d.n_i) : (int)(rel / d.n_i));
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
            d.slot = dec::partial_slot(a0, si * Hkv + d.g);
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

    dec::IssuePriority prio((int)((a1 - a0 + WAVES - 1) / WAVES));  // this wave's share, blocks

    // the first segment's q and each wave's first block go out together;
    // wave 0 then waits for q only
    Seg sg = describe(item, i, base_i, uniform(sm.range.len));  // the scan read the length
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
            nx = describe(item_n, i_n, base_n, i_n == i ? L : -1);
            issue_q(i_n, nx.g, qbi ^ 1);
        }
        // the partial slots [lo, hi] of this segment's (sequence, KV head),
        // worked out now so that the divisions stay off the hand-over
        const int pair = i * Hkv + g;
        int lo = 0, hi = 0;
        if (!direct) {
            if (PB > 0) {
                lo = (int)(item - x);
                hi = lo + n_i - 1;
            } else {
                dec::partial_slot_range(base_i + (long long)g * n_i, n_i, R,
                                        vbase_i + (long long)g * (n_i + ALPHA) + ALPHA, pair, lo, hi);
            }
            lo = uniform(lo);
            hi = uniform(hi);
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
        float acc[G][EV];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < EV; ++e)
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
            prio.step();
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
#pragma unroll
                    for (int s = 0; s < GP; ++s)
                        xs[s] = dec::dot_chunk<CDT, QW>(qr[s][c], kc, xs[s]);
                }
                const float s2 = dec::reduce_scatter<LPT, GP>(xs) * a.qk_scale;
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
                    for (int e = 0; e < EV; ++e)
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
                float pr[G];
#pragma unroll
                for (int h = 0; h < G; ++h)
                    pr[h] = sm.p[w][tk][h];
                float ve[EV];
                dec::widen_v<CDT, EV>(vrow[v], ve);
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < EV; ++e)
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

        // ---- the hand-over runs at the highest issue priority (the next
        // block's step sets the wave's own again)
        __builtin_amdgcn_s_setprio(3);
        prio.cur = 3;
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

        // ---- wave totals -> LDS, in the folded order of fold_totals: element
        // (h, e) of piece p at h * D + e * NCV + p --------------------------------
        const float ls = dec::token_total<LPT>(lane_owner ? lsum : 0.f);
        {
            constexpr int Q = G * EV / 4;
            float tot[Q];
            dec::fold_totals<G, EV, VTPR>(acc, tot);
            const int p = lane & 15, r = lane >> 4;
            if (p < NCV) {
                float *accw = (float *)&sm.ring[w][NSTAGE - 1][0] + r * Q * NCV + p;
#pragma unroll
                for (int k = 0; k < Q; ++k)
                    accw[k * NCV] = tot[k];
            }
        }
        if (lane < 16 && tr == 0 && lane_owner)
            sm.msum[w][1][lane_m] = ls;
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
                sm.msum[w][0][h] = mref[h];
        }
        barrier_lds();

        // ---- merge the waves; write the output, or a partial (kept in the
        // folded order) -----------------------------------------------------------
        // four neighbouring folded positions (pieces p .. p + 3 of one element
        // e) per thread: one 16-byte LDS read per wave, one store
        constexpr int MQ = G * D / 4, MITER = (MQ + NT - 1) / NT;
        const auto ws_rec = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(a.ws_acc + (int64_t)(direct ? 0 : slot) * G * D), (short)0, G * D * 4, dec::kBufferRsrcWord3);
#pragma unroll
        for (int it = 0; it < MITER; ++it) {
            const int f = 4 * (tid + it * NT);
            if (MQ % NT != 0 && f >= G * D)
                break;
            const int h = f / D, q = f - h * D;
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww)
                M = fmaxf(M, sm.msum[ww][0][h]);
            float A[4] = {0.f, 0.f, 0.f, 0.f}, Ls = 0.f;
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww) {
                const float m = sm.msum[ww][0][h];
                const float fw = m == -INFINITY ? 0.f : fast_exp2(m - M);
                const f32x4 v = *(const f32x4 *)((const float *)&sm.ring[ww][NSTAGE - 1][0] + f);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    A[j] = fmaf(fw, v[j], A[j]);
                Ls = fmaf(fw, sm.msum[ww][1][h], Ls);
            }
            if (direct) {
                const int e = q / NCV, p = q - e * NCV;  // columns (p + j) * EV + e
                float *dst = a.out + ((int64_t)i * Hq + g * G + h) * D + p * EV + e;
                const float inv = a.v_scale / Ls;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dst[j * EV] = A[j] * inv;
            } else {
                // partials are written and read with device-coherent (L2-bypassing)
                // accesses, so the hand-over below needs no cache flush
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{__float_as_uint(A[0]), __float_as_uint(A[1]), __float_as_uint(A[2]), __float_as_uint(A[3])},
                    ws_rec, f * 4, 0, dec::kBufferCoherent);
                if (q == 0)
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
            wait_vm<0>();
            barrier_lds();
            if (tid == 0)
                sm.last = __hip_atomic_fetch_add(&a.ws_count[pair], 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == hi - lo;
            barrier_lds();
            if (sm.last) {
                dec::merge_partials<G, D, NT, 8, NCV>(a.ws_ml, a.ws_acc, lo, hi - lo + 1,
                                                 a.out + ((int64_t)i * Hq + g * G) * D, a.v_scale, tid,
                                                 sm.merge);
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
