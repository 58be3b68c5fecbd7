// decode_hg.h -- decode attention by KV-head groups: the variant used when a
// model has at least two groups of four KV heads and G >= 2 (decode_hg4.hip
// instantiates it; decode.hip holds the other kernel and the choice).  The
// computation, the lane geometry, the start-up scan, the partial-record slots
// and the merge are those of decode_common.h, shared with decode.hip.
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

#include "decode_common.h"

namespace pa {
namespace hg {

using dec::u32x2;
using dec::row_token;
using dec::rows_shift_evenly;
using dec::wait_vm;

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
    dec::Range range;  // this work-group's range (start-up scan)
    // pending hand-overs: first slot, slot count, counter index, output row
    int def_lo[kDecodeDeferred], def_np[kDecodeDeferred], def_pair[kDecodeDeferred];
    long long def_out[kDecodeDeferred];
    int def_last[kDecodeDeferred];
    dec::MergeLds<HPG * G, 8> merge;  // merge of one (sequence, head group)
};

using dec::kBufferRsrcWord3;

template <int CDT, int D, int G, int HPG>
__global__ __launch_bounds__(64 * HPG, 2) void decode_hg_kernel(DecodeArgs a)
{
    using C = dec::DecodeCfg<CDT, D, G, CDT == DT_FP8 ? 8 : 16>;
    using SM = DecodeSmem<CDT, D, G, HPG>;
    constexpr int WAVES = HPG;
    constexpr bool HG_FOLD = G <= 4;  // partial records in the folded order
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

    // ---- this work-group's range of items (plain equal split); wave 0 scans,
    // the others wait at the barrier below
    if (w == 0) {
        const dec::Range R = dec::startup_scan<0>(a.context_lens, S, NHG, maxU, PB, lane);
        if (lane == 0)
            sm.range = R;
    }
    __syncthreads();
    dec::Range R;
    R.total = uniform64(sm.range.total);
    R.total_v = 0;
    dec::zero_empty_rows<D, NT>(a.context_lens, a.out, S, Hq, tid);
    const long long a0 = uniform64(sm.range.r0);
    const long long a1 = uniform64(sm.range.r1);
    if (a0 >= a1)
        return;
    int i = uniform(sm.range.seq);
    if (i < 0)  // unreachable while a0 < total; keeps every index in range
        return;
    long long base_i = uniform64(sm.range.base);  // first item index of sequence i
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
    const unsigned nblocks_pool = (unsigned)a.num_blocks;

    // per-lane byte offsets, inside one block (KV head 0), of the first K
    // chunk this lane scores and of the first V piece it accumulates; round j
    // (pass v) adds a whole number of token rows (a scalar offset), chunk c
    // adds c * LPT * 16 bytes (an immediate)
    static_assert(rows_shift_evenly<LPT, C::TRN, ROUNDS, C::TRN>(), "K rounds");
    static_assert(rows_shift_evenly<LPT, VTPR, VPASS, VTPR>(), "V passes");
    const int koff = (int)(row_token<LPT>(row, tr) * tok_bytes) + gl * 16;
    const int voff = (int)(row_token<LPT>(row, vh) * tok_bytes) + vc * C::VPB;

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
        int n = dec::items_of(L, maxU, PB);
        while (n == 0) {  // cannot happen for the first segment; skip empties
            ++si;
            L = lens_s[si];
            n = dec::items_of(L, maxU, PB);
        }
        d.L = uniform(L > maxU * 16 ? maxU * 16 : L);
        d.n_i = uniform(n);
        const long long rel = it - sbase;  // 32-bit division whenever it fits
        d.hg = uniform(rel < (1ll << 32) ? (int)((unsigned)rel / (unsigned)d.n_i) : (int)(rel / d.n_i));
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
            d.slot = dec::partial_slot(a0, si * NHG + d.hg);
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
            if constexpr (C::VPB == 16)
                vr[v] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, vrow, 0);
            else
                vr[v] = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, vrow, 0);
        }
    };
    auto head_base = [&](const void *cache, int hg) {
        return (const char *)cache + (int64_t)(hg * HPG + w) * D * C::EB;
    };

    dec::IssuePriority prio((int)(a1 - a0));  // blocks of this wave

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
        bool merged = false;
        for (int k = 0; k < ndef; ++k) {
            if (!sm.def_last[k])
                continue;
            if (merged)
                __syncthreads();  // the previous merge has read its scratch
            merged = true;
            dec::merge_partials<HG, D, NT, MB, HG_FOLD ? NCV : 0>(a.ws_ml, a.ws_acc, sm.def_lo[k], sm.def_np[k],
                                               a.out + sm.def_out[k], a.v_scale, tid, sm.merge);
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
    Seg sg = describe(item, i, base_i, uniform(sm.range.len));  // the scan read the length
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
            prio.step();

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
                    for (int j = 0; j < ROUNDS; ++j)
                        xs[j][s] = dec::dot_chunk<CDT, QW>(qc, kr[j][c], xs[j][s]);
                }
            }
            float sc[ROUNDS];
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j) {
                const float s2 = dec::reduce_scatter<LPT, GP>(xs[j]) * a.qk_scale;
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
                dec::widen_v<CDT, EV>(vv, ve);
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
        // Up to four heads per KV head the accumulators are summed over rows
        // by fold_totals (register k of a lane in row r then holds element
        // j = r * Q + k, j = h * EV + e, and the record keeps that folded
        // order); with more heads the per-element sums leave every lane of a
        // row with all totals (the fold's registers do not fit there).
        const float ls = dec::token_total<LPT>(lane_owner ? lsum : 0.f);
        constexpr int Q = HG_FOLD ? G * EV / 4 : 1;
        float tot[Q];
        if constexpr (HG_FOLD) {
            dec::fold_totals<G, EV, VTPR>(acc, tot);
        } else {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < EV; ++e)
                    acc[h][e] = dec::piece_total<VTPR>(acc[h][e]);
        }
        if (lane < 16 && tr == 0 && lane_owner)
            sm.lsum[w][lane_m] = ls;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float Lh[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
            Lh[h] = sm.lsum[w][h];
        const int pc = lane & 15, rw = lane >> 4;
        if (direct) {
            if constexpr (HG_FOLD) {
                if (pc < NCV) {
#pragma unroll
                    for (int k = 0; k < Q; ++k) {
                        const int j = rw * Q + k, h = j / EV, e = j - h * EV;
                        a.out[((int64_t)i * Hq + g * G + h) * D + pc * EV + e] = tot[k] * (a.v_scale / Lh[h]);
                    }
                }
            } else if (lane < NCV) {
                // lanes < NCV hold piece `lane` (EV elements) of every head's row
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
            if constexpr (HG_FOLD) {
                // element (h, e) of piece p at h * D + e * NCV + p
                if (pc < NCV) {
#pragma unroll
                    for (int k = 0; k < Q; ++k)
                        coherent_store(&a.ws_acc[(rec * G) * D + (rw * Q + k) * NCV + pc], tot[k]);
                }
            } else if (lane < NCV) {
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
                dec::partial_slot_range(base_i + (long long)hg * n_i, n_i, R, 0, pair, lo, hi);
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
