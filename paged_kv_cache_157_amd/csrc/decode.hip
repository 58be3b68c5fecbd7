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
//     persistent grid of work-groups takes equal contiguous ranges of the
//     list, so a 32k-token sequence is spread over many CUs as evenly as a
//     batch of short ones.  A run of items of one (sequence, KV head) inside
//     a range is a "segment".  A segment that covers its whole sequence
//     writes the output directly; otherwise it writes a partial
//     (max, sum, unnormalised accumulator) and a second kernel merges them.
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
    static constexpr int WAVES = 4;
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

// Sum of a value over the 64 lanes that share a "column" pattern: lanes that
// differ only in the row (bits 4-5) and in the bits selected by the pattern.
__device__ __forceinline__ float sum_rows(float v)
{
    v += __shfl_xor(v, 32);
    v += __shfl_xor(v, 16);
    return v;
}

struct SegInfo {
    int i, g;
    int b0, b1;      // block range
    int slot;
    int first, last;
};

template <int CDT, int D, int G>
struct DecodeSmem {
    using C = DecodeCfg<CDT, D, G>;
    float p[C::WAVES][16][8];       // probabilities of the current block
    float bmax[C::WAVES][4][8];     // row maxima (rescale path)
    float acc[C::WAVES][G][D];      // per-wave accumulators at a segment end
    float msum[C::WAVES][2][8];     // per-wave running max and sum
    long long scan[256];
    int seg_i, seg_x;
    long long seg_base;
};

template <int CDT, int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a)
{
    using C = DecodeCfg<CDT, D, G>;
    constexpr int LPT = C::LPT, GP = C::GP, CPL = C::CPL, ROUNDS = C::ROUNDS;
    constexpr int NC = C::NC, E = C::E, VTPR = C::VTPR, VPASS = C::VPASS, QW = C::QW;
    constexpr float TAU = 8.0f;
    __shared__ DecodeSmem<CDT, D, G> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int S = a.num_seqs, Hkv = a.num_kv_heads, Hq = a.num_q_heads, maxB = a.max_blocks;
    const int PB = a.part_blocks;

    auto items_of = [&](int L) -> int {
        L = L < 0 ? 0 : L;
        int nb = (L + 15) >> 4;
        nb = nb > maxB ? maxB : nb;
        return PB > 0 ? (nb + PB - 1) / PB : nb;
    };

    // ---- total item count and this work-group's range --------------------
    long long part = 0;
    for (int i = tid; i < S; i += 256)
        part += items_of(a.context_lens[i]);
    sm.scan[tid] = part;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s)
            sm.scan[tid] += sm.scan[tid + s];
        __syncthreads();
    }
    const long long total = sm.scan[0] * Hkv;
    __syncthreads();
    const long long a0 = total * blockIdx.x / gridDim.x;
    const long long a1 = total * (blockIdx.x + 1) / gridDim.x;
    if (a0 >= a1)
        return;

    // ---- locate the sequence holding item a0 (chunked inclusive scan) ----
    if (tid == 0)
        sm.seg_i = -1;
    long long carry = 0;
    for (int base = 0; base < S; base += 256) {
        const int i = base + tid;
        const long long v = i < S ? (long long)items_of(a.context_lens[i]) * Hkv : 0;
        __syncthreads();
        sm.scan[tid] = v;
        __syncthreads();
        for (int s = 1; s < 256; s <<= 1) {
            long long t = tid >= s ? sm.scan[tid - s] : 0;
            __syncthreads();
            sm.scan[tid] += t;
            __syncthreads();
        }
        const long long incl = carry + sm.scan[tid];
        const long long excl = incl - v;
        if (i < S && v > 0 && excl <= a0 && a0 < incl) {
            sm.seg_i = i;
            sm.seg_base = excl;
        }
        carry += sm.scan[255];
        __syncthreads();
        if (sm.seg_i >= 0)
            break;
    }
    int i = uniform(sm.seg_i);
    if (i < 0)  // unreachable while a0 < total; keeps every index in range
        return;
    long long base_i = sm.seg_base;  // first item index of sequence i
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
    const int64_t nslots = a.num_blocks;

    // per-lane byte offsets of K and V chunks inside one block (KV head 0)
    int koff[ROUNDS][CPL];
#pragma unroll
    for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            koff[j][c] = (int)(row_token<LPT>(row, tr + j * C::TRN) * tok_bytes) +
                         (gl + c * LPT) * 16;
    int voff[VPASS];
#pragma unroll
    for (int v = 0; v < VPASS; ++v)
        voff[v] = (int)(row_token<LPT>(row, v * VTPR + vh) * tok_bytes) + vc * 16;

    while (item < a1) {
        // ---- next segment ------------------------------------------------
        int L = a.context_lens[i];
        int n_i = items_of(L);
        while (n_i == 0) {  // cannot happen for the first segment; skip empties
            ++i;
            L = a.context_lens[i];
            n_i = items_of(L);
        }
        L = L > maxB * 16 ? maxB * 16 : L;
        const long long rel = item - base_i;
        const int g = (int)(rel / n_i);
        const int x = (int)(rel - (long long)g * n_i);
        const int nblk = (L + 15) >> 4;
        int seg_items, b0, b1, slot;
        if (PB > 0) {
            seg_items = 1;
            b0 = x * PB;
            b1 = b0 + PB < nblk ? b0 + PB : nblk;
            slot = (int)item;
        } else {
            const long long left = a1 - item;
            seg_items = (int)((long long)(n_i - x) < left ? (n_i - x) : left);
            b0 = x;
            b1 = x + seg_items;
            // rank of this work-group among those with a non-empty range: with at
            // least as many items as work-groups every range is non-empty (rank =
            // blockIdx.x); with fewer, each non-empty range holds one item (rank =
            // a0).  Ranks keep the partial slots of one (sequence, head) contiguous.
            slot = (int)(a0 < (long long)blockIdx.x ? a0 : (long long)blockIdx.x) + i * Hkv + g;
        }
        const bool first = x == 0;
        const bool last = x + seg_items == n_i;
        const bool direct = first && last;

        // ---- load q for this (sequence, KV head) --------------------------
        uint32_t qr[GP][CPL][QW];
        {
            const int hq0 = g * G;
#pragma unroll
            for (int s = 0; s < GP; ++s) {
                const int h = s ^ lane_m;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int chunk = gl + c * LPT;
                    if (h < G) {
                        const char *qp = (const char *)a.q;
                        if constexpr (CDT == DT_F32) {
                            const u32x4 t = *(const u32x4 *)(qp + (((int64_t)i * Hq + hq0 + h) * D +
                                                                   chunk * E) * 4);
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                qr[s][c][k] = t[k];
                        } else {
                            const u32x4 *t = (const u32x4 *)(qp + (((int64_t)i * Hq + hq0 + h) * D +
                                                                   chunk * E) * 2);
#pragma unroll
                            for (int k = 0; k < QW / 4; ++k) {
                                const u32x4 u = t[k];
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    qr[s][c][4 * k + e] = u[e];
                            }
                        }
                    } else {
#pragma unroll
                        for (int k = 0; k < QW; ++k)
                            qr[s][c][k] = 0;
                    }
                }
            }
        }

        // ---- per-wave streaming softmax over blocks b0+w, b0+w+4, ... -----
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

        const int32_t *table = a.block_tables + (int64_t)i * maxB;
        const char *kbase = (const char *)a.k_cache + (int64_t)g * D * C::EB;
        const char *vbase = (const char *)a.v_cache + (int64_t)g * D * C::EB;

        u32x4 kb[ROUNDS][CPL], vb[VPASS];
        auto load_block = [&](int b, u32x4 (&kd)[ROUNDS][CPL], u32x4 (&vd)[VPASS]) {
            int pb = table[b];
            pb = (unsigned)pb < (unsigned)nslots ? pb : 0;
            const char *kp = kbase + (int64_t)pb * blk_bytes;
            const char *vp = vbase + (int64_t)pb * blk_bytes;
#pragma unroll
            for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    kd[j][c] = *(const u32x4 *)(kp + koff[j][c]);
#pragma unroll
            for (int v = 0; v < VPASS; ++v)
                vd[v] = *(const u32x4 *)(vp + voff[v]);
        };

        int b = b0 + w;
        if (b < b1)
            load_block(b, kb, vb);
        for (; b < b1; b += C::WAVES) {
            u32x4 kn[ROUNDS][CPL], vn[VPASS];
            const bool has_next = b + C::WAVES < b1;
            if (has_next)
                load_block(b + C::WAVES, kn, vn);

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
                    if constexpr (CDT == DT_BF16) {
#pragma unroll
                        for (int s = 0; s < GP; ++s)
#pragma unroll
                            for (int p = 0; p < 4; ++p)
                                xs[s] = dot2_bf16(qr[s][c][p], kb[j][c][p], xs[s]);
                    } else if constexpr (CDT == DT_FP8) {
                        uint32_t kk[8];
#pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            kk[2 * p] = fp8x2_to_bf16x2<false>(kb[j][c][p]);
                            kk[2 * p + 1] = fp8x2_to_bf16x2<true>(kb[j][c][p]);
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
                                xs[s] = fmaf(__uint_as_float(qr[s][c][p]),
                                             __uint_as_float(kb[j][c][p]), xs[s]);
                    }
                }
                const float s2 = reduce_scatter<LPT, GP>(xs) * a.qk_scale;
                const int t = tbase + row_token<LPT>(row, tr + j * C::TRN);
                sc[j] = t < L ? s2 : -INFINITY;
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
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
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
            const bool partial = tbase + 16 > L;
#pragma unroll
            for (int v = 0; v < VPASS; ++v) {
                const int tk = row_token<LPT>(row, v * VTPR + vh);
                u32x4 vv = vb[v];
                if (partial && tbase + tk >= L)
                    vv = u32x4{0u, 0u, 0u, 0u};
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
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();

            if (has_next) {
#pragma unroll
                for (int j = 0; j < ROUNDS; ++j)
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
                        kb[j][c] = kn[j][c];
#pragma unroll
                for (int v = 0; v < VPASS; ++v)
                    vb[v] = vn[v];
            }
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
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    sm.acc[w][h][lane * E + e] = acc[h][e];
        }
        if (lane < 16 && tr == 0 && lane_owner)
            sm.msum[w][1][lane_m] = ls;
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
                sm.msum[w][0][h] = mref[h];
        }
        __syncthreads();

        // ---- merge the four waves; write output or a partial --------------
        for (int e = tid; e < G * D; e += 256) {
            const int h = e / D, c = e - h * D;
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < C::WAVES; ++ww)
                M = fmaxf(M, sm.msum[ww][0][h]);
            float A = 0.f, Ls = 0.f;
#pragma unroll
            for (int ww = 0; ww < C::WAVES; ++ww) {
                const float m = sm.msum[ww][0][h];
                const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
                A += f * sm.acc[ww][h][c];
                Ls += f * sm.msum[ww][1][h];
            }
            if (direct) {
                a.out[((int64_t)i * Hq + g * G + h) * D + c] = A / Ls * a.v_scale;
            } else {
                a.ws_acc[((int64_t)slot * G + h) * D + c] = A;
                if (c == 0) {
                    a.ws_ml[((int64_t)slot * G + h) * 2 + 0] = M;
                    a.ws_ml[((int64_t)slot * G + h) * 2 + 1] = Ls;
                }
            }
        }
        if (tid == 0) {
            if (first)
                a.ws_lohi[((int64_t)i * Hkv + g) * 2 + 0] = slot;
            if (last)
                a.ws_lohi[((int64_t)i * Hkv + g) * 2 + 1] = slot;
        }
        __syncthreads();

        // ---- advance ----------------------------------------------------------
        item += seg_items;
        if (last && g == Hkv - 1) {
            base_i += (long long)n_i * Hkv;
            ++i;
        }
    }
}

// Merge the partial results of every (sequence, KV head) that was split.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a)
{
    const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
    const int i = blockIdx.x / Hkv, g = blockIdx.x - (blockIdx.x / Hkv) * Hkv;
    const int L = a.context_lens[i];
    float *out = a.out + ((int64_t)i * Hq + g * G) * D;
    if (L <= 0) {
        for (int e = threadIdx.x; e < G * D; e += 256)
            out[e] = 0.f;
        return;
    }
    const int lo = a.ws_lohi[((int64_t)i * Hkv + g) * 2 + 0];
    const int hi = a.ws_lohi[((int64_t)i * Hkv + g) * 2 + 1];
    if (lo == hi)
        return;
    for (int e = threadIdx.x; e < G * D; e += 256) {
        const int h = e / D, c = e - h * D;
        float M = -INFINITY;
        for (int s = lo; s <= hi; ++s)
            M = fmaxf(M, a.ws_ml[((int64_t)s * G + h) * 2]);
        float num = 0.f, den = 0.f;
        for (int s = lo; s <= hi; ++s) {
            const float m = a.ws_ml[((int64_t)s * G + h) * 2];
            const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
            num += f * a.ws_acc[((int64_t)s * G + h) * D + c];
            den += f * a.ws_ml[((int64_t)s * G + h) * 2 + 1];
        }
        out[e] = num / den * a.v_scale;
    }
}

int64_t decode_partial_slots(int num_seqs, int num_kv_heads, int max_blocks, int part_blocks,
                             int grid)
{
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    if (part_blocks > 0)
        return pairs * ((max_blocks + part_blocks - 1) / part_blocks);
    return (int64_t)grid + pairs;
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
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream)
{
    decode_kernel<CDT, D, G><<<a.grid, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    decode_reduce_kernel<D, G><<<a.num_seqs * a.num_kv_heads, 256, 0, stream>>>(a);
    return hipGetLastError();
}

template <int CDT, int D>
static hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t stream)
{
    switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_t<CDT, D, 1>(a, stream);
    case 2: return launch_decode_t<CDT, D, 2>(a, stream);
    case 3: return launch_decode_t<CDT, D, 3>(a, stream);
    case 4: return launch_decode_t<CDT, D, 4>(a, stream);
    case 5: return launch_decode_t<CDT, D, 5>(a, stream);
    case 6: return launch_decode_t<CDT, D, 6>(a, stream);
    case 7: return launch_decode_t<CDT, D, 7>(a, stream);
    default: return launch_decode_t<CDT, D, 8>(a, stream);
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.cache_dtype == DT_F32)
        return launch_decode_d<DT_F32, 64>(a, stream);
    if (a.cache_dtype == DT_BF16)
        return a.head_dim == 64 ? launch_decode_d<DT_BF16, 64>(a, stream)
                                : launch_decode_d<DT_BF16, 128>(a, stream);
    if (a.head_dim == 64) {
        switch (a.num_q_heads / a.num_kv_heads) {
        case 1: return launch_decode_t<DT_FP8, 64, 1>(a, stream);
        case 2: return launch_decode_t<DT_FP8, 64, 2>(a, stream);
        case 3: return launch_decode_t<DT_FP8, 64, 3>(a, stream);
        default: return launch_decode_t<DT_FP8, 64, 4>(a, stream);
        }
    }
    return launch_decode_d<DT_FP8, 128>(a, stream);
}

}  // namespace pa
