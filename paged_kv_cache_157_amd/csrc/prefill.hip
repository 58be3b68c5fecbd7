// prefill.hip -- chunked-prefill attention over a paged history.
//
// What is computed ("Lecture 33" §4.2): a prompt chunk of n rows, written to
// the cache before the call, attends to everything cached before it (the
// earlier chunks, read through the block table) and causally to itself:
// row j of a request with C cached tokens attends keys [0, C - n + j].
//
// Here the query tile makes QK^T a dense contraction, so it runs on the
// matrix cores (v_mfma_f32_32x32x16_bf16):
//   * A work-group (4 waves) owns 128 "query rows" = (position, head) pairs of
//     one KV head (all G heads of a position are adjacent, so one K/V tile
//     feeds every head of the group), and one slice of the key range.
//   * Per 64-key tile, K and V rows are gathered through the block table into
//     LDS (fp8 caches are widened to bf16 there, exactly).  K keeps its row
//     layout; V is transposed to [d][key] so that keys are contiguous for the
//     PV contraction, with keys of each 16-key step stored in the order the
//     probabilities come out of the QK product.
//   * S^T = K Q^T puts one query row per lane (column of the MFMA result),
//     so the row maximum and sum are in-lane plus one exchange between the two
//     half-waves.  The probabilities are split into a bf16 head and a bf16
//     tail (together exact to about 2^-16) and both are multiplied with V on
//     the matrix cores (O = P V); a single bf16 rounding of P would cost up to
//     2^-8 relative weight error, too coarse for rows with few keys.
//   * The running maximum is raised only when a tile exceeds it by more than
//     8 (base 2); that rare path rescales the accumulators through LDS.
//   * When the key range is split over several work-groups, each writes
//     (max, sum, unnormalised O) and a second kernel merges them.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 pair -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    a += 0x7FFFu + ((a >> 16) & 1u);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (a >> 16) | (b & 0xFFFF0000u);
}

template <int D>
struct PrefillCfg {
    static constexpr int KT = 64;            // keys per tile
    static constexpr int MROWS = 128;        // query rows per work-group
    static constexpr int KSTR = D + 8;       // bf16 per K row in LDS (padded)
    static constexpr int VSTR = KT + 8;      // bf16 per V^T row in LDS (padded)
    static constexpr int DCH = D / 8;        // 16-byte chunks per row
};

template <int D>
struct PrefillSmem {
    using C = PrefillCfg<D>;
    uint16_t k[C::KT * C::KSTR];
    uint16_t vt[D * C::VSTR];
    float alpha[4][32];
    float ml[4][2][32];
};

// Position of key k (0..63) in a V^T row: inside each 16-key step the order is
// keys 0-3, 8-11, 4-7, 12-15, i.e. the order in which a lane half of the S^T
// result holds them.
__device__ __forceinline__ int vt_pos(int k)
{
    const int q = (k >> 2) & 3;
    const int perm = (q == 0) ? 0 : (q == 1) ? 8 : (q == 2) ? 4 : 12;
    return (k & ~15) + perm + (k & 3);
}

template <int CDT, int D>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a)
{
    using C = PrefillCfg<D>;
    constexpr int KT = C::KT, DCH = C::DCH;
    constexpr float TAU = 8.0f;
    __shared__ PrefillSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hl = lane >> 5, col = lane & 31;
    const int KS = a.kv_splits;
    const int r = blockIdx.z / KS, split = blockIdx.z - (blockIdx.z / KS) * KS;
    const int g = blockIdx.y;
    const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
    const int ppt = C::MROWS / G;  // positions per tile
    const int qs = a.query_start[r];
    const int n = a.query_start[r + 1] - qs;
    int Ctx = a.context_lens[r];
    Ctx = Ctx < 16 * a.max_blocks ? Ctx : 16 * a.max_blocks;  // caller precondition, enforced
    const int P = Ctx - n;
    const int pos0 = blockIdx.x * ppt;
    if (pos0 >= n)
        return;
    const int pos_end = pos0 + ppt < n ? pos0 + ppt : n;

    // this lane's query row (column of S^T)
    const int mrow = 32 * w + col;
    const int my_pos = pos0 + mrow / G;
    const int my_head = g * G + mrow % G;
    const bool row_ok = mrow < ppt * G && my_pos < pos_end;
    const int my_limit = P + my_pos;  // last key this row attends

    // key tiles of this split
    const int nkt = (Ctx + KT - 1) / KT;
    const int tps = (nkt + KS - 1) / KS;
    int t0 = split * tps;
    int t1 = t0 + tps < nkt ? t0 + tps : nkt;
    const int tile_limit = P + pos_end - 1;
    const int tmax = tile_limit / KT + 1;
    t1 = t1 < tmax ? t1 : tmax;

    // Q^T as the B operand: lane holds 8 consecutive d of its row per 16-d step
    u32x4 qb[D / 16];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)(qs + my_pos) * Hq + my_head) * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qb[s] = row_ok ? *(const u32x4 *)(qp + 16 * s + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = f32x16{};
    float mref = -INFINITY, lsum = 0.f;

    const int32_t *table = a.block_tables + (int64_t)r * a.max_blocks;
    constexpr int EB = Storage<CDT>::bytes;
    const int64_t tok_bytes = (int64_t)Hkv * D * EB;
    const char *kbase = (const char *)a.k_cache + (int64_t)g * D * EB;
    const char *vbase = (const char *)a.v_cache + (int64_t)g * D * EB;

    for (int kt = t0; kt < t1; ++kt) {
        // ---- gather the K tile: thread -> (key, 16-byte chunk of bf16) -------
        for (int e = tid; e < KT * DCH; e += 256) {
            const int key = e / DCH, ch = e - (e / DCH) * DCH;
            const int kabs = kt * KT + key;
            u32x4 val = u32x4{0u, 0u, 0u, 0u};
            if (kabs < Ctx) {
                int pb = table[kabs >> 4];
                pb = (unsigned)pb < (unsigned)a.num_blocks ? pb : 0;
                const char *src = kbase + ((int64_t)pb * 16 + (kabs & 15)) * tok_bytes;
                if constexpr (CDT == DT_BF16) {
                    val = *(const u32x4 *)(src + ch * 16);
                } else {
                    const u32x2 f8 = *(const u32x2 *)(src + ch * 8);
                    val = u32x4{fp8x2_to_bf16x2<false>(f8[0]), fp8x2_to_bf16x2<true>(f8[0]),
                                fp8x2_to_bf16x2<false>(f8[1]), fp8x2_to_bf16x2<true>(f8[1])};
                }
            }
            *(u32x4 *)&sm.k[key * C::KSTR + ch * 8] = val;
        }
        // ---- gather the V tile transposed: thread -> (4 keys, 8 d) ----------
        for (int e = tid; e < (KT / 4) * DCH; e += 256) {
            const int quad = e % (KT / 4), ch = e / (KT / 4);
            uint32_t rows[4][4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int kabs = kt * KT + quad * 4 + kk;
                u32x4 val = u32x4{0u, 0u, 0u, 0u};
                if (kabs < Ctx) {
                    int pb = table[kabs >> 4];
                    pb = (unsigned)pb < (unsigned)a.num_blocks ? pb : 0;
                    const char *src = vbase + ((int64_t)pb * 16 + (kabs & 15)) * tok_bytes;
                    if constexpr (CDT == DT_BF16) {
                        val = *(const u32x4 *)(src + ch * 16);
                    } else {
                        const u32x2 f8 = *(const u32x2 *)(src + ch * 8);
                        val = u32x4{fp8x2_to_bf16x2<false>(f8[0]), fp8x2_to_bf16x2<true>(f8[0]),
                                    fp8x2_to_bf16x2<false>(f8[1]), fp8x2_to_bf16x2<true>(f8[1])};
                    }
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    rows[kk][x] = val[x];
            }
            const int pos = vt_pos(quad * 4);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                // d = ch*8 + 2x (low halves) and ch*8 + 2x + 1 (high halves)
                const uint32_t lo01 = __builtin_amdgcn_perm(rows[1][x], rows[0][x], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(rows[3][x], rows[2][x], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(rows[1][x], rows[0][x], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(rows[3][x], rows[2][x], 0x07060302u);
                *(u32x2 *)&sm.vt[(ch * 8 + 2 * x) * C::VSTR + pos] = u32x2{lo01, lo23};
                *(u32x2 *)&sm.vt[(ch * 8 + 2 * x + 1) * C::VSTR + pos] = u32x2{hi01, hi23};
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T: two 32-key halves ------------------------------------
        f32x16 s[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            s[kc] = f32x16{};
#pragma unroll
            for (int st = 0; st < D / 16; ++st) {
                const u32x4 ka = *(const u32x4 *)&sm.k[(32 * kc + col) * C::KSTR + 16 * st + 8 * hl];
                s[kc] = mfma32(ka, qb[st], s[kc]);
            }
        }
        // scale, mask, tile maximum of this lane's row
        float tmax_row = -INFINITY;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kt * KT + 32 * kc + 8 * (i >> 2) + 4 * hl + (i & 3);
                const float v = s[kc][i] * a.qk_scale;
                s[kc][i] = (row_ok && key <= my_limit) ? v : -INFINITY;
                tmax_row = fmaxf(tmax_row, s[kc][i]);
            }
        tmax_row = fmaxf(tmax_row, __shfl_xor(tmax_row, 32));

        if (wave_any(tmax_row > mref + TAU)) {
            const float mnew = fmaxf(mref, tmax_row);
            const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(mref - mnew);
            lsum *= alpha;
            mref = mnew;
            if (hl == 0)
                sm.alpha[w][col] = alpha;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float al = sm.alpha[w][8 * (i >> 2) + 4 * hl + (i & 3)];
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
                    o[dt][i] *= al;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }

        // ---- probabilities and O += P V --------------------------------------------
        // P is split into a bf16 head and a bf16 tail (p = hi + lo to ~2^-16), so
        // the PV product keeps close to fp32 weights; both parts meet the same V.
        // a row with no valid key yet keeps mref = -inf: its probabilities are 0
        const float m_use = mref == -INFINITY ? 0.f : mref;
        u32x4 p_hi[4], p_lo[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kc = ks >> 1, base = 8 * (ks & 1);
            float p[8], r[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                p[j] = fast_exp2(s[kc][base + j] - m_use);
                lsum += p[j];
            }
            p_hi[ks] = u32x4{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                             pack_bf16(p[6], p[7])};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                r[2 * j] = p[2 * j] - bf16_lo(p_hi[ks][j]);
                r[2 * j + 1] = p[2 * j + 1] - bf16_hi(p_hi[ks][j]);
            }
            p_lo[ks] = u32x4{pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3]), pack_bf16(r[4], r[5]),
                             pack_bf16(r[6], r[7])};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const u32x4 vb =
                    *(const u32x4 *)&sm.vt[(32 * dt + col) * C::VSTR + 16 * ks + 8 * hl];
                o[dt] = mfma32(p_hi[ks], vb, o[dt]);
                o[dt] = mfma32(p_lo[ks], vb, o[dt]);
            }
        __syncthreads();
    }

    // ---- finish: row sums, then normalise or store a partial ------------------
    lsum += __shfl_xor(lsum, 32);
    if (hl == 0) {
        sm.ml[w][0][col] = mref;
        sm.ml[w][1][col] = lsum;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int orow = 8 * (i >> 2) + 4 * hl + (i & 3);
        const int mr = 32 * w + orow;
        const int pos = pos0 + mr / G;
        if (mr >= ppt * G || pos >= pos_end)
            continue;
        const int head = g * G + mr % G;
        const int64_t qrow = (int64_t)(qs + pos) * Hq + head;
        const float m = sm.ml[w][0][orow], l = sm.ml[w][1][orow];
        if (KS == 1) {
            const float inv = a.v_scale / l;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                a.out[qrow * D + 32 * dt + col] = o[dt][i] * inv;
        } else {
            float *dst = a.ws_acc + ((int64_t)split * a.total_rows * Hq + qrow) * D;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                dst[32 * dt + col] = o[dt][i];
            if (col == 0) {
                float *ml = a.ws_ml + ((int64_t)split * a.total_rows * Hq + qrow) * 2;
                ml[0] = m;
                ml[1] = l;
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillArgs a)
{
    const int64_t rows = a.total_rows * a.num_q_heads;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows * D)
        return;
    const int64_t qrow = e / D;
    const int KS = a.kv_splits;
    const int64_t stride = rows;
    float M = -INFINITY;
    for (int s = 0; s < KS; ++s)
        M = fmaxf(M, a.ws_ml[(s * stride + qrow) * 2]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < KS; ++s) {
        const float m = a.ws_ml[(s * stride + qrow) * 2];
        const float f = m == -INFINITY ? 0.f : fast_exp2(m - M);
        num += f * a.ws_acc[(s * stride) * D + e];
        den += f * a.ws_ml[(s * stride + qrow) * 2 + 1];
    }
    a.out[e] = num / den * a.v_scale;
}

bool prefill_supported(int cache_dtype, int head_dim, int group)
{
    return (cache_dtype == DT_BF16 || cache_dtype == DT_FP8) && (head_dim == 64 || head_dim == 128) &&
           group >= 1 && group <= 8;
}

int prefill_kv_splits(int64_t total_rows, int num_q_heads)
{
    // aim at roughly two work-groups per CU of a 256-CU device
    const int64_t tiles = (total_rows * num_q_heads + 127) / 128;
    int64_t ks = tiles > 0 ? 512 / tiles : 1;
    if (ks < 1)
        ks = 1;
    if (ks > 16)
        ks = 16;
    return (int)ks;
}

template <int CDT, int D>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    const int G = a.num_q_heads / a.num_kv_heads;
    const int ppt = 128 / G;
    const unsigned tiles = (unsigned)((a.total_rows + ppt - 1) / ppt);
    dim3 grid(tiles, a.num_kv_heads, a.num_reqs * a.kv_splits);
    prefill_kernel<CDT, D><<<grid, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.kv_splits == 1)
        return e;
    const int64_t n = a.total_rows * a.num_q_heads * D;
    prefill_reduce_kernel<D><<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream)
{
    if (a.cache_dtype == DT_BF16)
        return a.head_dim == 64 ? launch_prefill_t<DT_BF16, 64>(a, stream)
                                : launch_prefill_t<DT_BF16, 128>(a, stream);
    return a.head_dim == 64 ? launch_prefill_t<DT_FP8, 64>(a, stream)
                            : launch_prefill_t<DT_FP8, 128>(a, stream);
}

}  // namespace pa
