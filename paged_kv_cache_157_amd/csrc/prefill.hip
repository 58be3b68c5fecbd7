// prefill.hip -- chunked-prefill attention over a paged history.
//
// What is computed ("Lecture 33" §4.2): a prompt chunk of n rows, written to
// the cache before the call, attends to everything cached before it (the
// earlier chunks, read through the block table) and causally to itself:
// row j of a request with C cached tokens attends keys [0, C - n + j].
//
// Here the query tile makes QK^T a dense contraction, so it runs on the
// matrix cores (v_mfma_f32_32x32x16_bf16):
//   * A work-group (8 waves, two per SIMD so that one wave's softmax overlaps
//     the other's matrix products) owns 256 "query rows" = (position, head)
//     pairs of one KV head (all G heads of a position are adjacent, so one K/V
//     tile feeds every head of the group), and one slice of the key range.
//     Each wave holds one 32-row MFMA block.
//   * Per 64-key tile, K and V rows are gathered through the block table.
//     The loads for tile t+1 are issued into registers before tile t is
//     computed and land in the other half of a double-buffered LDS tile
//     afterwards (fp8 caches are widened to bf16 there, exactly).  K is stored
//     in MFMA operand order: each (32-key half, 16-d step) fragment is 1 KiB
//     that the wave reads with one contiguous 16-byte-per-lane access.  V is
//     transposed to [d][key] so that keys are contiguous for the PV
//     contraction, with keys of each 16-key step stored in the order the
//     probabilities come out of the QK product.
//   * S^T = K Q^T puts one query row per lane (column of the MFMA result),
//     so the row maximum and sum are in-lane plus one exchange between the two
//     half-waves.  Masks are applied only on tiles that cross the causal
//     diagonal or the end of the context.  The probabilities are split into a
//     bf16 head and a bf16 tail (together exact to about 2^-16) and both are
//     multiplied with V on the matrix cores (O = P V); a single bf16 rounding
//     of P would cost up to 2^-8 relative weight error, too coarse for rows
//     with few keys.
//   * The running maximum is raised only when a tile exceeds it by more than
//     8 (base 2); that rare path rescales the accumulators through LDS.
//   * When the key range is split over several work-groups, each writes
//     (max, sum, unnormalised O) and a second kernel merges them.
//   * Work-groups that share a (request, KV head, key slice) are numbered
//     Hkv*splits apart, so when that product is a multiple of the XCD count
//     they run on one XCD and its L2 serves their common K/V tiles.
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

// fp32 pair -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

template <int D>
struct PrefillCfg {
    static constexpr int KT = 64;              // keys per tile
    static constexpr int WAVES = 8;            // two per SIMD
    static constexpr int MROWS = 32 * WAVES;   // query rows per work-group
    static constexpr int ST = D / 16;          // 16-d steps of the QK contraction
    static constexpr int NKF = 2 * ST;         // 1 KiB K fragments per tile
    static constexpr int KWAVES = WAVES / 2;   // waves that stage K (the others stage V)
    static constexpr int KCH = NKF / KWAVES;   // K fragments each K-staging wave loads
    static constexpr int NVI = (KT / 4) * (D / 8);  // V staging items (4 keys x 8 d)
    static constexpr int VSTR = KT + 8;        // bf16 per V^T row in LDS (padded)
    static_assert(NKF % KWAVES == 0 && NVI <= 64 * (WAVES - KWAVES), "tile shape");
};

template <int D>
struct PrefillSmem {
    using C = PrefillCfg<D>;
    // 16-byte alignment lets the compiler use ds_read_b128 / ds_write_b128
    __attribute__((aligned(16))) uint16_t k[2][C::KT * D];     // [buffer][fragment][lane][8]
    __attribute__((aligned(16))) uint16_t vt[2][D * C::VSTR];  // [buffer][d][key position]
    float alpha[C::WAVES][32];
    float ml[C::WAVES][2][32];      // [wave][max, sum][row]
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

// One 16-byte chunk (8 elements) of a cached row as loaded, and widened to bf16.
template <int CDT>
struct RawChunk {
    using T = u32x4;
};
template <>
struct RawChunk<DT_FP8> {
    using T = u32x2;
};

template <int CDT>
__device__ __forceinline__ typename RawChunk<CDT>::T load_chunk(const char *p)
{
    return *(const typename RawChunk<CDT>::T *)p;
}

__device__ __forceinline__ u32x4 widen(u32x4 x) { return x; }
__device__ __forceinline__ u32x4 widen(u32x2 x)
{
    return u32x4{fp8x2_to_bf16x2<false>(x[0]), fp8x2_to_bf16x2<true>(x[0]),
                 fp8x2_to_bf16x2<false>(x[1]), fp8x2_to_bf16x2<true>(x[1])};
}

template <int CDT, int D>
__global__ __launch_bounds__(64 * PrefillCfg<D>::WAVES) void prefill_kernel(PrefillArgs a)
{
    using C = PrefillCfg<D>;
    using Raw = typename RawChunk<CDT>::T;
    constexpr int KT = C::KT, ST = C::ST, VSTR = C::VSTR;
    constexpr int EB = Storage<CDT>::bytes;
    constexpr float TAU = 8.0f;
    __shared__ PrefillSmem<D> sm;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int hl = lane >> 5, col = lane & 31;
    const int KS = a.kv_splits, Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = Hq / Hkv;
    int b = blockIdx.x;
    const int split = b % KS;
    b /= KS;
    const int g = b % Hkv;
    const int mt = b / Hkv;
    const int r = blockIdx.y;
    const int ppt = C::MROWS / G;  // positions per tile

    const int qs = a.query_start[r];
    int n = a.query_start[r + 1] - qs;
    if (qs < 0 || qs > a.total_rows)  // caller precondition; never write outside out
        return;
    n = n < a.total_rows - qs ? n : (int)(a.total_rows - qs);
    int Ctx = a.context_lens[r];
    Ctx = Ctx < 16 * a.max_blocks ? Ctx : 16 * a.max_blocks;  // caller precondition, enforced
    const int P = Ctx - n;
    const int pos0 = mt * ppt;
    if (pos0 >= n)
        return;
    const int pos_end = pos0 + ppt < n ? pos0 + ppt : n;

    // this lane's query row (column of S^T) and its Q^T fragments
    const int mrow = 32 * w + col;
    const int my_pos = pos0 + mrow / G;
    const int my_head = g * G + mrow % G;
    const bool row_ok = mrow < ppt * G && my_pos < pos_end;
    const int lim = row_ok ? P + my_pos : -1;  // last key this row attends
    u32x4 qb[ST];
    {
        const uint16_t *qp = (const uint16_t *)a.q + ((int64_t)(qs + my_pos) * Hq + my_head) * D;
#pragma unroll
        for (int s = 0; s < ST; ++s)
            qb[s] = row_ok ? *(const u32x4 *)(qp + 16 * s + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
    }

    // key tiles of this split
    const int nkt = (Ctx + KT - 1) / KT;
    const int tps = (nkt + KS - 1) / KS;
    const int t0 = split * tps;
    int t1 = t0 + tps < nkt ? t0 + tps : nkt;
    const int tmax = (P + pos_end - 1) / KT + 1;
    t1 = t1 < tmax ? t1 : tmax;

    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        o[dt] = f32x16{};
    float mref = -INFINITY, lsum = 0.f;

    const auto tab = scalar_view(a.block_tables + (int64_t)r * a.max_blocks);
    const int64_t tok_bytes = (int64_t)Hkv * D * EB;
    const char *kbase = (const char *)a.k_cache + (int64_t)g * D * EB;
    const char *vbase = (const char *)a.v_cache + (int64_t)g * D * EB;
    const float c = a.qk_scale;

    // ---- staging: tile kt -> registers -> LDS buffer --------------------------
    // Waves [KWAVES, WAVES) gather K fragments, the others gather V (4 keys x 8 d
    // per thread); either way a thread holds four 16-byte chunks in flight.
    const bool kstager = w >= C::KWAVES;
    Raw stg[4];
    auto issue_loads = [&](int kt) {
        int pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = kt * (KT / 16) + i;
            int e = 0;
            if (blk * 16 < Ctx)  // entries past the context are never read
                e = tab[blk];
            pb[i] = (unsigned)e < (unsigned)a.num_blocks ? e : 0;
        }
        if (kstager) {
#pragma unroll
            for (int j = 0; j < C::KCH; ++j) {
                const int f = (w - C::KWAVES) + C::KWAVES * j;  // (key half, d step)
                const int key = (f / ST) * 32 + col;
                const int ch = 2 * (f % ST) + hl;
                const int kb = key >> 4;
                const int p = kb == 0 ? pb[0] : kb == 1 ? pb[1] : kb == 2 ? pb[2] : pb[3];
                stg[j] = load_chunk<CDT>(kbase + ((int64_t)p * 16 + (key & 15)) * tok_bytes +
                                         ch * 8 * EB);
            }
        } else if (tid < C::NVI) {
            const int quad = tid & 15, vch = tid >> 4;
            const int kb = quad >> 2;
            const int p = kb == 0 ? pb[0] : kb == 1 ? pb[1] : kb == 2 ? pb[2] : pb[3];
            const char *src = vbase + ((int64_t)p * 16 + 4 * (quad & 3)) * tok_bytes + vch * 8 * EB;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                stg[kk] = load_chunk<CDT>(src + kk * tok_bytes);
        }
        // keep the loads ahead of the compute that follows
        asm volatile("" ::: "memory");
    };
    auto write_stage = [&](int bi, int kt) {
        if (kstager) {
#pragma unroll
            for (int j = 0; j < C::KCH; ++j) {
                const int f = (w - C::KWAVES) + C::KWAVES * j;
                *(u32x4 *)&sm.k[bi][(f * 64 + lane) * 8] = widen(stg[j]);
            }
        } else if (tid < C::NVI) {
            const int quad = tid & 15, vch = tid >> 4;
            u32x4 rows[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                // V rows past the context are zero (0 * garbage must not reach O)
                const bool ok = kt * KT + 4 * quad + kk < Ctx;
                rows[kk] = ok ? widen(stg[kk]) : u32x4{0u, 0u, 0u, 0u};
            }
            const int pos = vt_pos(4 * quad);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                // d = vch*8 + 2x (low halves) and vch*8 + 2x + 1 (high halves)
                const uint32_t lo01 = __builtin_amdgcn_perm(rows[1][x], rows[0][x], 0x05040100u);
                const uint32_t lo23 = __builtin_amdgcn_perm(rows[3][x], rows[2][x], 0x05040100u);
                const uint32_t hi01 = __builtin_amdgcn_perm(rows[1][x], rows[0][x], 0x07060302u);
                const uint32_t hi23 = __builtin_amdgcn_perm(rows[3][x], rows[2][x], 0x07060302u);
                *(u32x2 *)&sm.vt[bi][(vch * 8 + 2 * x) * VSTR + pos] = u32x2{lo01, lo23};
                *(u32x2 *)&sm.vt[bi][(vch * 8 + 2 * x + 1) * VSTR + pos] = u32x2{hi01, hi23};
            }
        }
    };

    if (t0 < t1) {
        issue_loads(t0);
        write_stage(0, t0);
        __syncthreads();
    }
    for (int kt = t0; kt < t1; ++kt) {
        const int bi = (kt - t0) & 1;
        if (kt + 1 < t1)
            issue_loads(kt + 1);

        const int key0 = kt * KT;
        const bool full = key0 + KT <= Ctx && key0 + KT - 1 <= P + pos0;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
            // ---- S^T = K Q^T for one 32-key half ------------------------------------
            f32x16 s = f32x16{};
#pragma unroll
            for (int st = 0; st < ST; ++st) {
                const u32x4 ka = *(const u32x4 *)&sm.k[bi][((kc * ST + st) * 64 + lane) * 8];
                s = mfma32(ka, qb[st], s);
            }

            // ---- mask (diagonal / ragged tiles only), row maximum, lazy rescale ----
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 32 * kc + 8 * (i >> 2) + 4 * hl + (i & 3);
                    s[i] = key <= lim ? s[i] : -INFINITY;
                }
            }
            float tm = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                tm = fmaxf(tm, s[i]);
            tm = fmaxf(tm, __shfl_xor(tm, 32)) * c;  // c > 0: scaled maximum
            if (wave_any(tm > mref + TAU)) {
                const float mnew = fmaxf(mref, tm);
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
            // a row with no valid key yet keeps mref = -inf: its probabilities are 0
            const float mu = mref == -INFINITY ? 0.f : mref;

            // ---- probabilities (bf16 head + tail) and O += P V ------------------------
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                const int ks = 2 * kc + h8;  // 16-key step of the tile
                float p[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    p[j] = fast_exp2(fmaf(s[8 * h8 + j], c, -mu));
                    lsum += p[j];
                }
                uint32_t h[4], t[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
                    t[j] = pack_bf16(p[2 * j] - bf16_lo(h[j]), p[2 * j + 1] - bf16_hi(h[j]));
                }
                const u32x4 ph = u32x4{h[0], h[1], h[2], h[3]};
                const u32x4 pl = u32x4{t[0], t[1], t[2], t[3]};
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) {
                    const u32x4 vb =
                        *(const u32x4 *)&sm.vt[bi][(32 * dt + col) * VSTR + 16 * ks + 8 * hl];
                    o[dt] = mfma32(ph, vb, o[dt]);
                    o[dt] = mfma32(pl, vb, o[dt]);
                }
            }
        }

        if (kt + 1 < t1)
            write_stage(bi ^ 1, kt + 1);
        __syncthreads();
    }

    // ---- finish: row sums, then normalise or store a partial ------------------
    lsum += __shfl_xor(lsum, 32);
    if (hl == 0) {
        sm.ml[w][0][col] = mref;
        sm.ml[w][1][col] = lsum;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
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

// Merge of the key-range splits: thread = (query row, 4 consecutive d).
template <int D>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillArgs a)
{
    typedef __attribute__((ext_vector_type(4))) float f32x4;
    const int64_t rows = a.total_rows * a.num_q_heads;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows * (D / 4))
        return;
    const int64_t qrow = e / (D / 4);
    const int d4 = (int)(e - qrow * (D / 4)) * 4;
    const int KS = a.kv_splits;
    float M = -INFINITY;
    for (int s = 0; s < KS; ++s)
        M = fmaxf(M, a.ws_ml[(s * rows + qrow) * 2]);
    f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int s = 0; s < KS; ++s) {
        const f32x2 ml = *(const f32x2 *)&a.ws_ml[(s * rows + qrow) * 2];
        const float f = ml[0] == -INFINITY ? 0.f : fast_exp2(ml[0] - M);
        num += f * *(const f32x4 *)&a.ws_acc[(s * rows + qrow) * D + d4];
        den += f * ml[1];
    }
    const float inv = a.v_scale / den;
    float *dst = a.out + qrow * D + d4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        dst[j] = num[j] * inv;
}

bool prefill_supported(int cache_dtype, int head_dim, int group)
{
    return (cache_dtype == DT_BF16 || cache_dtype == DT_FP8) && (head_dim == 64 || head_dim == 128) &&
           group >= 1 && group <= 8;
}

int prefill_m_tiles(int64_t total_rows, int num_q_heads, int num_kv_heads)
{
    const int ppt = PrefillCfg<128>::MROWS / (num_q_heads / num_kv_heads);
    return (int)((total_rows + ppt - 1) / ppt);
}

int prefill_kv_splits(int64_t total_rows, int num_q_heads)
{
    // one work-group per CU of a 256-CU device: split the key range until the
    // (row tile, KV head) work-groups reach that count
    const int64_t tiles = (total_rows * num_q_heads + PrefillCfg<128>::MROWS - 1) /
                          PrefillCfg<128>::MROWS;
    int64_t ks = tiles > 0 ? 256 / tiles : 1;
    if (ks < 1)
        ks = 1;
    if (ks > 16)
        ks = 16;
    return (int)ks;
}

template <int CDT, int D>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)(a.m_tiles * a.num_kv_heads * a.kv_splits), (unsigned)a.num_reqs);
    prefill_kernel<CDT, D><<<grid, 64 * PrefillCfg<D>::WAVES, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.kv_splits == 1)
        return e;
    const int64_t n = a.total_rows * a.num_q_heads * (D / 4);
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
