// prefill.hip -- chunked-prefill attention over a paged history.
//
// What is computed ("Lecture 33" §4.2): a prompt chunk of n rows, written to
// the cache before the call, attends to everything cached before it (the
// earlier chunks, read through the block table) and causally to itself:
// row j of a request with C cached tokens attends keys [0, C - n + j].
//
// Here the query tile makes QK^T a dense contraction, so it runs on the
// matrix cores (v_mfma_f32_32x32x16_bf16):
//   * A work-group (8 waves, two per SIMD) owns 256 "query rows" = (position,
//     head) pairs of one KV head (all G heads of a position are adjacent, so
//     one K/V tile feeds every head of the group), and one slice of the key
//     range.  Each wave holds one 32-row MFMA block.
//   * With a bf16 cache the two waves of a SIMD take turns (waves 0-3 and
//     4-7, half a tile apart, a work-group barrier between turns): one runs
//     its matrix phase (P V of the previous tile, S^T of this one) while the
//     other runs its vector phase (mask, maximum, exponentials, row sum, P in
//     bf16), so the matrix core and the vector ALU of a SIMD work at the same
//     time.  With an fp8 cache every wave runs a tile's steps in order.
//   * Per 64-key tile, K and V rows are gathered through the block table
//     straight into LDS (global_load_lds, 16 bytes per lane) through a ring of
//     four tiles, so two or three tiles are in flight while one is computed;
//     each wave counts its own loads (s_waitcnt vmcnt) and a work-group
//     barrier publishes a tile.  Both tiles stay row-major with XOR-swizzled
//     16-byte chunks: K fragments (MFMA A operand, 16 bytes per lane) and V^T
//     fragments (B operand, via the gfx950 transposing LDS read) come out
//     without bank conflicts.  fp8 rows arrive raw and are widened to bf16
//     (exactly) into a separate double buffer one tile ahead of the compute.
//   * S^T = K Q^T puts one query row per lane (column of the MFMA result),
//     so the row maximum and sum are in-lane plus one exchange between the two
//     half-waves.  Masks are applied only on tiles that cross the causal
//     diagonal or the end of the context.  With a bf16 cache the
//     probabilities are split into a bf16 head and a bf16 tail (together
//     exact to about 2^-16) and both are multiplied with V on the matrix cores
//     (O = P V): a single bf16 rounding of P costs up to 2^-8 relative weight
//     error, too coarse for rows with few keys at that cache's precision.
//     With an fp8 cache, whose values carry far coarser rounding, the head
//     alone is used (half the P V products).
//   * The running maximum is raised only when a tile exceeds it by more than
//     8 (base 2); that rare path rescales the accumulators through LDS.
//   * When the key range is split over several work-groups, each writes
//     (max, sum, unnormalised O) and a second kernel merges them.
//   * Work-groups that share a (request, KV head, key slice) are numbered
//     Hkv*splits apart, so when that product is a multiple of the XCD count
//     they run on one XCD and its L2 serves their common K/V tiles.
#include <type_traits>
#include <utility>

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

// bf16 (1.0, 1.0): v_dot2 against it sums a packed bf16 pair into fp32.
constexpr uint32_t kBf16OnePair = 0x3F803F80u;

// fp32 pair -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

constexpr int kPrefillWaves = 8;  // two per SIMD
constexpr int kPrefillThreads = 64 * kPrefillWaves;


template <int CDT, int D>
struct PrefillCfg {
    static constexpr int KT = 64;                  // keys per tile
    static constexpr int WAVES = kPrefillWaves;
    static constexpr int MROWS = 32 * WAVES;       // query rows per work-group
    static constexpr int ST = D / 16;              // 16-d steps of the QK contraction
    static constexpr int ROWB = 2 * D;             // bytes of a bf16 K or V row in LDS
    static constexpr int TILEB = KT * ROWB;        // bytes of a bf16 K (or V) tile
    static constexpr bool RAW = CDT == DT_FP8;     // fp8 rows are loaded raw, widened in LDS
    static constexpr int SROWB = RAW ? D : 2 * D;  // bytes of a row as cached
    static constexpr int DMA_ROWS = 1024 / SROWB;  // rows per global->LDS instruction
    static constexpr int DMA_TILE = 2 * KT / DMA_ROWS;  // instructions per tile (K, then V)
    static constexpr int DPW = DMA_TILE / WAVES;   // instructions per wave per tile
    static constexpr int NSTAGE = 4;               // tiles in the load ring
    static constexpr int STAGEB = 2 * KT * SROWB;  // bytes of one ring stage (K tile, V tile)
    static constexpr int CBUFB = RAW ? 2 * 2 * TILEB : 0;  // widened double buffer (fp8)
    static constexpr int LDSB = NSTAGE * STAGEB + CBUFB;
    static_assert(DMA_TILE % WAVES == 0 && DMA_ROWS <= 16 && 16 % DMA_ROWS == 0, "tile shape");
    static_assert(LDSB <= 128 * 1024, "LDS budget");
};

template <int CDT, int D>
struct PrefillSmem {
    using C = PrefillCfg<CDT, D>;
    __attribute__((aligned(1024))) char ring[C::LDSB];
    float alpha[C::WAVES][32];
    float ml[C::WAVES][2][32];  // [wave][max, sum][row]
};

// XOR swizzles of the 16-byte chunk index inside a K / V row of the LDS tile,
// chosen so that the fragment reads below hit distinct banks whether the LDS
// serves 128 or 256 bytes per cycle.  K rows are read 16 bytes per lane, 16
// consecutive keys at one chunk per 256 bytes; V rows are read with the
// transposing 8-byte reads, 4 consecutive keys x 2 (or 4) adjacent chunks per
// 128 (or 256) bytes.
template <int D>
__device__ __forceinline__ int swz_k(int key)
{
    return D == 128 ? (key & 15) : ((key & 7) ^ ((key >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int swz_v(int key)
{
    const int j = key & 3;
    return D == 128 ? 4 * j + 2 * (j >> 1) : 2 * j;
}

// max / sum of the values of lanes l and l ^ 32: gfx950's lane swap exchanges
// the two halves of the wave in registers; swapping a value with itself leaves
// {v(l), v(l ^ 32)} in the two results of every lane (in an order that depends
// on the half, hence only symmetric combinations).
__device__ __forceinline__ float max_halves(float v)
{
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}
__device__ __forceinline__ float sum_halves(float v)
{
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// Compile-time loop: f(std::integral_constant<int, 0>), ..., f(<N - 1>).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One 16-byte chunk of bf16 (8 values) from 8 fp8 bytes, exactly.
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1)
{
    return u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                 fp8x2_to_bf16x2<true>(w1)};
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4
// of the 4 x 16-bit values loaded by lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4 (checked on gfx950 with an in-bounds probe), i.e. a 4 x 16 block
// of a row-major tile arrives transposed.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ u32x2 lds_read_tr16(lds_char *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)p);
    return __builtin_bit_cast(u32x2, r);
}
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}
// keep(x): an empty asm that takes x in registers and may change it, so the
// computation of x cannot move past this point (the optimiser would otherwise
// sink pure arithmetic to where its result is used)
__device__ __forceinline__ void keep(float &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(u32x4 &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void keep(f32x16 &x) { asm volatile("" : "+v"(x)); }

// Work-group barrier that drains this wave's LDS operations only: the
// global->LDS loads of later tiles stay in flight (__syncthreads would wait
// for them too).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N): the global->LDS loads are counted there and the compiler
// does not wait for them by itself.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most n tiles of this wave's loads (DPW instructions each) are
// still in flight, n <= 2
template <int DPW>
__device__ __forceinline__ void wait_tiles_in_flight(int n)
{
    if (n >= 2)
        wait_vm<2 * DPW>();
    else if (n == 1)
        wait_vm<DPW>();
    else
        wait_vm<0>();
}

// 16 bytes per lane, global -> LDS at lds_dst + 16 * lane (lds_dst uniform).
// Issued as inline assembly so that the compiler, which would otherwise wait
// for these loads before every transposing LDS read, leaves the counting to
// wait_vm; the LDS reads then schedule freely between the matrix products.
// The LDS address is an input bound to m0 ("{m0}"), so the compiler writes
// that register itself and knows it is read here; the s_nop separates that
// write from the load that reads it.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_dst)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_dst) : "memory");
}

template <int CDT, int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs a)
{
    using C = PrefillCfg<CDT, D>;
    constexpr int KT = C::KT, ST = C::ST, ROWB = C::ROWB, NS = C::NSTAGE, DPW = C::DPW;
    constexpr int EB = Storage<CDT>::bytes;
    constexpr float TAU = 8.0f;
    __shared__ PrefillSmem<CDT, D> sm;

    const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
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
    // Rows are fetched in "parts" of PR = 2^hs consecutive rows held by one
    // physical location: 16-token units (a table entry names 2^ts of them),
    // or, with 8-token blocks (tbs_log2 < 0), single blocks.  Entry of part x:
    // tab[x >> tsp] << tsp, plus x's place among the parts of that entry.
    const bool h8 = a.tbs_log2 < 0;
    const int hs = h8 ? 3 : 4, PR = 1 << hs;
    const int tsp = h8 ? 0 : a.tbs_log2;
    const int max_ctx = a.max_blocks * (PR << tsp);  // tokens a table row addresses
    Ctx = Ctx < max_ctx ? Ctx : max_ctx;  // caller precondition, enforced
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
#pragma unroll
        for (int s = 0; s < ST; ++s)
            settle(qb[s][0]);  // q is in registers before the counted loads start
    }

    // key tiles of this split
    const int nkt = (Ctx + KT - 1) / KT;
    const int tps = (nkt + KS - 1) / KS;
    const int t0 = split * tps;
    int t1 = t0 + tps < nkt ? t0 + tps : nkt;
    const int tmax = (P + pos_end - 1) / KT + 1;
    t1 = t1 < tmax ? t1 : tmax;
    const int nt = t1 > t0 ? t1 - t0 : 0;

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

    // ---- global -> LDS: tile kt into ring stage s -----------------------------
    // Instruction i of a tile moves DMA_ROWS rows of K (i < DMA_TILE / 2) or V;
    // lane -> (row, 16-byte slot), fetching the source chunk that the row's
    // swizzle puts in that slot (fp8 rows are copied unswizzled and widened
    // later).  Rows past the context repeat the last context row, so every value
    // that reaches the products is finite.
    constexpr int SPR = C::SROWB / 16;  // 16-byte slots per cached row
    // per-lane byte offset of each of this wave's instructions inside its
    // part (the same for every tile)
    uint32_t doff[DPW];
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
        const int i = w + C::WAVES * j;
        const bool isv = i >= C::DMA_TILE / 2;
        const int ii = isv ? i - C::DMA_TILE / 2 : i;
        const int row = ii * C::DMA_ROWS + lane / SPR, slot = lane % SPR;
        const int ch = C::RAW ? slot : slot ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
        doff[j] = (uint32_t)((row & (PR - 1)) * tok_bytes + ch * 16);
    }
    const int64_t part_bytes = (int64_t)PR * tok_bytes;
    const int ppt_k = KT >> hs;  // parts per tile
    // parts holding context (>= 1 whenever a tile is issued)
    const int ctx_units = (Ctx + PR - 1) >> hs;
    // physical part of part kb of tile kt (parts past the context take the
    // last one's entry; no row of theirs is fetched)
    auto unit_entry = [&](int kt, int kb) -> int {
        int blk = kt * ppt_k + kb;
        blk = blk < ctx_units ? blk : ctx_units - 1;
        const int e = (tab[blk >> tsp] << tsp) + (blk & ((1 << tsp) - 1));
        return (unsigned)e < (unsigned)a.num_blocks ? e : 0;
    };
    // An instruction lies in one part when DMA_ROWS <= PR (not for 16-row fp8
    // instructions over 8-token blocks: those always take the per-lane path).
    // Instruction j of this wave then always moves rows of the same part of a
    // tile.  With two or more instructions per wave, K instruction j and V
    // instruction j + DPW / 2 move the same rows, so a wave needs the entries
    // of DPW / 2 parts; with one, of one part.  The table entries are read here
    // and used by issue_tile, so their loads go out back to back and are waited
    // for only where the entries are needed.
    const bool one_part = C::DMA_ROWS <= PR;
    static_assert((DPW == 1 || DPW % 2 == 0) && C::DMA_TILE == C::WAVES * DPW, "DMA layout");
    constexpr int NU = DPW >= 2 ? DPW / 2 : 1;
    struct Units {
        int blk[NU], raw[NU];
    };
    auto tile_units = [&](int kt, Units &un) {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int i = w + C::WAVES * j;
            const int ii = DPW >= 2 || i < C::DMA_TILE / 2 ? i : i - C::DMA_TILE / 2;
            int blk = kt * ppt_k + ((ii * C::DMA_ROWS) >> hs);
            blk = blk < ctx_units ? blk : ctx_units - 1;
            un.blk[j] = blk;
            un.raw[j] = tab[blk >> tsp];
        }
    };
    auto issue_tile = [&](int kt, int s, const Units &un) {
        int pb[NU];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
            const int e = (un.raw[j] << tsp) + (un.blk[j] & ((1 << tsp) - 1));
            pb[j] = (unsigned)e < (unsigned)a.num_blocks ? e : 0;
        }
        const int last = Ctx - 1 - kt * KT;  // last context row of this tile (may exceed KT)
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
            const int i = w + C::WAVES * j;
            const bool isv = i >= C::DMA_TILE / 2;  // uniform
            const int ii = isv ? i - C::DMA_TILE / 2 : i;
            const uint32_t dst =
                uniform(lds_addr(sm.ring + s * C::STAGEB + (isv ? KT * C::SROWB : 0) + ii * 1024));
            const char *base = isv ? vbase : kbase;
            const int row0 = ii * C::DMA_ROWS;
            if (one_part && row0 + C::DMA_ROWS - 1 <= last) {
                // whole instruction inside the context and one part: scalar base
                dma16(base + (int64_t)pb[j % NU] * part_bytes + doff[j], dst);
            } else {
                // the context ends inside this instruction (last tile only), or
                // the instruction spans two parts: each lane takes its row's
                // part, one of the (at most) two the aligned rows fall in
                // (DMA_ROWS <= 16, parts of 8 or 16 rows).  Rows past the
                // context read the last context row: in one of those two parts,
                // or, when the whole instruction is past the context, in an
                // earlier part whose entry both candidates then hold (a part past
                // the context takes the last context part's entry).
                static_assert(C::DMA_ROWS <= 16, "an instruction spans at most two parts");
                const int kb0 = row0 >> hs;
                const int pa0 = unit_entry(kt, kb0);
                const int pa1 = kb0 + 1 < ppt_k ? unit_entry(kt, kb0 + 1) : pa0;
                const int row = row0 + lane / SPR, slot = lane % SPR;
                const int key = row < last ? row : last;
                const int p = (key >> hs) == kb0 ? pa0 : pa1;
                const int ch = C::RAW ? slot : slot ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
                dma16(base + (int64_t)p * part_bytes + (int64_t)(key & (PR - 1)) * tok_bytes + ch * 16,
                      dst);
            }
        }
    };
    // fp8: widen ring stage s into compute buffer cb (bf16, swizzled rows)
    auto widen_tile = [&](int s, int cb) {
        constexpr int NCH = KT * D / 16;  // 16-byte raw chunks per K (or V) tile
#pragma unroll
        for (int e = tid; e < 2 * NCH; e += 64 * C::WAVES) {
            const bool isv = e >= NCH;
            const int e2 = isv ? e - NCH : e;
            const int row = e2 / (D / 16), c16 = e2 % (D / 16);
            const u32x4 raw = *(const u32x4 *)(sm.ring + s * C::STAGEB + (isv ? KT * D : 0) + e2 * 16);
            const int f = isv ? swz_v<D>(row) : swz_k<D>(row);
            char *dst = sm.ring + NS * C::STAGEB + cb * 2 * C::TILEB + (isv ? C::TILEB : 0) + row * ROWB;
            *(u32x4 *)(dst + ((2 * c16) ^ f) * 16) = widen8(raw[0], raw[1]);
            *(u32x4 *)(dst + ((2 * c16 + 1) ^ f) * 16) = widen8(raw[2], raw[3]);
        }
    };

    // per-lane parts of the fragment addresses (the rest are immediates)
    // K: lane reads key kc*32 + col, chunk 2 st + hl
    const int fk = swz_k<D>(col);
    int kofs[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st)
        kofs[st] = col * ROWB + ((2 * st + hl) ^ fk) * 16;
    // V: lane (hl, qd, j, m) of a transposing read loads key 4hl + j (+ 8, + 16 ks)
    // at d = 32 dt + 16 qd + 4 m
    const int jv = (lane >> 2) & 3, mv = lane & 3, qd = (lane >> 4) & 1;
    const int fv = swz_v<D>(jv);
    int vofs[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
        vofs[dt] = (4 * hl + jv) * ROWB + ((4 * dt + 2 * qd + (mv >> 1)) ^ fv) * 16 + (mv & 1) * 8;

    // ---- S^T = K Q^T of one tile (both 32-key halves) -------------------------------
    // K fragments are read two 16-d steps ahead of their products, so the LDS
    // latency of a step overlaps the products of the two before it
    auto s_tile = [&](const char *kt_lds, f32x16 (&s)[2], auto pin_) {
        constexpr int AH = ST < 3 ? ST : 3;  // steps of fragments in flight
        u32x4 ka[AH][2];
        auto read = [&](int st) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
                ka[st % AH][kc] = *(const u32x4 *)(kt_lds + kc * 32 * ROWB + kofs[st]);
        };
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int st = 0; st < AH - 1; ++st)
            read(st);
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            if (st + AH - 1 < ST)
                read(st + AH - 1);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
                s[kc] = mfma32(ka[st % AH][kc], qb[st], s[kc]);
        }
        // keep that order through scheduling (which would otherwise sink each
        // read to its product to save registers): the first reads, then per
        // step two products and the reads of a later step
        if constexpr (decltype(pin_)::value) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * (AH - 1), 0);
            static_for<ST>([&](auto st_) {
                constexpr int st = decltype(st_)::value;
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                if constexpr (st + AH - 1 < ST)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            });
        }
    };
    // ---- mask (diagonal / ragged tiles only), row maximum, lazy rescale --------------
    // Raises the running maximum when the tile exceeds it by more than TAU
    // (rescaling O and the row sum), and returns the maximum the tile's
    // probabilities are taken against.
    auto mask_max = [&](f32x16 (&s)[2], int kt) -> float {
        const int key0 = kt * KT;
        const bool full = key0 + KT <= Ctx && key0 + KT - 1 <= P + pos0;
        if (!full) {
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + 32 * kc + 8 * (i >> 2) + 4 * hl + (i & 3);
                    s[kc][i] = key <= lim ? s[kc][i] : -INFINITY;
                }
        }
        float tm = -INFINITY;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                tm = fmaxf(tm, s[kc][i]);
        tm = max_halves(tm) * c;  // c > 0: scaled maximum
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
        return mref == -INFINITY ? 0.f : mref;
    };
    // ---- fp8 caches: probabilities and O += P V, four 16-key steps ----------------
    // One bf16 rounding of P, and the rounded weights enter the row sum as they
    // enter the products, so the result stays a convex combination of V rows
    // (a row with one key returns its value exactly); that sum is formed with
    // v_dot2 against (1, 1): exact products, one fp32 sum per pair (four VALU
    // instructions fewer per pair than widening both halves and adding them).
    auto pv_tile = [&](const f32x16 (&s)[2], float mu, const char *vt_lds) {
        static_for<4>([&](auto ks_) {
            constexpr int ks = decltype(ks_)::value;
            constexpr int kc = ks >> 1, h8 = ks & 1;
            // V^T fragments: keys 4hl + (0..3) and 8 + 4hl + (0..3) of the step,
            // at d = 32 dt + col
            // (the LDS-space base keeps the constant offsets in the instructions)
            lds_char *vt3 = (lds_char *)vt_lds;
            u32x2 vr[2 * (D / 32)];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                lds_char *vp = vt3 + vofs[dt] + 16 * ks * ROWB;
                vr[2 * dt] = lds_read_tr16(vp);
                vr[2 * dt + 1] = lds_read_tr16(vp + 8 * ROWB);
            }
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                p[j] = fast_exp2(fmaf(s[kc][8 * h8 + j], c, -mu));
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
                lsum = dot2_bf16(h[j], kBf16OnePair, lsum);
            }
            const u32x4 ph = u32x4{h[0], h[1], h[2], h[3]};
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const u32x4 vb = u32x4{vr[2 * dt][0], vr[2 * dt][1], vr[2 * dt + 1][0], vr[2 * dt + 1][1]};
                o[dt] = mfma32(ph, vb, o[dt]);
            }
        });
    };

    using Pinned = std::true_type;
    auto compute_tile = [&](const char *kt_lds, const char *vt_lds, int kt) {
        f32x16 s[2];
        s_tile(kt_lds, s, Pinned{});
        const float mu = mask_max(s, kt);
        pv_tile(s, mu, vt_lds);
    };

    // ---- bf16 caches: the tile work as a vector and a matrix phase --------------
    // vec: mask, maximum, exponentials, row sum, and P as a bf16 head and a bf16
    // tail (weights exact to ~2^-16; a single bf16 rounding costs up to 2^-8
    // relative weight error, too coarse for rows with few keys at that cache's
    // precision); mat: P V of the previous tile (head and tail), then S^T of
    // this one.
    auto probs0 = [&](const f32x16 (&s)[2], float mu, u32x4 (&ph)[4], u32x4 (&pl)[4]) {
        static_for<4>([&](auto ks_) {
            constexpr int ks = decltype(ks_)::value;
            constexpr int kc = ks >> 1, h8 = ks & 1;
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                p[j] = fast_exp2(fmaf(s[kc][8 * h8 + j], c, -mu));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                lsum += p[j];
            uint32_t h[4], t[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                h[j] = pack_bf16(p[2 * j], p[2 * j + 1]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                t[j] = pack_bf16(p[2 * j] - bf16_lo(h[j]), p[2 * j + 1] - bf16_hi(h[j]));
            ph[ks] = u32x4{h[0], h[1], h[2], h[3]};
            pl[ks] = u32x4{t[0], t[1], t[2], t[3]};
        });
    };
    auto pv0 = [&](const u32x4 (&ph)[4], const u32x4 (&pl)[4], const char *vt_lds) {
        // V^T fragments of step ks + 1 are read while the products of step ks run
        lds_char *vt3 = (lds_char *)vt_lds;
        u32x4 vb[2][D / 32];
        auto read = [&](int ks) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                lds_char *vp = vt3 + vofs[dt] + 16 * ks * ROWB;
                const u32x2 a0 = lds_read_tr16(vp), a1 = lds_read_tr16(vp + 8 * ROWB);
                vb[ks & 1][dt] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
        };
        read(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4)
                read(ks + 1);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                o[dt] = mfma32(ph[ks], vb[ks & 1][dt], o[dt]);
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                o[dt] = mfma32(pl[ks], vb[ks & 1][dt], o[dt]);
        }
        // pin that order: reads of step 0, then per step its products and the
        // reads of the next
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);
        static_for<4>([&](auto ks_) {
            constexpr int ks = decltype(ks_)::value;
            if constexpr (ks + 1 < 4)
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 32), 0);
        });
    };
    // work-group barrier between phases; nothing is scheduled across it
    // (and keep() below stops the optimiser from sinking a phase's arithmetic
    // into the next one, where its results are used)
    auto phase_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        barrier_lds();
        __builtin_amdgcn_sched_barrier(0);
    };
    constexpr bool PP = !C::RAW;  // bf16 caches: the two waves of a SIMD take turns
    // The table entries of the next tile to issue are read right after a tile
    // is issued (fp8: at the end of the compute), so their scalar loads are in
    // flight while other work runs.
    Units pbn = {};
    if constexpr (PP) {
        // Waves w and w + 4 share a SIMD (work-group waves are placed on the
        // four SIMDs in turn).  Waves 0-3 and 4-7 run the phases half a tile
        // apart: in phase 2u the first group does mat(u) while the second does
        // vec(u - 1); in phase 2u + 1 the first does vec(u), the second mat(u).
        // A barrier separates phases, so while one wave of a SIMD keeps the
        // matrix core busy (at raised issue priority) the other has the vector
        // ALU.  Tile t is read in phases 2t .. 2t + 3, so with four ring stages
        // tile u + 2 is issued at the start of phase 2u into the stage tile
        // u - 2 has left.
        const bool mat_first = w < C::WAVES / 2;
        f32x16 s[2];
        u32x4 ph[4], pl[4];
        // Every wave runs the same sequence S(0), vec(0), PV(0) + S(1), vec(1),
        // ..., PV(nt - 1) with a barrier before each phase; the second group
        // passes one extra barrier first and the first group one at the end,
        // which puts them a phase apart.  The ring work of phase p (tile p / 2
        // landed and published, tile p / 2 + 2 issued) happens at the barrier
        // before phase p, whichever of its phases a wave is in.
        int gp = 0;  // global index of the phase about to start
        auto boundary = [&]() {
            if ((gp & 1) == 0) {
                const int u = gp >> 1;
                if (u < nt)
                    wait_tiles_in_flight<DPW>(nt - 1 - u < 1 ? nt - 1 - u : 1);  // tile u landed
                phase_barrier();  // tile u visible to all; tile u - 2's stage is free
                if (u + 2 < nt)
                    issue_tile(t0 + u + 2, (u + 2) % NS, pbn);
                if (u + 3 < nt)
                    tile_units(t0 + u + 3, pbn);
            } else {
                phase_barrier();
            }
            ++gp;
        };
        auto stage = [&](int u) { return sm.ring + (u % NS) * C::STAGEB; };
        auto vec = [&](int u) {
            const float mu = mask_max(s, t0 + u);
            probs0(s, mu, ph, pl);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                keep(ph[ks]);
                keep(pl[ks]);
            }
            keep(lsum);
        };
        auto kept_s = [&]() {
            keep(s[0]);
            keep(s[1]);
        };
        auto kept_o = [&]() {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
                keep(o[dt]);
        };
        for (int u = 0; u < 2 && u < nt; ++u) {
            tile_units(t0 + u, pbn);
            issue_tile(t0 + u, u, pbn);
        }
        if (2 < nt)
            tile_units(t0 + 2, pbn);
        if (!mat_first)
            boundary();
        boundary();
        if (nt > 0) {
            __builtin_amdgcn_s_setprio(1);
            s_tile(stage(0), s, Pinned{});
            __builtin_amdgcn_s_setprio(0);
            kept_s();
            for (int u = 0; u + 1 < nt; ++u) {
                boundary();
                vec(u);
                boundary();
                __builtin_amdgcn_s_setprio(1);
                pv0(ph, pl, stage(u) + C::TILEB);
                s_tile(stage(u + 1), s, Pinned{});
                __builtin_amdgcn_s_setprio(0);
                kept_s();
                kept_o();
            }
            boundary();
            vec(nt - 1);
            boundary();
            __builtin_amdgcn_s_setprio(1);
            pv0(ph, pl, stage(nt - 1) + C::TILEB);
            __builtin_amdgcn_s_setprio(0);
            kept_o();
        }
        if (mat_first)
            boundary();
    } else {
        // raw ring -> widened double buffer, one tile ahead of the compute
        for (int u = 0; u < NS - 1 && u < nt; ++u) {
            tile_units(t0 + u, pbn);
            issue_tile(t0 + u, u, pbn);
        }
        if (NS - 1 < nt)
            tile_units(t0 + NS - 1, pbn);
        if (nt > 0) {
            wait_tiles_in_flight<DPW>(nt - 1 < NS - 2 ? nt - 1 : NS - 2);
            barrier_lds();
            widen_tile(0, 0);
        }
        for (int u = 0; u < nt; ++u) {
            const int kt = t0 + u;
            if (u + 1 < nt) {
                const int ahead = nt - 2 - u < NS - 3 ? nt - 2 - u : NS - 3;
                wait_tiles_in_flight<DPW>(ahead);  // raw tile u + 1 landed
            }
            barrier_lds();  // widened tile u visible; raw stage of tile u - 1 is free
            if (u + NS - 1 < nt)
                issue_tile(kt + NS - 1, (u + NS - 1) % NS, pbn);
            const char *cb_lds = sm.ring + NS * C::STAGEB + (u & 1) * 2 * C::TILEB;
            compute_tile(cb_lds, cb_lds + C::TILEB, kt);
            if (u + 1 < nt)
                widen_tile((u + 1) % NS, (u + 1) & 1);
            if (u + NS < nt)
                tile_units(kt + NS, pbn);
        }
    }

    // ---- finish: row sums, then normalise or store a partial ------------------
    lsum = sum_halves(lsum);
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

// Merge of the key-range splits: thread = (query row, 4 consecutive d); the
// loads of all KS splits go out together.
template <int D, int KS>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillArgs a)
{
    const int64_t rows = a.total_rows * a.num_q_heads;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows * (D / 4))
        return;
    const int64_t qrow = e / (D / 4);
    const int d4 = (int)(e - qrow * (D / 4)) * 4;
    f32x2 ml[KS];
    f32x4 acc[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        ml[s] = *(const f32x2 *)&a.ws_ml[(s * rows + qrow) * 2];
        acc[s] = *(const f32x4 *)&a.ws_acc[(s * rows + qrow) * D + d4];
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < KS; ++s)
        M = fmaxf(M, ml[s][0]);
    f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const float f = ml[s][0] == -INFINITY ? 0.f : fast_exp2(ml[s][0] - M);
        num += f * acc[s];
        den += f * ml[s][1];
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
    const int ppt = PrefillCfg<DT_BF16, 128>::MROWS / (num_q_heads / num_kv_heads);
    return (int)((total_rows + ppt - 1) / ppt);
}

int prefill_kv_splits(int64_t total_rows, int num_q_heads, int cus)
{
    // one work-group per compute unit: split the key range until the
    // (row tile, KV head) work-groups reach the device's CU count
    const int64_t tiles = (total_rows * num_q_heads + PrefillCfg<DT_BF16, 128>::MROWS - 1) /
                          PrefillCfg<DT_BF16, 128>::MROWS;
    int64_t ks = tiles > 0 ? cus / tiles : 1;
    if (ks < 1)
        ks = 1;
    if (ks > 16)
        ks = 16;
    return (int)ks;
}

// the merge instance for the call's split count (2..16)
template <int D, int KS = 2>
static void launch_reduce(const PrefillArgs &a, hipStream_t stream)
{
    if constexpr (KS <= 16) {
        if (a.kv_splits != KS)
            return launch_reduce<D, KS + 1>(a, stream);
        const int64_t n = a.total_rows * a.num_q_heads * (D / 4);
        prefill_reduce_kernel<D, KS><<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a);
    }
}

template <int CDT, int D>
static hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t stream)
{
    dim3 grid((unsigned)(a.m_tiles * a.num_kv_heads * a.kv_splits), (unsigned)a.num_reqs);
    prefill_kernel<CDT, D><<<grid, kPrefillThreads, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.kv_splits == 1)
        return e;
    launch_reduce<D>(a, stream);
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
