// pa_api.cpp -- C ABI of libpa (declared in include/pa.h): argument checks on
// the host, workspace carving, and kernel launches.  No call allocates device
// memory, synchronises the host or copies data back.
#include "pa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "pa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status fail(pa_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

pa_status ok()
{
    g_last_error[0] = '\0';
    return PA_OK;
}

pa_status hip_fail(hipError_t e, const char *what)
{
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device.  Device properties (this count and
// the decode kernels' occupancy below) are memoised per device id in
// write-once tables under a mutex: they never change while the process runs,
// and no call's data passes through them.
int device_cus()
{
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Tokens per block (0 in the shape means 16) and the kernels' view of it:
// every kernel walks 16-token units, block b holding units b * 2^s .. + 2^s - 1;
// s = -1 for 8-token blocks, where a unit is the two blocks of entries 2u, 2u + 1.
int block_size_of(const pa_shape *s) { return s->block_size ? s->block_size : 16; }
int unit_shift(const pa_shape *s)
{
    const int b = block_size_of(s);
    return b == 64 ? 2 : b == 32 ? 1 : b == 8 ? -1 : 0;
}
// 16-token units a block table row can address.
int units_per_seq(const pa_shape *s)
{
    return unit_shift(s) < 0 ? (s->max_blocks_per_seq + 1) / 2 : s->max_blocks_per_seq << unit_shift(s);
}
// Pool size as the kernels count it: 16-token units, or 8-token blocks.
int64_t kernel_blocks(const pa_shape *s)
{
    return unit_shift(s) < 0 ? s->num_blocks : s->num_blocks << unit_shift(s);
}

// Work-groups per resident slot of the decode grid with fixed partitions.
constexpr int kPartitionGridFactor = 3;

// Persistent decode grid: as many work-groups as can be resident at once
// (compute units x occupancy of the kernel that serves this shape), so every
// work-group of the balanced split runs concurrently.
int decode_grid(const pa_shape *s)
{
    static std::mutex mu;
    static int cached[64][3][2][9][3] = {};
    const int G = s->num_q_heads / s->num_kv_heads;
    const int hpg = pa::decode_hpg(s->num_kv_heads, G, unit_shift(s));
    const int dt = s->cache_dtype, dh = s->head_dim == 128 ? 1 : 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    const bool h8 = unit_shift(s) < 0;
    int &slot = cached[dev][dt][dh][G][hpg == 4 ? 1 : h8 ? 2 : 0];
    if (slot == 0) {
        int per_cu = 0;
        const pa::DecodeKernels k = pa::decode_kernels(dt, s->head_dim, G, hpg, h8);
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.main, k.threads, 0) !=
                hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        slot = per_cu * device_cus();
    }
    return slot;
}

// Bytes of one block of one pool: block_size token rows of num_kv_heads x head_dim.
int64_t block_bytes_of(const pa_shape *s)
{
    return (int64_t)block_size_of(s) * s->num_kv_heads * s->head_dim *
           (s->cache_dtype == PA_F32 ? 4 : s->cache_dtype == PA_BF16 ? 2 : 1);
}

// The address a kernel uses for p: device memory as it is, pinned host memory
// through the device mapping the runtime reports; false for anything else
// (pageable host memory, which a kernel cannot reach).
bool device_address(const void *p, const void **out)
{
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();  // not an error of the next call
        return false;
    }
    if (at.type == hipMemoryTypeDevice) {
        *out = p;
        return true;
    }
    if (at.type == hipMemoryTypeHost && at.devicePointer && at.hostPointer) {
        *out = (const char *)at.devicePointer + ((const char *)p - (const char *)at.hostPointer);
        return true;
    }
    return false;
}

pa_status check_shape(const pa_shape *s, bool need_tables)
{
    if (!s)
        return fail(PA_ERR_INVALID, "shape is NULL");
    if (s->num_seqs < 0)
        return fail(PA_ERR_INVALID, "num_seqs < 0");
    if (s->num_q_heads <= 0 || s->num_kv_heads <= 0)
        return fail(PA_ERR_INVALID, "head counts must be positive");
    if (s->num_q_heads % s->num_kv_heads != 0)
        return fail(PA_ERR_INVALID, "num_q_heads %% num_kv_heads != 0 (%d, %d)", s->num_q_heads,
                    s->num_kv_heads);
    if (s->num_blocks <= 0)
        return fail(PA_ERR_INVALID, "num_blocks must be positive");
    if (s->block_size != 0 && s->block_size != 8 && s->block_size != 16 && s->block_size != 32 &&
        s->block_size != 64)
        return fail(PA_ERR_UNSUPPORTED, "block_size %d (8, 16, 32 or 64 are built)", s->block_size);
    if (kernel_blocks(s) > (int64_t)1 << 31)
        return fail(PA_ERR_UNSUPPORTED, "num_blocks * max(block_size / 16, 1) above 2^31");
    if (need_tables && s->max_blocks_per_seq <= 0)
        return fail(PA_ERR_INVALID, "max_blocks_per_seq must be positive");
    if (s->cache_dtype != PA_F32 && s->cache_dtype != PA_BF16 && s->cache_dtype != PA_FP8_E4M3)
        return fail(PA_ERR_INVALID, "unknown cache_dtype %d", s->cache_dtype);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d (64 or 128 are built)", s->head_dim);
    if (s->cache_dtype == PA_FP8_E4M3 && !(s->kv_scale > 0.f && std::isfinite(s->kv_scale)))
        return fail(PA_ERR_INVALID, "kv_scale must be finite and > 0 for an fp8 cache");
    return PA_OK;
}

int q_dtype_for(int cache_dtype) { return cache_dtype == PA_F32 ? PA_F32 : PA_BF16; }

float kv_scale_of(const pa_shape *s) { return s->cache_dtype == PA_FP8_E4M3 ? s->kv_scale : 1.f; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecodeLayout {
    int64_t slots;
    size_t count_bytes, acc_bytes, ml_bytes, total;
};

// Decode workspace: arrival counters (counter_slots int32), then the split-K
// partial records: (max, sum) pairs and accumulators.
DecodeLayout decode_layout(const pa_shape *s, int64_t counter_slots = pa::kDecodeCounterSlots)
{
    const int G = s->num_q_heads / s->num_kv_heads;
    const int pb = s->partition_tokens > 0 ? s->partition_tokens / 16 : 0;
    DecodeLayout L;
    L.slots = pa::decode_partial_slots(s->num_seqs, s->num_kv_heads, G, units_per_seq(s), pb,
                                       decode_grid(s), unit_shift(s));
    L.count_bytes = (size_t)counter_slots * sizeof(int32_t);
    L.ml_bytes = align256((size_t)L.slots * G * 2 * sizeof(float));
    L.acc_bytes = align256((size_t)L.slots * G * s->head_dim * sizeof(float));
    L.total = L.count_bytes + L.ml_bytes + L.acc_bytes;
    return L;
}

// Checks shared by the decode entry points; PA_OK means "launch".
pa_status check_decode(const float *out, const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, float scale,
                       const pa_shape *shape, int64_t counter_slots)
{
    pa_status st = check_shape(shape, true);
    if (st != PA_OK)
        return st;
    const int G = shape->num_q_heads / shape->num_kv_heads;
    if (shape->q_dtype != q_dtype_for(shape->cache_dtype))
        return fail(PA_ERR_UNSUPPORTED, "q_dtype %d with cache_dtype %d", shape->q_dtype,
                    shape->cache_dtype);
    if (!pa::decode_supported(shape->cache_dtype, shape->head_dim, G))
        return fail(PA_ERR_UNSUPPORTED, "decode not built for cache_dtype %d, head_dim %d, G %d",
                    shape->cache_dtype, shape->head_dim, G);
    if (shape->partition_tokens < 0 || shape->partition_tokens % 16 != 0)
        return fail(PA_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of 16");
    if (!std::isfinite(scale))
        return fail(PA_ERR_INVALID, "scale is not finite");
    if ((int64_t)shape->num_seqs * shape->num_kv_heads > counter_slots)
        return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_kv_heads above %lld",
                    (long long)counter_slots);
    if (shape->num_seqs > 0 && (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens))
        return fail(PA_ERR_INVALID, "NULL data pointer");
    return PA_OK;
}

// One decode launch over a workspace laid out by decode_layout(shape, L).
pa_status launch_decode_on(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           const pa_shape *shape, char *ws, const DecodeLayout &L, void *stream)
{
    pa::DecodeArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = shape->num_seqs;
    a.num_q_heads = shape->num_q_heads;
    a.num_kv_heads = shape->num_kv_heads;
    a.head_dim = shape->head_dim;
    a.max_blocks = shape->max_blocks_per_seq;
    a.tbs_log2 = unit_shift(shape);
    a.num_blocks = kernel_blocks(shape);
    a.cache_dtype = shape->cache_dtype;
    a.part_blocks = shape->partition_tokens / 16;
    // Fixed partitions are whole work items, so static ranges of them cannot
    // balance; three times the resident work-groups lets the dispatcher hand
    // the later ones to the CUs that finish first (measured: 2x and 4-8x are
    // slower on the 32k/short skewed batch; the balanced split balances by
    // itself and loses with any oversubscription).
    a.grid = decode_grid(shape) * (shape->partition_tokens > 0 ? kPartitionGridFactor : 1);
    const float kvs = kv_scale_of(shape);
    a.qk_scale = scale * 1.4426950408889634f * kvs;
    a.v_scale = kvs;
    a.ws_count = (int32_t *)ws;
    a.ws_ml = (float *)(ws + L.count_bytes);
    a.ws_acc = (float *)(ws + L.count_bytes + L.ml_bytes);
    hipError_t e = pa::launch_decode(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "decode launch");
}

// ---------------------------------------------------------------------------
// Scratch of pa_decode_static: one array per device, for callers that cannot
// allocate.  Arrival counters first (a fixed region, so that a later call with
// more (sequence, KV head) pairs never takes an earlier call's partial results
// for counters), then the partial records.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int64_t kStaticCounterSlots = (int64_t)1 << 18;  // 1 MiB of int32 counters
static_assert((size_t)kStaticCounterSlots * 4 < kStaticScratchBytes, "scratch layout");

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void zero_counters_kernel(int32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// Device address of `scratch` on the current device (the array's name is only
// a host-side stand-in), resolved once per device; the first call also queues
// a fill kernel on `stream` that zeroes the counter region.  Afterwards every
// decode leaves its counters zero again.
pa_status static_scratch(void *stream, char **out)
{
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64)
        return fail(PA_ERR_UNSUPPORTED, "device id %d above 63", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        zero_counters_kernel<<<256, 256, 0, (hipStream_t)stream>>>((int32_t *)p, kStaticCounterSlots);
        e = hipGetLastError();
        if (e != hipSuccess)
            return hip_fail(e, "zeroing the static scratch counters");
        addr[dev] = p;
    }
    *out = (char *)addr[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

const char *pa_status_string(pa_status s)
{
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *pa_last_error(void) { return g_last_error; }

pa_status pa_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int64_t num_tokens,
                               int32_t src_dtype, const pa_shape *shape, void *stream)
{
    pa_status st = check_shape(shape, false);
    if (st != PA_OK)
        return st;
    if (num_tokens < 0)
        return fail(PA_ERR_INVALID, "num_tokens < 0");
    if (src_dtype != q_dtype_for(shape->cache_dtype))
        return fail(PA_ERR_UNSUPPORTED, "src_dtype %d cannot feed cache_dtype %d", src_dtype,
                    shape->cache_dtype);
    if (num_tokens == 0)
        return ok();
    if (!k || !v || !k_cache || !v_cache || !slot_mapping)
        return fail(PA_ERR_INVALID, "NULL data pointer");
    pa::ReshapeArgs a;
    a.k = k;
    a.v = v;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.slot_mapping = slot_mapping;
    a.num_tokens = num_tokens;
    a.num_slots = shape->num_blocks * block_size_of(shape);
    a.row_elems = shape->num_kv_heads * shape->head_dim;
    a.src_dtype = src_dtype;
    a.cache_dtype = shape->cache_dtype;
    {
        volatile float one = 1.0f;
        a.inv_scale = one / kv_scale_of(shape);  // rounded once, in fp32
    }
    hipError_t e = pa::launch_reshape_and_cache(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "reshape_and_cache launch");
}

pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_pairs,
                         int64_t num_pairs, const pa_shape *shape, void *stream)
{
    pa_status st = check_shape(shape, false);
    if (st != PA_OK)
        return st;
    if (num_pairs < 0)
        return fail(PA_ERR_INVALID, "num_pairs < 0");
    if (num_pairs == 0)
        return ok();
    if (!k_cache || !v_cache || !block_pairs)
        return fail(PA_ERR_INVALID, "NULL data pointer");
    pa::CopyArgs a;
    a.src_k = k_cache;
    a.src_v = v_cache;
    a.dst_k = k_cache;
    a.dst_v = v_cache;
    a.block_pairs = block_pairs;
    a.num_pairs = num_pairs;
    a.src_blocks = a.dst_blocks = shape->num_blocks;
    a.block_bytes = block_bytes_of(shape);
    a.pieces = pa::copy_pieces(a.block_bytes);
    hipError_t e = pa::launch_copy_blocks(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "copy_blocks launch");
}

pa_status pa_swap_blocks(const void *src_k, const void *src_v, int64_t src_num_blocks, void *dst_k,
                         void *dst_v, int64_t dst_num_blocks, const int64_t *block_pairs,
                         int64_t num_pairs, const pa_shape *shape, void *stream)
{
    pa_status st = check_shape(shape, false);
    if (st != PA_OK)
        return st;
    if (num_pairs < 0 || src_num_blocks < 0 || dst_num_blocks < 0)
        return fail(PA_ERR_INVALID, "negative count");
    if (num_pairs == 0)
        return ok();
    if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs)
        return fail(PA_ERR_INVALID, "NULL data pointer");
    // every pointer the kernel uses: device memory, or pinned host memory
    // through its device mapping
    const void *ptrs[5] = {src_k, src_v, dst_k, dst_v, block_pairs};
    const void *dev[5];
    for (int i = 0; i < 5; ++i)
        if (!device_address(ptrs[i], &dev[i]))
            return fail(PA_ERR_INVALID,
                        "pointer %d is neither device memory nor pinned host memory", i);
    pa::CopyArgs a;
    a.src_k = dev[0];
    a.src_v = dev[1];
    a.dst_k = (void *)dev[2];
    a.dst_v = (void *)dev[3];
    a.block_pairs = (const int64_t *)dev[4];
    a.num_pairs = num_pairs;
    a.src_blocks = src_num_blocks;
    a.dst_blocks = dst_num_blocks;
    a.block_bytes = block_bytes_of(shape);
    a.pieces = pa::copy_pieces(a.block_bytes);
    hipError_t e = pa::launch_copy_blocks(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "swap_blocks launch");
}

size_t pa_decode_workspace_bytes(const pa_shape *shape)
{
    if (check_shape(shape, true) != PA_OK)
        return 0;
    if (!pa::decode_supported(shape->cache_dtype, shape->head_dim,
                              shape->num_q_heads / shape->num_kv_heads))
        return 0;
    return decode_layout(shape).total;
}

pa_status pa_decode(float *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    const pa_shape *shape, void *workspace, size_t workspace_bytes, void *stream)
{
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, shape,
                                pa::kDecodeCounterSlots);
    if (st != PA_OK)
        return st;
    if (shape->num_seqs == 0)
        return ok();
    const DecodeLayout L = decode_layout(shape);
    if (!workspace || workspace_bytes < L.total)
        return fail(PA_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    return launch_decode_on(out, q, k_cache, v_cache, block_tables, context_lens, scale, shape,
                            (char *)workspace, L, stream);
}

pa_status pa_decode_static(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           const pa_shape *shape, void *stream)
{
    pa_status st = check_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, shape,
                                kStaticCounterSlots);
    if (st != PA_OK)
        return st;
    if (shape->num_seqs == 0)
        return ok();
    const DecodeLayout L = decode_layout(shape, kStaticCounterSlots);
    if (L.total > kStaticScratchBytes)
        return fail(PA_ERR_WORKSPACE,
                    "decode of this shape needs %zu scratch bytes; the static scratch holds %zu "
                    "(use pa_decode with a workspace)", L.total, kStaticScratchBytes);
    char *ws = nullptr;
    st = static_scratch(stream, &ws);
    if (st != PA_OK)
        return st;
    return launch_decode_on(out, q, k_cache, v_cache, block_tables, context_lens, scale, shape, ws,
                            L, stream);
}

size_t pa_prefill_workspace_bytes(const pa_shape *shape, int64_t total_query_rows)
{
    if (check_shape(shape, true) != PA_OK || total_query_rows < 0)
        return 0;
    const int ks = pa::prefill_kv_splits(total_query_rows, shape->num_q_heads, device_cus());
    if (ks <= 1)
        return 0;
    const size_t rows = (size_t)total_query_rows * shape->num_q_heads;
    return align256((size_t)ks * rows * shape->head_dim * sizeof(float)) +
           align256((size_t)ks * rows * 2 * sizeof(float));
}

pa_status pa_prefill_chunk(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *query_start,
                           const int32_t *context_lens, int64_t total_query_rows, float scale,
                           const pa_shape *shape, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    pa_status st = check_shape(shape, true);
    if (st != PA_OK)
        return st;
    const int G = shape->num_q_heads / shape->num_kv_heads;
    if (shape->q_dtype != PA_BF16)
        return fail(PA_ERR_UNSUPPORTED, "prefill needs a bf16 q");
    if (!pa::prefill_supported(shape->cache_dtype, shape->head_dim, G))
        return fail(PA_ERR_UNSUPPORTED, "prefill not built for cache_dtype %d, head_dim %d, G %d",
                    shape->cache_dtype, shape->head_dim, G);
    if (total_query_rows < 0)
        return fail(PA_ERR_INVALID, "total_query_rows < 0");
    if (total_query_rows > (int64_t)1 << 24)
        return fail(PA_ERR_UNSUPPORTED, "more than 2^24 query rows");
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(PA_ERR_INVALID, "prefill scale must be finite and > 0");
    if (shape->num_seqs > 65535)
        return fail(PA_ERR_UNSUPPORTED, "more than 65535 prefill requests in one call");
    if (shape->num_seqs == 0 || total_query_rows == 0)
        return ok();
    const int m_tiles = pa::prefill_m_tiles(total_query_rows, shape->num_q_heads, shape->num_kv_heads);
    const int kv_splits = pa::prefill_kv_splits(total_query_rows, shape->num_q_heads, device_cus());
    if ((int64_t)m_tiles * shape->num_kv_heads * kv_splits > INT32_MAX)
        return fail(PA_ERR_UNSUPPORTED, "prefill grid too large");
    if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens)
        return fail(PA_ERR_INVALID, "NULL data pointer");
    const size_t need = pa_prefill_workspace_bytes(shape, total_query_rows);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PA_ERR_WORKSPACE, "prefill needs %zu workspace bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    pa::PrefillArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.query_start = query_start;
    a.context_lens = context_lens;
    a.total_rows = total_query_rows;
    a.num_reqs = shape->num_seqs;
    a.num_q_heads = shape->num_q_heads;
    a.num_kv_heads = shape->num_kv_heads;
    a.head_dim = shape->head_dim;
    a.max_blocks = shape->max_blocks_per_seq;
    a.tbs_log2 = unit_shift(shape);
    a.num_blocks = kernel_blocks(shape);
    a.cache_dtype = shape->cache_dtype;
    a.kv_splits = kv_splits;
    a.m_tiles = m_tiles;
    const float kvs = kv_scale_of(shape);
    a.qk_scale = scale * 1.4426950408889634f * kvs;
    a.v_scale = kvs;
    const size_t rows = (size_t)total_query_rows * shape->num_q_heads;
    a.ws_acc = (float *)workspace;
    a.ws_ml = need > 0 ? (float *)((char *)workspace +
                                   align256((size_t)a.kv_splits * rows * shape->head_dim * 4))
                       : nullptr;
    hipError_t e = pa::launch_prefill(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : hip_fail(e, "prefill launch");
}

}  // extern "C"
