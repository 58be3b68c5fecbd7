// pa_internal.h -- host-side interface between the C ABI layer (pa_api.cpp)
// and the kernel launchers (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct ReshapeArgs {
    const void *k, *v;
    void *k_cache, *v_cache;
    const int64_t *slot_mapping;
    int64_t num_tokens;
    int64_t num_slots;   // num_blocks * 16
    int row_elems;       // num_kv_heads * head_dim
    int src_dtype, cache_dtype;
    float inv_scale;     // fp32 reciprocal of kv_scale, rounded on the host
};
hipError_t launch_reshape_and_cache(const ReshapeArgs &a, hipStream_t stream);

struct CopyArgs {
    const void *src_k, *src_v;   // pools read (device addresses)
    void *dst_k, *dst_v;         // pools written (may be the same pools)
    const int64_t *block_pairs;  // [num_pairs][2] (src, dst)
    int64_t num_pairs;
    int64_t src_blocks, dst_blocks;  // blocks in the source / destination pools
    int64_t block_bytes;         // 16 * Hkv * head_dim * element bytes
    int64_t pieces;              // copy_pieces(block_bytes)
};
// 16 KiB pieces (one work-group each) of one block of one pool
int64_t copy_pieces(int64_t block_bytes);
hipError_t launch_copy_blocks(const CopyArgs &a, hipStream_t stream);

struct DecodeArgs {
    float *out;
    const void *q;
    const void *k_cache, *v_cache;
    const int32_t *block_tables, *context_lens;
    int num_seqs, num_q_heads, num_kv_heads, head_dim;
    int max_blocks;        // width of a block table row (entries)
    int tbs_log2;          // an entry names 2^tbs_log2 consecutive 16-token units; -1: an
                           // entry names one 8-token block (a unit is two entries)
    int64_t num_blocks;    // pool size in 16-token units (8-token blocks when tbs_log2 < 0)
    int cache_dtype;
    int part_blocks;       // 0: balanced split; else fixed partitions (16-token units)
    int grid;              // persistent work-group count
    float qk_scale;        // softmax scale * log2(e) (* kv_scale for fp8 K)
    float v_scale;         // 1, or kv_scale for fp8 V
    float *ws_acc;         // [records][G][D]
    float *ws_ml;          // [records][G][2]
    int32_t *ws_count;     // arrival counters (at most S * Hkv), zero between calls
};
// Arrival counters sit at the start of every decode workspace; this region
// must be zero before the first call and every call leaves it zero.
constexpr int64_t kDecodeCounterSlots = 1 << 20;
// Number of partial-result records the decode workspace must hold.
int64_t decode_partial_slots(int num_seqs, int num_kv_heads, int group, int max_blocks,
                             int part_blocks, int grid, int tbs_log2);
bool decode_supported(int cache_dtype, int head_dim, int group);
struct DecodeKernels {
    const void *main;    // persistent split-K decode kernel (merges its own partials)
    int threads;         // work-group size
};
// KV heads one decode work-group serves: 4 (the head-group kernel) when the
// model has at least two groups of four KV heads and G >= 2 and blocks hold 16
// or more tokens (tbs_log2 >= 0), else 1.
int decode_hpg(int num_kv_heads, int group, int tbs_log2);
// h8: the one-KV-head kernel built for 8-token blocks
DecodeKernels decode_kernels(int cache_dtype, int head_dim, int group, int hpg, bool h8);
// the head-group kernels (decode_hg4.hip)
DecodeKernels decode_hg4_kernels(int cache_dtype, int head_dim, int group);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

struct PrefillArgs {
    float *out;
    const void *q;
    const void *k_cache, *v_cache;
    const int32_t *block_tables, *query_start, *context_lens;
    int64_t total_rows;
    int num_reqs, num_q_heads, num_kv_heads, head_dim;
    int max_blocks;        // width of a block table row (entries)
    int tbs_log2;          // an entry names 2^tbs_log2 consecutive 16-token units; -1: an
                           // entry names one 8-token block (a unit is two entries)
    int64_t num_blocks;    // pool size in 16-token units (8-token blocks when tbs_log2 < 0)
    int cache_dtype;
    int kv_splits;
    int m_tiles;           // row tiles per (request, KV head), from the largest chunk
    float qk_scale, v_scale;
    float *ws_acc;         // [kv_splits][rows*Hq][D]
    float *ws_ml;          // [kv_splits][rows*Hq][2]
};
bool prefill_supported(int cache_dtype, int head_dim, int group);
// Key-range splits of a prefill call: enough (row tile, KV head, split)
// work-groups to give each of the device's `cus` compute units one, at most 16.
int prefill_kv_splits(int64_t total_rows, int num_q_heads, int cus);
int prefill_m_tiles(int64_t total_rows, int num_q_heads, int num_kv_heads);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

}  // namespace pa
