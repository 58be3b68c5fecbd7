/*
 * pa.h -- C ABI of libpa: paged KV-cache attention kernels for MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [L33] "Lecture 33: KV Cache memory management -- PagedAttention,
 *         Continuous Batching and Chunked Prefill" (lilinji.mintlify.site)
 *   [VM]  "PagedAttention: managing the KV cache like virtual memory"
 *         (inference-learning-path.pages.dev, Part 5)
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller.  Arrays are
 *     dense, row-major, with no padding between rows.
 *   - KV pool ([L33] §2.2: one tensor allocated once, holding every physical
 *     block): K and V are each [num_blocks, 16, num_kv_heads, head_dim].
 *     Token slot s = physical_block * 16 + offset; element (s, g, c) is at
 *     index (s * num_kv_heads + g) * head_dim + c.
 *   - block_tables: [num_seqs, max_blocks_per_seq] int32; entry [i][b] is the
 *     physical block of logical block b of sequence i ([L33] §2.2 walk-through,
 *     token t -> logical block t / 16, offset t % 16).  Only the first
 *     ceil(context_len / 16) entries of a row are read.
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - Softmax: out = softmax(scale * q K^T) V, with no bias, window or cap.
 *   - fp8 KV (PA_FP8_E4M3) is OCP E4M3FN: stored code = RNE(saturate(x / s))
 *     with the reciprocal 1/s and the product taken in fp32; value = code * s,
 *     s = kv_scale ([VM] §3.1 and §9 name an fp8 KV cache; the format is a
 *     reading).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream): it does no host synchronisation and no device-to-host copy.
 *   - Errors: shapes, dtypes, pointers and workspace sizes are checked on the
 *     host before any launch; PA_ERR_INVALID / PA_ERR_UNSUPPORTED /
 *     PA_ERR_WORKSPACE are returned without touching the device.  A failed
 *     launch returns PA_ERR_HIP.  pa_last_error() then holds a description
 *     (thread-local).  No C++ exception crosses this interface.
 *   - Caller preconditions that would need a device sync to check (not
 *     checked): 0 <= context_len <= 16 * max_blocks_per_seq; the table entries
 *     that are read lie in [0, num_blocks); non-negative slot_mapping entries
 *     are distinct.  Kernels skip cache writes whose slot is out of range.
 *   - The library allocates no device memory.  Scratch space is passed in as
 *     `workspace`, sized by the matching *_workspace_bytes() call.
 *   - Process-wide state: none that a call's data passes through.  The
 *     library memoises two device properties per device id (its compute-unit
 *     count, and how many work-groups of each decode kernel fit on a compute
 *     unit), in write-once tables guarded by a mutex; the decode grid, the
 *     prefill key split and the workspace sizes are derived from them, so
 *     they depend on the device the call runs on.  Every entry point may be
 *     called from several host threads at once.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID = 1,     /* bad pointer, size or combination            */
    PA_ERR_UNSUPPORTED = 2, /* valid but not built (head_dim, GQA ratio...) */
    PA_ERR_WORKSPACE = 3,   /* workspace missing or too small              */
    PA_ERR_HIP = 4          /* a HIP runtime call failed                   */
} pa_status;

typedef enum {
    PA_F32 = 0,      /* IEEE binary32                 */
    PA_BF16 = 1,     /* bfloat16                      */
    PA_FP8_E4M3 = 2  /* OCP E4M3FN, per-tensor scale  */
} pa_dtype;

/* Problem geometry shared by the calls. */
typedef struct {
    int32_t num_seqs;           /* decode: sequences S; prefill: requests R          */
    int32_t num_q_heads;        /* Hq                                                */
    int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 8              */
    int32_t head_dim;           /* d: 64 or 128 (f32 cache: 64 only)                 */
    int64_t num_blocks;         /* N physical blocks of block_size token slots       */
    int32_t max_blocks_per_seq; /* width of block_tables                             */
    int32_t q_dtype;            /* pa_dtype of q: PA_F32 with an f32 cache, else BF16 */
    int32_t cache_dtype;        /* pa_dtype of the pools                             */
    float kv_scale;             /* fp8 cache only: value = code * kv_scale (> 0)     */
    int32_t partition_tokens;   /* decode split-K: 0 = balanced split over the whole
                                   GPU, else fixed partitions of this many tokens
                                   (a multiple of 16)                               */
    int32_t block_size;         /* tokens per block: 8, 16 (0 also means 16), 32 or
                                   64; [L33] §2.2: token t of a sequence lives in slot
                                   table[t / block_size] * block_size
                                   + t % block_size.  With 8, decode always runs the
                                   one-KV-head kernel                                */
} pa_shape;

/*
 * pa_reshape_and_cache -- write this step's new K/V rows into their slots.
 *   [VM] §3.3: each new token fills the last block of its sequence (a new
 *   block when that one is full); [L33] §4.2: a prefill chunk's KV is written
 *   to the cache before later chunks use it as history.
 *   k, v:          [num_tokens, num_kv_heads, head_dim] of type src_dtype
 *                  (PA_F32 for an f32 cache, PA_BF16 for bf16 and fp8 caches)
 *   k_cache, v_cache: pools as above, of type shape->cache_dtype
 *   slot_mapping:  [num_tokens] int64; row n goes to slot slot_mapping[n];
 *                  a negative entry skips row n.
 *   Result: K/V pool rows of the mapped slots are overwritten (fp8: quantised
 *   as stated above); every other byte is left untouched.
 *   num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(const void *k, const void *v, void *k_cache, void *v_cache,
                               const int64_t *slot_mapping, int64_t num_tokens,
                               int32_t src_dtype, const pa_shape *shape, void *stream);

/*
 * pa_copy_blocks -- copy whole KV blocks inside both pools (copy-on-write).
 *   [L33] §2.4: before a sequence writes into a block that other sequences
 *   still reference (ref_cnt > 1), the block is copied to a private one and
 *   the writer's table points there; [VM] §3.4 the same for a forked prefix.
 *   k_cache, v_cache: the pools, [num_blocks, 16, num_kv_heads, head_dim]
 *   block_pairs:   [num_pairs, 2] int64 device array of (src, dst) block ids;
 *                  k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src]
 *   The copies run concurrently: dst ids must be distinct and no dst may be
 *   the src of another pair (else the result is unspecified).  A pair with
 *   an id outside [0, num_blocks) is skipped.  The shape is validated as for
 *   pa_reshape_and_cache; the copy uses its num_blocks, num_kv_heads,
 *   head_dim and cache_dtype.  num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int64_t *block_pairs,
                         int64_t num_pairs, const pa_shape *shape, void *stream);

/*
 * pa_swap_blocks -- move whole KV blocks between pools in different memories.
 *   [L33] §5.2: a preempted request's blocks are copied over PCIe to host
 *   memory, its device blocks freed, and copied back into free device blocks
 *   when it resumes ([L33] §5.4 prices a round trip at
 *   2 * S * KV_token / B_pcie).  One launch moves every pair; the GPU reads
 *   or writes host memory directly.
 *   src_k, src_v:  source pools, [src_num_blocks, 16, num_kv_heads, head_dim]
 *   dst_k, dst_v:  destination pools, [dst_num_blocks, 16, num_kv_heads, head_dim]
 *   block_pairs:   [num_pairs, 2] int64 (src, dst) block ids
 *   Every pointer must be device memory of the current device or pinned
 *   host memory (hipHostMalloc; torch's pin_memory); anything else gives
 *   PA_ERR_INVALID before any launch.  Pairs with an id outside its pool
 *   are skipped; dst ids must be distinct (the copies run concurrently).
 *   Pinned host buffers must stay allocated until the stream has finished
 *   the call.  The shape is validated as for pa_reshape_and_cache; its
 *   num_kv_heads, head_dim and cache_dtype give the block size.
 */
pa_status pa_swap_blocks(const void *src_k, const void *src_v, int64_t src_num_blocks,
                         void *dst_k, void *dst_v, int64_t dst_num_blocks,
                         const int64_t *block_pairs, int64_t num_pairs, const pa_shape *shape,
                         void *stream);

/* Workspace bytes pa_decode needs for this shape (depends on the shape and
 * on the device's compute-unit count only). */
size_t pa_decode_workspace_bytes(const pa_shape *shape);

/*
 * pa_decode -- single-query decode attention over a paged KV cache.
 *   [L33] §2.3: one query per sequence; its K/V blocks are read in place
 *   through the block table (no gather copy), Q K^T, softmax and the weighted
 *   sum of V are formed on chip with a streaming (online) softmax.
 *   out:           [num_seqs, num_q_heads, head_dim] fp32 (written)
 *   q:             [num_seqs, num_q_heads, head_dim] of type shape->q_dtype
 *   block_tables:  [num_seqs, max_blocks_per_seq] int32
 *   context_lens:  [num_seqs] int32, tokens each query attends (its own
 *                  token included, written beforehand); 0 gives a zero row
 *   scale:         softmax scale (1/sqrt(head_dim) in the usual case)
 *   workspace:     device scratch of pa_decode_workspace_bytes(shape) bytes:
 *                  arrival counters (its first 4 MiB), then split-K partial
 *                  results.  The counter region must be zero before the first
 *                  call that uses the buffer; every call leaves it zero again,
 *                  so a buffer zeroed once can be reused by calls of any shape.
 *                  Calls that may run at the same time (on different streams)
 *                  need separate workspaces: they would race on the counters
 *                  and partial results.  Calls queued on one stream may share
 *                  one.  A call that returns an error has launched nothing and
 *                  left the counters as they were; only a kernel aborted in
 *                  flight (a device fault, which ends the HIP context) can
 *                  leave them nonzero, so a workspace from before such a fault
 *                  must be zeroed again before reuse.
 *   A call is one kernel launch: partial results of a sequence split across
 *   work-groups are merged by the work-group that finishes last.
 *   Requires num_seqs * num_kv_heads <= 2^20.
 */
pa_status pa_decode(float *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    const pa_shape *shape, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * pa_decode_static -- pa_decode without a caller workspace, for callers that
 *   cannot allocate device memory (code under HIP graph capture, serving
 *   loops and harnesses that forbid allocation).  Same arguments, result and
 *   errors as pa_decode, minus the workspace: the arrival counters and split-K
 *   partial records live in a static device array of the library (32 MiB per
 *   device, held until the process ends: 1 MiB of counters, then the partial
 *   records).  The call allocates nothing; its first call on a device resolves
 *   the array's address and queues a fill kernel on `stream` that zeroes the
 *   counters, and every call leaves them zero again.
 *   Limits: num_seqs * num_kv_heads <= 2^18, and the shape's partial records
 *   (pa_decode_workspace_bytes(shape) minus its 4 MiB of counters) must fit in
 *   31 MiB, else PA_ERR_WORKSPACE before any launch.  The balanced split
 *   (partition_tokens 0) needs (grid + S*Hkv) * G * (head_dim + 2) * 4 bytes,
 *   a few MB for the usual batches; fixed partitions of long sequences can need
 *   more.  All calls on one device share the array: calls that may overlap in
 *   time (different streams, several host threads) race on it and must not
 *   be issued; calls queued on one stream are safe.
 */
pa_status pa_decode_static(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *context_lens, float scale,
                           const pa_shape *shape, void *stream);

/* Workspace bytes pa_prefill_chunk needs for total_query_rows rows (depends
 * on the shape, the row count and the device's compute-unit count, which
 * sets how many key-range splits the call uses). */
size_t pa_prefill_workspace_bytes(const pa_shape *shape, int64_t total_query_rows);

/*
 * pa_prefill_chunk -- attention of prefill chunks over their paged history.
 *   [L33] §4.2: a long prompt is split into chunks (e.g. 512 tokens); a chunk
 *   is written to the cache and attends to the cached earlier chunks as
 *   history, causally inside itself.
 *   out:           [total_query_rows, num_q_heads, head_dim] fp32 (written)
 *   q:             [total_query_rows, num_q_heads, head_dim] bf16; requests
 *                  stored back to back
 *   block_tables:  [num_seqs (= requests), max_blocks_per_seq] int32
 *   query_start:   [num_seqs + 1] int32 row offsets; request r owns rows
 *                  [query_start[r], query_start[r+1]), n_r rows
 *   context_lens:  [num_seqs] int32 total cached tokens of each request, its
 *                  chunk included (the chunk is written before the call)
 *   scale:         softmax scale, finite and > 0 (else PA_ERR_INVALID)
 *   Row j of request r attends keys [0, context_lens[r] - n_r + j].
 *   Requires a bf16 q, a bf16 or fp8 cache and at most 65535 requests.
 */
pa_status pa_prefill_chunk(float *out, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *query_start,
                           const int32_t *context_lens, int64_t total_query_rows, float scale,
                           const pa_shape *shape, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Static description of a status code. */
const char *pa_status_string(pa_status s);

/* Detail of the last failing call on this host thread ("" if none). */
const char *pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
