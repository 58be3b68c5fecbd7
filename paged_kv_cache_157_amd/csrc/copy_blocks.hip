// copy_blocks.hip -- copy whole KV blocks between pools: inside the device
// pools, the device half of copy-on-write ("Lecture 33" §2.4: a sequence that
// writes into a block other sequences still reference first gets a private
// copy of it); between the device pools and pools in pinned host memory,
// swapping a preempted request's blocks out and back in ("Lecture 33" §5.2:
// the blocks cross PCIe to host memory and return when there is room).
//
// A work-group copies one 16 KiB piece of one block of one pool (K or V) at
// a time: every thread moves four 16-byte words, all loads issued before any
// store.  Pieces of a block, both pools and all pairs are independent units
// spread over the grid, so a batch of copies fills the chip; the pair is
// read through the scalar path.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kCopyThreads = 256;
constexpr int kCopyWords = 4;  // 16-byte words per thread
constexpr int64_t kCopyPiece = (int64_t)kCopyThreads * kCopyWords * 16;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a)
{
    const int64_t per_pair = 2 * a.pieces;
    const int64_t units = a.num_pairs * per_pair;
    const auto pairs = scalar_view(a.block_pairs);
    // one unit (pair, pool, piece) per work-group and round
    for (int64_t id = blockIdx.x; id < units; id += gridDim.x) {
        const int64_t p = id / per_pair;
        const int64_t r = id - p * per_pair;
        const int side = r >= a.pieces;  // 0: K pool, 1: V pool
        const int64_t piece = side ? r - a.pieces : r;
        const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
        if (src < 0 || src >= a.src_blocks || dst < 0 || dst >= a.dst_blocks)
            continue;  // pairs naming a block outside its pool are skipped
        const char *sp = (const char *)(side ? a.src_v : a.src_k);
        char *dp = (char *)(side ? a.dst_v : a.dst_k);
        const int64_t off = piece * kCopyPiece;
        const u32x4 *s = (const u32x4 *)(sp + src * a.block_bytes + off);
        u32x4 *d = (u32x4 *)(dp + dst * a.block_bytes + off);
        const int64_t words = (a.block_bytes - off) / 16;  // this block's words from the piece on
        u32x4 t[kCopyWords];
#pragma unroll
        for (int u = 0; u < kCopyWords; ++u) {
            const int64_t wdx = (int64_t)u * kCopyThreads + threadIdx.x;
            if (wdx < words)
                t[u] = s[wdx];
        }
#pragma unroll
        for (int u = 0; u < kCopyWords; ++u) {
            const int64_t wdx = (int64_t)u * kCopyThreads + threadIdx.x;
            if (wdx < words)
                d[wdx] = t[u];
        }
    }
}

int64_t copy_pieces(int64_t block_bytes) { return (block_bytes + kCopyPiece - 1) / kCopyPiece; }

hipError_t launch_copy_blocks(const CopyArgs &a, hipStream_t stream)
{
    const int64_t units = a.num_pairs * 2 * a.pieces;
    if (units == 0)
        return hipSuccess;
    // at most 64 Ki work-groups (256 per compute unit); larger batches loop
    const unsigned groups = (unsigned)(units < 65536 ? units : 65536);
    copy_blocks_kernel<<<dim3(groups), kCopyThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace pa
