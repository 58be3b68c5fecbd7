// reshape.hip -- cache write: scatter this step's new K/V rows into their
// pool slots ("Lecture 33" §2.1 and §4.2; "PagedAttention: managing the KV
// cache like virtual memory" §3.3: the new token fills the last block).
//
// One thread moves 8 consecutive elements of one K or V row.  The slot index
// is read once per row by every thread of that row (L2-resident), the source
// read and the destination write are 16- or 32-byte vector accesses.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Saturating fp32 -> OCP E4M3FN with round-to-nearest-even (hardware
// v_cvt_pk_fp8_f32 after clamping to +-448); NaN keeps its sign.
__device__ __forceinline__ uint32_t encode_fp8x4(float a, float b, float c, float d)
{
    float x[4] = {a, b, c, d};
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        y[i] = fminf(fmaxf(x[i], -448.0f), 448.0f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    int both = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    uint32_t w = (uint32_t)both;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (__builtin_isnan(x[i])) {
            uint32_t code = 0x7Fu | ((__float_as_uint(x[i]) >> 24) & 0x80u);
            w = (w & ~(0xFFu << (8 * i))) | (code << (8 * i));
        }
    }
    return w;
}

template <int SRC, int DST>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(ReshapeArgs a)
{
    const int groups = a.row_elems >> 3;  // 8-element groups per row
    const int64_t per_side = a.num_tokens * groups;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= 2 * per_side)
        return;
    const int side = gid >= per_side;
    const int64_t r = side ? gid - per_side : gid;
    const int64_t n = r / groups;
    const int e8 = (int)(r - n * groups);
    const int64_t slot = a.slot_mapping[n];
    if (slot < 0 || slot >= a.num_slots)
        return;
    const int64_t src_elem = n * a.row_elems + (int64_t)e8 * 8;
    const int64_t dst_elem = slot * a.row_elems + (int64_t)e8 * 8;
    const char *src = (const char *)(side ? a.v : a.k);
    char *dst = (char *)(side ? a.v_cache : a.k_cache);

    if constexpr (SRC == DT_F32 && DST == DT_F32) {
        const u32x4 *s = (const u32x4 *)(src + src_elem * 4);
        u32x4 *d = (u32x4 *)(dst + dst_elem * 4);
        u32x4 v0 = s[0], v1 = s[1];
        d[0] = v0;
        d[1] = v1;
    } else if constexpr (SRC == DT_BF16 && DST == DT_BF16) {
        *(u32x4 *)(dst + dst_elem * 2) = *(const u32x4 *)(src + src_elem * 2);
    } else {  // bf16 -> fp8
        u32x4 w = *(const u32x4 *)(src + src_elem * 2);
        const float s = a.inv_scale;
        uint32_t lo = encode_fp8x4(bf16_lo(w[0]) * s, bf16_hi(w[0]) * s, bf16_lo(w[1]) * s,
                                   bf16_hi(w[1]) * s);
        uint32_t hi = encode_fp8x4(bf16_lo(w[2]) * s, bf16_hi(w[2]) * s, bf16_lo(w[3]) * s,
                                   bf16_hi(w[3]) * s);
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
        *(u32x2 *)(dst + dst_elem) = u32x2{lo, hi};
    }
}

hipError_t launch_reshape_and_cache(const ReshapeArgs &a, hipStream_t stream)
{
    const int64_t threads = 2 * a.num_tokens * (a.row_elems / 8);
    if (threads == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (a.src_dtype == DT_F32 && a.cache_dtype == DT_F32)
        reshape_and_cache_kernel<DT_F32, DT_F32><<<blocks, 256, 0, stream>>>(a);
    else if (a.src_dtype == DT_BF16 && a.cache_dtype == DT_BF16)
        reshape_and_cache_kernel<DT_BF16, DT_BF16><<<blocks, 256, 0, stream>>>(a);
    else
        reshape_and_cache_kernel<DT_BF16, DT_FP8><<<blocks, 256, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace pa
