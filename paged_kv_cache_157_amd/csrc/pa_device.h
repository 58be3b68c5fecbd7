// pa_device.h -- device-side building blocks shared by the HIP kernels of
// libpa (gfx950 / CDNA4, wave64).  Product code: nothing here is used by, or
// uses, the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Storage types (same numbering as pa_dtype in include/pa.h).
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

template <int DT>
struct Storage {
    static constexpr int bytes = DT == DT_F32 ? 4 : DT == DT_BF16 ? 2 : 1;
    static constexpr int per16 = 16 / bytes;  // elements in one 16-byte chunk
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

static constexpr float kLog2e = 1.4426950408889634f;

// bf16 halves of a packed dword, widened to fp32 exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// v_dot2_f32_bf16: a.lo*b.lo + a.hi*b.hi + c, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// Two OCP E4M3 bytes (low or high half of a dword) -> two bf16, exactly.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Two OCP E4M3 bytes -> two fp32, exactly.
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32x2(uint32_t w)
{
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// ---------------------------------------------------------------------------
// DPP lane exchange inside 16-lane rows (all row/bank masks enabled).
// ---------------------------------------------------------------------------
enum : int {
    DPP_QP_X1 = 0xB1,        // quad_perm [1,0,3,2]: partner lane ^ 1
    DPP_QP_X2 = 0x4E,        // quad_perm [2,3,0,1]: partner lane ^ 2
    DPP_ROW_ROR4 = 0x124,    // lane (l + 4) mod 16 within the row
    DPP_ROW_ROR8 = 0x128,    // lane (l + 8) mod 16 = l ^ 8 within the row
    DPP_HALF_MIRROR = 0x141, // lane l ^ 7 within each half row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T uniform(T v)
{
    return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ long long uniform64(long long v)
{
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return (long long)(((uint64_t)hi << 32) | lo);
}

// Read-only view of a global array through the constant address space: loads
// at wave-uniform indices become scalar loads (counted by lgkmcnt, not vmcnt).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *scalar_view(const T *p)
{
    return (const __attribute__((address_space(4))) T *)p;
}

// Make the compiler materialise a loaded value here (waiting for its load).
__device__ __forceinline__ void settle(uint32_t v) { asm volatile("" ::"v"(v)); }

// Device-coherent accesses: agent-scope relaxed atomics, which gfx950 performs
// at the coherence point shared by all XCDs (no L2 write-back or invalidate).
__device__ __forceinline__ void coherent_store(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two floats at once (p 8-byte aligned), device-coherent as above.
__device__ __forceinline__ void coherent_store2(float *p, float x, float y)
{
    const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
    __hip_atomic_store((uint64_t *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 coherent_load2(const float *p)
{
    const uint64_t v = __hip_atomic_load((const uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
