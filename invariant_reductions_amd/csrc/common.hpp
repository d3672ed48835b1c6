// common.hpp -- device helpers shared by the gfx950 kernels of libbi.
//
// Everything here is HIP for CDNA4 (wave64, MFMA).  No host fallback exists:
// the library is built for gfx950 only.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bi.h"

namespace bi {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
struct BF16 {
    using store_t = uint16_t;
    static constexpr int kElemsPer16B = 8;
    __device__ static inline float widen(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
    __device__ static inline uint16_t narrow(float f) {
        __bf16 h = (__bf16)f;                       // v_cvt_pk_bf16_f32: round to nearest even
        return __builtin_bit_cast(uint16_t, h);
    }
};
struct F16 {
    using store_t = uint16_t;
    static constexpr int kElemsPer16B = 8;
    __device__ static inline float widen(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
    __device__ static inline uint16_t narrow(float f) {
        _Float16 h = (_Float16)f;                   // v_cvt_f16_f32: round to nearest even
        return __builtin_bit_cast(uint16_t, h);
    }
};
struct F32 {
    using store_t = float;
    static constexpr int kElemsPer16B = 4;
    __device__ static inline float widen(float b) { return b; }
    __device__ static inline float narrow(float f) { return f; }
};

// ---------------------------------------------------------------------------
// bounded 16-byte chunk loads
// ---------------------------------------------------------------------------
// Loads elements [k, k + E) of a row (E = 16 bytes worth of elements), with
// every element at index >= limit, or the whole chunk when !ok, read as zero.
// VEC: the caller guarantees that a chunk is either entirely below `limit` or
// entirely at/above it and that the address is 16-byte aligned.
template <typename S, bool VEC>
__device__ inline uint4 load_chunk(const typename S::store_t *row, int64_t k, int64_t limit, bool ok)
{
    constexpr int E = S::kElemsPer16B;
    uint4 r = make_uint4(0, 0, 0, 0);
    if (VEC) {
        if (ok && k < limit) r = *reinterpret_cast<const uint4 *>(row + k);
    } else {
        typename S::store_t tmp[E];
#pragma unroll
        for (int e = 0; e < E; ++e) tmp[e] = (ok && k + e < limit) ? row[k + e] : (typename S::store_t)0;
        r = __builtin_bit_cast(uint4, tmp);
    }
    return r;
}

// SwiGLU activation of one bf16 pair: RNE(silu(g) * u) with
// silu(g) = g / (1 + exp(-g)), every step in fp32.  One definition for the
// stand-alone kernel and the fused matmul epilogue, so both give these bits.
__device__ inline uint16_t silu_mul1(uint16_t gb, uint16_t ub)
{
    const float g = BF16::widen(gb), u = BF16::widen(ub);
    const float sg = g / (1.0f + expf(-g));
    return BF16::narrow(sg * u);
}

// Calls f(std::integral_constant<int, I>{}) for I = B .. E-1: the index is a
// compile-time constant inside f, so register arrays indexed by it stay in
// registers.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Index of the calling wavefront within its workgroup, as a scalar (the
// compiler then treats loops and branches that depend on it as uniform).
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline bool host_aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// One-shot launch timing: when set (bi_time_next_launch), the next kernel
// the library launches on this host thread records `start` as it begins
// executing and `stop` as it ends (hipExtLaunchKernel), so the pair brackets
// the kernel itself rather than its dispatch.
// Measurement hook: the next `count` kernel launches of the calling thread
// carry `start` (recorded as the first one starts) and `stop` (as the last
// one ends), through the extended launch.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
    int count = 0;
};
inline LaunchTiming &launch_timing()
{
    static thread_local LaunchTiming t;
    return t;
}
template <typename... Params, typename... Args>
inline void launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, size_t smem, hipStream_t st,
                          Args... args)
{
    LaunchTiming &t = launch_timing();
    if (t.count > 0) {
        hipEvent_t start = t.start, stop = nullptr;
        t.start = nullptr;
        if (--t.count == 0) {
            stop = t.stop;
            t = LaunchTiming{};
        }
        hipExtLaunchKernelGGL(kernel, grid, block, smem, st, start, stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, smem, st, args...);
    }
}

// Compute units of the current device (cached per device; 256 if unknown).
inline int device_cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
        cached[dev] = cu;                       // benign race: every writer stores the same value
    }
    return cached[dev];
}

inline bi_status launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? BI_OK : BI_ERR_LAUNCH;
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace bi
