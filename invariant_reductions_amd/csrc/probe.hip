// probe.hip -- measurement probes: what this GPU sustains for a plain stream
// of HBM reads, a plain copy, and back-to-back bf16 MFMA.  They compute
// nothing of the library's; bench.py reports every kernel's rate against
// both the published peaks and these measured ones.
#include "common.hpp"

namespace bi {

// Streaming read: workgroup g reads 16-byte words g*256 + t, then every
// gridDim.x*256 words after, eight loads in flight per thread; each
// workgroup folds what it read (xor) into one word of `sink` so that the
// loads cannot be dropped.
__global__ __launch_bounds__(256)
void probe_read_kernel(const uint4 *__restrict__ src, int64_t nwords, uint4 *__restrict__ sink)
{
    uint4 acc = make_uint4(0, 0, 0, 0);
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 7 * stride < nwords; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc.x ^= v[u].x;
            acc.y ^= v[u].y;
            acc.z ^= v[u].z;
            acc.w ^= v[u].w;
        }
    }
    for (; i < nwords; i += stride) {
        const uint4 v = src[i];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    __shared__ uint4 red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint4 r = make_uint4(0, 0, 0, 0);
        for (int t = 0; t < 256; ++t) {
            r.x ^= red[t].x;
            r.y ^= red[t].y;
            r.z ^= red[t].z;
            r.w ^= red[t].w;
        }
        sink[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(256)
void probe_copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t nwords)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < nwords; i += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[i + u * stride] = v[u];
    }
    for (; i < nwords; i += stride) dst[i] = src[i];
}

// bf16 MFMA throughput: every wave issues `iters` rounds of eight
// independent v_mfma_f32_16x16x32_bf16 (2 * 16 * 16 * 32 flops each) on
// register operands, then stores one value per lane so that nothing is
// dropped.
__global__ __launch_bounds__(256)
void probe_mfma_kernel(float *__restrict__ sink, int64_t iters)
{
    const uint32_t seed = threadIdx.x * 2654435761u + blockIdx.x;
    const uint4 a = make_uint4(seed, seed ^ 0x3c003c00u, seed + 7u, seed * 3u);
    const uint4 b = make_uint4(seed ^ 0x40004000u, seed + 1u, seed * 5u, seed ^ 0x11111111u);
    f32x4 acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                             acc[u], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s = s + ((acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]));
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace bi

using namespace bi;

extern "C" bi_status bi_probe_read(const void *src, size_t bytes, void *sink, int32_t workgroups, hipStream_t stream)
{
    if (!src || !sink) return BI_ERR_NULL;
    if (bytes < 16 || bytes % 16 || workgroups < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(src) || !host_aligned16(sink)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    launch_kernel(probe_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, (const uint4 *)src,
                  (int64_t)(bytes / 16), (uint4 *)sink);
    return launch_status();
}

extern "C" bi_status bi_probe_copy(const void *src, void *dst, size_t bytes, int32_t workgroups, hipStream_t stream)
{
    if (!src || !dst) return BI_ERR_NULL;
    if (bytes < 16 || bytes % 16 || workgroups < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(src) || !host_aligned16(dst)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    launch_kernel(probe_copy_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, (const uint4 *)src,
                  (uint4 *)dst, (int64_t)(bytes / 16));
    return launch_status();
}

extern "C" bi_status bi_probe_mfma(void *sink, int32_t workgroups, int64_t iters, hipStream_t stream)
{
    if (!sink) return BI_ERR_NULL;
    if (workgroups < 1 || iters < 1) return BI_ERR_SHAPE;
    (void)hipGetLastError();
    launch_kernel(probe_mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, (float *)sink, iters);
    return launch_status();
}
