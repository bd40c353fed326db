// Bandwidth probe: the device's own read, write and copy rates, against which
// the parse and lex kernels' HBM traffic is measured. Not part of the method.
//
// Each kernel streams 16-byte words with a grid-stride loop, four loads or
// stores in flight per lane. Access pattern 0: wave-contiguous (lane l of a
// wave touches word base + l, so one instruction covers 1 KiB); pattern 1: 64
// contiguous bytes per lane (four consecutive words, the layout the CSV codes
// kernel reads its chunks in); pattern 2: wave-contiguous 4-byte words (one
// instruction covers 256 bytes, sixteen per lane in flight: the shape of the
// field and token stores).
#include <hip/hip_runtime.h>

#include "ppr.h"

namespace ppr {
namespace {

constexpr int kProbeBlock = 256;

template <int PAT>
__device__ __forceinline__ uint64_t word_index(uint64_t group, int j)
{
    // group = index of a run of 4 * kProbeBlock words handled by one workgroup pass
    if (PAT == 0) return group * 4 * kProbeBlock + (uint64_t)j * kProbeBlock + threadIdx.x;
    return group * 4 * kProbeBlock + (uint64_t)threadIdx.x * 4 + j;
}

template <int PAT>
__global__ void __launch_bounds__(kProbeBlock) probe_read_kernel(const uint4* src, uint64_t groups, uint32_t* sink)
{
    uint32_t acc = 0;
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
        uint4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = src[word_index<PAT>(g, j)];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc ^= x[j].x ^ x[j].y ^ x[j].z ^ x[j].w;
    }
    sink[(uint64_t)blockIdx.x * kProbeBlock + threadIdx.x] = acc;
}

template <int PAT>
__global__ void __launch_bounds__(kProbeBlock) probe_write_kernel(uint4* dst, uint64_t groups, uint32_t v)
{
    const uint4 x = make_uint4(v, v + 1, v + 2, v + 3);
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[word_index<PAT>(g, j)] = x;
    }
}

template <int PAT>
__global__ void __launch_bounds__(kProbeBlock) probe_copy_kernel(const uint4* src, uint4* dst, uint64_t groups)
{
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
        uint4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = src[word_index<PAT>(g, j)];
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[word_index<PAT>(g, j)] = x[j];
    }
}


// pattern 2: a pass covers the same 16 KiB per workgroup as the others, as
// 4-byte words: lane l touches word base + 256 j + l, j = 0..15
__device__ __forceinline__ uint64_t dword_index(uint64_t group, int j)
{
    return group * 16 * kProbeBlock + (uint64_t)j * kProbeBlock + threadIdx.x;
}

__global__ void __launch_bounds__(kProbeBlock) probe_read4_kernel(const uint32_t* src, uint64_t groups, uint32_t* sink)
{
    uint32_t acc = 0;
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
        uint32_t x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = src[dword_index(g, j)];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc ^= x[j];
    }
    sink[(uint64_t)blockIdx.x * kProbeBlock + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(kProbeBlock) probe_write4_kernel(uint32_t* dst, uint64_t groups, uint32_t v)
{
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[dword_index(g, j)] = v + (uint32_t)j;
    }
}

__global__ void __launch_bounds__(kProbeBlock) probe_copy4_kernel(const uint32_t* src, uint32_t* dst, uint64_t groups)
{
    for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
        uint32_t x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = src[dword_index(g, j)];
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[dword_index(g, j)] = x[j];
    }
}

}  // namespace
}  // namespace ppr

extern "C" PPR_API int ppr_bandwidth_probe(uint32_t mode, uint32_t pattern, const void* d_src, void* d_dst,
                                           uint64_t bytes, uint32_t grid, void* stream)
{
    using namespace ppr;
    const uint64_t gbytes = 16ull * 4 * kProbeBlock;
    if (bytes == 0 || bytes % gbytes || grid == 0 || mode > 2 || pattern > 2) return PPR_EINVAL;
    if ((mode != 1 && !d_src) || !d_dst) return PPR_EINVAL;
    if ((((uintptr_t)d_src) & 15u) || (((uintptr_t)d_dst) & 15u)) return PPR_EINVAL;
    const uint64_t groups = bytes / gbytes;
    hipStream_t s = (hipStream_t)stream;
    const uint4* src = (const uint4*)d_src;
    uint4* dst = (uint4*)d_dst;
    if (pattern == 2) {
        const uint32_t* src4 = (const uint32_t*)d_src;
        uint32_t* dst4 = (uint32_t*)d_dst;
        if (mode == 0) hipLaunchKernelGGL(probe_read4_kernel, dim3(grid), dim3(kProbeBlock), 0, s, src4, groups, dst4);
        else if (mode == 1) hipLaunchKernelGGL(probe_write4_kernel, dim3(grid), dim3(kProbeBlock), 0, s, dst4, groups, 7u);
        else hipLaunchKernelGGL(probe_copy4_kernel, dim3(grid), dim3(kProbeBlock), 0, s, src4, dst4, groups);
    } else if (mode == 0) {
        if (pattern == 0) hipLaunchKernelGGL(probe_read_kernel<0>, dim3(grid), dim3(kProbeBlock), 0, s, src, groups, (uint32_t*)d_dst);
        else hipLaunchKernelGGL(probe_read_kernel<1>, dim3(grid), dim3(kProbeBlock), 0, s, src, groups, (uint32_t*)d_dst);
    } else if (mode == 1) {
        if (pattern == 0) hipLaunchKernelGGL(probe_write_kernel<0>, dim3(grid), dim3(kProbeBlock), 0, s, dst, groups, 7u);
        else hipLaunchKernelGGL(probe_write_kernel<1>, dim3(grid), dim3(kProbeBlock), 0, s, dst, groups, 7u);
    } else {
        if (pattern == 0) hipLaunchKernelGGL(probe_copy_kernel<0>, dim3(grid), dim3(kProbeBlock), 0, s, src, dst, groups);
        else hipLaunchKernelGGL(probe_copy_kernel<1>, dim3(grid), dim3(kProbeBlock), 0, s, src, dst, groups);
    }
    return hipGetLastError() == hipSuccess ? PPR_OK : PPR_EHIP;
}
