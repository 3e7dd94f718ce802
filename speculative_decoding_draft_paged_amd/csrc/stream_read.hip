// Read-only streaming reference: the HBM read rate a plain kernel reaches on this GPU, the yardstick
// the attention kernels' KV read rate is compared with. Every byte of the source is read once with
// the same 16-byte non-temporal vector loads the attention kernels use for K and V, each workgroup
// walking a contiguous range; the loaded words are folded by XOR into one 32-bit result so no load
// can be dropped, and nothing else is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "blockattn.h"
#include "internal.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // independent 16-byte loads in flight per lane: 32 KB per workgroup

// Workgroup w reads its own contiguous range of the buffer, 32 KB at a time (each wave 1 KB per
// load instruction), as an attention work unit walks its key range.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* src, int64_t n16, int64_t chunk,
                                                               uint32_t* result) {
    const int64_t begin = (int64_t)blockIdx.x * chunk;
    const int64_t end = begin + chunk < n16 ? begin + chunk : n16;
    uint32_t acc = 0;
    int64_t i = begin + threadIdx.x;
    for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * kThreads);
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < end; i += kThreads) {
        const u32x4_t v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_xor(result, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

extern "C" int blockattn_stream_read(const void* src, size_t bytes, uint32_t* result, int32_t workgroups,
                                     void* stream) {
    if (!src || !result || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
        return blockattn::record_error(BLOCKATTN_ERR_INVALID_ARGUMENT,
                                       "src and result are required; src 16-byte aligned, bytes a positive multiple of 16");
    if (workgroups < 0 || workgroups > (1 << 20))
        return blockattn::record_error(BLOCKATTN_ERR_INVALID_ARGUMENT, "workgroups must be in [0, 2^20] (0: automatic)");
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t max_wg = (n16 + kThreads - 1) / kThreads;
    int64_t wg = workgroups > 0 ? workgroups : 1024;  // four 256-thread workgroups per compute unit
    if (wg > max_wg) wg = max_wg;
    const int64_t chunk = (n16 + wg - 1) / wg;  // 16-byte vectors per workgroup
    wg = (n16 + chunk - 1) / chunk;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)wg), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t*>(src), n16, chunk, result);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return blockattn::record_error(BLOCKATTN_ERR_HIP, hipGetErrorString(e));
    return blockattn::record_error(BLOCKATTN_OK, "");
}
