// Measurement support: a reference streaming read, for benchmarks that put
// the linear kernels' launches next to a kernel that only moves the same
// bytes (and, with zero bytes, next to the cost of a launch itself).  Not a
// step of the method.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "q4_0_internal.h"

namespace q4 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadPieces = 16;   // 16-byte pieces per thread: 64 KiB per workgroup

// Workgroup b reads its 64 KiB (nontemporal 16-byte loads, all issued before
// any is used; load p of thread t reads 16-byte chunk 4096 b + 256 p + t)
// and each thread writes the XOR of its 32-bit words to sink, so the loads
// cannot be removed.  Nothing else follows the loads: no cross-lane fold,
// LDS or barrier, which would keep the last workgroups of a launch busy
// after their data has arrived (a serial fold over the threads' words did,
// by about a microsecond per launch).  The sink adds 1/64 of the bytes read
// as writes.
__global__ __launch_bounds__(kReadThreads) void reference_read_kernel(const u32x4 *__restrict__ src, int64_t n16,
                                                                      uint32_t *__restrict__ sink) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kReadThreads * kReadPieces + threadIdx.x;
    u32x4 v[kReadPieces];
#pragma unroll
    for (int p = 0; p < kReadPieces; ++p) {
        const int64_t i = base + static_cast<int64_t>(p) * kReadThreads;
        v[p] = i < n16 ? __builtin_nontemporal_load(src + i) : (u32x4){0u, 0u, 0u, 0u};
    }
    uint32_t f = 0;
#pragma unroll
    for (int p = 0; p < kReadPieces; ++p) f ^= v[p].x ^ v[p].y ^ v[p].z ^ v[p].w;
    sink[static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x] = f;
}

}  // namespace

int64_t reference_read_workgroups(int64_t bytes) {
    const int64_t per = static_cast<int64_t>(kReadThreads) * kReadPieces * 16;
    return bytes == 0 ? 1 : (bytes + per - 1) / per;
}

int64_t reference_read_sink_words(int64_t bytes) { return reference_read_workgroups(bytes) * kReadThreads; }

hipError_t launch_reference_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
    const int64_t grid = reference_read_workgroups(bytes);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipEvent_t start = nullptr, stop = nullptr;
    if (take_launch_events(start, stop)) {
        hipExtLaunchKernelGGL(reference_read_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kReadThreads), 0, s,
                              start, stop, 0, static_cast<const u32x4 *>(src), bytes / 16, sink);
    } else {
        hipLaunchKernelGGL(reference_read_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kReadThreads), 0, s,
                           static_cast<const u32x4 *>(src), bytes / 16, sink);
    }
    return hipGetLastError();
}

}  // namespace q4
