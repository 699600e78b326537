// Measurement helper: a plain streaming device copy, the reference against
// which the kernels' achieved HBM bandwidth is compared (a measured peak next
// to the datasheet's 8 TB/s).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte accesses in flight per thread

// Every thread moves kCopyUnroll 16-byte pieces per round, the pieces of one
// round kCopyThreads apart (each wave's accesses are contiguous 1 KiB runs);
// rounds stride over the whole grid.  Nontemporal loads and stores: the data
// is streamed once.
__global__ void __launch_bounds__(kCopyThreads) stream_copy_kernel(u32x4_t* __restrict__ dst,
                                                                   const u32x4_t* __restrict__ src, int64_t n) {
    const int64_t step = int64_t(gridDim.x) * kCopyThreads * kCopyUnroll;
    for (int64_t base = int64_t(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x; base < n; base += step) {
        u32x4_t v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; u++) {
            const int64_t i = base + int64_t(u) * kCopyThreads;
            if (i < n) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; u++) {
            const int64_t i = base + int64_t(u) * kCopyThreads;
            if (i < n) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

}  // namespace

hipError_t launch_stream_copy(void* dst, const void* src, int64_t n16, int blocks, hipStream_t stream) {
    stream_copy_kernel<<<dim3(unsigned(blocks)), dim3(kCopyThreads), 0, stream>>>(
        static_cast<u32x4_t*>(dst), static_cast<const u32x4_t*>(src), n16);
    return hipGetLastError();
}

}  // namespace gdn
