// bw_copy.hip -- the plain device copy that bench.py measures beside the HC op,
// as the achievable HBM bandwidth of a streaming kernel on the same GPU (the
// op's roofline is HBM bandwidth). Not part of the op's C ABI; built into a
// library of its own, libds4hc_bw.so.
//
// Each thread copies four 16-byte vectors per grid-stride step with the
// non-temporal cache policy on loads and stores (every byte is touched once).
// On MI355X this reached 6.0 TB/s (read + write bytes) for 1 GiB, against
// ~5.2 TB/s for torch's elementwise copy.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef float f4_t __attribute__((ext_vector_type(4)));
constexpr int BW_THREADS = 256;
constexpr int BW_UNROLL = 4;
constexpr int BW_GRID = 8192;

__global__ __launch_bounds__(BW_THREADS) void bw_copy_kernel(const f4_t *__restrict__ src, f4_t *__restrict__ dst,
                                                             size_t n) {
    const size_t stride = (size_t)gridDim.x * BW_THREADS * BW_UNROLL;
    for (size_t base = (size_t)blockIdx.x * BW_THREADS * BW_UNROLL + threadIdx.x; base < n; base += stride) {
        f4_t v[BW_UNROLL];
#pragma unroll
        for (int u = 0; u < BW_UNROLL; ++u) {
            const size_t i = base + (size_t)u * BW_THREADS;
            if (i < n) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < BW_UNROLL; ++u) {
            const size_t i = base + (size_t)u * BW_THREADS;
            if (i < n) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

}  // namespace

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned device memory)
// from src to dst on `stream`. Returns 0, or a hipError_t code.
extern "C" int ds4hc_bw_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
        return (int)hipErrorInvalidValue;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(bw_copy_kernel, dim3(BW_GRID), dim3(BW_THREADS), 0, stream,
                       static_cast<const f4_t *>(src), static_cast<f4_t *>(dst), bytes / 16);
    return (int)hipGetLastError();
}
