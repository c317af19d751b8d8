// Measurement companion of the fused ShortConv K/V library (not part of its C ABI): a plain
// streaming copy, used by the bench to measure how fast this GPU moves the same number of bytes
// when nothing but moving them is asked for. Each lane copies 4 x 16 bytes with non-temporal loads
// and stores, the fastest plain copy form measured on MI355X.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 4;
constexpr int kBlock = 256;

__global__ void __launch_bounds__(kBlock) copy_nt(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * kBlock * kUnroll + threadIdx.x;
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kBlock;
        if (i < n) r[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kBlock;
        if (i < n) __builtin_nontemporal_store(r[u], dst + i);
    }
}

}  // namespace

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`. Returns 0, or -1
// for bad arguments, or -3 if the launch failed.
extern "C" __attribute__((visibility("default"))) int sc_probe_copy(const void* src, void* dst,
                                                                    int64_t bytes, void* stream) {
    if (!src || !dst || bytes < 0 || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) & 15) return -1;
    const int64_t n = bytes / 16;
    if (n == 0) return 0;
    const int64_t blocks = (n + kBlock * kUnroll - 1) / (kBlock * kUnroll);
    hipLaunchKernelGGL(copy_nt, dim3((unsigned)blocks), dim3(kBlock), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
