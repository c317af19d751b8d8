// Measurement companion of the fused ShortConv K/V library (not part of its C ABI): plain streaming
// copies, used by the bench to measure how fast this GPU moves the same number of bytes when
// nothing but moving them is asked for. Several forms, so that the ceiling is the best of them:
//   0  one-shot grid, each lane copies 4 x 16 bytes (non-temporal loads and stores);
//   1  one-shot grid, 8 x 16 bytes per lane;
//   2  one-shot grid, 2 x 16 bytes per lane;
//   3  persistent grid (a fixed number of workgroups per compute unit), each workgroup walking
//      chunks of 256 lanes x 4 x 16 bytes with the next chunk's loads issued before the current
//      chunk's stores (software pipelining: 8 x 16 bytes per lane in flight);
//   4  as 3 with 8 x 16 bytes per chunk (16 x 16 bytes per lane in flight);
//   5  as 0 with plain (cached) loads and stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlock = 256;

template <bool NT>
__device__ inline u32x4 ld(const u32x4* p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}
template <bool NT>
__device__ inline void st(u32x4* p, const u32x4& v) {
    if (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// One-shot: workgroup b copies elements [b * kBlock * U, (b + 1) * kBlock * U), lane-interleaved.
template <int U, bool NT>
__global__ void __launch_bounds__(kBlock) copy_oneshot(const u32x4* __restrict__ src,
                                                       u32x4* __restrict__ dst, int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * kBlock * U + threadIdx.x;
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kBlock;
        if (i < n) r[u] = ld<NT>(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kBlock;
        if (i < n) st<NT>(dst + i, r[u]);
    }
}

// Persistent: chunk c (kBlock * U elements) is handled by workgroup c mod gridDim.x; a workgroup
// loads its next chunk before storing the current one. Every workgroup leaves after its last
// chunk (the loop bound is the same fixed chunk count for all).
template <int U>
__global__ void __launch_bounds__(kBlock) copy_persistent(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, int64_t n) {
    constexpr int64_t C = (int64_t)kBlock * U;
    const int64_t chunks = (n + C - 1) / C;
    const int64_t step = gridDim.x;
    int64_t c = blockIdx.x;
    u32x4 cur[U], nxt[U];
    auto load = [&](int64_t chunk, u32x4 (&r)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = chunk * C + (int64_t)u * kBlock + threadIdx.x;
            if (chunk < chunks && i < n) r[u] = __builtin_nontemporal_load(src + i);
        }
    };
    load(c, cur);
    for (; c < chunks; c += step) {
        load(c + step, nxt);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = c * C + (int64_t)u * kBlock + threadIdx.x;
            if (i < n) __builtin_nontemporal_store(cur[u], dst + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
}

}  // namespace

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream` with copy form
// `variant` (see the top of this file); `blocks_per_cu` sizes the persistent grid (ignored by the
// one-shot forms). Returns 0, or -1 for bad arguments, or -3 if the launch failed.
extern "C" __attribute__((visibility("default"))) int sc_probe_copy_variant(
    const void* src, void* dst, int64_t bytes, int variant, int blocks_per_cu, void* stream) {
    if (!src || !dst || bytes < 0 || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) & 15) return -1;
    if (variant < 0 || variant > 5 || blocks_per_cu < 1 || blocks_per_cu > 32) return -1;
    const int64_t n = bytes / 16;
    if (n == 0) return 0;
    const u32x4* s = static_cast<const u32x4*>(src);
    u32x4* d = static_cast<u32x4*>(dst);
    hipStream_t st = (hipStream_t)stream;
    auto oneshot_blocks = [n](int u) { return (unsigned)((n + (int64_t)kBlock * u - 1) / (kBlock * u)); };
    int cus = 0;
    if (variant == 3 || variant == 4) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            return -3;
    }
    switch (variant) {
        case 0: hipLaunchKernelGGL((copy_oneshot<4, true>), dim3(oneshot_blocks(4)), dim3(kBlock), 0, st, s, d, n); break;
        case 1: hipLaunchKernelGGL((copy_oneshot<8, true>), dim3(oneshot_blocks(8)), dim3(kBlock), 0, st, s, d, n); break;
        case 2: hipLaunchKernelGGL((copy_oneshot<2, true>), dim3(oneshot_blocks(2)), dim3(kBlock), 0, st, s, d, n); break;
        case 3: hipLaunchKernelGGL((copy_persistent<4>), dim3((unsigned)(cus * blocks_per_cu)), dim3(kBlock), 0, st, s, d, n); break;
        case 4: hipLaunchKernelGGL((copy_persistent<8>), dim3((unsigned)(cus * blocks_per_cu)), dim3(kBlock), 0, st, s, d, n); break;
        default: hipLaunchKernelGGL((copy_oneshot<4, false>), dim3(oneshot_blocks(4)), dim3(kBlock), 0, st, s, d, n); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// The form the bench has always used: variant 0.
extern "C" __attribute__((visibility("default"))) int sc_probe_copy(const void* src, void* dst,
                                                                    int64_t bytes, void* stream) {
    return sc_probe_copy_variant(src, dst, bytes, 0, 1, stream);
}
