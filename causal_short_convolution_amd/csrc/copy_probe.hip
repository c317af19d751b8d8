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
// A second probe, sc_probe_scatter_rows, moves the rows a prefill call must move and nothing else:
// each token's K and V rows, read at the token's position, written to cache row slot[token]
// (dropped for a slot outside the pool). No state rows, no halo, no arithmetic. It measures how
// fast this access pattern runs on its own, again in several forms:
//   0..3  one-shot grid, each lane moving 16 bytes of 1, 2, 4 or 8 consecutive tokens;
//   4     persistent grid (a fixed number of workgroups per compute unit), 4 tokens per lane per
//         unit, the next unit's loads issued before the current unit's stores;
//   5, 6  the memory side of the fused prefill alone: each wave moves 8 (5) or 4 (6) consecutive
//         tokens of one 1 KB column slice, a workgroup's four waves consecutive spans, slices
//         varying fastest across workgroups; lane i reads token i's slot, every load and store is
//         issued unconditionally (loads past the end re-read the last row, stores go through a
//         buffer resource that is empty for a dropped slot). Needs row_bytes a multiple of 1 KB.
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

// The rows of one call: lane c of a token covers bytes [16 (c mod C/2), +16) of the K row
// (c < C/2) or the V row, C = 2 * row_bytes / 16 lanes per token over `lane_blocks` workgroups.
struct ScatterArgs {
    const char* src[2];
    int64_t src_stride[2];  // bytes between consecutive tokens
    char* dst[2];
    int64_t row_bytes;
    const int64_t* slot;
    int64_t tokens;
    int64_t num_slots;
    int lane_blocks;
};

__device__ inline void scatter_lane(const ScatterArgs& a, int lb, int& tensor, int64_t& col,
                                    bool& live) {
    const int64_t half = a.row_bytes / 16;
    const int64_t c = (int64_t)lb * kBlock + threadIdx.x;
    live = c < 2 * half;
    tensor = c >= half ? 1 : 0;
    col = (c - tensor * half) * 16;
}

template <int U>
__global__ void __launch_bounds__(kBlock) scatter_oneshot(ScatterArgs a) {
    const int64_t g = blockIdx.x / a.lane_blocks;
    const int lb = (int)(blockIdx.x % a.lane_blocks);
    int tensor;
    int64_t col;
    bool live;
    scatter_lane(a, lb, tensor, col, live);
    if (!live) return;
    const char* src = a.src[tensor] + col;
    char* dst = a.dst[tensor] + col;
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t t = g * U + u;
        if (t < a.tokens)
            r[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(src + t * a.src_stride[tensor]));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t t = g * U + u;
        if (t < a.tokens) {
            const int64_t s = a.slot[t];
            if (s >= 0 && s < a.num_slots)
                __builtin_nontemporal_store(r[u], reinterpret_cast<u32x4*>(dst + s * a.row_bytes));
        }
    }
}

// Unit q = (token group q / lane_blocks of U tokens, lane block q mod lane_blocks); workgroup b
// takes units b, b + G, ... (G = gridDim.x) and leaves after its last one.
template <int U>
__global__ void __launch_bounds__(kBlock) scatter_persistent(ScatterArgs a) {
    const int64_t groups = (a.tokens + U - 1) / U;
    const int64_t units = groups * a.lane_blocks;
    const int64_t G = gridDim.x;
    u32x4 cur[U], nxt[U];
    auto load = [&](int64_t q, u32x4 (&r)[U]) {
        if (q >= units) return;
        int tensor;
        int64_t col;
        bool live;
        scatter_lane(a, (int)(q % a.lane_blocks), tensor, col, live);
        const int64_t g = q / a.lane_blocks;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = g * U + u;
            if (live && t < a.tokens)
                r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                    a.src[tensor] + col + t * a.src_stride[tensor]));
        }
    };
    int64_t q = blockIdx.x;
    load(q, cur);
    for (; q < units; q += G) {
        load(q + G, nxt);
        int tensor;
        int64_t col;
        bool live;
        scatter_lane(a, (int)(q % a.lane_blocks), tensor, col, live);
        const int64_t g = q / a.lane_blocks;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = g * U + u;
            if (live && t < a.tokens) {
                const int64_t s = a.slot[t];
                if (s >= 0 && s < a.num_slots)
                    __builtin_nontemporal_store(
                        cur[u], reinterpret_cast<u32x4*>(a.dst[tensor] + col + s * a.row_bytes));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
}

// Fused-prefill memory side (forms 5, 6): see the top of this file.
template <int U>
__global__ void __launch_bounds__(kBlock) scatter_waves(ScatterArgs a) {
    const int64_t half = a.row_bytes / 16;                 // lanes per tensor row
    const int slices = (int)(2 * half / 64);
    const int slice = (int)(blockIdx.x % slices);
    const int64_t tile = blockIdx.x / slices;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wl = threadIdx.x & 63;
    const int tensor = __builtin_amdgcn_readfirstlane(slice * 64 >= half ? 1 : 0);
    const uint32_t col = (uint32_t)((slice * 64 + wl - tensor * half) * 16);
    const int64_t t0 = tile * 4 * U + (int64_t)w * U;
    const int64_t rem = a.tokens - t0;
    if (rem <= 0) return;
    const int n = rem < U ? (int)rem : U;
    const char* src = a.src[tensor] + t0 * a.src_stride[tensor];
    const int64_t stride = a.src_stride[tensor];
    const int64_t my_slot = a.slot[t0 + (wl < n ? wl : n - 1)];
    const int64_t lane_slot = wl < n ? my_slot : (int64_t)-1;
    u32x4 r[U];
#pragma unroll
    for (int i = 0; i < U; ++i)
        r[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(src + (i < n ? i : n - 1) * stride + col));
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)lane_slot, i);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(lane_slot >> 32), i);
        const int64_t s = (int64_t)(((uint64_t)hi << 32) | lo);
        const bool ok = s >= 0 && s < a.num_slots;
        char* row = a.dst[tensor] + (ok ? s : 0) * a.row_bytes;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            row, (short)0, ok ? (int)a.row_bytes : 0, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(r[i], rs, col, 0, 2);
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

// Moves the K and V rows of `tokens` tokens to their cache rows: row t of k (v), `k_stride`
// (`v_stride`) bytes apart, is written to row slot[t] of k_cache (v_cache), rows of `row_bytes`
// bytes (a multiple of 16, all pointers and strides 16-byte aligned, strides >= row_bytes); a slot
// outside [0, num_slots) drops the token. `slot` is a device array of int64. Form `variant` (see
// the top of this file); `blocks_per_cu` sizes the persistent grid. Returns 0, -1 for bad
// arguments, -3 if the launch failed.
extern "C" __attribute__((visibility("default"))) int sc_probe_scatter_rows(
    const void* k, const void* v, int64_t k_stride, int64_t v_stride, void* k_cache, void* v_cache,
    int64_t row_bytes, const int64_t* slot, int64_t tokens, int64_t num_slots, int variant,
    int blocks_per_cu, void* stream) {
    if (tokens < 0 || num_slots < 0 || row_bytes <= 0 || row_bytes % 16) return -1;
    if (tokens == 0) return 0;
    if (!k || !v || !k_cache || !v_cache || !slot) return -1;
    if (k_stride < row_bytes || v_stride < row_bytes || (k_stride | v_stride) & 15) return -1;
    if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache | (uintptr_t)v_cache) & 15) return -1;
    if (variant < 0 || variant > 6 || blocks_per_cu < 1 || blocks_per_cu > 32) return -1;
    if (variant >= 5 && (row_bytes % 1024 || row_bytes > (1 << 30))) return -1;
    ScatterArgs a;
    a.src[0] = static_cast<const char*>(k);
    a.src[1] = static_cast<const char*>(v);
    a.src_stride[0] = k_stride;
    a.src_stride[1] = v_stride;
    a.dst[0] = static_cast<char*>(k_cache);
    a.dst[1] = static_cast<char*>(v_cache);
    a.row_bytes = row_bytes;
    a.slot = slot;
    a.tokens = tokens;
    a.num_slots = num_slots;
    const int64_t lanes = 2 * row_bytes / 16;
    a.lane_blocks = (int)((lanes + kBlock - 1) / kBlock);
    hipStream_t st = (hipStream_t)stream;
    auto grid = [&](int u) {
        return (unsigned)(((tokens + u - 1) / u) * a.lane_blocks);
    };
    if (variant >= 5) {
        const int u = variant == 5 ? 8 : 4;
        const unsigned blocks =
            (unsigned)(((tokens + 4 * u - 1) / (4 * u)) * (2 * row_bytes / 1024));
        if (variant == 5)
            hipLaunchKernelGGL(scatter_waves<8>, dim3(blocks), dim3(kBlock), 0, st, a);
        else
            hipLaunchKernelGGL(scatter_waves<4>, dim3(blocks), dim3(kBlock), 0, st, a);
    } else if (variant == 4) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            return -3;
        hipLaunchKernelGGL(scatter_persistent<4>, dim3((unsigned)(cus * blocks_per_cu)),
                           dim3(kBlock), 0, st, a);
    } else if (variant == 0) {
        hipLaunchKernelGGL(scatter_oneshot<1>, dim3(grid(1)), dim3(kBlock), 0, st, a);
    } else if (variant == 1) {
        hipLaunchKernelGGL(scatter_oneshot<2>, dim3(grid(2)), dim3(kBlock), 0, st, a);
    } else if (variant == 2) {
        hipLaunchKernelGGL(scatter_oneshot<4>, dim3(grid(4)), dim3(kBlock), 0, st, a);
    } else {
        hipLaunchKernelGGL(scatter_oneshot<8>, dim3(grid(8)), dim3(kBlock), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
