// Device helpers shared by the HIP kernels of the fused ShortConv K/V step (forward, speculative
// verification, MXFP8 encoding and backward): element types, 16-byte row access with streaming
// hints, cross-lane moves and reductions, and the tile -> sequence search of the prefill grids.
// Internal to the library; not part of the C ABI.
#ifndef SHORTCONV_DEVICE_COMMON_H
#define SHORTCONV_DEVICE_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

// ------------------------------------------------------------------------------------------------
// Element types. A "packet" is the 16 bytes one lane moves: uint4.
// ------------------------------------------------------------------------------------------------
struct F32 {
    static constexpr int VEC = 4;
    static constexpr int BYTES = 4;
    __device__ static inline void widen(const uint4& r, float (&f)[VEC]) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    __device__ static inline uint4 narrow(const float (&f)[VEC]) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct BF16 {
    static constexpr int VEC = 8;
    static constexpr int BYTES = 2;
    __device__ static inline void widen(const uint4& r, float (&f)[VEC]) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    // Round to nearest even (one v_cvt_pk_bf16_f32 per pair on gfx950).
    __device__ static inline uint32_t pack2(float a, float b) {
        bf16x2_t p = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, p);
    }
    __device__ static inline uint4 narrow(const float (&f)[VEC]) {
        return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]),
                          pack2(f[6], f[7]));
    }
};

__device__ inline uint4 ld16(const void* base, int64_t elem_off, int bytes) {
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + elem_off * bytes);
}
__device__ inline void st16(void* base, int64_t elem_off, int bytes, const uint4& v) {
    *reinterpret_cast<uint4*>(static_cast<char*>(base) + elem_off * bytes) = v;
}
// Row access as (wave-uniform byte base, per-lane 32-bit byte offset). K/V rows are read once and
// cache rows are written once, so both stream with the non-temporal hint: they do not displace
// reusable lines (taps, gamma, metadata) from L2 and the Infinity Cache, and dirty cache rows do
// not linger there (measured on MI355X: a cold 140 MB copy streams at ~5.7 TB/s with the hint
// against ~3.0 TB/s without).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 ldrow(const char* base, uint32_t lane_off) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + lane_off));
    return make_uint4(v.x, v.y, v.z, v.w);
}
// The same load without the streaming hint. The kernels use it for a few rows of each span (a
// mix that measured faster than streaming every row; see where it is used).
__device__ inline uint4 ldrow_keep(const char* base, uint32_t lane_off) {
    return *reinterpret_cast<const uint4*>(base + lane_off);
}
__device__ inline void strow(char* base, uint32_t lane_off, const uint4& v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(base + lane_off));
}

// Waits until every vector memory access this wave has issued is complete (s_waitcnt vmcnt(0),
// other counters unconstrained). On gfx9 stores count in vmcnt too: where a span's row loads are
// followed by conditional cache stores, the compiler cannot tell how many operations follow a
// row and waits for all of them, stores included, before each row. One explicit wait for the
// rows before the loop leaves nothing in flight that a row could be waiting on.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Values that are the same in every lane, moved to scalar registers so that the compiler uses
// scalar loads for per-token metadata and scalar base addresses for the row accesses.
__device__ inline int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Per-lane choice between the K and the V member of a pair of kernel arguments. Both members are
// read as scalars and the lane selects; indexing the pair with the lane's tensor would instead be
// a vector load from the argument segment, and every address derived from it would wait for it.
template <class P>
__device__ inline P pick(const P (&pair)[2], int tensor) {
    const P k = pair[0];
    const P v = pair[1];
    return tensor ? v : k;
}

// Lane i's value of v, as a wave-uniform (scalar) value.
__device__ inline int64_t lane_value(int64_t v, int i) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, i);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), i);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Data-parallel-primitive lane moves (row = 16 lanes).
template <int CTRL>
__device__ inline float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each half row
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each row

// Sum over the LPH lanes that own one head (aligned groups, LPH | 64). A butterfly: at every step
// each lane adds its value and its partner's, the partner adds the same two values in the other
// order, so all lanes of the group end with the same bits. Within a 16-lane row the partners come
// from DPP moves; the quad steps make the 4 lanes of a quad equal, so the mirror moves pair each
// lane with a lane of the neighbouring quad (half row) or half row (row). Across rows, gfx950's
// permlane swaps give every lane its own value and its partner's (lane ^ 16, lane ^ 32) in one
// VALU instruction, as two outputs whose sum is own + partner in every lane.
template <int LPH>
__device__ inline float head_sum(float v) {
    static_assert(LPH == 8 || LPH == 16 || LPH == 32 || LPH == 64, "lanes per head");
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    v += dpp<kRowHalfMirror>(v);
    if (LPH >= 16) v += dpp<kRowMirror>(v);
    if (LPH >= 32) {
        const uint32_t u = __float_as_uint(v);
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    if (LPH >= 64) {
        const uint32_t u = __float_as_uint(v);
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    return v;
}

__device__ inline int32_t clamp_tok(int32_t v, int64_t T) {
    return v < 0 ? 0 : (v > T ? (int32_t)T : v);
}

template <int BB>
__device__ inline int64_t tile_base(const int32_t* cu, int s, int64_t T) {
    return (int64_t)(clamp_tok(cu[s], T) / BB) + s;
}

// The largest s in [0, n) with P(s) <= tile, P(s) = floor(cu[s] / BB) + s (strictly increasing).
// Wave-parallel: each round the 64 lanes test 64 evenly spaced candidates with one vector load and
// a ballot narrows the range 64-fold, so n <= 64 costs one memory round trip and n <= 4096 two,
// where a binary search would chain log2(n) dependent loads. Must be called by whole waves.
template <int BB>
__device__ inline int find_tile_seq(const int32_t* cu, int n, int64_t T, int64_t tile) {
    const int wl = threadIdx.x & 63;
    int base = 0, count = n;
    while (count > 1) {
        const int step = (count + 63) / 64;
        const int cand = base + wl * step;
        const bool ok = wl * step < count && tile_base<BB>(cu, cand, T) <= tile;
        const uint64_t mask = __ballot(ok);
        // P(base) <= tile always holds for a tile that belongs to some sequence; the prefix of
        // set bits ends at the last candidate that still starts at or before the tile.
        const int last = mask ? 63 - __builtin_clzll(mask) : 0;
        base += last * step;
        count = step < count - last * step ? step : count - last * step;
    }
    return uniform(base);
}

// find_tile_seq, also giving the sequence's bounds clamp_tok(cu[s]) and clamp_tok(cu[s + 1]) as
// wave-uniform values. For n <= 63 one round decides: lane l loads cu[min(l, n)], so the bounds
// are read from lanes s and s + 1 of that same load, with no further dependent load before the
// rows' addresses are known. Measured on MI355X (one process, medians of 5): varlen bf16 prefill
// of 8 sequences 28.03 -> 27.41 us, with MXFP8 rows 24.65 -> 23.76 us; in the backward neutral
// (57.8 us), and for one sequence (long prefill, W = 8) 1-3 % slower, where the plain search
// issues no vector load at all: there the kernels keep find_tile_seq. Must be called by whole
// waves.
template <int BB>
__device__ inline int tile_seq_bounds(const int32_t* cu, int n, int64_t T, int64_t tile,
                                      int64_t& start, int64_t& end) {
    if (n <= 63) {
        const int wl = threadIdx.x & 63;
        const int32_t c = clamp_tok(cu[wl <= n ? wl : n], T);
        const bool ok = wl < n && (int64_t)(c / BB) + wl <= tile;  // P(wl) <= tile
        const uint64_t mask = __ballot(ok);
        const int s = uniform(mask ? 63 - __builtin_clzll(mask) : 0);
        start = (int64_t)__builtin_amdgcn_readlane(c, s);
        end = (int64_t)__builtin_amdgcn_readlane(c, s + 1);
        return s;
    }
    const int s = find_tile_seq<BB>(cu, n, T, tile);
    start = uniform((int64_t)clamp_tok(cu[s], T));
    end = uniform((int64_t)clamp_tok(cu[s + 1], T));
    return s;
}

}  // namespace sc

#endif  // SHORTCONV_DEVICE_COMMON_H
