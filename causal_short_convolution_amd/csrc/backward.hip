// HIP kernels of the backward of the fused ShortConv K/V step for gfx950 (MI355X): the gradients
// that training needs for the K/V short convolution followed by the per-head RMSNorm (the English
// news item on SGLang/Miles Inkling support, paragraph 3, has the RL trainer run the model with
// train/infer-consistent kernels). The chain rule through the forward definition:
//   chat = c / r,  dchat = g * gamma,  proj = (1/D) sum_d dchat * chat
//   dc   = (dchat - chat * proj) / r
//   dgamma[d]    += g * chat                     (over tokens and heads)
//   dtaps[k,h,d] += dc[p] * e[p+k]               (over tokens)
//   de[i]         = sum_k taps[k] * dc[i-k]  (+ the loss on the new state for its rows)
//   dx = de of the input rows;  dstate = de of the initial window rows
//
// Like the forward this is a stencil, HBM-bound: per token it reads the K/V row and the gradient
// row and writes the input-gradient row (3 rows, 6 bytes per element in bf16), against ~3W+12
// flops per element. No matrix cores.
//
// Thread layout: one lane owns 4 channels of one head (8 bytes in bf16, 16 in fp32): the
// backward holds about twice the per-lane state of the forward (taps, their gradient
// accumulators, the input window and a ring of dc rows), and 4 channels keep the width-8 kernel
// within the register file. A wave covers one 64-lane column slice of the K|V rows.
//
// Grid: the forward's per-sequence tiles (4 waves x BT tokens of one sequence, found by the same
// wave-parallel search); each workgroup walks up to 4 consecutive tiles of its column slice
// (fewer when the problem is too small to fill the chip otherwise), so that each lane's fp32 sums
// of the tap and gamma gradients stay short. Per tile a wave:
//   phase 1: loads its W-1 halo rows, its BT input rows and BT gradient rows in one burst, then
//            for each token computes dc, accumulates the parameter gradients and emits the input
//            gradient of every token whose dc window (the token and the W-1 after it) lies inside
//            the span; its first W-1 dc rows go to LDS;
//   phase 2: after a barrier, emits the input gradient of its last W-1 tokens from the next
//            wave's first dc rows (LDS). The tile's last wave needs the next tile's first W-1 dc:
//            when the workgroup walks that tile next, it hands its own last W-1 dc rows through
//            LDS to that tile's wave 0, which finishes those rows in its own phase 2; otherwise it
//            recomputes the next tile's first W-1 tokens.
// The first wave of a sequence's first tile also writes the initial-window gradient.
// The parameter gradients leave each workgroup as one partial (the 4 waves summed through LDS,
// in wave order) in a workspace; further kernels add the partials in fp64 in a fixed order (by
// chunks of groups, then over chunks and heads). Results are therefore deterministic.
#include "device_common.h"
#include "shortconv_internal.h"

namespace sc {
namespace {

constexpr int kBwdBlock = 256;
constexpr int kBwdWaves = kBwdBlock / 64;
// Tiles a workgroup walks: as many as keep each lane's fp32 partial within kMaxPartialTokens
// tokens of its span (the rounding bound of the parameter gradients assumes no more), and fewer
// when that leaves too few workgroups to fill the chip (kFillBlocks); at most SC_BWD_MAX_TILES.
// Measured on MI355X with 4 / up to 6 tiles (bf16, 12-token spans at W = 4): the mixed W = 4
// backward 644 / 653 us (and, with the 10-token spans W = 8 had then, the long one 462 / 463 us).
constexpr int kMaxPartialTokens = 64;
#ifndef SC_BWD_MAX_TILES
#define SC_BWD_MAX_TILES 4
#endif
// Measured on MI355X (varlen bf16 backward, 8 rounds): 2048 65.5 us (one tile per workgroup),
// 1024 61.5 us (two tiles: the first tile's last rows are finished by the second); long and
// mixed backward unchanged (four tiles either way).
#ifndef SC_BWD_FILL_BLOCKS
#define SC_BWD_FILL_BLOCKS 1024
#endif
constexpr int64_t kFillBlocks = SC_BWD_FILL_BLOCKS;

// Span tokens per wave: a span's input and gradient rows are all in flight at once, so wide
// windows and fp32 rows take shorter spans to stay within the register file. Tuning knobs
// (chosen by measurement on MI355X).
#ifndef SC_BWD_BT_BF16
#define SC_BWD_BT_BF16 16       // bf16, W <= 5
#endif
#ifndef SC_BWD_BT_BF16_WIDE
#define SC_BWD_BT_BF16_WIDE 10  // bf16, W > 5
#endif
#ifndef SC_BWD_BT_F32
#define SC_BWD_BT_F32 16        // fp32, W == 1
#endif
#ifndef SC_BWD_BT_F32_WIDE
#define SC_BWD_BT_F32_WIDE 8    // fp32, W > 1
#endif
#ifndef SC_BWD_BT_BF16_PURE
#define SC_BWD_BT_BF16_PURE 12  // bf16, W <= 4, single-tensor slices (3 waves per SIMD)
#endif
// bf16, W > 5, single-tensor slices: the register count stays at ~242 (2 waves per SIMD) from
// 8 to 20 tokens here, so longer spans only shed halo rows, recomputed rows and partials.
// Measured on MI355X (W = 8, 131 072 tokens, one process, spans of 10 / 12 / 14 / 16 / 20):
// 461.7 / 447.8 / 438.9 / 424.1 / 423.8 us per backward; 24 spills.
#ifndef SC_BWD_BT_BF16_WIDE_PURE
#define SC_BWD_BT_BF16_WIDE_PURE 16
#endif
template <class E, int W, bool PURE = false>
constexpr int bwd_span() {
    return E::BYTES == 2
               ? (PURE && W <= 4 ? SC_BWD_BT_BF16_PURE
                                 : (W <= 5 ? SC_BWD_BT_BF16
                                           : (PURE ? SC_BWD_BT_BF16_WIDE_PURE : SC_BWD_BT_BF16_WIDE)))
               : (W <= 1 ? SC_BWD_BT_F32 : SC_BWD_BT_F32_WIDE);
}

// 4 channels of one lane, in the I/O element type, with streaming (non-temporal) access.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <class E>
struct Quad;
template <>
struct Quad<F32> {
    using Raw = uint4;
    static constexpr int BYTES = 4;
    __device__ static Raw load(const char* p) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    __device__ static Raw load_keep(const char* p) {  // without the streaming hint
        return *reinterpret_cast<const uint4*>(p);
    }
    __device__ static void store(char* p, const Raw& r) {
        const u32x4 v = {r.x, r.y, r.z, r.w};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    }
    __device__ static void widen(const Raw& r, float (&f)[4]) {
        f[0] = __uint_as_float(r.x);
        f[1] = __uint_as_float(r.y);
        f[2] = __uint_as_float(r.z);
        f[3] = __uint_as_float(r.w);
    }
    __device__ static Raw narrow(const float (&f)[4]) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
    __device__ static Raw zero() { return make_uint4(0, 0, 0, 0); }
};
template <>
struct Quad<BF16> {
    using Raw = uint2;
    static constexpr int BYTES = 2;
    __device__ static Raw load(const char* p) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return make_uint2(v.x, v.y);
    }
    __device__ static Raw load_keep(const char* p) {  // without the streaming hint
        return *reinterpret_cast<const uint2*>(p);
    }
    __device__ static void store(char* p, const Raw& r) {
        const u32x2 v = {r.x, r.y};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
    }
    __device__ static void widen(const Raw& r, float (&f)[4]) {
        f[0] = __uint_as_float(r.x << 16);
        f[1] = __uint_as_float(r.x & 0xffff0000u);
        f[2] = __uint_as_float(r.y << 16);
        f[3] = __uint_as_float(r.y & 0xffff0000u);
    }
    __device__ static Raw narrow(const float (&f)[4]) {
        return make_uint2(BF16::pack2(f[0], f[1]), BF16::pack2(f[2], f[3]));
    }
    __device__ static Raw zero() { return make_uint2(0, 0); }
};

// Input-gradient rows stored through a buffer resource whose range is the destination row: a row
// that must not be written gets an empty range and the hardware drops the store, so the store
// instruction is issued unconditionally (single-tensor slices, where the destination is uniform).
constexpr int kBufferDword3 = 0x00020000;  // raw (untyped, unswizzled) buffer resource, gfx9
constexpr int kNonTemporal = 2;            // cache policy of the streaming stores
template <class E>
__device__ inline void store_row(char* base, int64_t row, uint32_t bytes, bool valid,
                                 uint32_t lane_off, const typename Quad<E>::Raw& v) {
    char* p = base + (valid ? row : 0) * (int64_t)bytes;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(p, (short)0, valid ? (int)bytes : 0, kBufferDword3);
    if constexpr (E::BYTES == 2) {
        const u32x2 w = {v.x, v.y};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, lane_off, 0, kNonTemporal);
    } else {
        const u32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, lane_off, 0, kNonTemporal);
    }
}

// dc of one token from its window (ring: row k of the window is win[(off + k) % W]) and its
// output gradient; also returns chat for the gamma gradient. Same arithmetic order as the forward
// for c and r (FMA chain in k order, sum of squares, head butterfly, v_rsq_f32).
template <int W, int LPH>
__device__ inline void token_dc(const float (&win)[W][4], int off, const float (&tap)[W][4],
                                const float (&gam)[4], const float (&g)[4], float eps,
                                float inv_d, float (&dc)[4], float (&chat)[4]) {
    float c[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) c[v] = tap[0][v] * win[off % W][v];
#pragma unroll
    for (int k = 1; k < W; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v) c[v] = __builtin_fmaf(tap[k][v], win[(off + k) % W][v], c[v]);
    float ss = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) ss = __builtin_fmaf(c[v], c[v], ss);
    ss = head_sum<LPH>(ss);
    const float inv = __builtin_amdgcn_rsqf(__builtin_fmaf(ss, inv_d, eps));
    float dchat[4];
    float pj = 0.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        chat[v] = c[v] * inv;
        dchat[v] = g[v] * gam[v];
        pj = __builtin_fmaf(dchat[v], chat[v], pj);
    }
    pj = head_sum<LPH>(pj) * inv_d;
#pragma unroll
    for (int v = 0; v < 4; ++v) dc[v] = __builtin_fmaf(-chat[v], pj, dchat[v]) * inv;
}

// Input-window gradient of row q of a span: sum_k taps[k] * dc[q + R - k], where ring slot
// (j % W) holds dc of token j; the tokens' dc beyond the sequence are zero.
template <int W>
__device__ inline void row_grad(const float (&tap)[W][4], const float (&dcr)[W][4], int q,
                                float (&de)[4]) {
    constexpr int R = W - 1;
#pragma unroll
    for (int v = 0; v < 4; ++v) de[v] = tap[0][v] * dcr[(q + R) % W][v];
#pragma unroll
    for (int k = 1; k < W; ++k)
#pragma unroll
        for (int v = 0; v < 4; ++v) de[v] = __builtin_fmaf(tap[k][v], dcr[(q + R - k) % W][v], de[v]);
}

// Adds the new-state loss row jj = i - (L - R) to a row at sequence position i, if i falls in the
// last R rows (jj is a runtime value; the selection is unrolled so that gsr stays in registers).
template <class E, int R>
__device__ inline void add_state_loss(const typename Quad<E>::Raw (&gsr)[R > 0 ? R : 1], int64_t jj,
                                      float (&de)[4]) {
#pragma unroll
    for (int m = 0; m < R; ++m) {
        float f[4];
        Quad<E>::widen(gsr[m], f);
        const bool hit = jj == m;
#pragma unroll
        for (int v = 0; v < 4; ++v) de[v] += hit ? f[v] : 0.0f;
    }
}

// PURE: every 64-lane slice holds one tensor (H * D a multiple of 256), so the tensor and every
// destination are wave-uniform and the input-gradient rows are stored as they are computed;
// otherwise they are held until the span's loop ends (a conditional store between tokens would
// make the compiler wait for everything in flight).
#ifndef SC_BWD_WAVES_PURE
#define SC_BWD_WAVES_PURE 3
#endif
template <class E, int W, bool PURE>
constexpr int bwd_min_waves() {
    return PURE && W <= 4 && E::BYTES == 2 ? SC_BWD_WAVES_PURE : 2;
}

// Whether the tile's last wave loads the R rows after its span (for its phase 2) in its first
// burst, with everything else; otherwise it loads them after the barrier, and the whole workgroup
// waits for that round trip (measured on MI355X, bf16 W = 8, 131072 tokens: 530 us with the late
// loads, 408 us with no phase-2 recompute at all). Early loads hold 2R more rows in registers:
// every case but the ones where that spills (bf16 W = 8 over slices mixing K and V lanes, fp32
// W = 8, fp32 W = 7 over mixed slices).
#ifndef SC_BWD_PREFETCH_WIDE
#define SC_BWD_PREFETCH_WIDE 1
#endif
// 1: a tile's last R input-gradient rows may be finished by the next tile of the same workgroup
// (see `defer` in backward_kernel) instead of recomputing the next tile's first R tokens.
#ifndef SC_BWD_DEFER
#define SC_BWD_DEFER 1
#endif
template <class E, int W, bool PURE>
constexpr bool bwd_prefetch_next() {
    if (W <= 4) return true;
    if (!SC_BWD_PREFETCH_WIDE) return false;
    // with deferral (SC_BWD_DEFER) the bf16 W = 8 and fp32 W = 7 kernels over one-tensor slices
    // have no registers left for the early loads
    return E::BYTES == 2 ? (W < 8 || (PURE && !SC_BWD_DEFER))
                         : (W <= 6 || (PURE && W == 7 && !SC_BWD_DEFER));
}

template <class E, int D, int W, int BT, bool PURE>
__global__ void __launch_bounds__(kBwdBlock, (bwd_min_waves<E, W, PURE>())) backward_kernel(BwdArgs a) {
    using Q = Quad<E>;
    using Raw = typename Q::Raw;
    constexpr int LPH = D / 4;
    constexpr int R = W - 1;
    constexpr int RR = R > 0 ? R : 1;
    constexpr int NW = kBwdWaves;
    constexpr int BB = NW * BT;
    static_assert(BT >= R, "a wave's span must cover the window");
    // dc rows that wave w + 1 hands back to wave w (first R of its span), reused afterwards for
    // the workgroup's sum of the parameter-gradient partials.
    constexpr bool kPrefetchNext = bwd_prefetch_next<E, W, PURE>();
    constexpr bool kDefer = SC_BWD_DEFER && R > 0;
    // Row byte offsets (wave-uniform). For W <= 4 they are kept scalar through readfirstlane, so
    // each row address is one add to the lane's base rather than a quarter-rate 64-bit
    // multiply-add on the vector unit. Measured on MI355X (bf16, same process): varlen 61.5 ->
    // 61.0 us, mixed 650.7 -> 642.4 us; at W = 8 (431 against 427 us) it is left to the compiler.
    const auto roff = [](int64_t v) -> int64_t {
        if constexpr (W <= 4) return uniform(v);
        else return v;
    };

    // LDS: the first R dc rows of each wave's span (NW * RR rows), then two buffers (by tile
    // parity) for the last R dc rows of a tile's last span when it defers its last
    // input-gradient rows to the next tile (2 * RR rows).
    constexpr int kHand = NW * RR + 2 * RR;
    constexpr int kRed = (NW - 1) * (W + 1);
    __shared__ float4 lds[(kHand > kRed ? kHand : kRed) * 64];

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wl = threadIdx.x & 63;
    const int slices = a.slices;
    const int group = blockIdx.x / slices;
    const int slice = blockIdx.x - group * slices;
    const int lane = slice * 64 + wl;
    const bool active = lane < 2 * a.lanes_per_tensor;
    const int ln = active ? lane : 0;
    const int tensor = PURE ? uniform(slice * 64 >= a.lanes_per_tensor ? 1 : 0)
                            : (ln >= a.lanes_per_tensor ? 1 : 0);
    const int cch = ln - tensor * a.lanes_per_tensor;
    const int h = cch / LPH;
    const int d0 = (cch - h * LPH) * 4;
    const int64_t T = a.tokens;
    const int64_t row_elems = (int64_t)a.heads * D;
    const int64_t row_bytes = row_elems * Q::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * Q::BYTES);

    const char* x = static_cast<const char*>(pick(a.x, tensor));
    const int64_t xs = pick(a.x_stride, tensor) * Q::BYTES;
    const char* dy = static_cast<const char*>(pick(a.dy, tensor));
    char* dx = static_cast<char*>(pick(a.dx, tensor));
    const char* state = static_cast<const char*>(pick(a.state, tensor));
    const char* gs = static_cast<const char*>(pick(a.gs, tensor));
    char* dstate = static_cast<char*>(pick(a.dstate, tensor));
    const float* taps_p = pick(a.taps, tensor);

    float tap[W][4], gam[4];
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const float4 q = *reinterpret_cast<const float4*>(taps_p + (k * a.heads + h) * D + d0);
        tap[k][0] = q.x; tap[k][1] = q.y; tap[k][2] = q.z; tap[k][3] = q.w;
    }
    {
        const float4 q = *reinterpret_cast<const float4*>(pick(a.gamma, tensor) + d0);
        gam[0] = q.x; gam[1] = q.y; gam[2] = q.z; gam[3] = q.w;
    }
    const float inv_d = 1.0f / (float)D;
    float acc_t[W][4], acc_g[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        acc_g[v] = 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) acc_t[k][v] = 0.0f;
    }

    // The previous tile deferred its last R input-gradient rows (those at pending_t0 + BT - R ..)
    // to this one.
    bool pending = false;
    int64_t pending_t0 = 0;
#pragma unroll 1
    for (int gi = 0; gi < a.tiles_per_group; ++gi) {
        const int64_t tile = (int64_t)group * a.tiles_per_group + gi;
        if (tile >= a.tiles) break;  // the same for the whole workgroup
        const int s = find_tile_seq<BB>(a.cu, a.num_seqs, T, tile);
        const int64_t start = uniform((int64_t)clamp_tok(a.cu[s], T));
        int64_t end = uniform((int64_t)clamp_tok(a.cu[s + 1], T));
        if (end < start) end = start;
        const int64_t L = end - start;
        const int64_t j = tile - tile_base<BB>(a.cu, s, T);
        const int64_t ntiles = L > 0 ? (L + BB - 1) / BB : 1;
        if (j < 0 || j >= ntiles) {  // the same for the whole workgroup
            pending = false;  // (never set here: a deferring tile's successor is always walked)
            continue;
        }

        const int64_t p0 = j * BB + (int64_t)w * BT;  // span start, sequence position
        const int64_t t0 = start + p0;
        const int64_t rem = L - p0;
        const int n = rem <= 0 ? 0 : (rem < BT ? (int)rem : BT);
        const int next_n = rem <= BT ? 0 : (rem - BT < R ? (int)(rem - BT) : R);
        const bool first_span = j == 0 && w == 0;
        // Defer: when this workgroup walks the next tile too and the sequence continues into it,
        // the tile's last wave does not recompute the next tile's first R tokens; it hands the dc
        // of its own last R tokens to the next tile's wave 0 through LDS, which finishes the last
        // R input-gradient rows of this tile from them and its own first R dc. Not when those rows
        // carry the new-state loss. The same decision in every wave (uniform values only).
        const int64_t p0_last = j * BB + (int64_t)(NW - 1) * BT;
        const bool defer = kDefer && gi + 1 < a.tiles_per_group && tile + 1 < a.tiles &&
                           L - p0_last > BT && !(gs != nullptr && p0_last + BT > L - R);
        int32_t idx = -1;
        bool from_state = false;
        if (j == 0) {
            idx = uniform(a.state_idx ? a.state_idx[s] : s);
            from_state = R > 0 && state != nullptr && idx >= 0 && idx < a.num_state_slots &&
                         (a.has_init ? a.has_init[s] != 0 : true);
        }
        // this span holds some of the sequence's last R positions (the new-state loss rows)
        const bool has_tail = R > 0 && gs != nullptr && p0 + n > L - R;
        const char* gs_seq = gs + (int64_t)s * R * row_bytes;

        float win[W][4];
        float dcr[W][4];  // ring: slot (i % W) holds dc of span token i
        Raw gsr[RR];
        Raw xn[RR], gn[RR];  // the last wave's rows after its span (phase 2)
        if (n > 0) {
            // ---- phase 1: one burst of loads, then the span's tokens ----
            const char* hsrc = !first_span ? x + (t0 - R) * xs
                               : from_state ? state + (int64_t)idx * R * row_bytes
                                            : reinterpret_cast<const char*>(taps_p);
            const int64_t hstride = !first_span ? xs : row_bytes;
            // Loads, oldest first: the new-state loss rows (only in a span holding some of the
            // sequence's last R rows; being the oldest, the branch around them does not hide from
            // the compiler which later loads are still in flight), the halo, then the rows.
            Raw halo[RR], xr[BT], gr[BT];
            if (has_tail) {
#pragma unroll
                for (int m = 0; m < R; ++m) gsr[m] = Q::load(gs_seq + roff(m * row_bytes) + lane_off);
            }
            // the tile's last wave also fetches the R rows after its span now, for phase 2
            // (where the registers allow, see bwd_prefetch_next)
            if (kPrefetchNext && w == NW - 1 && next_n > 0 && !defer) {
                const int lastn = next_n - 1;
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    const int r = k < lastn ? k : lastn;
                    xn[k] = Q::load(x + roff((t0 + BT + r) * xs) + lane_off);
                    gn[k] = Q::load(dy + roff((t0 + BT + r) * row_bytes) + lane_off);
                }
            }
            // The halo and the span's last R input rows are loaded without the streaming hint,
            // the other rows with it, the mix that measured fastest (as in the forward).
#pragma unroll
            for (int k = 0; k < R; ++k) halo[k] = Q::load_keep(hsrc + roff(k * hstride) + lane_off);
            const int last = n - 1;
#pragma unroll
            for (int i = 0; i < BT; ++i) {
                const int r = i < last ? i : last;
                xr[i] = i >= BT - R ? Q::load_keep(x + roff((t0 + r) * xs) + lane_off)
                                    : Q::load(x + roff((t0 + r) * xs) + lane_off);
                gr[i] = Q::load(dy + roff((t0 + r) * row_bytes) + lane_off);
            }
            if (first_span && !from_state) {
#pragma unroll
                for (int k = 0; k < R; ++k) halo[k] = Q::zero();
            }
#pragma unroll
            for (int k = 0; k < R; ++k) Q::widen(halo[k], win[k]);
#pragma unroll
            for (int k = 0; k < W; ++k)
#pragma unroll
                for (int v = 0; v < 4; ++v) dcr[k][v] = 0.0f;

            // The tokens issue no store (their results stay in registers until the loop ends), so
            // the compiler waits for each token's rows alone and the first tokens are computed
            // while later rows arrive; a store among them would make it wait for everything.
            Raw dx_out[!PURE && BT - R > 0 ? BT - R : 1];
#pragma unroll
            for (int i = 0; i < BT; ++i) {
                float dci[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (i < n) {
                    Q::widen(xr[i], win[(i + R) % W]);
                    float g[4], chat[4];
                    Q::widen(gr[i], g);
                    token_dc<W, LPH>(win, i % W, tap, gam, g, a.eps, inv_d, dci, chat);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        acc_g[v] = __builtin_fmaf(g[v], chat[v], acc_g[v]);
#pragma unroll
                        for (int k = 0; k < W; ++k)
                            acc_t[k][v] = __builtin_fmaf(dci[v], win[(i + k) % W][v], acc_t[k][v]);
                    }
                }
#pragma unroll
                for (int v = 0; v < 4; ++v) dcr[i % W][v] = dci[v];
                if (i < R)
                    lds[(w * RR + i) * 64 + wl] = make_float4(dci[0], dci[1], dci[2], dci[3]);
                // rows whose dc window lies inside the span: q = i - R
                if constexpr (PURE) {
                    if (i >= R) {
                        const int q = i - R;
                        float de[4];
                        row_grad<W>(tap, dcr, q, de);
                        if (has_tail) add_state_loss<E, R>(gsr, p0 + q - (L - R), de);
                        store_row<E>(dx, t0 + q, (uint32_t)row_bytes, q < n, lane_off,
                                     Q::narrow(de));
                    }
                } else if (i >= R && i - R < n) {
                    const int q = i - R;
                    float de[4];
                    row_grad<W>(tap, dcr, q, de);
                    if (has_tail) add_state_loss<E, R>(gsr, p0 + q - (L - R), de);
                    dx_out[q] = Q::narrow(de);
                }
            }
            if constexpr (!PURE) {
                if (active) {
#pragma unroll
                    for (int q = 0; q < BT - R; ++q)
                        if (q < n) Q::store(dx + (t0 + q) * row_bytes + lane_off, dx_out[q]);
                }
            }
            // The initial window's gradient (first span): de[m] = sum_{k<=m} taps[k] dc[m-k],
            // from the span's first R dc, which this wave also left in LDS for its neighbour.
            if (R > 0 && first_span && dstate != nullptr) {
                float d0c[RR][4];
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    const float4 f = lds[(w * RR + k) * 64 + wl];
                    d0c[k][0] = f.x; d0c[k][1] = f.y; d0c[k][2] = f.z; d0c[k][3] = f.w;
                }
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    float de[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k <= m; ++k)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            de[v] = __builtin_fmaf(tap[k][v], d0c[m - k][v], de[v]);
                    if (has_tail) add_state_loss<E, R>(gsr, (int64_t)m - L, de);
                    if (!from_state) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) de[v] = 0.0f;
                    }
                    if (active)
                        Q::store(dstate + ((int64_t)s * R + m) * row_bytes + lane_off,
                                 Q::narrow(de));
                }
            }
        }
        __syncthreads();
        if (n > 0 && defer && w == NW - 1) {
            // ---- phase 2, deferring: hand the dc of the span's last R tokens to the next tile
            // (two buffers by tile parity: wave 0 reads the previous tile's while this is written)
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const float* f = dcr[(BT - R + k) % W];
                lds[((NW + (gi & 1)) * RR + k) * 64 + wl] = make_float4(f[0], f[1], f[2], f[3]);
            }
        } else if (n > 0) {
            // ---- phase 2: the last R rows of the span need dc of the R tokens after it ----
            float dcn[RR][4];  // dc of span tokens BT .. BT+R-1 (zero past the sequence)
#pragma unroll
            for (int k = 0; k < RR; ++k)
#pragma unroll
                for (int v = 0; v < 4; ++v) dcn[k][v] = 0.0f;
            if (R > 0 && next_n > 0) {
                if (w + 1 < NW) {
#pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const float4 f = lds[((w + 1) * RR + k) * 64 + wl];
                        dcn[k][0] = f.x; dcn[k][1] = f.y; dcn[k][2] = f.z; dcn[k][3] = f.w;
                    }
                } else {
                    // the tile's last wave: recompute the next tile's first next_n tokens (the
                    // input window continues from the span's last rows)
                    if (!kPrefetchNext) {
                        const int lastn = next_n - 1;
#pragma unroll
                        for (int k = 0; k < R; ++k) {
                            const int r = k < lastn ? k : lastn;
                            xn[k] = Q::load(x + roff((t0 + BT + r) * xs) + lane_off);
                            gn[k] = Q::load(dy + roff((t0 + BT + r) * row_bytes) + lane_off);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < R; ++k) {
                        const int i = BT + k;
                        if (k < next_n) {
                            Q::widen(xn[k], win[(i + R) % W]);
                            float g[4], chat[4];
                            Q::widen(gn[k], g);
                            token_dc<W, LPH>(win, i % W, tap, gam, g, a.eps, inv_d, dcn[k], chat);
                        }
                    }
                }
            }
#pragma unroll
            for (int q = BT - R; q < BT; ++q) {
                if (q < n) {
                    // sum_k taps[k] * dc[q + R - k]: own tokens from the ring, later ones from dcn
                    float de[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const int tk = q + R - k;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float dv = tk < BT ? dcr[tk % W][v] : dcn[tk - BT < RR ? tk - BT : 0][v];
                            de[v] = k == 0 ? tap[k][v] * dv : __builtin_fmaf(tap[k][v], dv, de[v]);
                        }
                    }
                    if (has_tail) add_state_loss<E, R>(gsr, p0 + q - (L - R), de);
                    if constexpr (PURE)
                        store_row<E>(dx, t0 + q, (uint32_t)row_bytes, true, lane_off,
                                     Q::narrow(de));
                    else if (active)
                        Q::store(dx + (t0 + q) * row_bytes + lane_off, Q::narrow(de));
                }
            }
            // The previous tile's deferred rows: row BT - R + m of its last span needs dc of
            // its tokens BT + m - k, k = 0..W-1: this span's token m - k when m >= k (this
            // wave's first R dc, left in LDS in phase 1), else the previous span's token
            // BT + m - k (handed over by the previous tile's last wave).
            if (kDefer && pending && w == 0) {
                const int hb = NW + ((gi - 1) & 1);
                float dn[RR][4], dp[RR][4];
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    const float4 f = lds[k * 64 + wl];
                    dn[k][0] = f.x; dn[k][1] = f.y; dn[k][2] = f.z; dn[k][3] = f.w;
                    const float4 g = lds[(hb * RR + k) * 64 + wl];
                    dp[k][0] = g.x; dp[k][1] = g.y; dp[k][2] = g.z; dp[k][3] = g.w;
                }
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    float de[4];
#pragma unroll
                    for (int k = 0; k < W; ++k) {
                        const int tk = m - k;
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const float dv = tk >= 0 ? dn[tk >= 0 ? tk : 0][v] : dp[tk >= 0 ? 0 : R + tk][v];
                            de[v] = k == 0 ? tap[k][v] * dv : __builtin_fmaf(tap[k][v], dv, de[v]);
                        }
                    }
                    const int64_t row = pending_t0 + BT - R + m;
                    if constexpr (PURE)
                        store_row<E>(dx, row, (uint32_t)row_bytes, true, lane_off, Q::narrow(de));
                    else if (active)
                        Q::store(dx + row * row_bytes + lane_off, Q::narrow(de));
                }
            }
        } else if (first_span && R > 0 && dstate != nullptr) {
            // an empty sequence: its new state is its initial window
#pragma unroll
            for (int m = 0; m < R; ++m) {
                float de[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (gs != nullptr && from_state) Q::widen(Q::load(gs_seq + roff(m * row_bytes) + lane_off), de);
                if (active)
                    Q::store(dstate + ((int64_t)s * R + m) * row_bytes + lane_off, Q::narrow(de));
            }
        }
        __syncthreads();  // the hand-off rows are rewritten by the next tile
        pending = defer;
        pending_t0 = start + p0_last;
    }

    // ---- the workgroup's partial of the parameter gradients: waves summed in order ----
    if (w > 0) {
#pragma unroll
        for (int k = 0; k <= W; ++k) {
            const float* f = k < W ? acc_t[k] : acc_g;
            lds[((w - 1) * (W + 1) + k) * 64 + wl] = make_float4(f[0], f[1], f[2], f[3]);
        }
    }
    __syncthreads();
    if (w == 0) {
        float4* out = reinterpret_cast<float4*>(a.partial) +
                      ((int64_t)group * slices + slice) * (W + 1) * 64;
#pragma unroll
        for (int k = 0; k <= W; ++k) {
            float f[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) f[v] = k < W ? acc_t[k][v] : acc_g[v];
#pragma unroll
            for (int ww = 0; ww < NW - 1; ++ww) {
                const float4 o = lds[(ww * (W + 1) + k) * 64 + wl];
                f[0] += o.x; f[1] += o.y; f[2] += o.z; f[3] += o.w;
            }
            out[k * 64 + wl] = make_float4(f[0], f[1], f[2], f[3]);
        }
    }
}

// The sum of the workgroup partials, in two fixed-order stages (so the result is the same on
// every run). A partial is [slices][W+1][64 lanes][4] fp32 = nb blocks of 256 floats.
//  stage A: block b of the partials summed over a chunk of kChunk groups, in group order, in fp64
//           (one thread per float, coalesced loads of all groups in flight);
//  stage B (one launch): the taps gradient sums its element's chunk sums in chunk order; the
//           gamma gradient, a sum over heads as well, takes one wave per output: lane l adds the
//           (head, chunk) pairs l, l+64, ... in order and a butterfly adds the 64 lane sums.
constexpr int kChunk = 64;

template <int W>
__global__ void __launch_bounds__(256) backward_chunk_kernel(BwdArgs a) {
    const int64_t nb = (int64_t)a.slices * (W + 1);
    const int64_t b = blockIdx.x;
    const int64_t c = blockIdx.y;
    const int64_t g0 = c * kChunk;
    const int64_t g1 = g0 + kChunk < a.groups ? g0 + kChunk : a.groups;
    const float* p = a.partial + b * 256 + threadIdx.x;
    double acc = 0.0;
#pragma unroll 16
    for (int64_t g = g0; g < g1; ++g) acc += (double)p[g * nb * 256];
    a.chunk[(c * nb + b) * 256 + threadIdx.x] = acc;
}

template <int W>
__device__ inline int64_t partial_index(const BwdArgs& a, int t, int k, int64_t ch) {
    const int64_t gl = (int64_t)t * a.lanes_per_tensor + ch / 4;  // lane holding the channel
    return ((gl / 64) * (W + 1) + k) * 256 + (gl % 64) * 4 + ch % 4;
}

// Stage B. Blocks [0, taps_blocks) give the taps gradient, one thread per element; the rest give
// the gamma gradient, one wave per element.
template <int W>
__global__ void __launch_bounds__(256) backward_final_kernel(BwdArgs a, int D, int taps_blocks) {
    const int64_t per_chunk = (int64_t)a.slices * (W + 1) * 256;
    if ((int)blockIdx.x < taps_blocks) {
        const int64_t HD = (int64_t)a.heads * D;
        const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
        if (id >= 2 * W * HD) return;
        const int t = (int)(id / (W * HD));
        const int64_t r = id - (int64_t)t * W * HD;
        const int k = (int)(r / HD);
        const int64_t ch = r - (int64_t)k * HD;
        const double* src = a.chunk + partial_index<W>(a, t, k, ch);
        double acc = 0.0;
#pragma unroll 8
        for (int c = 0; c < a.chunks; ++c) acc += src[c * per_chunk];
        pick(a.dtaps, t)[r] = (float)acc;
        return;
    }
    const int64_t wave = (int64_t)(blockIdx.x - taps_blocks) * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (wave >= 2 * D) return;  // whole waves leave together
    const int t = (int)(wave / D);
    const int d = (int)(wave - (int64_t)t * D);
    const int64_t pairs = (int64_t)a.heads * a.chunks;
    double acc = 0.0;
    for (int64_t i = lane; i < pairs; i += 64) {
        const int64_t hh = i / a.chunks, c = i - hh * a.chunks;
        acc += a.chunk[c * per_chunk + partial_index<W>(a, t, W, hh * D + d)];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) pick(a.dgamma, t)[d] = (float)acc;
}

using BwdFn = void (*)(BwdArgs);
template <class E, int D, int W>
constexpr BwdFn bwd_fn() { return backward_kernel<E, D, W, bwd_span<E, W>(), false>; }
template <class E, int D, int W>
constexpr BwdFn bwd_pure_fn() { return backward_kernel<E, D, W, bwd_span<E, W, true>(), true>; }

#define SC_BROW(K, E, D)                                                                  \
    { K<E, D, 1>(), K<E, D, 2>(), K<E, D, 3>(), K<E, D, 4>(), K<E, D, 5>(), K<E, D, 6>(),  \
      K<E, D, 7>(), K<E, D, 8>() }
const BwdFn kBackward[2][3][8] = {
    {SC_BROW(bwd_fn, F32, 64), SC_BROW(bwd_fn, F32, 128), SC_BROW(bwd_fn, F32, 256)},
    {SC_BROW(bwd_fn, BF16, 64), SC_BROW(bwd_fn, BF16, 128), SC_BROW(bwd_fn, BF16, 256)},
};
const BwdFn kBackwardPure[2][3][8] = {
    {SC_BROW(bwd_pure_fn, F32, 64), SC_BROW(bwd_pure_fn, F32, 128),
     SC_BROW(bwd_pure_fn, F32, 256)},
    {SC_BROW(bwd_pure_fn, BF16, 64), SC_BROW(bwd_pure_fn, BF16, 128),
     SC_BROW(bwd_pure_fn, BF16, 256)},
};
using ChunkFn = void (*)(BwdArgs);
using FinalFn = void (*)(BwdArgs, int, int);
#define SC_PER_W(K) {K<1>, K<2>, K<3>, K<4>, K<5>, K<6>, K<7>, K<8>}
const ChunkFn kChunkSum[8] = SC_PER_W(backward_chunk_kernel);
const FinalFn kFinal[8] = SC_PER_W(backward_final_kernel);

int d_index(int D) { return D == 64 ? 0 : (D == 128 ? 1 : 2); }

}  // namespace

BwdShape backward_shape(int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                        int32_t head_dim, int32_t width, int dtype) {
    BwdShape sh;
    sh.lanes_per_tensor = (int64_t)num_heads * head_dim / 4;
    sh.slices = (2 * sh.lanes_per_tensor + 63) / 64;
    const bool pure = sh.lanes_per_tensor % 64 == 0;  // the kernel launch_backward picks
    const int bt = dtype == 1 ? (pure && width <= 4 ? bwd_span<BF16, 1, true>()
                                 : width <= 5       ? bwd_span<BF16, 1>()
                                 : pure             ? bwd_span<BF16, 8, true>()
                                                    : bwd_span<BF16, 8>())
                              : (width <= 1 ? bwd_span<F32, 1>() : bwd_span<F32, 8>());
    const int64_t bb = (int64_t)kBwdWaves * bt;
    sh.tiles = total_tokens / bb + num_seqs;
    int64_t per = sh.tiles * sh.slices / kFillBlocks;
    int64_t max_per = kMaxPartialTokens / bt;
    max_per = max_per < 1 ? 1 : (max_per > SC_BWD_MAX_TILES ? SC_BWD_MAX_TILES : max_per);
    per = per < 1 ? 1 : (per > max_per ? max_per : per);
    sh.tiles_per_group = per;
    sh.groups = (sh.tiles + per - 1) / per;
    sh.chunks = (sh.groups + kChunk - 1) / kChunk;
    const int64_t nb = sh.slices * (width + 1);  // 256-float blocks per partial
    sh.partial_bytes = (size_t)sh.groups * nb * 256 * 4;
    sh.workspace_bytes = sh.partial_bytes + (size_t)sh.chunks * nb * 256 * 8;
    return sh;
}

hipError_t launch_backward(BwdArgs a, int dtype, int head_dim, int width, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.groups * a.slices;
    if (blocks > 0) {
        const bool pure = a.lanes_per_tensor % 64 == 0;
        hipLaunchKernelGGL((pure ? kBackwardPure : kBackward)[dtype][d_index(head_dim)][width - 1],
                           dim3((unsigned)blocks), dim3(kBwdBlock), 0, stream, a);
        hipLaunchKernelGGL(kChunkSum[width - 1],
                           dim3((unsigned)(a.slices * (width + 1)), (unsigned)a.chunks), dim3(256),
                           0, stream, a);
    }
    const int64_t taps = 2 * (int64_t)width * a.heads * head_dim;
    const int taps_blocks = (int)((taps + 255) / 256);
    const int gamma_blocks = (2 * head_dim + 3) / 4;
    hipLaunchKernelGGL(kFinal[width - 1], dim3((unsigned)(taps_blocks + gamma_blocks)), dim3(256),
                       0, stream, a, head_dim, taps_blocks);
    return hipGetLastError();
}

}  // namespace sc
