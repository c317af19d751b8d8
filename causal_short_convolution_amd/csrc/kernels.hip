// HIP kernels of the fused ShortConv K/V step for gfx950 (MI355X).
//
// The step is a memory-bound stencil over tokens (causal depthwise convolution of width W over the
// projected K and V, aib.vote English news item on SGLang/Miles Inkling support, paragraphs 1-2;
// the window is the current row and the W-1 before it, axbrief.com Inkling specifications blog,
// SConv section), followed by RMSNorm over head_dim, the paged KV-cache write and the
// conv-state update. It has ~(2W+4) flops per element against 2 bytes read and 2 written in bf16,
// far under the fp32 vector ridge of the chip, so no matrix cores are involved: the design is
// about moving each byte once with full-width memory instructions.
//
// Thread layout (prefill and decode alike): one lane owns 16 bytes of one token row of one tensor,
// i.e. VEC = 8 bf16 or 4 fp32 channels of one head. LPH = D / VEC lanes cover a head; a 64-wide
// wavefront covers 64 * 16 B = 1 KiB of a row, so every global load and store is a fully used,
// contiguous 16-byte-per-lane access. Lanes [0, lanes_per_tensor) work on K and the rest on V.
//
// Prefill tiles: a workgroup covers one 64-lane (1 KiB) column slice of the K|V rows over a tile of
// 4 * BT consecutive tokens of ONE sequence (BT = 8 for W <= 4, 16 for wider windows, whose
// halo is a larger share of a short span); each of its 4 wavefronts walks BT of those tokens,
// keeping the window in registers (each input row is loaded once and reused by the W outputs
// that read it). Wave w > 0 gets its W-1 halo rows from wave w-1 through LDS (an LDS-staged
// halo, so a row is fetched from HBM once); wave 0 reads the tail of the previous tile of the
// same sequence, or the sequence's conv state / zeros for its first tile. All 4 waves use the
// same taps and gamma, so 3 of 4 parameter loads hit in L1. Tiles never straddle sequences:
// sequence s owns tiles [P(s), P(s) + max(1, ceil(L_s / (4*BT)))) with P(s) = floor(cu[s] /
// (4*BT)) + s. P is strictly increasing and P(s) + max(1, ceil(L_s/(4*BT))) <= P(s+1), so a
// workgroup finds its sequence by a wave-parallel search over cu_seqlens (one vector load per 64x
// narrowing, whose lanes also hold the sequence's bounds when there are at most 63 sequences)
// with no host-side scan; at most one tile per sequence is empty.
//
// MXFP8 rows over one-tensor slices on large grids instead take one run of 16 tokens per wave
// (prefill_run_kernel): the run's rows are loaded one 4-token sub-span ahead of the arithmetic
// and the window is carried in registers, which hides the encoder's extra arithmetic.
//
// Memory order within a wave: after the search, every load of the span goes out back to back
// (parameters, halo, the rows the next wave needs first, the other rows, the span's slots as one
// vector load), with no branch between them; then the tokens are computed in order, each
// waiting only for its own row (see the token loop for why the first stores wait until half
// the span is computed).
//
// Conv-state ownership: only the first wave of a sequence's first tile reads the old state (its
// halo), so that wave also writes the new state (the sequence's last W-1 raw rows, taken from the
// read-only input and, when the sequence is shorter than W-1, from the surviving old rows). No
// other workgroup touches that state row, so no grid-wide synchronization is needed.
//
// Numerics (shared by prefill and decode through fused_row, so the two are bit-identical):
// inputs widen exactly to fp32; c = taps[0]*x[0], then fma over k = 1..W-1; the sum of squares is an
// fma chain over the lane's channels followed by a butterfly across the LPH lanes (every lane
// ends with the same bits, since each step adds the same two values); 1/sqrt(ss/D + eps) comes from
// the hardware reciprocal square root; y = (c * (1/r)) * gamma, rounded once to the element type
// (round to nearest even). With eps = 0, scaling the inputs by a power of two leaves y
// bit-identical.
#include "device_common.h"
#include "shortconv_internal.h"

namespace sc {
namespace {

constexpr int kBlock = 256;  // threads per workgroup (4 wavefronts)

// Build-time tuning knobs (defaults chosen by measurement on MI355X): tokens per wave span in
// prefill and the minimum resident waves per SIMD that the register budget must allow, for
// narrow (W <= 4) and wide windows, with plain and with MXFP8 cache rows.
#ifndef SC_BT_NARROW
#define SC_BT_NARROW 8
#endif
#ifndef SC_WAVES_NARROW
#define SC_WAVES_NARROW 4
#endif
#ifndef SC_BT_NARROW_MX
#define SC_BT_NARROW_MX 8
#endif
#ifndef SC_WAVES_NARROW_MX
#define SC_WAVES_NARROW_MX 3
#endif
#ifndef SC_BT_WIDE
#define SC_BT_WIDE 16
#endif
#ifndef SC_WAVES_WIDE
#define SC_WAVES_WIDE 2
#endif
#ifndef SC_BT_WIDE_MX
#define SC_BT_WIDE_MX 16
#endif
#ifndef SC_WAVES_WIDE_MX
#define SC_WAVES_WIDE_MX 2
#endif

// XCD-contiguous order of the units for W > 4 (see prefill_kernel). Measured on MI355X (bf16,
// W = 8, 131072 tokens, one process): 174.9 -> 171.9 us, MXFP8 rows 185.9 -> 183.6 us. (For
// narrow windows the same order measured neutral to slower.)
#ifndef SC_WIDE_XCD_ORDER
#define SC_WIDE_XCD_ORDER 1
#endif

template <int W, bool MX>
constexpr int span_tokens() {
    return W <= 4 ? (MX ? SC_BT_NARROW_MX : SC_BT_NARROW) : (MX ? SC_BT_WIDE_MX : SC_BT_WIDE);
}
template <int W, bool MX>
constexpr int span_min_waves() {
    return W <= 4 ? (MX ? SC_WAVES_NARROW_MX : SC_WAVES_NARROW)
                  : (MX ? SC_WAVES_WIDE_MX : SC_WAVES_WIDE);
}

// Per-lane constants of one (tensor, head, 16-byte column) position.
template <class E, int W>
struct LaneParams {
    float tap[W][E::VEC];
    float gam[E::VEC];
};

template <class E, int W>
__device__ inline void load_params(const float* taps, const float* gamma, int heads, int D, int h,
                                   int d0, LaneParams<E, W>& p) {
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const float* t = taps + ((int64_t)k * heads + h) * D + d0;
#pragma unroll
        for (int v = 0; v < E::VEC; v += 4) {
            const float4 q = *reinterpret_cast<const float4*>(t + v);
            p.tap[k][v] = q.x;
            p.tap[k][v + 1] = q.y;
            p.tap[k][v + 2] = q.z;
            p.tap[k][v + 3] = q.w;
        }
    }
#pragma unroll
    for (int v = 0; v < E::VEC; v += 4) {
        const float4 q = *reinterpret_cast<const float4*>(gamma + d0 + v);
        p.gam[v] = q.x;
        p.gam[v + 1] = q.y;
        p.gam[v + 2] = q.z;
        p.gam[v + 3] = q.w;
    }
}

// The row math of one output row slice: window row k (k = W-1 is the current token) is
// win[(off + k) % W], off being a compile-time constant after unrolling; o gets the normalized
// values in fp32, before the one rounding to the cache format.
template <class E, int W, int LPH>
__device__ inline void fused_row(const float (&win)[W][E::VEC], int off,
                                 const LaneParams<E, W>& p, float eps, float inv_d,
                                 float (&o)[E::VEC]) {
    constexpr int VEC = E::VEC;
    float c[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) c[v] = p.tap[0][v] * win[off % W][v];
#pragma unroll
    for (int k = 1; k < W; ++k)
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            c[v] = __builtin_fmaf(p.tap[k][v], win[(off + k) % W][v], c[v]);
    float ss = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) ss = __builtin_fmaf(c[v], c[v], ss);
    ss = head_sum<LPH>(ss);
    // v_rsq_f32: within ~1 ulp of 1/sqrt, one instruction instead of a correctly rounded square
    // root and divide; it scales exactly under power-of-4 scaling of its input.
    const float inv = __builtin_amdgcn_rsqf(__builtin_fmaf(ss, inv_d, eps));
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = (c[v] * inv) * p.gam[v];
}

// ------------------------------------------------------------------------------------------------
// Cache formats. A Sink takes one finished row slice (VEC fp32 values of one head) and writes it
// to cache row `slot`, unless the slot is outside [0, num_slots) or the lane is idle.
// ------------------------------------------------------------------------------------------------
// Plain rows in the I/O element type (one round-to-nearest-even conversion).
template <class E>
struct PlainSink {
    char* cache;
    int64_t row_bytes;
    uint32_t lane_off;
    int64_t num_slots;
    __device__ PlainSink(const StepArgs& a, int tensor, int h, int d0, int D)
        : cache(static_cast<char*>(pick(a.cache, tensor))),
          row_bytes((int64_t)a.heads * D * E::BYTES),
          lane_off((uint32_t)(((int64_t)h * D + d0) * E::BYTES)),
          num_slots(a.num_slots) {}
    // A row slice in its stored form, and its store (skipped for an idle lane or a slot outside
    // the pool).
    using Enc = uint4;
    __device__ Enc encode(const float (&o)[E::VEC]) const { return E::narrow(o); }
    // The slot is wave-uniform in every caller; its byte offset is kept scalar (read through
    // readfirstlane), so the address is one add to the lane's base instead of a 64-bit
    // multiply-add on the vector unit at quarter rate.
    __device__ void write(int64_t slot, bool active, const Enc& out) const {
        if (active && slot >= 0 && slot < num_slots)
            strow(cache + uniform(slot * row_bytes), lane_off, out);
    }
    __device__ void put(int64_t slot, bool active, const float (&o)[E::VEC]) const {
        write(slot, active, encode(o));
    }
};

// OCP FP8 E4M3 codes of v[b] * 2^-e for four finite values (byte b): nearest value, ties to even,
// saturating at +-448. gfx950's scaled conversion (v_cvt_scalef32_pk_fp8_f32) divides by its
// scale operand, here 2^e, exactly and rounds to nearest even into the OCP format, but does not
// saturate; clamping v to +-448 * 2^e first is the same as clamping v * 2^-e to +-448, scaling by
// a power of two being exact.
typedef short sc_i16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t e4m3x4_scaled(float v0, float v1, float v2, float v3, float scale,
                                         float lim) {
    v0 = __builtin_amdgcn_fmed3f(v0, -lim, lim);
    v1 = __builtin_amdgcn_fmed3f(v1, -lim, lim);
    v2 = __builtin_amdgcn_fmed3f(v2, -lim, lim);
    v3 = __builtin_amdgcn_fmed3f(v3, -lim, lim);
    // the two conversions write the low and the high half; the word they start from (any
    // register at hand) is overwritten entirely
    sc_i16x2 w = __builtin_bit_cast(sc_i16x2, __float_as_uint(v0));
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, v0, v1, scale, false);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, v2, v3, scale, true);
    return __builtin_bit_cast(uint32_t, w);
}

// The MXFP8 encoding of one lane's VEC values: the maximum over the 32/VEC lanes of a 32-element
// block (DPP), the E8M0 exponent e = floor(log2(max)) - 8 clamped to [-127, 127] (-127 for an
// all-zero block), and the saturated E4M3 codes of v * 2^-e. Across lanes the maximum of the
// magnitudes is taken on their bit patterns, which order non-negative finite floats as unsigned
// integers do; the pattern's exponent field E gives floor(log2(max)) = E - 127 for a normal
// maximum, so e = E - 135, which is at most 119, and every zero or subnormal maximum (E = 0)
// falls to the clamp at -127.
template <class E>
struct MxEnc {
    uint32_t packed[E::VEC / 4];
    int e;
};
template <class E>
__device__ inline MxEnc<E> mx_encode(const float (&o)[E::VEC]) {
    constexpr int VEC = E::VEC;
    constexpr int LPB = 32 / VEC;
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < VEC; ++v) amax = __builtin_fmaxf(amax, __builtin_fabsf(o[v]));
    uint32_t bits = __float_as_uint(amax);
    bits = max(bits, dpp_u32<kQuadXor1>(bits));
    bits = max(bits, dpp_u32<kQuadXor2>(bits));
    if (LPB == 8) bits = max(bits, dpp_u32<kRowHalfMirror>(bits));
    MxEnc<E> r;
    const int e = max((int)(bits >> 23) - 135, -127);
    r.e = e;
    const float scale = __builtin_ldexpf(1.0f, e);
    const float lim = __builtin_ldexpf(448.0f, e);  // +inf at e = 127: nothing saturates there
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q)
        r.packed[q] = e4m3x4_scaled(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3], scale, lim);
    return r;
}

// MXFP8 rows: 32-element blocks along head_dim share one E8M0 scale 2^e with
// e = floor(log2(max |v|)) - 8 (clamped to [-127, 127]; -127 for an all-zero block), and each
// element is stored as the E4M3 code of v * 2^-e. Codes [num_slots][H][D] bytes, scales
// [num_slots][H][D/32] bytes (e + 127). The 32/VEC lanes of a block exchange their maxima by DPP.
template <class E>
struct MxSink {
    static constexpr int VEC = E::VEC;
    static constexpr int LPB = 32 / VEC;  // lanes per block: 4 (bf16) or 8 (fp32)
    char* codes;
    char* scales;
    int64_t row_elems;
    uint32_t code_off;
    uint32_t scale_off;
    bool scale_lane;
    int64_t num_slots;
    __device__ MxSink(const StepArgs& a, int tensor, int h, int d0, int D)
        : codes(static_cast<char*>(pick(a.cache, tensor))),
          scales(static_cast<char*>(pick(a.scales, tensor))),
          row_elems((int64_t)a.heads * D),
          code_off((uint32_t)((int64_t)h * D + d0)),
          scale_off((uint32_t)(((int64_t)h * D + d0) / 32)),
          scale_lane(d0 % 32 == 0),
          num_slots(a.num_slots) {}
    using Enc = MxEnc<E>;  // the VEC codes, 4 per word, and the block's scale exponent
    __device__ Enc encode(const float (&o)[VEC]) const { return mx_encode<E>(o); }
    __device__ void write(int64_t slot, bool active, const Enc& enc) const {
        if (!(active && slot >= 0 && slot < num_slots)) return;
        char* row = codes + uniform(slot * row_elems) + code_off;  // (offset kept scalar)
        if (VEC == 8) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 w = {enc.packed[0], enc.packed[VEC / 4 - 1]};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(row));
        } else {
            __builtin_nontemporal_store(enc.packed[0], reinterpret_cast<uint32_t*>(row));
        }
        if (scale_lane)
            *reinterpret_cast<uint8_t*>(scales + uniform(slot * (row_elems / 32)) + scale_off) =
                (uint8_t)(enc.e + 127);
    }
    __device__ void put(int64_t slot, bool active, const float (&o)[VEC]) const {
        write(slot, active, encode(o));
    }
};

template <class E, bool MX>
struct SinkFor { using type = PlainSink<E>; };
template <class E>
struct SinkFor<E, true> { using type = MxSink<E>; };

// ------------------------------------------------------------------------------------------------
// Prefill
// ------------------------------------------------------------------------------------------------
// PURE: every 64-lane slice holds one tensor (H * D a multiple of 256 elements of each of K and
// V), so every lane is active and the tensor, with every base address picked by it, is
// wave-uniform: row and cache addresses are then a scalar base plus the lane's 32-bit offset
// (fewer 64-bit multiply-adds on the vector unit, at quarter rate). Measured on MI355X (W = 8,
// 131 072 tokens, same process): bf16 rows 169.2 -> 168.4 us, MXFP8 rows 179.2 -> 177.4 us,
// outputs bit-identical.
template <class E, int D, int W, int BT, bool MX, bool PURE>
__global__ void __launch_bounds__(kBlock, (span_min_waves<W, MX>())) prefill_kernel(StepArgs a) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    constexpr int R = W - 1;
    constexpr int NW = kBlock / 64;  // waves per workgroup, one BT-token span each
    constexpr int BB = NW * BT;      // tokens per workgroup tile
    // A wave's halo is the tail of the previous wave's span, and the tile holding a sequence's
    // first token holds every position that reads the old state.
    static_assert(BT >= R, "a wave's span must cover the conv halo");
    static_assert(BT <= 64, "a wave loads one slot per lane");
    // Tail rows that wave w hands to wave w+1 (an LDS-staged halo: HBM is read once per row).
    __shared__ uint4 handoff[NW - 1][R > 0 ? R : 1][64];

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wl = threadIdx.x & 63;
    // Linear workgroup id = tile * slices + slice: the slices of one tile (the 1 KiB pieces of the
    // same rows) are dispatched together, so each row is read and written in one burst.
    const int slices = a.lane_blocks;
    // Wide windows can order the units so that each XCD (workgroups are dealt to the 8 XCDs in
    // turn) takes a contiguous run of them: consecutive tiles of a slice then share an L2, where
    // a tile's first wave finds the halo rows the previous tile loaded.
    int unit = blockIdx.x;
    if constexpr (W > 4 && SC_WIDE_XCD_ORDER) {
        const int G = gridDim.x, b = blockIdx.x, x = b % 8, q = G / 8, r = G % 8;
        unit = x * q + (x < r ? x : r) + b / 8;
    }
    const int tile = unit / slices;
    const int slice = unit - tile * slices;
    const int lane = slice * 64 + wl;
    // idle lanes load lane 0's column and store nothing
    const bool active = PURE || lane < 2 * a.lanes_per_tensor;
    const int ln = active ? lane : 0;
    const int tensor = PURE ? uniform(slice * 64 >= a.lanes_per_tensor ? 1 : 0)
                            : (ln >= a.lanes_per_tensor ? 1 : 0);
    const int c = ln - tensor * a.lanes_per_tensor;
    const int h = c / LPH;
    const int d0 = (c - h * LPH) * VEC;
    const int64_t T = a.tokens;

    // Which sequence owns this tile (the same answer in every wave of the block).
    const int s = find_tile_seq<BB>(a.cu, a.num_seqs, T, tile);
    const int64_t start = uniform((int64_t)clamp_tok(a.cu[s], T));
    int64_t end = uniform((int64_t)clamp_tok(a.cu[s + 1], T));
    if (end < start) end = start;
    const int64_t L = end - start;
    const int64_t j = tile - tile_base<BB>(a.cu, s, T);
    const int64_t ntiles = L > 0 ? (L + BB - 1) / BB : 1;
    if (j < 0 || j >= ntiles) return;  // the whole workgroup leaves together

    const char* x = static_cast<const char*>(pick(a.x, tensor));
    const int64_t stride_bytes = pick(a.x_stride, tensor) * E::BYTES;
    const typename SinkFor<E, MX>::type sink(a, tensor, h, d0, D);
    char* state = static_cast<char*>(pick(a.state, tensor));
    const int64_t row_bytes = (int64_t)a.heads * D * E::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * E::BYTES);

    // This wave's span: tokens [t0, t0 + n) of the sequence.
    const int64_t t0 = start + j * BB + (int64_t)w * BT;
    const int64_t rem = end - t0;
    const int n = rem <= 0 ? 0 : (rem < BT ? (int)rem : BT);
    const char* xb = x + t0 * stride_bytes;

    int32_t idx = -1;
    bool slot_ok = false, read_state = false;
    if (j == 0) {
        idx = uniform(a.state_idx ? a.state_idx[s] : s);
        slot_ok = R > 0 && state != nullptr && idx >= 0 && idx < a.num_state_slots;
        read_state = slot_ok && (a.has_init ? a.has_init[s] != 0 : true);
    }

    // Every load of a span goes out back to back (vector loads return in order), with no branch
    // between them that could leave the compiler unsure how many are in flight: taps and gamma
    // (cache hits), the first wave's halo, the rows the next wave needs, the other rows, and the
    // span's cache slots. A wave whose span starts past its sequence's end loads nothing.
    const bool has_rows = n > 0;
    const bool first_span = j == 0 && w == 0;
    LaneParams<E, W> p;
    uint4 halo[R > 0 ? R : 1];
    uint4 raw[BT];
    int64_t lane_slot = -1;
    if (has_rows) {
        load_params<E, W>(pick(a.taps, tensor), pick(a.gamma, tensor), a.heads, D, h, d0, p);
        // The first wave's R window rows before its span: the previous tile's last rows, the
        // stored state, or zeros (loaded from a valid stand-in, the taps, and cleared later).
        // The other waves get theirs from the wave before through LDS.
        if (w == 0) {
            const char* state_row = state + (int64_t)(slot_ok ? idx : 0) * R * row_bytes;
            const char* hsrc = j > 0 ? x + (t0 - R) * stride_bytes
                               : read_state ? state_row
                                            : reinterpret_cast<const char*>(pick(a.taps, tensor));
            const int64_t hstride = j > 0 ? stride_bytes : row_bytes;
#pragma unroll
            for (int k = 0; k < R; ++k) halo[k] = ldrow_keep(hsrc + uniform(k * hstride), lane_off);
        }
        // Past a short span's end the last row is read again (and not used). Lane l < BT loads
        // token l's cache slot (one vector load instead of BT scalar ones, which the compiler
        // would issue only after the rows arrive).
        const int last = n - 1;
        // The R rows at the end of the span (and the first wave's halo rows, above) are loaded
        // without the streaming hint, the others with it: measured on MI355X, this mix is faster
        // than all streaming (varlen bf16 prefill 30.3 -> 28.1 us) or none, with unchanged HBM
        // reads in the counters; why it is faster is not established.
        // (row offsets kept scalar, as in the sinks)
#pragma unroll
        for (int i = BT - R; i < BT; ++i)
            raw[i] = ldrow_keep(xb + uniform((i < last ? i : last) * stride_bytes), lane_off);
#pragma unroll
        for (int i = 0; i < BT - R; ++i)
            raw[i] = ldrow(xb + uniform((i < last ? i : last) * stride_bytes), lane_off);
        lane_slot = a.slot[t0 + (wl < last ? wl : last)];
    }
    // LDS-staged halo: wave w hands its last R rows to wave w + 1, so a row is fetched once.
    // (A wave with a short span is the last with rows in its tile; what it hands on is unused.)
    if (R > 0) {
        if (has_rows && w + 1 < NW) {
#pragma unroll
            for (int k = 0; k < R; ++k) handoff[w][k][wl] = raw[BT - R + k];
        }
        __syncthreads();
        if (has_rows && w > 0) {
#pragma unroll
            for (int k = 0; k < R; ++k) halo[k] = handoff[w - 1][k][wl];
        }
    }

    if (has_rows) {
        if (first_span && !read_state) {
#pragma unroll
            for (int k = 0; k < R; ++k) halo[k] = make_uint4(0, 0, 0, 0);
        }
        float win[W][VEC];
#pragma unroll
        for (int k = 0; k < R; ++k) E::widen(halo[k], win[k]);
        const float inv_d = 1.0f / (float)D;
        // The window is a ring: token i's row goes to win[(i + R) % W], over the oldest row,
        // which no later token reads, so advancing it costs no register moves.
        // The first H1 tokens of the span are computed before any store is issued: with no store
        // among them, the compiler knows which loads are still in flight and waits for each
        // row just before its token, so those tokens are computed while later rows arrive. By
        // then every row is in (one wait makes sure), their rows are stored, and the remaining
        // tokens are computed and stored with nothing left in flight. (A conditional store
        // between tokens would make the compiler wait, at every later token, for everything
        // issued so far, that store included.) Holding H1 encoded rows costs registers; wide
        // windows, with fewer waves per SIMD anyway, hold the whole span.
        constexpr int H1 = W <= 4 ? BT / 2 : BT;
        typename SinkFor<E, MX>::type::Enc out[H1];
#pragma unroll
        for (int i = 0; i < H1; ++i) {
            if (i < n) {
                E::widen(raw[i], win[(i + R) % W]);
                float o[VEC];
                fused_row<E, W, LPH>(win, i % W, p, a.eps, inv_d, o);
                out[i] = sink.encode(o);
            }
            // Token by token: left free, the scheduler widens later rows early and runs out of
            // registers.
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_vmem();
#pragma unroll
        for (int i = 0; i < H1; ++i)
            if (i < n) sink.write(lane_value(lane_slot, i), active, out[i]);
#pragma unroll
        for (int i = H1; i < BT; ++i) {
            if (i < n) {
                E::widen(raw[i], win[(i + R) % W]);
                float o[VEC];
                fused_row<E, W, LPH>(win, i % W, p, a.eps, inv_d, o);
                sink.put(lane_value(lane_slot, i), active, o);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The sequence's first tile writes its new state (its first wave read the old one): row i =
    // e[L + i], e being the initial window followed by the sequence's rows. Rows are written in
    // increasing i and row i may read old row L + i > i, which is therefore still unmodified.
    if (R > 0 && j == 0 && w == 0 && slot_ok) {
        char* dst = state + (int64_t)idx * R * row_bytes;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t e = L + i;
            uint4 r = make_uint4(0, 0, 0, 0);
            if (e >= R)
                r = ldrow(x + (start + e - R) * stride_bytes, lane_off);
            else if (read_state)
                r = ldrow(dst + e * row_bytes, lane_off);
            if (active && (e != i || !read_state))  // e == i with a read state is a no-op copy
                strow(dst + i * row_bytes, lane_off, r);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Prefill over column slices that each hold one tensor (H * D a multiple of 64 lanes' worth of
// elements, so K and V never share a wavefront), for windows of width <= 4.
//
// The same tiles, spans, LDS hand-off and row math as prefill_kernel, with these differences:
//  - every cache store is issued unconditionally through a buffer resource whose range is the
//    destination row: a slot outside the pool (or a token past the span's end) gets an empty
//    range and the hardware drops the store. With no load or store under a branch, the compiler
//    knows exactly how many memory operations follow each row load and waits for that row alone,
//    so each token's row is stored as soon as it is computed and no finished rows are held in
//    registers (the MXFP8 variant fits 4 waves per SIMD, against 3 for prefill_kernel);
//  - the tensor, and so every base address, is wave-uniform;
//  - the workgroup walks units (tile, slice) g, g + G, ... (slice fastest, G a multiple of the
//    slice count) with the hand-off buffer alternating between two halves from one unit to the
//    next, so that a persistent grid can be used; by default G is the number of units (measured
//    fastest), and each workgroup handles one.
// ------------------------------------------------------------------------------------------------
constexpr int kBufferDword3 = 0x00020000;  // raw (untyped, unswizzled) buffer resource, gfx9
constexpr int kNonTemporal = 2;            // cache policy of the streaming stores

// A resource covering `bytes` bytes at row `row` of `base`, or an empty one (every access out of
// range, so stores are dropped and loads return zero) when !valid. All arguments wave-uniform.
__device__ inline __amdgpu_buffer_rsrc_t row_resource(char* base, int64_t row, uint32_t bytes,
                                                      bool valid) {
    char* p = base + (valid ? row : 0) * (int64_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, valid ? (int)bytes : 0, kBufferDword3);
}

// Plain cache rows of one tensor (wave-uniform destination).
template <class E>
struct PlainRows {
    char* cache;
    uint32_t row_bytes;
    uint32_t voff;
    int64_t num_slots;
    __device__ PlainRows(char* c, uint32_t rb, uint32_t lane_off, int64_t ns)
        : cache(c), row_bytes(rb), voff(lane_off), num_slots(ns) {}
    using Enc = uint4;
    __device__ Enc encode(const float (&o)[E::VEC]) const { return E::narrow(o); }
    __device__ void write(int64_t slot, const Enc& e) const {
        const bool ok = slot >= 0 && slot < num_slots;
        const u32x4 v = {e.x, e.y, e.z, e.w};
        __builtin_amdgcn_raw_buffer_store_b128(v, row_resource(cache, slot, row_bytes, ok), voff,
                                               0, kNonTemporal);
    }
};

// MXFP8 cache rows of one tensor: the codes row and the scales row each through its own resource;
// lanes that do not hold a block's first element aim their scale store past the range.
template <class E>
struct MxRows {
    static constexpr int VEC = E::VEC;
    char* codes;
    char* scales;
    uint32_t code_bytes;   // H * D
    uint32_t scale_bytes;  // H * D / 32
    uint32_t code_voff;
    uint32_t scale_voff;
    int64_t num_slots;
    __device__ MxRows(char* c, char* sc, uint32_t row_elems, int h, int d0, int D, int64_t ns)
        : codes(c), scales(sc), code_bytes(row_elems), scale_bytes(row_elems / 32),
          code_voff((uint32_t)(h * D + d0)),
          scale_voff(d0 % 32 == 0 ? (uint32_t)((h * D + d0) / 32) : row_elems / 32),
          num_slots(ns) {}
    using Enc = MxEnc<E>;
    __device__ Enc encode(const float (&o)[VEC]) const { return mx_encode<E>(o); }
    __device__ void write(int64_t slot, const Enc& enc) const {
        const bool ok = slot >= 0 && slot < num_slots;
        if (VEC == 8) {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t v = {enc.packed[0], enc.packed[VEC / 4 - 1]};
            __builtin_amdgcn_raw_buffer_store_b64(v, row_resource(codes, slot, code_bytes, ok),
                                                  code_voff, 0, kNonTemporal);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(enc.packed[0],
                                                  row_resource(codes, slot, code_bytes, ok),
                                                  code_voff, 0, kNonTemporal);
        }
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(enc.e + 127),
                                             row_resource(scales, slot, scale_bytes, ok),
                                             scale_voff, 0, 0);
    }
};

template <class E, bool MX>
struct RowsFor { using type = PlainRows<E>; };
template <class E>
struct RowsFor<E, true> { using type = MxRows<E>; };

#ifndef SC_SLICE_WAVES
#define SC_SLICE_WAVES 4
#endif
#ifndef SC_SLICE_WAVES_MX
#define SC_SLICE_WAVES_MX 4
#endif
// Windows of 5 and 6 fit 3 waves per SIMD in registers, 7 and 8 only 2.
#ifndef SC_SLICE_WAVES_WIDE
#define SC_SLICE_WAVES_WIDE 2
#endif

// Waves per workgroup of prefill_slice_kernel: a tile is this many consecutive spans of one
// column slice (see SC_SLICE_LDS_HALO for where each span's halo comes from). Measured on MI355X
// (varlen bf16 prefill, one process): 4 waves x 8-token spans 28.2 us; 8 x 4 33.6 us; 16 x 4
// 35.2 us; 8 x 8 29.4 us; 2 x 8 28.8 us; 1 x 8 (each wave reading its own halo) 30.8 us. Shorter
// spans keep fewer rows in flight per wave, and that costs more than the shorter tail of the grid
// gains; smaller workgroups re-read more halo rows from other workgroups.
#ifndef SC_SLICE_NW
#define SC_SLICE_NW 4
#endif
constexpr int kSliceBlock = 64 * SC_SLICE_NW;
// 1: a span's halo comes from the previous wave of its workgroup through LDS; 0: every wave loads
// its own halo rows, which the previous wave of the same workgroup is fetching at the same time
// (no workgroup barrier). For plain and for MXFP8 rows. Measured on MI355X, one process, LDS /
// own rows: bf16 rows, varlen 27.7 / 27.4 us, mixed 347.8 / 360.5 us; MXFP8 rows (6 rounds),
// varlen 25.6 / 25.2 us, mixed 325.5 / 320.8 us.
#ifndef SC_SLICE_LDS_HALO
#define SC_SLICE_LDS_HALO 1
#endif
#ifndef SC_SLICE_LDS_HALO_MX
#define SC_SLICE_LDS_HALO_MX 0
#endif

template <int W, bool MX>
constexpr int slice_min_waves() {
    return W <= 4 ? (MX ? SC_SLICE_WAVES_MX : SC_SLICE_WAVES) : (W <= 6 ? 3 : SC_SLICE_WAVES_WIDE);
}

template <class E, int D, int W, int BT, bool MX>
__global__ void __launch_bounds__(kSliceBlock, (slice_min_waves<W, MX>()))
    prefill_slice_kernel(StepArgs a) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    constexpr int R = W - 1;
    constexpr int NW = kSliceBlock / 64;
    constexpr int BB = NW * BT;
    static_assert(BT >= R && BT <= 64, "span length");
    using Rows = typename RowsFor<E, MX>::type;
    constexpr bool kLdsHalo = NW > 1 && (MX ? SC_SLICE_LDS_HALO_MX : SC_SLICE_LDS_HALO);
    __shared__ uint4 handoff[kLdsHalo ? 2 : 1][kLdsHalo ? NW - 1 : 1][R > 0 && kLdsHalo ? R : 1][64];

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wl = threadIdx.x & 63;
    const int slices = a.lane_blocks;
    const int64_t units = (int64_t)a.tiles * slices;
    if ((int64_t)blockIdx.x >= units) return;
    const int slice = uniform((int32_t)(blockIdx.x % slices));
    // whole slices hold one tensor: the tensor, and everything picked by it, is wave-uniform
    const int tensor = uniform(slice * 64 >= a.lanes_per_tensor ? 1 : 0);
    const int c = slice * 64 + wl - tensor * a.lanes_per_tensor;
    const int h = c / LPH;
    const int d0 = (c - h * LPH) * VEC;
    const int64_t T = a.tokens;
    const char* x = static_cast<const char*>(tensor ? a.x[1] : a.x[0]);
    const int64_t stride_bytes = (tensor ? a.x_stride[1] : a.x_stride[0]) * E::BYTES;
    char* state = static_cast<char*>(tensor ? a.state[1] : a.state[0]);
    const float* taps = tensor ? a.taps[1] : a.taps[0];
    const int64_t row_bytes = (int64_t)a.heads * D * E::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * E::BYTES);
    char* stand_in = reinterpret_cast<char*>(const_cast<float*>(taps));  // >= one row long
    const Rows rows = [&] {
        if constexpr (MX)
            return Rows(static_cast<char*>(tensor ? a.cache[1] : a.cache[0]),
                        static_cast<char*>(tensor ? a.scales[1] : a.scales[0]),
                        (uint32_t)(a.heads * D), h, d0, D, a.num_slots);
        else
            return Rows(static_cast<char*>(tensor ? a.cache[1] : a.cache[0]), (uint32_t)row_bytes,
                        lane_off, a.num_slots);
    }();

    LaneParams<E, W> p;
    load_params<E, W>(taps, tensor ? a.gamma[1] : a.gamma[0], a.heads, D, h, d0, p);
    const float inv_d = 1.0f / (float)D;
    int par = 0;

    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t tile = u / slices;
        int64_t start, end;
        const int s = tile_seq_bounds<BB>(a.cu, a.num_seqs, T, tile, start, end);
        if (end < start) end = start;
        const int64_t L = end - start;
        const int64_t j = tile - (start / BB + s);
        const int64_t ntiles = L > 0 ? (L + BB - 1) / BB : 1;
        if (j < 0 || j >= ntiles) continue;  // the same for the whole workgroup

        const int64_t t0 = start + j * BB + (int64_t)w * BT;
        const int64_t rem = end - t0;
        const int n = rem <= 0 ? 0 : (rem < BT ? (int)rem : BT);
        int32_t idx = -1;
        bool slot_ok = false, read_state = false;
        if (j == 0) {
            idx = uniform(a.state_idx ? a.state_idx[s] : s);
            slot_ok = R > 0 && state != nullptr && idx >= 0 && idx < a.num_state_slots;
            read_state = slot_ok && (a.has_init ? a.has_init[s] != 0 : true);
        }
        const bool first_span = j == 0 && w == 0;

        // Loads, all issued unconditionally and oldest first in the order of use: the span's
        // slots (lane i: token i's slot; a span with no rows reads a stand-in word), the halo
        // (the R rows before the span, for wave 0 only when the others get theirs through LDS;
        // the stored state for a sequence's first span; otherwise R stand-in rows, discarded),
        // the rows the next wave needs, then the other rows (past a short span's end the last
        // row again; a span with no rows reads the stand-in). The stand-in is the taps array, at
        // least W rows long.
        const int last = n > 0 ? n - 1 : 0;
        const int64_t* sp = n > 0 ? a.slot + t0 + (wl < last ? wl : last)
                                  : reinterpret_cast<const int64_t*>(taps);
        const int64_t slot_word = *sp;
        const int64_t lane_slot = wl < n ? slot_word : (int64_t)-1;  // -1: the store is dropped
        // with the LDS hand-off only wave 0 reads its halo rows; otherwise every wave with rows
        const bool halo_rows = kLdsHalo ? (w == 0 && j > 0) : (!first_span && n > 0);
        const char* hsrc = halo_rows ? x + (t0 - R) * stride_bytes
                           : (w == 0 && read_state) ? state + (int64_t)idx * R * row_bytes
                                                    : stand_in;
        const int64_t hstride = halo_rows ? stride_bytes : row_bytes;
        uint4 halo[R > 0 ? R : 1];
#pragma unroll
        for (int k = 0; k < R; ++k) halo[k] = ldrow_keep(hsrc + k * hstride, lane_off);
        const char* xb = n > 0 ? x + t0 * stride_bytes : stand_in;
        const int64_t rstride = n > 0 ? stride_bytes : 0;
        uint4 raw[BT];
#pragma unroll
        for (int i = BT - R; i < BT; ++i)
            raw[i] = ldrow_keep(xb + (i < last ? i : last) * rstride, lane_off);
#pragma unroll
        for (int i = 0; i < BT - R; ++i)
            raw[i] = ldrow(xb + (i < last ? i : last) * rstride, lane_off);

        if constexpr (kLdsHalo && R > 0) {
            if (w + 1 < NW) {
#pragma unroll
                for (int k = 0; k < R; ++k) handoff[par][w][k][wl] = raw[BT - R + k];
            }
            __syncthreads();
            if (w > 0) {
#pragma unroll
                for (int k = 0; k < R; ++k) halo[k] = handoff[par][w - 1][k][wl];
            }
            par ^= 1;
        }
        if (first_span && !read_state) {
#pragma unroll
            for (int k = 0; k < R; ++k) halo[k] = make_uint4(0, 0, 0, 0);
        }
        float win[W][VEC];
#pragma unroll
        for (int k = 0; k < R; ++k) E::widen(halo[k], win[k]);
        // Token i's row goes to win[(i + R) % W] (a ring). Every token is computed and its row
        // stored, tokens past the span's end (recomputing the last row) with an invalid slot,
        // so the store is dropped: no branch, and each token waits only for its own row.
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            E::widen(raw[i], win[(i + R) % W]);
            float o[VEC];
            fused_row<E, W, LPH>(win, i % W, p, a.eps, inv_d, o);
            rows.write(lane_value(lane_slot, i), rows.encode(o));
            __builtin_amdgcn_sched_barrier(0);
        }

        // The sequence's first tile writes its new state (its first wave read the old one), as in
        // prefill_kernel.
        if (R > 0 && first_span && slot_ok) {
            char* dst = state + (int64_t)idx * R * row_bytes;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int64_t e = L + i;
                uint4 r = make_uint4(0, 0, 0, 0);
                if (e >= R)
                    r = ldrow(x + (start + e - R) * stride_bytes, lane_off);
                else if (read_state)
                    r = ldrow(dst + e * row_bytes, lane_off);
                if (e != i || !read_state) strow(dst + i * row_bytes, lane_off, r);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Prefill over one-tensor slices, one run of RUN consecutive tokens of one 64-lane column slice
// per wave (no LDS, no workgroup barrier). The run is walked in sub-spans of ST tokens: the rows of
// sub-span n + 1 are loaded before sub-span n is computed, so a wave keeps loads in flight while
// it computes, at about the registers of one 8-token span. The window is carried in registers
// from one sub-span to the next; only the run's first R halo rows are loaded (from the previous
// run, the stored state, or zeros). Tiles, sequence search, state rule, stores and row math are
// those of prefill_slice_kernel, with a tile of RUN tokens per slice.
// ------------------------------------------------------------------------------------------------
#ifndef SC_RUN_TOKENS
#define SC_RUN_TOKENS 16  // tokens per run
#endif
#ifndef SC_RUN_ST
#define SC_RUN_ST 4
#endif
#ifndef SC_RUN_MIN_WAVES
#define SC_RUN_MIN_WAVES 4
#endif
constexpr int kRunWaves = 4;  // waves per workgroup (independent)

template <class E, int D, int W, int RUN, int ST, bool MX>
__global__ void __launch_bounds__(64 * kRunWaves, SC_RUN_MIN_WAVES) prefill_run_kernel(StepArgs a) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    constexpr int R = W - 1;
    constexpr int NS = RUN / ST;
    static_assert(RUN % ST == 0 && RUN <= 64 && ST >= 1 && RUN >= R, "run");
    using Rows = typename RowsFor<E, MX>::type;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wl = threadIdx.x & 63;
    const int slices = a.lane_blocks;
    const int64_t units = (int64_t)a.tiles * slices;
    const int64_t u = (int64_t)blockIdx.x * kRunWaves + w;
    if (u >= units) return;  // the whole wave
    const int slice = uniform((int32_t)(u % slices));
    const int64_t tile = u / slices;
    const int tensor = uniform(slice * 64 >= a.lanes_per_tensor ? 1 : 0);
    const int c = slice * 64 + wl - tensor * a.lanes_per_tensor;
    const int h = c / LPH;
    const int d0 = (c - h * LPH) * VEC;
    const int64_t T = a.tokens;
    const char* x = static_cast<const char*>(tensor ? a.x[1] : a.x[0]);
    const int64_t stride_bytes = (tensor ? a.x_stride[1] : a.x_stride[0]) * E::BYTES;
    char* state = static_cast<char*>(tensor ? a.state[1] : a.state[0]);
    const float* taps = tensor ? a.taps[1] : a.taps[0];
    const int64_t row_bytes = (int64_t)a.heads * D * E::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * E::BYTES);
    char* stand_in = reinterpret_cast<char*>(const_cast<float*>(taps));  // >= one row long
    const Rows rows = [&] {
        if constexpr (MX)
            return Rows(static_cast<char*>(tensor ? a.cache[1] : a.cache[0]),
                        static_cast<char*>(tensor ? a.scales[1] : a.scales[0]),
                        (uint32_t)(a.heads * D), h, d0, D, a.num_slots);
        else
            return Rows(static_cast<char*>(tensor ? a.cache[1] : a.cache[0]), (uint32_t)row_bytes,
                        lane_off, a.num_slots);
    }();

    int64_t start, end;
    const int s = tile_seq_bounds<RUN>(a.cu, a.num_seqs, T, tile, start, end);
    if (end < start) end = start;
    const int64_t L = end - start;
    const int64_t j = tile - (start / RUN + s);
    const int64_t ntiles = L > 0 ? (L + RUN - 1) / RUN : 1;
    if (j < 0 || j >= ntiles) return;  // the whole wave

    const int64_t t0 = start + j * RUN;
    const int64_t rem = end - t0;
    const int n = rem <= 0 ? 0 : (rem < RUN ? (int)rem : RUN);
    int32_t idx = -1;
    bool slot_ok = false, read_state = false;
    if (j == 0) {
        idx = uniform(a.state_idx ? a.state_idx[s] : s);
        slot_ok = R > 0 && state != nullptr && idx >= 0 && idx < a.num_state_slots;
        read_state = slot_ok && (a.has_init ? a.has_init[s] != 0 : true);
    }

    // Loads in the order of use, all unconditional: the run's slots (lane i: token i's; a run
    // with no rows reads a stand-in word), the halo (the R rows before the run, the stored state
    // for a sequence's first run, else R stand-in rows, discarded), the first sub-span's rows
    // (past the run's end the last row again; with no rows, the stand-in).
    const int last = n > 0 ? n - 1 : 0;
    const int64_t* sp = n > 0 ? a.slot + t0 + (wl < last ? wl : last)
                              : reinterpret_cast<const int64_t*>(taps);
    const int64_t slot_word = *sp;
    const int64_t lane_slot = wl < n ? slot_word : (int64_t)-1;  // -1: the store is dropped
    const char* hsrc = j > 0 ? x + (t0 - R) * stride_bytes
                       : read_state ? state + (int64_t)idx * R * row_bytes
                                    : stand_in;
    const int64_t hstride = j > 0 ? stride_bytes : row_bytes;
    uint4 halo[R > 0 ? R : 1];
#pragma unroll
    for (int k = 0; k < R; ++k) halo[k] = ldrow_keep(hsrc + k * hstride, lane_off);
    const char* xb = n > 0 ? x + t0 * stride_bytes : stand_in;
    const int64_t rstride = n > 0 ? stride_bytes : 0;
    // the run's last R rows are the next run's halo: loaded without the streaming hint
    const auto load_row = [&](int i) -> uint4 {
        const char* p = xb + (i < last ? i : last) * rstride;
        return i >= RUN - R ? ldrow_keep(p, lane_off) : ldrow(p, lane_off);
    };
    uint4 buf[2][ST];
#pragma unroll
    for (int i = 0; i < ST; ++i) buf[0][i] = load_row(i);

    LaneParams<E, W> p;
    load_params<E, W>(taps, tensor ? a.gamma[1] : a.gamma[0], a.heads, D, h, d0, p);
    const float inv_d = 1.0f / (float)D;
    if (j == 0 && !read_state) {
#pragma unroll
        for (int k = 0; k < R; ++k) halo[k] = make_uint4(0, 0, 0, 0);
    }
    float win[W][VEC];
#pragma unroll
    for (int k = 0; k < R; ++k) E::widen(halo[k], win[k]);

#pragma unroll
    for (int sub = 0; sub < NS; ++sub) {
        if (sub + 1 < NS) {
#pragma unroll
            for (int i = 0; i < ST; ++i) buf[(sub + 1) & 1][i] = load_row((sub + 1) * ST + i);
        }
        // token tk's row goes to win[(tk + R) % W]; tokens past the run's end recompute the last
        // row and their stores are dropped
#pragma unroll
        for (int i = 0; i < ST; ++i) {
            const int tk = sub * ST + i;
            E::widen(buf[sub & 1][i], win[(tk + R) % W]);
            float o[VEC];
            fused_row<E, W, LPH>(win, tk % W, p, a.eps, inv_d, o);
            rows.write(lane_value(lane_slot, tk), rows.encode(o));
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The sequence's first run writes its new state (it read the old one), as in prefill_kernel.
    if (R > 0 && j == 0 && slot_ok) {
        char* dst = state + (int64_t)idx * R * row_bytes;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t e = L + i;
            uint4 r = make_uint4(0, 0, 0, 0);
            if (e >= R)
                r = ldrow(x + (start + e - R) * stride_bytes, lane_off);
            else if (read_state)
                r = ldrow(dst + e * row_bytes, lane_off);
            if (e != i || !read_state) strow(dst + i * row_bytes, lane_off, r);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Decode: one token per sequence; window = [state rows 0..W-2, new row]; state shifts by one.
// ------------------------------------------------------------------------------------------------
template <class E, int D, int W, bool MX>
__global__ void __launch_bounds__(kBlock) decode_kernel(StepArgs a) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    constexpr int R = W - 1;
    const int64_t b = blockIdx.x;
    const int lane = blockIdx.y * kBlock + threadIdx.x;
    if (lane >= 2 * a.lanes_per_tensor) return;
    const int tensor = lane >= a.lanes_per_tensor;
    const int c = lane - tensor * a.lanes_per_tensor;
    const int h = c / LPH;
    const int d0 = (c - h * LPH) * VEC;
    const int64_t row_bytes = (int64_t)a.heads * D * E::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * E::BYTES);
    char* state = static_cast<char*>(pick(a.state, tensor));

    const int32_t idx = uniform(a.state_idx ? a.state_idx[b] : (int32_t)b);
    const bool slot_ok = R > 0 && state != nullptr && idx >= 0 && idx < a.num_state_slots;
    char* srow = state + (int64_t)idx * R * row_bytes;  // used only when slot_ok

    // Unconditional loads (a load under a branch makes the compiler wait for everything in flight
    // at the merge): a sequence without a state slot reads the taps as a stand-in for its state
    // rows (at least R rows long) and clears them afterwards.
    const char* src = slot_ok ? srow : reinterpret_cast<const char*>(pick(a.taps, tensor));
    const char* x = static_cast<const char*>(pick(a.x, tensor));
    uint4 raw[W];
#pragma unroll
    for (int k = 0; k < R; ++k) raw[k] = ldrow(src + k * row_bytes, lane_off);
    raw[R] = ldrow(x + b * pick(a.x_stride, tensor) * E::BYTES, lane_off);
    const int64_t slot = a.slot[b];

    LaneParams<E, W> p;
    load_params<E, W>(pick(a.taps, tensor), pick(a.gamma, tensor), a.heads, D, h, d0, p);
    if (!slot_ok) {
#pragma unroll
        for (int k = 0; k < R; ++k) raw[k] = make_uint4(0, 0, 0, 0);
    }
    float win[W][VEC];
#pragma unroll
    for (int k = 0; k < W; ++k) E::widen(raw[k], win[k]);
    float o[VEC];
    fused_row<E, W, LPH>(win, 0, p, a.eps, 1.0f / (float)D, o);
    const typename SinkFor<E, MX>::type sink(a, tensor, h, d0, D);
    sink.put(slot, true, o);
    if (slot_ok) {
#pragma unroll
        for (int k = 0; k < R; ++k) strow(srow + k * row_bytes, lane_off, raw[k + 1]);
    }
}

// ------------------------------------------------------------------------------------------------
// Speculative verification: each sequence runs its candidate tokens from the stored conv state,
// which it only reads; the state after every token goes to a snapshot buffer instead, so that the
// state of any accepted prefix can be installed afterwards (commit_kernel).
// ------------------------------------------------------------------------------------------------
// Tokens whose rows are loaded together per pass: about 16, a multiple of the window width.
template <int W>
constexpr int verify_chunk() { return W * (16 / W); }

template <class E, int D, int W>
__global__ void __launch_bounds__(kBlock) verify_kernel(StepArgs a, VerifyArgs va) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    constexpr int R = W - 1;
    constexpr int K = verify_chunk<W>();
    static_assert(K <= 64, "a wave loads one slot per lane");
    const int s = blockIdx.x;
    const int lane = blockIdx.y * kBlock + threadIdx.x;
    if (lane >= 2 * a.lanes_per_tensor) return;
    const int tensor = lane >= a.lanes_per_tensor;
    const int c = lane - tensor * a.lanes_per_tensor;
    const int h = c / LPH;
    const int d0 = (c - h * LPH) * VEC;
    const int64_t row_bytes = (int64_t)a.heads * D * E::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * E::BYTES);
    const char* x = static_cast<const char*>(pick(a.x, tensor));
    const int64_t stride_bytes = pick(a.x_stride, tensor) * E::BYTES;
    const PlainSink<E> sink(a, tensor, h, d0, D);
    const char* state = static_cast<const char*>(pick(a.state, tensor));
    char* snap = static_cast<char*>(pick(va.snap, tensor));

    const int64_t T = a.tokens;
    const int64_t start = uniform((int64_t)clamp_tok(a.cu[s], T));
    int64_t end = uniform((int64_t)clamp_tok(a.cu[s + 1], T));
    if (end < start) end = start;
    const int64_t L = end - start;
    const int32_t idx = uniform(a.state_idx ? a.state_idx[s] : s);
    const bool slot_ok = R > 0 && state != nullptr && idx >= 0 && idx < a.num_state_slots;

    LaneParams<E, W> p;
    load_params<E, W>(pick(a.taps, tensor), pick(a.gamma, tensor), a.heads, D, h, d0, p);
    // The window as two rings of W rows (raw, for bit-exact snapshots, and widened): token t's
    // row goes to slot (t + R) % W. A chunk is a multiple of W tokens, so every slot index is a
    // compile-time constant and advancing the window moves no registers. The stored state comes
    // in from a valid stand-in (the taps) when the sequence has no state slot, then is cleared.
    uint4 rr[W];
    float win[W][VEC];
    const char* src = slot_ok ? state + (int64_t)idx * R * row_bytes
                              : reinterpret_cast<const char*>(pick(a.taps, tensor));
#pragma unroll
    for (int k = 0; k < R; ++k) rr[k] = ldrow(src + k * row_bytes, lane_off);
    const float inv_d = 1.0f / (float)D;
    char* snap_seq = snap + (int64_t)s * va.max_tokens * R * row_bytes;
    const int wl = threadIdx.x & 63;

    for (int64_t c0 = 0; c0 < L; c0 += K) {
        // the chunk's rows (past the run's end the last row again, unused) and, in lane i, the
        // cache slot of its token i
        const int64_t last = (L - c0 < K ? L - c0 : K) - 1;
        uint4 raw[K];
#pragma unroll
        for (int i = 0; i < K; ++i)
            raw[i] = ldrow(x + (start + c0 + (i < last ? i : last)) * stride_bytes, lane_off);
        const int64_t lane_slot = a.slot[start + c0 + (wl < last ? wl : last)];
        if (c0 == 0) {  // the initial rows, the oldest loads, while this chunk's are in flight
#pragma unroll
            for (int k = 0; k < R; ++k) {
                if (!slot_ok) rr[k] = make_uint4(0, 0, 0, 0);
                E::widen(rr[k], win[k]);
            }
        }
        wait_vmem();  // the stores below then never wait for anything
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (c0 + i < L) {
                rr[(i + R) % W] = raw[i];
                E::widen(raw[i], win[(i + R) % W]);
                float o[VEC];
                fused_row<E, W, LPH>(win, i % W, p, a.eps, inv_d, o);
                sink.put(lane_value(lane_slot, i), true, o);
                if (R > 0 && snap != nullptr && c0 + i < va.max_tokens) {
                    // the state after this token: its row and the R - 1 before it, oldest first
                    char* dst = snap_seq + (c0 + i) * R * row_bytes;
#pragma unroll
                    for (int k = 0; k < R; ++k)
                        strow(dst + k * row_bytes, lane_off, rr[(i + 1 + k) % W]);
                }
            }
        }
    }
}

// Installs the snapshot of the accepted prefix: pool row state_idx[s] = snapshot (s, m - 1) with
// m = min(accepted[s], L_s, max_tokens); m == 0 leaves the row as it is.
template <class E, int D, int W>
__global__ void __launch_bounds__(kBlock) commit_kernel(StepArgs a, VerifyArgs va) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    constexpr int R = W - 1;
    const int s = blockIdx.x;
    const int lane = blockIdx.y * kBlock + threadIdx.x;
    if (R == 0 || lane >= 2 * a.lanes_per_tensor) return;
    const int tensor = lane >= a.lanes_per_tensor;
    const int c = lane - tensor * a.lanes_per_tensor;
    const int h = c / LPH;
    const int d0 = (c - h * LPH) * VEC;
    const int64_t row_bytes = (int64_t)a.heads * D * E::BYTES;
    const uint32_t lane_off = (uint32_t)(((int64_t)h * D + d0) * E::BYTES);
    char* state = static_cast<char*>(pick(a.state, tensor));
    const char* snap = static_cast<const char*>(pick(va.snap, tensor));

    const int64_t T = a.tokens;
    const int64_t start = (int64_t)clamp_tok(a.cu[s], T);
    int64_t end = (int64_t)clamp_tok(a.cu[s + 1], T);
    if (end < start) end = start;
    int64_t m = va.accepted[s];
    if (m > end - start) m = end - start;
    if (m > va.max_tokens) m = va.max_tokens;
    const int32_t idx = a.state_idx ? a.state_idx[s] : s;
    if (m < 1 || state == nullptr || snap == nullptr || idx < 0 || idx >= a.num_state_slots) return;
    const char* src = snap + ((int64_t)s * va.max_tokens + (m - 1)) * R * row_bytes;
    char* dst = state + (int64_t)idx * R * row_bytes;
    uint4 r[R > 0 ? R : 1];
#pragma unroll
    for (int k = 0; k < R; ++k) r[k] = ldrow(src + k * row_bytes, lane_off);
#pragma unroll
    for (int k = 0; k < R; ++k) strow(dst + k * row_bytes, lane_off, r[k]);
}

// ------------------------------------------------------------------------------------------------
// Standalone MXFP8 quantization of rows [rows][H][D] (e.g. to convert an existing cache), with
// exactly the quantizer the fused kernels use.
// ------------------------------------------------------------------------------------------------
template <class E, int D>
__global__ void __launch_bounds__(kBlock) mx_quantize_kernel(StepArgs a) {
    constexpr int VEC = E::VEC;
    constexpr int LPH = D / VEC;
    const int64_t r = blockIdx.x;
    const int lane = blockIdx.y * kBlock + threadIdx.x;
    if (lane >= a.lanes_per_tensor) return;
    const int h = lane / LPH;
    const int d0 = (lane - h * LPH) * VEC;
    const uint4 raw = ldrow(static_cast<const char*>(a.x[0]) + r * a.x_stride[0] * E::BYTES,
                            (uint32_t)(((int64_t)h * D + d0) * E::BYTES));
    float o[VEC];
    E::widen(raw, o);
    const MxSink<E> sink(a, 0, h, d0, D);
    sink.put(r, true, o);
}

// ------------------------------------------------------------------------------------------------
// Dispatch tables: [dtype][head_dim index][width - 1]
// ------------------------------------------------------------------------------------------------
using KernelFn = void (*)(StepArgs);

template <class E, int D, int W>
constexpr KernelFn prefill_fn() {
    return prefill_kernel<E, D, W, span_tokens<W, false>(), false, false>;
}
template <class E, int D, int W>
constexpr KernelFn prefill_mx_fn() {
    return prefill_kernel<E, D, W, span_tokens<W, true>(), true, false>;
}
#ifndef SC_SLICE_BT
#define SC_SLICE_BT 8
#endif
#ifndef SC_SLICE_BT_MX
#define SC_SLICE_BT_MX 8
#endif
#ifndef SC_SLICE_BT_WIDE
#define SC_SLICE_BT_WIDE 8
#endif
#ifndef SC_SLICE_BT_WIDE_MX
#define SC_SLICE_BT_WIDE_MX 8
#endif
// Widest window served by prefill_slice_kernel; wider ones over one-tensor slices use
// prefill_kernel's PURE form. Measured on MI355X (bf16, W = 8, 131072 tokens, 8 x 128 heads, one
// process): prefill_kernel (16-token spans held until every row is in, 2 waves per SIMD)
// 172.8 us; prefill_slice_kernel at 2 waves per SIMD with 16-token spans 179.8 us, with 8-token
// spans 223.8 us (at 3 waves per SIMD its registers spill). MXFP8 rows: 185.4 / 186.4 / 219.8 us.
#ifndef SC_SLICE_MAX_W
#define SC_SLICE_MAX_W 4
#endif
template <int W, bool MX>
constexpr int slice_span_tokens() {
    return W <= 4 ? (MX ? SC_SLICE_BT_MX : SC_SLICE_BT) : (MX ? SC_SLICE_BT_WIDE_MX : SC_SLICE_BT_WIDE);
}
// Prefill over one-tensor slices: prefill_slice_kernel up to SC_SLICE_MAX_W, then prefill_kernel
// in its PURE form.
template <class E, int D, int W>
constexpr KernelFn prefill_slice_fn() {
    if constexpr (W <= SC_SLICE_MAX_W)
        return prefill_slice_kernel<E, D, W, slice_span_tokens<W, false>(), false>;
    else return prefill_kernel<E, D, W, span_tokens<W, false>(), false, true>;
}
template <class E, int D, int W>
constexpr KernelFn prefill_slice_mx_fn() {
    if constexpr (W <= SC_SLICE_MAX_W)
        return prefill_slice_kernel<E, D, W, slice_span_tokens<W, true>(), true>;
    else return prefill_kernel<E, D, W, span_tokens<W, true>(), true, true>;
}
// MXFP8 rows over one-tensor slices in runs (large problems, see use_run_kernel)
template <class E, int D, int W>
constexpr KernelFn prefill_run_mx_fn() {
    if constexpr (W <= SC_SLICE_MAX_W)
        return prefill_run_kernel<E, D, W, SC_RUN_TOKENS, SC_RUN_ST, true>;
    else return nullptr;
}
template <class E, int D, int W>
constexpr KernelFn decode_fn() { return decode_kernel<E, D, W, false>; }
template <class E, int D, int W>
constexpr KernelFn decode_mx_fn() { return decode_kernel<E, D, W, true>; }
using VerifyFn = void (*)(StepArgs, VerifyArgs);
template <class E, int D, int W>
constexpr VerifyFn verify_fn() { return verify_kernel<E, D, W>; }
template <class E, int D, int W>
constexpr VerifyFn commit_fn() { return commit_kernel<E, D, W>; }

#define SC_ROW(KIND, E, D)                                                                   \
    { KIND##_fn<E, D, 1>(), KIND##_fn<E, D, 2>(), KIND##_fn<E, D, 3>(), KIND##_fn<E, D, 4>(), \
      KIND##_fn<E, D, 5>(), KIND##_fn<E, D, 6>(), KIND##_fn<E, D, 7>(), KIND##_fn<E, D, 8>() }
#define SC_TABLE(KIND)                                                          \
    {                                                                          \
        {SC_ROW(KIND, F32, 64), SC_ROW(KIND, F32, 128), SC_ROW(KIND, F32, 256)},    \
        {SC_ROW(KIND, BF16, 64), SC_ROW(KIND, BF16, 128), SC_ROW(KIND, BF16, 256)}, \
    }

const KernelFn kPrefill[2][3][8] = SC_TABLE(prefill);
const KernelFn kDecode[2][3][8] = SC_TABLE(decode);
const KernelFn kPrefillMx[2][3][8] = SC_TABLE(prefill_mx);
const KernelFn kPrefillSlice[2][3][8] = SC_TABLE(prefill_slice);
const KernelFn kPrefillSliceMx[2][3][8] = SC_TABLE(prefill_slice_mx);
const KernelFn kPrefillRunMx[2][3][8] = SC_TABLE(prefill_run_mx);
const KernelFn kDecodeMx[2][3][8] = SC_TABLE(decode_mx);
const KernelFn kQuantizeMx[2][3] = {
    {mx_quantize_kernel<F32, 64>, mx_quantize_kernel<F32, 128>, mx_quantize_kernel<F32, 256>},
    {mx_quantize_kernel<BF16, 64>, mx_quantize_kernel<BF16, 128>, mx_quantize_kernel<BF16, 256>},
};
const VerifyFn kVerify[2][3][8] = SC_TABLE(verify);
const VerifyFn kCommit[2][3][8] = SC_TABLE(commit);

int d_index(int D) { return D == 64 ? 0 : (D == 128 ? 1 : 2); }

// Workgroups per compute unit of a persistent prefill_slice_kernel grid; 0 = one workgroup per
// unit of work. Measured on MI355X (varlen bf16 prefill): one per unit 27.5 us; persistent grids
// of 2 / 3 / 4 workgroups per CU 30.1 / 28.6 / 28.8 us.
#ifndef SC_SLICE_WG_PER_CU
#define SC_SLICE_WG_PER_CU 0
#endif

// prefill_slice_kernel serves windows up to SC_SLICE_MAX_W over slices that each hold one tensor.
bool use_slice_kernel(int width, int64_t lanes_per_tensor) {
    return width <= SC_SLICE_MAX_W && lanes_per_tensor % 64 == 0;
}

// MXFP8 rows in runs (prefill_run_kernel) when the grid has at least SC_RUN_MIN_GRID_WAVES waves
// (4 rounds of the 4 096 wave slots MI355X has at 4 waves per SIMD): there its overlap of each
// wave's arithmetic with its next loads pays; on smaller grids the last partial round and the
// longer-lived waves cost more. Measured on MI355X (MXFP8 rows, bf16 inputs, 8 or 16 KV heads x
// 128, one process; runs of 16 tokens against prefill_slice_kernel): 64 chunks of 2 048 resumed
// tokens, 16 heads (65 536 waves) 313.6 against 351.3 us; 16 sequences of 4 096 tokens (16 384
// waves) 80.3 against 86.1 us; 16 of 2 048 (8 192 waves) 41.9 against 41.2 us; 17 060 packed
// tokens (4 265 waves) 26.4 against 24.8 us. bf16 rows were slower in runs at every size
// measured (65 536 waves: 398.0 against 368.0 us).
#ifndef SC_RUN_MIN_GRID_WAVES
#define SC_RUN_MIN_GRID_WAVES 16384
#endif
bool use_run_kernel(int width, bool mx, int64_t lanes_per_tensor, int64_t tokens) {
    if (!mx || !use_slice_kernel(width, lanes_per_tensor)) return false;
    const int64_t slices = 2 * lanes_per_tensor / 64;
    return tokens / SC_RUN_TOKENS * slices >= SC_RUN_MIN_GRID_WAVES;
}

int compute_units() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace

int prefill_tile_tokens(int width, bool mx, int64_t lanes_per_tensor, int64_t tokens) {
    if (use_run_kernel(width, mx, lanes_per_tensor, tokens)) return SC_RUN_TOKENS;
    if (use_slice_kernel(width, lanes_per_tensor)) {
        const int bt = width <= 4 ? (mx ? slice_span_tokens<1, true>() : slice_span_tokens<1, false>())
                                  : (mx ? slice_span_tokens<8, true>() : slice_span_tokens<8, false>());
        return SC_SLICE_NW * bt;
    }
    const int bt = width <= 4 ? (mx ? span_tokens<1, true>() : span_tokens<1, false>())
                              : (mx ? span_tokens<8, true>() : span_tokens<8, false>());
    return (kBlock / 64) * bt;
}

hipError_t launch_prefill(StepArgs a, int dtype, int head_dim, int width, bool mx,
                          hipStream_t stream) {
    // Units of work: (tile of 4 spans of tokens, 64-lane column slice of the K|V rows);
    // a.lane_blocks carries the number of slices. One-shot: one workgroup per unit; persistent:
    // a grid sized to the chip (a multiple of the slice count) walks the units.
    a.lane_blocks = (int32_t)((2 * (int64_t)a.lanes_per_tensor + 63) / 64);
    const int64_t units = (int64_t)a.tiles * a.lane_blocks;
    if (use_run_kernel(width, mx, a.lanes_per_tensor, a.tokens)) {  // one unit per wave
        hipLaunchKernelGGL(kPrefillRunMx[dtype][d_index(head_dim)][width - 1],
                           dim3((unsigned)((units + kRunWaves - 1) / kRunWaves)),
                           dim3(64 * kRunWaves), 0, stream, a);
        return hipGetLastError();
    }
    if (use_slice_kernel(width, a.lanes_per_tensor)) {
        int64_t grid = units;
        if (SC_SLICE_WG_PER_CU > 0) {
            int64_t cap = (int64_t)compute_units() * SC_SLICE_WG_PER_CU;
            cap = cap / a.lane_blocks * a.lane_blocks;
            if (cap < a.lane_blocks) cap = a.lane_blocks;
            grid = units < cap ? units : cap;
        }
        const KernelFn k = (mx ? kPrefillSliceMx : kPrefillSlice)[dtype][d_index(head_dim)][width - 1];
        hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kSliceBlock), 0, stream, a);
        return hipGetLastError();
    }
    // one-tensor slices (wider windows): prefill_kernel's PURE form; other shapes: the general one
    const bool pure = a.lanes_per_tensor % 64 == 0;
    const KernelFn k = (pure ? (mx ? kPrefillSliceMx : kPrefillSlice) : (mx ? kPrefillMx : kPrefill))
        [dtype][d_index(head_dim)][width - 1];
    hipLaunchKernelGGL(k, dim3((unsigned)units), dim3(kBlock), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(StepArgs a, int dtype, int head_dim, int width, bool mx,
                         hipStream_t stream) {
    const int64_t lanes = 2 * (int64_t)a.lanes_per_tensor;
    const int block = lanes >= kBlock ? kBlock : (int)((lanes + 63) / 64 * 64);
    const KernelFn k = (mx ? kDecodeMx : kDecode)[dtype][d_index(head_dim)][width - 1];
    hipLaunchKernelGGL(k, dim3((unsigned)a.tokens, (unsigned)a.lane_blocks), dim3(block), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_verify(StepArgs a, VerifyArgs va, int dtype, int head_dim, int width,
                         hipStream_t stream) {
    const int64_t lanes = 2 * (int64_t)a.lanes_per_tensor;
    const int block = lanes >= kBlock ? kBlock : (int)((lanes + 63) / 64 * 64);
    hipLaunchKernelGGL(kVerify[dtype][d_index(head_dim)][width - 1],
                       dim3((unsigned)a.num_seqs, (unsigned)a.lane_blocks), dim3(block), 0, stream,
                       a, va);
    return hipGetLastError();
}

hipError_t launch_commit(StepArgs a, VerifyArgs va, int dtype, int head_dim, int width,
                         hipStream_t stream) {
    const int64_t lanes = 2 * (int64_t)a.lanes_per_tensor;
    const int block = lanes >= kBlock ? kBlock : (int)((lanes + 63) / 64 * 64);
    hipLaunchKernelGGL(kCommit[dtype][d_index(head_dim)][width - 1],
                       dim3((unsigned)a.num_seqs, (unsigned)a.lane_blocks), dim3(block), 0, stream,
                       a, va);
    return hipGetLastError();
}

hipError_t launch_mx_quantize(StepArgs a, int dtype, int head_dim, hipStream_t stream) {
    const int64_t lanes = a.lanes_per_tensor;
    const int block = lanes >= kBlock ? kBlock : (int)((lanes + 63) / 64 * 64);
    hipLaunchKernelGGL(kQuantizeMx[dtype][d_index(head_dim)],
                       dim3((unsigned)a.tokens, (unsigned)((lanes + kBlock - 1) / kBlock)),
                       dim3(block), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sc
