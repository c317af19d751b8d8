// C ABI of the fused ShortConv K/V step: host-side validation, problem geometry and launch.
// The operation, layouts and error behaviour are specified in include/shortconv.h.
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "shortconv.h"
#include "shortconv_internal.h"

#define SC_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int element_bytes(int32_t dtype) { return dtype == SC_DTYPE_F32 ? 4 : 2; }

// Checks shared by both entry points. Returns SC_OK or an error (message set).
int check_common(const char* fn, const void* x0, const void* x1, int64_t s0, int64_t s1,
                 const float* t0, const float* t1, const float* g0, const float* g1, float eps,
                 const void* st0, const void* st1, int64_t num_state_slots, const int64_t* slot,
                 const void* c0, const void* c1, int64_t num_slots, int32_t heads, int32_t D,
                 int32_t W, int32_t dtype, int64_t tokens) {
    if (dtype != SC_DTYPE_F32 && dtype != SC_DTYPE_BF16)
        return fail(SC_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (D != 64 && D != 128 && D != 256)
        return fail(SC_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, D);
    if (W < 1 || W > 8) return fail(SC_ERR_UNSUPPORTED, "%s: width %d not in [1, 8]", fn, W);
    if (heads < 1) return fail(SC_ERR_INVALID, "%s: num_heads %d < 1", fn, heads);
    // Arrays with no elements may be null (an empty tensor's data pointer can be).
    if (tokens > 0 && (!x0 || !x1)) return fail(SC_ERR_INVALID, "%s: null K or V input", fn);
    if (tokens > 0 && !slot) return fail(SC_ERR_INVALID, "%s: null slot_mapping", fn);
    if (!t0 || !t1 || !g0 || !g1) return fail(SC_ERR_INVALID, "%s: null taps or gamma", fn);
    if (num_slots > 0 && (!c0 || !c1)) return fail(SC_ERR_INVALID, "%s: null K or V cache", fn);
    if (W > 1 && num_state_slots > 0 && (!st0 || !st1))
        return fail(SC_ERR_INVALID, "%s: null conv state with width %d > 1", fn, W);
    if (num_slots < 0) return fail(SC_ERR_INVALID, "%s: num_slots < 0", fn);
    if (num_state_slots < 0) return fail(SC_ERR_INVALID, "%s: num_state_slots < 0", fn);
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return fail(SC_ERR_INVALID, "%s: eps must be finite and >= 0", fn);
    const int64_t row = (int64_t)heads * D;
    if (row > (int64_t)1 << 20) return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    const int eb = element_bytes(dtype);
    if (s0 < row || s1 < row)
        return fail(SC_ERR_INVALID, "%s: token stride smaller than num_heads*head_dim", fn);
    if ((s0 * eb) % 16 || (s1 * eb) % 16)
        return fail(SC_ERR_INVALID, "%s: token stride must be a multiple of 16 bytes", fn);
    const void* ptrs[] = {x0, x1, t0, t1, g0, g1, c0, c1, st0, st1};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(SC_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    return SC_OK;
}

sc::StepArgs make_args(const void* k, const void* v, int64_t ks, int64_t vs, const float* kt,
                       const float* vt, const float* kg, const float* vg, float eps, void* kst,
                       void* vst, int64_t num_state_slots, const int32_t* state_idx,
                       const int64_t* slot, void* kc, void* vc, int64_t num_slots, int32_t heads,
                       int32_t D, int32_t W, int32_t dtype) {
    sc::StepArgs a = {};
    a.x[0] = k;
    a.x[1] = v;
    a.x_stride[0] = ks;
    a.x_stride[1] = vs;
    a.taps[0] = kt;
    a.taps[1] = vt;
    a.gamma[0] = kg;
    a.gamma[1] = vg;
    a.state[0] = W > 1 ? kst : nullptr;
    a.state[1] = W > 1 ? vst : nullptr;
    a.cache[0] = kc;
    a.cache[1] = vc;
    a.state_idx = state_idx;
    a.slot = slot;
    a.num_slots = num_slots;
    a.num_state_slots = W > 1 ? num_state_slots : 0;
    a.heads = heads;
    const int vec = 16 / element_bytes(dtype);
    a.lanes_per_tensor = heads * (D / vec);
    a.lane_blocks = (int32_t)((2 * (int64_t)a.lanes_per_tensor + 255) / 256);
    a.eps = eps;
    return a;
}

}  // namespace

namespace {

int prefill_impl(const char* fn, const void* k, const void* v, int64_t k_tok_stride,
                 int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t num_seqs,
                 int64_t total_tokens, const float* k_taps, const float* v_taps,
                 const float* k_gamma, const float* v_gamma, float eps, void* k_state,
                 void* v_state, int64_t num_state_slots, const int32_t* state_idx,
                 const uint8_t* has_initial_state, const int64_t* slot_mapping, void* k_cache,
                 void* v_cache, void* k_scales, void* v_scales, bool mx, int64_t num_slots,
                 int32_t num_heads, int32_t head_dim, int32_t width, int32_t dtype, void* stream) {
    g_err[0] = 0;
    int rc = check_common(fn, k, v, k_tok_stride, v_tok_stride, k_taps, v_taps, k_gamma, v_gamma,
                          eps, k_state, v_state, num_state_slots, slot_mapping, k_cache, v_cache,
                          num_slots, num_heads, head_dim, width, dtype, total_tokens);
    if (rc != SC_OK) return rc;
    if (num_seqs < 0) return fail(SC_ERR_INVALID, "%s: num_seqs < 0", fn);
    if (total_tokens < 0 || total_tokens > INT32_MAX)
        return fail(SC_ERR_INVALID, "%s: total_tokens must be in [0, 2^31)", fn);
    if (mx && num_slots > 0 && (!k_scales || !v_scales))
        return fail(SC_ERR_INVALID, "%s: null MXFP8 scale buffer", fn);
    if (num_seqs == 0) return SC_OK;  // no sequence owns any token: nothing to do
    if (!cu_seqlens) return fail(SC_ERR_INVALID, "%s: null cu_seqlens", fn);
    if (width == 1 && total_tokens == 0) return SC_OK;

    sc::StepArgs a = make_args(k, v, k_tok_stride, v_tok_stride, k_taps, v_taps, k_gamma, v_gamma,
                               eps, k_state, v_state, num_state_slots, state_idx, slot_mapping,
                               k_cache, v_cache, num_slots, num_heads, head_dim, width, dtype);
    a.scales[0] = k_scales;
    a.scales[1] = v_scales;
    a.cu = cu_seqlens;
    a.has_init = has_initial_state;
    a.tokens = total_tokens;
    a.num_seqs = num_seqs;
    const int bt = sc::prefill_tile_tokens(width, mx, a.lanes_per_tensor, total_tokens);
    const int64_t tiles = total_tokens / bt + num_seqs;  // upper bound, see kernels.hip
    if (tiles * ((2 * (int64_t)a.lanes_per_tensor + 63) / 64) > INT32_MAX)
        return fail(SC_ERR_UNSUPPORTED, "%s: problem too large for one launch", fn);
    a.tiles = (int32_t)tiles;
    hipError_t e = sc::launch_prefill(a, dtype, head_dim, width, mx, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SC_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SC_OK;
}

int decode_impl(const char* fn, const void* k_new, const void* v_new, int64_t k_tok_stride,
                int64_t v_tok_stride, int32_t batch, const float* k_taps, const float* v_taps,
                const float* k_gamma, const float* v_gamma, float eps, void* k_state,
                void* v_state, int64_t num_state_slots, const int32_t* state_idx,
                const int64_t* slot_mapping, void* k_cache, void* v_cache, void* k_scales,
                void* v_scales, bool mx, int64_t num_slots, int32_t num_heads, int32_t head_dim,
                int32_t width, int32_t dtype, void* stream) {
    g_err[0] = 0;
    int rc = check_common(fn, k_new, v_new, k_tok_stride, v_tok_stride, k_taps, v_taps, k_gamma,
                          v_gamma, eps, k_state, v_state, num_state_slots, slot_mapping, k_cache,
                          v_cache, num_slots, num_heads, head_dim, width, dtype, batch);
    if (rc != SC_OK) return rc;
    if (batch < 0) return fail(SC_ERR_INVALID, "%s: batch < 0", fn);
    if (mx && num_slots > 0 && (!k_scales || !v_scales))
        return fail(SC_ERR_INVALID, "%s: null MXFP8 scale buffer", fn);
    if (batch == 0) return SC_OK;
    sc::StepArgs a = make_args(k_new, v_new, k_tok_stride, v_tok_stride, k_taps, v_taps, k_gamma,
                               v_gamma, eps, k_state, v_state, num_state_slots, state_idx,
                               slot_mapping, k_cache, v_cache, num_slots, num_heads, head_dim,
                               width, dtype);
    a.scales[0] = k_scales;
    a.scales[1] = v_scales;
    a.tokens = batch;
    if (a.lane_blocks > 65535) return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    hipError_t e = sc::launch_decode(a, dtype, head_dim, width, mx, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SC_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SC_OK;
}

}  // namespace

SC_API int shortconv_kv_prefill(const void* k, const void* v, int64_t k_tok_stride,
                                int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t num_seqs,
                                int64_t total_tokens, const float* k_taps, const float* v_taps,
                                const float* k_gamma, const float* v_gamma, float eps,
                                void* k_state, void* v_state, int64_t num_state_slots,
                                const int32_t* state_idx, const uint8_t* has_initial_state,
                                const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                int64_t num_slots, int32_t num_heads, int32_t head_dim,
                                int32_t width, int32_t dtype, void* stream) {
    return prefill_impl("shortconv_kv_prefill", k, v, k_tok_stride, v_tok_stride, cu_seqlens,
                        num_seqs, total_tokens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                        v_state, num_state_slots, state_idx, has_initial_state, slot_mapping,
                        k_cache, v_cache, nullptr, nullptr, false, num_slots, num_heads, head_dim,
                        width, dtype, stream);
}

SC_API int shortconv_kv_prefill_mxfp8(const void* k, const void* v, int64_t k_tok_stride,
                                      int64_t v_tok_stride, const int32_t* cu_seqlens,
                                      int32_t num_seqs, int64_t total_tokens, const float* k_taps,
                                      const float* v_taps, const float* k_gamma,
                                      const float* v_gamma, float eps, void* k_state,
                                      void* v_state, int64_t num_state_slots,
                                      const int32_t* state_idx, const uint8_t* has_initial_state,
                                      const int64_t* slot_mapping, void* k_codes, void* v_codes,
                                      void* k_scales, void* v_scales, int64_t num_slots,
                                      int32_t num_heads, int32_t head_dim, int32_t width,
                                      int32_t dtype, void* stream) {
    return prefill_impl("shortconv_kv_prefill_mxfp8", k, v, k_tok_stride, v_tok_stride,
                        cu_seqlens, num_seqs, total_tokens, k_taps, v_taps, k_gamma, v_gamma, eps,
                        k_state, v_state, num_state_slots, state_idx, has_initial_state,
                        slot_mapping, k_codes, v_codes, k_scales, v_scales, true, num_slots,
                        num_heads, head_dim, width, dtype, stream);
}

SC_API int shortconv_kv_decode(const void* k_new, const void* v_new, int64_t k_tok_stride,
                               int64_t v_tok_stride, int32_t batch, const float* k_taps,
                               const float* v_taps, const float* k_gamma, const float* v_gamma,
                               float eps, void* k_state, void* v_state, int64_t num_state_slots,
                               const int32_t* state_idx, const int64_t* slot_mapping,
                               void* k_cache, void* v_cache, int64_t num_slots,
                               int32_t num_heads, int32_t head_dim, int32_t width, int32_t dtype,
                               void* stream) {
    return decode_impl("shortconv_kv_decode", k_new, v_new, k_tok_stride, v_tok_stride, batch,
                       k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state, num_state_slots,
                       state_idx, slot_mapping, k_cache, v_cache, nullptr, nullptr, false,
                       num_slots, num_heads, head_dim, width, dtype, stream);
}

SC_API int shortconv_kv_decode_mxfp8(const void* k_new, const void* v_new, int64_t k_tok_stride,
                                     int64_t v_tok_stride, int32_t batch, const float* k_taps,
                                     const float* v_taps, const float* k_gamma,
                                     const float* v_gamma, float eps, void* k_state,
                                     void* v_state, int64_t num_state_slots,
                                     const int32_t* state_idx, const int64_t* slot_mapping,
                                     void* k_codes, void* v_codes, void* k_scales, void* v_scales,
                                     int64_t num_slots, int32_t num_heads, int32_t head_dim,
                                     int32_t width, int32_t dtype, void* stream) {
    return decode_impl("shortconv_kv_decode_mxfp8", k_new, v_new, k_tok_stride, v_tok_stride,
                       batch, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                       num_state_slots, state_idx, slot_mapping, k_codes, v_codes, k_scales,
                       v_scales, true, num_slots, num_heads, head_dim, width, dtype, stream);
}

SC_API int shortconv_mxfp8_quantize(const void* x, int64_t tok_stride, int64_t rows,
                                    int32_t num_heads, int32_t head_dim, int32_t dtype,
                                    void* codes, void* scales, void* stream) {
    const char* fn = "shortconv_mxfp8_quantize";
    g_err[0] = 0;
    if (dtype != SC_DTYPE_F32 && dtype != SC_DTYPE_BF16)
        return fail(SC_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return fail(SC_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, head_dim);
    if (num_heads < 1 || (int64_t)num_heads * head_dim > (int64_t)1 << 20)
        return fail(SC_ERR_INVALID, "%s: bad num_heads %d", fn, num_heads);
    if (rows < 0 || rows > INT32_MAX) return fail(SC_ERR_INVALID, "%s: rows must be in [0, 2^31)", fn);
    if (rows == 0) return SC_OK;
    if (!x || !codes || !scales) return fail(SC_ERR_INVALID, "%s: null pointer", fn);
    const int eb = element_bytes(dtype);
    if (tok_stride < (int64_t)num_heads * head_dim || (tok_stride * eb) % 16)
        return fail(SC_ERR_INVALID, "%s: bad row stride", fn);
    if (!aligned16(x) || !aligned16(codes))
        return fail(SC_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    sc::StepArgs a = {};
    a.x[0] = x;
    a.x_stride[0] = tok_stride;
    a.cache[0] = codes;
    a.scales[0] = scales;
    a.tokens = rows;
    a.num_slots = rows;
    a.heads = num_heads;
    a.lanes_per_tensor = num_heads * (head_dim / (16 / eb));
    if ((a.lanes_per_tensor + 255) / 256 > 65535)
        return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    hipError_t e = sc::launch_mx_quantize(a, dtype, head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SC_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SC_OK;
}

SC_API int shortconv_kv_verify(const void* k, const void* v, int64_t k_tok_stride,
                               int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, const float* k_taps, const float* v_taps,
                               const float* k_gamma, const float* v_gamma, float eps,
                               const void* k_state, const void* v_state, int64_t num_state_slots,
                               const int32_t* state_idx, void* k_snap, void* v_snap,
                               int32_t max_tokens, const int64_t* slot_mapping, void* k_cache,
                               void* v_cache, int64_t num_slots, int32_t num_heads,
                               int32_t head_dim, int32_t width, int32_t dtype, void* stream) {
    const char* fn = "shortconv_kv_verify";
    g_err[0] = 0;
    int rc = check_common(fn, k, v, k_tok_stride, v_tok_stride, k_taps, v_taps, k_gamma, v_gamma,
                          eps, k_state, v_state, num_state_slots, slot_mapping, k_cache, v_cache,
                          num_slots, num_heads, head_dim, width, dtype, total_tokens);
    if (rc != SC_OK) return rc;
    if (num_seqs < 0) return fail(SC_ERR_INVALID, "%s: num_seqs < 0", fn);
    if (total_tokens < 0 || total_tokens > INT32_MAX)
        return fail(SC_ERR_INVALID, "%s: total_tokens must be in [0, 2^31)", fn);
    if (max_tokens < 1) return fail(SC_ERR_INVALID, "%s: max_tokens < 1", fn);
    if (num_seqs == 0 || total_tokens == 0) return SC_OK;  // nothing to compute or snapshot
    if (!cu_seqlens) return fail(SC_ERR_INVALID, "%s: null cu_seqlens", fn);
    if (width > 1 && (!k_snap || !v_snap))
        return fail(SC_ERR_INVALID, "%s: null snapshot buffer with width %d > 1", fn, width);
    if (!aligned16(k_snap) || !aligned16(v_snap))
        return fail(SC_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    sc::StepArgs a = make_args(k, v, k_tok_stride, v_tok_stride, k_taps, v_taps, k_gamma, v_gamma,
                               eps, const_cast<void*>(k_state), const_cast<void*>(v_state),
                               num_state_slots, state_idx, slot_mapping, k_cache, v_cache,
                               num_slots, num_heads, head_dim, width, dtype);
    a.cu = cu_seqlens;
    a.tokens = total_tokens;
    a.num_seqs = num_seqs;
    if (a.lane_blocks > 65535) return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    sc::VerifyArgs va = {};
    va.snap[0] = width > 1 ? k_snap : nullptr;
    va.snap[1] = width > 1 ? v_snap : nullptr;
    va.max_tokens = max_tokens;
    hipError_t e = sc::launch_verify(a, va, dtype, head_dim, width, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SC_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SC_OK;
}

SC_API int shortconv_state_commit(const void* k_snap, const void* v_snap, int32_t max_tokens,
                                  const int32_t* cu_seqlens, int64_t total_tokens,
                                  const int32_t* accepted, int32_t num_seqs, void* k_state,
                                  void* v_state, int64_t num_state_slots,
                                  const int32_t* state_idx, int32_t num_heads, int32_t head_dim,
                                  int32_t width, int32_t dtype, void* stream) {
    const char* fn = "shortconv_state_commit";
    g_err[0] = 0;
    if (dtype != SC_DTYPE_F32 && dtype != SC_DTYPE_BF16)
        return fail(SC_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return fail(SC_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, head_dim);
    if (width < 1 || width > 8)
        return fail(SC_ERR_UNSUPPORTED, "%s: width %d not in [1, 8]", fn, width);
    if (num_heads < 1) return fail(SC_ERR_INVALID, "%s: num_heads %d < 1", fn, num_heads);
    if (num_seqs < 0 || num_state_slots < 0 || total_tokens < 0 || total_tokens > INT32_MAX)
        return fail(SC_ERR_INVALID, "%s: negative size", fn);
    if (max_tokens < 1) return fail(SC_ERR_INVALID, "%s: max_tokens < 1", fn);
    if (width == 1 || num_seqs == 0 || num_state_slots == 0) return SC_OK;  // no state to install
    if (!k_snap || !v_snap || !k_state || !v_state || !cu_seqlens || !accepted)
        return fail(SC_ERR_INVALID, "%s: null pointer", fn);
    const void* ptrs[] = {k_snap, v_snap, k_state, v_state};
    for (const void* p : ptrs)
        if (!aligned16(p)) return fail(SC_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    if ((int64_t)num_heads * head_dim > (int64_t)1 << 20)
        return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    sc::StepArgs a = {};
    a.state[0] = k_state;
    a.state[1] = v_state;
    a.num_state_slots = num_state_slots;
    a.state_idx = state_idx;
    a.cu = cu_seqlens;
    a.tokens = total_tokens;
    a.num_seqs = num_seqs;
    a.heads = num_heads;
    a.lanes_per_tensor = num_heads * (head_dim / (16 / element_bytes(dtype)));
    a.lane_blocks = (int32_t)((2 * (int64_t)a.lanes_per_tensor + 255) / 256);
    if (a.lane_blocks > 65535) return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    sc::VerifyArgs va = {};
    va.snap[0] = const_cast<void*>(k_snap);
    va.snap[1] = const_cast<void*>(v_snap);
    va.accepted = accepted;
    va.max_tokens = max_tokens;
    hipError_t e = sc::launch_commit(a, va, dtype, head_dim, width, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SC_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SC_OK;
}

namespace {

// Shape checks of the backward (the same limits as the forward). Returns SC_OK or an error.
int check_backward_shape(const char* fn, int64_t total_tokens, int32_t num_seqs, int32_t heads,
                         int32_t D, int32_t W, int32_t dtype) {
    if (dtype != SC_DTYPE_F32 && dtype != SC_DTYPE_BF16)
        return fail(SC_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    if (D != 64 && D != 128 && D != 256)
        return fail(SC_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128, 256}", fn, D);
    if (W < 1 || W > 8) return fail(SC_ERR_UNSUPPORTED, "%s: width %d not in [1, 8]", fn, W);
    if (heads < 1) return fail(SC_ERR_INVALID, "%s: num_heads %d < 1", fn, heads);
    if ((int64_t)heads * D > (int64_t)1 << 20)
        return fail(SC_ERR_UNSUPPORTED, "%s: num_heads too large", fn);
    if (num_seqs < 0) return fail(SC_ERR_INVALID, "%s: num_seqs < 0", fn);
    if (total_tokens < 0 || total_tokens > INT32_MAX)
        return fail(SC_ERR_INVALID, "%s: total_tokens must be in [0, 2^31)", fn);
    const sc::BwdShape sh = sc::backward_shape(total_tokens, num_seqs, heads, D, W, dtype);
    if (sh.groups * sh.slices > INT32_MAX || sh.tiles > INT32_MAX)
        return fail(SC_ERR_UNSUPPORTED, "%s: problem too large for one launch", fn);
    return SC_OK;
}

}  // namespace

SC_API size_t shortconv_kv_backward_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                                   int32_t num_heads, int32_t head_dim,
                                                   int32_t width, int32_t dtype) {
    g_err[0] = 0;
    const char* fn = "shortconv_kv_backward_workspace_size";
    if (check_backward_shape(fn, total_tokens, num_seqs, num_heads, head_dim, width, dtype) !=
        SC_OK)
        return SIZE_MAX;
    return sc::backward_shape(total_tokens, num_seqs, num_heads, head_dim, width, dtype)
        .workspace_bytes;
}

namespace {

int backward_impl(
    const char* fn, const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, const float* k_taps,
    const float* v_taps, const float* k_gamma, const float* v_gamma, float eps, const void* k_state,
    const void* v_state, int64_t num_state_slots, const int32_t* state_idx,
    const uint8_t* has_initial_state, const void* dy_k, const void* dy_v, const void* dstate_out_k,
    const void* dstate_out_v, void* dk, void* dv, float* dk_taps, float* dv_taps, float* dk_gamma,
    float* dv_gamma, void* dstate_in_k, void* dstate_in_v, void* workspace,
    size_t workspace_bytes, int32_t num_heads, int32_t head_dim, int32_t width, int32_t dtype,
    void* stream) {
    int rc = check_backward_shape(fn, total_tokens, num_seqs, num_heads, head_dim, width, dtype);
    if (rc != SC_OK) return rc;
    if (!k_taps || !v_taps || !k_gamma || !v_gamma)
        return fail(SC_ERR_INVALID, "%s: null taps or gamma", fn);
    if (!dk_taps || !dv_taps || !dk_gamma || !dv_gamma)
        return fail(SC_ERR_INVALID, "%s: null taps or gamma gradient", fn);
    if (total_tokens > 0 && (!k || !v)) return fail(SC_ERR_INVALID, "%s: null K or V input", fn);
    if (total_tokens > 0 && (!dy_k || !dy_v))
        return fail(SC_ERR_INVALID, "%s: null output gradient", fn);
    if (total_tokens > 0 && (!dk || !dv)) return fail(SC_ERR_INVALID, "%s: null input gradient", fn);
    if (num_seqs > 0 && !cu_seqlens) return fail(SC_ERR_INVALID, "%s: null cu_seqlens", fn);
    if (num_state_slots < 0) return fail(SC_ERR_INVALID, "%s: num_state_slots < 0", fn);
    if (width > 1 && num_state_slots > 0 && (!k_state || !v_state))
        return fail(SC_ERR_INVALID, "%s: null conv state with width %d > 1", fn, width);
    if (!dstate_out_k != !dstate_out_v)
        return fail(SC_ERR_INVALID, "%s: new-state gradient given for one tensor only", fn);
    if (!dstate_in_k != !dstate_in_v)
        return fail(SC_ERR_INVALID, "%s: initial-state gradient requested for one tensor only", fn);
    if (!(eps >= 0.0f) || eps > 3.0e38f)
        return fail(SC_ERR_INVALID, "%s: eps must be finite and >= 0", fn);
    const int64_t row = (int64_t)num_heads * head_dim;
    const int eb = element_bytes(dtype);
    if (k_tok_stride < row || v_tok_stride < row)
        return fail(SC_ERR_INVALID, "%s: token stride smaller than num_heads*head_dim", fn);
    if ((k_tok_stride * eb) % 16 || (v_tok_stride * eb) % 16)
        return fail(SC_ERR_INVALID, "%s: token stride must be a multiple of 16 bytes", fn);
    const void* ptrs[] = {k, v, k_taps, v_taps, k_gamma, v_gamma, k_state, v_state, dy_k, dy_v,
                          dstate_out_k, dstate_out_v, dk, dv, dk_taps, dv_taps, dk_gamma,
                          dv_gamma, dstate_in_k, dstate_in_v, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(SC_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
    const sc::BwdShape sh =
        sc::backward_shape(total_tokens, num_seqs, num_heads, head_dim, width, dtype);
    if (sh.workspace_bytes > 0 && (!workspace || workspace_bytes < sh.workspace_bytes))
        return fail(SC_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", fn,
                    sh.workspace_bytes, workspace ? workspace_bytes : (size_t)0);

    sc::BwdArgs a = {};
    a.x[0] = k;
    a.x[1] = v;
    a.x_stride[0] = k_tok_stride;
    a.x_stride[1] = v_tok_stride;
    a.taps[0] = k_taps;
    a.taps[1] = v_taps;
    a.gamma[0] = k_gamma;
    a.gamma[1] = v_gamma;
    a.state[0] = width > 1 ? k_state : nullptr;
    a.state[1] = width > 1 ? v_state : nullptr;
    a.dy[0] = dy_k;
    a.dy[1] = dy_v;
    a.gs[0] = width > 1 ? dstate_out_k : nullptr;
    a.gs[1] = width > 1 ? dstate_out_v : nullptr;
    a.dx[0] = dk;
    a.dx[1] = dv;
    a.dstate[0] = width > 1 ? dstate_in_k : nullptr;
    a.dstate[1] = width > 1 ? dstate_in_v : nullptr;
    a.dtaps[0] = dk_taps;
    a.dtaps[1] = dv_taps;
    a.dgamma[0] = dk_gamma;
    a.dgamma[1] = dv_gamma;
    a.partial = static_cast<float*>(workspace);
    a.chunk = reinterpret_cast<double*>(static_cast<char*>(workspace) + sh.partial_bytes);
    a.cu = cu_seqlens;
    a.state_idx = state_idx;
    a.has_init = has_initial_state;
    a.tokens = total_tokens;
    a.num_state_slots = width > 1 ? num_state_slots : 0;
    a.num_seqs = num_seqs;
    a.heads = num_heads;
    a.lanes_per_tensor = (int32_t)sh.lanes_per_tensor;
    a.slices = (int32_t)sh.slices;
    a.tiles = (int32_t)sh.tiles;
    a.groups = num_seqs > 0 ? (int32_t)sh.groups : 0;  // no sequence: gradients of zero
    a.chunks = num_seqs > 0 ? (int32_t)sh.chunks : 0;
    a.tiles_per_group = (int32_t)sh.tiles_per_group;
    a.eps = eps;
    hipError_t e = sc::launch_backward(a, dtype, head_dim, width, (hipStream_t)stream);
    if (e != hipSuccess) return fail(SC_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return SC_OK;
}

}  // namespace

SC_API int shortconv_kv_backward(
    const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, const float* k_taps,
    const float* v_taps, const float* k_gamma, const float* v_gamma, float eps, const void* k_state,
    const void* v_state, int64_t num_state_slots, const int32_t* state_idx,
    const uint8_t* has_initial_state, const void* dy_k, const void* dy_v, const void* dstate_out_k,
    const void* dstate_out_v, void* dk, void* dv, float* dk_taps, float* dv_taps, float* dk_gamma,
    float* dv_gamma, void* dstate_in_k, void* dstate_in_v, void* workspace,
    size_t workspace_bytes, int32_t num_heads, int32_t head_dim, int32_t width, int32_t dtype,
    void* stream) {
    g_err[0] = 0;
    return backward_impl("shortconv_kv_backward", k, v, k_tok_stride, v_tok_stride, cu_seqlens,
                         num_seqs, total_tokens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state,
                         v_state, num_state_slots, state_idx, has_initial_state, dy_k, dy_v,
                         dstate_out_k, dstate_out_v, dk, dv, dk_taps, dv_taps, dk_gamma, dv_gamma,
                         dstate_in_k, dstate_in_v, workspace, workspace_bytes, num_heads, head_dim,
                         width, dtype, stream);
}

// ------------------------------------------------------------------------------------------------
// The backward for callers that cannot allocate: its workspace is a file-scope device array, one
// copy per GPU, held until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory, so its device address is looked up once per device (with that device
// current) and only that address is handed to the kernels.
// ------------------------------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[SHORTCONV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The device address of the current device's scratch array, or null with *code and the message
// set.
void* scratch_for_current_device(const char* fn, int* code) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *code = fail(SC_ERR_HIP, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        *code = fail(SC_ERR_UNSUPPORTED, "%s: device %d beyond the %d this library tracks", fn,
                     dev, kMaxDevices);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *code = fail(SC_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s",
                         fn, dev, hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

SC_API int shortconv_kv_backward_noalloc(
    const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, const float* k_taps,
    const float* v_taps, const float* k_gamma, const float* v_gamma, float eps, const void* k_state,
    const void* v_state, int64_t num_state_slots, const int32_t* state_idx,
    const uint8_t* has_initial_state, const void* dy_k, const void* dy_v, const void* dstate_out_k,
    const void* dstate_out_v, void* dk, void* dv, float* dk_taps, float* dv_taps, float* dk_gamma,
    float* dv_gamma, void* dstate_in_k, void* dstate_in_v, int32_t num_heads, int32_t head_dim,
    int32_t width, int32_t dtype, void* stream) {
    g_err[0] = 0;
    const char* fn = "shortconv_kv_backward_noalloc";
    int rc = check_backward_shape(fn, total_tokens, num_seqs, num_heads, head_dim, width, dtype);
    if (rc != SC_OK) return rc;
    const size_t need =
        sc::backward_shape(total_tokens, num_seqs, num_heads, head_dim, width, dtype)
            .workspace_bytes;
    if (need > (size_t)SHORTCONV_NOALLOC_SCRATCH_BYTES)
        return fail(SC_ERR_UNSUPPORTED,
                    "%s: this problem needs %zu bytes of workspace, more than the %zu bytes of "
                    "static scratch; use shortconv_kv_backward with a workspace",
                    fn, need, (size_t)SHORTCONV_NOALLOC_SCRATCH_BYTES);
    int code = SC_OK;
    void* ws = scratch_for_current_device(fn, &code);
    if (!ws) return code;
    return backward_impl(fn, k, v, k_tok_stride, v_tok_stride, cu_seqlens, num_seqs,
                         total_tokens, k_taps, v_taps, k_gamma, v_gamma, eps, k_state, v_state,
                         num_state_slots, state_idx, has_initial_state, dy_k, dy_v, dstate_out_k,
                         dstate_out_v, dk, dv, dk_taps, dv_taps, dk_gamma, dv_gamma, dstate_in_k,
                         dstate_in_v, ws, (size_t)SHORTCONV_NOALLOC_SCRATCH_BYTES, num_heads,
                         head_dim, width, dtype, stream);
}

SC_API const char* shortconv_last_error(void) { return g_err; }

SC_API int shortconv_abi_version(void) { return SHORTCONV_ABI_VERSION; }
