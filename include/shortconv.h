/*
 * shortconv.h -- C ABI of the fused ShortConv K/V step for AMD Instinct MI355X (gfx950).
 *
 * The step (aib.vote English news item "SGLang and Miles ... day-0 support for Inkling",
 * paragraphs 1-2: ShortConv is a causal convolution over the token dimension, and its fused
 * kernel combines the K/V convolution, a normalization and the KV-cache write), for each of K and
 * V with its own taps and gamma:
 *
 *   window    the current row and the W-1 rows before it in the same sequence (axbrief.com blog
 *             on Inkling's specifications, section on SConv and MoE); rows before the start of a
 *             sequence come from its conv state, or are zero for a fresh sequence;
 *   conv      c[h,d] = sum_{k=0}^{W-1} taps[k,h,d] * window[k][h,d]   (fp32 accumulation in
 *             order k = 0..W-1; window[W-1] is the current row, window[0] the oldest);
 *   norm      y[h,d] = c[h,d] / sqrt(mean_d c[h,:]^2 + eps) * gamma[d]  (RMSNorm over head_dim
 *             per (token, head), one gamma per tensor shared by all heads);
 *   write     cache[slot_mapping[t], h, d] = y[h,d] rounded once (to nearest even) to the element
 *             type, skipped when the slot is outside [0, num_slots);
 *   state     the sequence's conv state becomes its W-1 most recent raw rows (bit copies, oldest
 *             first), the per-request state pool of the serving engine (data-sketchers.com SGLang
 *             cookbook for Inkling-Small, section 2, memory-pool ratios).
 *
 * Conventions for every entry point:
 *  - Element type `dtype` (SC_DTYPE_F32 or SC_DTYPE_BF16) applies to K, V, the conv state and the
 *    caches alike. Taps and gamma are always fp32.
 *  - Layouts (all row-major, innermost dimension last, H = num_heads, D = head_dim):
 *      K, V          [tokens][H][D], token stride given in elements (>= H*D), rows 16-byte aligned;
 *      taps          fp32 [W][H][D] contiguous;   gamma fp32 [D];
 *      conv state    [num_state_slots][W-1][H][D] contiguous, row 0 = oldest;
 *      caches        [num_slots][H][D] contiguous (one paged-cache row per slot).
 *  - Every pointer except `stream` is a device pointer owned by the caller. The library never
 *    allocates, frees or synchronizes; it launches on `stream` (a hipStream_t, NULL = the null
 *    stream) and returns before the work is done.
 *  - Return value: SC_OK (0), or a negative SC_ERR_* code; shortconv_last_error() then describes
 *    it. Arguments are validated on the host before anything is launched. The contents of device
 *    index arrays are not read by the host; the kernels clamp them so that no invalid index is
 *    ever dereferenced (see each entry point).
 *  - Supported shapes: head_dim in {64, 128, 256}; 1 <= width <= 8; num_heads >= 1.
 *  - K/V and the cache or state must not overlap. Two calls that share a cache or state buffer
 *    must be ordered by the caller (same stream, or events).
 */
#ifndef SHORTCONV_H
#define SHORTCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SHORTCONV_ABI_VERSION 5

typedef enum {
    SC_DTYPE_F32 = 0,  /* IEEE binary32 */
    SC_DTYPE_BF16 = 1, /* bfloat16 (upper half of binary32), conversion rounds to nearest even */
} sc_dtype_t;

enum {
    SC_OK = 0,
    SC_ERR_INVALID = -1,     /* a null required pointer, a negative size, a bad stride */
    SC_ERR_UNSUPPORTED = -2, /* head_dim, width or dtype outside what the library is built for */
    SC_ERR_HIP = -3,         /* the HIP runtime refused the launch */
};

/*
 * Prefill over packed variable-length sequences.
 *
 *  k, v                [total_tokens][H][D] new projected rows of all sequences, packed in
 *                      sequence order; k_tok_stride / v_tok_stride in elements.
 *  cu_seqlens          int32 [num_seqs+1], cu_seqlens[0] = 0, non-decreasing, last = total_tokens.
 *                      Sequence s owns tokens [cu_seqlens[s], cu_seqlens[s+1]). Zero-length
 *                      sequences are allowed (their state is still rewritten, see below).
 *                      The kernel clamps every entry into [0, total_tokens].
 *  k_taps, v_taps      fp32 [W][H][D];  k_gamma, v_gamma fp32 [D];  eps >= 0 (e.g. 1e-6).
 *  k_state, v_state    [num_state_slots][W-1][H][D], read and rewritten in place. May be NULL
 *                      when width == 1 (num_state_slots is then ignored) or when
 *                      num_state_slots == 0 (no sequence has a state row: every window starts
 *                      from zeros and no state is written back).
 *  state_idx           int32 [num_seqs]: pool row of sequence s, or NULL for row s. Entries must
 *                      be distinct. An entry outside [0, num_state_slots) means the sequence has no
 *                      state row: its window starts from zeros and nothing is written back.
 *  has_initial_state   uint8 [num_seqs], or NULL for "all 1". 1 = the window before the first
 *                      token is the stored state row (a resumed sequence or chunk); 0 = zeros (a
 *                      fresh sequence). The new state is written in both cases: the last W-1 rows
 *                      of [initial window, new rows], so a sequence shorter than W-1 keeps the
 *                      newest surviving old rows ahead of its own.
 *  slot_mapping        int64 [total_tokens]: cache row of each token; a value outside
 *                      [0, num_slots) (e.g. -1 for padding) means the row is not written.
 *                      Non-negative entries must be distinct.
 *  k_cache, v_cache    [num_slots][H][D] written at the mapped rows only.
 *
 * total_tokens == 0 with num_seqs == 0 returns SC_OK without launching.
 */
int shortconv_kv_prefill(const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
                         const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         const float* k_taps, const float* v_taps, const float* k_gamma,
                         const float* v_gamma, float eps, void* k_state, void* v_state,
                         int64_t num_state_slots, const int32_t* state_idx,
                         const uint8_t* has_initial_state, const int64_t* slot_mapping,
                         void* k_cache, void* v_cache, int64_t num_slots, int32_t num_heads,
                         int32_t head_dim, int32_t width, int32_t dtype, void* stream);

/*
 * Decode: one new token for each of `batch` sequences, each resuming from its conv state.
 *
 *  k_new, v_new        [batch][H][D] (token strides in elements).
 *  k_state, v_state    [num_state_slots][W-1][H][D]; sequence b reads rows 0..W-2 of
 *                      pool row state_idx[b] as the past of its window and then shifts the pool
 *                      row by one (rows 1..W-2 move up, the new raw row goes last). May be NULL
 *                      when width == 1 or num_state_slots == 0 (zeros as the past, no write-back).
 *  state_idx           int32 [batch], or NULL for row b. Distinct. Out-of-pool entries: zeros as
 *                      the past, no write-back.
 *  slot_mapping        int64 [batch]: cache row of each new token (outside [0, num_slots) = skip).
 *
 * The result is bit-identical to shortconv_kv_prefill called with one token per sequence and
 * has_initial_state = 1. batch == 0 returns SC_OK without launching.
 */
int shortconv_kv_decode(const void* k_new, const void* v_new, int64_t k_tok_stride,
                        int64_t v_tok_stride, int32_t batch, const float* k_taps,
                        const float* v_taps, const float* k_gamma, const float* v_gamma, float eps,
                        void* k_state, void* v_state, int64_t num_state_slots,
                        const int32_t* state_idx, const int64_t* slot_mapping, void* k_cache,
                        void* v_cache, int64_t num_slots, int32_t num_heads, int32_t head_dim,
                        int32_t width, int32_t dtype, void* stream);

/*
 * MXFP8 cache rows. The serving cookbook's long-context recipe stores KV entries as block-scaled
 * MXFP8 instead of BF16, about doubling the tokens the pools hold (data-sketchers.com SGLang
 * cookbook for Inkling-Small, section 3.6). The page names the format only; the layout here is
 * the OCP Microscaling (MX) v1.0 one:
 *   - each (token, head) row of D elements is split into D/32 blocks of 32 consecutive elements;
 *   - a block has one E8M0 scale 2^e, e = floor(log2(max |y|)) - 8 clamped to [-127, 127]
 *     (an all-zero block gets e = -127), stored as the byte e + 127;
 *   - each element is stored as the OCP FP8 E4M3 code of y * 2^-e (bias 7, no infinity, largest
 *     finite 448): nearest value, ties to even, saturating at +-448.
 * Only the cache changes: the conv state stays in the I/O element type, so resuming a sequence is
 * exact. y is the same fp32 value the plain entry points round to bf16/fp32.
 *
 *  k_codes, v_codes    [num_slots][H][D] bytes (16-byte aligned), written at the mapped rows.
 *  k_scales, v_scales  [num_slots][H][D/32] bytes, written at the mapped rows.
 * All other arguments are those of shortconv_kv_prefill / shortconv_kv_decode.
 */
int shortconv_kv_prefill_mxfp8(const void* k, const void* v, int64_t k_tok_stride,
                               int64_t v_tok_stride, const int32_t* cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, const float* k_taps, const float* v_taps,
                               const float* k_gamma, const float* v_gamma, float eps,
                               void* k_state, void* v_state, int64_t num_state_slots,
                               const int32_t* state_idx, const uint8_t* has_initial_state,
                               const int64_t* slot_mapping, void* k_codes, void* v_codes,
                               void* k_scales, void* v_scales, int64_t num_slots,
                               int32_t num_heads, int32_t head_dim, int32_t width, int32_t dtype,
                               void* stream);

int shortconv_kv_decode_mxfp8(const void* k_new, const void* v_new, int64_t k_tok_stride,
                              int64_t v_tok_stride, int32_t batch, const float* k_taps,
                              const float* v_taps, const float* k_gamma, const float* v_gamma,
                              float eps, void* k_state, void* v_state, int64_t num_state_slots,
                              const int32_t* state_idx, const int64_t* slot_mapping,
                              void* k_codes, void* v_codes, void* k_scales, void* v_scales,
                              int64_t num_slots, int32_t num_heads, int32_t head_dim,
                              int32_t width, int32_t dtype, void* stream);

/*
 * The same MXFP8 quantizer on its own: rows x [rows][H][D] (element type `dtype`, row stride
 * tok_stride elements) -> codes [rows][H][D] and scales [rows][H][D/32] bytes. For converting
 * existing cache rows; it applies exactly the rounding the fused entry points apply.
 */
int shortconv_mxfp8_quantize(const void* x, int64_t tok_stride, int64_t rows, int32_t num_heads,
                             int32_t head_dim, int32_t dtype, void* codes, void* scales,
                             void* stream);

/*
 * Speculative verification. Serving engines verify the candidate tokens of a draft model or of
 * multi-token-prediction heads in one forward pass (aib.vote English news item on SGLang/Miles
 * Inkling support, paragraph 3; data-sketchers.com SGLang cookbook for Inkling-Small, section 2
 * on MTP and section 3.7 on DSpark). For the conv state this means: run each sequence's
 * candidates from its stored state, but install the state of only the prefix that the verifier
 * accepts, which is known after the call.
 *
 * shortconv_kv_verify: as shortconv_kv_prefill with has_initial_state = 1 for every sequence
 * (the same cache rows, bit for bit), except that the state pools are only READ. The state after
 * each token goes to the snapshot buffers instead:
 *  k_snap, v_snap   [num_seqs][max_tokens][W-1][H][D], element type `dtype`: snapshot (s, i) is
 *                   the conv state after the first i+1 tokens of sequence s (bit copies of raw
 *                   rows, oldest first), written for i < min(L_s, max_tokens); other entries are
 *                   not written. May be NULL when width == 1.
 *  max_tokens       >= 1, the snapshot capacity per sequence (the longest candidate run).
 * Sequences are processed in passes of about 16 tokens (a multiple of the width); candidate runs
 * are meant to be short.
 */
int shortconv_kv_verify(const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
                        const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const float* k_taps, const float* v_taps, const float* k_gamma,
                        const float* v_gamma, float eps, const void* k_state, const void* v_state,
                        int64_t num_state_slots, const int32_t* state_idx, void* k_snap,
                        void* v_snap, int32_t max_tokens, const int64_t* slot_mapping,
                        void* k_cache, void* v_cache, int64_t num_slots, int32_t num_heads,
                        int32_t head_dim, int32_t width, int32_t dtype, void* stream);

/*
 * shortconv_state_commit: installs the accepted prefix. For sequence s, m = min(accepted[s], L_s,
 * max_tokens) with L_s = cu_seqlens[s+1] - cu_seqlens[s] (cu_seqlens and total_tokens as given to
 * shortconv_kv_verify); if m >= 1 and state_idx[s] (or s when state_idx is NULL) is inside the
 * pool, that pool row becomes snapshot (s, m-1), bit for bit. m == 0 leaves the row unchanged.
 * accepted: device int32 [num_seqs]. A no-op when width == 1.
 */
int shortconv_state_commit(const void* k_snap, const void* v_snap, int32_t max_tokens,
                           const int32_t* cu_seqlens, int64_t total_tokens,
                           const int32_t* accepted, int32_t num_seqs, void* k_state,
                           void* v_state, int64_t num_state_slots, const int32_t* state_idx,
                           int32_t num_heads, int32_t head_dim, int32_t width, int32_t dtype,
                           void* stream);

/*
 * shortconv_kv_backward: the gradients of the prefill step, for training (the English news item's
 * paragraph 3: the RL trainer runs the model with train/infer-consistent kernels). Training reads
 * the step's output y = the rows shortconv_kv_prefill writes (slot_mapping = identity), so this
 * takes the gradient of a loss with respect to y and returns the gradients with respect to every
 * input of the step, by the chain rule through the definition at the top of this file:
 *
 *   chat = c / r, dchat = dy * gamma, proj = (1/D) sum_d dchat * chat, dc = (dchat - chat*proj) / r
 *   d_gamma[d]    = sum over tokens and heads of dy * chat
 *   d_taps[k,h,d] = sum over tokens p of dc[p] * window_p[k]
 *   d_input row   = sum_k taps[k] * dc[of the token whose window holds that row at position k]
 *                   (+ the new-state gradient, for the rows that become the new state)
 *
 * Inputs (as for shortconv_kv_prefill; the state pools are only read):
 *  k, v, k/v_tok_stride, cu_seqlens, num_seqs, total_tokens, taps, gamma, eps, k/v_state,
 *  num_state_slots, state_idx, has_initial_state
 *                   the forward call's arguments: the initial windows are the ones that call used
 *                   (so the state pools must hold the state from before that call).
 *  dy_k, dy_v       [total_tokens][H][D] contiguous, element type `dtype`: dLoss/dy.
 *  dstate_out_k/v   [num_seqs][W-1][H][D] contiguous, element type `dtype`: dLoss/d(new conv
 *                   state of sequence s), for chunked training where the state feeds the next
 *                   chunk; both NULL = no loss on the new state.
 * Outputs (overwritten):
 *  dk, dv           [total_tokens][H][D] contiguous, element type `dtype` (rounded once).
 *  dk/dv_taps       fp32 [W][H][D];   dk/dv_gamma fp32 [D].
 *  dstate_in_k/v    [num_seqs][W-1][H][D] contiguous, element type `dtype`: dLoss/d(initial
 *                   window rows) of each sequence; zero for a sequence that started from zeros
 *                   (has_initial_state = 0 or no state slot). Both NULL = not computed.
 *                   Indexed by sequence, not by pool row; add into the pool's gradient as needed.
 * Workspace: `workspace_bytes` >= shortconv_kv_backward_workspace_size(...) bytes of device
 *  memory (16-byte aligned), scratch for the parameter-gradient partials; its contents on entry
 *  do not matter and on exit are unspecified. Calls that share a workspace must be ordered.
 * Numerics: fp32 arithmetic (the forward's c and r are recomputed the same way). d_taps and
 *  d_gamma are deterministic: each workgroup sums at most 4 tiles of at most 64 tokens per lane
 *  in fp32, its 4 waves in order, and two further kernels add the workgroup partials in fp64 in
 *  a fixed order (chunks of 64 partials, then the chunks, and for d_gamma the heads), rounding
 *  once to fp32.
 * With num_seqs == 0 the parameter gradients are zero and nothing else is written.
 */
int shortconv_kv_backward(const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
                          const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                          const float* k_taps, const float* v_taps, const float* k_gamma,
                          const float* v_gamma, float eps, const void* k_state,
                          const void* v_state, int64_t num_state_slots, const int32_t* state_idx,
                          const uint8_t* has_initial_state, const void* dy_k, const void* dy_v,
                          const void* dstate_out_k, const void* dstate_out_v, void* dk, void* dv,
                          float* dk_taps, float* dv_taps, float* dk_gamma, float* dv_gamma,
                          void* dstate_in_k, void* dstate_in_v, void* workspace,
                          size_t workspace_bytes, int32_t num_heads, int32_t head_dim,
                          int32_t width, int32_t dtype, void* stream);

/*
 * Bytes of workspace shortconv_kv_backward needs for these sizes (a host-side computation, no
 * device access). SIZE_MAX when the sizes are invalid (shortconv_last_error() says why).
 */
size_t shortconv_kv_backward_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                            int32_t num_heads, int32_t head_dim, int32_t width,
                                            int32_t dtype);

/*
 * shortconv_kv_backward_noalloc: shortconv_kv_backward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc). It takes the same arguments except the workspace, and allocates nothing: its
 * workspace is a static device array of SHORTCONV_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (its address is looked up on the first call on each
 * device). Results are bit-identical to shortconv_kv_backward's.
 *  - A problem whose workspace (shortconv_kv_backward_workspace_size) exceeds
 *    SHORTCONV_NOALLOC_SCRATCH_BYTES is rejected with SC_ERR_UNSUPPORTED before anything is
 *    launched.
 *  - Every call on one GPU uses that GPU's one array: two calls that may overlap on the same GPU
 *    (different streams, no ordering) race on it and give undefined results. Order them.
 */
#define SHORTCONV_NOALLOC_SCRATCH_BYTES (16u << 20)

int shortconv_kv_backward_noalloc(
    const void* k, const void* v, int64_t k_tok_stride, int64_t v_tok_stride,
    const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens, const float* k_taps,
    const float* v_taps, const float* k_gamma, const float* v_gamma, float eps, const void* k_state,
    const void* v_state, int64_t num_state_slots, const int32_t* state_idx,
    const uint8_t* has_initial_state, const void* dy_k, const void* dy_v, const void* dstate_out_k,
    const void* dstate_out_v, void* dk, void* dv, float* dk_taps, float* dv_taps, float* dk_gamma,
    float* dv_gamma, void* dstate_in_k, void* dstate_in_v, int32_t num_heads, int32_t head_dim,
    int32_t width, int32_t dtype, void* stream);

/* Message for the last non-zero return on the calling thread ("" if none). Valid until the next
 * call on the same thread. */
const char* shortconv_last_error(void);

/* SHORTCONV_ABI_VERSION of the built library. */
int shortconv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SHORTCONV_H */
