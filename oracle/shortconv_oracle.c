/*
 * shortconv_oracle.c -- plain, slow, fp64 CPU statement of the fused ShortConv K/V step.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the bench's CPU-baseline leg are
 * the only callers. Nothing in the HIP library links, includes or calls this file, and this file
 * includes nothing of the HIP library. Its results are what the GPU path is judged against.
 *
 * What the step is, from the pages:
 *  - ShortConv is a causal convolution over the token dimension, applied to the projected K and V,
 *    fused with a normalization and the KV-cache write (aib.vote English news item "SGLang and
 *    Miles ... day-0 support for Inkling", paragraphs 1 and 2).
 *  - The short 1-D convolution reads the current token and the W-1 previous rows, W being the
 *    window width (axbrief.com blog on Inkling's specifications, section on SConv, MoE and the
 *    per-modality embedding towers).
 *  - The convolution keeps a per-request state in a pool next to the SWA pool (data-sketchers.com
 *    SGLang cookbook for Inkling-Small, section 2 "configuration tips", memory-pool ratios).
 *
 * Readings taken where the pages are silent (each is listed with its reason in the design notes):
 *  - depthwise taps, one per (tap k, head h, channel d), separate for K and V; tap W-1 multiplies
 *    the current token and tap 0 the row W-1 tokens back (cross-correlation, no flip);
 *  - no bias, no activation, no residual;
 *  - normalization = RMSNorm over head_dim per (token, head), eps inside the square root, one
 *    learned gamma[d] per tensor shared by all heads;
 *  - the conv state holds the W-1 most recent raw (pre-convolution) rows, oldest first;
 *  - the output goes to cache[slot_mapping[t]]; a slot outside [0, num_slots) is not written.
 *
 * Definition computed here, for one tensor X (K or V) and one sequence s of length L:
 *   z[i]      = initial window row i (0 <= i < W-1): the stored state row if the sequence has an
 *               initial state, else 0;
 *   e[i]      = z[i] for i < W-1, and x[cu[s] + i - (W-1)] for W-1 <= i < W-1+L;
 *   c[p,h,d]  = sum_{k=0}^{W-1} taps[k,h,d] * e[p+k,h,d]           for 0 <= p < L;
 *   r[p,h]    = sqrt( (1/D) * sum_d c[p,h,d]^2 + eps );
 *   y[p,h,d]  = c[p,h,d] / r[p,h] * gamma[d];
 *   new state = e[L .. L+W-2], copied bit for bit in the stored element type.
 * Decode is the same step for one token whose window is [state rows 0..W-2, x_new]; it is written
 * out separately below in its own (shift-register) form so that the two can be checked against
 * each other.
 *
 * Every input element is widened exactly to double (bf16 is the upper half of an IEEE binary32).
 * There is no blocking, fusion or reordering beyond the definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

static size_t elem_bytes(int dtype) { return dtype == ORC_F32 ? 4u : 2u; }

/* Exact widening of stored element number idx to double. */
static double widen(const void* base, int64_t idx, int dtype)
{
    float f;
    if (dtype == ORC_F32) {
        f = ((const float*)base)[idx];
    } else {
        uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
        memcpy(&f, &bits, sizeof f);
    }
    return (double)f;
}

/* Copy stored element src[si] to dst[di] bit for bit. */
static void copy_elem(void* dst, int64_t di, const void* src, int64_t si, int dtype)
{
    size_t b = elem_bytes(dtype);
    memcpy((char*)dst + (size_t)di * b, (const char*)src + (size_t)si * b, b);
}

static void zero_elem(void* dst, int64_t di, int dtype)
{
    size_t b = elem_bytes(dtype);
    memset((char*)dst + (size_t)di * b, 0, b);
}

/*
 * Prefill over packed variable-length sequences, one tensor.
 *
 *  x          stored [T][H][D], token stride x_stride elements (x_stride >= H*D)
 *  cu         int64 [n_seq+1], cu[0] = 0, non-decreasing
 *  taps       fp32 [W][H][D];   gamma fp32 [D];   eps >= 0 (fp32, widened)
 *  state      stored [n_state][W-1][H][D] or NULL when W == 1
 *  state_idx  int64 [n_seq]: pool row of sequence s; outside [0, n_state) means "no state slot"
 *  has_init   uint8 [n_seq]: 1 = the initial window is the stored state row, 0 = zeros
 *  y          out fp64 [T][H][D] (token order, contiguous)
 *  cond       out fp64 [T][H][D] or NULL: |gamma[d]| * sum_k |taps[k,h,d] * e[p+k,h,d]| / r[p,h],
 *             the scale of the rounding error a dot product of this shape can carry
 *  new_state  out stored [n_seq][W-1][H][D] or NULL (only meaningful when W > 1)
 *
 * Returns 0, or -1 on bad sizes.
 */
int sc_oracle_prefill(int dtype, int64_t H, int64_t D, int64_t W, int64_t n_seq, const int64_t* cu,
                      const void* x, int64_t x_stride, const float* taps, const float* gamma,
                      float eps, const void* state, int64_t n_state, const int64_t* state_idx,
                      const uint8_t* has_init, double* y, double* cond, void* new_state,
                      int nthreads)
{
    if (H <= 0 || D <= 0 || W <= 0 || n_seq < 0 || x_stride < H * D) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    const int64_t R = W - 1; /* rows of state */
    const int64_t units = n_seq * H;
    (void)nthreads;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t s = u / H, h = u % H;
        const int64_t start = cu[s], L = cu[s + 1] - cu[s];
        const int64_t idx = state_idx[s];
        const int slot_ok = state != NULL && idx >= 0 && idx < n_state;
        const int read_state = slot_ok && has_init[s];
        double* c = (double*)malloc((size_t)D * sizeof(double));
        double* a = (double*)malloc((size_t)D * sizeof(double));

        for (int64_t p = 0; p < L; ++p) {
            double ss = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    const int64_t i = p + k; /* index into e */
                    double e;
                    if (i < R)
                        e = read_state ? widen(state, ((idx * R + i) * H + h) * D + d, dtype) : 0.0;
                    else
                        e = widen(x, (start + i - R) * x_stride + h * D + d, dtype);
                    const double w = (double)taps[(k * H + h) * D + d];
                    acc += w * e;
                    mag += fabs(w * e);
                }
                c[d] = acc;
                a[d] = mag;
                ss += acc * acc;
            }
            const double r = sqrt(ss / (double)D + (double)eps);
            for (int64_t d = 0; d < D; ++d) {
                const int64_t o = ((start + p) * H + h) * D + d;
                y[o] = c[d] / r * (double)gamma[d];
                if (cond) cond[o] = fabs((double)gamma[d]) * a[d] / r;
            }
        }

        if (new_state && R > 0) {
            for (int64_t j = 0; j < R; ++j) {
                const int64_t i = L + j; /* row of e that becomes state row j */
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t o = ((s * R + j) * H + h) * D + d;
                    if (i < R) {
                        if (read_state)
                            copy_elem(new_state, o, state, ((idx * R + i) * H + h) * D + d, dtype);
                        else
                            zero_elem(new_state, o, dtype);
                    } else {
                        copy_elem(new_state, o, x, (start + i - R) * x_stride + h * D + d, dtype);
                    }
                }
            }
        }
        free(c);
        free(a);
    }
    return 0;
}

/*
 * Decode: one new token per sequence, written as a shift register.
 *
 *  x_new      stored [B][H][D], token stride x_stride
 *  state      stored [n_state][W-1][H][D] or NULL when W == 1 (row 0 = oldest)
 *  state_idx  int64 [B]; outside [0, n_state) means the window's past rows are zero and no state
 *             row is written
 *  y, cond    out fp64 [B][H][D] (cond may be NULL)
 *  new_state  out stored [B][W-1][H][D] or NULL: rows 1..W-2 of the old state, then x_new
 */
int sc_oracle_decode(int dtype, int64_t H, int64_t D, int64_t W, int64_t B, const void* x_new,
                     int64_t x_stride, const float* taps, const float* gamma, float eps,
                     const void* state, int64_t n_state, const int64_t* state_idx, double* y,
                     double* cond, void* new_state, int nthreads)
{
    if (H <= 0 || D <= 0 || W <= 0 || B < 0 || x_stride < H * D) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    const int64_t R = W - 1;
    const int64_t units = B * H;
    (void)nthreads;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H, h = u % H;
        const int64_t idx = state_idx[b];
        const int slot_ok = state != NULL && idx >= 0 && idx < n_state;
        double* c = (double*)malloc((size_t)D * sizeof(double));
        double* a = (double*)malloc((size_t)D * sizeof(double));
        double ss = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0, mag = 0.0;
            /* past rows: the W-1 state rows, oldest first, meet taps 0..W-2 */
            for (int64_t k = 0; k < R; ++k) {
                const double e = slot_ok ? widen(state, ((idx * R + k) * H + h) * D + d, dtype) : 0.0;
                const double w = (double)taps[(k * H + h) * D + d];
                acc += w * e;
                mag += fabs(w * e);
            }
            /* the new token meets the last tap */
            {
                const double e = widen(x_new, b * x_stride + h * D + d, dtype);
                const double w = (double)taps[(R * H + h) * D + d];
                acc += w * e;
                mag += fabs(w * e);
            }
            c[d] = acc;
            a[d] = mag;
            ss += acc * acc;
        }
        const double r = sqrt(ss / (double)D + (double)eps);
        for (int64_t d = 0; d < D; ++d) {
            const int64_t o = (b * H + h) * D + d;
            y[o] = c[d] / r * (double)gamma[d];
            if (cond) cond[o] = fabs((double)gamma[d]) * a[d] / r;
        }
        if (new_state && R > 0 && slot_ok) {
            for (int64_t j = 0; j < R; ++j) {
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t o = ((b * R + j) * H + h) * D + d;
                    if (j + 1 < R)
                        copy_elem(new_state, o, state, ((idx * R + j + 1) * H + h) * D + d, dtype);
                    else
                        copy_elem(new_state, o, x_new, b * x_stride + h * D + d, dtype);
                }
            }
        }
        free(c);
        free(a);
    }
    return 0;
}

/*
 * Backward of the prefill step, one tensor: the gradients of a loss through the definition at the
 * top of this file, for training (the news item's paragraph 3: the RL trainer runs the same model
 * with train/infer-consistent kernels). Nothing on the pages states it; it is the chain rule
 * applied to that definition, step by step:
 *   chat[p,h,d]  = c[p,h,d] / r[p,h]
 *   dchat        = g[p,h,d] * gamma[d]                            (g = dLoss/dy)
 *   dgamma[d]   += g[p,h,d] * chat[p,h,d]                         (over every token and head)
 *   dc[p,h,d]    = (dchat - chat * (1/D) sum_j dchat[j] chat[j]) / r[p,h]
 *   dtaps[k,h,d] += dc[p,h,d] * e[p+k,h,d]                        (over every sequence and token)
 *   de[i,h,d]    = sum_{k : 0 <= i-k < L} taps[k,h,d] * dc[i-k,h,d]
 *                  + gs[i-L,h,d] when L <= i < L+W-1               (gs = dLoss/d(new state))
 *   dx[cu[s]+t]  = de[t+W-1]
 *   dstate[s,i]  = de[i] for i < W-1 when the window came from the stored state, else 0
 *
 *  x, cu, taps, gamma, eps, state, n_state, state_idx, has_init   as for sc_oracle_prefill
 *  g          fp64 [T][H][D]
 *  gs         fp64 [n_seq][W-1][H][D] or NULL (no loss on the new state)
 *  dx         out fp64 [T][H][D]
 *  dtaps      out fp64 [W][H][D];   dgamma out fp64 [D]
 *  dstate     out fp64 [n_seq][W-1][H][D] or NULL
 *  cond_*     out fp64, shaped like dx / dtaps / dgamma / dstate, or NULL: the scale of the
 *             rounding error an fp32 evaluation of these formulas can carry (first order): per
 *             token, with A[d] = sum_k |taps[k] e[p+k]| (which bounds the error of c),
 *               M[p,d] = (|dchat| + (A/r) |proj| + |chat| (P1 + P2)) / r,
 *               P1 = (1/D) sum_j |dchat_j chat_j|,  P2 = (1/D) sum_j |dchat_j| A_j / r;
 *             cond_dx = sum_k |taps[k]| M[i-k] (+ |gs|), cond_dtaps = sum_p (M + |dc|) |e[p+k]|,
 *             cond_dgamma = sum |g| (|chat| + A/r).
 *
 * The sums over sequences (dtaps) and over sequences and heads (dgamma) are taken per
 * (sequence, head) unit first and then added in unit order, so the result does not depend on the
 * thread count. Returns 0, or -1 on bad sizes.
 */
int sc_oracle_backward(int dtype, int64_t H, int64_t D, int64_t W, int64_t n_seq,
                       const int64_t* cu, const void* x, int64_t x_stride, const float* taps,
                       const float* gamma, float eps, const void* state, int64_t n_state,
                       const int64_t* state_idx, const uint8_t* has_init, const double* g,
                       const double* gs, double* dx, double* dtaps, double* dgamma,
                       double* dstate, double* cond_dx, double* cond_dtaps, double* cond_dgamma,
                       double* cond_dstate, int nthreads)
{
    if (H <= 0 || D <= 0 || W <= 0 || n_seq < 0 || x_stride < H * D) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    const int64_t R = W - 1;
    const int64_t units = n_seq * H;
    double* part_taps = (double*)calloc((size_t)(units > 0 ? units : 1) * W * D, sizeof(double));
    double* part_gamma = (double*)calloc((size_t)(units > 0 ? units : 1) * D, sizeof(double));
    double* part_ctaps = (double*)calloc((size_t)(units > 0 ? units : 1) * W * D, sizeof(double));
    double* part_cgamma = (double*)calloc((size_t)(units > 0 ? units : 1) * D, sizeof(double));
    (void)nthreads;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t s = u / H, h = u % H;
        const int64_t start = cu[s], L = cu[s + 1] - cu[s];
        const int64_t idx = state_idx[s];
        const int from_state = state != NULL && idx >= 0 && idx < n_state && has_init[s];
        const int64_t E = R + L; /* rows of e */
        double* e = (double*)malloc((size_t)(E > 0 ? E : 1) * D * sizeof(double));
        double* dc = (double*)malloc((size_t)(L > 0 ? L : 1) * D * sizeof(double));
        double* mg = (double*)malloc((size_t)(L > 0 ? L : 1) * D * sizeof(double));
        double* c = (double*)malloc((size_t)D * sizeof(double));
        double* av = (double*)malloc((size_t)D * sizeof(double));
        double* pt = part_taps + u * W * D;
        double* pg = part_gamma + u * D;
        double* pct = part_ctaps + u * W * D;
        double* pcg = part_cgamma + u * D;

        /* the window rows e[0 .. R+L) of this sequence and head */
        for (int64_t i = 0; i < E; ++i)
            for (int64_t d = 0; d < D; ++d)
                e[i * D + d] = i < R ? (from_state ? widen(state, ((idx * R + i) * H + h) * D + d,
                                                           dtype)
                                                   : 0.0)
                                     : widen(x, (start + i - R) * x_stride + h * D + d, dtype);

        for (int64_t p = 0; p < L; ++p) {
            /* forward quantities of token p */
            double sumsq = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0, mag = 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    acc += (double)taps[(k * H + h) * D + d] * e[(p + k) * D + d];
                    mag += fabs((double)taps[(k * H + h) * D + d] * e[(p + k) * D + d]);
                }
                c[d] = acc;
                av[d] = mag;
                sumsq += acc * acc;
            }
            const double rp = sqrt(sumsq / (double)D + (double)eps);
            /* through the norm and gamma */
            double proj = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                const double gd = g[((start + p) * H + h) * D + d];
                const double chat = c[d] / rp;
                pg[d] += gd * chat;
                proj += gd * (double)gamma[d] * chat;
            }
            proj /= (double)D;
            for (int64_t d = 0; d < D; ++d) {
                const double gd = g[((start + p) * H + h) * D + d];
                const double chat = c[d] / rp;
                dc[p * D + d] = (gd * (double)gamma[d] - chat * proj) / rp;
            }
            /* through the convolution: the taps */
            for (int64_t k = 0; k < W; ++k)
                for (int64_t d = 0; d < D; ++d)
                    pt[k * D + d] += dc[p * D + d] * e[(p + k) * D + d];
            /* error scales (first-order model of an fp32 evaluation) */
            double p1 = 0.0, p2 = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                const double dch = fabs(g[((start + p) * H + h) * D + d] * (double)gamma[d]);
                p1 += dch * fabs(c[d] / rp);
                p2 += dch * av[d] / rp;
            }
            p1 /= (double)D;
            p2 /= (double)D;
            for (int64_t d = 0; d < D; ++d) {
                const double gd = g[((start + p) * H + h) * D + d];
                const double chat = fabs(c[d] / rp);
                mg[p * D + d] = (fabs(gd * (double)gamma[d]) + av[d] / rp * fabs(proj) +
                                 chat * (p1 + p2)) / rp;
                pcg[d] += fabs(gd) * (chat + av[d] / rp);
                for (int64_t k = 0; k < W; ++k)
                    pct[k * D + d] += (mg[p * D + d] + fabs(dc[p * D + d])) *
                                      fabs(e[(p + k) * D + d]);
            }
        }

        /* through the convolution: its input rows, plus the loss on the new state */
        for (int64_t i = 0; i < E; ++i) {
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0, cnd = 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    const int64_t p = i - k;
                    if (p >= 0 && p < L) acc += (double)taps[(k * H + h) * D + d] * dc[p * D + d];
                    if (p >= 0 && p < L) cnd += fabs((double)taps[(k * H + h) * D + d]) * mg[p * D + d];
                }
                if (gs && i >= L) acc += gs[((s * R + (i - L)) * H + h) * D + d];
                if (gs && i >= L) cnd += fabs(gs[((s * R + (i - L)) * H + h) * D + d]);
                if (i >= R) {
                    dx[((start + i - R) * H + h) * D + d] = acc;
                    if (cond_dx) cond_dx[((start + i - R) * H + h) * D + d] = cnd;
                } else {
                    if (dstate) dstate[((s * R + i) * H + h) * D + d] = from_state ? acc : 0.0;
                    if (cond_dstate) cond_dstate[((s * R + i) * H + h) * D + d] = from_state ? cnd : 0.0;
                }
            }
        }
        free(e);
        free(dc);
        free(mg);
        free(c);
        free(av);
    }

    for (int64_t k = 0; k < W; ++k)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0, cnd = 0.0;
                for (int64_t s = 0; s < n_seq; ++s) acc += part_taps[((s * H + h) * W + k) * D + d];
                for (int64_t s = 0; s < n_seq; ++s) cnd += part_ctaps[((s * H + h) * W + k) * D + d];
                dtaps[(k * H + h) * D + d] = acc;
                if (cond_dtaps) cond_dtaps[(k * H + h) * D + d] = cnd;
            }
    for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0, cnd = 0.0;
        for (int64_t u = 0; u < units; ++u) acc += part_gamma[u * D + d];
        for (int64_t u = 0; u < units; ++u) cnd += part_cgamma[u * D + d];
        dgamma[d] = acc;
        if (cond_dgamma) cond_dgamma[d] = cnd;
    }
    free(part_taps);
    free(part_gamma);
    free(part_ctaps);
    free(part_cgamma);
    return 0;
}
