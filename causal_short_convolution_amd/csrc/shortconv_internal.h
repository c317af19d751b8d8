// Internal interface between the C-ABI layer (abi.hip) and the kernels (kernels.hip,
// backward.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sc {

// Device-side arguments of one fused step. Index [0] is K, [1] is V.
struct StepArgs {
    const void* x[2];        // new rows, [tokens][H][D] with token stride x_stride[i] elements
    int64_t x_stride[2];
    const float* taps[2];    // fp32 [W][H][D]
    const float* gamma[2];   // fp32 [D]
    void* state[2];          // [num_state_slots][W-1][H][D] or null (W == 1)
    void* cache[2];          // [num_slots][H][D] rows, or MXFP8 codes [num_slots][H][D] bytes
    void* scales[2];         // MXFP8 scales [num_slots][H][D/32] bytes (null for plain rows)
    const int32_t* cu;       // prefill: int32 [num_seqs+1]
    const int32_t* state_idx;  // int32 [num_seqs] or null (identity)
    const uint8_t* has_init;   // prefill: uint8 [num_seqs] or null (all 1)
    const int64_t* slot;       // int64 [tokens]
    int64_t tokens;            // prefill: total packed tokens; decode: batch
    int64_t num_slots;
    int64_t num_state_slots;
    int32_t num_seqs;          // prefill only
    int32_t heads;
    int32_t lanes_per_tensor;  // heads * head_dim / (16 / element bytes)
    int32_t lane_blocks;       // blocks needed to cover 2 * lanes_per_tensor lanes
    int32_t tiles;             // prefill: number of logical tiles (upper bound, see kernels.hip)
    float eps;
};

// Extra arguments of speculative verification and of its commit.
struct VerifyArgs {
    void* snap[2];             // [num_seqs][max_tokens][W-1][H][D] per tensor, or null (W == 1)
    const int32_t* accepted;   // commit only: int32 [num_seqs]
    int32_t max_tokens;
};

// Device-side arguments of the backward. Index [0] is K, [1] is V.
struct BwdArgs {
    const void* x[2];          // forward inputs, [tokens][H][D], token stride x_stride[i]
    int64_t x_stride[2];
    const float* taps[2];      // fp32 [W][H][D]
    const float* gamma[2];     // fp32 [D]
    const void* state[2];      // forward's initial-state pool [num_state_slots][W-1][H][D] or null
    const void* dy[2];         // dLoss/d(output rows), [tokens][H][D] contiguous
    const void* gs[2];         // dLoss/d(new state), [num_seqs][W-1][H][D] or null
    void* dx[2];               // out: [tokens][H][D] contiguous
    void* dstate[2];           // out: [num_seqs][W-1][H][D] or null
    float* dtaps[2];           // out: fp32 [W][H][D]
    float* dgamma[2];          // out: fp32 [D]
    float* partial;            // workspace: [groups][slices][W+1][64 lanes][4] fp32
    double* chunk;             // workspace after the partials: [chunks][slices][W+1][64][4] fp64
    const int32_t* cu;         // int32 [num_seqs+1]
    const int32_t* state_idx;  // int32 [num_seqs] or null (identity)
    const uint8_t* has_init;   // uint8 [num_seqs] or null (all 1)
    int64_t tokens;
    int64_t num_state_slots;
    int32_t num_seqs;
    int32_t heads;
    int32_t lanes_per_tensor;  // heads * head_dim / 4 (4 channels per lane)
    int32_t slices;            // 64-lane column slices covering 2 * lanes_per_tensor lanes
    int32_t tiles;             // logical tiles (upper bound, as in prefill)
    int32_t groups;            // workgroups per column slice (each walks a few tiles)
    int32_t chunks;            // groups are first summed in chunks (of 64)
    int32_t tiles_per_group;   // consecutive tiles one workgroup walks (1..4)
    float eps;
};

// Grid shape and workspace size of the backward for one problem size.
struct BwdShape {
    int64_t lanes_per_tensor;
    int64_t slices;
    int64_t tiles;
    int64_t groups;
    int64_t tiles_per_group;
    int64_t chunks;
    size_t partial_bytes;      // the fp32 partials; the fp64 chunk sums follow them
    size_t workspace_bytes;
};
BwdShape backward_shape(int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                        int32_t head_dim, int32_t width, int dtype);
hipError_t launch_backward(BwdArgs a, int dtype, int head_dim, int width, hipStream_t stream);

// Returns hipSuccess or the launch error. `dtype`: 0 = fp32, 1 = bf16. Shapes already validated.
hipError_t launch_prefill(StepArgs a, int dtype, int head_dim, int width, bool mx,
                          hipStream_t stream);
hipError_t launch_decode(StepArgs a, int dtype, int head_dim, int width, bool mx,
                         hipStream_t stream);
hipError_t launch_mx_quantize(StepArgs a, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_verify(StepArgs a, VerifyArgs va, int dtype, int head_dim, int width,
                         hipStream_t stream);
hipError_t launch_commit(StepArgs a, VerifyArgs va, int dtype, int head_dim, int width,
                         hipStream_t stream);

// Tokens per prefill tile for a width, cache format, row width in lanes and token count (the
// kernel, and so the tile, depends on all four).
int prefill_tile_tokens(int width, bool mx, int64_t lanes_per_tensor, int64_t tokens);

}  // namespace sc
