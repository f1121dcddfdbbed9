// Host-side launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mu {

// Prep tile edge (elements) of the momentum / transpose kernel.
// Prep / finish tile over the U-oriented buffer: 32 x 128 with bf16
// Newton-Schulz operands (whole K-blocks, long row runs), 64 x 64 with fp32
// (buffers are padded to multiples of 64 only).
template <typename TX> constexpr int prep_rows() { return sizeof(TX) == 2 ? 32 : 64; }
template <typename TX> constexpr int prep_cols() { return sizeof(TX) == 2 ? 128 : 64; }
inline int prep_rows_dt(int ns_dtype) { return ns_dtype == DT_BF16 ? 32 : 64; }
inline int prep_cols_dt(int ns_dtype) { return ns_dtype == DT_BF16 ? 128 : 64; }

struct PrepArgs {
    const NsProb* probs;
    const int* prefix;   // nprobs+1 cumulative prep tiles
    int nprobs;
    int total_tiles;
    int src_dtype;       // element type of src/param/out
    int ns_dtype;        // element type of the X buffers
    int with_momentum;   // 1: Muon step, 0: orthogonalise-only (U = src)
    int nesterov;
    float mu;
};
hipError_t launch_prep(const PrepArgs& a, hipStream_t s);

struct NormArgs {
    const NsProb* probs;
    int nprobs;
    float eps;
};
hipError_t launch_norm(const NormArgs& a, hipStream_t s);

enum GemmMode : int {
    GM_GRAM = 0,        // B = f (a I + b f^2 X X^T), or A = f^2 X X^T when a quintic step follows  (upper, mirrored)
    GM_GRAM2 = 1,       // B = f (a I + b A + c A A^T)                                               (upper, mirrored)
    GM_APPLY = 2,       // X' = B X, B the matrix the Gram pass(es) left (f = 1/||U|| on the first step, else 1)
    GM_APPLY_LAST = 3,  // as GM_APPLY, result O goes to the update or to `out`
};

struct GemmArgs {
    const NsProb* probs;
    const int* prefix;   // nprobs+1 cumulative tiles for this mode
    const int* order;    // problem at each prefix position (the tile order runs
                         // through the problems in this order); null: identity
    int nprobs;
    int total_tiles;
    int mode;
    int src;             // which x[] buffer holds the current X
    int first;           // apply the fold (1/||U||) of the first step
    int use_b;           // quintic step: Gram writes A, the A^2 pass writes B, apply reads b
    int with_update;     // last step: 1 updates param, 0 writes out
    int src_dtype;       // element type of param/out
    int xcd_window;      // Gram tiles per XCD per window of the tile order (0: contiguous split)
    float ca, cb, cc;    // step coefficients
    float lr, wd;
};
// tile: 256 or 128 (square tiles, bf16) ; float32 uses 64.
hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);

// Newton-Schulz for problems with mp == 128 (bf16, cubic steps) up to the last
// apply, in one launch, one workgroup per problem. X0 is in x[0]; the steps
// ping-pong between x[0] and x[1] as on the tiled path, so the X of the last
// step is in x[(ns_steps - 1) & 1], and that step's B is left in `a` for the
// tiled last apply (GM_APPLY_LAST), which writes the update.
constexpr int SMALL_MAX_STEPS = 16;
struct SmallArgs {
    const NsProb* probs;
    int nprobs;
    int ns_steps;          // 1 .. SMALL_MAX_STEPS
    float ca[SMALL_MAX_STEPS], cb[SMALL_MAX_STEPS];
};
hipError_t launch_ns_small(const SmallArgs& a, hipStream_t s);

struct FinishArgs {      // ns_steps == 0: O = fold * X0
    const NsProb* probs;
    const int* prefix;   // prep-tile prefix
    int nprobs;
    int total_tiles;
    int ns_dtype;
    int src_dtype;
    int with_update;
    float lr, wd;
};
hipError_t launch_finish(const FinishArgs& a, hipStream_t s);

struct AdamWDesc {
    void* param;
    const void* grad;
    float* m;
    float* v;
    int64_t numel;
    int32_t dtype;
    int32_t vec;         // 16-byte aligned bases: vector path
    float lr, wd;
};
struct AdamWArgs {
    const AdamWDesc* descs;
    const int64_t* prefix;  // n+1 cumulative chunks
    int n;
    int64_t total_chunks;
    float beta1, beta2, eps;
    float bc1, bc2;         // 1 - beta^t
};
constexpr int ADAMW_CHUNK = 8192;  // elements per workgroup
hipError_t launch_adamw(const AdamWArgs& a, hipStream_t s);

// QK-Clip: one segment per (layer, query or key matrix, head) row block.
struct QkSeg {
    void* w;             // first element of the head's rows
    int64_t numel;
    int32_t dtype;
    int32_t vec;         // 16-byte aligned start: vector path
    const float* ml;     // max logits of the query heads this block follows
    int32_t nml;         // 1 for a query head, G for a key head
    int32_t pad;
    float* gamma_out;    // query heads: optional per-head gamma output
};
struct QkArgs {
    const QkSeg* segs;
    const int64_t* prefix;  // n+1 cumulative chunks
    int n;
    int64_t total_chunks;
    float tau;
};
constexpr int QK_CHUNK = 8192;  // elements per workgroup
hipError_t launch_qkclip(const QkArgs& a, hipStream_t s);

// Copy `bytes` from device-visible pinned host memory `src` (16-byte aligned)
// to device memory `dst` (16-byte aligned) on stream s.
hipError_t launch_table_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace mu
