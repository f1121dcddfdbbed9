// Device-side helpers and the internal descriptors shared by the kernels and
// the host launcher. gfx950 (CDNA4) only: 64-lane wavefronts, MFMA, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mu {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

enum : int { DT_F32 = 0, DT_BF16 = 1 };

// Pointers read from descriptor tables are generic; casting them to the global
// address space lets the compiler emit global_load/global_store (vmcnt only)
// instead of flat accesses that also hold lgkmcnt.
#define MU_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ MU_GLOBAL T* gp(T* p) {
    return (MU_GLOBAL T*)p;
}

// ---------------------------------------------------------------------------
// One Newton-Schulz problem: a (matrix, head) block in the Muon step, or one
// head of an input in the orthogonalise-only call.
//
// U-space is the head block as stored: hr rows x hc cols, row pitch ld. X-space
// is the wide orientation the iteration runs in: m = min(hr, hc) rows and
// n = max(hr, hc) cols, X = U when hr <= hc and X = U^T otherwise ("tall").
// The workspace keeps X (mp x np). The bf16 Gram X X^T reads it as both
// operands and the bf16 apply B X reads it as its right operand through
// transposing LDS reads (as does the fused short-block kernel). A transposed
// copy X^T (np x mp) exists only where a kernel reads X with its k down the
// columns from memory: the fp32 apply and the ns_steps == 0 finish of a tall
// block (xt_used). Buffers are padded with zeros to multiples of the GEMM tile;
// zero padding is preserved by every step, so the GEMM kernels need no bounds
// checks.
//
// Storage of the workspace operands (X, X^T, A, B): with bf16 Newton-Schulz
// they are K-blocked (see kb_off), with fp32 Newton-Schulz plain row-major.
// ---------------------------------------------------------------------------
struct NsProb {
    const void* src;   // gradient (step) or input (orthogonalise), U-space
    float* mom;        // momentum, U-space (step only)
    void* param;       // parameter, U-space (step only)
    void* out;         // output, U-space (orthogonalise only)
    int64_t ld;        // row pitch of src/mom/param/out in elements
    int32_t hr, hc;    // U-space shape
    int32_t m, n;      // X-space shape
    int32_t mp, np;    // padded X-space shape
    int32_t tall;      // X = U^T
    int32_t vec;       // 16-byte vector path is legal for the U-space buffers
    float scale;       // update scale
    int32_t xt_used;   // the X^T buffers exist (else xt[] are null)
    void* x[2];        // ping-pong X buffers, mp x np, NS element type
    void* xt[2];       // their transposes, np x mp, when xt_used
    void* a;           // a I + b A (cubic steps) or A = X X^T (quintic steps), mp x mp
    void* b;           // a I + b A + c A^2 (quintic steps), mp x mp, or null
    double* partials;  // per prep-tile sums of squares (float64: no overflow or
                       // underflow for any finite float32 U)
    float* fold;       // 2^-e / (||U||_F + eps), written by the norm kernel: the
                       // factor that turns the stored X0 into U / (||U||_F + eps)
    int32_t* xexp;     // e: the stored X0 is U * 2^e (0 unless ||U||_F lies
                       // outside the band where the unscaled Gram is exact)
    float* norm_out;   // optional ||U||_F
    float* oout;       // optional float32 copy of O in U-space (step only)
    int32_t nparts;    // number of prep tiles (see prep_rows / prep_cols)
    int32_t pad1;
};

// Binary search: index p with prefix[p] <= t < prefix[p+1].
__device__ inline int find_prob(const int* prefix, int nprobs, int t) {
    int lo = 0, hi = nprobs - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Map a workgroup id so that consecutive logical tiles land on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs; when the grid is a
// multiple of 8, XCD x receives ids x, x+8, ... and is given the contiguous
// logical block [x*G/8, (x+1)*G/8).
__device__ inline int xcd_remap(int wg, int grid) {
    if ((grid & 7) != 0) return wg;
    return (wg & 7) * (grid >> 3) + (wg >> 3);
}
// The same in windows: the grid is cut into windows of 8*W logical tiles and
// XCD x receives the contiguous block [x*W, (x+1)*W) of each window (the last
// window splits its remainder evenly), so the XCDs move through the logical
// order together. The Gram launches use it over a tile order sorted by K, so
// that the XCDs hold the X of only a few matrices of like K at a time (with
// a long K each tile streams two strips of X larger than an XCD's L2). W <= 0
// is the plain contiguous split.
__device__ inline int xcd_remap_window(int wg, int grid, int W) {
    if (W <= 0) return xcd_remap(wg, grid);
    if ((grid & 7) != 0) return wg;
    const int x = wg & 7, n = wg >> 3, nper = grid >> 3;
    const int base = (n / W) * W;
    const int c = min(W, nper - base);
    return base * 8 + x * c + (n - base);
}

// Element (r, k) of a K-blocked operand with R rows (R a multiple of 16, K a
// multiple of 32): 1 KB blocks of 16 rows x 32 k, ordered panel-major (block
// of k-panel k/32 and row group r/16 at index (k/32)*(R/16) + r/16); inside a
// block, the 16-byte chunk of k (k%32)/8 of row r%16 sits at byte
// 16*(16*((k%32)/8) + r%16). A block is the lane order of one 16x16x32 MFMA
// fragment, and the TS x 32 slice of a TS-row tile is one contiguous run.
__device__ inline int64_t kb_off(int r, int k, int R) {
    return ((int64_t)(k >> 5) * (R >> 4) + (r >> 4)) * 512 + ((k & 31) >> 3) * 128 + (r & 15) * 8 + (k & 7);
}
// Offset of element (r, k) of a workspace operand with R rows and K columns:
// K-blocked for bf16, row-major for fp32. k is a multiple of 4 whenever four
// or eight consecutive elements are accessed at once.
template <typename TX>
__device__ inline int64_t op_off(int r, int k, int R, int K) {
    if constexpr (sizeof(TX) == 2) return kb_off(r, k, R);
    else return (int64_t)r * K + k;
}

template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<bf16>(bf16 v) { return (float)v; }
template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Wavefront sum in a fixed order (butterfly over 64 lanes): every lane ends
// with the same value, and the order does not depend on timing.
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace mu
