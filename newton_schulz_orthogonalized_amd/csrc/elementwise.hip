// HBM-bound kernels of the Muon step and the AdamW step (gfx950).
//
//  k_prep    momentum EMA + Nesterov blend, write U into the workspace as X
//            (wide orientation; and X^T where a problem keeps it) with zero
//            padding, through an LDS tile, and one sum of squares per tile
//            (fixed order).
//  k_norm    per (matrix, head): fixed-order sum of the tile partials,
//            fold = 1/(||U||_F + eps).
//  k_finish  ns_steps == 0: O = fold * X0, then the update (or the output).
//  k_adamw   bias-corrected AdamW over a flat list of tensors, one launch.
//  k_qkclip  QK-Clip: per-head rescale of attention query/key weights.
//  k_table   copy of a call's descriptor table from pinned host memory into
//            the workspace.
//
// Momentum: MuonClip Optimizer page, section "Momentum" (EMA, decay 0.95).
// Nesterov blend: named on the nanochat optimizer page ("Muon Step
// Implementation") and as the nesterov flag of _prepare on the NeMo AutoModel
// muown_triton page; the blend used is U = (1-mu) G + mu M_new.
// AdamW: nanochat optimizer page, "AdamW Step Implementation" (exp_avg,
// exp_avg_sq, step, lr, betas, eps, weight decay).
#include "common.hpp"
#include "launch.hpp"

namespace mu {

namespace {

constexpr int NTHR = 256;

// Four consecutive U-space elements (row r, cols c0..c0+3) of a buffer whose
// element type is TS; out-of-range columns read as 0.
template <typename TS>
__device__ inline void load4(const void* base, int64_t off, int valid, bool vec, float v[4]) {
    const MU_GLOBAL TS* p = (const MU_GLOBAL TS*)base + off;
    if (vec && valid == 4) {
        if constexpr (sizeof(TS) == 2) {
            bf16x4 q = *(const MU_GLOBAL bf16x4*)p;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (float)q[e];
        } else {
            f32x4 q = *(const MU_GLOBAL f32x4*)p;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = q[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = e < valid ? to_f32<TS>(p[e]) : 0.f;
    }
}

template <typename TS>
__device__ inline void store4(void* base, int64_t off, int valid, bool vec, const float v[4]) {
    MU_GLOBAL TS* p = (MU_GLOBAL TS*)base + off;
    if (vec && valid == 4) {
        if constexpr (sizeof(TS) == 2) {
            bf16x4 q;
#pragma unroll
            for (int e = 0; e < 4; ++e) q[e] = (bf16)v[e];
            *(MU_GLOBAL bf16x4*)p = q;
        } else {
            f32x4 q = {v[0], v[1], v[2], v[3]};
            *(MU_GLOBAL f32x4*)p = q;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e < valid) p[e] = from_f32<TS>(v[e]);
    }
}

// Four consecutive X-space elements; the X workspace is always 4-aligned.
template <typename TX>
__device__ inline void store_x4(TX* p, const float v[4]) {
    if constexpr (sizeof(TX) == 2) {
        bf16x4 q;
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = (bf16)v[e];
        *(MU_GLOBAL bf16x4*)p = q;
    } else {
        f32x4 q = {v[0], v[1], v[2], v[3]};
        *(MU_GLOBAL f32x4*)p = q;
    }
}
template <typename TX>
__device__ inline void load_x4(const TX* p, float v[4]) {
    if constexpr (sizeof(TX) == 2) {
        bf16x4 q = *(const MU_GLOBAL bf16x4*)p;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (float)q[e];
    } else {
        f32x4 q = *(const MU_GLOBAL f32x4*)p;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = q[e];
    }
}

// Block-wide fixed-order sum (four waves); result valid in every thread.
template <typename T>
__device__ inline T block_sum(T v, T* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    T s = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    return s;
}

// Gradient and momentum of four consecutive elements of one U-space row
// (zeros outside the head block). Split from the arithmetic so that a thread
// can issue the loads of all its rows before the first momentum store (which
// the compiler would otherwise have to wait for, not knowing that the buffers
// are disjoint).
template <typename TS>
__device__ inline void load_gm(const NsProb& P, int r, int c0, bool with_m, float g[4], float m[4]) {
    const int valid = (r < P.hr) ? max(0, min(4, P.hc - c0)) : 0;
    const int64_t off = (int64_t)r * P.ld + c0;
    const bool vec = P.vec != 0;
    load4<TS>(P.src, off, valid, vec, g);
    if (with_m) load4<float>(P.mom, off, valid, vec, m);
    else {
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = 0.f;
    }
}

// U from G and M; the updated momentum is stored back. (MuonClip Optimizer
// page, "Momentum": M <- mu M + (1 - mu) G; the Nesterov blend
// U = (1 - mu) G + mu M_new.)
__device__ inline void make_u(const NsProb& P, int r, int c0, bool with_m, bool nesterov, float mu, const float g[4],
                              float m[4], float u[4]) {
    if (!with_m) {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[e] = g[e];
        return;
    }
    const float omm = 1.f - mu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        m[e] = mu * m[e] + omm * g[e];
        u[e] = nesterov ? omm * g[e] + mu * m[e] : m[e];
    }
    const int valid = (r < P.hr) ? max(0, min(4, P.hc - c0)) : 0;
    if (valid > 0) store4<float>(P.mom, (int64_t)r * P.ld + c0, valid, P.vec != 0, m);
}

// Tiles run over U's orientation (X for wide blocks, X^T for tall ones): U is
// computed into an LDS tile and written into X, straight for a wide block and
// transposed for a tall one, and into X^T too where the problem keeps it
// (xt_used). Out-of-range elements are written as zeros, which is the padding
// every later step relies on. Tile shape:
// prep_rows(TX) x prep_cols(TX) (32 x 128 for bf16, so a tile reads 256-byte
// gradient and 512-byte momentum runs per row). With bf16 Newton-Schulz both
// buffers are K-blocked: a tile is 8 whole 1 KB blocks in each of them, and
// thread q of a pass writes 16-byte chunk q, so a wave stores one whole block.
template <typename TS, typename TX>
__global__ __launch_bounds__(NTHR) void k_prep(PrepArgs A) {
    constexpr int TR = prep_rows<TX>(), TC = prep_cols<TX>();
    constexpr int TPR = TC / 4;          // threads per tile row
    constexpr int RSTEP = NTHR / TPR;    // rows between a thread's rows
    __shared__ float tile[TR][TC + 1];
    __shared__ double red[4];
    const int t = xcd_remap(blockIdx.x, gridDim.x);   // each XCD streams one contiguous run of tiles
    if (t >= A.total_tiles) return;
    const int p = __builtin_amdgcn_readfirstlane(find_prob(A.prefix, A.nprobs, t));
    const NsProb P = A.probs[p];   // by value: held in registers, never re-read after a store
    const int local = t - A.prefix[p];
    const bool wide = !P.tall;
    const int RD = wide ? P.mp : P.np;   // rows of the U-oriented buffer
    const int KD = wide ? P.np : P.mp;   // its columns = rows of the other one
    TX* D = (TX*)(wide ? P.x[0] : P.xt[0]);    // U's orientation
    TX* Tt = (TX*)(wide ? P.xt[0] : P.x[0]);   // transposed
    const bool wr_d = wide || P.xt_used, wr_t = !wide || P.xt_used;
    const int tiles_n = KD / TC;
    const int ti = local / tiles_n, tj = local - ti * tiles_n;
    const int tid = threadIdx.x;
    const int rr = tid / TPR, cc = (tid % TPR) * 4;
    const bool with_m = A.with_momentum != 0;
    const bool nest = gp(A.cs)->nesterov != 0;
    const float mu = gp(A.cs)->mu;
    float gk[4][4], mk[4][4];
    // a tile wholly inside the head block, on vector-capable buffers, loads
    // without per-lane range checks (no divergent branches between the loads)
    const bool inside = P.vec && (ti + 1) * TR <= P.hr && (tj + 1) * TC <= P.hc;
    if (inside) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t off = (int64_t)(ti * TR + rr + RSTEP * k) * P.ld + tj * TC + cc;
            if constexpr (sizeof(TS) == 2) {
                // the gradient is read once: a non-temporal load (8B-shaped
                // set, same process: 14.97 -> 14.90 ms)
                const bf16x4 q = __builtin_nontemporal_load((const MU_GLOBAL bf16x4*)((const bf16*)P.src + off));
#pragma unroll
                for (int e = 0; e < 4; ++e) gk[k][e] = (float)q[e];
            } else {
                const f32x4 q = *(const MU_GLOBAL f32x4*)((const float*)P.src + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) gk[k][e] = q[e];
            }
            if (with_m) {
                const f32x4 q = *(const MU_GLOBAL f32x4*)(P.mom + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) mk[k][e] = q[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) mk[k][e] = 0.f;
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) load_gm<TS>(P, ti * TR + rr + RSTEP * k, tj * TC + cc, with_m, gk[k], mk[k]);
    }
    // sum of squares in float64: squares of float32 values are exact there and
    // neither overflow nor underflow, whatever the magnitude of U
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = ti * TR + rr + RSTEP * k, c0 = tj * TC + cc;
        float u[4];
        make_u(P, r, c0, with_m, nest, mu, gk[k], mk[k], u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ss = fma((double)u[e], (double)u[e], ss);
            tile[rr + RSTEP * k][cc + e] = u[e];
        }
        if constexpr (sizeof(TX) == 4) {
            if (wr_d) store_x4<TX>(D + (int64_t)r * KD + c0, u);
        }
    }
    __syncthreads();
    if constexpr (sizeof(TX) == 2) {
        static_assert(TR % 32 == 0 && TC % 32 == 0, "whole K-blocks in both buffers");
#pragma unroll
        for (int pass = 0; pass < TR * TC / (NTHR * 8); ++pass) {
            const int q = pass * NTHR + tid;
            const int blk = q >> 6, c = (q >> 4) & 3, r16 = q & 15;
            // D: block (row group g, k-panel pl) of the tile; chunk c of row r16
            if (wr_d) {
                const int g = blk % (TR / 16), pl = blk / (TR / 16);
                const int row = g * 16 + r16, col = pl * 32 + c * 8;
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (bf16)tile[row][col + e];
                *(MU_GLOBAL bf16x8*)(D + kb_off(ti * TR + row, tj * TC + col, RD)) = o;
            }
            // the other buffer: its rows are tile columns, its k the tile rows
            if (wr_t) {
                const int g = blk % (TC / 16), pl = blk / (TC / 16);
                const int row = g * 16 + r16, col = pl * 32 + c * 8;
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (bf16)tile[col + e][row];
                *(MU_GLOBAL bf16x8*)(Tt + kb_off(tj * TC + row, ti * TR + col, KD)) = o;
            }
        }
    } else {
        static_assert(TR == TC, "the fp32 transpose pass walks a square tile");
#pragma unroll
        for (int k = 0; k < 4 && wr_t; ++k) {
            const int a = rr + RSTEP * k;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = tile[cc + e][a];
            store_x4<TX>(Tt + (int64_t)(tj * TC + a) * RD + ti * TR + cc, v);
        }
    }
    const double s = block_sum(ss, red);
    if (tid == 0) *gp(P.partials + local) = s;
}

// ||U||_F in float64 from the tile partials (fixed order), and the factors
// the Newton-Schulz kernels fold into their first step. X0 is stored as U;
// when ||U||_F lies outside [2^-NORM_BAND_LOG2, 2^NORM_BAND_LOG2] the stored
// X0 is to be multiplied by 2^e (||U||_F 2^e in [1, 2), done by k_rescale),
// and fold = 2^-e / (||U||_F + eps) turns the stored X0 back into
// U / (||U||_F + eps) either way. U = 0 gives fold = 0 (O = 0 for any eps,
// eps = 0 included); a non-finite norm keeps e = 0 and lets NaN propagate.
__global__ __launch_bounds__(NTHR) void k_norm(NormArgs A) {
    __shared__ double red[4];
    const NsProb& P = A.probs[blockIdx.x];
    double s = 0.0;
    for (int i = threadIdx.x; i < P.nparts; i += NTHR) s += *gp(P.partials + i);
    s = block_sum(s, red);
    if (threadIdx.x == 0) {
        const double nrm = sqrt(s);
        int e = 0;
        if (nrm > 0.0 && isfinite(nrm) &&
            (nrm < ldexp(1.0, -NORM_BAND_LOG2) || nrm > ldexp(1.0, NORM_BAND_LOG2)))
            e = -ilogb(nrm);
        const double f = nrm == 0.0 ? 0.0 : ldexp(1.0, -e) / (nrm + (double)gp(A.cs)->eps);
        *gp(P.fold) = (float)f;
        *gp(P.xexp) = e;
        if (P.norm_out) *gp(P.norm_out) = (float)nrm;
    }
}

// The stored X0 (and X0^T where the problem keeps it) times 2^e, for the
// problems whose exponent is nonzero. Every workgroup reads the exponents 256
// at a time and moves on when none is set, so with every norm inside the band
// (the usual case) the launch costs a few microseconds; otherwise all
// workgroups stride over each flagged problem's buffers, 16 bytes at a time.
// A power-of-two scale is exact: every stored value stays representable
// (values tiny against ||U||_F may become subnormal, at no cost to the result).
template <typename TX>
__device__ __forceinline__ void rescale_buf(void* buf, int64_t n16, int e) {
    const int64_t stride = (int64_t)gridDim.x * NTHR;
    for (int64_t i = (int64_t)blockIdx.x * NTHR + threadIdx.x; i < n16; i += stride) {
        MU_GLOBAL u32x4* q = (MU_GLOBAL u32x4*)buf + i;
        if constexpr (sizeof(TX) == 2) {
            bf16x8 v = __builtin_bit_cast(bf16x8, *q);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = (bf16)ldexpf((float)v[k], e);
            *q = __builtin_bit_cast(u32x4, v);
        } else {
            f32x4 v = __builtin_bit_cast(f32x4, *q);
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = ldexpf(v[k], e);
            *q = __builtin_bit_cast(u32x4, v);
        }
    }
}

template <typename TX>
__global__ __launch_bounds__(NTHR) void k_rescale(RescaleArgs A) {
    __shared__ int32_t se[NTHR];
    for (int base = 0; base < A.nprobs; base += NTHR) {
        const int p = base + (int)threadIdx.x;
        const int32_t e = p < A.nprobs ? *gp(A.xexp + p) : 0;
        if (!__syncthreads_or(e != 0)) continue;
        se[threadIdx.x] = e;
        __syncthreads();
        const int cnt = min(NTHR, A.nprobs - base);
        for (int q = 0; q < cnt; ++q) {
            const int eq = se[q];
            if (eq == 0) continue;
            const NsProb P = A.probs[base + q];
            const int64_t n16 = (int64_t)P.mp * P.np * (int64_t)sizeof(TX) / 16;
            rescale_buf<TX>(P.x[0], n16, eq);
            if (P.xt_used) rescale_buf<TX>(P.xt[0], n16, eq);
        }
        __syncthreads();   // `se` is rewritten by the next chunk
    }
}

// O = fold * X0 written back in U-space: update (W - lr*wd*W - lr*scale*O) or
// output. Same tiling as k_prep, over the U-oriented buffer (X for wide
// blocks, X^T for tall ones), which holds U in U's own orientation.
template <typename TS, typename TX>
__global__ __launch_bounds__(NTHR) void k_finish(FinishArgs A) {
    constexpr int TR = prep_rows<TX>(), TC = prep_cols<TX>();
    constexpr int TPR = TC / 4, RSTEP = NTHR / TPR;
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    if (t >= A.total_tiles) return;
    const int p = __builtin_amdgcn_readfirstlane(find_prob(A.prefix, A.nprobs, t));
    const NsProb P = A.probs[p];   // by value: held in registers, never re-read after a store
    const int local = t - A.prefix[p];
    const bool wide = !P.tall;
    const int RD = wide ? P.mp : P.np, KD = wide ? P.np : P.mp;
    const TX* D = (const TX*)(wide ? P.x[0] : P.xt[0]);
    const int tiles_n = KD / TC;
    const int ti = local / tiles_n, tj = local - ti * tiles_n;
    const int tid = threadIdx.x;
    const int rr = tid / TPR, cc = (tid % TPR) * 4;
    const float f = *gp(P.fold);
    const bool vec = P.vec != 0;
    const float lr = gp(A.cs)->lr, wd = gp(A.cs)->wd;
    const bool cautious = gp(A.cs)->cautious != 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = ti * TR + rr + RSTEP * k, c0 = tj * TC + cc;
        const int valid = (r < P.hr) ? max(0, min(4, P.hc - c0)) : 0;
        if (valid == 0) continue;
        float o[4];
        load_x4<TX>(D + op_off<TX>(r, c0, RD, KD), o);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= f;
        const int64_t off = (int64_t)r * P.ld + c0;
        if (P.oout) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e < valid) *gp(P.oout + off + e) = o[e];
        }
        if (A.with_update) {
            float w[4];
            load4<TS>(P.param, off, valid, vec, w);
            const float decay = lr * wd, step = lr * P.scale;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // cautious weight decay: no decay where the update opposes the weight's sign
                const float d = (cautious && w[e] * (step * o[e]) < 0.f) ? 0.f : decay;
                w[e] = (w[e] - d * w[e]) - step * o[e];
            }
            store4<TS>(P.param, off, valid, vec, w);
        } else {
            store4<TS>(P.out, off, valid, vec, o);
        }
    }
}

// ---------------------------------------------------------------------------
// AdamW. Workgroup c handles elements [k*CHUNK, (k+1)*CHUNK) of tensor i where
// prefix[i] <= c < prefix[i+1] and k = c - prefix[i]. Each thread handles two
// groups of 8 consecutive elements (16-byte bf16 / 32-byte fp32 accesses).
// ---------------------------------------------------------------------------
// One AdamW element in fp32, in the order of the formula, each operation
// rounded once: contraction into fused multiply-adds is off here, because the
// compiler fuses differently where the gradient arrives as a bf16 scalar (a
// float32 ulp apart in a quarter of the moments), and every path of k_adamw
// (band tile or contiguous chunk, vector or scalar accesses) must give an
// element the same result.
__device__ __forceinline__ void adamw1(float& p, float g, float& m, float& v, const AdamWArgs& A, float lr,
                                       float decay) {
#pragma clang fp contract(off)
    m = A.beta1 * m + (1.f - A.beta1) * g;
    v = A.beta2 * v + (1.f - A.beta2) * g * g;
    const float mhat = m / A.bc1;
    const float vhat = v / A.bc2;
    p = (p - decay * p) - lr * mhat / (sqrtf(vhat) + A.eps);
}

template <typename TP>
__device__ inline void adamw8(const AdamWDesc& D, int64_t i0, int cnt, const AdamWArgs& A) {
    MU_GLOBAL TP* p = (MU_GLOBAL TP*)D.param + i0;
    const MU_GLOBAL TP* g = (const MU_GLOBAL TP*)D.grad + i0;
    MU_GLOBAL float* m = (MU_GLOBAL float*)D.m + i0;
    MU_GLOBAL float* v = (MU_GLOBAL float*)D.v + i0;
    float pv[8], gv[8], mv[8], vv[8];
    const bool full = (cnt == 8) && D.vec;
    if (full) {
        if constexpr (sizeof(TP) == 2) {
            bf16x8 a = *(const MU_GLOBAL bf16x8*)p, b = *(const MU_GLOBAL bf16x8*)g;
#pragma unroll
            for (int e = 0; e < 8; ++e) { pv[e] = (float)a[e]; gv[e] = (float)b[e]; }
        } else {
            f32x4 a0 = ((const MU_GLOBAL f32x4*)p)[0], a1 = ((const MU_GLOBAL f32x4*)p)[1];
            f32x4 b0 = ((const MU_GLOBAL f32x4*)g)[0], b1 = ((const MU_GLOBAL f32x4*)g)[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) { pv[e] = a0[e]; pv[e + 4] = a1[e]; gv[e] = b0[e]; gv[e + 4] = b1[e]; }
        }
        f32x4 m0 = ((const MU_GLOBAL f32x4*)m)[0], m1 = ((const MU_GLOBAL f32x4*)m)[1];
        f32x4 v0 = ((const MU_GLOBAL f32x4*)v)[0], v1 = ((const MU_GLOBAL f32x4*)v)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { mv[e] = m0[e]; mv[e + 4] = m1[e]; vv[e] = v0[e]; vv[e + 4] = v1[e]; }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (e < cnt) { pv[e] = to_f32<TP>(p[e]); gv[e] = to_f32<TP>(g[e]); mv[e] = m[e]; vv[e] = v[e]; }
            else { pv[e] = gv[e] = mv[e] = vv[e] = 0.f; }
        }
    }
    const float lr = D.lr, decay = D.lr * D.wd;
#pragma unroll
    for (int e = 0; e < 8; ++e) adamw1(pv[e], gv[e], mv[e], vv[e], A, lr, decay);
    if (full) {
        if constexpr (sizeof(TP) == 2) {
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (bf16)pv[e];
            *(MU_GLOBAL bf16x8*)p = a;
        } else {
            ((MU_GLOBAL f32x4*)p)[0] = f32x4{pv[0], pv[1], pv[2], pv[3]};
            ((MU_GLOBAL f32x4*)p)[1] = f32x4{pv[4], pv[5], pv[6], pv[7]};
        }
        ((MU_GLOBAL f32x4*)m)[0] = f32x4{mv[0], mv[1], mv[2], mv[3]};
        ((MU_GLOBAL f32x4*)m)[1] = f32x4{mv[4], mv[5], mv[6], mv[7]};
        ((MU_GLOBAL f32x4*)v)[0] = f32x4{vv[0], vv[1], vv[2], vv[3]};
        ((MU_GLOBAL f32x4*)v)[1] = f32x4{vv[4], vv[5], vv[6], vv[7]};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < cnt) { p[e] = from_f32<TP>(pv[e]); m[e] = mv[e]; v[e] = vv[e]; }
    }
}

__device__ inline int find_tensor(const int64_t* prefix, int n, int64_t c) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= c) lo = mid; else hi = mid - 1;
    }
    return lo;
}


// Chunk layout. A tensor is cut into bands of ADAMW_BAND_ROWS rows of
// ADAMW_BAND_W elements (a band is a contiguous run of 65536 elements), and a
// band into ADAMW_BAND_W / ADAMW_TILE_C tiles of ADAMW_BAND_ROWS x
// ADAMW_TILE_C elements, one chunk (workgroup) each, taken column-fastest. A
// workgroup thus streams 16 pieces of 512 elements (1 KB of a bf16 parameter,
// 2 KB of a moment) 8 KB / 16 KB apart rather than one contiguous 8192-element
// run, which spreads each workgroup's requests over more memory channels.
// Measured on the 8B-shaped AdamW layout (bf16 parameter and gradient, float32
// moments, 2^30 elements), every variant in one process, two processes:
//   contiguous 8192-element chunks                       5.28-5.30 TB/s
//   16 x 512 tiles, 4096-wide view (this layout)         5.80-5.82
//   8 x 512 tiles, 8192-wide view (4096-element chunks)  5.83-5.85
//   16 x 256 tiles, 4096-wide view                       5.73-5.76
//   8 x 512 tiles, 4096-wide view                        5.57-5.59
//   4 x 1024 tiles, 16384-wide view                      5.52-5.54
//   plain 16-byte copy                                   5.62-5.63
// The 8192-element chunk is kept: the best layout was within 0.5 % of it.
// What is left of a tensor after its last whole band (and every chunk of a
// tensor whose buffers do not allow vector accesses) is taken in contiguous
// chunks of ADAMW_CHUNK elements.
constexpr int ADAMW_BAND_ROWS = 16, ADAMW_BAND_W = 4096, ADAMW_TILE_C = 512;
constexpr int64_t ADAMW_BAND = (int64_t)ADAMW_BAND_ROWS * ADAMW_BAND_W;
constexpr int ADAMW_TILES_PER_BAND = ADAMW_BAND_W / ADAMW_TILE_C;
static_assert(ADAMW_BAND_ROWS * ADAMW_TILE_C == ADAMW_CHUNK, "a band tile is one chunk");
static_assert(ADAMW_BAND % ADAMW_CHUNK == 0, "bands end on chunk boundaries");

// One band tile of a tensor whose four buffers are 16-byte aligned: each
// thread owns 4 consecutive elements in each of ADAMW_BAND_ROWS / 2 rows, and
// issues every load before any arithmetic.
template <typename TP>
__device__ __forceinline__ void adamw_band_tile(const AdamWDesc& D, int64_t q, const AdamWArgs& A) {
    constexpr int TPR = ADAMW_TILE_C / 4;       // threads per tile row
    constexpr int RSTEP = NTHR / TPR;           // rows between a thread's rows
    constexpr int RUNS = ADAMW_BAND_ROWS / RSTEP;
    static_assert(NTHR % TPR == 0 && ADAMW_BAND_ROWS % RSTEP == 0, "tile rows split evenly over the threads");
    const int64_t band = q / ADAMW_TILES_PER_BAND;
    const int tj = (int)(q - band * ADAMW_TILES_PER_BAND);
    const int rr = threadIdx.x / TPR, cc = (threadIdx.x % TPR) * 4;
    const int64_t base = band * ADAMW_BAND + (int64_t)rr * ADAMW_BAND_W + tj * ADAMW_TILE_C + cc;
    const MU_GLOBAL TP* pp = (const MU_GLOBAL TP*)D.param;
    const MU_GLOBAL TP* gg = (const MU_GLOBAL TP*)D.grad;
    float pv[RUNS][4], gv[RUNS][4];
    f32x4 mq[RUNS], vq[RUNS];
#pragma unroll
    for (int k = 0; k < RUNS; ++k) {
        const int64_t i0 = base + (int64_t)k * RSTEP * ADAMW_BAND_W;
        if constexpr (sizeof(TP) == 2) {
            const bf16x4 a = *(const MU_GLOBAL bf16x4*)(pp + i0);
            // the gradient is read once and never written: a non-temporal load
            // (A/B on the 8B-shaped AdamW set with contiguous chunks, same
            // process: +0.8 to +1.2 %)
            const bf16x4 b = __builtin_nontemporal_load((const MU_GLOBAL bf16x4*)(gg + i0));
#pragma unroll
            for (int e = 0; e < 4; ++e) { pv[k][e] = (float)a[e]; gv[k][e] = (float)b[e]; }
        } else {
            const f32x4 a = *(const MU_GLOBAL f32x4*)(pp + i0);
            const f32x4 b = __builtin_nontemporal_load((const MU_GLOBAL f32x4*)(gg + i0));
#pragma unroll
            for (int e = 0; e < 4; ++e) { pv[k][e] = a[e]; gv[k][e] = b[e]; }
        }
        mq[k] = *(const MU_GLOBAL f32x4*)(D.m + i0);
        vq[k] = *(const MU_GLOBAL f32x4*)(D.v + i0);
    }
    const float lr = D.lr, decay = D.lr * D.wd;
#pragma unroll
    for (int k = 0; k < RUNS; ++k) {
        const int64_t i0 = base + (int64_t)k * RSTEP * ADAMW_BAND_W;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float m = mq[k][e], v = vq[k][e];
            adamw1(pv[k][e], gv[k][e], m, v, A, lr, decay);
            mq[k][e] = m;
            vq[k][e] = v;
        }
        if constexpr (sizeof(TP) == 2) {
            bf16x4 po;
#pragma unroll
            for (int e = 0; e < 4; ++e) po[e] = (bf16)pv[k][e];
            *(MU_GLOBAL bf16x4*)((MU_GLOBAL TP*)D.param + i0) = po;
        } else {
            *(MU_GLOBAL f32x4*)((MU_GLOBAL TP*)D.param + i0) = f32x4{pv[k][0], pv[k][1], pv[k][2], pv[k][3]};
        }
        *(MU_GLOBAL f32x4*)(D.m + i0) = mq[k];
        *(MU_GLOBAL f32x4*)(D.v + i0) = vq[k];
    }
}

// Chunk c of the call: chunk q of tensor i. The grid is a multiple of 8 and
// xcd_remap gives each XCD one contiguous run of chunks. With the band layout
// that measured faster, and steadier, than consecutive chunks dealt
// round-robin over the XCDs: 16 x 256 tiles 5.73-5.76 against 5.65-5.66
// TB/s, 8 x 512 tiles in an 8192-wide view 5.83-5.85 against 5.71 and 5.31.
__global__ __launch_bounds__(NTHR) void k_adamw(AdamWArgs A) {
    const int64_t c = xcd_remap(blockIdx.x, gridDim.x);
    if (c >= A.total_chunks) return;
    const int i = __builtin_amdgcn_readfirstlane(find_tensor(A.prefix, A.n, c));
    const AdamWDesc D = A.descs[i];   // by value: held in registers, never re-read after a store
    const int64_t q = c - A.prefix[i];
    if (D.vec && q < D.numel / ADAMW_BAND * (ADAMW_BAND / ADAMW_CHUNK)) {
        if (D.dtype == DT_BF16) adamw_band_tile<bf16>(D, q, A);
        else adamw_band_tile<float>(D, q, A);
        return;
    }
    const int64_t base = q * ADAMW_CHUNK;
#pragma unroll
    for (int pass = 0; pass < ADAMW_CHUNK / (NTHR * 8); ++pass) {
        const int64_t i0 = base + (int64_t)pass * NTHR * 8 + threadIdx.x * 8;
        if (i0 >= D.numel) break;
        const int cnt = (int)min<int64_t>(8, D.numel - i0);
        if (D.dtype == DT_BF16) adamw8<bf16>(D, i0, cnt, A);
        else adamw8<float>(D, i0, cnt, A);
    }
}

// ---------------------------------------------------------------------------
// QK-Clip (MuonClip Optimizer page, "QK-Clip"). Workgroup c scales chunk k
// (QK_CHUNK elements) of segment i (a head's row block) by the segment's
// gamma: the smallest tau / max_logit over the query heads it follows that
// exceed tau, 1 if none does (then nothing is written). Chunks are laid out
// as AdamW's: bands of QK_BAND_ROWS rows of QK_BAND_W elements cut into
// QK_BAND_ROWS x QK_TILE_C tiles, the rest of a segment (and every chunk of
// a segment whose buffer does not allow vector accesses) in contiguous runs.
// Every load of a tile is issued before its first store. In-place bf16
// rescale of 2^29 elements, one process, two processes: 5.59-5.60 TB/s with
// contiguous chunks loaded, scaled and stored 16 bytes at a time, 5.62-5.63
// with all loads first, 5.92-5.93 for 32 x 256 tiles in a 4096-wide view
// (this layout), 6.00 for 8 x 512 tiles in an 8192-wide view (4096-element
// chunks).
// ---------------------------------------------------------------------------
template <typename TW>
__device__ __forceinline__ void qk_scale8(MU_GLOBAL TW* w, int cnt, bool vec, float g) {
    if (vec && cnt == 8) {
        if constexpr (sizeof(TW) == 2) {
            bf16x8 q = *(const MU_GLOBAL bf16x8*)w;
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = (bf16)(g * (float)q[e]);
            *(MU_GLOBAL bf16x8*)w = q;
        } else {
            f32x4 a = ((const MU_GLOBAL f32x4*)w)[0], b = ((const MU_GLOBAL f32x4*)w)[1];
            ((MU_GLOBAL f32x4*)w)[0] = g * a;
            ((MU_GLOBAL f32x4*)w)[1] = g * b;
        }
    } else {
        for (int e = 0; e < cnt; ++e) w[e] = from_f32<TW>(g * to_f32<TW>(w[e]));
    }
}

// Descriptor table upload: n16 16-byte chunks, then `tail` bytes, from
// pinned host memory (read over the host link) into the workspace. A kernel
// on the call's stream instead of an asynchronous host-to-device copy: on this
// platform the copy engine adds tens of microseconds to every call, which is
// most of a call on small parameter sets.
__global__ __launch_bounds__(NTHR) void k_table(const u32x4* src, u32x4* dst, int64_t n16, int tail) {
    const int64_t stride = (int64_t)gridDim.x * NTHR;
    for (int64_t i = (int64_t)blockIdx.x * NTHR + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
    if (blockIdx.x == 0 && (int)threadIdx.x < tail)
        ((unsigned char*)(dst + n16))[threadIdx.x] = ((const unsigned char*)(src + n16))[threadIdx.x];
}

constexpr int QK_BAND_ROWS = 32, QK_BAND_W = 4096, QK_TILE_C = 256;
constexpr int64_t QK_BAND = (int64_t)QK_BAND_ROWS * QK_BAND_W;
constexpr int QK_TILES_PER_BAND = QK_BAND_W / QK_TILE_C;
static_assert(QK_BAND_ROWS * QK_TILE_C == QK_CHUNK, "a band tile is one chunk");
static_assert(QK_BAND % QK_CHUNK == 0, "bands end on chunk boundaries");

// Tile q of a segment whose buffer is 16-byte aligned: 16-byte vectors, each
// thread owning one vector in each of QK_BAND_ROWS / RSTEP rows.
template <typename TW>
__device__ __forceinline__ void qk_band_tile(MU_GLOBAL TW* w, int64_t q, float g) {
    constexpr int EPT = 16 / (int)sizeof(TW);   // elements per vector
    constexpr int TPR = QK_TILE_C / EPT;        // threads per tile row
    constexpr int RSTEP = NTHR / TPR;
    constexpr int RUNS = QK_BAND_ROWS / RSTEP;
    static_assert(NTHR % TPR == 0 && QK_BAND_ROWS % RSTEP == 0, "tile rows split evenly over the threads");
    const int64_t band = q / QK_TILES_PER_BAND;
    const int tj = (int)(q - band * QK_TILES_PER_BAND);
    const int rr = threadIdx.x / TPR, cc = (threadIdx.x % TPR) * EPT;
    MU_GLOBAL TW* p = w + band * QK_BAND + (int64_t)rr * QK_BAND_W + tj * QK_TILE_C + cc;
    if constexpr (sizeof(TW) == 2) {
        bf16x8 v[RUNS];
#pragma unroll
        for (int k = 0; k < RUNS; ++k) v[k] = *(const MU_GLOBAL bf16x8*)(p + (int64_t)k * RSTEP * QK_BAND_W);
#pragma unroll
        for (int k = 0; k < RUNS; ++k) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[k][e] = (bf16)(g * (float)v[k][e]);
            *(MU_GLOBAL bf16x8*)(p + (int64_t)k * RSTEP * QK_BAND_W) = v[k];
        }
    } else {
        f32x4 v[RUNS];
#pragma unroll
        for (int k = 0; k < RUNS; ++k) v[k] = *(const MU_GLOBAL f32x4*)(p + (int64_t)k * RSTEP * QK_BAND_W);
#pragma unroll
        for (int k = 0; k < RUNS; ++k) *(MU_GLOBAL f32x4*)(p + (int64_t)k * RSTEP * QK_BAND_W) = g * v[k];
    }
}

__global__ __launch_bounds__(NTHR) void k_qkclip(QkArgs A) {
    const int64_t c = xcd_remap(blockIdx.x, gridDim.x);
    if (c >= A.total_chunks) return;
    const int i = __builtin_amdgcn_readfirstlane(find_tensor(A.prefix, A.n, c));
    const QkSeg S = A.segs[i];   // by value: held in registers, never re-read after a store
    const int64_t q = c - A.prefix[i];
    const int64_t base = q * QK_CHUNK;
    float g = 1.f;
    for (int j = 0; j < S.nml; ++j) {
        const float ml = *gp(S.ml + j);
        if (ml > A.tau) g = fminf(g, A.tau / ml);   // false for NaN; 0 for +inf
    }
    if (base == 0 && S.gamma_out && threadIdx.x == 0) *gp(S.gamma_out) = g;
    if (g == 1.f) return;
    if (S.vec && q < S.numel / QK_BAND * (QK_BAND / QK_CHUNK)) {
        if (S.dtype == DT_BF16) qk_band_tile<bf16>((MU_GLOBAL bf16*)S.w, q, g);
        else qk_band_tile<float>((MU_GLOBAL float*)S.w, q, g);
        return;
    }
#pragma unroll
    for (int pass = 0; pass < QK_CHUNK / (NTHR * 8); ++pass) {
        const int64_t i0 = base + (int64_t)pass * NTHR * 8 + threadIdx.x * 8;
        if (i0 >= S.numel) break;
        const int cnt = (int)min<int64_t>(8, S.numel - i0);
        if (S.dtype == DT_BF16) qk_scale8<bf16>((MU_GLOBAL bf16*)S.w + i0, cnt, S.vec != 0, g);
        else qk_scale8<float>((MU_GLOBAL float*)S.w + i0, cnt, S.vec != 0, g);
    }
}

}  // namespace

hipError_t launch_table_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const unsigned grid = (unsigned)std::min<size_t>(64, std::max<size_t>(1, (n16 + NTHR - 1) / NTHR));
    hipLaunchKernelGGL(k_table, dim3(grid), dim3(NTHR), 0, s, (const u32x4*)src, (u32x4*)dst, (int64_t)n16,
                       (int)(bytes % 16));
    return hipGetLastError();
}

// Grids of the streaming kernels are rounded up to a multiple of 8 (the
// extra workgroups exit at once) so that xcd_remap gives every XCD one
// contiguous run of tiles or chunks: prep measured 9 % faster that way than
// with consecutive workgroups spread round-robin over the XCDs.
inline unsigned grid8(int64_t n) { return (unsigned)((n + 7) / 8 * 8); }

hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    dim3 grid(grid8(a.total_tiles)), block(NTHR);
    if (a.src_dtype == DT_BF16) {
        if (a.ns_dtype == DT_BF16) hipLaunchKernelGGL((k_prep<bf16, bf16>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_prep<bf16, float>), grid, block, 0, s, a);
    } else {
        if (a.ns_dtype == DT_BF16) hipLaunchKernelGGL((k_prep<float, bf16>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_prep<float, float>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_norm(const NormArgs& a, hipStream_t s) {
    if (a.nprobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_norm, dim3(a.nprobs), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_rescale(const RescaleArgs& a, hipStream_t s) {
    if (a.nprobs <= 0) return hipSuccess;
    // enough workgroups to stream one flagged problem at full rate, at most 8
    // per compute unit; the exit path reads ceil(nprobs / 256) exponents each
    const int64_t per_wg = (int64_t)NTHR * 64;   // elements of one problem per workgroup
    const unsigned grid = (unsigned)std::min<int64_t>(2048, grid8(std::max<int64_t>(8, a.max_elems / per_wg)));
    if (a.ns_dtype == DT_BF16) hipLaunchKernelGGL(k_rescale<bf16>, dim3(grid), dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL(k_rescale<float>, dim3(grid), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_finish(const FinishArgs& a, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    dim3 grid(grid8(a.total_tiles)), block(NTHR);
    if (a.src_dtype == DT_BF16) {
        if (a.ns_dtype == DT_BF16) hipLaunchKernelGGL((k_finish<bf16, bf16>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_finish<bf16, float>), grid, block, 0, s, a);
    } else {
        if (a.ns_dtype == DT_BF16) hipLaunchKernelGGL((k_finish<float, bf16>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_finish<float, float>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamWArgs& a, hipStream_t s) {
    if (a.total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_adamw, dim3(grid8(a.total_chunks)), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_qkclip(const QkArgs& a, hipStream_t s) {
    if (a.total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_qkclip, dim3(grid8(a.total_chunks)), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

}  // namespace mu
