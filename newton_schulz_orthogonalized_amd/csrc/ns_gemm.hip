// Newton-Schulz products on MFMA (gfx950).
//
// One Newton-Schulz step on the wide X (m x n, m <= n) is
//     A  = X X^T                       (Gram, m x m, symmetric)
//     B  = b A + c A A^T               (only for steps with a quintic term)
//     X' = a X + b A X   or   a X + B X
// (MuonClip Optimizer page, section "Newton-Schulz Orthogonalization", gives
// the cubic step with a = 1.5, b = -0.5, written as X (X^T X), which equals
// (X X^T) X; the Gram side is kept on the short dimension.)
//
// All products are grouped GEMMs over every (matrix, head) problem of a call:
// one launch per mode covers all problems, each workgroup finds its problem
// by binary search over a tile prefix, and workgroup ids are remapped so that
// neighbouring tiles run on the same XCD (shared L2).
//
// Every product is "NT", C = P Q^T with both operands K-contiguous: the Gram
// X X^T reads X twice; the apply A X reads A and the transposed copy X^T that
// the previous step's epilogue (or the prep kernel) wrote. Gram products only
// compute tiles on or above the diagonal and also store the transposed tile.
//
// bf16: v_mfma_f32_16x16x32_bf16, fp32 accumulation, 256x256 or 128x128
// workgroup tiles, BK = 64, 4 waves in 2x2 (128x128 per wave for 256 tiles),
// operands moved with direct-to-LDS loads into two LDS stages.
// fp32: v_mfma_f32_16x16x4_f32, 64x64 tiles, BK = 32.
//
// Epilogue: accumulators are staged per wave through LDS in 16-row strips,
// then stored with 16-byte row-major accesses and, for transposed outputs
// (Gram mirror, X'^T, or a tall weight), a column pass. It applies the fold
// 1/||U||_F of the first step (so the normalised X0 is never materialised), the
// step coefficients, and on the last step the decoupled-weight-decay update
// W <- W - lr*wd*W - lr*scale*O straight into the parameter.
#include "common.hpp"
#include "launch.hpp"

namespace mu {

namespace {

constexpr int NTHR = 256;

// XOR swizzle of the eight 16-byte chunks of a 128-byte K-contiguous LDS row:
// physical chunk = logical chunk ^ (row & 7). A fragment read (16 rows at one
// logical chunk) then runs at the rate of a linear ds_read_b128 on gfx950, as
// measured; variants that also flip on row bit 3 ran about 1.45x slower.
__device__ __forceinline__ int swz_k(int r) { return r & 7; }


// ---------------------------------------------------------------------------
// Tile enumeration
// ---------------------------------------------------------------------------
__device__ __forceinline__ void upper_tile(int local, int T, int& ti, int& tj) {
    int i = 0;
    while (local >= T - i) { local -= T - i; ++i; }
    ti = i;
    tj = i + local;
}

// Groups of four tile rows, column-major inside a group: 4 A panels and a
// run of X panels are shared by the workgroups running together.
__device__ __forceinline__ void apply_tile(int local, int TM, int TN, int& ti, int& tj) {
    constexpr int G = 4;
    const int per_group = G * TN;
    const int g = local / per_group;
    const int w = local - g * per_group;
    const int gm = min(G, TM - g * G);
    ti = g * G + w % gm;
    tj = w / gm;
}

// ---------------------------------------------------------------------------
// U-space write of 8 consecutive values (update or plain output); row ur,
// columns uc0 .. uc0+7 (uc0 a multiple of 8), clipped to the head block.
// ---------------------------------------------------------------------------
template <typename TS>
__device__ __forceinline__ void emit_u8(const GemmArgs& A, const NsProb& P, int ur, int uc0, const float* v) {
    if (ur >= P.hr || uc0 >= P.hc) return;
    const int valid = min(8, P.hc - uc0);
    const int64_t off = (int64_t)ur * P.ld + uc0;
    const bool vec = P.vec != 0;
    if (P.oout) {
        float* o = P.oout + off;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < valid) o[e] = v[e];
    }
    if (A.with_update) {
        TS* w = (TS*)P.param + off;
        const float decay = A.lr * A.wd, step = A.lr * P.scale;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int cnt = min(4, valid - 4 * h);
            if (cnt <= 0) break;
            float x[4];
            if (vec && cnt == 4) {
                if constexpr (sizeof(TS) == 2) {
                    bf16x4 q = *(const bf16x4*)(w + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (float)q[e];
                } else {
                    f32x4 q = *(const f32x4*)(w + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = q[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = e < cnt ? to_f32<TS>(w[4 * h + e]) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (x[e] - decay * x[e]) - step * v[4 * h + e];
            if (vec && cnt == 4) {
                if constexpr (sizeof(TS) == 2) {
                    bf16x4 q;
#pragma unroll
                    for (int e = 0; e < 4; ++e) q[e] = (bf16)x[e];
                    *(bf16x4*)(w + 4 * h) = q;
                } else {
                    *(f32x4*)(w + 4 * h) = f32x4{x[0], x[1], x[2], x[3]};
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < cnt) w[4 * h + e] = from_f32<TS>(x[e]);
            }
        }
    } else {
        TS* o = (TS*)P.out + off;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < valid) o[e] = from_f32<TS>(v[e]);
    }
}

template <typename TX>
__device__ __forceinline__ void load8(const TX* p, float* v) {
    if constexpr (sizeof(TX) == 2) {
        bf16x8 q = *gp((const bf16x8*)p);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)q[e];
    } else {
        f32x4 a = gp((const f32x4*)p)[0], b = gp((const f32x4*)p)[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
    }
}
template <typename TX>
__device__ __forceinline__ void store8(TX* p, const float* v) {
    if constexpr (sizeof(TX) == 2) {
        bf16x8 q;
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (bf16)v[e];
        *gp((bf16x8*)p) = q;
    } else {
        gp((f32x4*)p)[0] = f32x4{v[0], v[1], v[2], v[3]};
        gp((f32x4*)p)[1] = f32x4{v[4], v[5], v[6], v[7]};
    }
}

// Eight consecutive X-space values of a bf16 or float buffer, held raw.
template <typename TX>
struct Vec8;
template <>
struct Vec8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *gp((const bf16x8*)p); }
    __device__ __forceinline__ float get(int e) const { return (float)v[e]; }
};
template <>
struct Vec8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = gp((const f32x4*)p)[0];
        b = gp((const f32x4*)p)[1];
    }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Order LDS accesses of this wave (a wave's LDS operations complete in issue
// order; only compiler reordering has to be prevented).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Epilogue shared by the bf16 and fp32 kernels. The accumulator layout is the
// 16x16 MFMA one: lane l holds C[4*(l>>4) + e][l & 15] of each fragment.
// `st` is this wave's LDS strip of 16 x (F*16 + 4) floats, not otherwise in
// use; each wave stages only its own strip, so syncs are wave-local. In the
// apply modes the X values of the whole tile are requested before the first
// strip, so their latency is paid once.
// ---------------------------------------------------------------------------
template <typename TX, typename TS, int F>
__device__ __forceinline__ void epilogue(const GemmArgs& A, const NsProb& P, int ti, int tj, int TS_, int wm0,
                                         int wn0, f32x4 (&acc)[F][F], float* st) {
    constexpr int WT = F * 16;
    constexpr int SP = WT + 4;
    constexpr int PASSES = (16 * WT / 8) / 64;
    const int lane = threadIdx.x & 63;
    const int mode = A.mode;
    const float f = A.first ? P.fold[0] : 1.f;
    const bool gram = mode == GM_GRAM || mode == GM_GRAM2;
    const bool apply = !gram;
    const bool mirror = gram && ti != tj;
    const bool last = mode == GM_APPLY_LAST;
    // transposed outputs: the Gram mirror, X'^T for the next apply, or the
    // parameter of a tall block on the last step
    const bool trans_out = mirror || (apply && !last) || (last && P.tall);
    const int row_base = ti * TS_ + wm0, col_base = tj * TS_ + wn0;
    const int mp = P.mp, np = P.np;
    const float cb_eff = A.use_b ? 1.f : A.cb;
    TX* gdst = (TX*)(mode == GM_GRAM ? P.a : P.b);
    const TX* xsrc = (const TX*)P.x[A.src];
    TX* xdst = (TX*)P.x[A.src ^ 1];
    TX* xtdst = (TX*)P.xt[A.src ^ 1];

    Vec8<TX> xv[F][PASSES];
    if (apply) {
#pragma unroll
        for (int fm = 0; fm < F; ++fm)
#pragma unroll
            for (int pass = 0; pass < PASSES; ++pass) {
                const int idx = pass * 64 + lane;
                const int rr = idx / (WT / 8), c8 = (idx % (WT / 8)) * 8;
                xv[fm][pass].load(xsrc + (int64_t)(row_base + fm * 16 + rr) * np + col_base + c8);
            }
    }

#pragma clang loop unroll(full)
    for (int fm = 0; fm < F; ++fm) {
        wave_lds_sync();
#pragma unroll
        for (int fn = 0; fn < F; ++fn)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(4 * (lane >> 4) + e) * SP + fn * 16 + (lane & 15)] = acc[fm][fn][e];
        wave_lds_sync();
        // row-major pass: 8 consecutive columns per lane
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int idx = pass * 64 + lane;
            const int rr = idx / (WT / 8), c8 = (idx % (WT / 8)) * 8;
            float v[8];
            {
                const f32x4 a = *(const f32x4*)(st + rr * SP + c8);
                const f32x4 b = *(const f32x4*)(st + rr * SP + c8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
            }
            const int r = row_base + fm * 16 + rr, c = col_base + c8;
            if (mode == GM_GRAM) {
                const float s = f * f;
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] *= s;
                store8<TX>(gdst + (int64_t)r * mp + c, v);
            } else if (mode == GM_GRAM2) {
                float a8[8];
                load8<TX>((const TX*)P.a + (int64_t)r * mp + c, a8);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = A.cb * a8[e] + A.cc * v[e];
                store8<TX>(gdst + (int64_t)r * mp + c, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = f * (A.ca * xv[fm][pass].get(e) + cb_eff * v[e]);
                if (!last) store8<TX>(xdst + (int64_t)r * np + c, v);
                else if (!P.tall) emit_u8<TS>(A, P, r, c, v);
            }
            if (trans_out) {
                *(f32x4*)(st + rr * SP + c8) = f32x4{v[0], v[1], v[2], v[3]};
                *(f32x4*)(st + rr * SP + c8 + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
        }
        if (trans_out) {
            wave_lds_sync();
            // column pass: lane takes one column and 8 consecutive rows
#pragma unroll
            for (int pass = 0; pass < (2 * WT) / 64; ++pass) {
                const int idx = pass * 64 + lane;
                const int jj = idx >> 1, half = idx & 1;
                float v[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = st[(half * 8 + t) * SP + jj];
                const int r = row_base + fm * 16 + half * 8, c = col_base + jj;
                if (mirror) store8<TX>(gdst + (int64_t)c * mp + r, v);
                else if (!last) store8<TX>(xtdst + (int64_t)c * mp + r, v);
                else emit_u8<TS>(A, P, c, r, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 kernel
//
// K loop, BK = 64, two LDS stages (separate arrays, so the compiler's wait
// insertion can tell a direct-to-LDS load into one stage from reads of the
// other). Operand tiles move HBM/L2 -> LDS with global_load_lds_dwordx4: each
// instruction writes 64 lanes x 16 B contiguously (LDS base + lane*16), so the
// XOR swizzle is applied by permuting the global addresses the lanes load.
//
// Iteration kt (stage S holds tile kt; fragments F0 = k-half 0 of tile kt are
// already in registers):
//   phase 1: read F1 (k-half 1 of tile kt) from stage S   | MFMAs on F0
//   phase 2: first MFMAs on F1; wait own loads; barrier    | (tile kt+1 ready,
//            all waves done with stage S)
//            DMA tile kt+2 into stage S; read F0 of tile kt+1 from stage S^1
//            | remaining MFMAs on F1
// One barrier per K step; loads run ~1.25 steps ahead of their use.
// ---------------------------------------------------------------------------
#define LDSP __attribute__((address_space(3)))

template <int N>
struct Stage {
    static constexpr int value = N;
};

// s_waitcnt with only vmcnt (gfx9 encoding: vmcnt[3:0] bits 3:0, [5:4] bits 15:14)
#define MU_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
#define MU_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8) | (3 << 14))

template <int TS, bool SYM, typename TSRC>
__global__ __launch_bounds__(NTHR) void k_gemm_bf16(GemmArgs A) {
    constexpr int BK = 64;
    constexpr int WT = TS / 2;
    constexpr int F = WT / 16;
    constexpr int LA = TS * BK;           // elements per operand tile
    constexpr int NBLK = LA * 2 / 1024;   // 1 KB direct-load blocks per operand tile
    constexpr int BPW = NBLK / 4;         // blocks per wave per operand
    __shared__ __attribute__((aligned(1024))) bf16 sA0[LA];
    __shared__ __attribute__((aligned(1024))) bf16 sB0[LA];
    __shared__ __attribute__((aligned(1024))) bf16 sA1[LA];
    __shared__ __attribute__((aligned(1024))) bf16 sB1[LA];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= A.total_tiles) return;
    const int p = find_prob(A.prefix, A.nprobs, wg);
    const NsProb& P = A.probs[p];
    const int local = wg - A.prefix[p];
    const int mode = A.mode;
    int ti, tj;
    if (SYM) upper_tile(local, P.mp / TS, ti, tj);
    else apply_tile(local, P.mp / TS, P.np / TS, ti, tj);

    // C = P Q^T, both operands with K contiguous
    const bf16 *pm, *qm;
    int ldp, ldq, K;
    if (mode == GM_GRAM) {
        pm = qm = (const bf16*)P.x[A.src]; ldp = ldq = P.np; K = P.np;
    } else if (mode == GM_GRAM2) {
        pm = qm = (const bf16*)P.a; ldp = ldq = P.mp; K = P.mp;
    } else {
        pm = (const bf16*)(A.use_b ? P.b : P.a); ldp = P.mp;
        qm = (const bf16*)P.xt[A.src]; ldq = P.mp; K = P.mp;
    }
    const bf16* pt = pm + (int64_t)ti * TS * ldp;
    const bf16* qt = qm + (int64_t)tj * TS * ldq;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;

    // Direct-load sources. Block b = s*4 + wave of an operand tile is 1 KB =
    // rows 8b .. 8b+7; lane -> row 8b + lane/8 and physical chunk lane%8, which
    // holds logical chunk (lane%8) ^ swz_k(row) = (lane%8) ^ (lane/8). Block s
    // is the block-0 address plus s*32 rows. Every source address is a
    // wave-uniform base (scalar registers) plus a fixed 32-bit lane offset.
    const int ca = (lane & 7) ^ (lane >> 3);
    const uint32_t offA = (uint32_t)((8 * wave + (lane >> 3)) * ldp + ca * 8) * 2u;
    const uint32_t offB = (uint32_t)((8 * wave + (lane >> 3)) * ldq + ca * 8) * 2u;
    const int64_t strideA = (int64_t)32 * ldp, strideB = (int64_t)32 * ldq;

    // direct load i of K step kt into stage S: i < BPW loads A block s = i,
    // otherwise B block s = i - BPW
    auto dma_one = [&](auto st, int kt, int i) {
        constexpr int S = decltype(st)::value;
        const bool isA = i < BPW;
        const int s = isA ? i : i - BPW;
        bf16* dst = isA ? (S ? sA1 : sA0) : (S ? sB1 : sB0);
        const char* src = isA ? (const char*)(pt + kt * BK) + s * strideA * 2 + offA
                              : (const char*)(qt + kt * BK) + s * strideB * 2 + offB;
        __builtin_amdgcn_global_load_lds((const void*)src, (LDSP void*)(dst + (s * 4 + wave) * 512), 16, 0, 0);
    };
    auto dma = [&](auto st, int kt) {
#pragma unroll
        for (int i = 0; i < 2 * BPW; ++i) dma_one(st, kt, i);
    };

    // Fragment reads: lane reads row (lane&15) of a 16-row fragment at logical
    // chunk kh*4 + lane/16, stored at that ^ swz_k(row) = ^ (lane&7).
    const int swl = lane & 7;
    const int offk0 = (lane & 15) * BK + (((lane >> 4) ^ swl) << 3);
    const int offk1 = (lane & 15) * BK + (((4 + (lane >> 4)) ^ swl) << 3);
    auto read_a = [&](auto st, int kh, int fm) -> bf16x8 {
        constexpr int S = decltype(st)::value;
        const bf16* as = S ? sA1 : sA0;
        return *(const bf16x8*)(as + (wm0 + fm * 16) * BK + (kh ? offk1 : offk0));
    };
    auto read_b = [&](auto st, int kh, int fn) -> bf16x8 {
        constexpr int S = decltype(st)::value;
        const bf16* bs = S ? sB1 : sB0;
        return *(const bf16x8*)(bs + (wn0 + fn * 16) * BK + (kh ? offk1 : offk0));
    };

    f32x4 acc[F][F];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 a0[F], b0[F], a1[F], b1[F];
    const int KT = K / BK;

    dma(Stage<0>{}, 0);
    MU_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    dma(Stage<1>{}, 1);
#pragma unroll
    for (int fn = 0; fn < F; ++fn) b0[fn] = read_b(Stage<0>{}, 0, fn);
#pragma unroll
    for (int fm = 0; fm < F; ++fm) a0[fm] = read_a(Stage<0>{}, 0, fm);

    // The body is emitted in the exact issue order wanted and fenced with
    // sched_barrier, so the MFMA stream is never starved: with one wave per
    // SIMD the matrix core drains within a couple of MFMAs of any gap.
    // Phase 1: 2F groups of {one k-half-1 fragment read, F/2 MFMAs on k-half 0}
    //          (B fragments first: the first MFMAs of phase 2 need all of them).
    // Phase 2: HEAD rows of MFMAs on k-half 1; wait own loads; barrier; then 2F
    //          groups of {a direct load of tile kt+2, one k-half-0 read of tile
    //          kt+1, the remaining k-half-1 MFMAs}.
    // K/BK is even (K is a multiple of the tile >= 128) and the body is
    // unrolled over the two stages, so every LDS access names one array; the
    // prefetch index is clamped, so the last two prefetches reload the final
    // tile into a stage nobody reads again instead of branching.
    constexpr int HEAD = F / 4 > 0 ? F / 4 : 1;
    constexpr int G = 2 * F;                 // fragment reads per k-half
    constexpr int NMF2 = (F - HEAD) * F;     // MFMAs after the barrier
    constexpr int NDMA = 2 * BPW;            // direct loads per K step
    auto mma1 = [&](int idx, const bf16x8 (&af)[F], const bf16x8 (&bfv)[F]) {
        const int fm = idx / F, fn = idx % F;
#pragma unroll
        for (int r = 0; r < F; ++r)
#pragma unroll
            for (int c = 0; c < F; ++c)
                if (r == fm && c == fn)
                    acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bfv[c], acc[r][c], 0, 0, 0);
    };
    auto half = [&](auto st, int kt) {
        constexpr int S = decltype(st)::value;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g < F) b1[g] = read_b(st, 1, g);
            else a1[g - F] = read_a(st, 1, g - F);
#pragma unroll
            for (int j = 0; j < F * F / G; ++j) mma1(g * (F * F / G) + j, a0, b0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < HEAD * F; ++j) mma1(j, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        MU_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        const int kn = min(kt + 2, KT - 1);
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int i = 0; i < NDMA; ++i)
                if (i * G / NDMA == g) dma_one(st, kn, i);
            if (g < F) b0[g] = read_b(Stage<1 - S>{}, 0, g);
            else a0[g - F] = read_a(Stage<1 - S>{}, 0, g - F);
#pragma unroll
            for (int j = g * NMF2 / G; j < (g + 1) * NMF2 / G; ++j) mma1(HEAD * F + j, a1, b1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (int kt = 0; kt < KT; kt += 2) {
        half(Stage<0>{}, kt);
        half(Stage<1>{}, kt + 1);
    }
    __syncthreads();
    // epilogue staging: waves 0-1 in stage 0's A array, waves 2-3 in its B array
    float* st = (float*)((wave < 2) ? sA0 : sB0) + (wave & 1) * 16 * (WT + 4);
    epilogue<bf16, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, st);
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64x64 tiles, BK = 32, v_mfma_f32_16x16x4_f32, operands staged
// through registers into padded LDS rows. Within a block of 16 k, lane l holds
// k = 4*(l>>4) + s in MFMA s for both operands (any permutation of k shared by
// both operands leaves the sum unchanged).
// ---------------------------------------------------------------------------
template <bool SYM, typename TSRC>
__global__ __launch_bounds__(NTHR) void k_gemm_f32(GemmArgs A) {
    constexpr int TS = 64, BK = 32, WT = 32, F = 2;
    constexpr int SPK = BK + 4;
    constexpr int LA = TS * SPK;
    __shared__ __attribute__((aligned(16))) float smem[2 * 2 * LA];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= A.total_tiles) return;
    const int p = find_prob(A.prefix, A.nprobs, wg);
    const NsProb& P = A.probs[p];
    const int local = wg - A.prefix[p];
    const int mode = A.mode;
    int ti, tj;
    if (SYM) upper_tile(local, P.mp / TS, ti, tj);
    else apply_tile(local, P.mp / TS, P.np / TS, ti, tj);

    const float *pm, *qm;
    int ldp, ldq, K;
    if (mode == GM_GRAM) {
        pm = qm = (const float*)P.x[A.src]; ldp = ldq = P.np; K = P.np;
    } else if (mode == GM_GRAM2) {
        pm = qm = (const float*)P.a; ldp = ldq = P.mp; K = P.mp;
    } else {
        pm = (const float*)(A.use_b ? P.b : P.a); ldp = P.mp;
        qm = (const float*)P.xt[A.src]; ldq = P.mp; K = P.mp;
    }
    const float* pt = pm + (int64_t)ti * TS * ldp;
    const float* qt = qm + (int64_t)tj * TS * ldq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;

    f32x4 ga[2], gb[2];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int q = s * NTHR + tid;
            ga[s] = *gp((const f32x4*)(pt + (int64_t)(q >> 3) * ldp + k0 + (q & 7) * 4));
            gb[s] = *gp((const f32x4*)(qt + (int64_t)(q >> 3) * ldq + k0 + (q & 7) * 4));
        }
    };
    auto sstore = [&](int stage) {
        float* as = smem + stage * 2 * LA;
        float* bs = as + LA;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int q = s * NTHR + tid;
            *(f32x4*)(as + (q >> 3) * SPK + (q & 7) * 4) = ga[s];
            *(f32x4*)(bs + (q >> 3) * SPK + (q & 7) * 4) = gb[s];
        }
    };

    f32x4 acc[F][F];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) gload(kt + 1);
        const float* as = smem + (kt & 1) * 2 * LA;
        const float* bs = as + LA;
#pragma unroll
        for (int kb = 0; kb < BK / 16; ++kb) {
            f32x4 af[F], bfv[F];
            const int kk = kb * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int fm = 0; fm < F; ++fm) af[fm] = *(const f32x4*)(as + (wm0 + fm * 16 + (lane & 15)) * SPK + kk);
#pragma unroll
            for (int fn = 0; fn < F; ++fn) bfv[fn] = *(const f32x4*)(bs + (wn0 + fn * 16 + (lane & 15)) * SPK + kk);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int fm = 0; fm < F; ++fm)
#pragma unroll
                    for (int fn = 0; fn < F; ++fn)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[fm][s], bfv[fn][s], acc[fm][fn], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore((kt + 1) & 1);
        __syncthreads();
    }
    epilogue<float, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, smem + wave * 16 * (WT + 4));
}

template <int TS, bool SYM>
hipError_t launch_bf16_t(const GemmArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)((a.total_tiles + 7) / 8 * 8);
    if (a.src_dtype == DT_BF16) hipLaunchKernelGGL((k_gemm_bf16<TS, SYM, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL((k_gemm_bf16<TS, SYM, float>), dim3(grid), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    const bool sym = a.mode == GM_GRAM || a.mode == GM_GRAM2;
    if (tile == 256) return sym ? launch_bf16_t<256, true>(a, s) : launch_bf16_t<256, false>(a, s);
    if (tile == 128) return sym ? launch_bf16_t<128, true>(a, s) : launch_bf16_t<128, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    const bool sym = a.mode == GM_GRAM || a.mode == GM_GRAM2;
    const unsigned grid = (unsigned)((a.total_tiles + 7) / 8 * 8);
    if (a.src_dtype == DT_BF16) {
        if (sym) hipLaunchKernelGGL((k_gemm_f32<true, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f32<false, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
    } else {
        if (sym) hipLaunchKernelGGL((k_gemm_f32<true, float>), dim3(grid), dim3(NTHR), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f32<false, float>), dim3(grid), dim3(NTHR), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mu
