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
//   Gram modes ("NT"): C = P Q^T with both operands K-contiguous rows. Only
//   tiles on or above the diagonal are computed; the epilogue also stores the
//   transposed tile, so A is written whole.
//   Apply mode ("NN"): C = P X with X row-major (N-contiguous). The X tile is
//   staged in LDS as stored and read with ds_read_b64_tr_b16, which hands each
//   lane four rows of one column: the MFMA B operand without any transposed
//   copy of X in memory.
//
// bf16: v_mfma_f32_16x16x32_bf16, fp32 accumulation, 256x256 or 128x128
// workgroup tiles, BK = 64, 4 waves in 2x2, LDS double buffer.
// fp32: v_mfma_f32_16x16x4_f32, 64x64 tiles, BK = 32.
//
// Epilogue: accumulators are staged per wave through LDS in 16-row strips,
// then stored with 16-byte row-major accesses (and, for the Gram mirror or a
// tall weight, a column pass for the transposed store). It applies the fold
// 1/||U||_F of the first step (so the normalised X0 is never materialised), the
// step coefficients, and on the last step the decoupled-weight-decay update
// W <- W - lr*wd*W - lr*scale*O straight into the parameter.
#include "common.hpp"
#include "launch.hpp"

namespace mu {

namespace {

constexpr int NTHR = 256;

// XOR swizzle of the eight 16-byte chunks of a 128-byte K-contiguous LDS row.
// Any 8 consecutive rows get distinct chunks, and any 16 consecutive rows get
// distinct (row parity, chunk) pairs, so ds_read_b128 of 16 rows at one logical
// chunk touches every bank once whether the LDS serves 128 or 256 bytes/clock.
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// XOR swizzle of the 32-byte groups of an N-contiguous LDS row (X tile of the
// apply). A transposed read touches rows 8g + {0..3} (+4) for g = 0..3 at one
// logical group; this maps rows {0..3, 8..11} to eight distinct groups.
__device__ __forceinline__ int swz_n(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

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

// ---------------------------------------------------------------------------
// Epilogue shared by the bf16 and fp32 kernels. The accumulator layout is the
// 16x16 MFMA one: lane l holds C[4*(l>>4) + e][l & 15] of each fragment.
// `stage` must hold 4 waves x 16 x (F*16 + 4) floats and not be in use.
// ---------------------------------------------------------------------------
template <typename TX, typename TS, int F>
__device__ __forceinline__ void epilogue(const GemmArgs& A, const NsProb& P, int ti, int tj, int TS_, int wm0,
                                int wn0, f32x4 (&acc)[F][F], float* stage) {
    constexpr int WT = F * 16;
    constexpr int SP = WT + 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float* st = stage + wave * 16 * SP;
    const int mode = A.mode;
    const float f = A.first ? P.fold[0] : 1.f;
    const bool gram = mode == GM_GRAM || mode == GM_GRAM2;
    const bool mirror = gram && ti != tj;
    const bool last = mode == GM_APPLY_LAST;
    const bool trans_out = mirror || (last && P.tall);
    const int row_base = ti * TS_ + wm0, col_base = tj * TS_ + wn0;
    const int mp = P.mp, np = P.np;
    const float cb_eff = A.use_b ? 1.f : A.cb;
    TX* gdst = (TX*)(mode == GM_GRAM ? P.a : P.b);
    const TX* xsrc = (const TX*)P.x[A.src];
    TX* xdst = (TX*)P.x[A.src ^ 1];

    for (int fm = 0; fm < F; ++fm) {
        __syncthreads();
        // static register indices: one uniform branch per fragment row
#pragma unroll
        for (int i = 0; i < F; ++i) {
            if (i == fm) {
#pragma unroll
                for (int fn = 0; fn < F; ++fn)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[(4 * (lane >> 4) + e) * SP + fn * 16 + (lane & 15)] = acc[i][fn][e];
            }
        }
        __syncthreads();
        // row-major pass: 8 consecutive columns per lane
#pragma unroll
        for (int pass = 0; pass < (16 * WT / 8) / 64; ++pass) {
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
                float x8[8];
                load8<TX>(xsrc + (int64_t)r * np + c, x8);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = f * (A.ca * x8[e] + cb_eff * v[e]);
                if (!last) store8<TX>(xdst + (int64_t)r * np + c, v);
                else if (!P.tall) emit_u8<TS>(A, P, r, c, v);
            }
            if (trans_out) {
                *(f32x4*)(st + rr * SP + c8) = f32x4{v[0], v[1], v[2], v[3]};
                *(f32x4*)(st + rr * SP + c8 + 4) = f32x4{v[4], v[5], v[6], v[7]};
            }
        }
        if (trans_out) {
            __syncthreads();
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
                else emit_u8<TS>(A, P, c, r, v);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
template <int TS, bool NN, typename TSRC>
__global__ __launch_bounds__(NTHR) void k_gemm_bf16(GemmArgs A) {
    constexpr int BK = 64;
    constexpr int WT = TS / 2;
    constexpr int F = WT / 16;
    constexpr int LA = TS * BK;                     // elements per operand tile
    constexpr int LOADS = LA / 8 / NTHR;            // 16-byte chunks per thread per operand
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * LA];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= A.total_tiles) return;
    const int p = find_prob(A.prefix, A.nprobs, wg);
    const NsProb& P = A.probs[p];
    const int local = wg - A.prefix[p];
    const int mode = A.mode;
    int ti, tj;
    if (NN) apply_tile(local, P.mp / TS, P.np / TS, ti, tj);
    else upper_tile(local, P.mp / TS, ti, tj);

    const bf16 *pm, *qm;
    int ldp, ldq, K;
    if (mode == GM_GRAM) {
        pm = qm = (const bf16*)P.x[A.src]; ldp = ldq = P.np; K = P.np;
    } else if (mode == GM_GRAM2) {
        pm = qm = (const bf16*)P.a; ldp = ldq = P.mp; K = P.mp;
    } else {
        pm = (const bf16*)(A.use_b ? P.b : P.a); ldp = P.mp;
        qm = (const bf16*)P.x[A.src]; ldq = P.np; K = P.mp;
    }
    const bf16* pt = pm + (int64_t)ti * TS * ldp;
    const bf16* qt = NN ? qm + tj * TS : qm + (int64_t)tj * TS * ldq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;

    u32x4 ga[LOADS], gb[LOADS];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int s = 0; s < LOADS; ++s) {
            const int q = s * NTHR + tid;
            ga[s] = *gp((const u32x4*)(pt + (int64_t)(q >> 3) * ldp + k0 + (q & 7) * 8));
            if (NN) {
                const int k = q / (TS / 8), c16 = q % (TS / 8);
                gb[s] = *gp((const u32x4*)(qt + (int64_t)(k0 + k) * ldq + c16 * 8));
            } else {
                gb[s] = *gp((const u32x4*)(qt + (int64_t)(q >> 3) * ldq + k0 + (q & 7) * 8));
            }
        }
    };
    auto sstore = [&](int stage) {
        bf16* as = smem + stage * 2 * LA;
        bf16* bs = as + LA;
#pragma unroll
        for (int s = 0; s < LOADS; ++s) {
            const int q = s * NTHR + tid;
            const int r = q >> 3, c = q & 7;
            *(u32x4*)(as + r * BK + ((c ^ swz_k(r)) << 3)) = ga[s];
            if (NN) {
                const int k = q / (TS / 8), c16 = q % (TS / 8);
                const int g = c16 >> 1, h = c16 & 1;
                *(u32x4*)(bs + k * TS + ((((g ^ swz_n(k)) << 1) | h) << 3)) = gb[s];
            } else {
                *(u32x4*)(bs + r * BK + ((c ^ swz_k(r)) << 3)) = gb[s];
            }
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
        const bf16* as = smem + (kt & 1) * 2 * LA;
        const bf16* bs = as + LA;
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            bf16x8 af[F], bfv[F];
            const int c = kh * 4 + (lane >> 4);
#pragma unroll
            for (int fm = 0; fm < F; ++fm) {
                const int r = wm0 + fm * 16 + (lane & 15);
                af[fm] = *(const bf16x8*)(as + r * BK + ((c ^ swz_k(r)) << 3));
            }
            if (NN) {
                const int G = lane >> 4, rq = (lane >> 2) & 3, q4 = lane & 3;
#pragma unroll
                for (int fn = 0; fn < F; ++fn) {
                    const int g = (wn0 + fn * 16) >> 4;
                    i16x4 lo, hi;
                    {
                        const int k = kh * 32 + 8 * G + rq;
                        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(bs + k * TS + ((g ^ swz_n(k)) << 4) + q4 * 4));
                    }
                    {
                        const int k = kh * 32 + 8 * G + 4 + rq;
                        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(bs + k * TS + ((g ^ swz_n(k)) << 4) + q4 * 4));
                    }
                    typedef short i16x8 __attribute__((ext_vector_type(8)));
                    i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    bfv[fn] = __builtin_bit_cast(bf16x8, both);
                }
            } else {
#pragma unroll
                for (int fn = 0; fn < F; ++fn) {
                    const int r = wn0 + fn * 16 + (lane & 15);
                    bfv[fn] = *(const bf16x8*)(bs + r * BK + ((c ^ swz_k(r)) << 3));
                }
            }
#pragma unroll
            for (int fm = 0; fm < F; ++fm)
#pragma unroll
                for (int fn = 0; fn < F; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfv[fn], acc[fm][fn], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore((kt + 1) & 1);
        __syncthreads();
    }
    epilogue<bf16, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, (float*)smem);
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64x64 tiles, BK = 32, v_mfma_f32_16x16x4_f32. Within a block
// of 16 k, lane l holds k = 4*(l>>4) + s in MFMA s for both operands (any
// permutation of k shared by both operands leaves the sum unchanged).
// ---------------------------------------------------------------------------
template <bool NN, typename TSRC>
__global__ __launch_bounds__(NTHR) void k_gemm_f32(GemmArgs A) {
    constexpr int TS = 64, BK = 32, WT = 32, F = 2;
    constexpr int SPK = BK + 4, SPN = TS + 4;
    constexpr int LA = TS * SPK;
    constexpr int LB = NN ? BK * SPN : TS * SPK;
    __shared__ __attribute__((aligned(16))) float smem[2 * (LA + LB)];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= A.total_tiles) return;
    const int p = find_prob(A.prefix, A.nprobs, wg);
    const NsProb& P = A.probs[p];
    const int local = wg - A.prefix[p];
    const int mode = A.mode;
    int ti, tj;
    if (NN) apply_tile(local, P.mp / TS, P.np / TS, ti, tj);
    else upper_tile(local, P.mp / TS, ti, tj);

    const float *pm, *qm;
    int ldp, ldq, K;
    if (mode == GM_GRAM) {
        pm = qm = (const float*)P.x[A.src]; ldp = ldq = P.np; K = P.np;
    } else if (mode == GM_GRAM2) {
        pm = qm = (const float*)P.a; ldp = ldq = P.mp; K = P.mp;
    } else {
        pm = (const float*)(A.use_b ? P.b : P.a); ldp = P.mp;
        qm = (const float*)P.x[A.src]; ldq = P.np; K = P.mp;
    }
    const float* pt = pm + (int64_t)ti * TS * ldp;
    const float* qt = NN ? qm + tj * TS : qm + (int64_t)tj * TS * ldq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;

    f32x4 ga[2], gb[2];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int q = s * NTHR + tid;
            ga[s] = *gp((const f32x4*)(pt + (int64_t)(q >> 3) * ldp + k0 + (q & 7) * 4));
            if (NN) gb[s] = *gp((const f32x4*)(qt + (int64_t)(k0 + (q >> 4)) * ldq + (q & 15) * 4));
            else gb[s] = *gp((const f32x4*)(qt + (int64_t)(q >> 3) * ldq + k0 + (q & 7) * 4));
        }
    };
    auto sstore = [&](int stage) {
        float* as = smem + stage * (LA + LB);
        float* bs = as + LA;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int q = s * NTHR + tid;
            *(f32x4*)(as + (q >> 3) * SPK + (q & 7) * 4) = ga[s];
            if (NN) *(f32x4*)(bs + (q >> 4) * SPN + (q & 15) * 4) = gb[s];
            else *(f32x4*)(bs + (q >> 3) * SPK + (q & 7) * 4) = gb[s];
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
        const float* as = smem + (kt & 1) * (LA + LB);
        const float* bs = as + LA;
#pragma unroll
        for (int kb = 0; kb < BK / 16; ++kb) {
            f32x4 af[F], bfv[F];
            const int kk = kb * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int fm = 0; fm < F; ++fm) af[fm] = *(const f32x4*)(as + (wm0 + fm * 16 + (lane & 15)) * SPK + kk);
#pragma unroll
            for (int fn = 0; fn < F; ++fn) {
                if (NN) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) bfv[fn][s] = bs[(kk + s) * SPN + wn0 + fn * 16 + (lane & 15)];
                } else {
                    bfv[fn] = *(const f32x4*)(bs + (wn0 + fn * 16 + (lane & 15)) * SPK + kk);
                }
            }
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
    epilogue<float, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, smem);
}

template <int TS, bool NN>
hipError_t launch_bf16_t(const GemmArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)((a.total_tiles + 7) / 8 * 8);
    if (a.src_dtype == DT_BF16) hipLaunchKernelGGL((k_gemm_bf16<TS, NN, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
    else hipLaunchKernelGGL((k_gemm_bf16<TS, NN, float>), dim3(grid), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    const bool nn = a.mode == GM_APPLY || a.mode == GM_APPLY_LAST;
    if (tile == 256) return nn ? launch_bf16_t<256, true>(a, s) : launch_bf16_t<256, false>(a, s);
    if (tile == 128) return nn ? launch_bf16_t<128, true>(a, s) : launch_bf16_t<128, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    const bool nn = a.mode == GM_APPLY || a.mode == GM_APPLY_LAST;
    const unsigned grid = (unsigned)((a.total_tiles + 7) / 8 * 8);
    if (a.src_dtype == DT_BF16) {
        if (nn) hipLaunchKernelGGL((k_gemm_f32<true, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f32<false, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
    } else {
        if (nn) hipLaunchKernelGGL((k_gemm_f32<true, float>), dim3(grid), dim3(NTHR), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f32<false, float>), dim3(grid), dim3(NTHR), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace mu
