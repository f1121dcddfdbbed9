// Newton-Schulz products on MFMA (gfx950).
//
// One Newton-Schulz step on the wide X (m x n, m <= n) is
//     A  = X X^T                       (Gram, m x m, symmetric)
//     X' = a X + b A X + c A A X  =  B X,   B = a I + b A + c A A^T
// (MuonClip Optimizer page, section "Newton-Schulz Orthogonalization", gives
// the cubic step with a = 1.5, b = -0.5, c = 0, written as X (X^T X), which
// equals (X X^T) X; the Gram side is kept on the short dimension.) B is formed
// in the Gram epilogue (cubic steps) or in an A A^T pass (quintic steps), so
// the apply is a plain product.
//
// Wide blocks with Gram-side steps (planned in capi.hip) run their first steps
// as m x m products instead: every iterate is X_k = Q_k X_0 with Q_k and
// A_k = X_k X_k^T polynomials in A_0, so S_k = B_k B_k, A_{k+1} = S_k A_k and
// Q_{k+1} = B_k Q_k are products of commuting symmetric matrices. They run on
// the Gram kernel with two operands (the pair product: upper tiles, mirrored),
// after a first Gram that also keeps A_0 and the unfolded B_0 (the dual Gram);
// the restart X_R = Q_R X_0 is a plain apply.
//
// All products are grouped GEMMs over every (matrix, head) problem of a call:
// one launch per mode covers all problems, each workgroup reads its problem
// and tile coordinates from the call's tile map (built once per call from the
// tile prefix over the problems), and workgroup ids are remapped so that
// neighbouring tiles run on the same XCD (shared L2).
//
// The Gram X X^T is "NT" (C = P Q^T, both operands K-contiguous) and reads X
// twice. The bf16 apply B X reads B (symmetric, K-contiguous) and X itself,
// whose k runs down its rows: fragments of X come out of LDS through
// ds_read_b64_tr_b16, so no transposed copy of X is ever written. (The fp32
// kernel reads a transposed copy X^T that the previous epilogue or the prep
// kernel wrote.) Gram products only compute tiles on or above the diagonal and
// also store the transposed tile.
//
// bf16: v_mfma_f32_16x16x32_bf16, fp32 accumulation, 256x256 or 128x128
// workgroup tiles, BK = 32, 4 waves in 2x2 (128x128 per wave for 256 tiles),
// K-blocked operands moved with direct-to-LDS buffer loads through a ring of
// four LDS slots.
// fp32: v_mfma_f32_16x16x4_f32, 64x64 tiles, BK = 32, row-major operands.
// Short blocks (mp == 128) of a call with many of them: k_ns_small runs every
// step but the last apply in one workgroup per block, with B kept in LDS.
//
// Epilogue: row-major outputs are staged per wave through LDS in 16-row strips
// and stored as 16-byte chunks; transposed outputs (Gram mirror, a tall
// weight, X'^T of the fp32 path) are formed in registers with
// v_permlane16_swap. The Gram
// epilogue applies the step coefficients and, on the first step, the fold
// f = 1/||U||_F (so the normalised X0 is never materialised); the last apply
// writes the decoupled-weight-decay update W <- W - lr*wd*W - lr*scale*O
// straight into the parameter.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mu {

namespace {

constexpr int NTHR = 256;

template <int N>
struct Stage {
    static constexpr int value = N;
};

// fn(Stage<i>{}) for i = B .. E-1, every index a compile-time constant
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
    if constexpr (B < E) {
        fn(Stage<B>{});
        static_for<B + 1, E>(fn);
    }
}

// ---------------------------------------------------------------------------
// Tile enumeration
// ---------------------------------------------------------------------------
// Upper-triangle tiles (ti <= tj) of a T x T tile grid in blocks of 8 x 8
// tiles (triangular on the diagonal), the blocks in row order and the tiles
// row by row inside a block. Runs of consecutive tiles then share fewer
// strips of X than in plain row order (a model of 32 consecutive tiles gives
// 11 % fewer strip loads at T = 16); the 8B-shaped Gram measured 1.5 % faster.
__device__ __forceinline__ void upper_tile(int local, int T, int& ti, int& tj) {
    constexpr int BB = 8;
    for (int I = 0; I < T; I += BB) {   // block row I: the triangle, then full-height blocks
        const int hI = min(BB, T - I);
        const int tri = hI * (hI + 1) / 2;
        if (local < tri) {
            int i = 0;
            while (local >= hI - i) { local -= hI - i; ++i; }
            ti = I + i;
            tj = I + i + local;
            return;
        }
        local -= tri;
        const int rest = hI * (T - I - hI);   // blocks right of the diagonal (hI == BB there)
        if (local < rest) {
            const int blk = local / (hI * BB);
            const int J = I + hI + blk * BB, wJ = min(BB, T - J);
            const int w = local - blk * hI * BB;
            ti = I + w / wJ;
            tj = J + w % wJ;
            return;
        }
        local -= rest;
    }
    ti = tj = 0;   // not reached: local < T (T + 1) / 2
}

// Groups of eight tile rows, column-major inside a group: 8 panels of B and a
// run of X panels are shared by the workgroups running together (32 tiles of
// an XCD: 8 B and 4 X panels). Same-box sweep on the 8B-shaped set, apply ms
// per launch: groups of 2: 45.4, 4: 42.0, 6: 41.9, 8: 41.4, 12: 42.3, 16: 45.0.
__device__ __forceinline__ void apply_tile(int local, int TM, int TN, int& ti, int& tj) {
    constexpr int G = 8;
    const int per_group = G * TN;
    const int g = local / per_group;
    const int w = local - g * per_group;
    const int gm = min(G, TM - g * G);
    ti = g * G + w % gm;
    tj = w / gm;
}

// Tile maps (see TileMapArgs): the same enumerations as the GEMMs above.
__global__ __launch_bounds__(NTHR) void k_tilemap(TileMapArgs A) {
    const int t = blockIdx.x * NTHR + threadIdx.x;
    if (t < A.nqueues) A.queues[t] = 0;
    if (t >= A.total) return;
    int s = 0;
    while (s + 1 < A.nseg && t >= A.seg[s + 1].start) ++s;
    const TileMapSeg S = A.seg[s];
    const int local = t - S.start;
    const int ps = find_prob(S.prefix, S.nprobs, local);
    const int p = S.order ? S.order[ps] : ps;
    const int in_prob = local - S.prefix[ps];
    const int T = S.probs[p].mp / S.ts;
    int ti, tj;
    if (S.sym) upper_tile(in_prob, T, ti, tj);
    else apply_tile(in_prob, T, S.probs[p].np / S.ts, ti, tj);
    S.out[local] = TileEntry{p, ti | (tj << 16)};
}

// ---------------------------------------------------------------------------
// U-space write of 8 consecutive values (update or plain output); row ur,
// columns uc0 .. uc0+7 (uc0 a multiple of 8), clipped to the head block. A
// whole run on vector-capable buffers takes two 4-wide read-modify-writes; a
// run cut by the block edge goes element by element in a loop that is kept
// rolled, so the many inlined copies of this stay small.
// ---------------------------------------------------------------------------
// The update's scalars, read from the call's CallScalars once per wave by the
// last-apply epilogue.
struct UpdScalars {
    float lr, wd;
    bool cautious;
};

// Decoupled decay factor of one element: lr*wd, or with cautious weight decay
// lr*wd only where the update u = step*v has the sign of x or is zero.
__device__ __forceinline__ float decay_of(const UpdScalars& us, float decay, float x, float u) {
    return (us.cautious && x * u < 0.f) ? 0.f : decay;
}

template <typename TS>
__device__ __forceinline__ void emit_u8(const GemmArgs& A, const NsProb& P, const UpdScalars& us, int ur, int uc0,
                                        const float* v) {
    if (ur >= P.hr || uc0 >= P.hc) return;
    const int64_t off = (int64_t)ur * P.ld + uc0;
    const float decay = us.lr * us.wd, step = us.lr * P.scale;
    if (P.vec && uc0 + 8 <= P.hc) {
        if (P.oout) {
#pragma unroll
            for (int e = 0; e < 8; ++e) P.oout[off + e] = v[e];
        }
        TS* dst = (TS*)(A.with_update ? P.param : P.out) + off;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float x[4];
            if (A.with_update) {
                if constexpr (sizeof(TS) == 2) {
                    const bf16x4 q = *gp((const bf16x4*)(dst + 4 * h));
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (float)q[e];
                } else {
                    const f32x4 q = *gp((const f32x4*)(dst + 4 * h));
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = q[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = decay_of(us, decay, x[e], step * v[4 * h + e]);
                    x[e] = (x[e] - d * x[e]) - step * v[4 * h + e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = v[4 * h + e];
            }
            if constexpr (sizeof(TS) == 2) {
                bf16x4 q;
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = (bf16)x[e];
                *gp((bf16x4*)(dst + 4 * h)) = q;
            } else {
                *gp((f32x4*)(dst + 4 * h)) = f32x4{x[0], x[1], x[2], x[3]};
            }
        }
        return;
    }
    const int valid = min(8, P.hc - uc0);
#pragma clang loop unroll(disable)
    for (int e = 0; e < valid; ++e) {
        const float ve = e == 0 ? v[0] : e == 1 ? v[1] : e == 2 ? v[2] : e == 3 ? v[3]
                       : e == 4 ? v[4] : e == 5 ? v[5] : e == 6 ? v[6] : v[7];
        if (P.oout) P.oout[off + e] = ve;
        if (A.with_update) {
            TS* w = (TS*)P.param + off + e;
            const float x = to_f32<TS>(*w);
            const float d = decay_of(us, decay, x, step * ve);
            *w = from_f32<TS>((x - d * x) - step * ve);
        } else {
            ((TS*)P.out)[off + e] = from_f32<TS>(ve);
        }
    }
}

// The update of emit_u8's vector path with the 8 parameter values already in
// registers (loaded ahead, see the last-apply epilogue); same arithmetic.
__device__ __forceinline__ void update8_pre(const NsProb& P, const UpdScalars& us, int ur, int uc0, const float* v,
                                            const bf16x4 (&q)[2]) {
    const int64_t off = (int64_t)ur * P.ld + uc0;
    const float decay = us.lr * us.wd, step = us.lr * P.scale;
    if (P.oout) {
#pragma unroll
        for (int e = 0; e < 8; ++e) P.oout[off + e] = v[e];
    }
    bf16* dst = (bf16*)P.param + off;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = (float)q[h][e];
            const float d = decay_of(us, decay, x, step * v[4 * h + e]);
            o[e] = (bf16)((x - d * x) - step * v[4 * h + e]);
        }
        *gp((bf16x4*)(dst + 4 * h)) = o;
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

// Copy one accumulator out of its AGPR at this point of the program (the
// compiler would otherwise hoist all 256 copies to the end of the K loop).
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// Order LDS accesses of this wave. A wave's LDS instructions execute in issue
// order, so lanes see each other's earlier writes without any wait; only the
// compiler must not move accesses across this point. (A memory fence would do
// that too, but it also waits for every global store still in flight.)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("" ::: "memory"); }

// ---------------------------------------------------------------------------
// Epilogue shared by the bf16 and fp32 kernels. The accumulator layout is the
// 16x16 MFMA one: lane l holds C[4*(l>>4) + e][l & 15] of each fragment.
//
// What each mode stores (f = 1/(||U||_F + eps) on the first step, else 1):
//   Gram, cubic step     B = f (a I + b f^2 X X^T)    -> P.a (mirrored)
//   Gram, quintic step   A = f^2 X X^T                -> P.a (mirrored)
//   A^2 pass             B = f (a I + b A + c A A^T)  -> P.b (mirrored)
//   apply                X' = B X                     -> X' (and X'^T, fp32 only)
//   last apply           O = B X -> parameter update (or output)
//   dual Gram (first step of a Gram-side block): B = f (a I + b f^2 X X^T)
//                        -> P.a, and also A0 = f^2 X X^T -> X' buffer (mp x mp),
//                        B0 = a I + b f^2 X X^T -> P.b (all mirrored)
//   pair product         C = P Q^T (P = x[0], Q = x[1], mp x mp, C symmetric)
//                        -> P.a, and B' = a I + b C -> P.b where P.b is set
//                        (both mirrored); with use_b only B' -> P.a
// On the first step X holds U itself, and f (a X0 + b (X0 X0^T) X0) with
// X0 = f U is exactly B U for these B. Folding a I and f into B keeps X and
// any scaling out of the apply epilogue; padding stays zero because a padded
// row of X' is f*a*0 + (rows of A that are zero).
//
// Transposed outputs (Gram mirror, fp32 X'^T, a tall block's parameter) come
// straight from registers: v_permlane16_swap on the accumulators of two
// neighbouring fragments leaves every lane with 8 consecutive rows of one
// column, one 16-byte chunk of the transposed (K-blocked) output.
// Row-major outputs go through `st`, this wave's LDS strip of 16 x (F*16 + 4)
// floats: lane -> row idx%16 and 8 consecutive columns, so with the K-blocked
// layout a wave writes whole 1 KB blocks. Each wave stages only its own strip,
// so syncs are wave-local.
// A tall block's parameter update is the exception to going straight from
// registers: there a 16-row strip is only 16 consecutive elements of each of
// 128 parameter rows, and updating 32-byte pieces of rows 8 KB apart makes the
// L2 fetch the same lines many times over. The bf16 kernel gives each wave a
// second slot array (`st2`): four strips are collected there as an F*16 x 64
// f32 block (first half of the rows in `st`, second half in `st2`; 16-byte
// chunk q of row c stored at chunk q ^ (c % 16), which keeps both the column
// writes and the row reads free of bank conflicts) and then written back as
// one 128-byte run of bf16 per parameter row.
// A wide block's update is staged the same way, four strips (64 rows x F*16)
// at a time in `st` and `st2`, and written back as whole F*16-wide runs of
// parameter rows. Besides the long runs, staging puts four strips of work
// between the load of the parameter values and their first use.
// ---------------------------------------------------------------------------
template <int MODE, typename TX, typename TS, int F>
__device__ __forceinline__ void epilogue_mode(const GemmArgs& A, const NsProb& P, int ti, int tj, int TS_, int wm0,
                                              int wn0, f32x4 (&acc)[F][F], float* st, float* st2) {
    static_assert(F % 2 == 0, "fragments are paired for the transposed stores");
    // staged tall update: four 16-row strips per WT x 64 block, in two halves
    // of WT/2 rows (one slot array each)
    constexpr bool staged_tall = MODE == GM_APPLY_LAST && F % 4 == 0;
    // staged wide update: four 16-row strips (64 rows x WT) at a time, rows
    // 0..31 in `st` and 32..63 in `st2`
    constexpr bool staged_wide = staged_tall;
    constexpr int WT = F * 16;
    constexpr int SP = WT + 4;
    constexpr int PASSES = WT / 32;            // row pass: 16 rows x 32 columns per pass
    // The last apply's update passes (the staged wide blocks, and the fp32
    // kernel's row passes) give each parameter row LPR lanes of 8 columns,
    // RPP whole rows per pass: a wave then reads and writes whole WT-wide
    // runs of parameter rows, where 16 x 32 passes would cut every row into
    // 64-byte pieces.
    constexpr int LPR = WT / 8, RPP = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4, l16 = lane & 15;
    constexpr int mode = MODE;
    UpdScalars us{0.f, 0.f, false};   // the update's scalars (last apply only)
    if constexpr (MODE == GM_APPLY_LAST) {
        us.lr = gp(A.cs)->lr;
        us.wd = gp(A.cs)->wd;
        us.cautious = gp(A.cs)->cautious != 0;
    }
    constexpr bool dual = mode == GM_GRAM_DUAL;
    constexpr bool pair = mode == GM_GRAM_PAIR;
    constexpr bool gram = mode == GM_GRAM || mode == GM_GRAM2 || dual || pair;
    const float f = gram && A.first ? P.fold[0] : 1.f;   // the apply takes it through B
    const bool diag = gram && ti == tj;
    if (diag && wm0 > wn0) return;   // below the diagonal: written by the mirror of the quadrant above
    // a wave block on the diagonal holds only its fragments on or above the
    // diagonal (fm <= fn); the others are written as their mirrors
    const bool tri = diag && wm0 == wn0;
    const bool mirror = gram && (ti != tj || wm0 < wn0 || tri);
    constexpr bool last = mode == GM_APPLY_LAST;
    // X'^T is kept only for the fp32 kernel; the bf16 apply reads X itself
    const bool trans_out = mirror || (!gram && !last && sizeof(TX) == 4) || (last && P.tall);
    const bool row_out = !(last && (P.tall || staged_wide));
    const int row_base = ti * TS_ + wm0, col_base = tj * TS_ + wn0;

    // Last apply with bf16 parameters: with one wave per SIMD nothing hides the
    // latency of a read-modify-write, so when the wave's whole WT x WT block is
    // in bounds its parameter values are all loaded up front (F*F/2 runs of 8
    // per lane, in the order the writes below consume them) and only the
    // stores remain in the strip loop.
    constexpr bool pre_ok = last && sizeof(TS) == 2 && F % 4 == 0;
    constexpr int NPRE = pre_ok ? F * F / 2 : 1;
    bf16x4 pre[NPRE][2];
    bool fast = false;
    if constexpr (pre_ok) {
        const int br = P.tall ? col_base : row_base;   // first parameter row of the block
        const int bc = P.tall ? row_base : col_base;   // first parameter column
        fast = A.with_update && P.vec && br + WT <= P.hr && bc + WT <= P.hc;
        if (fast) {
            const bf16* par = (const bf16*)P.param;
            static_for<0, NPRE>([&](auto ic) {
                constexpr int idx = decltype(ic)::value;
                int ur, uc0;
                if (P.tall) {   // staged block (idx / (WT/8)), row group idx % (WT/8)
                    ur = br + (idx % (WT / 8)) * 8 + (lane >> 3);
                    uc0 = bc + (idx / (WT / 8)) * 64 + 8 * (lane & 7);
                } else {        // staged half idx / LPR, pass idx % LPR
                    ur = br + (idx / LPR) * 64 + (idx % LPR) * RPP + lane / LPR;
                    uc0 = bc + (lane % LPR) * 8;
                }
                const bf16* src = par + (int64_t)ur * P.ld + uc0;
                pre[idx][0] = *gp((const bf16x4*)src);
                pre[idx][1] = *gp((const bf16x4*)(src + 4));
            });
        }
    }
    const int mp = P.mp, np = P.np;
    // Gram scale and diagonal term
    // Gram scale gs, diagonal term gd, and (A^2 pass) the factor on A
    float gs = f * f, gd = 0.f, ga = A.cb;
    if ((mode == GM_GRAM || dual) && !A.use_b) { gs = A.cb * f * f * f; gd = A.ca * f; }
    if (pair) { gs = A.use_b ? A.cb : 1.f; gd = A.use_b ? A.ca : 0.f; }   // use_b: B' alone, to a
    if (mode == GM_GRAM2) { gs = A.cc * f; gd = A.ca * f; ga = A.cb * f; }
    TX* gdst = (TX*)(mode == GM_GRAM2 ? P.b : P.a);
    // the extra outputs: A0 (scale f^2) and the unfolded B0 (scale b f^2,
    // diagonal a) of the dual Gram; B' = a I + b C of a pair product
    const float s_a0 = dual ? f * f : 0.f, s_b0 = dual ? A.cb * f * f : pair ? A.cb : 0.f;
    TX* a0dst = dual ? (TX*)(A.src ? P.x[0] : P.x[1]) : nullptr;
    TX* b0dst = (dual || pair) ? (TX*)P.b : nullptr;
    const bool with_b0 = dual || (pair && !A.use_b && P.b != nullptr);
    // A^2 pass: B = gd I + ga A + gs A A^T takes A over the whole block. The
    // stored A is exactly symmetric (the Gram writes both triangles from the
    // same values), so the four accumulator rows r .. r+3 of a lane's column
    // c are read as A[c][r .. r+3]: four consecutive k of operand row c, one
    // 8-byte piece (16 for fp32). All of them are loaded here, before the
    // strip loop: loaded next to their use, each waited behind the stores of
    // the strip before it (the A^2 pass ran 12-23 % slower that way).
    constexpr bool a2 = mode == GM_GRAM2;
    typedef typename std::conditional<sizeof(TX) == 2, bf16x4, f32x4>::type A4;
    A4 apre[a2 ? F : 1][a2 ? F : 1];
    if constexpr (a2) {
        const TX* ab = (const TX*)P.a;
#pragma unroll
        for (int fm = 0; fm < F; ++fm)
#pragma unroll
            for (int fn = 0; fn < F; ++fn) {
                const int c = col_base + fn * 16 + l16, r = row_base + fm * 16 + 4 * g4;
                apre[fm][fn] = *gp((const A4*)(ab + op_off<TX>(c, r, P.mp, P.mp)));
            }
    }
    TX* xdst = (TX*)(A.src ? P.x[0] : P.x[1]);
    TX* xtdst = (TX*)(A.src ? P.xt[0] : P.xt[1]);
    // Where this lane's run of 8 goes in a workspace operand with R rows and
    // K columns (element (row, k)). The bf16 operands are K-blocked: the 1 KB
    // block of a store is wave-uniform (row_base, col_base are multiples of
    // 64) and the place inside it a per-lane constant, so the address is a
    // scalar base plus a 32-bit lane offset. fp32 operands are row-major.
    //   transposed run: column c of C as operand row, C rows r0 .. r0+7 as k
    //   row run:        C row r, columns c .. c+7 as k
    const uint32_t lane_t = (uint32_t)(((g4 & 1) * 512 + (g4 >> 1) * 128 + l16 * 8) * sizeof(TX));
    const uint32_t lane_r = (uint32_t)((g4 * 128 + l16 * 8) * sizeof(TX));
    auto tdst = [&](TX* base, int R, int K, int c, int r0, int fm, int fp) -> TX* {
        if constexpr (sizeof(TX) == 2) {
            const int64_t blk = (int64_t)(row_base / 32 + (fm >> 1)) * (R >> 4) + col_base / 16 + fp;
            return (TX*)((char*)(base + blk * 512 + (fm & 1) * 256) + lane_t);
        } else {
            return base + op_off<TX>(c, r0, R, K);
        }
    };
    auto rdst = [&](TX* base, int R, int K, int r, int c, int fm, int pass) -> TX* {
        if constexpr (sizeof(TX) == 2) {
            const int64_t blk = (int64_t)(col_base / 32 + pass) * (R >> 4) + row_base / 16 + fm;
            return (TX*)((char*)(base + blk * 512) + lane_r);
        } else {
            return base + op_off<TX>(r, c, R, K);
        }
    };

#pragma clang loop unroll(full)
    for (int fm = 0; fm < F; ++fm) {
        // this strip's accumulators, copied out of the AGPRs here and only
        // here, so register use stays bounded by one strip
        float av[F][4];
#pragma unroll
        for (int fn = 0; fn < F; ++fn)
#pragma unroll
            for (int e = 0; e < 4; ++e) av[fn][e] = agpr_read(acc[fm][fn][e]);
        if constexpr (a2) {
            // B's values, in the accumulator layout (rows 4*g4 + e, column l16)
#pragma unroll
            for (int fn = 0; fn < F; ++fn)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[fn][e] = gs * av[fn][e] + ga * (float)apre[fm][fn][e];
                    if (diag && row_base + fm * 16 + 4 * g4 + e == col_base + fn * 16 + l16) av[fn][e] += gd;
                }
        }
        // the row-major copy is staged first: the swaps below then consume
        // the accumulator values in place instead of copying them
        if (row_out) {
            wave_lds_sync();
#pragma unroll
            for (int fn = 0; fn < F; ++fn)
#pragma unroll
                for (int e = 0; e < 4; ++e) st[(4 * g4 + e) * SP + fn * 16 + l16] = av[fn][e];
        }
        if constexpr (staged_wide) {
            if (!P.tall) {
                // strip fm -> rows (fm%4)*16 .. of the staged half; 4-float
                // chunk k of row h sits at chunk k ^ 4((h/4)%4), so the four
                // row groups of a write land in different banks
#pragma unroll
                for (int fn = 0; fn < F; ++fn)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int h = (fm & 3) * 16 + 4 * g4 + e, col = fn * 16 + l16;
                        float* row = (h < 32 ? st : st2) + (h & 31) * WT;
                        row[(((col >> 2) ^ (4 * g4)) << 2) | (col & 3)] = av[fn][e];
                    }
                if ((fm & 3) == 3) {
                    wave_lds_sync();
                    auto half_row = [&](int pass, float* v) {
                        const int h = pass * RPP + lane / LPR, k = (lane % LPR) * 2;
                        const float* row = (h < 32 ? st : st2) + (h & 31) * WT;
                        const int sw = 4 * ((h >> 2) & 3);
                        const f32x4 lo = *(const f32x4*)(row + ((k ^ sw) << 2));
                        const f32x4 hi = *(const f32x4*)(row + (((k + 1) ^ sw) << 2));
#pragma unroll
                        for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[4 + e] = hi[e]; }
                    };
                    const int ur0 = row_base + (fm >> 2) * 64, uc0 = col_base + (lane % LPR) * 8;
                    if (fast) {
                        if constexpr (pre_ok) {
#pragma unroll
                            for (int pass = 0; pass < LPR; ++pass) {
                                float v[8];
                                half_row(pass, v);
                                update8_pre(P, us, ur0 + pass * RPP + lane / LPR, uc0, v, pre[(fm >> 2) * LPR + pass]);
                            }
                        }
                    } else {
#pragma clang loop unroll(disable)
                        for (int pass = 0; pass < LPR; ++pass) {
                            float v[8];
                            half_row(pass, v);
                            emit_u8<TS>(A, P, us, ur0 + pass * RPP + lane / LPR, uc0, v);
                        }
                    }
                    wave_lds_sync();
                }
            }
        }
        if (trans_out) {
#pragma unroll
            for (int fp = 0; fp < F; fp += 2) {
                if (tri && fp + 1 <= fm) continue;   // both fragments at or below the diagonal
                float w[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(av[fp][e]),
                                                                     __float_as_uint(av[fp + 1][e]), false, false);
                    w[e] = __uint_as_float(sw[0]);
                    w[4 + e] = __uint_as_float(sw[1]);
                }
                // this lane: column c of C, rows r0 .. r0+7 (off the diagonal
                // for mirrored tiles)
                const int c = col_base + (fp + (g4 & 1)) * 16 + l16;
                const int r0 = row_base + fm * 16 + 8 * (g4 >> 1);
                float v[8];
                if constexpr (gram) {
                    // on a diagonal wave block only the fragments above the
                    // diagonal are mirrored (this lane's fragment: fp + (g4&1))
                    if (!tri || fp + (g4 & 1) > fm) {
                        // (the A^2 pass has B's values in w already; B is
                        // symmetric, so they are the mirrored ones too)
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = a2 ? w[e] : gs * w[e];
                        store8<TX>(tdst(gdst, mp, mp, c, r0, fm, fp), v);
                        if constexpr (dual) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] = s_a0 * w[e];
                            store8<TX>(tdst(a0dst, mp, mp, c, r0, fm, fp), v);
                        }
                        if ((dual || pair) && with_b0) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) v[e] = s_b0 * w[e];
                            store8<TX>(tdst(b0dst, mp, mp, c, r0, fm, fp), v);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = w[e];
                    if constexpr (!last) {
                        if constexpr (sizeof(TX) == 4) store8<TX>(tdst(xtdst, np, mp, c, r0, fm, fp), v);
                    } else if constexpr (staged_tall) {
                        // block row cl = c - col_base, columns rl .. rl+7
                        const int cl = (fp + (g4 & 1)) * 16 + l16;
                        const int q = ((fm & 3) * 16 + 8 * (g4 >> 1)) >> 2;
                        float* row = (fp < F / 2 ? st : st2) + (cl & (WT / 2 - 1)) * 64;
                        *(f32x4*)(row + ((q ^ l16) << 2)) = f32x4{v[0], v[1], v[2], v[3]};
                        *(f32x4*)(row + (((q + 1) ^ l16) << 2)) = f32x4{v[4], v[5], v[6], v[7]};
                    } else {
                        emit_u8<TS>(A, P, us, c, r0, v);
                    }
                }
            }
            if constexpr (staged_tall) {
                if ((fm & 3) == 3) {
                    // block complete: lane -> row it*8 + lane/8, columns 8*(lane%8) .. +7
                    wave_lds_sync();
                    const int j = lane & 7;
                    auto block_row = [&](int it, float* v) {
                        const int cl = it * 8 + (lane >> 3);
                        const float* row = (it < WT / 16 ? st : st2) + (cl & (WT / 2 - 1)) * 64;
                        const f32x4 lo = *(const f32x4*)(row + (((2 * j) ^ (cl & 15)) << 2));
                        const f32x4 hi = *(const f32x4*)(row + (((2 * j + 1) ^ (cl & 15)) << 2));
#pragma unroll
                        for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[4 + e] = hi[e]; }
                    };
                    const int uc0 = row_base + (fm >> 2) * 64 + 8 * j;
                    if (fast) {
                        if constexpr (pre_ok) {
#pragma unroll
                            for (int it = 0; it < WT / 8; ++it) {
                                float v[8];
                                block_row(it, v);
                                update8_pre(P, us, col_base + it * 8 + (lane >> 3), uc0, v,
                                            pre[(fm >> 2) * (WT / 8) + it]);
                            }
                        }
                    } else {
#pragma clang loop unroll(disable)
                        for (int it = 0; it < WT / 8; ++it) {
                            float v[8];
                            block_row(it, v);
                            emit_u8<TS>(A, P, us, col_base + it * 8 + (lane >> 3), uc0, v);
                        }
                    }
                    wave_lds_sync();
                }
            }
        }
        if (!row_out) continue;
        wave_lds_sync();
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            const int rr = last ? pass * RPP + lane / LPR : l16;
            const int c8 = last ? (lane % LPR) * 8 : pass * 32 + g4 * 8;
            float v[8];
            {
                const f32x4 lo = *(const f32x4*)(st + rr * SP + c8);
                const f32x4 hi = *(const f32x4*)(st + rr * SP + c8 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[e + 4] = hi[e]; }
            }
            const int r = row_base + fm * 16 + rr, c = col_base + c8;
            if constexpr (gram) {
                // a diagonal wave block stores its fragments on or above the
                // diagonal only (this lane's fragment: c8 / 16)
                if (tri && c8 / 16 < fm) continue;
                if ((dual || pair) && with_b0) {
                    float u[8];
                    if constexpr (dual) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) u[e] = s_a0 * v[e];
                        store8<TX>(rdst(a0dst, mp, mp, r, c, fm, pass), u);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) u[e] = s_b0 * v[e];
                    if (diag) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (r == c + e) u[e] += A.ca;
                    }
                    store8<TX>(rdst(b0dst, mp, mp, r, c, fm, pass), u);
                }
                if constexpr (!a2) {   // (the A^2 pass staged B's values)
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] *= gs;
                    if (diag) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (r == c + e) v[e] += gd;
                    }
                }
                store8<TX>(rdst(gdst, mp, mp, r, c, fm, pass), v);
            } else {
                if constexpr (!last) {
                    // X' is read back only by the next step's launches:
                    // stored non-temporally (0.1 ms per launch faster on
                    // the 8B-shaped set, same box)
                    if constexpr (sizeof(TX) == 2) {
                        bf16x8 q;
#pragma unroll
                        for (int e = 0; e < 8; ++e) q[e] = (bf16)v[e];
                        __builtin_nontemporal_store(q, gp((bf16x8*)rdst(xdst, mp, np, r, c, fm, pass)));
                    } else {
                        store8<TX>(rdst(xdst, mp, np, r, c, fm, pass), v);
                    }
                } else {
                    if constexpr (pre_ok) {
                        if (fast) update8_pre(P, us, r, c, v, pre[fm * PASSES + pass]);
                        else emit_u8<TS>(A, P, us, r, c, v);
                    } else {
                        emit_u8<TS>(A, P, us, r, c, v);
                    }
                }
            }
        }
    }
}

// One specialised, contiguous epilogue per mode: a generic one with every
// mode's code unrolled over the strips outgrows the instruction cache.
template <bool SYM, typename TX, typename TS, int F>
__device__ __forceinline__ void epilogue(const GemmArgs& A, const NsProb& P, int ti, int tj, int TS_, int wm0,
                                         int wn0, f32x4 (&acc)[F][F], float* st, float* st2) {
    // (the float32 kernel's: the dual modes run in bf16 only)
    if constexpr (SYM) {
        if (A.mode == GM_GRAM) epilogue_mode<GM_GRAM, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
        else epilogue_mode<GM_GRAM2, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
    } else {
        if (A.mode == GM_APPLY) epilogue_mode<GM_APPLY, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
        else epilogue_mode<GM_APPLY_LAST, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
    }
}
// The bf16 kernel's epilogues, one kernel instance each (EPI): the Gram and
// A^2 pass or the plain apply (0); the last apply, or for Gram kernels the
// dual Gram (1); the pair product (Gram kernels, 2). The modes of one
// instance share its code, and the others' code stays out of the instances
// the plain steps run.
template <bool SYM, int EPI, typename TX, typename TS, int F>
__device__ __forceinline__ void epilogue_k(const GemmArgs& A, const NsProb& P, int ti, int tj, int TS_, int wm0,
                                           int wn0, f32x4 (&acc)[F][F], float* st, float* st2) {
    if constexpr (SYM && EPI == 1) epilogue_mode<GM_GRAM_DUAL, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
    else if constexpr (SYM && EPI == 2) epilogue_mode<GM_GRAM_PAIR, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
    else if constexpr (SYM) {
        if (A.mode == GM_GRAM) epilogue_mode<GM_GRAM, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
        else epilogue_mode<GM_GRAM2, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
    } else if constexpr (EPI == 1) epilogue_mode<GM_APPLY_LAST, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
    else epilogue_mode<GM_APPLY, TX, TS, F>(A, P, ti, tj, TS_, wm0, wn0, acc, st, st2);
}

// ---------------------------------------------------------------------------
// bf16 kernel
//
// K loop over steps of BK = 32 through a ring of NS = 4 LDS slots (separate
// arrays, so the compiler's wait insertion can tell a direct-to-LDS load into
// one slot from reads of another). Operand slices move HBM/L2 -> LDS with
// global_load_lds_dwordx4: each instruction writes 64 lanes x 16 B
// contiguously (LDS base + lane*16). A slot holds an operand slice as 1 KB
// blocks of 16 rows x 32 k, chunk-major inside the block (16-byte chunk c of
// row r at byte 16*(16c + r)): that is exactly the lane order of a 16x16x32
// MFMA fragment, so a fragment read is one linear ds_read_b128 of a block
// (lane l at byte 16*l, free of bank conflicts) and one direct load fills one
// block. The apply's right operand, X, is the exception: its blocks hold rows
// of k, so its fragments come from two ds_read_b64_tr_b16 each (see read_b).
//
// Step kt (slot kt%NS holds slice kt, whose fragments are in registers; the
// slices up to kt+NS-1 are in flight):
//   phase A: the first HEAD fragment rows of MFMAs; wait until slice kt+1 has
//            landed and the reads of slice kt are done; barrier
//   phase B: direct loads of slice kt+NS into slot kt%NS, reads of slice
//            kt+1's fragments, the remaining MFMAs, interleaved in a fixed
//            order (loads spread out: a burst of them starves the MFMA stream)
// One barrier per step; each load has NS-1 steps (~1.5 us at 256x256 tiles)
// to arrive, which covers an L2 miss under full load.
// ---------------------------------------------------------------------------
#define LDSP __attribute__((address_space(3)))

// Word 3 of a raw buffer resource: 32-bit data format, no swizzle, no stride.
constexpr int BUF_RAW32 = 0x00020000;

// s_waitcnt with only vmcnt (gfx9 encoding: vmcnt[3:0] bits 3:0, [5:4] bits 15:14)
#define MU_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// s_waitcnt with vmcnt and lgkmcnt(0)
#define MU_WAIT_VMCNT_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (0 << 8) | (((n) >> 4) << 14))
// s_waitcnt lgkmcnt(0) only
#define MU_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14))

// Persistent launches. XCD x's queue is the list of tiles it receives in a
// one-tile-per-workgroup launch (positions x, x+8, .. of that grid through the
// window remap), handed out in that order by an atomic counter; a workgroup
// whose queue is empty moves on to the next XCD's. The clocks of the XCDs
// differ by up to 10 % under the GEMMs, so a fixed share per XCD leaves the
// fast ones idle at the end of every launch; this way they take over the
// slow ones' last tiles. Returns -1 once every queue is empty: a queue seen
// empty stays empty, so one pass over the eight ends the search.
__device__ __forceinline__ int xcc_id() {
    return (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 7);   // HW_REG_XCC_ID, bits 3:0
}
__device__ __forceinline__ int next_tile(const GemmArgs& A, int& q, int n, int gstat, int win) {
    const int nper = gstat >> 3;
    for (int empty = 0;;) {
        if (n < nper) {
            const int t = xcd_remap_window(q + 8 * n, gstat, win);
            if (t < A.total_tiles) return t;
        } else {
            if (++empty == 8) return -1;
            q = (q + 1) & 7;
        }
        n = atomicAdd(A.queues + q, 1);
    }
}

template <int TS, bool SYM, typename TSRC, int EPI>
__global__ __launch_bounds__(NTHR) void k_gemm_bf16(GemmArgs A) {
    constexpr int BK = 32;
    constexpr int NS = 4;
    constexpr int WT = TS / 2;
    constexpr int F = WT / 16;
    constexpr int LS = TS * BK;           // elements per operand slot
    constexpr int NBLK = TS / 16;         // 1 KB blocks per operand slot
    constexpr int BPW = NBLK / 4;         // blocks per wave per operand
    constexpr int NDMA = 2 * BPW;         // direct loads per wave per step
    static_assert((NS - 1) * NDMA <= 63, "vmcnt range");
    __shared__ __attribute__((aligned(1024))) bf16 sA0[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sA1[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sA2[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sA3[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sB0[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sB1[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sB2[LS];
    __shared__ __attribute__((aligned(1024))) bf16 sB3[LS];

    // Gram: the window the host chose (xcd_window). Apply: windows of 256
    // tiles per XCD (same-box sweep on the 8B-shaped set, ms per launch:
    // contiguous 40.2, windows of 128: 40.8, 256: 39.9, 512: 40.2, 1024: 40.2;
    // other sets unchanged)
    const int win = SYM ? A.xcd_window : 256;
    const int gstat = (A.total_tiles + 7) / 8 * 8;
    // not the last apply: its epilogue loads a whole block of parameters up
    // front, and with the loop its kernel spilled 57 registers (1-12 % slower)
    const bool persist = !(EPI == 1 && !SYM) && A.grid < gstat;
    __shared__ int s_tile;
    int q = 0, ticket = 0;   // persistent: thread 0's queue, and the ticket it took for the next tile
    int wg;
    if (!persist) {
        wg = xcd_remap_window(blockIdx.x, gstat, win);
        if (wg >= A.total_tiles) return;
    } else {
        if (threadIdx.x == 0) {
            q = xcc_id();
            s_tile = next_tile(A, q, atomicAdd(A.queues + q, 1), gstat, win);
        }
        __syncthreads();
        wg = __builtin_amdgcn_readfirstlane(s_tile);
        if (wg < 0) return;
    }
    for (;;) {
        // the tile, resolved ahead by k_tilemap: one load where a search over the
        // problems' tile prefix took a chain of dependent ones
        const TileEntry te = A.tmap[wg];
        const int p = __builtin_amdgcn_readfirstlane(te.p);
        const int tij = __builtin_amdgcn_readfirstlane(te.tij);
        const NsProb P = A.probs[p];   // by value: held in registers, never re-read after a store
        const int mode = A.mode;
        const int ti = tij & 0xffff, tj = tij >> 16;

        // Gram modes: C = P Q^T over K, P and Q K-blocked with RP and RQ rows.
        // Apply: C = B X, B K-blocked (mp rows, k = mp) and X itself (mp rows,
        // k = np) as the right operand, whose k runs down X's rows (see dma_slice
        // and read_b).
        const bf16 *pm, *qm;
        int RP, RQ, K;
        if (mode == GM_GRAM || (EPI == 1 && SYM)) {   // Gram, dual Gram
            pm = qm = (const bf16*)(A.src ? P.x[1] : P.x[0]); RP = RQ = P.mp; K = P.np;
        } else if (SYM && EPI == 2) {   // pair product: P = x[0], Q = x[1]
            pm = (const bf16*)P.x[0]; qm = (const bf16*)P.x[1]; RP = RQ = P.mp; K = P.np;
        } else if (mode == GM_GRAM2) {
            pm = qm = (const bf16*)P.a; RP = RQ = P.mp; K = P.mp;
        } else {
            pm = (const bf16*)(A.use_b ? P.b : P.a); RP = P.mp;
            qm = (const bf16*)(A.src ? P.x[1] : P.x[0]); RQ = P.mp; K = P.mp;
        }

        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;

        auto slot_a = [&](auto st) -> bf16* {
            constexpr int S = decltype(st)::value;
            if constexpr (S == 0) return sA0;
            else if constexpr (S == 1) return sA1;
            else if constexpr (S == 2) return sA2;
            else return sA3;
        };
        auto slot_b = [&](auto st) -> bf16* {
            constexpr int S = decltype(st)::value;
            if constexpr (S == 0) return sB0;
            else if constexpr (S == 1) return sB1;
            else if constexpr (S == 2) return sB2;
            else return sB3;
        };

        // Direct loads. The TS x 32 slice kt of a K-blocked operand tile is NBLK
        // contiguous 1 KB blocks starting at block kt*R/16 + tile*TS/16; a buffer
        // resource covering exactly that run (an offset outside it reads zeros
        // instead of faulting) is built per step from the wave-uniform address.
        // Block b of the slice goes to block b of the slot, lane l moving bytes
        // 16l..16l+15: a plain 1 KB copy, eight whole 128-byte lines per
        // instruction.
        // The apply's right operand is X: slice kt is rows 32kt .. 32kt+31 of the
        // tile's TS columns, i.e. row groups 2kt and 2kt+1 of TS/32 k-panels, two
        // adjacent blocks per panel with panels mp/16 blocks apart. Slot block
        // 2*panel + group holds it, its 16-byte chunks permuted: chunk (c, r) of
        // the X block (k chunk c, row r) sits at slot chunk (c, r ^ 4*(c&1)),
        // which keeps the transposed fragment reads below free of bank conflicts.
        const uint32_t lane_off = (uint32_t)lane * 16u;
        const uint32_t lane_xoff = (uint32_t)(256 * (lane >> 4) + 16 * ((lane & 15) ^ (4 * ((lane >> 4) & 1))));
        const uint32_t x_pan = (uint32_t)(RQ >> 4) * 1024u;   // bytes between k-panels of X
        auto slice = [&](const bf16* base, int R, int tile, int kt) {
            return __builtin_amdgcn_make_buffer_rsrc(
                (void*)(base + ((int64_t)kt * (R >> 4) + (int64_t)tile * (TS >> 4)) * 512), 0, NBLK * 1024, BUF_RAW32);
        };
        auto slice_x = [&](int kt) {
            return __builtin_amdgcn_make_buffer_rsrc(
                (void*)(qm + ((int64_t)tj * (TS / 32) * (RQ >> 4) + 2 * kt) * 512), 0, (TS / 32 - 1) * x_pan + 2048u,
                BUF_RAW32);
        };
        auto dma_slice = [&](auto st, int kt, auto first, auto count) {
            constexpr int I0 = decltype(first)::value, NI = decltype(count)::value;
            const __amdgpu_buffer_rsrc_t ra = slice(pm, RP, ti, kt);
            __amdgpu_buffer_rsrc_t rb;
            if constexpr (SYM) rb = slice(qm, RQ, tj, kt);
            else rb = slice_x(kt);
            static_for<I0, I0 + NI>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                constexpr bool isA = i < BPW;
                const int b = (isA ? i : i - BPW) * 4 + wave;
                bf16* dst = (isA ? slot_a(st) : slot_b(st)) + b * 512;
                if (isA || SYM)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? ra : rb, (LDSP void*)dst, 16, lane_off,
                                                             (uint32_t)b * 1024u, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rb, (LDSP void*)dst, 16, lane_xoff, (uint32_t)(b >> 1) * x_pan + (uint32_t)(b & 1) * 1024u, 0, 0);
            });
        };
        auto dma = [&](auto st, int kt) { dma_slice(st, kt, Stage<0>{}, Stage<NDMA>{}); };
        auto read_a = [&](auto st, int fm) -> bf16x8 {
            return *(const bf16x8*)(slot_a(st) + (wm0 + fm * 16) * BK + lane * 8);
        };
        // Apply fragment fn (X columns wn0 + 16fn ..): lane l needs rows
        // 8(l>>4) .. +7 of column l&15. ds_read_b64_tr_b16 hands lane i of each
        // 16-lane group element i%4 of the 4-element run addressed by lane
        // 4j + i/4 as its element j; lane i addresses row r0 + i/4, columns
        // 4(i%4) .. +3 (r0 = 8(l>>4), then r0 + 4), so it receives column i of
        // those four rows. Slot block 2*(wn0/32 + fn/2) + (l>>5), k chunk
        // 2(fn&1) + ((i>>1)&1).
        const int trs = (lane >> 1) & 1;
        const int tr_row = 8 * ((lane >> 4) & 1) + ((lane & 15) >> 2);
        const uint32_t tr_lane = (uint32_t)(1024 * (lane >> 5) + 256 * trs + 8 * (lane & 1));
        const uint32_t tr0 = tr_lane + 16u * (uint32_t)(tr_row + 4 * trs);
        const uint32_t tr1 = tr_lane + 16u * (uint32_t)(tr_row + 4 * (trs ^ 1));
        auto read_b = [&](auto st, int fn) -> bf16x8 {
            if constexpr (SYM) {
                return *(const bf16x8*)(slot_b(st) + (wn0 + fn * 16) * BK + lane * 8);
            } else {
                const char* blk = (const char*)slot_b(st) + (wn0 / 32 + fn / 2) * 2048 + (fn & 1) * 512;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP i16x4*)(blk + tr0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP i16x4*)(blk + tr1));
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        };

        f32x4 acc[F][F];
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
            for (int j = 0; j < F; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        bf16x8 a0[F], b0[F], a1[F], b1[F];
        const int KT = K / BK;   // a multiple of NS: K is a multiple of 128

        dma(Stage<0>{}, 0);
        dma(Stage<1>{}, 1);
        dma(Stage<2>{}, 2);
        dma(Stage<3>{}, 3);
        MU_WAIT_VMCNT((NS - 1) * NDMA);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int fn = 0; fn < F; ++fn) b0[fn] = read_b(Stage<0>{}, fn);
#pragma unroll
        for (int fm = 0; fm < F; ++fm) a0[fm] = read_a(Stage<0>{}, fm);

        // The body is emitted in the exact issue order wanted and fenced with
        // sched_barrier, so the MFMA stream is never starved: with one wave per
        // SIMD the matrix core drains within a couple of MFMAs of any gap. Next
        // fragments are read B first: phase A of the next step needs all of B and
        // the first HEAD rows of A. Slice indices past the end are clamped, so the
        // last loads refill slots nobody reads again instead of branching.
        constexpr int HEAD = F / 4 > 0 ? F / 4 : 1;
        constexpr int G = 2 * F;                 // fragment reads per step
        constexpr int NMB = (F - HEAD) * F;      // MFMAs after the barrier
        // one MFMA on accumulator tile idx (row-major over the F x F fragments);
        // the instruction is written out so that the accumulators stay pinned in
        // AGPRs across the loop (the builtin lets the allocator shuffle them)
        auto mma_acc = [](auto idx, f32x4 (&c)[F][F], const bf16x8 (&af)[F], const bf16x8 (&bfv)[F]) {
            constexpr int fm = decltype(idx)::value / F, fn = decltype(idx)::value % F;
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c[fm][fn]) : "v"(af[fm]), "v"(bfv[fn]));
        };
        auto mma = [&](auto idx, const bf16x8 (&af)[F], const bf16x8 (&bfv)[F]) { mma_acc(idx, acc, af, bfv); };
        auto step = [&](auto domma, auto st, int kt, const bf16x8 (&ac)[F], const bf16x8 (&bc)[F], bf16x8 (&an)[F],
                        bf16x8 (&bn)[F]) {
            constexpr int DM = decltype(domma)::value;
            constexpr bool DO = DM != 0;
            // one MFMA, or none for a fragment below the diagonal (DM == 2)
            auto mmaw = [&](auto j) {
                constexpr int idx = decltype(j)::value;
                if constexpr (DM != 2 || idx / F <= idx % F) mma(j, ac, bc);
            };
            constexpr int S = decltype(st)::value;
            using SN = Stage<(S + 1) % NS>;
            if constexpr (S == 0) {
                // loop head: two wait states after the accumulator zeroing
                // (a VALU write read as SrcC), which the compiler cannot see here
                asm volatile("s_nop 1");
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (DO) static_for<0, HEAD * F>([&](auto j) { mmaw(j); });
            __builtin_amdgcn_sched_barrier(0);
            MU_WAIT_VMCNT_LGKM0((NS - 2) * NDMA);
            __builtin_amdgcn_s_barrier();
            const int kn = min(kt + NS, KT - 1);
            static_for<0, G>([&](auto gc) {
                constexpr int g = decltype(gc)::value;
                // the loads of this group: i with i*G/NDMA == g
                constexpr int i0 = (g * NDMA + G - 1) / G, i1 = ((g + 1) * NDMA + G - 1) / G;
                if constexpr (i1 > i0) dma_slice(st, kn, Stage<i0>{}, Stage<i1 - i0>{});
                if constexpr (DO) {
                    if constexpr (g < F) bn[g] = read_b(SN{}, g);
                    else an[g - F] = read_a(SN{}, g - F);
                    static_for<HEAD * F + g * NMB / G, HEAD * F + (g + 1) * NMB / G>([&](auto j) { mmaw(j); });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        auto kloop = [&](auto domma) {
            for (int kt = 0; kt < KT; kt += NS) {
                step(domma, Stage<0>{}, kt, a0, b0, a1, b1);
                step(domma, Stage<1>{}, kt + 1, a1, b1, a0, b0);
                step(domma, Stage<2>{}, kt + 2, a0, b0, a1, b1);
                step(domma, Stage<3>{}, kt + 3, a1, b1, a0, b0);
            }
        };
        // On a diagonal Gram tile the wave below the diagonal would compute the
        // transpose of the wave above it: it only keeps the loads and barriers
        // going, and the epilogue of the wave above writes both quadrants. The
        // two waves on the diagonal compute only their fragments on or above it
        // and mirror those. Under the power limit the saved MFMA work (3 % of the
        // 8B-shaped Gram for the skipped quadrant) gave 0.7 %.
        if constexpr (SYM) {
            if (ti == tj && wm0 > wn0) kloop(Stage<0>{});
            else if (ti == tj && wm0 == wn0) kloop(Stage<2>{});
            else kloop(Stage<1>{});
        } else {
            kloop(Stage<1>{});
        }
        // The MFMAs above are opaque to the compiler's hazard recognizer: give the
        // last ones the wait states (>= passes + 2) that an accumulator read needs.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        MU_WAIT_VMCNT(0);
        __syncthreads();
        // epilogue staging: two slot arrays per wave
        static_assert(LS * sizeof(bf16) == (WT / 2) * 64 * sizeof(float), "a staging half is WT/2 x 64 floats");
        float* st = (float*)(wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sA2 : sA3);
        float* st2 = (float*)(wave == 0 ? sB0 : wave == 1 ? sB1 : wave == 2 ? sB2 : sB3);
        // the next tile's ticket, taken here so that the epilogue hides its latency
        // (and after the K loop, whose waits count only the direct loads)
        if (persist && threadIdx.x == 0) ticket = atomicAdd(A.queues + q, 1);
        epilogue_k<SYM, EPI, bf16, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, st, st2);
        if (!persist) return;
        __syncthreads();   // every wave is done with the LDS: its staging is the next tile's ring
        if (threadIdx.x == 0) s_tile = next_tile(A, q, ticket, gstat, win);
        __syncthreads();
        wg = __builtin_amdgcn_readfirstlane(s_tile);
        if (wg < 0) return;
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64x64 tiles, BK = 32, v_mfma_f32_16x16x4_f32, operands staged
// through registers into padded LDS rows. Within a block of 16 k, lane l holds
// k = 4*(l>>4) + s in MFMA s for both operands (any permutation of k shared by
// both operands leaves the sum unchanged).
// ---------------------------------------------------------------------------
template <int TS, bool SYM, typename TSRC>
__global__ __launch_bounds__(NTHR) void k_gemm_f32(GemmArgs A) {
    constexpr int BK = 32, WT = TS / 2, F = WT / 16;
    constexpr int SPK = BK + 4;
    constexpr int LA = TS * SPK;
    constexpr int NL = TS * BK / 4 / NTHR;   // 16-byte loads per operand per thread and step
    __shared__ __attribute__((aligned(16))) float smem[2 * 2 * LA];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    if (wg >= A.total_tiles) return;
    // the tile, resolved ahead by k_tilemap: one load where a search over the
    // problems' tile prefix took a chain of dependent ones
    const TileEntry te = A.tmap[wg];
    const int p = __builtin_amdgcn_readfirstlane(te.p);
    const int tij = __builtin_amdgcn_readfirstlane(te.tij);
    const NsProb P = A.probs[p];   // by value: held in registers, never re-read after a store
    const int mode = A.mode;
    const int ti = tij & 0xffff, tj = tij >> 16;

    const float *pm, *qm;
    int ldp, ldq, K;
    if (mode == GM_GRAM) {
        pm = qm = (const float*)(A.src ? P.x[1] : P.x[0]); ldp = ldq = P.np; K = P.np;
    } else if (mode == GM_GRAM2) {
        pm = qm = (const float*)P.a; ldp = ldq = P.mp; K = P.mp;
    } else {
        pm = (const float*)(A.use_b ? P.b : P.a); ldp = P.mp;
        qm = (const float*)(A.src ? P.xt[1] : P.xt[0]); ldq = P.mp; K = P.mp;
    }
    const float* pt = pm + (int64_t)ti * TS * ldp;
    const float* qt = qm + (int64_t)tj * TS * ldq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave >> 1) * WT, wn0 = (wave & 1) * WT;

    f32x4 ga[NL], gb[NL];
    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int s = 0; s < NL; ++s) {
            const int q = s * NTHR + tid;
            ga[s] = *gp((const f32x4*)(pt + (int64_t)(q >> 3) * ldp + k0 + (q & 7) * 4));
            gb[s] = *gp((const f32x4*)(qt + (int64_t)(q >> 3) * ldq + k0 + (q & 7) * 4));
        }
    };
    auto sstore = [&](int stage) {
        float* as = smem + stage * 2 * LA;
        float* bs = as + LA;
#pragma unroll
        for (int s = 0; s < NL; ++s) {
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
    // the epilogue reads the accumulators with opaque v_accvgpr_read: give the
    // last MFMAs their wait states
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // epilogue staging per wave: the 16-row strip, and with 4 x 4 fragments
    // the last apply's two halves of WT/2 x 64 floats
    if constexpr (F % 4 == 0) {
        constexpr int STG = (WT / 2) * 64;
        static_assert(STG >= 16 * (WT + 4) && 8 * STG <= 2 * 2 * LA, "staging fits the stage buffers");
        float* st = smem + wave * 2 * STG;
        epilogue<SYM, float, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, st, st + STG);
    } else {
        epilogue<SYM, float, TSRC, F>(A, P, ti, tj, TS, wm0, wn0, acc, smem + wave * 16 * (WT + 4), nullptr);
    }
}

// ---------------------------------------------------------------------------
// Newton-Schulz for one problem with mp == 128 (a 128-row head block, or any
// matrix whose short side is at most 128) in one workgroup, up to the last
// apply. Such short, wide problems are bound by HBM, and the tiled path moves X
// through it three times per step (the Gram reads X, the apply reads X and
// writes X'). Here B (128 x 128) stays on chip and each step streams X once,
// in blocks of 128 columns (one contiguous 32 KB run each):
//   X'_j^T = X_j^T B        (X_j through transposed LDS reads, B from
//                            registers; B is symmetric, so this is (B X_j)^T)
//   A' += X'_j X'_j^T       (from a K-blocked LDS copy of X'_j, bf16 as stored)
//   X'_j -> HBM             (that LDS copy, which has X's layout: the next
//                            step's input)
// and the next step's B = a' I + b' A' is written into LDS from the symmetric
// A'. The first B = f (a I + b f^2 X0 X0^T) comes from one pass over X0. The
// B of the last step is copied to the problem's `a` buffer, and the tiled last
// apply (which fuses the parameter update) finishes the run.
// LDS traffic is kept low: each wave holds its 64 rows of B in registers for
// the whole step (loaded from LDS once per step), and computing X'^T puts,
// after a lane swap, 8 consecutive columns of one row of X' in a lane: one
// 16-byte chunk of the K-blocked copy, written to LDS straight from registers
// with no float staging (288 KB of LDS traffic per block, against 480 KB for
// B X with B read from LDS and X' staged as floats). The loads of block j+1
// are issued before block j's apply; the barrier after the copy waits for LDS
// writes only, but the compiler drains the direct loads before the first
// write of X'_j into the staging buffer (it cannot tell the two LDS buffers
// apart), so the loads overlap the apply and not the store or the Gram.
// Per-head set, same process: 1.465 -> 1.399 ms per launch, results bit for
// bit the same. (Two workgroups per compute unit, with 64-column blocks in
// 80 KB of LDS, ran 6 % slower.)
// 4 waves in 2 x 2: the apply 64 x 64 of X'^T (64 AGPRs), the Gram 64 x 64 of
// A' (64 AGPRs).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTHR) void k_ns_small(SmallArgs A) {
    constexpr int M = 128, BK = 32, BW = 128;
    constexpr int SLICE = M * BK;   // a 32-wide k-slice of a 128-row K-blocked operand (8 KB)
    constexpr int OPB = 4 * SLICE;  // a 128 x 128 operand (32 KB)
    constexpr int XB = 4 * SLICE;   // a 128 x 128 block of X (32 KB)
    constexpr int FG = 4;           // Gram fragments per wave side (64 x 64)
    __shared__ __attribute__((aligned(1024))) bf16 sB[OPB];   // B
    __shared__ __attribute__((aligned(1024))) bf16 sX0[XB];   // X blocks, even j
    __shared__ __attribute__((aligned(1024))) bf16 sX1[XB];   // odd j
    __shared__ __attribute__((aligned(1024))) bf16 sG[XB];    // X'_j, both operands of the Gram

    if ((int)blockIdx.x >= A.nprobs) return;
    const NsProb P = A.probs[blockIdx.x];   // by value: held in registers
    const int np = P.np, NB = np / BW;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int gm0 = (wave >> 1) * 64, gn0 = (wave & 1) * 64;   // Gram: rows / columns of A'
    const int ar0 = (wave >> 1) * 64, ac0 = (wave & 1) * 64;   // apply: rows / columns of X'_j

    // Block j of X (columns 128j .. 128j+127) is one contiguous 32 KB run of
    // X's K-blocked layout (mp = 128): k-panel p (columns 32p ..) is the 8 KB
    // at 4096p, row group g the 1 KB at 512g inside it. It is copied into LDS
    // in that order; wave w moves 1 KB blocks w, w+4, .. With `permute`, each
    // block's 16-byte chunks are permuted as for the tiled apply (chunk (c, r)
    // at (c, r ^ 4(c&1))) for the transposed reads of the apply below.
    const uint32_t lane_off = (uint32_t)lane * 16u;
    const uint32_t lane_xoff = (uint32_t)(256 * (lane >> 4) + 16 * ((lane & 15) ^ (4 * ((lane >> 4) & 1))));
    auto dma_block = [&](bf16* dst, const bf16* base, int j, bool permute) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)j * XB), 0, XB * 2, BUF_RAW32);
#pragma unroll
        for (int i = 0; i < XB / 512 / 4; ++i) {
            const int b = i * 4 + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDSP void*)(dst + b * 512), 16,
                                                     permute ? lane_xoff : lane_off, (uint32_t)b * 1024u, 0, 0);
        }
    };
    // fragment of a K-blocked 128-row operand: rows row .. row+15, k-panel sl
    auto frag = [&](const bf16* buf, int sl, int row) -> bf16x8 {
        return *(const bf16x8*)(buf + sl * SLICE + row * BK + lane * 8);
    };
    // fragment of a permuted X block as the left operand of X^T B: column
    // col0 + (lane&15) of X, rows 32sl + 8(lane>>4) .. +7 (k); two transposed
    // reads, lane addressing as in the tiled apply
    const int trs = (lane >> 1) & 1;
    const int tr_row = 8 * ((lane >> 4) & 1) + ((lane & 15) >> 2);
    const uint32_t tr_lane = (uint32_t)(1024 * (lane >> 5) + 256 * trs + 8 * (lane & 1));
    const uint32_t tr0 = tr_lane + 16u * (uint32_t)(tr_row + 4 * trs);
    const uint32_t tr1 = tr_lane + 16u * (uint32_t)(tr_row + 4 * (trs ^ 1));
    auto frag_x = [&](const bf16* buf, int sl, int col0) -> bf16x8 {
        const char* blk = (const char*)buf + ((col0 >> 5) * 8 + 2 * sl) * 1024 + ((col0 >> 4) & 1) * 512;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP i16x4*)(blk + tr0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP i16x4*)(blk + tr1));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // apply accumulators: acc[i][jj] = X'^T rows ac0 + 16i .. (columns of X'),
    // columns ar0 + 16jj .. (rows of X')
    f32x4 acc[4][4], accg[FG][FG];
    bf16x8 bR[M / BK][4];   // this wave's rows ar0 .. ar0+63 of B, as the right operand of X^T B
    // one MFMA, written out so that the accumulators stay pinned in AGPRs
    auto mma = [](f32x4& c, const bf16x8& a, const bf16x8& b) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    };
    // A' (this wave's 64 x 64) += X'_j X'_j^T over the block's 64 columns
    auto gram_block = [&](const bf16* Gb) {
#pragma unroll
        for (int sl = 0; sl < BW / BK; ++sl) {
            bf16x8 a[FG], b[FG];
#pragma unroll
            for (int i = 0; i < FG; ++i) {
                a[i] = frag(Gb, sl, gm0 + i * 16);
                b[i] = frag(Gb, sl, gn0 + i * 16);
            }
#pragma unroll
            for (int i = 0; i < FG; ++i)
#pragma unroll
                for (int jn = 0; jn < FG; ++jn) mma(accg[i][jn], a[i], b[jn]);
        }
    };
    // B's rows ar0 .. ar0+63 into registers (B[k][r] = B[r][k]: a right-
    // operand fragment of column r is row r of B)
    auto load_b = [&]() {
#pragma unroll
        for (int sl = 0; sl < M / BK; ++sl)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bR[sl][jj] = frag(sB, sl, ar0 + jj * 16);
    };
    // X'_j^T (this wave's 64 x 64) = X_j^T B over the 128 rows of X_j
    auto apply_block = [&](const bf16* Xb) {
#pragma unroll
        for (int sl = 0; sl < M / BK; ++sl) {
            bf16x8 a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = frag_x(Xb, sl, ac0 + i * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) mma(acc[i][jj], a[i], bR[sl][jj]);
        }
    };
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        // two wait states before an MFMA reads the cleared accumulators
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 1");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto zero_gram = [&]() {
#pragma unroll
        for (int i = 0; i < FG; ++i)
#pragma unroll
            for (int jn = 0; jn < FG; ++jn) accg[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 1");
        __builtin_amdgcn_sched_barrier(0);
    };
    // the inline-asm MFMAs are opaque to the hazard recognizer: wait states
    // before their accumulators are read back
    auto mfma_drain = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // the lane swap of two fragments adjacent in columns: lane gets
    // w[e] = C[r0 + e][col], r0 = 8*(g4>>1) + the pair's first row, col =
    // (fp + (g4&1))*16 + l16 of the pair's columns
    auto swap_pair = [&](const float (&v0)[4], const float (&v1)[4], float* w) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto sw =
                __builtin_amdgcn_permlane16_swap(__float_as_uint(v0[e]), __float_as_uint(v1[e]), false, false);
            w[e] = __uint_as_float(sw[0]);
            w[4 + e] = __uint_as_float(sw[1]);
        }
    };
    // B = gd I + gs A' into sB from the symmetric A' (row col of B is column
    // col of A')
    auto build_b = [&](float gs, float gd) {
        mfma_drain();
#pragma unroll
        for (int fm = 0; fm < FG; ++fm) {
            float av[FG][4];
#pragma unroll
            for (int fn = 0; fn < FG; ++fn)
#pragma unroll
                for (int e = 0; e < 4; ++e) av[fn][e] = agpr_read(accg[fm][fn][e]);
#pragma unroll
            for (int fp = 0; fp < FG; fp += 2) {
                float w[8];
                swap_pair(av[fp], av[fp + 1], w);
                const int col = gn0 + (fp + (g4 & 1)) * 16 + l16, r0 = gm0 + fm * 16 + 8 * (g4 >> 1);
                bf16x8 q;
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = (bf16)(gs * w[e] + (col == r0 + e ? gd : 0.f));
                *(bf16x8*)(sB + kb_off(col, r0, M)) = q;
            }
        }
    };
    // X'_j from the apply accumulators into sG (K-blocked, 128 rows, 128
    // columns): after the swap a lane holds columns c0 .. c0+7 of row r
    auto store_xp = [&]() {
        mfma_drain();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float av[4][4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int e = 0; e < 4; ++e) av[jj][e] = agpr_read(acc[i][jj][e]);
#pragma unroll
            for (int jp = 0; jp < 4; jp += 2) {
                float w[8];
                swap_pair(av[jp], av[jp + 1], w);
                const int r = ar0 + (jp + (g4 & 1)) * 16 + l16, c0 = ac0 + i * 16 + 8 * (g4 >> 1);
                bf16x8 q;
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = (bf16)w[e];
                *(bf16x8*)(sG + kb_off(r, c0, M)) = q;
            }
        }
    };

    const bf16* x0 = (const bf16*)P.x[0];
    const float f = P.fold[0];

    // A0 = X0 X0^T, one pass over X0
    zero_gram();
    dma_block(sX0, x0, 0, false);
    auto gram0 = [&](int j, bf16* cur, bf16* nxt) {
        __syncthreads();   // block j landed; everyone is done with `nxt`
        if (j + 1 < NB) dma_block(nxt, x0, j + 1, false);
        gram_block(cur);
    };
    for (int j = 0; j < NB; j += 2) {
        gram0(j, sX0, sX1);
        if (j + 1 < NB) gram0(j + 1, sX1, sX0);
    }
    __syncthreads();
    build_b(A.cb[0] * f * f * f, A.ca[0] * f);

    // every step but the last: X' from x[k&1] into x[(k+1)&1], next B in sB
    // (the X of the last step is then in x[(ns_steps - 1) & 1])
    for (int k = 0; k + 1 < A.ns_steps; ++k) {
        const bf16* xin = (const bf16*)((k & 1) ? P.x[1] : P.x[0]);
        bf16* xout = (bf16*)((k & 1) ? P.x[0] : P.x[1]);
        __syncthreads();   // B written by every wave
        load_b();
        zero_gram();
        dma_block(sX0, xin, 0, true);
        auto step_block = [&](int j, bf16* cur, bf16* nxt) {
            __syncthreads();   // block j landed, the previous block's stores done; `nxt` and sG free
            if (j + 1 < NB) dma_block(nxt, xin, j + 1, true);
            zero_acc();
            apply_block(cur);
            store_xp();
            // X'_j complete in sG: a barrier on the LDS writes only (a full
            // __syncthreads would also wait for the loads of block j+1, just
            // issued, which then could not overlap this block's work)
            MU_WAIT_LGKM0();
            __builtin_amdgcn_s_barrier();
            {
                // sG is X'_j K-blocked with 128 rows, which is exactly the
                // 16 KB run of X (mp = 128) holding columns 64j .. 64j+63;
                // stored non-temporally (read back only by the next step)
                bf16* xd = xout + (int64_t)j * XB;
#pragma unroll
                for (int i = 0; i < XB / (NTHR * 8); ++i) {
                    const int o = (i * NTHR + tid) * 8;
                    __builtin_nontemporal_store(*(const bf16x8*)(sG + o), gp((bf16x8*)(xd + o)));
                }
            }
            gram_block(sG);
        };
        for (int j = 0; j < NB; j += 2) {
            step_block(j, sX0, sX1);
            if (j + 1 < NB) step_block(j + 1, sX1, sX0);
        }
        build_b(A.cb[k + 1], A.ca[k + 1]);
    }
    // the last step's B -> the problem's `a` buffer (same K-blocked layout)
    __syncthreads();
    bf16* ad = (bf16*)P.a;
#pragma unroll
    for (int i = 0; i < OPB / (NTHR * 8); ++i) {
        const int o = (i * NTHR + tid) * 8;
        *gp((bf16x8*)(ad + o)) = *(const bf16x8*)(sB + o);
    }
}

template <int TS, bool SYM>
hipError_t launch_bf16_t(const GemmArgs& a, hipStream_t s) {
    const unsigned grid = (unsigned)a.grid;
    // the parameter dtype matters only to the last apply's update
    if (!SYM && a.mode == GM_APPLY_LAST) {
        if (a.src_dtype == DT_BF16)
            hipLaunchKernelGGL((k_gemm_bf16<TS, false, bf16, 1>), dim3(grid), dim3(NTHR), 0, s, a);
        else
            hipLaunchKernelGGL((k_gemm_bf16<TS, false, float, 1>), dim3(grid), dim3(NTHR), 0, s, a);
    } else if (SYM && a.mode == GM_GRAM_DUAL) {
        hipLaunchKernelGGL((k_gemm_bf16<TS, true, bf16, 1>), dim3(grid), dim3(NTHR), 0, s, a);
    } else if (SYM && a.mode == GM_GRAM_PAIR) {
        hipLaunchKernelGGL((k_gemm_bf16<TS, true, bf16, 2>), dim3(grid), dim3(NTHR), 0, s, a);
    } else {
        hipLaunchKernelGGL((k_gemm_bf16<TS, SYM, bf16, 0>), dim3(grid), dim3(NTHR), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int tile, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    const int gstat = (a.total_tiles + 7) / 8 * 8;
    const bool sym = gemm_mode_sym(a.mode);
    if (a.grid < 1 || a.grid > gstat || (a.grid < gstat && (!a.queues || a.mode == GM_APPLY_LAST)))
        return hipErrorInvalidValue;
    if (tile == 256) return sym ? launch_bf16_t<256, true>(a, s) : launch_bf16_t<256, false>(a, s);
    if (tile == 128) return sym ? launch_bf16_t<128, true>(a, s) : launch_bf16_t<128, false>(a, s);
    return hipErrorInvalidValue;
}

template <int TS>
hipError_t launch_f32_t(const GemmArgs& a, hipStream_t s) {
    const bool sym = gemm_mode_sym(a.mode);
    const unsigned grid = (unsigned)((a.total_tiles + 7) / 8 * 8);
    if (a.src_dtype == DT_BF16) {
        if (sym) hipLaunchKernelGGL((k_gemm_f32<TS, true, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f32<TS, false, bf16>), dim3(grid), dim3(NTHR), 0, s, a);
    } else {
        if (sym) hipLaunchKernelGGL((k_gemm_f32<TS, true, float>), dim3(grid), dim3(NTHR), 0, s, a);
        else hipLaunchKernelGGL((k_gemm_f32<TS, false, float>), dim3(grid), dim3(NTHR), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, int tile, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    if (a.mode == GM_GRAM_DUAL || a.mode == GM_GRAM_PAIR) return hipErrorInvalidValue;   // bf16 only
    if (tile == 64) return launch_f32_t<64>(a, s);
    if (tile == 128) return launch_f32_t<128>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_tilemap(const TileMapArgs& a, hipStream_t s) {
    const int n = a.total > a.nqueues ? a.total : a.nqueues;
    if (n <= 0) return hipSuccess;
    if (a.nseg < 0 || a.nseg > TILEMAP_SEGS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_tilemap, dim3((unsigned)((n + NTHR - 1) / NTHR)), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ns_small(const SmallArgs& a, hipStream_t s) {
    if (a.nprobs <= 0) return hipSuccess;
    if (a.ns_steps < 1 || a.ns_steps > SMALL_MAX_STEPS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_ns_small, dim3(a.nprobs), dim3(NTHR), 0, s, a);
    return hipGetLastError();
}

}  // namespace mu
