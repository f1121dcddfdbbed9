// C ABI of the Muon + AdamW step: validation, planning, workspace layout,
// descriptor upload and launch order. Host code only; kernels live in
// elementwise.hip and ns_gemm.hip.
//
// Muon step order per call (MuonClip Optimizer page, "Momentum" and
// "Newton-Schulz Orthogonalization"; Qwen training-details page, "Confirmed",
// for per-head blocks):
//   prep (all problems) -> norm (all problems) ->
//   [fused short blocks: every step but the last apply, one launch] ->
//   for each step: Gram [-> Gram2 for a quintic term] -> apply
//   (the last apply writes the updated parameter, for the fused blocks too;
//   ns_steps == 0 uses finish).
// AdamW: one launch over the flat tensor list (nanochat optimizer page,
// "AdamW Step Implementation").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon_mi355x.h"
#include "common.hpp"
#include "launch.hpp"

using namespace mu;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MU_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x, size_t a = ALIGN) { return (x + a - 1) / a * a; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

size_t dtype_size(int dt) { return dt == MU_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// Buffer overlap check over all device ranges of one call.
// ---------------------------------------------------------------------------
struct Range {
    uintptr_t lo, hi;
    int owner;
};

bool ranges_overlap(std::vector<Range>& r) {
    std::sort(r.begin(), r.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < r.size(); ++i)
        if (r[i].lo < r[i - 1].hi) return true;
    return false;
}

// ---------------------------------------------------------------------------
// Coefficients
// ---------------------------------------------------------------------------
struct Coeff {
    float a, b, c;
};

std::vector<Coeff> coeffs_of(const mu_muon_hparams* hp) {
    std::vector<Coeff> out((size_t)hp->ns_steps);
    for (int k = 0; k < hp->ns_steps; ++k) {
        if (hp->coeffs) out[k] = {hp->coeffs[3 * k], hp->coeffs[3 * k + 1], hp->coeffs[3 * k + 2]};
        else out[k] = {1.5f, -0.5f, 0.f};  // cubic step of the pages
    }
    return out;
}

int check_hparams(const mu_muon_hparams* hp, bool need_update_terms) {
    if (!hp) return fail(MU_ERR_INVALID_ARG, "hparams is null");
    if (hp->ns_steps < 0) return fail(MU_ERR_INVALID_ARG, "ns_steps must be >= 0 (got %d)", hp->ns_steps);
    if (hp->ns_steps > 1000) return fail(MU_ERR_INVALID_ARG, "ns_steps too large (%d)", hp->ns_steps);
    if (hp->ns_precision != MU_NS_F32 && hp->ns_precision != MU_NS_BF16)
        return fail(MU_ERR_DTYPE, "unknown ns_precision %d", hp->ns_precision);
    if (!(hp->norm_eps >= 0.f) || !std::isfinite(hp->norm_eps)) return fail(MU_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
    if (need_update_terms) {
        if (!std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay) || !std::isfinite(hp->mu))
            return fail(MU_ERR_INVALID_ARG, "lr, weight_decay and mu must be finite");
    }
    if (hp->coeffs) {
        for (int i = 0; i < 3 * hp->ns_steps; ++i)
            if (!std::isfinite(hp->coeffs[i])) return fail(MU_ERR_INVALID_ARG, "coefficient %d is not finite", i);
    }
    return MU_OK;
}

// ---------------------------------------------------------------------------
// Planning. A problem is one head block. Problems are ordered by GEMM tile so
// that each tile group is contiguous in the descriptor table.
// ---------------------------------------------------------------------------
struct ProbPlan {
    NsProb d;          // device descriptor (buffer pointers filled at carve time)
    int tile;          // GEMM tile edge
    size_t x_bytes, a_bytes;
};

struct Group {
    int tile;
    int first, count;  // range in the problem array
    bool fused;        // mp == 128 problems run by k_ns_small up to the last apply
    int gram_window;   // GemmArgs::xcd_window of the Gram launches
    std::vector<int> gram_order;   // group-local problem index at each Gram prefix position
    std::vector<int> apply_order;  // the same for the apply
    std::vector<int> gram_prefix, apply_prefix;
};

// Gram tile order and XCD windows. The Gram launches walk a group's problems
// in order of falling K (np), then falling m (gram_order), and hand the tile
// order to the XCDs in windows, so that all XCDs work on problems of the same K
// at a time and the long ones start first. The apply walks the problems in the
// reverse order (apply_order), starting on those whose B the Gram wrote last
// and which the Infinity Cache still holds (same box, ms per apply launch,
// table order against reverse: GPT-2-small-shaped 0.162 -> 0.158,
// Llama-1B-shaped 4.09 -> 4.07, Llama-3-8B-shaped unchanged within 0.5 %).
// Window per XCD: 64 when most of the Gram flops come from K >= 12288 (a
// tile's two strips of X, 6 MB and more, exceed an XCD's 4 MB L2, and tiles
// sharing a strip must stay close), 4 for launches of under four tiles per
// CU, 8 otherwise. Same-box ms per Gram launch, table order with the plain
// contiguous split (windows of 64 on the 8B set) against this scheme:
// Llama-3-8B-shaped 21.56 -> 20.61, Llama-1B-shaped 2.00 -> 1.92 (windows of
// 8; the contiguous split on the sorted order: 3.76), GPT-2-small-shaped
// 0.101 -> 0.081 (windows of 4; of 8: 0.094).
constexpr int GW_SMALL = 4, GW_MID = 8;
constexpr int MI355X_CUS = 256;   // compute units of the one chip this library targets
int gram_window_for(const std::vector<ProbPlan>& probs, int first, int count, int tiles) {
    double all = 0, long_k = 0;
    for (int i = first; i < first + count; ++i) {
        const double m = probs[i].d.mp, k = probs[i].d.np;
        all += m * m * k;
        if (k >= 12288) long_k += m * m * k;
    }
    if (all > 0 && long_k > 0.5 * all) return 64;
    return tiles < 4 * MI355X_CUS ? GW_SMALL : GW_MID;
}

// Problems with mp == 128 go through the fused kernel (one workgroup per
// problem, every step but the last in one launch) when a call has at least
// this many of them; with fewer, the tiled path spreads each problem over more
// workgroups and wins. A fixed count, so that the workspace query and the call
// always plan alike.
constexpr int FUSED_MIN_PROBS = 256;

struct Plan {
    std::vector<ProbPlan> probs;
    std::vector<int> prep_prefix;
    std::vector<Group> groups;
    int ns_dt;
    bool quintic;
    // workspace layout
    size_t off_table, off_prep_prefix, off_group_prefix, table_bytes;
    size_t off_partials, off_fold, off_bufs, total;
    int64_t total_parts;
};

int choose_tile(int ns_dt, int64_t m, int64_t n) {
    if (ns_dt == DT_F32) return 64;
    if (m < 256) return 128;
    // prefer 256 unless its padding costs clearly more than 128's
    const double w256 = (double)round_up(m, 256) * round_up(m, 256) * round_up(n, 256);
    const double w128 = (double)round_up(m, 128) * round_up(m, 128) * round_up(n, 128);
    return w256 <= 1.15 * w128 ? 256 : 128;
}

struct Item {       // what the planner needs from one list entry
    const void* src;
    float* mom;
    void* param;
    void* out;
    int64_t rows, cols;
    int heads;
    float scale;
    float* norm_out;
    float* oout;
    int vec;
};

void build_plan(const std::vector<Item>& items, int ns_dt, const std::vector<Coeff>& co, int src_dt, Plan& pl) {
    pl.ns_dt = ns_dt;
    pl.quintic = false;
    for (const Coeff& c : co)
        if (c.c != 0.f) pl.quintic = true;
    std::vector<ProbPlan> all;
    for (const Item& it : items) {
        const int64_t hr = it.rows / it.heads, hc = it.cols;
        for (int h = 0; h < it.heads; ++h) {
            ProbPlan pp;
            std::memset(&pp.d, 0, sizeof(pp.d));
            const int64_t off = (int64_t)h * hr * it.cols;
            const size_t es = dtype_size(src_dt);
            pp.d.src = (const char*)it.src + off * es;
            pp.d.mom = it.mom ? it.mom + off : nullptr;
            pp.d.param = it.param ? (char*)it.param + off * es : nullptr;
            pp.d.out = it.out ? (char*)it.out + off * es : nullptr;
            pp.d.ld = it.cols;
            pp.d.hr = (int32_t)hr;
            pp.d.hc = (int32_t)hc;
            pp.d.tall = hr > hc;
            pp.d.m = (int32_t)std::min(hr, hc);
            pp.d.n = (int32_t)std::max(hr, hc);
            pp.tile = choose_tile(ns_dt, pp.d.m, pp.d.n);
            pp.d.mp = (int32_t)round_up(pp.d.m, pp.tile);
            pp.d.np = (int32_t)round_up(pp.d.n, pp.tile);
            pp.d.vec = it.vec;
            pp.d.scale = it.scale;
            pp.d.norm_out = it.norm_out ? it.norm_out + h : nullptr;
            pp.d.oout = it.oout ? it.oout + off : nullptr;
            {   // prep tiles over the U-oriented buffer (X if wide, X^T if tall)
                const int rd = pp.d.tall ? pp.d.np : pp.d.mp, kd = pp.d.tall ? pp.d.mp : pp.d.np;
                pp.d.nparts = (rd / prep_rows_dt(ns_dt)) * (kd / prep_cols_dt(ns_dt));
            }
            const size_t nes = ns_dt == DT_BF16 ? 2 : 4;
            pp.x_bytes = align_up((size_t)pp.d.mp * pp.d.np * nes);
            pp.a_bytes = align_up((size_t)pp.d.mp * pp.d.mp * nes);
            all.push_back(pp);
        }
    }
    // stable order: tile 256 first, then 128 (fused problems last), then 64
    const bool fuse_ok = ns_dt == DT_BF16 && !pl.quintic && !co.empty() && co.size() <= (size_t)SMALL_MAX_STEPS;
    int n_fused = 0;
    for (auto& pp : all)
        if (fuse_ok && pp.tile == 128 && pp.d.mp == 128) ++n_fused;
    const bool fuse = n_fused >= FUSED_MIN_PROBS;
    auto is_fused = [&](const ProbPlan& pp) { return fuse && pp.tile == 128 && pp.d.mp == 128; };
    // X^T buffers: read by the fp32 apply and by the finish kernel
    // (ns_steps == 0, tall blocks); the bf16 kernels read X only
    for (auto& pp : all) pp.d.xt_used = (ns_dt == DT_F32 || co.empty()) ? 1 : 0;
    pl.probs.clear();
    pl.groups.clear();
    for (int gi = 0; gi < 4; ++gi) {
        const int t = gi == 0 ? 256 : gi == 3 ? 64 : 128;
        const bool fused = gi == 2;
        Group g;
        g.tile = t;
        g.fused = fused;
        g.first = (int)pl.probs.size();
        for (auto& pp : all)
            if (pp.tile == t && is_fused(pp) == fused) pl.probs.push_back(pp);
        g.count = (int)pl.probs.size() - g.first;
        if (g.count == 0) continue;
        g.gram_order.resize(g.count);
        for (int i = 0; i < g.count; ++i) g.gram_order[i] = i;
        std::stable_sort(g.gram_order.begin(), g.gram_order.end(), [&](int u, int v) {
            const NsProb& a = pl.probs[g.first + u].d;
            const NsProb& b = pl.probs[g.first + v].d;
            return a.np != b.np ? a.np > b.np : a.mp > b.mp;
        });
        g.apply_order.resize(g.count);
        for (int i = 0; i < g.count; ++i)
            g.apply_order[i] = g.gram_order[g.count - 1 - i];
        g.gram_prefix.assign(1, 0);
        g.apply_prefix.assign(1, 0);
        for (int i = 0; i < g.count; ++i) {
            const NsProb& dg = pl.probs[g.first + g.gram_order[i]].d;
            const int Tg = dg.mp / t;
            g.gram_prefix.push_back(g.gram_prefix.back() + Tg * (Tg + 1) / 2);
            const NsProb& d = pl.probs[g.first + g.apply_order[i]].d;
            const int T = d.mp / t;
            g.apply_prefix.push_back(g.apply_prefix.back() + T * (d.np / t));
        }
        g.gram_window = gram_window_for(pl.probs, g.first, g.count, g.gram_prefix.back());
        pl.groups.push_back(std::move(g));
    }
    pl.prep_prefix.assign(1, 0);
    pl.total_parts = 0;
    for (auto& pp : pl.probs) {
        pl.prep_prefix.push_back(pl.prep_prefix.back() + pp.d.nparts);
        pl.total_parts += pp.d.nparts;
    }
    // layout
    const size_t P = pl.probs.size();
    size_t o = 0;
    pl.off_table = o;
    o += sizeof(NsProb) * P;
    pl.off_prep_prefix = o;
    o += sizeof(int) * (P + 1);
    pl.off_group_prefix = o;
    for (auto& g : pl.groups) o += sizeof(int) * (g.gram_order.size() + g.apply_order.size() + g.gram_prefix.size() + g.apply_prefix.size());
    pl.table_bytes = o;
    o = align_up(o);
    pl.off_partials = o;
    o = align_up(o + sizeof(float) * (size_t)pl.total_parts);
    pl.off_fold = o;
    o = align_up(o + sizeof(float) * P);
    pl.off_bufs = o;
    for (auto& pp : pl.probs) o += (pp.d.xt_used ? 4 : 2) * pp.x_bytes + pp.a_bytes * (pl.quintic ? 2 : 1);
    pl.total = o;
}

// Fill buffer pointers for a workspace base and serialise the table.
void carve(Plan& pl, char* ws, std::vector<char>& host_table) {
    float* partials = (float*)(ws + pl.off_partials);
    float* fold = (float*)(ws + pl.off_fold);
    size_t o = pl.off_bufs;
    int64_t part = 0;
    for (size_t i = 0; i < pl.probs.size(); ++i) {
        NsProb& d = pl.probs[i].d;
        d.x[0] = ws + o;
        o += pl.probs[i].x_bytes;
        d.x[1] = ws + o;
        o += pl.probs[i].x_bytes;
        if (d.xt_used) {
            d.xt[0] = ws + o;
            o += pl.probs[i].x_bytes;
            d.xt[1] = ws + o;
            o += pl.probs[i].x_bytes;
        } else {
            d.xt[0] = d.xt[1] = nullptr;
        }
        d.a = ws + o;
        o += pl.probs[i].a_bytes;
        if (pl.quintic) {
            d.b = ws + o;
            o += pl.probs[i].a_bytes;
        } else {
            d.b = nullptr;
        }
        d.partials = partials + part;
        part += d.nparts;
        d.fold = fold + i;
    }
    host_table.assign(pl.table_bytes, 0);
    char* h = host_table.data();
    for (size_t i = 0; i < pl.probs.size(); ++i) std::memcpy(h + pl.off_table + i * sizeof(NsProb), &pl.probs[i].d, sizeof(NsProb));
    std::memcpy(h + pl.off_prep_prefix, pl.prep_prefix.data(), sizeof(int) * pl.prep_prefix.size());
    size_t o2 = pl.off_group_prefix;
    for (auto& g : pl.groups) {
        std::memcpy(h + o2, g.gram_order.data(), sizeof(int) * g.gram_order.size());
        o2 += sizeof(int) * g.gram_order.size();
        std::memcpy(h + o2, g.apply_order.data(), sizeof(int) * g.apply_order.size());
        o2 += sizeof(int) * g.apply_order.size();
        std::memcpy(h + o2, g.gram_prefix.data(), sizeof(int) * g.gram_prefix.size());
        o2 += sizeof(int) * g.gram_prefix.size();
        std::memcpy(h + o2, g.apply_prefix.data(), sizeof(int) * g.apply_prefix.size());
        o2 += sizeof(int) * g.apply_prefix.size();
    }
}

// ---------------------------------------------------------------------------
// Pinned staging for descriptor tables: a small ring per device. A slot is
// reused only after the copy that last read it has completed.
// ---------------------------------------------------------------------------
struct Slot {
    void* host = nullptr;
    void* host_dev = nullptr;   // the device's address of `host`
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};
struct DevStaging {
    int device = -1;
    Slot slots[4];
    int next = 0;
};
std::mutex g_stage_mu;
std::vector<DevStaging> g_staging;

int upload(const void* src, size_t bytes, void* dst, hipStream_t s) {
    if (bytes == 0) return MU_OK;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lk(g_stage_mu);
    DevStaging* ds = nullptr;
    for (auto& d : g_staging)
        if (d.device == dev) ds = &d;
    if (!ds) {
        g_staging.emplace_back();
        ds = &g_staging.back();
        ds->device = dev;
    }
    Slot& sl = ds->slots[ds->next];
    ds->next = (ds->next + 1) % 4;
    if (sl.pending) {
        e = hipEventSynchronize(sl.ev);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
        sl.pending = false;
    }
    if (sl.cap < bytes) {
        if (sl.host) (void)hipHostFree(sl.host);
        sl.host = nullptr;
        sl.cap = 0;
        size_t cap = std::max<size_t>(bytes, 64 << 10);
        e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault);
        if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
        e = hipHostGetDevicePointer(&sl.host_dev, sl.host, 0);
        if (e != hipSuccess) {
            (void)hipHostFree(sl.host);
            sl.host = nullptr;
            return hip_fail(e, "hipHostGetDevicePointer(staging)");
        }
        sl.cap = cap;
    }
    if (!sl.ev) {
        e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate(staging)");
    }
    std::memcpy(sl.host, src, bytes);
    e = launch_table_copy(sl.host_dev, dst, bytes, s);
    if (e != hipSuccess) return hip_fail(e, "table copy launch");
    e = hipEventRecord(sl.ev, s);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
    sl.pending = true;
    return MU_OK;
}

// ---------------------------------------------------------------------------
// Profiling: events around each launch.
// ---------------------------------------------------------------------------
struct ProfRec {
    int kernel;
    hipEvent_t a, b;
    double flops, bytes;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_pending;
std::vector<hipEvent_t> g_event_pool;
double g_prof_ms[MU_K_COUNT], g_prof_flops[MU_K_COUNT], g_prof_bytes[MU_K_COUNT];
int64_t g_prof_n[MU_K_COUNT];

hipEvent_t get_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <typename F>
int timed_launch(int kernel, double flops, double bytes, hipStream_t s, F&& fn, const char* what) {
    hipEvent_t a = nullptr, b = nullptr;
    bool prof;
    {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        prof = g_prof_on;
        if (prof) {
            a = get_event();
            b = get_event();
        }
    }
    if (prof && a) (void)hipEventRecord(a, s);
    hipError_t e = fn();
    if (prof && b) (void)hipEventRecord(b, s);
    if (prof && a && b) {
        std::lock_guard<std::mutex> lk(g_prof_mu);
        g_prof_pending.push_back({kernel, a, b, flops, bytes});
    }
    if (e != hipSuccess) return hip_fail(e, what);
    return MU_OK;
}

// ---------------------------------------------------------------------------
// The NS pipeline shared by mu_muon_step and mu_muon_orthogonalize.
// ---------------------------------------------------------------------------
int run_pipeline(Plan& pl, char* ws, const mu_muon_hparams* hp, int src_dt, bool step_mode, hipStream_t s) {
    std::vector<char> table;
    carve(pl, ws, table);
    int rc = upload(table.data(), table.size(), ws, s);
    if (rc) return rc;
    const NsProb* dprobs = (const NsProb*)(ws + pl.off_table);
    const int* dprep = (const int*)(ws + pl.off_prep_prefix);
    const int P = (int)pl.probs.size();
    const int ns_dt = pl.ns_dt;
    const std::vector<Coeff> co = coeffs_of(hp);

    double elems = 0;
    for (auto& pp : pl.probs) elems += (double)pp.d.m * pp.d.n;
    const double src_es = (double)dtype_size(src_dt), ns_es = ns_dt == DT_BF16 ? 2.0 : 4.0;

    PrepArgs pa{dprobs, dprep, P, pl.prep_prefix.back(), src_dt, ns_dt, step_mode ? 1 : 0, hp->nesterov ? 1 : 0, hp->mu};
    const double prep_bytes = elems * (src_es + (step_mode ? 8.0 : 0.0) + ns_es);
    rc = timed_launch(MU_K_PREP, 0.0, prep_bytes, s, [&] { return launch_prep(pa, s); }, "prep launch");
    if (rc) return rc;
    NormArgs na{dprobs, P, hp->norm_eps};
    rc = timed_launch(MU_K_NORM, 0.0, 4.0 * (double)pl.total_parts, s, [&] { return launch_norm(na, s); }, "norm launch");
    if (rc) return rc;

    if (hp->ns_steps == 0) {
        FinishArgs fa{dprobs, dprep, P, pl.prep_prefix.back(), ns_dt, src_dt, step_mode ? 1 : 0, hp->lr, hp->weight_decay};
        const double fb = elems * (ns_es + (step_mode ? 2.0 * src_es : src_es));
        return timed_launch(MU_K_FINISH, 0.0, fb, s, [&] { return launch_finish(fa, s); }, "finish launch");
    }

    // group-level device pointers
    std::vector<const int*> gram_ord, apply_ord, gram_pf, apply_pf;
    {
        size_t o = pl.off_group_prefix;
        for (auto& g : pl.groups) {
            gram_ord.push_back((const int*)(ws + o));
            o += sizeof(int) * g.gram_order.size();
            apply_ord.push_back((const int*)(ws + o));
            o += sizeof(int) * g.apply_order.size();
            gram_pf.push_back((const int*)(ws + o));
            o += sizeof(int) * g.gram_prefix.size();
            apply_pf.push_back((const int*)(ws + o));
            o += sizeof(int) * g.apply_prefix.size();
        }
    }
    // fused problems: every step but the last apply in one launch
    for (const Group& g : pl.groups) {
        if (!g.fused) continue;
        SmallArgs sa{};
        sa.probs = dprobs + g.first;
        sa.nprobs = g.count;
        sa.ns_steps = hp->ns_steps;
        for (int k = 0; k < hp->ns_steps; ++k) {
            sa.ca[k] = co[k].a;
            sa.cb[k] = co[k].b;
        }
        double fl = 0, by = 0;
        for (int i = g.first; i < g.first + g.count; ++i) {
            const double m = pl.probs[i].d.m, n = pl.probs[i].d.n;
            const double xb = (double)pl.probs[i].d.mp * pl.probs[i].d.np * ns_es;
            fl += m * (m + 1) * n + (hp->ns_steps - 1) * (2 * m * m * n + 3 * m * n + m * (m + 1) * n);
            by += xb * (1 + 2 * (hp->ns_steps - 1));   // X0 once, then X in and X' out per step
        }
        rc = timed_launch(MU_K_FUSED, fl, by, s, [&] { return launch_ns_small(sa, s); }, "fused launch");
        if (rc) return rc;
    }
    int src = 0;
    for (int k = 0; k < hp->ns_steps; ++k) {
        const bool first = k == 0, last = k + 1 == hp->ns_steps;
        const bool quint = co[k].c != 0.f;
        for (size_t gi = 0; gi < pl.groups.size(); ++gi) {
            const Group& g = pl.groups[gi];
            if (g.fused && !last) continue;   // done by the fused launch
            double gflops = 0, g2flops = 0, aflops = 0, abytes = 0;
            for (int i = g.first; i < g.first + g.count; ++i) {
                const double m = pl.probs[i].d.m, n = pl.probs[i].d.n;
                gflops += m * (m + 1) * n;
                g2flops += m * (m + 1) * m;
                aflops += 2 * m * m * n + 3 * m * n;
                abytes += m * n * ns_es * (last ? 1.0 : 2.0) + (last ? m * n * (step_mode ? 2 * src_es : src_es) : 0.0);
            }
            GemmArgs ga{};
            ga.probs = dprobs + g.first;
            ga.nprobs = g.count;
            ga.src = src;
            ga.src_dtype = src_dt;
            ga.ca = co[k].a;
            ga.cb = co[k].b;
            ga.cc = co[k].c;
            ga.use_b = quint ? 1 : 0;   // the Gram writes B itself on cubic steps
            ga.lr = hp->lr;
            ga.wd = hp->weight_decay;
            ga.with_update = step_mode ? 1 : 0;
            auto launch = [&](const GemmArgs& a) {
                return ns_dt == DT_BF16 ? launch_gemm_bf16(a, g.tile, s) : launch_gemm_f32(a, s);
            };
            // Gram (the fused launch left a fused group's last B in `a`)
            if (g.fused) {
                GemmArgs ap = ga;
                ap.mode = GM_APPLY_LAST;
                ap.prefix = apply_pf[gi];
                ap.order = apply_ord[gi];
                ap.total_tiles = g.apply_prefix.back();
                rc = timed_launch(MU_K_APPLY, aflops, abytes, s, [&] { return launch(ap); }, "apply launch");
                if (rc) return rc;
                continue;
            }
            GemmArgs gg = ga;
            gg.mode = GM_GRAM;
            gg.prefix = gram_pf[gi];
            gg.order = gram_ord[gi];
            gg.total_tiles = g.gram_prefix.back();
            gg.first = first ? 1 : 0;
            gg.xcd_window = g.gram_window;
            rc = timed_launch(MU_K_GRAM, gflops, 0.0, s, [&] { return launch(gg); }, "gram launch");
            if (rc) return rc;
            if (quint) {
                GemmArgs g2 = ga;
                g2.mode = GM_GRAM2;
                g2.prefix = gram_pf[gi];
                g2.order = gram_ord[gi];
                g2.total_tiles = g.gram_prefix.back();
                g2.first = first ? 1 : 0;
                g2.xcd_window = g.gram_window;
                rc = timed_launch(MU_K_GRAM2, g2flops, 0.0, s, [&] { return launch(g2); }, "gram2 launch");
                if (rc) return rc;
            }
            GemmArgs ap = ga;
            ap.mode = last ? GM_APPLY_LAST : GM_APPLY;
            ap.prefix = apply_pf[gi];
            ap.order = apply_ord[gi];
            ap.total_tiles = g.apply_prefix.back();
            ap.first = first ? 1 : 0;
            rc = timed_launch(MU_K_APPLY, aflops, abytes, s, [&] { return launch(ap); }, "apply launch");
            if (rc) return rc;
        }
        src ^= 1;
    }
    return MU_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int validate_mats(const mu_matrix* m, int32_t n, std::vector<Item>& items, int& dt) {
    if (n < 0) return fail(MU_ERR_INVALID_ARG, "n must be >= 0");
    if (n > 0 && !m) return fail(MU_ERR_INVALID_ARG, "matrix list is null");
    std::vector<Range> ranges;
    dt = n > 0 ? m[0].dtype : MU_BF16;
    for (int i = 0; i < n; ++i) {
        const mu_matrix& x = m[i];
        if (x.dtype != MU_F32 && x.dtype != MU_BF16) return fail(MU_ERR_DTYPE, "matrix %d: unknown dtype %d", i, x.dtype);
        if (x.dtype != dt) return fail(MU_ERR_DTYPE, "matrix %d: all matrices of one call must share a dtype", i);
        if (!x.param || !x.grad || !x.momentum) return fail(MU_ERR_INVALID_ARG, "matrix %d: null param/grad/momentum", i);
        if (x.rows <= 0 || x.cols <= 0) return fail(MU_ERR_INVALID_ARG, "matrix %d: rows and cols must be > 0", i);
        if (x.rows > MU_MAX_DIM || x.cols > MU_MAX_DIM) return fail(MU_ERR_INVALID_ARG, "matrix %d: dimension above %d", i, MU_MAX_DIM);
        if (x.num_heads < 1 || x.rows % x.num_heads != 0)
            return fail(MU_ERR_INVALID_ARG, "matrix %d: num_heads (%d) must be >= 1 and divide rows (%lld)", i, x.num_heads,
                        (long long)x.rows);
        if (!std::isfinite(x.scale)) return fail(MU_ERR_INVALID_ARG, "matrix %d: scale must be finite", i);
        const size_t es = dtype_size(x.dtype);
        if (!aligned(x.param, es) || !aligned(x.grad, es) || !aligned(x.momentum, 4) || (x.norm_out && !aligned(x.norm_out, 4)))
            return fail(MU_ERR_LAYOUT, "matrix %d: misaligned buffer", i);
        const size_t ne = (size_t)x.rows * (size_t)x.cols;
        ranges.push_back({(uintptr_t)x.param, (uintptr_t)x.param + ne * es, i});
        ranges.push_back({(uintptr_t)x.grad, (uintptr_t)x.grad + ne * es, i});
        ranges.push_back({(uintptr_t)x.momentum, (uintptr_t)x.momentum + ne * 4, i});
        if (x.norm_out) ranges.push_back({(uintptr_t)x.norm_out, (uintptr_t)x.norm_out + 4 * (size_t)x.num_heads, i});
        if (x.ortho_out) {
            if (!aligned(x.ortho_out, 4)) return fail(MU_ERR_LAYOUT, "matrix %d: misaligned ortho_out", i);
            ranges.push_back({(uintptr_t)x.ortho_out, (uintptr_t)x.ortho_out + 4 * ne, i});
        }
        Item it{};
        it.oout = x.ortho_out;
        it.src = x.grad;
        it.mom = x.momentum;
        it.param = x.param;
        it.out = nullptr;
        it.rows = x.rows;
        it.cols = x.cols;
        it.heads = x.num_heads;
        it.scale = x.scale;
        it.norm_out = x.norm_out;
        it.vec = (x.cols % 4 == 0) && aligned(x.param, 16) && aligned(x.grad, 16) && aligned(x.momentum, 16);
        items.push_back(it);
    }
    if (ranges_overlap(ranges)) return fail(MU_ERR_LAYOUT, "buffers of the matrix list overlap");
    return MU_OK;
}

int validate_ortho(const mu_ortho* xs, int32_t n, std::vector<Item>& items, int& dt) {
    if (n < 0) return fail(MU_ERR_INVALID_ARG, "n must be >= 0");
    if (n > 0 && !xs) return fail(MU_ERR_INVALID_ARG, "input list is null");
    std::vector<Range> ranges;
    dt = n > 0 ? xs[0].dtype : MU_BF16;
    for (int i = 0; i < n; ++i) {
        const mu_ortho& x = xs[i];
        if (x.dtype != MU_F32 && x.dtype != MU_BF16) return fail(MU_ERR_DTYPE, "input %d: unknown dtype %d", i, x.dtype);
        if (x.dtype != dt) return fail(MU_ERR_DTYPE, "input %d: all inputs of one call must share a dtype", i);
        if (!x.input || !x.output) return fail(MU_ERR_INVALID_ARG, "input %d: null input/output", i);
        if (x.rows <= 0 || x.cols <= 0) return fail(MU_ERR_INVALID_ARG, "input %d: rows and cols must be > 0", i);
        if (x.rows > MU_MAX_DIM || x.cols > MU_MAX_DIM) return fail(MU_ERR_INVALID_ARG, "input %d: dimension above %d", i, MU_MAX_DIM);
        if (x.num_heads < 1 || x.rows % x.num_heads != 0)
            return fail(MU_ERR_INVALID_ARG, "input %d: num_heads (%d) must be >= 1 and divide rows", i, x.num_heads);
        const size_t es = dtype_size(x.dtype);
        if (!aligned(x.input, es) || !aligned(x.output, es) || (x.norm_out && !aligned(x.norm_out, 4)))
            return fail(MU_ERR_LAYOUT, "input %d: misaligned buffer", i);
        const size_t ne = (size_t)x.rows * (size_t)x.cols;
        ranges.push_back({(uintptr_t)x.input, (uintptr_t)x.input + ne * es, i});
        ranges.push_back({(uintptr_t)x.output, (uintptr_t)x.output + ne * es, i});
        if (x.norm_out) ranges.push_back({(uintptr_t)x.norm_out, (uintptr_t)x.norm_out + 4 * (size_t)x.num_heads, i});
        Item it{};
        it.src = x.input;
        it.mom = nullptr;
        it.param = nullptr;
        it.out = x.output;
        it.rows = x.rows;
        it.cols = x.cols;
        it.heads = x.num_heads;
        it.scale = 1.f;
        it.norm_out = x.norm_out;
        it.oout = nullptr;
        it.vec = (x.cols % 4 == 0) && aligned(x.input, 16) && aligned(x.output, 16);
        items.push_back(it);
    }
    if (ranges_overlap(ranges)) return fail(MU_ERR_LAYOUT, "buffers of the input list overlap");
    return MU_OK;
}

int ns_dtype(const mu_muon_hparams* hp) { return hp->ns_precision == MU_NS_BF16 ? DT_BF16 : DT_F32; }

int check_ws(const Plan& pl, void* ws, size_t ws_bytes) {
    if (pl.probs.empty()) return MU_OK;
    if (!ws) return fail(MU_ERR_WORKSPACE, "workspace is null (need %zu bytes)", pl.total);
    if (!aligned(ws, ALIGN)) return fail(MU_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < pl.total) return fail(MU_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, pl.total);
    return MU_OK;
}

}  // namespace

extern "C" {

int mu_version(void) { return MU_API_VERSION; }

const char* mu_last_error(void) { return g_err.c_str(); }

const char* mu_status_string(int s) {
    switch (s) {
        case MU_OK: return "ok";
        case MU_ERR_INVALID_ARG: return "invalid argument";
        case MU_ERR_DTYPE: return "unsupported dtype or precision";
        case MU_ERR_LAYOUT: return "bad layout (alignment or overlapping buffers)";
        case MU_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MU_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

int mu_muon_workspace_size(const mu_matrix* m, int32_t n, const mu_muon_hparams* hp, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(MU_ERR_INVALID_ARG, "bytes is null");
    int rc = check_hparams(hp, true);
    if (rc) return rc;
    std::vector<Item> items;
    int dt;
    rc = validate_mats(m, n, items, dt);
    if (rc) return rc;
    Plan pl;
    build_plan(items, ns_dtype(hp), coeffs_of(hp), dt, pl);
    *bytes = pl.probs.empty() ? 0 : pl.total;
    return MU_OK;
}

int mu_muon_step(const mu_matrix* m, int32_t n, const mu_muon_hparams* hp, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    int rc = check_hparams(hp, true);
    if (rc) return rc;
    std::vector<Item> items;
    int dt;
    rc = validate_mats(m, n, items, dt);
    if (rc) return rc;
    if (n == 0) return MU_OK;
    Plan pl;
    build_plan(items, ns_dtype(hp), coeffs_of(hp), dt, pl);
    rc = check_ws(pl, ws, ws_bytes);
    if (rc) return rc;
    return run_pipeline(pl, (char*)ws, hp, dt, true, (hipStream_t)stream);
}

int mu_ortho_workspace_size(const mu_ortho* xs, int32_t n, const mu_muon_hparams* hp, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(MU_ERR_INVALID_ARG, "bytes is null");
    int rc = check_hparams(hp, false);
    if (rc) return rc;
    std::vector<Item> items;
    int dt;
    rc = validate_ortho(xs, n, items, dt);
    if (rc) return rc;
    Plan pl;
    build_plan(items, ns_dtype(hp), coeffs_of(hp), dt, pl);
    *bytes = pl.probs.empty() ? 0 : pl.total;
    return MU_OK;
}

int mu_muon_orthogonalize(const mu_ortho* xs, int32_t n, const mu_muon_hparams* hp, void* ws, size_t ws_bytes,
                          void* stream) {
    g_err.clear();
    int rc = check_hparams(hp, false);
    if (rc) return rc;
    std::vector<Item> items;
    int dt;
    rc = validate_ortho(xs, n, items, dt);
    if (rc) return rc;
    if (n == 0) return MU_OK;
    Plan pl;
    build_plan(items, ns_dtype(hp), coeffs_of(hp), dt, pl);
    rc = check_ws(pl, ws, ws_bytes);
    if (rc) return rc;
    return run_pipeline(pl, (char*)ws, hp, dt, false, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// QK-Clip
// ---------------------------------------------------------------------------
namespace {
int64_t qk_segments(const mu_qk_pair* pairs, int32_t n) {
    int64_t s = 0;
    for (int i = 0; i < n; ++i) s += (int64_t)pairs[i].q_heads + pairs[i].k_heads;
    return s;
}
size_t qk_table_bytes(int64_t segs) { return sizeof(QkSeg) * (size_t)segs + sizeof(int64_t) * (size_t)(segs + 1); }
}  // namespace

int mu_qk_clip_workspace_size(const mu_qk_pair* pairs, int32_t n, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(MU_ERR_INVALID_ARG, "bytes is null");
    if (n < 0) return fail(MU_ERR_INVALID_ARG, "n must be >= 0");
    if (n > 0 && !pairs) return fail(MU_ERR_INVALID_ARG, "pair list is null");
    for (int i = 0; i < n; ++i)
        if (pairs[i].q_heads < 1 || pairs[i].k_heads < 1)
            return fail(MU_ERR_INVALID_ARG, "pair %d: head counts must be >= 1", i);
    *bytes = n == 0 ? 0 : align_up(qk_table_bytes(qk_segments(pairs, n)));
    return MU_OK;
}

int mu_qk_clip(const mu_qk_pair* pairs, int32_t n, float tau, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (n < 0) return fail(MU_ERR_INVALID_ARG, "n must be >= 0");
    if (n > 0 && !pairs) return fail(MU_ERR_INVALID_ARG, "pair list is null");
    if (!std::isfinite(tau) || !(tau > 0.f)) return fail(MU_ERR_INVALID_ARG, "tau must be finite and > 0");
    std::vector<QkSeg> segs;
    std::vector<int64_t> prefix(1, 0);
    std::vector<Range> ranges;
    double bytes = 0;
    for (int i = 0; i < n; ++i) {
        const mu_qk_pair& q = pairs[i];
        if (q.dtype != MU_F32 && q.dtype != MU_BF16) return fail(MU_ERR_DTYPE, "pair %d: unknown dtype %d", i, q.dtype);
        if (!q.wq || !q.wk || !q.max_logit) return fail(MU_ERR_INVALID_ARG, "pair %d: null wq/wk/max_logit", i);
        if (q.q_rows <= 0 || q.k_rows <= 0 || q.cols <= 0) return fail(MU_ERR_INVALID_ARG, "pair %d: sizes must be > 0", i);
        if (q.q_rows > MU_MAX_DIM || q.k_rows > MU_MAX_DIM || q.cols > MU_MAX_DIM)
            return fail(MU_ERR_INVALID_ARG, "pair %d: dimension above %d", i, MU_MAX_DIM);
        if (q.q_heads < 1 || q.k_heads < 1 || q.q_rows % q.q_heads != 0 || q.k_rows % q.k_heads != 0)
            return fail(MU_ERR_INVALID_ARG, "pair %d: head counts must be >= 1 and divide the rows", i);
        if (q.q_heads % q.k_heads != 0) return fail(MU_ERR_INVALID_ARG, "pair %d: k_heads must divide q_heads", i);
        const size_t es = dtype_size(q.dtype);
        if (!aligned(q.wq, es) || !aligned(q.wk, es) || !aligned(q.max_logit, 4) || (q.gamma_out && !aligned(q.gamma_out, 4)))
            return fail(MU_ERR_LAYOUT, "pair %d: misaligned buffer", i);
        const int64_t nq = q.q_rows * q.cols, nk = q.k_rows * q.cols;
        ranges.push_back({(uintptr_t)q.wq, (uintptr_t)q.wq + (size_t)nq * es, i});
        ranges.push_back({(uintptr_t)q.wk, (uintptr_t)q.wk + (size_t)nk * es, i});
        ranges.push_back({(uintptr_t)q.max_logit, (uintptr_t)q.max_logit + 4 * (size_t)q.q_heads, i});
        if (q.gamma_out) ranges.push_back({(uintptr_t)q.gamma_out, (uintptr_t)q.gamma_out + 4 * (size_t)q.q_heads, i});
        const int G = q.q_heads / q.k_heads;
        auto add = [&](void* base, int64_t rows, int heads, int h, const float* ml, int nml, float* gout) {
            const int64_t per = rows / heads * q.cols;
            char* w = (char*)base + (size_t)(h * per) * es;
            segs.push_back(QkSeg{w, per, q.dtype, (int32_t)aligned(w, 16), ml, nml, 0, gout});
            prefix.push_back(prefix.back() + (per + QK_CHUNK - 1) / QK_CHUNK);
        };
        for (int h = 0; h < q.q_heads; ++h)
            add(q.wq, q.q_rows, q.q_heads, h, q.max_logit + h, 1, q.gamma_out ? q.gamma_out + h : nullptr);
        for (int g = 0; g < q.k_heads; ++g) add(q.wk, q.k_rows, q.k_heads, g, q.max_logit + (size_t)g * G, G, nullptr);
        bytes += 2.0 * (double)(nq + nk) * (double)es + 4.0 * (q.q_heads + (double)q.q_heads);
    }
    if (ranges_overlap(ranges)) return fail(MU_ERR_LAYOUT, "buffers of the pair list overlap");
    if (n == 0 || prefix.back() == 0) return MU_OK;
    const size_t need = align_up(qk_table_bytes((int64_t)segs.size()));
    if (!ws) return fail(MU_ERR_WORKSPACE, "workspace is null (need %zu bytes)", need);
    if (!aligned(ws, ALIGN)) return fail(MU_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(MU_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    if (prefix.back() > 0x7fffffffLL || segs.size() > 0x7fffffffu)
        return fail(MU_ERR_INVALID_ARG, "too many elements for one launch");

    std::vector<char> table(qk_table_bytes((int64_t)segs.size()));
    std::memcpy(table.data(), segs.data(), sizeof(QkSeg) * segs.size());
    std::memcpy(table.data() + sizeof(QkSeg) * segs.size(), prefix.data(), sizeof(int64_t) * prefix.size());
    hipStream_t s = (hipStream_t)stream;
    int rc = upload(table.data(), table.size(), ws, s);
    if (rc) return rc;
    QkArgs a{};
    a.segs = (const QkSeg*)ws;
    a.prefix = (const int64_t*)((char*)ws + sizeof(QkSeg) * segs.size());
    a.n = (int)segs.size();
    a.total_chunks = prefix.back();
    a.tau = tau;
    return timed_launch(MU_K_QKCLIP, 0.0, bytes, s, [&] { return launch_qkclip(a, s); }, "qk_clip launch");
}

int mu_adamw_workspace_size(int32_t n, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(MU_ERR_INVALID_ARG, "bytes is null");
    if (n < 0) return fail(MU_ERR_INVALID_ARG, "n must be >= 0");
    *bytes = n == 0 ? 0 : align_up(sizeof(AdamWDesc) * n + sizeof(int64_t) * (n + 1));
    return MU_OK;
}

int mu_adamw_step(const mu_tensor* ts, int32_t n, const mu_adamw_hparams* hp, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!hp) return fail(MU_ERR_INVALID_ARG, "hparams is null");
    if (n < 0) return fail(MU_ERR_INVALID_ARG, "n must be >= 0");
    if (n > 0 && !ts) return fail(MU_ERR_INVALID_ARG, "tensor list is null");
    if (hp->step < 1) return fail(MU_ERR_INVALID_ARG, "step must be >= 1 (got %lld)", (long long)hp->step);
    if (!std::isfinite(hp->beta1) || !std::isfinite(hp->beta2) || !std::isfinite(hp->eps))
        return fail(MU_ERR_INVALID_ARG, "beta1, beta2 and eps must be finite");
    if (hp->beta1 < 0.f || hp->beta1 >= 1.f || hp->beta2 < 0.f || hp->beta2 >= 1.f)
        return fail(MU_ERR_INVALID_ARG, "betas must lie in [0, 1)");
    std::vector<AdamWDesc> d((size_t)n);
    std::vector<int64_t> prefix(1, 0);
    std::vector<Range> ranges;
    for (int i = 0; i < n; ++i) {
        const mu_tensor& t = ts[i];
        if (t.dtype != MU_F32 && t.dtype != MU_BF16) return fail(MU_ERR_DTYPE, "tensor %d: unknown dtype %d", i, t.dtype);
        if (t.numel < 0) return fail(MU_ERR_INVALID_ARG, "tensor %d: numel must be >= 0", i);
        if (t.numel > 0 && (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq))
            return fail(MU_ERR_INVALID_ARG, "tensor %d: null buffer", i);
        if (!std::isfinite(t.lr) || !std::isfinite(t.weight_decay))
            return fail(MU_ERR_INVALID_ARG, "tensor %d: lr and weight_decay must be finite", i);
        const size_t es = dtype_size(t.dtype);
        if (!aligned(t.param, es) || !aligned(t.grad, es) || !aligned(t.exp_avg, 4) || !aligned(t.exp_avg_sq, 4))
            return fail(MU_ERR_LAYOUT, "tensor %d: misaligned buffer", i);
        if (t.numel > 0) {
            ranges.push_back({(uintptr_t)t.param, (uintptr_t)t.param + t.numel * es, i});
            ranges.push_back({(uintptr_t)t.grad, (uintptr_t)t.grad + t.numel * es, i});
            ranges.push_back({(uintptr_t)t.exp_avg, (uintptr_t)t.exp_avg + t.numel * 4, i});
            ranges.push_back({(uintptr_t)t.exp_avg_sq, (uintptr_t)t.exp_avg_sq + t.numel * 4, i});
        }
        d[i] = AdamWDesc{t.param, t.grad, t.exp_avg, t.exp_avg_sq, t.numel, t.dtype,
                         (int32_t)(aligned(t.param, 16) && aligned(t.grad, 16) && aligned(t.exp_avg, 16) && aligned(t.exp_avg_sq, 16)),
                         t.lr, t.weight_decay};
        prefix.push_back(prefix.back() + (t.numel + ADAMW_CHUNK - 1) / ADAMW_CHUNK);
    }
    if (ranges_overlap(ranges)) return fail(MU_ERR_LAYOUT, "buffers of the tensor list overlap");
    if (n == 0 || prefix.back() == 0) return MU_OK;
    size_t need = 0;
    mu_adamw_workspace_size(n, &need);
    if (!ws) return fail(MU_ERR_WORKSPACE, "workspace is null (need %zu bytes)", need);
    if (!aligned(ws, ALIGN)) return fail(MU_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(MU_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    if (prefix.back() > 0x7fffffffLL) return fail(MU_ERR_INVALID_ARG, "too many elements for one launch");

    std::vector<char> table(sizeof(AdamWDesc) * n + sizeof(int64_t) * (n + 1));
    std::memcpy(table.data(), d.data(), sizeof(AdamWDesc) * n);
    std::memcpy(table.data() + sizeof(AdamWDesc) * n, prefix.data(), sizeof(int64_t) * (n + 1));
    hipStream_t s = (hipStream_t)stream;
    int rc = upload(table.data(), table.size(), ws, s);
    if (rc) return rc;
    AdamWArgs a{};
    a.descs = (const AdamWDesc*)ws;
    a.prefix = (const int64_t*)((char*)ws + sizeof(AdamWDesc) * n);
    a.n = n;
    a.total_chunks = prefix.back();
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.eps = hp->eps;
    a.bc1 = (float)(1.0 - std::pow((double)hp->beta1, (double)hp->step));
    a.bc2 = (float)(1.0 - std::pow((double)hp->beta2, (double)hp->step));
    double bytes = 0;
    for (int i = 0; i < n; ++i) bytes += (double)ts[i].numel * (3.0 * dtype_size(ts[i].dtype) + 16.0);
    return timed_launch(MU_K_ADAMW, 0.0, bytes, s, [&] { return launch_adamw(a, s); }, "adamw launch");
}

int mu_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (on) {
        for (auto& r : g_prof_pending) {
            (void)hipEventSynchronize(r.b);
            g_event_pool.push_back(r.a);
            g_event_pool.push_back(r.b);
        }
        g_prof_pending.clear();
        for (int k = 0; k < MU_K_COUNT; ++k) {
            g_prof_ms[k] = g_prof_flops[k] = g_prof_bytes[k] = 0.0;
            g_prof_n[k] = 0;
        }
    }
    g_prof_on = on != 0;
    return MU_OK;
}

int mu_profile_read(int kernel, double* total_ms, int64_t* launches, double* flops, double* bytes) {
    g_err.clear();
    if (kernel < 0 || kernel >= MU_K_COUNT) return fail(MU_ERR_INVALID_ARG, "unknown kernel class %d", kernel);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& r : g_prof_pending) {
        hipError_t e = hipEventSynchronize(r.b);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(profile)");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        g_prof_ms[r.kernel] += ms;
        g_prof_flops[r.kernel] += r.flops;
        g_prof_bytes[r.kernel] += r.bytes;
        g_prof_n[r.kernel] += 1;
        g_event_pool.push_back(r.a);
        g_event_pool.push_back(r.b);
    }
    g_prof_pending.clear();
    if (total_ms) *total_ms = g_prof_ms[kernel];
    if (launches) *launches = g_prof_n[kernel];
    if (flops) *flops = g_prof_flops[kernel];
    if (bytes) *bytes = g_prof_bytes[kernel];
    return MU_OK;
}

const char* mu_kernel_name(int k) {
    switch (k) {
        case MU_K_PREP: return "prep";
        case MU_K_NORM: return "norm";
        case MU_K_GRAM: return "gram";
        case MU_K_GRAM2: return "gram2";
        case MU_K_APPLY: return "apply";
        case MU_K_FINISH: return "finish";
        case MU_K_ADAMW: return "adamw";
        case MU_K_QKCLIP: return "qk_clip";
        case MU_K_FUSED: return "ns_fused";
        default: return "unknown";
    }
}

}  // extern "C"
