// Host side of the NVFP4 grouped GEMM C ABI: validation, planning and launch.
//
// Planning follows the host path of custom_kernel on the page "kernelindex submission
// 503584" in spirit (groups ordered by work, per-group tile counts and their prefix sum
// drive a persistent grid), with work units sized for gfx950:
//   * a unit is up to 32 NA rows of one group times 32 NB columns over the whole K; the
//     four waves of a workgroup split every K superstep and each holds the unit's NA x NB
//     accumulator blocks (at most 20), and the shapes the kernel is compiled for are
//     listed in nvfp4_gg_internal.h;
//   * a cost model (MFMA cycles, the conversion VALU that shares the MFMA's issue slots,
//     operand bytes, fixed prologue and epilogue cycles) prices a unit of each shape;
//   * each group gets one shape; starting from every group's most efficient shape, a
//     coordinate descent over the groups' shapes minimises the estimated makespan of the
//     kernel's own partition (workgroup v runs units [U v / V, U (v+1) / V) of the unit
//     sequence);
//   * the plan is the group table alone: it travels in the kernel arguments of every call,
//     so a plan holds host memory only and a call touches no device memory besides the
//     operands.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "nvfp4_gg.h"
#include "nvfp4_gg_internal.h"

using namespace nvfp4gg;

struct nvfp4_gg_plan_s {
    uint32_t magic;
    int g;
    int n, k;                    // shared by every group, or 0 where the groups differ
    int device;
    int num_cus;
    int scale_layout;            // nvfp4_gg_scale_layout_t
    int units;                   // units over all groups
    int vq;                      // virtual workgroups per XCD
    int grid;                    // 8 vq, or 0 when there is no work
    double est_cycles;           // estimated makespan (cycles of one CU)
    std::vector<int> m;          // caller order
    std::vector<int> ns, ks, ldcs;  // caller order
    std::vector<int> order;      // order[p] = caller group at schedule position p
    std::vector<int> na, nb;     // unit shape per schedule position (0 for m = 0)
    std::vector<int> unit_begin; // per-group unit prefix in schedule order (size g + 1)
};

namespace {

constexpr uint32_t kPlanMagic = 0x4E564634u;  // "NVF4"
constexpr int kMaxRows = 1 << 20;
constexpr int kNominalCUs = 256;               // MI355X
constexpr int kXcds = 8;                       // workgroup b runs on XCD b % 8

struct Shape {
    int na, nb;
};
const Shape kShapes[] = {
#define NVFP4GG_SHAPE(NA_, NB_) Shape{NA_, NB_},
    NVFP4GG_UNIT_SHAPES(NVFP4GG_SHAPE)
#undef NVFP4GG_SHAPE
};

bool plan_ok(const nvfp4_gg_plan_s* p) { return p != nullptr && p->magic == kPlanMagic; }

long ceil_div(long a, long b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Estimated cycles of one unit of shape (na, nb) with K = k on one CU, fitted to the
// kernel's own per-phase cycle counts on MI355X:
//   * the main loop issues, per superstep and wave, 4 na nb MFMAs 32x32x16 f16 and
//     ~33 (na + nb) conversion instructions (four FP4 conversions and four packed multiplies
//     per fragment and step); an MFMA holds the issue port ~19 of its 32 cycles, so the
//     conversions only partly hide behind it: ~110 na nb + 172 (na + nb) cycles per
//     superstep, barrier and LDS reads included; units of 11 operand blocks (their codes
//     read in 8-byte halves, the exchange in the most rounds) measure ~400 more per superstep
//     (with this term the short-K grouped shapes plan fewer of them: c3 -3 %, a 64-group
//     MoE-like workload -2.6 %);
//   * plus the pipeline fill (the first superstep's operands from HBM) and the epilogue
//     (the four K-quarter partial tiles added through LDS, fp16 rounding, stores).
double unit_cycles(int na, int nb, int k)
{
    const double nm = (double)na * nb;
    const double super = 110.0 * nm + 172.0 * (na + nb) + (na + nb >= 11 ? 400.0 : 0.0);
    const double nsup = (double)ceil_div(k, 256);
    return nsup * super + 8300.0 + 535.0 * nm;
}

struct GroupDims {
    int m, n, k;
};

long group_units(const GroupDims& d, const Shape& s)
{
    if (d.m == 0) return 0;
    return ceil_div(d.m, 32L * s.na) * ceil_div(d.n, 32L * s.nb);
}

// Makespan of the kernel's partition: the unit sequence (groups in schedule order, each
// group's units of equal cost) dealt in contiguous ranges of equal count to V workgroups.
double makespan(const std::vector<GroupDims>& dims, const std::vector<int>& shape, int num_cus, long* units_out,
                int* vq_out)
{
    long U = 0;
    std::vector<long> cnt(dims.size());
    std::vector<double> cost(dims.size());
    for (size_t i = 0; i < dims.size(); ++i) {
        cnt[i] = shape[i] < 0 ? 0 : group_units(dims[i], kShapes[shape[i]]);
        cost[i] = shape[i] < 0 ? 0.0 : unit_cycles(kShapes[shape[i]].na, kShapes[shape[i]].nb, dims[i].k);
        U += cnt[i];
    }
    if (units_out) *units_out = U;
    if (U == 0) {
        if (vq_out) *vq_out = 0;
        return 0.0;
    }
    const int vq = (int)ceil_div(std::min<long>(U, num_cus), kXcds);
    if (vq_out) *vq_out = vq;
    const long V = (long)kXcds * vq;
    // walk the ranges: range v is [U v / V, U (v+1) / V)
    double worst = 0.0;
    size_t gi = 0;
    long gbase = 0;
    for (long v = 0; v < V; ++v) {
        const long u0 = U * v / V, u1 = U * (v + 1) / V;
        double sum = 0.0;
        long u = u0;
        while (u < u1) {
            while (gi + 1 < dims.size() && u >= gbase + cnt[gi]) {
                gbase += cnt[gi];
                ++gi;
            }
            const long take = std::min(u1, gbase + cnt[gi]) - u;
            sum += take * cost[gi];
            u += take;
        }
        worst = std::max(worst, sum);
    }
    return worst;
}

// Candidate shapes of one group: the supported shapes, skipping a shape when a shape
// with fewer row blocks gives the same row chunk count and the same column blocks (it
// would only add padding rows).
std::vector<int> candidates(const GroupDims& d)
{
    std::vector<int> out;
    if (d.m == 0) return out;
    const int nshapes = (int)(sizeof(kShapes) / sizeof(kShapes[0]));
    for (int s = 0; s < nshapes; ++s) {
        const Shape& sh = kShapes[s];
        const long rch = ceil_div(d.m, 32L * sh.na);
        bool dominated = false;
        for (int t = 0; t < nshapes; ++t)
            if (kShapes[t].nb == sh.nb && kShapes[t].na < sh.na && ceil_div(d.m, 32L * kShapes[t].na) == rch)
                dominated = true;
        if (!dominated) out.push_back(s);
    }
    return out;
}

// Shapes for every group (schedule order) with at most `cap` accumulator blocks per unit:
// start from each group's cheapest shape per useful multiply-accumulate, then coordinate
// descent on the estimated makespan (ties: smaller total cost) until no single group's
// change helps.
std::vector<int> choose_shapes_capped(const std::vector<GroupDims>& dims, int num_cus, int cap, double* est)
{
    const size_t g = dims.size();
    std::vector<std::vector<int>> cand(g);
    std::vector<int> shape(g, -1);
    for (size_t i = 0; i < g; ++i) {
        for (int s : candidates(dims[i]))
            if (kShapes[s].na * kShapes[s].nb <= cap) cand[i].push_back(s);
        double best = 0.0;
        for (int s : cand[i]) {
            const Shape& sh = kShapes[s];
            const double work = (double)dims[i].m * dims[i].n;   // useful per unit of K
            const double eff = work / (group_units(dims[i], sh) * unit_cycles(sh.na, sh.nb, dims[i].k));
            if (shape[i] < 0 || eff > best) {
                best = eff;
                shape[i] = s;
            }
        }
        if (dims[i].m > 0 && shape[i] < 0) {   // no shape within the cap
            if (est) *est = 1e300;
            return shape;
        }
    }
    const auto total = [&](const std::vector<int>& sh) {
        double t = 0.0;
        for (size_t i = 0; i < g; ++i)
            if (sh[i] >= 0) t += group_units(dims[i], kShapes[sh[i]]) * unit_cycles(kShapes[sh[i]].na, kShapes[sh[i]].nb, dims[i].k);
        return t;
    };
    double cur = makespan(dims, shape, num_cus, nullptr, nullptr);
    double cur_total = total(shape);
    for (int pass = 0; pass < 8; ++pass) {
        bool improved = false;
        for (size_t i = 0; i < g; ++i) {
            for (int s : cand[i]) {
                if (s == shape[i]) continue;
                std::vector<int> trial = shape;
                trial[i] = s;
                const double ms = makespan(dims, trial, num_cus, nullptr, nullptr);
                const double tt = total(trial);
                if (ms < cur * 0.999 || (ms <= cur * 1.001 && tt < cur_total * 0.999)) {
                    shape = trial;
                    cur = ms;
                    cur_total = tt;
                    improved = true;
                }
            }
        }
        if (!improved) break;
    }
    if (est) *est = cur;
    return shape;
}

// The shape that NVFP4_GG_FORCE_SHAPE="na,nb" names, if it is a compiled shape; else -1.
int forced_shape()
{
    const char* e = std::getenv("NVFP4_GG_FORCE_SHAPE");
    int na = 0, nb = 0;
    if (e == nullptr || std::sscanf(e, "%d,%d", &na, &nb) != 2) return -1;
    const int nshapes = (int)(sizeof(kShapes) / sizeof(kShapes[0]));
    for (int s = 0; s < nshapes; ++s)
        if (kShapes[s].na == na && kShapes[s].nb == nb) return s;
    return -1;
}

// The best of the capped searches over every cap a compiled shape has (or the forced shape
// for every group).
std::vector<int> choose_shapes(const std::vector<GroupDims>& dims, int num_cus, double* est)
{
    const int forced = forced_shape();
    if (forced >= 0) {
        std::vector<int> sh(dims.size(), -1);
        for (size_t i = 0; i < dims.size(); ++i)
            if (dims[i].m > 0) sh[i] = forced;
        if (est) *est = makespan(dims, sh, num_cus, nullptr, nullptr);
        return sh;
    }
    std::vector<int> caps;
    for (const Shape& sh : kShapes) caps.push_back(sh.na * sh.nb);
    std::sort(caps.begin(), caps.end());
    caps.erase(std::unique(caps.begin(), caps.end()), caps.end());
    std::vector<int> best;
    double best_est = 0.0;
    for (int cap : caps) {
        double e = 0.0;
        std::vector<int> sh = choose_shapes_capped(dims, num_cus, cap, &e);
        if (best.empty() || e < best_est * 0.999) {
            best = sh;
            best_est = e;
        }
    }
    if (est) *est = best_est;
    return best;
}

}  // namespace

extern "C" const char* nvfp4_gg_status_string(nvfp4_gg_status_t s)
{
    switch (s) {
    case NVFP4_GG_OK: return "success";
    case NVFP4_GG_EINVAL: return "invalid argument";
    case NVFP4_GG_EALIGN: return "device pointer not 16-byte aligned";
    case NVFP4_GG_ENOMEM: return "host allocation failed";
    case NVFP4_GG_EHIP: return "HIP runtime error";
    case NVFP4_GG_EUNSUPPORTED: return "unsupported device or configuration";
    }
    return "unknown status";
}

extern "C" nvfp4_gg_status_t nvfp4_gg_plan(nvfp4_gg_plan_t* out, int g, const int* m, int n, int k, int device)
{
    return nvfp4_gg_plan_layout(out, g, m, n, k, device, NVFP4_GG_SCALES_ROW_MAJOR);
}

extern "C" nvfp4_gg_status_t nvfp4_gg_plan_layout(nvfp4_gg_plan_t* out, int g, const int* m, int n, int k,
                                                  int device, int scale_layout)
{
    if (out == nullptr) return NVFP4_GG_EINVAL;
    *out = nullptr;
    if (m == nullptr || g < 1) return NVFP4_GG_EINVAL;
    if (g > NVFP4_GG_MAX_GROUPS) return NVFP4_GG_EUNSUPPORTED;
    nvfp4_gg_problem_t probs[NVFP4_GG_MAX_GROUPS];
    for (int i = 0; i < g; ++i) probs[i] = nvfp4_gg_problem_t{m[i], n, k, 0};
    return nvfp4_gg_plan_problems(out, g, probs, device, scale_layout);
}

extern "C" nvfp4_gg_status_t nvfp4_gg_plan_problems(nvfp4_gg_plan_t* out, int g, const nvfp4_gg_problem_t* problems,
                                                    int device, int scale_layout)
{
    if (out == nullptr) return NVFP4_GG_EINVAL;
    *out = nullptr;
    if (scale_layout != NVFP4_GG_SCALES_ROW_MAJOR && scale_layout != NVFP4_GG_SCALES_BLOCKED) return NVFP4_GG_EINVAL;
    if (problems == nullptr || g < 1) return NVFP4_GG_EINVAL;
    if (g > NVFP4_GG_MAX_GROUPS) return NVFP4_GG_EUNSUPPORTED;
    for (int i = 0; i < g; ++i) {
        const nvfp4_gg_problem_t& q = problems[i];
        if (q.m < 0 || q.m > kMaxRows || q.n < 1 || q.n > kMaxRows || q.k < 64 || q.k > kMaxRows ||
            (q.k % 64) != 0 || q.ldc < 0 || (q.ldc != 0 && q.ldc < q.n))
            return NVFP4_GG_EINVAL;
    }
    if (device < NVFP4_GG_DEVICE_NONE) return NVFP4_GG_EINVAL;

    int num_cus = kNominalCUs;
    if (device != NVFP4_GG_DEVICE_NONE) {
        if (device == -1 && hipGetDevice(&device) != hipSuccess) return NVFP4_GG_EHIP;
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, device) != hipSuccess) return NVFP4_GG_EHIP;
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return NVFP4_GG_EUNSUPPORTED;
        num_cus = prop.multiProcessorCount;
    }

    nvfp4_gg_plan_s* p = new (std::nothrow) nvfp4_gg_plan_s();
    if (p == nullptr) return NVFP4_GG_ENOMEM;
    try {
        p->magic = kPlanMagic;
        p->g = g;
        p->device = device;
        p->num_cus = num_cus;
        p->scale_layout = scale_layout;
        p->m.resize(g);
        p->ns.resize(g);
        p->ks.resize(g);
        p->ldcs.resize(g);
        for (int i = 0; i < g; ++i) {
            p->m[i] = problems[i].m;
            p->ns[i] = problems[i].n;
            p->ks[i] = problems[i].k;
            p->ldcs[i] = problems[i].ldc ? problems[i].ldc : problems[i].n;
        }
        p->n = p->ns[0];
        p->k = p->ks[0];
        for (int i = 1; i < g; ++i) {
            if (p->ns[i] != p->n) p->n = 0;
            if (p->ks[i] != p->k) p->k = 0;
        }

        // schedule order of the groups: largest work first (stable for ties)
        const auto work = [&](int i) { return (double)p->m[i] * p->ns[i] * p->ks[i]; };
        p->order.resize(g);
        std::iota(p->order.begin(), p->order.end(), 0);
        std::stable_sort(p->order.begin(), p->order.end(), [&](int a, int b) { return work(a) > work(b); });
        std::vector<GroupDims> dims(g);
        for (int s = 0; s < g; ++s) dims[s] = GroupDims{p->m[p->order[s]], p->ns[p->order[s]], p->ks[p->order[s]]};

        const std::vector<int> shape = choose_shapes(dims, num_cus, &p->est_cycles);
        long units = 0;
        int vq = 0;
        (void)makespan(dims, shape, num_cus, &units, &vq);
        if (units > 0x7fffffffL) {
            delete p;
            return NVFP4_GG_EUNSUPPORTED;
        }
        p->units = (int)units;
        p->vq = vq;
        p->grid = kXcds * vq;
        p->na.assign(g, 0);
        p->nb.assign(g, 0);
        p->unit_begin.assign(g + 1, 0);
        for (int s = 0; s < g; ++s) {
            if (shape[s] >= 0) {
                p->na[s] = kShapes[shape[s]].na;
                p->nb[s] = kShapes[shape[s]].nb;
            }
            p->unit_begin[s + 1] = p->unit_begin[s] + (shape[s] >= 0 ? (int)group_units(dims[s], kShapes[shape[s]]) : 0);
        }
    } catch (...) {
        delete p;
        return NVFP4_GG_ENOMEM;
    }
    *out = p;
    return NVFP4_GG_OK;
}

extern "C" nvfp4_gg_status_t nvfp4_gg_run(nvfp4_gg_plan_t plan, const void* const* A, const void* const* B,
                                          const void* const* SFA, const void* const* SFB, void* const* C,
                                          hipStream_t stream)
{
    if (!plan_ok(plan)) return NVFP4_GG_EINVAL;
    if (!A || !B || !SFA || !SFB || !C) return NVFP4_GG_EINVAL;

    KernArgs args;
    std::memset(&args, 0, sizeof(args));
    args.g = plan->g;
    args.units = plan->units;
    args.vq = plan->vq;
    args.flags = plan->scale_layout == NVFP4_GG_SCALES_BLOCKED ? kFlagBlockedScales : 0;
    for (int s = 0; s < plan->g; ++s) {
        const int i = plan->order[s];
        const int mi = plan->m[i];
        GroupArgs& G = args.grp[s];
        G.m_shape = mi | (plan->na[s] << kNaShift) | (plan->nb[s] << kNbShift);
        G.n = plan->ns[i];
        G.k = plan->ks[i];
        G.ldc = plan->ldcs[i];
        if (mi > 0) {
            if (!A[i] || !B[i] || !SFA[i] || !SFB[i] || !C[i]) return NVFP4_GG_EINVAL;
            if (!aligned16(A[i]) || !aligned16(B[i]) || !aligned16(SFA[i]) || !aligned16(SFB[i]) || !aligned16(C[i]))
                return NVFP4_GG_EALIGN;
            G.a = static_cast<const uint8_t*>(A[i]);
            G.b = static_cast<const uint8_t*>(B[i]);
            G.sfa = static_cast<const uint8_t*>(SFA[i]);
            G.sfb = static_cast<const uint8_t*>(SFB[i]);
            G.c = static_cast<uint16_t*>(C[i]);
        }
    }

    if (plan->device == NVFP4_GG_DEVICE_NONE) return NVFP4_GG_EUNSUPPORTED;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return NVFP4_GG_EHIP;
    if (cur != plan->device) return NVFP4_GG_EINVAL;
    if (plan->units == 0) return NVFP4_GG_OK;
    if (launch_units(args, plan->grid, stream) != hipSuccess) return NVFP4_GG_EHIP;
    return NVFP4_GG_OK;
}

extern "C" nvfp4_gg_status_t nvfp4_gg_plan_info(nvfp4_gg_plan_t plan, nvfp4_gg_plan_info_t* info)
{
    if (!plan_ok(plan) || info == nullptr) return NVFP4_GG_EINVAL;
    std::memset(info, 0, sizeof(*info));
    info->g = plan->g;
    info->n = plan->n;
    info->k = plan->k;
    info->device = plan->device;
    info->num_cus = plan->num_cus;
    for (int s = 0; s < plan->g; ++s) {
        info->tile_m = std::max(info->tile_m, 32 * plan->na[s]);
        info->tile_n = std::max(info->tile_n, 32 * plan->nb[s]);
        info->unit_rows[s] = 32 * plan->na[s];
        info->unit_cols[s] = 32 * plan->nb[s];
    }
    info->total_tiles = plan->units;
    info->grid = plan->grid;
    info->block = kUnitThreads;
    info->lds_bytes = kUnitLdsBytes;
    info->variant = plan->scale_layout == NVFP4_GG_SCALES_BLOCKED ? 6 : 5;
    for (int s = 0; s < plan->g; ++s) info->order[s] = plan->order[s];
    for (int s = 0; s <= plan->g; ++s) info->tile_begin[s] = plan->unit_begin[s];
    info->scale_layout = plan->scale_layout;
    info->est_us = plan->est_cycles / 2.1e3;
    return NVFP4_GG_OK;
}

extern "C" size_t nvfp4_gg_blocked_scale_bytes(int rows, int k)
{
    if (rows <= 0 || k < 64 || (k % 64) != 0) return 0;
    return (size_t)blocked_scale_bytes(rows, k);
}

extern "C" nvfp4_gg_status_t nvfp4_gg_scales_to_blocked(void* dst, const void* src, int rows, int k,
                                                        hipStream_t stream)
{
    if (rows < 0 || rows > kMaxRows || k < 64 || k > kMaxRows || (k % 64) != 0) return NVFP4_GG_EINVAL;
    if (rows == 0) return NVFP4_GG_OK;
    if (dst == nullptr || src == nullptr) return NVFP4_GG_EINVAL;
    if (!aligned16(dst) || !aligned16(src)) return NVFP4_GG_EALIGN;
    if (launch_scales_to_blocked(dst, src, rows, k, stream) != hipSuccess) return NVFP4_GG_EHIP;
    return NVFP4_GG_OK;
}

extern "C" void nvfp4_gg_destroy(nvfp4_gg_plan_t plan)
{
    if (!plan_ok(plan)) return;
    plan->magic = 0;
    delete plan;
}
