// Host side of the NVFP4 grouped GEMM C ABI: validation, planning and launch.
//
// Planning follows the host path of custom_kernel on the page "kernelindex submission
// 503584" in spirit (groups ordered by work, tiles enumerated over per-group tile counts),
// but the tile list is built here once per shape and balanced across the compute units:
//   * every group's rows are cut into equal chunks of at most R rows (multiples of 32) and
//     the columns into 128-wide tiles, for each candidate R in {32, 64, 96};
//   * a cost model (MFMA cycles plus the dequantisation VALU cycles that the tile height
//     implies, per SIMD) prices each tile;
//   * tiles that read the same B columns (same group, same column tile) are kept on one
//     XCD, XCDs are balanced, and inside an XCD tiles are dealt largest first to the least
//     loaded workgroup (LPT);
//   * the candidate R with the smallest estimated makespan wins.
// The group table travels by value in the kernel arguments on every call; the tile list
// is uploaded to device memory once, when the plan is built.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
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
    int variant;
    int scale_layout;            // nvfp4_gg_scale_layout_t
    VariantShape shape;
    int chunk_rows;              // chosen maximum rows per tile
    int total_tiles;
    int grid;
    double est_cycles;           // estimated makespan of the tile schedule
    std::vector<int> m;          // caller order
    std::vector<int> ns, ks, ldcs;  // caller order
    std::vector<int> order;      // order[p] = caller group at schedule position p
    std::vector<int> tile_begin; // per-group tile prefix in schedule order (informational)
    std::vector<TileDesc> tiles; // tiles grouped by workgroup (group = schedule position)
    std::vector<int> wg_begin;   // size grid + 1
    TileDesc* d_tiles = nullptr;
    int* d_wg_begin = nullptr;
};

namespace {

constexpr uint32_t kPlanMagic = 0x4E564634u;  // "NVF4"
constexpr int kMaxRows = 1 << 20;
constexpr int kNominalCUs = 256;               // MI355X
constexpr int kXcds = 8;                       // workgroup b runs on XCD b % 8
constexpr int kTileCols = 128;
constexpr int kStepK = 64;

bool plan_ok(const nvfp4_gg_plan_s* p) { return p != nullptr && p->magic == kPlanMagic; }

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Estimated cycles of one tile on one CU, per compute step of 64 K (fitted on MI355X):
//   * MFMA: per SIMD 4 * rpad/32 MFMAs 32x32x16 f16 at ~35 cycles;
//   * VALU: per SIMD ~2 x 26 instructions for B plus 18 per 64 tile rows for A, at ~4.6
//     cycles (the conversions are not full rate);
//   * operand bytes: (128 + rows) rows x 36 B arrive at ~21 B per cycle per CU from L2.
// The slowest of the three sets the step; the first superstep's loads and the epilogue
// are not overlapped.  The model only has to rank the candidate chunk heights: timing every
// height on the box picks the same one as the model on each of the page shapes and on the
// dense 8192x4096x4096 shape (absolute times are ~2.5x the model's).
double tile_cycles(int rows, int k)
{
    const int rpad = (rows + 31) & ~31;
    const int steps = (k + 255) / 256 * (256 / kStepK);   // a short last superstep costs a full one
    const double mfma = 4.0 * (rpad / 32) * 35.0;
    const double valu = (2.0 * 26.0 + 18.0 * ((rpad + 63) / 64)) * 4.6;
    const double load = (kTileCols + rpad) * 36.0 / 21.0;
    return steps * std::max(std::max(mfma, valu), load) + 4.0 * load + 3000.0;
}

struct Schedule {
    int chunk_rows = 0;
    double makespan = 0;
    std::vector<std::vector<TileDesc>> per_wg;
};

// Build and balance the tile list for chunk height R (group indices are schedule positions;
// group gi has m_sched[gi] rows, n_sched[gi] columns and K = k_sched[gi]).
Schedule build_schedule(int R, const std::vector<int>& m_sched, const std::vector<int>& n_sched,
                        const std::vector<int>& k_sched, int num_wgs)
{
    Schedule S;
    S.chunk_rows = R;
    S.per_wg.assign(num_wgs, {});
    struct Cls {
        double cost;
        std::vector<std::pair<double, TileDesc>> tiles;
    };
    std::vector<Cls> classes;
    for (int gi = 0; gi < (int)m_sched.size(); ++gi) {
        const int mi = m_sched[gi], k = k_sched[gi];
        if (mi <= 0) continue;
        const int ntiles_n = ceil_div(n_sched[gi], kTileCols);
        const int chunks = ceil_div(mi, R);
        const int rp = (ceil_div(mi, chunks) + 31) / 32 * 32;
        for (int tn = 0; tn < ntiles_n; ++tn) {
            Cls c{0.0, {}};
            for (int row0 = 0; row0 < mi; row0 += rp) {
                const int rows = std::min(rp, mi - row0);
                const double cost = tile_cycles(rows, k);
                c.tiles.push_back({cost, TileDesc{gi, row0, rows, tn * kTileCols}});
                c.cost += cost;
            }
            classes.push_back(std::move(c));
        }
    }
    // classes (tiles sharing B columns) to XCDs, largest first, least-loaded XCD
    const int xcds = std::min(kXcds, num_wgs);
    std::vector<int> order(classes.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return classes[a].cost > classes[b].cost; });
    std::vector<double> xload(xcds, 0.0);
    std::vector<std::vector<std::pair<double, TileDesc>>> xtiles(xcds);
    for (int ci : order) {
        const int x = (int)(std::min_element(xload.begin(), xload.end()) - xload.begin());
        xload[x] += classes[ci].cost;
        for (auto& t : classes[ci].tiles) xtiles[x].push_back(t);
    }
    // inside an XCD: LPT over its workgroups (b = x + xcds * slot); stable order keeps the
    // tiles of one class next to each other, so they tend to run in the same round
    std::vector<double> wload(num_wgs, 0.0);
    for (int x = 0; x < xcds; ++x) {
        auto& v = xtiles[x];
        std::stable_sort(v.begin(), v.end(), [](const auto& a, const auto& b) { return a.first > b.first; });
        std::vector<int> wgs;
        for (int b = x; b < num_wgs; b += xcds) wgs.push_back(b);
        for (auto& t : v) {
            int best = wgs[0];
            for (int b : wgs)
                if (wload[b] < wload[best]) best = b;
            wload[best] += t.first;
            S.per_wg[best].push_back(t.second);
        }
    }
    S.makespan = num_wgs ? *std::max_element(wload.begin(), wload.end()) : 0.0;
    return S;
}

}  // namespace

extern "C" const char* nvfp4_gg_status_string(nvfp4_gg_status_t s)
{
    switch (s) {
    case NVFP4_GG_OK: return "success";
    case NVFP4_GG_EINVAL: return "invalid argument";
    case NVFP4_GG_EALIGN: return "device pointer not 16-byte aligned";
    case NVFP4_GG_ENOMEM: return "host or device allocation failed";
    case NVFP4_GG_EHIP: return "HIP runtime error";
    case NVFP4_GG_EUNSUPPORTED: return "unsupported device or configuration";
    }
    return "unknown status";
}

// Free the plan's device schedule on its device, after that device has finished the work
// already enqueued (a launch may still be reading the schedule).
static void free_device(nvfp4_gg_plan_s* p)
{
    if (p->d_tiles == nullptr && p->d_wg_begin == nullptr) return;
    int prev = -1;
    const bool switch_dev = hipGetDevice(&prev) == hipSuccess && prev != p->device;
    if (switch_dev) (void)hipSetDevice(p->device);
    (void)hipDeviceSynchronize();
    if (p->d_tiles) (void)hipFree(p->d_tiles);
    if (p->d_wg_begin) (void)hipFree(p->d_wg_begin);
    if (switch_dev) (void)hipSetDevice(prev);
    p->d_tiles = nullptr;
    p->d_wg_begin = nullptr;
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
        bool all256 = true;
        for (int i = 0; i < g; ++i) all256 = all256 && (problems[i].k % 256) == 0;
        p->variant = scale_layout == NVFP4_GG_SCALES_BLOCKED ? kVariantPersistentBlocked
                     : all256                                ? kVariantPersistent
                                                             : kVariantPersistentKTail;
        p->shape = variant_shape(p->variant);
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
        std::vector<int> m_sched(g), n_sched(g), k_sched(g);
        for (int s = 0; s < g; ++s) {
            m_sched[s] = p->m[p->order[s]];
            n_sched[s] = p->ns[p->order[s]];
            k_sched[s] = p->ks[p->order[s]];
        }

        // pick the chunk height with the smallest estimated makespan
        Schedule best;
        bool have = false;
        for (int R : {96, 64, 32}) {
            Schedule S = build_schedule(R, m_sched, n_sched, k_sched, num_cus);
            if (!have || S.makespan < best.makespan * 0.999) {
                best = std::move(S);
                have = true;
            }
        }
        p->chunk_rows = best.chunk_rows;
        p->est_cycles = best.makespan;

        // flatten: tiles[b] is the first tile of workgroup b (rows = 0 if it has none), so
        // that a workgroup can fetch it without first reading its range; the further tiles
        // of workgroup b follow at tiles[wg_begin[b] .. wg_begin[b+1]).  The grid ends at the
        // last busy workgroup.
        int last = -1;
        for (int b = 0; b < num_cus; ++b)
            if (!best.per_wg[b].empty()) last = b;
        p->grid = last + 1;
        p->tiles.assign(p->grid, TileDesc{0, 0, 0, 0});
        p->wg_begin.assign(p->grid + 1, p->grid);
        for (int b = 0; b < p->grid; ++b) {
            const auto& v = best.per_wg[b];
            if (!v.empty()) p->tiles[b] = v[0];
            p->wg_begin[b] = (int)p->tiles.size();
            for (size_t i = 1; i < v.size(); ++i) p->tiles.push_back(v[i]);
        }
        p->wg_begin[p->grid] = (int)p->tiles.size();
        p->total_tiles = 0;
        for (const auto& t : p->tiles) p->total_tiles += t.rows > 0 ? 1 : 0;

        // informational per-group tile prefix (schedule order)
        p->tile_begin.assign(g + 1, 0);
        for (int s = 0; s < g; ++s) {
            const int chunks = m_sched[s] ? ceil_div(m_sched[s], p->chunk_rows) : 0;
            p->tile_begin[s + 1] = p->tile_begin[s] + chunks * ceil_div(n_sched[s], kTileCols);
        }
    } catch (...) {
        delete p;
        return NVFP4_GG_ENOMEM;
    }

    if (device != NVFP4_GG_DEVICE_NONE && p->total_tiles > 0) {
        int prev = -1;
        if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) {
            delete p;
            return NVFP4_GG_EHIP;
        }
        bool ok = hipMalloc(reinterpret_cast<void**>(&p->d_tiles), sizeof(TileDesc) * p->tiles.size()) == hipSuccess &&
                  hipMalloc(reinterpret_cast<void**>(&p->d_wg_begin), sizeof(int) * p->wg_begin.size()) == hipSuccess;
        ok = ok &&
             hipMemcpy(p->d_tiles, p->tiles.data(), sizeof(TileDesc) * p->tiles.size(), hipMemcpyHostToDevice) ==
                 hipSuccess &&
             hipMemcpy(p->d_wg_begin, p->wg_begin.data(), sizeof(int) * p->wg_begin.size(), hipMemcpyHostToDevice) ==
                 hipSuccess;
        (void)hipSetDevice(prev);
        if (!ok) {
            free_device(p);
            delete p;
            return NVFP4_GG_ENOMEM;
        }
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
    args.ntiles = plan->total_tiles;
    for (int s = 0; s < plan->g; ++s) {
        const int i = plan->order[s];
        const int mi = plan->m[i];
        GroupArgs& G = args.grp[s];
        G.m = mi;
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
    if (plan->total_tiles == 0) return NVFP4_GG_OK;

    args.tiles = plan->d_tiles;
    args.wg_begin = plan->d_wg_begin;
    if (launch_variant(plan->variant, args, plan->grid, stream) != hipSuccess) return NVFP4_GG_EHIP;
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
    info->tile_m = plan->chunk_rows;
    info->tile_n = kTileCols;
    info->total_tiles = plan->total_tiles;
    info->grid = plan->grid;
    info->block = plan->shape.block;
    info->lds_bytes = plan->shape.lds_bytes;
    info->variant = plan->variant;
    for (int s = 0; s < plan->g; ++s) info->order[s] = plan->order[s];
    for (int s = 0; s <= plan->g; ++s) info->tile_begin[s] = plan->tile_begin[s];
    info->scale_layout = plan->scale_layout;
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
    free_device(plan);
    delete plan;
}
