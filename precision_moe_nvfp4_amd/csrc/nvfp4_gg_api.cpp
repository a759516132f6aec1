// Host side of the NVFP4 grouped GEMM C ABI: validation, planning and launch.
//
// Planning follows the host path of custom_kernel on the page "kernelindex submission
// 503584": groups are ordered by tile work, largest first, and tiles are numbered through
// the exclusive prefix sum of the per-group tile counts, m tile fastest inside a group.
// Unlike that page (which re-uploads a pointer table to device memory whenever the
// pointers change), the whole group table here travels by value in the kernel
// arguments, so a call needs no device allocation and no host-to-device copy.
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
    int g, n, k;
    int device;
    int num_cus;
    int variant;
    VariantShape shape;
    int total_tiles;
    int grid;
    std::vector<int> m;          // caller order
    std::vector<int> tiles_m;    // m chunks per group, caller order
    std::vector<int> rows_per;   // rows per m chunk, caller order
    std::vector<int> order;      // order[p] = caller group at schedule position p
    std::vector<int> tile_begin; // size g + 1, schedule order
};

namespace {

constexpr uint32_t kPlanMagic = 0x4E564634u;  // "NVF4"
constexpr int kMaxRows = 1 << 20;
constexpr int kNominalCUs = 256;               // MI355X

bool plan_ok(const nvfp4_gg_plan_s* p) { return p != nullptr && p->magic == kPlanMagic; }

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
    if (out == nullptr) return NVFP4_GG_EINVAL;
    *out = nullptr;
    if (m == nullptr || g < 1 || n < 1 || k < 256 || (k % 256) != 0) return NVFP4_GG_EINVAL;
    if (g > NVFP4_GG_MAX_GROUPS) return NVFP4_GG_EUNSUPPORTED;
    for (int i = 0; i < g; ++i)
        if (m[i] < 0 || m[i] > kMaxRows) return NVFP4_GG_EINVAL;
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
        p->n = n;
        p->k = k;
        p->device = device;
        p->num_cus = num_cus;
        p->variant = kVariantRing;
        p->shape = variant_shape(p->variant);
        p->m.assign(m, m + g);
        p->tiles_m.assign(g, 0);
        p->rows_per.assign(g, 0);

        // m chunks: as few as the tile height allows, equal sizes rounded up to whole
        // 32-row MFMA blocks; then tile counts and the largest-work-first order
        std::vector<long> work(g);
        std::vector<int> tiles(g);
        for (int i = 0; i < g; ++i) {
            const int tm = ceil_div(m[i], p->shape.tile_m);
            int rp = tm ? ceil_div(m[i], tm) : 0;
            rp = (rp + 31) / 32 * 32;
            p->tiles_m[i] = tm;
            p->rows_per[i] = rp;
            tiles[i] = tm * ceil_div(n, p->shape.tile_n);
            work[i] = (long)m[i];
        }
        p->order.resize(g);
        std::iota(p->order.begin(), p->order.end(), 0);
        std::stable_sort(p->order.begin(), p->order.end(), [&](int a, int b) { return work[a] > work[b]; });
        p->tile_begin.assign(g + 1, 0);
        for (int s = 0; s < g; ++s) p->tile_begin[s + 1] = p->tile_begin[s] + tiles[p->order[s]];
        p->total_tiles = p->tile_begin[g];
        p->grid = p->total_tiles;
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
    args.n = plan->n;
    args.k = plan->k;
    args.total_tiles = plan->total_tiles;
    for (int s = 0; s < plan->g; ++s) {
        const int i = plan->order[s];
        const int mi = plan->m[i];
        GroupArgs& G = args.grp[s];
        G.m = mi;
        G.tiles_m = plan->tiles_m[i];
        G.rows_per_tile = plan->rows_per[i];
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
    for (int s = 0; s <= plan->g; ++s) args.tile_begin[s] = plan->tile_begin[s];
    args.tile_begin[plan->g + 1] = plan->total_tiles;

    if (plan->device == NVFP4_GG_DEVICE_NONE) return NVFP4_GG_EUNSUPPORTED;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return NVFP4_GG_EHIP;
    if (cur != plan->device) return NVFP4_GG_EINVAL;
    if (plan->total_tiles == 0) return NVFP4_GG_OK;

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
    info->tile_m = plan->shape.tile_m;
    info->tile_n = plan->shape.tile_n;
    info->total_tiles = plan->total_tiles;
    info->grid = plan->grid;
    info->block = plan->shape.block;
    info->lds_bytes = plan->shape.lds_bytes;
    info->variant = plan->variant;
    for (int s = 0; s < plan->g; ++s) info->order[s] = plan->order[s];
    for (int s = 0; s <= plan->g; ++s) info->tile_begin[s] = plan->tile_begin[s];
    return NVFP4_GG_OK;
}

extern "C" void nvfp4_gg_destroy(nvfp4_gg_plan_t plan)
{
    if (!plan_ok(plan)) return;
    plan->magic = 0;
    delete plan;
}
