// Internal interface between the host planner (nvfp4_gg_api.cpp) and the gfx950
// kernels (nvfp4_gg_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "nvfp4_gg.h"

namespace nvfp4gg {

// One group as the kernel sees it (schedule order, not caller order).
struct GroupArgs {
    const uint8_t* a;    // [m][k/2] packed E2M1
    const uint8_t* b;    // [n][k/2] packed E2M1
    const uint8_t* sfa;  // [m][k/16] E4M3FN
    const uint8_t* sfb;  // [n][k/16] E4M3FN
    uint16_t* c;         // [m][ldc] fp16 bits (columns < n written)
    int m;               // rows of this group
    int n;               // columns of C (rows of B)
    int k;               // K (multiple of 64)
    int ldc;             // C row stride in elements (>= n)
};

// One output tile: rows [row0, row0 + rows) of group `group` (schedule index), columns
// [col0, col0 + 128).
struct TileDesc {
    int group;
    int row0;
    int rows;
    int col0;
};

// Kernel arguments, passed by value: the whole group table rides in the kernarg segment;
// the tile list (built once by the planner) lives in device memory owned by the plan.
struct KernArgs {
    int g;
    int ntiles;
    const TileDesc* tiles;  // tiles[b]: first tile of workgroup b (rows = 0: none)
    const int* wg_begin;    // workgroup b then processes tiles[wg_begin[b] .. wg_begin[b+1])
    GroupArgs grp[NVFP4_GG_MAX_GROUPS];
};
static_assert(sizeof(KernArgs) <= 4096, "kernel arguments must fit the 4 KiB kernarg segment");

// Launch shapes of the kernel variants.
struct VariantShape {
    int tile_m, tile_n, block, lds_bytes;
};

enum Variant : int {
    kVariantPersistent = 2,         // persistent 8-wave workgroups over a planned tile list
    kVariantPersistentBlocked = 3,  // the same, reading 128x4 blocked scale tensors
    kVariantPersistentKTail = 4,    // row-major scales when some k is not a multiple of 256
};

VariantShape variant_shape(int variant);

// Enqueue one launch of `variant` with `grid` workgroups.
hipError_t launch_variant(int variant, const KernArgs& args, int grid, hipStream_t stream);

// Bytes of a 128x4 blocked scale tensor: ceil(rows / 128) row blocks of k / 64 atoms of 512 B
// (k a multiple of 64).
inline long blocked_scale_bytes(int rows, int k)
{
    return rows <= 0 ? 0 : (long)((rows + 127) / 128) * (k / 64) * 512;
}

// Enqueue the row-major -> blocked scale conversion (padding rows written as zero).
hipError_t launch_scales_to_blocked(void* dst, const void* src, int rows, int k, hipStream_t stream);

}  // namespace nvfp4gg
