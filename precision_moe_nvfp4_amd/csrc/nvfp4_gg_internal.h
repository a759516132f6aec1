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
    uint16_t* c;         // [m][n] fp16 bits
    int m;               // rows of this group
    int tiles_m;         // m chunks of this group
    int rows_per_tile;   // rows of each m chunk (the last may have fewer)
    int pad_;
};

// Kernel arguments, passed by value: the whole group table rides in the kernarg segment.
struct KernArgs {
    int g;
    int n;
    int k;
    int total_tiles;
    int tile_begin[NVFP4_GG_MAX_GROUPS + 2];  // exclusive prefix of tiles, schedule order
    GroupArgs grp[NVFP4_GG_MAX_GROUPS];
};
static_assert(sizeof(KernArgs) <= 4096, "kernel arguments must fit the 4 KiB kernarg segment");

// Launch shapes of the kernel variants.
struct VariantShape {
    int tile_m, tile_n, block, lds_bytes;
};

enum Variant : int {
    kVariantRing = 1,  // (<= 128 rows) x 256 tile, 8 waves, 4-slot direct-to-LDS ring
};

VariantShape variant_shape(int variant);

// Enqueue one launch of `variant` with `grid` workgroups.
hipError_t launch_variant(int variant, const KernArgs& args, int grid, hipStream_t stream);

}  // namespace nvfp4gg
