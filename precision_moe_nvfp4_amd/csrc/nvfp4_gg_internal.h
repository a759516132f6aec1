// Internal interface between the host planner (nvfp4_gg_api.cpp) and the gfx950
// kernels (nvfp4_gg_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "nvfp4_gg.h"

namespace nvfp4gg {

// Unit shapes the kernel is compiled for: (row blocks NA, column blocks NB) of 32 each.  A
// unit covers up to 32 NA rows of one group times 32 NB columns over the whole K; the four
// waves of a workgroup each hold its NA x NB accumulator blocks (16 blocks in the 256
// accumulation registers of a lane, up to 4 more in ordinary VGPRs).
#define NVFP4GG_UNIT_SHAPES(X) \
    X(1, 1) X(1, 2) X(1, 4) X(1, 8) \
    X(2, 1) X(2, 2) X(2, 3) X(2, 4) X(2, 5) X(2, 6) X(2, 8) X(2, 9) \
    X(3, 2) X(3, 3) X(3, 4) X(3, 5) X(3, 6) \
    X(4, 1) X(4, 2) X(4, 3) X(4, 4) X(4, 5) \
    X(5, 2) X(5, 3) X(5, 4) \
    X(6, 1) X(6, 2) X(6, 3) \
    X(7, 2) \
    X(8, 1) X(8, 2)

// The group table entry of `m_shape`: rows m in bits 0..20, the unit shape's NA in bits
// 21..24 and NB in bits 25..29.
constexpr int kMMask = (1 << 21) - 1;
constexpr int kNaShift = 21;
constexpr int kNbShift = 25;

// One group as the kernel sees it (schedule order, not caller order).
struct GroupArgs {
    const uint8_t* a;    // [m][k/2] packed E2M1
    const uint8_t* b;    // [n][k/2] packed E2M1
    const uint8_t* sfa;  // [m][k/16] E4M3FN (or the blocked layout)
    const uint8_t* sfb;  // [n][k/16] E4M3FN (or the blocked layout)
    uint16_t* c;         // [m][ldc] fp16 bits (columns < n written)
    int m_shape;         // m | na << 21 | nb << 25 (see above)
    int n;               // columns of C (rows of B)
    int k;               // K (multiple of 64)
    int ldc;             // C row stride in elements (>= n)
};

constexpr int kFlagBlockedScales = 1;

// Kernel arguments, passed by value: the whole schedule is the group table (the unit
// sequence and every workgroup's share of it follow from it), so a call needs no device
// memory besides the operands.
struct KernArgs {
    int g;
    int units;   // units over all groups
    int vq;      // virtual workgroups per XCD; the grid is 8 vq
    int flags;   // kFlag*
    GroupArgs grp[NVFP4_GG_MAX_GROUPS];
};
static_assert(sizeof(GroupArgs) == 56, "group table entry layout");
static_assert(sizeof(KernArgs) <= 4096, "kernel arguments must fit the 4 KiB kernarg segment");

constexpr int kUnitThreads = 256;
constexpr int kUnitLdsBytes = 160 * 1024;

// Enqueue one launch of the unit kernel with `grid` workgroups.
hipError_t launch_units(const KernArgs& args, int grid, hipStream_t stream);

// Whether the kernel is compiled for unit shape (na, nb), and its ring depth.
bool unit_shape_supported(int na, int nb);
int unit_shape_slots(int na, int nb);

// Bytes of a 128x4 blocked scale tensor: ceil(rows / 128) row blocks of k / 64 atoms of 512 B
// (k a multiple of 64).
inline long blocked_scale_bytes(int rows, int k)
{
    return rows <= 0 ? 0 : (long)((rows + 127) / 128) * (k / 64) * 512;
}

// Enqueue the row-major -> blocked scale conversion (padding rows written as zero).
hipError_t launch_scales_to_blocked(void* dst, const void* src, int rows, int k, hipStream_t stream);

}  // namespace nvfp4gg
