// gfx950 (CDNA4) kernels of the NVFP4 grouped GEMM.
//
// C_i = dequant(A_i) * dequant(B_i)^T for every group i, fp32 accumulation, fp16 output
// rounded to nearest even (operation as on the page "kernelindex submission 503584",
// custom_kernel docstring and kernel configuration block; rounding as in epilogue_store of
// "kernelindex submission 498317").
//
// CDNA4's block-scaled FP4 matrix instructions take one power-of-two (E8M0) scale per 32
// K elements; NVFP4 carries one E4M3 scale (with 3 mantissa bits) per 16.  So both
// operands are dequantised exactly to fp16 in registers: an E2M1 value times an E4M3
// value has at most 6 significant bits and magnitude in [2^-10, 2688], so it is an
// exact normal fp16 number, and the contraction runs on the fp16 MFMA with fp32 sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_gg_internal.h"

namespace nvfp4gg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// Exact dequantisation helpers
// ---------------------------------------------------------------------------------------

// E4M3FN code -> fp16, exact for every finite code (bias 7; exponent field 0 is
// subnormal M * 2^-9).  Built through fp32 so that no fp16 subnormal is involved.
__device__ __forceinline__ _Float16 e4m3fn_to_f16(uint32_t q)
{
    const uint32_t E = (q >> 3) & 15u, M = q & 7u;
    const float mag = (E == 0u) ? (float)M * 0x1p-9f : __uint_as_float(((E + 120u) << 23) | (M << 20));
    return (_Float16)((q & 0x80u) ? -mag : mag);
}

__device__ __forceinline__ h2_t splat2(_Float16 s)
{
    h2_t r;
    r.x = s;
    r.y = s;
    return r;
}

// Eight E2M1 codes (one dword; nibble i is element i, i.e. low nibble = even K) sharing
// the scale `s` -> four dwords of fp16 pairs (element 2j in the low half of out[j]).
// Every E2M1 magnitude is an fp16 number whose low byte is zero, so a byte permute
// through an 8-entry table of fp16 high bytes decodes it; the sign bit is OR-ed in and
// one packed fp16 multiply applies the scale (exact, see above).
__device__ __forceinline__ void dequant8(uint32_t x, h2_t s, uint32_t out[4])
{
    const uint32_t kLutLo = 0x3E3C3800u;  // high bytes of fp16 0, 0.5, 1, 1.5
    const uint32_t kLutHi = 0x46444240u;  // high bytes of fp16 2, 3, 4, 6
    const uint32_t em_even = x & 0x07070707u;
    const uint32_t em_odd = (x >> 4) & 0x07070707u;
    const uint32_t hb_even = __builtin_amdgcn_perm(kLutHi, kLutLo, em_even) | ((x << 4) & 0x80808080u);
    const uint32_t hb_odd = __builtin_amdgcn_perm(kLutHi, kLutLo, em_odd) | (x & 0x80808080u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // bytes of the result: [0, hb_even.byte j, 0, hb_odd.byte j]; selector 12 gives 0x00
        const uint32_t sel = 0x0Cu | ((uint32_t)j << 8) | (0x0Cu << 16) | ((uint32_t)(4 + j) << 24);
        const uint32_t p = __builtin_amdgcn_perm(hb_odd, hb_even, sel);
        const h2_t v = __builtin_bit_cast(h2_t, p) * s;
        out[j] = __builtin_bit_cast(uint32_t, v);
    }
}

// ---------------------------------------------------------------------------------------
// Variant 0: one BMxBN output tile per workgroup, 4 waves in a 2x2 arrangement, each wave
// 64x64 = 4x4 MFMA blocks of 16x16.  Per K step of BK, the workgroup loads the packed
// A and B slabs (16-byte loads), dequantises them once into LDS as fp16 and runs
// v_mfma_f32_16x16x32_f16 out of LDS.
// ---------------------------------------------------------------------------------------
namespace v0 {
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int THREADS = 256;
constexpr int LDS_ROW = BK * 2 + 16;  // bytes per fp16 row, padded by 16 B
constexpr int LDS_BYTES = (BM + BN) * LDS_ROW;
}  // namespace v0

// Load a 128-row x BK slab of one operand (rows >= nrows read as zero), dequantise it
// and store it as fp16 rows of LDS_ROW bytes.
__device__ __forceinline__ void stage_operand_v0(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sf,
                                                 int row0, int nrows, int k, int k0, uint8_t* lds, int tid)
{
    using namespace v0;
    const long qstride = k / 2, sstride = k / 16;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = tid + THREADS * j;  // 512 chunks of 16 B: 128 rows x 4
        const int r = c >> 2, part = c & 3;
        const int grow = row0 + r;
        u4_t codes = {0u, 0u, 0u, 0u};
        uint32_t sc = 0u;
        if (grow < nrows) {
            codes = *reinterpret_cast<const u4_t*>(q + (long)grow * qstride + (k0 >> 1) + part * 16);
            sc = *reinterpret_cast<const uint16_t*>(sf + (long)grow * sstride + (k0 >> 4) + part * 2);
        }
        const h2_t s_lo = splat2(e4m3fn_to_f16(sc & 0xFFu));
        const h2_t s_hi = splat2(e4m3fn_to_f16(sc >> 8));
        uint32_t o[16];
        dequant8(codes.x, s_lo, o + 0);
        dequant8(codes.y, s_lo, o + 4);
        dequant8(codes.z, s_hi, o + 8);
        dequant8(codes.w, s_hi, o + 12);
        u4_t* dst = reinterpret_cast<u4_t*>(lds + r * LDS_ROW + part * 64);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            u4_t w = {o[4 * v], o[4 * v + 1], o[4 * v + 2], o[4 * v + 3]};
            dst[v] = w;
        }
    }
}

__global__ __launch_bounds__(v0::THREADS) void nvfp4_gg_tiled128(KernArgs args)
{
    using namespace v0;
    __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
    uint8_t* sA = smem;
    uint8_t* sB = smem + BM * LDS_ROW;

    // tile -> (group, m tile, n tile); groups are in schedule order, m tile fastest
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.g && t >= args.tile_begin[gi + 1]) ++gi;
    const GroupArgs& G = args.grp[gi];
    const int local = t - args.tile_begin[gi];
    const int tm = local % G.tiles_m, tn = local / G.tiles_m;
    const int row0 = tm * BM, col0 = tn * BN;
    const int n = args.n, k = args.k;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    f4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < k; k0 += BK) {
        __syncthreads();
        stage_operand_v0(G.a, G.sfa, row0, G.m, k, k0, sA, tid);
        stage_operand_v0(G.b, G.sfb, col0, n, k, k0, sB, tid);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            h8_t a[4], b[4];
            const int koff = (kk * 32 + (lane >> 4) * 8) * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const h8_t*>(sA + (wm * 64 + i * 16 + (lane & 15)) * LDS_ROW + koff);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const h8_t*>(sB + (wn * 64 + j * 16 + (lane & 15)) * LDS_ROW + koff);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // epilogue: lane holds rows 4*(lane/16)+s, column lane%16 of each 16x16 block
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = col0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int row = row0 + wm * 64 + i * 16 + (lane >> 4) * 4 + s;
                if (row < G.m && col < n) {
                    const _Float16 h = (_Float16)acc[i][j][s];
                    G.c[(long)row * n + col] = __builtin_bit_cast(uint16_t, h);
                }
            }
        }
    }
}

VariantShape variant_shape(int variant)
{
    switch (variant) {
    case kVariantTiled128:
        return VariantShape{v0::BM, v0::BN, v0::THREADS, v0::LDS_BYTES};
    default:
        return VariantShape{0, 0, 0, 0};
    }
}

hipError_t launch_variant(int variant, const KernArgs& args, int grid, hipStream_t stream)
{
    if (grid <= 0) return hipSuccess;
    switch (variant) {
    case kVariantTiled128: {
        KernArgs a = args;
        void* params[] = {&a};
        return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_tiled128), dim3(grid), dim3(v0::THREADS),
                               params, 0, stream);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4gg
