// gfx950 (CDNA4) kernel of the NVFP4 grouped GEMM.
//
// C_i = dequant(A_i) * dequant(B_i)^T for every group i, fp32 accumulation, fp16 output
// rounded to nearest even (operation as on the page "kernelindex submission 503584",
// custom_kernel docstring and kernel configuration block; rounding as in epilogue_store of
// "kernelindex submission 498317").
//
// CDNA4's block-scaled FP4 matrix instructions take one power-of-two (E8M0) scale per 32
// K elements; NVFP4 carries one E4M3 scale (with 3 mantissa bits) per 16.  So both
// operands are dequantised exactly to fp16: an E2M1 value times an E4M3 value has at most
// 6 significant bits and magnitude in [2^-10, 2688], so it is an exact normal fp16
// number, and the contraction runs on the fp16 MFMA with fp32 sums.
//
// Structure of one workgroup (8 waves, 2 per SIMD) working on a (<= 128 rows) x 256
// columns tile; wave w computes rows 64 (w >> 2) .. +64 and columns 64 (w & 3) .. +64:
//   * A 4-slot LDS ring receives, per K step of 128, the raw bytes of the step (B rows,
//     A rows and their scales) straight from HBM through direct-to-LDS loads (no VGPR
//     staging); three steps are in flight ahead of the one being computed.
//   * B (the large operand) is dequantised in registers right before its MFMAs, by the
//     two waves that own its columns.
//   * A (shared by the 4 waves of a row half) is dequantised once per workgroup into fp16
//     LDS buffers, half a step ahead, and read back as MFMA fragments.
//   * v_mfma_f32_32x32x16_f16 takes the B fragment as its M-side operand, so each lane
//     ends up holding runs of 4 consecutive C columns (8-byte fp16 stores).
// K is permuted inside each step, identically for A and B (the dot product is unchanged):
// MFMA sub-step t takes, in lane half h, the 8 K values starting at 64h + 8t.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_gg_internal.h"

namespace nvfp4gg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// Exact dequantisation helpers
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ h2_t splat2(_Float16 s)
{
    h2_t r;
    r.x = s;
    r.y = s;
    return r;
}

// E4M3FN byte SEL of x -> fp16 pair (hardware OCP E4M3 decode to fp32, exact; the value
// is a normal fp16 number or zero, so the conversion to fp16 is exact too).
template <int SEL>
__device__ __forceinline__ h2_t scale2(uint32_t x)
{
    return splat2((_Float16)__builtin_amdgcn_cvt_f32_fp8((int)x, SEL));
}

// 8 E2M1 codes (nibble i = element i, i.e. low nibble = even K) times one fp16 scale ->
// 4 dwords of fp16 pairs (element 2j in the low half of dword j).  The hardware FP4 ->
// fp16 conversion with scale 1.0 gives the exact E2M1 values; one packed fp16 multiply
// per pair applies the E4M3 scale exactly.
__device__ __forceinline__ u4_t dequant8(uint32_t x, h2_t s)
{
    u4_t o;
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * s);
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * s);
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * s);
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * s);
    return o;
}

// ---------------------------------------------------------------------------------------
// Tile geometry and LDS layout
// ---------------------------------------------------------------------------------------
namespace ring {
constexpr int THREADS = 512;
// 8 waves: wave w computes rows 64 (w >> 2) .. +64 and columns 64 (w & 3) .. +64
constexpr int BN = 256;              // columns per tile
constexpr int BM = 128;              // rows per tile
constexpr int BK = 128;              // K per step
constexpr int SLOTS = 4;             // ring depth: 3 steps in flight ahead of the one computed
// one ring slot: raw bytes of one step
constexpr int B_CODES = BN * (BK / 2);           // 16384: 256 rows x 64 B (chunk-swizzled)
constexpr int B_SCALES = BN * (BK / 16);         // 2048:  256 rows x 8 B
constexpr int A_CODES = BM * (BK / 2);           // 8192:  128 rows x 64 B
constexpr int A_SCALES = BM * (BK / 16);         // 1024:  128 rows x 8 B
constexpr int SLOT_BS = B_CODES;
constexpr int SLOT_A = B_CODES + B_SCALES;
constexpr int SLOT_AS = SLOT_A + A_CODES;
constexpr int SLOT = SLOT_AS + A_SCALES;         // 27648
// fp16 A, two half-step buffers of 64 K values per row
constexpr int A_ROW = 64 * 2 + 16;               // 144 B per row (padding spreads banks)
constexpr int A_HALF = BM * A_ROW;               // 18432
constexpr int A16 = SLOTS * SLOT;                // 110592
constexpr int LDS_BYTES = A16 + 2 * A_HALF;      // 147456
constexpr int VM_PER_STEP = 5;                   // direct-to-LDS loads per wave per step
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
}  // namespace ring

// Issue the direct-to-LDS loads of one K step into ring slot `slot`.  Per wave: 2 x 16 B
// (B codes), 1 x 4 B (B scales), 1 x 16 B (A codes) and 1 x 4 B on 32 lanes (A scales).
// B chunk q of row r is stored in 16-byte slot q ^ ((r >> 1) & 3) of the row, so that
// fragment reads of 8 consecutive rows hit 8 different bank groups.  Rows beyond n (B) or
// beyond the tile's rows (A) re-read the last valid row: those values only reach outputs
// that are never stored (B) or are replaced by zeros when dequantised (A).
__device__ __forceinline__ void ring_issue(uint8_t* smem, int slot, int step, const uint8_t* __restrict__ b,
                                           const uint8_t* __restrict__ sfb, int col0, int n,
                                           const uint8_t* __restrict__ a, const uint8_t* __restrict__ sfa, int rows,
                                           int k, int wave, int lane)
{
    using namespace ring;
    uint8_t* base = smem + slot * SLOT;
    const long qstride = k / 2, sstride = k / 16;
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * wave + ii;
        const int r = 16 * i + (lane >> 2);
        const int q = (lane & 3) ^ ((r >> 1) & 3);
        const long row = min(col0 + r, n - 1);
        __builtin_amdgcn_global_load_lds(b + row * qstride + step * (BK / 2) + 16 * q, base + i * 1024, 16, 0, 0);
    }
    {
        const int r = 32 * wave + (lane >> 1);
        const long row = min(col0 + r, n - 1);
        __builtin_amdgcn_global_load_lds(sfb + row * sstride + step * (BK / 16) + 4 * (lane & 1),
                                         base + SLOT_BS + wave * 256, 4, 0, 0);
    }
    {
        const int r = 16 * wave + (lane >> 2);
        const long row = min(r, rows - 1);
        __builtin_amdgcn_global_load_lds(a + row * qstride + step * (BK / 2) + 16 * (lane & 3), base + SLOT_A + wave * 1024,
                                         16, 0, 0);
    }
    if (lane < 32) {
        const int r = 16 * wave + (lane >> 1);
        const long row = min(r, rows - 1);
        __builtin_amdgcn_global_load_lds(sfa + row * sstride + step * (BK / 16) + 4 * (lane & 1),
                                         base + SLOT_AS + wave * 128, 4, 0, 0);
    }
}

// Wait until at most `steps_outstanding` (0, 1 or 2) later steps' loads of this wave are in
// flight.
__device__ __forceinline__ void vm_wait(int steps_outstanding)
{
    static_assert(ring::VM_PER_STEP == 5, "immediates below assume 5 loads per step");
    if (steps_outstanding >= 2) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else if (steps_outstanding == 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroup barrier for LDS hand-offs: waits for this wave's own LDS reads/writes, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding direct-to-LDS
// loads (those are waited for explicitly with vm_wait, so later steps stay in flight).
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Dequantise half p of a step's A bytes (ring slot `slot`) into the fp16 half buffer
// `dst`.  Half p holds, per row, the K values 32p + 64h' + [0, 32) for h' = 0, 1, stored
// at byte 64h' + 2 (K - 32p - 64h').  Thread t: row t / 4, 16 K values (one scale block)
// at h' = (t >> 1) & 1, sub-block t & 1.  Rows >= rows become zeros.
__device__ __forceinline__ void ring_dequant_a(const uint8_t* smem, int slot, int p, uint8_t* dst, int rows, int tid)
{
    using namespace ring;
    const int r = tid >> 2, hh = (tid >> 1) & 1, sub = tid & 1;
    const uint8_t* base = smem + slot * SLOT;
    const u2_t q = *reinterpret_cast<const u2_t*>(base + SLOT_A + r * 64 + 16 * p + 32 * hh + 8 * sub);
    const uint32_t sc = base[SLOT_AS + r * 8 + 2 * p + 4 * hh + sub];
    u4_t* d = reinterpret_cast<u4_t*>(dst + r * A_ROW + 64 * hh + 32 * sub);
    if (r < rows) {
        const h2_t s = scale2<0>(sc);
        d[0] = dequant8(q.x, s);
        d[1] = dequant8(q.y, s);
    } else {
        const u4_t z = {0u, 0u, 0u, 0u};
        d[0] = z;
        d[1] = z;
    }
}

// One wave's B bytes of a step, read from the ring: per 32-column block cb the lane's 32
// bytes of row 64 wn + 32 cb + j (K values 64h .. 64h+63) and their 4 scale bytes.
struct StepB {
    u4_t q[2][2];
    uint32_t s[2];
};

__device__ __forceinline__ void ring_read_b(StepB& r, const uint8_t* smem, int slot, int wn, int lane)
{
    using namespace ring;
    const int j = lane & 31, h = lane >> 5;
    const uint8_t* base = smem + slot * SLOT;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int row = 64 * wn + 32 * cb + j;
        const int sw = (row >> 1) & 3;
        r.q[cb][0] = *reinterpret_cast<const u4_t*>(base + row * 64 + 16 * ((2 * h) ^ sw));
        r.q[cb][1] = *reinterpret_cast<const u4_t*>(base + row * 64 + 16 * ((2 * h + 1) ^ sw));
        r.s[cb] = *reinterpret_cast<const uint32_t*>(base + SLOT_BS + row * 8 + 4 * h);
    }
}

// Fragments of MFMA sub-step T (0..7): B dequantised from the step's bytes (scale byte T/2
// of the lane's scale dword covers K values 64h + 8T ..), A read from the fp16 half buffer
// of sub-steps T & ~3 .. (T & ~3) + 3.
template <int NRB, int T>
__device__ __forceinline__ void frags(h8_t (&bf)[2], h8_t (&af)[NRB], const StepB& b, const uint8_t* arow)
{
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
        af[rb] = *reinterpret_cast<const h8_t*>(arow + rb * 32 * ring::A_ROW + 16 * (T & 3));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
        bf[cb] = __builtin_bit_cast(h8_t, dequant8(b.q[cb][T >> 2][T & 3], scale2<(T >> 1)>(b.s[cb])));
}

template <int NRB>
__device__ __forceinline__ void mfmas(f16v_t (&acc)[NRB][2], const h8_t (&bf)[2], const h8_t (&af)[NRB])
{
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[0], af[rb], acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[1], af[rb], acc[rb][1], 0, 0, 0);
    }
}

// Sub-steps T0 .. T0+3 (one half step): fetch and dequantise the fragments of T+1 while
// the MFMAs of T run.
template <int NRB, int T>
__device__ __forceinline__ void substep(f16v_t (&acc)[NRB][2], h8_t (&bf)[2][2], h8_t (&af)[2][NRB], const StepB& b,
                                        const uint8_t* arow)
{
    if constexpr ((T & 3) != 3) frags<NRB, T + 1>(bf[(T + 1) & 1], af[(T + 1) & 1], b, arow);
    mfmas<NRB>(acc, bf[T & 1], af[T & 1]);
    __builtin_amdgcn_sched_barrier(0);
}

template <int NRB, int T0>
__device__ __forceinline__ void compute_half(f16v_t (&acc)[NRB][2], const StepB& b, const uint8_t* ahalf, int mh,
                                             int lane)
{
    const int j = lane & 31, h = lane >> 5;
    const uint8_t* arow = ahalf + (64 * mh + j) * ring::A_ROW + 64 * h;
    h8_t bf[2][2], af[2][NRB];
    frags<NRB, T0>(bf[T0 & 1], af[T0 & 1], b, arow);
    substep<NRB, T0 + 0>(acc, bf, af, b, arow);
    substep<NRB, T0 + 1>(acc, bf, af, b, arow);
    substep<NRB, T0 + 2>(acc, bf, af, b, arow);
    substep<NRB, T0 + 3>(acc, bf, af, b, arow);
}

// fp32 -> fp16 (round to nearest even) and store: lane (j, h) holds
// C[32 rb + j][colw + 32 cb + 8 q + 4 h + e], e = 0..3, relative to the wave's first row.
template <int NRB>
__device__ __forceinline__ void store_c(const f16v_t (&acc)[NRB][2], uint16_t* __restrict__ c, int n, int rows,
                                        int colw, int lane)
{
    const int j = lane & 31, h = lane >> 5;
    const bool vec_ok = (n & 3) == 0;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        const int r = rb * 32 + j;
        if (r >= rows) continue;
        uint16_t* crow = c + (long)r * n;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = colw + cb * 32 + q * 8 + h * 4;
                const uint16_t v0 = __builtin_bit_cast(uint16_t, (_Float16)acc[rb][cb][4 * q + 0]);
                const uint16_t v1 = __builtin_bit_cast(uint16_t, (_Float16)acc[rb][cb][4 * q + 1]);
                const uint16_t v2 = __builtin_bit_cast(uint16_t, (_Float16)acc[rb][cb][4 * q + 2]);
                const uint16_t v3 = __builtin_bit_cast(uint16_t, (_Float16)acc[rb][cb][4 * q + 3]);
                if (vec_ok && col + 4 <= n) {
                    *reinterpret_cast<u2_t*>(crow + col) =
                        u2_t{(uint32_t)v0 | ((uint32_t)v1 << 16), (uint32_t)v2 | ((uint32_t)v3 << 16)};
                } else {
                    if (col + 0 < n) crow[col + 0] = v0;
                    if (col + 1 < n) crow[col + 1] = v1;
                    if (col + 2 < n) crow[col + 2] = v2;
                    if (col + 3 < n) crow[col + 3] = v3;
                }
            }
        }
    }
}

// One full-K tile: rows [row0, row0 + rows) of group G, columns [256 ntile, +256).  Each
// wave runs the MFMAs of its NRB (0, 1 or 2) row blocks; every wave takes part in the
// loads, the A dequantisation and the barriers.
template <int NRB>
__device__ __forceinline__ void ring_tile(const GroupArgs& G, int n, int k, int row0, int rows, int ntile,
                                          uint8_t* smem)
{
    using namespace ring;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int mh = wave >> 2, wn = wave & 3;
    const int col0 = ntile * BN;
    const uint8_t* a = G.a + (long)row0 * (k / 2);
    const uint8_t* sfa = G.sfa + (long)row0 * (k / 16);
    const int steps = k / BK;
    uint8_t* ah0 = smem + A16;
    uint8_t* ah1 = smem + A16 + A_HALF;

    f16v_t acc[NRB > 0 ? NRB : 1][2];
#pragma unroll
    for (int rb = 0; rb < (NRB > 0 ? NRB : 1); ++rb) {
        acc[rb][0] = f16v_t{};
        acc[rb][1] = f16v_t{};
    }

    // prologue: steps 0..2 in flight; wait for step 0, dequantise its first A half
    for (int s = 0; s < SLOTS - 1 && s < steps; ++s)
        ring_issue(smem, s, s, G.b, G.sfb, col0, n, a, sfa, rows, k, wave, lane);
    vm_wait(min(steps - 1, SLOTS - 2));
    barrier_lds();
    ring_dequant_a(smem, 0, 0, ah0, rows, tid);
    barrier_lds();

    for (int s = 0; s < steps; ++s) {
        if (s + SLOTS - 1 < steps)
            ring_issue(smem, (s + SLOTS - 1) % SLOTS, s + SLOTS - 1, G.b, G.sfb, col0, n, a, sfa, rows, k, wave, lane);
        const int slot = s % SLOTS;
        StepB b;
        if constexpr (NRB > 0) ring_read_b(b, smem, slot, wn, lane);
        // half 0: compute from ah0, dequantise the second A half of this step into ah1
        if constexpr (NRB > 0) compute_half<NRB, 0>(acc, b, ah0, mh, lane);
        ring_dequant_a(smem, slot, 1, ah1, rows, tid);
        // the next step's bytes must have landed before half 1 dequantises them
        vm_wait(min(steps - 1, s + SLOTS - 1) - (s + 1));
        barrier_lds();
        // half 1: compute from ah1, dequantise the first A half of the next step into ah0
        if constexpr (NRB > 0) compute_half<NRB, 4>(acc, b, ah1, mh, lane);
        if (s + 1 < steps) ring_dequant_a(smem, (s + 1) % SLOTS, 0, ah0, rows, tid);
        barrier_lds();
    }
    if constexpr (NRB > 0)
        store_c<NRB>(acc, G.c + (long)(row0 + 64 * mh) * n, n, rows - 64 * mh, col0 + 64 * wn, lane);
}

__global__ __launch_bounds__(ring::THREADS) void nvfp4_gg_ring(KernArgs args)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[ring::LDS_BYTES];
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.g && t >= args.tile_begin[gi + 1]) ++gi;
    const GroupArgs& G = args.grp[gi];
    const int local = t - args.tile_begin[gi];
    const int mchunk = local % G.tiles_m, ntile = local / G.tiles_m;
    const int row0 = mchunk * G.rows_per_tile;
    const int rows = min(G.rows_per_tile, G.m - row0);
    // row blocks of this wave's 64-row half (wave-uniform)
    const int mh = (threadIdx.x >> 6) >> 2;
    const int rows_h = min(max(rows - 64 * mh, 0), 64);
    switch ((rows_h + 31) >> 5) {
    case 0: ring_tile<0>(G, args.n, args.k, row0, rows, ntile, smem); break;
    case 1: ring_tile<1>(G, args.n, args.k, row0, rows, ntile, smem); break;
    default: ring_tile<2>(G, args.n, args.k, row0, rows, ntile, smem); break;
    }
}

VariantShape variant_shape(int variant)
{
    switch (variant) {
    case kVariantRing:
        return VariantShape{ring::BM, ring::BN, ring::THREADS, ring::LDS_BYTES};
    default:
        return VariantShape{0, 0, 0, 0};
    }
}

hipError_t launch_variant(int variant, const KernArgs& args, int grid, hipStream_t stream)
{
    if (grid <= 0) return hipSuccess;
    switch (variant) {
    case kVariantRing: {
        KernArgs a = args;
        void* params[] = {&a};
        return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_ring), dim3(grid), dim3(ring::THREADS), params, 0,
                               stream);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4gg
