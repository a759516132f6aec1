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
// Structure: a persistent grid (one workgroup of 8 waves, 2 per SIMD, per CU) walks a tile
// list built by the host planner.  A tile is up to 256 rows of one group x 256 columns;
// wave w owns columns 64 (w & 3) .. +64 and up to 128 rows, so each dequantised B fragment
// feeds up to 4 MFMAs:
//   * An LDS ring receives, per K step of 64, the raw bytes of the step (B rows, A rows
//     and their scales) straight from HBM through direct-to-LDS loads (no VGPR staging).
//     Its depth follows the tile height (4 slots at 256 rows, 14 at 32 rows), so tiles
//     with little MFMA work per step keep more steps in flight.
//   * B (the large operand) is dequantised in registers right before its MFMAs.
//   * A (shared by the waves) is dequantised once per workgroup into an fp16 LDS buffer,
//     one step ahead, and read back as MFMA fragments.
//   * v_mfma_f32_32x32x16_f16 takes the B fragment as its M-side operand, so each lane
//     ends up holding runs of 4 consecutive C columns (8-byte fp16 stores).
// K is permuted inside each step, identically for A and B (the dot product is unchanged):
// MFMA sub-step t takes, in lane half h, the 8 K values starting at 32h + 8t.
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

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default mode).
__device__ __forceinline__ uint16_t f16_bits_rne(float f)
{
    const _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
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
// Geometry and LDS layout
// ---------------------------------------------------------------------------------------
namespace pk {
constexpr int THREADS = 512;         // 8 waves, 2 per SIMD
constexpr int BN = 256;              // tile columns: wave w owns columns 64 (w & 3) .. +64
constexpr int RMAX = 128;            // tile rows (multiple of 32)
constexpr int BK = 64;               // K per compute step (4 MFMA sub-steps of 16)
constexpr int SK = 256;              // K per load superstep
constexpr int SUB = SK / BK;         // compute steps per superstep
constexpr int ROWB = SK / 2;         // code bytes per row and superstep: one 128-byte line
constexpr int SCB = SK / 16;         // scale bytes per row and superstep
constexpr int LDS_BYTES = 160 * 1024;
// LDS layout of a tile with rpad rows (all offsets multiples of 16 bytes):
//   [0, 2 * rpad * A_ROW)      fp16 A of two compute steps (double buffer)
//   then ring_slots(rpad) slots of slot_bytes(rpad), each holding the raw bytes of one
//   superstep:
//     B codes   256 rows x 128 B   at 0            (16-byte chunk c of row r at c ^ (r & 7))
//     B scales  256 rows x 16 B    at B_SCALES_AT
//     A codes   rpad rows x 128 B  at A_CODES_AT   (same chunk swizzle)
//     A scales  rpad rows x 16 B   at A_CODES_AT + 128 rpad
// Whole 128-byte lines per row and load instruction: a wave's 16-byte lanes cover 8 rows
// per instruction instead of 32, which is what lets a CU pull shared operand rows out of
// L2 at ~3x the rate of 32-byte row pieces.
constexpr int A_ROW = BK * 2 + 16;                    // 144 B per fp16 row (spreads banks)
constexpr int B_SCALES_AT = BN * ROWB;                // 32768
constexpr int A_CODES_AT = B_SCALES_AT + BN * SCB;    // 36864
__host__ __device__ constexpr int slot_bytes(int rpad) { return A_CODES_AT + rpad * (ROWB + SCB); }
__host__ __device__ constexpr int ring_base(int rpad) { return 2 * rpad * A_ROW; }
__host__ __device__ constexpr int ring_slots(int rpad)
{
    return (LDS_BYTES - ring_base(rpad)) / slot_bytes(rpad) > 3 ? 3 : (LDS_BYTES - ring_base(rpad)) / slot_bytes(rpad);
}
static_assert(ring_slots(RMAX) >= 2, "the tallest tile needs at least 2 ring slots");
static_assert(8 * 4 * 4 * 1024 <= LDS_BYTES, "pair-reduction area must fit in LDS");
}  // namespace pk

// Wave roles: both waves of a pair (x = w >> 2) take all tile rows and split the MFMA
// sub-steps (x takes sub-steps x and x + 2 of each compute step); the two partial sums
// are added through LDS at the end.

// Per-wave direct-to-LDS loads of one superstep.  Wave w fetches B rows 32w .. +32 (four
// instructions of 8 rows x 128 B) and their scales (lanes < 32, 16 B each); the A rows are
// dealt round-robin: code instruction i (rows 8i .. +8) to wave i % 8, scale instruction q
// (rows 32q .. +32) to wave 7 - q.
struct SuperLoads {
    const uint8_t* b[4];  // B codes of this lane, superstep 0
    const uint8_t* sb;    // B scales of this lane (lanes < 32)
    const uint8_t* a[2];  // A codes of this lane, for the wave's A code instructions
    const uint8_t* sa;    // A scales of this lane (lanes < 32)
    int na;               // A code instructions of this wave (0 .. 2)
    int nsa;              // A scale instructions of this wave (0 or 1)
    int a_dst[2];         // LDS offsets (inside a slot) of the A code instructions
    int sa_dst;           // LDS offset (inside a slot) of the A scale instruction
    int ops;              // loads per superstep issued by this wave
};

__device__ __forceinline__ void pk_issue(uint8_t* slot_base, int t, const SuperLoads& L, int wave, int lane)
{
    using namespace pk;
    const long kb = (long)t * ROWB, ks = (long)t * SCB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(L.b[i] + kb, slot_base + (32 * wave + 8 * i) * ROWB, 16, 0, 0);
    if (lane < 32) __builtin_amdgcn_global_load_lds(L.sb + ks, slot_base + B_SCALES_AT + 32 * wave * SCB, 16, 0, 0);
    if (L.na > 0) __builtin_amdgcn_global_load_lds(L.a[0] + kb, slot_base + L.a_dst[0], 16, 0, 0);
    if (L.na > 1) __builtin_amdgcn_global_load_lds(L.a[1] + kb, slot_base + L.a_dst[1], 16, 0, 0);
    if (L.nsa > 0 && lane < 32) __builtin_amdgcn_global_load_lds(L.sa + ks, slot_base + L.sa_dst, 16, 0, 0);
}

// Wait until at most n of this wave's loads are in flight (0 <= n <= 30).
__device__ __forceinline__ void pk_wait_loads(int n)
{
#define NVFP4GG_WAIT_CASE(N) \
    case N: asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory"); break;
    switch (n) {
        NVFP4GG_WAIT_CASE(30) NVFP4GG_WAIT_CASE(29) NVFP4GG_WAIT_CASE(28) NVFP4GG_WAIT_CASE(27)
        NVFP4GG_WAIT_CASE(26) NVFP4GG_WAIT_CASE(25) NVFP4GG_WAIT_CASE(24) NVFP4GG_WAIT_CASE(23)
        NVFP4GG_WAIT_CASE(22) NVFP4GG_WAIT_CASE(21) NVFP4GG_WAIT_CASE(20) NVFP4GG_WAIT_CASE(19)
        NVFP4GG_WAIT_CASE(18) NVFP4GG_WAIT_CASE(17) NVFP4GG_WAIT_CASE(16) NVFP4GG_WAIT_CASE(15)
        NVFP4GG_WAIT_CASE(14) NVFP4GG_WAIT_CASE(13) NVFP4GG_WAIT_CASE(12) NVFP4GG_WAIT_CASE(11)
        NVFP4GG_WAIT_CASE(10) NVFP4GG_WAIT_CASE(9) NVFP4GG_WAIT_CASE(8) NVFP4GG_WAIT_CASE(7)
        NVFP4GG_WAIT_CASE(6) NVFP4GG_WAIT_CASE(5) NVFP4GG_WAIT_CASE(4) NVFP4GG_WAIT_CASE(3)
        NVFP4GG_WAIT_CASE(2) NVFP4GG_WAIT_CASE(1)
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef NVFP4GG_WAIT_CASE
}

// Workgroup barrier for LDS hand-offs: waits for this wave's own LDS reads/writes, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding direct-to-LDS
// loads (those are waited for explicitly, so later supersteps stay in flight).
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Dequantise the A bytes of compute step U of the superstep held at `slot_base` into the
// fp16 buffer `dst` (natural K order, A_ROW-byte rows).  Waves 0..3 (one per SIMD) take
// rpad pieces each; piece id covers row id / 4, K values 16 (id % 4) .. +16 of the step
// (8 code bytes, one scale byte).  Rows in [rows, rpad) become zeros.
template <int U>
__device__ __forceinline__ void pk_dequant_a(const uint8_t* slot_base, uint8_t* dst, int rows, int rpad, int wave,
                                             int lane)
{
    using namespace pk;
    if (wave >= 4) return;
    const uint8_t* codes = slot_base + A_CODES_AT;
    const uint8_t* scales = codes + rpad * ROWB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int id = wave * rpad + lane + 64 * i;
        if (lane + 64 * i >= rpad) continue;
        const int r = id >> 2, p = id & 3;
        u4_t* d = reinterpret_cast<u4_t*>(dst + r * A_ROW + 32 * p);
        if (r < rows) {
            const int chunk = 2 * U + (p >> 1);
            const u2_t q = *reinterpret_cast<const u2_t*>(codes + r * ROWB + 16 * (chunk ^ (r & 7)) + 8 * (p & 1));
            const h2_t sc = scale2<0>(scales[r * SCB + 4 * U + p]);
            d[0] = dequant8(q.x, sc);
            d[1] = dequant8(q.y, sc);
        } else {
            const u4_t z = {0u, 0u, 0u, 0u};
            d[0] = z;
            d[1] = z;
        }
    }
}

// One wave's B bytes of a step: per 32-column block cb, the lane's 16 bytes of row
// 64 wn + 32 cb + j (K values 32h .. 32h+31) and the two scale bytes of those values.
struct PkB {
    u4_t q[2];
    uint32_t s[2];
};

// B codes of compute step U: lane (j, h) reads chunk 2U + h of its row.  The row's 16
// scale bytes of the superstep are read once per superstep (pk_read_bs).
template <int U>
__device__ __forceinline__ void pk_read_b(PkB& r, const uint8_t* slot_base, const u4_t (&bs)[2], int wn, int lane)
{
    using namespace pk;
    const int j = lane & 31, h = lane >> 5;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int row = 64 * wn + 32 * cb + j;
        r.q[cb] = *reinterpret_cast<const u4_t*>(slot_base + row * ROWB + 16 * ((2 * U + h) ^ (row & 7)));
        const uint32_t w = bs[cb][U];
        r.s[cb] = h ? (w >> 16) : w;
    }
}

__device__ __forceinline__ void pk_read_bs(u4_t (&bs)[2], const uint8_t* slot_base, int wn, int lane)
{
    using namespace pk;
    const int j = lane & 31;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
        bs[cb] = *reinterpret_cast<const u4_t*>(slot_base + B_SCALES_AT + (64 * wn + 32 * cb + j) * SCB);
}

// Fragments of MFMA sub-step T (lane half h: K values 32h + 8T ..): B dequantised from the
// step's bytes (scale byte T/2 of the lane's pair), A read from the fp16 buffer.
template <int NRB, int T>
__device__ __forceinline__ void pk_frags(h8_t (&bf)[2], h8_t (&af)[NRB], const PkB& b, const uint8_t* arow)
{
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
        af[rb] = *reinterpret_cast<const h8_t*>(arow + rb * 32 * pk::A_ROW + 16 * T);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
        bf[cb] = __builtin_bit_cast(h8_t, dequant8(b.q[cb][T], scale2<(T >> 1)>(b.s[cb])));
}

template <int NRB>
__device__ __forceinline__ void pk_mfmas(f16v_t (&acc)[NRB][2], const h8_t (&bf)[2], const h8_t (&af)[NRB])
{
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        acc[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[0], af[rb], acc[rb][0], 0, 0, 0);
        acc[rb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[1], af[rb], acc[rb][1], 0, 0, 0);
    }
}

// One compute step of this wave's MFMAs: sub-steps x and x + 2.  The fragments of both
// are prepared before the MFMAs run.
template <int NRB>
__device__ __forceinline__ void pk_compute(f16v_t (&acc)[NRB][2], const PkB& b, const uint8_t* arow, int x)
{
    h8_t bf[2][2], af[2][NRB];
    if (x == 0) {
        pk_frags<NRB, 0>(bf[0], af[0], b, arow);
        pk_frags<NRB, 2>(bf[1], af[1], b, arow);
    } else {
        pk_frags<NRB, 1>(bf[0], af[0], b, arow);
        pk_frags<NRB, 3>(bf[1], af[1], b, arow);
    }
    pk_mfmas<NRB>(acc, bf[0], af[0]);
    __builtin_amdgcn_sched_barrier(0);
    pk_mfmas<NRB>(acc, bf[1], af[1]);
}

// fp32 -> fp16 (round to nearest even) and store of column block CB: lane (j, h) holds
// C[32 rb + j][colw + 32 CB + 8 q + 4 h + e], e = 0..3, relative to the wave's first row.
template <int NRB, int CB>
__device__ __forceinline__ void pk_store_cb(const f16v_t (&acc)[NRB][2], uint16_t* __restrict__ c, int n, int rows,
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
        for (int q = 0; q < 4; ++q) {
            const int col = colw + CB * 32 + q * 8 + h * 4;
            const uint16_t v0 = f16_bits_rne(acc[rb][CB][4 * q + 0]);
            const uint16_t v1 = f16_bits_rne(acc[rb][CB][4 * q + 1]);
            const uint16_t v2 = f16_bits_rne(acc[rb][CB][4 * q + 2]);
            const uint16_t v3 = f16_bits_rne(acc[rb][CB][4 * q + 3]);
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

// K-split pair reduction, column block GIVE handed to the partner and block KEEP kept:
// write acc[.][GIVE] to this wave's LDS area, wait for the partner, add the partner's
// contribution to acc[.][KEEP].  Area of wave (wn, x): 16 KiB at (wn * 2 + x) * 16 KiB.
template <int NRB, int GIVE, int KEEP>
__device__ __forceinline__ void pk_pair_reduce(f16v_t (&acc)[NRB][2], u4_t* red, int wn, int x, int lane)
{
    u4_t* mine = red + (wn * 2 + x) * 1024;
    const u4_t* theirs = red + (wn * 2 + (1 - x)) * 1024;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            mine[(rb * 4 + e) * 64 + lane] =
                u4_t{__float_as_uint(acc[rb][GIVE][4 * e + 0]), __float_as_uint(acc[rb][GIVE][4 * e + 1]),
                     __float_as_uint(acc[rb][GIVE][4 * e + 2]), __float_as_uint(acc[rb][GIVE][4 * e + 3])};
    barrier_lds();
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const u4_t o = theirs[(rb * 4 + e) * 64 + lane];
            // (element-wise __uint_as_float: __builtin_bit_cast of an ext-vector element
            // reads element 0 with this compiler)
            acc[rb][KEEP][4 * e + 0] += __uint_as_float(o.x);
            acc[rb][KEEP][4 * e + 1] += __uint_as_float(o.y);
            acc[rb][KEEP][4 * e + 2] += __uint_as_float(o.z);
            acc[rb][KEEP][4 * e + 3] += __uint_as_float(o.w);
        }
}

// Compute step U of superstep t (slot `cur`), then the A dequantisation of the next step
// (from `cur`, or from `nxt` when U is the last step of the superstep).
template <int NRB, int U>
__device__ __forceinline__ void pk_step(f16v_t (&acc)[NRB][2], const uint8_t* cur, const uint8_t* nxt,
                                        const u4_t (&bs)[2], uint8_t* a16, int s, int steps, int rows, int rpad,
                                        int wave, int lane)
{
    using namespace pk;
    const int wn = wave & 3, x = wave >> 2;
    const int j = lane & 31, h = lane >> 5;
    PkB b;
    pk_read_b<U>(b, cur, bs, wn, lane);
    pk_compute<NRB>(acc, b, a16 + (s & 1) * rpad * A_ROW + j * A_ROW + 64 * h, x);
    if (s + 1 < steps) {
        uint8_t* dst = a16 + ((s + 1) & 1) * rpad * A_ROW;
        if constexpr (U + 1 < SUB) pk_dequant_a<U + 1>(cur, dst, rows, rpad, wave, lane);
        else pk_dequant_a<0>(nxt, dst, rows, rpad, wave, lane);
    }
}

// One full-K tile (rows [row0, row0 + rows) of group G, columns [col0, col0 + 256)).  All
// 8 waves execute the same sequence of loads, dequantisations and barriers; NRB = rpad / 32
// only changes this wave's MFMAs and epilogue.
template <int NRB>
__device__ __noinline__ void pk_tile(const GroupArgs& G, int n_, int k_, int row0_, int rows_, int col0_, uint8_t* smem)
{
    using namespace pk;
    // workgroup-uniform scalars (the call passes them in vector registers)
    const int n = __builtin_amdgcn_readfirstlane(n_), k = __builtin_amdgcn_readfirstlane(k_);
    const int row0 = __builtin_amdgcn_readfirstlane(row0_), rows = __builtin_amdgcn_readfirstlane(rows_);
    const int col0 = __builtin_amdgcn_readfirstlane(col0_);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 3, x = wave >> 2;
    const int rpad = 32 * NRB;
    const int steps = k / BK, supers = k / SK;
    const long qs = k / 2, ss = k / 16;

    const int sbytes = slot_bytes(rpad), nslots = ring_slots(rpad);
    uint8_t* a16 = smem;
    uint8_t* ring = smem + ring_base(rpad);

    // this wave's loads (see SuperLoads); lane l of a code instruction covers row
    // (first row + l / 8) and stores LDS chunk l % 8, which holds global chunk
    // (l % 8) ^ (row & 7)
    SuperLoads L;
    {
        const int rl = lane >> 3, pos = lane & 7;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 32 * wave + 8 * i + rl;
            const long brow = min(col0 + r, n - 1);
            L.b[i] = G.b + brow * qs + 16 * (pos ^ (r & 7));
        }
        L.sb = G.sfb + (long)min(col0 + 32 * wave + (lane & 31), n - 1) * ss;
        const int na_total = rpad / 8, nsa_total = rpad / 32;
        L.na = 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int i = wave + 8 * q;    // A code instruction handled by this wave
            const int r = 8 * i + rl;
            L.a[q] = G.a + (long)(row0 + min(r, rows - 1)) * qs + 16 * (pos ^ (r & 7));
            L.a_dst[q] = A_CODES_AT + 8 * i * ROWB;
            if (i < na_total) L.na = q + 1;
        }
        const int qa = 7 - wave;            // A scale instruction handled by this wave
        L.nsa = qa < nsa_total ? 1 : 0;
        L.sa = G.sfa + (long)(row0 + min(32 * qa + (lane & 31), rows - 1)) * ss;
        L.sa_dst = A_CODES_AT + rpad * ROWB + 32 * qa * SCB;
        L.ops = 5 + L.na + L.nsa;
    }

    f16v_t acc[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
        acc[rb][0] = f16v_t{};
        acc[rb][1] = f16v_t{};
    }

    // prologue: supersteps 0 .. nslots-1 in flight; wait for superstep 0; dequantise A of
    // compute step 0
    const int first = min(nslots, supers);
    for (int t = 0; t < first; ++t) pk_issue(ring + t * sbytes, t, L, wave, lane);
    pk_wait_loads((first - 1) * L.ops);
    barrier_lds();
    pk_dequant_a<0>(ring, a16, rows, rpad, wave, lane);
    barrier_lds();

    int cs = 0;   // slot of superstep t
    for (int t = 0; t < supers; ++t) {
        // the slot of superstep t - 1 is free since the last barrier: refill it with
        // superstep t - 1 + nslots
        if (t > 0 && t - 1 + nslots < supers) {
            const int fs = (cs == 0) ? nslots - 1 : cs - 1;
            pk_issue(ring + fs * sbytes, t - 1 + nslots, L, wave, lane);
        }
        const int ns = (cs + 1 == nslots) ? 0 : cs + 1;
        const uint8_t* cur = ring + cs * sbytes;
        const uint8_t* nxt = ring + ns * sbytes;
        u4_t bs[2];
        pk_read_bs(bs, cur, wn, lane);
        const int s0 = SUB * t;
        pk_step<NRB, 0>(acc, cur, nxt, bs, a16, s0 + 0, steps, rows, rpad, wave, lane);
        barrier_lds();
        pk_step<NRB, 1>(acc, cur, nxt, bs, a16, s0 + 1, steps, rows, rpad, wave, lane);
        barrier_lds();
        pk_step<NRB, 2>(acc, cur, nxt, bs, a16, s0 + 2, steps, rows, rpad, wave, lane);
        // superstep t + 1 must have landed before the next step dequantises its A bytes
        {
            const int last = min(supers - 1, t - 1 + nslots);   // last superstep issued
            const int need = min(supers - 1, t + 1);
            pk_wait_loads((last - need) * L.ops);
        }
        barrier_lds();
        pk_step<NRB, 3>(acc, cur, nxt, bs, a16, s0 + 3, steps, rows, rpad, wave, lane);
        barrier_lds();
        cs = ns;
    }

    // pair reduction: wave x keeps column block x and hands block 1 - x to its partner
    const int colw = col0 + 64 * wn;
    u4_t* red = reinterpret_cast<u4_t*>(smem);
    uint16_t* c = G.c + (long)row0 * n;
    if (x == 0) {
        pk_pair_reduce<NRB, 1, 0>(acc, red, wn, x, lane);
        pk_store_cb<NRB, 0>(acc, c, n, rows, colw, lane);
    } else {
        pk_pair_reduce<NRB, 0, 1>(acc, red, wn, x, lane);
        pk_store_cb<NRB, 1>(acc, c, n, rows, colw, lane);
    }
    // the next tile's loads reuse the LDS just read
    barrier_lds();
}

// Persistent kernel: workgroup b processes tiles list[begin[b] .. begin[b+1]) in order.
__global__ __launch_bounds__(pk::THREADS) void nvfp4_gg_persistent(KernArgs args_byval)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[pk::LDS_BYTES];
    // index the group table in place in the kernarg segment (scalar loads), rather than
    // through the by-value copy
    (void)args_byval;
    const KernArgs& args = *(const KernArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    const int b = blockIdx.x;
    for (int i = args.wg_begin[b]; i < args.wg_begin[b + 1]; ++i) {
        // the tile is workgroup-uniform: keep it in scalar registers so that the group
        // table is read from the kernel arguments with scalar loads
        const TileDesc tv = args.tiles[i];
        const TileDesc t = {__builtin_amdgcn_readfirstlane(tv.group), __builtin_amdgcn_readfirstlane(tv.row0),
                            __builtin_amdgcn_readfirstlane(tv.rows), __builtin_amdgcn_readfirstlane(tv.col0)};
        const GroupArgs& G = args.grp[t.group];
        const int n = args.n, k = args.k;
        switch ((t.rows + 31) >> 5) {   // the planner keeps tiles within 1 .. RMAX rows
        case 1: pk_tile<1>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        case 2: pk_tile<2>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        case 3: pk_tile<3>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        case 4: pk_tile<4>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        default: break;
        }
    }
}

VariantShape variant_shape(int variant)
{
    switch (variant) {
    case kVariantPersistent:
        return VariantShape{pk::RMAX, pk::BN, pk::THREADS, pk::LDS_BYTES};
    default:
        return VariantShape{0, 0, 0, 0};
    }
}

hipError_t launch_variant(int variant, const KernArgs& args, int grid, hipStream_t stream)
{
    if (grid <= 0) return hipSuccess;
    switch (variant) {
    case kVariantPersistent: {
        KernArgs a = args;
        void* params[] = {&a};
        return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_persistent), dim3(grid), dim3(pk::THREADS),
                               params, 0, stream);
    }
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace nvfp4gg
