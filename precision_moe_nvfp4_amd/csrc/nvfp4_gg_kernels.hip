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
// list built by the host planner.  A tile is up to 96 rows of one group x 128 columns.
// Wave w owns the 64 columns 64 (w & 1) .. +64 and all tile rows, and one quarter of every
// K step (w >> 1); the four partial sums of a column half are added through LDS at the
// end.  So each dequantised B fragment feeds one MFMA per 32 tile rows, and each A
// fragment feeds two MFMAs:
//   * An LDS ring receives, per superstep of K = 256, the raw bytes of the superstep (B
//     rows, A rows and their scales) straight from HBM through direct-to-LDS loads (no
//     VGPR staging), one whole 128-byte line per row and load instruction; LDS holds
//     nothing else, so 5 to 7 slots fit and 3 to 5 supersteps stay in flight.
//   * Every wave reads the raw bytes of its own K quarter of both operands from the ring
//     and dequantises them in registers into MFMA fragments, one half superstep ahead of
//     their use, while the MFMAs of the current half run.
//   * One barrier per superstep both publishes the next superstep's slot and frees the
//     slot just consumed, which is refilled at once.
//   * v_mfma_f32_32x32x16_f16 takes the B fragment as its M-side operand, so each lane
//     ends up holding runs of 4 consecutive C columns (8-byte fp16 stores).
// K is permuted inside each half superstep, identically for A and B (the dot product is
// unchanged): lane half h, K quarter t and step u take the 8 K values starting at
// 64h + 16t + 8u, so that a lane's bytes of a whole half are 8 contiguous bytes.
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
constexpr int BN = 128;              // tile columns: wave w owns columns 64 (w & 1) .. +64
constexpr int RMAX = 96;             // tile rows (multiple of 32)

constexpr int SK = 256;              // K per load superstep
constexpr int ROWB = SK / 2;         // code bytes per row and superstep: one 128-byte line
constexpr int SCB = SK / 16;         // scale bytes per row and superstep
constexpr int MAX_SLOTS = 7;
constexpr int LDS_BYTES = 160 * 1024;
// LDS holds only the ring: ring_slots(rpad) slots of slot_bytes(rpad) for a tile with rpad
// rows, each holding the raw bytes of one superstep (all offsets multiples of 16 bytes):
//     B codes   128 rows x 128 B   at 0            (16-byte chunk c of row r at c ^ swz(r))
//     B scales  128 rows x 16 B    at B_SCALES_AT
//     A codes   rpad rows x 128 B  at A_CODES_AT   (same chunk swizzle)
//     A scales  rpad rows x 16 B   at A_CODES_AT + 128 rpad
// (5 slots of 96-row tiles, 5 of 64-row tiles, 7 of 32-row tiles).  Whole 128-byte lines
// per row and load instruction: a wave's 16-byte lanes cover 8 rows per instruction
// instead of 32, which is what lets a CU pull shared operand rows out of L2 at ~3x the
// rate of 32-byte row pieces.
// Chunk swizzle of the raw rows: the 3-bit reversal of (r >> 1) & 7, so that the 8-byte
// reads of one chunk half from 32 consecutive rows spread over 16 chunk positions.
__host__ __device__ constexpr int swz(int r)
{
    return (((r >> 1) & 1) << 2) | ((r >> 1) & 2) | ((r >> 3) & 1);
}
constexpr int B_SCALES_AT = BN * ROWB;                // 16384
constexpr int A_CODES_AT = B_SCALES_AT + BN * SCB;    // 18432
__host__ __device__ constexpr int slot_bytes(int rpad) { return A_CODES_AT + rpad * (ROWB + SCB); }
__host__ __device__ constexpr int ring_slots(int rpad)
{
    return LDS_BYTES / slot_bytes(rpad) > MAX_SLOTS ? MAX_SLOTS : LDS_BYTES / slot_bytes(rpad);
}
// reduction area (overlays the ring after the last superstep): per wave, for each column
// block and 32-row block, the three element groups handed to the other K quarters (one u4
// per lane each)
constexpr int RED_WAVE = 2 * (RMAX / 32) * 3 * 64 * 16;
// staged output rows of the epilogue (fp16, 128 columns, padded to spread banks)
constexpr int STAGE_ROW = BN * 2 + 16;
static_assert(RMAX * STAGE_ROW <= LDS_BYTES, "staged output tile must fit in LDS");
static_assert(ring_slots(RMAX) >= 3, "the tallest tile needs at least 3 ring slots");
static_assert(8 * RED_WAVE <= LDS_BYTES, "reduction area must fit in LDS");
}  // namespace pk

// ---------------------------------------------------------------------------------------
// Loads
// ---------------------------------------------------------------------------------------

// How the scales are fetched (see SuperLoads).
enum ScaleMode : int {
    SCL_ROW16 = 0,    // row-major scales, 16 bytes per lane (k % 256 == 0: 16-byte rows)
    SCL_BLOCKED = 1,  // 128x4 blocked scales, 4 bytes per lane
    SCL_ROW4 = 2,     // row-major scales, 4 bytes per lane (rows only 4-byte aligned)
};

// Per-wave direct-to-LDS loads of one superstep.  B code instruction i (rows 8i .. +8,
// i < 16) goes to wave i % 8 and A code instruction a (rows 8a .. +8) to wave (a + 4) % 8.
// Scales, SCL_ROW16: B scale instruction q (rows 32q .. +32, 16 bytes per lane, lanes < 32)
// to wave q < 4, A scale instruction q to wave 7 - q.  Scales, SCL_BLOCKED and SCL_ROW4:
// 4 bytes per lane, so instruction q covers rows 16q .. +16 (lane l: row 16q + l / 4,
// scale dword l % 4 of the superstep); B scale instruction q to wave q (all 8), A scale
// instruction q to wave q.  Either way the LDS copy of a superstep's scales is the same:
// row r's 16 bytes at 16 r.  In a last superstep that holds fewer than 256 K values, lanes
// whose code chunk or scale dword lies beyond K store zeros to their LDS place instead of
// loading (zero codes and zero scales contribute exact zeros); every instruction keeps at
// least one loading lane, so the per-superstep load count is unchanged.
// Source addresses are a workgroup-uniform base (first row of the tile, superstep 0) plus a
// 32-bit per-lane offset, so that the loads address memory as scalar base + vector offset
// and the per-superstep advance is a scalar add.
struct SuperLoads {
    const uint8_t* bb;    // B codes: uniform base
    const uint8_t* sbb;   // B scales: uniform base
    const uint8_t* ab;    // A codes: uniform base
    const uint8_t* sab;   // A scales: uniform base
    __amdgpu_buffer_rsrc_t rb, rsb, ra, rsa;   // buffer resources of the four bases
    uint32_t b[2];        // this lane's offsets from the bases
    uint32_t sb;
    uint32_t a[2];
    uint32_t sa;
    int b_dst[2];         // LDS offsets (inside a slot) of the B code instructions
    int sb_dst;
    int a_dst[2];
    int sa_dst;
    int nsb;              // B scale instructions of this wave (0 or 1)
    int na;               // A code instructions of this wave (0 .. 2)
    int nsa;              // A scale instructions of this wave (0 or 1)
    int ops;              // loads per superstep issued by this wave
    int b_chunk[2];       // global 16-byte chunk (0 .. 7) of a row that this lane loads
    int a_chunk[2];
    int s_dword;          // scale dword (0 .. 3) of the superstep this lane loads (4-byte modes)
    long sstride;         // scale bytes between consecutive supersteps of this lane
};

// Loads per superstep issued by wave w for tiles of 32 nrb rows (the assignment above).
__host__ __device__ constexpr int pk_ops(int w, int nrb, bool blocked)   // blocked: 4-byte scale loads
{
    int ops = 2;                                            // B codes: instructions w, w + 8
    ops += blocked ? 1 : (w < 4 ? 1 : 0);                   // B scales
    for (int q = 0; q < 2; ++q) ops += ((w + 4) & 7) + 8 * q < 4 * nrb ? 1 : 0;   // A codes
    ops += blocked ? (w < 2 * nrb ? 1 : 0) : (7 - w < nrb ? 1 : 0);             // A scales
    return ops;
}
__host__ __device__ constexpr int pk_ops_min(int nrb, bool blocked)
{
    int v = pk_ops(0, nrb, blocked);
    for (int w = 1; w < 8; ++w) v = pk_ops(w, nrb, blocked) < v ? pk_ops(w, nrb, blocked) : v;
    return v;
}
__host__ __device__ constexpr int pk_ops_max(int nrb, bool blocked)
{
    int v = pk_ops(0, nrb, blocked);
    for (int w = 1; w < 8; ++w) v = pk_ops(w, nrb, blocked) > v ? pk_ops(w, nrb, blocked) : v;
    return v;
}

// Raw buffer resource over [base, base + 2^31): loads address it as scalar base + 32-bit
// vector offset + scalar offset, so the per-lane part needs no 64-bit address arithmetic
// and the per-superstep advance rides in the scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pk_rsrc(const uint8_t* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Direct-to-LDS buffer loads of 16 / 4 bytes per lane at voff + soff into lds_base + 16 (4)
// times the lane index.
__device__ __forceinline__ void pk_bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voff, soff,
                                             0, 0);
}
__device__ __forceinline__ void pk_bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds_base)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, (int)voff, soff,
                                             0, 0);
}

// 16 code bytes of this lane, or zeros when its chunk lies beyond the superstep's K.
__device__ __forceinline__ void pk_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds_base,
                                          int lane, bool valid)
{
    if (valid) {
        pk_bload16(r, voff, soff, lds_base);
    } else {
        *reinterpret_cast<u4_t*>(lds_base + 16 * lane) = u4_t{0u, 0u, 0u, 0u};
    }
}

// Issue the loads of superstep t (kt = K values it holds, 256 except maybe in the last).
template <int SCL>
__device__ __forceinline__ void pk_issue(uint8_t* slot_base, int t, int kt, const SuperLoads& L, int lane)
{
    using namespace pk;
    const int kb = t * ROWB;                      // scalar offsets of superstep t
    const int ks = t * (int)L.sstride;
    if (SCL == SCL_ROW16 || kt == SK) {   // (SCL_ROW16 plans have no short supersteps)
        pk_bload16(L.rb, L.b[0], kb, slot_base + L.b_dst[0]);
        pk_bload16(L.rb, L.b[1], kb, slot_base + L.b_dst[1]);
        if constexpr (SCL == SCL_ROW16) {
            if (L.nsb > 0 && lane < 32) pk_bload16(L.rsb, L.sb, ks, slot_base + L.sb_dst);
            if (L.nsa > 0 && lane < 32) pk_bload16(L.rsa, L.sa, ks, slot_base + L.sa_dst);
        } else {
            if (L.nsb > 0) pk_bload4(L.rsb, L.sb, ks, slot_base + L.sb_dst);
            if (L.nsa > 0) pk_bload4(L.rsa, L.sa, ks, slot_base + L.sa_dst);
        }
        if (L.na > 0) pk_bload16(L.ra, L.a[0], kb, slot_base + L.a_dst[0]);
        if (L.na > 1) pk_bload16(L.ra, L.a[1], kb, slot_base + L.a_dst[1]);
    } else {
        // a short last superstep: kt / 32 code chunks and kt / 64 scale dwords per row
        const int vchunks = kt >> 5, vdw = kt >> 6;
        pk_load16(L.rb, L.b[0], kb, slot_base + L.b_dst[0], lane, L.b_chunk[0] < vchunks);
        pk_load16(L.rb, L.b[1], kb, slot_base + L.b_dst[1], lane, L.b_chunk[1] < vchunks);
        if constexpr (SCL != SCL_ROW16) {
            const bool sv = L.s_dword < vdw;
            if (L.nsb > 0) {
                if (sv) pk_bload4(L.rsb, L.sb, ks, slot_base + L.sb_dst);
                else *reinterpret_cast<uint32_t*>(slot_base + L.sb_dst + 4 * lane) = 0u;
            }
            if (L.nsa > 0) {
                if (sv) pk_bload4(L.rsa, L.sa, ks, slot_base + L.sa_dst);
                else *reinterpret_cast<uint32_t*>(slot_base + L.sa_dst + 4 * lane) = 0u;
            }
        }
        if (L.na > 0) pk_load16(L.ra, L.a[0], kb, slot_base + L.a_dst[0], lane, L.a_chunk[0] < vchunks);
        if (L.na > 1) pk_load16(L.ra, L.a[1], kb, slot_base + L.a_dst[1], lane, L.a_chunk[1] < vchunks);
    }
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

// ---------------------------------------------------------------------------------------
// Scales
// ---------------------------------------------------------------------------------------

// fp16 scale pair (column block 0, column block 1) of half HALF: byte 8 HALF + 4h + t of
// each row's scale bytes, i.e. byte t of the lane's word for that half.
template <int HALF>
__device__ __forceinline__ h2_t pk_scales(const u2_t (&srow)[2], uint32_t tsel)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(srow[1][HALF], srow[0][HALF], tsel), 1.0f,
                                                    false);
}

// ---------------------------------------------------------------------------------------
// Compute
// ---------------------------------------------------------------------------------------

// MFMAs of one step: B fragments of the two column blocks, A fragments of the row blocks.
template <int NRB>
__device__ __forceinline__ void pk_mfmas(f16v_t (&acc)[2][NRB], const h8_t (&bf)[2], const h8_t (&af)[NRB])
{
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
            acc[c][rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[c], af[rb], acc[c][rb], 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// Epilogue
// ---------------------------------------------------------------------------------------

// Reduction over the four K quarters and store.  Lane (j, h) holds, in acc[c][rb] element
// 4q + e, the partial sum of C[32 rb + j][64 cw + 32 c + 8 q + 4 h + e].  The wave with K
// quarter T keeps element group q = T and hands the other three to the waves that keep
// them (same column half) through LDS.  T is a template parameter so that every element
// and LDS slot index is static (no register indexing, no per-partner branches) and all
// partner reads are in flight together.
template <int NRB, int T>
__device__ __forceinline__ void pk_reduce_store_q(const f16v_t (&acc)[2][NRB], uint8_t* smem,
                                                  uint16_t* __restrict__ c0, int n, int ldc, int rows, int col, int wave,
                                                  int lane)
{
    using namespace pk;
    const int cw = wave & 1;
    u4_t* mine = reinterpret_cast<u4_t*>(smem + wave * RED_WAVE);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q == T) continue;
                const int slot = q - (q > T ? 1 : 0);
                mine[((c * NRB + rb) * 3 + slot) * 64 + lane] =
                    u4_t{__float_as_uint(acc[c][rb][4 * q + 0]), __float_as_uint(acc[c][rb][4 * q + 1]),
                         __float_as_uint(acc[c][rb][4 * q + 2]), __float_as_uint(acc[c][rb][4 * q + 3])};
            }
    barrier_lds();
    u4_t o[2][NRB][3];   // group T of the three partner waves
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
            for (int p = 0, i = 0; p < 4; ++p) {
                if (p == T) continue;
                const int slot = T - (T > p ? 1 : 0);   // where partner p put group T
                o[c][rb][i++] = reinterpret_cast<const u4_t*>(smem + (cw + 2 * p) * RED_WAVE)[((c * NRB + rb) * 3 + slot) * 64 + lane];
            }
    const int j = lane & 31, h = lane >> 5;
    // all 128 columns in bounds and 16-byte aligned rows (one uniform test): the reduced fp16
    // tile is staged in LDS as rows and leaves in whole 128-byte lines, 16 bytes per lane,
    // with the non-temporal hint (C is written once and not read again here); otherwise
    // each lane stores its own 4 columns (8 bytes, or element-wise at the edge)
    const bool staged = (ldc & 7) == 0 && col + BN <= n;
    const bool full = (ldc & 3) == 0 && col + BN <= n;
    if (staged) barrier_lds();   // the staged rows overwrite the exchange area: all reads done
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // (element-wise __uint_as_float: __builtin_bit_cast of an ext-vector element
                // reads element 0 with this compiler)
                v[e] = acc[c][rb][4 * T + e] + __uint_as_float(o[c][rb][0][e]) + __uint_as_float(o[c][rb][1][e]) +
                       __uint_as_float(o[c][rb][2][e]);
            }
            const int r = rb * 32 + j;
            const uint16_t h0 = f16_bits_rne(v[0]), h1 = f16_bits_rne(v[1]);
            const uint16_t h2 = f16_bits_rne(v[2]), h3 = f16_bits_rne(v[3]);
            const int tc = 64 * cw + 32 * c + 8 * T + 4 * h;   // column inside the tile
            if (staged) {
                *reinterpret_cast<u2_t*>(smem + r * STAGE_ROW + 2 * tc) =
                    u2_t{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
                continue;
            }
            if (r >= rows) continue;
            uint16_t* crow = c0 + (long)r * ldc;
            const int cc = col + tc;
            if (full) {
                *reinterpret_cast<u2_t*>(crow + cc) =
                    u2_t{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
            } else {
                if (cc + 0 < n) crow[cc + 0] = h0;
                if (cc + 1 < n) crow[cc + 1] = h1;
                if (cc + 2 < n) crow[cc + 2] = h2;
                if (cc + 3 < n) crow[cc + 3] = h3;
            }
        }
    if (staged) {
        barrier_lds();
        // 16 lanes per 256-byte tile row, 32 rows per pass of the 512 threads
        const int tid = threadIdx.x, chunk = tid & 15;
        for (int r = tid >> 4; r < rows; r += THREADS / 16) {
            const u4_t val = *reinterpret_cast<const u4_t*>(smem + r * STAGE_ROW + 16 * chunk);
            __builtin_nontemporal_store(val, reinterpret_cast<u4_t*>(c0 + (long)r * ldc + col + 8 * chunk));
        }
    }
}

template <int NRB>
__device__ __forceinline__ void pk_reduce_store(const f16v_t (&acc)[2][NRB], uint8_t* smem, uint16_t* __restrict__ c0,
                                                int n, int ldc, int rows, int col, int wave, int lane)
{
    switch (wave >> 1) {   // the wave's K quarter (wave-uniform)
    case 0: pk_reduce_store_q<NRB, 0>(acc, smem, c0, n, ldc, rows, col, wave, lane); break;
    case 1: pk_reduce_store_q<NRB, 1>(acc, smem, c0, n, ldc, rows, col, wave, lane); break;
    case 2: pk_reduce_store_q<NRB, 2>(acc, smem, c0, n, ldc, rows, col, wave, lane); break;
    default: pk_reduce_store_q<NRB, 3>(acc, smem, c0, n, ldc, rows, col, wave, lane); break;
    }
}

// ---------------------------------------------------------------------------------------
// Tile
// ---------------------------------------------------------------------------------------

// This wave's loads of a tile (see SuperLoads): lane l of a code instruction covers row
// (first row + l / 8) and stores LDS chunk l % 8, which holds global chunk (l % 8) ^ swz(row).
template <int SCL>
__device__ __forceinline__ SuperLoads pk_super_loads(const GroupArgs& G, int n, int k, int row0, int rows, int col0,
                                                     int rpad, int wave, int lane)
{
    using namespace pk;
    const long qs = k / 2, ss = k / 16;
    SuperLoads L;
    const int rl = lane >> 3, pos = lane & 7;
    L.bb = G.b + (long)col0 * qs;
    L.ab = G.a + (long)row0 * qs;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i = wave + 8 * q;   // B code instruction
        const int r = 8 * i + rl;
        L.b[q] = (uint32_t)((long)(min(col0 + r, n - 1) - col0) * qs + 16 * (pos ^ swz(r)));
        L.b_dst[q] = 8 * i * ROWB;
        L.b_chunk[q] = pos ^ swz(r);
    }
    const int na_total = rpad / 8;
    L.na = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int a = ((wave + 4) & 7) + 8 * q;   // A code instruction
        const int r = 8 * a + rl;
        L.a[q] = (uint32_t)((long)min(r, rows - 1) * qs + 16 * (pos ^ swz(r)));
        L.a_dst[q] = A_CODES_AT + 8 * a * ROWB;
        L.a_chunk[q] = pos ^ swz(r);
        if (a < na_total) L.na = q + 1;
    }
    L.s_dword = lane & 3;
    if constexpr (SCL == SCL_BLOCKED) {
        // 128x4 blocked scales: the scale of (row r, K block c) sits in 512-byte atom
        // (r / 128) * (k / 64) + c / 4 at byte 16 (r % 32) + 4 ((r / 32) % 4) + c % 4, so
        // the 4 scales of a row in one atom are contiguous.  Lane l of scale instruction
        // q = wave loads the 4 bytes of row 16 q + l / 4 in the superstep's atom l % 4
        // (K blocks 16 t + 4 (l % 4) .. +4), which land at LDS byte 16 (row) + 4 (l % 4).
        // (bases: the tile's first 128-row block; col0 is a multiple of 128, so all B rows
        // of the tile sit in that block, A rows in it or the next)
        const long atoms = k / 64;
        const int piece = lane & 3;
        const int gb = min(col0 + 16 * wave + (lane >> 2), n - 1);
        L.sbb = G.sfb + (long)(col0 >> 7) * atoms * 512;
        L.nsb = 1;
        L.sb = (uint32_t)((((long)(gb >> 7) - (col0 >> 7)) * atoms + piece) * 512 + 16 * (gb & 31) +
                          4 * ((gb >> 5) & 3));
        L.sb_dst = B_SCALES_AT + 16 * wave * SCB;
        const int ga = row0 + min(16 * wave + (lane >> 2), rows - 1);
        L.sab = G.sfa + (long)(row0 >> 7) * atoms * 512;
        L.nsa = wave < rpad / 16 ? 1 : 0;
        L.sa = (uint32_t)((((long)(ga >> 7) - (row0 >> 7)) * atoms + piece) * 512 + 16 * (ga & 31) +
                          4 * ((ga >> 5) & 3));
        L.sa_dst = A_CODES_AT + rpad * ROWB + 16 * wave * SCB;
        L.sstride = 4 * 512;             // four atoms per superstep
    } else if constexpr (SCL == SCL_ROW4) {
        // row-major scales, lane l of scale instruction q = wave: dword l % 4 of the
        // superstep's 16 scale bytes of row 16 q + l / 4
        const int gb = min(col0 + 16 * wave + (lane >> 2), n - 1);
        L.sbb = G.sfb + (long)col0 * ss;
        L.nsb = 1;
        L.sb = (uint32_t)((long)(gb - col0) * ss + 4 * (lane & 3));
        L.sb_dst = B_SCALES_AT + 16 * wave * SCB;
        const int ga = min(16 * wave + (lane >> 2), rows - 1);
        L.sab = G.sfa + (long)row0 * ss;
        L.nsa = wave < rpad / 16 ? 1 : 0;
        L.sa = (uint32_t)((long)ga * ss + 4 * (lane & 3));
        L.sa_dst = A_CODES_AT + rpad * ROWB + 16 * wave * SCB;
        L.sstride = SCB;
    } else {
        L.sstride = SCB;
        L.sbb = G.sfb + (long)col0 * ss;
        L.sab = G.sfa + (long)row0 * ss;
        L.nsb = wave < 4 ? 1 : 0;        // B scale instruction q = wave
        L.sb = (uint32_t)((long)(min(col0 + 32 * (wave & 3) + (lane & 31), n - 1) - col0) * ss);
        L.sb_dst = B_SCALES_AT + 32 * (wave & 3) * SCB;
        const int qa = 7 - wave;         // A scale instruction
        L.nsa = qa < rpad / 32 ? 1 : 0;
        L.sa = (uint32_t)((long)min(32 * qa + (lane & 31), rows - 1) * ss);
        L.sa_dst = A_CODES_AT + rpad * ROWB + 32 * qa * SCB;
    }
    L.ops = 2 + L.nsb + L.na + L.nsa;
    L.rb = pk_rsrc(L.bb);
    L.ra = pk_rsrc(L.ab);
    L.rsb = pk_rsrc(L.sbb);
    L.rsa = pk_rsrc(L.sab);
    return L;
}

// ---------------------------------------------------------------------------------------
// Tile
// ---------------------------------------------------------------------------------------
//
// Every wave reads the raw A bytes of its own K quarter for all tile rows straight from the
// ring slot, exactly as it reads its B bytes, and dequantises both into MFMA fragments in
// registers.  The two column halves thus both convert the A rows (a shared fp16 A buffer in
// LDS would convert them once), which measured cheaper than that buffer's LDS writes,
// fragment reads and second barrier per superstep; the LDS it would take holds more ring
// slots instead.

// This lane's LDS byte offsets inside a ring slot: raw codes of half 0 / 1 (column block
// cb0, row block 0) and the scale words, for B and A.  Both operands use the same lane
// mapping (lane (j, h), K quarter tq: row j of a 32-row block, chunk 4 half + 2h + tq / 2,
// bytes 8 (tq % 2) .. +8), and rows 32 apart share the chunk swizzle.
struct LdsOffs {
    int ob[2];
    int oa[2];
    int obs;
    int osa;
};

template <int NRB>
__device__ __forceinline__ LdsOffs pk_lds_offsets(int lane, int cw, int tq)
{
    using namespace pk;
    const int j = lane & 31, h = lane >> 5;
    const int brow = 64 * cw + j;
    LdsOffs o;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int chunk = 4 * half + 2 * h + (tq >> 1);
        o.ob[half] = brow * ROWB + 16 * (chunk ^ swz(brow)) + 8 * (tq & 1);
        o.oa[half] = A_CODES_AT + j * ROWB + 16 * (chunk ^ swz(j)) + 8 * (tq & 1);
    }
    o.obs = B_SCALES_AT + brow * SCB + 4 * h;
    o.osa = A_CODES_AT + 32 * NRB * ROWB + j * SCB + 4 * h;
    return o;
}

// Raw bytes of half HALF: 8 code bytes (steps u = 0, 1 in dwords x, y) of B column block c
// or A row block rb.
template <int HALF>
__device__ __forceinline__ u2_t pk_rd_b(const uint8_t* slot, int c, const LdsOffs& o)
{
    return *reinterpret_cast<const u2_t*>(slot + o.ob[HALF] + 32 * pk::ROWB * c);
}
template <int HALF>
__device__ __forceinline__ u2_t pk_rd_a(const uint8_t* slot, int rb, const LdsOffs& o)
{
    return *reinterpret_cast<const u2_t*>(slot + o.oa[HALF] + 32 * pk::ROWB * rb);
}
// The two scale words of a row that the lane needs in a superstep: words h (half 0) and
// 2 + h (half 1) of the row's 16 scale bytes; byte tq of a word is the lane's scale.
__device__ __forceinline__ u2_t pk_rd_s(const uint8_t* slot, int off)
{
    const uint32_t* w = reinterpret_cast<const uint32_t*>(slot + off);
    return u2_t{w[0], w[2]};
}

// Dequantise the raw bytes of half HALF into the MFMA fragments bf[u][c] and af[u][rb].
template <int NRB, int HALF>
__device__ __forceinline__ void pk_dequant(h8_t (&bf)[2][2], h8_t (&af)[2][NRB], const u2_t (&qb)[2],
                                             const u2_t (&qa)[NRB], const u2_t (&srow)[2], const u2_t (&arow)[NRB],
                                             uint32_t tsel)
{
    const h2_t sc = pk_scales<HALF>(srow, tsel);
    const h2_t s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
    bf[0][0] = __builtin_bit_cast(h8_t, dequant8(qb[0].x, s0));
    bf[1][0] = __builtin_bit_cast(h8_t, dequant8(qb[0].y, s0));
    bf[0][1] = __builtin_bit_cast(h8_t, dequant8(qb[1].x, s1));
    bf[1][1] = __builtin_bit_cast(h8_t, dequant8(qb[1].y, s1));
#pragma unroll
    for (int rb = 0; rb < NRB; rb += 2) {
        const int r1 = rb + 1 < NRB ? rb + 1 : rb;
        const h2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(arow[r1][HALF], arow[rb][HALF], tsel),
                                                                 1.0f, false);
        const h2_t a0 = {sa.x, sa.x};
        af[0][rb] = __builtin_bit_cast(h8_t, dequant8(qa[rb].x, a0));
        af[1][rb] = __builtin_bit_cast(h8_t, dequant8(qa[rb].y, a0));
        if (rb + 1 < NRB) {
            const h2_t a1 = {sa.y, sa.y};
            af[0][rb + 1] = __builtin_bit_cast(h8_t, dequant8(qa[rb + 1].x, a1));
            af[1][rb + 1] = __builtin_bit_cast(h8_t, dequant8(qa[rb + 1].y, a1));
        }
    }
}

// Raw operand bytes of one half superstep in registers: B code bytes of the two column
// blocks, A code bytes of the row blocks.  Scale words of one superstep: B column blocks,
// A row blocks.
template <int NRB>
struct RawHalf {
    u2_t b[2];
    u2_t a[NRB];
};
template <int NRB>
struct ScaleWords {
    u2_t b[2];
    u2_t a[NRB];
};

template <int NRB, int HALF>
__device__ __forceinline__ void pk_read_raw(RawHalf<NRB>& q, const uint8_t* slot, const LdsOffs& o)
{
#pragma unroll
    for (int c = 0; c < 2; ++c) q.b[c] = pk_rd_b<HALF>(slot, c, o);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) q.a[rb] = pk_rd_a<HALF>(slot, rb, o);
}

template <int NRB>
__device__ __forceinline__ void pk_read_scales(ScaleWords<NRB>& s, const uint8_t* slot, const LdsOffs& o)
{
#pragma unroll
    for (int c = 0; c < 2; ++c) s.b[c] = pk_rd_s(slot, o.obs + 32 * pk::SCB * c);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) s.a[rb] = pk_rd_s(slot, o.osa + 32 * pk::SCB * rb);
}

// One half superstep.  The MFMAs consume the fragments bf, af (converted during the
// previous half); meanwhile the raw bytes q of the next half (read from LDS during the
// previous half, so their reads have had a whole half to land) are converted into bf, af,
// and the raw bytes of the half after that are read from `nxt` (the next superstep's slot)
// into q.  HALF = 0: the next half is half 1 of this superstep (scales s); the half after
// is half 0 of the next superstep, whose scale words are read too and replace s once this
// half's conversions are done.  HALF = 1: the next half is half 0 of the next superstep;
// the half after is its half 1.
template <int NRB, int HALF>
__device__ __forceinline__ void pk_half(f16v_t (&acc)[2][NRB], h8_t (&bf)[2][2], h8_t (&af)[2][NRB], RawHalf<NRB>& q,
                                        ScaleWords<NRB>& s, const uint8_t* nxt, const LdsOffs& o, uint32_t tsel)
{
    RawHalf<NRB> qn;
    ScaleWords<NRB> sn;
    if constexpr (HALF == 0) {
        pk_read_scales<NRB>(sn, nxt, o);
        pk_read_raw<NRB, 0>(qn, nxt, o);
    } else {
        pk_read_raw<NRB, 1>(qn, nxt, o);
    }
    pk_mfmas<NRB>(acc, bf[0], af[0]);
    pk_mfmas<NRB>(acc, bf[1], af[1]);
    pk_dequant<NRB, 1 - HALF>(bf, af, q.b, q.a, s.b, s.a, tsel);
    q = qn;
    if constexpr (HALF == 0) s = sn;
}

// The steady-state load wait of the ring above: AHEAD = slots - 2 supersteps stay in flight.
template <int NRB, int SCL>
__device__ __forceinline__ void pk_wait_steady(int n)
{
    constexpr bool B4 = SCL != SCL_ROW16;
    constexpr int AHEAD = pk::ring_slots(32 * NRB) - 2;
    constexpr int LO = AHEAD * pk_ops_min(NRB, B4), HI = AHEAD * pk_ops_max(NRB, B4);
    static_assert(HI <= 63, "vmcnt has 6 bits");
    // s_waitcnt: vmcnt bits 3..0 and 15..14; expcnt (6..4) and lgkmcnt (11..8) not waited for
    constexpr int EHI = 0x0f70 | (HI & 15) | ((HI >> 4) << 14);
    constexpr int ELO = 0x0f70 | (LO & 15) | ((LO >> 4) << 14);
    if (n == HI) {
        __builtin_amdgcn_s_waitcnt(EHI);
    } else if (n == LO) {
        __builtin_amdgcn_s_waitcnt(ELO);
    } else {
        pk_wait_loads(n);
    }
}

// One full-K tile (rows [row0, row0 + rows) of group G, columns [col0, col0 + 128)), K a
// multiple of 64 (the last superstep holds k - 256 (supers - 1) K values).  All 8 waves
// execute the same sequence of loads and barriers; NRB = rpad / 32 sets the MFMAs per B
// fragment; SCL is how the scales are fetched (ScaleMode).  Raw bytes are read from LDS two
// halves before their MFMAs and converted one half before.  At the start of superstep t the
// wave waits for its own loads of superstep t + 1, and the barrier both publishes
// superstep t + 1 (read during superstep t) and frees slot t (already read during
// superstep t - 1), which is refilled at once with superstep t + slots.
template <int NRB, int SCL>
__device__ __forceinline__ void pk_tile(const GroupArgs& G, int n_, int k_, int row0_, int rows_, int col0_,
                                        uint8_t* smem)
{
    using namespace pk;
    const int n = __builtin_amdgcn_readfirstlane(n_), k = __builtin_amdgcn_readfirstlane(k_);
    const int row0 = __builtin_amdgcn_readfirstlane(row0_), rows = __builtin_amdgcn_readfirstlane(rows_);
    const int col0 = __builtin_amdgcn_readfirstlane(col0_);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = wave & 1, tq = wave >> 1;
    const int rpad = 32 * NRB;
    const int supers = (k + SK - 1) / SK;
    const int klast = k - SK * (supers - 1);
    const int sbytes = slot_bytes(rpad), nslots = ring_slots(rpad);
    uint8_t* ring = smem;
    const SuperLoads L = pk_super_loads<SCL>(G, n, k, row0, rows, col0, rpad, wave, lane);

    f16v_t acc[2][NRB];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) acc[c][rb] = f16v_t{};

    // prologue: superstep 0 on its own, then supersteps 1 .. slots-1; convert half 0 of
    // superstep 0
    const int first = min(nslots, supers);
    const auto kt_of = [&](int t) { return t == supers - 1 ? klast : SK; };
    pk_issue<SCL>(ring, 0, kt_of(0), L, lane);
    pk_wait_loads(0);
    for (int t = 1; t < first; ++t) pk_issue<SCL>(ring + t * sbytes, t, kt_of(t), L, lane);
    barrier_lds();
    const uint32_t tsel = 0x0c0c0000u | ((uint32_t)(4 + tq) << 8) | (uint32_t)tq;
    const LdsOffs lo = pk_lds_offsets<NRB>(lane, cw, tq);
    // fragments of half 0 of superstep 0, raw bytes of its half 1 and its scale words
    h8_t bf[2][2], af[2][NRB];
    RawHalf<NRB> q;
    ScaleWords<NRB> sw;
    {
        RawHalf<NRB> q0;
        pk_read_scales<NRB>(sw, ring, lo);
        pk_read_raw<NRB, 0>(q0, ring, lo);
        pk_read_raw<NRB, 1>(q, ring, lo);
        pk_dequant<NRB, 0>(bf, af, q0.b, q0.a, sw.b, sw.a, tsel);
    }

    const int wait_steady = (nslots - 2) * L.ops;
    int cs = 0;   // slot of superstep t
    for (int t = 0; t < supers; ++t) {
        // superstep t + 1 must have landed (this wave's loads; loads complete in issue
        // order, so later supersteps stay in flight) before the barrier publishes it; the
        // barrier also frees slot t, whose bytes are all in registers by now: refill it
        if (t + nslots - 1 < supers) {
            pk_wait_steady<NRB, SCL>(wait_steady);   // supersteps t + 2 .. t + slots - 1 in flight
        } else if (t + 1 < supers) {
            pk_wait_loads((supers - 2 - t) * L.ops);
        }
        barrier_lds();
        if (t + nslots < supers) pk_issue<SCL>(ring + cs * sbytes, t + nslots, kt_of(t + nslots), L, lane);
        const int ns = (cs + 1 == nslots) ? 0 : cs + 1;
        // in the last superstep the reads of the "next" slot land on bytes that are no
        // superstep's: harmless, and their results are unused
        const uint8_t* nxt = ring + ns * sbytes;
        pk_half<NRB, 0>(acc, bf, af, q, sw, nxt, lo, tsel);
        pk_half<NRB, 1>(acc, bf, af, q, sw, nxt, lo, tsel);
        cs = ns;
    }
    // every ring read has completed and every load has landed before the reduction area
    // overwrites the ring
    barrier_lds();
    const int ldc = __builtin_amdgcn_readfirstlane(G.ldc);
    pk_reduce_store<NRB>(acc, smem, G.c + (long)row0 * ldc, n, ldc, rows, col0, wave, lane);
    barrier_lds();
}

// Persistent kernel body: workgroup b processes its first tile tiles[b], then tiles
// list[begin[b] .. begin[b+1]) in order.
template <int SCL>
__device__ __forceinline__ void pk_persistent(uint8_t* smem)
{
    // index the group table in place in the kernarg segment (scalar loads), rather than
    // through the by-value copy
    const KernArgs& args = *(const KernArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    const int b = blockIdx.x;
    // the first tile sits at tiles[b], so its fetch does not wait for the range fetch; the
    // range is read once (the C stores could alias it as far as the compiler knows)
    const int i_begin = args.wg_begin[b], i_end = args.wg_begin[b + 1];
    int idx = b, next = i_begin;
    while (true) {
        // the tile is workgroup-uniform: keep it in scalar registers so that the group
        // table is read from the kernel arguments with scalar loads
        const TileDesc tv = args.tiles[idx];
        const TileDesc t = {__builtin_amdgcn_readfirstlane(tv.group), __builtin_amdgcn_readfirstlane(tv.row0),
                            __builtin_amdgcn_readfirstlane(tv.rows), __builtin_amdgcn_readfirstlane(tv.col0)};
        const GroupArgs& G = args.grp[t.group];
        const int n = G.n, k = G.k;
        switch ((t.rows + 31) >> 5) {   // the planner keeps tiles within 0 .. RMAX rows
        case 1: pk_tile<1, SCL>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        case 2: pk_tile<2, SCL>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        case 3: pk_tile<3, SCL>(G, n, k, t.row0, t.rows, t.col0, smem); break;
        default: break;
        }
        if (next >= i_end) break;
        idx = next++;
    }
}

// Row-major scales ([rows][k/16]), every k a multiple of 256.
__global__ __launch_bounds__(pk::THREADS) void nvfp4_gg_persistent(KernArgs args_byval)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[pk::LDS_BYTES];
    (void)args_byval;
    pk_persistent<SCL_ROW16>(smem);
}

// 128x4 blocked scales (512-byte atoms), k a multiple of 64.
__global__ __launch_bounds__(pk::THREADS) void nvfp4_gg_persistent_blocked(KernArgs args_byval)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[pk::LDS_BYTES];
    (void)args_byval;
    pk_persistent<SCL_BLOCKED>(smem);
}

// Row-major scales with some k not a multiple of 256 (scale rows only 4-byte aligned).
__global__ __launch_bounds__(pk::THREADS) void nvfp4_gg_persistent_ktail(KernArgs args_byval)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[pk::LDS_BYTES];
    (void)args_byval;
    pk_persistent<SCL_ROW4>(smem);
}

VariantShape variant_shape(int variant)
{
    switch (variant) {
    case kVariantPersistent:
    case kVariantPersistentBlocked:
    case kVariantPersistentKTail:
        return VariantShape{pk::RMAX, pk::BN, pk::THREADS, pk::LDS_BYTES};
    default:
        return VariantShape{0, 0, 0, 0};
    }
}

hipError_t launch_variant(int variant, const KernArgs& args, int grid, hipStream_t stream)
{
    if (grid <= 0) return hipSuccess;
    KernArgs a = args;
    void* params[] = {&a};
    switch (variant) {
    case kVariantPersistent:
        return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_persistent), dim3(grid), dim3(pk::THREADS),
                               params, 0, stream);
    case kVariantPersistentBlocked:
        return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_persistent_blocked), dim3(grid),
                               dim3(pk::THREADS), params, 0, stream);
    case kVariantPersistentKTail:
        return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_persistent_ktail), dim3(grid),
                               dim3(pk::THREADS), params, 0, stream);
    default:
        return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------------------
// Scale layout conversion
// ---------------------------------------------------------------------------------------

// Row-major scales [rows][k/16] -> 128x4 blocked layout.  One thread per output dword:
// dword w of atom a holds the 4 scales of row 128 (a / (k/64)) + 32 (w % 4) + w / 4 in
// K blocks 4 (a % (k/64)) .. +4, which are one aligned dword of that source row.  Rows
// at or beyond `rows` (the padding of the last 128-row block) are written as zero.
__global__ __launch_bounds__(256) void nvfp4_gg_scales_to_blocked_kernel(uint32_t* __restrict__ dst,
                                                                         const uint8_t* __restrict__ src, int rows,
                                                                         int k, long ndw)
{
    const long d = (long)blockIdx.x * 256 + threadIdx.x;
    if (d >= ndw) return;
    const long atoms = k / 64;
    const long a = d >> 7;
    const int w = (int)(d & 127);
    const long row = (a / atoms) * 128 + 32 * (w & 3) + (w >> 2);
    const long c4 = a % atoms;
    uint32_t v = 0;
    if (row < rows) v = *reinterpret_cast<const uint32_t*>(src + row * (k / 16) + 4 * c4);
    dst[d] = v;
}

hipError_t launch_scales_to_blocked(void* dst, const void* src, int rows, int k, hipStream_t stream)
{
    const long ndw = blocked_scale_bytes(rows, k) / 4;
    if (ndw == 0) return hipSuccess;
    const long grid = (ndw + 255) / 256;
    void* d = dst;
    const void* s_ = src;
    long nd = ndw;
    void* params[] = {&d, &s_, &rows, &k, &nd};
    return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_scales_to_blocked_kernel), dim3((unsigned)grid),
                           dim3(256), params, 0, stream);
}

}  // namespace nvfp4gg
