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
// Structure.  One workgroup of 4 waves (one per SIMD) per CU walks a range of work units;
// a unit is up to 32*NA rows of one group times 32*NB columns, over the whole K.  Every
// wave owns the whole unit tile (NB x NA blocks of 32x32 fp32 accumulators, kept in the
// accumulation registers) and one quarter of every K superstep:
//   * K runs in supersteps of 256 (128 bytes of codes per row: one cache line).  The four
//     waves together fetch a superstep's lines (A and B codes, both scale sets) straight
//     from HBM/L2 into a ring slot in LDS (direct-to-LDS buffer loads, one whole line per
//     8 lanes); a ring of 3 slots (4 for 1x1 units) keeps 2 to 3 supersteps in flight.
//   * Wave w consumes K values 64w .. 64w+63 of each superstep: each lane reads its 16
//     code bytes per 32-row block with one LDS read, or two 8-byte reads in the units with
//     the most registers in use (rows are stored with an XOR swizzle of their 16-byte
//     chunks, so the 16-byte reads are bank-conflict free; the 8-byte reads pair lanes on
//     banks), and its two scale bytes, converts them to MFMA fragments in registers and
//     issues the MFMAs.  No LDS
//     holds converted values, so each FP4 byte is converted exactly once per unit.
//   * One barrier per superstep publishes the next superstep and frees the slot that was
//     read during the previous one.
//   * At the end of a unit the four K-quarter partial sums are added through LDS, rounded
//     to fp16 and stored.
// v_mfma_f32_32x32x16_f16 takes a B fragment (32 columns of C) as its first operand and
// an A fragment (32 rows of C) as its second, so a lane ends up holding runs of 4
// consecutive columns of one C row.  Inside each 64-K quarter the K order is permuted
// identically for A and B (the dot product is unchanged): lane half h, step s takes the
// 8 K values 64w + 32h + 8s .. +8, so a lane's 16 bytes are contiguous in the row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "nvfp4_gg_internal.h"

namespace nvfp4gg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f16v_t __attribute__((ext_vector_type(16)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// Exact dequantisation
// ---------------------------------------------------------------------------------------

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default mode).
__device__ __forceinline__ uint16_t f16_bits_rne(float f)
{
    const _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// A fragment dword holds 2 elements: the hardware FP4 -> fp16 conversion of one code byte
// (low nibble = even K) with scale 1.0 gives the exact E2M1 values, and one packed fp16
// multiply applies the block's E4M3 scale exactly (convert_dword below).

// Calls f(integral_constant<int, i>) for i = B .. E-1 in order.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------------------
// Geometry
// ---------------------------------------------------------------------------------------
namespace gk {
constexpr int THREADS = 256;           // 4 waves, one per SIMD
constexpr int SK = 256;                // K per superstep
constexpr int ROWB = SK / 2;           // code bytes per row and superstep: one 128-byte line
constexpr int BLK_CODE = 32 * ROWB;    // one 32-row block's codes per superstep (4 KiB)
constexpr int LDS_BYTES = 160 * 1024;
constexpr int MAX_SLOTS = 4;
// Ring depth of units of at least this many operand blocks (every shape but 1x1).  When many
// CUs stream at once, a shallow ring keeps each CU's reads in flight on the supersteps needed
// next and asks for fewer bytes when all workgroups start together, so every CU's superstep
// lands sooner (measured: 3 slots instead of 5-6 cut 2x4 launches of 256 units by 9 %, 2x3 by
// 10 %, 2x2 and 1x2 launches by 4-8 %, 4x4 units 3 instead of 4 by 3 %).  1x1 units, planned
// for launches with few CUs busy, take MAX_SLOTS: 4 hides their latency best (3 slots cost
// them up to 2.6 %, 5 or 6 up to 5 %).
constexpr int LARGE_UNIT_BLOCKS = 3;
constexpr int LARGE_UNIT_SLOTS = 3;

// Chunk swizzle: row r of a block keeps its 16-byte chunk c at position c ^ swz(r).  The
// 16-byte reads of one chunk from rows 0..7 (or 0..15) of a block then fall on distinct
// bank groups for 32 banks (8 lanes per cycle) and for 64 banks (16 lanes per cycle).
__host__ __device__ constexpr int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Ring slot of a unit with NA row blocks (A) and NB column blocks (B):
//   codes   block x (B blocks 0..NB-1, then A blocks NB..NB+NA-1): 32 rows x 128 B at
//           x * 4096, row r at 128 r, chunk c at 16 (c ^ swz(r));
//   scales  four row-quarter regions (rows 8q..8q+7 of every block, loaded by wave q),
//           SREG bytes apart; inside region q, scale block y (B blocks 0..NB-1, then A
//           blocks from NBp = NB rounded up to even) row 8q + i: 16 bytes at 128 y + 16 i.
//           The regions are 4 bytes more than a multiple of 256 apart, so that the scale
//           reads of rows 0..31 (one dword each) fall on 32 distinct banks.
template <int NA, int NB>
struct Geo {
    static constexpr int NBLK = NA + NB;
    static constexpr int NBP = (NB + 1) & ~1;
    static constexpr int NAP = (NA + 1) & ~1;
    static constexpr int SREG = 128 * (NBP + NAP) + 4;
    static constexpr int SCALE_AT = NBLK * BLK_CODE;
    static constexpr int SLOT = (SCALE_AT + 4 * SREG + 15) & ~15;
    static constexpr int SLOT_CAP = NBLK >= LARGE_UNIT_BLOCKS ? LARGE_UNIT_SLOTS : MAX_SLOTS;
    static constexpr int SLOTS = LDS_BYTES / SLOT > SLOT_CAP ? SLOT_CAP : LDS_BYTES / SLOT;
    static constexpr int NSI = (NBP + NAP) / 2;    // scale load instructions per wave
    static constexpr int OPS = NBLK + NSI;         // loads per wave and superstep
    static constexpr int NACC = NA * NB;           // accumulator blocks
    // each lane reads its 16 code bytes of a block in one LDS read per superstep, except in
    // the units with the most registers in use (20 accumulator blocks, or 11 operand blocks),
    // which read them in two 8-byte halves (two fewer code registers per block)
    static constexpr bool FULL_READS = NACC < 20 && NBLK < 11;
    // epilogue exchange: per block, 4 element groups x 3 partner copies x 1 KiB
    static constexpr int RED_BLK = 3 * 4 * 1024;
    // the exchange region starts after ring slot 0, which may meanwhile take the first
    // superstep of the workgroup's next unit
    static constexpr int RED_AT = SLOT;
    static constexpr int RED_FIT = (LDS_BYTES - RED_AT) / RED_BLK;
    static constexpr int RED_ROUND = RED_FIT < NACC ? RED_FIT : NACC;
    static_assert(RED_FIT >= 1, "the exchange region must hold one block");
    static_assert(SLOTS >= 3, "a unit shape needs at least 3 ring slots");
    static_assert((SLOTS - 2) * OPS <= 63, "the steady-state wait count must fit vmcnt");
};
}  // namespace gk

// ---------------------------------------------------------------------------------------
// Loads
// ---------------------------------------------------------------------------------------

// Raw buffer resource over `bytes` bytes at base (at most 2^31 - 1): loads address it as
// scalar base + 32-bit vector offset + scalar offset, and vector offsets at or beyond
// `bytes` read as zero (a direct-to-LDS load then stores zeros).  The base and size are
// the same in every lane; saying so (readfirstlane) keeps the resource in scalar registers,
// where a buffer instruction needs it (otherwise every load becomes a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, long bytes)
{
    const int n = __builtin_amdgcn_readfirstlane(bytes >= 0x7fffffffL ? 0x7fffffff : (int)bytes);
    const uint64_t p = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// A vector offset beyond every buffer range (all ranges are below 2^31 bytes).
constexpr uint32_t kOffNone = 0x80000000u;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, uint8_t* lds)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, (int)voff, soff, 0, 0);
}

// What one wave loads for one unit, per superstep (addresses relative to the unit):
//   codes: for every block, the 8 rows 8w .. 8w+7 (lane l: row 8w + l/8, global chunk
//          (l%8) ^ swz(row), stored at LDS chunk position l%8);
//   scales: for every pair of scale blocks, rows 8w .. 8w+7 x the superstep's four 4-byte
//          scale words (lane l: block 2p + l/32, row 8w + (l%32)/4, word l%4).
// B rows beyond n and A rows beyond m read as zero codes (buffer range); their scale rows
// are clamped to the last row, so that padding scales are never read.
template <int NA, int NB>
struct UnitLoads {
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    uint32_t code[(NA > NB ? NA : NB)];       // per-lane code offset of block b' of a side
    uint32_t scl[gk::Geo<NA, NB>::NSI];       // per-lane scale offset of scale instruction p
    int scl_step;                             // scale bytes between supersteps
    int code_chunk;                           // global 16-byte chunk of this lane's code loads
    int scl_word;                             // scale word (0..3) of this lane's scale loads
};

// Issue wave w's loads of superstep t (kt = K values it holds: 256 except maybe in the
// last) into `slot`.  In a short superstep, lanes whose 16-byte code chunk or 4-byte scale
// word lies beyond K load from an offset outside the buffer, which stores zeros to their
// LDS place (zero codes and zero scales add exact zeros).  The code is the same for every
// superstep (no branch), so every wait count is the same in all supersteps too.
template <int NA, int NB>
struct Refill {
    uint8_t* slot;   // this wave's slot base
    int soff, ssoff; // code and scale offsets of the superstep
    bool cv, sv;     // this lane's code chunk / scale word lies inside K
};

template <int NA, int NB>
__device__ __forceinline__ Refill<NA, NB> refill_of(const UnitLoads<NA, NB>& L, uint8_t* slot, int t, int kt)
{
    return Refill<NA, NB>{slot, t * gk::ROWB, t * L.scl_step, L.code_chunk < (kt >> 5), L.scl_word < (kt >> 6)};
}

// Load OP of a superstep: B code blocks 0..NB-1, A code blocks, then the scale pairs.
template <int NA, int NB, int OP>
__device__ __forceinline__ void issue_op(const UnitLoads<NA, NB>& L, const Refill<NA, NB>& R, int wave)
{
    using G = gk::Geo<NA, NB>;
    if constexpr (OP < NB)
        dma16(L.rb, R.cv ? L.code[OP] : kOffNone, R.soff, R.slot + OP * gk::BLK_CODE + wave * 1024);
    else if constexpr (OP < G::NBLK)
        dma16(L.ra, R.cv ? L.code[OP - NB] : kOffNone, R.soff, R.slot + OP * gk::BLK_CODE + wave * 1024);
    else
        dma4(OP - G::NBLK < G::NBP / 2 ? L.rsb : L.rsa, R.sv ? L.scl[OP - G::NBLK] : kOffNone, R.ssoff,
             R.slot + G::SCALE_AT + wave * G::SREG + (OP - G::NBLK) * 256);
}

template <int NA, int NB>
__device__ __forceinline__ void issue_superstep(const UnitLoads<NA, NB>& L, uint8_t* slot, int t, int kt, int wave)
{
    const Refill<NA, NB> R = refill_of<NA, NB>(L, slot, t, kt);
    static_for<0, gk::Geo<NA, NB>::OPS>([&](auto op) { issue_op<NA, NB, decltype(op)::value>(L, R, wave); });
}

// Per-lane load offsets and buffer resources of one unit (see UnitLoads).  `rows` / `cols`
// are the unit's valid A rows / B rows (C columns).
template <int NA, int NB>
__device__ __forceinline__ UnitLoads<NA, NB> unit_loads(const GroupArgs& G, int k, int row0, int rows, int col0,
                                                        int cols, bool blocked, int wave, int lane)
{
    using Gm = gk::Geo<NA, NB>;
    UnitLoads<NA, NB> L;
    const long qs = k / 2;
    const int rb8 = 8 * wave + (lane >> 3);   // row inside a block of this lane's code loads
    L.code_chunk = (lane & 7) ^ gk::swz(rb8);
#pragma unroll
    for (int b = 0; b < (NA > NB ? NA : NB); ++b) L.code[b] = (uint32_t)((32 * b + rb8) * qs + 16 * L.code_chunk);
    L.rb = make_rsrc(G.b + (long)col0 * qs, (long)cols * qs);
    L.ra = make_rsrc(G.a + (long)row0 * qs, (long)rows * qs);
    L.scl_word = lane & 3;
    const int srow = 8 * wave + ((lane & 31) >> 2);   // row inside a block of this lane's scale loads
    if (!blocked) {
        // row-major [rows][k/16]: superstep t's 16 scales of a row are its bytes 16t .. 16t+15
        const long ss = k / 16;
#pragma unroll
        for (int p = 0; p < Gm::NSI; ++p) {
            const int y = 2 * p + (lane >> 5);
            const bool bside = p < Gm::NBP / 2;
            const int bl = bside ? min(y, NB - 1) : min(y - Gm::NBP, NA - 1);
            const int r = min(32 * bl + srow, (bside ? cols : rows) - 1);
            L.scl[p] = (uint32_t)(r * ss + 4 * L.scl_word);
        }
        L.rsb = make_rsrc(G.sfb + (long)col0 * ss, 0x7fffffffL);
        L.rsa = make_rsrc(G.sfa + (long)row0 * ss, 0x7fffffffL);
        L.scl_step = gk::SK / 16;
    } else {
        // 128x4 blocked: scale (row R, K block c) at ((R/128) (k/64) + c/4) 512 + 16 (R%32)
        // + 4 ((R/32)%4) + c%4; superstep t covers the four atoms 4t .. 4t+3 of a row block
        const long atoms = k / 64;
        const int b0 = col0 >> 7, a0 = row0 >> 7;
#pragma unroll
        for (int p = 0; p < Gm::NSI; ++p) {
            const int y = 2 * p + (lane >> 5);
            const bool bside = p < Gm::NBP / 2;
            const int bl = bside ? min(y, NB - 1) : min(y - Gm::NBP, NA - 1);
            const int r = min(32 * bl + srow, (bside ? cols : rows) - 1);
            const int R = (bside ? col0 : row0) + r;
            const int rb0 = bside ? b0 : a0;
            L.scl[p] = (uint32_t)((((long)(R >> 7) - rb0) * atoms + L.scl_word) * 512 + 16 * (R & 31) +
                                  4 * ((R >> 5) & 3));
        }
        L.rsb = make_rsrc(G.sfb + (long)b0 * atoms * 512, 0x7fffffffL);
        L.rsa = make_rsrc(G.sfa + (long)a0 * atoms * 512, 0x7fffffffL);
        L.scl_step = 4 * 512;
    }
    return L;
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier for LDS hand-offs: waits for this wave's own LDS reads and writes, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding direct-to-LDS loads
// (those are waited for explicitly, so later supersteps stay in flight).
__device__ __forceinline__ void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the same wait as an instruction the compiler sees (it cannot read the asm): it then
    // knows every earlier LDS read has returned and adds no wait of its own for them; the
    // count is already zero, so this costs nothing
    __builtin_amdgcn_s_waitcnt(0xc07f);
}

// ---------------------------------------------------------------------------------------
// Compute
// ---------------------------------------------------------------------------------------

// This wave's raw code dwords (one per 16-K step) of a superstep, W = 4: all four steps
// (one 16-byte read per block), or W = 2: one half of it (steps 0-1 or 2-3, one 8-byte
// read per block).
template <int NA, int NB, int W>
struct RawCodes {
    using V = std::conditional_t<W == 4, u4_t, u2_t>;
    V cb[NB], ca[NA];
};

// The two scale bytes of each block's row in one superstep (low byte: steps 0 and 1, high
// byte: steps 2 and 3).
template <int NA, int NB>
struct RawScales {
    uint32_t sb[NB], sa[NA];
};

// The code read of block Y (B blocks first, then A blocks).
template <int NA, int NB, int W, int OFF, int Y>
__device__ __forceinline__ void read_code(RawCodes<NA, NB, W>& R, const uint8_t* slot, int code_off)
{
    using V = typename RawCodes<NA, NB, W>::V;
    if constexpr (Y < NB)
        R.cb[Y] = *reinterpret_cast<const V*>(slot + Y * gk::BLK_CODE + code_off + OFF);
    else
        R.ca[Y - NB] = *reinterpret_cast<const V*>(slot + Y * gk::BLK_CODE + code_off + OFF);
}

template <int NA, int NB, int W, int OFF>
__device__ __forceinline__ void read_codes(RawCodes<NA, NB, W>& R, const uint8_t* slot, int code_off)
{
    using V = typename RawCodes<NA, NB, W>::V;
#pragma unroll
    for (int x = 0; x < NB; ++x) R.cb[x] = *reinterpret_cast<const V*>(slot + x * gk::BLK_CODE + code_off + OFF);
#pragma unroll
    for (int i = 0; i < NA; ++i)
        R.ca[i] = *reinterpret_cast<const V*>(slot + (NB + i) * gk::BLK_CODE + code_off + OFF);
}

// The scale read of block Y (B blocks first, then A blocks).
template <int NA, int NB, int Y>
__device__ __forceinline__ void read_scale(RawScales<NA, NB>& R, const uint8_t* slot, int scale_off)
{
    using Gm = gk::Geo<NA, NB>;
    if constexpr (Y < NB)
        R.sb[Y] = *reinterpret_cast<const uint16_t*>(slot + Gm::SCALE_AT + scale_off + 128 * Y);
    else
        R.sa[Y - NB] = *reinterpret_cast<const uint16_t*>(slot + Gm::SCALE_AT + scale_off + 128 * (Gm::NBP + Y - NB));
}

template <int NA, int NB>
__device__ __forceinline__ void read_scales(RawScales<NA, NB>& R, const uint8_t* slot, int scale_off)
{
    using Gm = gk::Geo<NA, NB>;
#pragma unroll
    for (int x = 0; x < NB; ++x) R.sb[x] = *reinterpret_cast<const uint16_t*>(slot + Gm::SCALE_AT + scale_off + 128 * x);
#pragma unroll
    for (int i = 0; i < NA; ++i)
        R.sa[i] = *reinterpret_cast<const uint16_t*>(slot + Gm::SCALE_AT + scale_off + 128 * (Gm::NBP + i));
}

// MFMA fragments of one 16-K step: one per B block and one per A block (dword e holds
// elements 2e and 2e + 1 as fp16).
template <int NA, int NB>
struct Frags {
    u4_t b[NB], a[NA];
};

// The fp16 scale pairs of a superstep (element 0: steps 0 and 1, element 1: steps 2 and 3).
template <int NA, int NB>
struct Scales {
    h2_t b[NB], a[NA];
};

// Scale pair of block Y (B blocks first, then A blocks) from its two raw E4M3 bytes.
template <int NA, int NB, int Y>
__device__ __forceinline__ void convert_scale(Scales<NA, NB>& S, const RawScales<NA, NB>& R)
{
    if constexpr (Y < NB)
        S.b[Y] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(R.sb[Y], 1.0f, false);
    else
        S.a[Y - NB] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(R.sa[Y - NB], 1.0f, false);
}

// Dword E of fragment Y (B blocks first, then A blocks) of step ST (0..3) of a superstep,
// from dword D of the raw codes that hold it: two E2M1 codes (byte E of the step's code
// dword) converted exactly by the hardware, times the block's E4M3 scale in fp16 (exact,
// see above).
template <int NA, int NB, int ST, int D, int Y, int E, int W>
__device__ __forceinline__ void convert_dword(Frags<NA, NB>& F, const RawCodes<NA, NB, W>& R, const Scales<NA, NB>& S)
{
    if constexpr (Y < NB) {
        const _Float16 c = ST < 2 ? S.b[Y].x : S.b[Y].y;
        F.b[Y][E] = __builtin_bit_cast(uint32_t,
                                       __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(R.cb[Y][D], 1.0f, E) * h2_t{c, c});
    } else {
        const _Float16 c = ST < 2 ? S.a[Y - NB].x : S.a[Y - NB].y;
        F.a[Y - NB][E] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(R.ca[Y - NB][D], 1.0f, E) * h2_t{c, c});
    }
}

template <int NA, int NB>
__device__ __forceinline__ void convert_scales(Scales<NA, NB>& S, const RawScales<NA, NB>& R)
{
    static_for<0, NA + NB>([&](auto y) { convert_scale<NA, NB, decltype(y)::value>(S, R); });
}

template <int NA, int NB, int ST, int D, int W>
__device__ __forceinline__ void convert_step(Frags<NA, NB>& F, const RawCodes<NA, NB, W>& R, const Scales<NA, NB>& S)
{
    static_for<0, 4 * (NA + NB)>([&](auto j) {
        constexpr int J = decltype(j)::value;
        convert_dword<NA, NB, ST, D, J / 4, J % 4>(F, R, S);
    });
}

// Accumulator blocks 0..15 (x * NA + i) live in the 256 accumulation registers; a unit with
// more blocks keeps the rest in ordinary VGPRs.  The compiler places every accumulator of
// its MFMA builtin in one register class, so the extra blocks use the same instruction
// written out, with its operands pinned to VGPRs; the s_nop before it covers the VALU
// writes of its fragments (and of the zero start value) just before, the s_nop after it
// the reads of its source fragments by the VALU that may overwrite them next.
constexpr int kAgprBlocks = 16;

__device__ __forceinline__ void mfma_vgpr_acc(f16v_t& acc, const u4_t& b, const u4_t& a)
{
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\ts_nop 1" : "+v"(acc) : "v"(b), "v"(a));
}

// MFMA of accumulator block Q (column block Q / NA, row block Q % NA).
template <int NA, int NB, int Q>
__device__ __forceinline__ void mfma_block(f16v_t (&acc)[NB][NA], const Frags<NA, NB>& F)
{
    constexpr int x = Q / NA, i = Q % NA;
    if constexpr (Q < kAgprBlocks)
        acc[x][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, F.b[x]),
                                                         __builtin_bit_cast(h8_t, F.a[i]), acc[x][i], 0, 0, 0);
    else
        mfma_vgpr_acc(acc[x][i], F.b[x], F.a[i]);
}

// One 16-K step in program order: the NA * NB MFMAs, each followed by its share of the NR
// LDS reads, the NL loads and the NJ VALU jobs that prepare later steps, fenced so that the
// compiler keeps this order (a VALU job issues while the MFMA before it runs; reads and
// loads reach the LDS and memory pipelines spread over the step instead of in a burst that
// the four waves would queue on).
template <int NM, int NJ, int NL, int NR, class M, class J, class L, class R>
__device__ __forceinline__ void bundled_step(M&& mfma, J&& job, L&& load, R&& read)
{
    static_for<0, NM>([&](auto q) {
        constexpr int Q = decltype(q)::value;
        mfma(q);
        static_for<Q * NR / NM, (Q + 1) * NR / NM>(read);
        static_for<Q * NL / NM, (Q + 1) * NL / NM>(load);
        static_for<Q * NJ / NM, (Q + 1) * NJ / NM>(job);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// After the last MFMA of a unit: the written-out MFMAs' results become readable by the VALU
// only after the pipeline has drained (the compiler cannot count for them), so wait it out
// once, with the extra blocks as operands so that no read of them moves above the wait.
template <int NA, int NB>
__device__ __forceinline__ void drain_vgpr_acc(f16v_t (&acc)[NB][NA])
{
    if constexpr (NA * NB > kAgprBlocks) {
#pragma unroll
        for (int x = 0; x < NB; ++x)
#pragma unroll
            for (int i = 0; i < NA; ++i)
                if (x * NA + i >= kAgprBlocks) asm volatile("" : "+v"(acc[x][i]));
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int x = 0; x < NB; ++x)
#pragma unroll
            for (int i = 0; i < NA; ++i)
                if (x * NA + i >= kAgprBlocks) asm volatile("" : "+v"(acc[x][i]));
    }
}

// ---------------------------------------------------------------------------------------
// Epilogue
// ---------------------------------------------------------------------------------------

// Sum of the four K-quarter partial tiles, fp16 rounding and stores.  Lane (j, h) holds in
// acc[x][i] element 4q + e the partial sum of C[32 i + j][32 x + 8 q + 4 h + e].  Wave W
// keeps element group q = W and hands the other three groups to their owners through LDS,
// RED_ROUND blocks at a time.  W is a template parameter so that every element index is
// static (the accumulators live in registers that cannot be indexed at run time).
template <int NA, int NB, int W>
__device__ __forceinline__ void epilogue_w(const f16v_t (&acc)[NB][NA], uint8_t* smem, uint16_t* __restrict__ c0,
                                           int rows, int cols, int ldc, int lane)
{
    using Gm = gk::Geo<NA, NB>;
    constexpr int RR = Gm::RED_ROUND;
    const int j = lane & 31, h = lane >> 5;
    const bool vec = (ldc & 3) == 0;
    // every column of the unit exists and rows are 8-byte aligned: one 8-byte store per lane,
    // masked by the row only (and not at all when every row exists)
    const bool colfull = cols == 32 * NB && vec;
    // exchange place of element group q's copy from partner slot sl, round block xr
    const auto at = [&](int xr, int q, int sl) {
        return smem + Gm::RED_AT + (((xr * 4 + q) * 3 + sl) * 64 + lane) * 16;
    };
    // this lane's first C element of row block ib (row 32 ib + j, columns 8 W + 4 h ..)
    uint16_t* rowp[NA];
#pragma unroll
    for (int ib = 0; ib < NA; ++ib) rowp[ib] = c0 + (long)(32 * ib + j) * ldc + 8 * W + 4 * h;
    static_for<0, (Gm::NACC + RR - 1) / RR>([&](auto rd) {
        constexpr int R0 = decltype(rd)::value * RR;
        constexpr int NR = Gm::NACC - R0 < RR ? Gm::NACC - R0 : RR;
        barrier_lds();   // the ring, or the previous round's exchange, is no longer read
        static_for<0, NR>([&](auto xr_) {
            constexpr int XR = decltype(xr_)::value;
            constexpr int xb = (R0 + XR) / NA, ib = (R0 + XR) % NA;
            static_for<0, 4>([&](auto q_) {
                constexpr int Q = decltype(q_)::value;
                if constexpr (Q != W) {
                    constexpr int SL = W - (W > Q ? 1 : 0);
                    *reinterpret_cast<u4_t*>(at(XR, Q, SL)) =
                        u4_t{__float_as_uint(acc[xb][ib][4 * Q + 0]), __float_as_uint(acc[xb][ib][4 * Q + 1]),
                             __float_as_uint(acc[xb][ib][4 * Q + 2]), __float_as_uint(acc[xb][ib][4 * Q + 3])};
                }
            });
            __builtin_amdgcn_sched_barrier(0);   // one block's copies at a time (register pressure)
        });
        barrier_lds();
        // read the partner copies RD blocks ahead of the sums that use them
        constexpr int RD = 4;
        u4_t o[RD][3];
        static_for<0, (RD - 1 < NR ? RD - 1 : NR)>([&](auto x_) {
            constexpr int X = decltype(x_)::value;
            static_for<0, 3>([&](auto sl) {
                o[X % RD][decltype(sl)::value] = *reinterpret_cast<const u4_t*>(at(X, W, sl));
            });
        });
        static_for<0, NR>([&](auto xr_) {
            constexpr int XR = decltype(xr_)::value;
            constexpr int xb = (R0 + XR) / NA, ib = (R0 + XR) % NA;
            if constexpr (XR + RD - 1 < NR)
                static_for<0, 3>([&](auto sl) {
                    o[(XR + RD - 1) % RD][decltype(sl)::value] =
                        *reinterpret_cast<const u4_t*>(at(XR + RD - 1, W, sl));
                });
            __builtin_amdgcn_sched_barrier(0);
            float v[4];
            static_for<0, 4>([&](auto e_) {
                constexpr int E = decltype(e_)::value;
                v[E] = acc[xb][ib][4 * W + E] + __uint_as_float(o[XR % RD][0][E]) +
                       __uint_as_float(o[XR % RD][1][E]) + __uint_as_float(o[XR % RD][2][E]);
            });
            const int r = 32 * ib + j;
            const int cc = 32 * xb + 8 * W + 4 * h;
            if (colfull) {
                if (r < rows)
                    *reinterpret_cast<u2_t*>(rowp[ib] + 32 * xb) =
                        u2_t{(uint32_t)f16_bits_rne(v[0]) | ((uint32_t)f16_bits_rne(v[1]) << 16),
                             (uint32_t)f16_bits_rne(v[2]) | ((uint32_t)f16_bits_rne(v[3]) << 16)};
            } else if (r < rows) {
                uint16_t* crow = c0 + (long)r * ldc;
                const uint16_t h0 = f16_bits_rne(v[0]), h1 = f16_bits_rne(v[1]);
                const uint16_t h2 = f16_bits_rne(v[2]), h3 = f16_bits_rne(v[3]);
                if (vec && cc + 4 <= cols) {
                    *reinterpret_cast<u2_t*>(crow + cc) =
                        u2_t{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
                } else {
                    if (cc + 0 < cols) crow[cc + 0] = h0;
                    if (cc + 1 < cols) crow[cc + 1] = h1;
                    if (cc + 2 < cols) crow[cc + 2] = h2;
                    if (cc + 3 < cols) crow[cc + 3] = h3;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    });
    barrier_lds();   // every exchange read is done before the LDS is reused
}

// ---------------------------------------------------------------------------------------
// One unit
// ---------------------------------------------------------------------------------------

// One unit of the schedule: group gi, rows [row0, row0 + rows) times columns
// [col0, col0 + cols), unit shape na x nb.
struct Unit {
    int gi, row0, rows, col0, cols, na, nb;
};

// Unit cu over the whole K of its group.  If `prefetched`, the previous unit already issued
// this unit's superstep 0 (same shape); if `pf_next`, this unit issues that of the next unit
// nx (same shape) before its own epilogue, so that its fetch overlaps the K reduction and the
// C stores.  (One superstep measured better than S-1 of them: a smaller burst while the
// epilogue runs, and more LDS for the exchange.)  All four waves run the same sequence of
// loads and barriers.
template <int NA, int NB>
__device__ __forceinline__ void run_unit(const KernArgs& A, const Unit& cu, const GroupArgs G, bool prefetched, bool pf_next,
                                         const Unit& nx, bool blocked, uint8_t* smem)
{
    using Gm = gk::Geo<NA, NB>;
    const int k = G.k, row0 = cu.row0, rows = cu.rows, col0 = cu.col0, cols = cu.cols, ldc = G.ldc;
    constexpr int S = Gm::SLOTS;
    // the thread index through an instruction the compiler cannot hoist: values derived from
    // it are then recomputed per unit instead of being kept live across all of them (the
    // kernel has no scratch)
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nsup = (k + gk::SK - 1) / gk::SK;
    const int klast = k - gk::SK * (nsup - 1);
    // K values of superstep t: 256, the tail in the last, none beyond (such supersteps are
    // still "loaded", every lane from outside the buffers, which stores zeros: so every
    // superstep issues the same loads and waits with the same count)
    const auto kt_of = [&](int t) { return t < nsup - 1 ? gk::SK : t == nsup - 1 ? klast : 0; };

    // The ring's first S supersteps go out first (superstep 0 only if the previous unit has
    // not issued it).  The previous unit's C stores may still be in flight: they touch
    // neither LDS nor this unit's operands, and loads complete in issue order among
    // themselves, so whatever the stores do, the wait below means that superstep 0 has
    // landed.
    const UnitLoads<NA, NB> L = unit_loads<NA, NB>(G, k, row0, rows, col0, cols, blocked, wave, lane);
    if (!prefetched)
        issue_superstep<NA, NB>(L, smem, 0, kt_of(0), wave);
    static_for<1, S - 1>([&](auto t) { issue_superstep<NA, NB>(L, smem + t * Gm::SLOT, t, kt_of(t), wave); });
    issue_superstep<NA, NB>(L, smem + (S - 1) * Gm::SLOT, S - 1, kt_of(S - 1), wave);
    __builtin_amdgcn_sched_barrier(0);

    // The accumulators start at zero.  The zero comes from an instruction the compiler cannot
    // hoist: a zero vector hoisted out of the unit loop would stay live across every unit and
    // be spilled to scratch (and a kernel with a larger scratch allocation launches its waves
    // markedly slower: measured 2x on the 1-unit-per-workgroup shapes at 96 bytes per lane).
    float zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    const f16v_t zv = {zero, zero, zero, zero, zero, zero, zero, zero, zero, zero, zero, zero, zero, zero, zero, zero};
    f16v_t acc[NB][NA];
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int i = 0; i < NA; ++i) acc[x][i] = zv;

    // this lane's LDS read offsets inside a slot (wave's K quarter, lane half h, row j)
    const int j = lane & 31, h = lane >> 5;
    const int code_off = j * gk::ROWB + 16 * ((2 * wave + h) ^ gk::swz(j));
    const int scale_off = (j >> 3) * Gm::SREG + 16 * (j & 7) + 4 * wave + 2 * h;

    wait_vm<(S - 1) * Gm::OPS>();   // superstep 0 has landed (this wave's part)
    barrier_lds();
    constexpr bool FULL = Gm::FULL_READS;
    constexpr int W = FULL ? 4 : 2;
    RawCodes<NA, NB, W> rc[2];   // a superstep's codes (FULL) or its first half
    RawCodes<NA, NB, 2> h1;      // the second half (not FULL)
    RawScales<NA, NB> rs[2];
    Scales<NA, NB> sc[2];
    Frags<NA, NB> fr[2];
    read_codes<NA, NB, W, 0>(rc[0], smem, code_off);
    read_scales<NA, NB>(rs[0], smem, scale_off);
    convert_scales<NA, NB>(sc[0], rs[0]);
    convert_step<NA, NB, 0, 0>(fr[0], rc[0], sc[0]);

    // One superstep t (its codes, or their first half, in rc[P], scales in sc[P], step 0's
    // fragments in fr[0]).  Unless its whole codes are already in rc[P], the second half is
    // read at once; steps 0 and 1 run (MFMAs of a step beside the next step's
    // conversions).  Then the wave waits for its own loads of superstep t+1, and the
    // barrier publishes them and frees slot cs (superstep t has been read by every wave),
    // which is refilled with superstep t+S; the codes (or first half) and the scales of
    // superstep t+1 are read, and steps 2 and 3 run, step 3 beside the conversion of step 0
    // of superstep t+1.  In the last superstep the "next" reads and
    // conversions touch no superstep's bytes: harmless, and their results are unused.
    // Every superstep refills its slot (with zeros beyond the last superstep) and waits with
    // the same count; the refill's loads are spread over step 2.
    constexpr int NM = NA * NB;
    constexpr int NJ = 4 * Gm::NBLK;   // VALU jobs of one step's conversion
    const auto no_op = [](auto) {};
    int cs = 0;
    const auto superstep = [&](auto P_, int t) {
        constexpr int P = decltype(P_)::value;
        const int ns = cs + 1 == S ? 0 : cs + 1;
        const uint8_t* cur = smem + cs * Gm::SLOT;
        const uint8_t* nxt = smem + ns * Gm::SLOT;
        // step 0 (and, with half reads, the second half's reads)
        bundled_step<NM, NJ, 0, FULL ? 0 : Gm::NBLK>(
            [&](auto q) { mfma_block<NA, NB, decltype(q)::value>(acc, fr[0]); },
            [&](auto j) {
                constexpr int J = decltype(j)::value;
                convert_dword<NA, NB, 1, 1, J / 4, J % 4>(fr[1], rc[P], sc[P]);
            },
            no_op, [&](auto y) { read_code<NA, NB, 2, 8, decltype(y)::value>(h1, cur, code_off); });
        bundled_step<NM, NJ, 0, 0>([&](auto q) { mfma_block<NA, NB, decltype(q)::value>(acc, fr[1]); },
                                [&](auto j) {
                                    constexpr int J = decltype(j)::value;
                                    if constexpr (FULL)
                                        convert_dword<NA, NB, 2, 2, J / 4, J % 4>(fr[0], rc[P], sc[P]);
                                    else
                                        convert_dword<NA, NB, 2, 0, J / 4, J % 4>(fr[0], h1, sc[P]);
                                },
                                no_op, no_op);
        wait_vm<(S - 2) * Gm::OPS>();
        barrier_lds();
        const auto step2_jobs = [&](auto j) {
            constexpr int J = decltype(j)::value;
            if constexpr (FULL)
                convert_dword<NA, NB, 3, 3, J / 4, J % 4>(fr[1], rc[P], sc[P]);
            else
                convert_dword<NA, NB, 3, 1, J / 4, J % 4>(fr[1], h1, sc[P]);
        };
        const auto step2_mfma = [&](auto q) { mfma_block<NA, NB, decltype(q)::value>(acc, fr[0]); };
        const Refill<NA, NB> R = refill_of<NA, NB>(L, const_cast<uint8_t*>(cur), t + S, kt_of(t + S));
        // step 2, with the refill's loads and the reads of superstep t+1 (scales first, which
        // step 3 converts first)
        bundled_step<NM, NJ, Gm::OPS, 2 * Gm::NBLK>(
            step2_mfma, step2_jobs, [&](auto op) { issue_op<NA, NB, decltype(op)::value>(L, R, wave); },
            [&](auto r) {
                constexpr int RD = decltype(r)::value;
                if constexpr (RD < Gm::NBLK)
                    read_scale<NA, NB, RD>(rs[1 - P], nxt, scale_off);
                else
                    read_code<NA, NB, W, 0, RD - Gm::NBLK>(rc[1 - P], nxt, code_off);
            });
        // step 3: first the next superstep's scales, then its step 0 fragments
        bundled_step<NM, NJ + Gm::NBLK, 0, 0>([&](auto q) { mfma_block<NA, NB, decltype(q)::value>(acc, fr[1]); },
                                           [&](auto j) {
                                               constexpr int J = decltype(j)::value;
                                               if constexpr (J < Gm::NBLK)
                                                   convert_scale<NA, NB, J>(sc[1 - P], rs[1 - P]);
                                               else
                                                   convert_dword<NA, NB, 0, 0, (J - Gm::NBLK) / 4, (J - Gm::NBLK) % 4>(
                                                       fr[0], rc[1 - P], sc[1 - P]);
                                           },
                                           no_op, no_op);
        cs = ns;
    };
    for (int t = 0; t < nsup; t += 2) {
        superstep(std::integral_constant<int, 0>{}, t);
        if (t + 1 < nsup) superstep(std::integral_constant<int, 1>{}, t + 1);
    }
    wait_vm<0>();   // the zero refills beyond the last superstep have landed before the LDS is reused

    if (pf_next) {
        // every wave has read the ring for the last time: slot 0 takes the next unit's first
        // superstep (the exchange region lies beyond it)
        barrier_lds();
        const GroupArgs& Gn = A.grp[nx.gi];
        const UnitLoads<NA, NB> Ln =
            unit_loads<NA, NB>(Gn, Gn.k, nx.row0, nx.rows, nx.col0, nx.cols, blocked, wave, lane);
        issue_superstep<NA, NB>(Ln, smem, 0, Gn.k < gk::SK ? Gn.k : gk::SK, wave);   // K of superstep 0
    }
    drain_vgpr_acc<NA, NB>(acc);
    uint16_t* c0 = G.c + (long)row0 * ldc + col0;
    switch (wave) {
    case 0: epilogue_w<NA, NB, 0>(acc, smem, c0, rows, cols, ldc, lane); break;
    case 1: epilogue_w<NA, NB, 1>(acc, smem, c0, rows, cols, ldc, lane); break;
    case 2: epilogue_w<NA, NB, 2>(acc, smem, c0, rows, cols, ldc, lane); break;
    default: epilogue_w<NA, NB, 3>(acc, smem, c0, rows, cols, ldc, lane); break;
    }
}

// ---------------------------------------------------------------------------------------
// Persistent grouped scheduler
// ---------------------------------------------------------------------------------------

// Workgroup b is virtual workgroup v = (b % 8) * vq + b / 8 of V = 8 vq (workgroups are
// dealt to the 8 XCDs round-robin, so consecutive v share an XCD and its L2); it runs
// the units [U v / V, U (v+1) / V) of the unit sequence, which lists every group's units
// in schedule order, row chunks fastest (so the units that read one B column tile are
// consecutive).  This is the prefix-sum tile enumeration of the persistent scheduler on
// the page "kernelindex submission 503584" (a group's units are ceil(m / 32 na) row chunks
// times ceil(n / 32 nb) column tiles; a unit's group is found from the running sums of these
// counts, its tile from its rank inside the group).
constexpr int kEagerGroups = 8;

__global__ __launch_bounds__(gk::THREADS) void nvfp4_gg_units(KernArgs args_byval)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[gk::LDS_BYTES];
    (void)args_byval;
    const KernArgs& A = *(const KernArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    // Lane l reads entry l of the group table, the first kEagerGroups lanes together with the
    // header (lanes < NVFP4_GG_MAX_GROUPS, so every read lies inside the kernel arguments).
    // Units are then found from registers, and the first unit's group entry comes from them
    // too: one memory round trip before the first operand load for tables of up to
    // kEagerGroups groups (two beyond), where walking the table entry by entry costs one
    // round trip per group passed.  Reading only a few entries eagerly keeps the requests of
    // all waves at kernel start to a few cache lines.
    const int lane0 = threadIdx.x & 63;
    GroupArgs ent{};
    if (lane0 < kEagerGroups) ent = A.grp[lane0];
    // (used here together with the header, so that all of these reads are in flight at once)
    asm volatile("" ::"v"(ent.a), "v"(ent.b), "v"(ent.sfa), "v"(ent.sfb), "v"(ent.c), "v"(ent.m_shape), "v"(ent.n),
                 "v"(ent.k), "v"(ent.ldc), "s"(A.g), "s"(A.units), "s"(A.vq), "s"(A.flags));
    // tables of more groups: the rest of the entries, now that g is known
    if (lane0 >= kEagerGroups && lane0 < A.g) ent = A.grp[lane0];
    const int b = blockIdx.x;
    const unsigned V = 8u * (unsigned)A.vq, v = (unsigned)(b & 7) * (unsigned)A.vq + (unsigned)(b >> 3);
    // U v / V without 64-bit division: U = per V + rem, so U v / V = per v + rem v / V
    // (rem v < V^2 fits in 32 bits)
    const unsigned U = (unsigned)A.units, per = U / V, rem = U % V;
    const int u0 = (int)(per * v + rem * v / V), u1 = (int)(per * (v + 1) + rem * (v + 1) / V);
    const bool blocked = (A.flags & kFlagBlockedScales) != 0;
    if (u0 >= u1) return;
    const int g = A.g;
    // lane l < g: group l's shape word, columns and first unit past its units (the running
    // sum of the unit counts); lanes beyond g take no part
    const int ms_l = ent.m_shape, n_l = ent.n;
    int end_l = 0;
    {
        const int m = ms_l & kMMask, na = (ms_l >> kNaShift) & 15, nb = (ms_l >> kNbShift) & 31;
        const int cnt = lane0 < g && m > 0 ? ((m + 32 * na - 1) / (32 * na)) * ((n_l + 32 * nb - 1) / (32 * nb)) : 0;
        int sum = 0;
        for (int i = 0; i < g; ++i) {
            sum += __builtin_amdgcn_readlane(cnt, i);
            if (lane0 == i) end_l = sum;
        }
    }
    // unit u's group (the first whose units end beyond u; the ends never decrease) and tile
    const auto decode = [&](int u) {
        const int gi = __popcll(__ballot(lane0 < g && end_l <= u));
        const int gbase = gi > 0 ? __builtin_amdgcn_readlane(end_l, gi - 1) : 0;
        const int ms = __builtin_amdgcn_readlane(ms_l, gi), n = __builtin_amdgcn_readlane(n_l, gi);
        const int m = ms & kMMask;
        const int na = (ms >> kNaShift) & 15, nb = (ms >> kNbShift) & 31;
        const int rch = (m + 32 * na - 1) / (32 * na);
        const int l = u - gbase;
        const int rc = l % rch, ct = l / rch;
        const int row0 = rc * 32 * na, col0 = ct * 32 * nb;
        return Unit{gi, row0, min(32 * na, m - row0), col0, min(32 * nb, n - col0), na, nb};
    };
    const auto lane_ptr = [](const void* p, int i) {
        const unsigned long long x = (unsigned long long)p;
        return (unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)x, i) |
               (unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)(x >> 32), i) << 32;
    };
    Unit cu = decode(u0);
    // the first unit's group entry, from the lane that read it
    GroupArgs gcur;
    gcur.a = (const uint8_t*)lane_ptr(ent.a, cu.gi);
    gcur.b = (const uint8_t*)lane_ptr(ent.b, cu.gi);
    gcur.sfa = (const uint8_t*)lane_ptr(ent.sfa, cu.gi);
    gcur.sfb = (const uint8_t*)lane_ptr(ent.sfb, cu.gi);
    gcur.c = (uint16_t*)lane_ptr(ent.c, cu.gi);
    gcur.m_shape = __builtin_amdgcn_readlane(ent.m_shape, cu.gi);
    gcur.n = __builtin_amdgcn_readlane(ent.n, cu.gi);
    gcur.k = __builtin_amdgcn_readlane(ent.k, cu.gi);
    gcur.ldc = __builtin_amdgcn_readlane(ent.ldc, cu.gi);
    bool prefetched = false;
    for (int u = u0; u < u1; ++u) {
        const bool has_next = u + 1 < u1;
        const Unit nx = has_next ? decode(u + 1) : cu;
        const bool pf_next = has_next && nx.na == cu.na && nx.nb == cu.nb;
        switch ((cu.na << 8) | cu.nb) {
#define NVFP4GG_CASE(NA_, NB_) \
    case ((NA_) << 8) | (NB_): run_unit<NA_, NB_>(A, cu, gcur, prefetched, pf_next, nx, blocked, smem); break;
            NVFP4GG_UNIT_SHAPES(NVFP4GG_CASE)
#undef NVFP4GG_CASE
        default: break;
        }
        prefetched = pf_next;
        cu = nx;
        if (has_next) gcur = A.grp[cu.gi];
    }
}



hipError_t launch_units(const KernArgs& args, int grid, hipStream_t stream)
{
    if (grid <= 0) return hipSuccess;
    KernArgs a = args;
    void* params[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&nvfp4_gg_units), dim3(grid), dim3(gk::THREADS), params, 0,
                           stream);
}

bool unit_shape_supported(int na, int nb)
{
    switch ((na << 8) | nb) {
#define NVFP4GG_CASE(NA_, NB_) \
    case ((NA_) << 8) | (NB_): return true;
        NVFP4GG_UNIT_SHAPES(NVFP4GG_CASE)
#undef NVFP4GG_CASE
    default: return false;
    }
}

int unit_shape_slots(int na, int nb)
{
    switch ((na << 8) | nb) {
#define NVFP4GG_CASE(NA_, NB_) \
    case ((NA_) << 8) | (NB_): return gk::Geo<NA_, NB_>::SLOTS;
        NVFP4GG_UNIT_SHAPES(NVFP4GG_CASE)
#undef NVFP4GG_CASE
    default: return 0;
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
