/*
 * CPU oracle for the NVFP4 grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library; the product
 * (precision_moe_nvfp4_amd) never does, and shares no code with it.
 *
 * What it computes (the plain definition, written out):
 *
 *   C_i[r][c] = RNE_fp16( sum_{kk<k} a(r,kk) * sa(r,kk/16) * b(c,kk) * sb(c,kk/16) )
 *
 * for every group i, row r < m_i and column c < n, where a, b are FP4 E2M1
 * values and sa, sb are FP8 E4M3FN scale values, one per 16 consecutive K.
 *   - Each operand scaled by its own scale factors, then multiplied (the
 *     comment before the kernel launch), and the operand shapes a[m, k/2],
 *     b[n, k/2], sfa[m, k/16], sfb[n, k/16], c[m, n] fp16 (the custom_kernel
 *     docstring) are from the page "kernelindex submission 503584"; the data
 *     types (Float4E2M1FN data,
 *     Float8E4M3FN scales, 16 elements per scale, Float16 output) are that
 *     page's kernel configuration block.
 *   - The products are summed in fp64.  Every product is an integer multiple of
 *     2^-20 and, for the shapes used here, |partial sums| < 2^12, so every fp64
 *     sum is exact in any order; the single rounding to fp16 is round to nearest
 *     even, the rounding of the fp16 conversion in the epilogue_store function
 *     of the page "kernelindex submission 498317".
 *
 * Readings where the pages are silent (listed with the rest in the design notes):
 *   - E2M1 is the OCP Microscaling FP4 format (bias 1, no Inf/NaN).
 *   - E4M3FN is the OCP FP8 E4M3 format (bias 7, S.1111.111 is NaN, max 448).
 *   - Packing: two E2M1 codes per byte along K, low nibble = even K index.
 *   - Scales are row-major [rows][k/16] (the plain definition); the 128x4 blocked
 *     scale layout is an index permutation of it, written out in
 *     nvfp4_oracle_blocked_offset below.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* FP4 E2M1 (OCP MX): s | e1 e0 | m.  e == 0: m * 2^-1;  else 2^(e-1) * (1 + m/2). */
double nvfp4_oracle_e2m1(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* FP8 E4M3FN (OCP): s | E(4) | M(3), bias 7.  E == 15 && M == 7: NaN (no Inf).
 * E == 0: M * 2^-9 (subnormal);  else (1 + M/8) * 2^(E-7). */
double nvfp4_oracle_e4m3fn(unsigned code)
{
    unsigned s = (code >> 7) & 1u, E = (code >> 3) & 15u, M = code & 7u;
    if (E == 15u && M == 7u) return NAN;
    double mag = (E == 0) ? ldexp((double)M, -9) : ldexp(1.0 + (double)M / 8.0, (int)E - 7);
    return s ? -mag : mag;
}

/* Round a double to the nearest IEEE binary16 value, ties to even; returns the bits.
 * |x| beyond the largest finite half rounds to +-Inf as the IEEE rule says. */
uint16_t nvfp4_oracle_f16_rne(double x)
{
    if (isnan(x)) return 0x7E00u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a < ldexp(1.0, -14)) {
        /* subnormal (or zero): quantum 2^-24; 1024 quanta is the smallest normal */
        double q = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e;
    (void)frexp(a, &e);            /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                 /* a in [2^E, 2^(E+1)) */
    double q = nearbyint(ldexp(a, 10 - E));   /* significand with 10 fraction bits */
    if (q == 2048.0) { q = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* Element (row, kk) of a packed E2M1 matrix with k columns. */
static unsigned fp4_code_at(const uint8_t* rows, int k, long row, int kk)
{
    uint8_t byte = rows[row * (long)(k / 2) + kk / 2];
    return (kk & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 0x0F);
}

/* Dequantised operand row: value(kk) = e2m1(code) * e4m3fn(scale of block kk/16). */
static void dequant_row(const uint8_t* q, const uint8_t* sf, int k, long row, double* out)
{
    for (int kk = 0; kk < k; ++kk) {
        double v = nvfp4_oracle_e2m1(fp4_code_at(q, k, row, kk));
        double s = nvfp4_oracle_e4m3fn(sf[row * (long)(k / 16) + kk / 16]);
        out[kk] = v * s;
    }
}

/*
 * Grouped oracle.  For each group i: C[i] (fp16 bits, [m_i][n] row-major) and,
 * when non-null, exact[i] (the fp64 sum before rounding) and abssum[i]
 * (sum_k |a*sa*b*sb|, used for the tolerance).  nthreads <= 0: OpenMP default.
 * Returns 0, or -1 on an argument error.
 */
int nvfp4_oracle_grouped(int g, const int* m, int n, int k,
                         const uint8_t* const* A, const uint8_t* const* B,
                         const uint8_t* const* SFA, const uint8_t* const* SFB,
                         uint16_t* const* C, double* const* exact, double* const* abssum,
                         int nthreads)
{
    if (g < 0 || n < 0 || k < 0 || (k % 16) != 0 || !m || !A || !B || !SFA || !SFB || !C)
        return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (int i = 0; i < g; ++i) {
        const int mi = m[i];
        if (mi <= 0 || n == 0) continue;
        double* ad = (double*)malloc(sizeof(double) * (size_t)mi * (size_t)k);
        if (!ad) return -1;
        for (int r = 0; r < mi; ++r) dequant_row(A[i], SFA[i], k, r, ad + (size_t)r * k);
        int failed = 0;
#pragma omp parallel
        {
            double* bd = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
            if (!bd) {
#pragma omp atomic write
                failed = 1;
            }
#pragma omp for schedule(static)
            for (int c = 0; c < n; ++c) {
                if (!bd) continue;
                dequant_row(B[i], SFB[i], k, c, bd);
                for (int r = 0; r < mi; ++r) {
                    const double* ar = ad + (size_t)r * k;
                    double sum = 0.0, asum = 0.0;
                    for (int kk = 0; kk < k; ++kk) {
                        double p = ar[kk] * bd[kk];
                        sum += p;
                        asum += fabs(p);
                    }
                    size_t at = (size_t)r * (size_t)n + (size_t)c;
                    C[i][at] = nvfp4_oracle_f16_rne(sum);
                    if (exact && exact[i]) exact[i][at] = sum;
                    if (abssum && abssum[i]) abssum[i][at] = asum;
                }
            }
            free(bd);
        }
        free(ad);
        if (failed) return -1;
    }
    return 0;
}

/* Number of OpenMP threads the grouped oracle uses by default. */
int nvfp4_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * 128x4 blocked scale layout: byte offset of scale (row r, K block c = kk / 16) of a
 * scale matrix for K = k.
 *   - Atoms of 512 bytes are ordered row block (128 rows) major, K block of 64 values
 *     (4 scales) minor: atom (r / 128) * (k / 64) + c / 4.  This is the address of the
 *     SFA/SFB scale blocks in the producer branch of the kernel on the page "kernelindex
 *     submission 498317" (row offset / 128 times K / 16 / 4, plus K offset / 64, times 512).
 *   - Inside an atom, the row splits into (r % 32, (r / 32) % 4) with byte strides (16, 4)
 *     and the scale into (c % 4) with stride 1: the scale atom of the page "kernelindex
 *     submission 402102" (shape ((32, 4), (16, 4)), stride ((16, 4), (0, 1)), where the
 *     16 K values sharing a scale have stride 0).
 */
long nvfp4_oracle_blocked_offset(long r, long c, int k)
{
    const long atom = (r / 128) * (long)(k / 64) + c / 4;
    return atom * 512 + 16 * (r % 32) + 4 * ((r / 32) % 4) + (c % 4);
}

/* Bytes of the blocked layout for `rows` rows: whole 128-row blocks of k / 64 atoms. */
long nvfp4_oracle_blocked_bytes(long rows, int k)
{
    return rows <= 0 ? 0 : ((rows + 127) / 128) * (long)(k / 64) * 512;
}

/*
 * src [rows][k/16] row-major -> dst in the blocked layout; dst bytes that no (r, c) maps
 * to (the rows of the last block beyond `rows`) are set to `pad`.  Returns 0, or -1 on an
 * argument error (k must be a positive multiple of 64).
 */
int nvfp4_oracle_scales_to_blocked(uint8_t* dst, const uint8_t* src, long rows, int k, int pad)
{
    if (rows < 0 || k <= 0 || (k % 64) != 0 || (rows > 0 && (!dst || !src))) return -1;
    if (rows == 0) return 0;
    memset(dst, pad & 0xFF, (size_t)nvfp4_oracle_blocked_bytes(rows, k));
    const long cols = k / 16;
    for (long r = 0; r < rows; ++r)
        for (long c = 0; c < cols; ++c) dst[nvfp4_oracle_blocked_offset(r, c, k)] = src[r * cols + c];
    return 0;
}
