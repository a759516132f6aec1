/*
 * nvfp4_gg.h -- C ABI of the MI355X (gfx950) NVFP4 grouped GEMM.
 *
 * Operation (per group i = 0..g-1):
 *
 *   C_i[m_i x n] (fp16) = dequant(A_i[m_i x k]) * dequant(B_i[n x k])^T,  fp32 accumulation,
 *
 * where dequant(X)[r][kk] = e2m1(X[r][kk]) * e4m3fn(SFX[r][kk / 16]).  This is the
 * operation of the leaderboard task nvfp4_group_gemm: the custom_kernel docstring of the
 * page "kernelindex submission 503584" gives the operands (a[m, k/2] and b[n, k/2] of
 * packed FP4 E2M1 codes, sfa[m, k/16] and sfb[n, k/16] of FP8 E4M3 scales, c[m, n] fp16,
 * one (m, n, k) problem per group), its kernel configuration block the data types
 * (Float4E2M1FN, Float8E4M3FN, 16 elements per scale, Float16 output, Float32
 * accumulator), and the comment before its kernel launch states that each operand is
 * multiplied by its own scale factors before the product is formed.
 * Output rounding is round-to-nearest-even, as in the epilogue_store function of the page
 * "kernelindex submission 498317".
 *
 * Data layout (all row-major, no batch dimension):
 *   A_i   [m_i][k/2] bytes: two E2M1 codes per byte along K, low nibble = even K index.
 *   B_i   [n  ][k/2] bytes: same packing.
 *   SFA_i [m_i][k/16] bytes: E4M3FN codes (finite; 0x7F/0xFF are NaN and not supported).
 *   SFB_i [n  ][k/16] bytes: E4M3FN codes.
 *   C_i   [m_i][n] fp16 (IEEE binary16).
 * n and k are the same for every group; m_i varies (m_i = 0 is allowed and writes nothing).
 *
 * Ownership: the caller owns every device buffer it passes.  A plan owns host memory only:
 * its schedule travels in the kernel arguments of every call, so nvfp4_gg_plan allocates
 * nothing on a device and nvfp4_gg_destroy performs no device work (no synchronisation).
 * Asynchrony: nvfp4_gg_run only enqueues work on the given stream; it never synchronises,
 * allocates memory, prints or throws.  A call captured into a HIP graph carries everything
 * it needs in its kernel node, so the graph stays valid after the plan is destroyed.
 * Threading: a plan is immutable after nvfp4_gg_plan returns; several threads may call
 * nvfp4_gg_run on one plan concurrently.  Distinct plans are independent.
 * Errors: every entry point returns a status code; nothing is thrown across this ABI.
 */
#ifndef NVFP4_GG_H
#define NVFP4_GG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest number of groups one plan accepts: the whole per-group table travels in the
 * kernel arguments (no device allocation, no host-to-device copy per call). */
#define NVFP4_GG_MAX_GROUPS 64

/* Pass as `device` to nvfp4_gg_plan to build a plan for a nominal MI355X (256 compute
 * units) without touching the HIP runtime.  Such a plan can be inspected with
 * nvfp4_gg_plan_info but nvfp4_gg_run rejects it with NVFP4_GG_EUNSUPPORTED. */
#define NVFP4_GG_DEVICE_NONE (-2)

typedef enum {
    NVFP4_GG_OK = 0,
    NVFP4_GG_EINVAL = 1,       /* bad argument: null pointer, bad size, unknown plan */
    NVFP4_GG_EALIGN = 2,       /* a device pointer is not 16-byte aligned */
    NVFP4_GG_ENOMEM = 3,       /* host allocation failed */
    NVFP4_GG_EHIP = 4,         /* a HIP runtime call failed (device query or launch) */
    NVFP4_GG_EUNSUPPORTED = 5  /* device is not gfx950, g too large, or a host-only plan */
} nvfp4_gg_status_t;

typedef struct nvfp4_gg_plan_s* nvfp4_gg_plan_t;

/*
 * Layout of the scale tensors SFA_i and SFB_i.
 *
 * NVFP4_GG_SCALES_ROW_MAJOR: [rows][k/16] bytes (the sfa/sfb operands of the custom_kernel
 * docstring on the page "kernelindex submission 503584").
 *
 * NVFP4_GG_SCALES_BLOCKED: the pre-arranged layout the kernels on the pages consume
 * (their sfasfb_reordered tensors).  The scales are stored in 512-byte atoms, each holding
 * 128 rows x 4 consecutive K blocks (64 K values).  Scale (row r, K block c = kk / 16) is
 * at byte
 *     ((r / 128) * (k / 64) + c / 4) * 512  +  16 * (r % 32) + 4 * ((r / 32) % 4) + c % 4.
 * The atom order (row block major, K block of 64 minor, 512 bytes each) is the scale-block
 * address arithmetic of the B and SFA/SFB producer in "kernelindex submission 498317"; the
 * arrangement inside an atom is the scale atom of "kernelindex submission 402102" (shape
 * (32, 4) rows x (16, 4) K with strides (16, 4) and (0, 1)).  A tensor for `rows` rows
 * holds nvfp4_gg_blocked_scale_bytes(rows, k) bytes: rows are padded to a multiple of 128;
 * padding bytes are never read by nvfp4_gg_run.
 */
typedef enum {
    NVFP4_GG_SCALES_ROW_MAJOR = 0,
    NVFP4_GG_SCALES_BLOCKED = 1
} nvfp4_gg_scale_layout_t;

/*
 * One problem of a grouped call with its own sizes (nvfp4_gg_plan_problems): the custom_kernel
 * of "kernelindex submission 503584" takes one (m, n, k, l) per group, and its kernel
 * addresses C through per-group strides.
 *   m   rows of A_i and C_i (0 <= m <= 2^20; 0: nothing is read or written for the group)
 *   n   rows of B_i and columns of C_i (1 <= n <= 2^20)
 *   k   K of the group (64 <= k <= 2^20, k % 64 == 0)
 *   ldc elements between the starts of consecutive rows of C_i: 0 means n, otherwise >= n;
 *       the elements of a row beyond column n are never written
 */
typedef struct {
    int m, n, k, ldc;
} nvfp4_gg_problem_t;

/* What a plan decided; filled by nvfp4_gg_plan_info.  A work unit is up to unit_rows[p]
 * rows of the group at schedule position p times unit_cols[p] columns, over its whole K. */
typedef struct {
    int g, n, k;           /* n and k shared by every group, or 0 where they differ */
    int device;            /* HIP device ordinal, or NVFP4_GG_DEVICE_NONE */
    int num_cus;           /* compute units the schedule was sized for */
    int tile_m, tile_n;    /* largest unit of the plan (rows, columns) */
    int total_tiles;       /* work units over all groups */
    int grid;              /* workgroups launched per call */
    int block;             /* threads per workgroup */
    int lds_bytes;         /* LDS per workgroup */
    int variant;           /* kernel variant id: 5 row-major scales, 6 blocked scales */
    int order[NVFP4_GG_MAX_GROUPS];       /* group processed at schedule position p */
    int tile_begin[NVFP4_GG_MAX_GROUPS + 1]; /* exclusive unit prefix in schedule order */
    int scale_layout;      /* nvfp4_gg_scale_layout_t the plan's runs read */
    int unit_rows[NVFP4_GG_MAX_GROUPS];   /* unit height at schedule position p (0: m = 0) */
    int unit_cols[NVFP4_GG_MAX_GROUPS];   /* unit width at schedule position p */
    double est_us;         /* the planner's cost-model estimate of one call (microseconds) */
} nvfp4_gg_plan_info_t;

/*
 * Build a plan for g groups with row counts m[0..g-1] (host array, copied), and shared
 * n and k: validation, the largest-work-first group order and its per-group unit counts
 * and prefix sum (the host planning of custom_kernel on the page "kernelindex submission
 * 503584": groups sorted by tile work, prefix of per-group tile counts), and each group's
 * unit shape, chosen by a cost model so that the persistent grid's contiguous shares of
 * the unit sequence take about the same time.  Host work only: nothing is allocated on
 * or copied to a device.  Plans are meant to be built once per shape and reused.
 *   device: HIP device ordinal, -1 for the current device, or NVFP4_GG_DEVICE_NONE (host
 *   only: the HIP runtime is not touched).
 * Requirements: 1 <= g <= NVFP4_GG_MAX_GROUPS, 1 <= n <= 2^20, 64 <= k <= 2^20 and
 * k % 64 == 0, 0 <= m_i <= 2^20; else NVFP4_GG_EINVAL (g above the maximum:
 * NVFP4_GG_EUNSUPPORTED).  (The group_gemm host function of "kernelindex submission
 * 498317" requires k % 256 == 0; here K values beyond the last multiple of 256 are handled
 * by a shorter last K step, so every multiple of 64 is accepted.)  A device that is not
 * gfx950: NVFP4_GG_EUNSUPPORTED.  Host allocation failure: NVFP4_GG_ENOMEM.
 * On success *out holds a new plan, released with nvfp4_gg_destroy; on failure *out = NULL.
 * Diagnostics: if the environment variable NVFP4_GG_FORCE_SHAPE holds "na,nb" naming a
 * compiled unit shape (32 na rows x 32 nb columns), every group of the plan uses it instead
 * of the planner's choice (for tests and measurements; results are the same, only the
 * schedule differs).
 */
nvfp4_gg_status_t nvfp4_gg_plan(nvfp4_gg_plan_t* out, int g, const int* m, int n, int k,
                                int device);

/*
 * nvfp4_gg_plan for scale tensors in `scale_layout` (an nvfp4_gg_scale_layout_t; any other
 * value: NVFP4_GG_EINVAL).  nvfp4_gg_plan(...) is nvfp4_gg_plan_layout(...,
 * NVFP4_GG_SCALES_ROW_MAJOR).  With NVFP4_GG_SCALES_BLOCKED, each SFA_i passed to
 * nvfp4_gg_run must hold nvfp4_gg_blocked_scale_bytes(m_i, k) bytes and each SFB_i
 * nvfp4_gg_blocked_scale_bytes(n, k) bytes; everything else is as for nvfp4_gg_run.
 */
nvfp4_gg_status_t nvfp4_gg_plan_layout(nvfp4_gg_plan_t* out, int g, const int* m, int n, int k,
                                       int device, int scale_layout);

/*
 * The general plan: group i has its own sizes problems[i] (host array of g, copied; see
 * nvfp4_gg_problem_t for the limits, NVFP4_GG_EINVAL outside them) and the operand shapes
 * of group i are A_i [m][k/2], B_i [n][k/2], SFA_i [m][k/16] and SFB_i [n][k/16] (or their
 * blocked-layout sizes for NVFP4_GG_SCALES_BLOCKED), C_i rows of ldc (or n) fp16 elements.
 * Everything else is as nvfp4_gg_plan_layout; nvfp4_gg_plan_layout(out, g, m, n, k, device,
 * layout) is this call with problems[i] = {m[i], n, k, 0}.  With a nonzero ldc the row starts
 * of C_i must stay 2-byte aligned; 8-byte stores are used when ldc % 4 == 0.
 */
nvfp4_gg_status_t nvfp4_gg_plan_problems(nvfp4_gg_plan_t* out, int g, const nvfp4_gg_problem_t* problems,
                                         int device, int scale_layout);

/* Bytes of a NVFP4_GG_SCALES_BLOCKED scale tensor with `rows` rows (0 if rows <= 0 or
 * k is not a positive multiple of 64). */
size_t nvfp4_gg_blocked_scale_bytes(int rows, int k);

/*
 * Enqueue on `stream` (0 = null stream of the current device) the conversion of one
 * row-major scale tensor src[rows][k/16] into the NVFP4_GG_SCALES_BLOCKED layout at dst
 * (nvfp4_gg_blocked_scale_bytes(rows, k) bytes, every one written; padding rows are
 * written as zero).  Both are device pointers of the current device, 16-byte aligned
 * (else NVFP4_GG_EALIGN), non-null for rows > 0, not overlapping (else undefined).
 * rows = 0 does nothing.  Requirements: 0 <= rows <= 2^20, 64 <= k <= 2^20, k % 64 == 0,
 * else NVFP4_GG_EINVAL.  A failed launch returns NVFP4_GG_EHIP.  Asynchronous, like
 * nvfp4_gg_run; it allocates nothing.
 */
nvfp4_gg_status_t nvfp4_gg_scales_to_blocked(void* dst, const void* src, int rows, int k,
                                             hipStream_t stream);

/*
 * Enqueue one grouped GEMM on `stream` (0 = the null stream of the plan's device).
 * A, B, SFA, SFB, C: host arrays of g device pointers (read before returning; the caller
 * may reuse the arrays at once), in the caller's group order.  Every pointer of a group
 * with m_i > 0 must be non-null (else NVFP4_GG_EINVAL) and 16-byte aligned (else
 * NVFP4_GG_EALIGN); pointers of groups with m_i = 0 are ignored.  C must not overlap any
 * input.  Each element of every C_i[m_i x n] is written exactly once; nothing else is
 * written and C is never read.  The current HIP device must be the plan's device
 * (else NVFP4_GG_EINVAL).  A failed launch returns NVFP4_GG_EHIP.
 */
nvfp4_gg_status_t nvfp4_gg_run(nvfp4_gg_plan_t plan,
                               const void* const* A, const void* const* B,
                               const void* const* SFA, const void* const* SFB,
                               void* const* C, hipStream_t stream);

/* Copy the plan's decisions into *info.  NVFP4_GG_EINVAL on a null argument. */
nvfp4_gg_status_t nvfp4_gg_plan_info(nvfp4_gg_plan_t plan, nvfp4_gg_plan_info_t* info);

/* Release a plan's host memory (NULL is ignored).  No device work and no synchronisation:
 * calls already enqueued with the plan, and graphs that captured them, do not read it. */
void nvfp4_gg_destroy(nvfp4_gg_plan_t plan);

/* Static English text for a status code; never NULL. */
const char* nvfp4_gg_status_string(nvfp4_gg_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_GG_H */
