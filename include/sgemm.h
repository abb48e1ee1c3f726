/*
 * sgemm.h -- C ABI of the MI355X (gfx950) FP32 SGEMM library.
 *
 * The operation.  C = alpha * A * B + beta * C on row-major matrices: A is
 * M x K, B is K x N, C is M x N, alpha and beta are scalars, and alpha scales
 * the finished dot product once ("如何高效实现矩阵乘？CUDA初学者的角度入门",
 * section "樸素 GEMM 與前置知識", the naive GEMM with alpha and beta).
 * Element (r, c) of a matrix with leading dimension ld sits at r*ld + c
 * ("SGEMM CUDA kernel (Second Half)", Part 8, where the OFFSET(row, col, ld)
 * macro is used for every global access).  Partial tiles at the right and
 * bottom edges are handled by zero-filling out-of-range operand elements and
 * masking out-of-range stores ("3.3 Shared memory ו tiling תרגול", exercise 1,
 * zero padding of partial tiles).
 *
 * Precision.  Every product and every sum is an IEEE float32 operation (FMA
 * on the VALU path, v_mfma_f32_*_f32 on the matrix path); there is no
 * reduced-precision input rounding and no multi-pass emulation.  The
 * summation order differs from a sequential loop, so results match a float64
 * reference within |C - ref| <= 1e-5 * (|alpha| sum_k |A_ik||B_kj| +
 * |beta||C_ij|), not bit for bit.  A given variant (and split count) on
 * given inputs is deterministic run to run.
 *
 * Pointers.  A, B and C are DEVICE pointers owned by the caller.  The library
 * allocates no memory, copies nothing and keeps no handles (split-K takes a
 * caller-owned workspace, below).  Its only state is a per-device cache of
 * the machine shape (compute units and XCDs, sgemm_device_shape), read from
 * the device's attributes on first use; the choice of kernel depends on the
 * sizes and that shape only.  No alignment is required: 16-byte aligned bases with leading
 * dimensions and N that are multiples of 4 take 128-bit global accesses
 * (and K a multiple of 4 for the variants that read A 128 bits at a time);
 * other 4-byte aligned operands take 16-byte loads of A and B at 4-byte
 * alignment and 32-bit accesses to C on the K-ordered blocks; anything else
 * takes 32-bit ones (see sgemm_variant_access for the access modes).  C must not overlap A or B (undefined
 * behaviour).  Dimensions and leading dimensions are int; address arithmetic
 * is 64-bit.
 *
 * Asynchrony.  The kernel is enqueued on `stream` (0 = the null stream) and
 * the call returns without synchronising.  Faults inside the kernel (for
 * example a device pointer that does not cover the stated extent) surface at
 * the next synchronisation, not here.
 *
 * Special cases.  M == 0 or N == 0: nothing is launched, returns 0.
 * (alpha == 0 or K == 0) and beta == 1: nothing is launched, returns 0.
 * alpha == 0 or K == 0 otherwise: C = beta * C, with A and B not read.
 * beta == 0: C is not read (NaN or Inf already in C does not propagate).
 *
 * Return value.  0 on success.  Negative: an invalid argument, numbered by its
 * position in sgemm() (-1 M < 0, -2 N < 0, -3 K < 0, -5 A == NULL while
 * M*K > 0 and alpha != 0, -6 lda < max(1, K), -7 B == NULL while K*N > 0 and
 * alpha != 0, -8 ldb < max(1, N), -10 C == NULL while M*N > 0, -11
 * ldc < max(1, N)); -20 unknown path; -21 unknown variant; -22 the tile grid
 * does not fit one launch; -23 an unknown access mode, or one these arguments
 * do not allow; -24 a split-K or stream-K workspace that is missing, too
 * small or not 256-byte aligned; -25 a split count outside 1..64, a worker
 * count outside 1..4096, or a variant without a split-K (stream-K) build;
 * -26 a machine shape or tile grid out of range (sgemm_plan_for,
 * sgemm_tile_order); -27 a plan that needs more scratch than
 * sgemm_ws_noalloc's static buffer holds.  Argument checks run before any HIP call, so they
 * need no GPU.  Positive: the hipError_t reported for the launch.  The library
 * never exits or aborts the process.
 */
#ifndef SGEMM_MI355X_H
#define SGEMM_MI355X_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGEMM_PATH_AUTO 0 /* the library picks the inner product and tile */
#define SGEMM_PATH_VALU 1 /* FP32 FMA on the vector ALU, register outer product */
#define SGEMM_PATH_MFMA 2 /* v_mfma_f32_32x32x2_f32 matrix-core inner product */

/* How a kernel reaches global memory (sgemm_variant_access). */
#define SGEMM_ACCESS_AUTO 0       /* the library's choice, as sgemm_variant() */
#define SGEMM_ACCESS_BUFFER_128 1 /* range-checked buffer accesses, 128-bit on B and C (and A) */
#define SGEMM_ACCESS_BUFFER_32 2  /* range-checked buffer accesses, 32-bit */
#define SGEMM_ACCESS_CHECKED 3    /* per-element checked pointer accesses */
#define SGEMM_ACCESS_BUFFER_128_AB 4 /* 16-byte loads of A and B at 4-byte alignment, 32-bit C */

#define SGEMM_OK 0
#define SGEMM_ERR_PATH (-20)
#define SGEMM_ERR_VARIANT (-21)
#define SGEMM_ERR_TOO_LARGE (-22)
#define SGEMM_ERR_ACCESS (-23)
#define SGEMM_ERR_WORKSPACE (-24)
#define SGEMM_ERR_SPLITS (-25)
#define SGEMM_ERR_MACHINE (-26)
#define SGEMM_ERR_SCRATCH (-27)

/* C = alpha*A*B + beta*C, automatic choice of inner product and tile.  One
 * kernel launch, or two or three on the same stream when sgemm_select_rows()
 * is positive (C cut into pieces by sgemm_select_pieces(), each a whole
 * product of its own; nothing allocated, no order between the pieces'
 * results). */
int sgemm(int M, int N, int K, float alpha, const float *A, int lda,
          const float *B, int ldb, float beta, float *C, int ldc,
          hipStream_t stream);

/* As sgemm(), restricted to one inner product: SGEMM_PATH_AUTO, _VALU or _MFMA.
 * The tile is still chosen by shape.  Argument codes are sgemm()'s. */
int sgemm_path(int path, int M, int N, int K, float alpha, const float *A,
               int lda, const float *B, int ldb, float beta, float *C, int ldc,
               hipStream_t stream);

/* As sgemm(), with one compiled kernel variant (inner product + tile shape)
 * forced by index, 0 <= variant < sgemm_variant_count().  For tests and
 * benchmarks that must cover or time every variant. */
int sgemm_variant(int variant, int M, int N, int K, float alpha,
                  const float *A, int lda, const float *B, int ldb, float beta,
                  float *C, int ldc, hipStream_t stream);

/* As sgemm_variant(), with the global-memory access mode forced as well
 * (SGEMM_ACCESS_*).  Each variant is compiled three ways:
 *   BUFFER_128  raw buffer accesses whose descriptors end at each matrix's
 *               last element, so partial tiles need no branch; 128-bit on B
 *               and C.  Needs 16-byte aligned B and C, N, ldb and ldc
 *               multiples of 4, and byte offsets inside one block tile below
 *               2^31 (about (BM+1)*lda*4, (BK+1)*ldb*4 and (BM+1)*ldc*4).
 *               A variant for which sgemm_variant_reads_a128() is 1 also
 *               reads A 128 bits at a time along K in this mode, and needs a
 *               16-byte aligned A and K and lda multiples of 4 as well.
 *   BUFFER_32   the same with 32-bit accesses: any alignment.
 *   CHECKED     plain pointers with every element checked: any arguments.
 * and the K-ordered blocks (`_kcd`) once more:
 *   BUFFER_128_AB  16-byte loads of A and B at any 4-byte alignment (rows of
 *               any length and leading dimension; a 16-byte buffer load is
 *               range-checked per 4 bytes, so one that straddles a matrix's
 *               end keeps what lies inside, and the columns of A past K that
 *               a load brings along are cleared in LDS), 32-bit accesses to
 *               C.  Needs 4-byte aligned A, B and C and the in-tile offset
 *               bound above.
 * SGEMM_ACCESS_AUTO takes the first of BUFFER_128, BUFFER_128_AB, BUFFER_32
 * and CHECKED the arguments allow.  A forced
 * mode the arguments do not allow returns SGEMM_ERR_ACCESS.  The small
 * wave-group blocks (32 x 32 and 32 x 64 tiles) have no plain-pointer build:
 * their CHECKED build uses buffer accesses too, so with in-tile offsets of
 * 2^31 bytes or more every mode returns SGEMM_ERR_ACCESS for them.  For tests and
 * benchmarks that must cover every compiled kernel. */
int sgemm_variant_access(int variant, int access, int M, int N, int K,
                         float alpha, const float *A, int lda, const float *B,
                         int ldb, float beta, float *C, int ldc,
                         hipStream_t stream);

/* ---- split-K (for shapes too small to fill the chip with tiles) ----------
 * The K range is cut into `splits` parts.  A first launch has every (tile,
 * part) workgroup write its partial tile to the workspace; a second launch
 * on the same stream has one workgroup per tile sum the partials in part
 * order 0, 1, ..., splits-1 and apply alpha and beta ("如何高效实现矩阵乘？CUDA
 * 初学者的角度入门", section "Epilogue", names split-K for the long tail of
 * small shapes).  The order of the sum is fixed, so results are
 * deterministic run to run.
 *
 * Workspace: caller-owned device memory, 256-byte aligned, at least
 * sgemm_splitk_workspace_size() bytes, any contents.  Calls that share a
 * workspace must not overlap in time (same stream, or synchronised).  The
 * library allocates nothing. */

/* C = alpha*A*B + beta*C like sgemm(), using split-K or stream-K (below)
 * when the auto choice calls for it, the operands allow 16-byte loads
 * (sgemm_operands_load16) and `workspace_bytes` holds sgemm_workspace_size(M,
 * N, K); otherwise exactly sgemm(). */
int sgemm_ws(int M, int N, int K, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc,
             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- no allocation at all --------------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Exactly sgemm_ws() with enough workspace (the same plan and
 * kernels, so the same results bit for bit), with the split-K / stream-K
 * partial tiles kept in a static device array of the library,
 * SGEMM_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held from the first call on
 * that GPU until the process ends.  That covers every split-K plan and
 * stream-K on the 64 x 64 and 128 x 128 blocks; a plan that needs more
 * (stream-K on the 128 x 256 and 256 x 256 blocks of large squares, 64 and
 * 128 MiB) returns SGEMM_ERR_SCRATCH before any HIP call: use sgemm_ws() with
 * a workspace, or sgemm().  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine); its first call on a GPU looks the array's
 * address up once.  The array needs no clearing: a call writes every partial
 * tile it reads.  Calls on one GPU share the array, so calls that overlap in
 * time on one GPU (different streams, not ordered) race and give wrong
 * results; calls on one stream are ordered and safe. */
#define SGEMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int sgemm_ws_noalloc(int M, int N, int K, float alpha, const float *A, int lda,
                     const float *B, int ldb, float beta, float *C, int ldc,
                     hipStream_t stream);

/* Workspace bytes sgemm_ws() can use for these sizes (0: it never splits).
 * Only operands that allow 16-byte loads of A and B (sgemm_operands_load16)
 * split K or run stream-K: for others sgemm_ws() is exactly sgemm() (loading
 * 4 bytes per lane, split launches were slower than whole tiles). */
size_t sgemm_workspace_size(int M, int N, int K);

/* The plan queries below (sgemm_select_splits, sgemm_select_streamk,
 * sgemm_ws_plan, sgemm_select_variant, sgemm_select_rows) answer for
 * operands that allow 16-byte loads of A and B: A, B and C 4-byte aligned
 * and leading dimensions below about 2^24 (sgemm_operands_load16), however N,
 * K and the leading dimensions fall against multiples of 4.  Other operands
 * split nothing and
 * take neither small block (32 x 32, 32 x 64), so their plan may differ:
 * sgemm_select_variant_for() and sgemm_plan_for() answer for any operands. */

/* The split count sgemm_ws() uses with enough workspace (1: no split), or a
 * negative argument code.  Host logic only. */
int sgemm_select_splits(int M, int N, int K);

/* The stream-K worker count sgemm_ws() uses with enough workspace (0: no
 * stream-K), or a negative argument code.  Host logic only. */
int sgemm_select_streamk(int M, int N, int K);

/* What sgemm_ws() runs with enough workspace: the variant, the split count
 * (1: none) and the stream-K worker count (0: none), through the pointers
 * (each may be NULL).  Returns 0 or a negative argument code (-1..-3).
 * Host logic only. */
int sgemm_ws_plan(int M, int N, int K, int *variant, int *splits, int *workers);

/* One variant with a forced split count (1 = no split, same as
 * sgemm_variant()).  SGEMM_ERR_SPLITS for a variant without a split-K build;
 * SGEMM_ERR_ACCESS (split-K and stream-K alike) for operands that allow no
 * 16-byte loads of A and B: the split builds load 16 bytes at a time only. */
int sgemm_splitk(int variant, int splits, int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb, float beta,
                 float *C, int ldc, void *workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Workspace bytes sgemm_splitk(variant, splits, M, N, ...) needs (0 for
 * splits == 1, an empty C, or invalid arguments). */
size_t sgemm_splitk_workspace_size(int variant, int splits, int M, int N);

/* ---- stream-K (for shapes whose last round of tiles leaves slots idle) ---
 * With T tiles and W workers, the first T - (T mod W) tiles (whole rounds)
 * are computed whole, and the K tiles of the remaining R = T mod W tiles,
 * R * ceil(K / BK) in all, are shared by the W workers in equal contiguous
 * ranges: worker w takes [w I / W, (w + 1) I / W) with I = R ceil(K / BK),
 * in tile order.  A range is shorter than one tile, so a worker holds at
 * most the end of one tile and the start of the next; it writes each as a
 * partial tile to the workspace, or, when it holds a whole tile, C itself.
 * A second launch on the same stream sums each shared tile's partials in
 * worker order and applies alpha and beta, so results are deterministic run
 * to run.  No atomics, flags or waits between workgroups.  R = 0 (whole
 * rounds) is an ordinary launch.
 *
 * Workspace: caller-owned device memory, 256-byte aligned, at least
 * sgemm_streamk_workspace_size() bytes, any contents; the same sharing rule
 * as split-K. */

/* One variant with stream-K over `workers` workers (1 .. 4096; one per
 * workgroup slot of the chip fills it evenly).  SGEMM_ERR_SPLITS for a
 * worker count out of range or a variant without stream-K. */
int sgemm_streamk(int variant, int workers, int M, int N, int K, float alpha,
                  const float *A, int lda, const float *B, int ldb, float beta,
                  float *C, int ldc, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* Workspace bytes sgemm_streamk(variant, workers, ...) needs (0 for a
 * variant without stream-K or a worker count out of range): two partial
 * tiles per worker. */
size_t sgemm_streamk_workspace_size(int variant, int workers);

/* Number of compiled kernel variants. */
int sgemm_variant_count(void);

/* The builds a variant has, as a bit mask (SGEMM_BUILD_*), or
 * SGEMM_ERR_VARIANT.  CHECKED is set only where that build uses plain
 * pointers (any leading dimension).  Host logic only. */
#define SGEMM_BUILD_BUFFER_128 1
#define SGEMM_BUILD_BUFFER_32 2
#define SGEMM_BUILD_CHECKED 4
#define SGEMM_BUILD_BUFFER_128_AB 8
#define SGEMM_BUILD_SPLITK 16
#define SGEMM_BUILD_STREAMK 32
int sgemm_variant_builds(int variant);

/* Static, NUL-terminated name of a variant ("mfma_256x256x32_w128x128" ...),
 * or NULL for an index out of range. */
const char *sgemm_variant_name(int variant);

/* SGEMM_PATH_VALU or SGEMM_PATH_MFMA for a variant, SGEMM_ERR_VARIANT if out of range. */
int sgemm_variant_path(int variant);

/* Block tile (rows, columns of C) of a variant through *bm and *bn; returns 0
 * or SGEMM_ERR_VARIANT.  Either pointer may be NULL. */
int sgemm_variant_tile(int variant, int *bm, int *bn);

/* 1 if the variant's SGEMM_ACCESS_BUFFER_128 build reads A 128 bits at a time
 * along K (so that mode also needs K, lda multiples of 4 and A 16-byte
 * aligned), 0 if it reads A 32 bits at a time, SGEMM_ERR_VARIANT if out of
 * range.  Host logic only. */
int sgemm_variant_reads_a128(int variant);

/* The variant sgemm_path(path, M, N, K, ...) launches for these sizes with
 * operands that allow 16-byte loads (above), or a negative code (-1..-3,
 * SGEMM_ERR_PATH).  Host logic only, no HIP call.  When sgemm_select_rows()
 * is positive, an AUTO or MFMA call cuts C into pieces instead (below). */
int sgemm_select_variant(int path, int M, int N, int K);

/* The same for these operands: the pointers and leading dimensions decide
 * whether 16-byte loads are possible (the pointers are only inspected for
 * alignment, never dereferenced; they may be NULL where sgemm() allows it).
 * Host logic only. */
int sgemm_select_variant_for(int path, int M, int N, int K, const float *A, int lda,
                             const float *B, int ldb, const float *C, int ldc);

/* 1 if these operands allow 16-byte loads of A and B, which the small
 * blocks, split-K and stream-K need (A, B and C 4-byte aligned; leading
 * dimensions below about 2^24, so that in-tile byte offsets fit 31 bits),
 * else 0: the operands_load16 argument of sgemm_plan_for() that describes
 * them.  The pointers are only inspected.  Host logic only. */
int sgemm_operands_load16(const float *A, int lda, const float *B, int ldb, const float *C, int ldc);

/* How sgemm() (path AUTO or MFMA), and sgemm_ws() when it neither splits
 * K nor runs stream-K, cut C into pieces, one launch each, so that the first
 * piece's tiles fill their rounds of the device's compute units: through
 * *rows, *cols and *first_variant (each may be NULL) the first piece, C's
 * rows [0, rows) and columns [0, cols), and the variant it runs on (a block
 * of one workgroup per CU: 256 x 256, or 128 x 256 or 128 x 128 where the
 * 256 x 256 block gives no cut), or rows = 0 (and first_variant -1) for one
 * launch.  rows is a multiple of the block's rows up to M; cols is N (a cut
 * by rows alone) or a multiple of the block's columns below N.  After the
 * first piece come, when cols < N, the columns
 * [cols, N) of the same rows (with the variant
 * sgemm_select_variant(AUTO, rows, N - cols, K)), then, when rows < M, the
 * rows [rows, M) over all N columns (sgemm_select_variant(AUTO, M - rows, N,
 * K)).  Returns 0 or a negative argument code (-1..-3).  Host logic only.
 * (Quantisation of tiles over the compute units: "如何高效实现矩阵乘？CUDA
 * 初学者的角度入门", section "Wave & L2 cache Hit Rate".) */
int sgemm_select_pieces(int M, int N, int K, int *rows, int *cols, int *first_variant);

/* The rows of sgemm_select_pieces()'s first piece (0: one launch), or a
 * negative argument code (-1..-3).  Host logic only. */
int sgemm_select_rows(int M, int N, int K);

/* The machine shape the current device's choices use: its compute units and
 * XCDs, read once per device from hipDeviceAttributeMultiprocessorCount and
 * hipDeviceAttributeNumberOfXccs (256 and 8, an MI355X, when no device can
 * be queried, so the host-only queries above answer without a GPU; an XCD
 * count that is not a power of two is taken as 1).  Either
 * pointer may be NULL.  Returns 0.  (Tile quantisation over the compute
 * units and the XCDs' separate L2 caches: "如何高效实现矩阵乘？CUDA初学者的角度
 * 入门", section "Wave & L2 cache Hit Rate".) */
int sgemm_device_shape(int *compute_units, int *xcds);

/* The plan the library makes for these sizes on a device of
 * `compute_units` compute units: with with_workspace != 0 what sgemm_ws()
 * runs with enough workspace, else what sgemm() runs; operands_load16 != 0
 * for operands that allow 16-byte loads (above), 0 for others.  Through
 * the pointers (each may be NULL): the variant, the split count (1: none),
 * the stream-K worker count (0: none) and the rows of the first piece when
 * C is cut into pieces (sgemm_select_pieces(); 0: one launch).  Returns 0, a
 * negative argument code (-1..-3 for M, N, K), or SGEMM_ERR_MACHINE for
 * compute_units outside 1..2^20.  Host logic only. */
int sgemm_plan_for(int compute_units, int M, int N, int K, int with_workspace, int operands_load16,
                   int *variant, int *splits, int *workers, int *rows);

/* sgemm_plan_for() that also gives the first piece's columns through *cols
 * (N for a cut by rows alone, 0 with rows = 0) and its variant through
 * *first_variant (-1 with rows = 0); either may be NULL. */
int sgemm_plan_pieces_for(int compute_units, int M, int N, int K, int with_workspace,
                          int operands_load16, int *variant, int *splits, int *workers, int *rows,
                          int *cols, int *first_variant);

/* The workgroup -> tile order of the K-ordered blocks on a device of `xcds`
 * XCDs, for a grid of nbm x nbn tiles: workgroup p computes tile
 * (tile_m[p], tile_n[p]).  The arrays hold nbm * nbn ints each (caller-owned
 * host memory; may be NULL when the grid is empty).  Returns 0 or
 * SGEMM_ERR_MACHINE (xcds not a power of two in 1..1024, a negative or too
 * large grid, NULL arrays).
 * Host logic only.  (Block order and L2 locality: "如何高效实现矩阵乘？CUDA
 * 初学者的角度入门", section "Wave & L2 cache Hit Rate".) */
int sgemm_tile_order(int xcds, int nbm, int nbn, int *tile_m, int *tile_n);

/* Static text for a status code returned by any entry point above. */
const char *sgemm_status_string(int status);

/* The FP32 peak of a device from its properties: compute units x 256 FLOP per
 * clock (4 SIMDs, each one v_mfma_f32_32x32x2_f32 = 4096 FLOP per 64 cycles,
 * which is also the FP32 vector FMA rate) x the peak engine clock.  Any output
 * pointer may be NULL.  Returns 0 or the hipError_t of the property query.
 * For reports that state the peak they divide by. */
int sgemm_device_fp32_peak(int device, int *compute_units, int *clock_khz, double *tflops);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_MI355X_H */
