/*
 * pgemm -- dense matrix multiply C <- alpha*A*B + beta*C for AMD Instinct
 * MI355X (gfx950), fp32 and fp64, column-major with leading dimensions.
 *
 * Plain C ABI: device pointers, sizes, scalars and an opaque HIP stream.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Column-major, neither operand transposed, as in the SGEMM study
 *   "optimizing-sgemm-on-nvidia-turing-gpus" (introduction).  Element (i, j)
 *   of a matrix X with leading dimension ldx is X[i + j*ldx].  A is m x k,
 *   B is k x n, C is m x n.  Only the logical block of C is written; its
 *   padding rows (between the logical extent and the leading dimension) are
 *   never written.  A column of A other than the last may be read up to
 *   the next 16-byte boundary past row m-1 (whole 16-byte loads at the edge
 *   of the block; with lda < m rounded up to 16 bytes this reaches the first
 *   rows of the next column).  Those values never reach C, and every read
 *   stays inside the (k-1)*lda + m elements of A.  Nothing else outside the
 *   logical blocks is read.
 * Memory.  A, B, C are DEVICE pointers on the current HIP device, owned by
 *   the caller (matmat_f64_host alone takes host pointers).  The library
 *   allocates nothing per call and keeps no state besides read-only kernel
 *   code, a per-device compute-unit count and, for gemm_f32_noalloc alone, a
 *   fixed scratch array per device; the scratch memory of every other entry
 *   point that uses any is a caller workspace.  C must not overlap A or B; A
 *   may equal B.
 * Stream.  `stream` is a hipStream_t passed as void*; NULL means the default
 *   stream.  Every call is stream-ordered and asynchronous: it returns after
 *   enqueueing work; the caller synchronizes (matmat_f64_host alone returns
 *   after its result is back in host memory).
 * Semantics (BLAS convention where the pages are silent).
 *   m == 0 or n == 0: nothing is touched, returns 0.
 *   k == 0 or alpha == 0: C <- beta*C; A and B are not read (may be NULL).
 *   beta == 0: C is write-only (NaN or Inf already in C does not propagate).
 * Accuracy.  Products and sums are formed in the working precision (fp32 or
 *   fp64) by matrix-core multiply-accumulate; the summation order differs
 *   from a sequential loop, so results are not bitwise equal to one, but a
 *   given build is deterministic: identical inputs give identical bits.
 * Errors.  Returns 0 on success.  An invalid argument returns -p, where p is
 *   the 1-based position of the first offending argument in the signature
 *   (e.g. -6 for a bad lda in gemm_f32).  A failed kernel launch (or copy)
 *   returns PGEMM_EHIP.  Nothing aborts and nothing prints.  Argument checking
 *   happens before any HIP call.
 */
#ifndef PGEMM_H
#define PGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PGEMM_OK 0
#define PGEMM_EHIP (-100)      /* a HIP launch, copy or synchronization failed */
#define PGEMM_EVARIANT (-101)  /* unknown kernel variant id */
#define PGEMM_ESCRATCH (-102)  /* the shape needs more than PGEMM_SCRATCH_BYTES of scratch */

/* Size of the library-owned scratch array of gemm_f32_noalloc, per device. */
#define PGEMM_SCRATCH_BYTES (32u << 20)

/*
 * Single precision.  C(m x n) <- alpha * A(m x k) * B(k x n) + beta * C.
 *
 *   m, n, k >= 0                       (arguments 1, 2, 3)
 *   A: lda >= max(1, m)                (arguments 5, 6)
 *   B: ldb >= max(1, k)                (arguments 7, 8)
 *   C: ldc >= max(1, m)                (arguments 10, 11)
 *   A, B may be NULL only if k == 0 or alpha == 0; C only if m == 0 or n == 0.
 *
 * Any leading dimension and any 4-byte-aligned pointer is accepted.  Global
 * memory is moved in 16-byte accesses either way (gfx950 needs only dword
 * alignment for them); 16-byte aligned pointers with leading dimensions that
 * are multiples of 4 select kernels that also assume that alignment.  The
 * tile size is chosen per call from the shape; when only a few rows (at most
 * 8) lie below the last whole row of tiles, a second kernel may compute them
 * (both kernels are launched on `stream`).  Leading dimensions so large
 * that one tile's columns span 2 GiB (about ldb >= 2^21 or lda >= 2^24
 * elements) take a slower loading path with 64-bit addresses; the results
 * are the same.
 */
int gemm_f32(int m, int n, int k, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc,
             void *stream);

/*
 * Double precision, same contract as gemm_f32 with 8-byte elements
 * (pointers 8-byte aligned; the aligned kernels need 16-byte pointers and
 * even leading dimensions).
 */
int gemm_f64(int m, int n, int k, double alpha, const double *A, int lda,
             const double *B, int ldb, double beta, double *C, int ldc,
             void *stream);

/*
 * The lecture's double-precision matmat interface ("HPC - Lecture 13 -
 * MatMat GPU", section "function matmatgpu1"), on device pointers:
 * ROW-major A (N1 x N2), B (N2 x N3), C (N1 x N3), row i of X starting at
 * X + i*ldx, and C <- C + A*B (alpha = beta = 1, as the lecture's kernel
 * starts each dot product from the old C value).
 *
 * A row-major matrix is the column-major storage of its transpose, so this is
 * gemm_f64(N3, N1, N2, 1, B, ldb, A, lda, 1, C, ldc, stream): no data moves.
 *   lda >= max(1, N2), ldb >= max(1, N3), ldc >= max(1, N3)   (args 1, 2, 3)
 *   N1, N2, N3 >= 0                                            (args 7, 8, 9)
 * Error codes refer to this signature's argument positions.
 */
int matmat_f64(int lda, int ldb, int ldc, const double *A, const double *B,
               double *C, int N1, int N2, int N3, void *stream);

/*
 * Same as gemm_f32 / gemm_f64, with a caller-provided device workspace that
 * lets the library balance the last, partly filled round of tiles by
 * stream-K: the tiles of the full rounds run one per workgroup as in
 * gemm_f32, while the K iterations of the remaining tiles are shared evenly
 * by up to one more workgroup per compute unit.  Each such workgroup writes
 * the partial sums of its range (the end of one tile and the start of the
 * next at most) to the workspace, and a second kernel adds each tile's
 * pieces, always in K order, and applies alpha and beta.  The library uses
 * it only where its model of the kernel estimates a gain; the tile size may
 * then differ from gemm_f32's for the same shape.  Results stay
 * deterministic (identical inputs give identical bits) but are not bitwise
 * equal to gemm_f32's, whose summation order differs.
 *
 *   workspace        device pointer, 16-byte aligned (argument 12), or NULL
 *   workspace_bytes  its size; pgemm_workspace_f32/f64(m, n, k) returns the
 *                    size this shape can use (0 when stream-K does not
 *                    apply): two tiles of partial sums per stream-K
 *                    workgroup, at most 32 MiB (fp32) or 64 MiB (fp64) on
 *                    256 compute units
 * With NULL or a smaller workspace the call behaves exactly like gemm_f32.
 * The workspace is scratch owned by the caller; calls that share one
 * workspace must be ordered (e.g. on one stream).
 */
int gemm_f32_ws(int m, int n, int k, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc,
                void *workspace, size_t workspace_bytes, void *stream);
int gemm_f64_ws(int m, int n, int k, double alpha, const double *A, int lda,
                const double *B, int ldb, double beta, double *C, int ldc,
                void *workspace, size_t workspace_bytes, void *stream);
size_t pgemm_workspace_f32(int m, int n, int k);
size_t pgemm_workspace_f64(int m, int n, int k);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * contract and same result bits as gemm_f32_ws given a workspace of
 * pgemm_workspace_f32(m, n, k) bytes, but the stream-K partial sums go to a
 * scratch array that the library itself holds in device memory: a
 * file-scope array of PGEMM_SCRATCH_BYTES (32 MiB) per device, reserved
 * when the library's code is loaded on that device and kept until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller passes A, B and C as for
 * gemm_f32.
 *
 *   returns PGEMM_ESCRATCH, before any launch, if the shape's stream-K
 *   workspace would exceed PGEMM_SCRATCH_BYTES (it never does on a device of
 *   up to 256 compute units: the largest plan there is 2 x 256 tiles of
 *   128 x 128 fp32 partial sums, exactly 32 MiB); PGEMM_EHIP if the array's
 *   device address cannot be obtained.
 *
 * Every call on one device shares that device's array, which keeps the last
 * call's contents; no part of it needs to start at zero (each partial sum is
 * written before the fix-up kernel reads it).  Calls on one device must
 * therefore be ordered (e.g. issued on one stream): two calls that overlap
 * on one device race on the array and may return wrong results.
 */
int gemm_f32_noalloc(int m, int n, int k, float alpha, const float *A, int lda,
                     const float *B, int ldb, float beta, float *C, int ldc,
                     void *stream);

/*
 * The lecture's matmat on HOST memory ("HPC - Lecture 13 - MatMat GPU",
 * section "function matmatgpu1": A, B, C start in host memory, go to the
 * device, the kernel runs, C comes back).  Same arguments and meaning as
 * matmat_f64 (row-major, C <- C + A*B), but A, B, C are host pointers, plus
 * a caller-owned DEVICE workspace that receives copies of the three
 * matrices with the same leading dimensions:
 *   workspace        device pointer, 16-byte aligned            (argument 10)
 *   workspace_bytes  at least pgemm_matmat_host_workspace(lda, ldb, ldc,
 *                    N1, N2, N3)                                (argument 11)
 * Each operand moves as one flat copy of its strided block (the padding
 * between rows is read but never used; flat copies are much faster than
 * pitched ones from pageable memory), the product runs as matmat_f64 on the
 * workspace copies, and C's N1 x N3 block comes back (row by row when ldc >
 * N3: the padding of C is never written).  The call returns after C is back
 * in host memory (it synchronizes `stream`).  Pinned host memory transfers
 * faster than pageable.  N1 = 0, N3 = 0 or N2 = 0 return 0 without touching
 * memory (C + A*B = C when N2 = 0).  PGEMM_EHIP if a copy, the launch or the
 * synchronization fails.
 */
int matmat_f64_host(int lda, int ldb, int ldc, const double *A, const double *B,
                    double *C, int N1, int N2, int N3, void *workspace,
                    size_t workspace_bytes, void *stream);
/* Workspace bytes matmat_f64_host needs (0 for an empty product or invalid
 * leading dimensions). */
size_t pgemm_matmat_host_workspace(int lda, int ldb, int ldc, int N1, int N2, int N3);

/* Static text for a status code returned by any entry point. */
const char *pgemm_status_string(int status);

/*
 * Diagnostics.  pgemm_select_f32 / pgemm_select_f64 return the kernel
 * variant id gemm_f32 / gemm_f64 would launch for these arguments (host
 * logic only; it may query the current device's compute-unit count, and
 * without a device assumes 256), or a negative status for invalid
 * arguments, or 0 for calls
 * that launch no GEMM kernel (quick return or the beta-scaling path).
 * Variant ids are positive; pgemm_variant_name() describes one (NULL if the
 * id is unknown).  gemm_f32_variant / gemm_f64_variant run the GEMM with a
 * forced variant (same contract as gemm_f32 / gemm_f64, plus
 * PGEMM_EVARIANT for an unknown id, one of the other precision, an aligned
 * ("vec") variant with unaligned arguments, or an ldc beyond the variant's
 * limit: the 64 x 64 variants store C with 32-bit offsets from a tile's
 * first element and take ldc <= 8388606 (fp32) or 4194302 (fp64); gemm_f32
 * and gemm_f64 do not choose them beyond that); they let tests cover every
 * compiled tile configuration.
 */
int pgemm_select_f32(int m, int n, int k, float alpha, const float *A, int lda,
                     const float *B, int ldb, float beta, const float *C, int ldc);
int pgemm_select_f64(int m, int n, int k, double alpha, const double *A, int lda,
                     const double *B, int ldb, double beta, const double *C, int ldc);
/* The variant gemm_f32_ws / gemm_f64_ws would launch with a workspace of
 * ws_bytes bytes (0: as without one, i.e. gemm_f32 / gemm_f64), same return
 * values as above.  If sk_wgs is not NULL it receives the number of
 * stream-K workgroups that share the last, partly filled round (0: none;
 * otherwise the call also launches the fix-up kernel that sums the pieces).
 * If strip_rows is not NULL it receives the number of rows of C below the
 * last whole tile row that a separate strip kernel computes (0: none; at
 * most 8; the tiles then cover the first m - strip_rows rows). */
int pgemm_select_ws_f32(int m, int n, int k, float alpha, const float *A, int lda,
                        const float *B, int ldb, float beta, const float *C, int ldc,
                        size_t ws_bytes, int *sk_wgs, int *strip_rows);
int pgemm_select_ws_f64(int m, int n, int k, double alpha, const double *A, int lda,
                        const double *B, int ldb, double beta, const double *C, int ldc,
                        size_t ws_bytes, int *sk_wgs, int *strip_rows);
const char *pgemm_variant_name(int variant);
int pgemm_num_variants(void);
/* The current device's compute units and peak clock (kHz), as the HIP
 * runtime reports them: the matrix peaks are cus * clock * 256 flop per
 * cycle (fp32) and * 128 (fp64).  Returns 0, -1 / -2 for a NULL argument,
 * or PGEMM_EHIP when no device answers. */
int pgemm_device_info(int *cus, int *clock_khz);
int gemm_f32_variant(int variant, int m, int n, int k, float alpha, const float *A,
                     int lda, const float *B, int ldb, float beta, float *C, int ldc,
                     void *stream);
int gemm_f64_variant(int variant, int m, int n, int k, double alpha, const double *A,
                     int lda, const double *B, int ldb, double beta, double *C, int ldc,
                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PGEMM_H */
