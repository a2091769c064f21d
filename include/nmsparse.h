/*
 * nmsparse — N:M fine-grained structured-sparse matrix multiply for AMD
 * Instinct MI355X (gfx950).
 *
 *   D = alpha * op(A) * op(B) + beta * C
 *
 * A is the sparse operand: in every group of M consecutive elements along the
 * reduction dimension k of op(A), at most N are non-zero (2:4 is the case the
 * matrix cores run natively; general N:M with M in {4, 8, 16, 32} runs on the
 * gather paths). B, C and D are dense.
 *
 * The operation, its layouts and the set-up-once / multiply-many workflow
 * follow the NVIDIA developer blog "Exploiting Ampere structured sparsity with
 * cuSPARSELt" (the section defining D = alpha*op(A)*op(B) + beta*C with N/T
 * layouts, the workflow list, and the code example: prune, prune check,
 * compressed size, compress, matmul). The magnitude top-N rule follows the
 * apex pull request "[sparse] update support for arbitrary N:M settings
 * sparse" (extension 1, the greedy per-group mask); the transposable 4x4-tile
 * mask follows pytorch issue 126420 "backpropagation for sparse
 * semi-structured" (the maintainer reply on forward and backward needing
 * 2:4 in both directions).
 *
 * Conventions used by every entry point
 * -------------------------------------
 *  - A and B are row-major. op_a / op_b say whether the stored array is
 *    used as is (NM_OP_N) or transposed (NM_OP_T):
 *      op_a = N: A stored m x k (lda >= k);  op_a = T: A stored k x m (lda >= m)
 *      op_b = N: B stored k x n (ldb >= n);  op_b = T: B stored n x k (ldb >= k)
 *      C and D: m x n, row-major (ldc, ldd >= n) or, with order_cd =
 *      NM_COL_MAJOR, column-major (ldc, ldd >= m).
 *    (The blog defines N/T on column-major storage; its column-major "TN" is
 *    byte-for-byte this library's "NT" with order_cd = NM_COL_MAJOR.)
 *  - Element types (type_ab, type_cd): (NM_F16, NM_F16), (NM_BF16, NM_BF16)
 *    with fp32 accumulation; (NM_I8, NM_I32) with exact int32 accumulation
 *    (the blog's type list; C and D are int32 for the integer path); and
 *    (NM_I8, NM_I8), the blog's int8 output: C and D int8, D = alpha * acc +
 *    beta * C evaluated exactly and saturated to [-128, 127].
 *  - Leading dimensions are in elements. All device pointers must be 16-byte
 *    aligned, and every stored row (column, for column-major C/D) that is at
 *    least 16 bytes long must start on a 16-byte boundary
 *    (ld * element size % 16 == 0).
 *  - Ownership: the caller allocates and owns every device buffer. A plan owns
 *    host memory only. The library never allocates device memory and never
 *    synchronises the device: device work is enqueued on the caller's stream
 *    (`stream` is a hipStream_t passed as void*, NULL = the null stream).
 *  - Errors: invalid arguments, shapes and alignment are reported before
 *    anything is enqueued (nothing runs). A failed kernel launch returns
 *    NM_ERR_HIP. nm_last_error() gives a message for the last failure on the
 *    calling thread.
 *
 * Compressed layout (this library's definition; the blog only says the sparse
 * matrix is stored as its non-zeros at half size plus "a small amount of
 * metadata"). For every row r of op(A) and group g (columns gM .. gM+M-1),
 * the kept in-group offsets i_0 < ... < i_{N-1} are those the 1-D rule below
 * selects. Then
 *     values[r * values_ld + g*N + s] = op(A)[r][g*M + i_s]
 *     bits [(g*N + s)*b, (g*N + s + 1)*b) of row r of meta  = i_s
 * with b = ceil(log2 M) (2 bits for M = 4, 5 bits for M = 32). Each meta row
 * is a little-endian bit stream (bit t is bit t%8 of byte t/8) of meta_ld
 * bytes. values_ld (elements) and meta_ld (bytes) are the row lengths rounded
 * up to 16 bytes; every padding bit and element is zero. For 2:4 a group is
 * the nibble i_0 | i_1 << 2, which is also the index format the gfx950 sparse
 * matrix instructions consume.
 *
 * 1-D selection rule: in every group keep the N elements of largest |x|;
 * among equal magnitudes the lower offset wins (for fp16/bf16 the magnitude
 * order is the order of the bit pattern with the sign cleared, so +0 and -0
 * are equal). Exactly N slots are kept per group even when some are zero.
 *
 * Vector-wise N:M (vector_rows = V > 1; the apex pull request's extension 2,
 * vector-wise N:M for nmSPARSE): the V consecutive rows bV .. bV+V-1 of op(A)
 * share one set of kept offsets in every group. A vector is the V values of
 * one column of such a block; its score is |v_0 + v_1 + ... + v_{V-1}| (the
 * signed values summed first, as the pull request's vector-wise calculator
 * does), accumulated in fp64 in increasing row order. In every group the N
 * vectors of largest score are kept for all V rows, ties to the lower offset
 * (scores compare as the bit patterns of the non-negative fp64 values, so a
 * NaN score ranks above +Inf). The compressed values keep the element-wise
 * layout (row r holds its own kept values); the metadata has one row per
 * block: m / V rows of meta_ld bytes, block row b holding the element-wise
 * bit stream of its offsets. Requires op_a = NM_OP_N (NM_ERR_UNSUPPORTED
 * otherwise) and m % V == 0 (NM_ERR_SHAPE); the prune check counts the
 * (block, group) pairs whose V rows hold non-zeros at more than N offsets;
 * NM_PRUNE_TILE4X4 does not apply (NM_ERR_INVALID_ARG).
 */
#ifndef NMSPARSE_H
#define NMSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_ERR_INVALID_ARG = 1, /* null pointer, unknown enum, bad N:M, non-integral alpha/beta on the int path */
  NM_ERR_SHAPE = 2,       /* k % M != 0, tile mode on dims not divisible by 4, ld too small, size overflow */
  NM_ERR_ALIGN = 3,       /* pointer or leading dimension breaks the 16-byte rule */
  NM_ERR_UNSUPPORTED = 4, /* valid request this build does not implement (vector-wise N:M with op_a = T) */
  NM_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} nm_status_t;

typedef enum { NM_F16 = 0, NM_BF16 = 1, NM_I8 = 2, NM_I32 = 3 } nm_dtype_t;
typedef enum { NM_OP_N = 0, NM_OP_T = 1 } nm_op_t;
/* Storage order of C and D. NM_ROW_MAJOR: element (i, j) at i * ld + j
 * (ld >= n). NM_COL_MAJOR: element (i, j) at j * ld + i (ld >= m), the
 * column-major output of the cuSPARSELt blog's matmul descriptors (its
 * Table 1 runs use column-major matrices); D^T is then a row-major n x m
 * matrix, e.g. Y = X W^T for activations X stored tokens x features. */
typedef enum { NM_ROW_MAJOR = 0, NM_COL_MAJOR = 1 } nm_order_t;
typedef enum { NM_PRUNE_1D = 0, NM_PRUNE_TILE4X4 = 1 } nm_prune_mode_t;

/* Problem descriptor: the blog's structured / dense / matmul descriptors
 * folded into one struct. All fields are read by nm_plan_init and copied. */
typedef struct {
  int64_t m, n, k;          /* D is m x n; k is the reduction dimension */
  int32_t nm_n, nm_m;       /* N kept of every M along k of op(A); 1 <= N < M, M in {4, 8, 16, 32} */
  int32_t op_a, op_b;       /* nm_op_t */
  int32_t type_ab, type_cd; /* nm_dtype_t pair, see above */
  int64_t lda, ldb, ldc, ldd;
  int32_t order_cd;         /* nm_order_t of C and D (both the same order) */
  int32_t vector_rows;      /* V: 0 or 1 = element-wise N:M (every row of op(A) has its own kept offsets);
                               V in {2, 4, ..., 256} (a power of two) = vector-wise N:M (see below) */
} nm_problem_t;

typedef struct nm_plan* nm_plan_t;

/* Validate a problem and build a plan (host only, no device call). The plan
 * fixes shapes, layouts, compressed sizes and the SpMM kernel. On failure
 * *plan is set to NULL. */
nm_status_t nm_plan_init(nm_plan_t* plan, const nm_problem_t* problem);

/* Release a plan (host memory only). NULL is accepted. */
nm_status_t nm_plan_destroy(nm_plan_t plan);

/* Sizes of the compressed form of op(A) (the blog's compressed-size query):
 * values_bytes = m * values_ld * sizeof(type_ab); meta_bytes = (m / V) *
 * meta_ld (V = vector_rows, 1 for element-wise N:M).
 * Any output pointer may be NULL. */
nm_status_t nm_compressed_size(nm_plan_t plan, size_t* values_bytes, size_t* meta_bytes,
                               int64_t* values_ld_elems, int64_t* meta_ld_bytes);

/* Size of the optional keep mask written by nm_prune: one bit per element of
 * the stored A (rows x cols as stored), uint32 words, least significant bit
 * first, each stored row starting a new word: mask_ld_words = ceil(cols/32). */
nm_status_t nm_mask_size(nm_plan_t plan, size_t* mask_bytes, int64_t* mask_ld_words);

/* Prune the stored A (lda) into dA_pruned (same shape and lda; may equal dA).
 *  NM_PRUNE_1D:      the 1-D rule above along k of op(A); kept values copied
 *                    bit for bit, every other element written as +0.
 *  NM_PRUNE_TILE4X4: requires N:M = 2:4 and both stored dimensions divisible
 *                    by 4. On every 4x4 tile of the stored matrix keep the
 *                    pattern with exactly two elements per row and per column
 *                    (90 candidates) that maximises the kept sum of |x|,
 *                    summed in fp64 as ((s0 + s1) + s2) + s3 over tile rows;
 *                    ties go to the first candidate when candidates are
 *                    ordered lexicographically by their per-row pair index
 *                    (pairs ordered (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)).
 *                    The result is 2:4 along both dimensions, so it serves
 *                    op_a = N (forward) and op_a = T (backward).
 * d_mask may be NULL; otherwise it receives the keep mask (nm_mask_size). */
nm_status_t nm_prune(nm_plan_t plan, const void* dA, void* dA_pruned, int32_t mode,
                     uint32_t* d_mask, void* stream);

/* Apply a keep mask written by nm_prune to another matrix of the stored A's
 * shape and leading dimension (lda): elements whose bit is clear become +0,
 * the others are left as they are. This masks a gradient with the sparsity
 * pattern of the weight it belongs to (the pytorch issue's sparse training
 * setting: the masked weight gradient keeps the pruned weights at zero). */
nm_status_t nm_mask_apply(nm_plan_t plan, const uint32_t* d_mask, void* dX, void* stream);

/* Conformance check (the blog's prune check, with its flag made a count):
 * writes to *d_violations (device int32) the number of groups of op(A) that
 * hold more than N non-zeros (1-D), or the number of 4x4-tile rows plus
 * tile columns with more than two non-zeros (TILE4X4). 0 means conforming.
 * -0.0 counts as zero. The count overwrites *d_violations. */
nm_status_t nm_prune_check(nm_plan_t plan, const void* dA, int32_t mode, int32_t* d_violations,
                           void* stream);

/* Compress the stored A into (values, meta) in the layout above. The
 * selection is the 1-D rule, so compress(A) == compress(prune(A)); on an
 * input that already conforms, the kept slots are its non-zeros plus the
 * lowest-offset zeros. Padding is written as zero. */
nm_status_t nm_compress(nm_plan_t plan, const void* dA, void* d_values, void* d_meta, void* stream);

/* Inverse of nm_compress: writes the dense stored A (lda, op_a orientation):
 * kept values at their offsets, +0 everywhere else. */
nm_status_t nm_decompress(nm_plan_t plan, const void* d_values, const void* d_meta, void* dA_out,
                          void* stream);

/* D = alpha * op(A) * op(B) + beta * C with A given as (values, meta).
 * alpha and beta are host floats (the blog's example passes host floats);
 * on the int8 path both must be integers. dC may be NULL when *beta == 0 and
 * may equal dD. C and D are stored in the plan's order_cd (row- or
 * column-major). fp16/bf16 outputs are alpha*acc + beta*C evaluated in fp32
 * and rounded to nearest even.
 * d_workspace: device memory of at least nm_spmm_workspace_size bytes, 16-byte
 * aligned, when that size is non-zero (a split-k plan); it must not overlap
 * any operand, its contents on entry do not matter, and it is scratch after
 * the call (the blog's matmul takes its workspace the same way). When the size
 * is zero d_workspace is not read and may be NULL. A missing workspace is
 * NM_ERR_INVALID_ARG, returned before anything is enqueued. */
nm_status_t nm_spmm(nm_plan_t plan, const float* alpha, const void* d_values, const void* d_meta,
                    const void* dB, const float* beta, const void* dC, void* dD, void* d_workspace,
                    void* stream);

/* nm_spmm without a workspace argument and without any device allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. A split-k
 * plan's partial sums go to a static device array of the library,
 * NM_NOALLOC_SCRATCH_BYTES (32 MiB) on every GPU the library runs on, held
 * until the process ends; its address is looked up once per device on the
 * first call that needs it (the device of `stream`, the current device for
 * the null stream). Plans whose workspace (nm_spmm_workspace_size) exceeds
 * that size get NM_ERR_SHAPE before anything is enqueued; plans that need no
 * workspace run exactly as nm_spmm. All calls on one GPU share that GPU's
 * array, which keeps the last call's contents (every element a call reads
 * was written earlier in the same call, so nothing has to be cleared): calls
 * that may overlap on one GPU (different streams, no ordering between them)
 * race on it and must be serialised by the caller. Arguments and results
 * otherwise as nm_spmm. */
#define NM_NOALLOC_SCRATCH_BYTES (32u << 20)
nm_status_t nm_spmm_noalloc(nm_plan_t plan, const float* alpha, const void* d_values, const void* d_meta,
                            const void* dB, const float* beta, const void* dC, void* dD, void* stream);

/* Same-shape dense product D = alpha * op(A) * op(B) + beta * C with A dense
 * (stored with lda and op_a as in the plan). This is the in-library
 * comparator for the sparse speed-up (the blog's dense-vs-sparse table); it
 * ignores N:M. */
nm_status_t nm_dense_gemm(nm_plan_t plan, const float* alpha, const void* dA, const void* dB,
                          const float* beta, const void* dC, void* dD, void* stream);

/* Algorithm selection: the blog's algorithm-selection object with its
 * configuration-id attribute, reduced to one id on the plan. The ids pin the
 * block tile of the matrix-core products (nm_spmm on the 2:4 and general N:M
 * paths and nm_dense_gemm): NM_ALG_AUTO (the default: the plan picks by shape),
 * NM_ALG_TILE128 (128 x 128), NM_ALG_TILE256X128 (256 x 128),
 * NM_ALG_TILE256 (256 x 256; for the dense product on whole tiles a two-stage
 * ring, which the automatic choice does not take). The
 * general N:M expansion always uses 128 x 128 and small n (n <= 16) its own
 * kernel; there the id has no effect. Results do not depend on the id beyond
 * fp32 summation order (bit-exact for int8). Host-only; invalid ids give
 * NM_ERR_INVALID_ARG and leave the plan unchanged. */
enum { NM_ALG_AUTO = 0, NM_ALG_TILE128 = 1, NM_ALG_TILE256X128 = 2, NM_ALG_TILE256 = 3, NM_ALG_COUNT = 4 };
int32_t nm_plan_algorithm_count(nm_plan_t plan);   /* NM_ALG_COUNT (0 for a NULL plan) */
nm_status_t nm_plan_set_algorithm(nm_plan_t plan, int32_t alg);
nm_status_t nm_plan_get_algorithm(nm_plan_t plan, int32_t* alg);

/* nm_spmm over several streams (the blog's matmul takes an array of streams):
 * the rows of D are split into at most num_streams blocks of whole 256-row
 * multiples, and block i is enqueued on streams[i] as its own product (the
 * same kernels nm_spmm picks for a problem of that many rows; a split-k
 * plan's workspace is shared out between the blocks, so the workspace size is
 * the plan's). The caller orders the streams after the call (each stream's
 * work is independent). num_streams in [1, 64]; 1 is nm_spmm on streams[0].
 * Results equal nm_spmm's up to fp32 summation order (bit-identical for int8).
 * Errors and arguments as nm_spmm. */
nm_status_t nm_spmm_streams(nm_plan_t plan, const float* alpha, const void* d_values, const void* d_meta,
                            const void* dB, const float* beta, const void* dC, void* dD, void* d_workspace,
                            void* const* streams, int32_t num_streams);

/* Split-k: the blog's split-k setting of the algorithm selection, with the
 * workspace its matmul call takes (the workspace-size query and the
 * d_workspace argument of the code example). With splits S > 1, the 2:4
 * product on whole tiles (m and n multiples of the block tile, k a multiple of
 * 64 fp16/bf16 or 128 int8 elements, 16-byte rows) runs S blocks per output
 * tile, each over one contiguous range of the k-steps (range z covers steps
 * [z T / S, (z + 1) T / S) of the T = k / 64 (128 for int8) steps), writes its
 * raw fp32 (int32) partial sums to plane z of the workspace, and a second
 * kernel adds the planes in the order z = 0, 1, ..., applies alpha and beta
 * and rounds once. int8 results are bit-identical to the unsplit product;
 * fp16/bf16 differ only by fp32 summation order. Shapes the split does not
 * apply to (other tiles, general N:M, small n) run unsplit and need no
 * workspace. Host-only.
 *   nm_plan_set_split_k: S in [1, 16] (1 = no split, the default); invalid
 *     values give NM_ERR_INVALID_ARG and leave the plan unchanged.
 *   nm_plan_get_split_k: the requested S and the S nm_spmm will launch
 *     (min(S, T) where the split applies, else 1); either pointer may be NULL.
 *   nm_spmm_workspace_size: S_eff * m * n * 4 bytes when S_eff > 1, else 0. */
nm_status_t nm_plan_set_split_k(nm_plan_t plan, int32_t splits);
nm_status_t nm_plan_get_split_k(nm_plan_t plan, int32_t* requested, int32_t* effective);
nm_status_t nm_spmm_workspace_size(nm_plan_t plan, size_t* bytes);

/* Name of the SpMM kernel the plan dispatches to (static string). */
const char* nm_plan_kernel_name(nm_plan_t plan);

/* The device kernel nm_spmm launches for this plan (whenever m, n > 0), named
   as profilers print it: demangled, e.g. "void nm::gemm_dma_kernel<0, 0, 256,
   256, 3, 2, 4, 1>(nm::GemmArgs)". The first call runs the same host logic as
   nm_spmm without launching anything and caches the result in the plan; the
   string lives as long as the plan. Needs the HIP runtime to resolve the name
   ("unknown" otherwise). Calls on one plan must not run concurrently. */
const char* nm_plan_spmm_kernel(nm_plan_t plan);

/* Static text for a status code. */
const char* nm_status_string(nm_status_t status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* nm_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t nm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NMSPARSE_H */
