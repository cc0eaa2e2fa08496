/*
 * dgt_gemm.h -- C ABI of the MI355X (gfx950) dense GEMM library.
 *
 * Operation (every entry point): the BLAS GEMM form
 *
 *     C <- alpha * op(A) * op(B) + beta * C
 *
 * with C(i,j) = sum_k op(A)(i,k) * op(B)(k,j) (element formula:
 * dilfish.github.io section 5.2; chongfengling.github.io section 1;
 * elainafan.one "稠密矩阵乘法", where alpha and beta let one call both scale
 * and accumulate).  op(X) is X, or X transposed when gemm_ex is asked for it
 * (every other entry point: no transposes).
 *
 * Layout: row-major with leading dimensions, the column index contiguous
 * (chongfengling.github.io section 2.2; elainafan.one "行主序"):
 *     op(A)(i,k) = A[i*lda + k]  trans_a = 0: A stored M x K, lda >= max(1, K)
 *     op(A)(i,k) = A[k*lda + i]  trans_a = 1: A stored K x M, lda >= max(1, M)
 *     op(B)(k,j) = B[k*ldb + j]  trans_b = 0: B stored K x N, ldb >= max(1, N)
 *     op(B)(k,j) = B[j*ldb + k]  trans_b = 1: B stored N x K, ldb >= max(1, K)
 *     C(i,j)     = C[i*ldc + j]  C is M x N,                  ldc >= max(1, N)
 * The transposed forms are the operands of a linear layer stored as in
 * elainafan.one "全连接层" (input X [batch, in], weight W [out, in], output
 * gradient G [batch, out]): the forward pass X*W^T is trans_b = 1, the
 * weight gradient G^T*X is trans_a = 1, the input gradient G*W needs
 * neither.  A column-major caller passes its storage with the flags set.
 *
 * Precision: gemm_f32 takes fp32 A and B; gemm_bf16 takes A and B as raw
 * bf16 bit patterns (uint16_t, the upper half of an fp32 value: 8-bit
 * exponent, 7-bit mantissa); gemm_f16 takes raw IEEE binary16 bit patterns
 * (5-bit exponent, 10-bit mantissa) -- the BF16 and FP16 rows of the
 * dilfish.github.io section 5.5 precision table.  All accumulate in fp32 on
 * the matrix cores and read/write C in fp32.  The
 * summation order is the kernel's own; results agree with an exact
 * reference to fp32 accumulation accuracy, and bit for bit whenever every
 * partial sum is exactly representable (e.g. small-integer inputs).
 *
 * Semantics of the edge cases (the pages leave them open; BLAS readings):
 *   - beta == 0: C is write-only; NaN/Inf already in C never propagate.
 *   - alpha == 0 or K == 0: A and B are not read; C <- beta*C (zeros when
 *     beta == 0 too).
 *   - M == 0 or N == 0: nothing is done; returns GEMM_OK.
 *
 * Memory and ownership: A, B and C are DEVICE pointers owned by the caller;
 * they must stay valid until the work queued on `stream` has finished.  The
 * library allocates nothing, frees nothing, keeps no per-call state and is
 * safe to call from several host threads.  A misaligned pointer or leading
 * dimension is accepted (fp32: 4-byte, bf16/fp16: 2-byte alignment); it only
 * selects a slower load path, never a fault.
 *
 * Ordering: asynchronous.  Work is queued on `stream` (a hipStream_t cast
 * to void*; NULL = the null stream) and the call returns without waiting.
 *
 * Errors: every entry point returns GEMM_OK (0) or a negative status; on an
 * argument error nothing is queued.  The library never aborts or prints.
 * Argument checks run on the host in this order: dtype and transpose flags,
 * dimensions, leading dimensions, variant id, quick return for an empty C,
 * null pointers, overlap of C with A or B, variant support for the shape.
 * gemm_status_string() names a status.
 */
#ifndef DGT_GEMM_H
#define DGT_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DGT_GEMM_ABI_VERSION 9

/* Input formats (the dtype argument of gemm_ex and gemm_select_variant). */
enum gemm_dtype { GEMM_DTYPE_F32 = 0, GEMM_DTYPE_BF16 = 1, GEMM_DTYPE_F16 = 2 };

enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_DIM = -1,          /* M, N or K negative                        */
    GEMM_ERR_LD = -2,           /* lda < max(1,K), ldb < max(1,N) or
                                   ldc < max(1,N)                            */
    GEMM_ERR_NULL = -3,         /* NULL A/B (when read) or C with a
                                   non-empty extent                          */
    GEMM_ERR_OVERLAP = -4,      /* the byte range of C overlaps A's, B's or
                                   the bias's, or two problems of a batch
                                   share C elements                          */
    GEMM_ERR_VARIANT = -5,      /* unknown variant, or one that does not
                                   support this shape / size                 */
    GEMM_ERR_LAUNCH = -6,       /* the HIP runtime rejected a kernel launch  */
    GEMM_ERR_ARG = -7,          /* dtype not a gemm_dtype, a transpose flag
                                   other than 0 or 1, a negative batch,
                                   splits or workspace size, or a stride
                                   outside [0, 2^48)                         */
    GEMM_ERR_WORKSPACE = -8,    /* gemm_splitk: workspace NULL or smaller
                                   than gemm_splitk_workspace_size           */
    GEMM_ERR_SCRATCH = -9       /* gemm_splitk_noalloc: the shape's partials
                                   (gemm_splitk_workspace_size) exceed
                                   DGT_GEMM_NOALLOC_SCRATCH_BYTES            */
};

/* Kernel ladder (for measurement and tests; GEMM_VARIANT_AUTO is what
 * gemm_f32 / gemm_bf16 / gemm_f16 use).  Every variant computes the same operation
 * and handles any shape that it accepts, ragged edges included. */
enum gemm_variant {
    GEMM_VARIANT_AUTO = 0,      /* MFMA tiles; skinny path when M <= 64       */
    GEMM_VARIANT_NAIVE = 1,     /* one lane per output, K-loop of two global
                                   loads and an FMA (dilfish.github.io 5.2;
                                   chongfengling.github.io 2.1 and 2.4:
                                   the contiguous column index on the
                                   64-wide lane index)                        */
    GEMM_VARIANT_LDS = 2,       /* LDS-staged 128x128 macro tiles, 128-bit
                                   global loads, double-buffered, padded LDS
                                   rows, 8x8 outputs per lane on the vector
                                   ALU (dilfish.github.io 5.3 and 5.4)        */
    GEMM_VARIANT_MFMA = 3,      /* LDS-staged macro tiles, double-buffered,
                                   per-wavefront MFMA micro-tiles, masked
                                   ragged edges (dilfish.github.io 5.4-5.5;
                                   qwbw.cn section 三); the workgroup tile
                                   (256 x 256 or 128 x 128; 64 x 64 for fp32
                                   launches with at most 128 tiles of 128 x
                                   128) is chosen per launch                  */
    GEMM_VARIANT_SKINNY = 4,    /* M <= 64: streams B once from HBM (copied
                                   straight into LDS when B is stored N x K
                                   with 16-byte aligned rows), A held in
                                   registers per step (up to four 16-row
                                   blocks), K split over waves and reduced
                                   in LDS (dilfish.github.io 5.1 GEMV row and
                                   batching; qwbw.cn section 四)              */
    GEMM_VARIANT_MFMA_T256 = 5, /* the MFMA rung's global->LDS DMA kernel with
                                   a fixed 256 x 256 workgroup tile (one
                                   workgroup per CU): the block-size choice
                                   of dilfish.github.io 5.3-5.4 made
                                   explicit.  Needs 16-byte aligned operand
                                   rows (pitch and base) and pitches below
                                   2^23 (fp32) or 2^24 (16-bit) elements;
                                   GEMM_ERR_VARIANT otherwise                */
    GEMM_VARIANT_MFMA_T128 = 6, /* the same with 128 x 128 tiles, two
                                   workgroups per CU                          */
    GEMM_VARIANT_MFMA_REGS = 7  /* the MFMA rung without the DMA pipeline:
                                   LDS tiles filled through registers by
                                   128-bit loads, double-buffered
                                   (dilfish.github.io 5.4's double buffer),
                                   MFMA micro-tiles, workgroup tiles of
                                   128 x 128 (fp32) or 256 x 256 (16-bit
                                   inputs); any alignment.  GEMM_VARIANT_MFMA
                                   uses this kernel for operands the DMA
                                   kernels do not take (rows not 16-byte
                                   aligned, pitches past their limits) and,
                                   on 64 x 64 tiles, for the small fp32
                                   launches                                   */
};

/* C <- alpha*A*B + beta*C, fp32 inputs, fp32 accumulate/output. */
int gemm_f32(int M, int N, int K, float alpha, const float* A, int lda,
             const float* B, int ldb, float beta, float* C, int ldc,
             void* stream);

/* C <- alpha*A*B + beta*C, bf16 inputs (raw bits), fp32 accumulate/output. */
int gemm_bf16(int M, int N, int K, float alpha, const uint16_t* A, int lda,
              const uint16_t* B, int ldb, float beta, float* C, int ldc,
              void* stream);

/* C <- alpha*A*B + beta*C, fp16 inputs (raw IEEE binary16 bits), fp32
 * accumulate/output: the half-input / fp32-accumulate matrix-unit path of
 * dilfish.github.io 5.5 (WMMA listing) and qwbw.cn Level 2. */
int gemm_f16(int M, int N, int K, float alpha, const uint16_t* A, int lda,
             const uint16_t* B, int ldb, float beta, float* C, int ldc,
             void* stream);

/* Same as gemm_f32 / gemm_bf16 / gemm_f16 with an explicit ladder rung (enum
 * gemm_variant).  GEMM_VARIANT_SKINNY requires M <= 64, and the fixed-tile
 * MFMA rungs 16-byte aligned operand rows, and return GEMM_ERR_VARIANT
 * otherwise (checked on the host before anything is queued; alpha == 0 or
 * K == 0 never reads A or B and so never fails this check). */
int gemm_f32_variant(int variant, int M, int N, int K, float alpha,
                     const float* A, int lda, const float* B, int ldb,
                     float beta, float* C, int ldc, void* stream);
int gemm_bf16_variant(int variant, int M, int N, int K, float alpha,
                      const uint16_t* A, int lda, const uint16_t* B, int ldb,
                      float beta, float* C, int ldc, void* stream);
int gemm_f16_variant(int variant, int M, int N, int K, float alpha,
                     const uint16_t* A, int lda, const uint16_t* B, int ldb,
                     float beta, float* C, int ldc, void* stream);

/* General form: C <- alpha*op(A)*op(B) + beta*C with the input format
 * `dtype` (enum gemm_dtype; A and B point to float for GEMM_DTYPE_F32, to
 * raw uint16_t bits otherwise), transpose flags trans_a / trans_b (0 or 1,
 * storage as in the layout table above) and a ladder rung `variant` (enum
 * gemm_variant; every rung takes every layout).  The untransposed call is
 * the same operation as gemm_f32 / gemm_bf16 / gemm_f16 (_variant), with the
 * same kernels. */
int gemm_ex(int dtype, int trans_a, int trans_b, int variant, int M, int N,
            int K, float alpha, const void* A, int lda, const void* B, int ldb,
            float beta, float* C, int ldc, void* stream);

/* Strided batch with the bias of a linear layer: for z = 0 .. batch-1,
 *
 *   C_z <- alpha * op(A_z) * op(B_z) + beta * C_z + 1 * bias_z^T
 *
 * where X_z = X + z * stride_x (strides in ELEMENTS of the operand: A and B
 * in their input format, C and bias in floats; 0 repeats one operand for
 * every problem, e.g. a shared weight), and bias_z is a row of N floats
 * added to every row of C_z (elainafan.one "全连接层": the linear layer
 * computes X*W^T + b; its input keeps a batch dimension).  bias may be NULL
 * (no bias); it is added after the BLAS form, unscaled, also when
 * alpha == 0 or K == 0.  Every other argument is as for gemm_ex.
 * Requirements: batch >= 0 (0 does nothing), strides in [0, 2^48), the
 * problems' C ranges disjoint (stride_c * 4 bytes at least the span of one
 * C when batch > 1), C disjoint from every A, B and bias range.  Any batch
 * size is accepted; the library splits it into launches of at most 65535
 * problems, queued in order on `stream`. */
int gemm_strided_batched(int dtype, int trans_a, int trans_b, int variant,
                         int M, int N, int K, float alpha,
                         const void* A, int lda, int64_t stride_a,
                         const void* B, int ldb, int64_t stride_b,
                         float beta, float* C, int ldc, int64_t stride_c,
                         const float* bias, int64_t stride_bias, int batch,
                         void* stream);

/* Split-K, for shapes with too few output tiles to fill the GPU (e.g. a
 * small M x N with a long K).  Same operation and arguments as gemm_ex with
 * GEMM_VARIANT_AUTO, computed in two phases queued on `stream`: the K range
 * is cut into slices (whole multiples of 128 except the last), each slice's
 * product is written to the caller's `workspace` as fp32 partials (M x N
 * per slice), and a second kernel sums the slices in a fixed order and
 * applies alpha and beta -- deterministic, no atomics, nothing allocated.
 * The pages do not describe split-K; they note that a launch whose blocks
 * are partly idle leaves compute unused (elainafan.one "朴素 CUDA 实现",
 * after the launch code), and this is the case where the whole grid is too
 * small: the reduction dimension supplies the missing parallelism.
 * `splits` = 0 picks the number of slices that fills the GPU's workgroup
 * slots (128 x 128 tiles: one per CU for fp32, two for 16-bit inputs; a
 * skinny column strip per CU for M <= 64; each slice at least 128 deep)
 * and runs them as one launch; a positive value is a request (at
 * most 64; rounding of the slice length may give fewer).  With one slice
 * the call is gemm_ex and needs no workspace.  The workspace (device
 * memory, 16-byte aligned, at least gemm_splitk_workspace_size bytes) must
 * not overlap A, B or C and must stay untouched until the work on `stream`
 * has finished; its contents on return are unspecified. */
int gemm_splitk(int dtype, int trans_a, int trans_b, int M, int N, int K,
                float alpha, const void* A, int lda, const void* B, int ldb,
                float beta, float* C, int ldc, int splits, void* workspace,
                int64_t workspace_bytes, void* stream);

/* gemm_splitk for callers that cannot allocate device memory at all --
 * code recorded under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation -- and so cannot hand in a workspace either.
 * Same operation, arguments, slicing and kernels as gemm_splitk (results
 * are bit-identical to it), but the fp32 partials go to a fixed scratch
 * array of DGT_GEMM_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it has run on until the process ends.  The call allocates nothing:
 * no hipMalloc, no hipFree, no allocating library routine.
 *   - Size limit: a shape whose partials (gemm_splitk_workspace_size for
 *     the same dtype, shape and splits) exceed the scratch returns
 *     GEMM_ERR_SCRATCH before anything is queued; a shape that needs no
 *     split runs as gemm_ex and uses no scratch.
 *   - Sharing: all calls on one GPU share that GPU's scratch, which keeps
 *     the last call's partials.  Calls on one GPU must not overlap in time
 *     (queue them on one stream, or order their streams); overlapping calls
 *     race on the scratch and give wrong results.  No part of the scratch
 *     needs to start at zero (every partial is written before it is read).
 *   - The first call on a GPU looks up that GPU's scratch address (a host
 *     query, no allocation); a failure there returns GEMM_ERR_LAUNCH.
 * Every other error is as for gemm_splitk. */
#define DGT_GEMM_NOALLOC_SCRATCH_BYTES (64ll << 20)
int gemm_splitk_noalloc(int dtype, int trans_a, int trans_b, int M, int N,
                        int K, float alpha, const void* A, int lda,
                        const void* B, int ldb, float beta, float* C, int ldc,
                        int splits, void* stream);

/* Number of K slices gemm_splitk uses for this shape and request (>= 1), or
 * a negative status.  Host only. */
int gemm_splitk_slices(int dtype, int M, int N, int K, int splits);

/* Bytes of workspace gemm_splitk needs for this shape and request: slices x
 * M x N x 4, or 0 with one slice; a negative status for bad arguments.
 * Host only. */
int64_t gemm_splitk_workspace_size(int dtype, int M, int N, int K, int splits);

/* Stream-K: the same operation and arguments as gemm_ex with
 * GEMM_VARIANT_AUTO, for shapes whose 256 x 256 output tiles do not divide
 * evenly among the 256 compute units (the last wave of tiles of a
 * data-parallel launch then runs on part of the chip).  The pages note that
 * a launch whose blocks are partly idle leaves compute unused
 * (elainafan.one "朴素 CUDA 实现", after the launch code); stream-K deals out
 * the tiles' K iterations (128 k each for 16-bit inputs, 64 k for FP32) in
 * equal contiguous ranges to one workgroup per compute unit instead of whole
 * tiles.  A tile covered by one workgroup is written directly; the parts of
 * a tile split between workgroups go to the caller's `workspace` as fp32
 * partial sums, and a second kernel queued on `stream` sums them in k order
 * and applies alpha, beta -- deterministic, no atomics, nothing allocated.
 * Covered: FP32, BF16 and FP16 inputs, M > 64, operands whose stored rows
 * are 16-byte aligned with pitches below 2^24 elements (2^23 for FP32).
 * Anything else (M <= 64, unaligned operands, alpha == 0 or K == 0) runs as
 * gemm_ex with GEMM_VARIANT_AUTO and needs no workspace.  The workspace (device memory,
 * 16-byte aligned, at least gemm_streamk_workspace_size bytes: two
 * 256 x 256 fp32 tiles per workgroup, 128 MiB at most) must not overlap A, B
 * or C and must stay untouched until the work on `stream` has finished; its
 * contents on return are unspecified.  Errors as for gemm_splitk.
 * gemm_f32 / gemm_bf16 / gemm_f16 and GEMM_VARIANT_AUTO take no workspace
 * and never split K; for the shapes above this call is the faster form. */
int gemm_streamk(int dtype, int trans_a, int trans_b, int M, int N, int K,
                 float alpha, const void* A, int lda, const void* B, int ldb,
                 float beta, float* C, int ldc, void* workspace,
                 int64_t workspace_bytes, void* stream);

/* Bytes of workspace gemm_streamk needs for this shape (0 when the call
 * runs as gemm_ex), or a negative status for bad arguments.  Host only. */
int64_t gemm_streamk_workspace_size(int dtype, int M, int N, int K);

/* The rung GEMM_VARIANT_AUTO picks for this call (dtype: enum gemm_dtype;
 * trans_a, trans_b as for gemm_ex), or a negative status if the arguments
 * are invalid.  Host only: touches no device and queues nothing. */
int gemm_select_variant(int dtype, int trans_a, int trans_b, int M, int N,
                        int K, int lda, int ldb, int ldc);

/* Static string naming a status code (never NULL). */
const char* gemm_status_string(int status);

/* DGT_GEMM_ABI_VERSION of the built library. */
int gemm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DGT_GEMM_H */
