// gemm_api.cpp -- the C ABI declared in include/dgt_gemm.h: host-side
// argument checks, the choice of kernel, and the launch on the caller's
// stream.  Nothing here allocates, synchronises or keeps state.
//
// Argument checks run before any HIP call, so an invalid call never touches
// the device (and the checks can be exercised on a machine without a GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/dgt_gemm.h"
#include "gemm_common.hpp"

static_assert(dgt::kScratchBytes == DGT_GEMM_NOALLOC_SCRATCH_BYTES,
              "the header states the scratch size of gemm_splitk_noalloc");

namespace {

using dgt::GemmParams;

enum class DType { F32, BF16, F16 };

int elem_size(DType t) { return t == DType::F32 ? 4 : 2; }

bool valid_flag(int f) { return f == 0 || f == 1; }

// Flag, shape and leading-dimension checks (no pointers involved).  A is
// stored M x K (ta == 0) or K x M (ta == 1); B is stored K x N (tb == 0) or
// N x K (tb == 1); ld is the stored row pitch.
int check_shape(int ta, int tb, int M, int N, int K, int lda, int ldb, int ldc) {
    if (!valid_flag(ta) || !valid_flag(tb)) return GEMM_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    if (lda < std::max(1, ta ? M : K) || ldb < std::max(1, tb ? K : N) ||
        ldc < std::max(1, N))
        return GEMM_ERR_LD;
    return GEMM_OK;
}

// Bytes spanned by a rows x cols row-major operand with leading dim ld.
uint64_t span_bytes(int rows, int cols, int ld, int esz) {
    if (rows == 0 || cols == 0) return 0;
    return ((uint64_t)(rows - 1) * (uint64_t)ld + (uint64_t)cols) * (uint64_t)esz;
}

// The rung AUTO resolves to; the alpha == 0 / K == 0 case is handled before.
// Both input types have a skinny kernel, so the choice depends on M only.
int auto_variant(int M) {
    return M <= dgt::kSkinnyMaxM ? GEMM_VARIANT_SKINNY : GEMM_VARIANT_MFMA;
}

// One call of the library: the operation, the batch and the stream.
struct Call {
    DType t;
    int ta, tb, variant;
    int M, N, K;
    float alpha, beta;
    const void* A;
    int lda;
    int64_t stride_a;  // elements
    const void* B;
    int ldb;
    int64_t stride_b;  // elements
    float* C;
    int ldc;
    int64_t stride_c;  // floats
    const float* bias;
    int64_t stride_bias;  // floats
    int batch;
    void* stream;
    int k_last = 0;  // K of the last problem when > 0 (a split-K tail slice)
};

// [lo, hi) byte range covered by `batch` problems of `span` bytes, `stride`
// bytes apart (empty when span == 0).
struct Range {
    uintptr_t lo, hi;
};
Range batch_range(const void* base, uint64_t span, int64_t stride_bytes, int batch) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    if (span == 0 || batch <= 0) return {b, b};
    return {b, b + (uint64_t)(batch - 1) * (uint64_t)stride_bytes + span};
}
bool overlaps(const Range& x, const Range& y) {
    return x.lo < x.hi && y.lo < y.hi && x.lo < y.hi && y.lo < x.hi;
}

// Largest gridDim.y of one launch; longer batches take several launches.
constexpr int kMaxBatchPerLaunch = 65535;

hipError_t dispatch(DType t, int variant, const GemmParams& p, bool reads_ab, hipStream_t s) {
    using dgt::In;
    if (!reads_ab) return dgt::launch_scale(p, s);
    switch (variant) {
        case GEMM_VARIANT_NAIVE:
            return t == DType::F32    ? dgt::launch_naive<In::F32>(p, s)
                   : t == DType::BF16 ? dgt::launch_naive<In::BF16>(p, s)
                                      : dgt::launch_naive<In::F16>(p, s);
        case GEMM_VARIANT_LDS:
            return t == DType::F32    ? dgt::launch_lds<In::F32>(p, s)
                   : t == DType::BF16 ? dgt::launch_lds<In::BF16>(p, s)
                                      : dgt::launch_lds<In::F16>(p, s);
        case GEMM_VARIANT_MFMA:
            return t == DType::F32    ? dgt::launch_mfma_f32(p, s)
                   : t == DType::BF16 ? dgt::launch_mfma16<In::BF16>(p, s)
                                      : dgt::launch_mfma16<In::F16>(p, s);
        case GEMM_VARIANT_SKINNY:
            // B stored N x K with A stored M x K: B streamed through LDS by copies
            if (t == DType::F32) {
                if (dgt::skinny_bt_dma_eligible<In::F32>(p))
                    return dgt::launch_skinny_bt_dma<In::F32>(p, s);
                return dgt::launch_skinny_f32(p, s);
            }
            if (t == DType::BF16 ? dgt::skinny_bt_dma_eligible<In::BF16>(p)
                                 : dgt::skinny_bt_dma_eligible<In::F16>(p))
                return t == DType::BF16 ? dgt::launch_skinny_bt_dma<In::BF16>(p, s)
                                        : dgt::launch_skinny_bt_dma<In::F16>(p, s);
            return t == DType::BF16 ? dgt::launch_skinny16<In::BF16>(p, s)
                                    : dgt::launch_skinny16<In::F16>(p, s);
        case GEMM_VARIANT_MFMA_REGS:
            return t == DType::F32    ? dgt::launch_mfma_f32_regs(p, s)
                   : t == DType::BF16 ? dgt::launch_mfma16_regs<In::BF16>(p, s)
                                      : dgt::launch_mfma16_regs<In::F16>(p, s);
        case GEMM_VARIANT_MFMA_T256:
        case GEMM_VARIANT_MFMA_T128: {
            const int tile = variant == GEMM_VARIANT_MFMA_T128 ? 128 : 256;
            return t == DType::F32    ? dgt::launch_mfma_f32_dma_tile(p, s, tile)
                   : t == DType::BF16 ? dgt::launch_mfma16_dma_tile<In::BF16>(p, s, tile)
                                      : dgt::launch_mfma16_dma_tile<In::F16>(p, s, tile);
        }
        default:
            return hipErrorInvalidConfiguration;
    }
}

// Strides beyond this (in elements) cannot describe device memory; rejecting
// them keeps the range arithmetic below from overflowing.
constexpr int64_t kMaxStride = int64_t(1) << 48;

bool valid_stride(int64_t s) { return s >= 0 && s < kMaxStride; }

int run(const Call& c) {
    if (c.batch < 0 || !valid_stride(c.stride_a) || !valid_stride(c.stride_b) ||
        !valid_stride(c.stride_c) || !valid_stride(c.stride_bias))
        return GEMM_ERR_ARG;
    int st = check_shape(c.ta, c.tb, c.M, c.N, c.K, c.lda, c.ldb, c.ldc);
    if (st != GEMM_OK) return st;
    if (c.k_last < 0 || c.k_last > c.K) return GEMM_ERR_ARG;
    if (c.variant < GEMM_VARIANT_AUTO || c.variant > GEMM_VARIANT_MFMA_REGS)
        return GEMM_ERR_VARIANT;
    if (c.M == 0 || c.N == 0 || c.batch == 0) return GEMM_OK;  // empty C: nothing to do
    const bool reads_ab = (c.alpha != 0.0f) && (c.K > 0);
    if (c.C == nullptr) return GEMM_ERR_NULL;
    if (reads_ab && (c.A == nullptr || c.B == nullptr)) return GEMM_ERR_NULL;
    const int esz = elem_size(c.t);
    const uint64_t c_span = span_bytes(c.M, c.N, c.ldc, 4);
    // the problems of a batch must not write over each other
    if (c.batch > 1 && (uint64_t)c.stride_c * 4 < c_span) return GEMM_ERR_OVERLAP;
    const Range rc = batch_range(c.C, c_span, c.stride_c * 4, c.batch);
    if (reads_ab) {
        // operand z spans span(K_z) bytes from its start; with a shorter last
        // problem (k_last) the others and the last are checked apart
        auto reads = [&](const void* X, int64_t stride, bool rows_k, int rows, int ld) {
            auto span = [&](int k) {
                return rows_k ? span_bytes(k, rows, ld, esz) : span_bytes(rows, k, ld, esz);
            };
            const int64_t sb = stride * esz;
            if (c.k_last == 0) return overlaps(rc, batch_range(X, span(c.K), sb, c.batch));
            const void* last = static_cast<const char*>(X) + (int64_t)(c.batch - 1) * sb;
            return overlaps(rc, batch_range(X, span(c.K), sb, c.batch - 1)) ||
                   overlaps(rc, batch_range(last, span(c.k_last), 0, 1));
        };
        if (reads(c.A, c.stride_a, c.ta, c.M, c.lda) || reads(c.B, c.stride_b, !c.tb, c.N, c.ldb))
            return GEMM_ERR_OVERLAP;
    }
    if (c.bias && overlaps(rc, batch_range(c.bias, (uint64_t)c.N * 4, c.stride_bias * 4, c.batch)))
        return GEMM_ERR_OVERLAP;
    int variant = c.variant;
    if (variant == GEMM_VARIANT_SKINNY && c.M > dgt::kSkinnyMaxM) return GEMM_ERR_VARIANT;
    if (variant == GEMM_VARIANT_AUTO) variant = auto_variant(c.M);

    GemmParams p;
    p.M = c.M; p.N = c.N; p.K = c.K;
    p.alpha = c.alpha; p.beta = c.beta;
    p.A = c.A; p.lda = c.lda;
    p.B = c.B; p.ldb = c.ldb;
    p.C = c.C; p.ldc = c.ldc;
    p.ta = c.ta; p.tb = c.tb;
    p.stride_a = c.stride_a * esz;
    p.stride_b = c.stride_b * esz;
    p.stride_c = c.stride_c;
    p.stride_bias = c.stride_bias;
    p.bias = c.bias;
    p.batch = std::min(kMaxBatchPerLaunch, c.batch);
    hipStream_t s = static_cast<hipStream_t>(c.stream);
    // the fixed-tile rungs run only the DMA kernels (16-byte aligned rows)
    if (reads_ab && (variant == GEMM_VARIANT_MFMA_T256 || variant == GEMM_VARIANT_MFMA_T128)) {
        const bool ok = c.t == DType::F32 ? dgt::mfma_f32_dma_eligible(p)
                                          : dgt::mfma16_dma_eligible(p);
        if (!ok) return GEMM_ERR_VARIANT;
    }

    for (int z0 = 0; z0 < c.batch; z0 += kMaxBatchPerLaunch) {
        GemmParams q = p;
        q.batch = std::min(kMaxBatchPerLaunch, c.batch - z0);
        q.A = static_cast<const char*>(p.A) + (int64_t)z0 * p.stride_a;
        q.B = static_cast<const char*>(p.B) + (int64_t)z0 * p.stride_b;
        q.C = p.C + (int64_t)z0 * p.stride_c;
        if (p.bias) q.bias = p.bias + (int64_t)z0 * p.stride_bias;
        q.k_last = z0 + q.batch == c.batch ? c.k_last : 0;
        const hipError_t e = dispatch(c.t, variant, q, reads_ab, s);
        if (e == hipErrorInvalidConfiguration) return GEMM_ERR_VARIANT;
        if (e != hipSuccess) return GEMM_ERR_LAUNCH;
    }
    return GEMM_OK;
}

// The single-problem entry points.
int run1(DType t, int ta, int tb, int variant, int M, int N, int K, float alpha,
         const void* A, int lda, const void* B, int ldb, float beta, float* C, int ldc,
         void* stream) {
    Call c{t, ta, tb, variant, M, N, K, alpha, beta, A, lda, 0, B, ldb, 0, C, ldc, 0,
           nullptr, 0, 1, stream};
    return run(c);
}

// ------------------------------------------------------------- split-K

// K slices: kc columns of op(A) / rows of op(B) each (a multiple of 128, so
// every slice keeps the whole-tile kernels' K granularity and 16-byte
// alignment), the last one shorter when K is not a multiple.
struct SplitPlan {
    int splits, kc;
};

// Workgroup slots of the kernel AUTO picks, and its output tiles.
void tile_budget(DType t, int M, int N, int64_t& tiles, int64_t& slots) {
    if (M <= dgt::kSkinnyMaxM) {  // skinny: a column strip per workgroup
        const int cols = t == DType::F32 ? 64 : 128;
        tiles = (N + cols - 1) / cols;
        slots = 256;
    } else {  // 128 x 128 tiles (the smaller DMA tile)
        tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
        // 16-bit: two workgroups per CU.  FP32: one; a second on the same CU
        // only shares its matrix cores (an FP32 MFMA is twice as long as a
        // 16-bit one per k) while doubling the partials the reduction reads
        // (1000^3: 4 slices 32 us, 8 slices 37 us; 512^2 x 8192: 16 slices
        // 42 us, 32 slices 48 us).
        slots = t == DType::F32 ? 256 : 512;
    }
}

constexpr int kSliceAlign = 128;   // K granularity of a slice
constexpr int kMinSliceK = 128;    // no slice shorter than this when chosen automatically
constexpr int kMaxSplits = 64;

SplitPlan plan_splitk(DType t, int M, int N, int K, int requested) {
    if (K <= 0 || requested == 1) return {1, K};
    int want = requested;
    if (want == 0) {  // enough slices to fill the workgroup slots
        int64_t tiles, slots;
        tile_budget(t, M, N, tiles, slots);
        const int64_t fill = tiles > 0 ? slots / tiles : 1;
        const int64_t most = (K + kMinSliceK - 1) / kMinSliceK;  // slices of kMinSliceK
        want = (int)std::max<int64_t>(1, std::min<int64_t>(fill, most));
    }
    want = std::min(want, kMaxSplits);
    if (want <= 1) return {1, K};
    int kc = (K + want - 1) / want;
    kc = (kc + kSliceAlign - 1) / kSliceAlign * kSliceAlign;
    const int splits = (K + kc - 1) / kc;
    if (splits <= 1) return {1, K};
    return {splits, kc};
}

bool dtype_of(int dtype, DType& t) {
    if (dtype < GEMM_DTYPE_F32 || dtype > GEMM_DTYPE_F16) return false;
    t = dtype == GEMM_DTYPE_F32 ? DType::F32 : dtype == GEMM_DTYPE_BF16 ? DType::BF16 : DType::F16;
    return true;
}

// Both split-K entry points.  noalloc: the partials go to the library's fixed
// scratch (shapes whose partials exceed it are refused, nothing is
// allocated); otherwise to the caller's workspace of workspace_bytes.
int splitk(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
           const void* A, int lda, const void* B, int ldb, float beta, float* C, int ldc,
           int splits, void* workspace, int64_t workspace_bytes, bool noalloc, void* stream) {
    DType t;
    if (!dtype_of(dtype, t) || splits < 0 || workspace_bytes < 0) return GEMM_ERR_ARG;
    int st = check_shape(trans_a, trans_b, M, N, K, lda, ldb, ldc);
    if (st != GEMM_OK) return st;
    const SplitPlan plan = plan_splitk(t, M, N, K, splits);
    const bool reads_ab = alpha != 0.0f && K > 0;
    if (plan.splits == 1 || !reads_ab || M == 0 || N == 0)
        return run1(t, trans_a, trans_b, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb,
                    beta, C, ldc, stream);
    if (C == nullptr || A == nullptr || B == nullptr) return GEMM_ERR_NULL;
    const int64_t ws_need = (int64_t)plan.splits * M * N * 4;
    if (noalloc) {
        if (ws_need > dgt::kScratchBytes) return GEMM_ERR_SCRATCH;
        if (dgt::splitk_scratch(&workspace) != hipSuccess || workspace == nullptr)
            return GEMM_ERR_LAUNCH;
        workspace_bytes = dgt::kScratchBytes;
    }
    if (workspace == nullptr || workspace_bytes < ws_need) return GEMM_ERR_WORKSPACE;
    float* W = static_cast<float*>(workspace);
    const int esz = elem_size(t);
    const Range rw = batch_range(W, (uint64_t)ws_need, 0, 1);
    const Range rc = batch_range(C, span_bytes(M, N, ldc, 4), 0, 1);
    const uint64_t a_span = trans_a ? span_bytes(K, M, lda, esz) : span_bytes(M, K, lda, esz);
    const uint64_t b_span = trans_b ? span_bytes(N, K, ldb, esz) : span_bytes(K, N, ldb, esz);
    if (overlaps(rw, rc) || overlaps(rw, batch_range(A, a_span, 0, 1)) ||
        overlaps(rw, batch_range(B, b_span, 0, 1)))
        return GEMM_ERR_OVERLAP;

    // Phase 1: slice z covers k in [z*kc, z*kc + K_z), into W + z*M*N: one
    // strided batch, whose last problem takes the shorter last slice.
    const int64_t sa = trans_a ? (int64_t)plan.kc * lda : plan.kc;   // elements
    const int64_t sb = trans_b ? plan.kc : (int64_t)plan.kc * ldb;
    const int last_k = K - (plan.splits - 1) * plan.kc;
    Call c{t, trans_a, trans_b, GEMM_VARIANT_AUTO, M, N, plan.kc, 1.0f, 0.0f, A, lda, sa, B,
           ldb, sb, W, N, (int64_t)M * N, nullptr, 0, plan.splits, stream};
    c.k_last = last_k == plan.kc ? 0 : last_k;
    st = run(c);
    if (st != GEMM_OK) return st;
    // Phase 2: C <- alpha * sum_z W_z + beta * C, in slice order.
    const hipError_t e = dgt::launch_splitk_reduce(W, plan.splits, M, N, alpha, beta, C, ldc,
                                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_splitk_slices(int dtype, int M, int N, int K, int splits) {
    DType t;
    if (!dtype_of(dtype, t) || splits < 0) return GEMM_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    return plan_splitk(t, M, N, K, splits).splits;
}

int64_t gemm_splitk_workspace_size(int dtype, int M, int N, int K, int splits) {
    const int s = gemm_splitk_slices(dtype, M, N, K, splits);
    if (s < 0) return s;
    return s > 1 ? (int64_t)s * M * N * 4 : 0;
}

int gemm_splitk(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                const void* A, int lda, const void* B, int ldb, float beta, float* C, int ldc,
                int splits, void* workspace, int64_t workspace_bytes, void* stream) {
    return splitk(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                  workspace, workspace_bytes, false, stream);
}

int64_t gemm_streamk_workspace_size(int dtype, int M, int N, int K) {
    DType t;
    if (!dtype_of(dtype, t)) return GEMM_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    if (M <= dgt::kSkinnyMaxM || N == 0 || K == 0) return 0;
    GemmParams p;
    p.M = M; p.N = N; p.K = K;
    return dgt::streamk_workspace_bytes(p, t == DType::F32);
}

int gemm_streamk(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                 const void* A, int lda, const void* B, int ldb, float beta, float* C, int ldc,
                 void* workspace, int64_t workspace_bytes, void* stream) {
    DType t;
    if (!dtype_of(dtype, t) || workspace_bytes < 0) return GEMM_ERR_ARG;
    int st = check_shape(trans_a, trans_b, M, N, K, lda, ldb, ldc);
    if (st != GEMM_OK) return st;
    const bool reads_ab = alpha != 0.0f && K > 0;
    GemmParams p;
    p.M = M; p.N = N; p.K = K;
    p.alpha = alpha; p.beta = beta;
    p.A = A; p.lda = lda;
    p.B = B; p.ldb = ldb;
    p.C = C; p.ldc = ldc;
    p.ta = trans_a; p.tb = trans_b;
    p.stride_a = p.stride_b = p.stride_c = p.stride_bias = 0;
    p.bias = nullptr;
    p.batch = 1;
    // what stream-K does not cover runs as gemm_ex with the automatic choice
    const bool dma = t == DType::F32 ? dgt::mfma_f32_dma_eligible(p) : dgt::mfma16_dma_eligible(p);
    if (M <= dgt::kSkinnyMaxM || !reads_ab || M == 0 || N == 0 || !dma)
        return run1(t, trans_a, trans_b, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb,
                    beta, C, ldc, stream);
    if (C == nullptr || A == nullptr || B == nullptr) return GEMM_ERR_NULL;
    const int64_t ws_need = dgt::streamk_workspace_bytes(p, t == DType::F32);
    if (workspace == nullptr || workspace_bytes < ws_need ||
        reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return GEMM_ERR_WORKSPACE;
    const int esz = elem_size(t);
    const Range rw = batch_range(workspace, (uint64_t)ws_need, 0, 1);
    const Range rc = batch_range(C, span_bytes(M, N, ldc, 4), 0, 1);
    const uint64_t a_span = trans_a ? span_bytes(K, M, lda, esz) : span_bytes(M, K, lda, esz);
    const uint64_t b_span = trans_b ? span_bytes(N, K, ldb, esz) : span_bytes(K, N, ldb, esz);
    const Range ra = batch_range(A, a_span, 0, 1), rb = batch_range(B, b_span, 0, 1);
    if (overlaps(rc, ra) || overlaps(rc, rb) || overlaps(rw, rc) || overlaps(rw, ra) ||
        overlaps(rw, rb))
        return GEMM_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);
    const hipError_t e = t == DType::F32    ? dgt::launch_mfma_f32_streamk(p, ws, s)
                         : t == DType::BF16 ? dgt::launch_mfma16_streamk<dgt::In::BF16>(p, ws, s)
                                            : dgt::launch_mfma16_streamk<dgt::In::F16>(p, ws, s);
    if (e == hipErrorInvalidConfiguration) return GEMM_ERR_VARIANT;
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_splitk_noalloc(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const void* A, int lda, const void* B, int ldb, float beta, float* C,
                        int ldc, int splits, void* stream) {
    return splitk(dtype, trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                  nullptr, 0, true, stream);
}

int gemm_f32(int M, int N, int K, float alpha, const float* A, int lda,
             const float* B, int ldb, float beta, float* C, int ldc, void* stream) {
    return run1(DType::F32, 0, 0, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta,
               C, ldc, stream);
}

int gemm_bf16(int M, int N, int K, float alpha, const uint16_t* A, int lda,
              const uint16_t* B, int ldb, float beta, float* C, int ldc, void* stream) {
    return run1(DType::BF16, 0, 0, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta,
               C, ldc, stream);
}

int gemm_f16(int M, int N, int K, float alpha, const uint16_t* A, int lda,
             const uint16_t* B, int ldb, float beta, float* C, int ldc, void* stream) {
    return run1(DType::F16, 0, 0, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta,
               C, ldc, stream);
}

int gemm_f16_variant(int variant, int M, int N, int K, float alpha, const uint16_t* A,
                     int lda, const uint16_t* B, int ldb, float beta, float* C, int ldc,
                     void* stream) {
    return run1(DType::F16, 0, 0, variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               stream);
}

int gemm_f32_variant(int variant, int M, int N, int K, float alpha, const float* A,
                     int lda, const float* B, int ldb, float beta, float* C, int ldc,
                     void* stream) {
    return run1(DType::F32, 0, 0, variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               stream);
}

int gemm_bf16_variant(int variant, int M, int N, int K, float alpha,
                      const uint16_t* A, int lda, const uint16_t* B, int ldb,
                      float beta, float* C, int ldc, void* stream) {
    return run1(DType::BF16, 0, 0, variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               stream);
}

int gemm_ex(int dtype, int trans_a, int trans_b, int variant, int M, int N, int K,
            float alpha, const void* A, int lda, const void* B, int ldb, float beta,
            float* C, int ldc, void* stream) {
    if (dtype < GEMM_DTYPE_F32 || dtype > GEMM_DTYPE_F16) return GEMM_ERR_ARG;
    const DType t = dtype == GEMM_DTYPE_F32    ? DType::F32
                    : dtype == GEMM_DTYPE_BF16 ? DType::BF16
                                               : DType::F16;
    return run1(t, trans_a, trans_b, variant, M, N, K, alpha, A, lda, B, ldb, beta, C,
                ldc, stream);
}

int gemm_strided_batched(int dtype, int trans_a, int trans_b, int variant, int M, int N,
                         int K, float alpha, const void* A, int lda, int64_t stride_a,
                         const void* B, int ldb, int64_t stride_b, float beta, float* C,
                         int ldc, int64_t stride_c, const float* bias, int64_t stride_bias,
                         int batch, void* stream) {
    if (dtype < GEMM_DTYPE_F32 || dtype > GEMM_DTYPE_F16) return GEMM_ERR_ARG;
    if (!valid_flag(trans_a) || !valid_flag(trans_b)) return GEMM_ERR_ARG;
    const DType t = dtype == GEMM_DTYPE_F32    ? DType::F32
                    : dtype == GEMM_DTYPE_BF16 ? DType::BF16
                                               : DType::F16;
    Call c{t, trans_a, trans_b, variant, M, N, K, alpha, beta, A, lda, stride_a, B, ldb,
           stride_b, C, ldc, stride_c, bias, stride_bias, batch, stream};
    return run(c);
}

int gemm_select_variant(int dtype, int trans_a, int trans_b, int M, int N, int K,
                        int lda, int ldb, int ldc) {
    if (dtype < GEMM_DTYPE_F32 || dtype > GEMM_DTYPE_F16) return GEMM_ERR_ARG;
    const int st = check_shape(trans_a, trans_b, M, N, K, lda, ldb, ldc);
    if (st != GEMM_OK) return st;
    return auto_variant(M);
}

const char* gemm_status_string(int status) {
    switch (status) {
        case GEMM_OK: return "GEMM_OK: success";
        case GEMM_ERR_DIM: return "GEMM_ERR_DIM: M, N or K is negative";
        case GEMM_ERR_LD: return "GEMM_ERR_LD: leading dimension too small";
        case GEMM_ERR_NULL: return "GEMM_ERR_NULL: null pointer for a non-empty operand";
        case GEMM_ERR_OVERLAP: return "GEMM_ERR_OVERLAP: C overlaps A or B";
        case GEMM_ERR_VARIANT: return "GEMM_ERR_VARIANT: variant unknown or unsupported for this shape";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: the HIP runtime rejected the launch";
        case GEMM_ERR_ARG: return "GEMM_ERR_ARG: unknown dtype or transpose flag, negative batch, splits or size, or stride out of range";
        case GEMM_ERR_WORKSPACE: return "GEMM_ERR_WORKSPACE: workspace missing or smaller than gemm_splitk_workspace_size";
        case GEMM_ERR_SCRATCH: return "GEMM_ERR_SCRATCH: gemm_splitk_noalloc: the partials (slices x M x N x 4 bytes) exceed the library's fixed scratch of DGT_GEMM_NOALLOC_SCRATCH_BYTES";
        default: return "unknown gemm status";
    }
}

int gemm_abi_version(void) { return DGT_GEMM_ABI_VERSION; }

}  // extern "C"
