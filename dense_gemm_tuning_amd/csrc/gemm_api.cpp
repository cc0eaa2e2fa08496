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

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// The rung AUTO resolves to; the alpha == 0 / K == 0 case is handled before.
// Both input types have a skinny kernel, so the choice depends on M only.
int auto_variant(int M) {
    return M <= dgt::kSkinnyMaxM ? GEMM_VARIANT_SKINNY : GEMM_VARIANT_MFMA;
}

int run(DType t, int ta, int tb, int variant, int M, int N, int K, float alpha,
        const void* A, int lda, const void* B, int ldb, float beta, float* C, int ldc,
        void* stream) {
    int st = check_shape(ta, tb, M, N, K, lda, ldb, ldc);
    if (st != GEMM_OK) return st;
    if (variant < GEMM_VARIANT_AUTO || variant > GEMM_VARIANT_SKINNY)
        return GEMM_ERR_VARIANT;
    if (M == 0 || N == 0) return GEMM_OK;  // empty C: nothing to do
    const bool reads_ab = (alpha != 0.0f) && (K > 0);
    if (C == nullptr) return GEMM_ERR_NULL;
    if (reads_ab && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL;
    const int esz = elem_size(t);
    const uint64_t c_bytes = span_bytes(M, N, ldc, 4);
    const uint64_t a_bytes = ta ? span_bytes(K, M, lda, esz) : span_bytes(M, K, lda, esz);
    const uint64_t b_bytes = tb ? span_bytes(N, K, ldb, esz) : span_bytes(K, N, ldb, esz);
    if (reads_ab && (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes)))
        return GEMM_ERR_OVERLAP;
    if (variant == GEMM_VARIANT_SKINNY && M > dgt::kSkinnyMaxM) return GEMM_ERR_VARIANT;

    GemmParams p;
    p.M = M; p.N = N; p.K = K;
    p.alpha = alpha; p.beta = beta;
    p.A = A; p.lda = lda;
    p.B = B; p.ldb = ldb;
    p.C = C; p.ldc = ldc;
    p.ta = ta; p.tb = tb;
    hipStream_t s = static_cast<hipStream_t>(stream);

    hipError_t e;
    if (!reads_ab) {
        e = dgt::launch_scale(p, s);
    } else {
        if (variant == GEMM_VARIANT_AUTO) variant = auto_variant(M);
        using dgt::In;
        switch (variant) {
            case GEMM_VARIANT_NAIVE:
                e = t == DType::F32    ? dgt::launch_naive<In::F32>(p, s)
                    : t == DType::BF16 ? dgt::launch_naive<In::BF16>(p, s)
                                       : dgt::launch_naive<In::F16>(p, s);
                break;
            case GEMM_VARIANT_LDS:
                e = t == DType::F32    ? dgt::launch_lds<In::F32>(p, s)
                    : t == DType::BF16 ? dgt::launch_lds<In::BF16>(p, s)
                                       : dgt::launch_lds<In::F16>(p, s);
                break;
            case GEMM_VARIANT_MFMA:
                e = t == DType::F32    ? dgt::launch_mfma_f32(p, s)
                    : t == DType::BF16 ? dgt::launch_mfma16<In::BF16>(p, s)
                                       : dgt::launch_mfma16<In::F16>(p, s);
                break;
            case GEMM_VARIANT_SKINNY:
                e = t == DType::F32    ? dgt::launch_skinny_f32(p, s)
                    : t == DType::BF16 ? dgt::launch_skinny16<In::BF16>(p, s)
                                       : dgt::launch_skinny16<In::F16>(p, s);
                break;
            default:
                return GEMM_ERR_VARIANT;
        }
    }
    if (e == hipErrorInvalidConfiguration) return GEMM_ERR_VARIANT;
    return e == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int gemm_f32(int M, int N, int K, float alpha, const float* A, int lda,
             const float* B, int ldb, float beta, float* C, int ldc, void* stream) {
    return run(DType::F32, 0, 0, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta,
               C, ldc, stream);
}

int gemm_bf16(int M, int N, int K, float alpha, const uint16_t* A, int lda,
              const uint16_t* B, int ldb, float beta, float* C, int ldc, void* stream) {
    return run(DType::BF16, 0, 0, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta,
               C, ldc, stream);
}

int gemm_f16(int M, int N, int K, float alpha, const uint16_t* A, int lda,
             const uint16_t* B, int ldb, float beta, float* C, int ldc, void* stream) {
    return run(DType::F16, 0, 0, GEMM_VARIANT_AUTO, M, N, K, alpha, A, lda, B, ldb, beta,
               C, ldc, stream);
}

int gemm_f16_variant(int variant, int M, int N, int K, float alpha, const uint16_t* A,
                     int lda, const uint16_t* B, int ldb, float beta, float* C, int ldc,
                     void* stream) {
    return run(DType::F16, 0, 0, variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               stream);
}

int gemm_f32_variant(int variant, int M, int N, int K, float alpha, const float* A,
                     int lda, const float* B, int ldb, float beta, float* C, int ldc,
                     void* stream) {
    return run(DType::F32, 0, 0, variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               stream);
}

int gemm_bf16_variant(int variant, int M, int N, int K, float alpha,
                      const uint16_t* A, int lda, const uint16_t* B, int ldb,
                      float beta, float* C, int ldc, void* stream) {
    return run(DType::BF16, 0, 0, variant, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               stream);
}

int gemm_ex(int dtype, int trans_a, int trans_b, int variant, int M, int N, int K,
            float alpha, const void* A, int lda, const void* B, int ldb, float beta,
            float* C, int ldc, void* stream) {
    if (dtype < GEMM_DTYPE_F32 || dtype > GEMM_DTYPE_F16) return GEMM_ERR_ARG;
    const DType t = dtype == GEMM_DTYPE_F32    ? DType::F32
                    : dtype == GEMM_DTYPE_BF16 ? DType::BF16
                                               : DType::F16;
    return run(t, trans_a, trans_b, variant, M, N, K, alpha, A, lda, B, ldb, beta, C,
               ldc, stream);
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
        case GEMM_ERR_ARG: return "GEMM_ERR_ARG: unknown dtype or transpose flag";
        default: return "unknown gemm status";
    }
}

int gemm_abi_version(void) { return DGT_GEMM_ABI_VERSION; }

}  // extern "C"
