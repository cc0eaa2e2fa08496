// gemm_common.hpp -- types and small device helpers shared by the kernels.
//
// All kernels compute C <- alpha*A*B + beta*C on row-major operands
// (A(i,k) = A[i*lda+k], B(k,j) = B[k*ldb+j], C(i,j) = C[i*ldc+j]) with fp32
// accumulation; inputs are fp32 or raw bf16 bits.  Offsets are 64-bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dgt {

struct GemmParams {
    int M, N, K;
    float alpha, beta;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
};

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bits are the upper half of an fp32 value: widening is a shift.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// Scalar input load widened to fp32.
__device__ __forceinline__ float load_in(const float* p) { return *p; }
__device__ __forceinline__ float load_in(const uint16_t* p) {
    return bf16_bits_to_f32(*p);
}

// Epilogue of the BLAS form: alpha*acc + beta*c, where C is read only when
// beta != 0 (so NaN/Inf in a write-only C never propagate).
__device__ __forceinline__ float epilogue(float acc, float alpha, float beta,
                                          const float* c) {
    return beta == 0.0f ? alpha * acc : alpha * acc + beta * (*c);
}

// Host-side launchers; each returns the hipError_t of its launch.
hipError_t launch_scale(const GemmParams& p, hipStream_t s);
hipError_t launch_naive_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_naive_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_lds_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_lds_bf16(const GemmParams& p, hipStream_t s);
hipError_t launch_mfma_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_mfma_bf16(const GemmParams& p, hipStream_t s);
bool mfma_bf16_dma_eligible(const GemmParams& p);
hipError_t launch_mfma_bf16_dma(const GemmParams& p, hipStream_t s);
hipError_t launch_skinny_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_skinny_bf16(const GemmParams& p, hipStream_t s);

// Largest M the skinny (decode) path accepts.
constexpr int kSkinnyMaxM = 16;

// True when every row start of a row-major operand is 16-byte aligned, so
// 128-bit loads are legal at any chunk whose column is a multiple of
// 16 / elem_size.
inline bool rows_16b_aligned(const void* base, int64_t ld, int elem_size) {
    return (reinterpret_cast<uintptr_t>(base) % 16 == 0) &&
           ((ld * elem_size) % 16 == 0);
}

}  // namespace dgt
