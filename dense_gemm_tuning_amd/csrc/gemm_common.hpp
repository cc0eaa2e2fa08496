// gemm_common.hpp -- types and small device helpers shared by the kernels.
//
// All kernels compute C <- alpha*op(A)*op(B) + beta*C on row-major storage
// with fp32 accumulation; inputs are fp32, or raw bf16 / IEEE binary16 bits.
// op(A)(i,k) = A[i*lda+k] (ta == 0) or A[k*lda+i] (ta == 1, A stored K x M);
// op(B)(k,j) = B[k*ldb+j] (tb == 0) or B[j*ldb+k] (tb == 1, B stored N x K);
// C(i,j) = C[i*ldc+j].  Offsets are 64-bit.
//
// The tiled kernels treat the two operands alike: what matters for staging
// is whether an operand's stored rows run along k ("K-contiguous": A with
// ta == 0, B with tb == 1) or along m / n ("MN-contiguous": A with ta == 1,
// B with tb == 0), not whether it is A or B.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
    int ta, tb;  // 1: the operand is stored transposed
    // Strided batch: problem z of a launch (blockIdx.y, z < batch) reads
    // A + z*stride_a bytes and B + z*stride_b bytes, writes C + z*stride_c
    // floats and adds bias + z*stride_bias floats.  bias (N floats per
    // problem, broadcast over the rows of C) is optional: nullptr = none.
    int64_t stride_a, stride_b, stride_c, stride_bias;
    const float* bias;
    int batch;
    // K of the launch's last problem when > 0 (split-K's shorter last
    // slice); otherwise every problem has K.
    int k_last = 0;
};

// Point p at problem z of a strided batch.
__device__ __forceinline__ void select_problem(GemmParams& p, int64_t z) {
    if (p.k_last > 0 && z == p.batch - 1) p.K = p.k_last;
    p.A = static_cast<const char*>(p.A) + z * p.stride_a;
    p.B = static_cast<const char*>(p.B) + z * p.stride_b;
    p.C += z * p.stride_c;
    if (p.bias) p.bias += z * p.stride_bias;
}
__device__ __forceinline__ void select_problem(GemmParams& p) { select_problem(p, blockIdx.y); }

// Tile order.  A launch's workgroups go to the 8 XCDs (each with its own L2)
// round-robin by linear id.
//  * linear (grouped == false): workgroup x of problem blockIdx.y takes tile
//    (x / tiles_n, x % tiles_n).  For one problem an XCD then holds tiles of
//    8 tile-rows x 4 tile-columns (columns 8 apart), but in a batch its
//    tiles come from several problems and share few panels.
//  * grouped: XCD x takes a contiguous range of the launch's tiles
//    (problem-major), and inside a problem the tiles run in groups of
//    kGroupM tile-rows, column by column, so the tiles an XCD holds at one
//    time form a compact block of one problem (8 x 4 for 32 resident tiles).
// Measured on the whole-tile 16-bit kernel: grouped is 4-6% faster for a
// batch of 16 x 2048^3, the same for one 8192^3 problem with A or B stored
// m/n-contiguous, and 5% slower for one 8192^3 problem with both operands
// k-contiguous (B stored N x K), which therefore keeps the linear order.
// Both maps are bijections on [0, tiles) for any tile count.
struct TileIdx {
    int z, bm, bn;
};
constexpr int kXcds = 8;
constexpr int kGroupM = 8;
__device__ __forceinline__ TileIdx xcd_tile(int tiles_m, int tiles_n, bool grouped) {
    if (!grouped) return TileIdx{(int)blockIdx.y, (int)(blockIdx.x / tiles_n),
                                 (int)(blockIdx.x % tiles_n)};
    const int64_t per_problem = (int64_t)tiles_m * tiles_n;
    const int64_t total = per_problem * gridDim.y;
    const int64_t lin = blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
    const int64_t x = lin % kXcds, q = lin / kXcds;
    const int64_t per = total / kXcds, rem = total % kXcds;
    const int64_t g = x < rem ? x * (per + 1) + q : rem * (per + 1) + (x - rem) * per + q;
    TileIdx t;
    t.z = (int)(g / per_problem);
    const int64_t idx = g % per_problem;
    const int64_t group = idx / ((int64_t)kGroupM * tiles_n);
    const int first_m = (int)(group * kGroupM);
    const int gm = min(tiles_m - first_m, kGroupM);
    const int64_t in_group = idx - group * kGroupM * tiles_n;
    t.bm = first_m + (int)(in_group % gm);
    t.bn = (int)(in_group / gm);
    return t;
}

// Calls fn(TA, TB) with std::bool_constant arguments matching p.ta, p.tb, so
// that launchers can pick a kernel specialised for the operand layout.
template <typename Fn>
inline hipError_t with_layout(const GemmParams& p, Fn&& fn) {
    using T = std::true_type;
    using F = std::false_type;
    if (p.ta) return p.tb ? fn(T{}, T{}) : fn(T{}, F{});
    return p.tb ? fn(F{}, T{}) : fn(F{}, F{});
}

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

// Input formats.  The 16-bit ones are passed as raw uint16_t bit patterns.
enum class In { F32, BF16, F16 };

// bf16 bits are the upper half of an fp32 value: widening is a shift.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

template <In T> struct InFmt;
template <> struct InFmt<In::F32> {
    using S = float;
    __device__ static float widen(float x) { return x; }
};
template <> struct InFmt<In::BF16> {
    using S = uint16_t;
    __device__ static float widen(uint16_t x) { return bf16_bits_to_f32(x); }
};
template <> struct InFmt<In::F16> {
    using S = uint16_t;
    __device__ static float widen(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }
};

// Scalar input load widened to fp32.
template <In T>
__device__ __forceinline__ float load_in(const typename InFmt<T>::S* p) {
    return InFmt<T>::widen(*p);
}

// Matrix-core products of 8 16-bit values per lane (raw 16-byte operands),
// fp32 accumulate: 32x32x16 and 16x16x32 shapes.
template <In T>
__device__ __forceinline__ floatx16 mfma32x32x16(u32x4 a, u32x4 b, floatx16 c) {
    if constexpr (T == In::BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}
template <In T>
__device__ __forceinline__ floatx4 mfma16x16x32(u32x4 a, u32x4 b, floatx4 c) {
    if constexpr (T == In::BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
}

// Epilogue of the BLAS form plus the optional bias of a linear layer:
// (alpha*acc + beta*c) + bias[col], where C is read only when beta != 0 (so
// NaN/Inf in a write-only C never propagate).
__device__ __forceinline__ float epilogue(float acc, const GemmParams& p, const float* c,
                                          int col) {
    const float r = p.beta == 0.0f ? p.alpha * acc : p.alpha * acc + p.beta * (*c);
    return p.bias ? r + p.bias[col] : r;
}

// Host-side launchers; each returns the hipError_t of its launch.
hipError_t launch_scale(const GemmParams& p, hipStream_t s);
template <In T> hipError_t launch_naive(const GemmParams& p, hipStream_t s);
template <In T> hipError_t launch_lds(const GemmParams& p, hipStream_t s);
hipError_t launch_mfma_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_mfma_f32_regs(const GemmParams& p, hipStream_t s);
bool mfma_f32_dma_eligible(const GemmParams& p);
hipError_t launch_mfma_f32_dma(const GemmParams& p, hipStream_t s);
hipError_t launch_mfma_f32_dma_tile(const GemmParams& p, hipStream_t s, int tile);
template <In T> hipError_t launch_mfma16(const GemmParams& p, hipStream_t s);
template <In T> hipError_t launch_mfma16_regs(const GemmParams& p, hipStream_t s);
bool mfma16_dma_eligible(const GemmParams& p);
template <In T> hipError_t launch_mfma16_dma(const GemmParams& p, hipStream_t s);
template <In T> hipError_t launch_mfma16_dma_tile(const GemmParams& p, hipStream_t s, int tile);
// Stream-K on 256 x 256 tiles (one problem, DMA-eligible operands) into a
// workspace of streamk_workspace_bytes(p, f32) bytes.
int64_t streamk_workspace_bytes(const GemmParams& p, bool f32);
template <In T> hipError_t launch_mfma16_streamk(const GemmParams& p, float* ws, hipStream_t s);
hipError_t launch_mfma_f32_streamk(const GemmParams& p, float* ws, hipStream_t s);
hipError_t launch_skinny_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_splitk_reduce(const float* W, int splits, int M, int N, float alpha,
                                float beta, float* C, int64_t ldc, hipStream_t s);
// Fixed split-K scratch of gemm_splitk_noalloc: its size, and its device
// address on the current GPU.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
hipError_t splitk_scratch(void** ptr);
template <In T> hipError_t launch_skinny16(const GemmParams& p, hipStream_t s);
template <In T> bool skinny_bt_dma_eligible(const GemmParams& p);
template <In T> hipError_t launch_skinny_bt_dma(const GemmParams& p, hipStream_t s);

// Largest M the skinny (decode) path accepts: four blocks of 16 rows.
constexpr int kSkinnyMaxM = 64;

// Buffer descriptors for the global -> LDS copies (buffer_load ... lds):
// word 3 of a raw 32-bit-data descriptor, and the row pitch (elements) below
// which a workgroup's rows of lane offsets fit the 32-bit buffer offset.
constexpr int kBufferRsrcW3 = 0x00020000;
constexpr int64_t kMaxBufferPitch = int64_t(1) << 24;

// True when every row start of a row-major operand is 16-byte aligned, so
// 128-bit loads are legal at any chunk whose column is a multiple of
// 16 / elem_size.
inline bool rows_16b_aligned(const void* base, int64_t ld, int elem_size) {
    return (reinterpret_cast<uintptr_t>(base) % 16 == 0) &&
           ((ld * elem_size) % 16 == 0);
}

// The same for A and B of every problem of a batch (batch strides are in
// bytes and must keep the alignment too).
// True when every problem's K (the last one's too) is a multiple of q.
inline bool k_multiple(const GemmParams& p, int q) {
    return p.K % q == 0 && (p.k_last <= 0 || p.k_last % q == 0);
}

inline bool operands_16b_aligned(const GemmParams& p, int elem_size) {
    return rows_16b_aligned(p.A, p.lda, elem_size) && rows_16b_aligned(p.B, p.ldb, elem_size) &&
           p.stride_a % 16 == 0 && p.stride_b % 16 == 0;
}

}  // namespace dgt
