// k_naive.hip -- baseline rung: one lane per output element, plus the
// alpha == 0 / K == 0 scaling kernel.
//
// The naive mapping (dilfish.github.io section 5.2; chongfengling.github.io
// section 2.1) gives every output C(i,j) its own lane, which walks k and does
// two global loads and one FMA per step.  The column index, contiguous in
// row-major memory, is bound to the lane index so that a wavefront reads one
// contiguous run of B and one broadcast element of A per step
// (chongfengling.github.io sections 2.2 and 2.4).  On gfx950 a wavefront is
// 64 lanes, so the x-extent of the workgroup is 64, not 16 or 32.  Ragged
// shapes are handled by the per-lane bounds check (chongfengling.github.io
// section 2.1; elainafan.one, paragraph after the naive launch).  Arithmetic
// intensity is 0.25 FLOP/B from the per-lane view (dilfish.github.io 5.2);
// caches recover part of that, the layout does not.  Transposed operands
// only change the stride along k; with B stored N x K the wavefront's B
// reads are strided (this rung does not restage them).
#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int kNaiveX = 64;  // one wavefront along the contiguous columns
constexpr int kNaiveY = 4;   // four rows per workgroup (256 lanes)

template <In T>
__global__ __launch_bounds__(kNaiveX * kNaiveY) void naive_kernel(GemmParams p,
                                                                  int tiles_n) {
    using S = typename InFmt<T>::S;
    select_problem(p);
    const int bn = blockIdx.x % tiles_n;
    const int bm = blockIdx.x / tiles_n;
    const int col = bn * kNaiveX + threadIdx.x;
    const int row = bm * kNaiveY + threadIdx.y;
    if (row >= p.M || col >= p.N) return;
    // op(A)(row, k) and op(B)(k, col) walk k with a stride of 1 or ld,
    // depending on how each operand is stored.
    const S* a = static_cast<const S*>(p.A) + (p.ta ? (int64_t)row : (int64_t)row * p.lda);
    const S* b = static_cast<const S*>(p.B) + (p.tb ? (int64_t)col * p.ldb : (int64_t)col);
    const int64_t sa = p.ta ? p.lda : 1, sb = p.tb ? 1 : p.ldb;
    float acc = 0.0f;
    for (int k = 0; k < p.K; ++k)
        acc = fmaf(load_in<T>(a + k * sa), load_in<T>(b + k * sb), acc);
    float* c = p.C + (int64_t)row * p.ldc + col;
    *c = epilogue(acc, p, c, col);
}

// C <- beta*C (+ bias) when A*B contributes nothing (alpha == 0 or K == 0);
// beta == 0 writes zeros (or the bias) without reading C.
__global__ __launch_bounds__(256) void scale_kernel(GemmParams p) {
    select_problem(p);
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / p.N, j = e % p.N;
        float* c = p.C + i * p.ldc + j;
        const float r = p.beta == 0.0f ? 0.0f : p.beta * (*c);
        *c = p.bias ? r + p.bias[j] : r;
    }
}

}  // namespace

template <In T>
hipError_t launch_naive(const GemmParams& p, hipStream_t s) {
    const int tiles_n = (p.N + kNaiveX - 1) / kNaiveX;
    const int64_t tiles_m = (p.M + kNaiveY - 1) / kNaiveY;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(naive_kernel<T>, dim3((unsigned)blocks, p.batch),
                       dim3(kNaiveX, kNaiveY), 0, s, p, tiles_n);
    return hipGetLastError();
}
template hipError_t launch_naive<In::F32>(const GemmParams&, hipStream_t);
template hipError_t launch_naive<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_naive<In::F16>(const GemmParams&, hipStream_t);

hipError_t launch_scale(const GemmParams& p, hipStream_t s) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;  // grid-stride loop covers the rest
    hipLaunchKernelGGL(scale_kernel, dim3((unsigned)blocks, p.batch), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace dgt
