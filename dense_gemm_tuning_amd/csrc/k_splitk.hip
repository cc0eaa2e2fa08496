// k_splitk.hip -- the second phase of split-K: sum the partial products of
// the K slices and apply the BLAS epilogue.
//
// Split-K is for shapes with too few output tiles to fill the 256 compute
// units (a 1000 x 1000 C has 64 tiles of 128 x 128): the first phase runs
// the ordinary kernels as a strided batch, one problem per K slice, writing
// fp32 partial products W_z (M x N, packed) into a caller-provided
// workspace; this kernel then forms
//
//     C(i,j) <- alpha * (W_0(i,j) + W_1(i,j) + ... + W_{S-1}(i,j)) + beta * C(i,j)
//
// summing the slices in a fixed order, so results are deterministic.  It is
// bound by HBM: S reads of M*N floats and one write (a read too when
// beta != 0), in 16-byte pieces along rows when the row pitch allows.
#include <mutex>

#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int NT = 256;

// The split-K partials of gemm_splitk_noalloc: a fixed device array instead
// of a caller's workspace, for callers that cannot allocate (code under HIP
// graph capture, serving loops, harnesses that forbid allocation).  Every
// GPU the library runs on holds its own copy until the process ends; every
// call on that GPU shares it, so such calls must not overlap in time.
// Phase 1 writes every element of every slice it later reads, so nothing in
// it needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The scratch array's device address on each GPU.  In host code the array's
// name stands for a host-side shadow, never a device address: kernels get
// only the address hipGetSymbolAddress returns for the current device.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

template <bool kVec>
__global__ __launch_bounds__(NT) void splitk_reduce_kernel(const float* W, int splits, int M,
                                                           int N, float alpha, float beta,
                                                           float* C, int64_t ldc) {
    constexpr int V = kVec ? 4 : 1;
    const int64_t slice = (int64_t)M * N;
    const int64_t per_row = (N + V - 1) / V;
    const int64_t total = (int64_t)M * per_row;
    for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * NT) {
        const int64_t i = e / per_row;
        const int j = (int)(e % per_row) * V;
        const float* w = W + i * N + j;
        float* c = C + i * ldc + j;
        if (kVec && j + 4 <= N) {
            float4 s = *reinterpret_cast<const float4*>(w);
            for (int z = 1; z < splits; ++z) {
                const float4 t = *reinterpret_cast<const float4*>(w + z * slice);
                s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
            }
            float4 r;
            if (beta == 0.0f) {
                r = make_float4(alpha * s.x, alpha * s.y, alpha * s.z, alpha * s.w);
            } else {
                const float4 c0 = *reinterpret_cast<const float4*>(c);
                r = make_float4(alpha * s.x + beta * c0.x, alpha * s.y + beta * c0.y,
                                alpha * s.z + beta * c0.z, alpha * s.w + beta * c0.w);
            }
            *reinterpret_cast<float4*>(c) = r;
        } else {
            for (int v = 0; v < V && j + v < N; ++v) {
                float s = w[v];
                for (int z = 1; z < splits; ++z) s += w[v + z * slice];
                c[v] = beta == 0.0f ? alpha * s : alpha * s + beta * c[v];
            }
        }
    }
}

}  // namespace

// Device address of this GPU's scratch array (looked up once per device,
// with that device current), or the HIP error of the lookup.
hipError_t splitk_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    *ptr = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

hipError_t launch_splitk_reduce(const float* W, int splits, int M, int N, float alpha,
                                float beta, float* C, int64_t ldc, hipStream_t s) {
    // float4 pieces need 16-byte aligned rows of C; W rows (N floats) then
    // are too when N is a multiple of 4.
    const bool vec = reinterpret_cast<uintptr_t>(C) % 16 == 0 && ldc % 4 == 0 && N % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(W) % 16 == 0;
    const int64_t items = (int64_t)M * ((N + (vec ? 3 : 0)) / (vec ? 4 : 1));
    int64_t blocks = (items + NT - 1) / NT;
    if (blocks > 8192) blocks = 8192;  // grid-stride loop covers the rest
    if (blocks < 1) blocks = 1;
    if (vec)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(NT), 0, s, W,
                           splits, M, N, alpha, beta, C, ldc);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(NT), 0, s, W,
                           splits, M, N, alpha, beta, C, ldc);
    return hipGetLastError();
}

}  // namespace dgt
