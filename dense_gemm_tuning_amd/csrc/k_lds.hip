// k_lds.hip -- LDS-staged macro tiles with per-lane register tiles on the
// vector ALU (the rung below the matrix cores).
//
// A workgroup owns a 128 x 128 tile of C and walks K in slices of 16.  Each
// slice of A (128 x 16) and B (16 x 128) is fetched once with coalesced
// 128-bit loads and parked in LDS, where every lane of the workgroup reuses
// it (dilfish.github.io section 5.3; elainafan.one "Shared Memory Tiling").
// Each lane owns 8 x 8 outputs and, per k, reads 8 values of A and 8 of B
// from LDS for 64 FMAs, four FMAs per LDS read (dilfish.github.io 5.4); with
// a 128-wide tile the global-side intensity is 32 FLOP/B (same section).
//
// Double buffering (dilfish.github.io 5.4, "software pipeline"): the next
// slice is loaded from global memory into registers while the current one is
// consumed from LDS, then written to the other LDS buffer; one barrier per
// slice suffices because a buffer is only rewritten one slice after its last
// read (the second barrier the pages insist on, dilfish.github.io 5.7 and
// elainafan.one after the tiled listing, is the previous slice's barrier).
//
// LDS layout: both operands k-major (As[k][m], Bs[k][n]) so that a lane's
// 4 consecutive m or n are one 128-bit read.  An operand whose stored rows
// run along k (A, or B stored transposed) is written to LDS transposed; rows
// are padded by 4 floats (132 floats), which makes those transposing writes
// land on distinct banks (dilfish.github.io 5.7 and qwbw.cn's "Pad" row on
// padding the second dimension).  Ragged shapes: out-of-range loads are zero-filled and stores
// masked (dilfish.github.io 5.7; elainafan.one masked tiled listing).
#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int BM = 128, BN = 128, BK = 16, PAD = 4, NT = 256;

// A 16-byte chunk of inputs widened to fp32.
template <In T> struct Chunk {
    static constexpr int V = 8;  // 16-bit formats: 8 per chunk
    __device__ static void unpack(const uint4& u, float* o) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = InFmt<T>::widen((uint16_t)(w[i] & 0xffffu));
            o[2 * i + 1] = InFmt<T>::widen((uint16_t)(w[i] >> 16));
        }
    }
};
template <> struct Chunk<In::F32> {
    static constexpr int V = 4;
    __device__ static void unpack(const uint4& u, float* o) {
        o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
        o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
    }
};

// Load the 16-byte chunk [col, col+V) of one row, zero-filling whatever lies
// outside the row range or beyond `limit` columns.
template <In T, bool kVec>
__device__ __forceinline__ void load_chunk(const typename InFmt<T>::S* rowp, int col,
                                           int limit, bool row_ok, float* out) {
    constexpr int V = Chunk<T>::V;
    if (!row_ok) {
#pragma unroll
        for (int v = 0; v < V; ++v) out[v] = 0.0f;
        return;
    }
    if (kVec && col + V <= limit) {
        Chunk<T>::unpack(*reinterpret_cast<const uint4*>(rowp + col), out);
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
            out[v] = (col + v < limit) ? load_in<T>(rowp + col + v) : 0.0f;
    }
}

// One operand's share of a K slice, fetched as 16-byte chunks along its
// stored rows and parked in LDS as [k][mn] (both operands alike).  kKC: the
// stored rows run along k (A untransposed, B transposed): the slice is 128
// rows of 16 k, written to LDS transposed; otherwise the stored rows run
// along m / n: the slice is 16 rows of 128, written as is.
template <In T, bool kVec, bool kKC>
struct OpSlice {
    using S = typename InFmt<T>::S;
    static constexpr int V = Chunk<T>::V;
    static constexpr int CPR = kKC ? BK / V : BM / V;          // chunks per stored row
    static constexpr int CH = (kKC ? BM : BK) * CPR / NT;      // chunks per lane
    float r[CH][V];

    // mn0: first m (or n) of the tile, mn_lim: M (or N).
    __device__ void load(const S* X, int64_t ld, int mn0, int mn_lim, int k0, int K,
                         int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int f = tid + NT * c, row = f / CPR, q = f % CPR;
            if (kKC) {
                const bool ok = mn0 + row < mn_lim;
                load_chunk<T, kVec>(X + (int64_t)(ok ? mn0 + row : 0) * ld, k0 + q * V, K,
                                    ok, r[c]);
            } else {
                const bool ok = k0 + row < K;
                load_chunk<T, kVec>(X + (int64_t)(ok ? k0 + row : 0) * ld, mn0 + q * V,
                                    mn_lim, ok, r[c]);
            }
        }
    }
    __device__ void store(float (*dst)[BM + PAD], int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int f = tid + NT * c, row = f / CPR, q = f % CPR;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if (kKC) dst[q * V + v][row] = r[c][v];
                else dst[row][q * V + v] = r[c][v];
            }
        }
    }
};

template <In T, bool kVec, bool TA, bool TB>
__global__ __launch_bounds__(NT, 2) void lds_kernel(GemmParams p, int tiles_n) {
    using S = typename InFmt<T>::S;
    select_problem(p);
    __shared__ float As[2][BK][BM + PAD];
    __shared__ float Bs[2][BK][BN + PAD];

    const int tid = threadIdx.x;
    const int m0 = (blockIdx.x / tiles_n) * BM;
    const int n0 = (blockIdx.x % tiles_n) * BN;
    const S* A = static_cast<const S*>(p.A);
    const S* B = static_cast<const S*>(p.B);

    OpSlice<T, kVec, !TA> ra;
    OpSlice<T, kVec, TB> rb;
    auto load_slice = [&](int k0) {
        ra.load(A, p.lda, m0, p.M, k0, p.K, tid);
        rb.load(B, p.ldb, n0, p.N, k0, p.K, tid);
    };
    auto store_slice = [&](int buf) {
        ra.store(As[buf], tid);
        rb.store(Bs[buf], tid);
    };

    const int ty = tid / 16, tx = tid % 16;
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    const int nk = (p.K + BK - 1) / BK;
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
        if (t + 1 < nk) load_slice((t + 1) * BK);
#pragma unroll 2
        for (int k = 0; k < BK; ++k) {
            float a[8], b[8];
            *reinterpret_cast<float4*>(&a[0]) = *reinterpret_cast<const float4*>(&As[buf][k][ty * 4]);
            *reinterpret_cast<float4*>(&a[4]) = *reinterpret_cast<const float4*>(&As[buf][k][64 + ty * 4]);
            *reinterpret_cast<float4*>(&b[0]) = *reinterpret_cast<const float4*>(&Bs[buf][k][tx * 4]);
            *reinterpret_cast<float4*>(&b[4]) = *reinterpret_cast<const float4*>(&Bs[buf][k][64 + tx * 4]);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        if (t + 1 < nk) store_slice(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + (i - 4));
        if (row >= p.M) continue;
        float* crow = p.C + (int64_t)row * p.ldc;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + (j < 4 ? tx * 4 + j : 64 + tx * 4 + (j - 4));
            if (col < p.N) crow[col] = epilogue(acc[i][j], p, crow + col, col);
        }
    }
}

}  // namespace

template <In T>
hipError_t launch_lds(const GemmParams& p, hipStream_t s) {
    const int tiles_n = (p.N + BN - 1) / BN;
    const int64_t blocks = (int64_t)((p.M + BM - 1) / BM) * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool vec = operands_16b_aligned(p, sizeof(typename InFmt<T>::S));
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (vec)
            hipLaunchKernelGGL((lds_kernel<T, true, TA, TB>), dim3((unsigned)blocks, p.batch),
                               dim3(NT), 0, s, p, tiles_n);
        else
            hipLaunchKernelGGL((lds_kernel<T, false, TA, TB>), dim3((unsigned)blocks, p.batch),
                               dim3(NT), 0, s, p, tiles_n);
        return hipGetLastError();
    });
}
template hipError_t launch_lds<In::F32>(const GemmParams&, hipStream_t);
template hipError_t launch_lds<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_lds<In::F16>(const GemmParams&, hipStream_t);

}  // namespace dgt
