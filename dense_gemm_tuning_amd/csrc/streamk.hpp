// streamk.hpp -- the stream-K schedule shared by the 16-bit and the FP32 DMA
// kernels (a persistent grid that deals out K iterations rather than whole
// tiles).
//
// For launches whose 256 x 256 tiles do not divide evenly among the CUs, a
// data-parallel launch runs its last wave of tiles on part of the chip, and
// splitting K in equal slices for every tile multiplies the partial sums.
// Here G = min(256, tiles * I) workgroups (an iteration is one group of the
// tile body's four K slices: 128 k for 16-bit inputs, 64 k for fp32, I per
// tile) first run the whole waves of tiles data-parallel (tile j*G + g of
// wave j to workgroup g: the dp first tiles), then deal out the T remaining
// tiles' T*I iterations: cut into GS = min(G, T*I) equal contiguous ranges,
// workgroup g < GS owns iterations [start(g), start(g+1)), start(g) =
// floor(g * T*I / GS), and walks them tile by tile.  A tile it covers whole
// gets the ordinary epilogue into C; a part of a tile goes, as bare fp32
// sums, to workspace slot 2g (the first tile of its range) or 2g + 1 (the
// last).  A second kernel then sums each split tile's parts in k order
// (workgroup order) and applies the epilogue -- deterministic, no atomics,
// no waiting between workgroups.  Every part runs the tile body on its
// sub-range of k (A and B offset by the part's first k); whole-tile
// launches with K a multiple of the iteration keep the whole-tile instance
// (every part is then whole groups of slices), others take the edge-tile /
// K-tail one.  The data-parallel waves keep the tiles a wave's workgroups
// on one XCD hold at one time in step along k (as in the data-parallel
// kernels), which the dealt-out ranges do not.
#pragma once

#include "dma_common.hpp"

namespace dgt {
namespace streamk {

using dma::kCUs;

constexpr int R = 256;          // workgroup tile, one workgroup per CU
constexpr int kFixSplit = 16;   // fix-up workgroups per tile: 16 rows each
constexpr int kIterK16 = 128;   // k per iteration, 16-bit inputs (four 32-deep slices)
constexpr int kIterKF32 = 64;   // k per iteration, fp32 inputs (four 16-deep slices)

struct StreamK {
    int64_t T, I, W;  // dealt-out tiles (after the first dp), iterations per tile, T*I
    int64_t dp;       // tiles run whole, a multiple of G
    int G;            // workgroups
    int GS;           // workgroups sharing the dealt-out iterations (<= G; 0 when W == 0)
    int tiles_m, tiles_n;
    int IK;           // k per iteration
    __host__ __device__ int64_t start(int g) const { return g * W / GS; }
    // the workgroup owning dealt-out iteration x
    __host__ __device__ int owner(int64_t x) const {
        int g = (int)((x * GS) / W);
        while (g + 1 < GS && start(g + 1) <= x) ++g;
        while (g > 0 && start(g) > x) --g;
        return g;
    }
    // tile t as (tile row, tile column): groups of kGroupM tile rows, column
    // by column inside a group (the tiles a workgroup range and its XCD
    // neighbours cover share A and B panels)
    __host__ __device__ void coords(int64_t t, int& bm, int& bn) const {
        const int64_t group = t / ((int64_t)kGroupM * tiles_n);
        const int first_m = (int)(group * kGroupM);
        const int gm = tiles_m - first_m < kGroupM ? tiles_m - first_m : kGroupM;
        const int64_t in_group = t - group * kGroupM * tiles_n;
        bm = first_m + (int)(in_group % gm);
        bn = (int)(in_group / gm);
    }
    // workspace slot of workgroup g's part of dealt-out tile t
    __host__ __device__ int slot(int g, int64_t t) const {
        return t == start(g) / I ? 2 * g : 2 * g + 1;
    }
    // true when some tile is split between workgroups (the fix-up has work)
    __host__ bool split() const { return W > 0 && !(W % GS == 0 && (W / GS) % I == 0); }
};

inline StreamK plan(const GemmParams& p, int iter_k) {
    StreamK sk;
    sk.tiles_m = (p.M + R - 1) / R;
    sk.tiles_n = (p.N + R - 1) / R;
    const int64_t tiles = (int64_t)sk.tiles_m * sk.tiles_n;
    sk.IK = iter_k;
    sk.I = (p.K + iter_k - 1) / iter_k;
    sk.G = (int)(tiles * sk.I < kCUs ? tiles * sk.I : kCUs);
    sk.dp = sk.G > 0 ? tiles / sk.G * sk.G : 0;
    sk.T = tiles - sk.dp;
    sk.W = sk.T * sk.I;
    sk.GS = (int)(sk.W < sk.G ? sk.W : sk.G);
    return sk;
}

// Two R x R fp32 tiles per workgroup.
inline int64_t workspace_bytes(const GemmParams& p, int iter_k) {
    return (int64_t)2 * plan(p, iter_k).G * R * R * 4;
}

// Workgroup blockIdx.x's range, its parts in order: tile(q, m0, n0, raw)
// runs the tile body on part q (p restricted to the part's k range, A and B
// offset by ESZ-byte elements) with raw == nullptr for a whole tile or its
// workspace slot otherwise.
template <bool TA, bool TB, int ESZ, class Tile>
__device__ __forceinline__ void walk(const GemmParams& p, const StreamK& sk, float* ws,
                                     Tile&& tile) {
    // consecutive tiles / ranges on one XCD (workgroups reach the 8 XCDs
    // round-robin)
    const int per = sk.G / kXcds;
    const int b = blockIdx.x;
    const int g = (sk.G % kXcds == 0) ? (b % kXcds) * per + b / kXcds : b;
    // whole tiles g, g + G, ... below dp, then the dealt-out range (one call
    // site for the tile body, so that it is inlined once)
    int64_t t = g;
    int64_t a = g < sk.GS ? sk.start(g) : 0;
    const int64_t end = g < sk.GS ? sk.start(g + 1) : 0;
    while (t < sk.dp || a < end) {
        GemmParams q = p;
        int64_t tile_id;
        float* raw = nullptr;
        if (t < sk.dp) {
            tile_id = t;
            t += sk.G;
        } else {
            const int64_t u = a / sk.I;  // dealt-out tile
            const int64_t e = end < (u + 1) * sk.I ? end : (u + 1) * sk.I;
            const int s0 = (int)(a - u * sk.I), s1 = (int)(e - u * sk.I);
            const int k0 = s0 * sk.IK;
            q.K = (s1 * sk.IK < p.K ? s1 * sk.IK : p.K) - k0;
            q.A = static_cast<const char*>(p.A) + (TA ? (int64_t)k0 * p.lda : (int64_t)k0) * ESZ;
            q.B = static_cast<const char*>(p.B) + (TB ? (int64_t)k0 : (int64_t)k0 * p.ldb) * ESZ;
            if (!(s0 == 0 && s1 == sk.I)) raw = ws + (int64_t)sk.slot(g, u) * R * R;
            tile_id = sk.dp + u;
            a = e;
        }
        int bm, bn;
        sk.coords(tile_id, bm, bn);
        dma::barrier();  // every wave is done with the previous tile's LDS stages
        tile(q, bm * R, bn * R, raw);
    }
}

namespace {

// C <- alpha * (sum of a split tile's parts, in k order) + beta * C: a
// dealt-out tile of 256 x 256 in kFixSplit workgroups of 256 threads, each
// thread 4 consecutive columns per row it takes (tiles covered whole by one
// workgroup return).  The parts' workspace offsets are worked out once per
// workgroup, in LDS.
__global__ __launch_bounds__(256) void streamk_fixup_kernel(GemmParams p, StreamK sk,
                                                            const float* ws) {
    __shared__ int64_t part[kCUs];  // workspace offsets (floats) of the tile's parts
    const int64_t t = blockIdx.x / kFixSplit;
    const int g0 = sk.owner(t * sk.I), g1 = sk.owner((t + 1) * sk.I - 1);
    if (g0 == g1) return;
    const int nparts = g1 - g0 + 1;
    for (int j = threadIdx.x; j < nparts; j += 256)
        part[j] = (int64_t)sk.slot(g0 + j, t) * R * R;
    __syncthreads();
    int bm, bn;
    sk.coords(sk.dp + t, bm, bn);
    const int r = (int)(blockIdx.x % kFixSplit) * (R / kFixSplit) + threadIdx.x / 64;
    const int c = 4 * (threadIdx.x % 64);
    const bool vec = p.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(p.C) % 16 == 0;
#pragma unroll 1
    for (int rr = r; rr < r + R / kFixSplit; rr += 4) {
        const int m = bm * R + rr, n = bn * R + c;
        if (m >= p.M || n >= p.N) continue;
        const int e = rr * R + c;
        float4 sum = *reinterpret_cast<const float4*>(ws + part[0] + e);
        for (int j = 1; j < nparts; ++j) {
            const float4 v = *reinterpret_cast<const float4*>(ws + part[j] + e);
            sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
        }
        float* cp = p.C + (int64_t)m * p.ldc + n;
        if (vec && n + 4 <= p.N && p.beta == 0.0f) {
            *reinterpret_cast<float4*>(cp) = make_float4(p.alpha * sum.x, p.alpha * sum.y,
                                                         p.alpha * sum.z, p.alpha * sum.w);
        } else {
            const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
            for (int v = 0; v < 4 && n + v < p.N; ++v) cp[v] = epilogue(sv[v], p, cp + v, n + v);
        }
    }
}

}  // namespace

// The fix-up launch after the stream-K kernel (nothing when no tile is
// split).
inline hipError_t launch_fixup(const GemmParams& p, const StreamK& sk, const float* ws,
                               hipStream_t s) {
    if (!sk.split()) return hipSuccess;
    if (sk.T * kFixSplit > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(streamk_fixup_kernel, dim3((unsigned)(sk.T * kFixSplit)), dim3(256), 0, s,
                       p, sk, ws);
    return hipGetLastError();
}

}  // namespace streamk
}  // namespace dgt
