// skinny_common.hpp -- pieces shared by the bandwidth-bound skinny kernels
// (k_skinny16.hip, k_skinny_f32.hip).
//
// With few rows of op(A) (M <= kSkinnyMaxM), every element of B is used
// only M times: the arithmetic intensity is about M FLOP per byte of 16-bit
// B (2M / 2) or M/2 per byte of fp32 B, below the ridge, so the time is the
// time to stream B from HBM once (dilfish.github.io 5.1: GEMV is
// bandwidth-bound at 0.5 FLOP/B and batching scales it by the batch;
// qwbw.cn section 四: at batch 1 the cost is loading the weights).  The
// kernels read B exactly once, in 16-byte pieces whose lanes cover
// contiguous row segments, with non-temporal hints, one step ahead; A is
// re-read from cache.  M is covered by RB blocks of 16 rows (RB <= 4): each
// B operand feeds RB MFMAs.
//
// Work split: a workgroup owns one column strip over the whole of K; its NW
// wavefronts each take one NW-th of the K steps, and the NW partial tiles
// are summed in LDS in a fixed order, one 16-row block at a time
// (deterministic, no atomics, no workspace).  Ragged shapes: zero-filled
// loads, masked stores.
#pragma once

#include "gemm_common.hpp"

namespace dgt {
namespace skinny {

constexpr int KSTEP = 32;

// A 16-byte piece at an element-aligned address: loaded as one
// global_load_dwordx4 whatever the row pitch (the GPU runs with unaligned
// memory access enabled; the parity tests include pitches of a few elements
// past a 16-byte multiple).
typedef uint32_t u32x4_any __attribute__((ext_vector_type(4), aligned(2)));

// 16-byte piece [col, col + 16/esz) of one row, zero outside; streamed.
// kVec: 16-byte loads (element-aligned operands, any pitch); pieces that
// straddle the limit, and every piece without kVec, are gathered element by
// element.
template <typename T, bool kVec, bool kGuard>
__device__ __forceinline__ u32x4 load16(const T* rowp, int col, int limit, bool row_ok) {
    constexpr int V = 16 / sizeof(T);
    if (!kGuard || (row_ok && kVec && col + V <= limit)) {
        const u32x4_any v =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_any*>(rowp + col));
        return u32x4{v[0], v[1], v[2], v[3]};
    }
    u32x4 out = {0u, 0u, 0u, 0u};
    if (!row_ok) return out;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[v] = (col + v < limit)
                         ? __float_as_uint(reinterpret_cast<const float*>(rowp)[col + v])
                         : 0u;
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint32_t lo = (col + 2 * v < limit) ? rowp[col + 2 * v] : 0u;
            const uint32_t hi = (col + 2 * v + 1 < limit) ? rowp[col + 2 * v + 1] : 0u;
            out[v] = lo | (hi << 16);
        }
    }
    return out;
}

// A is small and shared by every workgroup: ordinary (cached) loads.
template <typename T, bool kVec, bool kGuard>
__device__ __forceinline__ u32x4 load16_cached(const T* rowp, int col, int limit, bool row_ok) {
    constexpr int V = 16 / sizeof(T);
    if (!kGuard || (row_ok && kVec && col + V <= limit)) {
        const u32x4_any v = *reinterpret_cast<const u32x4_any*>(rowp + col);
        return u32x4{v[0], v[1], v[2], v[3]};
    }
    return load16<T, kVec, true>(rowp, col, limit, row_ok);
}

// Row 16*rb + i of op(A) for the RB row blocks: a stored row (k contiguous)
// or, with A stored K x M, column 16*rb + i (stride lda).  Rows past M point
// at row 0 and are computed but never stored.
template <typename S, int RB, bool TA>
struct ARows {
    const S* row[RB];
    bool ok[RB];
    __device__ ARows(const S* A, const GemmParams& p, int i) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int r = 16 * rb + i;
            ok[rb] = r < p.M;
            const int64_t rr = ok[rb] ? r : 0;
            row[rb] = A + (TA ? rr : rr * p.lda);
        }
    }
};

// Sum the NW partial tiles of rows m0 .. m0+15 held in red, in wave order,
// and apply the epilogue.  The caller brackets it with barriers.
template <int NW, int NTH, int COLS>
__device__ __forceinline__ void reduce_rows(const float (*red)[16][COLS + 4], const GemmParams& p,
                                            int n0, int m0) {
    for (int o = threadIdx.x; o < 16 * COLS; o += NTH) {
        const int m = m0 + o / COLS, nl = o % COLS, n = n0 + nl;
        if (m >= p.M || n >= p.N) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += red[w][o / COLS][nl];
        float* c = p.C + (int64_t)m * p.ldc + n;
        *c = epilogue(s, p, c, n);
    }
}

// Wavefronts per workgroup: 8 (a wave then has 256 registers) keep twice
// the bytes in flight per CU of 4 (512 registers each), and the skinny path
// is latency-bound without them; 4 only where a wave's operands and RB x 8
// accumulators do not fit 256 registers: with A stored K x M (gathered
// element by element) from 3 row blocks, and for B stored N x K (two 8-KiB
// groups and four k-quarters of A per row block in flight) from 2.
template <int RB, bool TA>
constexpr int waves_for() { return (TA && RB >= 3) ? 4 : 8; }
template <int RB>
constexpr int bt_waves_for() { return RB == 1 ? 8 : 4; }

// The step range [s0, s1) of wave w when nsteps are split over NW waves.
__device__ __forceinline__ void wave_steps(int nsteps, int NW, int wave, int& s0, int& s1) {
    const int per = (nsteps + NW - 1) / NW;
    s0 = wave * per;
    s1 = min(s0 + per, nsteps);
}

}  // namespace skinny
}  // namespace dgt
