// k_skinny_f32.hip -- the bandwidth-bound path for M <= 64 with fp32 inputs
// (see skinny_common.hpp for the reasoning and the work split).
//
// v_mfma_f32_16x16x4_f32 (one k per lane, no transpose): rows = a block of
// 16 rows of op(A), columns = 16 columns.  Lane (g = l/16, i = l%16) holds
// columns n0 + 4i .. +3 and k = k0 + 8g .. +7 of a 32-deep step: slot t of
// MFMA c is k = k0 + 8g + t, column n0 + 4i + c, so a lane's A operands for
// one row are two 16-byte reads, and one step covers 64 columns with 32
// MFMAs per row block.  B stored K x N: a lane's loads are 8 stored rows x
// 16 bytes; B stored N x K: 4 stored rows (columns of op(B)) x 2 pieces of
// 16 bytes along k.  A stored K x M is read element by element.
#include "skinny_common.hpp"

namespace dgt {

namespace {

using namespace skinny;

constexpr int COLS = 64;  // columns per workgroup
constexpr int NW = 8;
constexpr int NTH = NW * 64;

template <bool kVec, bool kGuard, bool TA, bool TB, int RB>
__global__ __launch_bounds__(NTH, 1) void skinny_f32_kernel(GemmParams p) {
    select_problem(p);
    __shared__ float red[NW][16][COLS + 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * COLS;
    const int col = n0 + 4 * i;
    // B as K x N: a lane whose 4 columns run past N reads the row's last 4
    // columns instead, as in the 16-bit kernel (its duplicate results go to
    // the same places, bit for bit).
    const int bcol = (!TB && kVec && kGuard && p.N >= 4 && col + 4 > p.N) ? p.N - 4 : col;
    const int sh = col - bcol;
    const float* B = static_cast<const float*>(p.B);
    const ARows<float, RB, TA> ar(static_cast<const float*>(p.A), p, i);

    int s0, s1;
    wave_steps((p.K + KSTEP - 1) / KSTEP, NW, wave, s0, s1);

    floatx4 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // B as K x N: dst[t] = stored row k = kb + t, columns col .. col+3.  B
    // stored N x K: dst[2c + x] = stored row n = col + c, k = kb + 4x .. +3.
    auto load_b = [&](int step, u32x4 (&dst)[8]) {
        const int kb = step * KSTEP + 8 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (TB) {
                const int n = col + (t >> 1);
                const bool ok = n < p.N;
                dst[t] = load16<float, kVec, kGuard>(B + (int64_t)(ok ? n : 0) * p.ldb,
                                                     kb + 4 * (t & 1), p.K, ok);
            } else {
                const int krow = kb + t;
                const bool ok = krow < p.K;
                dst[t] = load16<float, kVec, kGuard>(B + (int64_t)(ok ? krow : 0) * p.ldb,
                                                     bcol, p.N, ok);
            }
        }
    };
    // a[rb][x] holds k = ka + 4x .. +3 of row 16*rb + i of op(A).
    auto load_a = [&](int step, u32x4 (&a)[RB][2]) {
        const int ka = step * KSTEP + 8 * g;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if constexpr (TA) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    a[rb][t >> 2][t & 3] = (!kGuard || ka + t < p.K)
                                               ? __float_as_uint(ar.row[rb][(int64_t)(ka + t) * p.lda])
                                               : 0u;
            } else {
                a[rb][0] = load16_cached<float, kVec, kGuard>(ar.row[rb], ka, p.K, ar.ok[rb]);
                a[rb][1] = load16_cached<float, kVec, kGuard>(ar.row[rb], ka + 4, p.K, ar.ok[rb]);
            }
        }
    };
    auto compute = [&](const u32x4 (&a)[RB][2], const u32x4 (&rbk)[8]) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float bv = __uint_as_float(TB ? rbk[2 * c + (t >> 2)][t & 3] : rbk[t][c]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        __uint_as_float(a[rb][t >> 2][t & 3]), bv, acc[rb][c], 0, 0, 0);
            }
    };

    // Two steps in flight, as in the 16-bit kernel.
    u32x4 b0[8], b1[8], a0[RB][2], a1[RB][2];
    int s = s0;
    if (s < s1) {
        load_a(s, a0);
        load_b(s, b0);
    }
    for (; s + 2 < s1; s += 2) {
        load_a(s + 1, a1);
        load_b(s + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        load_a(s + 2, a0);
        load_b(s + 2, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(a1, b1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (s + 1 < s1) {
        load_a(s + 1, a1);
        load_b(s + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(a1, b1);
    } else if (s < s1) {
        compute(a0, b0);
    }

    // MFMA c holds column 4*(l%16) + c of the strip; row 4*(l/16) + r.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (rb > 0) __syncthreads();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int cc = 4 * i + c - sh;
            if (cc < 0) continue;  // a column of the previous strip
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][4 * g + r][cc] = acc[rb][c][r];
        }
        __syncthreads();
        reduce_rows<NW, NTH, COLS>(red, p, n0, 16 * rb);
    }
}

template <int RB>
hipError_t launch_rb(const GemmParams& p, hipStream_t s) {
    const int blocks = (p.N + COLS - 1) / COLS;
    // 16-byte loads need element-aligned operands (any pitch)
    const bool vec = reinterpret_cast<uintptr_t>(p.A) % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(p.B) % 4 == 0 && p.stride_a % 4 == 0 &&
                     p.stride_b % 4 == 0;
    const bool full = vec && p.N % COLS == 0 && k_multiple(p, KSTEP);
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        const dim3 grid(blocks, p.batch), block(NTH);
        if (full)
            hipLaunchKernelGGL((skinny_f32_kernel<true, false, TA, TB, RB>), grid, block, 0, s, p);
        else if (vec)
            hipLaunchKernelGGL((skinny_f32_kernel<true, true, TA, TB, RB>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((skinny_f32_kernel<false, true, TA, TB, RB>), grid, block, 0, s, p);
        return hipGetLastError();
    });
}

}  // namespace

hipError_t launch_skinny_f32(const GemmParams& p, hipStream_t s) {
    switch ((p.M + 15) / 16) {
        case 1: return launch_rb<1>(p, s);
        case 2: return launch_rb<2>(p, s);
        case 3: return launch_rb<3>(p, s);
        case 4: return launch_rb<4>(p, s);
        default: return hipErrorInvalidConfiguration;
    }
}

}  // namespace dgt
