// k_skinny16.hip -- the bandwidth-bound path for M <= 64 with 16-bit inputs
// (decode-shaped GEMM; see skinny_common.hpp for the reasoning and the work
// split).
//
// Compute still goes to the matrix cores, because the vector ALU would need
// about 80% of its peak just for the FMAs at full HBM bandwidth.  The
// operand freedom used: MFMA sums over k, so any assignment of k and of the
// output columns to MFMA slots is valid if A and B agree and the store
// inverts the column map.  v_mfma_f32_16x16x32_{bf16,f16}: rows = a block of
// 16 rows of op(A), columns = 16 columns of op(B), 32 k.
//
//  * B stored K x N (skinny16_kernel): lane l (g = l/16, i = l%16) loads the
//    8 x 8 block B[k0+8g .. +7][n0+8i .. +7] and transposes it in registers
//    into eight k-contiguous column pieces; MFMA c (c = 0..7) takes column
//    n0 + 8i + c from lane i, so one 32-deep K step covers 128 columns with
//    8 MFMAs per row block.
//  * B stored N x K (skinny16_bt_kernel; a linear layer's [out, in] weight):
//    every column of op(B) is a stored row with k contiguous.  The MFMA lane
//    layout would let one load instruction fetch only 64 B from each of 16
//    rows, which halves the rate the memory side delivers; instead each
//    instruction fetches 256 B from each of 4 rows (16 lanes per row, as the
//    K x N layout does), the wave parks the piece in a private LDS region,
//    and reads the MFMA operands back from there.  A group is 32 columns
//    (stored rows) x 128 k = 8 KiB, eight load instructions; a 128-deep step
//    is four groups (the workgroup's 128 columns).  LDS rows are 256 B with
//    chunk c of row r at c ^ (r & 15), so both the writes (16 lanes of one
//    row) and the operand reads (16 rows, one chunk) touch 16 distinct
//    16-byte bank groups.
//  * A stored K x M is read element by element (it is tiny and cached).
#include "skinny_common.hpp"

namespace dgt {

namespace {

using namespace skinny;

constexpr int COLS = 128;  // columns per workgroup

// 8 consecutive k (from ka) of one row of op(A) as an MFMA operand.
template <bool kVec, bool kGuard, bool TA>
__device__ __forceinline__ u32x4 load_a16(const uint16_t* arow, int ka, const GemmParams& p,
                                          bool a_ok) {
    if constexpr (TA) {
        u32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k0 = ka + 2 * e, k1 = k0 + 1;
            const uint32_t lo = (!kGuard || k0 < p.K) ? arow[(int64_t)k0 * p.lda] : 0u;
            const uint32_t hi = (!kGuard || k1 < p.K) ? arow[(int64_t)k1 * p.lda] : 0u;
            a[e] = lo | (hi << 16);
        }
        return a;
    } else {
        return load16_cached<uint16_t, kVec, kGuard>(arow, ka, p.K, a_ok);
    }
}

// Column j of an 8 x 8 16-bit block (rows = k): dword e = rows 2e (low), 2e+1.
__device__ __forceinline__ u32x4 column8(const u32x4 (&r)[8], int j) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = r[2 * e][j >> 1], hi = r[2 * e + 1][j >> 1];
        o[e] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    return o;
}

// Write the accumulators of row block rb as this wave's partial tile, then
// sum the waves' partials for those 16 rows.  acc[c][r]: row 4*(l/16) + r,
// column col_of(c, l%16) of the strip.
template <int NW, int NTH, typename ColOf>
__device__ __forceinline__ void store_block(float (*red)[16][COLS + 4], const floatx4 (&acc)[8],
                                            int wave, int g, int i, ColOf col_of,
                                            const GemmParams& p, int n0, int m0, bool first) {
    if (!first) __syncthreads();  // the previous block's sums have been read
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int cc = col_of(c, i);
        if (cc < 0) continue;  // a column of the previous strip
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * g + r][cc] = acc[c][r];
    }
    __syncthreads();
    reduce_rows<NW, NTH, COLS>(red, p, n0, m0);
}

// ---------------------------------------------------------- B stored K x N

template <In T, bool kVec, bool kGuard, bool TA, int RB>
__global__ __launch_bounds__((waves_for<RB, TA>() * 64), 1) void skinny16_kernel(GemmParams p) {
    constexpr int NW = waves_for<RB, TA>(), NTH = NW * 64;
    select_problem(p);
    __shared__ float red[NW][16][COLS + 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * COLS;
    const int col = n0 + 8 * i;
    // A lane whose 8 columns run past N (the last strip of a ragged N) reads
    // the row's last 8 columns instead, with whole 16-byte loads: its
    // results for the columns below col repeat a neighbour's bit for bit
    // (same operands, same order) and go to the same places.  Element-wise
    // loads there instead would hold that strip's waves, and the launch,
    // back at every load.
    const int bcol = (kVec && kGuard && p.N >= 8 && col + 8 > p.N) ? p.N - 8 : col;
    const int sh = col - bcol;
    const uint16_t* B = static_cast<const uint16_t*>(p.B);
    const ARows<uint16_t, RB, TA> ar(static_cast<const uint16_t*>(p.A), p, i);

    int s0, s1;
    wave_steps((p.K + KSTEP - 1) / KSTEP, NW, wave, s0, s1);

    floatx4 acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // dst[r] = stored row k = kb + r, columns col .. col+7; the MFMA operand
    // is a column of that block.
    auto load_b = [&](int step, u32x4 (&dst)[8]) {
        const int kb = step * KSTEP + 8 * g;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int krow = kb + r;
            const bool ok = krow < p.K;
            dst[r] = load16<uint16_t, kVec, kGuard>(B + (int64_t)(ok ? krow : 0) * p.ldb,
                                                    bcol, p.N, ok);
        }
    };
    auto load_a = [&](int step, u32x4 (&a)[RB]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            a[rb] = load_a16<kVec, kGuard, TA>(ar.row[rb], step * KSTEP + 8 * g, p, ar.ok[rb]);
    };
    auto compute = [&](const u32x4 (&a)[RB], const u32x4 (&rbk)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const u32x4 bop = column8(rbk, c);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc[rb][c] = mfma16x16x32<T>(a[rb], bop, acc[rb][c]);
        }
    };

    // Two steps in flight: each phase issues the next step's loads (A with
    // B, so that waiting for A never drains the B prefetch), then consumes
    // the step loaded one phase earlier.  The scheduling barriers keep the
    // phases in this order; unrolled by two so that the buffers alternate
    // without a branch in the loop body.
    u32x4 b0[8], b1[8], a0[RB], a1[RB];
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

    // MFMA c holds column 8*(l%16) + c of the strip (less the lane's shift).
    auto col_of = [sh](int c, int ii) { return 8 * ii + c - sh; };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        store_block<NW, NTH>(red, acc[rb], wave, g, i, col_of, p, n0, 16 * rb, rb == 0);
}

// ---------------------------------------------------------- B stored N x K

constexpr int BT_KSTEP = 128;
constexpr int BT_GROUP_ROWS = 32;
constexpr int BT_STAGE = BT_GROUP_ROWS * 256;  // bytes per wave

template <In T, bool kVec, bool kGuard, bool TA, int RB>
__global__ __launch_bounds__(bt_waves_for<RB>() * 64, 1) void skinny16_bt_kernel(GemmParams p) {
    constexpr int NW = bt_waves_for<RB>(), NTH = NW * 64;
    select_problem(p);
    __shared__ float red[NW][16][COLS + 4];
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[NW][BT_STAGE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * COLS;
    const uint16_t* B = static_cast<const uint16_t*>(p.B);
    const ARows<uint16_t, RB, TA> ar(static_cast<const uint16_t*>(p.A), p, i);
    uint8_t* stage = stage_all[wave];

    int s0, s1;
    wave_steps((p.K + BT_KSTEP - 1) / BT_KSTEP, NW, wave, s0, s1);

    floatx4 acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Group cp of step s: instruction j fetches local rows 4j .. 4j+3; lane
    // l takes local row 4j + l/16, chunk l%16 (k = 128s + 8*(l%16)).
    auto load_group = [&](int s, int cp, u32x4 (&r)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = n0 + BT_GROUP_ROWS * cp + 4 * j + g;
            const bool ok = row < p.N;
            r[j] = load16<uint16_t, kVec, kGuard>(B + (int64_t)(ok ? row : 0) * p.ldb,
                                                  s * BT_KSTEP + 8 * i, p.K, ok);
        }
    };
    auto park = [&](const u32x4 (&r)[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int lr = 4 * j + g;
            *reinterpret_cast<u32x4*>(stage + lr * 256 + ((i ^ (lr & 15)) << 4)) = r[j];
        }
    };
    // MFMA block b of the group (local rows 16b + i), quarter u (chunk 4u + g).
    auto compute = [&](auto cpc, const u32x4 (&a)[RB][4]) {
        constexpr int cp = decltype(cpc)::value;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 bop = *reinterpret_cast<const u32x4*>(
                    stage + (16 * b + i) * 256 + (((4 * u + g) ^ i) << 4));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][2 * cp + b] = mfma16x16x32<T>(a[rb][u], bop, acc[rb][2 * cp + b]);
            }
    };
    auto load_a = [&](int s, u32x4 (&a)[RB][4]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                a[rb][u] = load_a16<kVec, kGuard, TA>(ar.row[rb], s * BT_KSTEP + 32 * u + 8 * g,
                                                      p, ar.ok[rb]);
    };

    // Two groups in flight.  Each phase issues the next group's loads, then
    // parks and consumes the group loaded one phase earlier; the scheduling
    // barriers keep the compiler from gathering several phases' loads into
    // one burst or from sinking them below the waits of the park.  The last
    // step is peeled (no prefetch), so the loop body has no branch and the
    // loads stay in flight across the back edge.  LDS operations of one wave
    // complete in order, so parking a group after the previous group's
    // operand reads needs no wait.
    u32x4 r0[8], r1[8], a0[RB][4], a1[RB][4];
    auto step = [&](int s, auto prefetch) {
        constexpr bool kPrefetch = decltype(prefetch)::value;
        load_group(s, 1, r1);
        __builtin_amdgcn_sched_barrier(0);
        park(r0);
        compute(std::integral_constant<int, 0>{}, a0);
        __builtin_amdgcn_sched_barrier(0);
        load_group(s, 2, r0);
        __builtin_amdgcn_sched_barrier(0);
        park(r1);
        compute(std::integral_constant<int, 1>{}, a0);
        __builtin_amdgcn_sched_barrier(0);
        load_group(s, 3, r1);
        __builtin_amdgcn_sched_barrier(0);
        park(r0);
        compute(std::integral_constant<int, 2>{}, a0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kPrefetch) {
            load_a(s + 1, a1);
            load_group(s + 1, 0, r0);
        }
        __builtin_amdgcn_sched_barrier(0);
        park(r1);
        compute(std::integral_constant<int, 3>{}, a0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int u = 0; u < 4; ++u) a0[rb][u] = a1[rb][u];
        }
    };
    if (s0 < s1) {
        load_a(s0, a0);
        load_group(s0, 0, r0);
        for (int s = s0; s + 1 < s1; ++s) step(s, std::true_type{});
        step(s1 - 1, std::false_type{});
    }

    // Accumulator c holds columns 16c .. 16c+15 of the strip.
    auto col_of = [](int c, int ii) { return 16 * c + ii; };
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
        store_block<NW, NTH>(red, acc[rb], wave, g, i, col_of, p, n0, 16 * rb, rb == 0);
}

template <In T, int RB>
hipError_t launch_rb(const GemmParams& p, hipStream_t s) {
    const int NTH = (p.tb ? bt_waves_for<RB>() : p.ta ? waves_for<RB, true>() : waves_for<RB, false>()) * 64;
    const int blocks = (p.N + COLS - 1) / COLS;
    // 16-byte loads need element-aligned operands (any pitch)
    const bool vec = reinterpret_cast<uintptr_t>(p.A) % 2 == 0 &&
                     reinterpret_cast<uintptr_t>(p.B) % 2 == 0 && p.stride_a % 2 == 0 &&
                     p.stride_b % 2 == 0;
    const int kstep = p.tb ? BT_KSTEP : KSTEP;
    const bool full = vec && p.N % COLS == 0 && k_multiple(p, kstep);
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        const dim3 grid(blocks, p.batch), block(NTH);
        if constexpr (TB) {
            if (full)
                hipLaunchKernelGGL((skinny16_bt_kernel<T, true, false, TA, RB>), grid, block, 0, s, p);
            else if (vec)
                hipLaunchKernelGGL((skinny16_bt_kernel<T, true, true, TA, RB>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((skinny16_bt_kernel<T, false, true, TA, RB>), grid, block, 0, s, p);
        } else {
            if (full)
                hipLaunchKernelGGL((skinny16_kernel<T, true, false, TA, RB>), grid, block, 0, s, p);
            else if (vec)
                hipLaunchKernelGGL((skinny16_kernel<T, true, true, TA, RB>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((skinny16_kernel<T, false, true, TA, RB>), grid, block, 0, s, p);
        }
        return hipGetLastError();
    });
}

}  // namespace

template <In T>
hipError_t launch_skinny16(const GemmParams& p, hipStream_t s) {
    switch ((p.M + 15) / 16) {
        case 1: return launch_rb<T, 1>(p, s);
        case 2: return launch_rb<T, 2>(p, s);
        case 3: return launch_rb<T, 3>(p, s);
        case 4: return launch_rb<T, 4>(p, s);
        default: return hipErrorInvalidConfiguration;
    }
}
template hipError_t launch_skinny16<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_skinny16<In::F16>(const GemmParams&, hipStream_t);

}  // namespace dgt
