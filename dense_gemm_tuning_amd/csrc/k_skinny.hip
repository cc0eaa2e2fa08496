// k_skinny.hip -- the bandwidth-bound path for M <= 16 (decode-shaped GEMM).
//
// With a handful of rows of A, every element of B is used only M times:
// the arithmetic intensity is about M FLOP per byte of 16-bit B (2M / 2) or
// M/2 per byte of fp32 B, far below the ridge, so the time is the time to
// stream B from HBM once (dilfish.github.io 5.1: GEMV is bandwidth-bound at
// 0.5 FLOP/B and batching only scales it by the batch; qwbw.cn section 四:
// at batch 1 the cost is loading the weights).  The kernel is built for
// that: B is read exactly once, in 16-byte pieces whose lanes cover
// contiguous row segments, with non-temporal hints (nothing else reuses it),
// one K step ahead in registers; A (at most 16 rows) is re-read from cache;
// no LDS staging of B at all.
//
// Compute still goes to the matrix cores, because the vector ALU would need
// about 80% of its peak just for the FMAs at full HBM bandwidth.  The
// operand freedom used: MFMA sums over k, so any assignment of k and of the
// output columns to MFMA slots is valid if A and B agree and the store
// inverts the column map.
//
//  * bf16 / fp16: v_mfma_f32_16x16x32_{bf16,f16} with rows = the (up to 16) rows of A
//    and columns = 16 columns of B.  Lane l (g = l/16, i = l%16) loads the
//    8 x 8 block B[k0+8g .. +7][n0+8i .. +7] and transposes it in registers
//    into eight k-contiguous column pieces; MFMA c (c = 0..7) takes column
//    n0 + 8i + c from lane i, so one 32-deep K step covers 128 columns with
//    8 MFMAs and a single 16-byte read of A per lane.
//  * fp32: v_mfma_f32_16x16x4_f32 (one k per lane, no transpose).  Lane
//    (g, i) loads B[k0+8g+t][n0+4i .. +3] for t = 0..7; slot t of the MFMA
//    is k = k0 + 8g + t, so a lane's A operands are two 16-byte reads; one
//    32-deep K step covers 64 columns with 32 MFMAs.
//
// Transposed operands: with B stored N x K (a linear layer's [out, in]
// weight) a lane's 16-byte load already holds 8 (or 4) consecutive k of one
// column, so no register transpose is needed (16-bit inputs: a kernel of
// its own, below); A stored K x M is read element by element (it is tiny
// and cached).
//
// Work split: a workgroup of 8 wavefronts owns one column strip (128 bf16
// or 64 fp32 columns) over the whole of K; wavefront w takes the w-th
// eighth of the K steps, and the eight partial tiles are summed in LDS in a
// fixed order (deterministic, no atomics, no workspace).  Ragged shapes:
// zero-filled loads, masked stores.
#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int NT = 512;      // 8 wavefronts
constexpr int NW = NT / 64;
constexpr int KSTEP = 32;

// 16-byte piece [col, col + 16/esz) of one row, zero outside; streamed.
template <typename T, bool kVec, bool kGuard>
__device__ __forceinline__ u32x4 load16(const T* rowp, int col, int limit, bool row_ok) {
    constexpr int V = 16 / sizeof(T);
    if (!kGuard || (row_ok && kVec && col + V <= limit))
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + col));
    u32x4 out = {0u, 0u, 0u, 0u};
    if (!row_ok) return out;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[v] = (col + v < limit) ? __float_as_uint(reinterpret_cast<const float*>(rowp)[col + v]) : 0u;
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
    if (!kGuard || (row_ok && kVec && col + V <= limit))
        return *reinterpret_cast<const u32x4*>(rowp + col);
    return load16<T, kVec, true>(rowp, col, limit, row_ok);
}

// Column j of an 8 x 8 bf16 block (rows = k): dword e = rows 2e (low), 2e+1.
__device__ __forceinline__ u32x4 column8(const u32x4 (&r)[8], int j) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = r[2 * e][j >> 1], hi = r[2 * e + 1][j >> 1];
        o[e] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    return o;
}

// Sum the NW partial tiles in a fixed order and apply the epilogue.
template <int COLS>
__device__ __forceinline__ void reduce_store(float (*red)[16][COLS + 4],
                                             const GemmParams& p, int n0) {
    __syncthreads();
    for (int o = threadIdx.x; o < 16 * COLS; o += NT) {
        const int m = o / COLS, nl = o % COLS, n = n0 + nl;
        if (m >= p.M || n >= p.N) continue;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += red[w][m][nl];
        float* c = p.C + (int64_t)m * p.ldc + n;
        *c = epilogue(s, p, c, n);
    }
}

// ---------------------------------------------------------------- bf16

constexpr int BF_COLS = 128;

// 8 consecutive k (from ka) of row i of op(A) as one MFMA operand.  arow is
// row i of A (stored M x K), or column i of A stored K x M, read element by
// element with stride lda (A is tiny and cached).
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

template <In T, bool kVec, bool kGuard, bool TA>
__global__ __launch_bounds__(NT, 1) void skinny16_kernel(GemmParams p) {
    select_problem(p);
    __shared__ float red[NW][16][BF_COLS + 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * BF_COLS;
    const int col = n0 + 8 * i;
    const uint16_t* A = static_cast<const uint16_t*>(p.A);
    const uint16_t* B = static_cast<const uint16_t*>(p.B);
    const bool a_ok = i < p.M;
    // Row i of op(A): a stored row (k contiguous), or column i of A stored
    // K x M (stride lda).  Rows past M use row 0 and are never stored.
    const uint16_t* arow = A + (TA ? (int64_t)(a_ok ? i : 0) : (int64_t)(a_ok ? i : 0) * p.lda);

    const int nsteps = (p.K + KSTEP - 1) / KSTEP;
    const int per = (nsteps + NW - 1) / NW;
    const int s0 = wave * per;
    const int s1 = min(s0 + per, nsteps);

    floatx4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // dst[r] = stored row k = kb + r, columns col .. col+7; the MFMA operand
    // is a column of that block.
    auto load_b = [&](int step, u32x4 (&dst)[8]) {
        const int kb = step * KSTEP + 8 * g;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int krow = kb + r;
            const bool ok = krow < p.K;
            dst[r] = load16<uint16_t, kVec, kGuard>(B + (int64_t)(ok ? krow : 0) * p.ldb,
                                                    col, p.N, ok);
        }
    };
    auto load_a = [&](int step) {
        return load_a16<kVec, kGuard, TA>(arow, step * KSTEP + 8 * g, p, a_ok);
    };
    auto compute = [&](const u32x4& a, const u32x4 (&rb)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = mfma16x16x32<T>(a, column8(rb, c), acc[c]);
    };

    // Two steps in flight: each phase issues the next step's loads (A with
    // B, so that waiting for A never drains the B prefetch), then consumes
    // the step loaded one phase earlier.  The scheduling barriers keep the
    // phases in this order; unrolled by two so that the buffers alternate
    // without a branch in the loop body.
    u32x4 b0[8], b1[8], a0, a1;
    int s = s0;
    if (s < s1) {
        a0 = load_a(s);
        load_b(s, b0);
    }
    for (; s + 2 < s1; s += 2) {
        a1 = load_a(s + 1);
        load_b(s + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        a0 = load_a(s + 2);
        load_b(s + 2, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(a1, b1);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (s + 1 < s1) {
        a1 = load_a(s + 1);
        load_b(s + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute(a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute(a1, b1);
    } else if (s < s1) {
        compute(a0, b0);
    }

    // 16x16 accumulator layout: register r of lane l is row 4*(l/16) + r,
    // column l%16; MFMA c holds column n0 + 8*(l%16) + c.
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * g + r][8 * i + c] = acc[c][r];
    reduce_store<BF_COLS>(red, p, n0);
}

// ------------------------------------------- 16-bit, B stored N x K

// B stored N x K (a linear layer's [out, in] weight): every column of op(B)
// is a stored row with k contiguous.  The MFMA lane layout would let one
// load instruction fetch only 64 B from each of 16 rows, which halves the
// rate the memory side delivers; instead each instruction fetches 256 B from
// each of 4 rows (16 lanes per row, as the K x N layout does), the wave
// parks the piece in a private LDS region, and reads the MFMA operands back
// from there.  A group is 32 columns (stored rows) x 128 k = 8 KiB, eight
// load instructions; a 128-deep step is four groups (the workgroup's 128
// columns).  LDS rows are 256 B with chunk c of row r at c ^ (r & 15), so
// both the writes (16 lanes of one row) and the operand reads (16 rows, one
// chunk) touch 16 distinct 16-byte bank groups.
constexpr int BT_KSTEP = 128;
constexpr int BT_GROUP_ROWS = 32;
constexpr int BT_STAGE = BT_GROUP_ROWS * 256;  // bytes per wave

template <In T, bool kVec, bool kGuard, bool TA>
__global__ __launch_bounds__(NT, 1) void skinny16_bt_kernel(GemmParams p) {
    select_problem(p);
    __shared__ float red[NW][16][BF_COLS + 4];
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[NW][BT_STAGE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * BF_COLS;
    const uint16_t* A = static_cast<const uint16_t*>(p.A);
    const uint16_t* B = static_cast<const uint16_t*>(p.B);
    const bool a_ok = i < p.M;
    const uint16_t* arow = A + (TA ? (int64_t)(a_ok ? i : 0) : (int64_t)(a_ok ? i : 0) * p.lda);
    uint8_t* stage = stage_all[wave];

    const int nsteps = (p.K + BT_KSTEP - 1) / BT_KSTEP;
    const int per = (nsteps + NW - 1) / NW;
    const int s0 = wave * per;
    const int s1 = min(s0 + per, nsteps);

    floatx4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

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
    auto compute = [&](auto cpc, const u32x4 (&a)[4]) {
        constexpr int cp = decltype(cpc)::value;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4 bop = *reinterpret_cast<const u32x4*>(
                    stage + (16 * b + i) * 256 + (((4 * u + g) ^ i) << 4));
                acc[2 * cp + b] = mfma16x16x32<T>(a[u], bop, acc[2 * cp + b]);
            }
    };
    auto load_a = [&](int s, u32x4 (&a)[4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            a[u] = load_a16<kVec, kGuard, TA>(arow, s * BT_KSTEP + 32 * u + 8 * g, p, a_ok);
    };

    // Two groups in flight.  Each phase issues the next group's loads, then
    // parks and consumes the group loaded one phase earlier; the scheduling
    // barriers keep the compiler from gathering several phases' loads into
    // one burst or from sinking them below the waits of the park.  The last
    // step is peeled (no prefetch), so the loop body has no branch and the
    // loads stay in flight across the back edge.  LDS operations of one wave
    // complete in order, so parking a group after the previous group's
    // operand reads needs no wait.
    u32x4 r0[8], r1[8], a0[4], a1[4];
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
            for (int u = 0; u < 4; ++u) a0[u] = a1[u];
        }
    };
    if (s0 < s1) {
        load_a(s0, a0);
        load_group(s0, 0, r0);
        for (int s = s0; s + 1 < s1; ++s) step(s, std::true_type{});
        step(s1 - 1, std::false_type{});
    }

    // 16x16 accumulator layout: register r of lane l is row 4*(l/16) + r,
    // column l%16; accumulator c holds columns n0 + 16c .. +15.
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * g + r][16 * c + i] = acc[c][r];
    reduce_store<BF_COLS>(red, p, n0);
}

// ---------------------------------------------------------------- fp32

constexpr int F_COLS = 64;

template <bool kVec, bool kGuard, bool TA, bool TB>
__global__ __launch_bounds__(NT, 1) void skinny_f32_kernel(GemmParams p) {
    select_problem(p);
    __shared__ float red[NW][16][F_COLS + 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * F_COLS;
    const int col = n0 + 4 * i;
    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    const bool a_ok = i < p.M;
    const float* arow = A + (TA ? (int64_t)(a_ok ? i : 0) : (int64_t)(a_ok ? i : 0) * p.lda);

    const int nsteps = (p.K + KSTEP - 1) / KSTEP;
    const int per = (nsteps + NW - 1) / NW;
    const int s0 = wave * per;
    const int s1 = min(s0 + per, nsteps);

    floatx4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

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
                                                     col, p.N, ok);
            }
        }
    };
    auto compute = [&](int step, const u32x4 (&rb)[8]) {
        const int ka = step * KSTEP + 8 * g;
        float av[8];
        if constexpr (TA) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                av[t] = (!kGuard || ka + t < p.K) ? arow[(int64_t)(ka + t) * p.lda] : 0.0f;
        } else {
            const u32x4 a0 = load16_cached<float, kVec, kGuard>(arow, ka, p.K, a_ok);
            const u32x4 a1 = load16_cached<float, kVec, kGuard>(arow, ka + 4, p.K, a_ok);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                av[t] = __uint_as_float(a0[t]);
                av[t + 4] = __uint_as_float(a1[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t bv = TB ? rb[2 * c + (t >> 2)][t & 3] : rb[t][c];
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], __uint_as_float(bv),
                                                              acc[c], 0, 0, 0);
            }
        }
    };

    u32x4 b0[8], b1[8];
    if (s0 < s1) load_b(s0, b0);
    for (int s = s0; s < s1; s += 2) {
        if (s + 1 < s1) load_b(s + 1, b1);
        compute(s, b0);
        if (s + 1 < s1) {
            if (s + 2 < s1) load_b(s + 2, b0);
            compute(s + 1, b1);
        }
    }

    // MFMA c holds column n0 + 4*(l%16) + c.
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * g + r][4 * i + c] = acc[c][r];
    reduce_store<F_COLS>(red, p, n0);
}

}  // namespace

template <In T>
hipError_t launch_skinny16(const GemmParams& p, hipStream_t s) {
    const int blocks = (p.N + BF_COLS - 1) / BF_COLS;
    const bool vec = operands_16b_aligned(p, 2);
    const int kstep = p.tb ? BT_KSTEP : KSTEP;
    const bool full = vec && p.N % BF_COLS == 0 && p.K % kstep == 0;
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        const dim3 grid(blocks, p.batch), block(NT);
        if constexpr (TB) {
            if (full)
                hipLaunchKernelGGL((skinny16_bt_kernel<T, true, false, TA>), grid, block, 0, s, p);
            else if (vec)
                hipLaunchKernelGGL((skinny16_bt_kernel<T, true, true, TA>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((skinny16_bt_kernel<T, false, true, TA>), grid, block, 0, s, p);
        } else {
            if (full)
                hipLaunchKernelGGL((skinny16_kernel<T, true, false, TA>), grid, block, 0, s, p);
            else if (vec)
                hipLaunchKernelGGL((skinny16_kernel<T, true, true, TA>), grid, block, 0, s, p);
            else
                hipLaunchKernelGGL((skinny16_kernel<T, false, true, TA>), grid, block, 0, s, p);
        }
        return hipGetLastError();
    });
}
template hipError_t launch_skinny16<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_skinny16<In::F16>(const GemmParams&, hipStream_t);

hipError_t launch_skinny_f32(const GemmParams& p, hipStream_t s) {
    const int blocks = (p.N + F_COLS - 1) / F_COLS;
    const bool vec = operands_16b_aligned(p, 4);
    const bool full = vec && p.N % F_COLS == 0 && p.K % KSTEP == 0;
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (full)
            hipLaunchKernelGGL((skinny_f32_kernel<true, false, TA, TB>), dim3(blocks, p.batch), dim3(NT),
                               0, s, p);
        else if (vec)
            hipLaunchKernelGGL((skinny_f32_kernel<true, true, TA, TB>), dim3(blocks, p.batch), dim3(NT),
                               0, s, p);
        else
            hipLaunchKernelGGL((skinny_f32_kernel<false, true, TA, TB>), dim3(blocks, p.batch), dim3(NT),
                               0, s, p);
        return hipGetLastError();
    });
}

}  // namespace dgt
