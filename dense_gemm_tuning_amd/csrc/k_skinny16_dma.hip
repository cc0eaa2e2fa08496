// k_skinny16_dma.hip -- the bandwidth-bound path for a linear layer's
// decode-shaped product: 16-bit inputs, M <= 64 rows of A stored M x K and
// the weight B stored N x K (every column of op(B) a stored row, k
// contiguous).  Same reasoning as the register-staged skinny kernels: the
// time is the time to stream B once, so what matters is how many bytes are
// in flight per CU (Little's law: about 8 TB/s x a few microseconds of
// loaded latency, spread over the CUs).
//
// With several 16-row blocks of A the register-staged kernel runs out of
// registers (RB x 8 accumulators plus two steps of A operands): it keeps
// four waves per CU with at most two 8-KiB groups of B each.  Here B never
// passes through registers: each wave copies its groups straight into LDS
// with buffer loads that write LDS (one 16-byte piece per lane, 1 KiB per
// instruction), into a private ring of four stages, so three groups (24 KiB)
// per wave, 96 KiB per CU, are in flight while it computes on the fourth.
// No wave reads another wave's stages, so the loop has no workgroup barrier;
// each wave waits only for its own copies (vector-memory loads complete in
// issue order, so one wait count per group suffices).
//
// Work split as in the register-staged kernel: a workgroup owns a strip of
// 128 columns (stored rows of B) over all of K, its four waves one K-quarter
// each; a 128-deep step is four groups of 32 stored rows x 128 k (8 KiB).
// The partial tiles are summed in LDS in wave order (deterministic, no
// atomics, no workspace).  A (at most 64 x K, shared by every workgroup and
// re-read from cache) is loaded into registers one step ahead with plain
// buffer loads, so that a wave issues the same number of vector-memory
// instructions per step whatever the shape (the wait counts rely on it).
//
// Operands through buffer descriptors: a 16-byte piece past a descriptor's
// range reads as zeros.  Each group has a descriptor that ends at its last
// valid stored row (k = K - 1), so rows past N read zeros; pieces at k >= K
// (K a multiple of 8, so a piece is all inside or all outside) get an
// offset at the range end and read zeros too, as do rows of A past M.
#include "skinny_common.hpp"
#include "dma_common.hpp"

namespace dgt {

namespace {

using namespace skinny;

constexpr int COLS = 128;        // columns (stored rows of B) per workgroup
constexpr int STEP_K = 128;      // k per step
constexpr int GROUP_ROWS = 32;   // stored rows per group (four groups a step)
constexpr int STAGE = GROUP_ROWS * STEP_K * 2;  // bytes of one group: 8 KiB
constexpr int kBPolicy = 2;      // cache policy of the B copies: nt (streamed once)

static_assert(STAGE == 16 * COLS * 4, "one stage holds a wave's 16-row partial tile");

// One 16-byte piece per lane of B into LDS: lane l's bytes at base + voff
// land at lds + 16*l.
__device__ __forceinline__ void copy_b(const void* base, uint32_t range, uint8_t* lds,
                                       uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, range, kBufferRsrcW3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (dma::lds_void*)lds, 16, voff, 0, 0, kBPolicy);
}

// NW waves (one K-range each), a ring of NS stages per wave (NS divides the
// four groups of a step, so group cp of any step uses stage cp % NS).
template <In T, int RB, int NW, int NS>
__global__ __launch_bounds__(NW * 64, 1) void skinny16_bt_dma_kernel(GemmParams p) {
    static_assert(NS == 2 || NS == 4, "a step's four groups map onto the ring");
    constexpr int D = NS - 1;  // groups copied ahead of the one being read
    select_problem(p);
    // One __shared__ object per stage (so the compiler's wait-count pass can
    // tell a copy into one stage from reads of another); stage q of wave w
    // is stq + STAGE*w.
    __shared__ __attribute__((aligned(16))) uint8_t st0[NW * STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[NW * STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[NS > 2 ? NW * STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st3[NS > 2 ? NW * STAGE : 16];
    // The wave index is uniform over the wave; saying so keeps the step
    // range, the loop branches and every descriptor in scalar registers.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int n0 = blockIdx.x * COLS;
    const int64_t ldb2 = p.ldb * 2, lda2 = p.lda * 2;

    // Group cp of a step: stored rows n0 + 32cp .. +31; its descriptor ends
    // at the last valid row's k = K - 1 (range 0 when no row is valid).
    const uint8_t* gbase[4];
    uint32_t grange[4];
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) {
        const int row0 = n0 + GROUP_ROWS * cp;
        const int rows = min(GROUP_ROWS, p.N - row0);
        gbase[cp] = static_cast<const uint8_t*>(p.B) + (int64_t)row0 * ldb2;
        grange[cp] = rows <= 0 ? 0u : (uint32_t)((int64_t)(rows - 1) * ldb2 + 2 * (int64_t)p.K);
    }
    // Instruction j of a group fills local rows 4j .. 4j+3 (256 B each);
    // lane l writes row lr = 4j + l/16 at position l%16 and fetches the
    // chunk c = (l%16) ^ (lr%16) of it, so chunk c of row lr sits at
    // position c ^ (lr%16): the operand reads below (16 rows, one chunk)
    // then touch 16 distinct 16-byte bank groups.
    uint32_t vrow[8];
    int kc[4];  // first k of this lane's chunk for instructions j = 4h + (j%4)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int lr = 4 * j + g;
        const int c = i ^ (lr & 15);
        vrow[j] = (uint32_t)(lr * ldb2 + 16 * c);
        kc[j & 3] = 8 * c;
    }

    // A: row 16rb + i of the RB row blocks; the descriptor covers rows 0 ..
    // M-1 (k = K - 1 of the last).
    const uint32_t arange = (uint32_t)((int64_t)(p.M - 1) * lda2 + 2 * (int64_t)p.K);
    const __amdgpu_buffer_rsrc_t rsa =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), 0, arange, kBufferRsrcW3);
    uint32_t arow[RB];
    bool aok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        aok[rb] = 16 * rb + i < p.M;
        arow[rb] = aok[rb] ? (uint32_t)((16 * rb + i) * lda2) : 0u;
    }

    const int nsteps = (p.K + STEP_K - 1) / STEP_K;
    int s0, s1;
    wave_steps(nsteps, NW, wave, s0, s1);

    floatx4 acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Eight copy instructions: group cp of step s into stage cp % NS.
    auto issue = [&](auto cpc, int s) {
        constexpr int cp = decltype(cpc)::value;
        uint8_t* dst = dma::pick<cp % NS>(st0, st1, st2, st3) + STAGE * wave;
        const int lim = p.K - STEP_K * s;  // chunks at k >= K read zeros
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t voff = kc[j & 3] < lim ? vrow[j] + (uint32_t)(256 * s) : grange[cp];
            copy_b(gbase[cp], grange[cp], dst + 1024 * j, voff);
        }
    };
    // RB x 4 loads: a[rb][u] = row 16rb + i, k = 128s + 32u + 8g .. +7.
    auto load_a = [&](int s, u32x4 (&a)[RB][4]) {
        const int lim = p.K - STEP_K * s;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = aok[rb] && 32 * u + 8 * g < lim;
                const uint32_t voff = ok ? arow[rb] + (uint32_t)(256 * s + 64 * u + 16 * g) : arange;
                a[rb][u] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsa, (int)voff, 0, 0));
            }
    };
    // Group cp from stage cp % NS: MFMA block b (local rows 16b + i), quarter
    // u (chunk 4u + g); accumulator 2cp + b holds columns 32cp + 16b .. +15.
    auto compute = [&](auto cpc, const u32x4 (&a)[RB][4]) {
        constexpr int cp = decltype(cpc)::value;
        const uint8_t* st = dma::pick<cp % NS>(st0, st1, st2, st3) + STAGE * wave;
        // All eight operand reads first, so that their LDS round trips
        // overlap each other.
        u32x4 bop[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                bop[b][u] = *reinterpret_cast<const u32x4*>(
                    st + (16 * b + i) * 256 + (((4 * u + g) ^ i) << 4));
        __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the MFMAs
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][2 * cp + b] = mfma16x16x32<T>(a[rb][u], bop[b][u], acc[rb][2 * cp + b]);
    };
    // Before a copy overwrites a stage, this wave's reads of it must have
    // returned (they have: their MFMAs came first; the wait makes it explicit).
    auto wait_reads = [] { DMA_WAIT_VMCNT_LGKM0(63); };
    auto fence = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Group cp of step s.  Before reading it the wave copies the group D
    // places ahead (group cp + D of this step, or of the next), and at cp = 0
    // of a step that is not its last it loads A of the next step right after
    // that copy.  The wait then lets through everything issued after the copy
    // of group cp: the D later groups' copies (8 instructions each), plus the
    // RB x 4 A loads when they came after it, which is when that copy was
    // issued in this step's cp = 0 phase or earlier (cp <= D).  A loads of
    // earlier steps always precede it.  In the wave's last step nothing is
    // loaded past its group 3, so only min(D, 3 - cp) copies follow.  The
    // prologue loads A of the first step and then copies its groups 0 .. D-1,
    // which gives the first step the same counts.
    auto phase = [&](auto cpc, auto lastc, int s, const u32x4 (&a)[RB][4], u32x4 (&an)[RB][4]) {
        constexpr int cp = decltype(cpc)::value;
        constexpr bool kLast = decltype(lastc)::value;
        constexpr int ahead = cp + D;  // group copied now, counted from this step
        if constexpr (!kLast || ahead <= 3) {
            wait_reads();
            issue(std::integral_constant<int, ahead % 4>{}, s + ahead / 4);
            fence();
        }
        if constexpr (!kLast && cp == 0) {
            load_a(s + 1, an);
            fence();
        }
        constexpr int after = kLast ? 8 * (D < 3 - cp ? D : 3 - cp)
                                    : 8 * D + (cp <= D ? 4 * RB : 0);
        static_assert(after <= 63, "vmcnt holds 6 bits");
        DMA_WAIT_VMCNT(after);
        fence();
        compute(cpc, a);
        fence();
    };
    auto step = [&](auto lastc, int s, const u32x4 (&a)[RB][4], u32x4 (&an)[RB][4]) {
        phase(std::integral_constant<int, 0>{}, lastc, s, a, an);
        phase(std::integral_constant<int, 1>{}, lastc, s, a, an);
        phase(std::integral_constant<int, 2>{}, lastc, s, a, an);
        phase(std::integral_constant<int, 3>{}, lastc, s, a, an);
    };

    if (s0 < s1) {
        u32x4 a0[RB][4], a1[RB][4];
        load_a(s0, a0);
        fence();
        issue(std::integral_constant<int, 0>{}, s0);
        if constexpr (D > 1) issue(std::integral_constant<int, 1>{}, s0);
        if constexpr (D > 2) issue(std::integral_constant<int, 2>{}, s0);
        fence();
        // Unrolled by two so that the A buffers alternate without copies.
        using Full = std::false_type;
        using Last = std::true_type;
        int s = s0;
        for (; s + 2 < s1; s += 2) {
            step(Full{}, s, a0, a1);
            step(Full{}, s + 1, a1, a0);
        }
        if (s + 1 < s1) {
            step(Full{}, s, a0, a1);
            step(Last{}, s + 1, a1, a0);
        } else {
            step(Last{}, s, a0, a1);
        }
    }

    // Every wave's copies have landed (its last wait counted none) and its
    // reads returned: stage 0 becomes the reduction buffer, one 16-row block
    // at a time: red[w][row][col] at float (16w + row)*COLS + (col ^ 16*(row/4
    // % 4)), so the four row quarters of a write land in distinct banks.
    __syncthreads();
    float* red = reinterpret_cast<float*>(st0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        if (rb) __syncthreads();  // the previous block's sums have been read
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                red[(16 * wave + 4 * g + r) * COLS + ((16 * c + i) ^ (16 * g))] = acc[rb][c][r];
        __syncthreads();
        for (int o = threadIdx.x; o < 16 * COLS; o += NW * 64) {
            const int row = o / COLS, cl = o % COLS;
            const int m = 16 * rb + row, n = n0 + cl;
            if (m >= p.M || n >= p.N) continue;
            const int at = row * COLS + (cl ^ (16 * ((row >> 2) & 3)));
            float sum = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[16 * COLS * w + at];
            float* cptr = p.C + (int64_t)m * p.ldc + n;
            *cptr = epilogue(sum, p, cptr, n);
        }
    }
}

template <In T, int RB>
hipError_t launch_rb(const GemmParams& p, hipStream_t s) {
    constexpr int NW = RB <= 2 ? 8 : 4, NS = NW == 8 ? 2 : 4;
    const dim3 grid((p.N + COLS - 1) / COLS, p.batch), block(NW * 64);
    hipLaunchKernelGGL((skinny16_bt_dma_kernel<T, RB, NW, NS>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

// A stored M x K and B stored N x K, 1 <= M <= 64, K a multiple of 8 (a
// 16-byte piece is then all inside or all outside k < K), 16-byte aligned
// rows, and every offset within a descriptor below 2^31 (pitches below
// 2^24 elements: at most 64 rows of A or 32 of B per descriptor).
bool skinny16_bt_dma_eligible(const GemmParams& p) {
    return !p.ta && p.tb && p.M >= 1 && p.M <= kSkinnyMaxM && p.N >= 1 && p.K >= 8 &&
           p.K % 8 == 0 && operands_16b_aligned(p, 2) && p.lda < kMaxBufferPitch &&
           p.ldb < kMaxBufferPitch;
}

template <In T>
hipError_t launch_skinny16_bt_dma(const GemmParams& p, hipStream_t s) {
    if (!skinny16_bt_dma_eligible(p)) return hipErrorInvalidValue;
    switch ((p.M + 15) / 16) {
        case 1: return launch_rb<T, 1>(p, s);
        case 2: return launch_rb<T, 2>(p, s);
        case 3: return launch_rb<T, 3>(p, s);
        case 4: return launch_rb<T, 4>(p, s);
        default: return hipErrorInvalidConfiguration;
    }
}
template hipError_t launch_skinny16_bt_dma<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_skinny16_bt_dma<In::F16>(const GemmParams&, hipStream_t);

}  // namespace dgt
