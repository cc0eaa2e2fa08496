// k_skinny_dma.hip -- the bandwidth-bound path for a linear layer's
// decode-shaped product: M <= 64 rows of A stored M x K and the weight B
// stored N x K (every column of op(B) a stored row, k contiguous), 16-bit
// or fp32 inputs.  Same reasoning as the register-staged skinny kernels:
// the time is the time to stream B once.
//
// The kernel works in bytes: a step covers a 256- or 128-byte piece of each
// stored row (128 or 64 k of 16-bit inputs, 64 or 32 of fp32), and a lane's
// 16-byte chunk of A meets the same 16 bytes of B in one 16x16x32 product
// (16-bit) or four 16x16x4 ones (fp32).  With fp32 B the register-staged
// kernel's loads touch 16 stored rows with 64 bytes each per instruction;
// through this kernel the same B streams 1.5-2x faster (28672 x 8192
// weights: M = 8 142.5 against 219.9 us, M = 64 277.9 against 554.3).
//
// B never passes through registers: each wave copies its groups of B
// straight into LDS with buffer loads that write LDS (one 16-byte piece per
// lane, 1 KiB per instruction), into a private ring of stages.  No wave
// reads another wave's stages, so the loop has no workgroup barrier; each
// wave waits only for its own copies (vector-memory loads complete in issue
// order, so one wait count per group suffices).  The registers this frees
// buy waves: measured on 28672 x 8192 weights, the rate follows the number
// of waves per CU far more than the bytes each wave keeps in flight (four
// waves with three 8-KiB groups each in flight stream no faster than four
// register-staged waves with one or two).  So the configuration per row
// count is the one with the most waves that fits without spilling (a
// kernel that spills is also held to fewer concurrent waves by its scratch):
//   M <= 32: eight waves, 256-byte steps, two stages (one group in flight),
//            A for the next step loaded a step ahead into a second buffer;
//   M <= 64: eight waves, 128-byte steps (4-KiB groups, half the A
//            registers), four stages, and one A buffer reloaded after each
//            step's last MFMAs: at four row blocks the 128 accumulator
//            registers leave no room for a second (with it the kernel
//            spills), and one buffer is faster at three as well.
// Splitting a strip's columns over two waves instead (halving the
// accumulators) was slower: both waves then read every A slice, and the
// extra A requests cost more than the waves gain.
//
// Work split as in the register-staged kernel: a workgroup owns a strip of
// up to 128 columns (stored rows of B) over all of K, each wave one K-range;
// a step is four groups of 32 stored rows.  The strip width is chosen per
// launch so that the strips fill the 256 CUs (strip_cols).  The partial tiles are summed in
// LDS in wave order (deterministic, no atomics, no workspace).  A (at most
// 64 x K, shared by every workgroup and re-read from cache) is loaded into
// registers one step ahead with plain buffer loads, so that a wave issues
// the same number of vector-memory instructions per step whatever the shape
// (the wait counts rely on it).
//
// Operands through buffer descriptors: a 16-byte piece past a descriptor's
// range reads as zeros.  Each group has a descriptor that ends at its last
// valid stored row (k = K - 1), so rows past N read zeros; pieces at k >= K
// (K a multiple of the elements in 16 bytes, so a piece is all inside or
// all outside) get an offset at the range end and read zeros too, as do
// rows of A past M.
#include <algorithm>

#include "skinny_common.hpp"
#include "dma_common.hpp"

namespace dgt {

namespace {

using namespace skinny;

constexpr int COLS = 128;        // columns (stored rows of B) per workgroup
constexpr int GR = 32;           // stored rows per group (four groups a step)
constexpr int kBPolicy = 2;      // cache policy of the B copies: nt (streamed once)

// Geometry of a step whose row pieces are ROWB bytes (256 or 128: 128 or
// 64 k of 16-bit inputs, 64 or 32 of fp32): a group is GR stored rows x one
// piece, copied by INSTR instructions of RPI rows each (LPR lanes per row).  In LDS chunk c of local row r sits at
// position c ^ swz(r), so that the operand reads (16 rows, one chunk) touch
// 16 distinct 16-byte bank groups: with 256-byte rows 16 positions per row
// serve; with 128-byte rows two rows share a 256-byte bank line, so rows r
// and r + 8 (same line half) must differ: the swizzle uses r / 2.
template <int ROWB_>
struct Geo {
    static_assert(ROWB_ == 256 || ROWB_ == 128, "a row piece is 256 or 128 bytes");
    static constexpr int ROWB = ROWB_;
    static constexpr int STAGE = GR * ROWB;           // bytes of one group
    static constexpr int INSTR = STAGE / 1024;        // copy instructions per group
    static constexpr int RPI = 1024 / ROWB;           // rows per copy instruction
    static constexpr int LPR = ROWB / 16;             // lanes per row
    static constexpr int U = ROWB / 64;               // 64-byte MFMA k-slices per step
    static constexpr int RED_ROWS = STAGE / (COLS * 4);  // C rows per reduction pass
    __device__ static int swz(int r) { return ROWB == 256 ? (r & 15) : ((r >> 1) & 7); }
};

// The products of one 16-byte chunk of A and of B per lane (lane group g =
// l/16 holding the chunk's k): one 16x16x32 instruction for 16-bit inputs;
// four 16x16x4 ones for fp32, the j-th taking element j of each chunk, so
// that k-slot g of product j is the chunk's element j (every k of the 64
// bytes lands in the sum once, as with the 16-bit form).
template <In T>
__device__ __forceinline__ floatx4 mfma_chunk(u32x4 a, u32x4 b, floatx4 c) {
    if constexpr (T == In::F32) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]),
                                                     c, 0, 0, 0);
        return c;
    } else {
        return mfma16x16x32<T>(a, b, c);
    }
}

// One 16-byte piece per lane of B into LDS: lane l's bytes at base + voff
// land at lds + 16*l.
__device__ __forceinline__ void copy_b(const void* base, uint32_t range, uint8_t* lds,
                                       uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, range, kBufferRsrcW3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (dma::lds_void*)lds, 16, voff, 0, 0, kBPolicy);
}

// NW waves (one K-range each), a ring of NS stages per wave (NS divides the
// four groups of a step, so group cp of any step uses stage cp % NS), steps
// of ROWB bytes per row (SK elements); kSingleA: one register buffer of A
// operands, reloaded after each step's last MFMAs (else two, the next
// step's loaded one step ahead).
template <In T, int RB, int NW, int NS, int ROWB, bool kSingleA>
__global__ __launch_bounds__(NW * 64, 1) void skinny_bt_dma_kernel(GemmParams p, int cols) {
    using G = Geo<ROWB>;
    constexpr int ESZ = T == In::F32 ? 4 : 2;  // bytes per element
    constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
    constexpr int SK = ROWB / ESZ;             // k per step
    static_assert(NS == 2 || NS == 4, "a step's four groups map onto the ring");
    constexpr int D = NS - 1;  // groups copied ahead of the one being read
    constexpr int STAGE = G::STAGE;
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
    // The workgroup's strip: `cols` (<= COLS, a multiple of 16) stored rows
    // from n0; the four groups of a step always span COLS rows, and the rows
    // past the strip read zeros through the group descriptors.
    const int n0 = blockIdx.x * cols;
    const int nlim = min(n0 + cols, p.N);
    const int64_t ldb2 = p.ldb * ESZ, lda2 = p.lda * ESZ;  // bytes

    // Group cp of a step: stored rows n0 + 32cp .. +31; its descriptor ends
    // at the last valid row's k = K - 1 (range 0 when no row is valid).
    const uint8_t* gbase[4];
    uint32_t grange[4];
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) {
        const int row0 = n0 + GR * cp;
        const int rows = min(GR, nlim - row0);
        gbase[cp] = static_cast<const uint8_t*>(p.B) + (int64_t)row0 * ldb2;
        grange[cp] = rows <= 0 ? 0u : (uint32_t)((int64_t)(rows - 1) * ldb2 + ESZ * (int64_t)p.K);
    }
    // Instruction j of a group fills local rows RPI*j .. +RPI-1; lane l
    // writes row lr = RPI*j + l/LPR at position l%LPR, so it fetches chunk
    // (l%LPR) ^ swz(lr) of that row.
    uint32_t vrow[G::INSTR];
    int kc[G::INSTR];  // first k of the lane's chunk, within the step
#pragma unroll
    for (int j = 0; j < G::INSTR; ++j) {
        const int lr = G::RPI * j + lane / G::LPR;
        const int c = (lane % G::LPR) ^ G::swz(lr);
        vrow[j] = (uint32_t)(lr * ldb2 + 16 * c);
        kc[j] = EPC * c;
    }

    // A: row 16rb + i of the RB row blocks; the descriptor covers rows 0 ..
    // M-1 (k = K - 1 of the last).
    const uint32_t arange = (uint32_t)((int64_t)(p.M - 1) * lda2 + ESZ * (int64_t)p.K);
    const __amdgpu_buffer_rsrc_t rsa =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.A), 0, arange, kBufferRsrcW3);
    uint32_t arow[RB];
    bool aok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        aok[rb] = 16 * rb + i < p.M;
        arow[rb] = aok[rb] ? (uint32_t)((16 * rb + i) * lda2) : 0u;
    }

    const int nsteps = (p.K + SK - 1) / SK;
    int s0, s1;
    wave_steps(nsteps, NW, wave, s0, s1);

    floatx4 acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rb][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    // INSTR copy instructions: group cp of step s into stage cp % NS.
    auto issue = [&](auto cpc, int s) {
        constexpr int cp = decltype(cpc)::value;
        uint8_t* dst = dma::pick<cp % NS>(st0, st1, st2, st3) + STAGE * wave;
        const int lim = p.K - SK * s;  // chunks at k >= K read zeros
#pragma unroll
        for (int j = 0; j < G::INSTR; ++j) {
            const uint32_t voff = kc[j] < lim ? vrow[j] + (uint32_t)(G::ROWB * s) : grange[cp];
            copy_b(gbase[cp], grange[cp], dst + 1024 * j, voff);
        }
    };
    // RB x U loads: a[rb][u] = row 16rb + i, bytes 64u + 16g of the step's
    // piece (k = SK*s + 4*EPC*u + EPC*g .. +EPC-1).
    auto load_a = [&](int s, u32x4 (&a)[RB][G::U]) {
        const int lim = p.K - SK * s;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int u = 0; u < G::U; ++u) {
                const bool ok = aok[rb] && 4 * EPC * u + EPC * g < lim;
                const uint32_t voff =
                    ok ? arow[rb] + (uint32_t)(G::ROWB * s + 64 * u + 16 * g) : arange;
                a[rb][u] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsa, (int)voff, 0, 0));
            }
    };
    // Group cp from stage cp % NS: MFMA block b (local rows 16b + i), k-slice
    // u (chunk 4u + g); accumulator 2cp + b holds columns 32cp + 16b .. +15.
    auto compute = [&](auto cpc, const u32x4 (&a)[RB][G::U]) {
        constexpr int cp = decltype(cpc)::value;
        const uint8_t* st = dma::pick<cp % NS>(st0, st1, st2, st3) + STAGE * wave;
        // All operand reads first, so that their LDS round trips overlap.
        u32x4 bop[2][G::U];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int u = 0; u < G::U; ++u)
                bop[b][u] = *reinterpret_cast<const u32x4*>(
                    st + (16 * b + i) * G::ROWB + (((4 * u + g) ^ G::swz(16 * b + i)) << 4));
        __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the MFMAs
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int u = 0; u < G::U; ++u)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][2 * cp + b] = mfma_chunk<T>(a[rb][u], bop[b][u], acc[rb][2 * cp + b]);
    };
    // Before a copy overwrites a stage, this wave's reads of it must have
    // returned (they have: their MFMAs came first; the wait makes it explicit).
    auto wait_reads = [] { DMA_WAIT_VMCNT_LGKM0(63); };
    auto fence = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Group cp of step s.  Before reading it the wave copies the group D
    // places ahead (group cp + D of this step, or of the next).  The wait then
    // lets through everything issued after the copy of group cp: the D later
    // groups' copies (INSTR instructions each; in the wave's last step nothing
    // is copied past its group 3, so only min(D, 3 - cp)), plus the RB x U A
    // loads when they came after it.
    //  * Two A buffers: at cp = 0 of a step that is not its last, A of the
    //    next step is loaded right after that phase's copy; it follows the
    //    copy of group cp when that copy was issued in this cp = 0 phase or
    //    earlier (cp <= D).  The prologue loads A of the first step and then
    //    copies its groups 0 .. D-1, which gives the first step the same
    //    counts, and no A load follows any copy of the wave's last step.
    //  * One A buffer: A of step s is loaded at the end of the previous step's
    //    cp = 3 phase, after that phase's copy, so it follows the copy of
    //    group cp of step s when that copy was issued in the previous step's
    //    cp = 3 phase or earlier (cp <= D - 1), the last step included.  The
    //    prologue copies groups 0 .. D-1 and then loads A of the first step,
    //    which again gives the same counts.
    using AOps = u32x4[RB][G::U];
    auto phase = [&](auto cpc, auto lastc, int s, const AOps& a, AOps& an) {
        constexpr int cp = decltype(cpc)::value;
        constexpr bool kLast = decltype(lastc)::value;
        constexpr int ahead = cp + D;  // group copied now, counted from this step
        if constexpr (!kLast || ahead <= 3) {
            wait_reads();
            issue(std::integral_constant<int, ahead % 4>{}, s + ahead / 4);
            fence();
        }
        if constexpr (!kSingleA && !kLast && cp == 0) {
            load_a(s + 1, an);
            fence();
        }
        constexpr int copies = G::INSTR * (kLast ? (D < 3 - cp ? D : 3 - cp) : D);
        constexpr bool a_after = kSingleA ? cp <= D - 1 : (!kLast && cp <= D);
        constexpr int after = copies + (a_after ? RB * G::U : 0);
        static_assert(after <= 63, "vmcnt holds 6 bits");
        DMA_WAIT_VMCNT(after);
        fence();
        compute(cpc, a);
        fence();
        if constexpr (kSingleA && !kLast && cp == 3) {  // a and an are one buffer
            load_a(s + 1, an);
            fence();
        }
    };
    auto step = [&](auto lastc, int s, const AOps& a, AOps& an) {
        phase(std::integral_constant<int, 0>{}, lastc, s, a, an);
        phase(std::integral_constant<int, 1>{}, lastc, s, a, an);
        phase(std::integral_constant<int, 2>{}, lastc, s, a, an);
        phase(std::integral_constant<int, 3>{}, lastc, s, a, an);
    };

    using Full = std::false_type;
    using Last = std::true_type;
    auto prologue_copies = [&] {
        issue(std::integral_constant<int, 0>{}, s0);
        if constexpr (D > 1) issue(std::integral_constant<int, 1>{}, s0);
        if constexpr (D > 2) issue(std::integral_constant<int, 2>{}, s0);
        fence();
    };
    if (s0 < s1) {
        if constexpr (kSingleA) {
            AOps a0;
            prologue_copies();
            load_a(s0, a0);
            fence();
            int s = s0;
            for (; s + 1 < s1; ++s) step(Full{}, s, a0, a0);
            step(Last{}, s, a0, a0);
        } else {
            AOps a0, a1;
            load_a(s0, a0);
            fence();
            prologue_copies();
            // Unrolled by two so that the A buffers alternate without copies.
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
    }

    // Every wave's copies have landed (its last wait counted none) and its
    // reads returned: stage 0 becomes the reduction buffer, RR rows of C at a
    // time.  Wave w's partial for a row and a strip column col sits at float
    // (RR*w + row)*COLS + (col ^ 16*(grow/4 % 4)), grow the row within the
    // 16-row block, so the four row quarters of a write land in distinct
    // banks; the sums run over the waves in order.
    constexpr int RR = G::RED_ROWS;
    __syncthreads();
    float* red = reinterpret_cast<float*>(st0);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int h = 0; h < 16 / RR; ++h) {
            if (rb + h) __syncthreads();  // the previous pass's sums have been read
            if ((4 * g) / RR == h) {
#pragma unroll
                for (int c = 0; c < 8; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[(RR * wave + 4 * g + r - RR * h) * COLS + ((16 * c + i) ^ (16 * g))] =
                            acc[rb][c][r];
            }
            __syncthreads();
            for (int o = threadIdx.x; o < RR * COLS; o += NW * 64) {
                const int row = o / COLS, cl = o % COLS;
                const int grow = RR * h + row;
                const int m = 16 * rb + grow, n = n0 + cl;
                if (m >= p.M || n >= nlim) continue;
                const int at = row * COLS + (cl ^ (16 * ((grow >> 2) & 3)));
                float sum = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum += red[RR * COLS * w + at];
                float* cptr = p.C + (int64_t)m * p.ldc + n;
                *cptr = epilogue(sum, p, cptr, n);
            }
        }
}

// Strip width.  A launch takes about the longer of the time HBM needs to
// deliver B (about 6.5 TB/s to this kernel) and the time one CU needs to
// stream its strips' share of B: (waves of workgroups) x (strip width) x K x
// 2 bytes at the rate one workgroup pulls, measured on 28672 x 8192 weights:
// 29 GB/s with one row block of A, 24 GB/s with four (A's loads compete with
// B's), interpolated in between.  The width (a multiple of 16 from 64 to
// COLS) with the least time wins, ties (within 1%) to the wider strip, which
// re-reads A less.  So one row block keeps 128 on N = 28672 (224 strips
// already saturate HBM: 71.8 us), four take 112 (256 strips, one per CU:
// 83.5 us against 87.4 with 128), and a narrow N spreads over more CUs.
int strip_cols(const GemmParams& p, int rb, int esz) {
    constexpr int64_t kCUs = 256;
    const double hbm = 6.5e12, per_wg = 29e9 - (rb - 1) * (29e9 - 24e9) / 3.0;
    const double bytes_col = (double)esz * p.K;  // one column of B over all of K
    const double floor_s = bytes_col * p.N * p.batch / hbm;
    int best = COLS;
    double best_t = 0.0;
    for (int c = COLS; c >= 64; c -= 16) {
        const int64_t wgs = (int64_t)((p.N + c - 1) / c) * p.batch;
        const double t = std::max(floor_s, (double)((wgs + kCUs - 1) / kCUs) * c * bytes_col / per_wg);
        if (c == COLS || t < 0.99 * best_t) best = c, best_t = t;
    }
    return best;
}

template <In T, int RB, int NW, int NS, int ROWB, bool kSingleA>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
    const int cols = strip_cols(p, RB, T == In::F32 ? 4 : 2);
    const dim3 grid((p.N + cols - 1) / cols, p.batch), block(NW * 64);
    hipLaunchKernelGGL((skinny_bt_dma_kernel<T, RB, NW, NS, ROWB, kSingleA>), grid, block, 0,
                       s, p, cols);
    return hipGetLastError();
}

template <In T, int RB>
hipError_t launch_rb(const GemmParams& p, hipStream_t s) {
    if constexpr (RB <= 2) return launch_cfg<T, RB, 8, 2, 256, false>(p, s);
    else return launch_cfg<T, RB, 8, 4, 128, true>(p, s);
}

}  // namespace

// A stored M x K and B stored N x K, 1 <= M <= 64, K a multiple of the
// elements in 16 bytes (a 16-byte piece is then all inside or all outside
// k < K), 16-byte aligned rows, and every offset within a descriptor below
// 2^31 (at most 64 rows of A or 32 of B per descriptor).
template <In T>
bool skinny_bt_dma_eligible(const GemmParams& p) {
    constexpr int esz = T == In::F32 ? 4 : 2, epc = 16 / esz;
    if (p.ta || !p.tb || p.M < 1 || p.M > kSkinnyMaxM || p.N < 1 || p.K < epc ||
        !k_multiple(p, epc) || !operands_16b_aligned(p, esz) || p.lda < p.K || p.ldb < p.K)
        return false;
    const int64_t lim = int64_t(1) << 31;
    return (int64_t)(p.M - 1) * p.lda * esz + esz * (int64_t)p.K < lim &&
           (int64_t)(GR - 1) * p.ldb * esz + esz * (int64_t)p.K < lim;
}
template bool skinny_bt_dma_eligible<In::F32>(const GemmParams&);
template bool skinny_bt_dma_eligible<In::BF16>(const GemmParams&);
template bool skinny_bt_dma_eligible<In::F16>(const GemmParams&);

template <In T>
hipError_t launch_skinny_bt_dma(const GemmParams& p, hipStream_t s) {
    if (!skinny_bt_dma_eligible<T>(p)) return hipErrorInvalidValue;
    switch ((p.M + 15) / 16) {
        case 1: return launch_rb<T, 1>(p, s);
        case 2: return launch_rb<T, 2>(p, s);
        case 3: return launch_rb<T, 3>(p, s);
        case 4: return launch_rb<T, 4>(p, s);
        default: return hipErrorInvalidConfiguration;
    }
}
template hipError_t launch_skinny_bt_dma<In::F32>(const GemmParams&, hipStream_t);
template hipError_t launch_skinny_bt_dma<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_skinny_bt_dma<In::F16>(const GemmParams&, hipStream_t);

}  // namespace dgt
