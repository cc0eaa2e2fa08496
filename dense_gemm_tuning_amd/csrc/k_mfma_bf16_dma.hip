// k_mfma_bf16_dma.hip -- 16-bit-input (BF16 or FP16) / FP32-accumulate GEMM:
// global -> LDS by DMA up to three K slices ahead, operands stored with m / n
// contiguous transposed by the LDS read.
//
// Tiling as in the register-staged kernel (256 x 256 workgroup tile, 2 x 2
// wavefronts of 128 x 128, v_mfma_f32_32x32x16: dilfish.github.io 5.3-5.5,
// qwbw.cn Level 2), or, for launches with few such tiles, 128 x 128 (two
// workgroups per CU, wavefronts of 64 x 64), with a deeper software
// pipeline than the pages' double buffer (dilfish.github.io 5.4; qwbw.cn's
// double-buffering row).  The notes below give the 256 x 256 sizes; at 128
// a stage holds half the rows or columns and each wave half the copies:
//
//  * K advances in slices of 32.  Copies use buffer_load_dwordx4 ... lds:
//    lane l's 16 bytes land at LDS base + 16*l, so one instruction fills
//    1 KiB and no operand byte passes through a VGPR; a swizzle is applied by
//    the choice of which global chunk each lane fetches.  Each wave addresses
//    its rows through a buffer descriptor (wave-uniform base, 32-bit lane
//    offsets, range-checked by the hardware); against the same copies as
//    global_load_lds the L2 requests return sooner and the kernel is ~2%
//    faster.
//  * An operand is staged by how it is stored, not by whether it is A or B.
//    K-contiguous (A as M x K, B transposed as N x K): two LDS stages of two
//    slices each, 256 rows of 128 B (chunk q of row r at q ^ ((r ^ r>>3) & 7)),
//    so each copy request covers a 128-byte row segment; a lane reads its 8
//    consecutive k with one 16-byte LDS read.  MN-contiguous (B as K x N, A
//    transposed as K x M): four stages of one slice, 32 k-rows of 512 B
//    (chunk c of row k at c ^ (4*(k & 3))); ds_read_b64_tr_b16 transposes
//    on the read: within each 16-lane group, source lane 4r+q names row r,
//    columns 4q..4q+3, and destination lane j receives column j, rows 0..3;
//    two reads give a lane its 8 consecutive k (the pages warn that an
//    operand in the wrong major order still "looks right": dilfish.github.io
//    5.5).  Either way 64 KiB per operand, 128 KiB of the 160 KiB LDS.
//  * Copies start as soon as a stage is retired, 1.25 to 2.5 slices (1200 to
//    2500 MFMA cycles) before the data is needed, which covers L2-miss
//    latency to the memory side.  Each wave's copies are spread one per two
//    MFMAs; issued in bursts they queue at the address unit and in L1 and
//    hold back the wave's MFMA issue.  Copies past the last slice re-read the last
//    slice (never consumed) so every step waits on the same count.
//  * Per slice each wavefront issues 32 MFMAs in two 16-deep steps; the LDS
//    reads of the next step are interleaved with them.  The workgroup
//    barrier sits between the two steps: it publishes slice t+1 (every wave
//    has waited for its own copies) and retires slice t's stage, so the
//    first operands of slice t+1 are read while step 2 of slice t computes.
//
// Used for any M, N and K with 16-byte aligned rows and row pitches below
// 2^24 elements (so that a wave's rows of lane offsets fit 32 bits).  On edge
// tiles the copy descriptors' ranges stop at the operands' last elements and
// the epilogue stores only the valid part.  When K is not a multiple of 128
// the K loop runs in groups of four 32-deep slices and the last group (1 to
// 4 slices) after it as ordinary slices (each keeps its copies, waits and
// barrier, so every wait count holds); in a partial last slice the
// k-contiguous fragments are masked past K, and m/n-contiguous rows past K
// read as zeros through the descriptor range.  The register-staged kernel
// handles unaligned operands.
#include "dma_common.hpp"
#include "streamk.hpp"

namespace dgt {

namespace {

using namespace dma;

constexpr int BK = 32, NT = 256, NSTAGE = 4;
constexpr double kCost128 = 1.22;           // a 128-tile's time, in quarters of a 256-tile's

// Geometry of a workgroup tile of R x R (R = 256 or 128; a 2 x 2 grid of
// wavefronts of R/2 x R/2).  A k-contiguous stage holds R rows of 128 B (two
// slices), copied 8 rows per instruction; an m/n-contiguous stage holds 32
// k-rows of 2R bytes, 512/R k-rows per instruction; each wave copies a
// quarter of either.
template <int R>
struct Geo {
    static constexpr int TM = R / 64;          // 32 x 32 MFMA tiles per wave and dimension
    static constexpr int KC_ROWS = R / 4;      // k-contiguous rows per wave
    static constexpr int KC_INSTR = R / 32;    // their copy instructions per pair
    static constexpr int KC_STAGE = R * 128;   // bytes
    static constexpr int MN_ROW = 2 * R;       // bytes per k-row
    static constexpr int MN_LPR = R / 8;       // 16-byte chunks (lanes) per k-row
    static constexpr int MN_INSTR = R / 64;    // copy instructions per slice and wave
    static constexpr int MN_STAGE = BK * MN_ROW;
};

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;







// A K-contiguous operand: stage = a pair of slices, R rows x 128 B.  Wave w
// issues copy instructions j = (R/32)w + i per pair, instruction j filling
// rows 8j .. 8j+7 (8 lanes per row), as two halves.  The wave's descriptor
// covers its R/4 rows; pair pr adds 128*pr bytes through the scalar offset.
template <int R>
struct KcOperand {
    using G = Geo<R>;
    const uint16_t* base;         // row (R/4)*wave of the tile (wave-uniform)
    uint32_t voff[G::KC_INSTR];   // lane byte offsets from base, per instruction
    uint32_t bytes;               // descriptor range: the wave's rows
    int off[G::TM][2][2];         // LDS read offset: tile t, slice-in-pair u, step s
    int npair;

    // mn0: first row (m or n) of the workgroup tile; w: this wave's half of
    // it (wm or wn); mn_lim: rows of the operand (M or N), K its row length.
    // The descriptor range ends at the wave's last element (k = K - 1 of its
    // last row, or of row mn_lim - 1 on an edge tile), so rows past mn_lim
    // and the k past K of a final half pair are never read from memory (they
    // return zeros; they only feed outputs that are not stored, or slices
    // that are not computed).
    template <bool kEdge>
    __device__ void init(const uint16_t* X, int64_t ld, int mn0, int w, int wave, int lane,
                         int nk, int mn_lim, int K) {
#pragma unroll
        for (int i = 0; i < G::KC_INSTR; ++i) {
            const int row = 8 * (G::KC_INSTR * wave + i) + (lane >> 3);
            const int q = (lane & 7) ^ swz_kc(row);
            voff[i] = (uint32_t)(((int64_t)(row - G::KC_ROWS * wave) * ld + 8 * q) * 2);
        }
        base = X + (int64_t)(mn0 + G::KC_ROWS * wave) * ld;
        int rows = G::KC_ROWS;
        if constexpr (kEdge) rows = min(G::KC_ROWS, mn_lim - (mn0 + G::KC_ROWS * wave));
        bytes = rows <= 0 ? 0u : (uint32_t)(((int64_t)(rows - 1) * ld + round_chunk<8>(K)) * 2);
        // rows w*R/2 + t*32 + l%32; half-wave h reads chunk 4u + 2s + h
        const int h = lane >> 5;
#pragma unroll
        for (int t = 0; t < G::TM; ++t) {
            const int row = w * (R / 2) + t * 32 + (lane & 31);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    off[t][u][s] = row * 128 + (((4 * u + 2 * s + h) ^ swz_kc(row)) << 4);
        }
        npair = (nk + 1) / 2;  // an odd slice count ends with half a pair
    }
    // Half `half` of pair pr into stage st (past the end: the last pair).
    // With a K tail (kTail) the descriptor starts at the pair, so the whole
    // offset of every lane is range-checked (the scalar offset is not) and
    // the k past K of a final half pair is never read; pair and range are
    // wave-uniform, which readfirstlane tells the compiler.  Otherwise every
    // k read is below K and the pair's offset goes in the scalar offset.
    template <bool kEdge = false, bool kTail = false>
    __device__ void copy(uint8_t* st, int pr, int half, int wave) const {
        pr = pr < npair ? pr : npair - 1;
        const uint8_t* from = reinterpret_cast<const uint8_t*>(base);
        uint32_t range = bytes, soff = (uint32_t)pr * (2 * BK * 2);
        if constexpr (kTail) {
            pr = __builtin_amdgcn_readfirstlane(pr);
            const uint32_t skip = (uint32_t)pr * (2 * BK * 2);
            range = __builtin_amdgcn_readfirstlane(bytes > skip ? bytes - skip : 0u);
            from += skip;
            soff = 0;
        }
        constexpr int HALF = G::KC_INSTR / 2;
#pragma unroll
        for (int i = HALF * half; i < HALF * half + HALF; ++i)
            dma16(from, range, st + (G::KC_INSTR * wave + i) * 1024, voff[i], soff);
    }
    // Operands of step s of the slice in half u of stage st.
    __device__ void frags(const uint8_t* st, int u, int s, u32x4 (&f)[G::TM]) const {
#pragma unroll
        for (int t = 0; t < G::TM; ++t) f[t] = *reinterpret_cast<const u32x4*>(st + off[t][u][s]);
    }
    static constexpr int kReads = G::TM;  // LDS reads per step
    static constexpr int kHalfCopies = G::KC_INSTR / 2;
    static constexpr int kStage = G::KC_STAGE;
};

// Transposing LDS read of 4 k-rows x 4 columns per 16-lane group (a plain
// function, like dma16).
__device__ __forceinline__ shortx4 read_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)p);
}

// An MN-contiguous operand: stage = one slice, 32 k-rows x 2R bytes.  Wave w
// copies k-rows 8w .. 8w+7 with R/64 instructions (512/R k-rows each, R/8
// lanes per k-row), as two halves.
template <int R>
struct MnOperand {
    using G = Geo<R>;
    const uint16_t* base;        // k-row 8*wave of slice 0, first column of the tile
    uint32_t voff[G::MN_INSTR];  // lane byte offsets from base, per instruction
    uint32_t bytes;              // descriptor range: 8 k-rows
    int off[G::TM];
    int64_t slice;
    int nk;
    int64_t ld_;
    int rows_left0;        // k-rows from this wave's first one to the end
    int cols;              // valid columns of the tile (edge tiles)

    // mn_lim, K: columns and rows of the stored operand.  On an edge tile the
    // range of slice kt's descriptor stops at the operand's last element;
    // columns past mn_lim in earlier rows are read (they belong to the next
    // row) but only feed outputs the epilogue does not store.
    template <bool kEdge>
    __device__ void init(const uint16_t* X, int64_t ld, int mn0, int w, int wave, int lane,
                         int nk_, int mn_lim, int K) {
#pragma unroll
        for (int i = 0; i < G::MN_INSTR; ++i) {
            const int krow = 8 * wave + (512 / R) * i + lane / G::MN_LPR;
            const int c = (lane % G::MN_LPR) ^ (4 * (krow & 3));
            voff[i] = (uint32_t)(((int64_t)(krow - 8 * wave) * ld + 8 * c) * 2);
        }
        base = X + (int64_t)(8 * wave) * ld + mn0;
        bytes = (uint32_t)(8 * ld * 2);
        ld_ = ld;
        rows_left0 = K - 8 * wave;
        cols = kEdge ? round_chunk<8>(mn_lim - mn0) : 0;
        // Source lane 4r+q of 16-lane group G reads k-row 16s + 8h + 4t + r,
        // columns w*R/2 + tile*32 + 16*(G%2) + 4q .. +3 (t = which of the two
        // reads); k & 3 == r.
        const int r = (lane & 15) >> 2, q = lane & 3, g = (lane >> 4) & 1, h = lane >> 5;
#pragma unroll
        for (int t = 0; t < G::TM; ++t) {
            const int chunk = (w * (R / 16) + t * 4 + 2 * g + (q >> 1)) ^ (4 * r);
            off[t] = (8 * h + r) * G::MN_ROW + chunk * 16 + (q & 1) * 8;
        }
        slice = (int64_t)BK * ld;
        nk = nk_;
    }
    // Half `half` of slice kt into stage st (past the end: the last slice).
    template <bool kEdge = false, bool kTail = false>
    __device__ void copy(uint8_t* st, int kt, int half, int wave) const {
        kt = kt < nk ? kt : nk - 1;
        uint32_t range = bytes;
        if constexpr (kEdge) {
            const int64_t end = (int64_t)(rows_left0 - BK * kt - 1) * ld_ + cols;  // elements
            if (end < 8 * ld_) range = end <= 0 ? 0u : (uint32_t)(end * 2);
        }
        constexpr int HALF = G::MN_INSTR / 2;
#pragma unroll
        for (int i = HALF * half; i < HALF * half + HALF; ++i)
            dma16(base + kt * slice, range, st + (G::MN_INSTR * wave + i) * 1024, voff[i], 0);
    }
    __device__ void frags(const uint8_t* st, int s, u32x4 (&f)[G::TM]) const {
#pragma unroll
        for (int t = 0; t < G::TM; ++t) {
            const uint8_t* base = st + off[t] + s * 16 * G::MN_ROW;
            const shortx4 lo = read_tr16(base);
            const shortx4 hi = read_tr16(base + 4 * G::MN_ROW);
            const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            f[t] = __builtin_bit_cast(u32x4, v);
        }
    }
    static constexpr int kReads = 2 * G::TM;
    static constexpr int kHalfCopies = G::MN_INSTR / 2;
    static constexpr int kStage = G::MN_STAGE;
};


// TA / TB: A / B stored transposed.  A is K-contiguous unless TA, B is
// K-contiguous when TB.
// kEdge: M or N not a multiple of the tile (edge tiles read through
// clipped descriptor ranges and store only their valid part).  kTail: K is
// not a multiple of 128 (a last group of 1 to 4 slices after the loop, the
// last slice possibly partial).
// R: workgroup tile R x R (256: one workgroup per CU; 128: two).
// One R x R output tile at (m0, n0) over k = 0 .. p.K-1 of p's operands:
// the body of mfma16_dma_kernel, shared with the stream-K kernel.  raw ==
// nullptr: the BLAS epilogue into p.C; otherwise the bare fp32 sums go to
// raw (R x R, row pitch R, every element written; a stream-K partial tile).
template <In T, int R, bool TA, bool TB, bool kEdge, bool kTail>
__device__ __forceinline__ void dma_tile(const GemmParams& p, int m0, int n0, float* raw) {
    constexpr bool AK = !TA, BKc = TB;
    constexpr int TM = Geo<R>::TM;
    using OpA = typename std::conditional<AK, KcOperand<R>, MnOperand<R>>::type;
    using OpB = typename std::conditional<BKc, KcOperand<R>, MnOperand<R>>::type;
    constexpr int SA01 = OpA::kStage, SA23 = AK ? 16 : OpA::kStage;
    constexpr int SB01 = OpB::kStage, SB23 = BKc ? 16 : OpB::kStage;
    constexpr int CKC = AK ? OpA::kHalfCopies : BKc ? OpB::kHalfCopies : 0;
    constexpr int CMN = !AK ? OpA::kHalfCopies : !BKc ? OpB::kHalfCopies : 0;
    // One LDS object per operand and stage (K-contiguous operands use two).
    __shared__ __attribute__((aligned(1024))) uint8_t sA0[SA01];
    __shared__ __attribute__((aligned(1024))) uint8_t sA1[SA01];
    __shared__ __attribute__((aligned(1024))) uint8_t sA2[SA23];
    __shared__ __attribute__((aligned(1024))) uint8_t sA3[SA23];
    __shared__ __attribute__((aligned(1024))) uint8_t sB0[SB01];
    __shared__ __attribute__((aligned(1024))) uint8_t sB1[SB01];
    __shared__ __attribute__((aligned(1024))) uint8_t sB2[SB23];
    __shared__ __attribute__((aligned(1024))) uint8_t sB3[SB23];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
    const int nk = (p.K + BK - 1) / BK;  // slices (the last one partial when K % 32 != 0)

    OpA opa;
    OpB opb;
    opa.template init<kEdge>(static_cast<const uint16_t*>(p.A), p.lda, m0, wm, wave, lane, nk,
                             p.M, p.K);
    opb.template init<kEdge>(static_cast<const uint16_t*>(p.B), p.ldb, n0, wn, wave, lane, nk,
                             p.N, p.K);

    floatx16 acc[TM][TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Operands of step s of slice position J (0..3 within a group of four
    // slices: a K-contiguous operand has it in stage J/2, half J%2; an
    // MN-contiguous one in stage J).
    auto frags = [&](auto Jc, int s, u32x4 (&a)[TM], u32x4 (&b)[TM]) {
        constexpr int J = decltype(Jc)::value;
        if constexpr (AK) opa.frags(pick<J / 2>(sA0, sA1, sA2, sA3), J % 2, s, a);
        else opa.frags(pick<J>(sA0, sA1, sA2, sA3), s, a);
        if constexpr (BKc) opb.frags(pick<J / 2>(sB0, sB1, sB2, sB3), J % 2, s, b);
        else opb.frags(pick<J>(sB0, sB1, sB2, sB3), s, b);
    };

    // 16 MFMAs on (a, b).  The LDS reads and the copies issued just before
    // in program order are spread between them (per 4 MFMAs: 2 to 4 LDS
    // reads; a copy after every second MFMA), so the address unit never sees
    // a burst that would hold the wave, and its MFMA issue, back.
    // (At 128 x 128 a step is 4 MFMAs: after each, two LDS reads and a copy.)
    constexpr int DS_PER = (OpA::kReads + OpB::kReads) / 4;
    auto mfma_step = [&](const u32x4 (&a)[TM], const u32x4 (&b)[TM]) {
#pragma unroll
        for (int ti = 0; ti < TM; ++ti)
#pragma unroll
            for (int tj = 0; tj < TM; ++tj)
                acc[ti][tj] = mfma32x32x16<T>(a[ti], b[tj], acc[ti][tj]);
        if constexpr (TM == 4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
                    if (m < DS_PER) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
                    if (m & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // copy
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < TM * TM; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // copy
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    u32x4 a0[TM], b0[TM], a1[TM], b1[TM];


    // Slice kt at position J of its group of four.  Copies, per wave:
    //   before the barrier: MN-contiguous operands the second half of slice
    //     kt+3 (into stage (J+3)%4); for even J, K-contiguous operands the
    //     second half of pair kt/2+1 (into the other pair stage);
    //   after the barrier: MN-contiguous operands the first half of slice
    //     kt+4 into stage J (just retired); for odd J, K-contiguous operands
    //     the first half of pair (kt+3)/2 into the pair stage retired by this
    //     barrier.
    // The barrier of slice kt publishes slice kt+1.
    // In a partial last slice (K % 32 != 0), k-contiguous fragments hold
    // whatever follows k = K - 1 in the row; they are masked to zero element
    // by element (a lane's fragment of step s holds k = 32kt + 16s + 8h ..
    // +7).  m/n-contiguous operands need no mask: their rows past K lie past
    // the copy descriptor's range and read as zeros.
    auto mask_k = [&](int kt, int s, u32x4 (&f)[TM]) {
        const int valid = p.K - (BK * kt + 16 * s + 8 * h);  // elements of the 8 still below K
        uint32_t m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m[e] = (2 * e < valid ? 0x0000ffffu : 0u) | (2 * e + 1 < valid ? 0xffff0000u : 0u);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[t][e] &= m[e];
    };
    auto slice = [&](auto Jc, int kt, auto maskc) {
        constexpr int J = decltype(Jc)::value;
        constexpr bool kEven = J % 2 == 0;
        constexpr bool kMask = decltype(maskc)::value;
        frags(Jc, 1, a1, b1);  // step 2 operands of this slice
        if constexpr (kMask) {
            if (kt == nk - 1 && p.K % BK != 0) {
                if constexpr (AK) { mask_k(kt, 0, a0); mask_k(kt, 1, a1); }
                if constexpr (BKc) { mask_k(kt, 0, b0); mask_k(kt, 1, b1); }
            }
        }
        if constexpr (!AK) opa.template copy<kEdge, kTail>(pick<(J + 3) % 4>(sA0, sA1, sA2, sA3), kt + 3, 1, wave);
        if constexpr (!BKc) opb.template copy<kEdge, kTail>(pick<(J + 3) % 4>(sB0, sB1, sB2, sB3), kt + 3, 1, wave);
        if constexpr (kEven && AK) opa.template copy<kEdge, kTail>(pick<(J / 2 + 1) % 2>(sA0, sA1, sA2, sA3), kt / 2 + 1, 1, wave);
        if constexpr (kEven && BKc) opb.template copy<kEdge, kTail>(pick<(J / 2 + 1) % 2>(sB0, sB1, sB2, sB3), kt / 2 + 1, 1, wave);
        mfma_step(a0, b0);  // step 1 (operands read earlier)
        DMA_WAIT_VMCNT_LGKM0((copies_after<AK, BKc, kEven>(CKC, CMN)));  // own copies landed, reads returned
        barrier();                                           // ... for every wave
        frags(std::integral_constant<int, (J + 1) % 4>{}, 0, a0, b0);  // next slice, step 1
        if constexpr (!AK) opa.template copy<kEdge, kTail>(pick<J>(sA0, sA1, sA2, sA3), kt + NSTAGE, 0, wave);
        if constexpr (!BKc) opb.template copy<kEdge, kTail>(pick<J>(sB0, sB1, sB2, sB3), kt + NSTAGE, 0, wave);
        if constexpr (!kEven && AK) opa.template copy<kEdge, kTail>(pick<((J + 3) / 2) % 2>(sA0, sA1, sA2, sA3), (kt + 3) / 2, 0, wave);
        if constexpr (!kEven && BKc) opb.template copy<kEdge, kTail>(pick<((J + 3) / 2) % 2>(sB0, sB1, sB2, sB3), (kt + 3) / 2, 0, wave);
        mfma_step(a1, b1);  // step 2
    };

    // Prologue: K-contiguous operands pair 0; MN-contiguous ones slices 0..2
    // and the first half of slice 3; then K-contiguous ones the first half of
    // pair 1.
    if constexpr (AK) { opa.template copy<kEdge, kTail>(sA0, 0, 0, wave); opa.template copy<kEdge, kTail>(sA0, 0, 1, wave); }
    if constexpr (BKc) { opb.template copy<kEdge, kTail>(sB0, 0, 0, wave); opb.template copy<kEdge, kTail>(sB0, 0, 1, wave); }
    if constexpr (!AK) { opa.template copy<kEdge, kTail>(sA0, 0, 0, wave); opa.template copy<kEdge, kTail>(sA0, 0, 1, wave); }
    if constexpr (!BKc) { opb.template copy<kEdge, kTail>(sB0, 0, 0, wave); opb.template copy<kEdge, kTail>(sB0, 0, 1, wave); }
    if constexpr (!AK) { opa.template copy<kEdge, kTail>(sA1, 1, 0, wave); opa.template copy<kEdge, kTail>(sA1, 1, 1, wave); }
    if constexpr (!BKc) { opb.template copy<kEdge, kTail>(sB1, 1, 0, wave); opb.template copy<kEdge, kTail>(sB1, 1, 1, wave); }
    if constexpr (!AK) { opa.template copy<kEdge, kTail>(sA2, 2, 0, wave); opa.template copy<kEdge, kTail>(sA2, 2, 1, wave); }
    if constexpr (!BKc) { opb.template copy<kEdge, kTail>(sB2, 2, 0, wave); opb.template copy<kEdge, kTail>(sB2, 2, 1, wave); }
    if constexpr (!AK) opa.template copy<kEdge, kTail>(sA3, 3, 0, wave);
    if constexpr (!BKc) opb.template copy<kEdge, kTail>(sB3, 3, 0, wave);
    if constexpr (AK) opa.template copy<kEdge, kTail>(sA1, 1, 0, wave);
    if constexpr (BKc) opb.template copy<kEdge, kTail>(sB1, 1, 0, wave);
    DMA_WAIT_VMCNT((prologue_after<AK, BKc>(CKC, CMN)));  // slice 0 of both operands landed
    barrier();
    frags(std::integral_constant<int, 0>{}, 0, a0, b0);
    using NoMask = std::false_type;
    int kt = 0;
    // with a K tail the last group (1 to 4 slices, the last possibly
    // partial) runs after the loop
    for (; kt + NSTAGE < nk + (kTail ? 0 : 1); kt += NSTAGE) {
        slice(std::integral_constant<int, 0>{}, kt, NoMask{});
        slice(std::integral_constant<int, 1>{}, kt + 1, NoMask{});
        slice(std::integral_constant<int, 2>{}, kt + 2, NoMask{});
        slice(std::integral_constant<int, 3>{}, kt + 3, NoMask{});
    }
    if constexpr (kTail) {
        const int rest = nk - kt;
        slice(std::integral_constant<int, 0>{}, kt, std::true_type{});
        if (rest >= 2) slice(std::integral_constant<int, 1>{}, kt + 1, std::true_type{});
        if (rest >= 3) slice(std::integral_constant<int, 2>{}, kt + 2, std::true_type{});
        if (rest >= 4) slice(std::integral_constant<int, 3>{}, kt + 3, std::true_type{});
    }
    DMA_WAIT_VMCNT(0);  // no copy may still target LDS when the workgroup ends

    // 32x32 accumulator layout: register r of lane l is row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the MFMA tile.  C is read
    // only when beta != 0, an MFMA tile at a time.  Every workgroup stores its
    // tile at about the same time, so the stores of a wave of tiles arrive
    // as one burst that the memory system drains at its write rate (about
    // 6% of the 8192^3 time); stores marked non-temporal drain ~2% sooner.  A lane's four bias values (one per column tile)
    // are read once; without a bias it adds -0.0, which leaves every value,
    // signed zeros included, unchanged.
    if (raw) {
        // stream-K partial: every element of the R x R tile, no epilogue
        float* rbase = raw + (int64_t)(wm * (R / 2) + 4 * h) * R + wn * (R / 2) + (lane & 31);
#pragma unroll
        for (int ti = 0; ti < TM; ++ti)
#pragma unroll
            for (int tj = 0; tj < TM; ++tj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    rbase[(ti * 32 + 8 * (r >> 2) + (r & 3)) * R + tj * 32] = acc[ti][tj][r];
        return;
    }
    const int col0 = n0 + wn * (R / 2) + (lane & 31);
    float* cbase = p.C + (int64_t)(m0 + wm * (R / 2) + 4 * h) * p.ldc + col0;
    const float alpha = p.alpha, beta = p.beta;
    float bias[TM];
#pragma unroll
    for (int tj = 0; tj < TM; ++tj)
        bias[tj] = p.bias && (!kEdge || col0 + tj * 32 < p.N) ? p.bias[col0 + tj * 32] : -0.0f;
    // on edge tiles only rows < M and columns < N are stored
    const int row0 = m0 + wm * (R / 2) + 4 * h;
    auto ok = [&](int ti, int tj, int r) {
        return !kEdge || (row0 + ti * 32 + 8 * (r >> 2) + (r & 3) < p.M && col0 + tj * 32 < p.N);
    };
    if (beta == 0.0f) {
#pragma unroll
        for (int ti = 0; ti < TM; ++ti)
#pragma unroll
            for (int tj = 0; tj < TM; ++tj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (ok(ti, tj, r))
                        __builtin_nontemporal_store(
                            alpha * acc[ti][tj][r] + bias[tj],
                            &cbase[(int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32]);
    } else {
        // C is read one 32 x 32 MFMA tile (16 values a lane) at a time
        // before those values are stored, so the reads of a tile overlap.
#pragma unroll
        for (int ti = 0; ti < TM; ++ti)
#pragma unroll
            for (int tj = 0; tj < TM; ++tj) {
                float cv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    cv[r] = ok(ti, tj, r)
                                ? cbase[(int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32]
                                : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (ok(ti, tj, r))
                        __builtin_nontemporal_store(
                            (alpha * acc[ti][tj][r] + beta * cv[r]) + bias[tj],
                            &cbase[(int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32]);
            }
    }
}

template <In T, int R, bool TA, bool TB, bool kEdge, bool kTail>
__global__ __launch_bounds__(NT, R == 256 ? 1 : 2) void mfma16_dma_kernel(GemmParams p,
                                                                        int tiles_m,
                                                                        int tiles_n,
                                                                        int grouped) {
    const TileIdx tile = xcd_tile(tiles_m, tiles_n, grouped != 0);
    select_problem(p, tile.z);
    dma_tile<T, R, TA, TB, kEdge, kTail>(p, tile.bm * R, tile.bn * R, nullptr);
}


// ------------------------------------------------------------- stream-K
// (the schedule and the fix-up kernel: streamk.hpp)

constexpr int kSkIterK = streamk::kIterK16;
static_assert(kSkIterK == BK * NSTAGE, "a stream-K iteration is one group of four slices");

template <In T, bool TA, bool TB, bool kRagged>
__global__ __launch_bounds__(NT, 1) void mfma16_streamk_kernel(GemmParams p, streamk::StreamK sk,
                                                               float* ws) {
    streamk::walk<TA, TB, 2>(p, sk, ws, [&](const GemmParams& q, int m0, int n0, float* raw) {
        dma_tile<T, streamk::R, TA, TB, kRagged, kRagged>(q, m0, n0, raw);
    });
}

}  // namespace

int64_t streamk_workspace_bytes(const GemmParams& p, bool f32) {
    return streamk::workspace_bytes(p, f32 ? streamk::kIterKF32 : streamk::kIterK16);
}

template <In T>
hipError_t launch_mfma16_streamk(const GemmParams& p, float* ws, hipStream_t s) {
    if (p.batch != 1 || p.k_last > 0 || !mfma16_dma_eligible(p)) return hipErrorInvalidConfiguration;
    const streamk::StreamK sk = streamk::plan(p, kSkIterK);
    if (sk.T > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool ragged = p.M % 256 != 0 || p.N % 256 != 0 || p.K % kSkIterK != 0;
    hipError_t e = with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (ragged)
            hipLaunchKernelGGL((mfma16_streamk_kernel<T, TA, TB, true>), dim3(sk.G), dim3(NT), 0,
                               s, p, sk, ws);
        else
            hipLaunchKernelGGL((mfma16_streamk_kernel<T, TA, TB, false>), dim3(sk.G), dim3(NT), 0,
                               s, p, sk, ws);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    return streamk::launch_fixup(p, sk, ws, s);
}
template hipError_t launch_mfma16_streamk<In::BF16>(const GemmParams&, float*, hipStream_t);
template hipError_t launch_mfma16_streamk<In::F16>(const GemmParams&, float*, hipStream_t);

// Any M, N and K (edge tiles and a K tail are clipped or masked), 16-byte
// aligned rows, and pitches within the 32-bit buffer offsets.
bool mfma16_dma_eligible(const GemmParams& p) {
    return operands_16b_aligned(p, 2) && p.M > 0 && p.N > 0 && p.K > 0 &&
           p.lda < kMaxBufferPitch && p.ldb < kMaxBufferPitch;
}

namespace {

template <In T, int R>
hipError_t launch_tiles(const GemmParams& p, hipStream_t s) {
    const int tiles_m = (p.M + R - 1) / R, tiles_n = (p.N + R - 1) / R;
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool edge = p.M % R != 0 || p.N % R != 0;
    const bool tail = !k_multiple(p, BK * NSTAGE);
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        // linear order only for one problem with both operands k-contiguous
        const int grouped = !(p.batch == 1 && !TA && TB);
        const dim3 grid((unsigned)blocks, p.batch);
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(NT), 0, s, p, tiles_m, tiles_n, grouped);
        };
        // a K tail takes the edge-tile instance whatever M and N (its guards
        // then always pass); built without edges it spills registers
        if (tail) go(mfma16_dma_kernel<T, R, TA, TB, true, true>);
        else if (edge) go(mfma16_dma_kernel<T, R, TA, TB, true, false>);
        else go(mfma16_dma_kernel<T, R, TA, TB, false, false>);
        return hipGetLastError();
    });
}

}  // namespace

template <In T>
hipError_t launch_mfma16_dma_tile(const GemmParams& p, hipStream_t s, int tile) {
    return tile == 128 ? launch_tiles<T, 128>(p, s) : launch_tiles<T, 256>(p, s);
}

// Tile size by the waves of tiles the CUs work through.  A CU runs one
// 256-tile, or two 128-tiles side by side (alone, a 128-tile leaves the CU
// about as slow as a pair does), and a 128-tile costs kCost128 quarters of a
// 256-tile's time (measured at 8192^3: 0.932 against 0.766 ms).  In units
// of a quarter 256-tile: 4 per wave of 256 tiles against 2 * kCost128 per
// wave of 512.  Ties keep the larger tile.
template <In T>
hipError_t launch_mfma16_dma(const GemmParams& p, hipStream_t s) {
    const int64_t t256 = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
    const int64_t t128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
    const double time256 = (double)((t256 + kCUs - 1) / kCUs) * 4.0;
    const double time128 = (double)((t128 + 2 * kCUs - 1) / (2 * kCUs)) * 2.0 * kCost128;
    return time128 < time256 ? launch_tiles<T, 128>(p, s) : launch_tiles<T, 256>(p, s);
}
template hipError_t launch_mfma16_dma<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_mfma16_dma<In::F16>(const GemmParams&, hipStream_t);
template hipError_t launch_mfma16_dma_tile<In::BF16>(const GemmParams&, hipStream_t, int);
template hipError_t launch_mfma16_dma_tile<In::F16>(const GemmParams&, hipStream_t, int);

}  // namespace dgt
