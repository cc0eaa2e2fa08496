// k_mfma_f32_dma.hip -- FP32 GEMM: global -> LDS by DMA up to three K
// slices ahead, a wavefront's tile of C held in accumulation registers.
//
// The pages' register-tiled SGEMM (dilfish.github.io 5.4: block tile, a
// per-thread register tile, double buffering) becomes, on the matrix cores,
// an R/2 x R/2 tile of C per wavefront (R/64 x R/64 v_mfma_f32_32x32x2_f32
// tiles) and a 2 x 2 grid of wavefronts per R x R workgroup tile.  It is
// the 16-bit DMA kernel's structure with fp32 elements: at R = 256 the byte
// geometry of its LDS stages is the same, so are its copy counts per slice,
// waits and barrier placement.
//
//  * K advances in slices of 16.  Copies use buffer_load_dwordx4 ... lds:
//    lane l's 16 bytes land at LDS base + 16*l; a swizzle is applied by the
//    choice of which global chunk each lane fetches.  Each wave addresses its
//    rows through a buffer descriptor (wave-uniform base, 32-bit lane
//    offsets).
//  * K-contiguous operand (A as M x K, B transposed as N x K): two LDS stages
//    of two slices each, R rows of 128 B (32 floats; chunk q of row r at
//    q ^ ((r ^ r>>3) & 7)).  A lane reads its 4 k of a half slice with one
//    16-byte LDS read.
//  * MN-contiguous operand (B as K x N, A transposed as K x M): four stages
//    of one slice, 16 k-rows of 4R bytes; chunk c of k-row k at
//    c ^ 8((k>>3)&1), so the two half-wavefronts, which read k-rows 8 apart,
//    use opposite halves of the LDS banks.  A lane reads one float per k (no
//    transposing LDS read exists for 32-bit data).
//  * The 32x32x2 instruction sums over two k, one per half-wavefront: half
//    h feeds k = 8h + 4s + j at sub-step j of half slice s, so a lane's 4 k of
//    a k-contiguous operand are adjacent; every product still lands in the
//    same sum.
//  * Per slice each wavefront issues 8 (R/64)^2 MFMAs in two half slices;
//    the LDS reads of the next half slice and the copies are spread between
//    them.  The workgroup barrier sits between the two halves: it publishes
//    slice t+1 and retires slice t's stage.
//
// Tiles of 256 x 256 (one workgroup per CU) or 128 x 128 (two per CU, each
// wave 64 x 64), chosen per launch by the waves of tiles the CUs work
// through.  Used for any M, N and K with 16-byte aligned rows and row
// pitches below 2^23 elements (so a wave's rows of lane offsets fit 32
// bits); the register-staged 128 x 128 kernel takes unaligned operands.
// On edge tiles the copy descriptors' ranges stop at the operands' last
// elements and the epilogue stores only the valid part.  When K is not a multiple of 64 the
// last group of 1 to 4 slices runs after the loop; in a partial last slice
// the k-contiguous fragments are masked past K, and m/n-contiguous rows past
// K read as zeros through the descriptor range.
#include "dma_common.hpp"
#include "streamk.hpp"

namespace dgt {

namespace {

using namespace dma;

constexpr int BK = 16, NT = 256, NSTAGE = 4;

// Geometry of a workgroup tile of R x R (R = 256 or 128; a 2 x 2 grid of
// wavefronts of R/2 x R/2).  A k-contiguous stage holds R rows of 128 B (two
// slices), copied 8 rows per instruction; an m/n-contiguous stage holds 16
// k-rows of 4R bytes, 256/R k-rows per instruction; each wave copies a
// quarter of either.
template <int R>
struct Geo {
    static constexpr int TM = R / 64;         // 32 x 32 MFMA tiles per wave and dimension
    static constexpr int KC_ROWS = R / 4;     // k-contiguous rows per wave
    static constexpr int KC_INSTR = R / 32;   // their copy instructions per pair
    static constexpr int KC_STAGE = R * 128;  // bytes
    static constexpr int MN_ROW = 4 * R;      // bytes per k-row
    static constexpr int MN_LPR = R / 4;      // 16-byte chunks (lanes) per k-row
    static constexpr int MN_INSTR = R / 64;   // copy instructions per slice and wave
    static constexpr int MN_STAGE = BK * MN_ROW;
};
constexpr int64_t kMaxPitchF32 = int64_t(1) << 23;

// m/n-contiguous k-rows: chunk c of k-row k sits at c ^ swz_mn(k), so the
// two half-wavefronts, which read k-rows 8 apart, use opposite halves of
// the LDS banks.
__device__ __forceinline__ int swz_mn(int k) { return ((k >> 3) & 1) * 8; }

// A K-contiguous operand: stage = a pair of slices, R rows x 128 B.  Wave w
// issues copy instructions j = (R/32)w + i per pair, instruction j filling
// rows 8j .. 8j+7 (8 lanes per row), as two halves.  The wave's descriptor
// covers its R/4 rows; pair pr adds 128*pr bytes through the scalar offset.
template <int R>
struct KcOperand {
    using G = Geo<R>;
    const float* base;             // row (R/4)*wave of the tile (wave-uniform)
    uint32_t voff[G::KC_INSTR];    // lane byte offsets from base, per instruction
    uint32_t bytes;                // descriptor range: the wave's rows
    int off[G::TM][2][2];          // LDS read offset: tile t, slice-in-pair u, half slice s
    int npair;

    // mn0: first row (m or n) of the workgroup tile; w: this wave's half of
    // it (wm or wn); mn_lim: rows of the operand (M or N), K its row length.
    // The descriptor range ends at the wave's last element (k = K - 1 of its
    // last row, or of row mn_lim - 1 on an edge tile), so rows past mn_lim
    // and the k past K of a final half pair are never read from memory.
    template <bool kEdge>
    __device__ void init(const float* X, int64_t ld, int mn0, int w, int wave, int lane, int nk,
                         int mn_lim, int K) {
#pragma unroll
        for (int i = 0; i < G::KC_INSTR; ++i) {
            const int row = 8 * (G::KC_INSTR * wave + i) + (lane >> 3);
            const int q = (lane & 7) ^ swz_kc(row);
            voff[i] = (uint32_t)(((int64_t)(row - G::KC_ROWS * wave) * ld + 4 * q) * 4);
        }
        base = X + (int64_t)(mn0 + G::KC_ROWS * wave) * ld;
        int rows = G::KC_ROWS;
        if constexpr (kEdge) rows = min(G::KC_ROWS, mn_lim - (mn0 + G::KC_ROWS * wave));
        bytes = rows <= 0 ? 0u : (uint32_t)(((int64_t)(rows - 1) * ld + round_chunk<4>(K)) * 4);
        // rows w*R/2 + t*32 + l%32; half-wave h, half slice s read chunk 4u + 2h + s
        const int h = lane >> 5;
#pragma unroll
        for (int t = 0; t < G::TM; ++t) {
            const int row = w * (R / 2) + t * 32 + (lane & 31);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    off[t][u][s] = row * 128 + (((4 * u + 2 * h + s) ^ swz_kc(row)) << 4);
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
        uint32_t range = bytes, soff = (uint32_t)pr * 128;
        if constexpr (kTail) {
            pr = __builtin_amdgcn_readfirstlane(pr);
            const uint32_t skip = (uint32_t)pr * 128;
            range = __builtin_amdgcn_readfirstlane(bytes > skip ? bytes - skip : 0u);
            from += skip;
            soff = 0;
        }
        constexpr int HALF = G::KC_INSTR / 2;
#pragma unroll
        for (int i = HALF * half; i < HALF * half + HALF; ++i)
            dma16(from, range, st + (G::KC_INSTR * wave + i) * 1024, voff[i], soff);
    }
    // Operands of half slice s of the slice in half u of stage st: f[t][j] is
    // k = 8h + 4s + j of row w*R/2 + t*32 + l%32.
    __device__ void frags(const uint8_t* st, int u, int s, u32x4 (&f)[G::TM]) const {
#pragma unroll
        for (int t = 0; t < G::TM; ++t) f[t] = *reinterpret_cast<const u32x4*>(st + off[t][u][s]);
    }
    static constexpr int kReads = G::TM;        // LDS reads per half slice
    static constexpr int kHalfCopies = G::KC_INSTR / 2;
    static constexpr int kStage = G::KC_STAGE;
};

// An MN-contiguous operand: stage = one slice, 16 k-rows x 4R bytes.  Wave w
// copies k-rows 4w .. 4w+3 with R/64 instructions (256/R k-rows each, R/4
// lanes per k-row), as two halves.
template <int R>
struct MnOperand {
    using G = Geo<R>;
    const float* base;           // k-row 4*wave of slice 0, first column of the tile
    uint32_t voff[G::MN_INSTR];  // lane byte offsets from base, per instruction
    uint32_t bytes;              // descriptor range: 4 k-rows
    int off[G::TM];
    int64_t slice;
    int nk;
    int64_t ld_;
    int rows_left0;     // k-rows from this wave's first one to the end
    int cols;           // valid columns of the tile, rounded to a chunk (edge tiles)

    // mn_lim, K: columns and rows of the stored operand.  On an edge tile the
    // range of slice kt's descriptor stops at the operand's last element;
    // columns past mn_lim in earlier rows are read (they belong to the next
    // row) but only feed outputs the epilogue does not store, and k-rows
    // past K read as zeros.
    template <bool kEdge>
    __device__ void init(const float* X, int64_t ld, int mn0, int w, int wave, int lane, int nk_,
                         int mn_lim, int K) {
#pragma unroll
        for (int i = 0; i < G::MN_INSTR; ++i) {
            const int krow = 4 * wave + (256 / R) * i + lane / G::MN_LPR;
            const int c = (lane % G::MN_LPR) ^ swz_mn(krow);
            voff[i] = (uint32_t)(((int64_t)(krow - 4 * wave) * ld + 4 * c) * 4);
        }
        base = X + (int64_t)(4 * wave) * ld + mn0;
        bytes = (uint32_t)(4 * ld * 4);
        // lane (h, l%32) reads k-rows 8h + 4s + j, column w*R/2 + t*32 + l%32
        const int h = lane >> 5, r = lane & 31;
#pragma unroll
        for (int t = 0; t < G::TM; ++t) {
            const int chunk = (w * (R / 8) + t * 8 + (r >> 2)) ^ (8 * h);
            off[t] = 8 * h * G::MN_ROW + chunk * 16 + (r & 3) * 4;
        }
        slice = (int64_t)BK * ld;
        nk = nk_;
        ld_ = ld;
        rows_left0 = K - 4 * wave;
        cols = kEdge ? round_chunk<4>(mn_lim - mn0) : 0;
    }
    // Half `half` of slice kt into stage st (past the end: the last slice).
    template <bool kEdge = false, bool kTail = false>
    __device__ void copy(uint8_t* st, int kt, int half, int wave) const {
        kt = kt < nk ? kt : nk - 1;
        uint32_t range = bytes;
        if constexpr (kEdge) {
            const int64_t end = (int64_t)(rows_left0 - BK * kt - 1) * ld_ + cols;  // elements
            if (end < 4 * ld_) range = end <= 0 ? 0u : (uint32_t)(end * 4);
        }
        constexpr int HALF = G::MN_INSTR / 2;
#pragma unroll
        for (int i = HALF * half; i < HALF * half + HALF; ++i)
            dma16(base + kt * slice, range, st + (G::MN_INSTR * wave + i) * 1024, voff[i], 0);
    }
    __device__ void frags(const uint8_t* st, int s, u32x4 (&f)[G::TM]) const {
#pragma unroll
        for (int t = 0; t < G::TM; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f[t][j] = *reinterpret_cast<const uint32_t*>(st + off[t] + (4 * s + j) * G::MN_ROW);
    }
    static constexpr int kReads = 4 * G::TM;
    static constexpr int kHalfCopies = G::MN_INSTR / 2;
    static constexpr int kStage = G::MN_STAGE;
};


// TA / TB: A / B stored transposed.  A is K-contiguous unless TA, B is
// K-contiguous when TB.
// kEdge: M or N not a multiple of the tile (edge tiles read through
// clipped descriptor ranges and store only their valid part).  kTail: K is
// not a multiple of 64 (a last group of 1 to 4 slices after the loop, the
// last slice possibly partial).
// R: workgroup tile R x R (256: one workgroup per CU; 128: two).
// One R x R output tile at (m0, n0) over k = 0 .. p.K-1 of p's operands:
// the body of mfma_f32_dma_kernel, shared with the stream-K kernel.  raw ==
// nullptr: the BLAS epilogue into p.C; otherwise the bare fp32 sums go to
// raw (R x R, row pitch R, every element written; a stream-K partial tile).
template <int R, bool TA, bool TB, bool kEdge, bool kTail>
__device__ __forceinline__ void f32_tile(const GemmParams& p, int m0, int n0, float* raw) {
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
    const int nk = (p.K + BK - 1) / BK;  // slices (the last one partial when K % 16 != 0)

    OpA opa;
    OpB opb;
    opa.template init<kEdge>(static_cast<const float*>(p.A), p.lda, m0, wm, wave, lane, nk, p.M,
                             p.K);
    opb.template init<kEdge>(static_cast<const float*>(p.B), p.ldb, n0, wn, wave, lane, nk, p.N,
                             p.K);

    floatx16 acc[TM][TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Operands of half slice s of slice position J (0..3 within a group of
    // four slices: a K-contiguous operand has it in stage J/2, half J%2; an
    // MN-contiguous one in stage J).
    auto frags = [&](auto Jc, int s, u32x4 (&a)[TM], u32x4 (&b)[TM]) {
        constexpr int J = decltype(Jc)::value;
        if constexpr (AK) opa.frags(pick<J / 2>(sA0, sA1, sA2, sA3), J % 2, s, a);
        else opa.frags(pick<J>(sA0, sA1, sA2, sA3), s, a);
        if constexpr (BKc) opb.frags(pick<J / 2>(sB0, sB1, sB2, sB3), J % 2, s, b);
        else opb.frags(pick<J>(sB0, sB1, sB2, sB3), s, b);
    };

    // 4 TM^2 MFMAs on (a, b): four sub-steps of TM x TM tiles.  The LDS reads
    // and the copies issued just before in program order are spread between
    // them (both evenly, up to 8 copy slots), so the address unit never sees
    // a burst that would hold the wave, and its MFMA issue, back.
    constexpr int NMFMA = 4 * TM * TM;
    constexpr int RD_EVERY = NMFMA / (OpA::kReads + OpB::kReads) > 0
                                 ? NMFMA / (OpA::kReads + OpB::kReads) : 1;
    constexpr int CP_EVERY = NMFMA / 8;
    auto mfma_step = [&](const u32x4 (&a)[TM], const u32x4 (&b)[TM]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int ti = 0; ti < TM; ++ti)
#pragma unroll
                for (int tj = 0; tj < TM; ++tj)
                    acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        __uint_as_float(a[ti][j]), __uint_as_float(b[tj][j]), acc[ti][tj], 0, 0,
                        0);
#pragma unroll
        for (int m = 0; m < NMFMA; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
            if (m % RD_EVERY == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            if (m % CP_EVERY == 1 % CP_EVERY) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // copy
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
    // In a partial last slice (K % 16 != 0), k-contiguous fragments hold
    // whatever follows k = K - 1 in the row; they are masked to zero element
    // by element (a lane's fragment of half slice s holds k = 16kt + 8h + 4s
    // .. +3).  m/n-contiguous operands need no mask: their rows past K lie
    // past the copy descriptor's range and read as zeros.
    auto mask_k = [&](int kt, int s, u32x4 (&f)[TM]) {
        const int valid = p.K - (BK * kt + 8 * h + 4 * s);  // of the 4 still below K
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) f[t][j] = j < valid ? f[t][j] : 0u;
    };
    auto slice = [&](auto Jc, int kt, auto maskc) {
        constexpr int J = decltype(Jc)::value;
        constexpr bool kEven = J % 2 == 0;
        constexpr bool kMask = decltype(maskc)::value;
        frags(Jc, 1, a1, b1);  // second half-slice operands of this slice
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
        mfma_step(a0, b0);  // first half slice (operands read earlier)
        DMA_WAIT_VMCNT_LGKM0((copies_after<AK, BKc, kEven>(CKC, CMN)));  // own copies landed, reads returned
        barrier();                                           // ... for every wave
        frags(std::integral_constant<int, (J + 1) % 4>{}, 0, a0, b0);  // next slice, first half
        if constexpr (!AK) opa.template copy<kEdge, kTail>(pick<J>(sA0, sA1, sA2, sA3), kt + NSTAGE, 0, wave);
        if constexpr (!BKc) opb.template copy<kEdge, kTail>(pick<J>(sB0, sB1, sB2, sB3), kt + NSTAGE, 0, wave);
        if constexpr (!kEven && AK) opa.template copy<kEdge, kTail>(pick<((J + 3) / 2) % 2>(sA0, sA1, sA2, sA3), (kt + 3) / 2, 0, wave);
        if constexpr (!kEven && BKc) opb.template copy<kEdge, kTail>(pick<((J + 3) / 2) % 2>(sB0, sB1, sB2, sB3), (kt + 3) / 2, 0, wave);
        mfma_step(a1, b1);  // second half slice
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
    // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the MFMA tile.  C is read only
    // when beta != 0, an MFMA tile at a time, before those values are
    // stored.  Without a bias the epilogue adds -0.0, which leaves every
    // value, signed zeros included, unchanged.  The lane index is counted
    // afresh here rather than kept live through the K loop.
    const int el = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int eh = el >> 5;
    if (raw) {
        // stream-K partial: every element of the R x R tile, no epilogue
        float* rbase = raw + (int64_t)(wm * (R / 2) + 4 * eh) * R + wn * (R / 2) + (el & 31);
#pragma unroll
        for (int ti = 0; ti < TM; ++ti)
#pragma unroll
            for (int tj = 0; tj < TM; ++tj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    rbase[(ti * 32 + 8 * (r >> 2) + (r & 3)) * R + tj * 32] = acc[ti][tj][r];
        return;
    }
    const int col0 = n0 + wn * (R / 2) + (el & 31);
    float* cbase = p.C + (int64_t)(m0 + wm * (R / 2) + 4 * eh) * p.ldc + col0;
    const float alpha = p.alpha, beta = p.beta;
    float bias[TM];
#pragma unroll
    for (int tj = 0; tj < TM; ++tj)
        bias[tj] = p.bias && (!kEdge || col0 + tj * 32 < p.N) ? p.bias[col0 + tj * 32] : -0.0f;
    // on edge tiles only rows < M and columns < N are stored
    const int row0 = m0 + wm * (R / 2) + 4 * eh;
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
                        cbase[(int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32] =
                            alpha * acc[ti][tj][r] + bias[tj];
    } else {
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
                        cbase[(int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32] =
                            (alpha * acc[ti][tj][r] + beta * cv[r]) + bias[tj];
            }
    }
}

template <int R, bool TA, bool TB, bool kEdge, bool kTail>
__global__ __launch_bounds__(NT, R == 256 ? 1 : 2) void mfma_f32_dma_kernel(GemmParams p,
                                                                          int tiles_m,
                                                                          int tiles_n,
                                                                          int grouped) {
    const TileIdx tile = xcd_tile(tiles_m, tiles_n, grouped != 0);
    select_problem(p, tile.z);
    f32_tile<R, TA, TB, kEdge, kTail>(p, tile.bm * R, tile.bn * R, nullptr);
}

// Stream-K (streamk.hpp) on 256 x 256 tiles; an iteration is a group of
// four 16-deep slices.
static_assert(streamk::kIterKF32 == BK * NSTAGE, "a stream-K iteration is one group of four slices");

template <bool TA, bool TB, bool kRagged>
__global__ __launch_bounds__(NT, 1) void mfma_f32_streamk_kernel(GemmParams p, streamk::StreamK sk,
                                                                 float* ws) {
    streamk::walk<TA, TB, 4>(p, sk, ws, [&](const GemmParams& q, int m0, int n0, float* raw) {
        f32_tile<streamk::R, TA, TB, kRagged, kRagged>(q, m0, n0, raw);
    });
}

}  // namespace

hipError_t launch_mfma_f32_streamk(const GemmParams& p, float* ws, hipStream_t s) {
    if (p.batch != 1 || p.k_last > 0 || !mfma_f32_dma_eligible(p))
        return hipErrorInvalidConfiguration;
    const streamk::StreamK sk = streamk::plan(p, streamk::kIterKF32);
    if (sk.T > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool ragged = p.M % 256 != 0 || p.N % 256 != 0 || p.K % streamk::kIterKF32 != 0;
    hipError_t e = with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (ragged)
            hipLaunchKernelGGL((mfma_f32_streamk_kernel<TA, TB, true>), dim3(sk.G), dim3(NT), 0, s,
                               p, sk, ws);
        else
            hipLaunchKernelGGL((mfma_f32_streamk_kernel<TA, TB, false>), dim3(sk.G), dim3(NT), 0, s,
                               p, sk, ws);
        return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    return streamk::launch_fixup(p, sk, ws, s);
}

// Aligned rows and pitches within the buffer offsets: every other shape
// takes the register-staged 128 x 128 kernel.
bool mfma_f32_dma_eligible(const GemmParams& p) {
    if (!operands_16b_aligned(p, 4) || p.M <= 0 || p.N <= 0 || p.K <= 0) return false;
    return p.lda < kMaxPitchF32 && p.ldb < kMaxPitchF32;
}

namespace {

template <int R>
hipError_t launch_tiles(const GemmParams& p, hipStream_t s) {
    const int tiles_m = (p.M + R - 1) / R, tiles_n = (p.N + R - 1) / R;
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool edge = p.M % R != 0 || p.N % R != 0;
    const bool tail = !k_multiple(p, BK * NSTAGE);
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        const dim3 grid((unsigned)blocks, p.batch);
        auto go = [&](auto kernel) {
            hipLaunchKernelGGL(kernel, grid, dim3(NT), 0, s, p, tiles_m, tiles_n, 1);
        };
        // a K tail takes the edge-tile instance whatever M and N (its guards
        // then always pass)
        if (tail) go(mfma_f32_dma_kernel<R, TA, TB, true, true>);
        else if (edge) go(mfma_f32_dma_kernel<R, TA, TB, true, false>);
        else go(mfma_f32_dma_kernel<R, TA, TB, false, false>);
        return hipGetLastError();
    });
}

}  // namespace

hipError_t launch_mfma_f32_dma_tile(const GemmParams& p, hipStream_t s, int tile) {
    return tile == 128 ? launch_tiles<128>(p, s) : launch_tiles<256>(p, s);
}

// Tile size by the waves of tiles the CUs work through: both sizes reach
// ~0.96 of the MFMA peak (a CU runs one 256-tile or two 128-tiles at a
// time), so a CU's time is its share of tiles rounded up, counted in
// 128-tiles (a 256-tile is four).  Ties keep the larger tile.
hipError_t launch_mfma_f32_dma(const GemmParams& p, hipStream_t s) {
    const int64_t t256 = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
    const int64_t t128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
    const int64_t time256 = (t256 + kCUs - 1) / kCUs * 4;
    const int64_t time128 = (t128 + kCUs - 1) / kCUs;
    return time128 < time256 ? launch_tiles<128>(p, s) : launch_tiles<256>(p, s);
}

}  // namespace dgt
