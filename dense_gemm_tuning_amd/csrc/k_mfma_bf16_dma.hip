// k_mfma_bf16_dma.hip -- 16-bit-input (BF16 or FP16) / FP32-accumulate GEMM
// for whole tiles:
// global -> LDS by DMA three K slices ahead, B transposed by the LDS read.
//
// Tiling as in the register-staged kernel (256 x 256 workgroup tile, 2 x 2
// wavefronts of 128 x 128, v_mfma_f32_32x32x16_bf16: dilfish.github.io
// 5.3-5.5, qwbw.cn Level 2), with a deeper software pipeline than the pages'
// double buffer (dilfish.github.io 5.4; qwbw.cn's double-buffering row):
//
//  * K advances in slices of 32.  Each slice of A (256 x 32) and B (32 x 256)
//    is copied by global_load_lds_dwordx4: lane l's 16 bytes land at LDS base
//    + 16*l, so one instruction fills 1 KiB and no operand byte passes through
//    a VGPR.  Four LDS stages (4 x 32 KiB) hold slices t .. t+3; the copy of
//    slice t+4 starts as soon as stage t%4 has been read, about 2.5 slices
//    (2500 MFMA cycles) before it is needed, which covers L2-miss latency to
//    the memory side.  Each wave's 8 copy instructions per slice are spread
//    one per 4 MFMAs; issued in a burst they queue at the address unit and
//    hold back the wave's MFMA issue.  Copies past the last slice re-read the
//    last slice (never consumed) so every step waits on the same count.
//  * A rows (32 bf16 = 4 chunks of 16 B): chunk q of row r sits at
//    q ^ ((r >> 2) & 3); the DMA writes lanes in order, so the swizzle is
//    applied by the choice of which global chunk each lane fetches.
//  * B stays row-major in LDS (k rows of 256 bf16 = 32 chunks; chunk c of row
//    k at c ^ (4*(k & 3))).  ds_read_b64_tr_b16 transposes on the read:
//    within each 16-lane group, source lane 4r+q names row r, columns
//    4q..4q+3, and destination lane j receives column j, rows 0..3; two reads
//    give a lane its 8 consecutive k (the pages warn that an operand in the
//    wrong major order still "looks right": dilfish.github.io 5.5).
//  * Per slice each wavefront issues 32 MFMAs in two 16-deep steps; the LDS
//    reads of the next step are interleaved one per MFMA.  The workgroup
//    barrier sits between the two steps: it publishes slice t+1 (every wave
//    has waited for its own copies) and retires slice t's stage, so the
//    first operands of slice t+1 are read while step 2 of slice t computes.
//
// Used for shapes that are whole tiles (M, N multiples of 256, K of 128) with
// 16-byte aligned rows; the register-staged kernel handles everything else.
#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int BM = 256, BN = 256, BK = 32, NT = 256, NSTAGE = 4;
constexpr int A_STAGE = BM * 2 * BK * 2;  // 32 KiB: 256 rows x 128 B (two slices)
constexpr int B_STAGE = BK * BN * 2;      // 16 KiB: 32 rows x 512 B (one slice)
constexpr int KALIGN = BK * NSTAGE;       // K multiple handled here
constexpr int CPOL = 1;                   // sc0 on the copies

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// A rows are 128 B = 8 chunks of 16 B; chunk q of row r sits at q ^ swz_a(r).
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt in 6:4,
// lgkmcnt in 11:8); WAIT_VMCNT_LGKM0 also drains this wave's LDS reads.
#define WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)
#define WAIT_VMCNT_LGKM0(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0070)

// Workgroup barrier without a memory fence: LDS data written by copies is
// published by each wave waiting for its own copies first.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <In T>
__global__ __launch_bounds__(NT, 1) void mfma16_dma_kernel(GemmParams p, int tiles_n) {
    // One LDS object per operand and stage, so that the compiler sees that a
    // copy in flight into one stage does not alias reads of another.  A has
    // two stages of two slices each, B four stages of one slice.
    __shared__ __attribute__((aligned(1024))) uint8_t sA0[A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sA1[A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sB0[B_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sB1[B_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sB2[B_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t sB3[B_STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;
    const int m0 = (blockIdx.x / tiles_n) * BM;
    const int n0 = (blockIdx.x % tiles_n) * BN;
    const uint16_t* A = static_cast<const uint16_t*>(p.A);
    const uint16_t* B = static_cast<const uint16_t*>(p.B);
    const int nk = p.K / BK;      // slices
    const int npair = nk / 2;     // slice pairs

    // Copy sources.  A: wave w issues instructions j = 8w + i (i = 0..7) per
    // pair, instruction j filling rows 8j .. 8j+7 with 128 B each (8 lanes per
    // row).  B: wave w issues j = 4w + i (i = 0..3) per slice, instruction j
    // filling k-rows 2j and 2j+1 (32 lanes per row).
    const uint16_t* asrc[8];
    const uint16_t* bsrc[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int arow = 8 * (8 * wave + i) + (lane >> 3);
        const int aq = (lane & 7) ^ swz_a(arow);
        asrc[i] = A + (int64_t)(m0 + arow) * p.lda + 8 * aq;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int brow = 2 * (4 * wave + i) + (lane >> 5);
        const int bc = (lane & 31) ^ (4 * (brow & 3));
        bsrc[i] = B + (int64_t)brow * p.ldb + n0 + 8 * bc;
    }
    const int64_t b_slice = (int64_t)BK * p.ldb;

    // Half `half` (instructions 4*half .. 4*half+3) of A pair `pr` into sa.
    auto copy_a = [&](uint8_t* sa, int pr, int half) {
        pr = pr < npair ? pr : npair - 1;  // past the end: re-read the last pair
#pragma unroll
        for (int i = 4 * half; i < 4 * half + 4; ++i)
            __builtin_amdgcn_global_load_lds(asrc[i] + (int64_t)pr * (2 * BK),
                                             (lds_void*)(sa + (8 * wave + i) * 1024), 16, 0,
                                             CPOL);
    };
    // Half `half` (instructions 2*half, 2*half+1) of B slice kt into sb.
    auto copy_b = [&](uint8_t* sb, int kt, int half) {
        kt = kt < nk ? kt : nk - 1;        // past the end: re-read the last slice
#pragma unroll
        for (int i = 2 * half; i < 2 * half + 2; ++i)
            __builtin_amdgcn_global_load_lds(bsrc[i] + kt * b_slice,
                                             (lds_void*)(sb + (4 * wave + i) * 1024), 16, 0,
                                             CPOL);
    };

    // LDS read offsets.  A: row wm*128 + ti*32 + l%32; slice-in-pair u, step s,
    // half-wave h -> chunk 4u + 2s + h.
    int a_off[4][2][2];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
        const int row = wm * 128 + ti * 32 + (lane & 31);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                a_off[ti][u][s] = row * 128 + (((4 * u + 2 * s + h) ^ swz_a(row)) << 4);
    }
    // B: source lane 4r+q of 16-lane group G reads k-row 16s + 8h + 4t + r,
    // columns wn*128 + tj*32 + 16*(G%2) + 4q .. +3; k & 3 == r.
    int b_off[4];
    {
        const int r = (lane & 15) >> 2, q = lane & 3, gn = (lane >> 4) & 1;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const int chunk = (wn * 16 + tj * 4 + 2 * gn + (q >> 1)) ^ (4 * r);
            b_off[tj] = (8 * h + r) * 512 + chunk * 16 + (q & 1) * 8;
        }
    }

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Operands of step s of the slice held in (sa half u, sb).
    auto load_frags = [&](const uint8_t* sa, int u, const uint8_t* sb, int s,
                          u32x4 (&a)[4], u32x4 (&b)[4]) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
            a[ti] = *reinterpret_cast<const u32x4*>(sa + a_off[ti][u][s]);
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const uint8_t* base = sb + b_off[tj] + s * 8192;
            const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(base));
            const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(base + 2048));
            const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            b[tj] = __builtin_bit_cast(u32x4, v);
        }
    };

    // 16 MFMAs on (a, b).  The 12 LDS reads and the copies issued just before
    // in program order are spread between them (3 LDS reads and one copy per
    // 4 MFMAs), so the address unit never sees a burst that would hold the
    // wave, and its MFMA issue, back.
    auto mfma_step = [&](const u32x4 (&a)[4], const u32x4 (&b)[4]) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < 4; ++tj)
                acc[ti][tj] = mfma32x32x16<T>(a[ti], b[tj], acc[ti][tj]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // copies (VMEM read)
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    u32x4 a0[4], b0[4], a1[4], b1[4];

    // Slice kt (its A in half u of sa, its B in sb); the next slice's A is in
    // half nu of na, its B in nb.  Copies, per wave:
    //   before the barrier: second half of B slice kt+3 into fb, and for even
    //     kt the second half of A pair kt/2+1 into fa;
    //   after the barrier: first half of B slice kt+4 into sb (just retired),
    //     and for odd kt the first half of A pair (kt+3)/2 into fa (the pair
    //     stage retired by this barrier).
    // The barrier of slice kt publishes slice kt+1.  Counting the copies
    // issued after the last one it needs gives 16 for even kt and 4 for odd kt
    // (odd kt also needs the A pair finished in the previous region).
    auto slice = [&](const uint8_t* sa, int u, uint8_t* sb, const uint8_t* na, int nu,
                     const uint8_t* nb, uint8_t* fb, uint8_t* fa, int kt, bool even) {
        load_frags(sa, u, sb, 1, a1, b1);  // step 2 operands of this slice
        copy_b(fb, kt + 3, 1);
        if (even) copy_a(fa, kt / 2 + 1, 1);
        mfma_step(a0, b0);                 // step 1 (operands read earlier)
        if (even) WAIT_VMCNT_LGKM0(16);    // own copies landed, own reads returned
        else WAIT_VMCNT_LGKM0(4);
        barrier();                         // ... for every wave
        load_frags(na, nu, nb, 0, a0, b0); // step 1 operands of the next slice
        copy_b(sb, kt + NSTAGE, 0);
        if (!even) copy_a(fa, (kt + 3) / 2, 0);
        mfma_step(a1, b1);                 // step 2
    };

    // Prologue: A pair 0, B slices 0..2, first halves of B slice 3 and A pair 1.
    copy_a(sA0, 0, 0);
    copy_a(sA0, 0, 1);
    copy_b(sB0, 0, 0);
    copy_b(sB0, 0, 1);
    copy_b(sB1, 1, 0);
    copy_b(sB1, 1, 1);
    copy_b(sB2, 2, 0);
    copy_b(sB2, 2, 1);
    copy_b(sB3, 3, 0);
    copy_a(sA1, 1, 0);
    WAIT_VMCNT(14);  // A pair 0 and B slice 0 landed
    barrier();
    load_frags(sA0, 0, sB0, 0, a0, b0);
    for (int kt = 0; kt < nk; kt += NSTAGE) {
        // A pair kt/2 in sA0, pair kt/2+1 in sA1
        slice(sA0, 0, sB0, sA0, 1, sB1, sB3, sA1, kt, true);
        slice(sA0, 1, sB1, sA1, 0, sB2, sB0, sA0, kt + 1, false);
        slice(sA1, 0, sB2, sA1, 1, sB3, sB1, sA0, kt + 2, true);
        slice(sA1, 1, sB3, sA0, 0, sB0, sB2, sA1, kt + 3, false);
    }
    WAIT_VMCNT(0);  // no copy may still target LDS when the workgroup ends

    // 32x32 accumulator layout: register r of lane l is row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the MFMA tile.  C is read
    // only when beta != 0.
    float* cbase = p.C + (int64_t)(m0 + wm * 128 + 4 * h) * p.ldc + n0 + wn * 128 + (lane & 31);
    const float alpha = p.alpha, beta = p.beta;
    if (beta == 0.0f) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < 4; ++tj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    cbase[(int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32] =
                        alpha * acc[ti][tj][r];
    } else {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int tj = 0; tj < 4; ++tj)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float* c = cbase + (int64_t)(ti * 32 + 8 * (r >> 2) + (r & 3)) * p.ldc + tj * 32;
                    *c = alpha * acc[ti][tj][r] + beta * (*c);
                }
    }
}

}  // namespace

bool mfma16_dma_eligible(const GemmParams& p) {
    return rows_16b_aligned(p.A, p.lda, 2) && rows_16b_aligned(p.B, p.ldb, 2) &&
           p.M % BM == 0 && p.N % BN == 0 && p.K % KALIGN == 0 && p.K > 0;
}

template <In T>
hipError_t launch_mfma16_dma(const GemmParams& p, hipStream_t s) {
    const int tiles_n = p.N / BN;
    const int64_t blocks = (int64_t)(p.M / BM) * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mfma16_dma_kernel<T>, dim3((unsigned)blocks), dim3(NT), 0, s, p,
                       tiles_n);
    return hipGetLastError();
}
template hipError_t launch_mfma16_dma<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_mfma16_dma<In::F16>(const GemmParams&, hipStream_t);

}  // namespace dgt
