// k_mfma_f32.hip -- FP32 GEMM on the CDNA4 matrix cores.
//
// The pages' register-tiled kernel (dilfish.github.io 5.4: 128 x 128 block
// tile, 8 x 8 outputs per thread, double buffering) is rebuilt around
// wavefront-wide MFMA tiles: the register micro-tile of a lane becomes a
// 64 x 64 tile per wavefront computed by 2 x 2 v_mfma_f32_32x32x2_f32
// instructions, whose accumulators (64 fp32 per lane) stay in registers for
// the whole K loop.  The pages' matrix-unit sections (dilfish.github.io 5.5,
// qwbw.cn Level 2) use 16-bit inputs; on gfx950 the matrix cores also take
// fp32 operands at the full fp32 rate, so SGEMM keeps fp32 inputs and
// accumulation, with no TF32-style input truncation (dilfish.github.io 5.7
// warns that TF32 is not lossless).
//
// Workgroup: 256 lanes = 4 wavefronts in a 2 x 2 grid over a 128 x 128 tile
// of C; K advances in slices of 16.  Global -> LDS: each slice of A
// (128 x 16) and B (16 x 128) is read with coalesced 128-bit loads into
// one of two register sets two slices ahead and written to the other half
// of a double LDS buffer (dilfish.github.io 5.4 keeps one slice in flight;
// two hide more of the load latency), one barrier per slice.  Each operand is
// staged by how it is stored: rows along k (A, or B stored N x K) go to LDS
// as 128 rows of 16 k; rows along m / n (B, or A stored K x M) as 16 rows of
// 128.  Transposed operands therefore cost no extra pass.
//
// Operand order inside a slice: the 32x32x2 instruction sums over two k
// values, one per half-wavefront.  Half h of the wavefront feeds k = 8h + j
// at step j (j = 0..7), so each lane reads its 8 A values as two 128-bit
// LDS reads; any fixed assignment of k to steps is valid because every
// product lands in the same sum.
//
// LDS layout: a k-contiguous operand keeps 64-byte rows with its 16-byte
// chunks XOR-swizzled by row (kc_chunk), so that neither its 128-bit writes
// nor its 128-bit reads meet bank conflicts; an m/n-contiguous one has its
// rows padded to T + 4 floats (the two half-wavefronts read rows 8 apart and
// land on opposite halves of the 64 banks).  Ragged
// shapes: zero-filled loads outside A and B and masked stores
// (dilfish.github.io 5.7; elainafan.one masked tiled listing); the
// specialisation for shapes that are multiples of the tile skips the checks.
#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int BK = 16, NT = 256;
constexpr int KC_PITCH = BK;        // floats, rows along k (unpadded, chunks swizzled)

// Position of 16-byte chunk c (k 4c .. 4c+3) within k-contiguous row `row`
// in LDS.  Sixteen lanes of a 128-bit access meet in the same bank cycle;
// with 64-byte rows the swizzle spreads both access patterns over all 64
// banks: a write of 4 rows x 4 chunks (row % 4 gives the bank quarter,
// the chunk its position in it) and a read of one chunk from 16
// consecutive rows (row % 4 the quarter, row / 4 % 4 the XOR).  A padded
// pitch cannot serve both: 20 floats make the reads distinct but send rows
// 0 and 3 of a write to the same banks.
__device__ __forceinline__ int kc_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

// All ones when ok, else zero, through an empty asm statement the optimiser
// cannot see into, applied when the chunk is written to LDS: the load stays
// an ordinary unconditional load whose wait comes only at that write.
// (Zeroing by `ok ? v : 0` lets the optimiser recover the condition and turn
// the load into a branch around it; the wait for such a load lands right
// after it, at the branch's end, and the slice in flight no longer overlaps
// the MFMAs.)
__device__ __forceinline__ uint32_t keep_mask(bool ok) {
    uint32_t m = ok ? 0xffffffffu : 0u;
    asm("" : "+v"(m));
    return m;
}

__device__ __forceinline__ float masked(float x, uint32_t m) {
    return __uint_as_float(__float_as_uint(x) & m);
}

// 16 bytes from a 4-byte aligned address: one global_load_dwordx4 whatever
// the row pitch (the GPU runs with unaligned memory access enabled; the
// parity tests include pitches of a few floats past a 16-byte multiple).
__device__ __forceinline__ float4 load16(const float* src) {
    float4 v;
    __builtin_memcpy(&v, src, 16);
    return v;
}

// A 16-byte chunk of 4 floats at [col, col+4) of one row, zero outside: the
// raw load in v and, for the guarded forms, the mask(s) that zero what lies
// outside (NMASK: one for the whole chunk, or one per float).  rowp is a row
// that exists (a missing row is replaced by row 0 and row_ok is false); every
// lane loads from an address inside the operand (column 0 of its row when
// the chunk lies outside).  kVec with kGuard requires the limits (K, and M or
// N) to be multiples of 4, so that a chunk is either wholly inside or wholly
// outside; otherwise four 4-byte loads.
template <bool kVec, bool kGuard>
struct Chunk {
    static constexpr int NMASK = kGuard && !kVec ? 4 : 1;
    float4 v;
    uint32_t m[NMASK];

    __device__ __forceinline__ void load(const float* rowp, int col, int limit, bool row_ok) {
        if (!kGuard) {
            v = load16(rowp + col);
        } else if (kVec) {
            const bool ok = row_ok && col < limit;
            v = load16(rowp + (ok ? col : 0));
            m[0] = keep_mask(ok);
        } else {
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = row_ok && col + i < limit;
                x[i] = rowp[ok ? col + i : 0];
                m[i] = keep_mask(ok);
            }
            v = make_float4(x[0], x[1], x[2], x[3]);
        }
    }
    __device__ __forceinline__ float4 value() const {
        if (!kGuard) return v;
        const uint32_t* mm = m;
        return make_float4(masked(v.x, mm[0]), masked(v.y, mm[NMASK > 1 ? 1 : 0]),
                           masked(v.z, mm[NMASK > 1 ? 2 : 0]), masked(v.w, mm[NMASK > 1 ? 3 : 0]));
    }
};

// One operand's share of a K slice in LDS, for a T x T workgroup tile (T =
// 128 or 64).  kKC (stored rows run along k: A untransposed, B transposed):
// T mn-rows of 16 k, 64 bytes each with swizzled chunks (kc_chunk), and a
// lane reads its 8 k of one row as two 128-bit reads.  Otherwise (stored rows run along m / n): 16
// k-rows of T, pitch T + 4, and a lane reads one float per k.  Each lane
// moves T/64 16-byte chunks per slice.
template <bool kVec, bool kGuard, bool kKC, int T>
struct OpF32 {
    static constexpr int MN_PITCH = T + 4;       // floats, rows along m or n
    static constexpr int CH = T / 64;            // chunks per lane and slice
    static constexpr int TM = T / 64;            // 32 x 32 MFMA tiles per wave and dimension
    static constexpr int SIZE = kKC ? T * KC_PITCH : BK * MN_PITCH;  // floats per buffer
    Chunk<kVec, kGuard> r[CH];

    __device__ void load(const float* X, int64_t ld, int mn0, int mn_lim, int k0, int K,
                         int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int f = tid + NT * c;
            if (kKC) {  // chunk f: mn-row f/4, k 4*(f%4)
                const int row = mn0 + (f >> 2), col = k0 + 4 * (f & 3);
                const bool ok = row < mn_lim;
                r[c].load(X + (int64_t)(ok ? row : 0) * ld, col, K, ok);
            } else {    // chunk f: k-row f/(T/4), mn 4*(f%(T/4))
                const int krow = k0 + f / (T / 4), col = mn0 + 4 * (f % (T / 4));
                const bool ok = krow < K;
                r[c].load(X + (int64_t)(ok ? krow : 0) * ld, col, mn_lim, ok);
            }
        }
    }
    __device__ void store(float* dst, int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int f = tid + NT * c;
            float* d = kKC ? &dst[(f >> 2) * KC_PITCH + 4 * kc_chunk(f >> 2, f & 3)]
                           : &dst[(f / (T / 4)) * MN_PITCH + 4 * (f % (T / 4))];
            *reinterpret_cast<float4*>(d) = r[c].value();
        }
    }
    // The operand of MFMA tile t (rows / columns w*T/2 + t*32 + l%32) for
    // k = 8h + j: for kKC all eight j at once into v[t][0..7] ...
    __device__ void read_all(const float* src, int w, int h, int r32, float (&v)[TM][8]) const {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int row = w * (T / 2) + t * 32 + r32;
            const float* a = &src[row * KC_PITCH];
            *reinterpret_cast<float4*>(&v[t][0]) =
                *reinterpret_cast<const float4*>(a + 4 * kc_chunk(row, 2 * h));
            *reinterpret_cast<float4*>(&v[t][4]) =
                *reinterpret_cast<const float4*>(a + 4 * kc_chunk(row, 2 * h + 1));
        }
    }
    // ... otherwise one j at a time.
    __device__ float read_one(const float* src, int w, int h, int r32, int t, int j) const {
        return src[(8 * h + j) * MN_PITCH + w * (T / 2) + t * 32 + r32];
    }
};

// T x T workgroup tile (T = 128: waves of 64 x 64, two workgroups per CU;
// T = 64: waves of 32 x 32, for launches with few 128-tiles, four per CU).
template <bool kVec, bool kGuard, bool TA, bool TB, int T>
__global__ __launch_bounds__(NT, T == 64 ? 4 : 2) void mfma_f32_kernel(GemmParams p, int tiles_n) {
    constexpr int BM = T, BN = T, TM = T / 64;
    select_problem(p);
    using OpA = OpF32<kVec, kGuard, !TA, T>;
    using OpB = OpF32<kVec, kGuard, TB, T>;
    __shared__ float As[2][OpA::SIZE];
    __shared__ float Bs[2][OpB::SIZE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int m0 = (blockIdx.x / tiles_n) * BM;
    const int n0 = (blockIdx.x % tiles_n) * BN;
    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);

    floatx16 acc[TM][TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One slice's MFMAs from LDS buffer buf.  Operands: A rows
    // wm*T/2 + ti*32 + r32, B columns wn*T/2 + tj*32 + r32, k = 8h .. 8h+7.
    auto compute = [&](const OpA& ra, const OpB& rb, int buf) {
        float a[TM][8], b[TM][8];
        if constexpr (!TA) ra.read_all(As[buf], wm, h, r32, a);
        if constexpr (TB) rb.read_all(Bs[buf], wn, h, r32, b);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int x = 0; x < TM; ++x) {
                if constexpr (TA) a[x][j] = ra.read_one(As[buf], wm, h, r32, x, j);
                if constexpr (!TB) b[x][j] = rb.read_one(Bs[buf], wn, h, r32, x, j);
            }
        // 64-tiles: every operand read before the MFMAs, so that the LDS
        // round trips overlap (a wave's 8 MFMAs a slice leave little to hide
        // them behind; measured 4-8% faster).  128-tiles keep the compiler's
        // interleaving (measured 1.5% faster for them).
        if constexpr (T == 64) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float aj[TM], bj[TM];
#pragma unroll
            for (int x = 0; x < TM; ++x) {
                aj[x] = a[x][j];
                bj[x] = b[x][j];
            }
#pragma unroll
            for (int ti = 0; ti < TM; ++ti)
#pragma unroll
                for (int tj = 0; tj < TM; ++tj)
                    acc[ti][tj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        aj[ti], bj[tj], acc[ti][tj], 0, 0, 0);
        }
    };

    const int nk = (p.K + BK - 1) / BK;
    {
        // Two slices in flight (a 64-tile gives a CU little compute per
        // slice to hide a global load behind): slice s lives in register
        // set s % 2 from its load (at the start of iteration s - 2) until it
        // is written to LDS buffer s % 2 (at the end of iteration s - 1).
        // The loads and writes are unconditional (past the last slice a set
        // reloads slice nk - 1 and is written to the buffer no iteration
        // reads), so that every iteration issues the same loads and the
        // wait before a write covers only the older set's loads.
        OpA ra0, ra1;
        OpB rb0, rb1;
        auto load = [&](OpA& ra, OpB& rb, int s) {
            s = min(s, nk - 1);
            ra.load(A, p.lda, m0, p.M, s * BK, p.K, tid);
            rb.load(B, p.ldb, n0, p.N, s * BK, p.K, tid);
            // guarded: issue the loads before the MFMAs (whole tiles keep
            // the compiler's own schedule, measured faster for them)
            if constexpr (kGuard) __builtin_amdgcn_sched_barrier(0);
        };
        auto store = [&](const OpA& ra, const OpB& rb, int buf) {
            // keeps the masking of a guarded chunk (which waits for its
            // load) from being scheduled ahead of this point
            if constexpr (kGuard) __builtin_amdgcn_sched_barrier(0);
            ra.store(As[buf], tid);
            rb.store(Bs[buf], tid);
        };
        load(ra0, rb0, 0);
        load(ra1, rb1, 1);
        store(ra0, rb0, 0);
        __syncthreads();
        // iteration t: load slice t+2 into set t%2 (free: slice t is in LDS),
        // compute slice t, write slice t+1 to LDS buffer (t+1)%2
        auto iter = [&](int t, OpA& ra_cur, OpB& rb_cur, const OpA& ra_next,
                        const OpB& rb_next) {
            load(ra_cur, rb_cur, t + 2);
            compute(ra_cur, rb_cur, t & 1);
            store(ra_next, rb_next, (t + 1) & 1);
            __syncthreads();
        };
        int t = 0;
        for (; t + 1 < nk; t += 2) {
            iter(t, ra0, rb0, ra1, rb1);
            iter(t + 1, ra1, rb1, ra0, rb0);
        }
        if (t < nk) iter(t, ra0, rb0, ra1, rb1);
    }

    // Accumulator layout of a 32x32 MFMA tile: register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int ti = 0; ti < TM; ++ti)
#pragma unroll
        for (int tj = 0; tj < TM; ++tj) {
            const int col = n0 + wn * (T / 2) + tj * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * (T / 2) + ti * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (kGuard && (row >= p.M || col >= p.N)) continue;
                float* c = p.C + (int64_t)row * p.ldc + col;
                *c = epilogue(acc[ti][tj][r], p, c, col);
            }
        }
}

template <int T>
hipError_t launch_regs_tiles(const GemmParams& p, hipStream_t s) {
    const int tiles_n = (p.N + T - 1) / T;
    const int64_t blocks = (int64_t)((p.M + T - 1) / T) * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // 16-byte loads need 4-byte aligned operands (any pitch)
    const bool vec = reinterpret_cast<uintptr_t>(p.A) % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(p.B) % 4 == 0 && p.stride_a % 4 == 0 &&
                     p.stride_b % 4 == 0;
    const bool full = vec && p.M % T == 0 && p.N % T == 0 && k_multiple(p, BK);
    // guarded 16-byte chunks need every limit a multiple of 4 (see Chunk)
    const bool vec_edge = vec && p.M % 4 == 0 && p.N % 4 == 0 && p.K % 4 == 0;
    const dim3 grid((unsigned)blocks, p.batch), block(NT);
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (full)
            hipLaunchKernelGGL((mfma_f32_kernel<true, false, TA, TB, T>), grid, block, 0, s, p,
                               tiles_n);
        else if (vec_edge)
            hipLaunchKernelGGL((mfma_f32_kernel<true, true, TA, TB, T>), grid, block, 0, s, p,
                               tiles_n);
        else
            hipLaunchKernelGGL((mfma_f32_kernel<false, true, TA, TB, T>), grid, block, 0, s, p,
                               tiles_n);
        return hipGetLastError();
    });
}

}  // namespace

// The register-staged kernel on 128 x 128 tiles for any operands (the
// ladder's explicit rung, and what operands whose rows are not 16-byte
// aligned take when there are enough 128-tiles).
hipError_t launch_mfma_f32_regs(const GemmParams& p, hipStream_t s) {
    return launch_regs_tiles<128>(p, s);
}

// A launch with fewer 128-tiles than half the CUs leaves most of the chip
// idle whichever 128- or 256-tile kernel runs it; 64-tiles (four workgroups
// a CU) spread the same work over four times as many workgroups.
bool mfma_f32_small(const GemmParams& p) {
    const int64_t t128 = (int64_t)((p.M + 127) / 128) * ((p.N + 127) / 128) * p.batch;
    return t128 * 2 <= 256;
}

hipError_t launch_mfma_f32(const GemmParams& p, hipStream_t s) {
    if (mfma_f32_small(p)) return launch_regs_tiles<64>(p, s);
    if (mfma_f32_dma_eligible(p)) return launch_mfma_f32_dma(p, s);
    return launch_mfma_f32_regs(p, s);
}

}  // namespace dgt
