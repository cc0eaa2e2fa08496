// k_mfma_bf16.hip -- 16-bit-input (BF16 or FP16) / FP32-accumulate GEMM on
// the CDNA4 matrix cores, register-staged (any shape, any alignment).  FP16
// takes the same path with v_mfma_f32_32x32x16_f16 (the pages' matrix-unit
// listings use half inputs: dilfish.github.io 5.5, qwbw.cn Level 2).
//
// The pages' matrix-unit rung (dilfish.github.io 5.5 WMMA listing; qwbw.cn
// Level 2 and its double-buffering row) feeds 16-bit inputs to the matrix
// unit and accumulates in fp32.  Here every wavefront owns a 128 x 128 tile
// of C built from 4 x 4 v_mfma_f32_32x32x16_bf16 instructions (256 fp32
// accumulators per lane, held in the accumulation registers for the whole K
// loop); four wavefronts in a 2 x 2 grid cover a 256 x 256 workgroup tile,
// so a 64-deep K slice of A and B (64 KiB) is read from memory once and
// reused 256 times per element from LDS (dilfish.github.io 5.3-5.4: tile
// size sets the arithmetic intensity, 2*256*256*64 / 65536 B = 128 FLOP/B
// here).  The products of two bf16 values are exact in fp32.
//
// Operand layout.  The MFMA takes, per lane, 8 consecutive k of one row of
// A and 8 consecutive k of one column of B.  An operand stored with k
// contiguous (A as M x K, or B stored transposed as N x K) has its 16-byte
// chunks go to LDS unchanged.  One stored with m or n contiguous (B as
// K x N, or A stored transposed as K x M): each lane loads an 8 (k) x 8
// (mn) block as eight 16-byte row pieces and transposes it in registers
// (byte permutes), then writes eight 16-byte column pieces, so both
// operands sit in LDS as 256 x 64 with k contiguous.  The
// pages warn that a fragment declared in the wrong major order still "looks
// right" (dilfish.github.io 5.5); the tests check with permutation and
// rank-1 inputs that rows and columns are not swapped.
//
// LDS layout (both operands): rows of 64 bf16 = eight 16-byte chunks; chunk
// q of row r is stored at position q ^ ((r ^ (r >> 3)) & 7).  Eight lanes
// reading the same chunk of 8 consecutive rows, and eight lanes writing
// rows 8 apart, both land on 8 distinct 16-byte bank groups (the XOR form
// of the padding remedy of dilfish.github.io 5.7 / qwbw.cn "Pad").
//
// Pipeline: the next K slice is loaded from global memory into registers
// while the current one is consumed from LDS; it is then written to the other
// LDS buffer (two 64 KiB stages in the 160 KiB LDS), one barrier per
// slice (dilfish.github.io 5.4 double buffering; 5.7 second barrier).
// Ragged shapes: zero-filled loads and masked stores; shapes that are tile
// multiples with 16-byte aligned rows use an unchecked specialisation.
#include "gemm_common.hpp"

namespace dgt {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int CPR = BK / 8;  // 16-byte chunks per LDS row (8)

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// 16 bytes from a 2-byte aligned address: one global_load_dwordx4 whatever
// the row pitch (the GPU runs with unaligned memory access enabled; the
// parity tests include pitches of a few elements past a 16-byte multiple).
__device__ __forceinline__ uint4 load16(const uint16_t* src) {
    uint4 v;
    __builtin_memcpy(&v, src, 16);
    return v;
}

// All ones when ok, else zero, through an empty asm statement the optimiser
// cannot see into, applied when the chunk is written to LDS: the load stays
// an ordinary unconditional load whose wait comes only at that write
// (zeroing by a select lets the optimiser turn the load into a branch
// around it, and the wait for it then comes right after it).
__device__ __forceinline__ uint32_t keep_mask(bool ok) {
    uint32_t m = ok ? 0xffffffffu : 0u;
    asm("" : "+v"(m));
    return m;
}

__device__ __forceinline__ uint4 masked(const uint4& v, uint32_t m) {
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// 8 elements at [col, col+8) of one row as a 16-byte chunk, zero outside,
// element by element (the form for limits that are not multiples of 8).
template <bool kVec, bool kGuard>
__device__ __forceinline__ uint4 load8(const uint16_t* rowp, int col, int limit,
                                       bool row_ok) {
    if (!kGuard) return load16(rowp + col);
    if (!row_ok) return make_uint4(0, 0, 0, 0);
    if (kVec && col + 8 <= limit) return load16(rowp + col);
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (col + 2 * i < limit) ? rowp[col + 2 * i] : 0u;
        const uint32_t hi = (col + 2 * i + 1 < limit) ? rowp[col + 2 * i + 1] : 0u;
        w[i] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Column j (0..7) of the 8 x 8 bf16 block r[0..7] (row k = index, 8 n per
// row) as 8 k-consecutive values: dword e holds rows 2e (low) and 2e+1.
__device__ __forceinline__ uint4 column8(const uint4 (&r)[8], int j) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = word(r[2 * e], j >> 1), hi = word(r[2 * e + 1], j >> 1);
        o[e] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                       : ((lo & 0xffffu) | (hi << 16));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ u32x4 as_u32x4(const uint4& v) {
    return u32x4{v.x, v.y, v.z, v.w};
}

// One operand's share of a 64-deep K slice, staged in LDS as 256 mn-rows of
// 64 k (eight swizzled 16-byte chunks per row) whichever way it is stored.
// kKC (stored rows run along k: A untransposed, B transposed): lane chunk i
// is row (tid>>3) + 32*i, chunk tid&7, stored unchanged.  Otherwise (stored
// rows run along m / n): the lane covers stored rows (k) 8*(tid>>5) .. +7
// and columns (mn) 8*(tid&31) .. +7, transposed in registers on the store.
//
// kVec with kGuard (limits, K and M or N, multiples of 8: a chunk is wholly
// inside or wholly outside): every lane loads its chunk unconditionally from
// an address inside the operand (column 0 of its row when the chunk lies
// outside) and the chunk is masked when written to LDS.  Without kVec the
// chunks are gathered element by element (load8).
template <bool kVec, bool kGuard, bool kKC>
struct Op16 {
    static constexpr bool kMasked = kVec && kGuard;
    uint4 r[8];
    uint32_t m[kMasked ? 8 : 1];

    __device__ __forceinline__ void load_chunk(int i, const uint16_t* rowp, int col, int limit,
                                               bool row_ok) {
        if constexpr (kMasked) {
            const bool ok = row_ok && col < limit;
            r[i] = load16(rowp + (ok ? col : 0));
            m[i] = keep_mask(ok);
        } else {
            r[i] = load8<kVec, kGuard>(rowp, col, limit, row_ok);
        }
    }
    __device__ __forceinline__ uint4 chunk(int i) const {
        if constexpr (kMasked) return masked(r[i], m[i]);
        else return r[i];
    }

    // mn0: first m (or n) of the tile, mn_lim: M (or N).
    __device__ void load(const uint16_t* X, int64_t ld, int mn0, int mn_lim, int k0, int K,
                         int tid) {
        if (kKC) {
            const int q = tid & 7, row0 = tid >> 3;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = mn0 + row0 + 32 * i;
                const bool ok = row < mn_lim;
                load_chunk(i, X + (int64_t)(ok ? row : 0) * ld, k0 + 8 * q, K, ok);
            }
        } else {
            const int c = tid & 31, g = tid >> 5;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int krow = k0 + 8 * g + i;
                const bool ok = krow < K;
                load_chunk(i, X + (int64_t)(ok ? krow : 0) * ld, mn0 + 8 * c, mn_lim, ok);
            }
        }
    }
    __device__ void store(uint4* dst, int tid) const {
        if (kKC) {
            const int q = tid & 7, row0 = tid >> 3;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = row0 + 32 * i;
                dst[row * CPR + (q ^ swz(row))] = chunk(i);
            }
        } else {
            const int c = tid & 31, g = tid >> 5;
            uint4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = chunk(i);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int n = 8 * c + j;
                dst[n * CPR + (g ^ swz(n))] = column8(v, j);
            }
        }
    }
};

template <In T, bool kVec, bool kGuard, bool TA, bool TB>
__global__ __launch_bounds__(NT, 1) void mfma16_kernel(GemmParams p, int tiles_n) {
    select_problem(p);
    __shared__ uint4 As[2][BM * CPR];
    __shared__ uint4 Bt[2][BN * CPR];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5, r32 = lane & 31;
    const int m0 = (blockIdx.x / tiles_n) * BM;
    const int n0 = (blockIdx.x % tiles_n) * BN;
    const uint16_t* A = static_cast<const uint16_t*>(p.A);
    const uint16_t* B = static_cast<const uint16_t*>(p.B);

    Op16<kVec, kGuard, !TA> ra;
    Op16<kVec, kGuard, TB> rb;
    auto load_slice = [&](int k0) {
        ra.load(A, p.lda, m0, p.M, k0, p.K, tid);
        rb.load(B, p.ldb, n0, p.N, k0, p.K, tid);
    };
    auto store_slice = [&](int buf) {
        ra.store(As[buf], tid);
        rb.store(Bt[buf], tid);
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // One slice in flight.  With guards the load is unconditional (past the
    // last slice it reloads slice nk - 1, written to the buffer no iteration
    // reads), so that the wait before the LDS write covers just this load,
    // and scheduling barriers keep the loads ahead of the MFMAs and the
    // masking and writes after them; whole tiles keep the compiler's own
    // schedule (measured faster for them).
    const int nk = (p.K + BK - 1) / BK;
    load_slice(0);
    store_slice(0);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
        if (kGuard || t + 1 < nk) load_slice(min(t + 1, nk - 1) * BK);
        if constexpr (kGuard) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            // half-wave h supplies k = 16s + 8h .. +7 for both operands
            const int q = 2 * s + h;
            u32x4 a[4], b[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int row = wm * 128 + ti * 32 + r32;
                a[ti] = as_u32x4(As[buf][row * CPR + (q ^ swz(row))]);
            }
#pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const int n = wn * 128 + tj * 32 + r32;
                b[tj] = as_u32x4(Bt[buf][n * CPR + (q ^ swz(n))]);
            }
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < 4; ++tj)
                    acc[ti][tj] = mfma32x32x16<T>(a[ti], b[tj], acc[ti][tj]);
        }
        if constexpr (kGuard) __builtin_amdgcn_sched_barrier(0);
        if (kGuard || t + 1 < nk) store_slice(buf ^ 1);
        __syncthreads();
    }

    // 32x32 accumulator layout: register r of lane l is row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the MFMA tile.
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const int col = n0 + wn * 128 + tj * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + ti * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (kGuard && (row >= p.M || col >= p.N)) continue;
                float* c = p.C + (int64_t)row * p.ldc + col;
                *c = epilogue(acc[ti][tj][r], p, c, col);
            }
        }
}

}  // namespace

template <In T>
hipError_t launch_mfma16_regs(const GemmParams& p, hipStream_t s) {
    const int tiles_n = (p.N + BN - 1) / BN;
    const int64_t blocks = (int64_t)((p.M + BM - 1) / BM) * tiles_n;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // 16-byte loads need 2-byte aligned operands (any pitch); guarded ones
    // limits that are multiples of 8 (see Op16)
    const bool vec = reinterpret_cast<uintptr_t>(p.A) % 2 == 0 &&
                     reinterpret_cast<uintptr_t>(p.B) % 2 == 0 && p.stride_a % 2 == 0 &&
                     p.stride_b % 2 == 0;
    const bool full = vec && p.M % BM == 0 && p.N % BN == 0 && k_multiple(p, BK);
    const bool vec_edge = vec && p.M % 8 == 0 && p.N % 8 == 0 && p.K % 8 == 0;
    const dim3 grid((unsigned)blocks, p.batch), block(NT);
    return with_layout(p, [&](auto ta, auto tb) {
        constexpr bool TA = decltype(ta)::value, TB = decltype(tb)::value;
        if (full)
            hipLaunchKernelGGL((mfma16_kernel<T, true, false, TA, TB>), grid, block, 0, s, p,
                               tiles_n);
        else if (vec_edge)
            hipLaunchKernelGGL((mfma16_kernel<T, true, true, TA, TB>), grid, block, 0, s, p,
                               tiles_n);
        else
            hipLaunchKernelGGL((mfma16_kernel<T, false, true, TA, TB>), grid, block, 0, s, p,
                               tiles_n);
        return hipGetLastError();
    });
}
// Operands with 16-byte aligned rows take the DMA kernel (any M, N and K);
// the register-staged kernel takes the others.
template <In T>
hipError_t launch_mfma16(const GemmParams& p, hipStream_t s) {
    if (mfma16_dma_eligible(p)) return launch_mfma16_dma<T>(p, s);
    return launch_mfma16_regs<T>(p, s);
}

template hipError_t launch_mfma16<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_mfma16<In::F16>(const GemmParams&, hipStream_t);
template hipError_t launch_mfma16_regs<In::BF16>(const GemmParams&, hipStream_t);
template hipError_t launch_mfma16_regs<In::F16>(const GemmParams&, hipStream_t);

}  // namespace dgt
