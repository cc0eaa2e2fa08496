// dma_common.hpp -- pieces shared by the global->LDS DMA GEMM kernels
// (k_mfma_bf16_dma.hip for 16-bit inputs, k_mfma_f32_dma.hip for fp32): the
// copy through a buffer descriptor, the K-contiguous swizzle, the wait and
// barrier helpers, compile-time stage selection, and the wait counts of
// their common copy schedule.
#pragma once

#include "gemm_common.hpp"

namespace dgt {
namespace dma {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kCopyPolicy = 1;  // sc0 on the copies (sc1 or sc0 sc1: 10-20% slower)
constexpr int64_t kCUs = 256;

// A copy descriptor's range ends at an operand's last element rounded up to
// a whole 16-byte chunk (kElems elements): the hardware returns zeros for a
// 16-byte load that reaches past the range, even for its bytes inside it.
// The rounding never reads another page (a 16-byte aligned chunk lies within
// one), and what it reads past the element only feeds outputs that are not
// stored or k that are masked.
template <int kElems>
__device__ __forceinline__ int round_chunk(int n) {
    return (n + kElems - 1) & ~(kElems - 1);
}

// One 16-byte-per-lane copy, global -> LDS, through a buffer descriptor of
// `range` bytes from `base`: lane l's bytes at base + voff + soff land at
// lds + 16*l.  (A plain function: the host pass of the kernels' templates
// then never sees the device-only descriptor type.)
__device__ __forceinline__ void dma16(const void* base, uint32_t range, uint8_t* lds,
                                      uint32_t voff, uint32_t soff) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, range, kBufferRsrcW3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, kCopyPolicy);
}

// K-contiguous rows are 128 B = 8 chunks of 16 B; chunk q of row r sits at
// q ^ swz_kc(r).
__device__ __forceinline__ int swz_kc(int r) { return (r ^ (r >> 3)) & 7; }

// Workgroup barrier without a memory fence: LDS data written by copies is
// published by each wave waiting for its own copies first.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Stage I of an operand, chosen at compile time so that every LDS access
// names one __shared__ object (the compiler's wait-count pass then sees that
// a copy in flight into one stage does not alias reads of another).
template <int I>
__device__ __forceinline__ uint8_t* pick(uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3) {
    if constexpr (I == 0) return s0;
    else if constexpr (I == 1) return s1;
    else if constexpr (I == 2) return s2;
    else return s3;
}

// Copies a wave has issued after the last one that slice kt+1 needs, at the
// wait in slice kt (steady state; the prologue is laid out to match), for
// ckc copy instructions per half pair of a K-contiguous operand and cmn per
// half slice of an MN-contiguous one.  Per slice: K-contiguous operands
// copy half a pair before the barrier of even slices and after the barrier
// of odd ones; MN-contiguous ones copy half a slice before and half after
// every barrier, and are issued first.  With one operand of each kind the
// last copy slice kt+1 needs is the K-contiguous half pair issued before
// the barrier of slice kt-2 (kt even) or kt-1 (kt odd); with two
// MN-contiguous ones, the second's half slice before the barrier of kt-2.
template <bool AK, bool BKc, bool kEven>
constexpr int copies_after(int ckc, int cmn) {
    if (AK != BKc) return kEven ? 4 * cmn + 2 * ckc : 2 * cmn;  // one operand of each kind
    if (AK) return kEven ? 4 * ckc : 0;                         // both K-contiguous
    return 8 * cmn;                                             // both MN-contiguous
}

// Copies issued by the prologue after the last one slice 0 needs: every
// MN-contiguous operand still has slices 1 and 2 and half of slice 3 after
// it (5 half slices), every K-contiguous one the first half of pair 1.
template <bool AK, bool BKc>
constexpr int prologue_after(int ckc, int cmn) {
    constexpr int nmn = (AK ? 0 : 1) + (BKc ? 0 : 1), nkc = 2 - nmn;
    return nmn ? 5 * cmn * nmn + ckc * nkc : ckc * nkc;
}
static_assert(copies_after<true, false, true>(4, 2) == 16 && copies_after<true, false, false>(4, 2) == 4 &&
              copies_after<true, true, true>(4, 2) == 16 && copies_after<true, true, false>(4, 2) == 0 &&
              copies_after<false, false, true>(4, 2) == 16 && prologue_after<true, false>(4, 2) == 14 &&
              prologue_after<true, true>(4, 2) == 8 && prologue_after<false, false>(4, 2) == 20,
              "the 256-tile wait counts");

}  // namespace dma
}  // namespace dgt

// s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima (gfx9
// encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt in 6:4,
// lgkmcnt in 11:8); DMA_WAIT_VMCNT_LGKM0 also drains this wave's LDS reads.
#define DMA_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)
#define DMA_WAIT_VMCNT_LGKM0(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0070)
