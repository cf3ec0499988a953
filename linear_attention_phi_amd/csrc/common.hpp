// common.hpp -- device helpers shared by the linear-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace linattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;    // tokens per chunk (one MFMA-tiled step of the chunked form)
constexpr int kThreads = 256; // four 64-wide waves per workgroup

// ---------------------------------------------------------------- feature map
// phi(x) = elu(x) + 1: x + 1 for x >= 0 and exp(x) for x < 0 (elu's exp(x) - 1,
// plus one).  Mode 1 is the identity map used for the post-feature-map worked
// examples.  Mode 2 (kFeatElu) is elu itself, phi - 1: the backward writes
// phi(x) = 1 + elu(x) and carries the constant part separately, so that the
// bf16 copy of a feature keeps its varying part at full relative precision
// (bf16 of 1 + x keeps only the bits of x above 2^-8).
constexpr int kFeatElu = 2;
__device__ __forceinline__ float phi_fast(float x, int mode) {
    if (mode == 1) return x;
    // exp(x) = 2^(x log2 e) on the hardware exp2; relative error ~1e-7 for the
    // |x| seen here, far below the bf16 rounding that follows.
    const float e = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
    if (mode == kFeatElu) return x >= 0.f ? x : e - 1.f;
    return x >= 0.f ? x + 1.f : e;
}
__device__ __forceinline__ float phi_exact(float x, int mode) {
    if (mode) return x;
    return x >= 0.f ? x + 1.f : expf(x);
}

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16, returned as raw bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return (uint32_t)__builtin_bit_cast(unsigned short, b);
}
// x rounded to the nearest bf16 (ties to even), as a float.
__device__ __forceinline__ float bf16_round(float x) { return __uint_as_float(f32_to_bf16_bits(x) << 16); }
// Two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The wave index as a scalar, so that conditions on it branch on the scalar unit.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------- MFMA
// 16x16x32 bf16 -> fp32.  Lane l supplies A[l%16][8(l/16)+i], B[8(l/16)+i][l%16]
// (i = 0..7) and receives D[4(l/16)+i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
// Eight bf16 ones (0x3f80): an MFMA operand that turns a product into row or
// column sums.
__device__ __forceinline__ bf16x8 bf16_ones8() { return as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u)); }

// Streaming (non-temporal) 16-byte global load: every input row is read once,
// so it should not displace cache lines that are reused.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

// Buffer resource over [base, base + nbytes): raw (stride 0) buffer loads at a
// byte offset at or past nbytes return zero instead of touching memory.  The
// last descriptor word is the gfx9 default data format (32-bit, no swizzle).
// Base and size are the same in every lane of a wave; they are taken from the
// first lane so that the descriptor sits in scalar registers even where the
// compiler formed them on the vector unit (a clamp lowers to v_med3, for one),
// which would otherwise make it loop over the lanes' distinct descriptors.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t chunk_rsrc(const void *base, int nbytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
}
// 16-byte buffer load at byte offset voff (bounds-checked).  STREAM marks it
// non-temporal (cache-policy bit 1).
template <bool STREAM>
__device__ __forceinline__ uint4 buffer_load16(rsrc_t rs, int voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, STREAM ? 2 : 0));
}

// 4-byte buffer load (bounds-checked: 0 past the range).
__device__ __forceinline__ float buffer_load_f32(rsrc_t rs, int voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, 0));
}

// Buffer stores at byte offset voff: a store at or past the descriptor's size
// is dropped by the hardware.  Rows past the end of a sequence are skipped
// this way instead of under a branch, so that every store is an instruction
// the compiler counts: waits for loads issued before a chunk's stores then
// need not wait for the stores too.
__device__ __forceinline__ void buffer_store16(uint4 v, rsrc_t rs, int voff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff, 0, 0);
}
__device__ __forceinline__ void buffer_store8(uint2 v, rsrc_t rs, int voff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, voff, 0, 0);
}
__device__ __forceinline__ void buffer_store_f32(float v, rsrc_t rs, int voff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, voff, 0, 0);
}
// An offset past every descriptor the kernels form: each covers under 1 GiB
// (a chunk's rows, or one (b, h)'s state cells, which the host keeps below it).
constexpr int kDropOffset = 1 << 30;

// ---------------------------------------------------------------- cross-lane
// Sum over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15), the same in
// each of them: rotations by 8, 4, 2 and 1 within the row (every step adds two
// values that the row's lanes pair symmetrically, so all lanes round alike).
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
    return x;
}

// Sum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
// On the gfx950 row swaps (VALU, no LDS round trip): with both operands v,
// v_permlane16_swap returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of v, and
// v_permlane32_swap its lower and upper halves each twice, so the two adds
// are (v0 + v1) + (v2 + v3) in every lane, in the same order everywhere.
__device__ __forceinline__ float sum_over_groups(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
    const unsigned w = __builtin_bit_cast(unsigned, v);
    const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// ---------------------------------------------------------------- gating
// In-chunk decay bookkeeping.  Within a chunk the decay between key j and
// query t (j <= t) is prod_{m=j+1..t} a_m.  It is carried as a pair (count of
// exactly-zero gates, sum of log of the nonzero gates) over the inclusive
// prefix (log base 2), so that a zero gate clears exactly and no -inf - -inf
// arises:
//   decay(j -> t) = 0                       if zeros(t) > zeros(j)
//                 = 2^(lsum(t) - lsum(j))   otherwise.
// A gate below the smallest normal float counts as zero.
__device__ __forceinline__ float decay_between(float to_lsum, int to_zeros, float from_lsum, int from_zeros) {
    return to_zeros > from_zeros ? 0.f : __builtin_amdgcn_exp2f(to_lsum - from_lsum);
}
// The same decay from one number per token, kappa = lsum - kZeroShift * zeros
// (both prefixes still scanned exactly, then combined): across a zero gate the
// exponent is below -kZeroShift, far under the smallest float, so exp2 gives
// exactly 0; between tokens with the same zero count the shift cancels, up to
// the rounding of kappa (for z zeros, about 2^-23 * 256 z of the exponent:
// 3e-5 relative in the decay per zero before the pair).  The exponent is
// positive only for pairs out of causal order, which callers mask after the
// product (it can overflow to inf there).
constexpr float kZeroShift = 256.f;
__device__ __forceinline__ float decay_k(float to_kappa, float from_kappa) {
    return __builtin_amdgcn_exp2f(to_kappa - from_kappa);
}
__device__ __forceinline__ bool gate_is_zero(float a) { return a < 1.17549435e-38f; }  // NaN stays NaN
__device__ __forceinline__ float gate_log2(float a) { return gate_is_zero(a) ? 0.f : __builtin_amdgcn_logf(a); }

// Inclusive scan over the 64 lanes of a wave (lane order = token order), on
// DPP: shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in from
// outside the row add 0), then the last lane of row 0 added to row 1 and of
// row 2 to row 3 (row_bcast:15), then lane 31 added to rows 2 and 3
// (row_bcast:31).  Rows not selected by a step's row mask add 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_or_zero(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ void scan_step(float &lsum, int &zeros) {
    lsum += __builtin_bit_cast(float, dpp_or_zero<CTRL, ROWS>(__builtin_bit_cast(int, lsum)));
    zeros += dpp_or_zero<CTRL, ROWS>(zeros);
}
__device__ __forceinline__ void wave_inclusive_scan(float &lsum, int &zeros) {
    scan_step<0x111, 0xf>(lsum, zeros); // row_shr:1
    scan_step<0x112, 0xf>(lsum, zeros); // row_shr:2
    scan_step<0x114, 0xf>(lsum, zeros); // row_shr:4
    scan_step<0x118, 0xf>(lsum, zeros); // row_shr:8
    scan_step<0x142, 0xa>(lsum, zeros); // row_bcast:15 into rows 1, 3
    scan_step<0x143, 0xc>(lsum, zeros); // row_bcast:31 into rows 2, 3
}

} // namespace linattn
