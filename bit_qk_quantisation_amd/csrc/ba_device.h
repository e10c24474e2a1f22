// Device-side building blocks for the gfx950 BinaryAttention kernels.
//
// Everything here is shared by the prologue (which expands the key signs),
// the fused forward kernel and the QK integer-dot kernel, so the integer dots
// that ba_qk_int_dot returns come from the very code the fused kernel runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ba {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v3f __attribute__((ext_vector_type(3)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Sign bit of the scaled binary representation: 1 iff x < 0 (an IEEE
// compare, so +0.0 and -0.0 both give 0, i.e. sign +1).  The sign function
// of s_i = mu_q sign(q_i) ("Representaciones Binarias Escaladas").
__device__ __forceinline__ uint32_t neg_bit(float x) { return x < 0.0f ? 1u : 0u; }

// Sign byte (bit b set iff channel b of the 8-channel chunk is negative) and
// the sum of |x| over the chunk, in a fixed order.
__device__ __forceinline__ uint32_t chunk_signs(const uint4& raw, float& part) {
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t byte = 0;
  float a[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = bf16_to_f32(static_cast<uint16_t>(wv[k] & 0xffffu));
    const float hi = bf16_to_f32(static_cast<uint16_t>(wv[k] >> 16));
    byte |= neg_bit(lo) << (2 * k);
    byte |= neg_bit(hi) << (2 * k + 1);
    a[2 * k] = fabsf(lo);
    a[2 * k + 1] = fabsf(hi);
  }
  part = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  return byte;
}

// --------------------------------------------------------------------------
// +/-1 operands in fp4 (e2m1) for the scaled f8f6f4 MFMA.
//
// In e2m1, +1.0 = 0b0010, -1.0 = 0b1010 and 0 = 0b0000.  A product of two
// +/-1 values is exact and the MFMA accumulates in fp32, so the result is the
// exact integer <sign q, sign k> = d - 2 popcount(q XOR k) (|D| <= 256).
//
// One 32-bit sign word (32 channels) fills the four operand dwords of one
// MFMA lane: dword k, nibble n holds the channel of bit 4n+k.  Every operand
// (query and key side alike) uses this same channel-to-slot map, and the
// contraction runs over all slots, so the slot order cancels out.  Channels
// past d carry sign bit 0 and get magnitude 0, so they contribute nothing.
// --------------------------------------------------------------------------

// Magnitude nibbles (0x2) for the valid channels of a word with `nvalid`
// channels (0, 8, 16, 24 or 32: d is a multiple of 8).  Bit 4n+k is valid iff
// 4n+k < nvalid, i.e. n < nvalid/4 for every k.
__device__ __forceinline__ uint32_t fp4_magnitude(int nvalid) {
  if (nvalid >= 32) return 0x22222222u;
  if (nvalid <= 0) return 0u;
  return 0x22222222u & ((1u << nvalid) - 1u);
}

// Valid channels of word `w` for head dim d.
__device__ __forceinline__ int word_valid(int d, int w) {
  int v = d - 32 * w;
  return v < 0 ? 0 : (v > 32 ? 32 : v);
}

__device__ __forceinline__ v4i expand_signs_fp4(uint32_t w, uint32_t mag) {
  v4i r;
  r[0] = static_cast<int>(((w << 3) & 0x88888888u) | mag);
  r[1] = static_cast<int>(((w << 2) & 0x88888888u) | mag);
  r[2] = static_cast<int>(((w << 1) & 0x88888888u) | mag);
  r[3] = static_cast<int>((w & 0x88888888u) | mag);
  return r;
}

// 32x32 block of sign dots over 64 channels: rows from `a` (lane = row % 32,
// channel group = lane / 32), columns from `b` (same map), accumulated into
// acc.  Output layout (CDNA 32x32 accumulator): lane l holds column l % 32
// and, in register r, row 8*(r/4) + 4*(l/32) + r%4.  The E8M0 scales are
// 127, i.e. 1.0.
__device__ __forceinline__ v16f mfma_signs_32x32x64(v4i a, v4i b, v16f acc) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc, 4, 4, 0, 127, 0, 127);
}

// bf16 32x32x16: lane l supplies row (A) / column (B) l % 32 and the eight
// k-slots 8*(l/32) .. 8*(l/32)+7.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// ---- scale products on the matrix cores ------------------------------------
// The logit of query i and key j multiplies the integer dot by
// w_ij = (alpha_q,i * scale * log2e) * alpha_k,j, an outer product.  A bf16
// 32x32x16 product computes a 32 x 32 block of it at fp32 precision when
// each factor enters as three bf16 terms x = x0 + x1 + x2 (each the
// round-to-nearest-even bf16 of what the earlier ones leave; every remainder
// is exact in fp32, so the terms carry x to within 2^-24 of itself): k-slots
// 0..5 hold the six products a_i b_j with i + j <= 2, which are exact, and
// the terms left out (i + j >= 3) add up to about 2^-25 a b.  So w is the
// product to within a few fp32 roundings.  Keys supply the A operand (row =
// key), queries the B operand (column = query); slots 6..15 hold zeros.

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split3_bf16(float x, uint32_t (&t)[3]) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    t[i] = bf16_rne_bits(x);
    x -= __uint_as_float(t[i] << 16);
  }
}

// The three A operand words of one key: slots 0..5 = b0 b1 b2 b0 b1 b0 (the
// fourth word, slots 6 and 7, is zero).
__device__ __forceinline__ void scale_split_a(float alpha_k, uint32_t (&w)[3]) {
  uint32_t b[3];
  split3_bf16(alpha_k, b);
  w[0] = b[0] | (b[1] << 16);
  w[1] = b[2] | (b[0] << 16);
  w[2] = b[1] | (b[0] << 16);
}

// B operand words of one query (slots 0..5 = a0 a0 a0 a1 a1 a2) for a lane
// of the low half; zeros for the high half (slots 8..15).
__device__ __forceinline__ v4u scale_split_b(float aq, bool low_half) {
  uint32_t a[3];
  split3_bf16(aq, a);
  if (!low_half) return v4u{0u, 0u, 0u, 0u};
  return v4u{a[0] | (a[0] << 16), a[0] | (a[1] << 16), a[1] | (a[2] << 16), 0u};
}

// Value of x in lane n of this lane's row of 16 lanes (DPP row_newbcast:n).
// n must be a constant once loops are unrolled; the broadcast then folds
// into the instruction that uses it as a DPP source operand.
template <int N>
__device__ __forceinline__ float row_bcast_c(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_bcast(float x, int n) {
  switch (n) {
    case 0: return row_bcast_c<0>(x);
    case 1: return row_bcast_c<1>(x);
    case 2: return row_bcast_c<2>(x);
    case 3: return row_bcast_c<3>(x);
    case 4: return row_bcast_c<4>(x);
    case 5: return row_bcast_c<5>(x);
    case 6: return row_bcast_c<6>(x);
    case 7: return row_bcast_c<7>(x);
    case 8: return row_bcast_c<8>(x);
    case 9: return row_bcast_c<9>(x);
    case 10: return row_bcast_c<10>(x);
    case 11: return row_bcast_c<11>(x);
    case 12: return row_bcast_c<12>(x);
    case 13: return row_bcast_c<13>(x);
    case 14: return row_bcast_c<14>(x);
    default: return row_bcast_c<15>(x);
  }
}

// DPP shifts inside each row of 16 lanes, zero where the source lane falls
// outside the row: row_shl:N gives lane l the value of lane l + N, row_shr:N
// that of lane l - N.  ROWS selects the rows that take the result; the other
// rows keep `old`.
template <int N, int ROWS = 0xF>
__device__ __forceinline__ float row_shl_c(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), 0x100 + N, ROWS, 0xF, true));
}
template <int N, int ROWS = 0xF>
__device__ __forceinline__ float row_shr_c(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), 0x110 + N, ROWS, 0xF, true));
}
// x in the rows ROWS selects, 0 in the others.
template <int ROWS>
__device__ __forceinline__ float rows_only(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xE4, ROWS, 0xF, true));
}

// Cross-half reductions for the 32x32 layout: lanes l and l^32 hold the two
// halves of one query's keys.  v_permlane32_swap of x with itself leaves
// (lower, lower) in r[0] and (upper, upper) in r[1], so r[0] op r[1] is the
// same value in both lanes of the pair.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  v2f f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, v2bf));
}

// acc + lo + hi of a packed bf16 pair (v_dot2 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  const v2bf one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, pair), one, acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- raw buffer access -------------------------------------------------------
// A buffer resource holds a uniform base address and a byte range; loads then
// take a per-lane 32-bit offset and a uniform (scalar) offset, so no per-lane
// 64-bit address arithmetic is needed.  A load whose offset falls outside the
// range returns 0.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw (untyped) buffer, 32-bit elements
constexpr uint32_t kOutOfRange = 0x80000000u; // an offset past every range used here

// `base` and `bytes` must be the same in every lane of the wave; they are
// moved to scalar registers here, so the compiler never has to assume
// otherwise (a resource it takes for per-lane would cost a loop per load).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)),
                                           kRsrcWord3);
}

// 16 bytes per lane from the buffer straight into LDS: lane l writes
// lds[16 l, 16 l + 16).  `lds` must be wave-uniform.
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16,
                                           voff, soff, 0, 0);
}

// As dma16, for data read once (a dense bias tile): the load is marked
// nontemporal, so it streams through L2 without displacing the key and value
// tiles that the other query tiles of the head read again.
__device__ __forceinline__ void dma16_nt(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16,
                                           voff, soff, 0, 2);
}

// 4 bytes per lane into LDS: lane l writes lds[4 l, 4 l + 4).
__device__ __forceinline__ void dma4(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 4,
                                           voff, soff, 0, 0);
}

__device__ __forceinline__ uint32_t buffer_u32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// MFMA results must be formed while every lane of the wave is active: a
// matrix instruction mixes data across lanes, and one issued under a partial
// EXEC mask drops the inactive lanes' rows.  LLVM treats the MFMA intrinsics
// as speculatable, so it may sink one below a divergent branch when its
// result is only used inside that branch.  Passing the result through an
// empty volatile asm in uniform control flow pins the MFMA above it.
__device__ __forceinline__ void pin_uniform(v16f& x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float e = x[i];
    asm volatile("" : "+v"(e));
    x[i] = e;
  }
}

}  // namespace ba
