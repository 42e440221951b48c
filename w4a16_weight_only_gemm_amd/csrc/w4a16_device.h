// w4a16_device.h -- device helpers shared by the gfx950 kernels: operand types,
// in-register dequantization of packed int4 words, and number conversions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4a16_internal {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global (address space 1) views of pointers. Pointers read from a descriptor
// in memory are generic to the compiler; through these, loads and stores are
// global_* instructions (counted only by vmcnt) rather than flat_* (counted by
// vmcnt and lgkmcnt, which would make every LDS wait also wait for them).
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

template <typename T>
__device__ __forceinline__ gptr<T> to_global(T* p) {
  return (gptr<T>)(p);  // address-space cast (generic to global)
}

// A value read through the constant address space: the memory must not be
// written while the kernel runs (a plan's problem table), and a uniform
// address then becomes a scalar load into SGPRs.
template <typename T>
__device__ __forceinline__ T load_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// s_waitcnt vmcnt(0) alone (expcnt and lgkmcnt left at their maxima). Stores
// and loads share the vector-memory counter but may retire out of order, so
// while a store is outstanding the compiler must wait for every load in
// flight before using any of them. Draining right after a rare store keeps a
// hot loop's later waits exact.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that orders LDS accesses only: global loads in flight
// keep flying (a plain __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave-uniform value moved to a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// bf16 bit pattern of -24.0 (sign 1, exponent 131 = 2^4, fraction 64/128), twice.
constexpr uint32_t kBiasPair = 0xC1C0C1C0u;

// Biased dequantization of one packed word: eight 4-bit two's-complement
// codes of k = 8j..8j+7, interleaved so that nibble v holds the code of
// k = 8j+2v and nibble v+4 that of k = 8j+2v+1. Output register v holds, as a
// bf16 pair, codes 2v (low half) and 2v+1 (high half), each as the exact
// value 24 + q: (c ^ 8) is the offset code q + 8 in 0..15, and placed in
// fraction bits 3..6 of 16.0 (0x4180, whose fraction step there is 1) it gives
// 16 + q + 8. The nibbles are moved to bits 3..6 and 19..22 of the register
// (one shift), then masked and xor-ed with 0x41C0 = 0x4180 ^ (8 << 3) (one
// and-xor): 0x41C0 ^ (c << 3) = 0x4180 | ((c ^ 8) << 3).
//
// Why 24 and not a larger base such as 128 + 8: the kernels remove the bias
// through fp32 sums of base * x, which round at the magnitude of base * sum|x|;
// 24 is the smallest base for which one or-into-the-fraction yields all sixteen
// codes as exact integers, so the rounding that large activations leave on a
// result near zero is 5.7 times smaller than with 136.
//
// MFMA consumes the eight bf16 of a register quad as k-slots 0..7, so the
// operand is in natural k order and pairs with eight consecutive bf16
// activations loaded as they are stored.
__device__ __forceinline__ bf16x8 dequant_biased(uint32_t w) {
  u32x4 r;
  r[0] = ((w << 3) & 0x00780078u) ^ 0x41C041C0u;
  r[1] = ((w >> 1) & 0x00780078u) ^ 0x41C041C0u;
  r[2] = ((w >> 5) & 0x00780078u) ^ 0x41C041C0u;
  r[3] = ((w >> 9) & 0x00780078u) ^ 0x41C041C0u;
  return __builtin_bit_cast(bf16x8, r);
}

// Eight consecutive bf16 activations (four dwords) as an MFMA operand.
__device__ __forceinline__ bf16x8 act_frag(u32x4 d) { return __builtin_bit_cast(bf16x8, d); }

__device__ __forceinline__ bf16x8 bias_operand() {
  u32x4 r = {kBiasPair, kBiasPair, kBiasPair, kBiasPair};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A lane permutation within rows of 16 lanes whose sources all exist.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF,
                                                     true));
}

// -24 times the sum of the 8 bf16 values of a 16-byte piece, in fp32: four
// bf16 dot products against the pair (-24, -24). Each product is exact in
// fp32 (8-bit by 2-bit significands); only the additions round.
__device__ __forceinline__ float neg_bias_sum8(u32x4 d) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 k = __builtin_bit_cast(bf16x2, kBiasPair);
  // Elements are copied to scalars first: this compiler's __builtin_bit_cast
  // of a vector-element expression (d[1]) reads the vector's first element.
  const uint32_t e0 = d[0], e1 = d[1], e2 = d[2], e3 = d[3];
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e0), k, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e1), k, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e2), k, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e3), k, s, false);
}

// Sum over the aligned group of LPG consecutive lanes containing this lane,
// returned in every lane of the group (butterfly within quads, half rows,
// rows of 16 lanes and pairs of rows). Each step adds two values in an order
// that does not matter (a + b = b + a), so every lane gets the same bits.
// All LPG lanes of the group must be active.
template <int LPG>
__device__ __forceinline__ float group_lane_sum(float v) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16 || LPG == 32, "group of 32, 64, 128 or 256");
  v += dpp_f32<0xB1>(v);                           // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);                           // quad_perm [2,3,0,1]
  if constexpr (LPG >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if constexpr (LPG >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if constexpr (LPG >= 32) v += __shfl_xor(v, 16);
  return v;
}

// Buffer resource over [base, base + bytes): loads at offsets at or beyond
// `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// LDS slot of 16-byte piece p of row r of the activation tile (256-byte
// rows: one row per line of the 64 banks): p ^ r' ^ ((r' & 4) << 1), r' = r
// mod 16. A 128-bit LDS read is served in four passes of 16 lanes, the lanes
// of a pass being those with equal (l5, l2 ^ l3 ^ l4) (found by counting
// SQ_LDS_BANK_CONFLICT over address patterns on gfx950). A fragment read
// puts rows 0..15 in lanes 0..15 and pieces p + WPL j in lane group j; with
// the plain p ^ r' two rows of one pass share a slot at group 128 (four
// conflict cycles per 128-bit read, as counted). With the extra bit
// every pass reads 16 distinct slots at groups 128, 64 and 32, and the
// staging writes (four rows of 16 pieces per wave) stay conflict-free.
__device__ __forceinline__ int lg_slot(int piece, int row) {
  const int r = row & 15;
  return piece ^ r ^ ((r & 4) << 1);
}

// Workgroup b of `total` in XCD-grouped order: XCD x (= b % 8) owns a
// contiguous range of the indices.
__device__ __forceinline__ int xcd_grouped(int b, int total) {
  const int xcd = b & 7, slot = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace w4a16_internal
