// Device helpers shared by the W4A16 decode kernels (single linear and
// stacked): the register unpack of packed nibbles into fp16 operands, fp16
// dot products and DPP lane sums, and raw buffer loads.
#pragma once

#include "awq_common.h"

namespace awq {

// Constants of the nibble unpack, made opaque to constant folding (the empty
// asm statements emit nothing).  gfx9 VOP3 encodings take no literal
// constants, so with literal masks the compiler splits (w & mask) | magic into
// v_and + v_or; with the masks in SGPRs and the magic numbers in VGPRs it
// selects a single v_and_or_b32 per fp16 pair.
struct UnpackConsts {
  uint32_t m_lo, m_hi, mag1024, mag64;
};
__device__ __forceinline__ UnpackConsts unpack_consts() {
  UnpackConsts u;
  u.m_lo = 0x000F000Fu;
  u.m_hi = 0x00F000F0u;
  u.mag1024 = 0x64006400u;
  u.mag64 = 0x54005400u;
  asm volatile("" : "+s"(u.m_lo));
  asm volatile("" : "+s"(u.m_hi));
  asm volatile("" : "+v"(u.mag1024));
  asm volatile("" : "+v"(u.mag64));
  return u;
}

// Unpack one qweight word into four fp16 pairs in slot order:
// (1024+q0, 1024+q4), (64+q1, 64+q5), (1024+q2, 1024+q6), (64+q3, 64+q7).
// Masking a nibble into the mantissa of 1024.0 (bits 0-3) or 64.0 (bits 4-7)
// gives offset + q exactly, with no conversion instruction: 5 instructions
// per 8 weights.
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t out[4], const UnpackConsts& k) {
  out[0] = (w & k.m_lo) | k.mag1024;
  out[1] = (w & k.m_hi) | k.mag64;
  const uint32_t w8 = w >> 8;
  out[2] = (w8 & k.m_lo) | k.mag1024;
  out[3] = (w8 & k.m_hi) | k.mag64;
}

// fp32 accumulate of a two-term fp16 dot product (v_dot2_f32_f16)
__device__ __forceinline__ float dot2_f16(half2_t a, half2_t b, float c) {
  typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2_t, a), __builtin_bit_cast(fp16x2_t, b), c,
                                false);
}

// Sum over aligned groups of N = 4, 8 or 16 lanes, returned in every lane of
// the group, with DPP lane moves inside a 16-lane row: swap neighbours, swap
// pairs (quad permutes), then the mirror of each 8-lane half and of the row.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   CTRL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ float row_group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  v = dpp_add<0xB1>(v);                       // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);                       // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) v = dpp_add<0x141>(v);    // row_half_mirror
  if constexpr (N >= 16) v = dpp_add<0x140>(v);   // row_mirror
  return v;
}

// Raw buffer loads: the resource records the tensor's byte size, and the
// hardware returns zero for any lane whose offset reaches it, so a partial
// last column block needs no per-lane clamp, and each load is a loop-invariant
// per-lane offset plus a scalar offset (no vector address arithmetic in the
// loop).  Sizes are below 4 GiB (checked at the C ABI).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
template <int WPL>
__device__ __forceinline__ void buf_words(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                          uint32_t (&w)[WPL]) {
  if constexpr (WPL == 4) {
    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (WPL == 2) {
    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  }
}

}  // namespace awq
