// Device helpers shared by the gfx950 kernels of the AWQ W4A16 path.
//
// Exactness rules the kernels rely on (compiled with -ffp-contract=off, IEEE
// division, fp16/fp32/fp64 denormals kept):
//  * fp16 x fp16 products are exact in fp32 (11 + 11 significant bits), so
//    W' = fp16_rn(W * s) is one product and one hardware RNE conversion;
//  * per-group ranges are formed in float64 (the difference of two fp16 values
//    can need 40 bits) and rounded to fp16 by f64_to_f16_rn (single rounding);
//  * RNE(w / D) for fp16 w, D is one correctly rounded fp32 quotient followed by
//    rintf; the quotient comes from a correctly rounded reciprocal refined by
//    one fused residual step (rne_quot).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr uint16_t kF16NaN = 0x7E00;
constexpr uint16_t kF16One = 0x3C00;

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(half_t, b);
}
__device__ __forceinline__ uint16_t f2h_rn(float f) {
  return __builtin_bit_cast(uint16_t, (half_t)f);   // v_cvt_f16_f32, RNE
}
__device__ __forceinline__ bool f16_nonfinite(uint16_t b) {
  return (b & 0x7C00u) == 0x7C00u;
}

// binary16 round-to-nearest-even of a float64, from the float64 bits (one
// rounding; subnormal results kept; overflow to inf; NaN stays NaN).
// bf16 activations: a bf16 bit pattern as float (exact), a float rounded to
// bf16 (nearest, ties to even; NaN stays NaN), and 16-bit activation patterns
// as fp16: fp16 patterns unchanged, bf16 patterns rounded once to fp16 (exact
// for |x| in the fp16 normal range [2^-14, 65504]).
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f2bf_rn(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t act_h(uint16_t raw, bool bf) {
  return bf ? f2h_rn(bf2f(raw)) : raw;
}
__device__ __forceinline__ uint32_t act2_h(uint32_t raw, bool bf) {
  if (!bf) return raw;
  return (uint32_t)f2h_rn(bf2f((uint16_t)raw)) | ((uint32_t)f2h_rn(bf2f((uint16_t)(raw >> 16))) << 16);
}
__device__ __forceinline__ uint4 act8_h(uint4 raw, bool bf) {
  if (!bf) return raw;
  return make_uint4(act2_h(raw.x, true), act2_h(raw.y, true), act2_h(raw.z, true), act2_h(raw.w, true));
}
// an output value rounded once to the activation type
__device__ __forceinline__ uint16_t f2act(float f, bool bf) { return bf ? f2bf_rn(f) : f2h_rn(f); }

__host__ __device__ __forceinline__ uint16_t f64_to_f16_rn(double d) {
  uint64_t b = __builtin_bit_cast(uint64_t, d);
  uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
  int e = (int)((b >> 52) & 0x7FF);
  uint64_t m = b & ((1ull << 52) - 1);
  if (e == 0x7FF) return (uint16_t)(sign | 0x7C00u | (m ? 0x200u : 0u));
  if (e == 0) return (uint16_t)sign;          // zero or float64-subnormal: < 2^-1022
  int E = e - 1023;
  if (E > 15) return (uint16_t)(sign | 0x7C00u);
  uint64_t mant = m | (1ull << 52);            // value = mant * 2^(E-52)
  int qexp = (E >= -14) ? (E - 10) : -24;      // quantum of the fp16 result
  int shift = qexp - (E - 52);                 // >= 42
  if (shift >= 64) return (uint16_t)sign;      // below half the quantum
  uint64_t q = mant >> shift;
  uint64_t rem = mant & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1ull))) q++;
  if (qexp == -24) return (uint16_t)(sign | (uint32_t)q);   // subnormal (q may reach 1024 = min normal)
  if (q == 2048) { q = 1024; E += 1; }
  if (E > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | ((uint32_t)(E + 15) << 10) | ((uint32_t)q & 0x3FFu));
}

// Round-half-even of w / d for fp16 values w, d > 0 held in fp32, given
// rd = 1.0f / d correctly rounded.  t1 is within one ulp of w/d; the residual
// w - t1*d is exact in one fma; t1 + residual*rd is then the correctly
// rounded quotient, so exact ties k + 1/2 come out exactly and rintf applies
// the tie-to-even rule.  Away from ties the quotient of two fp16 values lies
// at least 2^-12 from any half-integer (for |w/d| <= 2^10), far beyond the
// fp32 error, so rintf never picks the wrong side.
__device__ __forceinline__ float rne_quot(float w, float d, float rd) {
  float t1 = w * rd;
  float r = __builtin_fmaf(-t1, d, w);
  float t2 = __builtin_fmaf(r, rd, t1);
  return __builtin_rintf(t2);
}

// Per-group step, zero and reciprocal from the group's fp16 max and min, for
// codes 0..qmax (qmax = 2^w_bit - 1: 15 for 4-bit weights, 7 and 255 for the
// 3- and 8-bit variants).  rne_quot is exact for |w / D| <= 2^10; beyond that
// the clamp to -z .. qmax - z decides whatever the rounding, as qmax <= 255.
struct GroupQ {
  float d;      // step D (an fp16 value)
  float rd;     // 1/D, correctly rounded fp32
  float z;      // zero point, integer 0..qmax
  float qmax;
  uint16_t d_bits;
};

__device__ __forceinline__ GroupQ group_q(float mx, float mn, float qmax = 15.0f) {
  GroupQ gq;
  double r = (double)mx - (double)mn;          // exact in float64
  r = r > 0x1p-16 ? r : 0x1p-16;
  gq.d_bits = f64_to_f16_rn(r / (double)qmax);
  gq.d = h2f(gq.d_bits);
  gq.rd = 1.0f / gq.d;
  gq.qmax = qmax;
  float z = rne_quot(-mn, gq.d, gq.rd);
  gq.z = __builtin_fminf(__builtin_fmaxf(z, 0.0f), qmax);
  return gq;
}

// (q - z) for one element: clamp(RNE(w/D) + z, 0, qmax) - z as a float.
__device__ __forceinline__ float code_minus_zero(float w, const GroupQ& gq) {
  float t = rne_quot(w, gq.d, gq.rd);
  return __builtin_fminf(__builtin_fmaxf(t, -gq.z), gq.qmax - gq.z);
}

// Tile t of a linear's tiles_m x tiles_n output tiles in banded order: bands
// of GM row tiles, each band column by column with its row tiles fastest.  A
// contiguous run of the order (the work-groups resident on one XCD at a time)
// then covers a few row tiles and a few column tiles rather than every row
// tile of a few columns, so both operands' tiles are shared in that XCD's L2.
// A bijection of [0, tiles_m * tiles_n); with at most GM row tiles it is the
// plain rows-fastest order.
template <int GM>
__device__ __forceinline__ void banded_tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  if (tiles_m <= GM) {
    tm = t % tiles_m;
    tn = t / tiles_m;
    return;
  }
  const int span = GM * tiles_n;
  const int band = t / span, first = band * GM;
  const int rows = tiles_m - first < GM ? tiles_m - first : GM;
  const int r = t - band * span;
  tm = first + r % rows;
  tn = r / rows;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ double shfl_xor_d(double v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace awq
