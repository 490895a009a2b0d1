// W4A16 linear: y = x_tilde W_deq^T with 4-bit group-quantized weights
// (layout v1) and fp16 activations.  bjdmk.com.cn page, section
// "量化参数配置" / "技术选型决策树": a GEMV mode for batch-1 decode and a GEMM
// mode for long inputs; zeeklog.com page: W4A16 kernels; jsqmd.com page,
// section 二.1 (3): the activation is divided by s at inference
// (x_tilde = x * inv_s16).
//
// Decode path (m <= 32): two kernels.
//  * linear_prep stages x_tilde once per call as the MFMA A operand: every
//    token contributes an fp16 hi row and an fp16 lo row (x_tilde = hi + lo,
//    so the staged activation carries ~22 bits), 8 tokens per 16-row chunk,
//    with the channels of each 8-channel word permuted into the order the
//    weight nibbles come out of the register unpack.  It also stores, per
//    (row, group), U = sum of the staged values and T = sum of the staged
//    values times the unpack offset (1024 or 64, see below).
//  * linear_skinny streams the packed weights once.  Lane l of a wave owns
//    output column n0 + l%16 and loads g/32 consecutive qweight words (one
//    16-byte load at g=128).  Each word becomes four fp16 pairs by masking
//    nibbles into the mantissa of 1024.0 (bits 0-3) or 64.0 (bits 4-7), so
//    the B operand holds offset + q exactly, with no conversion instruction.
//    v_mfma_f32_16x16x32_f16 multiplies them with the staged activations; per
//    group, y += D * (C - T - z U) removes the offset and the zero point
//    exactly in fp32.  Waves of a work-group split the groups of K; their
//    partial sums meet in LDS in a fixed order.
// Prefill path (m > 32): linear_gemm, 128 x 128 output tiles; each K-step
// dequantizes a 128 x 32 weight tile ((q - z) * D * inv_s, rounded once to
// fp16) into LDS next to the fp16 activation tile and runs
// v_mfma_f32_32x32x16_f16 with fp32 accumulation.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kSkinnyTok = 8;          // tokens per 16-row A chunk (hi + lo rows)
constexpr int kSkinnyWaves = 8;        // waves per work-group

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t linear_scratch_bytes(int64_t m, int64_t k, int32_t g) {
  if (m > 32) return 0;
  const int64_t tc = (m + kSkinnyTok - 1) / kSkinnyTok;
  const int64_t ng = k / g;
  size_t a = (size_t)tc * (size_t)k * 16 * 2;          // [tc][ng][4][16][g/4] halves
  size_t tu = (size_t)tc * (size_t)ng * 16 * 8;        // [tc][ng][16] float2
  return align256(a) + align256(tu);
}

// slot s (0..7) of an 8-channel word in unpack order -> nibble index
__device__ __forceinline__ int slot_nibble(int s) { return (s >> 1) + 4 * (s & 1); }

template <int G>
__global__ __launch_bounds__(256) void linear_prep_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s, int64_t m, int64_t k,
    int64_t n_pairs, uint16_t* __restrict__ a_st, float2* __restrict__ tu) {
  constexpr int WPL = G / 32;                  // qweight words per lane per group
  constexpr int HPL = G / 4;                   // staged halves per lane per group
  const int64_t ng = k / G;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (tc, j)
  if (pair >= n_pairs) return;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t tc = pair / ng, j = pair % ng;
  const int64_t t = tc * kSkinnyTok + (r & 7);
  const bool lo_row = r >= 8;
  uint16_t vals[HPL];
  double tsum = 0.0, usum = 0.0;
#pragma unroll
  for (int i = 0; i < WPL; ++i) {
    const int64_t kw = j * G + 8 * (WPL * c + i);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int nib = slot_nibble(s);
      uint16_t h = 0;
      if (t < m) {
        float xv = h2f(x[t * k + kw + nib]);
        if (inv_s != nullptr) xv *= h2f(inv_s[kw + nib]);   // exact: fp16 x fp16
        uint16_t hb = f2h_rn(xv);
        h = lo_row ? f2h_rn(xv - h2f(hb)) : hb;
      }
      vals[i * 8 + s] = h;
      const double hv = (double)h2f(h);
      usum += hv;
      tsum += hv * ((nib & 1) ? 64.0 : 1024.0);
    }
  }
  uint16_t* dst = a_st + ((pair * 4 + c) * 16 + r) * HPL;
#pragma unroll
  for (int i = 0; i < HPL; i += 8) {
    uint4 v;
    v.x = (uint32_t)vals[i + 0] | ((uint32_t)vals[i + 1] << 16);
    v.y = (uint32_t)vals[i + 2] | ((uint32_t)vals[i + 3] << 16);
    v.z = (uint32_t)vals[i + 4] | ((uint32_t)vals[i + 5] << 16);
    v.w = (uint32_t)vals[i + 6] | ((uint32_t)vals[i + 7] << 16);
    *reinterpret_cast<uint4*>(dst + i) = v;
  }
  // sum over the 4 lane groups c holding the same row r (lanes r, r+16, r+32, r+48)
  tsum += shfl_xor_d(tsum, 16);
  tsum += shfl_xor_d(tsum, 32);
  usum += shfl_xor_d(usum, 16);
  usum += shfl_xor_d(usum, 32);
  if (c == 0) tu[pair * 16 + r] = make_float2((float)tsum, (float)usum);
}

// Unpack one qweight word into four fp16 pairs in slot order:
// (1024+q0, 1024+q4), (64+q1, 64+q5), (1024+q2, 1024+q6), (64+q3, 64+q7).
__device__ __forceinline__ void unpack_word(uint32_t w, uint32_t out[4]) {
  out[0] = (w & 0x000F000Fu) | 0x64006400u;
  out[1] = (w & 0x00F000F0u) | 0x54005400u;
  const uint32_t w8 = w >> 8;
  out[2] = (w8 & 0x000F000Fu) | 0x64006400u;
  out[3] = (w8 & 0x00F000F0u) | 0x54005400u;
}

template <int G, int TC>
__global__ __launch_bounds__(kSkinnyWaves * 64) void linear_skinny_kernel(
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, const uint16_t* __restrict__ a_st,
    const float2* __restrict__ tu, int64_t m, int64_t n, int64_t k, uint16_t* __restrict__ y) {
  constexpr int WPL = G / 32;
  constexpr int HPL = G / 4;
  __shared__ floatx4_t red[kSkinnyWaves][TC][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t col = n0 + (lane & 15);
  const bool col_ok = col < n;
  const int64_t ng = k / G;
  const int64_t nzw = (ng + 7) / 8;
  const int64_t kw_row = k / 8;

  floatx4_t ytot[TC];
#pragma unroll
  for (int i = 0; i < TC; ++i) ytot[i] = floatx4_t{};

  for (int64_t j = wave; j < ng; j += kSkinnyWaves) {
    uint32_t wq[WPL];
    float dsc = 0.0f, zf = 0.0f;
    if (col_ok) {
      const uint32_t* src = qweight + col * kw_row + j * (G / 8) + WPL * c;
      if constexpr (WPL == 4) {
        uint4 v = *reinterpret_cast<const uint4*>(src);
        wq[0] = v.x; wq[1] = v.y; wq[2] = v.z; wq[3] = v.w;
      } else if constexpr (WPL == 2) {
        uint2 v = *reinterpret_cast<const uint2*>(src);
        wq[0] = v.x; wq[1] = v.y;
      } else {
        wq[0] = *src;
      }
      dsc = h2f(scales[col * ng + j]);
      zf = (float)((qzeros[col * nzw + (j >> 3)] >> (4 * (j & 7))) & 0xFu);
    } else {
#pragma unroll
      for (int i = 0; i < WPL; ++i) wq[i] = 0x00000000u;
    }
    half8_t bop[WPL];
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
      uint32_t u[4];
      unpack_word(wq[i], u);
      bop[i] = __builtin_bit_cast(half8_t, make_uint4(u[0], u[1], u[2], u[3]));
    }
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      const int64_t pair = tc * ng + j;
      const uint16_t* asrc = a_st + ((pair * 4 + c) * 16 + (lane & 15)) * HPL;
      floatx4_t cacc = floatx4_t{};
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        half8_t aop = *reinterpret_cast<const half8_t*>(asrc + 8 * i);
        cacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[i], cacc, 0, 0, 0);
      }
      // rows 4c .. 4c+3 of this chunk live in this lane's accumulator
      const float4* tup = reinterpret_cast<const float4*>(tu + pair * 16 + 4 * c);
      const float4 t01 = tup[0], t23 = tup[1];
      const float tt[4] = {t01.x, t01.z, t23.x, t23.z};
      const float uu[4] = {t01.y, t01.w, t23.y, t23.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = __builtin_fmaf(-zf, uu[i], cacc[i] - tt[i]);
        ytot[tc][i] = __builtin_fmaf(dsc, v, ytot[tc][i]);
      }
    }
  }
#pragma unroll
  for (int tc = 0; tc < TC; ++tc) red[wave][tc][lane] = ytot[tc];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      floatx4_t s = red[0][tc][lane];
#pragma unroll
      for (int wv = 1; wv < kSkinnyWaves; ++wv) s += red[wv][tc][lane];
      // lanes 0..31 hold hi rows 0..7, lanes 32..63 the matching lo rows 8..15
      floatx4_t o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(s[i], 32, 64);
      if (lane < 32 && col_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t t = (int64_t)tc * kSkinnyTok + 4 * c + i;
          if (t < m) y[t * n + col] = f2h_rn(s[i] + o[i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- prefill GEMM
constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 32;

template <int G>
__global__ __launch_bounds__(256) void linear_gemm_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ inv_s, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t a_l[kGemmBM * kGemmBK];
  __shared__ __attribute__((aligned(16))) uint16_t b_l[kGemmBN * kGemmBK];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;     // 2 x 2 waves, 64 x 64 each
  const int64_t m0 = (int64_t)blockIdx.y * kGemmBM;
  const int64_t n0 = (int64_t)blockIdx.x * kGemmBN;
  const int64_t ng = k / G;
  const int64_t nzw = (ng + 7) / 8;
  const int64_t kw_row = k / 8;

  floatx16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = floatx16_t{};

  // loader roles
  const int b_row = tid >> 1;                  // 0..127
  const int b_half = tid & 1;                  // which 16 channels of the 32
  const int64_t b_col = n0 + b_row;

  for (int64_t k0 = 0; k0 < k; k0 += kGemmBK) {
    // A tile: 128 tokens x 32 channels, 2 x 16 bytes per thread
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int idx = tid + it * 256;          // 0..511
      const int ar = idx >> 2, ac = (idx & 3) * 8;
      const int64_t t = m0 + ar;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < m) v = *reinterpret_cast<const uint4*>(x + t * k + k0 + ac);
      *reinterpret_cast<uint4*>(&a_l[ar * kGemmBK + ac]) = v;
    }
    // B tile: 128 output rows x 32 channels, dequantized to fp16
    {
      uint16_t outv[16];
      if (b_col < n) {
        const int64_t kk = k0 + b_half * 16;
        const int64_t j = kk / G;
        const uint2 wv = *reinterpret_cast<const uint2*>(qweight + b_col * kw_row + kk / 8);
        const float d = h2f(scales[b_col * ng + j]);
        const float z = (float)((qzeros[b_col * nzw + (j >> 3)] >> (4 * (j & 7))) & 0xFu);
        const uint32_t ww[2] = {wv.x, wv.y};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float q = (float)((ww[e >> 3] >> (4 * (e & 7))) & 0xFu);
          float v = (q - z) * d;                                   // exact
          if (inv_s != nullptr) v *= h2f(inv_s[kk + e]);
          outv[e] = f2h_rn(v);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) outv[e] = 0;
      }
      uint4 p0, p1;
      p0.x = outv[0] | ((uint32_t)outv[1] << 16);  p0.y = outv[2] | ((uint32_t)outv[3] << 16);
      p0.z = outv[4] | ((uint32_t)outv[5] << 16);  p0.w = outv[6] | ((uint32_t)outv[7] << 16);
      p1.x = outv[8] | ((uint32_t)outv[9] << 16);  p1.y = outv[10] | ((uint32_t)outv[11] << 16);
      p1.z = outv[12] | ((uint32_t)outv[13] << 16); p1.w = outv[14] | ((uint32_t)outv[15] << 16);
      *reinterpret_cast<uint4*>(&b_l[b_row * kGemmBK + b_half * 16]) = p0;
      *reinterpret_cast<uint4*>(&b_l[b_row * kGemmBK + b_half * 16 + 8]) = p1;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kGemmBK / 16; ++ks) {
      half8_t av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ar = wm * 64 + i * 32 + (lane & 31);
        av[i] = *reinterpret_cast<const half8_t*>(&a_l[ar * kGemmBK + ks * 16 + (lane >> 5) * 8]);
        const int br = wn * 64 + i * 32 + (lane & 31);
        bv[i] = *reinterpret_cast<const half8_t*>(&b_l[br * kGemmBK + ks * 16 + (lane >> 5) * 8]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[jj], acc[i][jj], 0, 0, 0);
    }
    __syncthreads();
  }
  // epilogue: 32x32 accumulator layout, value e of lane l is
  // row 8*(e/4) + 4*(l/32) + e%4, column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = m0 + wm * 64 + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int64_t c = n0 + wn * 64 + jj * 32 + (lane & 31);
        if (t < m && c < n) y[t * n + c] = f2h_rn(acc[i][jj][e]);
      }
}

template <int G>
static hipError_t launch_linear_g(const uint16_t* x, const uint32_t* qweight,
                                  const uint16_t* scales, const uint32_t* qzeros,
                                  const uint16_t* inv_s16, int64_t m, int64_t n, int64_t k,
                                  uint16_t* y, void* scratch, hipStream_t stream) {
  if (m > 32) {
    dim3 grid((unsigned)((n + kGemmBN - 1) / kGemmBN), (unsigned)((m + kGemmBM - 1) / kGemmBM));
    hipLaunchKernelGGL(linear_gemm_kernel<G>, grid, dim3(256), 0, stream, x, qweight, scales,
                       qzeros, inv_s16, m, n, k, y);
    return hipGetLastError();
  }
  const int64_t tc = (m + kSkinnyTok - 1) / kSkinnyTok;
  const int64_t ng = k / G;
  char* sp = static_cast<char*>(scratch);
  uint16_t* a_st = reinterpret_cast<uint16_t*>(sp);
  float2* tu = reinterpret_cast<float2*>(sp + align256((size_t)tc * (size_t)k * 16 * 2));
  const int64_t n_pairs = tc * ng;
  hipLaunchKernelGGL(linear_prep_kernel<G>, dim3((unsigned)((n_pairs + 3) / 4)), dim3(256), 0,
                     stream, x, inv_s16, m, k, n_pairs, a_st, tu);
  dim3 grid((unsigned)((n + 15) / 16));
  dim3 block(kSkinnyWaves * 64);
  switch (tc) {
    case 1:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 1>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y);
      break;
    case 2:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 2>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y);
      break;
    case 3:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 3>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y);
      break;
    default:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 4>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_linear(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                         const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m, int64_t n,
                         int64_t k, int32_t g, uint16_t* y, void* scratch, hipStream_t stream) {
  switch (g) {
    case 32:
      return launch_linear_g<32>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, scratch, stream);
    case 64:
      return launch_linear_g<64>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, scratch, stream);
    default:
      return launch_linear_g<128>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, scratch, stream);
  }
}

}  // namespace awq
