// Real quantization and nibble packing (layout v1) of scaled weights.
// Passage: CSDN page "LLM-AWQ学术影响力…", section "量化流程优化" (real 4-bit,
// group-128 quantization into a packed dump) and bjdmk.com.cn page, section
// "量化参数配置" (4 bit, group 128, zero point on).
//
// Launch: grid (n, ceil(k/2048)); one work-group of 256 threads per row chunk
// of 2048 input channels; thread t owns qweight word t of the chunk (8
// consecutive channels, one 16-byte load of W and of s).  A group of g
// channels spans g/8 adjacent lanes (4, 8 or 16), reduced with xor shuffles.
// The chunk holds a whole number of zero-point words (8g divides 2048), which
// are assembled from LDS after a barrier.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

template <int G>
__global__ __launch_bounds__(256) void pack_int4_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ s16, int64_t n, int64_t k,
    uint32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
    uint32_t* __restrict__ qzeros, int32_t* __restrict__ nonfinite) {
  constexpr int L = G / 8;                 // lanes per group
  constexpr int GROUPS_PER_CHUNK = 2048 / G;
  __shared__ uint32_t zbuf[GROUPS_PER_CHUNK];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t wi = (int64_t)blockIdx.y * 256 + tid;       // word index in the row
  const int64_t k0 = wi * 8;
  const bool valid = k0 < k;

  float v[8];
  float mx = -__builtin_inff(), mn = __builtin_inff();
  int bad = 0;
  if (valid) {
    uint4 wv = *reinterpret_cast<const uint4*>(w + row * k + k0);
    uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
    uint32_t ss[4] = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    if (s16 != nullptr) {
      uint4 sv = *reinterpret_cast<const uint4*>(s16 + k0);
      ss[0] = sv.x; ss[1] = sv.y; ss[2] = sv.z; ss[3] = sv.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t wb = (uint16_t)(ww[i >> 1] >> ((i & 1) * 16));
      uint16_t sb = (uint16_t)(ss[i >> 1] >> ((i & 1) * 16));
      // fp16 * fp16 is exact in fp32; one RNE rounding back to fp16
      uint16_t pb = f2h_rn(h2f(wb) * h2f(sb));
      bad |= f16_nonfinite(pb) ? 1 : 0;
      v[i] = h2f(pb);
      mx = __builtin_fmaxf(mx, v[i]);
      mn = __builtin_fminf(mn, v[i]);
    }
  }
#pragma unroll
  for (int off = 1; off < L; off <<= 1) {
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, off));
    mn = __builtin_fminf(mn, shfl_xor_f(mn, off));
    bad |= __shfl_xor(bad, off, 64);
  }
  const int64_t j = k0 / G;                  // group index in the row
  const int64_t ng = k / G;
  const int jl = tid / L;                    // group index in the chunk
  if (valid) {
    uint32_t word = 0;
    uint32_t zq = 0;
    uint16_t dbits = kF16NaN;
    if (!bad) {
      GroupQ gq = group_q(mx, mn);
      dbits = gq.d_bits;
      zq = (uint32_t)gq.z;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t q = (uint32_t)(code_minus_zero(v[i], gq) + gq.z);
        word |= (q & 0xFu) << (4 * i);
      }
    }
    qweight[row * (k / 8) + wi] = word;
    if ((tid % L) == 0) {
      scales[row * ng + j] = dbits;
      zbuf[jl] = zq;
      if (bad && nonfinite != nullptr) atomicAdd(nonfinite, 1);
    }
  }
  __syncthreads();
  // zero-point words of this chunk
  const int64_t j0 = (int64_t)blockIdx.y * GROUPS_PER_CHUNK;
  const int64_t groups_here = (ng - j0) < GROUPS_PER_CHUNK ? (ng - j0) : GROUPS_PER_CHUNK;
  const int64_t zwords = (groups_here + 7) / 8;
  const int64_t nzw = (ng + 7) / 8;
  if (tid < zwords) {
    uint32_t word = 0;
    for (int i = 0; i < 8; ++i) {
      int64_t jj = (int64_t)tid * 8 + i;
      if (jj < groups_here) word |= (zbuf[jj] & 0xFu) << (4 * i);
    }
    qzeros[row * nzw + j0 / 8 + tid] = word;
  }
}

// 3- and 8-bit packing: the 4-bit kernel's work split and group reduction,
// codes 0..2^BITS - 1.  8-bit: thread t writes qweight words 2t, 2t + 1 (one
// byte per code); zeros one byte per group.  3-bit: the 4 threads of a pack
// of 32 channels hold bits 24q .. 24q + 23 of its 96-bit value and threads
// q = 0, 1, 2 write its words (each taking the next thread's bits through a
// shuffle); zeros one nibble per group, as for 4 bits.
template <int G, int BITS>
__global__ __launch_bounds__(256) void pack_wbit_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ s16, int64_t n, int64_t k,
    uint32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
    uint32_t* __restrict__ qzeros, int32_t* __restrict__ nonfinite) {
  constexpr int L = G / 8;                 // lanes per group
  constexpr int GROUPS_PER_CHUNK = 2048 / G;
  constexpr float QMAX = (float)((1 << BITS) - 1);
  constexpr int ZPW = BITS == 8 ? 4 : 8;   // zero points per 32-bit word
  constexpr uint32_t ZMASK = BITS == 8 ? 0xFFu : 0xFu;
  __shared__ uint32_t zbuf[GROUPS_PER_CHUNK];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t wi = (int64_t)blockIdx.y * 256 + tid;       // 8-channel unit of the row
  const int64_t k0 = wi * 8;
  const bool valid = k0 < k;

  float v[8];
  float mx = -__builtin_inff(), mn = __builtin_inff();
  int bad = 0;
  if (valid) {
    uint4 wv = *reinterpret_cast<const uint4*>(w + row * k + k0);
    uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
    uint32_t ss[4] = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
    if (s16 != nullptr) {
      uint4 sv = *reinterpret_cast<const uint4*>(s16 + k0);
      ss[0] = sv.x; ss[1] = sv.y; ss[2] = sv.z; ss[3] = sv.w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t wb = (uint16_t)(ww[i >> 1] >> ((i & 1) * 16));
      uint16_t sb = (uint16_t)(ss[i >> 1] >> ((i & 1) * 16));
      uint16_t pb = f2h_rn(h2f(wb) * h2f(sb));
      bad |= f16_nonfinite(pb) ? 1 : 0;
      v[i] = h2f(pb);
      mx = __builtin_fmaxf(mx, v[i]);
      mn = __builtin_fminf(mn, v[i]);
    }
  }
#pragma unroll
  for (int off = 1; off < L; off <<= 1) {
    mx = __builtin_fmaxf(mx, shfl_xor_f(mx, off));
    mn = __builtin_fminf(mn, shfl_xor_f(mn, off));
    bad |= __shfl_xor(bad, off, 64);
  }
  const int64_t j = k0 / G;
  const int64_t ng = k / G;
  const int jl = tid / L;
  uint32_t w8[2] = {0u, 0u}, c24 = 0u, zq = 0u;
  uint16_t dbits = kF16NaN;
  if (valid && !bad) {
    const GroupQ gq = group_q(mx, mn, QMAX);
    dbits = gq.d_bits;
    zq = (uint32_t)gq.z;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t q = (uint32_t)(code_minus_zero(v[i], gq) + gq.z);
      if constexpr (BITS == 8) w8[i >> 2] |= (q & 0xFFu) << (8 * (i & 3));
      else c24 |= (q & 7u) << (3 * i);
    }
  }
  if (valid) {
    if constexpr (BITS == 8) {
      qweight[row * (k / 4) + 2 * wi] = w8[0];
      qweight[row * (k / 4) + 2 * wi + 1] = w8[1];
    }
    if ((tid % L) == 0) {
      scales[row * ng + j] = dbits;
      zbuf[jl] = zq;
      if (bad && nonfinite != nullptr) atomicAdd(nonfinite, 1);
    }
  }
  if constexpr (BITS == 3) {
    const uint32_t nx = __shfl_down(c24, 1, 64);       // the next thread's 24 bits
    const int q = tid & 3;
    if (valid && q < 3) {
      const uint32_t word = q == 0 ? (c24 | (nx << 24)) : q == 1 ? ((c24 >> 8) | (nx << 16))
                                                                 : ((c24 >> 16) | (nx << 8));
      qweight[row * (3 * k / 32) + 3 * (wi >> 2) + q] = word;
    }
  }
  __syncthreads();
  const int64_t j0 = (int64_t)blockIdx.y * GROUPS_PER_CHUNK;
  const int64_t groups_here = (ng - j0) < GROUPS_PER_CHUNK ? (ng - j0) : GROUPS_PER_CHUNK;
  const int64_t zwords = (groups_here + ZPW - 1) / ZPW;
  const int64_t nzw = (ng + ZPW - 1) / ZPW;
  if (tid < zwords) {
    uint32_t word = 0;
    for (int i = 0; i < ZPW; ++i) {
      const int64_t jj = (int64_t)tid * ZPW + i;
      if (jj < groups_here) word |= (zbuf[jj] & ZMASK) << ((32 / ZPW) * i);
    }
    qzeros[row * nzw + j0 / ZPW + tid] = word;
  }
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

hipError_t launch_pack_wbit(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                            int32_t g, int32_t w_bit, uint32_t* qweight, uint16_t* scales,
                            uint32_t* qzeros, int32_t* nonfinite, hipStream_t stream) {
  if (w_bit == 4) return launch_pack(w, s16, n, k, g, qweight, scales, qzeros, nonfinite, stream);
  if (nonfinite != nullptr) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, stream, nonfinite);
  const dim3 grid((unsigned)n, (unsigned)((k + 2047) / 2048));
#define AWQ_PACKW(GG, BB)                                                                      \
  hipLaunchKernelGGL((pack_wbit_kernel<GG, BB>), grid, dim3(256), 0, stream, w, s16, n, k, qweight, \
                     scales, qzeros, nonfinite)
  if (w_bit == 8) {
    if (g == 32) AWQ_PACKW(32, 8); else if (g == 64) AWQ_PACKW(64, 8); else AWQ_PACKW(128, 8);
  } else {
    if (g == 32) AWQ_PACKW(32, 3); else if (g == 64) AWQ_PACKW(64, 3); else AWQ_PACKW(128, 3);
  }
#undef AWQ_PACKW
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                       int32_t g, uint32_t* qweight, uint16_t* scales, uint32_t* qzeros,
                       int32_t* nonfinite, hipStream_t stream) {
  if (nonfinite != nullptr) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, stream, nonfinite);
  dim3 grid((unsigned)n, (unsigned)((k + 2047) / 2048));
  switch (g) {
    case 32:
      hipLaunchKernelGGL(pack_int4_kernel<32>, grid, dim3(256), 0, stream, w, s16, n, k, qweight,
                         scales, qzeros, nonfinite);
      break;
    case 64:
      hipLaunchKernelGGL(pack_int4_kernel<64>, grid, dim3(256), 0, stream, w, s16, n, k, qweight,
                         scales, qzeros, nonfinite);
      break;
    default:
      hipLaunchKernelGGL(pack_int4_kernel<128>, grid, dim3(256), 0, stream, w, s16, n, k, qweight,
                         scales, qzeros, nonfinite);
      break;
  }
  return hipGetLastError();
}

// fold of 1/s into the per-channel weight of the operation that produces a
// linear's input: out_k = fp16_rn(v_k / s_k), the float64 quotient of two
// fp16 values rounded once (a float64 quotient of 11-bit significands cannot
// land on an fp16 rounding midpoint unless the exact quotient does, so the
// result is the correctly rounded one)
__global__ __launch_bounds__(256) void fold_inv_scale_kernel(const uint16_t* __restrict__ v,
                                                             const uint16_t* __restrict__ s16,
                                                             int64_t k, uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < k; i += (int64_t)gridDim.x * 256)
    out[i] = f64_to_f16_rn((double)h2f(v[i]) / (double)h2f(s16[i]));
}

// the same fold into the output rows of a linear [n][k] that produces the
// input: out_jc = fp16_rn(w_jc / s_j)
__global__ __launch_bounds__(256) void fold_inv_scale_rows_kernel(const uint16_t* __restrict__ w,
                                                                  const uint16_t* __restrict__ s16,
                                                                  int64_t n, int64_t k,
                                                                  uint16_t* __restrict__ out) {
  const int64_t total = n * k;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
    out[e] = f64_to_f16_rn((double)h2f(w[e]) / (double)h2f(s16[e / k]));
}

hipError_t launch_fold_inv_scale_rows(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                                      uint16_t* out, hipStream_t stream) {
  const int64_t total = n * k;
  const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
  hipLaunchKernelGGL(fold_inv_scale_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, s16, n,
                     k, out);
  return hipGetLastError();
}

hipError_t launch_fold_inv_scale(const uint16_t* v, const uint16_t* s16, int64_t k, uint16_t* out,
                                 hipStream_t stream) {
  const int64_t blocks = (k + 255) / 256 < 1024 ? (k + 255) / 256 : 1024;
  hipLaunchKernelGGL(fold_inv_scale_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, v, s16, k,
                     out);
  return hipGetLastError();
}

}  // namespace awq
