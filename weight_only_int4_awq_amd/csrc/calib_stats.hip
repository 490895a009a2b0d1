// Per-input-channel mean absolute activation (the activation statistic of
// activation-aware weight quantization: jsqmd.com page, section 二.1 (2)).
//
// Every |fp16| times 2^24 is an integer below 2^40, so the kernel sums
// integers: the column sums are exact and independent of the order.  With
// m <= 8192 the sum stays below 2^53, so (double)S * 2^-24 is exact and the
// final division by m is the only rounding.
//
// Launch: one work-group of 256 threads per 64 columns; thread (r, c) with
// c = tid % 8 owns 8 consecutive columns (one 16-byte load per row) and sums
// rows r, r + 32, ...; the 32 row slices are combined in LDS in a fixed order.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

__device__ __forceinline__ uint64_t abs_f16_as_int(uint32_t h) {
  uint32_t e = (h >> 10) & 0x1Fu;
  uint32_t m = h & 0x3FFu;
  // normal: (1.m) * 2^(e-15) * 2^24 = (m | 0x400) << (e - 1); subnormal: m
  return e == 0 ? (uint64_t)m : ((uint64_t)(m | 0x400u) << (e - 1));
}

__global__ __launch_bounds__(256) void calib_stats_kernel(
    const uint16_t* __restrict__ x, int64_t m, int64_t k, double* __restrict__ out) {
  __shared__ uint64_t part[32][64];
  __shared__ uint32_t flags[32][64];
  const int tid = threadIdx.x;
  const int c = tid & 7;
  const int r = tid >> 3;
  const int64_t col0 = (int64_t)blockIdx.x * 64 + c * 8;
  uint64_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint32_t fl[8] = {0, 0, 0, 0, 0, 0, 0, 0};   // bit0: inf seen, bit1: NaN seen
  if (col0 < k) {
    for (int64_t row = r; row < m; row += 32) {
      uint4 v = *reinterpret_cast<const uint4*>(x + row * k + col0);
      uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t h = (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
        if ((h & 0x7C00u) == 0x7C00u) {
          fl[i] |= (h & 0x3FFu) ? 2u : 1u;
        } else {
          acc[i] += abs_f16_as_int(h);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    part[r][c * 8 + i] = acc[i];
    flags[r][c * 8 + i] = fl[i];
  }
  __syncthreads();
  if (tid < 64) {
    int64_t col = (int64_t)blockIdx.x * 64 + tid;
    if (col < k) {
      uint64_t s = 0;
      uint32_t f = 0;
      for (int i = 0; i < 32; ++i) {
        s += part[i][tid];
        f |= flags[i][tid];
      }
      double a;
      if (f & 2u) {
        a = __builtin_nan("");
      } else if (f & 1u) {
        a = __builtin_inf();
      } else {
        a = ((double)s * 0x1p-24) / (double)m;
      }
      out[col] = a;
    }
  }
}

hipError_t launch_calib_stats(const uint16_t* x, int64_t m, int64_t k, double* out,
                              hipStream_t stream) {
  dim3 grid((unsigned)((k + 63) / 64));
  hipLaunchKernelGGL(calib_stats_kernel, grid, dim3(256), 0, stream, x, m, k, out);
  return hipGetLastError();
}

}  // namespace awq
