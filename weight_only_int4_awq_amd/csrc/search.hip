// Grid search of the AWQ channel scale s = a^alpha (jsqmd.com page, section
// 二.1 (3): scale the salient input channels of W by s, divide the activation
// by s, choose s to minimise the output error of the quantized layer).
//
// Three kernels, all on the caller's stream:
//  1. search_prep: s_ik = fp16_rn(max(a_k^alpha_i, 2^-14)) and 1/s_ik (fp32)
//     for every grid point and channel (float64 pow, single fp16 rounding).
//  2. search_blockscale: a power-of-two factor per 32-row block that keeps the
//     fp16 split of the weight error in the normal range (see below).
//  3. search_loss: one work-group per (32-row block, alpha).  For every group
//     of g channels it fake-quantizes the 32 x g block of W' = fp16(W s_i)
//     (exact per-element codes, see awq_common.h), forms the weight error
//     dW = ((q - z) D - W s) / s in fp32 (no cancellation: both terms of the
//     difference are exact), splits it into fp16 hi + lo, stages both
//     in LDS in the MFMA A-operand layout and multiplies them with the
//     calibration tokens (B operand, straight from global memory) into fp32
//     accumulators E = dW X^T.  After the last group it squares E in float64
//     and writes the block's partial loss.
//  4. search_select: sums the partials of each alpha in block order (fixed),
//     takes the first minimum over finite losses and writes s16 and
//     inv_s16 = fp16_rn(1/s16) (float64 quotient).
#include <math.h>

#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kSearchRows = 32;        // rows of W per work-group
constexpr int kSearchTokPass = 512;    // tokens per pass (4 waves x 4 tiles x 32)

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

SearchLayout search_layout(int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid) {
  (void)m; (void)g;
  SearchLayout L;
  L.n_blocks = (n + kSearchRows - 1) / kSearchRows;
  size_t off = 0;
  L.off_s16 = off;  off = align256(off + (size_t)n_grid * (size_t)k * 2);
  L.off_rs = off;   off = align256(off + (size_t)n_grid * (size_t)k * 4);
  L.off_part = off; off = align256(off + (size_t)n_grid * (size_t)L.n_blocks * 8);
  L.off_cblk = off; off = align256(off + (size_t)L.n_blocks * 4);
  L.total = off;
  return L;
}

__global__ __launch_bounds__(256) void search_prep_kernel(const double* __restrict__ a,
                                                          int64_t k, int32_t n_grid,
                                                          uint16_t* __restrict__ s16,
                                                          float* __restrict__ rs) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y;
  if (col >= k) return;
  const double alpha = (double)i / (double)n_grid;
  double p;
  if (i == 0) {
    p = 1.0;                                  // x^0 = 1 for every x
  } else {
    p = pow(a[col], alpha);
  }
  if (!(p != p)) p = p > 0x1p-14 ? p : 0x1p-14;   // lower clamp; NaN stays NaN
  const uint16_t sb = f64_to_f16_rn(p);
  s16[(int64_t)i * k + col] = sb;
  rs[(int64_t)i * k + col] = 1.0f / h2f(sb);
}

// Per 32-row block: a power-of-two factor c for the weight error dW.  Every
// |dW_nk| is at most about 1.03 |W_nk| (an element on quantization level 0 has
// dW = -W; on any other level |W'| >= D/2, so |deq - W'| <= 0.51 D <= 1.02 |W'|).
// With max|W| < 2^e the factor c = 2^(14 - e) keeps c |dW| below 17000, inside
// fp16, while lifting small errors far above the fp16 subnormal range, so the
// fp16 hi + lo split of c dW keeps about 22 significant bits.
__global__ __launch_bounds__(256) void search_blockscale_kernel(const uint16_t* __restrict__ w,
                                                                int64_t n, int64_t k,
                                                                float* __restrict__ cblk) {
  __shared__ uint32_t red[4];
  const int64_t rb = blockIdx.x;
  const int64_t r0 = rb * kSearchRows;
  const int64_t rows = (n - r0) < kSearchRows ? (n - r0) : kSearchRows;
  const int64_t words = rows * k / 8;          // 8 halves per 16-byte load
  const uint4* base = reinterpret_cast<const uint4*>(w + r0 * k);
  uint32_t mx = 0;
  for (int64_t i = threadIdx.x; i < words; i += 256) {
    uint4 v = base[i];
    uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      uint32_t b = (ww[h >> 1] >> ((h & 1) * 16)) & 0x7FFFu;
      if (b < 0x7C00u && b > mx) mx = b;         // |fp16| bits order like the values
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(mx, off, 64);
    mx = o > mx ? o : mx;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int i = 1; i < 4; ++i) m = red[i] > m ? red[i] : m;
    float c = 1.0f;
    if (m != 0) {
      int e;
      (void)__builtin_frexpf(h2f((uint16_t)m), &e);   // max|W| < 2^e
      c = __builtin_ldexpf(1.0f, 14 - e);
    }
    cblk[rb] = c;
  }
}

template <int G>
__global__ __launch_bounds__(256) void search_loss_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ x, int64_t n, int64_t k,
    int64_t m, int32_t n_grid, int64_t n_blocks, const uint16_t* __restrict__ s16_all,
    const float* __restrict__ rs_all, const float* __restrict__ cblk, double* __restrict__ part) {
  constexpr int EPT = G / 8;          // elements of one row-group per thread
  constexpr int KSTEPS = G / 16;      // MFMA k-steps per group
  __shared__ __attribute__((aligned(16))) uint16_t a_hi[KSTEPS * 32 * 16];
  __shared__ __attribute__((aligned(16))) uint16_t a_lo[KSTEPS * 32 * 16];
  __shared__ double red[4];

  // XCD-aware order: consecutive logical ids (the alphas of one row block)
  // land on the same XCD, so they share W through that XCD's L2.
  const int64_t total = n_blocks * (int64_t)n_grid;
  const int64_t p = blockIdx.x;
  const int64_t per = total / 8, rem = total % 8;
  const int64_t xcd = p % 8, slot = p / 8;
  const int64_t logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int ai = (int)(logical % n_grid);
  const int64_t rb = logical / n_grid;

  const uint16_t* __restrict__ s16 = s16_all + (int64_t)ai * k;
  const float* __restrict__ rs = rs_all + (int64_t)ai * k;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = tid >> 3;             // row of the block this thread quantizes
  const int sub = tid & 7;            // which EPT-slice of the group
  const int64_t row = rb * kSearchRows + r;
  const bool row_ok = row < n;
  const float cscale = cblk[rb];

  double loss = 0.0;
  for (int64_t t0 = 0; t0 < m; t0 += kSearchTokPass) {
    const int64_t tpass = (m - t0) < kSearchTokPass ? (m - t0) : kSearchTokPass;
    const int ntiles = (int)((tpass + 31) / 32);
    floatx16_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = floatx16_t{};

    for (int64_t j = 0; j < k / G; ++j) {
      // ---- stage 1: fake-quantize this thread's EPT elements, stage dW in LDS
      const int64_t kb = j * G + sub * EPT;
      float wsx[EPT], wp[EPT], rsv[EPT];
      float mx = -__builtin_inff(), mn = __builtin_inff();
      int bad = 0;
      if (row_ok) {
#pragma unroll
        for (int e = 0; e < EPT; e += 4) {
          uint2 wr = *reinterpret_cast<const uint2*>(w + row * k + kb + e);
          uint2 sr = *reinterpret_cast<const uint2*>(s16 + kb + e);
          float4 rr = *reinterpret_cast<const float4*>(rs + kb + e);
          uint32_t ww[2] = {wr.x, wr.y};
          uint32_t ss[2] = {sr.x, sr.y};
          float rq[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint16_t wb = (uint16_t)(ww[i >> 1] >> ((i & 1) * 16));
            uint16_t sb = (uint16_t)(ss[i >> 1] >> ((i & 1) * 16));
            const float prod = h2f(wb) * h2f(sb);      // W s, exact in fp32
            uint16_t pb = f2h_rn(prod);
            bad |= f16_nonfinite(pb) ? 1 : 0;
            wsx[e + i] = prod;
            wp[e + i] = h2f(pb);
            rsv[e + i] = rq[i];
            mx = __builtin_fmaxf(mx, wp[e + i]);
            mn = __builtin_fminf(mn, wp[e + i]);
          }
        }
      }
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        mx = __builtin_fmaxf(mx, shfl_xor_f(mx, off));
        mn = __builtin_fminf(mn, shfl_xor_f(mn, off));
        bad |= __shfl_xor(bad, off, 64);
      }
      uint16_t hi[EPT], lo[EPT];
      if (row_ok) {
        GroupQ gq = group_q(mx, mn);
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          // dW = (deq - W s) / s: deq and W s are exact, so the small difference is
          // rounded once, then scaled by the block factor c (a power of two)
          float deq = code_minus_zero(wp[e], gq) * gq.d;          // exact
          float dw = bad ? __builtin_nanf("") : (deq - wsx[e]) * (rsv[e] * cscale);
          uint16_t h = f2h_rn(dw);
          hi[e] = h;
          lo[e] = f2h_rn(dw - h2f(h));
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) { hi[e] = 0; lo[e] = 0; }
      }
      {
        const int kloc = sub * EPT;
        const int s = kloc / 16, kk = kloc % 16;
        const int base = (s * 32 + r) * 16 + kk;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          a_hi[base + e] = hi[e];
          a_lo[base + e] = lo[e];
        }
      }
      __syncthreads();
      // ---- stage 2: E += dW_hi X^T + dW_lo X^T on the matrix cores
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int aoff = (s * 32 + (lane & 31)) * 16 + (lane >> 5) * 8;
        half8_t ah = *reinterpret_cast<const half8_t*>(&a_hi[aoff]);
        half8_t al = *reinterpret_cast<const half8_t*>(&a_lo[aoff]);
        const int64_t kx = j * G + s * 16 + (lane >> 5) * 8;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const int tile = wave + 4 * ti;
          if (tile < ntiles) {
            const int64_t tok = t0 + tile * 32 + (lane & 31);
            half8_t b = half8_t{};
            if (tok < m) b = *reinterpret_cast<const half8_t*>(x + tok * k + kx);
            acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, b, acc[ti], 0, 0, 0);
            acc[ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, b, acc[ti], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }
    // ---- square and reduce (float64, fixed order)
    double sq = 0.0;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        double e = (double)acc[ti][i];
        sq += e * e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sq += shfl_xor_d(sq, off);
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    loss += ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
  }
  const double inv_c = 1.0 / (double)cscale;       // exact: c is a power of two
  if (tid == 0) part[(int64_t)ai * n_blocks + rb] = loss * inv_c * inv_c;
}

__global__ __launch_bounds__(256) void search_select_kernel(
    const double* __restrict__ part, int64_t n_blocks, int32_t n_grid, int64_t k,
    const uint16_t* __restrict__ s16_all, int32_t* __restrict__ best_idx,
    uint16_t* __restrict__ s16, uint16_t* __restrict__ inv_s16, double* __restrict__ losses) {
  __shared__ double L[64];
  __shared__ int best_s;
  const int tid = threadIdx.x;
  if (tid < n_grid) {
    double s = 0.0;
    for (int64_t b = 0; b < n_blocks; ++b) s += part[(int64_t)tid * n_blocks + b];
    L[tid] = s;
    if (losses != nullptr) losses[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    int best = -1;
    double bv = 0.0;
    for (int i = 0; i < n_grid; ++i) {
      double v = L[i];
      if (!__builtin_isfinite(v)) continue;
      if (best < 0 || v < bv) { best = i; bv = v; }
    }
    best_s = best;
    *best_idx = best;
  }
  __syncthreads();
  const int best = best_s;
  for (int64_t col = tid; col < k; col += 256) {
    uint16_t sb = best >= 0 ? s16_all[(int64_t)best * k + col] : kF16One;
    s16[col] = sb;
    inv_s16[col] = f64_to_f16_rn(1.0 / (double)h2f(sb));
  }
}

hipError_t launch_search(const uint16_t* w, const uint16_t* x, const double* mean_abs,
                         int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid,
                         int32_t* best_idx, uint16_t* s16, uint16_t* inv_s16,
                         double* losses, void* workspace, hipStream_t stream) {
  const SearchLayout L = search_layout(n, k, m, g, n_grid);
  char* ws = static_cast<char*>(workspace);
  uint16_t* s16_all = reinterpret_cast<uint16_t*>(ws + L.off_s16);
  float* rs_all = reinterpret_cast<float*>(ws + L.off_rs);
  double* part = reinterpret_cast<double*>(ws + L.off_part);
  float* cblk = reinterpret_cast<float*>(ws + L.off_cblk);

  hipLaunchKernelGGL(search_prep_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)n_grid),
                     dim3(256), 0, stream, mean_abs, k, n_grid, s16_all, rs_all);
  hipLaunchKernelGGL(search_blockscale_kernel, dim3((unsigned)L.n_blocks), dim3(256), 0, stream, w,
                     n, k, cblk);
  const unsigned nwg = (unsigned)(L.n_blocks * n_grid);
  switch (g) {
    case 32:
      hipLaunchKernelGGL(search_loss_kernel<32>, dim3(nwg), dim3(256), 0, stream, w, x, n, k, m,
                         n_grid, L.n_blocks, s16_all, rs_all, cblk, part);
      break;
    case 64:
      hipLaunchKernelGGL(search_loss_kernel<64>, dim3(nwg), dim3(256), 0, stream, w, x, n, k, m,
                         n_grid, L.n_blocks, s16_all, rs_all, cblk, part);
      break;
    default:
      hipLaunchKernelGGL(search_loss_kernel<128>, dim3(nwg), dim3(256), 0, stream, w, x, n, k, m,
                         n_grid, L.n_blocks, s16_all, rs_all, cblk, part);
      break;
  }
  hipLaunchKernelGGL(search_select_kernel, dim3(1), dim3(256), 0, stream, part, L.n_blocks,
                     n_grid, k, s16_all, best_idx, s16, inv_s16, losses);
  return hipGetLastError();
}

}  // namespace awq
