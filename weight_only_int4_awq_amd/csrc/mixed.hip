// Mixed-precision baseline: a small share of input channels (those with the
// largest mean |x|) keeps its fp16 weights, the rest is quantized with plain
// round-to-nearest.  jsqmd.com page, section 二.1 (1): 0.1 - 1 % of the
// weights, on the channels with large activations, decide the accuracy and
// suffer most from direct quantization; section 五.1: protection ratio 0.1 - 1
// % by default; CSDN page: mixed-precision optimisation named beside the
// scaling.  The baseline the search is measured against.
//
//  * salient_select_kernel: the indices (ascending) of the `count` largest
//    a_k, ties to the lower index, NaN above +inf: one work-group, a radix
//    select over an order-preserving 64-bit key (8 passes of 8 bits, LDS
//    histograms), then an ordered compaction.
//  * channel_keep_kernel / channel_zero_kernel: the fp16 keep mask (1.0, and
//    0.0 on the protected channels).  As inv_s16 of the 4-bit linear it removes
//    the protected channels from the quantized product.
//  * gather_channels_kernel: the protected columns of W, channel-major
//    [count][n] fp16 (a wave's 64 columns of one channel are contiguous).
//  * mask_rows_kernel: activations with the protected channels set to zero
//    (the mixed loss is the s = 1 search loss on them).
//  * salient_add_kernel: y = fp16_rn(y + sum_j x[:, idx_j] W_S[j, :]) after the
//    quantized product, fp32 accumulation (eight interleaved slices of j,
//    added in slice order).
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

// order-preserving key of a double: equal values (+0 and -0 included) get
// equal keys, NaN the largest key
__device__ __forceinline__ uint64_t rank_key(double a) {
  if (a != a) return ~0ull;
  const uint64_t b = __builtin_bit_cast(uint64_t, a == 0.0 ? 0.0 : a);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

constexpr int kSelThreads = 1024;

// inclusive prefix sum over the work-group of one int per thread (wave scans
// in registers, wave totals through LDS); returns the thread's inclusive sum
// and the group total in *total
__device__ __forceinline__ int block_scan_incl(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int s = wsum[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

__global__ __launch_bounds__(kSelThreads) void salient_select_kernel(
    const double* __restrict__ a, int64_t k, int32_t count, int32_t* __restrict__ idx) {
  __shared__ int hist[256];
  __shared__ int wsum[kSelThreads / 64];
  __shared__ uint64_t s_prefix;
  __shared__ int s_need;
  const int tid = threadIdx.x;
  // ---- radix select: the count-th largest key T and how many keys == T to take
  uint64_t prefix = 0, mask = 0;
  int need = count;
  for (int d = 7; d >= 0; --d) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t i = tid; i < k; i += kSelThreads) {
      const uint64_t key = rank_key(a[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(int)((key >> (8 * d)) & 0xFF)], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= need) break;
        above += hist[b];
      }
      s_prefix = prefix | ((uint64_t)b << (8 * d));
      s_need = need - above;
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    mask |= 0xFFull << (8 * d);
    __syncthreads();
  }
  // ---- ordered compaction: keys > T, and the first `need` keys == T by index
  int eq_base = 0, out_base = 0;
  for (int64_t c0 = 0; c0 < k; c0 += kSelThreads) {
    const int64_t i = c0 + tid;
    const uint64_t key = i < k ? rank_key(a[i]) : 0ull;
    const int eq = (i < k && key == prefix) ? 1 : 0;
    int eq_total = 0;
    const int eq_incl = block_scan_incl(eq, wsum, &eq_total);
    const int take = (i < k && (key > prefix || (eq && eq_base + eq_incl - 1 < need))) ? 1 : 0;
    int take_total = 0;
    const int take_incl = block_scan_incl(take, wsum, &take_total);
    if (take) idx[out_base + take_incl - 1] = (int32_t)i;
    eq_base += eq_total;
    out_base += take_total;
  }
}

__global__ __launch_bounds__(256) void channel_keep_kernel(int64_t k, uint16_t* __restrict__ keep) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < k; i += (int64_t)gridDim.x * 256)
    keep[i] = 0x3C00u;                                   // 1.0
}

__global__ __launch_bounds__(256) void channel_zero_kernel(const int32_t* __restrict__ idx,
                                                           int32_t count, uint16_t* __restrict__ keep) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j < count) keep[idx[j]] = 0u;
}

__global__ __launch_bounds__(256) void gather_channels_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, const int32_t* __restrict__ idx,
    int32_t count, uint16_t* __restrict__ w_s) {
  const int64_t total = n * count;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e / n);
    const int64_t row = e - (int64_t)j * n;
    w_s[e] = w[row * k + idx[j]];
  }
}

// x with the channels whose keep entry is 0 set to +0 (a select, not a
// product, so non-finite values in those channels become 0 too)
__global__ __launch_bounds__(256) void mask_rows_kernel(const uint16_t* __restrict__ x,
                                                        const uint16_t* __restrict__ keep, int64_t m,
                                                        int64_t k, uint16_t* __restrict__ out) {
  const int64_t total = m * k;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256)
    out[e] = keep[e % k] == 0 ? (uint16_t)0 : x[e];
}

// Tiles of 64 columns x kAddTok tokens, 512 threads: thread (column c =
// tid % 64, slice q = tid / 64) sums channels j = q, q + 8, ... of the
// protected set (coalesced loads of w_s[j][col], 8 in flight); the eight
// slice sums meet in LDS and slice 0 adds them in slice order.  The tile's protected activations
// are staged in LDS as float [kAddTok][count].
constexpr int kAddTok = 16;
constexpr int kAddSlices = 8;

__global__ __launch_bounds__(64 * kAddSlices) void salient_add_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ idx, int32_t count,
    const uint16_t* __restrict__ w_s, int64_t m, int64_t n, int64_t k, uint16_t* __restrict__ y) {
  extern __shared__ float xs[];                          // [kAddTok][count]
  __shared__ float part[kAddSlices - 1][kAddTok][64];
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 64 + c;
  const int64_t t0 = (int64_t)blockIdx.y * kAddTok;
  const int tt_n = (m - t0) < kAddTok ? (int)(m - t0) : kAddTok;
  for (int e = threadIdx.x; e < tt_n * count; e += 64 * kAddSlices) {
    const int tt = e / count, j = e - tt * count;
    xs[e] = h2f(x[(t0 + tt) * k + idx[j]]);
  }
  __syncthreads();
  const int64_t cc = col < n ? col : n - 1;
  float acc[kAddTok];
#pragma unroll
  for (int tt = 0; tt < kAddTok; ++tt) acc[tt] = 0.0f;
#pragma unroll 8
  for (int j = q; j < count; j += kAddSlices) {
    const float wv = h2f(w_s[(int64_t)j * n + cc]);
#pragma unroll
    for (int tt = 0; tt < kAddTok; ++tt)
      if (tt < tt_n) acc[tt] = __builtin_fmaf(xs[tt * count + j], wv, acc[tt]);
  }
  if (q > 0) {
#pragma unroll
    for (int tt = 0; tt < kAddTok; ++tt) part[q - 1][tt][c] = acc[tt];
  }
  __syncthreads();
  if (q == 0 && col < n) {
#pragma unroll
    for (int tt = 0; tt < kAddTok; ++tt) {
      if (tt < tt_n) {
        float v = acc[tt];
#pragma unroll
        for (int qq = 0; qq < kAddSlices - 1; ++qq) v += part[qq][tt][c];
        uint16_t* yp = y + (t0 + tt) * n + col;
        *yp = f2h_rn(h2f(*yp) + v);
      }
    }
  }
}

__global__ __launch_bounds__(256) void fill_one_f64_kernel(int64_t k, double* __restrict__ a) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < k; i += (int64_t)gridDim.x * 256)
    a[i] = 1.0;
}

hipError_t launch_salient_select(const double* a, int64_t k, int32_t count, int32_t* idx,
                                 hipStream_t stream) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(salient_select_kernel, dim3(1), dim3(kSelThreads), 0, stream, a, k, count, idx);
  return hipGetLastError();
}

hipError_t launch_channel_mask(const int32_t* idx, int32_t count, int64_t k, uint16_t* keep,
                               hipStream_t stream) {
  const int64_t blocks = (k + 255) / 256 < 1024 ? (k + 255) / 256 : 1024;
  hipLaunchKernelGGL(channel_keep_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, keep);
  if (count > 0)
    hipLaunchKernelGGL(channel_zero_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream,
                       idx, count, keep);
  return hipGetLastError();
}

hipError_t launch_gather_channels(const uint16_t* w, int64_t n, int64_t k, const int32_t* idx,
                                  int32_t count, uint16_t* w_s, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const int64_t total = n * count;
  const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
  hipLaunchKernelGGL(gather_channels_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, n, k, idx,
                     count, w_s);
  return hipGetLastError();
}

hipError_t launch_mask_rows(const uint16_t* x, const uint16_t* keep, int64_t m, int64_t k,
                            uint16_t* out, hipStream_t stream) {
  const int64_t total = m * k;
  const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
  hipLaunchKernelGGL(mask_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, keep, m, k, out);
  return hipGetLastError();
}

hipError_t launch_salient_add(const uint16_t* x, const int32_t* idx, int32_t count,
                              const uint16_t* w_s, int64_t m, int64_t n, int64_t k, uint16_t* y,
                              hipStream_t stream) {
  if (count == 0 || m == 0) return hipSuccess;
  const int64_t ty = (m + kAddTok - 1) / kAddTok;
  const dim3 grid((unsigned)((n + 63) / 64), (unsigned)ty);
  const size_t lds = (size_t)kAddTok * count * 4;
  const size_t lds_static = (size_t)(kAddSlices - 1) * kAddTok * 64 * 4;
  if (lds + lds_static > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&salient_add_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(salient_add_kernel, grid, dim3(64 * kAddSlices), lds, stream, x, idx, count, w_s, m, n,
                     k, y);
  return hipGetLastError();
}

// workspace of the mixed loss: masked activations | a = 1 | s16, inv_s16 |
// best index | the search's own workspace
struct MixedLossLayout {
  size_t off_x, off_a, off_s, off_inv, off_best, off_search, total;
};
static size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }
static MixedLossLayout mixed_loss_layout(int64_t n, int64_t k, int64_t m, int32_t g) {
  MixedLossLayout L;
  size_t o = 0;
  L.off_x = o;      o += al256((size_t)m * k * 2);
  L.off_a = o;      o += al256((size_t)k * 8);
  L.off_s = o;      o += al256((size_t)k * 2);
  L.off_inv = o;    o += al256((size_t)k * 2);
  L.off_best = o;   o += 256;
  L.off_search = o; o += search_layout(n, k, m, g, 1).total;
  L.total = o;
  return L;
}

size_t mixed_loss_workspace_bytes(int64_t n, int64_t k, int64_t m, int32_t g) {
  return mixed_loss_layout(n, k, m, g).total;
}

// L_mixed = the s = 1 (alpha = 0) search loss of W on x with the protected
// channels zeroed: removing those channels' activations removes exactly the
// error columns that the fp16 weights would have fixed
hipError_t launch_mixed_loss(const uint16_t* w, const uint16_t* x, const uint16_t* keep, int64_t n,
                             int64_t k, int64_t m, int32_t g, double* loss, void* workspace,
                             hipStream_t stream) {
  const MixedLossLayout L = mixed_loss_layout(n, k, m, g);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xm = reinterpret_cast<uint16_t*>(ws + L.off_x);
  double* a = reinterpret_cast<double*>(ws + L.off_a);
  hipError_t e = launch_mask_rows(x, keep, m, k, xm, stream);
  if (e != hipSuccess) return e;
  const int64_t blocks = (k + 255) / 256 < 1024 ? (k + 255) / 256 : 1024;
  hipLaunchKernelGGL(fill_one_f64_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_search(w, xm, a, n, k, m, g, 1, 4, reinterpret_cast<int32_t*>(ws + L.off_best),
                       reinterpret_cast<uint16_t*>(ws + L.off_s), reinterpret_cast<uint16_t*>(ws + L.off_inv),
                       loss, ws + L.off_search, stream);
}

}  // namespace awq
