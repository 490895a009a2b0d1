// Linear for 3- and 8-bit group-quantized weights: y = x_tilde W_deq^T with
// the packed layouts of awq_pack_wbit.  csdn.net page, section "量化流程优化":
// the bit width is a parameter of the quantizer; jsqmd.com page, section 五:
// 3- and 4-bit weights; bjdmk.com.cn page: INT4 and INT8 weight formats;
// zeeklog.com page: INT3 weights.
//
// Layouts (codes q in 0 .. 2^b - 1, zero points z in the same range):
//  * 8 bits: qweight[n][k/4], code k at byte k % 4 of word k/4;
//    qzeros[n][ceil(ng/4)], zero j at byte j % 4 of word j/4.
//  * 3 bits: qweight[n][3k/32]; the 32 codes 32p .. 32p + 31 of a row fill
//    the 96-bit little-endian value of words 3p .. 3p + 2, code 32p + i at
//    bits 3i .. 3i + 2 (codes 10 and 21 straddle a word boundary);
//    qzeros[n][ceil(ng/8)], zero j at bits 4(j % 8) of word j/8.
// Scales are fp16 [n][ng] as for 4 bits.
//
// One kernel serves every m.  These widths have no per-token tuning: the
// 4-bit path is the product path and the one tuned to the roofline.
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

// linear_wbit_kernel<G, BITS>: one work-group of 4 waves per 16-column block
// and 16-token chunk (grid y strides over the chunks); the waves split K by
// groups.  For group j, lane (r = lane % 16, c = lane / 16) takes the G/4
// consecutive channels jG + cG/4 .. of column n0 + r (at 3 bits and g = 128
// exactly one 3-word pack) and the same channels of token t0 + r.  Sub-step
// i < G/32 is one v_mfma_f32_16x16x32_f16 whose k-block of lane c is its i-th
// run of 8 channels; A and B follow the same order, so every channel of the
// group meets its weight once.  Weights become fp16_rn((q - z) D): the codes
// sit in the mantissa of 1024, 1024 + z is subtracted exactly, and the product
// with D rounds once.  Activations become fp16_rn(x inv_s).  The waves' fp32
// partial tiles are summed in wave order through LDS.
template <int G, int BITS>
__global__ __launch_bounds__(256) void linear_wbit_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y) {
  constexpr int SUB = G / 32;                 // MFMAs per group
  constexpr int RUN = G / 4;                  // channels per lane per group
  constexpr int ZPW = BITS == 8 ? 4 : 8;      // zero points per word
  constexpr uint32_t ZMASK = BITS == 8 ? 0xFFu : 0xFu;
  // 3 bits: words a lane's run touches (first bit 3(jG + cG/4) mod 32 is 0
  // at G = 128, 0 or 16 at G = 64, a multiple of 8 at G = 32)
  constexpr int NW = BITS == 8 ? RUN / 4 : (G == 128 ? 3 : 2);
  __shared__ floatx4_t red[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int ng = (int)(k / G), nzw = (ng + ZPW - 1) / ZPW;
  const int jb = ng * wave / 4, je = ng * (wave + 1) / 4;
  int64_t col = n0 + r;
  col = col < n ? col : n - 1;                // columns past n compute a copy, not stored
  const uint16_t* __restrict__ srow = scales + col * ng;
  const uint32_t* __restrict__ zrow = qzeros + col * nzw;
  const int64_t row_words = BITS == 8 ? k / 4 : 3 * k / 32;
  const uint32_t* __restrict__ wrow = qweight + col * row_words;
  const bool has_inv = inv_s != nullptr;
  const uint32_t shift0 = BITS == 8 ? 0u : (uint32_t)(3 * c * RUN) & 31u;
  const int64_t nchunks = (m + 15) / 16;
  for (int64_t tc = blockIdx.y; tc < nchunks; tc += gridDim.y) {
    const int64_t tok = tc * 16 + r;
    const bool tok_ok = tok < m;
    const uint16_t* __restrict__ xrow = x + (tok_ok ? tok : 0) * k;
    floatx4_t acc = floatx4_t{};
    for (int j = jb; j < je; ++j) {
      const int64_t kb = (int64_t)j * G + (int64_t)c * RUN;    // first channel of the run
      const float d = h2f(srow[j]);
      const float z = (float)((zrow[j / ZPW] >> ((32 / ZPW) * (j % ZPW))) & ZMASK);
      const half2_t dd = {(half_t)d, (half_t)d};
      const half2_t oz = {(half_t)(-1024.0f - z), (half_t)(-1024.0f - z)};
      uint32_t cw[NW];
      if constexpr (BITS == 8) {
#pragma unroll
        for (int q = 0; q < NW; ++q) cw[q] = wrow[kb / 4 + q];
      } else {
        const int64_t w0 = (3 * kb) >> 5;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          const int64_t wi = w0 + q < row_words ? w0 + q : row_words - 1;   // a word past the
          cw[q] = wrow[wi];                                                  // row is not used
        }
      }
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        // B: the 8 codes of run i as (1024 + q) halves, in channel order
        uint32_t hq[4];
        if constexpr (BITS == 8) {
          const uint32_t lo = cw[2 * i], hi = cw[2 * i + 1];
          hq[0] = (lo & 0xFFu) | ((lo & 0xFF00u) << 8) | 0x64006400u;
          hq[1] = ((lo >> 16) & 0xFFu) | ((lo >> 8) & 0xFF0000u) | 0x64006400u;
          hq[2] = (hi & 0xFFu) | ((hi & 0xFF00u) << 8) | 0x64006400u;
          hq[3] = ((hi >> 16) & 0xFFu) | ((hi >> 8) & 0xFF0000u) | 0x64006400u;
        } else {
          uint32_t c24;
          if constexpr (G == 128) {
            // bits 24i .. 24i + 23 of the pack
            const uint64_t v = i == 0 ? (uint64_t)cw[0]
                             : i == 1 ? ((uint64_t)cw[0] | ((uint64_t)cw[1] << 32)) >> 24
                             : i == 2 ? ((uint64_t)cw[1] | ((uint64_t)cw[2] << 32)) >> 16
                                      : (uint64_t)cw[2] >> 8;
            c24 = (uint32_t)v & 0xFFFFFFu;
          } else {
            const uint32_t bit = shift0 + 24u * (uint32_t)i;        // < 64 - 24
            const uint64_t v = ((uint64_t)cw[0] | ((uint64_t)cw[1] << 32)) >> bit;
            c24 = (uint32_t)v & 0xFFFFFFu;
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t qa = (c24 >> (6 * e)) & 7u, qb = (c24 >> (6 * e + 3)) & 7u;
            hq[e] = qa | (qb << 16) | 0x64006400u;
          }
        }
        uint32_t bw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bw[e] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, hq[e]) + oz) * dd);
        const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
        // A: x of the lane's token, the same 8 channels, times inv_s
        const uint4 xv = tok_ok ? *reinterpret_cast<const uint4*>(xrow + kb + 8 * i)
                                : make_uint4(0u, 0u, 0u, 0u);
        const uint4 sv = has_inv ? *reinterpret_cast<const uint4*>(inv_s + kb + 8 * i)
                                 : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, sw[4] = {sv.x, sv.y, sv.z, sv.w};
        uint32_t aw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          aw[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xw[e]) *
                                                   __builtin_bit_cast(half2_t, sw[e]));
        const half8_t aop = __builtin_bit_cast(half8_t, make_uint4(aw[0], aw[1], aw[2], aw[3]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc, 0, 0, 0);
      }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      floatx4_t sum = red[0][lane];
#pragma unroll
      for (int wv = 1; wv < 4; ++wv) sum += red[wv][lane];
      const int64_t cc = n0 + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t t = tc * 16 + 4 * c + e;
        if (t < m && cc < n) y[t * n + cc] = f2h_rn(sum[e]);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_linear_wbit(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                              const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m,
                              int64_t n, int64_t k, int32_t g, int32_t w_bit, uint16_t* y,
                              hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int64_t chunks = (m + 15) / 16;
  const dim3 grid((unsigned)((n + 15) / 16), (unsigned)(chunks < 65535 ? chunks : 65535));
#define AWQ_LWB(GG, BB)                                                                        \
  hipLaunchKernelGGL((linear_wbit_kernel<GG, BB>), grid, dim3(256), 0, stream, x, inv_s16,      \
                     qweight, scales, qzeros, m, n, k, y)
  if (w_bit == 8) {
    if (g == 32) AWQ_LWB(32, 8); else if (g == 64) AWQ_LWB(64, 8); else AWQ_LWB(128, 8);
  } else {
    if (g == 32) AWQ_LWB(32, 3); else if (g == 64) AWQ_LWB(64, 3); else AWQ_LWB(128, 3);
  }
#undef AWQ_LWB
  return hipGetLastError();
}

}  // namespace awq
