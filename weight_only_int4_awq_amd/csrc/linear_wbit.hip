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
// Up to 32 tokens one kernel streams the weights once per 16-token chunk
// (linear_wbit_kernel); from 33 tokens a GEMM with the 4-bit GEMM's tiling
// dequantizes each weight tile once per 256 (or 64) tokens
// (linear_wbit_gemm_kernel).
#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

// B operand of sub-step i of a group: the 8 codes of the lane's run i as
// (1024 + q) fp16 pairs, in channel order.  8 bits: words 2i, 2i + 1 of the
// run; 3 bits: bits 24i + sh .. of the run's words (sh = first bit of the
// run in its first word).
template <int G, int BITS, int NW>
__device__ __forceinline__ void wb_run_codes(const uint32_t (&cw)[NW], int i, uint32_t sh,
                                             uint32_t* hq) {
  if constexpr (BITS == 8) {
    const uint32_t lo = cw[2 * i], hi = cw[2 * i + 1];
    hq[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u);
    hq[1] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u);
    hq[2] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u);
    hq[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u);
  } else {
    uint32_t c24;
    if constexpr (G == 128) {
      c24 = i == 0 ? (cw[0] & 0xFFFFFFu)
          : i == 1 ? ((cw[0] >> 24) | (cw[1] << 8)) & 0xFFFFFFu
          : i == 2 ? ((cw[1] >> 16) | (cw[2] << 16)) & 0xFFFFFFu
                   : (cw[2] >> 8);
    } else {
      const uint64_t v = ((uint64_t)cw[0] | ((uint64_t)cw[1] << 32)) >> (sh + 24u * (uint32_t)i);
      c24 = (uint32_t)v & 0xFFFFFFu;
    }
    // codes e (bits 3e .. 3e+2 of c24) in the pair order (e0, e4), (e1, e5),
    // (e2, e6), (e3, e7): the two codes of a pair lie 12 bits apart, so one
    // shift places both inside the mantissas of the two halves, at bit a of
    // the low and b of the high half; a half whose exponent is 2^(10 - a)
    // then holds 2^(10 - a) + q exactly (a, b = 4/0, 7/3, 6/2, 4/0)
    const uint32_t x4 = c24 << 4, x5 = c24 >> 5;
    hq[0] = (x4 & 0x00070070u) | 0x64005400u;       // 64 + e0, 1024 + e4
    hq[1] = (x4 & 0x00380380u) | 0x58004800u;       // 8 + e1, 128 + e5
    hq[2] = (c24 & 0x001C01C0u) | 0x5C004C00u;      // 16 + e2, 256 + e6
    hq[3] = (x5 & 0x00070070u) | 0x64005400u;       // 64 + e3, 1024 + e7
  }
}

// The offsets that turn the halves of wb_run_codes into q - z, from
// oz = (-1024 - z, -1024 - z): at 8 bits every pair is 1024 + q; at 3 bits
// the bases of the pairs above (every sum exact in fp16)
template <int BITS>
__device__ __forceinline__ void wb_offsets(half2_t oz, half2_t (&o)[4]) {
  if constexpr (BITS == 8) {
    o[0] = oz; o[1] = oz; o[2] = oz; o[3] = oz;
  } else {
    o[0] = oz + half2_t{(half_t)960.0f, (half_t)0.0f};
    o[1] = oz + half2_t{(half_t)1016.0f, (half_t)896.0f};
    o[2] = oz + half2_t{(half_t)1008.0f, (half_t)768.0f};
    o[3] = o[0];
  }
}

// 8 activation channels (k0 .. k7, two per word) into the 3-bit pair order
// (k0, k4), (k1, k5), (k2, k6), (k3, k7); the 8-bit order is the natural one
template <int BITS>
__device__ __forceinline__ uint4 wb_act_order(uint4 v) {
  if constexpr (BITS == 8) {
    return v;
  } else {
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
  }
}

// Lane geometry shared by the two decode kernels.  Lane (r = lane % 16,
// c = lane / 16) of a wave serves column n0 + r and a quarter of the channels
// of each group; sub-step i < G/32 multiplies 8 of them, starting at channel
// chan(i) of the group.  The 4 lanes of a row read contiguous bytes per load
// instruction, so each instruction fetches whole 64-byte sectors:
//  * 8 bits (G bytes per row and group): load q < G/64 of lane c is bytes
//    64q + 16c .. + 15 (G = 32: bytes 8c .. + 7); sub-step i takes channels
//    64(i/2) + 16c + 8(i%2) .. + 7.
//  * 3 bits (3G/32 words): lane c takes the run of channels cG/4 .. + G/4 - 1
//    and the words that hold its 3G/4 bits: at g = 128 exactly one 3-word
//    pack (one 12-byte load); at g = 64 and 32 two words from the run's first
//    word, a second word that the run does not reach repeating the first, so
//    no load leaves the group.  sh = first bit of the run in its first word.
template <int G, int BITS>
struct WbLane {
  static constexpr int RUN = G / 4;
  static constexpr int GW = BITS == 8 ? G / 4 : 3 * G / 32;     // words per group per row
  static constexpr int NW = BITS == 8 ? G / 16 : (G == 128 ? 3 : 2);
  uint32_t off[NW];
  uint32_t sh;
  int cc;
  __device__ explicit WbLane(int c) : cc(c) {
    if constexpr (BITS == 8) {
      if constexpr (G >= 64) {
#pragma unroll
        for (int q = 0; q < NW; ++q) off[q] = (uint32_t)(16 * (q / 4) + 4 * c + (q % 4));
      } else {
#pragma unroll
        for (int q = 0; q < NW; ++q) off[q] = (uint32_t)(2 * c + q);
      }
      sh = 0;
    } else {
      const uint32_t b0 = 3u * (uint32_t)(c * RUN);
      const uint32_t w0 = b0 >> 5;
      sh = b0 & 31u;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const uint32_t bits_end = sh + 3u * RUN;        // bits of the run from word w0
        off[q] = (32u * q < bits_end) ? w0 + q : w0;
      }
    }
  }
  __device__ int chan(int i) const {
    if constexpr (BITS == 8) return G >= 64 ? 64 * (i >> 1) + 16 * cc + 8 * (i & 1) : 8 * cc;
    return cc * RUN + 8 * i;
  }
  // the lane's words of group word base `go` (a word offset in its row)
  __device__ void load(const uint32_t* __restrict__ wrow, uint32_t go, uint32_t (&w)[NW]) const {
    if constexpr (BITS == 8 && G >= 64) {
#pragma unroll
      for (int q = 0; q < NW / 4; ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(wrow + go + off[4 * q]);
        w[4 * q] = v.x; w[4 * q + 1] = v.y; w[4 * q + 2] = v.z; w[4 * q + 3] = v.w;
      }
    } else if constexpr (BITS == 8) {
      const uint2 v = *reinterpret_cast<const uint2*>(wrow + go + off[0]);
      w[0] = v.x; w[1] = v.y;
    } else if constexpr (G == 128) {
      __builtin_memcpy(w, wrow + go + off[0], 12);        // one 12-byte load
    } else {
#pragma unroll
      for (int q = 0; q < NW; ++q) w[q] = wrow[go + off[q]];
    }
  }
};

// linear_wbit_kernel<G, BITS, W>: the general decode kernel (up to 16 tokens,
// any k).  One work-group of W waves per 16-column block and 16-token chunk
// (grid y strides over the chunks); the waves split the groups of K into W
// contiguous ranges.  Sub-step i < G/32 of a group is one
// v_mfma_f32_16x16x32_f16 whose k-block of lane c is its i-th run of 8
// channels (at 3 bits in the pair order (k0, k4), (k1, k5), (k2, k6), (k3, k7)
// of the code extraction); A (x_tilde of token t0 + r) and B follow the same
// order, so every channel meets its weight once.  Weights become
// fp16_rn((q - z) D): the codes sit in the mantissa of a power of two
// (1024 at 8 bits, 8 .. 1024 by position at 3 bits), base + z is subtracted
// exactly, and the product with D rounds once.  Activations become
// fp16_rn(x inv_s).  The waves' fp32 partial tiles are summed in wave order
// through LDS.
#ifndef AWQ_WB_GROUP_M
#define AWQ_WB_GROUP_M 4
#endif

template <int G, int BITS, int W>
__global__ __launch_bounds__(W * 64) void linear_wbit_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y) {
  using LG = WbLane<G, BITS>;
  constexpr int SUB = G / 32, NW = LG::NW, RUN = LG::RUN;
  constexpr int ZPW = BITS == 8 ? 4 : 8;      // zero points per word
  constexpr uint32_t ZMASK = BITS == 8 ? 0xFFu : 0xFu;
  __shared__ floatx4_t red[W][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, c = lane >> 4;
  const LG lg(c);
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int ng = (int)(k / G), nzw = (ng + ZPW - 1) / ZPW;
  const int jb = ng * wave / W, je = ng * (wave + 1) / W;
  int64_t col = n0 + r;
  col = col < n ? col : n - 1;                // columns past n compute a copy, not stored
  const uint16_t* __restrict__ srow = scales + col * ng;
  const uint32_t* __restrict__ zrow = qzeros + col * nzw;
  const int64_t row_words = BITS == 8 ? k / 4 : 3 * k / 32;
  const uint32_t* __restrict__ wrow = qweight + col * row_words;
  const bool has_inv = inv_s != nullptr;
  const int64_t nchunks = (m + 15) / 16;
  for (int64_t tc = blockIdx.y; tc < nchunks; tc += gridDim.y) {
    const int64_t tok = tc * 16 + r;
    const bool tok_ok = tok < m;
    const uint16_t* __restrict__ xrow = x + (tok_ok ? tok : 0) * k;
    floatx4_t acc = floatx4_t{};
    for (int j = jb; j < je; ++j) {
      uint32_t cw[NW];
      lg.load(wrow, (uint32_t)j * (uint32_t)LG::GW, cw);
      const float z = (float)((zrow[j / ZPW] >> ((32 / ZPW) * (j % ZPW))) & ZMASK);
      const uint32_t db = srow[j];
      const half2_t dd = __builtin_bit_cast(half2_t, db | (db << 16));
      const half2_t oz = {(half_t)(-1024.0f - z), (half_t)(-1024.0f - z)};
      half2_t oe[4];
      wb_offsets<BITS>(oz, oe);
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int64_t kb = (int64_t)j * G + lg.chan(i);
        uint32_t hq[4];
        wb_run_codes<G, BITS, NW>(cw, i, lg.sh, hq);
        uint32_t bw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bw[e] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, hq[e]) + oe[e]) * dd);
        const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
        const uint4 xv = tok_ok ? *reinterpret_cast<const uint4*>(xrow + kb)
                                : make_uint4(0u, 0u, 0u, 0u);
        const uint4 sv = has_inv ? *reinterpret_cast<const uint4*>(inv_s + kb)
                                 : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, sw[4] = {sv.x, sv.y, sv.z, sv.w};
        uint32_t aw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          aw[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xw[e]) *
                                                   __builtin_bit_cast(half2_t, sw[e]));
        const half8_t aop =
            __builtin_bit_cast(half8_t, wb_act_order<BITS>(make_uint4(aw[0], aw[1], aw[2], aw[3])));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc, 0, 0, 0);
      }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      floatx4_t sum = red[0][lane];
#pragma unroll
      for (int wv = 1; wv < W; ++wv) sum += red[wv][lane];
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

// linear_wbit_decode_kernel<G, BITS, W>: the decode kernel for up to 16
// tokens whose x_tilde fits LDS (m = 1 always does), with the lane geometry,
// sub-steps and rounding of linear_wbit_kernel.  Work-group b owns the
// 16-column blocks b, b + grid, ... (at most kWbMaxBlk).
//  * Prologue: the staging loads (x, inv_s, scales, zeros: cache-resident and
//    shared by all work-groups) are issued first, then the first kWbPF weight
//    loads of every wave; x_tilde = fp16_rn(x inv_s) of all m tokens (each
//    8-channel run in the code order) and the blocks' (D, -1024 - z) pairs
//    go to LDS, so weights are the only global loads of the main loop.
//  * Main loop: each wave owns a contiguous range of groups along K and walks
//    the sequence (block, group) with its weight loads in two halves of kWbPF
//    items, one in flight while the other is multiplied, across block
//    boundaries.  Loads are unconditional (the issue cursor stops on the
//    last item) and their offsets opaque to the optimiser, so the compiler
//    keeps exact counts of the loads in flight instead of waiting for all.
//  * At a block's end each wave leaves its fp32 partial tile in LDS; after
//    the last block the partial tiles are summed in wave order.
#ifndef AWQ_WB_PF
#define AWQ_WB_PF 2
#endif
#ifndef AWQ_WB_MAXBLK
#define AWQ_WB_MAXBLK 4
#endif
#ifndef AWQ_WB_SZPRE
#define AWQ_WB_SZPRE 2
#endif
#ifndef AWQ_WB_PF3
#define AWQ_WB_PF3 2
#endif
// items per prefetch half: a 3-bit item is 768 bytes per wave (at g = 128),
// an 8-bit one 2 KiB
template <int BITS>
constexpr int wb_pf() { return BITS == 3 ? AWQ_WB_PF3 : AWQ_WB_PF; }
constexpr int kWbMaxBlk = AWQ_WB_MAXBLK;

// dynamic LDS of the staged decode kernel
// (x_tilde [m][k] | table [nb][ng][17] words | 16-byte aligned partial tiles [nb][w][64])
__host__ __device__ inline size_t wbit_decode_red_off(int64_t m, int64_t k, int64_t ng, int nb) {
  return ((size_t)m * (size_t)k * 2 + (size_t)nb * ng * 17 * 4 + 15) & ~(size_t)15;
}
__host__ __device__ inline size_t wbit_decode_lds(int64_t m, int64_t k, int64_t ng, int nb, int w) {
  return wbit_decode_red_off(m, k, ng, nb) + (size_t)nb * w * 64 * 16;
}

template <int G, int BITS, int W>
__global__ __launch_bounds__(W * 64) void linear_wbit_decode_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y) {
  using LG = WbLane<G, BITS>;
  constexpr int SUB = G / 32, NW = LG::NW;
  constexpr int ZPW = BITS == 8 ? 4 : 8;
  constexpr uint32_t ZMASK = BITS == 8 ? 0xFFu : 0xFu;
  const int ng = (int)(k / G), nzw = (ng + ZPW - 1) / ZPW;
  const int nblk = (int)((n + 15) / 16);
  const int grid = (int)gridDim.x, bid = (int)blockIdx.x;
  const int my_blocks = (nblk - bid + grid - 1) / grid;          // 1 .. kWbMaxBlk
  extern __shared__ __attribute__((aligned(16))) uint16_t dyn_l[];
  uint16_t* xs_l = dyn_l;                                                    // [m][k]
  uint32_t* sz_l = reinterpret_cast<uint32_t*>(dyn_l + m * k);               // [blk][ng][17]
  floatx4_t* red = reinterpret_cast<floatx4_t*>(reinterpret_cast<char*>(dyn_l) +
                                                 wbit_decode_red_off(m, k, ng, my_blocks));  // [blk][W][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, c = lane >> 4;
  const LG lg(c);
  const int jb = ng * wave / W, je = ng * (wave + 1) / W;
  const int cnt = je - jb;
  const int total = my_blocks * cnt;                              // (block, group) items of this wave
  const int64_t row_words = BITS == 8 ? k / 4 : 3 * k / 32;
  auto col_of = [&](int bi, int rr) {
    const int64_t cq = (int64_t)(bid + bi * grid) * 16 + rr;
    return cq < n ? cq : n - 1;
  };

  // ---- 1. staging loads first
  const bool has_inv = inv_s != nullptr;
  const uint32_t kc = (uint32_t)(k / 8), xchunks = (uint32_t)m * kc;
  const uint16_t* __restrict__ sbase = has_inv ? inv_s : x;    // a valid address either way
  const int szn = my_blocks * 16 * ng;                         // table entries
  constexpr int XPRE = 2, SZPRE = AWQ_WB_SZPRE;
  uint4 xp[XPRE], sp[XPRE];
#pragma unroll
  for (int i = 0; i < XPRE; ++i) {
    uint32_t q = (uint32_t)tid + (uint32_t)(i * W * 64);
    q = q < xchunks ? q : xchunks - 1;                  // clamped: unconditional loads
    xp[i] = *reinterpret_cast<const uint4*>(x + (size_t)q * 8);
    sp[i] = *reinterpret_cast<const uint4*>(sbase + (size_t)(q % kc) * 8);
  }
  // entry q of the table: block q / (16 ng), column (q / ng) % 16, group q % ng
  auto sz_src = [&](int q, int64_t& cq, int& j) {
    const int bi = q / (16 * ng), rest = q - bi * 16 * ng;
    cq = col_of(bi, rest / ng);
    j = rest % ng;
  };
  uint32_t dp[SZPRE], zp[SZPRE];
#pragma unroll
  for (int i = 0; i < SZPRE; ++i) {
    int q = tid + i * W * 64;
    q = q < szn ? q : szn - 1;
    int64_t cq;
    int j;
    sz_src(q, cq, j);
    dp[i] = scales[cq * ng + j];
    zp[i] = qzeros[cq * nzw + j / ZPW];
  }

  // ---- 2. the first half of the weight loads
  constexpr int kWbPF = wb_pf<BITS>();
  uint32_t wq[2 * kWbPF][NW];
  int i_blk = 0, i_j = jb, i_left = total;    // issue cursor (wave-uniform)
  auto issue = [&](int slot) {
    const int64_t cq = col_of(i_blk, r);
    uint32_t go = (uint32_t)i_j * (uint32_t)LG::GW;
    asm volatile("" : "+v"(go));              // a repeated address stays a load
    lg.load(qweight + cq * row_words, go, wq[slot]);
    if (i_left > 1) {
      --i_left;
      if (++i_j == je) { i_j = jb; ++i_blk; }
    }
  };
  if (cnt > 0) {
#pragma unroll
    for (int p = 0; p < kWbPF; ++p) issue(p);
  }

  // ---- 3. x_tilde and the (D, -1024 - z) table in LDS
  auto stage_x = [&](uint32_t q, uint4 xv, uint4 sv) {
    if (!has_inv) sv = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.x) * __builtin_bit_cast(half2_t, sv.x));
    v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.y) * __builtin_bit_cast(half2_t, sv.y));
    v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.z) * __builtin_bit_cast(half2_t, sv.z));
    v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.w) * __builtin_bit_cast(half2_t, sv.w));
    *reinterpret_cast<uint4*>(xs_l + (size_t)q * 8) = wb_act_order<BITS>(v);
  };
  auto stage_sz = [&](int q, uint32_t d, uint32_t zw) {
    const int bi = q / (16 * ng), rest = q - bi * 16 * ng;
    const int rr = rest / ng, j = rest % ng;
    const float z = (float)((zw >> ((32 / ZPW) * (j % ZPW))) & ZMASK);
    const uint32_t zb = __builtin_bit_cast(uint16_t, (half_t)(-1024.0f - z));
    sz_l[((size_t)bi * ng + j) * 17 + rr] = (d & 0xFFFFu) | (zb << 16);
  };
#pragma unroll
  for (int i = 0; i < XPRE; ++i) {
    const uint32_t q = (uint32_t)tid + (uint32_t)(i * W * 64);
    if (q < xchunks) stage_x(q, xp[i], sp[i]);
  }
#pragma unroll
  for (int i = 0; i < SZPRE; ++i) {
    const int q = tid + i * W * 64;
    if (q < szn) stage_sz(q, dp[i], zp[i]);
  }
  // the rest (long k, several blocks): these loads wait behind the weights
  for (uint32_t q = (uint32_t)tid + (uint32_t)(XPRE * W * 64); q < xchunks; q += W * 64)
    stage_x(q, *reinterpret_cast<const uint4*>(x + (size_t)q * 8),
            *reinterpret_cast<const uint4*>(sbase + (size_t)(q % kc) * 8));
  for (int q = tid + SZPRE * W * 64; q < szn; q += W * 64) {
    int64_t cq;
    int j;
    sz_src(q, cq, j);
    stage_sz(q, scales[cq * ng + j], qzeros[cq * nzw + j / ZPW]);
  }
  __syncthreads();

  // ---- 4. the (block, group) loop
  const bool tok_ok = r < m;
  const uint16_t* xa = xs_l + (tok_ok ? r : 0) * k;
  floatx4_t acc = floatx4_t{};
  int c_blk = 0, c_j = jb, c_left = total;    // consume cursor
  auto consume = [&](int slot, bool guarded) {
    if (!guarded || c_left > 0) {             // wave-uniform
      const int j = c_j;
      const uint32_t t = sz_l[((size_t)c_blk * ng + j) * 17 + r];
      const uint32_t dl = t & 0xFFFFu, zl = t >> 16;
      const half2_t dd = __builtin_bit_cast(half2_t, dl | (dl << 16));
      const half2_t oz = __builtin_bit_cast(half2_t, zl | (zl << 16));
      half2_t oe[4];
      wb_offsets<BITS>(oz, oe);
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        uint32_t hq[4];
        wb_run_codes<G, BITS, NW>(wq[slot], i, lg.sh, hq);
        uint32_t bw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bw[e] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, hq[e]) + oe[e]) * dd);
        const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));
        // rows r >= m read token 0: they only reach output rows that are not stored
        const half8_t aop = *reinterpret_cast<const half8_t*>(xa + j * G + lg.chan(i));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc, 0, 0, 0);
      }
      --c_left;
      if (++c_j == je) {                      // the block's partial tile of this wave
        red[((size_t)c_blk * W + wave) * 64 + lane] = acc;
        acc = floatx4_t{};
        c_j = jb;
        ++c_blk;
      }
    }
  };
  if (cnt > 0) {
    // half 0 (slots 0 .. PF-1) is in flight on entry; the other half is
    // issued only while items remain beyond the current half
    int rem = total;
    while (true) {
      if (rem > kWbPF) {
#pragma unroll
        for (int p = 0; p < kWbPF; ++p) issue(kWbPF + p);
#pragma unroll
        for (int p = 0; p < kWbPF; ++p) consume(p, false);
        rem -= kWbPF;
      } else {
#pragma unroll
        for (int p = 0; p < kWbPF; ++p) consume(p, true);
        break;
      }
      if (rem > kWbPF) {
#pragma unroll
        for (int p = 0; p < kWbPF; ++p) issue(p);
#pragma unroll
        for (int p = 0; p < kWbPF; ++p) consume(kWbPF + p, false);
        rem -= kWbPF;
      } else {
#pragma unroll
        for (int p = 0; p < kWbPF; ++p) consume(kWbPF + p, true);
        break;
      }
    }
  } else {
    // a wave without groups (fewer than W groups in k) leaves zero tiles
    for (int bi = 0; bi < my_blocks; ++bi) red[((size_t)bi * W + wave) * 64 + lane] = acc;
  }

  // ---- 5. wave bi % W sums block bi's W partial tiles in wave order
  __syncthreads();
  for (int bi = wave; bi < my_blocks; bi += W) {
    floatx4_t sum = red[((size_t)bi * W) * 64 + lane];
#pragma unroll
    for (int wv = 1; wv < W; ++wv) sum += red[((size_t)bi * W + wv) * 64 + lane];
    const int64_t cc = (int64_t)(bid + bi * grid) * 16 + r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t t = 4 * c + e;
      if (t < m && cc < n) y[t * n + cc] = f2h_rn(sum[e]);
    }
  }
}

// ---------------------------------------------------------------- prefill GEMM (m > 32)
// linear_wbit_gemm_kernel<G, BITS, BM>: work-group tile BM (256, or 64 for
// few tokens) x 128 columns, K-step 64, 4 waves (2 x 2 of 128 x 64, or 1 x 4
// of 64 x 32), v_mfma_f32_32x32x16_f16 with fp32 accumulators.
//  * A: x_tilde rows (fp16, natural channel order; written once per call by
//    linear_wbit_xprep_kernel, or x itself when there is no inv_s) copied
//    global -> LDS with global_load_lds, two stages, 16-byte chunks
//    XOR-swizzled by row so a fragment read hits distinct banks.
//  * B: lane (column j = lane % 32, half c = lane / 32) owns channels
//    32c .. 32c + 31 of the K-step: at 8 bits 32 bytes (two 16-byte loads),
//    at 3 bits exactly one 3-word pack.  Sub-step s < 4 multiplies their
//    8-channel chunk s; the A fragment of lane half c reads chunk 4c + s of
//    the tile row, so both operands agree on the K order.  Codes are placed
//    in the mantissa of 1024 (a byte permute at 8 bits, 3-bit fields at 3
//    bits); (1024 + z) is removed exactly and D applied with one rounding.
//  * D and (-1024 - z) of the tile's 128 columns are staged in LDS as one
//    fp16 pair per (group, column) for a window of kWbWin groups, restaged
//    at each window boundary (windows hold an even number of K-steps).
//  * The next K-step's activations and weights are in flight while the
//    current one is multiplied.
constexpr int kWbBN = 128, kWbBK = 64;
constexpr int kWbWin = 28;                 // groups per staged window
constexpr int kWbTRow = kWbBN + 1;         // padded table row (words)
#ifndef AWQ_WBIT_SWZ_SHIFT
#define AWQ_WBIT_SWZ_SHIFT 1
#endif

// x_tilde = fp16_rn(x * inv_s), natural channel order
__global__ __launch_bounds__(256) void linear_wbit_xprep_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s, int64_t m, int64_t k,
    uint16_t* __restrict__ xt) {
  const int64_t chunks = m * (k / 8);
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t kk = (c % (k / 8)) * 8;
    const uint4 xv = *reinterpret_cast<const uint4*>(x + c * 8);
    const uint4 iv = *reinterpret_cast<const uint4*>(inv_s + kk);
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.x) * __builtin_bit_cast(half2_t, iv.x));
    v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.y) * __builtin_bit_cast(half2_t, iv.y));
    v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.z) * __builtin_bit_cast(half2_t, iv.z));
    v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.w) * __builtin_bit_cast(half2_t, iv.w));
    *reinterpret_cast<uint4*>(xt + c * 8) = v;
  }
}

template <int BITS>
struct WbRegs;
template <>
struct WbRegs<8> { uint4 a, b; };
template <>
struct WbRegs<3> { uint32_t a, b, c; };

// the 8 codes of sub-step s (channels 8s .. 8s + 7 of a lane's 32) as four
// fp16 pairs (1024 + q), in channel order
template <int BITS>
__device__ __forceinline__ void wb_codes(const WbRegs<BITS>& w, int s, uint32_t* hq);

template <>
__device__ __forceinline__ void wb_codes<8>(const WbRegs<8>& w, int s, uint32_t* hq) {
  const uint4 v = s < 2 ? w.a : w.b;
  const uint32_t lo = (s & 1) ? v.z : v.x, hi = (s & 1) ? v.w : v.y;
  // bytes 0/1 and 2/3 of a word into the low bytes of two halves of 0x64..
  hq[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u);
  hq[1] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u);
  hq[2] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u);
  hq[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u);
}

template <>
__device__ __forceinline__ void wb_codes<3>(const WbRegs<3>& w, int s, uint32_t* hq) {
  // bits 24s .. 24s + 23 of the 96-bit pack
  const uint32_t c24 = s == 0 ? (w.a & 0xFFFFFFu)
                     : s == 1 ? ((w.a >> 24) | (w.b << 8)) & 0xFFFFFFu
                     : s == 2 ? ((w.b >> 16) | (w.c << 16)) & 0xFFFFFFu
                              : (w.c >> 8);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    hq[e] = ((c24 >> (6 * e)) & 7u) | (((c24 >> (6 * e + 3)) & 7u) << 16) | 0x64006400u;
}

template <int G, int BITS, int BM>
__global__ __launch_bounds__(256, 2) void linear_wbit_gemm_kernel(
    const uint16_t* __restrict__ xt, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros, int64_t m,
    int64_t n, int64_t k, uint16_t* __restrict__ y, int tiles_m, int tiles_total, int ks,
    float* __restrict__ part) {
  constexpr int WM = BM == 256 ? 2 : 1;
  constexpr int WN = 4 / WM;
  constexpr int RW = BM / WM, CW = kWbBN / WN;      // rows and columns per wave
  constexpr int BMB = RW / 32, BNB = CW / 32;       // 32 x 32 blocks per wave
  constexpr int AR = BM / 32;                       // A copy instructions per wave
  constexpr int ZPW = BITS == 8 ? 4 : 8;
  constexpr uint32_t ZMASK = BITS == 8 ? 0xFFu : 0xFu;
  constexpr int SPW = kWbWin * G / kWbBK;           // K-steps per window (even)
  static_assert(BM == 256 || BM == 64, "tile rows");
  static_assert(SPW % 2 == 0, "windows hold an even number of K-steps");
  __shared__ __attribute__((aligned(16))) uint16_t a_st0[BM * kWbBK];
  __shared__ __attribute__((aligned(16))) uint16_t a_st1[BM * kWbBK];
  __shared__ uint32_t t_l[kWbWin * kWbTRow];        // (D, -1024 - z) per (group, column)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  // XCD-aware tile order: each XCD gets a contiguous run of the tiles in
  // banded order (bands of AWQ_WB_GROUP_M row tiles)
  const int bid = blockIdx.x;
  const int per = tiles_total / 8, rem = tiles_total % 8;
  const int xcd = bid % 8, slot = bid / 8;
  const int wgi = xcd * per + (xcd < rem ? xcd : rem) + slot;
  // work-group wgi: tile wgi / ks of the order, slice wgi % ks of its K range;
  // slices start on group boundaries (units of max(1, G / 64) K-steps); tl is
  // the tile's slot among the partial tiles (rows fastest)
  const int t_ord = wgi / ks, sl = wgi - t_ord * ks;
  int tm, tn;
  banded_tile_coords<AWQ_WB_GROUP_M>(t_ord, tiles_m, tiles_total / ks / tiles_m, tm, tn);
  const int tl = tm + tn * tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * kWbBN;
  const int ng = (int)(k / G), nzw = (ng + ZPW - 1) / ZPW;
  constexpr int UNIT = G / kWbBK > 1 ? G / kWbBK : 1;
  const int nu = (int)(k / kWbBK) / UNIT;
  const int kt0 = (int)((int64_t)sl * nu / ks) * UNIT, kt1 = (int)((int64_t)(sl + 1) * nu / ks) * UNIT;

  // ---- A loader (as in the 4-bit GEMM): lane (row r, slot p) of a copy
  // instruction fetches logical chunk p ^ ((r >> S) & 7) of its row
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int a_lr = lane >> 3, a_p = lane & 7;
  const char* xbytes = reinterpret_cast<const char*>(xt);
  // row of copy i: wave BM/4 + 8 i + a_lr (clamped to m - 1); its swizzle
  // (row >> 1) & 7 takes two values, by the parity of i (BM/4 is a multiple
  // of 16).  The offsets are formed at each copy to spare registers.
  const int64_t a_row0 = m0 + wave * (BM / 4) + a_lr;
  const uint32_t a_sw[2] = {(uint32_t)((a_p ^ ((a_lr >> 1) & 7)) * 16),
                            (uint32_t)((a_p ^ ((4 + (a_lr >> 1)) & 7)) * 16)};
#define AWQ_WB_LOAD_A(KT, STAGE_PTR)                                                    \
  {                                                                                     \
    const char* xk_ = xbytes + (int64_t)(KT) * kWbBK * 2;                               \
    _Pragma("unroll") for (int i = 0; i < AR; ++i) {                                    \
      const int64_t r_ = a_row0 + 8 * i < m ? a_row0 + 8 * i : m - 1;                   \
      const uint32_t o_ = (uint32_t)(r_ * k * 2) + a_sw[i & 1];                        \
      __builtin_amdgcn_global_load_lds(                                                 \
          (const void*)(xk_ + o_),                                                      \
          (lds_void_t*)((STAGE_PTR) + (wave * (BM / 4) + 8 * i) * 64), 16, 0, 0);       \
    }                                                                                   \
  }

  // ---- B loader: lane (j, c) of block bn, channels 32c .. 32c + 31 of the K-step
  const int bj = lane & 31, bc = lane >> 5;
  constexpr int64_t kStepWords = BITS == 8 ? 16 : 6;     // qweight words per row per K-step
  const int64_t row_words = BITS == 8 ? k / 4 : 3 * k / 32;
  const uint32_t* b_src[BNB];
#pragma unroll
  for (int bn = 0; bn < BNB; ++bn) {
    int64_t col = n0 + wn * CW + bn * 32 + bj;
    col = col < n ? col : n - 1;
    b_src[bn] = qweight + col * row_words + (BITS == 8 ? 8 : 3) * bc;
  }
  WbRegs<BITS> wb[BNB];
#define AWQ_WB_LOAD_B(KT)                                                                  \
  {                                                                                        \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                                   \
      const uint32_t* p_ = b_src[bn] + (int64_t)(KT) * kStepWords;                         \
      if constexpr (BITS == 8) {                                                           \
        wb[bn].a = *reinterpret_cast<const uint4*>(p_);                                    \
        wb[bn].b = *reinterpret_cast<const uint4*>(p_ + 4);                                \
      } else {                                                                             \
        wb[bn].a = p_[0];                                                                  \
        wb[bn].b = p_[1];                                                                  \
        wb[bn].c = p_[2];                                                                  \
      }                                                                                    \
    }                                                                                      \
  }

  floatx16_t acc[BMB][BNB];
#pragma unroll
  for (int i = 0; i < BMB; ++i)
#pragma unroll
    for (int jj = 0; jj < BNB; ++jj) acc[i][jj] = floatx16_t{};

  uint32_t a_base[BMB];
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm) {
    const int row = wm * RW + bm * 32 + (lane & 31);
    a_base[bm] = (uint32_t)(row * 128 + ((4 * bc) ^ ((row >> AWQ_WBIT_SWZ_SHIFT) & 7)) * 16);
  }

  AWQ_WB_LOAD_A(kt0, a_st0);
  AWQ_WB_LOAD_B(kt0);

  int gwin0 = 0;
#define AWQ_WB_STEP(KT, CUR, NXT)                                                       \
  {                                                                                     \
    WbRegs<BITS> wc[BNB];                                                               \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) wc[bn] = wb[bn];                 \
    const int ktn_ = (KT) + 1 < kt1 ? (KT) + 1 : (KT);                                 \
    AWQ_WB_LOAD_A(ktn_, NXT);                                                           \
    AWQ_WB_LOAD_B(ktn_);                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    const int ti_ = ((KT) * kWbBK + 32 * bc) / G - gwin0;                               \
    half2_t dd[BNB], oz[BNB];                                                           \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                                \
      const uint32_t t_ = t_l[ti_ * kWbTRow + wn * CW + bn * 32 + bj];                  \
      const uint32_t dl_ = t_ & 0xFFFFu, zl_ = t_ >> 16;                                \
      dd[bn] = __builtin_bit_cast(half2_t, dl_ | (dl_ << 16));                          \
      oz[bn] = __builtin_bit_cast(half2_t, zl_ | (zl_ << 16));                          \
    }                                                                                   \
    half8_t af[BMB];                                                                    \
    _Pragma("unroll") for (int bm = 0; bm < BMB; ++bm)                                  \
      af[bm] = *reinterpret_cast<const half8_t*>(reinterpret_cast<const char*>(CUR) + a_base[bm]); \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                     \
      half8_t bq[BNB];                                                                  \
      _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                              \
        uint32_t hq[4];                                                                 \
        wb_codes<BITS>(wc[bn], s, hq);                                                  \
        uint32_t bw[4];                                                                 \
        _Pragma("unroll") for (int e = 0; e < 4; ++e)                                   \
          bw[e] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2_t, hq[e]) + oz[bn]) * dd[bn]); \
        bq[bn] = __builtin_bit_cast(half8_t, make_uint4(bw[0], bw[1], bw[2], bw[3]));   \
      }                                                                                 \
      _Pragma("unroll") for (int bm = 0; bm < BMB; ++bm) {                              \
        _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn)                              \
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[bm], bq[bn], acc[bm][bn], 0, 0, 0); \
        if (s + 1 < 4)                                                                  \
          af[bm] = *reinterpret_cast<const half8_t*>(                                   \
              reinterpret_cast<const char*>(CUR) + (a_base[bm] ^ (uint32_t)(16 * (s + 1)))); \
      }                                                                                 \
    }                                                                                   \
    __builtin_amdgcn_s_waitcnt(0);                                                      \
    __syncthreads();                                                                    \
  }

  for (int ws = kt0; ws < kt1; ws += SPW) {
    const int we = ws + SPW < kt1 ? ws + SPW : kt1;
    // stage the window's (D, -1024 - z): every wave has passed the last
    // step's barrier, so the previous window is no longer read
    gwin0 = ws * kWbBK / G;
    const int gw = (we * kWbBK + G - 1) / G - gwin0;      // <= kWbWin
    for (int i = tid; i < kWbBN * gw; i += 256) {
      const int r = i / gw, gi = i - r * gw;
      int64_t col = n0 + r;
      col = col < n ? col : n - 1;
      const int gg = gwin0 + gi;
      const uint32_t d = scales[col * ng + gg];
      const uint32_t zw = qzeros[col * nzw + gg / ZPW];
      const float z = (float)((zw >> ((32 / ZPW) * (gg % ZPW))) & ZMASK);
      const uint32_t zb = __builtin_bit_cast(uint16_t, (half_t)(-1024.0f - z));
      t_l[gi * kWbTRow + r] = d | (zb << 16);
    }
    __builtin_amdgcn_s_waitcnt(0);       // also the direct-to-LDS copies of the first step
    __syncthreads();
    int kt = ws;
#pragma unroll 1
    for (; kt + 1 < we; kt += 2) {
      AWQ_WB_STEP(kt, a_st0, a_st1);
      AWQ_WB_STEP(kt + 1, a_st1, a_st0);
    }
    if (kt < we) AWQ_WB_STEP(kt, a_st0, a_st1);    // only in the last window
  }
#undef AWQ_WB_STEP
#undef AWQ_WB_LOAD_A
#undef AWQ_WB_LOAD_B

  // value e of lane l in block (bm, bn) is row 8(e/4) + 4(l/32) + e%4, column l%32
  if (ks == 1) {
#pragma unroll
    for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
      for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = m0 + wm * RW + bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
          const int64_t cidx = n0 + wn * CW + bn * 32 + (lane & 31);
          const float v = acc[bm][bn][e];
          if (t < m && cidx < n) y[t * n + cidx] = f2h_rn(v);
        }
    return;
  }
  // split along K: the fp32 partial tile (its valid rows) goes to slice sl of
  // the tile's partials; linear_wbit_reduce_kernel sums them in slice order
  const int rows_t = m < BM ? (int)m : BM;
  const int mrow = (m - m0) < rows_t ? (int)(m - m0) : rows_t;
  float* __restrict__ pt = part + ((size_t)tl * ks + sl) * rows_t * kWbBN;
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
    for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * RW + bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int col = wn * CW + bn * 32 + (lane & 31);
        const float v = acc[bm][bn][e];
        if (row < mrow) pt[row * kWbBN + col] = v;
      }
}

// Sums the K slices of a split GEMM in slice order: thread item = 4 adjacent
// columns of one row of one tile.
__global__ __launch_bounds__(256) void linear_wbit_reduce_kernel(
    const float* __restrict__ part, int64_t m, int64_t n, int bm, int tiles_m, int tiles_total,
    int ks, uint16_t* __restrict__ y) {
  const int rows_t = m < bm ? (int)m : bm;
  const int64_t items = (int64_t)tiles_total * rows_t * (kWbBN / 4);
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * 256) {
    const int c4 = (int)(it % (kWbBN / 4));
    const int64_t rr = it / (kWbBN / 4);
    const int row = (int)(rr % rows_t);
    const int tl = (int)(rr / rows_t);
    const int tm = tl % tiles_m, tn = tl / tiles_m;
    const int64_t t = (int64_t)tm * bm + row;
    if (t >= m) continue;
    const float* __restrict__ src = part + ((size_t)tl * ks) * rows_t * kWbBN +
                                    (size_t)row * kWbBN + 4 * c4;
    float4 sum = *reinterpret_cast<const float4*>(src);
    for (int sl = 1; sl < ks; ++sl) {
      const float4 v = *reinterpret_cast<const float4*>(src + (size_t)sl * rows_t * kWbBN);
      sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
    }
    const int64_t c0 = (int64_t)tn * kWbBN + 4 * c4;
    const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c0 + e < n) y[t * n + c0 + e] = f2h_rn(sv[e]);
  }
}

// the smallest m that takes the GEMM (at 17-32 tokens its 64-row tiles with
// split K stream the weights 1.6-2.3x faster than one 16-token-chunk pass
// per chunk of the general kernel: 3-bit gate/up at 32 tokens 106 -> 47 us)
#ifndef AWQ_WBIT_GEMM_MIN_M
#define AWQ_WBIT_GEMM_MIN_M 17
#endif

static int64_t wbit_gemm_bm(int64_t m) { return m <= 128 ? 64 : 256; }

// rows per GEMM launch: the 32-bit activation offsets stay below 2^31 bytes
static int64_t wbit_row_chunk(int64_t k) {
  const int64_t c = (((int64_t)1 << 31) / (k * 2)) / 256 * 256;
  return c > 0 ? c : 256;
}

// K slices per tile where the tiles alone leave CUs idle: enough for about
// 256 work-groups, at most 16, each slice at least two group-aligned units of
// K-steps; none beyond 512 tokens, 128 tiles or one row chunk.
static int wbit_split(int64_t m, int64_t n, int64_t k, int32_t g) {
  const int64_t bm = wbit_gemm_bm(m);
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + kWbBN - 1) / kWbBN);
  if (m > 512 || tiles > 128 || m > wbit_row_chunk(k)) return 1;
  const int64_t unit = g / kWbBK > 1 ? g / kWbBK : 1;
  const int64_t nu = k / kWbBK / unit;
  // two work-groups per CU for 64-row tiles with a long K loop (as the 4-bit GEMM)
  const int64_t target = (bm == 64 && k >= 8192) ? 512 : 256;
  int64_t sk = (target + tiles - 1) / tiles;
  const int64_t smax = nu / 2 < 16 ? nu / 2 : 16;
  sk = sk < smax ? sk : smax;
  return sk > 1 ? (int)sk : 1;
}

static size_t align256w(size_t v) { return (v + 255) & ~(size_t)255; }

size_t linear_wbit_scratch_bytes(int64_t m, int64_t n, int64_t k, int32_t g, bool has_inv) {
  if (m < AWQ_WBIT_GEMM_MIN_M) return 0;
  size_t b = has_inv ? align256w((size_t)m * (size_t)k * 2) : 0;
  const int sk = wbit_split(m, n, k, g);
  if (sk > 1) {
    const int64_t bm = wbit_gemm_bm(m);
    const int64_t tiles = ((m + bm - 1) / bm) * ((n + kWbBN - 1) / kWbBN);
    const int64_t rows_t = m < bm ? m : bm;
    b += align256w((size_t)sk * tiles * rows_t * kWbBN * 4);
  }
  return b;
}

template <int G, int BITS>
static void launch_wbit_gemm(const uint16_t* xt, const uint32_t* qweight, const uint16_t* scales,
                             const uint32_t* qzeros, int64_t m, int64_t n, int64_t k, uint16_t* y,
                             float* part, hipStream_t stream) {
  const int64_t bm = wbit_gemm_bm(m);
  const int64_t chunk = wbit_row_chunk(k);
  const int ks = wbit_split(m, n, k, G);
  const int tiles_n = (int)((n + kWbBN - 1) / kWbBN);
  for (int64_t r0 = 0; r0 < m; r0 += chunk) {
    const int64_t mc = (m - r0) < chunk ? (m - r0) : chunk;
    const int tiles_m = (int)((mc + bm - 1) / bm);
    const int tiles = tiles_m * tiles_n;
    const unsigned grid = (unsigned)tiles * (unsigned)ks;
    if (bm == 64)
      hipLaunchKernelGGL((linear_wbit_gemm_kernel<G, BITS, 64>), dim3(grid), dim3(256), 0, stream,
                         xt + r0 * k, qweight, scales, qzeros, mc, n, k, y + r0 * n, tiles_m,
                         (int)grid, ks, part);
    else
      hipLaunchKernelGGL((linear_wbit_gemm_kernel<G, BITS, 256>), dim3(grid), dim3(256), 0, stream,
                         xt + r0 * k, qweight, scales, qzeros, mc, n, k, y + r0 * n, tiles_m,
                         (int)grid, ks, part);
    if (ks > 1)
      hipLaunchKernelGGL(linear_wbit_reduce_kernel, dim3(512), dim3(256), 0, stream, part, mc, n,
                         (int)bm, tiles_m, tiles, ks, y + r0 * n);
  }
}

// decode launch: waves per work-group give each wave at least two groups of
// K; up to 16 tokens whose x_tilde and scale table fit LDS (with the
// reduction buffer) take the staged kernel
template <int G, int BITS, int WW>
static hipError_t launch_wbit_decode_w(const uint16_t* x, const uint32_t* qweight,
                                       const uint16_t* scales, const uint32_t* qzeros,
                                       const uint16_t* inv_s16, int64_t m, int64_t n, int64_t k,
                                       uint16_t* y, hipStream_t stream) {
  const int64_t ng = k / G;
  const int64_t nblk = (n + 15) / 16;
  // blocks per work-group: about two work-groups per CU, at most kWbMaxBlk,
  // fewer where LDS would not hold them
  int nb = (int)((nblk + 511) / 512);
  nb = nb < 1 ? 1 : (nb > kWbMaxBlk ? kWbMaxBlk : nb);
  while (nb > 1 && wbit_decode_lds(m, k, ng, nb, WW) > 80 * 1024) --nb;
  const size_t lds = wbit_decode_lds(m, k, ng, nb, WW);
  if (m <= 16 && lds <= 160 * 1024) {
    const void* fn = reinterpret_cast<const void*>(&linear_wbit_decode_kernel<G, BITS, WW>);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    const int64_t grid = (nblk + nb - 1) / nb;
    hipLaunchKernelGGL((linear_wbit_decode_kernel<G, BITS, WW>), dim3((unsigned)grid), dim3(WW * 64),
                       lds, stream, x, inv_s16, qweight, scales, qzeros, m, n, k, y);
  } else {
    const int64_t chunks = (m + 15) / 16;
    const dim3 grid((unsigned)nblk, (unsigned)(chunks < 65535 ? chunks : 65535));
    hipLaunchKernelGGL((linear_wbit_kernel<G, BITS, WW>), grid, dim3(WW * 64), 0, stream, x, inv_s16,
                       qweight, scales, qzeros, m, n, k, y);
  }
  return hipGetLastError();
}

template <int G, int BITS>
static hipError_t launch_wbit_decode(const uint16_t* x, const uint32_t* qweight,
                                     const uint16_t* scales, const uint32_t* qzeros,
                                     const uint16_t* inv_s16, int64_t m, int64_t n, int64_t k,
                                     uint16_t* y, hipStream_t stream) {
  if (k / G >= 16)
    return launch_wbit_decode_w<G, BITS, 8>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
  return launch_wbit_decode_w<G, BITS, 4>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
}

hipError_t launch_linear_wbit(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                              const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m,
                              int64_t n, int64_t k, int32_t g, int32_t w_bit, uint16_t* y,
                              void* scratch, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (m >= AWQ_WBIT_GEMM_MIN_M) {
    const uint16_t* xt = x;
    char* sp = static_cast<char*>(scratch);
    if (inv_s16 != nullptr) {
      uint16_t* xs = reinterpret_cast<uint16_t*>(sp);
      sp += align256w((size_t)m * (size_t)k * 2);
      const int64_t chunks = m * (k / 8);
      const int64_t pgrid = (chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096;
      hipLaunchKernelGGL(linear_wbit_xprep_kernel, dim3((unsigned)pgrid), dim3(256), 0, stream, x,
                         inv_s16, m, k, xs);
      xt = xs;
    }
    float* part = reinterpret_cast<float*>(sp);
#define AWQ_LWG(GG, BB) launch_wbit_gemm<GG, BB>(xt, qweight, scales, qzeros, m, n, k, y, part, stream)
    if (w_bit == 8) {
      if (g == 32) AWQ_LWG(32, 8); else if (g == 64) AWQ_LWG(64, 8); else AWQ_LWG(128, 8);
    } else {
      if (g == 32) AWQ_LWG(32, 3); else if (g == 64) AWQ_LWG(64, 3); else AWQ_LWG(128, 3);
    }
#undef AWQ_LWG
    return hipGetLastError();
  }
  switch (w_bit * 1000 + g) {
    case 8032: return launch_wbit_decode<32, 8>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
    case 8064: return launch_wbit_decode<64, 8>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
    case 8128: return launch_wbit_decode<128, 8>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
    case 3032: return launch_wbit_decode<32, 3>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
    case 3064: return launch_wbit_decode<64, 3>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
    default: return launch_wbit_decode<128, 3>(x, qweight, scales, qzeros, inv_s16, m, n, k, y, stream);
  }
}

}  // namespace awq
