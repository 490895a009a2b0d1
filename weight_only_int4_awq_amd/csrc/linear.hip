// W4A16 linear: y = x_tilde W_deq^T with 4-bit group-quantized weights
// (layout v1) and fp16 activations.  bjdmk.com.cn page, section
// "量化参数配置" / "技术选型决策树": a GEMV mode for batch-1 decode and a GEMM
// mode for long inputs; zeeklog.com page: W4A16 kernels; jsqmd.com page,
// section 二.1 (3): the activation is divided by s at inference
// (x_tilde = x * inv_s16).
//
// Decode path, m = 1: linear_gemv (one kernel, activations staged in LDS; see
// below).  Decode path, 2 <= m <= 32: two kernels.
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
// Prefill path (m > 32): linear_gemm (see its comment below).
#include "awq_common.h"
#include "awq_internal.h"
#include "decode_common.h"

namespace awq {

constexpr int kSkinnyTok = 8;          // tokens per 16-row A chunk (hi + lo rows)
constexpr int kSkinnyWaves = 8;        // waves per work-group

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int64_t gemm_row_chunk(int64_t k);

static size_t gemm_part_bytes(int64_t m, int64_t n, int64_t k, int32_t g);

// slot s (0..7) of an 8-channel word in unpack order -> nibble index
__device__ __forceinline__ int slot_nibble(int s) { return (s >> 1) + 4 * (s & 1); }

template <int G>
__global__ __launch_bounds__(256) void linear_prep_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s, int64_t m, int64_t k,
    int64_t n_pairs, uint16_t* __restrict__ a_st, float2* __restrict__ tu, bool bf) {
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
        float xv = h2f(act_h(x[t * k + kw + nib], bf));
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


template <int G, int TC>
__global__ __launch_bounds__(kSkinnyWaves * 64) void linear_skinny_kernel(
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, const uint16_t* __restrict__ a_st,
    const float2* __restrict__ tu, int64_t m, int64_t n, int64_t k, uint16_t* __restrict__ y,
    bool bf) {
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
  const UnpackConsts uc = unpack_consts();

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
      unpack_word(wq[i], u, uc);
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
          if (t < m) y[t * n + col] = f2act(s[i] + o[i], bf);
        }
      }
    }
  }
}


// ---------------------------------------------------------------- linear groups
// The decode kernels take up to kGroupMax independent linears of the same k
// (and m) in one launch: work-groups [wg0[l], wg0[l + 1]) serve linear l,
// each exactly as a launch of that linear alone with wg0[l + 1] - wg0[l]
// work-groups would (the arithmetic of a column block does not depend on the
// grid, so the outputs are the same bits).
struct LinGroup {
  const uint16_t* x[kGroupMax];
  const uint16_t* inv[kGroupMax];
  const uint32_t* qw[kGroupMax];
  const uint16_t* sc[kGroupMax];
  const uint32_t* qz[kGroupMax];
  uint16_t* y[kGroupMax];
  int64_t n[kGroupMax];
  int32_t wg0[kGroupMax + 1];
  int32_t count;
  // prefill GEMM only: slices of K per tile and fp32 partial tiles of the
  // linears split along K (ks = 1: not split)
  int32_t ks[kGroupMax];
  float* part[kGroupMax];
  int32_t gmax;                      // most groups of a K slice (LDS rows)
  int32_t bf;                        // 1: x and y hold bf16 patterns (else fp16)
};
struct LinPick {
  const uint16_t* x;
  const uint16_t* inv;
  const uint32_t* qw;
  const uint16_t* sc;
  const uint32_t* qz;
  uint16_t* y;
  int64_t n;
  int bid, grid;
  int ks;
  float* part;
};
// the linear that work-group (or tile) b of a group launch belongs to, and
// b's index within that linear's range
__device__ __forceinline__ LinPick pick_linear_at(const LinGroup& gp, int b) {
  int li = 0;
#pragma unroll
  for (int i = 1; i < kGroupMax; ++i)
    if (i < gp.count && b >= gp.wg0[i]) li = i;
  LinPick L;
  L.x = gp.x[li];
  L.inv = gp.inv[li];
  L.qw = gp.qw[li];
  L.sc = gp.sc[li];
  L.qz = gp.qz[li];
  L.y = gp.y[li];
  L.n = gp.n[li];
  L.bid = b - gp.wg0[li];
  L.grid = gp.wg0[li + 1] - gp.wg0[li];
  L.ks = gp.ks[li];
  L.part = gp.part[li];
  return L;
}
__device__ __forceinline__ LinPick pick_linear(const LinGroup& gp) {
  return pick_linear_at(gp, (int)blockIdx.x);
}

// ---------------------------------------------------------------- decode GEMV (m = 1)
// Work-groups of W = 8 or 16 waves (16 where one work-group per CU is all
// that fits or is needed, so that as many weight bytes are in flight per CU);
// work-group b owns the 16-column blocks b, b + grid,
// ... (at most kGemvMaxBlk of them: the grid is sized for that).
//  * Prologue.  Every load is issued before the first wait, in the order the
//    data is needed: the scale and zero words of all the work-group's blocks,
//    the activations (x and inv_s), then the first kGemvPF weight items of
//    every wave.  The activations are staged in LDS as rows 0 (fp16 hi) and 8
//    (fp16 lo) of the MFMA A operand (the other 14 rows read a zero block),
//    with the per-group offset sums T and U; the scales and zero points as
//    packed words (fp16 scale | zero << 16) laid out [block][group][column].
//  * Main loop.  Every wave owns a contiguous range of groups along K and walks
//    the flattened sequence (block, group) with a double-buffered prefetch of
//    packed weights that runs across block boundaries.  Weight loads are the
//    only memory instructions in the loop: memory counters retire in order,
//    and a load or store of anything else there (behind the branch of a block
//    end) would make the compiler wait for the whole prefetch.
//  * At the end of a block the waves meet at one barrier and a designated wave
//    sums the W partial rows in a fixed order into an LDS output row; the
//    outputs are written after the last block.
#ifndef AWQ_GEMV_PF
#define AWQ_GEMV_PF 4
#endif
constexpr int kGemvPF = AWQ_GEMV_PF;
constexpr int kGemvCUs = 256;
constexpr int kGemvMaxBlk = 4;         // column blocks per work-group
constexpr int kGemvSzRounds = 4;       // scale/zero octets per thread in the prologue
constexpr int kGemvXPre = 4;           // activation chunks per thread loaded up front

// LDS: x_tilde [ng][4][2][g/4] halves, T/U [ng] float4, zero block [g/4]
// halves, scale|zero words [nb][ng][16], partial rows [nb][W][16] floats.
size_t gemv_lds_bytes(int64_t k, int32_t g, int nb, int waves) {
  const size_t ng = (size_t)(k / g);
  return (size_t)k * 4 + ng * 16 + (size_t)(g / 4) * 2 + (size_t)nb * ng * 16 * 4 +
         (size_t)nb * waves * 16 * 4;
}

template <int WPL>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&w)[WPL]) {
  if constexpr (WPL == 4) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (WPL == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *p;
  }
}

// SZV: the scale rows are 16-byte aligned octets (k / g a multiple of 8 and an
// aligned base), read with one 16-byte load per octet.
template <int G, bool SZV, int W>
__device__ __forceinline__ void gemv_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t n, int64_t k, uint16_t* __restrict__ y,
    int bid, int grid_in, bool bf) {
  constexpr int WPL = G / 32;            // qweight words per lane per group
  constexpr int HPL = G / 4;             // staged halves per (group, lane group, row)
  constexpr int LPG = G / 8;             // words per group
  constexpr int kGemvWaves = W;
  constexpr int kGemvThreads = W * 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ng = (int)(k / G);
  const int nblk = (int)((n + 15) / 16);
  const int grid = grid_in;
  const int my_blocks = (nblk - bid + grid - 1) / grid;   // 1 .. kGemvMaxBlk
  unsigned char* sp = smem;
  uint16_t* xa = reinterpret_cast<uint16_t*>(sp);          sp += (size_t)k * 4;     // [ng][4][2][HPL]
  float4* tu = reinterpret_cast<float4*>(sp);              sp += (size_t)ng * 16;   // (T_hi, U_hi, T_lo, U_lo)
  uint16_t* zblk = reinterpret_cast<uint16_t*>(sp);        sp += HPL * 2;           // zeros
  uint32_t* szw = reinterpret_cast<uint32_t*>(sp);         sp += (size_t)my_blocks * ng * 16 * 4;
  float* red = reinterpret_cast<float*>(sp);               // [nb][W][16] partial rows

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave: keep it (and every group index
  // and group base address derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int jb = ng * wave / kGemvWaves, je = ng * (wave + 1) / kGemvWaves;
  const int cnt = je - jb;                            // groups of this wave per block
  const int total = my_blocks * cnt;                  // (block, group) items of this wave
  const int nzw = (ng + 7) / 8, kw_row = (int)(k / 8);

  // ---- 1. scale and zero words of every block of the work-group.  Octet o
  // (8 groups of one column) of block slot bs: o = (bs * 16 + row) * nzw + oct.
  // These loads are lane-predicated; they come first, so that the waits for
  // the loads after them stay exact.
  const int n_oct = my_blocks * 16 * nzw;
  uint4 sz_s[kGemvSzRounds];
  uint32_t sz_z[kGemvSzRounds];
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    sz_s[i] = make_uint4(0, 0, 0, 0);
    sz_z[i] = 0;
    const int o = tid + i * kGemvThreads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      int col = (bid + bs * grid) * 16 + row;
      col = col < (int)n ? col : (int)n - 1;
      const uint16_t* srow = scales + (int64_t)col * ng + oct * 8;
      if constexpr (SZV) {
        sz_s[i] = *reinterpret_cast<const uint4*>(srow);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (oct * 8 + e < ng) ? srow[e] : (uint16_t)0;
        sz_s[i] = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                             h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
      sz_z[i] = qzeros[(int64_t)col * nzw + oct];
    }
  }

  // ---- 2. activations: chunk i of thread t is the 8 channels of word
  // t + 512 i.  Clamped indices: the loads are unconditional.
  const bool has_inv = inv_s != nullptr;
  const uint16_t* sbase = has_inv ? inv_s : x;        // any readable row when inv_s is absent
  uint4 xv[kGemvXPre], sv[kGemvXPre];
#pragma unroll
  for (int i = 0; i < kGemvXPre; ++i) { xv[i] = make_uint4(0, 0, 0, 0); sv[i] = xv[i]; }
  {
    const int wi = tid < kw_row ? tid : kw_row - 1;
    xv[0] = *reinterpret_cast<const uint4*>(x + (int64_t)wi * 8);
    sv[0] = *reinterpret_cast<const uint4*>(sbase + (int64_t)wi * 8);
  }
  if (kw_row > kGemvThreads) {                        // uniform
#pragma unroll
    for (int i = 1; i < kGemvXPre; ++i) {
      int wi = tid + i * kGemvThreads;
      wi = wi < kw_row ? wi : kw_row - 1;
      xv[i] = *reinterpret_cast<const uint4*>(x + (int64_t)wi * 8);
      sv[i] = *reinterpret_cast<const uint4*>(sbase + (int64_t)wi * 8);
    }
  }

  // ---- 3. first weights.  Prefetch slots hold raw loaded bits only
  // (converting at issue time would make the wave wait there), every load is
  // unconditional (the cursor stops on the last item, the column and group are
  // clamped), and the (block, group) cursors advance in scalar registers.
  uint32_t wq[2 * kGemvPF][WPL];
  const char* qbase = reinterpret_cast<const char*>(qweight);
  int i_blk = bid, i_j = jb, i_left = total;    // issue cursor
  auto issue = [&](int slot) {
    int col = i_blk * 16 + r;
    col = col < (int)n ? col : (int)n - 1;
    // 32-bit per-lane byte offset (the packed tensors of one call are below 4 GiB)
    uint32_t qoff = ((uint32_t)col * (uint32_t)kw_row + (uint32_t)(WPL * c)) * 4u;
    // opaque to the optimiser: a clamped cursor repeats an address, and the
    // compiler would otherwise replace that load by a copy of the previous
    // slot behind a branch and a full wait
    asm volatile("" : "+v"(qoff));
    const int jj = i_j < ng ? i_j : ng - 1;
    load_words<WPL>(reinterpret_cast<const uint32_t*>(qbase + (int64_t)jj * (LPG * 4) + qoff), wq[slot]);
    if (i_left > 1) {
      --i_left;
      if (++i_j == je) { i_j = jb; i_blk += grid; }
    }
  };
#pragma unroll
  for (int p = 0; p < kGemvPF; ++p) issue(p);         // a wave without groups loads group ng - 1

  // ---- 4. stage x_tilde (hi, lo) and the offset sums in LDS
  if (tid < HPL / 2) reinterpret_cast<uint32_t*>(zblk)[tid] = 0u;
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  auto stage = [&](int wi, const uint4& xraw, const uint4& sq) {
    const uint4 sv_ = has_inv ? sq : ones;
    const uint4 xq = act8_h(xraw, bf);
    const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w};
    const uint32_t sw[4] = {sv_.x, sv_.y, sv_.z, sv_.w};
    // hi = fp16_rn(x s) (v_pk_mul_f16) and lo = fp16_rn(x s - hi)
    // (v_pk_fma_f16): each is one rounding of an exact value, and
    // x_tilde = hi + lo to about 22 bits.  T and U accumulate in fp32 with
    // v_dot2 against (1024, 64) and (1, 1): channels 2i and 2i + 1 of a pair
    // carry the unpack offsets 1024 and 64.
    const half2_t one2 = {(half_t)1.0f, (half_t)1.0f};
    const half2_t off2 = {(half_t)1024.0f, (half_t)64.0f};
    uint32_t hw[4], lw[4];
    float th = 0.f, uh = 0.f, tl = 0.f, ul = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t xx = __builtin_bit_cast(half2_t, xw[i]);
      const half2_t ss = __builtin_bit_cast(half2_t, sw[i]);
      const half2_t h = xx * ss;
      const half2_t l = __builtin_elementwise_fma(xx, ss, -h);
      hw[i] = __builtin_bit_cast(uint32_t, h);
      lw[i] = __builtin_bit_cast(uint32_t, l);
      uh = dot2_f16(h, one2, uh);
      th = dot2_f16(h, off2, th);
      ul = dot2_f16(l, one2, ul);
      tl = dot2_f16(l, off2, tl);
    }
    const int j = wi / LPG;
    const int wg = wi % LPG;
    const int cc = wg / WPL, i = wg % WPL;
    uint16_t* dh = xa + ((j * 4 + cc) * 2 + 0) * HPL + i * 8;
    uint16_t* dl = xa + ((j * 4 + cc) * 2 + 1) * HPL + i * 8;
    // slot order (k0, k4, k1, k5, k2, k6, k3, k7) matches unpack_word
    uint4 vh, vl;
    vh.x = __builtin_amdgcn_perm(hw[2], hw[0], 0x05040100u);
    vh.y = __builtin_amdgcn_perm(hw[2], hw[0], 0x07060302u);
    vh.z = __builtin_amdgcn_perm(hw[3], hw[1], 0x05040100u);
    vh.w = __builtin_amdgcn_perm(hw[3], hw[1], 0x07060302u);
    vl.x = __builtin_amdgcn_perm(lw[2], lw[0], 0x05040100u);
    vl.y = __builtin_amdgcn_perm(lw[2], lw[0], 0x07060302u);
    vl.z = __builtin_amdgcn_perm(lw[3], lw[1], 0x05040100u);
    vl.w = __builtin_amdgcn_perm(lw[3], lw[1], 0x07060302u);
    *reinterpret_cast<uint4*>(dh) = vh;
    *reinterpret_cast<uint4*>(dl) = vl;
    // the LPG words of a group sit in LPG consecutive, aligned lanes, all
    // active or all inactive together (kw_row and the thread count are
    // multiples of LPG)
    th = row_group_sum<LPG>(th); uh = row_group_sum<LPG>(uh);
    tl = row_group_sum<LPG>(tl); ul = row_group_sum<LPG>(ul);
    if (wg == 0) tu[j] = make_float4(th, uh, tl, ul);
  };
#pragma unroll
  for (int i = 0; i < kGemvXPre; ++i) {
    const int wi = tid + i * kGemvThreads;
    if (wi < kw_row) stage(wi, xv[i], sv[i]);
  }
  for (int wi = tid + kGemvXPre * kGemvThreads; wi < kw_row; wi += kGemvThreads) {
    const uint4 xq = *reinterpret_cast<const uint4*>(x + (int64_t)wi * 8);
    const uint4 sq = *reinterpret_cast<const uint4*>(sbase + (int64_t)wi * 8);
    stage(wi, xq, sq);
  }

  // ---- 5. scale|zero words into LDS
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    const int o = tid + i * kGemvThreads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      const uint32_t sw[4] = {sz_s[i].x, sz_s[i].y, sz_s[i].z, sz_s[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = oct * 8 + e;
        if (j < ng)
          szw[((size_t)bs * ng + j) * 16 + row] =
              ((sw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) | (((sz_z[i] >> (4 * e)) & 0xFu) << 16);
      }
    }
  }
  __syncthreads();

  // rows 0 (hi) and 8 (lo) of the A operand are live; the others read zeros
  const int part = r >> 3;
  const bool arow = (r == 0) || (r == 8);
  const uint32_t a_lane = arow ? (uint32_t)(((c * 2 + part) * HPL) * 2) : 0u;
  const char* a_base = arow ? reinterpret_cast<const char*>(xa) : reinterpret_cast<const char*>(zblk);
  const uint32_t a_step = arow ? (uint32_t)(4 * 2 * HPL * 2) : 0u;      // bytes per group
  const char* tu_lane = reinterpret_cast<const char*>(tu) + ((c >= 2) ? 8 : 0);
  const int reducer = kGemvWaves - 1;                 // always owns at least one group
  const UnpackConsts uc = unpack_consts();
  float yacc = 0.0f;
  int blocks_done = 0;

  // end of a column block: combine the hi + lo rows into the wave's partial
  // row of the block (LDS; each block has its own rows, so no wave waits for
  // another until all blocks are done)
  auto finish_block = [&]() {
    const float other = __shfl_xor(yacc, 32, 64);
    if (lane < 16) red[(blocks_done * kGemvWaves + wave) * 16 + lane] = yacc + other;
    yacc = 0.0f;
    ++blocks_done;
  };
  int c_j = jb, c_left = total;                       // consume cursor
  // GUARDED only in the tail: a consume skipped behind a branch would leave
  // its slot's loads pending in the compiler's view, and the next reuse of
  // those registers would then wait for every outstanding load
  auto consume = [&](int p, bool guarded) {
    if (!guarded || c_left > 0) {                     // wave-uniform
      const int j = c_j;
      const char* asrc = a_base + a_lane + (uint32_t)j * a_step;
      half8_t aop[WPL];
#pragma unroll
      for (int i = 0; i < WPL; ++i) aop[i] = *reinterpret_cast<const half8_t*>(asrc + 16 * i);
      const float2 tv = *reinterpret_cast<const float2*>(tu_lane + (uint32_t)j * 16);
      const uint32_t szv = szw[((size_t)blocks_done * ng + j) * 16 + r];
      floatx4_t cacc = floatx4_t{};
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        uint32_t u[4];
        unpack_word(wq[p][i], u, uc);
        const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(u[0], u[1], u[2], u[3]));
        cacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[i], bop, cacc, 0, 0, 0);
      }
      // lanes with c >= 2 hold the lo row and read (T_lo, U_lo)
      const float zf = (float)(szv >> 16);
      yacc = __builtin_fmaf(h2f((uint16_t)szv), __builtin_fmaf(-zf, tv.y, cacc[0] - tv.x), yacc);
      --c_left;
      if (++c_j == je) {
        finish_block();
        c_j = jb;
      }
    }
  };
  if (cnt > 0) {
    // Half A (slots 0..PF-1) is in flight on entry.  The next half is issued
    // only while items remain beyond the current one, so no load outlives the
    // last item; the branches are wave-uniform and each path has a fixed
    // number of loads in flight at every wait.
    int left = total;
    while (true) {
      if (left > kGemvPF) {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) issue(kGemvPF + p);
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(p, false);
        left -= kGemvPF;
      } else {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(p, true);
        break;
      }
      if (left > kGemvPF) {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) issue(p);
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(kGemvPF + p, false);
        left -= kGemvPF;
      } else {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(kGemvPF + p, true);
        break;
      }
    }
  } else {
    // a wave without groups (fewer than W groups in k) still meets every block's barrier
    for (int bi = 0; bi < my_blocks; ++bi) finish_block();
  }

  // ---- outputs: one barrier, then the reducer wave sums each block's W
  // partial rows in wave order and stores the block
  __syncthreads();
  if (wave == reducer && lane < 16) {
    for (int bi = 0; bi < my_blocks; ++bi) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kGemvWaves; ++wv) sum += red[(bi * kGemvWaves + wv) * 16 + lane];
      const int64_t col = ((int64_t)bid + (int64_t)bi * grid) * 16 + lane;
      if (col < n) y[col] = f2act(sum, bf);
    }
  }
}

template <int G, bool SZV, int W>
__global__ __launch_bounds__(W * 64, 2) void linear_gemv_kernel(const LinGroup gp, int64_t k) {
  const LinPick L = pick_linear(gp);
  gemv_body<G, SZV, W>(L.x, L.inv, L.qw, L.sc, L.qz, L.n, k, L.y, L.bid, L.grid, gp.bf != 0);
}

// ---------------------------------------------------------------- decode GEMV, 2 <= m <= 8
// The decode GEMV with the tokens as rows 0 .. m-1 of the MFMA A operand
// (x_tilde = fp16_rn(x inv_s), one rounding, as in the skinny kernels; rows
// m .. 15 read the zero block), staged once per work-group in LDS as
// [group][lane group c][token][g/4 halves] with the offset sums T, U per
// (group, token) in [group][16] float pairs.  Weights, scales and the
// (block, group) walk of every wave are the decode GEMV's.  Lane (c, r) holds
// rows 4c .. 4c + 3 of column r of the MFMA result, and per item adds
// D (C_t - T_t - z U_t) for each of them (rows past m are never stored).  At
// the end of a block a wave writes its partial rows to LDS as
// [block][wave][column][8 tokens]; after the loop every thread sums one
// output over the waves in wave order.
constexpr int kRowsMaxBlk = 8;         // column blocks per work-group
constexpr int kRowsMaxTok = 8;

size_t gemv_rows_lds_bytes(int64_t k, int32_t g, int64_t m, int nb, int waves) {
  const size_t ng = (size_t)(k / g);
  return (size_t)k * (size_t)m * 2 + ng * 16 * 8 + (size_t)(g / 4) * 2 + (size_t)nb * ng * 16 * 4 +
         (size_t)nb * waves * 16 * kRowsMaxTok * 4;
}

template <int G, bool SZV, int W>
__device__ __forceinline__ void gemv_rows_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t n, int64_t k, int64_t m_in,
    uint16_t* __restrict__ y, int bid, int grid, bool bf) {
  constexpr int WPL = G / 32, HPL = G / 4, LPG = G / 8;
  constexpr int kThreads = W * 64;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int m = (int)m_in;                              // 2 .. 8
  const int ng = (int)(k / G);
  const int nblk = (int)((n + 15) / 16);
  const int my_blocks = (nblk - bid + grid - 1) / grid;   // 1 .. kRowsMaxBlk
  unsigned char* sp = smem;
  uint16_t* xa = reinterpret_cast<uint16_t*>(sp);      sp += (size_t)k * m * 2;      // [ng][4][m][HPL]
  float2* tu = reinterpret_cast<float2*>(sp);          sp += (size_t)ng * 16 * 8;    // [ng][16] (T, U)
  uint16_t* zblk = reinterpret_cast<uint16_t*>(sp);    sp += HPL * 2;
  uint32_t* szw = reinterpret_cast<uint32_t*>(sp);     sp += (size_t)my_blocks * ng * 16 * 4;
  float* red = reinterpret_cast<float*>(sp);           // [nb][W][16][kRowsMaxTok]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int jb = ng * wave / W, je = ng * (wave + 1) / W;
  const int cnt = je - jb;
  const int total = my_blocks * cnt;
  const int nzw = (ng + 7) / 8, kw_row = (int)(k / 8);

  // ---- 1. scale and zero words of every block (lane-predicated, first)
  const int n_oct = my_blocks * 16 * nzw;
  uint4 sz_s[kGemvSzRounds];
  uint32_t sz_z[kGemvSzRounds];
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    sz_s[i] = make_uint4(0, 0, 0, 0);
    sz_z[i] = 0;
    const int o = tid + i * kThreads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      int col = (bid + bs * grid) * 16 + row;
      col = col < (int)n ? col : (int)n - 1;
      const uint16_t* srow = scales + (int64_t)col * ng + oct * 8;
      if constexpr (SZV) {
        sz_s[i] = *reinterpret_cast<const uint4*>(srow);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (oct * 8 + e < ng) ? srow[e] : (uint16_t)0;
        sz_s[i] = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                             h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
      sz_z[i] = qzeros[(int64_t)col * nzw + oct];
    }
  }

  // ---- 2. activations: item i of thread t is word (t + threads i) of the
  // m rows, row-major (clamped: the loads are unconditional)
  const int n_items = m * kw_row;
  const bool has_inv = inv_s != nullptr;
  const uint16_t* sbase = has_inv ? inv_s : x;
  uint4 xv[kGemvXPre], sv[kGemvXPre];
#pragma unroll
  for (int i = 0; i < kGemvXPre; ++i) {
    int it = tid + i * kThreads;
    it = it < n_items ? it : n_items - 1;
    const int t = it / kw_row, wi = it - t * kw_row;
    xv[i] = *reinterpret_cast<const uint4*>(x + (int64_t)t * k + (int64_t)wi * 8);
    sv[i] = *reinterpret_cast<const uint4*>(sbase + (int64_t)wi * 8);
  }

  // ---- 3. first weights (as in the decode GEMV)
  uint32_t wq[2 * kGemvPF][WPL];
  const char* qbase = reinterpret_cast<const char*>(qweight);
  int i_blk = bid, i_j = jb, i_left = total;
  auto issue = [&](int slot) {
    int col = i_blk * 16 + r;
    col = col < (int)n ? col : (int)n - 1;
    uint32_t qoff = ((uint32_t)col * (uint32_t)kw_row + (uint32_t)(WPL * c)) * 4u;
    asm volatile("" : "+v"(qoff));
    const int jj = i_j < ng ? i_j : ng - 1;
    load_words<WPL>(reinterpret_cast<const uint32_t*>(qbase + (int64_t)jj * (LPG * 4) + qoff), wq[slot]);
    if (i_left > 1) {
      --i_left;
      if (++i_j == je) { i_j = jb; i_blk += grid; }
    }
  };
#pragma unroll
  for (int p = 0; p < kGemvPF; ++p) issue(p);

  // ---- 4. stage x_tilde and the offset sums
  if (tid < HPL / 2) reinterpret_cast<uint32_t*>(zblk)[tid] = 0u;
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  auto stage = [&](int it, const uint4& xraw, const uint4& sq) {
    const int t = it / kw_row, wi = it - t * kw_row;
    const uint4 sv_ = has_inv ? sq : ones;
    const uint4 xq = act8_h(xraw, bf);
    const uint32_t xw[4] = {xq.x, xq.y, xq.z, xq.w};
    const uint32_t sw[4] = {sv_.x, sv_.y, sv_.z, sv_.w};
    const half2_t one2 = {(half_t)1.0f, (half_t)1.0f};
    const half2_t off2 = {(half_t)1024.0f, (half_t)64.0f};
    uint32_t hw[4];
    float th = 0.f, uh = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t h = __builtin_bit_cast(half2_t, xw[i]) * __builtin_bit_cast(half2_t, sw[i]);
      hw[i] = __builtin_bit_cast(uint32_t, h);
      uh = dot2_f16(h, one2, uh);
      th = dot2_f16(h, off2, th);
    }
    const int j = wi / LPG;
    const int wg = wi % LPG;
    const int cc = wg / WPL, i = wg % WPL;
    uint4 vh;
    vh.x = __builtin_amdgcn_perm(hw[2], hw[0], 0x05040100u);
    vh.y = __builtin_amdgcn_perm(hw[2], hw[0], 0x07060302u);
    vh.z = __builtin_amdgcn_perm(hw[3], hw[1], 0x05040100u);
    vh.w = __builtin_amdgcn_perm(hw[3], hw[1], 0x07060302u);
    *reinterpret_cast<uint4*>(xa + ((size_t)(j * 4 + cc) * m + t) * HPL + i * 8) = vh;
    // the LPG words of a group are LPG consecutive, aligned lanes of one row
    th = row_group_sum<LPG>(th);
    uh = row_group_sum<LPG>(uh);
    if (wg == 0) tu[j * 16 + t] = make_float2(th, uh);
  };
#pragma unroll
  for (int i = 0; i < kGemvXPre; ++i) {
    const int it = tid + i * kThreads;
    if (it < n_items) stage(it, xv[i], sv[i]);
  }
  for (int it = tid + kGemvXPre * kThreads; it < n_items; it += kThreads) {
    const int t = it / kw_row, wi = it - t * kw_row;
    const uint4 xq = *reinterpret_cast<const uint4*>(x + (int64_t)t * k + (int64_t)wi * 8);
    const uint4 sq = *reinterpret_cast<const uint4*>(sbase + (int64_t)wi * 8);
    stage(it, xq, sq);
  }

  // ---- 5. scale|zero words into LDS
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    const int o = tid + i * kThreads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      const uint32_t sw[4] = {sz_s[i].x, sz_s[i].y, sz_s[i].z, sz_s[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = oct * 8 + e;
        if (j < ng)
          szw[((size_t)bs * ng + j) * 16 + row] =
              ((sw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) | (((sz_z[i] >> (4 * e)) & 0xFu) << 16);
      }
    }
  }
  __syncthreads();

  const bool arow = r < m;
  const uint32_t a_lane = arow ? (uint32_t)((c * m + r) * HPL * 2) : 0u;
  const char* a_base = arow ? reinterpret_cast<const char*>(xa) : reinterpret_cast<const char*>(zblk);
  const uint32_t a_step = arow ? (uint32_t)(4 * m * HPL * 2) : 0u;      // bytes per group
  const char* tu_lane = reinterpret_cast<const char*>(tu) + c * 32;
  const UnpackConsts uc = unpack_consts();
  float yacc[4] = {0.f, 0.f, 0.f, 0.f};
  int blocks_done = 0;
  auto finish_block = [&]() {
    if (c < 2)
      *reinterpret_cast<float4*>(red + (((size_t)blocks_done * W + wave) * 16 + r) * kRowsMaxTok + 4 * c) =
          make_float4(yacc[0], yacc[1], yacc[2], yacc[3]);
    yacc[0] = yacc[1] = yacc[2] = yacc[3] = 0.f;
    ++blocks_done;
  };
  int c_j = jb, c_left = total;
  auto consume = [&](int p, bool guarded) {
    if (!guarded || c_left > 0) {
      const int j = c_j;
      const char* asrc = a_base + a_lane + (uint32_t)j * a_step;
      half8_t aop[WPL];
#pragma unroll
      for (int i = 0; i < WPL; ++i) aop[i] = *reinterpret_cast<const half8_t*>(asrc + 16 * i);
      const float4 t01 = *reinterpret_cast<const float4*>(tu_lane + (uint32_t)j * 128);
      const float4 t23 = *reinterpret_cast<const float4*>(tu_lane + (uint32_t)j * 128 + 16);
      const uint32_t szv = szw[((size_t)blocks_done * ng + j) * 16 + r];
      floatx4_t cacc = floatx4_t{};
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        uint32_t u[4];
        unpack_word(wq[p][i], u, uc);
        const half8_t bop = __builtin_bit_cast(half8_t, make_uint4(u[0], u[1], u[2], u[3]));
        cacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[i], bop, cacc, 0, 0, 0);
      }
      const float d = h2f((uint16_t)szv), zf = (float)(szv >> 16);
      const float c0 = cacc[0], c1 = cacc[1], c2 = cacc[2], c3 = cacc[3];
      yacc[0] = __builtin_fmaf(d, __builtin_fmaf(-zf, t01.y, c0 - t01.x), yacc[0]);
      yacc[1] = __builtin_fmaf(d, __builtin_fmaf(-zf, t01.w, c1 - t01.z), yacc[1]);
      yacc[2] = __builtin_fmaf(d, __builtin_fmaf(-zf, t23.y, c2 - t23.x), yacc[2]);
      yacc[3] = __builtin_fmaf(d, __builtin_fmaf(-zf, t23.w, c3 - t23.z), yacc[3]);
      --c_left;
      if (++c_j == je) {
        finish_block();
        c_j = jb;
      }
    }
  };
  if (cnt > 0) {
    int left = total;
    while (true) {
      if (left > kGemvPF) {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) issue(kGemvPF + p);
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(p, false);
        left -= kGemvPF;
      } else {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(p, true);
        break;
      }
      if (left > kGemvPF) {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) issue(p);
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(kGemvPF + p, false);
        left -= kGemvPF;
      } else {
#pragma unroll
        for (int p = 0; p < kGemvPF; ++p) consume(kGemvPF + p, true);
        break;
      }
    }
  } else {
    for (int bi = 0; bi < my_blocks; ++bi) finish_block();
  }

  // ---- outputs: every thread sums outputs (block, token, column) over the
  // waves in wave order
  __syncthreads();
  const int n_out = my_blocks * m * 16;
  for (int o = tid; o < n_out; o += kThreads) {
    const int bs = o / (m * 16), rem = o - bs * (m * 16);
    const int t = rem >> 4, cl = rem & 15;
    float sum = 0.0f;
#pragma unroll
    for (int wv = 0; wv < W; ++wv) sum += red[(((size_t)bs * W + wv) * 16 + cl) * kRowsMaxTok + t];
    const int64_t col = ((int64_t)bid + (int64_t)bs * grid) * 16 + cl;
    if (col < n) y[(int64_t)t * n + col] = f2act(sum, bf);
  }
}

template <int G, bool SZV, int W>
__global__ __launch_bounds__(W * 64, W == 16 ? 1 : 2) void linear_gemv_rows_kernel(const LinGroup gp, int64_t m, int64_t k) {
  const LinPick L = pick_linear(gp);
  gemv_rows_body<G, SZV, W>(L.x, L.inv, L.qw, L.sc, L.qz, L.n, k, m, L.y, L.bid, L.grid, gp.bf != 0);
}

// ---------------------------------------------------------------- skinny, 2 <= m <= 32
// linear_prep16 writes x_tilde = fp16_rn(x * inv_s) once per call as the MFMA
// A operand, 16 tokens per chunk (one chunk for m <= 16, two for m <= 32):
// [chunk][group][lane group c][row][g/4 halves], channels of every 8-channel
// word in the nibble-unpack order, plus the offset sums T, U per (chunk,
// group, row).  linear_skinny16 follows the decode GEMV: 8 waves split K,
// 16-column blocks (up to 4 per work-group), scale|zero words and the offset
// sums staged in LDS up front, each wave's (block, group) items prefetched
// with their weight words and activation fragments (unconditional loads, so
// the waits stay exact), one barrier per block and outputs stored at the end.
template <int G>
__global__ __launch_bounds__(256) void linear_prep16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s, int64_t m, int64_t k,
    int64_t n_pairs, uint16_t* __restrict__ a16, float2* __restrict__ tu16, bool bf) {
  constexpr int WPL = G / 32, HPL = G / 4;
  const int64_t ng = k / G;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (chunk, group)
  if (pair >= n_pairs) return;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c = lane >> 4;
  const int64_t tc = pair / ng, j = pair % ng;
  const int64_t t = tc * 16 + r;
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
        float xv = h2f(act_h(x[t * k + kw + nib], bf));
        if (inv_s != nullptr) xv *= h2f(inv_s[kw + nib]);   // exact: fp16 x fp16
        h = f2h_rn(xv);
      }
      vals[i * 8 + s] = h;
      const double hv = (double)h2f(h);
      usum += hv;
      tsum += hv * ((nib & 1) ? 64.0 : 1024.0);
    }
  }
  uint16_t* dst = a16 + ((pair * 4 + c) * 16 + r) * HPL;
#pragma unroll
  for (int i = 0; i < HPL; i += 8) {
    uint4 v;
    v.x = (uint32_t)vals[i + 0] | ((uint32_t)vals[i + 1] << 16);
    v.y = (uint32_t)vals[i + 2] | ((uint32_t)vals[i + 3] << 16);
    v.z = (uint32_t)vals[i + 4] | ((uint32_t)vals[i + 5] << 16);
    v.w = (uint32_t)vals[i + 6] | ((uint32_t)vals[i + 7] << 16);
    *reinterpret_cast<uint4*>(dst + i) = v;
  }
  tsum += shfl_xor_d(tsum, 16);
  tsum += shfl_xor_d(tsum, 32);
  usum += shfl_xor_d(usum, 16);
  usum += shfl_xor_d(usum, 32);
  if (c == 0) tu16[pair * 16 + r] = make_float2((float)tsum, (float)usum);
}

constexpr int kSk16Waves = 8;
constexpr int kSk16Threads = kSk16Waves * 64;

// LDS: scale|zero words [nb][ng][16], offset sums [tc][ng][16] float2 (rounded
// up to whole 1 KiB copies), reduction rows [2][8][tc][64] float4, outputs
// [nb][tc][64] float4.
size_t skinny16_lds_bytes(int64_t k, int32_t g, int nb, int tc) {
  const size_t ng = (size_t)(k / g);
  const size_t tu = ((size_t)tc * ng * 16 * 8 + 1023) & ~(size_t)1023;
  return (size_t)nb * ng * 16 * 4 + tu + (size_t)2 * kSk16Waves * tc * 64 * 16 +
         (size_t)nb * tc * 64 * 16;
}

template <int G, int TC, bool SZV, int PF>
__global__ __launch_bounds__(kSk16Threads, 4) void linear_skinny16_kernel(
    const uint16_t* __restrict__ a16, const float2* __restrict__ tu16,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y, bool bf) {
  constexpr int WPL = G / 32, HPL = G / 4, LPG = G / 8;
  constexpr int W = kSk16Waves;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ng = (int)(k / G);
  const int nblk = (int)((n + 15) / 16);
  const int grid = (int)gridDim.x;
  const int my_blocks = (nblk - (int)blockIdx.x + grid - 1) / grid;   // 1 .. kGemvMaxBlk
  const size_t tu_bytes = ((size_t)TC * ng * 16 * 8 + 1023) & ~(size_t)1023;
  unsigned char* sp = smem;
  uint32_t* szw = reinterpret_cast<uint32_t*>(sp);   sp += (size_t)my_blocks * ng * 16 * 4;
  float2* tu_l = reinterpret_cast<float2*>(sp);      sp += tu_bytes;
  floatx4_t* red = reinterpret_cast<floatx4_t*>(sp); sp += (size_t)2 * W * TC * 64 * 16;
  floatx4_t* ybuf = reinterpret_cast<floatx4_t*>(sp);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int jb = ng * wave / W, je = ng * (wave + 1) / W;
  const int cnt = je - jb;
  const int total = my_blocks * cnt;
  const int nzw = (ng + 7) / 8, kw_row = (int)(k / 8);

  // ---- 1. offset sums: straight global -> LDS copies of 1 KiB per wave
  // instruction (lane i copies 16 bytes; the tail is clamped to the last
  // 16 bytes of the source and lands in the rounded-up LDS pad)
  {
    typedef __attribute__((address_space(3))) void lds_void_t;
    const int64_t src_bytes = (int64_t)TC * ng * 16 * 8;
    const char* srcb = reinterpret_cast<const char*>(tu16);
    const int n_copy = (int)(tu_bytes / 1024);
    for (int i = wave; i < n_copy; i += W) {
      int64_t off = (int64_t)i * 1024 + lane * 16;
      off = off + 16 <= src_bytes ? off : src_bytes - 16;
      __builtin_amdgcn_global_load_lds((const void*)(srcb + off),
                                       (lds_void_t*)(reinterpret_cast<char*>(tu_l) + i * 1024),
                                       16, 0, 0);
    }
  }
  // ---- 2. scale and zero words of every block (lane-predicated, first)
  const int n_oct = my_blocks * 16 * nzw;
  uint4 sz_s[kGemvSzRounds];
  uint32_t sz_z[kGemvSzRounds];
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    sz_s[i] = make_uint4(0, 0, 0, 0);
    sz_z[i] = 0;
    const int o = tid + i * kSk16Threads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      int col = ((int)blockIdx.x + bs * grid) * 16 + row;
      col = col < (int)n ? col : (int)n - 1;
      const uint16_t* srow = scales + (int64_t)col * ng + oct * 8;
      if constexpr (SZV) {
        sz_s[i] = *reinterpret_cast<const uint4*>(srow);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (oct * 8 + e < ng) ? srow[e] : (uint16_t)0;
        sz_s[i] = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                             h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
      sz_z[i] = qzeros[(int64_t)col * nzw + oct];
    }
  }

  // ---- 3. first items: weight words and activation fragments (unconditional
  // buffer loads; a lane past the last column reads zeros)
  uint32_t wq[2 * PF][WPL];
  uint4 aq[2 * PF][TC][WPL];          // raw bits, like the weight words
  const __amdgpu_buffer_rsrc_t rs_w = buf_rsrc(qweight, (uint32_t)((uint64_t)n * (uint64_t)k / 2));
  const __amdgpu_buffer_rsrc_t rs_a = buf_rsrc(a16, (uint32_t)((uint64_t)TC * (uint64_t)k * 32));
  // the row (which decides whether a load is past the end) is in the VGPR
  // offset, the group along K in the scalar one
  const uint32_t w_voff = ((uint32_t)r * (uint32_t)kw_row + (uint32_t)(WPL * c)) * 4u;
  const uint32_t a_voff = (uint32_t)((c * 16 + r) * HPL) * 2u;
  int i_blk = (int)blockIdx.x, i_j = jb, i_left = total;
  auto issue = [&](int slot) {
    const int jj = i_j < ng ? i_j : ng - 1;
    const uint32_t wvo = w_voff + (uint32_t)i_blk * 16u * (uint32_t)kw_row * 4u;
    buf_words<WPL>(rs_w, wvo, (uint32_t)(jj * LPG) * 4u, wq[slot]);
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      const uint32_t aso = (uint32_t)((tc * ng + jj) * 64 * HPL) * 2u;
#pragma unroll
      for (int i = 0; i < WPL; ++i)
        aq[slot][tc][i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_voff + 16u * i, aso, 0));
    }
    if (i_left > 1) {
      --i_left;
      if (++i_j == je) { i_j = jb; i_blk += grid; }
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p);

  // ---- 4. scale|zero words into LDS as [block][group][column]
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    const int o = tid + i * kSk16Threads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      const uint32_t sw[4] = {sz_s[i].x, sz_s[i].y, sz_s[i].z, sz_s[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = oct * 8 + e;
        if (j < ng)
          szw[((size_t)bs * ng + j) * 16 + row] =
              ((sw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) | (((sz_z[i] >> (4 * e)) & 0xFu) << 16);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);      // the offset-sum copies have landed
  __syncthreads();

  const UnpackConsts uc = unpack_consts();
  const int reducer = W - 1;          // always owns at least one group
  floatx4_t yacc[TC];
#pragma unroll
  for (int tc = 0; tc < TC; ++tc) yacc[tc] = floatx4_t{};
  int blocks_done = 0;
  auto finish_block = [&]() {
    floatx4_t* rb = red + (size_t)(blocks_done & 1) * W * TC * 64;
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      rb[(wave * TC + tc) * 64 + lane] = yacc[tc];
      yacc[tc] = floatx4_t{};
    }
    __syncthreads();
    if (wave == reducer) {
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        floatx4_t sacc = rb[tc * 64 + lane];
#pragma unroll
        for (int wv = 1; wv < W; ++wv) sacc += rb[(wv * TC + tc) * 64 + lane];
        ybuf[((size_t)blocks_done * TC + tc) * 64 + lane] = sacc;
      }
    }
    ++blocks_done;
  };
  int c_j = jb, c_left = total;
  auto consume = [&](int p, bool guarded) {   // guarded only in the tail (see the GEMV)
    if (!guarded || c_left > 0) {
      const int j = c_j;
      const uint32_t szv = szw[((size_t)blocks_done * ng + j) * 16 + r];
      const float dsc = h2f((uint16_t)szv), zf = (float)(szv >> 16);
      half8_t bop[WPL];
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        uint32_t u[4];
        unpack_word(wq[p][i], u, uc);
        bop[i] = __builtin_bit_cast(half8_t, make_uint4(u[0], u[1], u[2], u[3]));
      }
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        floatx4_t cacc = floatx4_t{};
#pragma unroll
        for (int i = 0; i < WPL; ++i)
          cacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, aq[p][tc][i]), bop[i],
                                                        cacc, 0, 0, 0);
        // rows 4c .. 4c+3 of the chunk (tokens) for column r
        const float4* tup = reinterpret_cast<const float4*>(tu_l + ((size_t)tc * ng + j) * 16 + 4 * c);
        const float4 t01 = tup[0], t23 = tup[1];
        const float tt[4] = {t01.x, t01.z, t23.x, t23.z};
        const float uu[4] = {t01.y, t01.w, t23.y, t23.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          yacc[tc][e] = __builtin_fmaf(dsc, __builtin_fmaf(-zf, uu[e], cacc[e] - tt[e]), yacc[tc][e]);
      }
      --c_left;
      if (++c_j == je) {
        finish_block();
        c_j = jb;
      }
    }
  };
  if (cnt > 0) {
    int left = total;
    while (true) {
      if (left > PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(PF + p);
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(p, false);
        left -= PF;
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(p, true);
        break;
      }
      if (left > PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(p);
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(PF + p, false);
        left -= PF;
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(PF + p, true);
        break;
      }
    }
  } else {
    for (int bi = 0; bi < my_blocks; ++bi) finish_block();
  }

  // ---- outputs: the reducer wave wrote every row of ybuf itself
  if (wave == reducer) {
    for (int bi = 0; bi < my_blocks; ++bi) {
      const int64_t col = ((int64_t)blockIdx.x + (int64_t)bi * grid) * 16 + r;
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        const floatx4_t v = ybuf[((size_t)bi * TC + tc) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t t = (int64_t)tc * 16 + 4 * c + e;
          if (t < m && col < n) y[t * n + col] = f2act(v[e], bf);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- skinny, fused
// linear_skinny_fused: one kernel for 2 <= m <= 32 with the decode GEMV's
// layout (8 waves split K, 16-column blocks, scale|zero words staged up front,
// one barrier per block, outputs stored at the end), but no staged activation
// operand: every (block, group) item loads, next to its weight words, the raw
// 16-byte activation rows of its tokens (tokens 16 tc + lane % 16; buffer
// loads, so rows past m read zeros and cost nothing), and the MFMA A operand
// x_tilde = fp16_rn(x * inv_s) is formed in registers (v_pk_mul_f16 against
// inv_s staged in LDS, then the channels permuted into the unpack order).
// The weights are dequantized in registers to fp16_rn((q - z) D) as in the
// prefill GEMM, so the MFMA accumulates whole groups with no offset sums.
template <int G, int TC, bool SZV, int PF>
__device__ __forceinline__ void skinny_fused_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y, int bid, int grid_in, bool bf) {
  constexpr int WPL = G / 32, LPG = G / 8;
  constexpr int W = kSk16Waves;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ng = (int)(k / G);
  const int nblk = (int)((n + 15) / 16);
  const int grid = grid_in;
  const int my_blocks = (nblk - bid + grid - 1) / grid;   // 1 .. kGemvMaxBlk
  const size_t inv_bytes = ((size_t)k * 2 + 1023) & ~(size_t)1023;
  unsigned char* sp = smem;
  uint16_t* inv_l = reinterpret_cast<uint16_t*>(sp);  sp += inv_bytes;
  uint32_t* szw = reinterpret_cast<uint32_t*>(sp);    sp += (size_t)my_blocks * ng * 16 * 4;
  floatx4_t* red = reinterpret_cast<floatx4_t*>(sp);  sp += (size_t)2 * W * TC * 64 * 16;
  floatx4_t* ybuf = reinterpret_cast<floatx4_t*>(sp);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int jb = ng * wave / W, je = ng * (wave + 1) / W;
  const int cnt = je - jb;
  const int total = my_blocks * cnt;
  const int nzw = (ng + 7) / 8, kw_row = (int)(k / 8);
  const bool has_inv = inv_s != nullptr;

  // ---- 1. inv_s into LDS: straight global -> LDS copies of 1 KiB per wave
  // instruction (the tail clamped to the last 16 source bytes, landing in the
  // rounded-up pad)
  if (has_inv) {
    typedef __attribute__((address_space(3))) void lds_void_t;
    const int64_t src_bytes = k * 2;
    const char* srcb = reinterpret_cast<const char*>(inv_s);
    const int n_copy = (int)(inv_bytes / 1024);
    for (int i = wave; i < n_copy; i += W) {
      int64_t off = (int64_t)i * 1024 + lane * 16;
      off = off + 16 <= src_bytes ? off : src_bytes - 16;
      __builtin_amdgcn_global_load_lds((const void*)(srcb + off),
                                       (lds_void_t*)(reinterpret_cast<char*>(inv_l) + i * 1024),
                                       16, 0, 0);
    }
  }
  // ---- 2. scale and zero words of every block (lane-predicated, first)
  const int n_oct = my_blocks * 16 * nzw;
  uint4 sz_s[kGemvSzRounds];
  uint32_t sz_z[kGemvSzRounds];
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    sz_s[i] = make_uint4(0, 0, 0, 0);
    sz_z[i] = 0;
    const int o = tid + i * kSk16Threads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      int col = (bid + bs * grid) * 16 + row;
      col = col < (int)n ? col : (int)n - 1;
      const uint16_t* srow = scales + (int64_t)col * ng + oct * 8;
      if constexpr (SZV) {
        sz_s[i] = *reinterpret_cast<const uint4*>(srow);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (oct * 8 + e < ng) ? srow[e] : (uint16_t)0;
        sz_s[i] = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                             h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
      sz_z[i] = qzeros[(int64_t)col * nzw + oct];
    }
  }

  // ---- 3. first items (unconditional buffer loads; rows past m and columns
  // past n read zeros)
  uint32_t wq[2 * PF][WPL];
  uint4 xq[2 * PF][TC][WPL];
  const __amdgpu_buffer_rsrc_t rs_w = buf_rsrc(qweight, (uint32_t)((uint64_t)n * (uint64_t)k / 2));
  const __amdgpu_buffer_rsrc_t rs_x = buf_rsrc(x, (uint32_t)((uint64_t)m * (uint64_t)k * 2));
  // the row or token (which decides whether a load is past the end) is in the
  // VGPR offset, the group along K in the scalar one
  const uint32_t w_voff = ((uint32_t)r * (uint32_t)kw_row + (uint32_t)(WPL * c)) * 4u;
  uint32_t x_voff[TC];
#pragma unroll
  for (int tc = 0; tc < TC; ++tc)
    x_voff[tc] = ((uint32_t)(tc * 16 + r) * (uint32_t)k + (uint32_t)(8 * WPL * c)) * 2u;
  int i_blk = bid, i_j = jb, i_left = total;
  auto issue = [&](int slot) {
    const int jj = i_j < ng ? i_j : ng - 1;
    const uint32_t wvo = w_voff + (uint32_t)i_blk * 16u * (uint32_t)kw_row * 4u;
    buf_words<WPL>(rs_w, wvo, (uint32_t)(jj * LPG) * 4u, wq[slot]);
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      const uint32_t xso = (uint32_t)(jj * G) * 2u;
#pragma unroll
      for (int i = 0; i < WPL; ++i)
        xq[slot][tc][i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, x_voff[tc] + 16u * i, xso, 0));
    }
    if (i_left > 1) {
      --i_left;
      if (++i_j == je) { i_j = jb; i_blk += grid; }
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p);

  // ---- 4. scale|zero words into LDS as [block][group][column]
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    const int o = tid + i * kSk16Threads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      const uint32_t sw[4] = {sz_s[i].x, sz_s[i].y, sz_s[i].z, sz_s[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = oct * 8 + e;
        if (j < ng)
          szw[((size_t)bs * ng + j) * 16 + row] =
              ((sw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) | (((sz_z[i] >> (4 * e)) & 0xFu) << 16);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);      // the inv_s copies have landed
  __syncthreads();

  const UnpackConsts uc = unpack_consts();
  const int reducer = W - 1;
  floatx4_t acc[TC];
#pragma unroll
  for (int tc = 0; tc < TC; ++tc) acc[tc] = floatx4_t{};
  int blocks_done = 0;
  auto finish_block = [&]() {
    floatx4_t* rb = red + (size_t)(blocks_done & 1) * W * TC * 64;
#pragma unroll
    for (int tc = 0; tc < TC; ++tc) {
      rb[(wave * TC + tc) * 64 + lane] = acc[tc];
      acc[tc] = floatx4_t{};
    }
    __syncthreads();
    if (wave == reducer) {
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        floatx4_t sacc = rb[tc * 64 + lane];
#pragma unroll
        for (int wv = 1; wv < W; ++wv) sacc += rb[(wv * TC + tc) * 64 + lane];
        ybuf[((size_t)blocks_done * TC + tc) * 64 + lane] = sacc;
      }
    }
    ++blocks_done;
  };
  int c_j = jb, c_left = total;
  auto consume = [&](int p, bool guarded) {   // guarded only in the tail (see the GEMV)
    if (!guarded || c_left > 0) {
      const int j = c_j;
      const uint32_t szv = szw[((size_t)blocks_done * ng + j) * 16 + r];
      const float d = h2f((uint16_t)szv), z = (float)(szv >> 16);
      const half2_t dd = {(half_t)d, (half_t)d};
      const half2_t o1024 = {(half_t)(-1024.0f - z), (half_t)(-1024.0f - z)};
      const half2_t o64 = {(half_t)(-64.0f - z), (half_t)(-64.0f - z)};
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        // B: the 8 weights of word i, fp16_rn((q - z) D) in unpack order
        uint32_t u[4];
        unpack_word(wq[p][i], u, uc);
        const half2_t q0 = (__builtin_bit_cast(half2_t, u[0]) + o1024) * dd;
        const half2_t q1 = (__builtin_bit_cast(half2_t, u[1]) + o64) * dd;
        const half2_t q2 = (__builtin_bit_cast(half2_t, u[2]) + o1024) * dd;
        const half2_t q3 = (__builtin_bit_cast(half2_t, u[3]) + o64) * dd;
        const half8_t bop = __builtin_bit_cast(
            half8_t, make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                                __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)));
        // inv_s of the same 8 channels
        const uint4 sv = has_inv ? *reinterpret_cast<const uint4*>(inv_l + j * G + 8 * (WPL * c + i))
                                 : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
#pragma unroll
        for (int tc = 0; tc < TC; ++tc) {
          const uint4 xv = act8_h(xq[p][tc][i], bf);
          const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.x) * __builtin_bit_cast(half2_t, sv.x));
          const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.y) * __builtin_bit_cast(half2_t, sv.y));
          const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.z) * __builtin_bit_cast(half2_t, sv.z));
          const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.w) * __builtin_bit_cast(half2_t, sv.w));
          // channels (k0..k7) -> unpack order (k0, k4, k1, k5, k2, k6, k3, k7)
          const uint4 av = make_uint4(__builtin_amdgcn_perm(p2, p0, 0x05040100u),
                                      __builtin_amdgcn_perm(p2, p0, 0x07060302u),
                                      __builtin_amdgcn_perm(p3, p1, 0x05040100u),
                                      __builtin_amdgcn_perm(p3, p1, 0x07060302u));
          acc[tc] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), bop,
                                                           acc[tc], 0, 0, 0);
        }
      }
      --c_left;
      if (++c_j == je) {
        finish_block();
        c_j = jb;
      }
    }
  };
  if (cnt > 0) {
    int left = total;
    while (true) {
      if (left > PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(PF + p);
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(p, false);
        left -= PF;
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(p, true);
        break;
      }
      if (left > PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(p);
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(PF + p, false);
        left -= PF;
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(PF + p, true);
        break;
      }
    }
  } else {
    for (int bi = 0; bi < my_blocks; ++bi) finish_block();
  }

  // ---- outputs: lane (c, r) holds tokens 16 tc + 4c + e of column r
  if (wave == reducer) {
    for (int bi = 0; bi < my_blocks; ++bi) {
      const int64_t col = ((int64_t)bid + (int64_t)bi * grid) * 16 + r;
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        const floatx4_t v = ybuf[((size_t)bi * TC + tc) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t t = (int64_t)tc * 16 + 4 * c + e;
          if (t < m && col < n) y[t * n + col] = f2act(v[e], bf);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- skinny, group-major
// linear_skinny_gm: the fused skinny kernel with a work-group's (block, group)
// items walked group-major.  One unit of a wave is group j of all NB column
// blocks of its work-group, so the 16 activation rows of group j are loaded,
// scaled and permuted into the MFMA A operand once for NB blocks (block-major
// does that once per block, which at 16 tokens moves four times the weight
// bytes through the caches).  The NB accumulators stay in registers over the
// wave's K range, so the main loop has no barrier; after it the waves meet
// once per block to sum their partial rows, and the reducing wave stores the
// outputs.  Block slots past the linear's last block point one block past its
// end: their weight loads read zeros, and they are not stored.  TC = 2 (17 to
// 32 tokens) gives every dequantized weight fragment two A fragments, tokens
// 0-15 and 16-31, so the weights are read and dequantized once for both.
template <int G, bool SZV, int NB, int PF, int TC>
__device__ __forceinline__ void skinny_gm_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t m, int64_t n, int64_t k,
    uint16_t* __restrict__ y, int bid, int grid, bool bf) {
  constexpr int WPL = G / 32, LPG = G / 8;
  constexpr int W = kSk16Waves;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ng = (int)(k / G);
  const int nblk = (int)((n + 15) / 16);
  const int my_blocks = (nblk - bid + grid - 1) / grid;   // 1 .. NB
  const size_t inv_bytes = ((size_t)k * 2 + 1023) & ~(size_t)1023;
  unsigned char* sp = smem;
  uint16_t* inv_l = reinterpret_cast<uint16_t*>(sp);  sp += inv_bytes;
  uint32_t* szw = reinterpret_cast<uint32_t*>(sp);    sp += (size_t)NB * ng * 16 * 4;
  floatx4_t* red = reinterpret_cast<floatx4_t*>(sp);  // [2][W][64]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int jb = ng * wave / W, je = ng * (wave + 1) / W;
  const int cnt = je - jb;
  const int nzw = (ng + 7) / 8, kw_row = (int)(k / 8);
  const bool has_inv = inv_s != nullptr;

  // ---- 1. inv_s into LDS (straight global -> LDS copies, as the fused kernel)
  if (has_inv) {
    typedef __attribute__((address_space(3))) void lds_void_t;
    const int64_t src_bytes = k * 2;
    const char* srcb = reinterpret_cast<const char*>(inv_s);
    const int n_copy = (int)(inv_bytes / 1024);
    for (int i = wave; i < n_copy; i += W) {
      int64_t off = (int64_t)i * 1024 + lane * 16;
      off = off + 16 <= src_bytes ? off : src_bytes - 16;
      __builtin_amdgcn_global_load_lds((const void*)(srcb + off),
                                       (lds_void_t*)(reinterpret_cast<char*>(inv_l) + i * 1024),
                                       16, 0, 0);
    }
  }
  // ---- 2. scale and zero words of the work-group's blocks
  const int n_oct = my_blocks * 16 * nzw;
  uint4 sz_s[kGemvSzRounds];
  uint32_t sz_z[kGemvSzRounds];
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    sz_s[i] = make_uint4(0, 0, 0, 0);
    sz_z[i] = 0;
    const int o = tid + i * kSk16Threads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      int col = (bid + bs * grid) * 16 + row;
      col = col < (int)n ? col : (int)n - 1;
      const uint16_t* srow = scales + (int64_t)col * ng + oct * 8;
      if constexpr (SZV) {
        sz_s[i] = *reinterpret_cast<const uint4*>(srow);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (oct * 8 + e < ng) ? srow[e] : (uint16_t)0;
        sz_s[i] = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                             h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
      sz_z[i] = qzeros[(int64_t)col * nzw + oct];
    }
  }

  // ---- 3. first units (unconditional buffer loads: rows past n, block slots
  // past the last block and tokens past m read zeros; the row or token is in
  // the VGPR offset, the group along K in the scalar one)
  uint32_t wq[2 * PF][NB][WPL];
  uint4 xq[2 * PF][TC][WPL];
  const __amdgpu_buffer_rsrc_t rs_w = buf_rsrc(qweight, (uint32_t)((uint64_t)n * (uint64_t)k / 2));
  const __amdgpu_buffer_rsrc_t rs_x = buf_rsrc(x, (uint32_t)((uint64_t)m * (uint64_t)k * 2));
  uint32_t w_voff[NB];
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    int blk = bid + bb * grid;
    blk = blk < nblk ? blk : nblk;
    w_voff[bb] = ((uint32_t)(blk * 16 + r) * (uint32_t)kw_row + (uint32_t)(WPL * c)) * 4u;
  }
  const uint32_t x_voff = ((uint32_t)r * (uint32_t)k + (uint32_t)(8 * WPL * c)) * 2u;
  const uint32_t x_chunk = (uint32_t)k * 32u;     // 16 token rows
  int i_j = jb, i_left = cnt;
  auto issue = [&](int slot) {
    const int jj = i_j < ng ? i_j : ng - 1;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
      buf_words<WPL>(rs_w, w_voff[bb], (uint32_t)(jj * LPG) * 4u, wq[slot][bb]);
#pragma unroll
    for (int t = 0; t < TC; ++t)
#pragma unroll
      for (int i = 0; i < WPL; ++i)
        xq[slot][t][i] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_x, x_voff + x_chunk * t + 16u * i,
                                                         (uint32_t)(jj * G) * 2u, 0));
    if (i_left > 1) {
      --i_left;
      ++i_j;
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) issue(p);

  // ---- 4. scale|zero words into LDS as [block][group][column]
#pragma unroll
  for (int i = 0; i < kGemvSzRounds; ++i) {
    const int o = tid + i * kSk16Threads;
    if (o < n_oct) {
      const int row_all = o / nzw, oct = o - row_all * nzw;
      const int bs = row_all >> 4, row = row_all & 15;
      const uint32_t sw[4] = {sz_s[i].x, sz_s[i].y, sz_s[i].z, sz_s[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = oct * 8 + e;
        if (j < ng)
          szw[((size_t)bs * ng + j) * 16 + row] =
              ((sw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu) | (((sz_z[i] >> (4 * e)) & 0xFu) << 16);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);      // the inv_s copies have landed
  __syncthreads();

  const UnpackConsts uc = unpack_consts();
  floatx4_t acc[TC][NB];
#pragma unroll
  for (int t = 0; t < TC; ++t)
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[t][bb] = floatx4_t{};
  int c_j = jb, c_left = cnt;
  auto consume = [&](int p, bool guarded) {   // guarded only in the tail
    if (!guarded || c_left > 0) {
      const int j = c_j;
      // A: x_tilde = fp16_rn(x inv_s) of the 16 token rows of each chunk,
      // channels permuted into the unpack order (k0, k4, k1, k5, k2, k6, k3, k7)
      half8_t av[TC][WPL];
#pragma unroll
      for (int i = 0; i < WPL; ++i) {
        const uint4 sv = has_inv ? *reinterpret_cast<const uint4*>(inv_l + j * G + 8 * (WPL * c + i))
                                 : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
#pragma unroll
        for (int t = 0; t < TC; ++t) {
          const uint4 xv = act8_h(xq[p][t][i], bf);
          const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.x) * __builtin_bit_cast(half2_t, sv.x));
          const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.y) * __builtin_bit_cast(half2_t, sv.y));
          const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.z) * __builtin_bit_cast(half2_t, sv.z));
          const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.w) * __builtin_bit_cast(half2_t, sv.w));
          av[t][i] = __builtin_bit_cast(half8_t, make_uint4(__builtin_amdgcn_perm(p2, p0, 0x05040100u),
                                                            __builtin_amdgcn_perm(p2, p0, 0x07060302u),
                                                            __builtin_amdgcn_perm(p3, p1, 0x05040100u),
                                                            __builtin_amdgcn_perm(p3, p1, 0x07060302u)));
        }
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        // B: the 8 weights of word i of block bb, fp16_rn((q - z) D) in unpack order
        const uint32_t szv = szw[((size_t)bb * ng + j) * 16 + r];
        const float d = h2f((uint16_t)szv), z = (float)(szv >> 16);
        const half2_t dd = {(half_t)d, (half_t)d};
        const half2_t o1024 = {(half_t)(-1024.0f - z), (half_t)(-1024.0f - z)};
        const half2_t o64 = {(half_t)(-64.0f - z), (half_t)(-64.0f - z)};
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
          uint32_t u[4];
          unpack_word(wq[p][bb][i], u, uc);
          const half2_t q0 = (__builtin_bit_cast(half2_t, u[0]) + o1024) * dd;
          const half2_t q1 = (__builtin_bit_cast(half2_t, u[1]) + o64) * dd;
          const half2_t q2 = (__builtin_bit_cast(half2_t, u[2]) + o1024) * dd;
          const half2_t q3 = (__builtin_bit_cast(half2_t, u[3]) + o64) * dd;
          const half8_t bop = __builtin_bit_cast(
              half8_t, make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                                  __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)));
#pragma unroll
          for (int t = 0; t < TC; ++t)
            acc[t][bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[t][i], bop, acc[t][bb], 0, 0, 0);
        }
      }
      --c_left;
      ++c_j;
    }
  };
  if (cnt > 0) {
    int left = cnt;
    while (true) {
      if (left > PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(PF + p);
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(p, false);
        left -= PF;
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(p, true);
        break;
      }
      if (left > PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(p);
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(PF + p, false);
        left -= PF;
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p) consume(PF + p, true);
        break;
      }
    }
  }

  // ---- 5. per block and chunk: the W partial rows summed in wave order by
  // the last wave, which stores them (lane (c, r) holds tokens 16 tc + 4c + e
  // of column r); the two reduction buffers alternate
  const int reducer = W - 1;
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    if (bb < my_blocks) {
#pragma unroll
      for (int tc = 0; tc < TC; ++tc) {
        floatx4_t* rb = red + (size_t)((bb * TC + tc) & 1) * W * 64;
        rb[wave * 64 + lane] = acc[tc][bb];
        __syncthreads();
        if (wave == reducer) {
          floatx4_t sacc = rb[lane];
#pragma unroll
          for (int wv = 1; wv < W; ++wv) sacc += rb[wv * 64 + lane];
          const int64_t col = ((int64_t)bid + (int64_t)bb * grid) * 16 + r;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = sacc[e];
            const int64_t t = 16 * tc + 4 * c + e;
            if (t < m && col < n) y[t * n + col] = f2act(v, bf);
          }
        }
      }
    }
  }
}

#ifndef AWQ_SKINNY_GM_MINW
#define AWQ_SKINNY_GM_MINW 2
#endif
template <int G, bool SZV, int NB, int PF>
__global__ __launch_bounds__(kSk16Threads, AWQ_SKINNY_GM_MINW) void linear_skinny_gm_kernel(const LinGroup gp,
                                                                           int64_t m, int64_t k) {
  const LinPick L = pick_linear(gp);
  skinny_gm_body<G, SZV, NB, PF, 1>(L.x, L.inv, L.qw, L.sc, L.qz, m, L.n, k, L.y, L.bid, L.grid,
                                    gp.bf != 0);
}
// 17 to 32 tokens: two A chunks per weight fragment; one work-group per CU
// (the second chunk's activations and accumulators double those registers)
template <int G, bool SZV, int NB, int PF>
__global__ __launch_bounds__(kSk16Threads, 1) void linear_skinny_gm2_kernel(const LinGroup gp,
                                                                             int64_t m, int64_t k) {
  const LinPick L = pick_linear(gp);
  skinny_gm_body<G, SZV, NB, PF, 2>(L.x, L.inv, L.qw, L.sc, L.qz, m, L.n, k, L.y, L.bid, L.grid,
                                    gp.bf != 0);
}

// LDS of the group-major skinny kernel: inv_s (whole 1 KiB copies), scale|zero
// words [NB][ng][16], reduction rows [2][8][64] float4.
size_t skinny_gm_lds_bytes(int64_t k, int32_t g, int nb) {
  const size_t ng = (size_t)(k / g);
  const size_t inv = ((size_t)k * 2 + 1023) & ~(size_t)1023;
  return inv + (size_t)nb * ng * 16 * 4 + (size_t)2 * kSk16Waves * 64 * 16;
}

// LDS of the fused skinny kernel: inv_s (rounded up to whole 1 KiB copies),
// scale|zero words [nb][ng][16], reduction rows [2][8][tc][64] float4,
// outputs [nb][tc][64] float4.

template <int G, int TC, bool SZV, int PF>
__global__ __launch_bounds__(kSk16Threads, 2) void linear_skinny_fused_kernel(const LinGroup gp,
                                                                              int64_t m, int64_t k) {
  const LinPick L = pick_linear(gp);
  skinny_fused_body<G, TC, SZV, PF>(L.x, L.inv, L.qw, L.sc, L.qz, m, L.n, k, L.y, L.bid, L.grid,
                                    gp.bf != 0);
}

size_t skinny_fused_lds_bytes(int64_t k, int32_t g, int nb, int tc) {
  const size_t ng = (size_t)(k / g);
  const size_t inv = ((size_t)k * 2 + 1023) & ~(size_t)1023;
  return inv + (size_t)nb * ng * 16 * 4 + (size_t)2 * kSk16Waves * tc * 64 * 16 +
         (size_t)nb * tc * 64 * 16;
}

// ---------------------------------------------------------------- prefill GEMM, 33-128 tokens
// Work-group tile 64 tokens x 128 output columns, K-step 64, 4 waves side by
// side along N, each 64 x 32 = 2 x 1 blocks of v_mfma_f32_32x32x16_f16 (fp32
// accumulators).  Also taken beyond 128 tokens where a column has an odd
// number of groups (the 128-row kernel below copies scales in pairs).
//  * A (activations): linear_xprep first writes x_tilde = fp16(x * inv_s)
//    once per call, every 8-channel chunk permuted into the nibble-unpack
//    slot order.  Each K-step the work-group copies its 64 x 64 tile straight
//    from global memory into one of two LDS stages (global_load_lds, 16 bytes
//    per lane; 16-byte chunks XOR-swizzled by row, so the lanes served per
//    LDS cycle hit distinct banks).
//  * B (weights) never touches LDS: lane (column j, half c) of a wave loads
//    the 4 qweight words of its column for the K-step directly (one 16-byte
//    load), and dequantizes them in registers: nibbles masked into fp16
//    (offset + q), the offset and zero point removed exactly with
//    v_pk_add_f16, the step applied with v_pk_mul_f16 (one rounding).  MFMA
//    step s of the K-step uses word 4c + s, and the A fragment of lane half c
//    reads the matching channel chunk 4c + s, so both operands agree on the
//    K order.
//  * Scales and zero words of the work-group's 128 columns are staged in LDS
//    once.  The next K-step's global loads are in flight while the current
//    one is multiplied.
constexpr int kGemmBM = 64, kGemmBN = 128, kGemmBK = 64;
constexpr int kGemmSRow = kGemmBN + 2, kGemmZRow = kGemmBN + 1;   // padded LDS rows

// dynamic LDS of the GEMM (the two activation stages are static): the
// scales [gmax][kGemmSRow] halves and zero words [gmax / 8 + 2][kGemmZRow] of
// the groups one K slice spans
__host__ __device__ inline size_t gemm_s_bytes(int gmax) {
  return ((size_t)kGemmSRow * gmax * 2 + 15) & ~(size_t)15;
}
static size_t gemm_lds_bytes(int gmax) {
  return gemm_s_bytes(gmax) + (size_t)kGemmZRow * (gmax / 8 + 2) * 4;
}
// most groups a slice of ks slices of the K-steps spans
static int gemm_slice_groups(int64_t k, int32_t g, int ks) {
  const int64_t nk = k / kGemmBK;
  const int64_t steps = (nk + ks - 1) / ks;
  return (int)((steps * kGemmBK + g - 1) / g + 1);
}
// the 128-row kernel: tile, stages of its copy ring and their bytes (x_tilde,
// packed words, scale and zero words)
constexpr int kG2BM = 128, kG2BN = 256, kG2Stages = 3;
constexpr int kG2AStage = kG2BM * kGemmBK * 2;
constexpr int kG2BStage = kG2BN * 32;
constexpr int kG2Stage = kG2AStage + kG2BStage + 2 * kG2BN * 4;
static size_t gemm_static_lds(int bm) {
  return bm == 64 ? (size_t)2 * bm * kGemmBK * 2 : (size_t)kG2Stages * kG2Stage;
}

// rows of one GEMM launch: its x_tilde stays below 2^31 bytes
static int64_t gemm_row_chunk(int64_t k) {
  const int64_t c = (((int64_t)1 << 31) / (k * 2)) / kG2BM * kG2BM;
  return c > 0 ? c : kG2BM;
}

#ifndef AWQ_GEMM_SMALL_M
#define AWQ_GEMM_SMALL_M 128
#endif
#ifndef AWQ_GEMM_SPLIT_TARGET
#define AWQ_GEMM_SPLIT_TARGET 256
#endif
// tile rows: 64 for few tokens (64 x 128 tiles), else 128 (128 x 256 tiles;
// the 128-row kernel copies the scales as 32-bit words of two groups, so it
// needs an even number of groups per column)
static int gemm_bm(int64_t m, int64_t k, int32_t g) {
  return (m <= AWQ_GEMM_SMALL_M || (k / g) % 2 != 0) ? 64 : kG2BM;
}
static int gemm_bn(int bm) { return bm == 64 ? kGemmBN : kG2BN; }

// Slices of K per tile for a linear whose tiles alone leave CUs idle: enough
// slices for one work-group per CU (two for 64-row tiles where K >= 8192: a
// long tile K loop runs one K-step ahead and stalls on its loads, and a
// second resident work-group per CU hides that; measured at 24-128 tokens,
// down 30 -> 25.5 us, 70B-shaped down 79 -> 58 us, while at K = 4096 and with
// 128 x 256 tiles the extra partial tiles cost more), at least two K-steps
// each, at most 16.
// With 64-row tiles (m <= 128) whenever the linear has fewer tiles than CUs;
// with 128 x 256 tiles up to 512 tokens and 64 tiles, or 128 tiles where
// K >= 8192 makes a tile's K loop long (beyond that the partial tiles' round
// trip costs more than the idle CUs: measured on the Llama-shaped linears with
// tiles of the same area, 256 x 128).  A property of the linear alone, so a
// group call computes every linear exactly as a call of it alone.
static int gemm_split_occupancy(int64_t m, int64_t n, int64_t k, int32_t g) {
  const int bm = gemm_bm(m, k, g), bn = gemm_bn(bm);
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  if (m > gemm_row_chunk(k) || tiles >= AWQ_GEMM_SPLIT_TARGET) return 1;
  if (bm != 64 && (m > 512 || tiles > 128 || (tiles > 64 && k < 8192))) return 1;
  const int64_t nk = k / kGemmBK;
  const int64_t target = (bm == 64 && k >= 8192) ? 2 * AWQ_GEMM_SPLIT_TARGET : AWQ_GEMM_SPLIT_TARGET;
  int64_t sk = (target + tiles - 1) / tiles;
  const int64_t smax = nk / 2 < 16 ? nk / 2 : 16;
  sk = sk < smax ? sk : smax;
  return sk > 1 ? (int)sk : 1;
}
// With 64-row tiles also split where the scales and zero words of a tile's
// whole K range would not fit LDS (long K with small groups: K / g beyond
// about 300; the 128-row kernel keeps them in registers); 0 when that would
// need a split and the call's activations are too large for one launch.
static int gemm_split(int64_t m, int64_t n, int64_t k, int32_t g) {
  int sk = gemm_split_occupancy(m, n, k, g);
  const int64_t nk = k / kGemmBK;
  const int bm = gemm_bm(m, k, g);
  const size_t budget = (size_t)160 * 1024 - gemm_static_lds(bm);
  while (bm == 64 && gemm_lds_bytes(gemm_slice_groups(k, g, sk)) > budget && sk < nk) ++sk;
  if (sk > 1 && m > gemm_row_chunk(k)) return 0;
  return sk;
}

// fp32 partial tiles of a split linear: [tile][slice][min(m, BM) rows][BN]
static size_t gemm_part_bytes(int64_t m, int64_t n, int64_t k, int32_t g) {
  const int sk = gemm_split(m, n, k, g);
  if (sk <= 1) return 0;
  const int bm = gemm_bm(m, k, g), bn = gemm_bn(bm);
  const int64_t tiles = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
  const int64_t rows_t = m < bm ? m : bm;
  return align256((size_t)sk * (size_t)tiles * (size_t)rows_t * bn * 4);
}
#ifndef AWQ_GEMM_SWZ_SHIFT
#define AWQ_GEMM_SWZ_SHIFT 1
#endif

__device__ __forceinline__ uint32_t perm_bytes(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// x_tilde = fp16_rn(x * inv_s), every 8-channel chunk permuted into the
// nibble-unpack slot order (k0,k4) (k1,k5) (k2,k6) (k3,k7); one pass over the
// activations per call, so the GEMM's activation staging is a plain copy.
// Item blockIdx.y of the group: x = gp.x, inv_s = gp.inv, x_tilde written to
// gp.y (the scratch slot of that item).
__global__ __launch_bounds__(256) void linear_xprep_kernel(const LinGroup gp, int64_t m,
                                                           int64_t k) {
  int li = 0;
#pragma unroll
  for (int i = 1; i < kGroupMax; ++i)
    if (i == (int)blockIdx.y) li = i;
  const uint16_t* __restrict__ x = gp.x[li];
  const uint16_t* __restrict__ inv_s = gp.inv[li];
  uint16_t* __restrict__ xt = gp.y[li];
  const int64_t chunks = m * (k / 8);
  const bool has_inv = inv_s != nullptr;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t kk = (c % (k / 8)) * 8;
    const uint4 xv = act8_h(*reinterpret_cast<const uint4*>(x + c * 8), gp.bf != 0);
    const uint4 iv = has_inv ? *reinterpret_cast<const uint4*>(inv_s + kk)
                             : make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    const uint32_t p0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.x) * __builtin_bit_cast(half2_t, iv.x));
    const uint32_t p1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.y) * __builtin_bit_cast(half2_t, iv.y));
    const uint32_t p2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.z) * __builtin_bit_cast(half2_t, iv.z));
    const uint32_t p3 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, xv.w) * __builtin_bit_cast(half2_t, iv.w));
    uint4 v;
    v.x = perm_bytes(p2, p0, 0x05040100u);
    v.y = perm_bytes(p2, p0, 0x07060302u);
    v.z = perm_bytes(p3, p1, 0x05040100u);
    v.w = perm_bytes(p3, p1, 0x07060302u);
    *reinterpret_cast<uint4*>(xt + c * 8) = v;
  }
}

template <int G>
__global__ __launch_bounds__(256, 2) void linear_gemm_kernel(const LinGroup gp, int64_t m,
                                                             int64_t k, int tiles_m) {
  // waves 1 (M) x 4 (N), each 64 x 32 = 2 x 1 blocks of 32 x 32
  constexpr int BM = kGemmBM;
  constexpr int WM = 1;
  constexpr int WN = 4 / WM;
  constexpr int RW = BM / WM, CW = kGemmBN / WN;    // rows and columns per wave
  constexpr int BMB = RW / 32, BNB = CW / 32;       // 32 x 32 blocks per wave
  constexpr int AR = BM / 32;                       // A copy instructions per wave (8 rows each)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // two distinct stage objects: the compiler can see that the copies into one
  // stage never alias the fragment reads of the other, so it does not wait for
  // the copies before reading
  __shared__ __attribute__((aligned(16))) uint16_t a_st0[BM * kGemmBK];
  __shared__ __attribute__((aligned(16))) uint16_t a_st1[BM * kGemmBK];
  const int ng = (int)(k / G), nzw = (ng + 7) / 8;
  // scales and zero words of the tile's columns for the groups of this
  // work-group's K slice, column fastest with a padded row (kGemmSRow halves,
  // kGemmZRow words): the lanes of a wave read 32 consecutive columns of one
  // group, and the staging writes of consecutive groups of one column land in
  // different banks.  Sized on the host for the longest slice of the launch.
  uint16_t* s_l = reinterpret_cast<uint16_t*>(smem);                          // [gmax][kGemmSRow]
  uint32_t* z_l = reinterpret_cast<uint32_t*>(smem + gemm_s_bytes(gp.gmax));  // [gmax/8+2][kGemmZRow]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  // XCD-aware tile order: each XCD gets a contiguous range of tiles, M fastest,
  // so the work-groups that share a weight tile share that XCD's L2
  const int total = gp.wg0[gp.count];
  const int bid = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, slot = bid / 8;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const LinPick L = pick_linear_at(gp, tile);
  const uint16_t* __restrict__ x = L.x;
  const uint32_t* __restrict__ qweight = L.qw;
  const uint16_t* __restrict__ scales = L.sc;
  const uint32_t* __restrict__ qzeros = L.qz;
  uint16_t* __restrict__ y = L.y;
  const int64_t n = L.n;
  // work-group L.bid of the linear: tile L.bid / ks, slice L.bid % ks of its K-steps
  const int ks = L.ks;
  const int tl = L.bid / ks, sl = L.bid - tl * ks;
  const int tm = tl % tiles_m, tn = tl / tiles_m;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * kGemmBN;
  const int64_t kw_row = k / 8;
  const int nk = (int)(k / kGemmBK);
  const int kt0 = (int)((int64_t)sl * nk / ks), kt1 = (int)((int64_t)(sl + 1) * nk / ks);

  // ---- scales and zero words of this tile's columns (rows of W)
  // (consecutive threads read consecutive groups of one column)
  const int g0 = (kt0 * kGemmBK) / G, g1 = (kt1 * kGemmBK + G - 1) / G;
  const int w0 = g0 >> 3, w1 = ((g1 - 1) >> 3) + 1;
  const int gn = g1 - g0, wn_ = w1 - w0;
  for (int i = tid; i < kGemmBN * gn; i += 256) {
    const int r = i / gn, gi = i - r * gn;
    int64_t col = n0 + r;
    col = col < n ? col : n - 1;
    s_l[gi * kGemmSRow + r] = scales[col * ng + g0 + gi];
  }
  for (int i = tid; i < kGemmBN * wn_; i += 256) {
    const int r = i / wn_, wi = i - r * wn_;
    int64_t col = n0 + r;
    col = col < n ? col : n - 1;
    z_l[wi * kGemmZRow + r] = qzeros[col * nzw + w0 + wi];
  }

  // ---- A loader: direct global -> LDS copies (global_load_lds_dwordx4).  One
  // wave instruction fills 64 consecutive 16-byte LDS slots (8 rows x 8
  // chunks); lane i writes slot i, so the XOR swizzle of the chunk position is
  // applied on the global side: lane (row r, slot p) fetches logical chunk
  // p ^ ((r >> S) & 7).  Wave w fills rows BM/4 w .. BM/4 (w + 1) - 1 of the stage.
  // The activations arrive already scaled and slot-permuted (linear_xprep).
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int a_lr = lane >> 3, a_p = lane & 7;
  // 32-bit byte offsets from the activation base (one launch covers fewer
  // than 2^31 bytes of x_tilde; the host splits larger M)
  const char* xbytes = reinterpret_cast<const char*>(x);
  uint32_t a_off[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int lrow = wave * (BM / 4) + 8 * i + a_lr;
    int64_t row = m0 + lrow;
    row = row < m ? row : m - 1;
    a_off[i] = (uint32_t)((row * k + (a_p ^ ((lrow >> AWQ_GEMM_SWZ_SHIFT) & 7)) * 8) * 2);
  }
#define AWQ_GEMM_LOAD_A(KT, STAGE_PTR)                                                  \
  {                                                                                     \
    const char* xk_ = xbytes + (int64_t)(KT) * kGemmBK * 2;                             \
    _Pragma("unroll") for (int i = 0; i < AR; ++i)                                      \
      __builtin_amdgcn_global_load_lds(                                                 \
          (const void*)(xk_ + a_off[i]),                                                \
          (lds_void_t*)((STAGE_PTR) + (wave * (BM / 4) + 8 * i) * 64), 16, 0, 0);       \
  }

  // ---- B loader: lane (j = lane % 32, c = lane / 32) of block bn loads words 4c..4c+3
  const int bj = lane & 31, bc = lane >> 5;
  const uint32_t* b_src[BNB];
#pragma unroll
  for (int bn = 0; bn < BNB; ++bn) {
    int64_t col = n0 + wn * CW + bn * 32 + bj;
    col = col < n ? col : n - 1;
    b_src[bn] = qweight + col * kw_row + 4 * bc;
  }
  uint4 wb[BNB];
#define AWQ_GEMM_LOAD_B(KT)                                                        \
  {                                                                                \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn)                             \
      wb[bn] = *reinterpret_cast<const uint4*>(b_src[bn] + (int64_t)(KT) * 8);     \
  }

  floatx16_t acc[BMB][BNB];
#pragma unroll
  for (int i = 0; i < BMB; ++i)
#pragma unroll
    for (int jj = 0; jj < BNB; ++jj) acc[i][jj] = floatx16_t{};

  AWQ_GEMM_LOAD_A(kt0, a_st0);
  AWQ_GEMM_LOAD_B(kt0);
  __builtin_amdgcn_s_waitcnt(0);       // the direct-to-LDS copies have landed
  __syncthreads();
  const UnpackConsts uc = unpack_consts();
  // byte offset of this lane's A fragment of row block bm at sub-step 0: row
  // r = wm RW + bm 32 + lane % 32 holds logical chunk ch = 4 (lane / 32) + s
  // at physical chunk ch ^ ((r >> S) & 7); s only flips chunk bits 0-1, so
  // sub-step s reads a_base[bm] ^ (16 s)
  uint32_t a_base[BMB];
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm) {
    const int row = wm * RW + bm * 32 + (lane & 31);
    a_base[bm] = (uint32_t)(row * 128 + ((4 * bc) ^ ((row >> AWQ_GEMM_SWZ_SHIFT) & 7)) * 16);
  }

  // One K-step: copy the next step's activations into the other stage and
  // load its weights, then four 16-channel sub-steps: the A fragments of the
  // next sub-step are read from LDS while the current one's 8 MFMAs run, and
  // each sub-step dequantizes only its own two weight words; then wait for the
  // copies and meet at the barrier.
#define AWQ_GEMM_A_READ(CUR, S, DST)                                                    \
  {                                                                                     \
    _Pragma("unroll") for (int bm = 0; bm < BMB; ++bm)                                  \
      DST[bm] = *reinterpret_cast<const half8_t*>(                                      \
          reinterpret_cast<const char*>(CUR) + (a_base[bm] ^ (uint32_t)(16 * (S))));     \
  }
#define AWQ_GEMM_STEP(KT, CUR, NXT)                                                     \
  {                                                                                     \
    uint4 wc[BNB];                                                                      \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) wc[bn] = wb[bn];                 \
    const int ktn_ = (KT) + 1 < kt1 ? (KT) + 1 : (KT);                                 \
    AWQ_GEMM_LOAD_A(ktn_, NXT);                                                         \
    AWQ_GEMM_LOAD_B(ktn_);                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    const int grp = ((KT) * kGemmBK + 32 * bc) / G;                                     \
    half2_t dd[BNB], o1024[BNB], o64[BNB];                                              \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                                \
      const int r = wn * CW + bn * 32 + bj;                                             \
      const float d = h2f(s_l[(grp - g0) * kGemmSRow + r]);                             \
      const float z = (float)((z_l[((grp >> 3) - w0) * kGemmZRow + r] >> (4 * (grp & 7))) & 0xFu); \
      dd[bn] = half2_t{(half_t)d, (half_t)d};                                           \
      o1024[bn] = half2_t{(half_t)(-1024.0f - z), (half_t)(-1024.0f - z)};             \
      o64[bn] = half2_t{(half_t)(-64.0f - z), (half_t)(-64.0f - z)};                    \
    }                                                                                   \
    half8_t af[BMB];                                                                    \
    AWQ_GEMM_A_READ(CUR, 0, af)                                                         \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                     \
      half8_t bq[BNB];                                                                  \
      _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                              \
        const uint32_t wsel = s == 0 ? wc[bn].x : s == 1 ? wc[bn].y : s == 2 ? wc[bn].z : wc[bn].w; \
        uint32_t u[4];                                                                  \
        unpack_word(wsel, u, uc);                                                       \
        const half2_t q0 = (__builtin_bit_cast(half2_t, u[0]) + o1024[bn]) * dd[bn];    \
        const half2_t q1 = (__builtin_bit_cast(half2_t, u[1]) + o64[bn]) * dd[bn];      \
        const half2_t q2 = (__builtin_bit_cast(half2_t, u[2]) + o1024[bn]) * dd[bn];    \
        const half2_t q3 = (__builtin_bit_cast(half2_t, u[3]) + o64[bn]) * dd[bn];      \
        bq[bn] = __builtin_bit_cast(                                                    \
            half8_t, make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1), \
                                __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3))); \
      }                                                                                 \
      /* each A fragment is reloaded for the next sub-step right after its last use */  \
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
  int kt = kt0;
  for (; kt + 1 < kt1; kt += 2) {
    AWQ_GEMM_STEP(kt, a_st0, a_st1);
    AWQ_GEMM_STEP(kt + 1, a_st1, a_st0);
  }
  if (kt < kt1) AWQ_GEMM_STEP(kt, a_st0, a_st1);
#undef AWQ_GEMM_STEP
#undef AWQ_GEMM_A_READ
#undef AWQ_GEMM_LOAD_A
#undef AWQ_GEMM_LOAD_B

  // ---- epilogue: value e of lane l in block (bm, bn) is row 8(e/4) + 4(l/32) + e%4, column l%32
  if (ks == 1) {
#pragma unroll
    for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
      for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = m0 + wm * RW + bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
          const int64_t cidx = n0 + wn * CW + bn * 32 + (lane & 31);
          if (t < m && cidx < n) y[t * n + cidx] = f2act(acc[bm][bn][e], gp.bf != 0);
        }
    return;
  }
  // split along K: the fp32 partial tile (its valid rows) goes to slice sl of
  // the tile's partials; linear_gemm_reduce_kernel, the next launch, sums the
  // slices in slice order
  const int rows_t = m < BM ? (int)m : BM;                   // partial rows per tile
  const int mrow = (m - m0) < rows_t ? (int)(m - m0) : rows_t;
  float* __restrict__ part = L.part + ((size_t)tl * ks + sl) * rows_t * kGemmBN;
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
    for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * RW + bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int col = wn * CW + bn * 32 + (lane & 31);
        // the element goes through a scalar first (a bit cast of an element of
        // a vector value reads the vector's first element on this compiler)
        const float v = acc[bm][bn][e];
        if (row < mrow) part[row * kGemmBN + col] = v;
      }
}

// ---------------------------------------------------------------- prefill GEMM, m > 128
// Work-group tile 128 tokens x 256 output columns, K-step 64, 4 waves side by
// side along N, each wave 128 x 64 = 4 x 2 blocks of v_mfma_f32_32x32x16_f16.
// Against a 256 x 128 tile in a 2 x 2 wave arrangement the same MFMA work
// reads 26 instead of 40 KB per K-step (16 KB of activations, 8 KB of packed
// weights loaded once, 2 KB of scales and zero words) and every column is
// dequantized by one wave only.
//  * Every global load of the K loop is a 16- or 4-byte global -> LDS copy
//    into a ring of three stages, issued two K-steps ahead, so that a copy has
//    two K-steps of MFMA work to land.  A stage holds the x_tilde tile (rows
//    of 64 channels, chunks XOR-swizzled by row as in the 64-row kernel), the
//    packed words of the 256 columns (two 16-byte chunks per column, swapped
//    on every other column quad so that 8 lanes reading 8 columns hit 32
//    distinct banks), and per column the 32-bit word holding the step's fp16
//    scale (with its neighbour group) and the zero word.
//  * The copies are inline asm: the compiler neither sees nor waits for them.
//    Per K-step one explicit wait and one barrier: the wave's own copies of
//    the step have landed (those of the next step stay in flight), then every
//    wave's copies are visible and no wave still reads the stage the next
//    copies overwrite.  Every K-step issues the same copies (past the last
//    step they repeat it), so the wait count is a constant.
//  * Dequantization as in the 64-row kernel, the scale and zero point formed
//    as fp16 pairs straight from their bits.
// Needs 4-byte aligned scales and an even number of groups per column (the
// scale words); the host takes the 64-row kernel otherwise.

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// lane i copies 16 (resp. 4) bytes from sbase + voff (sbase wave-uniform, in
// SGPRs; voff the lane's 32-bit byte offset) to LDS bytes lds_base + 16 i
// (resp. 4 i); no output register, the caller waits with an explicit vmcnt
__device__ __forceinline__ void g2_copy16(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void g2_copy4(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop
#define AWQ_G2_WAIT_VMCNT(N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory")
// A work-group barrier without the memory fence of __syncthreads (which
// waits for every outstanding global load, the look-ahead included); the
// empty statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void g2_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

#ifndef AWQ_G2_GROUP_M
#define AWQ_G2_GROUP_M 4
#endif
// The 128-row kernel walks each linear's tiles in bands of AWQ_G2_GROUP_M row
// tiles (banded_tile_coords): at m = 2048 the ~64 work-groups resident on an
// XCD share 4 row tiles of activations and 16 column tiles of weights instead
// of 16 row tiles of 4 columns (the prefill layer 926 -> 938 TFLOP/s with
// bands of 4, 935 with bands of 8).

template <int G, int KG>
__global__ __launch_bounds__(256 * KG, KG == 1 ? 2 : 1) void linear_gemm2_kernel(const LinGroup gp, int64_t m,
                                                                                 int64_t k, int tiles_m) {
  constexpr int BM = kG2BM, BN = kG2BN, BK = kGemmBK;
  constexpr int BMB = BM / 32, BNB = 2;               // 32 x 32 blocks per wave
  constexpr int AR = BM / 32;                         // A copies per wave and step (8 rows each)
  constexpr int kCopiesPerStep = AR + 2 + 2;          // + 2 KB of packed words, scale and zero words
  static_assert(kG2Stages == 3 && BN == 4 * 64, "three stages, four waves of 64 columns");
  static_assert(KG == 1 || KG == 2, "one or two K groups");
  // stage s, K group g: bytes (s KG + g) kG2Stage ..
  __shared__ __attribute__((aligned(16))) unsigned char ring[kG2Stages * KG * kG2Stage];
  const int ng = (int)(k / G), nzw = (ng + 7) / 8;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = wave >> 2, wv = wave & 3;          // K group, wave within the group
  // XCD-aware order: each XCD takes a contiguous run of the tile order
  // (banded within each linear)
  const int total = gp.wg0[gp.count];
  const int bid = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, slot = bid / 8;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const LinPick L = pick_linear_at(gp, tile);
  uint16_t* __restrict__ y = L.y;
  const int64_t n = L.n;
  const int ks = L.ks;
  const int t_ord = L.bid / ks, sl = L.bid - t_ord * ks;
  int tm, tn;
  banded_tile_coords<AWQ_G2_GROUP_M>(t_ord, tiles_m, (int)((n + BN - 1) / BN), tm, tn);
  const int tl = tm + tn * tiles_m;                   // the tile's slot among the partial tiles
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kw_row = k / 8;
  const int nk = (int)(k / BK);
  const int kt0 = (int)((int64_t)sl * nk / ks), kt1 = (int)((int64_t)(sl + 1) * nk / ks);
  // round P: K group g multiplies K-step kt0 + KG P + g
  const int nr = (kt1 - kt0 + KG - 1) / KG;

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(&ring[0]) + (uint32_t)(kgrp * kG2Stage);
  const unsigned char* ring_g = ring + kgrp * kG2Stage;
  // ---- copy sources: a wave-uniform base per K-step (SGPRs) plus the lane's
  // fixed 32-bit byte offset (x_tilde of one launch and the packed tensors of
  // one linear stay below 2^31 resp. 2^32 bytes).
  // A: wave w of a K group copies rows 32 w .. 32 w + 31 of the tile, lane
  // (row r = 8 i + lane / 8, slot p = lane % 8) the logical chunk
  // p ^ swizzle(r), so that lane i fills LDS slot i.
  const int a_lr = lane >> 3, a_p = lane & 7;
  uint32_t a_voff[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int lrow = wv * (BM / 4) + 8 * i + a_lr;
    int64_t row = m0 + lrow;
    row = row < m ? row : m - 1;
    a_voff[i] = (uint32_t)((row * k + (a_p ^ ((lrow >> AWQ_GEMM_SWZ_SHIFT) & 7)) * 8) * 2);
  }
  // B: wave w copies the 32-byte K-step slices of columns 64 w .. 64 w + 63,
  // two per copy instruction: lane i fills slot i of column 32 h + i / 2,
  // taking chunk (i % 2) ^ (bit 2 of the column)
  uint32_t b_voff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int lcol = wv * 64 + 32 * h + (lane >> 1);
    int64_t col = n0 + lcol;
    col = col < n ? col : n - 1;
    b_voff[h] = (uint32_t)(col * kw_row * 4 + (((lane & 1) ^ ((lcol >> 2) & 1)) * 16));
  }
  // scale and zero words: lane i of wave w, column 64 w + i
  int64_t sz_col = n0 + wv * 64 + lane;
  sz_col = sz_col < n ? sz_col : n - 1;
  const uint32_t s_voff = (uint32_t)(sz_col * ng * 2), z_voff = (uint32_t)(sz_col * nzw * 4);
  const char* xb = reinterpret_cast<const char*>(L.x);
  const char* qb = reinterpret_cast<const char*>(L.qw);
  const char* sb = reinterpret_cast<const char*>(L.sc);
  const char* zb = reinterpret_cast<const char*>(L.qz);
  // the copies of the K group's K-step of round P (clamped to the slice's
  // last step) into stage ST
#define AWQ_G2_LOAD(P, ST)                                                               \
  {                                                                                     \
    int kt_ = kt0 + KG * (P) + kgrp;                                                    \
    kt_ = kt_ < kt1 ? kt_ : kt1 - 1;                                                    \
    const uint32_t st_ = ring_lds + (uint32_t)((ST) * KG * kG2Stage);                   \
    const char* xk_ = xb + (int64_t)kt_ * BK * 2;                                       \
    _Pragma("unroll") for (int i = 0; i < AR; ++i)                                      \
      g2_copy16(a_voff[i], xk_, st_ + (uint32_t)((wv * (BM / 4) + 8 * i) * 128));       \
    const char* qk_ = qb + (int64_t)kt_ * 32;                                           \
    _Pragma("unroll") for (int h = 0; h < 2; ++h)                                       \
      g2_copy16(b_voff[h], qk_, st_ + (uint32_t)(kG2AStage + (wv * 64 + 32 * h) * 32));  \
    const int g0_ = (kt_ * BK) / G;                                                     \
    g2_copy4(s_voff, sb + (int64_t)(g0_ & ~1) * 2,                                      \
             st_ + (uint32_t)(kG2AStage + kG2BStage + wv * 256));                       \
    g2_copy4(z_voff, zb + (int64_t)(g0_ >> 3) * 4,                                      \
             st_ + (uint32_t)(kG2AStage + kG2BStage + BN * 4 + wv * 256));              \
  }

  floatx16_t acc[BMB][BNB];
#pragma unroll
  for (int i = 0; i < BMB; ++i)
#pragma unroll
    for (int jj = 0; jj < BNB; ++jj) acc[i][jj] = floatx16_t{};
  const UnpackConsts uc = unpack_consts();
  // ---- fragment reads.  A: byte offset of lane's fragment of row block bm at
  // sub-step 0 (row bm 32 + lane % 32, logical chunk 4 (lane / 32) + s stored
  // at chunk ^ swizzle(row); s flips chunk bits 0-1 only)
  const int bj = lane & 31, bc = lane >> 5;
  uint32_t a_base[BMB];
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm) {
    const int row = bm * 32 + bj;
    a_base[bm] = (uint32_t)(row * 128 + ((4 * bc) ^ ((row >> AWQ_GEMM_SWZ_SHIFT) & 7)) * 16);
  }
  // B: lane (column j, half c) of block bn reads the 4 words 4c .. 4c + 3 of
  // column 64 w + 32 bn + j; scale and zero words of that column
  uint32_t b_off[BNB], s_off[BNB], z_off[BNB];
#pragma unroll
  for (int bn = 0; bn < BNB; ++bn) {
    const int lcol = wv * 64 + bn * 32 + bj;
    b_off[bn] = (uint32_t)(kG2AStage + lcol * 32 + ((bc ^ ((lcol >> 2) & 1)) * 16));
    s_off[bn] = (uint32_t)(kG2AStage + kG2BStage + lcol * 4);
    z_off[bn] = (uint32_t)(kG2AStage + kG2BStage + BN * 4 + lcol * 4);
  }

  // The operands a wave copied itself (the packed words, scale and zero words
  // of its own 64 columns) need only its own wait, not the barrier: they are
  // read from LDS, and the step's scale and zero point formed as fp16 pairs
  // (d, d), (-1024 - z) and (-64 - z) straight from their bits, at the end of
  // the previous round, so that after the barrier only the shared activation
  // fragments stand between the wave and its first MFMA.
  struct BSet {
    uint4 wb[BNB];
    half2_t dd[BNB], o1024[BNB], o64[BNB];
  };
#define AWQ_G2_PREP(P, ST, R)                                                            \
  {                                                                                     \
    const unsigned char* p_ = ring_g + (ST) * KG * kG2Stage;                            \
    const int grp_ = ((kt0 + KG * (P) + kgrp) * BK + 32 * bc) / G;                      \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                                \
      R.wb[bn] = *reinterpret_cast<const uint4*>(p_ + b_off[bn]);                       \
      const uint32_t sw_ = *reinterpret_cast<const uint32_t*>(p_ + s_off[bn]);          \
      const uint32_t zw_ = *reinterpret_cast<const uint32_t*>(p_ + z_off[bn]);          \
      const uint32_t s_ = (sw_ >> (16 * (grp_ & 1))) & 0xFFFFu;                         \
      const uint32_t z_ = (zw_ >> (4 * (grp_ & 7))) & 0xFu;                             \
      R.dd[bn] = __builtin_bit_cast(half2_t, s_ | (s_ << 16));                          \
      R.o1024[bn] = __builtin_bit_cast(half2_t, (0xE400u + z_) * 0x10001u);             \
      R.o64[bn] = __builtin_bit_cast(half2_t, (0xD400u + (z_ << 4)) * 0x10001u);        \
    }                                                                                   \
  }
  // dequantized B fragments of sub-step S (word S of each block) from R
#define AWQ_G2_DQ(R, S, OUT)                                                             \
  {                                                                                     \
    _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) {                                \
      const uint32_t wsel = (S) == 0 ? R.wb[bn].x : (S) == 1 ? R.wb[bn].y : (S) == 2 ? R.wb[bn].z : R.wb[bn].w; \
      uint32_t u[4];                                                                    \
      unpack_word(wsel, u, uc);                                                         \
      const half2_t q0 = (__builtin_bit_cast(half2_t, u[0]) + R.o1024[bn]) * R.dd[bn];    \
      const half2_t q1 = (__builtin_bit_cast(half2_t, u[1]) + R.o64[bn]) * R.dd[bn];      \
      const half2_t q2 = (__builtin_bit_cast(half2_t, u[2]) + R.o1024[bn]) * R.dd[bn];    \
      const half2_t q3 = (__builtin_bit_cast(half2_t, u[3]) + R.o64[bn]) * R.dd[bn];      \
      OUT[bn] = __builtin_bit_cast(                                                     \
          half8_t, make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1), \
                              __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3))); \
    }                                                                                   \
  }
  // Round P (stage ST, weights in R, the B fragments of its first sub-step in
  // bq): meet (every wave has its copies of P), then four 16-channel
  // sub-steps as in the 64-row kernel.  Each sub-step's MFMAs run while the
  // B fragments of the next are dequantized; the copies of round P + 2 go
  // into the stage round P - 1 used once the first sub-step's MFMAs are
  // issued; the last sub-step waits for the wave's own copies of round P + 1,
  // prepares its weights into RN and dequantizes its first B fragments.  With
  // two K groups the second has no K-step in the last round when the slice's
  // step count is odd: it only copies and prepares.
#define AWQ_G2_STEP(P, ST, STN, STP, R, RN)                                              \
  {                                                                                     \
    /* the previous round's work (the first B fragments of this one          */       \
    /* included) is issued before the barrier, not after it                  */       \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    g2_barrier();                                                                       \
    if (KG == 1 || kt0 + KG * (P) + kgrp < kt1) {                                       \
      const unsigned char* cur_ = ring_g + (ST) * KG * kG2Stage;                        \
      half8_t af[BMB];                                                                  \
      _Pragma("unroll") for (int bm = 0; bm < BMB; ++bm)                                \
        af[bm] = *reinterpret_cast<const half8_t*>(cur_ + a_base[bm]);                  \
      _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                   \
        half8_t bqn[BNB];                                                               \
        if (s < 3) {                                                                    \
          AWQ_G2_DQ(R, s + 1, bqn)                                                      \
        } else {                                                                        \
          AWQ_G2_WAIT_VMCNT(kCopiesPerStep);                                            \
          AWQ_G2_PREP((P) + 1, STP, RN)                                                 \
          AWQ_G2_DQ(RN, 0, bqn)                                                         \
        }                                                                               \
        _Pragma("unroll") for (int bm = 0; bm < BMB; ++bm) {                            \
          _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn)                            \
            acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[bm], bq[bn], acc[bm][bn], 0, 0, 0); \
          if (s + 1 < 4)                                                                \
            af[bm] = *reinterpret_cast<const half8_t*>(cur_ + (a_base[bm] ^ (uint32_t)(16 * (s + 1)))); \
        }                                                                               \
        if (s == 0) AWQ_G2_LOAD((P) + 2, STN)                                           \
        _Pragma("unroll") for (int bn = 0; bn < BNB; ++bn) bq[bn] = bqn[bn];            \
      }                                                                                 \
    } else {                                                                            \
      AWQ_G2_LOAD((P) + 2, STN)                                                         \
      AWQ_G2_WAIT_VMCNT(kCopiesPerStep);                                                \
      AWQ_G2_PREP((P) + 1, STP, RN)                                                     \
      AWQ_G2_DQ(RN, 0, bq)                                                              \
    }                                                                                   \
  }
  BSet r0, r1;
  half8_t bq[BNB];
  AWQ_G2_LOAD(0, 0)
  AWQ_G2_LOAD(1, 1)
  AWQ_G2_WAIT_VMCNT(kCopiesPerStep);
  AWQ_G2_PREP(0, 0, r0)
  AWQ_G2_DQ(r0, 0, bq)
  int rp = 0;
  for (; rp + 3 <= nr; rp += 3) {
    AWQ_G2_STEP(rp, 0, 2, 1, r0, r1)
    AWQ_G2_STEP(rp + 1, 1, 0, 2, r1, r0)
    AWQ_G2_STEP(rp + 2, 2, 1, 0, r0, r1)
    r0 = r1;
  }
  if (rp < nr) {
    AWQ_G2_STEP(rp, 0, 2, 1, r0, r1)
    r0 = r1;
  }
  if (rp + 1 < nr) {
    AWQ_G2_STEP(rp + 1, 1, 0, 2, r0, r1)
  }
  AWQ_G2_WAIT_VMCNT(0);               // the look-ahead copies have landed before the wave ends
#undef AWQ_G2_STEP
#undef AWQ_G2_DQ
#undef AWQ_G2_PREP
#undef AWQ_G2_LOAD

  // ---- two K groups: the second hands its sums to the first through LDS
  // (element-major, 16 bytes per lane: consecutive lanes, consecutive bytes)
  if constexpr (KG == 2) {
    g2_barrier();                     // every copy landed, every fragment read done
    float* red = reinterpret_cast<float*>(ring) + wv * (BMB * BNB * 16 * 64);
    if (kgrp == 1) {
#pragma unroll
      for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
        for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(red + (((bm * BNB + bn) * 4 + q) * 64 + lane) * 4) =
                make_float4(acc[bm][bn][4 * q], acc[bm][bn][4 * q + 1], acc[bm][bn][4 * q + 2],
                            acc[bm][bn][4 * q + 3]);
    }
    g2_barrier();
    if (kgrp == 1) return;
#pragma unroll
    for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
      for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(red + (((bm * BNB + bn) * 4 + q) * 64 + lane) * 4);
          acc[bm][bn][4 * q] += v.x;
          acc[bm][bn][4 * q + 1] += v.y;
          acc[bm][bn][4 * q + 2] += v.z;
          acc[bm][bn][4 * q + 3] += v.w;
        }
  }

  // ---- epilogue: value e of lane l in block (bm, bn) is row 8(e/4) + 4(l/32) + e%4, column l%32
  if (ks == 1) {
    if (n % 8 == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
      // through LDS (free once every wave's copies have landed and its last
      // fragments are read; with two K groups each wave reuses its own part
      // of the hand-over area, already read): the wave's 128 x 64 outputs
      // into rows of 72 halves (the two lane halves of a write land 16 banks
      // apart), read back as 16-byte row chunks and stored 8 lanes per row
      constexpr int ER = 72;
      if constexpr (KG == 1) g2_barrier();
      uint16_t* ep = reinterpret_cast<uint16_t*>(ring) + wv * (KG == 1 ? BM * ER : BMB * BNB * 16 * 64 * 2);
#pragma unroll
      for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
        for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int row = bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
            ep[row * ER + bn * 32 + (lane & 31)] = f2act(acc[bm][bn][e], gp.bf != 0);
          }
#pragma unroll
      for (int i = 0; i < BM / 8; ++i) {
        const int row = 8 * i + (lane >> 3), c8 = (lane & 7) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(ep + row * ER + c8);
        const int64_t t = m0 + row, cidx = n0 + wv * 64 + c8;
        if (t < m && cidx < n) *reinterpret_cast<uint4*>(y + t * n + cidx) = v;
      }
    } else {
#pragma unroll
      for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
        for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t t = m0 + bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
            const int64_t cidx = n0 + wv * 64 + bn * 32 + (lane & 31);
            if (t < m && cidx < n) y[t * n + cidx] = f2act(acc[bm][bn][e], gp.bf != 0);
          }
    }
    return;
  }
  // split along K: the fp32 partial tile (its valid rows) goes to slice sl
  const int rows_t = m < BM ? (int)m : BM;
  const int mrow = (m - m0) < rows_t ? (int)(m - m0) : rows_t;
  float* __restrict__ part = L.part + ((size_t)tl * ks + sl) * rows_t * BN;
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
    for (int bn = 0; bn < BNB; ++bn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int col = wv * 64 + bn * 32 + (lane & 31);
        const float v = acc[bm][bn][e];
        if (row < mrow) part[row * BN + col] = v;
      }
}

// Sums the K slices of the split linears of a GEMM launch (linear
// blockIdx.y; a linear that was not split has no work here): every thread
// takes 4 adjacent columns of one row of one tile and adds the slices in
// slice order, all slice loads of a batch of 8 in flight together.
template <int BM, int BN>
__global__ __launch_bounds__(256) void linear_gemm_reduce_kernel(const LinGroup gp, int64_t m,
                                                                 int tiles_m) {
  int li = 0;
#pragma unroll
  for (int i = 1; i < kGroupMax; ++i)
    if (i == (int)blockIdx.y) li = i;
  const int ks = gp.ks[li];
  if (ks == 1) return;
  const int64_t n = gp.n[li];
  const float* __restrict__ part = gp.part[li];
  uint16_t* __restrict__ y = gp.y[li];
  const int rows_t = m < BM ? (int)m : BM;
  const int tiles = tiles_m * (int)((n + BN - 1) / BN);
  const int64_t chunks = (int64_t)tiles * rows_t * (BN / 4);
  const size_t slice_floats = (size_t)rows_t * BN;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
    const int tl = (int)(c / ((int64_t)rows_t * (BN / 4)));
    const int w = (int)(c - (int64_t)tl * rows_t * (BN / 4));
    const int row = w / (BN / 4), c4 = (w - row * (BN / 4)) * 4;
    const int tm = tl % tiles_m, tn = tl / tiles_m;
    const int64_t t = (int64_t)tm * BM + row, col = (int64_t)tn * BN + c4;
    if (t >= m) continue;
    const float* src = part + (size_t)tl * ks * slice_floats + (size_t)row * BN + c4;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ks; s0 += 8) {
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < ks) v[j] = *reinterpret_cast<const float4*>(src + (size_t)(s0 + j) * slice_floats);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (s0 + j < ks) {
          sum[0] += v[j].x;
          sum[1] += v[j].y;
          sum[2] += v[j].z;
          sum[3] += v[j].w;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (col + i < n) y[t * n + col + i] = f2act(sum[i], gp.bf != 0);
  }
}

// Work-groups of a group launch: the grid one launch of all the column blocks
// would take (fill the chip first, then at most nb_cap blocks per
// work-group), split over the linears in proportion to their blocks.  For a
// single linear this is that launch's grid.  Returns the most blocks any
// work-group gets.
static int split_group_grid(const LinItem* items, int count, int64_t slots, int nb_cap,
                            LinGroup& gp) {
  int64_t nblk[kGroupMax], total = 0;
  for (int l = 0; l < count; ++l) {
    nblk[l] = (items[l].n + 15) / 16;
    total += nblk[l];
  }
  int64_t grid_total = total < slots ? total : slots;
  const int64_t need = (total + nb_cap - 1) / nb_cap;
  grid_total = grid_total > need ? grid_total : need;
  int start = 0, nb = 1;
  for (int l = 0; l < count; ++l) {
    int64_t gl = grid_total * nblk[l] / total;
    const int64_t need_l = (nblk[l] + nb_cap - 1) / nb_cap;
    gl = gl > need_l ? gl : need_l;
    gl = gl < nblk[l] ? gl : nblk[l];
    gl = gl > 0 ? gl : 1;
    gp.x[l] = items[l].x;
    gp.inv[l] = items[l].inv;
    gp.qw[l] = items[l].qw;
    gp.sc[l] = items[l].sc;
    gp.qz[l] = items[l].qz;
    gp.y[l] = items[l].y;
    gp.n[l] = items[l].n;
    gp.wg0[l] = start;
    start += (int)gl;
    const int nbl = (int)((nblk[l] + gl - 1) / gl);
    nb = nb > nbl ? nb : nbl;
  }
  for (int l = count; l < kGroupMax; ++l) {
    gp.x[l] = nullptr; gp.inv[l] = nullptr; gp.qw[l] = nullptr; gp.sc[l] = nullptr;
    gp.qz[l] = nullptr; gp.y[l] = nullptr; gp.n[l] = 0;
  }
  for (int l = count; l <= kGroupMax; ++l) gp.wg0[l] = start;
  gp.count = count;
  gp.bf = items[0].bf;
  return nb;
}

// The decode kernels address the packed weights with 32-bit byte offsets
// (including the up to 16 rows past n of the last column block, and one block
// past the end), the activations of up to 32 tokens likewise.
static bool offsets32_ok(const LinItem* items, int count, int64_t k) {
  const uint64_t lim = (uint64_t)1 << 32;
  if ((uint64_t)32 * (uint64_t)k * 2 >= lim) return false;
  for (int l = 0; l < count; ++l) {
    const uint64_t rows = (uint64_t)((items[l].n + 15) / 16) * 16 + 16;
    if (rows * (uint64_t)k / 2 >= lim) return false;
  }
  return true;
}

static bool scales_octets(const LinItem* items, int count, int64_t ng) {
  if (ng % 8 != 0) return false;
  for (int l = 0; l < count; ++l)
    if (reinterpret_cast<uintptr_t>(items[l].sc) % 16 != 0) return false;
  return true;
}

template <int G>
static hipError_t launch_linear_one(const LinItem& it, int64_t m, int64_t k, Scratch& scr,
                                    hipStream_t stream) {
  const uint16_t* x = it.x;
  const uint32_t* qweight = it.qw;
  const uint16_t* scales = it.sc;
  const uint32_t* qzeros = it.qz;
  const uint16_t* inv_s16 = it.inv;
  uint16_t* y = it.y;
  const int64_t n = it.n;
  const bool bf = it.bf != 0;
  // 16 < m <= 32: prep16 + skinny16 when its LDS plan fits (with 32 tokens the
  // activation operand formed once per call beats forming it per item)
  if (m > 16 && m <= 32 && offsets32_ok(&it, 1, k)) {
    const int tcs = 2;
    const int64_t ng_all = k / G, nzw_all = (ng_all + 7) / 8;
    const int64_t nblk = (n + 15) / 16;
    int nb_cap = kGemvMaxBlk;
    while (nb_cap > 0 && ((int64_t)nb_cap * 16 * nzw_all > (int64_t)kGemvSzRounds * kSk16Threads ||
                          skinny16_lds_bytes(k, G, nb_cap, tcs) > 160 * 1024))
      --nb_cap;
    if (nb_cap > 0) {
      int64_t per_cu = (int64_t)(160 * 1024) / (int64_t)skinny16_lds_bytes(k, G, nb_cap, tcs);
      per_cu = per_cu < 2 ? per_cu : 2;
      const int64_t slots = (int64_t)kGemvCUs * per_cu;
      int64_t grid = nblk < slots ? nblk : slots;
      const int64_t need = (nblk + nb_cap - 1) / nb_cap;
      grid = grid > need ? grid : need;
      const int nb = (int)((nblk + grid - 1) / grid);
      const size_t lds = skinny16_lds_bytes(k, G, nb, tcs);
      const bool szv = (ng_all % 8 == 0) && (reinterpret_cast<uintptr_t>(scales) % 16 == 0);
      // x_tilde [2][ng][4][16][g/4] halves, then T, U [2][ng][16] float2
      const size_t a_bytes = align256((size_t)tcs * (size_t)k * 16 * 2);
      char* sp16 = scr.at(0, a_bytes + (size_t)tcs * (size_t)ng_all * 16 * 8);
      if (scr.dry) return hipSuccess;
      uint16_t* a16 = reinterpret_cast<uint16_t*>(sp16);
      float2* tu16 = reinterpret_cast<float2*>(sp16 + a_bytes);
      const int64_t n_pairs = tcs * ng_all;
      hipLaunchKernelGGL(linear_prep16_kernel<G>, dim3((unsigned)((n_pairs + 3) / 4)), dim3(256), 0,
                         stream, x, inv_s16, m, k, n_pairs, a16, tu16, bf);
      const dim3 gd((unsigned)grid), bd(kSk16Threads);
#define AWQ_SK16(SZ)                                                                           \
  {                                                                                            \
    const void* fn_ = reinterpret_cast<const void*>(&linear_skinny16_kernel<G, 2, SZ, 1>);      \
    if (lds > 65536) {                                                                         \
      hipError_t e_ = hipFuncSetAttribute(fn_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e_ != hipSuccess) return e_;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((linear_skinny16_kernel<G, 2, SZ, 1>), gd, bd, lds, stream, a16, tu16,   \
                       qweight, scales, qzeros, m, n, k, y, bf);                               \
  }
      if (szv) AWQ_SK16(true) else AWQ_SK16(false)
#undef AWQ_SK16
      return hipGetLastError();
    }
  }
  // the staged two-kernel decode path (any m <= 32 whose plans above do not fit)
  const int64_t tc = (m + kSkinnyTok - 1) / kSkinnyTok;
  const int64_t ng = k / G;
  // x_tilde [tc][ng][4][16][g/4] halves, then T, U [tc][ng][16] float2
  const size_t a_bytes = align256((size_t)tc * (size_t)k * 16 * 2);
  char* sp = scr.at(0, a_bytes + (size_t)tc * (size_t)ng * 16 * 8);
  if (scr.dry) return hipSuccess;
  uint16_t* a_st = reinterpret_cast<uint16_t*>(sp);
  float2* tu = reinterpret_cast<float2*>(sp + a_bytes);
  const int64_t n_pairs = tc * ng;
  hipLaunchKernelGGL(linear_prep_kernel<G>, dim3((unsigned)((n_pairs + 3) / 4)), dim3(256), 0,
                     stream, x, inv_s16, m, k, n_pairs, a_st, tu, bf);
  dim3 grid((unsigned)((n + 15) / 16));
  dim3 block(kSkinnyWaves * 64);
  switch (tc) {
    case 1:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 1>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y, bf);
      break;
    case 2:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 2>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y, bf);
      break;
    case 3:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 3>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y, bf);
      break;
    default:
      hipLaunchKernelGGL((linear_skinny_kernel<G, 4>), grid, block, 0, stream, qweight, scales,
                         qzeros, a_st, tu, m, n, k, y, bf);
      break;
  }
  return hipGetLastError();
}

// 17 <= m <= 32: a linear that a call of it alone would not run fused (more
// than 16 MiB of packed weights) and that is wide (at least 12288 columns)
// takes the GEMM.  A property of the linear alone, as every plan choice.
// 17 to 32 tokens: the linears that run the grouped GEMM (64-row tiles, split
// along K) rather than the two-chunk group-major kernel: more than 16 MiB of
// packed weights with either more column blocks than one round of one
// work-group per CU takes at two blocks each, or k > 8192.  Measured at 20 and
// 32 tokens: the kernel is faster for q/k/v (12 MiB) and o (8 MiB) of
// Llama-3-8B and the 70B-shaped 8192 x 8192 (32 MiB, 512 blocks), the GEMM for
// gate/up (28 MiB each, 896 blocks each) and down (28 MiB at k = 14336).
static bool skinny_wide(const LinItem& it, int64_t m, int64_t k) {
  const int64_t blocks = (it.n + 15) / 16;
  return m > 16 && m <= 32 && it.n * k / 2 > ((int64_t)16 << 20) &&
         (blocks > 2 * (int64_t)kGemvCUs || k > 8192);
}

// The prefill GEMM of a group (m > 32): x_tilde of every linear into a
// scratch slot of its own (one launch for all), then one GEMM launch over
// the tiles of all linears.  The kernel addresses its activations with 32-bit
// byte offsets: an m whose x_tilde reaches 2^31 bytes runs linear after
// linear, in row chunks, through scratch slot 0.
template <int G>
static hipError_t launch_gemm_group(const LinItem* items, int count, int64_t m, int64_t k,
                                    Scratch& scr, hipStream_t stream) {
  const int bm = gemm_bm(m, k, G), bn = gemm_bn(bm);
  const int64_t chunk = gemm_row_chunk(k);
  const bool whole = m <= chunk;
  // slices of every linear (one when the call runs in row chunks), and the
  // LDS for the longest slice of the launch
  int sks[kGroupMax];
  int gmax = 0;
  for (int l = 0; l < count; ++l) {
    sks[l] = whole ? gemm_split(m, items[l].n, k, G) : 1;
    const int gl = gemm_slice_groups(k, G, sks[l]);
    gmax = gmax > gl ? gmax : gl;
  }
  // dynamic LDS: the scales and zero words of the 64-row kernel (the 128-row
  // kernel has only its static stages)
  const size_t lds = bm == 64 ? gemm_lds_bytes(gmax) : 0;
  const size_t lds_static = gemm_static_lds(bm);
  const void* fn = reinterpret_cast<const void*>(&linear_gemm_kernel<G>);
  if (lds + lds_static > 160 * 1024) return hipErrorInvalidValue;
  // scratch: one x_tilde slot per linear and the fp32 partial tiles of the
  // split linears (whole m in one launch), else slot 0 reused linear by linear
  const size_t slot_bytes = align256((size_t)m * (size_t)k * 2);
  size_t scratch_bytes = whole ? (size_t)count * slot_bytes : slot_bytes;
  if (whole)
    for (int l = 0; l < count; ++l)
      if (sks[l] > 1) scratch_bytes += gemm_part_bytes(m, items[l].n, k, G);
  char* const scratch = scr.at(0, scratch_bytes);
  if (scr.dry) return hipSuccess;
  if (bm == 64 && lds + lds_static > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int n_batch = whole ? 1 : count;
  for (int bt = 0; bt < n_batch; ++bt) {
    const LinItem* its = whole ? items : items + bt;
    const int cnt = whole ? count : 1;
    LinGroup xg = {};
    for (int l = 0; l < cnt; ++l) {
      xg.x[l] = its[l].x;
      xg.inv[l] = its[l].inv;
      xg.y[l] = reinterpret_cast<uint16_t*>(scratch + (size_t)l * slot_bytes);
    }
    xg.count = cnt;
    xg.bf = its[0].bf;
    const int64_t chunks = m * (k / 8);
    const int64_t pgrid = (chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096;
    hipLaunchKernelGGL(linear_xprep_kernel, dim3((unsigned)pgrid, (unsigned)cnt), dim3(256), 0,
                       stream, xg, m, k);
    for (int64_t r0 = 0; r0 < m; r0 += chunk) {
      const int64_t mc = (m - r0) < chunk ? (m - r0) : chunk;
      const int tiles_m = (int)((mc + bm - 1) / bm);
      // the work-groups of every linear and, for the 128-row kernel, its
      // K groups: two where the linear, not split along K, has at most one
      // work-group per CU (a property of the linear, so that a group call
      // gives the bits of the single calls; linears of both kinds take one
      // launch per kind).  A split linear has work-groups enough for two per
      // CU, and so has a group of them.
      int wgs[kGroupMax], kgs[kGroupMax];
      char* parts[kGroupMax];
      char* part = scratch + (size_t)cnt * slot_bytes;
      for (int l = 0; l < cnt; ++l) {
        // split along K only where the whole m is one launch (mc == m)
        const int sk = whole ? sks[l] : 1;
        wgs[l] = tiles_m * (int)((its[l].n + bn - 1) / bn) * sk;
        kgs[l] = (bm != 64 && sk == 1 && wgs[l] <= kGemvCUs) ? 2 : 1;
        parts[l] = nullptr;
        if (sk > 1) {
          parts[l] = part;
          part += gemm_part_bytes(m, its[l].n, k, G);
        }
      }
      for (int kg = 1; kg <= 2; ++kg) {
        LinGroup gg = {};
        int total = 0, c = 0;
        bool split = false;
        for (int l = 0; l < cnt; ++l) {
          if (kgs[l] != kg) continue;
          const int64_t n = its[l].n;
          gg.x[c] = xg.y[l] + r0 * k;
          gg.qw[c] = its[l].qw;
          gg.sc[c] = its[l].sc;
          gg.qz[c] = its[l].qz;
          gg.y[c] = its[l].y + r0 * n;
          gg.n[c] = n;
          gg.wg0[c] = total;
          gg.ks[c] = whole ? sks[l] : 1;
          if (parts[l]) {
            gg.part[c] = reinterpret_cast<float*>(parts[l]);
            split = true;
          }
          total += wgs[l];
          ++c;
        }
        if (c == 0) continue;
        for (int l = c; l <= kGroupMax; ++l) gg.wg0[l] = total;
        gg.count = c;
        gg.bf = its[0].bf;
        gg.gmax = gmax;
        if (bm == 64)
          hipLaunchKernelGGL((linear_gemm_kernel<G>), dim3((unsigned)total), dim3(256), lds, stream,
                             gg, mc, k, tiles_m);
        else if (kg == 2)
          hipLaunchKernelGGL((linear_gemm2_kernel<G, 2>), dim3((unsigned)total), dim3(512), 0, stream,
                             gg, mc, k, tiles_m);
        else
          hipLaunchKernelGGL((linear_gemm2_kernel<G, 1>), dim3((unsigned)total), dim3(256), 0, stream,
                             gg, mc, k, tiles_m);
        if (split) {
          // the slices of every split linear (a few MB of fp32 partials, still
          // in the caches): a grid over the chip per linear
          const dim3 rg(256u, (unsigned)c);
          if (bm == 64)
            hipLaunchKernelGGL((linear_gemm_reduce_kernel<64, kGemmBN>), rg, dim3(256), 0, stream, gg, mc,
                               tiles_m);
          else
            hipLaunchKernelGGL((linear_gemm_reduce_kernel<kG2BM, kG2BN>), rg, dim3(256), 0, stream, gg,
                               mc, tiles_m);
        }
      }
    }
  }
  return hipGetLastError();
}

template <int G>
static hipError_t launch_linear_group_g(const LinItem* items, int count, int64_t m, int64_t k,
                                        Scratch& scr, hipStream_t stream) {
  // fused skinny plan above 16 tokens: groups of at most this many packed bytes
  constexpr int64_t kFusedMax = (int64_t)16 << 20;
  if (m > 32) return launch_gemm_group<G>(items, count, m, k, scr, stream);
  // the decode GEMV (m = 1): at most kGemvMaxBlk column blocks per
  // work-group, whose scale/zero octets fit the prologue (kGemvSzRounds per
  // thread) and whose LDS plan fits 160 KiB
  const bool off32 = offsets32_ok(items, count, k);
  if (m == 1 && off32) {
    const int64_t ng_all = k / G, nzw_all = (ng_all + 7) / 8;
    auto plan = [&](int waves, int& nb_cap, int64_t& per_cu) {
      nb_cap = kGemvMaxBlk;
      while (nb_cap > 0 && ((int64_t)nb_cap * 16 * nzw_all > (int64_t)kGemvSzRounds * waves * 64 ||
                            gemv_lds_bytes(k, G, nb_cap, waves) > 160 * 1024))
        --nb_cap;
      per_cu = nb_cap > 0 ? (int64_t)(160 * 1024) / (int64_t)gemv_lds_bytes(k, G, nb_cap, waves) : 0;
      const int64_t wg_cap = 16 / waves;            // 16 waves per CU (4 per SIMD)
      per_cu = per_cu < wg_cap ? per_cu : wg_cap;
    };
    int nb_cap = 0;
    int64_t per_cu = 0;
    plan(8, nb_cap, per_cu);
    int waves = 8;
    // LDS leaves room for one 8-wave work-group per CU: 16 waves put twice
    // the weight bytes in flight.  Also 16 waves for long K (>= 8192) and at
    // most two blocks per CU: half the work-groups, each staging its K once
    // for up to two blocks, with as many waves per CU (Llama-3-70B-shaped
    // 8192<-8192 11.9 -> 11.5 us, 1024<-8192 7.0 -> 6.8 us; at K = 4096 the
    // stack's q/k/v and o were 3 % slower so)
    int64_t blocks_all = 0;
    for (int l = 0; l < count; ++l) blocks_all += (items[l].n + 15) / 16;
    if (nb_cap > 0 && (per_cu < 2 || (k >= 8192 && blocks_all <= 2 * kGemvCUs))) {
      int nb16 = 0;
      int64_t pc16 = 0;
      plan(16, nb16, pc16);
      if (nb16 > 0 && pc16 >= 1) { waves = 16; nb_cap = nb16; per_cu = pc16; }
    }
    if (nb_cap > 0 && per_cu >= 1) {
      LinGroup gp = {};
      const int nb = split_group_grid(items, count, (int64_t)kGemvCUs * per_cu, nb_cap, gp);
      const size_t lds = gemv_lds_bytes(k, G, nb, waves);
      const bool szv = scales_octets(items, count, ng_all);
      if (scr.dry) return hipSuccess;               // the decode GEMV takes no scratch
      const void* fn =
          waves == 16 ? (szv ? reinterpret_cast<const void*>(&linear_gemv_kernel<G, true, 16>)
                             : reinterpret_cast<const void*>(&linear_gemv_kernel<G, false, 16>))
                      : (szv ? reinterpret_cast<const void*>(&linear_gemv_kernel<G, true, 8>)
                             : reinterpret_cast<const void*>(&linear_gemv_kernel<G, false, 8>));
      if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
      }
      const dim3 gd((unsigned)gp.wg0[count]), bd((unsigned)(waves * 64));
      if (waves == 16) {
        if (szv)
          hipLaunchKernelGGL((linear_gemv_kernel<G, true, 16>), gd, bd, lds, stream, gp, k);
        else
          hipLaunchKernelGGL((linear_gemv_kernel<G, false, 16>), gd, bd, lds, stream, gp, k);
      } else {
        if (szv)
          hipLaunchKernelGGL((linear_gemv_kernel<G, true, 8>), gd, bd, lds, stream, gp, k);
        else
          hipLaunchKernelGGL((linear_gemv_kernel<G, false, 8>), gd, bd, lds, stream, gp, k);
      }
      return hipGetLastError();
    }
  }
  // 2 <= m <= 8: the decode GEMV with token rows for every linear whose
  // activations fit its LDS plan with all its column blocks in one round of
  // work-groups (a property of the linear, so a group call gives the bits of
  // the single calls; a group with linears of both kinds runs them one by one)
#ifndef AWQ_GEMV_ROWS
#define AWQ_GEMV_ROWS 1
#endif
  if (AWQ_GEMV_ROWS && m >= 2 && m <= kRowsMaxTok && off32) {
    const int64_t ng_all = k / G, nzw_all = (ng_all + 7) / 8;
    auto plan = [&](int waves, int cap, int& nb_cap, int64_t& per_cu) {
      nb_cap = cap;
      while (nb_cap > 0 && ((int64_t)nb_cap * 16 * nzw_all > (int64_t)kGemvSzRounds * waves * 64 ||
                            gemv_rows_lds_bytes(k, G, m, nb_cap, waves) > 160 * 1024))
        --nb_cap;
      per_cu = nb_cap > 0 ? (int64_t)(160 * 1024) / (int64_t)gemv_rows_lds_bytes(k, G, m, nb_cap, waves) : 0;
      const int64_t wg_cap = 16 / waves;
      per_cu = per_cu < wg_cap ? per_cu : wg_cap;
    };
    int nb_cap = 0, waves = 8;
    int64_t per_cu = 0;
    plan(8, kGemvMaxBlk, nb_cap, per_cu);
    if (nb_cap > 0 && per_cu < 2) {
      int nb16 = 0;
      int64_t pc16 = 0;
      plan(16, kRowsMaxBlk, nb16, pc16);
      if (nb16 > 0 && pc16 >= 1) { waves = 16; nb_cap = nb16; per_cu = pc16; }
    }
    int fits = 0;
    if (nb_cap > 0 && per_cu >= 1)
      for (int l = 0; l < count; ++l)
        if ((items[l].n + 15) / 16 <= (int64_t)kGemvCUs * per_cu * nb_cap) ++fits;
    if (fits == count) {
      LinGroup gp = {};
      const int nb = split_group_grid(items, count, (int64_t)kGemvCUs * per_cu, nb_cap, gp);
      const size_t lds = gemv_rows_lds_bytes(k, G, m, nb, waves);
      const bool szv = scales_octets(items, count, ng_all);
      if (scr.dry) return hipSuccess;               // no scratch
      const dim3 gd((unsigned)gp.wg0[count]), bd((unsigned)(waves * 64));
#define AWQ_GR(SZ, WW)                                                                         \
  {                                                                                            \
    const void* fn_ = reinterpret_cast<const void*>(&linear_gemv_rows_kernel<G, SZ, WW>);      \
    if (lds > 65536) {                                                                         \
      hipError_t e_ = hipFuncSetAttribute(fn_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e_ != hipSuccess) return e_;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((linear_gemv_rows_kernel<G, SZ, WW>), gd, bd, lds, stream, gp, m, k);   \
  }
      if (waves == 16) {
        if (szv) AWQ_GR(true, 16) else AWQ_GR(false, 16)
      } else {
        if (szv) AWQ_GR(true, 8) else AWQ_GR(false, 8)
      }
#undef AWQ_GR
      return hipGetLastError();
    }
    if (fits > 0) {
      for (int l = 0; l < count; ++l) {
        hipError_t e = launch_linear_group_g<G>(items + l, 1, m, k, scr, stream);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  // 17 <= m <= 32: the wide linears as one grouped GEMM launch, the others
  // as one launch of the group-major kernel with two token chunks (one
  // work-group per CU), when its LDS plan fits
#ifndef AWQ_SKINNY_GM2
#define AWQ_SKINNY_GM2 1
#endif
#ifndef AWQ_SKINNY_GM2_PF
#define AWQ_SKINNY_GM2_PF 1
#endif
  if (AWQ_SKINNY_GM2 && off32 && m > 16 && m <= 32) {
    const int64_t ng_all = k / G, nzw_all = (ng_all + 7) / 8;
    // at g = 128 three or more blocks spill registers
    int nb_cap = G == 128 ? 2 : kGemvMaxBlk;
    while (nb_cap > 0 && ((int64_t)nb_cap * 16 * nzw_all > (int64_t)kGemvSzRounds * kSk16Threads ||
                          skinny_gm_lds_bytes(k, G, nb_cap) > 160 * 1024))
      --nb_cap;
    if (nb_cap > 0) {
      LinItem wide[kGroupMax], rest[kGroupMax];
      int nw = 0, nr = 0;
      for (int l = 0; l < count; ++l) {
        if (skinny_wide(items[l], m, k)) wide[nw++] = items[l];
        else rest[nr++] = items[l];
      }
      if (nw > 0) {
        hipError_t e = launch_gemm_group<G>(wide, nw, m, k, scr, stream);
        if (e != hipSuccess || nr == 0) return e;
      }
      LinGroup gp = {};
      const int nb = split_group_grid(rest, nr, (int64_t)kGemvCUs, nb_cap, gp);
      const size_t lds = skinny_gm_lds_bytes(k, G, nb);
      const bool szv = scales_octets(rest, nr, ng_all);
      if (scr.dry) return hipSuccess;               // no scratch of its own
      const dim3 gd((unsigned)gp.wg0[nr]), bd(kSk16Threads);
#define AWQ_SKG2(SZ, NBB)                                                                      \
  {                                                                                            \
    const void* fn_ = reinterpret_cast<const void*>(&linear_skinny_gm2_kernel<G, SZ, NBB, AWQ_SKINNY_GM2_PF>); \
    if (lds > 65536) {                                                                         \
      hipError_t e_ = hipFuncSetAttribute(fn_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e_ != hipSuccess) return e_;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((linear_skinny_gm2_kernel<G, SZ, NBB, AWQ_SKINNY_GM2_PF>), gd, bd, lds, stream, gp, \
                       m, k);                                                                  \
  }
      if (nb == 1) {
        if (szv) AWQ_SKG2(true, 1) else AWQ_SKG2(false, 1)
      } else if (G == 128 || nb == 2) {
        if (szv) AWQ_SKG2(true, 2) else AWQ_SKG2(false, 2)
      } else {
        if constexpr (G != 128) {
          if (nb == 3) {
            if (szv) AWQ_SKG2(true, 3) else AWQ_SKG2(false, 3)
          } else {
            if (szv) AWQ_SKG2(true, 4) else AWQ_SKG2(false, 4)
          }
        }
      }
#undef AWQ_SKG2
      return hipGetLastError();
    }
  }
  // skinny 2 <= m <= 32: one fused kernel when its LDS plan fits (16-token
  // chunks: one for m <= 16, two above).  Above 16 tokens the fused kernel
  // reads every activation row once per 16-column block, which costs more than
  // a separate activation-prep launch per linear once the group holds more
  // than 16 MiB of packed weights (measured: q/k/v and o faster fused,
  // gate/up, down and the 70B-shaped linears faster staged).
  int64_t packed_bytes = 0;
  for (int l = 0; l < count; ++l) packed_bytes += items[l].n * k / 2;
  if (off32 && m >= 2 && (m <= 16 || (m <= 32 && packed_bytes <= kFusedMax))) {
    const int tcs = m <= 16 ? 1 : 2;
    const int64_t ng_all = k / G, nzw_all = (ng_all + 7) / 8;
    int nb_cap = kGemvMaxBlk;
    while (nb_cap > 0 && ((int64_t)nb_cap * 16 * nzw_all > (int64_t)kGemvSzRounds * kSk16Threads ||
                          skinny_fused_lds_bytes(k, G, nb_cap, tcs) > 160 * 1024))
      --nb_cap;
    if (nb_cap > 0) {
      int64_t per_cu = (int64_t)(160 * 1024) / (int64_t)skinny_fused_lds_bytes(k, G, nb_cap, tcs);
      per_cu = per_cu < 2 ? per_cu : 2;
      LinGroup gp = {};
      const int nb = split_group_grid(items, count, (int64_t)kGemvCUs * per_cu, nb_cap, gp);
      const size_t lds = skinny_fused_lds_bytes(k, G, nb, tcs);
      const bool szv = scales_octets(items, count, ng_all);
      if (scr.dry) return hipSuccess;               // the fused skinny kernels take no scratch
      const dim3 gd((unsigned)gp.wg0[count]), bd(kSk16Threads);
#define AWQ_SKF(TCC, SZ, PFF)                                                                  \
  {                                                                                            \
    const void* fn_ = reinterpret_cast<const void*>(&linear_skinny_fused_kernel<G, TCC, SZ, PFF>); \
    if (lds > 65536) {                                                                         \
      hipError_t e_ = hipFuncSetAttribute(fn_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); \
      if (e_ != hipSuccess) return e_;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((linear_skinny_fused_kernel<G, TCC, SZ, PFF>), gd, bd, lds, stream, gp,  \
                       m, k);                                                                  \
  }
#ifndef AWQ_SKINNY_GM_PF
#define AWQ_SKINNY_GM_PF 1
#endif
#define AWQ_SKG(SZ, NBB)                                                                       \
  {                                                                                            \
    const size_t lg_ = skinny_gm_lds_bytes(k, G, NBB);                                         \
    const void* fn_ = reinterpret_cast<const void*>(&linear_skinny_gm_kernel<G, SZ, NBB, AWQ_SKINNY_GM_PF>); \
    if (lg_ > 65536) {                                                                         \
      hipError_t e_ = hipFuncSetAttribute(fn_, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lg_); \
      if (e_ != hipSuccess) return e_;                                                         \
    }                                                                                          \
    hipLaunchKernelGGL((linear_skinny_gm_kernel<G, SZ, NBB, AWQ_SKINNY_GM_PF>), gd, bd, lg_, stream, gp, \
                       m, k);                                                                  \
  }
      // several blocks per work-group: group-major (the same sums in the same
      // order, so the same bits as the block-major kernel)
      if (tcs == 1 && nb >= 2) {
        if (nb == 2) {
          if (szv) AWQ_SKG(true, 2) else AWQ_SKG(false, 2)
        } else if (nb == 3) {
          if (szv) AWQ_SKG(true, 3) else AWQ_SKG(false, 3)
        } else {
          if (szv) AWQ_SKG(true, 4) else AWQ_SKG(false, 4)
        }
      } else if (tcs == 1) {
        if (szv) AWQ_SKF(1, true, 2) else AWQ_SKF(1, false, 2)
      } else {
        if (szv) AWQ_SKF(2, true, 1) else AWQ_SKF(2, false, 1)
      }
#undef AWQ_SKF
#undef AWQ_SKG
      return hipGetLastError();
    }
  }
  // 17 <= m <= 32: linears of more than 16 MiB of packed weights that do not
  // take the fused kernel run as one grouped GEMM launch (64-row tiles, split
  // along K), which streams their weights faster than the staged skinny pair
  // (measured at 32 tokens: gate/up 67 -> 37 us, down 34 -> 30 us, 70B-shaped
  // gate/up 93 -> 62 us, down 97 -> 80 us); the others as calls alone
  if (m > 16 && m <= 32) {
    LinItem wide[kGroupMax], rest[kGroupMax];
    int nw = 0, nr = 0;
    for (int l = 0; l < count; ++l) {
      if (skinny_wide(items[l], m, k)) wide[nw++] = items[l];
      else rest[nr++] = items[l];
    }
    if (nw > 0) {
      hipError_t e = launch_gemm_group<G>(wide, nw, m, k, scr, stream);
      if (e != hipSuccess) return e;
      for (int l = 0; l < nr; ++l) {
        e = launch_linear_group_g<G>(rest + l, 1, m, k, scr, stream);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  // every other case: one linear after another on the stream, each planned as
  // a call of it alone (the staged kernels share the scratch buffer, in
  // stream order)
  if (count == 1) return launch_linear_one<G>(items[0], m, k, scr, stream);
  for (int l = 0; l < count; ++l) {
    hipError_t e = launch_linear_group_g<G>(items + l, 1, m, k, scr, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_linear_group(const LinItem* items, int count, int64_t m, int64_t k, int32_t g,
                               Scratch& scr, hipStream_t stream) {
  switch (g) {
    case 32:
      return launch_linear_group_g<32>(items, count, m, k, scr, stream);
    case 64:
      return launch_linear_group_g<64>(items, count, m, k, scr, stream);
    default:
      return launch_linear_group_g<128>(items, count, m, k, scr, stream);
  }
}

size_t linear_group_scratch_bytes(const LinItem* items, int count, int64_t m, int64_t k, int32_t g) {
  Scratch scr;
  scr.dry = true;
  (void)launch_linear_group(items, count, m, k, g, scr, nullptr);
  return scr.need;
}

}  // namespace awq
