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

namespace awq {

constexpr int kSkinnyTok = 8;          // tokens per 16-row A chunk (hi + lo rows)
constexpr int kSkinnyWaves = 8;        // waves per work-group

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t linear_scratch_bytes(int64_t m, int64_t k, int32_t g) {
  if (m > 32) return align256((size_t)m * (size_t)k * 2);     // scaled, permuted activations
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
          if (t < m) y[t * n + col] = f2h_rn(s[i] + o[i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- decode GEMV (m = 1)
// Persistent work-groups of 8 waves.  A work-group stages x_tilde once in LDS
// as the two live rows of the MFMA A operand (row 0 = fp16 hi, row 8 = fp16
// lo; the other 14 rows read a zero block) together with the per-group offset
// sums T and U, then walks its 16-column blocks (block b, b + grid, ...).
// Every wave owns a fixed contiguous range of groups along K; it walks the
// flattened sequence (block, group) with a double-buffered prefetch of packed
// weights that runs across block boundaries.  The per-group scales and zero
// points of a block are staged in LDS one block ahead with 16-byte loads (one
// per 8 groups of a column), as packed words (fp16 scale | zero << 16) laid
// out [group][column]: scattered 2- and 4-byte loads of them would cost as
// many memory requests as the weights themselves.  At the end of a block the
// waves meet at one barrier; a designated wave sums the 8 partial rows in a
// fixed order and stores 16 outputs while the others go on.
#ifndef AWQ_GEMV_PF
#define AWQ_GEMV_PF 4
#endif
#ifndef AWQ_GEMV_WG_PER_CU
#define AWQ_GEMV_WG_PER_CU 2
#endif
constexpr int kGemvWaves = 8;
constexpr int kGemvPF = AWQ_GEMV_PF;
constexpr int kGemvCUs = 256;

// LDS: x_tilde [ng][4][2][g/4] halves, T/U [ng] float4, zero block, scale|zero
// words [2][ng][16], reduction rows [2][8][16] floats.
size_t gemv_lds_bytes(int64_t k, int32_t g) {
  const size_t ng = (size_t)(k / g);
  return (size_t)k * 4 + ng * 16 + (size_t)(g / 4) * 2 + 2 * ng * 16 * 4 + 2 * kGemvWaves * 16 * 4;
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

template <int G>
__global__ __launch_bounds__(kGemvWaves * 64, AWQ_GEMV_WG_PER_CU) void linear_gemv_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ inv_s,
    const uint32_t* __restrict__ qweight, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, int64_t n, int64_t k, uint16_t* __restrict__ y) {
  constexpr int WPL = G / 32;            // qweight words per lane per group
  constexpr int HPL = G / 4;             // staged halves per (group, lane group, row)
  constexpr int LPG = G / 8;             // words per group
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ng = (int)(k / G);
  unsigned char* sp = smem;
  uint16_t* xa = reinterpret_cast<uint16_t*>(sp);          sp += (size_t)k * 4;     // [ng][4][2][HPL]
  float4* tu = reinterpret_cast<float4*>(sp);              sp += (size_t)ng * 16;   // (T_hi, U_hi, T_lo, U_lo)
  uint16_t* zblk = reinterpret_cast<uint16_t*>(sp);        sp += HPL * 2;           // zeros
  uint32_t* szw = reinterpret_cast<uint32_t*>(sp);         sp += (size_t)2 * ng * 16 * 4;  // [2][ng][16]
  float* red = reinterpret_cast<float*>(sp);                                         // [2][8][16]

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across the wave: keep it (and every group index
  // and group base address derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane >> 4, r = lane & 15;
  const int nblk = (int)((n + 15) / 16);
  const int grid = (int)gridDim.x;
  const int my_blocks = (nblk - (int)blockIdx.x + grid - 1) / grid;   // >= 1
  const int jb = ng * wave / kGemvWaves, je = ng * (wave + 1) / kGemvWaves;
  const int cnt = je - jb;                            // groups of this wave per block
  const int total = my_blocks * cnt;                  // (block, group) items of this wave
  const int nzw = (ng + 7) / 8, kw_row = (int)(k / 8);

  // ---- scale / zero staging: thread t < 16 * nzw owns (column t / nzw, octet t % nzw)
  const bool sz_thread = tid < 16 * nzw;
  const int sz_row = sz_thread ? tid / nzw : 0;
  const int sz_oct = sz_thread ? tid % nzw : 0;
  const bool sz_vec = (ng % 8) == 0;                  // 16-byte aligned octets
  auto sz_load = [&](int blk, uint4& ss, uint32_t& zz) {   // registers <- global, block blk
    blk = blk < nblk ? blk : nblk - 1;
    int col = blk * 16 + sz_row;
    col = col < (int)n ? col : (int)n - 1;
    if (sz_thread) {
      const uint16_t* srow = scales + (int64_t)col * ng + sz_oct * 8;
      if (sz_vec) {
        ss = *reinterpret_cast<const uint4*>(srow);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (sz_oct * 8 + i < ng) ? srow[i] : (uint16_t)0;
        ss = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                        h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
      }
      zz = qzeros[(int64_t)col * nzw + sz_oct];
    }
  };
  uint4 sz_s = make_uint4(0, 0, 0, 0);                // block staged at the next block end
  uint32_t sz_z = 0;
  auto sz_store_regs = [&](int buf, const uint4& ss, uint32_t zz) {   // LDS <- registers
    if (sz_thread) {
      const uint32_t sw[4] = {ss.x, ss.y, ss.z, ss.w};
      const uint32_t sz_zv = zz;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int j = sz_oct * 8 + i;
        if (j < ng)
          szw[((size_t)buf * ng + j) * 16 + sz_row] =
              ((sw[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu) | (((sz_zv >> (4 * i)) & 0xFu) << 16);
      }
    }
  };

  // Prefetch slots hold raw loaded bits only (converting at issue time would
  // make the wave wait there: memory counters retire in order), and every
  // load is unconditional (the cursor stops on the last item, the column is
  // clamped), so no branch separates a load from its use and the waits stay
  // precise.  The (block, group) cursors advance incrementally in scalar
  // registers: no division per item.
  uint32_t wq[2 * kGemvPF][WPL];
  const char* qbase = reinterpret_cast<const char*>(qweight);
  int i_blk = (int)blockIdx.x, i_j = jb, i_left = total;    // issue cursor
  auto issue = [&](int slot) {
    int col = i_blk * 16 + r;
    col = col < (int)n ? col : (int)n - 1;
    // 32-bit per-lane byte offset (the packed tensors of one call are below 4 GiB)
    const uint32_t qoff = ((uint32_t)col * (uint32_t)kw_row + (uint32_t)(WPL * c)) * 4u;
    load_words<WPL>(reinterpret_cast<const uint32_t*>(qbase + (int64_t)i_j * (LPG * 4) + qoff), wq[slot]);
    if (i_left > 1) {
      --i_left;
      if (++i_j == je) { i_j = jb; i_blk += grid; }
    }
  };
  const bool active = cnt > 0;                        // wave-uniform
  if (active) {
#pragma unroll
    for (int p = 0; p < kGemvPF; ++p) issue(p);
  }
  // every prologue load is issued before anything waits on one (memory
  // counters retire in order): weights, the scales of blocks 0 and 1, then x
  uint4 sz_s0 = make_uint4(0, 0, 0, 0);
  uint32_t sz_z0 = 0;
  sz_load((int)blockIdx.x, sz_s0, sz_z0);             // block 0 of this work-group
  sz_load((int)blockIdx.x + grid, sz_s, sz_z);        // block 1, stored at the first block end

  // ---- stage x_tilde (hi, lo) and the offset sums in LDS
  if (tid < HPL / 2) reinterpret_cast<uint32_t*>(zblk)[tid] = 0u;
  const bool has_inv = inv_s != nullptr;
  for (int wi = tid; wi < kw_row; wi += kGemvWaves * 64) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + (int64_t)wi * 8);
    uint4 sv = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    if (has_inv) sv = *reinterpret_cast<const uint4*>(inv_s + (int64_t)wi * 8);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
    uint16_t hi[8], lo[8];
    float th = 0.f, uh = 0.f, tl = 0.f, ul = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xt = h2f((uint16_t)(xw[e >> 1] >> ((e & 1) * 16))) *
                       h2f((uint16_t)(sw[e >> 1] >> ((e & 1) * 16)));     // exact
      hi[e] = f2h_rn(xt);
      lo[e] = f2h_rn(xt - h2f(hi[e]));
      const float off = (e & 1) ? 64.0f : 1024.0f;
      th += off * h2f(hi[e]);
      uh += h2f(hi[e]);
      tl += off * h2f(lo[e]);
      ul += h2f(lo[e]);
    }
    const int j = wi / LPG;
    const int wg = wi % LPG;
    const int cc = wg / WPL, i = wg % WPL;
    uint16_t* dh = xa + ((j * 4 + cc) * 2 + 0) * HPL + i * 8;
    uint16_t* dl = xa + ((j * 4 + cc) * 2 + 1) * HPL + i * 8;
    // slot order (k0, k4, k1, k5, k2, k6, k3, k7) matches unpack_word
    uint4 vh, vl;
    vh.x = hi[0] | ((uint32_t)hi[4] << 16); vh.y = hi[1] | ((uint32_t)hi[5] << 16);
    vh.z = hi[2] | ((uint32_t)hi[6] << 16); vh.w = hi[3] | ((uint32_t)hi[7] << 16);
    vl.x = lo[0] | ((uint32_t)lo[4] << 16); vl.y = lo[1] | ((uint32_t)lo[5] << 16);
    vl.z = lo[2] | ((uint32_t)lo[6] << 16); vl.w = lo[3] | ((uint32_t)lo[7] << 16);
    *reinterpret_cast<uint4*>(dh) = vh;
    *reinterpret_cast<uint4*>(dl) = vl;
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) {
      th += shfl_xor_f(th, off); uh += shfl_xor_f(uh, off);
      tl += shfl_xor_f(tl, off); ul += shfl_xor_f(ul, off);
    }
    if (wg == 0) tu[j] = make_float4(th, uh, tl, ul);
  }
  sz_store_regs(0, sz_s0, sz_z0);
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

  // end of a column block: stage the scales of the block after next, combine
  // hi + lo rows, meet the other waves, reduce
  auto finish_block = [&](int blk) {
    sz_store_regs((blocks_done + 1) & 1, sz_s, sz_z);
    const float other = __shfl_xor(yacc, 32, 64);
    float* rb = red + (blocks_done & 1) * (kGemvWaves * 16);
    if (lane < 16) rb[wave * 16 + lane] = yacc + other;
    yacc = 0.0f;
    __syncthreads();
    if (wave == reducer && lane < 16) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kGemvWaves; ++wv) sum += rb[wv * 16 + lane];
      const int64_t col = (int64_t)blk * 16 + lane;
      if (col < n) y[col] = f2h_rn(sum);
    }
    ++blocks_done;
    sz_load(blk + 2 * grid, sz_s, sz_z);
  };
  int c_blk = (int)blockIdx.x, c_j = jb, c_left = total;    // consume cursor
  auto consume = [&](int p) {
    if (c_left > 0) {                                 // wave-uniform
      const int j = c_j;
      const char* asrc = a_base + a_lane + (uint32_t)j * a_step;
      half8_t aop[WPL];
#pragma unroll
      for (int i = 0; i < WPL; ++i) aop[i] = *reinterpret_cast<const half8_t*>(asrc + 16 * i);
      const float2 tv = *reinterpret_cast<const float2*>(tu_lane + (uint32_t)j * 16);
      const uint32_t szv = szw[((blocks_done & 1) * ng + j) * 16 + r];
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
        finish_block(c_blk);
        c_j = jb;
        c_blk += grid;
      }
    }
  };
  if (active) {
    for (int s0 = 0; s0 < total; s0 += 2 * kGemvPF) {
#pragma unroll
      for (int p = 0; p < kGemvPF; ++p) issue(kGemvPF + p);
#pragma unroll
      for (int p = 0; p < kGemvPF; ++p) consume(p);
#pragma unroll
      for (int p = 0; p < kGemvPF; ++p) issue(p);
#pragma unroll
      for (int p = 0; p < kGemvPF; ++p) consume(kGemvPF + p);
    }
  } else {
    // a wave without groups (fewer than 8 groups in k) still meets every block's barrier
    for (int bi = 0; bi < my_blocks; ++bi) finish_block((int)blockIdx.x + bi * grid);
  }
}

// ---------------------------------------------------------------- prefill GEMM
// Work-group tile 256 tokens x 128 output columns, K-step 64, 4 waves in a
// 2 x 2 arrangement, each wave 128 x 64 = 4 x 2 blocks of
// v_mfma_f32_32x32x16_f16 (fp32 accumulators).
//  * A (activations): linear_xprep first writes x_tilde = fp16(x * inv_s)
//    once per call, every 8-channel chunk permuted into the nibble-unpack
//    slot order.  Each K-step the work-group copies its 256 x 64 tile straight
//    from global memory into one of two LDS stages (global_load_lds, 16 bytes
//    per lane; 16-byte chunks XOR-swizzled by row, so the 16 lanes served per
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
constexpr int kGemmBM = 256, kGemmBN = 128, kGemmBK = 64;
#ifndef AWQ_GEMM_SWZ_SHIFT
#define AWQ_GEMM_SWZ_SHIFT 1
#endif

__device__ __forceinline__ uint32_t perm_bytes(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// x_tilde = fp16_rn(x * inv_s), every 8-channel chunk permuted into the
// nibble-unpack slot order (k0,k4) (k1,k5) (k2,k6) (k3,k7); one pass over the
// activations per call, so the GEMM's activation staging is a plain copy.
__global__ __launch_bounds__(256) void linear_xprep_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ inv_s,
                                                           int64_t m, int64_t k,
                                                           uint16_t* __restrict__ xt) {
  const int64_t chunks = m * (k / 8);
  const bool has_inv = inv_s != nullptr;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * 256) {
    const int64_t kk = (c % (k / 8)) * 8;
    const uint4 xv = *reinterpret_cast<const uint4*>(x + c * 8);
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

// dynamic LDS of the GEMM (the two activation stages are static: 64 KiB)
size_t gemm_lds_bytes(int64_t k, int32_t g) {
  const size_t ng = (size_t)(k / g), nzw = (ng + 7) / 8;
  const size_t s_bytes = ((size_t)kGemmBN * ng * 2 + 15) & ~(size_t)15;
  return s_bytes + (size_t)kGemmBN * nzw * 4;
}

template <int G>
__global__ __launch_bounds__(256, 2) void linear_gemm_kernel(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint32_t* __restrict__ qzeros,
    int64_t m, int64_t n, int64_t k, uint16_t* __restrict__ y, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // two distinct stage objects: the compiler can see that the copies into one
  // stage never alias the fragment reads of the other, so it does not wait for
  // the copies before reading
  __shared__ __attribute__((aligned(16))) uint16_t a_st0[kGemmBM * kGemmBK];
  __shared__ __attribute__((aligned(16))) uint16_t a_st1[kGemmBM * kGemmBK];
  const int ng = (int)(k / G), nzw = (ng + 7) / 8;
  uint16_t* s_l = reinterpret_cast<uint16_t*>(smem);                          // [128][ng]
  const size_t s_bytes = ((size_t)kGemmBN * ng * 2 + 15) & ~(size_t)15;
  uint32_t* z_l = reinterpret_cast<uint32_t*>(smem + s_bytes);                // [128][nzw]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // XCD-aware tile order: each XCD gets a contiguous range of tiles, M fastest,
  // so the work-groups that share a weight tile share that XCD's L2
  const int total = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, slot = bid / 8;
  const int tile = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int64_t m0 = (int64_t)tm * kGemmBM, n0 = (int64_t)tn * kGemmBN;
  const int64_t kw_row = k / 8;
  const int nk = (int)(k / kGemmBK);

  // ---- scales and zero words of this tile's columns (rows of W)
  for (int i = tid; i < kGemmBN * ng; i += 256) {
    const int r = i / ng, gg = i % ng;
    int64_t col = n0 + r;
    col = col < n ? col : n - 1;
    s_l[i] = scales[col * ng + gg];
  }
  for (int i = tid; i < kGemmBN * nzw; i += 256) {
    const int r = i / nzw, w = i % nzw;
    int64_t col = n0 + r;
    col = col < n ? col : n - 1;
    z_l[i] = qzeros[col * nzw + w];
  }

  // ---- A loader: direct global -> LDS copies (global_load_lds_dwordx4).  One
  // wave instruction fills 64 consecutive 16-byte LDS slots (8 rows x 8
  // chunks); lane i writes slot i, so the XOR swizzle of the chunk position is
  // applied on the global side: lane (row r, slot p) fetches logical chunk
  // p ^ ((r >> S) & 7).  Wave w fills rows 64 w .. 64 w + 63 of the stage.
  // The activations arrive already scaled and slot-permuted (linear_xprep).
  typedef __attribute__((address_space(3))) void lds_void_t;
  const int a_lr = lane >> 3, a_p = lane & 7;
  const uint16_t* a_src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lrow = wave * 64 + 8 * i + a_lr;
    int64_t row = m0 + lrow;
    row = row < m ? row : m - 1;
    a_src[i] = x + row * k + (a_p ^ ((lrow >> AWQ_GEMM_SWZ_SHIFT) & 7)) * 8;
  }
#define AWQ_GEMM_LOAD_A(KT, STAGE_PTR)                                                  \
  {                                                                                     \
    const int64_t kk_ = (int64_t)(KT) * kGemmBK;                                        \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                       \
      __builtin_amdgcn_global_load_lds(                                                 \
          (const void*)(a_src[i] + kk_),                                                \
          (lds_void_t*)((STAGE_PTR) + (wave * 64 + 8 * i) * 64), 16, 0, 0);             \
  }

  // ---- B loader: lane (j = lane % 32, c = lane / 32) of block bn loads words 4c..4c+3
  const int bj = lane & 31, bc = lane >> 5;
  const uint32_t* b_src[2];
#pragma unroll
  for (int bn = 0; bn < 2; ++bn) {
    int64_t col = n0 + wn * 64 + bn * 32 + bj;
    col = col < n ? col : n - 1;
    b_src[bn] = qweight + col * kw_row + 4 * bc;
  }
  uint4 wb0, wb1;
#define AWQ_GEMM_LOAD_B(KT)                                                        \
  {                                                                                \
    wb0 = *reinterpret_cast<const uint4*>(b_src[0] + (int64_t)(KT) * 8);           \
    wb1 = *reinterpret_cast<const uint4*>(b_src[1] + (int64_t)(KT) * 8);           \
  }

  floatx16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = floatx16_t{};

  AWQ_GEMM_LOAD_A(0, a_st0);
  AWQ_GEMM_LOAD_B(0);
  __builtin_amdgcn_s_waitcnt(0);       // the direct-to-LDS copies have landed
  __syncthreads();
  const UnpackConsts uc = unpack_consts();
  const int a_row_base = wm * 128 + (lane & 31);

  // One K-step: copy the next step's activations into the other stage and
  // load its weights, dequantize this step's weights, 32 MFMAs, then wait for
  // the copies and meet at the barrier.
#define AWQ_GEMM_STEP(KT, CUR, NXT)                                                     \
  {                                                                                     \
    const uint4 wc0 = wb0, wc1 = wb1;                                                   \
    const int ktn_ = (KT) + 1 < nk ? (KT) + 1 : (KT);                                  \
    AWQ_GEMM_LOAD_A(ktn_, NXT);                                                         \
    AWQ_GEMM_LOAD_B(ktn_);                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    half8_t bq[2][4];                                                                   \
    const int grp = ((KT) * kGemmBK + 32 * bc) / G;                                     \
    _Pragma("unroll") for (int bn = 0; bn < 2; ++bn) {                                  \
      const int r = wn * 64 + bn * 32 + bj;                                             \
      const float d = h2f(s_l[r * ng + grp]);                                           \
      const float z = (float)((z_l[r * nzw + (grp >> 3)] >> (4 * (grp & 7))) & 0xFu);   \
      const half2_t dd = {(half_t)d, (half_t)d};                                        \
      const half2_t o1024 = {(half_t)(-1024.0f - z), (half_t)(-1024.0f - z)};          \
      const half2_t o64 = {(half_t)(-64.0f - z), (half_t)(-64.0f - z)};                 \
      const uint4 wv = bn == 0 ? wc0 : wc1;                                             \
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};                                  \
      _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                   \
        uint32_t u[4];                                                                  \
        unpack_word(ww[s], u, uc);                                                      \
        const half2_t q0 = (__builtin_bit_cast(half2_t, u[0]) + o1024) * dd;            \
        const half2_t q1 = (__builtin_bit_cast(half2_t, u[1]) + o64) * dd;              \
        const half2_t q2 = (__builtin_bit_cast(half2_t, u[2]) + o1024) * dd;            \
        const half2_t q3 = (__builtin_bit_cast(half2_t, u[3]) + o64) * dd;              \
        bq[bn][s] = __builtin_bit_cast(                                                 \
            half8_t, make_uint4(__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1), \
                                __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3))); \
      }                                                                                 \
    }                                                                                   \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                     \
      const int ch = 4 * bc + s;                                                        \
      _Pragma("unroll") for (int bm = 0; bm < 4; ++bm) {                                \
        const int row = a_row_base + bm * 32;                                           \
        const half8_t av = *reinterpret_cast<const half8_t*>(                           \
            (CUR) + ((size_t)row * 8 + (ch ^ ((row >> AWQ_GEMM_SWZ_SHIFT) & 7))) * 8);  \
        _Pragma("unroll") for (int bn = 0; bn < 2; ++bn)                                \
          acc[bm][bn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bq[bn][s], acc[bm][bn], 0, 0, 0); \
      }                                                                                 \
    }                                                                                   \
    __builtin_amdgcn_s_waitcnt(0);                                                      \
    __syncthreads();                                                                    \
  }
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    AWQ_GEMM_STEP(kt, a_st0, a_st1);
    AWQ_GEMM_STEP(kt + 1, a_st1, a_st0);
  }
  if (kt < nk) AWQ_GEMM_STEP(kt, a_st0, a_st1);
#undef AWQ_GEMM_STEP
#undef AWQ_GEMM_LOAD_A
#undef AWQ_GEMM_LOAD_B

  // ---- epilogue: value e of lane l in block (bm, bn) is row 8(e/4) + 4(l/32) + e%4, column l%32
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 2; ++bn)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = m0 + wm * 128 + bm * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int64_t cidx = n0 + wn * 64 + bn * 32 + (lane & 31);
        if (t < m && cidx < n) y[t * n + cidx] = f2h_rn(acc[bm][bn][e]);
      }
}

template <int G>
static hipError_t launch_linear_g(const uint16_t* x, const uint32_t* qweight,
                                  const uint16_t* scales, const uint32_t* qzeros,
                                  const uint16_t* inv_s16, int64_t m, int64_t n, int64_t k,
                                  uint16_t* y, void* scratch, hipStream_t stream) {
  if (m > 32) {
    const size_t lds = gemm_lds_bytes(k, G);
    const size_t lds_static = (size_t)2 * kGemmBM * kGemmBK * 2;
    if (lds + lds_static > 160 * 1024) return hipErrorInvalidValue;
    if (lds + lds_static > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&linear_gemm_kernel<G>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    uint16_t* xt = static_cast<uint16_t*>(scratch);
    const int64_t chunks = m * (k / 8);
    const int64_t pgrid = (chunks + 255) / 256 < 4096 ? (chunks + 255) / 256 : 4096;
    hipLaunchKernelGGL(linear_xprep_kernel, dim3((unsigned)pgrid), dim3(256), 0, stream, x, inv_s16,
                       m, k, xt);
    const int tiles_m = (int)((m + kGemmBM - 1) / kGemmBM);
    const int tiles_n = (int)((n + kGemmBN - 1) / kGemmBN);
    hipLaunchKernelGGL(linear_gemm_kernel<G>, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), lds,
                       stream, xt, qweight, scales, qzeros, m, n, k, y, tiles_m, tiles_n);
    return hipGetLastError();
  }
  // the fused decode kernel needs its LDS plan to fit (160 KiB) and one
  // scale/zero octet per thread (16 columns x ceil(ng/8) octets <= 512);
  // other shapes take the staged two-kernel path below
  const int64_t ng_all = k / G;
  if (m == 1 && gemv_lds_bytes(k, G) <= 160 * 1024 && 16 * ((ng_all + 7) / 8) <= kGemvWaves * 64) {
    const size_t lds = gemv_lds_bytes(k, G);
    const void* fn = reinterpret_cast<const void*>(&linear_gemv_kernel<G>);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    const int64_t nblk = (n + 15) / 16;
    // work-groups resident at once: bounded by the launch bound and by LDS
    int64_t per_cu = (int64_t)(160 * 1024) / (int64_t)lds;
    per_cu = per_cu < AWQ_GEMV_WG_PER_CU ? per_cu : AWQ_GEMV_WG_PER_CU;
    per_cu = per_cu > 0 ? per_cu : 1;
    const int64_t slots = (int64_t)kGemvCUs * per_cu;
    // as many work-groups as fit at once; blocks go round-robin
    const int64_t grid = nblk < slots ? nblk : slots;
    hipLaunchKernelGGL((linear_gemv_kernel<G>), dim3((unsigned)grid), dim3(kGemvWaves * 64), lds,
                       stream, x, inv_s16, qweight, scales, qzeros, n, k, y);
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
