// Grid search of the AWQ channel scale s = a^alpha (jsqmd.com page, section
// 二.1 (3): scale the salient input channels of W by s, divide the activation
// by s, choose s to minimise the output error of the quantized layer).
//
// Four kernels, all on the caller's stream:
//  1. search_prep: s_ik = fp16_rn(max(a_k^alpha_i, 2^-14)) and 1/s_ik (fp32)
//     for every grid point and channel (float64 pow, single fp16 rounding).
//  2. search_blockmax: the largest finite |W| of every 64-row block, from
//     which the loss kernel takes a power-of-two factor that keeps the fp16
//     split of the weight error in the normal range (see below).
//  3. search_loss: one work-group per (64-row block, alpha).  For every group
//     of g channels it fake-quantizes the 64 x g block of W' = fp16(W s_i)
//     (exact per-element codes, see awq_common.h), forms the weight error
//     dW = ((q - z) D - W s) / s in fp32 (no cancellation: both terms of the
//     difference are exact), splits it into fp16 hi + lo, stages both in LDS
//     in the MFMA A-operand layout and multiplies them with the calibration
//     tokens (B operand, copied into LDS three steps ahead) into fp32
//     accumulators E = dW X^T.  After the last group it squares E in float64
//     and writes the block's partial loss.
//  4. search_select: sums the partials of each alpha in block order (fixed),
//     takes the first minimum over finite losses and writes s16 and
//     inv_s16 = fp16_rn(1/s16) (float64 quotient).
// A non-finite W' (W s overflowing fp16, or a NaN scale) makes its group's
// step D non-finite or its own error NaN; either reaches E through the MFMAs,
// so that alpha's loss is not finite and it is never chosen.
#include <math.h>

#include "awq_common.h"
#include "awq_internal.h"

namespace awq {

constexpr int kSearchRows = 64;        // rows of W per work-group

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
                                                          float* __restrict__ rs,
                                                          uint32_t* __restrict__ bmax,
                                                          int64_t n_blocks) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y;
  if (i == 0)   // the block maxima of |W| start from zero (filled by search_blockmax)
    for (int64_t b = col; b < n_blocks; b += (int64_t)gridDim.x * 256) bmax[b] = 0u;
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

// Per 64-row block: a power-of-two factor c for the weight error dW.  Every
// |dW_nk| is at most about 1.03 |W_nk| (an element on quantization level 0 has
// dW = -W; on any other level |W'| >= D/2, so |deq - W'| <= 0.51 D <= 1.02 |W'|).
// With max|W| < 2^e the factor c = 2^(14 - e) keeps c |dW| below 17000, inside
// fp16, while lifting small errors far above the fp16 subnormal range, so the
// fp16 hi + lo split of c dW keeps about 22 significant bits.
//
// search_blockmax: work-group (block, 512-column chunk) folds the finite |W|
// of its 64 x 512 tile into the block maximum with an integer atomic max on
// the fp16 bit patterns (|fp16| bits order like the values; max is
// order-independent, so the result is deterministic).
constexpr int kBlockMaxCols = 512;
__global__ __launch_bounds__(256) void search_blockmax_kernel(const uint16_t* __restrict__ w,
                                                              int64_t n, int64_t k,
                                                              uint32_t* __restrict__ bmax) {
  __shared__ uint32_t red[4];
  const int64_t rb = blockIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * kBlockMaxCols;
  const int64_t r0 = rb * kSearchRows;
  const int64_t rows = (n - r0) < kSearchRows ? (n - r0) : kSearchRows;
  const int64_t cols = (k - c0) < kBlockMaxCols ? (k - c0) : kBlockMaxCols;   // multiple of 8
  const int64_t cw = cols / 8;
  uint32_t mx = 0;
  for (int64_t i = threadIdx.x; i < rows * cw; i += 256) {
    const int64_t rr = i / cw, cc = i % cw;
    const uint4 v = *reinterpret_cast<const uint4*>(w + (r0 + rr) * k + c0 + cc * 8);
    const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const uint32_t bits = (ww[h >> 1] >> ((h & 1) * 16)) & 0x7FFFu;
      if (bits < 0x7C00u && bits > mx) mx = bits;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(mx, off, 64);
    mx = o > mx ? o : mx;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int i = 1; i < 4; ++i) m = red[i] > m ? red[i] : m;
    if (m != 0) atomicMax(&bmax[rb], m);
  }
}

// c = 2^(14 - e) for a block whose largest finite |W| (fp16 bits m) is below 2^e
__device__ __forceinline__ float block_factor(uint32_t m) {
  if (m == 0) return 1.0f;
  int e;
  (void)__builtin_frexpf(h2f((uint16_t)m), &e);
  return __builtin_ldexpf(1.0f, 14 - e);
}

// One 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane i
// writes LDS bytes lds_base + 16 i .. +15.  Issued from inline asm so that the
// compiler, which would otherwise drain every outstanding copy before any read
// of the destination array, leaves the waits to the caller: the destination
// must not be read before an explicit s_waitcnt vmcnt that covers the copy,
// and every copy must have landed before the wave ends.  No output register.
// M0 is reserved for the compiler, which uses it only to address LDS copies
// of its own; none is live across this statement in the kernels below.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* gsrc, uint32_t lds_base) {
  // one wait state between the M0 write and the copy that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt on the vector memory counter only, as inline asm: the compiler
// does not see the copies above and would drop a wait it thinks is idle.  The
// memory clobber keeps the LDS reads that follow below it.
// The producer's per-element arithmetic in the fewest instructions, each
// result bit-identical to the plain float form:
//  * the code of an fp16 w' takes w' straight into the quotient's fmas
//    (v_fma_mix_f32 reads fp16 operands), as rne_quot and code_minus_zero do
//    with a float w' (the two differ at most in the sign of a zero t1, which
//    the following fmas turn into the same +0);
//  * dw - hi for the fp16 hi half of a packed pair is one v_fma_mix_f32
//    (-hi * 1 + dw, one rounding of the exact difference, as dw - (float)hi).
__device__ __forceinline__ float code_minus_zero_h(half_t w, const GroupQ& gq) {
  const float t1 = __builtin_fmaf((float)w, gq.rd, 0.0f);
  const float r = __builtin_fmaf(-t1, gq.d, (float)w);
  const float t = __builtin_rintf(__builtin_fmaf(r, gq.rd, t1));
  return __builtin_fminf(__builtin_fmaxf(t, -gq.z), gq.qmax - gq.z);
}
__device__ __forceinline__ float sub_f16_lo(float dw, half2_t h) {
  float o;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(o) : "v"(h), "v"(dw));
  return o;
}
__device__ __forceinline__ float sub_f16_hi(float dw, half2_t h) {
  float o;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(o) : "v"(h), "v"(dw));
  return o;
}

#define AWQ_WAIT_VMCNT(N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory")

// Lane moves inside aligned groups of 4 lanes (DPP quad permutes).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Work-group: 64 rows of W (two 32-row MFMA blocks) x one alpha x all tokens
// in passes of 128 NT, as 4 + NP waves in two roles that run concurrently on
// each SIMD, one group of g channels apart:
//  * producer waves 4 .. 3 + NP (stage 1): thread (row t / NP, part t % NP)
//    fake-quantizes g / NP elements of group i (eight producers where the
//    tokens are few and quantizing a group would outlast its MFMAs): W' =
//    fp16(W s) two at a time (v_pk_mul_f16), the group max/min two at a time
//    and across the row's lanes (DPP), then per element the exact code,
//    deq = (q - z) D, the scaled error
//    dW c = (deq - W s)(c/s) and its fp16 split hi = rtz(dW c),
//    lo = rtz(dW c - hi) (v_cvt_pkrtz, two at a time), stored in LDS buffer
//    i % 2 in the MFMA A layout with 16-byte stores.  The next group's
//    weights, scales and scaled reciprocals load meanwhile.
//  * consumer waves 0..3 (stage 2): E += dW_hi X^T + dW_lo X^T for group
//    i - 1 from the other buffer; wave w owns the token tiles w, w + 4, ... of
//    the pass and both row blocks, so each activation fragment feeds four
//    MFMAs.  A wave copies its own activation fragments straight into a
//    private 4-slot LDS ring (global_load_lds, 16 bytes per lane, read back
//    by the same lane), three 16-channel steps ahead of the MFMAs.
//  * dW sits in LDS as [step][k half][row][8 halves]: the 32 lanes that read
//    one k half of an A fragment read 512 contiguous bytes (no bank
//    conflicts).
// One barrier per group separates the roles.  Every load is unconditional
// (indices clamped), so the waits stay exact.  After the last group of a pass
// the consumers square E in float64 over the valid tokens; fixed-order
// reductions give one partial loss per (alpha, block).
template <int G, int NT, int NP>
__global__ __launch_bounds__(64 * (4 + NP), 1) void search_loss_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ x, int64_t n, int64_t k,
    int64_t m, int32_t n_grid, int64_t n_blocks, const uint16_t* __restrict__ s16_all,
    const float* __restrict__ rs_all, const uint32_t* __restrict__ bmax, double* __restrict__ part,
    float qmax) {
  static_assert((NP == 4 || NP == 8) && G / NP >= 8, "four or eight producer waves");
  constexpr int NC = 4;               // consumer waves
  constexpr int EPT = G / NP;         // elements of one row-group per producer thread
  constexpr int KSTEPS = G / 16;      // MFMA k-steps per group (even)
  constexpr int TOK = 32 * NC * NT;   // tokens per pass
  constexpr int WLD = EPT / 8;        // 16-byte weight loads per producer thread per group
  // LDS padding, so that the 8 lanes an LDS cycle serves hit distinct banks:
  // a producer's 16-byte dW stores (lanes: 2 rows x 4 quarters, or 1 row x 8
  // eighths) shift by 32 (16) bytes per part of the group; its scale reads
  // (the parts, the rows broadcast) by 16 bytes per part, its reciprocal
  // reads likewise
  constexpr int CPQ = EPT / 8;                     // 8-channel chunks per part
  constexpr int PADS = NP == 4 ? 16 : 8;           // dW pad (halves) per part of the group
  constexpr int DWN = KSTEPS * kSearchRows * 16 + (NP - 1) * PADS;   // halves per dW buffer
  __shared__ __attribute__((aligned(16))) uint16_t dh0[DWN];
  __shared__ __attribute__((aligned(16))) uint16_t dl0[DWN];
  __shared__ __attribute__((aligned(16))) uint16_t dh1[DWN];
  __shared__ __attribute__((aligned(16))) uint16_t dl1[DWN];
  __shared__ __attribute__((aligned(16))) uint16_t s_l[2][G + (NP - 1) * 8];   // candidate scales
  __shared__ __attribute__((aligned(16))) float rc_l[2][G + (NP - 1) * 4];     // c / s
  __shared__ double red[NC];
  // activation ring: [slot][wave][tile][lane][8 halves]
  constexpr int XSN = NC * NT * 64 * 8;
  // the global -> LDS copies write 64 lanes x 16 bytes from a base that
  // must be aligned to that 1 KB (a 64-byte offset gave wrong data)
  __shared__ __attribute__((aligned(1024))) uint16_t xring[4 * XSN];

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool consumer = wave < NC;    // wave-uniform role
  const float cscale = block_factor(bmax[rb]);
  const int ng = (int)(k / G);

  // ---- producer state
  const int ptid = tid - 64 * NC;     // producers are the last NP waves
  const int r = ptid / NP;            // row of the block this thread quantizes
  const int sub = ptid % NP;          // which part of the group
  const int64_t row = rb * kSearchRows + r;
  const bool row_ok = row < n;
  // rows past n load row n - 1 and zero it: a zero row has zero errors
  const uint16_t* wrow = w + (row_ok ? row : n - 1) * k + sub * EPT;
  // scale / reciprocal staging: producer thread t loads halves 8 (t % (G/8))
  // of the scales and floats 4 (t % (G/4)) of the reciprocals (clamped: every
  // producer loads, the first G/8 resp. G/4 store)
  const int s_i = ptid % (G / 8), r_i = ptid % (G / 4);
  uint4 wa[WLD], wb[WLD];             // weights of the current / next group
  uint4 sn;                           // scales / reciprocals of the next group:
  float4 rn;                          // loaded at the top of an iteration, stored to LDS at its end
  auto store_sr = [&](int buf, const uint4& sv, const float4& rv) {
    if (ptid < G / 8) *reinterpret_cast<uint4*>(&s_l[buf][8 * s_i + (8 * s_i / EPT) * 8]) = sv;
    if (ptid < G / 4)
      *reinterpret_cast<float4*>(&rc_l[buf][4 * r_i + (4 * r_i / EPT) * 4]) =
          make_float4(rv.x * cscale, rv.y * cscale, rv.z * cscale, rv.w * cscale);
  };
#define AWQ_LOAD_W(WV, J)                                                                   \
  {                                                                                         \
    _Pragma("unroll") for (int q_ = 0; q_ < WLD; ++q_) {                                    \
      const uint4 v_ = *reinterpret_cast<const uint4*>(wrow + (int64_t)(J) * G + 8 * q_);  \
      WV[q_] = row_ok ? v_ : make_uint4(0u, 0u, 0u, 0u);                                    \
    }                                                                                       \
  }
#define AWQ_LOAD_SR(SV, RV, J)                                                              \
  {                                                                                         \
    SV = *reinterpret_cast<const uint4*>(s16 + (int64_t)(J) * G + 8 * s_i);                \
    RV = *reinterpret_cast<const float4*>(rs + (int64_t)(J) * G + 4 * r_i);                \
  }
  // With four token tiles per consumer wave the accumulators leave no room
  // for a second weight buffer: the next group's weights are then loaded right
  // after stage 1 (still under the consumers' MFMAs) into the same registers.
  constexpr bool kWDouble = NT < 4;

  // stage 1 for one group: weights in WV, scales / reciprocals in LDS buffer
  // SB, errors into LDS buffers DH / DL
#define AWQ_PRODUCE(WV, SB, DH, DL)                                                         \
  {                                                                                         \
    half2_t pmx = {(half_t)-__builtin_inff(), (half_t)-__builtin_inff()};                   \
    half2_t pmn = {(half_t)__builtin_inff(), (half_t)__builtin_inff()};                     \
    _Pragma("unroll") for (int q = 0; q < WLD; ++q) {                                       \
      const uint4 sv = *reinterpret_cast<const uint4*>(&s_l[SB][sub * (EPT + 8) + 8 * q]); \
      const uint32_t wq4[4] = {WV[q].x, WV[q].y, WV[q].z, WV[q].w};                         \
      const uint32_t sq4[4] = {sv.x, sv.y, sv.z, sv.w};                                     \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                       \
        const half2_t wp = __builtin_bit_cast(half2_t, wq4[i]) * __builtin_bit_cast(half2_t, sq4[i]); \
        pmx = __builtin_elementwise_max(pmx, wp);                                           \
        pmn = __builtin_elementwise_min(pmn, wp);                                           \
      }                                                                                     \
    }                                                                                       \
    float mx = __builtin_fmaxf((float)pmx.x, (float)pmx.y);                                 \
    float mn = __builtin_fminf((float)pmn.x, (float)pmn.y);                                 \
    mx = __builtin_fmaxf(mx, dpp_mov<0xB1>(mx));                                            \
    mn = __builtin_fminf(mn, dpp_mov<0xB1>(mn));                                            \
    mx = __builtin_fmaxf(mx, dpp_mov<0x4E>(mx));                                            \
    mn = __builtin_fminf(mn, dpp_mov<0x4E>(mn));                                            \
    if constexpr (NP == 8) { /* the other quad of the row's 8 lanes (row_half_mirror) */    \
      mx = __builtin_fmaxf(mx, dpp_mov<0x141>(mx));                                         \
      mn = __builtin_fminf(mn, dpp_mov<0x141>(mn));                                         \
    }                                                                                       \
    const GroupQ gq = group_q(mx, mn, qmax);                                                \
    _Pragma("unroll") for (int q = 0; q < WLD; ++q) {                                       \
      __builtin_amdgcn_sched_barrier(0);                                                    \
      const uint4 sv = *reinterpret_cast<const uint4*>(&s_l[SB][sub * (EPT + 8) + 8 * q]); \
      const float4 rc0 = *reinterpret_cast<const float4*>(&rc_l[SB][sub * (EPT + 4) + 8 * q]);     \
      const float4 rc1 = *reinterpret_cast<const float4*>(&rc_l[SB][sub * (EPT + 4) + 8 * q + 4]); \
      const uint32_t wq4[4] = {WV[q].x, WV[q].y, WV[q].z, WV[q].w};                         \
      const uint32_t sq4[4] = {sv.x, sv.y, sv.z, sv.w};                                     \
      const float rcv[8] = {rc0.x, rc0.y, rc0.z, rc0.w, rc1.x, rc1.y, rc1.z, rc1.w};        \
      uint32_t hw[4], lw[4];                                                                \
      _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                       \
        const half2_t wv = __builtin_bit_cast(half2_t, wq4[i]);                             \
        const half2_t sv2 = __builtin_bit_cast(half2_t, sq4[i]);                            \
        const half2_t wp = wv * sv2;                                                        \
        float dw[2];                                                                        \
        _Pragma("unroll") for (int e = 0; e < 2; ++e) {                                     \
          const float deq = code_minus_zero_h(wp[e], gq) * gq.d;                            \
          /* deq - W s: the exact product, one rounding (v_fma_mix_f32) */                  \
          dw[e] = __builtin_fmaf(-(float)wv[e], (float)sv2[e], deq) * rcv[2 * i + e];       \
        }                                                                                   \
        const half2_t hi = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(dw[0], dw[1])); \
        const half2_t lo = __builtin_bit_cast(                                              \
            half2_t, __builtin_amdgcn_cvt_pkrtz(sub_f16_lo(dw[0], hi), sub_f16_hi(dw[1], hi))); \
        hw[i] = __builtin_bit_cast(uint32_t, hi);                                           \
        lw[i] = __builtin_bit_cast(uint32_t, lo);                                           \
      }                                                                                     \
      const int kloc = sub * EPT + 8 * q;                                                   \
      const int off = ((kloc / 8) * kSearchRows + r) * 8 + sub * PADS; /* [step][half][row][8] */ \
      *reinterpret_cast<uint4*>(&DH[off]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);         \
      *reinterpret_cast<uint4*>(&DL[off]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);         \
    }                                                                                       \
  }

  // ---- consumer state
  floatx16_t acc[2][NT];
  uint32_t xoff[NT];                  // byte offsets of this lane's fragment rows (m k < 2^31)
  const char* xbytes = reinterpret_cast<const char*>(x);
  // LDS byte address of this wave's part of ring slot 0
  const uint32_t xring_wave =
      (uint32_t)(uintptr_t)(&xring[0]) + (uint32_t)(wave * NT * 64 * 16);
  // copy step T of the pass (group T / KSTEPS, step T % KSTEPS; groups past
  // the last are clamped) into ring slot T % 4
#define AWQ_LOAD_X(T)                                                                       \
  {                                                                                         \
    int jj_ = (T) / KSTEPS;                                                                 \
    jj_ = jj_ < ng ? jj_ : ng - 1;                                                          \
    const char* xs_ = xbytes + ((int64_t)jj_ * G + 16 * ((T) % KSTEPS)) * 2;                \
    const uint32_t slot_ = xring_wave + (uint32_t)(((T) % 4) * XSN * 2);                    \
    _Pragma("unroll") for (int ti_ = 0; ti_ < NT; ++ti_)                                    \
      lds_copy16(xs_ + xoff[ti_], slot_ + (uint32_t)(ti_ * 64 * 16));                      \
  }
  // stage 2 for group J from LDS buffers DH / DL.  Software-pipelined: the
  // fragments of step s + 1 (dW from DH / DL, activations from the ring) are
  // read while the MFMAs of step s run, so an MFMA waits on LDS only at the
  // group's first step.  Ring slot (t + 3) % 4, filled at step t, held step
  // t - 1, whose fragments were read at step t - 2.
#define AWQ_CONSUME(J, DH, DL)                                                              \
  {                                                                                         \
    half8_t fa_[4], fb_[NT];                                                                \
    auto frags_ = [&](int s_, int t_, half8_t* a_, half8_t* b_) {                           \
      const uint16_t* xsl_ = xring + (t_ % 4) * XSN;                                        \
      const int ch_ = s_ * 2 + (lane >> 5);                                                 \
      const int aoff0 = (ch_ * kSearchRows + (lane & 31)) * 8 + (ch_ / CPQ) * PADS;         \
      const int aoff1 = aoff0 + 32 * 8;                                                     \
      a_[0] = *reinterpret_cast<const half8_t*>(&DH[aoff0]);                                \
      a_[1] = *reinterpret_cast<const half8_t*>(&DH[aoff1]);                                \
      a_[2] = *reinterpret_cast<const half8_t*>(&DL[aoff0]);                                \
      a_[3] = *reinterpret_cast<const half8_t*>(&DL[aoff1]);                                \
      _Pragma("unroll") for (int ti = 0; ti < NT; ++ti)                                     \
        b_[ti] = *reinterpret_cast<const half8_t*>(xsl_ + ((wave * NT + ti) * 64 + lane) * 8); \
    };                                                                                      \
    /* copies of steps t .. t + 2 are in flight: wait for step t's */                      \
    AWQ_WAIT_VMCNT(2 * NT);                                                                 \
    frags_(0, (J) * KSTEPS, fa_, fb_);                                                      \
    _Pragma("unroll") for (int s = 0; s < KSTEPS; ++s) {                                    \
      const int t_ = (J) * KSTEPS + s;                                                      \
      AWQ_LOAD_X(t_ + 3)                                                                    \
      half8_t na_[4], nb_[NT];                                                              \
      if (s + 1 < KSTEPS) {                                                                 \
        AWQ_WAIT_VMCNT(2 * NT);       /* step t + 1's copies have landed */                 \
        frags_(s + 1, t_ + 1, na_, nb_);                                                    \
      }                                                                                     \
      _Pragma("unroll") for (int ti = 0; ti < NT; ++ti) {                                   \
        acc[0][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa_[0], fb_[ti], acc[0][ti], 0, 0, 0); \
        acc[1][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa_[1], fb_[ti], acc[1][ti], 0, 0, 0); \
        acc[0][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa_[2], fb_[ti], acc[0][ti], 0, 0, 0); \
        acc[1][ti] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa_[3], fb_[ti], acc[1][ti], 0, 0, 0); \
      }                                                                                     \
      if (s + 1 < KSTEPS) {                                                                 \
        _Pragma("unroll") for (int q_ = 0; q_ < 4; ++q_) fa_[q_] = na_[q_];                 \
        _Pragma("unroll") for (int ti = 0; ti < NT; ++ti) fb_[ti] = nb_[ti];                \
      }                                                                                     \
    }                                                                                       \
  }

  // Iteration I: producers quantize group I (weights CUR, scales buffer I%2,
  // errors into dW buffer I%2) and load group I+1 into NXT; consumers multiply
  // group I-1 from the other dW buffer.  PB is I%2, known statically.  The two
  // roles run separate loops with the same barriers: in one shared loop the
  // producers' weight loads, pending across the loop head, make the compiler
  // wait for every outstanding load of the consumers too (their activation
  // copies, three steps ahead) before it reuses a register.
#define AWQ_PRODUCE_STEP(I, PB, WCUR, WNXT, DHP, DLP)                                        \
  {                                                                                         \
    const int jn_ = (I) + 1 < ng ? (I) + 1 : ng - 1;                                        \
    AWQ_LOAD_SR(sn, rn, jn_)                                                                \
    if constexpr (kWDouble) AWQ_LOAD_W(WNXT, jn_)                                           \
    AWQ_PRODUCE(WCUR, PB, DHP, DLP)                                                         \
    if constexpr (!kWDouble) AWQ_LOAD_W(WCUR, jn_)                                          \
    store_sr((PB) ^ 1, sn, rn);                                                             \
  }

  double loss = 0.0;
  for (int64_t t0 = 0; t0 < m; t0 += TOK) {
    if (consumer) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[b][i] = floatx16_t{};
      // activation fragment rows of this wave's tiles (clamped tokens; tokens
      // past m are left out of the squares)
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) {
        int64_t tok = t0 + (int64_t)(wave + NC * ti) * 32 + (lane & 31);
        tok = tok < m ? tok : m - 1;
        xoff[ti] = (uint32_t)((tok * k + 8 * (lane >> 5)) * 2);
      }
      AWQ_LOAD_X(0)
      AWQ_LOAD_X(1)
      AWQ_LOAD_X(2)
      __syncthreads();
      for (int i = 0; i <= ng; i += 2) {
        if (i >= 1) AWQ_CONSUME(i - 1, dh1, dl1)
        __syncthreads();
        if (i + 1 <= ng) {
          AWQ_CONSUME(i, dh0, dl0)
          __syncthreads();
        }
      }
      // ---- square and reduce (float64, fixed order) over the valid tokens
      AWQ_WAIT_VMCNT(0);              // the ring's look-ahead copies have landed
      double sq = 0.0;
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) {
        const int64_t tok = t0 + (int64_t)(wave + NC * ti) * 32 + (lane & 31);
        if (tok < m) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const double e = (double)acc[b][ti][i];
              sq += e * e;
            }
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sq += shfl_xor_d(sq, off);
      if (lane == 0) red[wave] = sq;
    } else {
      AWQ_LOAD_W(wa, 0)
      AWQ_LOAD_SR(sn, rn, 0)
      store_sr(0, sn, rn);
      __syncthreads();
      for (int i = 0; i <= ng; i += 2) {
        if (i < ng) {
          if constexpr (kWDouble) AWQ_PRODUCE_STEP(i, 0, wa, wb, dh0, dl0)
          else AWQ_PRODUCE_STEP(i, 0, wa, wa, dh0, dl0)
        }
        __syncthreads();
        if (i + 1 <= ng) {
          if (i + 1 < ng) {
            if constexpr (kWDouble) AWQ_PRODUCE_STEP(i + 1, 1, wb, wa, dh1, dl1)
            else AWQ_PRODUCE_STEP(i + 1, 1, wa, wa, dh1, dl1)
          }
          __syncthreads();
        }
      }
    }
    __syncthreads();
    double pass = red[0];
#pragma unroll
    for (int i = 1; i < NC; ++i) pass += red[i];
    loss += pass;
    __syncthreads();
  }
#undef AWQ_PRODUCE_STEP
#undef AWQ_CONSUME

#undef AWQ_LOAD_X
#undef AWQ_PRODUCE
#undef AWQ_LOAD_SR
#undef AWQ_LOAD_W
  const double inv_c = 1.0 / (double)cscale;       // exact: c is a power of two
  if (tid == 0) part[(int64_t)ai * n_blocks + rb] = loss * inv_c * inv_c;
}

// One wave per alpha (alpha = wave, wave + 4, ...): lane l sums the partials
// of blocks l, l + 64, ... in order, then a fixed butterfly combines the lanes,
// so the sum is deterministic.  Thread 0 takes the first minimum over finite
// losses.  Every work-group of the grid computes the same sums and minimum and
// writes s16 and inv_s16 for its 256 channels; work-group 0 also writes the
// losses and the index.
__global__ __launch_bounds__(256) void search_select_kernel(
    const double* __restrict__ part, int64_t n_blocks, int32_t n_grid, int64_t k,
    const uint16_t* __restrict__ s16_all, int32_t* __restrict__ best_idx,
    uint16_t* __restrict__ s16, uint16_t* __restrict__ inv_s16, double* __restrict__ losses) {
  __shared__ double L[64];
  __shared__ int best_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = wave; i < n_grid; i += 4) {
    double sacc = 0.0;
    for (int64_t b = lane; b < n_blocks; b += 64) sacc += part[(int64_t)i * n_blocks + b];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sacc += shfl_xor_d(sacc, off);
    if (lane == 0) {
      L[i] = sacc;
      if (losses != nullptr && blockIdx.x == 0) losses[i] = sacc;
    }
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
    if (blockIdx.x == 0) *best_idx = best;
  }
  __syncthreads();
  const int best = best_s;
  const int64_t col = (int64_t)blockIdx.x * 256 + tid;
  if (col < k) {
    uint16_t sb = best >= 0 ? s16_all[(int64_t)best * k + col] : kF16One;
    s16[col] = sb;
    inv_s16[col] = f64_to_f16_rn(1.0 / (double)h2f(sb));
  }
}

hipError_t launch_search(const uint16_t* w, const uint16_t* x, const double* mean_abs,
                         int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid,
                         int32_t w_bit, int32_t* best_idx, uint16_t* s16, uint16_t* inv_s16,
                         double* losses, void* workspace, hipStream_t stream) {
  const float qmax = (float)((1 << w_bit) - 1);
  const SearchLayout L = search_layout(n, k, m, g, n_grid);
  char* ws = static_cast<char*>(workspace);
  uint16_t* s16_all = reinterpret_cast<uint16_t*>(ws + L.off_s16);
  float* rs_all = reinterpret_cast<float*>(ws + L.off_rs);
  double* part = reinterpret_cast<double*>(ws + L.off_part);
  uint32_t* bmax = reinterpret_cast<uint32_t*>(ws + L.off_cblk);

  hipLaunchKernelGGL(search_prep_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)n_grid),
                     dim3(256), 0, stream, mean_abs, k, n_grid, s16_all, rs_all, bmax, L.n_blocks);
  hipLaunchKernelGGL(search_blockmax_kernel,
                     dim3((unsigned)L.n_blocks, (unsigned)((k + kBlockMaxCols - 1) / kBlockMaxCols)),
                     dim3(256), 0, stream, w, n, k, bmax);
  const unsigned nwg = (unsigned)(L.n_blocks * n_grid);
  // token tiles per wave and pass: 128 NT tokens per pass
  // token tiles per consumer wave and pass (128 NT tokens) and producer
  // waves: up to 128 tokens, where quantizing a group takes longer than its
  // MFMAs, eight producers (g >= 64), else four
  const int nt = m <= 128 ? 1 : (m <= 256 ? 2 : 4);
  const bool np8 = m <= 128 && g >= 64;
#define AWQ_SEARCH_LAUNCH(GG, NTT, NPP)                                                         \
  hipLaunchKernelGGL((search_loss_kernel<GG, NTT, NPP>), dim3(nwg), dim3(64 * (4 + NPP)), 0,  \
                     stream, w, x, n, k, m, n_grid, L.n_blocks, s16_all, rs_all, bmax, part, qmax)
#define AWQ_SEARCH_NT(GG)                        \
  switch (nt) {                                  \
    case 1: AWQ_SEARCH_LAUNCH(GG, 1, 4); break;  \
    case 2: AWQ_SEARCH_LAUNCH(GG, 2, 4); break;  \
    default: AWQ_SEARCH_LAUNCH(GG, 4, 4); break; \
  }
  switch (g) {
    case 32: AWQ_SEARCH_NT(32); break;
    case 64:
      if (np8) AWQ_SEARCH_LAUNCH(64, 1, 8);
      else AWQ_SEARCH_NT(64);
      break;
    default:
      if (np8) AWQ_SEARCH_LAUNCH(128, 1, 8);
      else AWQ_SEARCH_NT(128);
      break;
  }
#undef AWQ_SEARCH_NT
#undef AWQ_SEARCH_LAUNCH
  hipLaunchKernelGGL(search_select_kernel, dim3((unsigned)((k + 255) / 256)), dim3(256), 0, stream,
                     part, L.n_blocks,
                     n_grid, k, s16_all, best_idx, s16, inv_s16, losses);
  return hipGetLastError();
}

}  // namespace awq
