// Internal launch functions behind the C ABI (host side).  Arguments are
// already validated by the entry points in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

hipError_t launch_calib_stats(const uint16_t* x, int64_t m, int64_t k, double* out,
                              hipStream_t stream);

// Search workspace layout (bytes, 256-aligned sections):
//   s16  [n_grid][k]        fp16 candidate scales
//   rs   [n_grid][k]        fp32 reciprocals of the candidates
//   part [n_grid][n_blocks] float64 per-row-block partial losses
//   cblk [n_blocks]         uint32 largest finite |W| (fp16 bits) of each 64-row block
struct SearchLayout {
  size_t off_s16, off_rs, off_part, off_cblk, total;
  int64_t n_blocks;
};
SearchLayout search_layout(int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid);

hipError_t launch_search(const uint16_t* w, const uint16_t* x, const double* mean_abs,
                         int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid,
                         int32_t w_bit, int32_t* best_idx, uint16_t* s16, uint16_t* inv_s16,
                         double* losses, void* workspace, hipStream_t stream);

hipError_t launch_fold_inv_scale_rows(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                                      uint16_t* out, hipStream_t stream);
hipError_t launch_fold_inv_scale(const uint16_t* v, const uint16_t* s16, int64_t k, uint16_t* out,
                                 hipStream_t stream);

hipError_t launch_pack(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                       int32_t g, uint32_t* qweight, uint16_t* scales, uint32_t* qzeros,
                       int32_t* nonfinite, hipStream_t stream);

// 3- or 8-bit packing (layouts of awq_pack_wbit)
hipError_t launch_pack_wbit(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                            int32_t g, int32_t w_bit, uint32_t* qweight, uint16_t* scales,
                            uint32_t* qzeros, int32_t* nonfinite, hipStream_t stream);

// Most linears one grouped decode launch takes.
constexpr int kGroupMax = 4;

// One linear of a group (device pointers, validated by the caller): x [m][k],
// inv_s16 [k] or null, packed weights in layout v1, y [m][n].
struct LinItem {
  const uint16_t* x;
  const uint16_t* inv;
  const uint32_t* qw;
  const uint16_t* sc;
  const uint32_t* qz;
  uint16_t* y;
  int64_t n;
  int32_t bf = 0;          // 1: x and y hold bf16 patterns (the same for every item of a call)
};

// Device scratch of one linear call: the caller's workspace (base), or a
// plan-only pass (dry) in which the launch code records the bytes its plan
// would use (need) and launches nothing.  One code path decides the plan for
// both, so the size the library asks for is exactly what the launches touch.
struct Scratch {
  char* base = nullptr;
  size_t need = 0;
  bool dry = false;
  // the scratch bytes [off, off + bytes) of this call (nullptr in a dry pass)
  char* at(size_t off, size_t bytes) {
    if (off + bytes > need) need = off + bytes;
    return base ? base + off : nullptr;
  }
};

// 1..kGroupMax independent linears of the same m, k and g: one launch for the
// kernels that take groups (decode GEMV, fused skinny, prefill GEMM),
// consecutive launches otherwise.  Each y holds the bits a call of that
// linear alone writes.  Scratch: linear_group_scratch_bytes bytes,
// 256-byte aligned (0 for the decode GEMV and the fused skinny kernels).
hipError_t launch_linear_group(const LinItem* items, int count, int64_t m, int64_t k, int32_t g,
                               Scratch& scr, hipStream_t stream);
size_t linear_group_scratch_bytes(const LinItem* items, int count, int64_t m, int64_t k,
                                  int32_t g);

// mixed-precision baseline (mixed.hip)
hipError_t launch_salient_select(const double* a, int64_t k, int32_t count, int32_t* idx,
                                 hipStream_t stream);
hipError_t launch_channel_mask(const int32_t* idx, int32_t count, int64_t k, uint16_t* keep,
                               hipStream_t stream);
hipError_t launch_gather_channels(const uint16_t* w, int64_t n, int64_t k, const int32_t* idx,
                                  int32_t count, uint16_t* w_s, hipStream_t stream);
hipError_t launch_mask_rows(const uint16_t* x, const uint16_t* keep, int64_t m, int64_t k,
                            uint16_t* out, hipStream_t stream);
hipError_t launch_salient_add(const uint16_t* x, const int32_t* idx, int32_t count,
                              const uint16_t* w_s, int64_t m, int64_t n, int64_t k, uint16_t* y,
                              hipStream_t stream);
size_t mixed_loss_workspace_bytes(int64_t n, int64_t k, int64_t m, int32_t g);
hipError_t launch_mixed_loss(const uint16_t* w, const uint16_t* x, const uint16_t* keep, int64_t n,
                             int64_t k, int64_t m, int32_t g, double* loss, void* workspace,
                             hipStream_t stream);
constexpr int32_t kMixedMaxCount = 1024;       // protected channels per linear (LDS of the add)

// the linear for 3- and 8-bit weights (layouts of awq_pack_wbit); scratch of
// linear_wbit_scratch_bytes(m, n, k, g, inv_s16 != NULL) bytes, 256-byte aligned
size_t linear_wbit_scratch_bytes(int64_t m, int64_t n, int64_t k, int32_t g, bool has_inv);
hipError_t launch_linear_wbit(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                              const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m,
                              int64_t n, int64_t k, int32_t g, int32_t w_bit, uint16_t* y,
                              void* scratch, hipStream_t stream);

}  // namespace awq
