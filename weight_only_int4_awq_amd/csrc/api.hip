// C ABI entry points: argument validation on the host, then launches on the
// caller's stream.  No entry point synchronises.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/awq_mi355x.h"
#include "awq_common.h"
#include "awq_internal.h"

namespace {

thread_local char g_err[512] = "";

awq_status fail(awq_status s, const char* fmt, long long a = 0, long long b = 0) {
  snprintf(g_err, sizeof(g_err), fmt, a, b);
  return s;
}

awq_status hip_fail(hipError_t e, const char* where) {
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
  return AWQ_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool group_ok(int32_t g) { return g == 32 || g == 64 || g == 128; }

}  // namespace

extern "C" {

int32_t awq_abi_version(void) { return 2; }

const char* awq_last_error(void) { return g_err; }

awq_status awq_calib_stats(const uint16_t* x, int64_t m, int64_t k, double* mean_abs,
                           void* stream) {
  g_err[0] = 0;
  if (!x || !mean_abs) return fail(AWQ_ERR_NULL, "awq_calib_stats: null pointer");
  if (m < 1 || m > 8192) return fail(AWQ_ERR_SHAPE, "awq_calib_stats: m=%lld outside 1..8192", m);
  if (k < 8 || k % 8 != 0) return fail(AWQ_ERR_SHAPE, "awq_calib_stats: k=%lld must be a positive multiple of 8", k);
  if (!aligned(x, 16) || !aligned(mean_abs, 8)) return fail(AWQ_ERR_ALIGN, "awq_calib_stats: x must be 16-byte aligned");
  hipError_t e = awq::launch_calib_stats(x, m, k, mean_abs, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_calib_stats launch");
  return AWQ_OK;
}

size_t awq_search_workspace_size(int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid) {
  if (n < 1 || k < 1 || m < 1 || n_grid < 1 || n_grid > 64 || !group_ok(g)) return 0;
  return awq::search_layout(n, k, m, g, n_grid).total;
}

static awq_status search_scale_impl(const char* fn, const uint16_t* w, const uint16_t* x,
                                    const double* mean_abs, int64_t n, int64_t k, int64_t m,
                                    int32_t g, int32_t n_grid, int32_t w_bit, int32_t* best_idx,
                                    uint16_t* s16, uint16_t* inv_s16, double* losses,
                                    void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  char msg[96];
  auto err = [&](awq_status st, const char* what, long long a = 0, long long b = 0) {
    snprintf(msg, sizeof(msg), "%s: %s", fn, what);
    return fail(st, msg, a, b);
  };
  if (!w || !x || !mean_abs || !best_idx || !s16 || !inv_s16) return err(AWQ_ERR_NULL, "null pointer");
  if (w_bit != 3 && w_bit != 4 && w_bit != 8) return err(AWQ_ERR_SHAPE, "w_bit=%lld not in {3,4,8}", w_bit);
  if (!group_ok(g)) return err(AWQ_ERR_SHAPE, "g=%lld not in {32,64,128}", g);
  if (k < g || k % g != 0) return err(AWQ_ERR_SHAPE, "k=%lld not a positive multiple of g=%lld", k, g);
  if (n < 1) return err(AWQ_ERR_SHAPE, "n=%lld < 1", n);
  if (m < 1 || m > 8192) return err(AWQ_ERR_SHAPE, "m=%lld outside 1..8192", m);
  if (n_grid < 1 || n_grid > 64) return err(AWQ_ERR_SHAPE, "n_grid=%lld outside 1..64", n_grid);
  if (!aligned(w, 16) || !aligned(x, 16)) return err(AWQ_ERR_ALIGN, "w and x must be 16-byte aligned");
  if (!aligned(mean_abs, 8) || !aligned(s16, 2) || !aligned(inv_s16, 2) || (losses && !aligned(losses, 8)))
    return err(AWQ_ERR_ALIGN, "misaligned output");
  const size_t need = awq::search_layout(n, k, m, g, n_grid).total;
  if (!workspace || ws_bytes < need)
    return err(AWQ_ERR_WORKSPACE, "workspace of %lld bytes < %lld needed", (long long)ws_bytes, (long long)need);
  if (!aligned(workspace, 256)) return err(AWQ_ERR_ALIGN, "workspace must be 256-byte aligned");
  hipError_t e = awq::launch_search(w, x, mean_abs, n, k, m, g, n_grid, w_bit, best_idx, s16,
                                    inv_s16, losses, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return AWQ_OK;
}

awq_status awq_search_scale(const uint16_t* w, const uint16_t* x, const double* mean_abs,
                            int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid,
                            int32_t* best_idx, uint16_t* s16, uint16_t* inv_s16,
                            double* losses, void* workspace, size_t ws_bytes, void* stream) {
  return search_scale_impl("awq_search_scale", w, x, mean_abs, n, k, m, g, n_grid, 4, best_idx,
                           s16, inv_s16, losses, workspace, ws_bytes, stream);
}

awq_status awq_search_scale_wbit(const uint16_t* w, const uint16_t* x, const double* mean_abs,
                                 int64_t n, int64_t k, int64_t m, int32_t g, int32_t n_grid,
                                 int32_t w_bit, int32_t* best_idx, uint16_t* s16,
                                 uint16_t* inv_s16, double* losses, void* workspace,
                                 size_t ws_bytes, void* stream) {
  return search_scale_impl("awq_search_scale_wbit", w, x, mean_abs, n, k, m, g, n_grid, w_bit,
                           best_idx, s16, inv_s16, losses, workspace, ws_bytes, stream);
}

static awq_status pack_impl(const char* fn, const uint16_t* w, const uint16_t* s16, int64_t n,
                            int64_t k, int32_t g, int32_t w_bit, uint32_t* qweight,
                            uint16_t* scales, uint32_t* qzeros, int32_t* nonfinite_groups,
                            void* stream) {
  g_err[0] = 0;
  char msg[96];
  auto err = [&](awq_status st, const char* what, long long a = 0, long long b = 0) {
    snprintf(msg, sizeof(msg), "%s: %s", fn, what);
    return fail(st, msg, a, b);
  };
  if (!w || !qweight || !scales || !qzeros) return err(AWQ_ERR_NULL, "null pointer");
  if (w_bit != 3 && w_bit != 4 && w_bit != 8) return err(AWQ_ERR_SHAPE, "w_bit=%lld not in {3,4,8}", w_bit);
  if (!group_ok(g)) return err(AWQ_ERR_SHAPE, "g=%lld not in {32,64,128}", g);
  if (k < g || k % g != 0) return err(AWQ_ERR_SHAPE, "k=%lld not a positive multiple of g=%lld", k, g);
  if (n < 1 || n > 0x7FFFFFFF) return err(AWQ_ERR_SHAPE, "n=%lld out of range", n);
  if (!aligned(w, 16) || !aligned(qweight, 16) || (s16 && !aligned(s16, 16)))
    return err(AWQ_ERR_ALIGN, "w, s16 and qweight must be 16-byte aligned");
  if (!aligned(scales, 2) || !aligned(qzeros, 4) || (nonfinite_groups && !aligned(nonfinite_groups, 4)))
    return err(AWQ_ERR_ALIGN, "misaligned output");
  hipError_t e = awq::launch_pack_wbit(w, s16, n, k, g, w_bit, qweight, scales, qzeros,
                                       nonfinite_groups, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return AWQ_OK;
}

awq_status awq_pack_int4(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k, int32_t g,
                         uint32_t* qweight, uint16_t* scales, uint32_t* qzeros,
                         int32_t* nonfinite_groups, void* stream) {
  return pack_impl("awq_pack_int4", w, s16, n, k, g, 4, qweight, scales, qzeros, nonfinite_groups,
                   stream);
}

awq_status awq_pack_wbit(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k, int32_t g,
                         int32_t w_bit, uint32_t* qweight, uint16_t* scales, uint32_t* qzeros,
                         int32_t* nonfinite_groups, void* stream) {
  return pack_impl("awq_pack_wbit", w, s16, n, k, g, w_bit, qweight, scales, qzeros,
                   nonfinite_groups, stream);
}

awq_status awq_fold_inv_scale_rows(const uint16_t* w, const uint16_t* s16, int64_t n, int64_t k,
                                   uint16_t* out, void* stream) {
  g_err[0] = 0;
  if (!w || !s16 || !out) return fail(AWQ_ERR_NULL, "awq_fold_inv_scale_rows: null pointer");
  if (n < 1 || k < 1) return fail(AWQ_ERR_SHAPE, "awq_fold_inv_scale_rows: n=%lld, k=%lld must be >= 1", n, k);
  if (!aligned(w, 2) || !aligned(s16, 2) || !aligned(out, 2))
    return fail(AWQ_ERR_ALIGN, "awq_fold_inv_scale_rows: misaligned pointer");
  hipError_t e = awq::launch_fold_inv_scale_rows(w, s16, n, k, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_fold_inv_scale_rows launch");
  return AWQ_OK;
}

awq_status awq_fold_inv_scale(const uint16_t* v, const uint16_t* s16, int64_t k, uint16_t* out,
                              void* stream) {
  g_err[0] = 0;
  if (!v || !s16 || !out) return fail(AWQ_ERR_NULL, "awq_fold_inv_scale: null pointer");
  if (k < 1) return fail(AWQ_ERR_SHAPE, "awq_fold_inv_scale: k=%lld < 1", k);
  if (!aligned(v, 2) || !aligned(s16, 2) || !aligned(out, 2))
    return fail(AWQ_ERR_ALIGN, "awq_fold_inv_scale: misaligned pointer");
  hipError_t e = awq::launch_fold_inv_scale(v, s16, k, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_fold_inv_scale launch");
  return AWQ_OK;
}

}  // extern "C"

namespace {

// checks shared by awq_linear_w4a16 and awq_linear_w4a16_group
awq_status check_linear_args(const char* fn, const uint16_t* x, const uint32_t* qweight,
                             const uint16_t* scales, const uint32_t* qzeros,
                             const uint16_t* inv_s16, int64_t m, int64_t n, int64_t k, int32_t g,
                             const uint16_t* y) {
  if (!x || !qweight || !scales || !qzeros || !y) {
    snprintf(g_err, sizeof(g_err), "%s: null pointer", fn);
    return AWQ_ERR_NULL;
  }
  if (!group_ok(g)) {
    snprintf(g_err, sizeof(g_err), "%s: g=%lld not in {32,64,128}", fn, (long long)g);
    return AWQ_ERR_SHAPE;
  }
  if (k < 64 || k % g != 0 || k % 64 != 0) {
    snprintf(g_err, sizeof(g_err), "%s: k=%lld must be a multiple of g=%lld and of 64", fn, (long long)k,
             (long long)g);
    return AWQ_ERR_SHAPE;
  }
  if (m < 1 || m > 0x7FFFFFFF) {
    snprintf(g_err, sizeof(g_err), "%s: m=%lld out of range", fn, (long long)m);
    return AWQ_ERR_SHAPE;
  }
  if (n < 1 || n > 0x7FFFFFFF) {
    snprintf(g_err, sizeof(g_err), "%s: n=%lld out of range", fn, (long long)n);
    return AWQ_ERR_SHAPE;
  }
  // x, inv_s16 and qweight are read with 16-byte loads and direct-to-LDS copies
  if (!aligned(x, 16) || !aligned(qweight, 16) || (inv_s16 && !aligned(inv_s16, 16))) {
    snprintf(g_err, sizeof(g_err), "%s: x, inv_s16 and qweight must be 16-byte aligned", fn);
    return AWQ_ERR_ALIGN;
  }
  // scales are read as 32-bit words of two groups by the prefill GEMM
  if (!aligned(scales, 4) || !aligned(qzeros, 4) || !aligned(y, 2)) {
    snprintf(g_err, sizeof(g_err), "%s: misaligned pointer", fn);
    return AWQ_ERR_ALIGN;
  }
  if ((unsigned long long)n * (unsigned long long)k / 2 >= (1ull << 32)) {
    snprintf(g_err, sizeof(g_err), "%s: packed weights of n=%lld x k=%lld exceed 4 GiB", fn, (long long)n,
             (long long)k);
    return AWQ_ERR_SHAPE;
  }
  return AWQ_OK;
}

// the caller's workspace against what the call's plan needs
awq_status check_workspace(const char* fn, size_t need, const void* workspace, size_t ws_bytes) {
  if (need == 0) return AWQ_OK;
  if (!workspace || ws_bytes < need) {
    snprintf(g_err, sizeof(g_err), "%s: workspace of %llu bytes < %llu needed", fn,
             (unsigned long long)(workspace ? ws_bytes : 0), (unsigned long long)need);
    return AWQ_ERR_WORKSPACE;
  }
  if (!aligned(workspace, 256)) {
    snprintf(g_err, sizeof(g_err), "%s: workspace must be 256-byte aligned", fn);
    return AWQ_ERR_ALIGN;
  }
  return AWQ_OK;
}

awq_status run_linear_group(const char* fn, const awq::LinItem* li, int32_t count, int64_t m, int64_t k,
                            int32_t g, void* workspace, size_t ws_bytes, void* stream) {
  const size_t need = awq::linear_group_scratch_bytes(li, count, m, k, g);
  awq_status st = check_workspace(fn, need, workspace, ws_bytes);
  if (st != AWQ_OK) return st;
  awq::Scratch scr;
  scr.base = static_cast<char*>(workspace);
  hipError_t e = awq::launch_linear_group(li, count, m, k, g, scr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return AWQ_OK;
}

awq_status linear_impl(const char* fn, const uint16_t* x, const uint32_t* qweight,
                       const uint16_t* scales, const uint32_t* qzeros, const uint16_t* inv_s16,
                       int64_t m, int64_t n, int64_t k, int32_t g, uint16_t* y, int32_t bf,
                       void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  awq_status st0 = check_linear_args(fn, x, qweight, scales, qzeros, inv_s16, m, n, k, g, y);
  if (st0 != AWQ_OK) return st0;
  awq::LinItem it{x, inv_s16, qweight, scales, qzeros, y, n};
  it.bf = bf;
  return run_linear_group(fn, &it, 1, m, k, g, workspace, ws_bytes, stream);
}

awq_status linear_group_impl(const char* fn, const awq_linear_item* items, int32_t count, int64_t m,
                             int64_t k, int32_t g, int32_t bf, void* workspace, size_t ws_bytes,
                             void* stream) {
  g_err[0] = 0;
  if (!items) {
    snprintf(g_err, sizeof(g_err), "%s: null items", fn);
    return AWQ_ERR_NULL;
  }
  if (count < 1 || count > awq::kGroupMax) {
    snprintf(g_err, sizeof(g_err), "%s: count=%lld outside 1..%lld", fn, (long long)count,
             (long long)awq::kGroupMax);
    return AWQ_ERR_SHAPE;
  }
  awq::LinItem li[awq::kGroupMax];
  for (int32_t i = 0; i < count; ++i) {
    const awq_linear_item& it = items[i];
    awq_status st = check_linear_args(fn, it.x, it.qweight, it.scales, it.qzeros, it.inv_s16, m, it.n,
                                      k, g, it.y);
    if (st != AWQ_OK) return st;
    li[i] = awq::LinItem{it.x, it.inv_s16, it.qweight, it.scales, it.qzeros, it.y, it.n};
    li[i].bf = bf;
  }
  return run_linear_group(fn, li, count, m, k, g, workspace, ws_bytes, stream);
}

bool linear_shape_ok(int64_t m, int64_t n, int64_t k, int32_t g) {
  return group_ok(g) && k >= 64 && k % g == 0 && k % 64 == 0 && m >= 1 && m <= 0x7FFFFFFF && n >= 1 &&
         n <= 0x7FFFFFFF;
}

}  // namespace

extern "C" {

size_t awq_linear_workspace_size(int64_t m, int64_t n, int64_t k, int32_t g) {
  if (!linear_shape_ok(m, n, k, g)) return 0;
  awq::LinItem it{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, n};
  return awq::linear_group_scratch_bytes(&it, 1, m, k, g);
}

size_t awq_linear_group_workspace_size(const int64_t* n, int32_t count, int64_t m, int64_t k,
                                       int32_t g) {
  if (!n || count < 1 || count > awq::kGroupMax) return 0;
  awq::LinItem li[awq::kGroupMax];
  for (int32_t i = 0; i < count; ++i) {
    if (!linear_shape_ok(m, n[i], k, g)) return 0;
    li[i] = awq::LinItem{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, n[i]};
  }
  return awq::linear_group_scratch_bytes(li, count, m, k, g);
}

awq_status awq_linear_w4a16(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m, int64_t n,
                            int64_t k, int32_t g, uint16_t* y, void* workspace, size_t ws_bytes,
                            void* stream) {
  return linear_impl("awq_linear_w4a16", x, qweight, scales, qzeros, inv_s16, m, n, k, g, y, 0,
                     workspace, ws_bytes, stream);
}

awq_status awq_linear_w4a16_bf16(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                                 const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m,
                                 int64_t n, int64_t k, int32_t g, uint16_t* y, void* workspace,
                                 size_t ws_bytes, void* stream) {
  return linear_impl("awq_linear_w4a16_bf16", x, qweight, scales, qzeros, inv_s16, m, n, k, g, y, 1,
                     workspace, ws_bytes, stream);
}

awq_status awq_linear_w4a16_group(const awq_linear_item* items, int32_t count, int64_t m, int64_t k,
                                  int32_t g, void* workspace, size_t ws_bytes, void* stream) {
  return linear_group_impl("awq_linear_w4a16_group", items, count, m, k, g, 0, workspace, ws_bytes,
                           stream);
}

awq_status awq_linear_w4a16_group_bf16(const awq_linear_item* items, int32_t count, int64_t m,
                                       int64_t k, int32_t g, void* workspace, size_t ws_bytes,
                                       void* stream) {
  return linear_group_impl("awq_linear_w4a16_group_bf16", items, count, m, k, g, 1, workspace,
                           ws_bytes, stream);
}

size_t awq_linear_wbit_workspace_size(int64_t m, int64_t n, int64_t k, int32_t g, int32_t w_bit,
                                      int32_t has_inv_s16) {
  if (w_bit == 4) return awq_linear_workspace_size(m, n, k, g);
  if ((w_bit != 3 && w_bit != 8) || !linear_shape_ok(m, n, k, g)) return 0;
  return awq::linear_wbit_scratch_bytes(m, n, k, g, has_inv_s16 != 0);
}

awq_status awq_linear_wbit(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* qzeros, const uint16_t* inv_s16, int64_t m, int64_t n,
                           int64_t k, int32_t g, int32_t w_bit, uint16_t* y, void* workspace,
                           size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (w_bit == 4) {
    awq_status st = awq_linear_w4a16(x, qweight, scales, qzeros, inv_s16, m, n, k, g, y, workspace,
                                     ws_bytes, stream);
    if (st != AWQ_OK) {
      char msg[512];
      snprintf(msg, sizeof(msg), "awq_linear_wbit (w_bit 4) -> %s", g_err);
      snprintf(g_err, sizeof(g_err), "%s", msg);
    }
    return st;
  }
  if (!x || !qweight || !scales || !qzeros || !y) return fail(AWQ_ERR_NULL, "awq_linear_wbit: null pointer");
  if (w_bit != 3 && w_bit != 8) return fail(AWQ_ERR_SHAPE, "awq_linear_wbit: w_bit=%lld not in {3,4,8}", w_bit);
  if (!group_ok(g)) return fail(AWQ_ERR_SHAPE, "awq_linear_wbit: g=%lld not in {32,64,128}", g);
  if (k < 64 || k % g != 0 || k % 64 != 0)
    return fail(AWQ_ERR_SHAPE, "awq_linear_wbit: k=%lld must be a multiple of g=%lld and of 64", k, g);
  if (m < 1 || m > 0x7FFFFFFF) return fail(AWQ_ERR_SHAPE, "awq_linear_wbit: m=%lld out of range", m);
  if (n < 1 || n > 0x7FFFFFFF) return fail(AWQ_ERR_SHAPE, "awq_linear_wbit: n=%lld out of range", n);
  if (!aligned(x, 16) || !aligned(qweight, 16) || (inv_s16 && !aligned(inv_s16, 16)))
    return fail(AWQ_ERR_ALIGN, "awq_linear_wbit: x, qweight and inv_s16 must be 16-byte aligned");
  if (!aligned(qzeros, 4) || !aligned(scales, 2) || !aligned(y, 2))
    return fail(AWQ_ERR_ALIGN, "awq_linear_wbit: misaligned pointer");
  const size_t need = awq::linear_wbit_scratch_bytes(m, n, k, g, inv_s16 != nullptr);
  awq_status st = check_workspace("awq_linear_wbit", need, workspace, ws_bytes);
  if (st != AWQ_OK) return st;
  hipError_t e = awq::launch_linear_wbit(x, qweight, scales, qzeros, inv_s16, m, n, k, g, w_bit, y,
                                         workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_linear_wbit launch");
  return AWQ_OK;
}

awq_status awq_salient_channels(const double* mean_abs, int64_t k, int32_t count, int32_t* idx,
                                void* stream) {
  g_err[0] = 0;
  if (!mean_abs || (!idx && count > 0)) return fail(AWQ_ERR_NULL, "awq_salient_channels: null pointer");
  if (k < 1 || k > 0x7FFFFFFF) return fail(AWQ_ERR_SHAPE, "awq_salient_channels: k=%lld out of range", k);
  if (count < 0 || count > k || count > awq::kMixedMaxCount)
    return fail(AWQ_ERR_SHAPE, "awq_salient_channels: count=%lld outside 0..min(k, %lld)", count,
                awq::kMixedMaxCount);
  if (!aligned(mean_abs, 8) || (idx && !aligned(idx, 4)))
    return fail(AWQ_ERR_ALIGN, "awq_salient_channels: misaligned pointer");
  hipError_t e = awq::launch_salient_select(mean_abs, k, count, idx, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_salient_channels launch");
  return AWQ_OK;
}

awq_status awq_channel_mask(const int32_t* idx, int32_t count, int64_t k, uint16_t* keep16,
                            void* stream) {
  g_err[0] = 0;
  if (!keep16 || (!idx && count > 0)) return fail(AWQ_ERR_NULL, "awq_channel_mask: null pointer");
  if (k < 1 || count < 0 || count > k) return fail(AWQ_ERR_SHAPE, "awq_channel_mask: count=%lld, k=%lld", count, k);
  if (!aligned(keep16, 2) || (idx && !aligned(idx, 4))) return fail(AWQ_ERR_ALIGN, "awq_channel_mask: misaligned pointer");
  hipError_t e = awq::launch_channel_mask(idx, count, k, keep16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_channel_mask launch");
  return AWQ_OK;
}

awq_status awq_gather_channels(const uint16_t* w, int64_t n, int64_t k, const int32_t* idx,
                               int32_t count, uint16_t* w_s, void* stream) {
  g_err[0] = 0;
  if (!w || ((!idx || !w_s) && count > 0)) return fail(AWQ_ERR_NULL, "awq_gather_channels: null pointer");
  if (n < 1 || k < 1 || count < 0 || count > k)
    return fail(AWQ_ERR_SHAPE, "awq_gather_channels: n=%lld, k=%lld out of range", n, k);
  if (!aligned(w, 2) || (w_s && !aligned(w_s, 2)) || (idx && !aligned(idx, 4)))
    return fail(AWQ_ERR_ALIGN, "awq_gather_channels: misaligned pointer");
  hipError_t e = awq::launch_gather_channels(w, n, k, idx, count, w_s, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_gather_channels launch");
  return AWQ_OK;
}

size_t awq_mixed_loss_workspace_size(int64_t n, int64_t k, int64_t m, int32_t g) {
  if (n < 1 || k < 1 || m < 1 || !group_ok(g)) return 0;
  return awq::mixed_loss_workspace_bytes(n, k, m, g);
}

awq_status awq_mixed_loss(const uint16_t* w, const uint16_t* x, const uint16_t* keep16, int64_t n,
                          int64_t k, int64_t m, int32_t g, double* loss, void* workspace,
                          size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!w || !x || !keep16 || !loss) return fail(AWQ_ERR_NULL, "awq_mixed_loss: null pointer");
  if (!group_ok(g)) return fail(AWQ_ERR_SHAPE, "awq_mixed_loss: g=%lld not in {32,64,128}", g);
  if (k < g || k % g != 0) return fail(AWQ_ERR_SHAPE, "awq_mixed_loss: k=%lld not a positive multiple of g=%lld", k, g);
  if (n < 1) return fail(AWQ_ERR_SHAPE, "awq_mixed_loss: n=%lld < 1", n);
  if (m < 1 || m > 8192) return fail(AWQ_ERR_SHAPE, "awq_mixed_loss: m=%lld outside 1..8192", m);
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(keep16, 2) || !aligned(loss, 8))
    return fail(AWQ_ERR_ALIGN, "awq_mixed_loss: w and x must be 16-byte aligned");
  const size_t need = awq::mixed_loss_workspace_bytes(n, k, m, g);
  if (!workspace || ws_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "awq_mixed_loss: workspace of %lld bytes < %lld needed", (long long)ws_bytes, (long long)need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_ALIGN, "awq_mixed_loss: workspace must be 256-byte aligned");
  hipError_t e = awq::launch_mixed_loss(w, x, keep16, n, k, m, g, loss, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_mixed_loss launch");
  return AWQ_OK;
}

awq_status awq_linear_mixed(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                            const uint32_t* qzeros, const uint16_t* keep16, const uint16_t* w_s,
                            const int32_t* idx, int32_t count, int64_t m, int64_t n, int64_t k,
                            int32_t g, uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!keep16 || ((!w_s || !idx) && count > 0)) return fail(AWQ_ERR_NULL, "awq_linear_mixed: null pointer");
  if (count < 0 || count > k || count > awq::kMixedMaxCount)
    return fail(AWQ_ERR_SHAPE, "awq_linear_mixed: count=%lld outside 0..min(k, %lld)", count, awq::kMixedMaxCount);
  if (m > (int64_t)65535 * 16) return fail(AWQ_ERR_SHAPE, "awq_linear_mixed: m=%lld too large", m);
  if (!aligned(keep16, 16) || (w_s && !aligned(w_s, 2)) || (idx && !aligned(idx, 4)))
    return fail(AWQ_ERR_ALIGN, "awq_linear_mixed: misaligned pointer (keep16 must be 16-byte aligned)");
  awq_status st = linear_impl("awq_linear_mixed", x, qweight, scales, qzeros, keep16, m, n, k, g, y, 0,
                              workspace, ws_bytes, stream);
  if (st != AWQ_OK) return st;
  hipError_t e = awq::launch_salient_add(x, idx, count, w_s, m, n, k, y, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "awq_linear_mixed launch");
  return AWQ_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- no allocation
// awq_linear_w4a16_group_noalloc: the group call with its device scratch in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate (code under graph capture, tight serving loops, harnesses
// that forbid allocation).  Each GPU the library runs on holds its own copy of
// the array until the process ends.  In host code the array's name is only a
// host-side stand-in: its device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept per device; that
// address, never the name, is what the kernels receive.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[kMaxDevices] = {};

// the device address of `scratch` on the current device
awq_status noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "awq_linear_w4a16_group_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(AWQ_ERR_UNSUPPORTED, "awq_linear_w4a16_group_noalloc: device index %lld out of range", dev);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "awq_linear_w4a16_group_noalloc: hipGetSymbolAddress");
    if (ptr == nullptr)
      return fail(AWQ_ERR_HIP, "awq_linear_w4a16_group_noalloc: no device address for the scratch array");
    g_noalloc_ptr[dev] = ptr;
  }
  *out = g_noalloc_ptr[dev];
  return AWQ_OK;
}

}  // namespace

extern "C" {

size_t awq_linear_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

awq_status awq_linear_w4a16_group_noalloc(const awq_linear_item* items, int32_t count, int64_t m,
                                          int64_t k, int32_t g, void* stream) {
  const char* fn = "awq_linear_w4a16_group_noalloc";
  g_err[0] = 0;
  if (!items) return fail(AWQ_ERR_NULL, "awq_linear_w4a16_group_noalloc: null items");
  if (count < 1 || count > awq::kGroupMax)
    return fail(AWQ_ERR_SHAPE, "awq_linear_w4a16_group_noalloc: count=%lld outside 1..%lld", count,
                awq::kGroupMax);
  awq::LinItem li[awq::kGroupMax];
  for (int32_t i = 0; i < count; ++i) {
    const awq_linear_item& it = items[i];
    awq_status st = check_linear_args(fn, it.x, it.qweight, it.scales, it.qzeros, it.inv_s16, m, it.n,
                                      k, g, it.y);
    if (st != AWQ_OK) return st;
    li[i] = awq::LinItem{it.x, it.inv_s16, it.qweight, it.scales, it.qzeros, it.y, it.n};
  }
  const size_t need = awq::linear_group_scratch_bytes(li, count, m, k, g);
  if (need > kNoallocScratchBytes)
    return fail(AWQ_ERR_WORKSPACE,
                "awq_linear_w4a16_group_noalloc: the call needs %lld scratch bytes, beyond the %lld of the "
                "static scratch (use awq_linear_w4a16_group with a workspace)",
                (long long)need, (long long)kNoallocScratchBytes);
  void* ptr = nullptr;
  awq_status st = noalloc_scratch(&ptr);
  if (st != AWQ_OK) return st;
  awq::Scratch scr;
  scr.base = static_cast<char*>(ptr);
  hipError_t e = awq::launch_linear_group(li, count, m, k, g, scr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return AWQ_OK;
}

}  // extern "C"
