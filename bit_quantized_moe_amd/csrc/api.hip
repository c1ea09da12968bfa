// C ABI of the MoE library: host-side argument checks, workspace sizing,
// dispatch to the kernel launchers and error reporting.  Nothing here touches
// the GPU before every argument of a call has been checked.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "bqmoe.h"
#include "common.cuh"
#include "internal.h"

using namespace bqmoe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status from_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kMaxDevices = 64;
std::mutex g_dev_mu;
DeviceInfo g_dev[kMaxDevices];
bool g_dev_ok[kMaxDevices];

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

std::atomic<int> g_wait_spins{kDefaultWaitSpins};

// ---- workspace of moe_layer_w4a16_noalloc: a file-scope device array.
// Each device the library runs on holds its own copy (reserved when the code
// object is loaded, kept until the process ends).  In host code the name
// `scratch` is only a host-side stand-in for the symbol, not a device
// address: host code uses the address hipGetSymbolAddress returns for the
// current device, looked up once per device on the first call there.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

moe_status check_common_moe(int T, int H, int E, int k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E must be in [1, 1024] (got %d)", E);
  if (k < 1 || k > 32 || k > E) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, min(E, 32)] (got k=%d, E=%d)", k, E);
  if (H < 128 || H % 128) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 (got %d)", H);
  if ((long long)T * k > (1LL << 24)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*k must be <= 2^24");
  return MOE_OK;
}

}  // namespace

namespace bqmoe {

int wait_spin_limit() { return g_wait_spins.load(std::memory_order_relaxed); }

hipError_t current_device_info(DeviceInfo *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_ok[dev]) {
    DeviceInfo d;
    d.device = dev;
    e = hipDeviceGetAttribute(&d.num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_dev[dev] = d;
    g_dev_ok[dev] = true;
  }
  *out = g_dev[dev];
  return hipSuccess;
}

// NVFP4: control block, h (tagged 32-bit words on the decode path, bf16 on
// the grouped GEMMs), then the quantised activations (bf16)
static size_t ffn_nvfp4_h_bytes(int T, int k, int E, int I) {
  return (size_t)T * k * I * (decode_path(T, k, E) ? sizeof(uint32_t) : sizeof(uint16_t));
}
static size_t ffn_nvfp4_workspace_bytes(int T, int k, int E, int H, int I) {
  return round_up(ffn_ctl_bytes(T, k, E) + ffn_nvfp4_h_bytes(T, k, E, I) + (size_t)T * H * sizeof(uint16_t), 256);
}

size_t ffn_workspace_bytes(int T, int k, int E, int H, int I) {
  (void)E;
  (void)H;
  // h: 32-bit tagged words on the decode path, bf16 on the grouped-GEMM path
  const size_t h_elem = decode_path(T, k, E) ? sizeof(uint32_t) : sizeof(uint16_t);
  return round_up(ffn_ctl_bytes(T, k, E) + (size_t)T * k * I * h_elem, 256);
}

}  // namespace bqmoe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *moe_last_error(void) { return g_err; }

moe_status moe_workspace_status(void *workspace, size_t workspace_bytes, int clear, uint32_t *flags, void *stream) {
  if (!workspace || !flags) return fail(MOE_ERR_INVALID_ARG, "moe_workspace_status: workspace and flags are required");
  if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "moe_workspace_status: workspace needs 256-byte alignment");
  if (workspace_bytes < kCtlBytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_workspace_status: %zu bytes hold no control block (%zu)",
                workspace_bytes, (size_t)kCtlBytes);
  const hipStream_t st = (hipStream_t)stream;
  int *ctl = (int *)workspace;
  int host = 0;
  hipError_t e = hipMemcpyAsync(&host, ctl + kCtlError, sizeof host, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return from_hip(e, "moe_workspace_status");
  *flags = (uint32_t)host;
  // words 0..3 of the control block hold only the flags word
  if (clear && host) return from_hip(launch_zero16(ctl, 16, st), "moe_workspace_status clear");
  return MOE_OK;
}

int moe_set_wait_limit(int spins) {
  const int prev = g_wait_spins.load();
  g_wait_spins.store(spins < 0 ? kDefaultWaitSpins : spins);
  return prev;
}

size_t moe_route_workspace_size(int T, int E) {
  if (T < 0 || E < 1) return 0;
  return round_up(route_workspace_bytes(T, E), 256);
}

moe_status moe_route(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H, int E,
                     int k, int32_t *topk_ids, float *topk_weights, float *logits, void *workspace,
                     size_t workspace_bytes, void *stream) {
  moe_status s = check_common_moe(T, H, E, k);
  if (s != MOE_OK) return s;
  if (!x || !w_router || !topk_ids || !topk_weights || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: x, w_router, topk_ids, topk_weights and workspace are required");
  if (!aligned(x, 16) || !aligned(w_router, 16)) return fail(MOE_ERR_MISALIGNED, "moe_route: x and w_router need 16-byte alignment");
  if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "moe_route: workspace needs 256-byte alignment");
  if (!aligned(topk_ids, 4) || !aligned(topk_weights, 4) || (logits && !aligned(logits, 4)) ||
      (logit_bias && !aligned(logit_bias, 4)))
    return fail(MOE_ERR_MISALIGNED, "moe_route: 4-byte arrays must be 4-byte aligned");
  if (workspace_bytes < moe_route_workspace_size(T, E))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_route: workspace %zu < %zu bytes", workspace_bytes,
                moe_route_workspace_size(T, E));
  if (T == 0) return MOE_OK;
  return from_hip(launch_route(x, w_router, logit_bias, T, H, E, k, topk_ids, topk_weights, logits, workspace,
                               (hipStream_t)stream),
                  "moe_route launch");
}

size_t moe_permute_workspace_size(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return permute_workspace_bytes(T, k, E);
}

moe_status moe_permute(const int32_t *topk_ids, int T, int k, int E, int32_t *expert_offsets, int32_t *sorted_rows,
                       int32_t *row_pos, int32_t *active, void *workspace, size_t workspace_bytes, void *stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E must be in [1, 1024] (got %d)", E);
  if (k < 1 || k > 32) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, 32] (got %d)", k);
  if ((long long)T * k > (1LL << 24)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*k must be <= 2^24");
  if (!topk_ids || !expert_offsets || !sorted_rows || !row_pos || !active)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: all arrays are required");
  if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_rows, 4) || !aligned(row_pos, 4) ||
      !aligned(active, 4))
    return fail(MOE_ERR_MISALIGNED, "moe_permute: int32 arrays must be 4-byte aligned");
  const size_t need = moe_permute_workspace_size(T, k, E);
  if (need && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_permute: workspace %zu < %zu bytes", workspace_bytes, need);
  if (need && !aligned(workspace, 256))
    return fail(MOE_ERR_MISALIGNED, "moe_permute: workspace needs 256-byte alignment");
  if (T == 0) return MOE_OK;
  return from_hip(launch_permute(topk_ids, T, k, E, expert_offsets, sorted_rows, row_pos, active, workspace,
                                 (hipStream_t)stream),
                  "moe_permute launch");
}

size_t moe_route_permute_workspace_size(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const size_t r = moe_route_workspace_size(T, E), p = round_up(permute_workspace_bytes(T, k, E), 256);
  return r > p ? r : p;
}

moe_status moe_route_permute(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H,
                             int E, int k, int32_t *topk_ids, float *topk_weights, float *logits,
                             int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos, int32_t *active,
                             void *workspace, size_t workspace_bytes, void *stream) {
  moe_status s = check_common_moe(T, H, E, k);
  if (s != MOE_OK) return s;
  if (!x || !w_router || !topk_ids || !topk_weights || !workspace || !expert_offsets || !sorted_rows || !row_pos ||
      !active)
    return fail(MOE_ERR_INVALID_ARG, "moe_route_permute: a required pointer is NULL");
  if (!aligned(x, 16) || !aligned(w_router, 16))
    return fail(MOE_ERR_MISALIGNED, "moe_route_permute: x and w_router need 16-byte alignment");
  if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "moe_route_permute: workspace needs 256-byte alignment");
  if (!aligned(topk_ids, 4) || !aligned(topk_weights, 4) || (logits && !aligned(logits, 4)) ||
      (logit_bias && !aligned(logit_bias, 4)) || !aligned(expert_offsets, 4) || !aligned(sorted_rows, 4) ||
      !aligned(row_pos, 4) || !aligned(active, 4))
    return fail(MOE_ERR_MISALIGNED, "moe_route_permute: 4-byte arrays must be 4-byte aligned");
  const size_t need = moe_route_permute_workspace_size(T, k, E);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "moe_route_permute: workspace %zu < %zu bytes", workspace_bytes, need);
  if (T == 0) return MOE_OK;
  const hipStream_t st = (hipStream_t)stream;
  if (route_groups_rows(T, k))
    return from_hip(launch_route_group(x, w_router, logit_bias, T, H, E, k, topk_ids, topk_weights, logits,
                                       expert_offsets, sorted_rows, row_pos, active, workspace, st),
                    "moe_route_permute launch");
  hipError_t e = launch_route(x, w_router, logit_bias, T, H, E, k, topk_ids, topk_weights, logits, workspace, st);
  if (e != hipSuccess) return from_hip(e, "moe_route_permute: route launch");
  return from_hip(launch_permute(topk_ids, T, k, E, expert_offsets, sorted_rows, row_pos, active, workspace, st),
                  "moe_route_permute: permute launch");
}

size_t moe_expert_ffn_workspace_size(int T, int k, int E, int H, int I) {
  if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return 0;
  return ffn_workspace_bytes(T, k, E, H, I);
}

// The integer-code and FP6 formats of the wna16 calls: INT4 and INT8 with
// groups of 128 or 32, 2-bit and FP6 with groups of 128.
static bool wna16_format_ok(int bits, int group) {
  return ((bits == 4 || bits == 8) && (group == 128 || group == 32)) || ((bits == 2 || bits == 6) && group == 128);
}

// The expert-FFN path of a shape and format (MOE_FFN_PATH_*); group 16 with
// 4 bits is NVFP4, whose decode kernel reads 128-K units of E4M3 pairs.
static int ffn_path_of(int T, int k, int E, int H, int I, int bits, int group) {
  const bool nv = bits == 4 && group == 16;
  if (decode_path(T, k, E) && decode_layout_ok(H, I, bits, nv ? 32 : group)) return MOE_FFN_PATH_DECODE;
  if (!nv && mid_path(T, k, E) && mid_layout_ok(H, I, bits, group)) return MOE_FFN_PATH_MID;
  return MOE_FFN_PATH_GEMM;
}

static moe_status expert_ffn(const char *name, int bits, const uint16_t *x, const int32_t *expert_offsets,
                             const int32_t *sorted_rows, const int32_t *active, int T, int k, int E, int H, int I,
                             const uint32_t *w13_codes, const uint16_t *w13_scales, const uint8_t *w13_zeros,
                             const uint32_t *w2_codes, const uint16_t *w2_scales, const uint8_t *w2_zeros,
                             uint16_t *y_perm, void *workspace, size_t workspace_bytes, void *stream,
                             const uint64_t *table = nullptr, int group = 128) {
  moe_status s = check_common_moe(T, H, E, k);
  if (s != MOE_OK) return s;
  if (I < 128 || I % 128) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: I must be a positive multiple of 128 (got %d)", name, I);
  if (!x || !expert_offsets || !sorted_rows || !active || !y_perm || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
  if (table) {
    if (!aligned(table, 8)) return fail(MOE_ERR_MISALIGNED, "%s: the expert table needs 8-byte alignment", name);
  } else {
    if (!w13_codes || !w13_scales || !w2_codes || !w2_scales)
      return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
    if (bits == 2 && (!w13_zeros || !w2_zeros)) return fail(MOE_ERR_INVALID_ARG, "%s: zero-points are required", name);
    if (!aligned(w13_codes, 16) || !aligned(w2_codes, 16) || !aligned(w13_scales, 2) || !aligned(w2_scales, 2))
      return fail(MOE_ERR_MISALIGNED, "%s: code arrays need 16-byte and scale arrays 2-byte alignment", name);
  }
  if (!aligned(x, 16)) return fail(MOE_ERR_MISALIGNED, "%s: x needs 16-byte alignment", name);
  if (!aligned(y_perm, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_rows, 4) || !aligned(active, 4))
    return fail(MOE_ERR_MISALIGNED, "%s: array alignment", name);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "%s: workspace needs 256-byte alignment", name);
  const size_t need = moe_expert_ffn_workspace_size(T, k, E, H, I);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", name, workspace_bytes, need);
  if (T == 0) return MOE_OK;
  DeviceInfo dev;
  hipError_t he = current_device_info(&dev);
  if (he != hipSuccess) return from_hip(he, name);
  FfnArgs a{x, expert_offsets, sorted_rows, active, T, k, E, H, I, bits, w13_codes, w13_scales, w13_zeros,
            w2_codes, w2_scales, w2_zeros, y_perm, workspace, table, group};
  const int path = ffn_path_of(T, k, E, H, I, bits, group);
  if (path == MOE_FFN_PATH_DECODE) return from_hip(launch_ffn_decode(a, dev, (hipStream_t)stream), name);
  // the grouped GEMMs and the middle-batch kernel address x and one expert's
  // codes with 32-bit offsets
  if ((long long)T * H > (1LL << 30) || (long long)I * H > (1LL << 30))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: T*H and I*H must be <= 2^30 on the grouped-GEMM path (T=%d)", name, T);
  if (path == MOE_FFN_PATH_MID) return from_hip(launch_ffn_mid(a, (hipStream_t)stream), name);
  return from_hip(launch_ffn_prefill(a, dev, (hipStream_t)stream), name);
}

moe_status moe_expert_ffn_w4a16(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                const int32_t *active, int T, int k, int E, int H, int I, const uint32_t *w13_codes,
                                const uint16_t *w13_scales, const uint32_t *w2_codes, const uint16_t *w2_scales,
                                uint16_t *y_perm, void *workspace, size_t workspace_bytes, void *stream) {
  return expert_ffn("moe_expert_ffn_w4a16", 4, x, expert_offsets, sorted_rows, active, T, k, E, H, I, w13_codes,
                    w13_scales, nullptr, w2_codes, w2_scales, nullptr, y_perm, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_w2a16(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                const int32_t *active, int T, int k, int E, int H, int I, const uint32_t *w13_codes,
                                const uint16_t *w13_scales, const uint8_t *w13_zeros, const uint32_t *w2_codes,
                                const uint16_t *w2_scales, const uint8_t *w2_zeros, uint16_t *y_perm,
                                void *workspace, size_t workspace_bytes, void *stream) {
  return expert_ffn("moe_expert_ffn_w2a16", 2, x, expert_offsets, sorted_rows, active, T, k, E, H, I, w13_codes,
                    w13_scales, w13_zeros, w2_codes, w2_scales, w2_zeros, y_perm, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_wna16(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                const int32_t *active, int T, int k, int E, int H, int I, int bits, int group_size,
                                const uint32_t *w13_codes, const uint16_t *w13_scales, const uint8_t *w13_zeros,
                                const uint32_t *w2_codes, const uint16_t *w2_scales, const uint8_t *w2_zeros,
                                uint16_t *y_perm, void *workspace, size_t workspace_bytes, void *stream) {
  if (!wna16_format_ok(bits, group_size))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_wna16: unsupported format: %d bits, group %d", bits, group_size);
  return expert_ffn("moe_expert_ffn_wna16", bits, x, expert_offsets, sorted_rows, active, T, k, E, H, I, w13_codes,
                    w13_scales, bits == 2 ? w13_zeros : nullptr, w2_codes, w2_scales, bits == 2 ? w2_zeros : nullptr,
                    y_perm, workspace, workspace_bytes, stream, nullptr, group_size);
}

moe_status moe_expert_ffn_wna16_table(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                      const int32_t *active, int T, int k, int E, int H, int I, int bits,
                                      int group_size, const uint64_t *expert_table, uint16_t *y_perm,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  if (!wna16_format_ok(bits, group_size))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_wna16_table: unsupported format: %d bits, group %d", bits,
                group_size);
  if (!expert_table) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_wna16_table: expert_table is NULL");
  return expert_ffn("moe_expert_ffn_wna16_table", bits, x, expert_offsets, sorted_rows, active, T, k, E, H, I,
                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, y_perm, workspace, workspace_bytes, stream,
                    expert_table, group_size);
}

int moe_expert_ffn_path(int T, int k, int E, int H, int I, int bits, int group_size) {
  if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return -1;
  const bool nv = bits == 4 && group_size == 16;
  if (!nv && !wna16_format_ok(bits, group_size)) return -1;
  return ffn_path_of(T, k, E, H, I, bits, group_size);
}

size_t moe_expert_ffn_nvfp4_workspace_size(int T, int k, int E, int H, int I) {
  if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return 0;
  return ffn_nvfp4_workspace_bytes(T, k, E, H, I);
}

static moe_status expert_ffn_nvfp4(const char *name, const uint16_t *x, const int32_t *expert_offsets,
                                   const int32_t *sorted_rows, const int32_t *active, int T, int k, int E, int H,
                                   int I, float x_gscale, float h_gscale, const uint32_t *w13_codes,
                                   const uint8_t *w13_scales, const float *w13_gscale, const uint32_t *w2_codes,
                                   const uint8_t *w2_scales, const float *w2_gscale, uint16_t *y_perm,
                                   void *workspace, size_t workspace_bytes, void *stream,
                                   const uint64_t *table = nullptr) {
  moe_status s = check_common_moe(T, H, E, k);
  if (s != MOE_OK) return s;
  if (I < 128 || I % 128) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: I must be a positive multiple of 128 (got %d)", name, I);
  if (!x || !expert_offsets || !sorted_rows || !active || !y_perm || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
  if (table) {
    if (!aligned(table, 8)) return fail(MOE_ERR_MISALIGNED, "%s: the expert table needs 8-byte alignment", name);
  } else {
    if (!w13_codes || !w13_scales || !w13_gscale || !w2_codes || !w2_scales || !w2_gscale)
      return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
    if (!aligned(w13_codes, 16) || !aligned(w2_codes, 16) || !aligned(w13_scales, 2) || !aligned(w2_scales, 2) ||
        !aligned(w13_gscale, 4) || !aligned(w2_gscale, 4))
      return fail(MOE_ERR_MISALIGNED, "%s: code arrays need 16-byte, scale arrays 2-byte and tensor-scale arrays "
                  "4-byte alignment", name);
  }
  if (!(x_gscale > 0.f) || !(h_gscale > 0.f) || x_gscale > 3.0e38f || h_gscale > 3.0e38f)
    return fail(MOE_ERR_INVALID_ARG, "%s: the tensor scales must be positive and finite", name);
  if (!aligned(x, 16)) return fail(MOE_ERR_MISALIGNED, "%s: x needs 16-byte alignment", name);
  if (!aligned(y_perm, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_rows, 4) || !aligned(active, 4))
    return fail(MOE_ERR_MISALIGNED, "%s: array alignment", name);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "%s: workspace needs 256-byte alignment", name);
  const size_t need = ffn_nvfp4_workspace_bytes(T, k, E, H, I);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", name, workspace_bytes, need);
  if (T == 0) return MOE_OK;
  if ((long long)T * H > (1LL << 30) || (long long)I * H > (1LL << 30))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: T*H and I*H must be <= 2^30 (T=%d)", name, T);
  DeviceInfo dev;
  hipError_t he = current_device_info(&dev);
  if (he != hipSuccess) return from_hip(he, name);
  FfnArgs a{x, expert_offsets, sorted_rows, active, T, k, E, H, I, 4, w13_codes, (const uint16_t *)w13_scales, nullptr,
            w2_codes, (const uint16_t *)w2_scales, nullptr, y_perm, workspace, table, 16};
  a.nvfp4 = true;
  a.w13_g = w13_gscale;
  a.w2_g = w2_gscale;
  a.gx = x_gscale;
  a.gh = h_gscale;
  const hipStream_t st = (hipStream_t)stream;
  if (ffn_path_of(T, k, E, H, I, 4, 16) == MOE_FFN_PATH_DECODE) {
    // decode path: quantise x after the h words, run the GEMV kernel on it, clear it again
    uint16_t *xq = (uint16_t *)((char *)workspace + ffn_ctl_bytes(T, k, E) + ffn_nvfp4_h_bytes(T, k, E, I));
    hipError_t e = launch_quant_nvfp4(x, (int64_t)T * H, x_gscale, xq, nullptr, st);
    if (e == hipSuccess) {
      FfnArgs d = a;
      d.x = xq;
      e = launch_ffn_decode(d, dev, st);
    }
    if (e == hipSuccess) e = launch_zero16(xq, (size_t)T * H * sizeof(uint16_t), st);
    return from_hip(e, name);
  }
  return from_hip(launch_ffn_prefill(a, dev, st), name);
}

moe_status moe_expert_ffn_nvfp4(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                const int32_t *active, int T, int k, int E, int H, int I, float x_gscale,
                                float h_gscale, const uint32_t *w13_codes, const uint8_t *w13_scales,
                                const float *w13_gscale, const uint32_t *w2_codes, const uint8_t *w2_scales,
                                const float *w2_gscale, uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                void *stream) {
  return expert_ffn_nvfp4("moe_expert_ffn_nvfp4", x, expert_offsets, sorted_rows, active, T, k, E, H, I, x_gscale,
                          h_gscale, w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, y_perm,
                          workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_nvfp4_table(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                      const int32_t *active, int T, int k, int E, int H, int I, float x_gscale,
                                      float h_gscale, const uint64_t *expert_table, uint16_t *y_perm,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  if (!expert_table) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_nvfp4_table: expert_table is NULL");
  return expert_ffn_nvfp4("moe_expert_ffn_nvfp4_table", x, expert_offsets, sorted_rows, active, T, k, E, H, I,
                          x_gscale, h_gscale, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, y_perm,
                          workspace, workspace_bytes, stream, expert_table);
}

moe_status moe_quant_act_nvfp4(const uint16_t *x, int64_t n, float gscale, uint16_t *values, uint8_t *scales,
                               void *stream) {
  if (n < 0 || n % 16) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_quant_act_nvfp4: n must be a multiple of 16");
  if (!x || !values) return fail(MOE_ERR_INVALID_ARG, "moe_quant_act_nvfp4: x and values are required");
  if (!(gscale > 0.f) || gscale > 3.0e38f) return fail(MOE_ERR_INVALID_ARG, "moe_quant_act_nvfp4: bad tensor scale");
  if (!aligned(x, 16) || !aligned(values, 16)) return fail(MOE_ERR_MISALIGNED, "moe_quant_act_nvfp4: 16-byte alignment");
  if (n == 0) return MOE_OK;
  return from_hip(launch_quant_nvfp4(x, n, gscale, values, scales, (hipStream_t)stream), "moe_quant_act_nvfp4");
}

moe_status moe_expert_ffn_w4a16_table(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                      const int32_t *active, int T, int k, int E, int H, int I,
                                      const uint64_t *expert_table, uint16_t *y_perm, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (!expert_table) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_w4a16_table: expert_table is NULL");
  return expert_ffn("moe_expert_ffn_w4a16_table", 4, x, expert_offsets, sorted_rows, active, T, k, E, H, I, nullptr,
                    nullptr, nullptr, nullptr, nullptr, nullptr, y_perm, workspace, workspace_bytes, stream,
                    expert_table);
}

moe_status moe_expert_ffn_w2a16_table(const uint16_t *x, const int32_t *expert_offsets, const int32_t *sorted_rows,
                                      const int32_t *active, int T, int k, int E, int H, int I,
                                      const uint64_t *expert_table, uint16_t *y_perm, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  if (!expert_table) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_w2a16_table: expert_table is NULL");
  return expert_ffn("moe_expert_ffn_w2a16_table", 2, x, expert_offsets, sorted_rows, active, T, k, E, H, I, nullptr,
                    nullptr, nullptr, nullptr, nullptr, nullptr, y_perm, workspace, workspace_bytes, stream,
                    expert_table);
}

moe_status moe_device_address(const void *ptr, uint64_t *out) {
  if (!ptr || !out) return fail(MOE_ERR_INVALID_ARG, "moe_device_address: NULL argument");
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // an unknown pointer leaves a sticky error code behind
    return fail(MOE_ERR_INVALID_ARG, "moe_device_address: %p is not memory the HIP runtime knows (%s)", ptr,
                hipGetErrorString(e));
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = (uint64_t)(uintptr_t)ptr;
    return MOE_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer) {
    // The runtime may report the mapping of the allocation's base or of ptr
    // itself; the offset from the reported host pointer covers both.
    const char *hp = at.hostPointer ? (const char *)at.hostPointer : (const char *)ptr;
    *out = (uint64_t)(uintptr_t)((const char *)at.devicePointer + ((const char *)ptr - hp));
    return MOE_OK;
  }
  return fail(MOE_ERR_INVALID_ARG, "moe_device_address: %p is not device-readable (pageable host memory?)", ptr);
}

size_t moe_layer_workspace_size(int T, int k, int E, int H, int I) {
  if (T < 1 || k < 1 || E < 1 || H < 1 || I < 1) return 0;
  return round_up(layer_workspace_bytes(T, k, E, H, I), 256);
}

static moe_status layer(const char *name, int bits, const uint16_t *x, const uint16_t *w_router,
                        const float *logit_bias, int T, int H, int E, int k, int I, const uint32_t *w13_codes,
                        const uint16_t *w13_scales, const uint8_t *w13_zeros, const uint32_t *w2_codes,
                        const uint16_t *w2_scales, const uint8_t *w2_zeros, uint16_t *y, int32_t *topk_ids,
                        float *topk_weights, void *workspace, size_t workspace_bytes, void *stream,
                        int group = 128, bool use_scratch = false) {
  moe_status s = check_common_moe(T, H, E, k);
  if (s != MOE_OK) return s;
  if (I < 128 || I % 128) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: I must be a positive multiple of 128 (got %d)", name, I);
  if (T == 0) return MOE_OK;
  if (!layer_shape_ok(T, k, E, H, I, bits, group))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "%s: one-launch layer needs 1 <= T <= %d and a decode-path shape (T=%d, k=%d, E=%d, H=%d, I=%d); "
                "call the stages instead",
                name, kLayerMaxT, T, k, E, H, I);
  if (!x || !w_router || !w13_codes || !w13_scales || !w2_codes || !w2_scales || !y || (!workspace && !use_scratch))
    return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
  if (bits == 2 && (!w13_zeros || !w2_zeros)) return fail(MOE_ERR_INVALID_ARG, "%s: zero-points are required", name);
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(w13_codes, 16) || !aligned(w2_codes, 16))
    return fail(MOE_ERR_MISALIGNED, "%s: x, w_router and code arrays need 16-byte alignment", name);
  if (!aligned(w13_scales, 2) || !aligned(w2_scales, 2) || !aligned(y, 4) || (topk_ids && !aligned(topk_ids, 4)) ||
      (topk_weights && !aligned(topk_weights, 4)) || (logit_bias && !aligned(logit_bias, 4)))
    return fail(MOE_ERR_MISALIGNED, "%s: array alignment", name);
  const size_t need = moe_layer_workspace_size(T, k, E, H, I);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                  "%s: this shape needs %zu bytes of workspace, more than the %zu-byte scratch; call the entry point "
                  "that takes a workspace",
                  name, need, kScratchBytes);
  } else {
    if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "%s: workspace needs 256-byte alignment", name);
    if (workspace_bytes < need)
      return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", name, workspace_bytes, need);
  }
  DeviceInfo dev;
  hipError_t he = current_device_info(&dev);
  if (he != hipSuccess) return from_hip(he, name);
  if (use_scratch) {
    // The scratch keeps the previous call's contents (left zero unless a wait
    // timed out), so every call clears the region it uses before its launch;
    // with a fill kernel, not a memset, since callers may capture the call in
    // a graph.
    he = scratch_address(&workspace);
    if (he == hipSuccess) he = launch_zero16(workspace, need, (hipStream_t)stream);
    if (he != hipSuccess) return from_hip(he, name);
  }
  FfnArgs a{x, nullptr, nullptr, nullptr, T, k, E, H, I, bits, w13_codes, w13_scales, w13_zeros,
            w2_codes, w2_scales, w2_zeros, nullptr, workspace, nullptr, group};
  LayerArgs l{w_router, logit_bias, y, topk_ids, topk_weights, nullptr};
  return from_hip(launch_layer_decode(a, l, dev, (hipStream_t)stream), name);
}

moe_status moe_layer_nvfp4(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H, int E,
                           int k, int I, float x_gscale, float h_gscale, const uint32_t *w13_codes,
                           const uint8_t *w13_scales, const float *w13_gscale, const uint32_t *w2_codes,
                           const uint8_t *w2_scales, const float *w2_gscale, uint16_t *y, int32_t *topk_ids,
                           float *topk_weights, void *workspace, size_t workspace_bytes, void *stream) {
  const char *name = "moe_layer_nvfp4";
  moe_status s = check_common_moe(T, H, E, k);
  if (s != MOE_OK) return s;
  if (I < 128 || I % 128) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s: I must be a positive multiple of 128 (got %d)", name, I);
  if (T == 0) return MOE_OK;
  if (!layer_shape_ok(T, k, E, H, I, 4, 16))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                "%s: one-launch layer needs 1 <= T <= %d and a decode-path shape (T=%d, k=%d, E=%d, H=%d, I=%d); "
                "call the stages instead",
                name, kLayerMaxT, T, k, E, H, I);
  if (!x || !w_router || !w13_codes || !w13_scales || !w13_gscale || !w2_codes || !w2_scales || !w2_gscale || !y ||
      !workspace)
    return fail(MOE_ERR_INVALID_ARG, "%s: a required pointer is NULL", name);
  if (!(x_gscale > 0.f) || !(h_gscale > 0.f) || x_gscale > 3.0e38f || h_gscale > 3.0e38f)
    return fail(MOE_ERR_INVALID_ARG, "%s: the tensor scales must be positive and finite", name);
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(w13_codes, 16) || !aligned(w2_codes, 16))
    return fail(MOE_ERR_MISALIGNED, "%s: x, w_router and code arrays need 16-byte alignment", name);
  if (!aligned(w13_scales, 2) || !aligned(w2_scales, 2) || !aligned(w13_gscale, 4) || !aligned(w2_gscale, 4) ||
      !aligned(y, 4) || (topk_ids && !aligned(topk_ids, 4)) || (topk_weights && !aligned(topk_weights, 4)) ||
      (logit_bias && !aligned(logit_bias, 4)))
    return fail(MOE_ERR_MISALIGNED, "%s: array alignment", name);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_MISALIGNED, "%s: workspace needs 256-byte alignment", name);
  const size_t need = moe_layer_workspace_size(T, k, E, H, I);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu < %zu bytes", name, workspace_bytes, need);
  DeviceInfo dev;
  hipError_t he = current_device_info(&dev);
  if (he != hipSuccess) return from_hip(he, name);
  FfnArgs a{x, nullptr, nullptr, nullptr, T, k, E, H, I, 4, w13_codes, (const uint16_t *)w13_scales, nullptr,
            w2_codes, (const uint16_t *)w2_scales, nullptr, nullptr, workspace, nullptr, 16};
  a.nvfp4 = true;
  a.w13_g = w13_gscale;
  a.w2_g = w2_gscale;
  a.gx = x_gscale;
  a.gh = h_gscale;
  LayerArgs l{w_router, logit_bias, y, topk_ids, topk_weights, nullptr};
  return from_hip(launch_layer_decode(a, l, dev, (hipStream_t)stream), name);
}

moe_status moe_layer_wna16(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H, int E,
                           int k, int I, int bits, int group_size, const uint32_t *w13_codes,
                           const uint16_t *w13_scales, const uint8_t *w13_zeros, const uint32_t *w2_codes,
                           const uint16_t *w2_scales, const uint8_t *w2_zeros, uint16_t *y, int32_t *topk_ids,
                           float *topk_weights, void *workspace, size_t workspace_bytes, void *stream) {
  if (!wna16_format_ok(bits, group_size))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_wna16: unsupported format: %d bits, group %d", bits, group_size);
  return layer("moe_layer_wna16", bits, x, w_router, logit_bias, T, H, E, k, I, w13_codes, w13_scales,
               bits == 2 ? w13_zeros : nullptr, w2_codes, w2_scales, bits == 2 ? w2_zeros : nullptr, y, topk_ids,
               topk_weights, workspace, workspace_bytes, stream, group_size);
}

moe_status moe_layer_w4a16(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H, int E,
                           int k, int I, const uint32_t *w13_codes, const uint16_t *w13_scales,
                           const uint32_t *w2_codes, const uint16_t *w2_scales, uint16_t *y, int32_t *topk_ids,
                           float *topk_weights, void *workspace, size_t workspace_bytes, void *stream) {
  return layer("moe_layer_w4a16", 4, x, w_router, logit_bias, T, H, E, k, I, w13_codes, w13_scales, nullptr,
               w2_codes, w2_scales, nullptr, y, topk_ids, topk_weights, workspace, workspace_bytes, stream);
}

moe_status moe_layer_w4a16_noalloc(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H,
                                   int E, int k, int I, const uint32_t *w13_codes, const uint16_t *w13_scales,
                                   const uint32_t *w2_codes, const uint16_t *w2_scales, uint16_t *y,
                                   int32_t *topk_ids, float *topk_weights, void *stream) {
  return layer("moe_layer_w4a16_noalloc", 4, x, w_router, logit_bias, T, H, E, k, I, w13_codes, w13_scales, nullptr,
               w2_codes, w2_scales, nullptr, y, topk_ids, topk_weights, nullptr, 0, stream, 128, true);
}

moe_status moe_layer_w2a16(const uint16_t *x, const uint16_t *w_router, const float *logit_bias, int T, int H, int E,
                           int k, int I, const uint32_t *w13_codes, const uint16_t *w13_scales,
                           const uint8_t *w13_zeros, const uint32_t *w2_codes, const uint16_t *w2_scales,
                           const uint8_t *w2_zeros, uint16_t *y, int32_t *topk_ids, float *topk_weights,
                           void *workspace, size_t workspace_bytes, void *stream) {
  return layer("moe_layer_w2a16", 2, x, w_router, logit_bias, T, H, E, k, I, w13_codes, w13_scales, w13_zeros,
               w2_codes, w2_scales, w2_zeros, y, topk_ids, topk_weights, workspace, workspace_bytes, stream);
}

moe_status moe_combine(const uint16_t *y_perm, const int32_t *row_pos, const float *topk_weights, int T, int k, int H,
                       uint16_t *y, void *stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  if (k < 1 || k > 32) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, 32] (got %d)", k);
  if (H < 8 || H % 8) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "moe_combine: H must be a positive multiple of 8");
  if (!y_perm || !row_pos || !topk_weights || !y) return fail(MOE_ERR_INVALID_ARG, "moe_combine: all arrays are required");
  if (!aligned(y_perm, 16) || !aligned(y, 16) || !aligned(row_pos, 4) || !aligned(topk_weights, 4))
    return fail(MOE_ERR_MISALIGNED, "moe_combine: y_perm and y need 16-byte alignment");
  if ((long long)T * k > (1LL << 24)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*k must be <= 2^24");
  if (T == 0) return MOE_OK;
  return from_hip(launch_combine(y_perm, row_pos, topk_weights, T, k, H, y, (hipStream_t)stream), "moe_combine launch");
}

moe_status moe_unpack_codes(const uint32_t *words, int bits, int64_t n_words, int8_t *out, void *stream) {
  if (bits != 2 && bits != 4 && bits != 6 && bits != 8)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "bits must be 2, 4, 6 or 8 (got %d)", bits);
  if (n_words < 0) return fail(MOE_ERR_INVALID_ARG, "n_words must be >= 0");
  if (bits == 6 && n_words % 6)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "FP6: n_words must be a multiple of 6 (32 codes)");
  if (n_words > (1LL << 36)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "n_words too large");
  if (!words || !out) return fail(MOE_ERR_INVALID_ARG, "moe_unpack_codes: words and out are required");
  if (!aligned(words, 4)) return fail(MOE_ERR_MISALIGNED, "moe_unpack_codes: words must be 4-byte aligned");
  if (n_words == 0) return MOE_OK;
  return from_hip(launch_unpack(words, bits, n_words, out, (hipStream_t)stream), "moe_unpack_codes launch");
}

moe_status moe_dequant_bf16_grouped(const uint32_t *words, const uint16_t *scales, const uint8_t *zeros, int bits,
                                    int group_size, int N, int K, uint16_t *out, void *stream) {
  if (bits != 2 && bits != 4 && bits != 6 && bits != 8)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "bits must be 2, 4, 6 or 8 (got %d)", bits);
  if (group_size != 128 && !(group_size == 32 && (bits == 4 || bits == 8)))
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "group size 128, or 32 for INT4 / INT8 (got %d)", group_size);
  if (N < 0 || K < 0) return fail(MOE_ERR_INVALID_ARG, "N and K must be >= 0");
  if (K % 128) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K must be a multiple of 128 (got %d)", K);
  if ((long long)N * K > (1LL << 36)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "N*K too large");
  if (!words || !scales || !out || (bits == 2 && !zeros))
    return fail(MOE_ERR_INVALID_ARG, "moe_dequant_bf16: a required pointer is NULL");
  if (!aligned(words, 4) || !aligned(scales, 2) || !aligned(out, 4))
    return fail(MOE_ERR_MISALIGNED, "moe_dequant_bf16: array alignment");
  if (N == 0 || K == 0) return MOE_OK;
  return from_hip(launch_dequant_bf16(words, scales, zeros, bits, group_size, N, K, out, (hipStream_t)stream),
                  "moe_dequant_bf16 launch");
}

moe_status moe_dequant_bf16(const uint32_t *words, const uint16_t *scales, const uint8_t *zeros, int bits, int N, int K,
                            uint16_t *out, void *stream) {
  return moe_dequant_bf16_grouped(words, scales, zeros, bits, 128, N, K, out, stream);
}

size_t moe_probe_stream_blocks(size_t bytes) { return probe_stream_blocks(bytes); }

moe_status moe_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (!buf || !out) return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream_read: buf and out are required");
  if (!aligned(buf, 16) || bytes % 16) return fail(MOE_ERR_MISALIGNED, "moe_probe_stream_read: 16-byte units");
  if (probe_stream_blocks(bytes) > (1u << 31) - 1) return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream_read: too large");
  return from_hip(launch_probe_stream(buf, bytes, out, (hipStream_t)stream), "moe_probe_stream_read");
}

moe_status moe_probe_mfma(int blocks, int iters, float *out, void *stream) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_probe_mfma: out is required");
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return fail(MOE_ERR_INVALID_ARG, "moe_probe_mfma: sizes");
  return from_hip(launch_probe_mfma(blocks, iters, out, (hipStream_t)stream), "moe_probe_mfma");
}

}  // extern "C"
