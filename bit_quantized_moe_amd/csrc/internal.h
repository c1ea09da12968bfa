// Host-side launchers of the MoE kernels.  Each returns the hipError_t of its
// launch; argument checking happens in api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bqmoe {

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
};

// Properties of the current device (cached per device, thread-safe).
hipError_t current_device_info(DeviceInfo *out);

// Polling rounds after which a bounded cross-block wait gives up and raises
// the workspace's sticky error flag (kDefaultWaitSpins unless a test lowered
// it through moe_set_wait_limit).
constexpr int kDefaultWaitSpins = 1 << 22;
int wait_spin_limit();

// route.hip
constexpr int kRouteSmallT = 256;  // T at or below: one block per expert (tagged logits) + selector blocks (measured faster than the token-tiled kernel up to T = 256 at H = 4096, E = 256)
size_t route_workspace_bytes(int T, int E);
hipError_t launch_route(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                        int k, int32_t *ids, float *gates, float *logits, void *ws, hipStream_t st);
// Router launch that also groups the rows by expert (the outputs of
// launch_permute), for shapes where route_groups_rows(T, k) holds.
bool route_groups_rows(int T, int k);
hipError_t launch_route_group(const uint16_t *x, const uint16_t *w_router, const float *bias, int T, int H, int E,
                              int k, int32_t *ids, float *gates, float *logits, int32_t *offsets,
                              int32_t *sorted_rows, int32_t *row_pos, int32_t *active, void *ws, hipStream_t st);

// permute.hip
size_t permute_workspace_bytes(int T, int k, int E);
hipError_t launch_permute(const int32_t *ids, int T, int k, int E, int32_t *offsets, int32_t *sorted_rows,
                          int32_t *row_pos, int32_t *active, void *ws, hipStream_t st);

// ffn_decode.hip / ffn_prefill.hip
// Expert FFN dispatch: the decode path (weights streamed once per expert,
// rows in passes of four) while the rows per expert stay few, the grouped
// MFMA GEMMs above.  Measured at H = 4096, I = 1024, E = 256, top-8 (INT4):
// the decode path is faster up to T = 192 (6 rows per expert when every
// expert is active) and even at T = 256.
constexpr int kDecodeMaxT = 512;       // never the decode path above this T
constexpr int kDecodeRowsPerExpert = 6;
inline bool decode_path(int T, int k, int E) {
  return T <= kDecodeMaxT && (long)T * k <= (long)kDecodeRowsPerExpert * E;
}
constexpr int kLayerMaxT = 16;  // the one-launch decode layer
size_t ffn_workspace_bytes(int T, int k, int E, int H, int I);
size_t ffn_ctl_bytes(int T, int k, int E);  // control block at the start of the FFN workspace (x256)
bool decode_layout_ok(int H, int I, int bits, int group = 128);

struct FfnArgs {
  const uint16_t *x;
  const int32_t *offsets;
  const int32_t *sorted_rows;
  const int32_t *active;
  int T, k, E, H, I, bits;
  const uint32_t *w13_codes;
  const uint16_t *w13_scales;
  const uint8_t *w13_zeros;
  const uint32_t *w2_codes;
  const uint16_t *w2_scales;
  const uint8_t *w2_zeros;
  uint16_t *y_perm;
  void *ws;
  // optional per-expert address table (device memory, kTabStride uint64 per
  // expert: w13 codes, w13 scales, w13 zeros, w2 codes, w2 scales, w2 zeros,
  // each the expert's own block); when set the array pointers are unused
  const uint64_t *tab = nullptr;
  // quantisation group along K: 128, or 32 for the INT4 / INT8 group-32 formats
  int group = 128;
  // NVFP4 W4A4 (bits 4, E2M1 codes, E4M3 scales per 16 K in the scale arrays):
  // per-expert float32 weight tensor scales and the activation / h tensor scales
  bool nvfp4 = false;
  const float *w13_g = nullptr, *w2_g = nullptr;
  float gx = 0.f, gh = 0.f;
};
constexpr int kTabStride = 6;
hipError_t launch_ffn_decode(const FfnArgs &a, const DeviceInfo &dev, hipStream_t st);

// Fused decode layer (ffn_decode.hip): router, grouping, expert FFN and combine in one launch.
struct LayerArgs {
  const uint16_t *w_router;
  const float *bias;
  uint16_t *y;
  int32_t *ids;    // optional outputs
  float *gates;
  float *logits;
};
bool layer_shape_ok(int T, int k, int E, int H, int I, int bits, int group = 128);
size_t layer_workspace_bytes(int T, int k, int E, int H, int I);
hipError_t launch_layer_decode(const FfnArgs &a, const LayerArgs &l, const DeviceInfo &dev, hipStream_t st);
hipError_t launch_ffn_prefill(const FfnArgs &a, const DeviceInfo &dev, hipStream_t st);

// ffn_mid.hip: the middle-batch expert FFN (two launches, rows staged per
// K step, weights read once per 32 rows of an expert) between the decode
// path and the grouped GEMMs: INT4 and 2-bit with groups of 128, while an
// active expert averages at most kMidRowsPerExpert rows.
constexpr int kMidRowsPerExpert = 24;
inline bool mid_path(int T, int k, int E) {
  return !decode_path(T, k, E) && (long)T * k <= (long)kMidRowsPerExpert * E;
}
bool mid_layout_ok(int H, int I, int bits, int group);
hipError_t launch_ffn_mid(const FfnArgs &a, hipStream_t st);
// One of the mid path's two launches (gate_up into hbuf, or down from it)
// for the experts with at most max_rows rows; the grouped-GEMM path uses it
// for its small experts.
hipError_t launch_mid_gemm(const FfnArgs &a, uint16_t *hbuf, int max_rows, bool gate_up, hipStream_t st);

// combine.hip
hipError_t launch_combine(const uint16_t *y_perm, const int32_t *row_pos, const float *gates, int T, int k,
                          int H, uint16_t *y, hipStream_t st);

// unpack.hip
hipError_t launch_unpack(const uint32_t *words, int bits, int64_t n_words, int8_t *out, hipStream_t st);
hipError_t launch_zero16(void *p, size_t bytes, hipStream_t st);  // bytes % 16 == 0, 16-byte aligned
hipError_t launch_quant_nvfp4(const uint16_t *x, int64_t n, float G, uint16_t *vals, uint8_t *scales, hipStream_t st);
hipError_t launch_dequant_bf16(const uint32_t *words, const uint16_t *scales, const uint8_t *zeros, int bits,
                               int group, int N, int K, uint16_t *out, hipStream_t st);

// probe.hip: the achievable HBM read rate and bf16 MFMA rate of the device
size_t probe_stream_blocks(size_t bytes);  // blocks (and words of out) of one stream probe launch
hipError_t launch_probe_stream(const void *buf, size_t bytes, uint32_t *out, hipStream_t st);
hipError_t launch_probe_mfma(int blocks, int iters, float *out, hipStream_t st);

}  // namespace bqmoe
