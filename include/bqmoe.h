/*
 * bqmoe.h -- C ABI of the routed-expert mixture-of-experts layer with low-bit
 * (weight-only INT4 / 2-bit / INT8 / FP6) experts, for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer, per batch of T tokens with hidden size H, E experts, top-k routing
 * and expert intermediate size I:
 *
 *   moe_route       router logits, top-k experts and their softmax gates
 *   moe_permute     stable grouping of the T*k (token, slot) rows by expert
 *   moe_expert_ffn_w4a16 / _w2a16
 *                   per-expert gate_up -> SwiGLU -> down with the expert weights
 *                   dequantised on the fly from packed codes
 *   moe_expert_ffn_wna16
 *                   the same for any supported format: INT4 or INT8 with
 *                   groups of 128 or 32, 2-bit or FP6 e2m3 with groups of 128
 *   moe_expert_ffn_nvfp4 (+ moe_quant_act_nvfp4)
 *                   the same with NVFP4 W4A4 experts (activations quantised too)
 *   moe_expert_ffn_w4a16_table / _w2a16_table / _wna16_table / _nvfp4_table
 *                   the same, each expert's weights located through a
 *                   per-expert address table
 *   moe_combine     gate-weighted sum of each token's k expert outputs
 *
 * Weight formats.  INT4 symmetric with one bf16 scale per 128 consecutive K
 * (weight-only, activations stay 16-bit): page "Qwen3.8-Flash-Next on 2x RTX
 * 3090", storage-format table; page "Qwen3.8-Flash-Next on dual RTX 3090: W4A16
 * + FP8 PLE + MTP3", "Composition".  2-bit with group 128 and 16 codes per
 * 32-bit word along K: page "Qwen3.8-Flash-Next on one 24 GB GPU", "What the
 * patch does" and "Hardware and software requirements".  Field i of word kw
 * (bits [b*i, b*i+b), least significant first) holds the code of K index
 * P*kw + i, P = 32/b.  INT4 fields hold q + 8 with q in [-8, 7] and the weight
 * is q*s; 2-bit fields hold u in {0..3} and the weight is (u - z)*s with an
 * integer zero-point z per group.  Two more formats share the layout: INT4
 * symmetric with one scale per 32 K (the draft-layer experts of the same two
 * pages' format tables), and INT8 symmetric, fields q + 128 with q in
 * [-127, 127], group 128 or 32 (page "Qwen3.8-Flash-Next on one 24 GB GPU",
 * "What the patch does": INT8 g128; page "Qwen3.8-Flash-Next FP6-INT8",
 * "Precision map" and "Kernel-level verification": an int8 g32 tier).  FP6
 * e2m3 codes with fp16 scales (same page, opening paragraph and
 * "Kernel-level verification"): a row's codes form one little-endian bit
 * stream, code k in bits [6k, 6k+6) (16 codes per 3 words); bit 5 is the
 * sign, bits 4..3 the exponent e (bias 1), bits 2..0 the mantissa m; the
 * value is m/8 for e = 0 and 2^(e-1) * (1 + m/8) otherwise; W = value * s
 * with one fp16 scale per 128 K.
 *
 * Conventions shared by every entry point:
 *  - Every array argument is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or retains memory and never synchronises.
 *  - Arrays are row-major and contiguous.  bf16 values are passed as uint16_t
 *    holding the bfloat16 bit pattern.
 *  - Each call checks its arguments on the host first; on any error it returns
 *    a status != MOE_OK, enqueues nothing and moe_last_error() describes the
 *    problem.  Otherwise it enqueues its kernels on `stream` (a hipStream_t
 *    passed as void*; NULL = the default stream) and returns MOE_OK without
 *    waiting.  A failed kernel launch returns MOE_ERR_HIP.
 *  - T = 0 is a valid empty batch: the call checks its arguments and enqueues
 *    nothing.
 *  - Results are bitwise deterministic for given inputs on a given device.
 *  - Workspaces: device memory of at least the size returned by the matching
 *    *_workspace_size() function, 256-byte aligned.  A workspace must be
 *    all-zero before the first call that uses it (allocate it zeroed); every
 *    call leaves it all-zero again, because kernels tell values written in
 *    this call from unwritten ones by a nonzero tag.  Two calls that overlap
 *    in time must not share a workspace.  After a call that reported an
 *    error, zero the workspace again.
 *  - Entry points are thread-safe; the only library state is a per-device
 *    cache of device properties and a thread-local error string.
 */
#ifndef BQMOE_H
#define BQMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,         /* null pointer, negative size, k outside [1, min(E, 32)] ... */
    MOE_ERR_UNSUPPORTED_SHAPE = 2,   /* H or I not a multiple of 128, E > 1024, ... */
    MOE_ERR_MISALIGNED = 3,          /* a pointer lacks the alignment its loads need */
    MOE_ERR_WORKSPACE_TOO_SMALL = 4,
    MOE_ERR_HIP = 5                  /* a HIP runtime call or kernel launch failed */
} moe_status;

/* Library ABI version (MOE_ABI_VERSION at build time). */
int moe_abi_version(void);

/* Static text for a status code. */
const char *moe_status_string(int status);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *moe_last_error(void);

/* ---------------------------------------------------------------- workspace status
 * Kernels that hand values from one block to another (the decode-path expert
 * FFN, the one-launch layer, the small-batch router) wait for them in bounded
 * polling loops.  Those kernels size their grids so that every block is
 * resident at once (from the device's occupancy), so in a lone launch every
 * wait ends.  A kernel of another stream or process that holds compute units
 * at the same time can keep some blocks from starting; a wait then gives up
 * after moe_set_wait_limit rounds (several seconds by default), the kernel
 * finishes with unreliable outputs and sets a sticky flag in the control
 * block at the start of the workspace, and the workspace may keep nonzero
 * words.  Concurrent launches of these kernels on one device are therefore
 * not supported.
 *
 * moe_workspace_status: reads the flags of a workspace of moe_route,
 * moe_route_permute, moe_expert_ffn_* or moe_layer_* (each starts with the
 * control block) once the calls that used it have finished.  It enqueues a
 * 4-byte copy on `stream` and waits for the stream: the one entry point that
 * synchronises.  flags (out): 0, or MOE_WS_WAIT_TIMEOUT when some wait gave
 * up; the outputs of the calls since the flags were last cleared are then
 * unreliable and the workspace must be zeroed before it is used again.
 * clear != 0 resets the flags (enqueued on `stream`).  workspace: 256-byte
 * aligned, workspace_bytes >= 4096.
 */
#define MOE_WS_WAIT_TIMEOUT 1u
moe_status moe_workspace_status(void *workspace, size_t workspace_bytes, int clear, uint32_t *flags, void *stream);

/* moe_set_wait_limit: polling rounds after which the bounded waits above give
 * up, for launches made after the call (process-wide; spins < 0 restores the
 * default of 4194304).  Returns the previous limit.  A test hook: a small
 * limit forces the timeout path (outputs unreliable, MOE_WS_WAIT_TIMEOUT set,
 * every kernel still ends normally). */
int moe_set_wait_limit(int spins);

/* ---------------------------------------------------------------- routing
 * moe_route: logits l[t,e] = sum_h x[t,h] * w_router[e,h] (+ logit_bias[e]),
 * then the k largest logits of each token, listed in order (logit descending,
 * expert index ascending on ties), and their softmax gates.  The pages keep
 * the router in 16-bit precision because a small logit perturbation changes
 * routing on near-ties (page "Qwen3.8-Flash-Next FP6-INT8", "Precision map");
 * to make the selection reproducible the float32 additions follow one fixed
 * order: h is split into 64 contiguous slices of H/64 elements, each slice is
 * summed in ascending h starting from 0, the 64 slice sums are added as a
 * balanced pairwise tree in index order, then the bias is added.
 *
 *   x           [T, H] bf16, 16-byte aligned
 *   w_router    [E, H] bf16, 16-byte aligned
 *   logit_bias  [E] float32, or NULL for none (e.g. a log-prior over experts)
 *   topk_ids    [T, k] int32 out
 *   topk_weights[T, k] float32 out: exp(l_j - l_max) / sum over the k selected
 *   logits      [T, E] float32 out, or NULL (exported for inspection)
 * Requirements: H % 128 == 0, 1 <= E <= 1024, 1 <= k <= min(E, 32).
 * Non-finite logits give unspecified (but in-bounds) ids.
 */
size_t moe_route_workspace_size(int T, int E);
moe_status moe_route(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                     int T, int H, int E, int k,
                     int32_t *topk_ids, float *topk_weights, float *logits,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- permutation
 * moe_permute: groups the n = T*k rows r = t*k + j (token t, slot j) by expert
 * topk_ids[r], keeping r ascending inside each expert (a stable counting sort).
 * Grouping the rows is what lets each selected expert's weights be read once
 * for all of its rows, and only the selected experts at all (page
 * "Qwen3.8-Flash-Next on one 24 GB GPU", "What the patch does": the decode
 * GEMV reads only the selected experts, in place).
 *
 *   topk_ids       [T, k] int32 in
 *   expert_offsets [E+1] int32 out: rows of expert e are sorted positions
 *                  [expert_offsets[e], expert_offsets[e+1])
 *   sorted_rows    [n] int32 out: the row r at each sorted position
 *   row_pos        [n] int32 out: the sorted position of row r (inverse of
 *                  sorted_rows); -1 for a row whose id is outside [0, E)
 *   active         [1 + min(E, n)] int32 out: active[0] = A, the number of
 *                  experts with at least one row, then their ids ascending,
 *                  then -1 padding
 * Rows whose id lies outside [0, E) are dropped (they get no sorted position).
 * Workspace: moe_permute_workspace_size(T, k, E) bytes, 256-byte aligned,
 * all-zero and left zero (the conventions above); the size is 0 for
 * T*k <= 4096, and then workspace may be NULL.  Larger batches keep a block
 * counter and a table of per-block expert counts there.
 */
size_t moe_permute_workspace_size(int T, int k, int E);
moe_status moe_permute(const int32_t *topk_ids, int T, int k, int E,
                       int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos,
                       int32_t *active, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- route + permutation
 * moe_route_permute: moe_route, then moe_permute on its topk_ids, with the
 * outputs of both bit for bit (same arguments, same meaning).  For
 * T*k <= 256 both steps run in one launch: the block that finishes the
 * top-k last groups the rows by expert in LDS, which saves a launch on the
 * decode path.  Other shapes run the two launches in order.  topk_ids are
 * always valid expert ids here, so row_pos has no -1 entries.
 * The workspace (moe_route_permute_workspace_size bytes, 256-byte aligned)
 * starts with the router's control block; the library leaves all of it zero.
 */
size_t moe_route_permute_workspace_size(int T, int k, int E);
moe_status moe_route_permute(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                             int T, int H, int E, int k,
                             int32_t *topk_ids, float *topk_weights, float *logits,
                             int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos,
                             int32_t *active, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- expert FFN
 * moe_expert_ffn_w4a16: for every active expert e and each of its rows
 * (sorted positions p in [expert_offsets[e], expert_offsets[e+1]), token
 * t = sorted_rows[p] / k):
 *     a = W13_e x_t                     gate_up, 2I outputs; rows [0, I) of
 *                                       W13 are gate, rows [I, 2I) are up
 *     h = silu(a[0:I]) * a[I:2I]        silu(v) = v / (1 + exp(-v))
 *     y_perm[p] = W2_e h                down, H outputs, stored as bf16
 * with W = q * s dequantised from INT4 symmetric group-128 codes.  The dot
 * products accumulate in float32; h is rounded to bf16 before the down
 * projection.  Three paths, chosen on the host from the sizes alone
 * (moe_expert_ffn_path reports the choice):
 *   decode  T <= 512 and T*k <= 6*E (at most about six rows per expert): one
 *           fused GEMV kernel streaming each selected expert's packed weights
 *           once, rows in passes of four;
 *   mid     otherwise while T*k <= 24*E (INT4 / 2-bit g128, H and I
 *           multiples of 256): two launches that stage up to 32 rows of an
 *           expert per K step and read its weights once per 32 rows;
 *   GEMM    otherwise: grouped bf16-MFMA GEMMs on dequantised tiles; for
 *           INT4 / 2-bit g128 (H, I multiples of 256) the experts with at
 *           most 64 rows run the mid kernel inside the same call.
 * The pages dispatch between a GEMV and dequantise-then-GEMM at 16 rows (page
 * "Qwen3.8-Flash-Next FP6-INT8", "Quantization quality"); the crossovers used
 * here were measured on MI355X instead.  The permutation arrays must come
 * from moe_permute with the same T, k, E.
 *
 *   x           [T, H] bf16, 16-byte aligned
 *   w13_codes   [E, 2I, H/8]  uint32, 16-byte aligned
 *   w13_scales  [E, 2I, H/128] bf16
 *   w2_codes    [E, H, I/8]   uint32, 16-byte aligned
 *   w2_scales   [E, H, I/128] bf16
 *   y_perm      [T*k, H] bf16 out, in sorted order (rows of dropped ids untouched)
 *   workspace   moe_expert_ffn_workspace_size bytes; all of it must be zero
 *               before the first call (allocate it zeroed) and every call
 *               leaves all of it zero again (the decode path tells written
 *               intermediate values from unwritten ones by a nonzero tag)
 * Requirements: H % 128 == 0, I % 128 == 0, 1 <= E <= 1024, 1 <= k <= 32;
 * on the grouped-GEMM path also T*H <= 2^30 and I*H <= 2^30 (32-bit offsets).
 */
size_t moe_expert_ffn_workspace_size(int T, int k, int E, int H, int I);

/* moe_expert_ffn_path: the path the expert-FFN calls take for these sizes and
 * format (bits, group_size as for moe_expert_ffn_wna16; bits 4 with group 16
 * is NVFP4, which has no mid path): MOE_FFN_PATH_DECODE, _MID or _GEMM, or -1
 * for a negative size or an unsupported format.  Pure host arithmetic. */
#define MOE_FFN_PATH_DECODE 0
#define MOE_FFN_PATH_MID 1
#define MOE_FFN_PATH_GEMM 2
int moe_expert_ffn_path(int T, int k, int E, int H, int I, int bits, int group_size);

moe_status moe_expert_ffn_w4a16(const uint16_t *x, const int32_t *expert_offsets,
                                const int32_t *sorted_rows, const int32_t *active,
                                int T, int k, int E, int H, int I,
                                const uint32_t *w13_codes, const uint16_t *w13_scales,
                                const uint32_t *w2_codes, const uint16_t *w2_scales,
                                uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                void *stream);

/* moe_expert_ffn_w2a16: as moe_expert_ffn_w4a16 with 2-bit codes (16 per
 * uint32 along K: w13_codes [E, 2I, H/16], w2_codes [E, H, I/16]) and
 * W = (u - z) * s, z an integer zero-point per (row, group):
 *   w13_zeros [E, 2I, H/128] uint8, w2_zeros [E, H, I/128] uint8. */
moe_status moe_expert_ffn_w2a16(const uint16_t *x, const int32_t *expert_offsets,
                                const int32_t *sorted_rows, const int32_t *active,
                                int T, int k, int E, int H, int I,
                                const uint32_t *w13_codes, const uint16_t *w13_scales,
                                const uint8_t *w13_zeros,
                                const uint32_t *w2_codes, const uint16_t *w2_scales,
                                const uint8_t *w2_zeros,
                                uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                void *stream);

/* moe_expert_ffn_wna16: the expert FFN of moe_expert_ffn_w4a16 for a format
 * given by bits and group_size:
 *   bits 4, group 128 or 32   W = (field - 8) * s
 *   bits 8, group 128 or 32   W = (field - 128) * s
 *   bits 2, group 128         W = (field - z) * s   (zero-points required)
 *   bits 6, group 128         W = e2m3(code) * s    (FP6; s is fp16)
 * with s (and z) the value of the group that holds the K index:
 *   w13_codes [E, 2I, H*bits/32] uint32, w13_scales [E, 2I, H/G] bf16 (fp16 for FP6),
 *   w13_zeros [E, 2I, H/G] uint8 (bits == 2, else ignored; may be NULL),
 *   w2_codes [E, H, I*bits/32], w2_scales [E, H, I/G], w2_zeros [E, H, I/G].
 * Other arguments, requirements, dispatch (the decode path streams each
 * selected expert once; with groups of 32 each MFMA covers one group) and
 * workspace are those of moe_expert_ffn_w4a16; (4, 128) and (2, 128) give
 * the results of moe_expert_ffn_w4a16 / _w2a16 bit for bit.  Any other
 * (bits, group_size) returns MOE_ERR_INVALID_ARG. */
moe_status moe_expert_ffn_wna16(const uint16_t *x, const int32_t *expert_offsets,
                                const int32_t *sorted_rows, const int32_t *active,
                                int T, int k, int E, int H, int I, int bits, int group_size,
                                const uint32_t *w13_codes, const uint16_t *w13_scales,
                                const uint8_t *w13_zeros,
                                const uint32_t *w2_codes, const uint16_t *w2_scales,
                                const uint8_t *w2_zeros,
                                uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                void *stream);

/* moe_expert_ffn_nvfp4: the expert FFN with NVFP4 W4A4 experts (page
 * "Qwen3.8-Flash-Next NVFP4", "Format": E2M1 values in groups of 16; the
 * group scale is FP8 E4M3 and one float32 scale covers a tensor, as NVFP4
 * defines them).  Weights: w13_codes [E, 2I, H/8], w2_codes [E, H, I/8] uint32
 * with eight 4-bit E2M1 codes per word along K (field i of word w is K index
 * 8w + i; bit 3 sign, bits 2..1 exponent with bias 1, bit 0 mantissa),
 * w13_scales [E, 2I, H/16] and w2_scales [E, H, I/16] E4M3 codes (uint8, one
 * per 16 K), w13_gscale [E] and w2_gscale [E] float32 tensor scales.  The
 * activations are quantised on the fly (moe_quant_act_nvfp4) with tensor
 * scale x_gscale before gate_up, and h with h_gscale before down:
 *   a = NVFP4(x) . W13' * (x_gscale * w13_gscale[e]),  h = silu(a_gate) * a_up
 *   y = NVFP4(h) . W2'  * (h_gscale * w2_gscale[e])
 * with W' = e2m1 * e4m3 (exact in bf16) and float32 accumulation.  Dispatch
 * as for moe_expert_ffn_w4a16 (the decode GEMV kernel, which quantises each
 * item's 16 h outputs itself, while T <= 512 and T*k <= 6*E; the grouped
 * GEMMs above).  Workspace: moe_expert_ffn_nvfp4_workspace_size bytes,
 * zero before the first call and left zero.  Other arguments and
 * requirements as for moe_expert_ffn_w4a16; the scales must be positive and
 * finite. */
size_t moe_expert_ffn_nvfp4_workspace_size(int T, int k, int E, int H, int I);
moe_status moe_expert_ffn_nvfp4(const uint16_t *x, const int32_t *expert_offsets,
                                const int32_t *sorted_rows, const int32_t *active,
                                int T, int k, int E, int H, int I, float x_gscale, float h_gscale,
                                const uint32_t *w13_codes, const uint8_t *w13_scales, const float *w13_gscale,
                                const uint32_t *w2_codes, const uint8_t *w2_scales, const float *w2_gscale,
                                uint16_t *y_perm, void *workspace, size_t workspace_bytes, void *stream);

/* moe_quant_act_nvfp4: the NVFP4 activation quantiser of moe_expert_ffn_nvfp4
 * on n bf16 values (n % 16 == 0; groups of 16 consecutive values).  Per group:
 * amax = max |x|, s = E4M3(amax / (6 G)), q = E2M1(x / (s G)) (0 when s = 0),
 * every rounding to nearest even and saturating (448, 6), every step one
 * float32 operation in that order.  values [n] bf16 = q * s (exact); scales
 * [n/16] uint8 E4M3 codes of s, or NULL. */
moe_status moe_quant_act_nvfp4(const uint16_t *x, int64_t n, float gscale, uint16_t *values, uint8_t *scales,
                               void *stream);

/* moe_expert_ffn_w4a16_table / moe_expert_ffn_w2a16_table: the same
 * computation, with each expert's weights found through a per-expert address
 * table instead of three stacked arrays per projection, so that every expert
 * is read where it lives (device memory, or pinned host memory that the device
 * can address) and moving an expert is a write of its table entry.  Page
 * "Qwen3.8-Flash-Next on one 24 GB GPU", "What the patch does" (experts read
 * in place through an int64 address table; placement as a table write).
 *   expert_table  [E, 6] uint64, device-readable (device or pinned host
 *                 memory), 8-byte aligned, not modified.  Row e holds the
 *                 addresses of expert e's own blocks, in this order:
 *                   0  w13 codes   [2I, H/P] uint32 (P = 8 INT4, 16 2-bit)
 *                   1  w13 scales  [2I, H/128] bf16
 *                   2  w13 zeros   [2I, H/128] uint8  (2-bit only, else unused)
 *                   3  w2 codes    [H, I/P] uint32
 *                   4  w2 scales   [H, I/128] bf16
 *                   5  w2 zeros    [H, I/128] uint8   (2-bit only, else unused)
 *                 i.e. the slices [e] of the stacked arrays above.  Code blocks
 *                 must be 16-byte aligned and scale blocks 2-byte aligned; each
 *                 entry must be a valid device-visible address while the call
 *                 runs (rows of inactive experts are never read).
 * All other arguments, the requirements, the dispatch and the results are
 * those of moe_expert_ffn_w4a16 / _w2a16: with the same weights the output is
 * bit-identical.  A NULL table returns MOE_ERR_INVALID_ARG. */
moe_status moe_expert_ffn_w4a16_table(const uint16_t *x, const int32_t *expert_offsets,
                                      const int32_t *sorted_rows, const int32_t *active,
                                      int T, int k, int E, int H, int I,
                                      const uint64_t *expert_table,
                                      uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                      void *stream);
moe_status moe_expert_ffn_w2a16_table(const uint16_t *x, const int32_t *expert_offsets,
                                      const int32_t *sorted_rows, const int32_t *active,
                                      int T, int k, int E, int H, int I,
                                      const uint64_t *expert_table,
                                      uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* moe_expert_ffn_wna16_table: moe_expert_ffn_wna16 (any of its formats,
 * chosen by bits and group_size as there) with each expert found through the
 * table above.  Row e holds the addresses of the [e] slices of the six stacked
 * arrays of moe_expert_ffn_wna16: code blocks [N, K*bits/32] uint32 (FP6: the
 * row's bit stream, 3 words per 16 codes), 16-byte aligned; scale blocks
 * [N, K/group] bf16 (FP6: fp16), 2-byte aligned; zero-point blocks
 * [N, K/group] uint8 for 2-bit only (entries 2 and 5 are not read for the
 * other formats).  With the same weights the output is bit-identical to
 * moe_expert_ffn_wna16.  A NULL table returns MOE_ERR_INVALID_ARG, an
 * unsupported format MOE_ERR_INVALID_ARG. */
moe_status moe_expert_ffn_wna16_table(const uint16_t *x, const int32_t *expert_offsets,
                                      const int32_t *sorted_rows, const int32_t *active,
                                      int T, int k, int E, int H, int I, int bits, int group_size,
                                      const uint64_t *expert_table,
                                      uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* moe_expert_ffn_nvfp4_table: moe_expert_ffn_nvfp4 with each expert found
 * through the table above (same page and section).  Row e holds, in order:
 *   0  w13 codes   [2I, H/8] uint32 E2M1 fields, 16-byte aligned
 *   1  w13 scales  [2I, H/16] uint8 E4M3 codes
 *   2  w13 tensor scale: the address of one float32 (4-byte aligned)
 *   3  w2 codes    [H, I/8] uint32, 16-byte aligned
 *   4  w2 scales   [H, I/16] uint8
 *   5  w2 tensor scale: the address of one float32
 * i.e. the [e] slices and elements of the stacked arrays of
 * moe_expert_ffn_nvfp4.  Workspace: moe_expert_ffn_nvfp4_workspace_size.  With
 * the same weights the output is bit-identical to moe_expert_ffn_nvfp4.  A
 * NULL table returns MOE_ERR_INVALID_ARG. */
moe_status moe_expert_ffn_nvfp4_table(const uint16_t *x, const int32_t *expert_offsets,
                                      const int32_t *sorted_rows, const int32_t *active,
                                      int T, int k, int E, int H, int I, float x_gscale, float h_gscale,
                                      const uint64_t *expert_table,
                                      uint16_t *y_perm, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* moe_device_address: the address under which the kernels read ptr, for
 * filling an expert table.  Device (and managed) memory is returned as is;
 * pinned host memory (hipHostMalloc, torch pin_memory) through the runtime's
 * device mapping, offset kept.  Pageable host memory and pointers the runtime
 * does not know return MOE_ERR_INVALID_ARG: the kernels cannot read them. */
moe_status moe_device_address(const void *ptr, uint64_t *out);

/* ---------------------------------------------------------------- combine
 * moe_combine: y[t] = sum over j = 0..k-1 (ascending) of
 *   topk_weights[t, j] * y_perm[row_pos[t*k + j]]   in float32, stored as bf16.
 * The pages name top-k routing with softmax gates but do not spell out the
 * combine; this gate-weighted sum of the k expert outputs is the plainest
 * reading, accumulated in float32 like every other sum of the layer (page
 * "Qwen3.8-Flash-Next FP6-INT8", "Precision map": bf16 activations, float32
 * accumulation).
 * Rows with row_pos < 0 contribute nothing.
 *   y_perm [T*k, H] bf16, row_pos [T*k] int32, topk_weights [T, k] float32,
 *   y [T, H] bf16 out.  y_perm and y 16-byte aligned, H % 8 == 0.
 */
moe_status moe_combine(const uint16_t *y_perm, const int32_t *row_pos, const float *topk_weights,
                       int T, int k, int H, uint16_t *y, void *stream);

/* ---------------------------------------------------------------- whole decode layer
 * moe_layer_w4a16 / moe_layer_w2a16: the whole layer of a small batch in one
 * launch: y = moe_combine(expert FFN(moe_route_permute(x))), with the same
 * bits as those calls made one after another (router order, ties, gates,
 * grouping, FFN arithmetic and combine order are shared).  The blocks of the
 * launch first compute the router logits, one block runs every token's top-k
 * and publishes the rows grouped by expert, every block streams its share of
 * the selected experts' weights, and finally some blocks combine y.  This
 * removes the launches and hand-offs between the stages on the decode path.
 *
 *   x, w_router, logit_bias, T, H, E, k   as for moe_route
 *   I, w13_*, w2_*                        as for moe_expert_ffn_w4a16 / _w2a16
 *   y             [T, H] bf16 out
 *   topk_ids      [T, k] int32 out, or NULL;  topk_weights [T, k] float32 out, or NULL
 *   workspace     moe_layer_workspace_size(T, k, E, H, I) bytes, all-zero
 *                 before the first call, left all-zero by every call
 * Requirements: those of the stages, plus 1 <= T <= 16, T*k <= 256,
 * E <= 65536 and a shape the decode path supports (I % 16 == 0, and its LDS
 * fits); otherwise the call returns MOE_ERR_UNSUPPORTED_SHAPE and the stage
 * calls are the way to run the layer.
 */
size_t moe_layer_workspace_size(int T, int k, int E, int H, int I);
/* moe_layer_wna16: the one-launch layer for any format of moe_expert_ffn_wna16
 * (bits / group_size: 4 / 128 or 32, 8 / 128 or 32, 2 / 128, 6 / 128 (FP6,
 * fp16 scales)); arguments as for moe_layer_w2a16 with the two format
 * integers after I (zero-points used for bits == 2 only).  Results equal the
 * stage calls with moe_expert_ffn_wna16 bit for bit. */
/* moe_layer_nvfp4: the one-launch layer with NVFP4 W4A4 experts (the weights,
 * scales and the two tensor scales of moe_expert_ffn_nvfp4).  The router
 * reads x as given; each block quantises the activation rows it stages for
 * the experts (moe_quant_act_nvfp4's steps), so the results equal the stage
 * calls (moe_route_permute, moe_expert_ffn_nvfp4, moe_combine) bit for bit.
 * Workspace: moe_layer_workspace_size. */
moe_status moe_layer_nvfp4(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                           int T, int H, int E, int k, int I, float x_gscale, float h_gscale,
                           const uint32_t *w13_codes, const uint8_t *w13_scales, const float *w13_gscale,
                           const uint32_t *w2_codes, const uint8_t *w2_scales, const float *w2_gscale,
                           uint16_t *y, int32_t *topk_ids, float *topk_weights,
                           void *workspace, size_t workspace_bytes, void *stream);
moe_status moe_layer_wna16(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                           int T, int H, int E, int k, int I, int bits, int group_size,
                           const uint32_t *w13_codes, const uint16_t *w13_scales, const uint8_t *w13_zeros,
                           const uint32_t *w2_codes, const uint16_t *w2_scales, const uint8_t *w2_zeros,
                           uint16_t *y, int32_t *topk_ids, float *topk_weights,
                           void *workspace, size_t workspace_bytes, void *stream);
moe_status moe_layer_w4a16(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                           int T, int H, int E, int k, int I,
                           const uint32_t *w13_codes, const uint16_t *w13_scales,
                           const uint32_t *w2_codes, const uint16_t *w2_scales,
                           uint16_t *y, int32_t *topk_ids, float *topk_weights,
                           void *workspace, size_t workspace_bytes, void *stream);
moe_status moe_layer_w2a16(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                           int T, int H, int E, int k, int I,
                           const uint32_t *w13_codes, const uint16_t *w13_scales, const uint8_t *w13_zeros,
                           const uint32_t *w2_codes, const uint16_t *w2_scales, const uint8_t *w2_zeros,
                           uint16_t *y, int32_t *topk_ids, float *topk_weights,
                           void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- the layer without a workspace
 * moe_layer_w4a16_noalloc: moe_layer_w4a16 for callers that cannot allocate
 * device memory - code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments without the workspace,
 * same kernels, same results bit for bit.  The workspace is a file-scope
 * device array of the library (8 MiB, one per GPU, reserved when the library's
 * code is loaded on that GPU and kept until the process ends); the call
 * allocates and frees nothing.  Shapes whose moe_layer_workspace_size exceeds
 * 8 MiB return MOE_ERR_UNSUPPORTED_SHAPE (T*k <= 256 with H = 4096, I = 1024
 * and E <= 1024 fit).  Every call first clears the part of the array it uses
 * with a fill kernel on `stream`, then launches the layer.  All calls on one
 * GPU share that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued.  A wait that timed out
 * inside such a call is not reported (there is no caller-visible workspace to
 * read the flag from); the next call starts from a cleared array.
 */
moe_status moe_layer_w4a16_noalloc(const uint16_t *x, const uint16_t *w_router, const float *logit_bias,
                                   int T, int H, int E, int k, int I,
                                   const uint32_t *w13_codes, const uint16_t *w13_scales,
                                   const uint32_t *w2_codes, const uint16_t *w2_scales,
                                   uint16_t *y, int32_t *topk_ids, float *topk_weights, void *stream);

/* ---------------------------------------------------------------- diagnostics
 * moe_unpack_codes: the signed codes of n_words packed words, unpacked by the
 * same device routine the decode kernels use (INT4: q = field - 8; 2-bit:
 * u = field; INT8: q = field - 128; FP6: 8 * e2m3 value, an integer in
 * [-60, 60]).  out holds n_words * 32/bits int8 values in K order.  bits: 2,
 * 4, 6 (n_words a multiple of 6) or 8.
 */
moe_status moe_unpack_codes(const uint32_t *words, int bits, int64_t n_words, int8_t *out,
                            void *stream);

/* moe_dequant_bf16: one [N, K] matrix dequantised to bf16 by the same device
 * routine the grouped-GEMM kernels use: round-to-nearest-even of (q - z) * s.
 *   words [N, K*bits/32] uint32 (16-byte aligned), scales [N, K/128] bf16,
 *   zeros [N, K/128] uint8 (bits == 2 only, else NULL), out [N, K] bf16.
 * Requirements: K % 128 == 0; bits 2, 4 or 8. */
moe_status moe_dequant_bf16(const uint32_t *words, const uint16_t *scales, const uint8_t *zeros,
                            int bits, int N, int K, uint16_t *out, void *stream);
/* moe_dequant_bf16_grouped: the same with group_size 128, or 32 (bits 4 or 8;
 * scales [N, K/32]); bits 6 (FP6, group 128) takes fp16 scales. */
moe_status moe_dequant_bf16_grouped(const uint32_t *words, const uint16_t *scales, const uint8_t *zeros,
                                    int bits, int group_size, int N, int K, uint16_t *out, void *stream);

/* ---------------------------------------------------------------- measurement probes
 * The device's achievable rates, measured by the benchmark next to the spec
 * sheet's peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA):
 * moe_probe_stream_read: reads `bytes` (a multiple of 16; buf 16-byte
 *   aligned) once in one launch, each thread eight 16-byte loads all in flight
 *   together, and writes one folded word per block to out
 *   [moe_probe_stream_blocks(bytes)] (so the reads cannot be dropped).
 * moe_probe_mfma: `blocks` blocks of four waves, each wave issuing 8 * iters
 *   v_mfma_f32_16x16x32_bf16 (16384 flops each) on register operands with eight
 *   independent accumulators; out [4 * blocks] float32 (the folded sums). */
size_t moe_probe_stream_blocks(size_t bytes);
moe_status moe_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream);
moe_status moe_probe_mfma(int blocks, int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BQMOE_H */
