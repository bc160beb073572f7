/*
 * kk.h -- C ABI of the MI355X (gfx950) library for KV-Kaizen compressed
 * decode attention: a per-layer compressed MLA cache (depth, rank and
 * precision choices per layer) and one decode step of absorbed-MLA attention
 * over it.
 *
 * Method source: "KV-Kaizen: Learning Context-Adaptive Cache Compression
 * Choices" (arXiv 2609.37988), picx.dev whiteboard summary page:
 *   - "Three Non-Eviction Compression Axes": depth (an anchor layer owns a
 *     cache, later layers inherit it), rank (the MLA cache keeps the first
 *     d <= r coordinates of the latent c^KV plus the decoupled RoPE key k^R),
 *     precision (stored at b <= 16 bits, symmetric uniform quantization, one
 *     scale per token);
 *   - "Action Space and Cost Model": per-layer actions {inherit} U {(d, b)},
 *     b in {2, 4, 8, 16}; cost (d + d_R) * b bits per token;
 *   - "Selector Architecture and Training", Inference item: the per-layer
 *     configuration is chosen once before pre-fill and fixed for every
 *     generated token (here: an input table, constant across calls);
 *   - "Background: The KV Cache Bottleneck": every decoded token reads the
 *     whole cache, so decode is bound by memory bandwidth.
 *
 * Conventions shared by every entry point
 *   - All device pointers are HIP device allocations owned by the caller.
 *     The library never allocates or frees device memory, never
 *     synchronizes, and keeps no mutable global state (planning uses host
 *     memory local to the call); calls are thread-safe.  The one exception is
 *     kk_decode_attn_noalloc, which keeps its partials in a static device
 *     array per device (see there).
 *   - Every call validates its arguments on the host before enqueueing
 *     anything; a non-KK_OK status means nothing was enqueued.
 *   - Work is enqueued on the caller's stream and returns asynchronously;
 *     a kernel fault surfaces at the caller's next synchronization.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified results.
 *
 * Cache layout (one anchor layer)
 *   codes  : uint8 [batch][t_cap][row_stride]; row = d + d_R fields of b bits,
 *            field j (latent coordinate j for j < d, RoPE coordinate j - d
 *            after) is the two's-complement code at bit offset j*b of the row,
 *            bytes little-endian (b = 2, 4, 8).  b = 16 is stored as two
 *            byte planes: bytes [0, K) hold the high bytes of fields 0..K-1,
 *            bytes [K, 2K) their low bytes with bit 7 flipped (K = d + d_R),
 *            so that the integer MFMA reads each plane as int8 operands.
 *            row_stride = ceil((d + d_R)*b/8 / 16) * 16, padding bytes are
 *            zero.  16-byte aligned.
 *   scales : float32 [batch][t_cap], one per token.  16-byte aligned.
 *   Quantization of one token v = [c[0:d] || k^R[0:d_R]] (fp32):
 *     qmax = 2^(b-1) - 1; amax = max |v_j|; scale = amax / qmax (IEEE fp32
 *     division, round to nearest even); code_j = clamp(rint(v_j / scale),
 *     -qmax, qmax) with IEEE fp32 division and ties to even; amax = 0 gives
 *     scale 0 and all codes 0.  Dequantized value: code * scale.
 *
 * Decode output layout: float32, packed per layer as [batch][n_heads][d_eff]
 * at the float offsets returned by kk_out_offsets (layer order), where d_eff
 * is the d of the layer's anchor.
 */
#ifndef KK_H_
#define KK_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KK_OK = 0,
  KK_ERR_INVALID_ARGUMENT = 1,   /* a rule below is broken (null, misaligned, out of range) */
  KK_ERR_UNSUPPORTED = 2,        /* valid for the method but outside this library's limits */
  KK_ERR_WORKSPACE_TOO_SMALL = 3,
  KK_ERR_DEVICE = 4              /* a HIP launch or query failed */
} kk_status;

typedef enum { KK_DTYPE_F32 = 0, KK_DTYPE_BF16 = 1 } kk_dtype;

/* Build limits (KK_ERR_UNSUPPORTED beyond them). */
#define KK_MAX_LAYERS 64
#define KK_MAX_D 512           /* kept latent width d (and r >= d, any r) */
#define KK_MAX_K 576           /* d + d_R (512 + 64, the MLA shape) */
#define KK_MAX_TABLES 1024     /* tables of one heterogeneous step */

/* One layer's action ("Action Space and Cost Model").
 *   anchor == own index : the layer is an anchor with action (d, bits);
 *   anchor <  own index : the layer inherits the cache of layer `anchor`,
 *                         which must itself be an anchor; d and bits are
 *                         ignored (the anchor's are used).
 * sm_scale is the layer's softmax scale (any finite value; the workloads use
 * 1/sqrt(d_eff + d_R)).
 * Rules: layer 0 is an anchor; 0 < d <= r, d % 16 == 0; bits in {2,4,8,16};
 * d_R % 16 == 0; d + d_R <= KK_MAX_K; d <= KK_MAX_D; ceil(d / 64) +
 * ceil(d_R / 64) <= 9 (the decode reads the latent and the RoPE part of a row
 * in separate 64-field chunks). */
typedef struct {
  int32_t anchor;
  int32_t d;
  int32_t bits;
  float sm_scale;
} kk_layer_cfg;

typedef struct {
  int32_t n_layers;             /* 1 .. KK_MAX_LAYERS */
  int32_t n_heads;              /* query heads per layer, >= 1 */
  int32_t r;                    /* full latent width (q_lat row length) */
  int32_t d_rope;               /* RoPE key width d_R, 16 .. 128, multiple of 16 */
  const kk_layer_cfg* layers;   /* host array [n_layers] */
} kk_model_cfg;

/* Device buffers of one anchor layer's cache (see layout above). */
typedef struct {
  uint8_t* codes;
  float* scales;
} kk_cache;

/* Row stride in bytes of a (d, d_rope, bits) cache; 0 if the combination is
 * invalid (bits not in {2,4,8,16}, non-positive widths, or (d+d_rope)*bits
 * not a multiple of 8).
 * Follows the per-token cost of an action on the KV-Kaizen summary page
 * ("Action Space and Cost Model", cost equation: (d + d_R) * b bits), rounded
 * up to whole 16-byte segments. */
size_t kk_row_stride_bytes(int32_t d, int32_t d_rope, int32_t bits);

/* Checks the table rules above (the action set of "Action Space and Cost
 * Model"; the depth item of "Three Non-Eviction Compression Axes": an
 * inheriting layer names an earlier anchor). */
kk_status kk_validate_model(const kk_model_cfg* cfg);

/* Bytes of the codes and scales buffers of anchor `layer` for [batch][t_cap]:
 * batch * t_cap rows of kk_row_stride_bytes, and one float32 scale per token
 * (precision item of "Three Non-Eviction Compression Axes": one scale per
 * token).  Inheriting layers own no cache (depth item): KK_ERR_INVALID_ARGUMENT.
 * Host outputs; no device access. */
kk_status kk_cache_bytes(const kk_model_cfg* cfg, int32_t layer, int32_t batch, int32_t t_cap,
                         size_t* codes_bytes, size_t* scales_bytes);

/* Float offsets of each layer's output block in the packed decode output:
 * offsets[l] for l in [0, n_layers], offsets[n_layers] = total floats.
 * `offsets` is a host array of n_layers + 1 entries.  Each layer's block is
 * [batch][n_heads][d_eff]: the absorbed output lives in the latent space kept
 * by the layer's anchor (rank item of "Three Non-Eviction Compression Axes"). */
kk_status kk_out_offsets(const kk_model_cfg* cfg, int32_t batch, int64_t* offsets);

/* Quantize-and-pack cache write (pre-fill and append) for anchor `layer`:
 * the cache keeps the first d latent coordinates and the RoPE key (rank item
 * of "Three Non-Eviction Compression Axes"), as b-bit symmetric uniform codes
 * with one scale per token (precision item), quantized as stated at the top
 * of this file.
 *
 * Source rows: latent [n_src][latent_ld] (first d of r coordinates used) and
 * rope [n_src][rope_ld] (first d_rope used), both `src_dtype` (float32, or
 * bf16 widened exactly), device, 4-byte aligned.  Token i (0 <= i < n_tokens)
 * reads source row src_index[i] (device int32, nullable: identity) and writes
 * cache slot dst_slot[i] (device int64: seq * t_cap + position).  A token
 * whose source row is outside [0, n_src) or whose slot is outside
 * [0, batch * t_cap) is skipped.  Gathering by src_index composes eviction:
 * the kept positions of a longer context are packed densely.
 * Two tokens writing the same slot race. */
kk_status kk_quantize_write(const kk_model_cfg* cfg, int32_t layer,
                            const void* latent, const void* rope, kk_dtype src_dtype,
                            int64_t latent_ld, int64_t rope_ld, int64_t n_src, int32_t n_tokens,
                            const int32_t* src_index, const int64_t* dst_slot,
                            kk_cache dst, int32_t batch, int32_t t_cap, hipStream_t stream);

/* Workspace bytes kk_decode_attn needs for this model, batch and
 * max_seq_len, with the same split_tokens argument (0 = automatic).
 * The workspace holds split partials only; it need not be zeroed.
 * Automatic splits are planned for the compute units of the current HIP
 * device (hipGetDevice); with no device, KK_ERR_DEVICE.  kk_decode_attn plans
 * for the device of its stream, so size the workspace on that device. */
kk_status kk_decode_workspace_bytes(const kk_model_cfg* cfg, int32_t batch, int32_t max_seq_len,
                                    int32_t split_tokens, size_t* bytes);

/* The work plan of one kk_decode_attn step (host only; no device access when
 * n_cus > 0).  The decode step splits each sequence's tokens so that the work
 * items fill the device (every decoded token reads the whole cache: "Background:
 * The KV Cache Bottleneck"); the split count depends on the compute units.
 * n_cus > 0 plans for that many compute units, n_cus == 0 for the current
 * device's.  Outputs: the compute units used, the decode work items (one
 * workgroup each), the merge workgroups (one per split (row chunk, sequence),
 * or up to 4 feature ranges of one when merges are fewer than 4 per compute
 * unit), the largest split count of any
 * (row chunk, sequence), and the workspace bytes (as kk_decode_workspace_bytes
 * on a device with n_cus compute units). */
typedef struct {
  int32_t n_cus;
  int32_t work_items;
  int32_t merge_blocks;
  int32_t max_splits;
  size_t workspace_bytes;
} kk_plan_info;
kk_status kk_decode_plan_info(const kk_model_cfg* cfg, int32_t batch, int32_t max_seq_len, int32_t split_tokens,
                              int32_t n_cus, kk_plan_info* info);

/* One decode step of absorbed-MLA attention for every layer of the table
 * (the step that reads the whole compressed cache for every generated token:
 * "Background: The KV Cache Bottleneck"; the cache of the depth, rank and
 * precision items of "Three Non-Eviction Compression Axes").
 *
 * For layer l with anchor a = cfg->layers[l].anchor, d = d_a, b = b_a, each
 * sequence s and head h, over the cached tokens t < len_s:
 *   z_t = sm_scale_l * (q_lat[l,s,h,0:d] . c_a[s,t,0:d] + q_rope[l,s,h,:] . kR_a[s,t,:])
 *   out[l,s,h,i] = sum_t softmax(z)_t * c_a[s,t,i],  i < d
 * with c_a, kR_a the dequantized anchor cache (code * scale).  Inheriting
 * layers read their anchor's buffers (no copy); len_s = 0 gives zeros.
 *
 * caches     : host array [n_layers]; entries of inheriting layers are ignored.
 * seq_lens   : device int32 [batch]; each value is clamped to [0, t_cap].
 * max_seq_len: host planning hint in [0, t_cap]: the expected longest
 *              sequence, which sets how many splits each sequence's tokens
 *              are cut into.  It never truncates: every sequence is attended
 *              over all of its (clamped) seq_lens tokens, also above it.
 * q_lat      : device [n_layers][batch][n_heads][r], q_dtype.
 * q_rope     : device [n_layers][batch][n_heads][d_rope], q_dtype.
 * out        : device float32, packed as kk_out_offsets describes.
 * split_tokens: tokens per split of one sequence (multiple of 32), or 0 to let
 *              the library choose; results agree across choices within
 *              floating-point rounding and are bitwise reproducible for a
 *              fixed choice.
 * workspace  : device, >= kk_decode_workspace_bytes, 256-byte aligned.
 *
 * Arithmetic and the range it is checked over: the latent part of each query
 * row is rounded once to a 15-bit fixed-point number relative to its largest
 * magnitude (two int8 limbs) and the RoPE part to a 22-bit one relative to its
 * own (three limbs); the integer scores of the two parts are exact (b = 16: up
 * to a left-out low-byte term of 2^-15 resp. 2^-22 of the leading one) and are
 * joined in fp32; softmax in fp32; the P.V operands are P' (numerator times
 * token scale) in fp16 and the codes in fp16 (exact for b <= 8, rounded to 11
 * significant bits for b = 16), accumulated in fp32.  Against an exact fp64
 * evaluation of the formula above, the output stays within 2e-3 * max|out| per
 * layer for N(0, 1) queries, for queries whose RoPE part is up to 256x the
 * latent part or whose latent part is 64x the RoPE part, and for one
 * coordinate per row scaled 64x in either part (all tested, with and without
 * token splits).  The logit error is about 2^-15 of the latent part's largest
 * term plus 2^-22 of the RoPE part's, so it grows with |q| * |cache|: queries
 * far outside that range can exceed the bound. */
kk_status kk_decode_attn(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                         const int32_t* seq_lens, int32_t max_seq_len,
                         const void* q_lat, const void* q_rope, kk_dtype q_dtype, float* out,
                         int32_t split_tokens, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Size of the device array that kk_decode_attn_noalloc keeps its split
 * partials in: 256 MiB, held on each device the entry point runs on until the
 * process ends.  It covers the automatic plan (split_tokens = 0) of 32
 * sequences of 8192 tokens on the 7B (28 layers, d = 512, b = 16: 227 MiB)
 * and 14B (48 layers, mixed table: 159 MiB) shapes on a 256-CU device;
 * kk_decode_workspace_bytes gives the need of any other step. */
#define KK_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* kk_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, checks, kernels, results
 * and error statuses as kk_decode_attn; the split partials go to a static
 * device array of KK_NOALLOC_SCRATCH_BYTES instead of a workspace.
 *   - Calls no hipMalloc, hipFree or other device-allocating routine.  The
 *     first call on a device looks the array's device address up
 *     (hipGetSymbolAddress, device switched to the stream's device and back)
 *     and may load its code object: make that first call outside stream
 *     capture.
 *   - KK_ERR_WORKSPACE_TOO_SMALL, with nothing enqueued, when the step needs
 *     more than KK_NOALLOC_SCRATCH_BYTES (kk_decode_workspace_bytes with the
 *     same batch, max_seq_len and split_tokens on the same device); pass a
 *     larger split_tokens or use kk_decode_attn.
 *   - Every call on one device shares that device's array: calls that overlap
 *     in time on one device (two streams, or two host threads) race and give
 *     wrong results.  Calls on one stream are ordered and safe.  Nothing in
 *     the array has to start at zero: each step writes every partial it reads.
 *   - KK_ERR_UNSUPPORTED for device ordinals >= 64. */
kk_status kk_decode_attn_noalloc(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                                 const int32_t* seq_lens, int32_t max_seq_len,
                                 const void* q_lat, const void* q_rope, kk_dtype q_dtype, float* out,
                                 int32_t split_tokens, hipStream_t stream);

/* One generated token per sequence: append it to every anchor cache, then
 * attend (the decode step right after the write; KV-Kaizen summary page,
 * "Background: The KV Cache Bottleneck": every new token is cached and then
 * the whole cache is read).
 *
 * seq_lens   : device int32 [batch], lengths AFTER the append.  For each s
 *              with 1 <= seq_lens[s] <= t_cap and each anchor a, row
 *              seq_lens[s] - 1 of sequence s in a's cache is written with the
 *              quantized [new_latent[a][s][0:d_a] || new_rope[a][s]] (as
 *              kk_quantize_write would); other sequences append nothing.
 * new_latent : device [n_layers][batch][r], src_dtype (rows of inheriting
 *              layers are not read).
 * new_rope   : device [n_layers][batch][d_rope], src_dtype.
 * Every other argument is as for kk_decode_attn, which then runs over the
 * extended caches.  All checks of both steps happen before anything is
 * enqueued; the write and the decode go to `stream` in that order (two
 * launches, no host synchronization). */
kk_status kk_append_decode(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                           const int32_t* seq_lens, int32_t max_seq_len, const void* new_latent,
                           const void* new_rope, kk_dtype src_dtype, const void* q_lat, const void* q_rope,
                           kk_dtype q_dtype, float* out, int32_t split_tokens, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---- Heterogeneous tables in one batch -------------------------------------
 * The selector chooses a table per prompt, from that prompt's context, before
 * its pre-fill (KV-Kaizen summary page, "Selector Architecture and Training":
 * the context-adaptive selector and its Inference item), so the sequences of
 * one serving batch can carry different tables.  One call decodes them all in
 * one fused launch.
 *
 * The batch is cut into n_tables contiguous runs of sequences: run k holds
 * tables[k].batch sequences, starting at the sum of the earlier runs' sizes,
 * and is decoded exactly as kk_decode_attn would decode it with table
 * tables[k].cfg over caches tables[k].caches (whose sequence index is the
 * position within the run).  Every table has the same n_layers, n_heads, r
 * and d_rope (they describe one model); anchors, widths, precisions and
 * softmax scales may differ.  One table per sequence is n_tables = batch. */
typedef struct {
  const kk_model_cfg* cfg;     /* the table (host) */
  int32_t batch;               /* sequences of the run, >= 1 */
  const kk_cache* caches;      /* host [n_layers]: the run's anchor caches, each
                                  [batch][t_cap] as for kk_decode_attn (may be
                                  NULL for the size queries) */
} kk_table_batch;

/* Float offsets of the output blocks: offsets[k * n_layers + l] is where layer
 * l of run k starts, as [tables[k].batch][n_heads][d_eff(k, l)] float32;
 * offsets[n_tables * n_layers] = total floats.  Host array. */
kk_status kk_multi_out_offsets(const kk_table_batch* tables, int32_t n_tables, int64_t* offsets);

/* Workspace bytes of kk_multi_decode_attn (always > 0: the work plan lives in
 * the workspace next to the split partials). */
kk_status kk_multi_decode_workspace_bytes(const kk_table_batch* tables, int32_t n_tables, int32_t max_seq_len,
                                          int32_t split_tokens, size_t* bytes);

/* One decode step over a heterogeneous batch of B = sum of tables[k].batch
 * sequences.
 * seq_lens : device int32 [B], clamped to [0, t_cap] as for kk_decode_attn.
 * q_lat    : device [n_layers][B][n_heads][r], q_dtype.
 * q_rope   : device [n_layers][B][n_heads][d_rope], q_dtype.
 * out      : device float32, packed as kk_multi_out_offsets describes.
 * workspace: device, >= kk_multi_decode_workspace_bytes, 256-byte aligned.
 *            The call first writes its work plan into the workspace (small
 *            launches whose arguments carry it), then decodes; calls that
 *            share a workspace must be ordered on one stream.
 * max_seq_len and split_tokens as for kk_decode_attn.  Results for a run are
 * those kk_decode_attn gives for it alone, within floating-point rounding
 * (the split choice depends on the whole batch). */
kk_status kk_multi_decode_attn(const kk_table_batch* tables, int32_t n_tables, int32_t t_cap, const int32_t* seq_lens,
                               int32_t max_seq_len, const void* q_lat, const void* q_rope, kk_dtype q_dtype,
                               float* out, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* ---- Grouped-query (non-MLA) cache: precision + depth --------------------------
 * The same per-layer table on a model without a latent: an anchor caches its
 * keys K and values V per KV head at b bits, later layers may inherit an
 * anchor's cache; there is no rank axis (KV-Kaizen summary page: the "Precision
 * (non-MLA)", "Depth (non-MLA)" and "Precision + depth" rows of Table 1, the
 * KVK 4x row of Table 2; the non-MLA cost C0 = L * 2 * n_kv * d_h * 16 bits of
 * "Action Space and Cost Model").
 *
 * Layout (one anchor): codes uint8 [batch][n_kv][t_cap][row_stride], one row
 * per (sequence, KV head, token) holding 2 d_h fields, the head's values then
 * its keys ([V_g || K_g], fields packed as for the latent cache, b = 16 as two
 * byte planes); row_stride = kk_row_stride_bytes(d_h, d_h, b).  scales float32
 * [batch][n_kv][t_cap]: one scale per token over its K and V of every KV head
 * (amax / qmax, as for the latent cache), repeated for each KV head's row.
 *
 * Decode, for layer l with anchor a, sequence s, query head h and its KV head
 * g = h / (n_q_heads / n_kv_heads), over t < len_s:
 *   z_t = sm_scale_l * q[l,s,h,:] . K_a[s,g,t,:],  out[l,s,h,:] = sum_t softmax(z)_t V_a[s,g,t,:]
 * (dequantized codes).  Keys are cached after RoPE. */
typedef struct {
  int32_t n_layers;             /* 1 .. KK_MAX_LAYERS */
  int32_t n_q_heads;            /* H, a multiple of n_kv_heads */
  int32_t n_kv_heads;           /* n_kv */
  int32_t d_head;               /* d_h: 64 or 128 */
  const kk_layer_cfg* layers;   /* host [n_layers]: anchor, bits and sm_scale as for
                                   kk_layer_cfg; d is ignored (every coordinate kept) */
} kk_gqa_cfg;

/* Bytes of anchor `layer`'s codes and scales for [batch][n_kv][t_cap]. */
kk_status kk_gqa_cache_bytes(const kk_gqa_cfg* cfg, int32_t layer, int32_t batch, int32_t t_cap,
                             size_t* codes_bytes, size_t* scales_bytes);

/* Quantize-and-pack write of anchor `layer`: token i reads k and v row
 * src_index[i] (nullable: identity), each [n_src][n_kv][d_h] contiguous
 * `src_dtype` (4-byte aligned for f32), and writes position dst_slot[i] =
 * seq * t_cap + pos of every KV head.  Out-of-range tokens are skipped; two
 * tokens writing one slot race. */
kk_status kk_gqa_quantize_write(const kk_gqa_cfg* cfg, int32_t layer, const void* k, const void* v,
                                kk_dtype src_dtype, int64_t n_src, int32_t n_tokens, const int32_t* src_index,
                                const int64_t* dst_slot, kk_cache dst, int32_t batch, int32_t t_cap,
                                hipStream_t stream);

/* Workspace bytes of kk_gqa_decode_attn (0 when no sequence is split). */
kk_status kk_gqa_decode_workspace_bytes(const kk_gqa_cfg* cfg, int32_t batch, int32_t max_seq_len,
                                        int32_t split_tokens, size_t* bytes);

/* One decode step of every layer.
 * q   : device [n_layers][batch][n_q_heads][d_h], q_dtype, 16-byte aligned.
 * out : device float32 [n_layers][batch][n_q_heads][d_h].
 * caches, seq_lens, max_seq_len, split_tokens, workspace: as for kk_decode_attn. */
kk_status kk_gqa_decode_attn(const kk_gqa_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                             const int32_t* seq_lens, int32_t max_seq_len, const void* q, kk_dtype q_dtype,
                             float* out, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ---- Latent epilogue ---------------------------------------------------------
 * Absorbed-MLA decode returns each head's output in the latent space (a
 * weighted sum of the cached latents c^KV, truncated to the d_eff kept
 * coordinates: KV-Kaizen summary page, "Three Non-Eviction Compression
 * Axes", rank item).  The epilogue maps it to the model's output: head h's
 * value is its block of the value up-projection on the kept coordinates, and
 * the output projection mixes the heads.  For every layer l, sequence s:
 *   v[l,s,h,j] = sum_{i < d_eff(l)} W_UV[l][h*d_v + j][i] * o_lat[l,s,h,i]
 *   y[l,s,n]   = sum_{h, j} W_O[l][n][h*d_v + j] * v[l,s,h,j]
 * Every layer has its own weights (inheriting layers share a cache, not
 * weights).
 *
 * o_lat : device float32, packed as kk_out_offsets (the kk_decode_attn output).
 * w_uv  : host array [n_layers] of device bf16 pointers; layer l's is
 *         [n_heads * d_v][r] row-major (the full up-projection; columns
 *         d_eff(l) .. r-1 are not read).  16-byte aligned.
 * w_o   : host array [n_layers] of device bf16 pointers; layer l's is
 *         [d_model][n_heads * d_v] row-major.  16-byte aligned.
 * v     : device float32 [n_layers][batch][n_heads * d_v] (written: the
 *         per-head values).
 * y     : device float32 [n_layers][batch][d_model] (written).
 * d_v, d_model: multiples of 8.
 * Arithmetic: the bf16 weights are used exactly; each fp32 activation enters
 * as the sum of two bf16 parts (16 significant bits); products accumulate in
 * fp32.  Two launches on `stream` (up-projection of all layers, then output
 * projection of all layers); no workspace. */
kk_status kk_latent_epilogue(const kk_model_cfg* cfg, int32_t batch, int32_t d_v, int32_t d_model,
                             const float* o_lat, const void* const* w_uv, const void* const* w_o, float* v, float* y,
                             hipStream_t stream);

/* Static description of a status code. */
const char* kk_status_string(kk_status status);

#ifdef __cplusplus
}
#endif

#endif /* KK_H_ */
