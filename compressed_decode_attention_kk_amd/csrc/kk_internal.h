// Internal launch descriptors shared by the host planner and the gfx950
// kernels of the compressed decode-attention library.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kk {

// ---- decode kernel geometry -------------------------------------------------
constexpr int kWaves = 4;            // waves per workgroup (256 threads)
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;            // token granularity of splits (tiles are 32 or 16 tokens)
constexpr int kMaxRowBlocks = 3;     // 16-row MFMA blocks per work item (<= 48 query rows)
constexpr int kMaxMergeSplits = 64;  // token splits of one sequence
constexpr int kMaxMergeParts = 4;    // merge workgroups of one (entry, sequence, row chunk)
constexpr int kMaxK = 576;           // d + d_R (the ABI limit)
constexpr int kMaxEntries = 88;      // group entries held in the launch arguments
constexpr int kMaxLayers = 64;
// Decode kernel variants (register budgets) and workgroups per CU: kFull, any
// latent row (256 VGPRs: two workgroups, the second hides the fixed latencies
// of the first); kLean, steps whose anchors all have d <= 256 and at most
// five 64-field Q.K chunks, in items of at most 2 row blocks (three); kGqa,
// grouped-query rows (four).
constexpr int kFull = 0, kLean = 1, kGqa = 2;
constexpr int decode_wg_per_cu(int variant) { return variant == kGqa ? 4 : variant == kLean ? 3 : 2; }
constexpr int kLeanMaxD = 256, kLeanMaxChunks = 5;
// Q.K chunks of a row: the latent part and the RoPE part, each in chunks of 64 fields
constexpr int qk_chunks_of(int d, int d_rope) { return ((d + 63) >> 6) + ((d_rope + 63) >> 6); }
constexpr int kMaxQkChunks = (kMaxK + 63) / 64;
constexpr float kLazyRescale = 8.0f; // log2 headroom before the running max is moved

// One layer of one table: softmax scale, kept width of its anchor and the
// float offset of its block in the packed output.
struct LayerArg {
  float sm_scale;
  int32_t d_eff;
  int64_t out_off;
};

// One group entry: the query rows [row_begin, row_end) of one anchor group
// (an anchor and the layers that inherit its cache) of one table, cut into nrc
// chunks of at most 64 rows, over the n_seq sequences [seq_base, seq_base +
// n_seq) of the batch that use the table; every (chunk, sequence, split)
// triple is one work item.  The cache holds those sequences at indices
// [0, n_seq); the layers of the group are group_layers[lay_begin ...], indices
// into the layer array whose table starts at layer_base (model layer =
// index - layer_base).
struct EntryArg {
  const uint8_t* codes;
  const float* scales;
  int64_t ws_off;        // float offset of this entry's split partials
  int32_t item_base;     // first work item (decode kernel block)
  int32_t merge_base;    // first merge block (monotone over entries)
  int32_t row_stride;    // bytes per cached row
  int32_t row_begin, row_end;
  int32_t seq_base, n_seq;
  int32_t lay_begin, layer_base;
  int16_t d, bits;
  int16_t nrc, chunk_rows;
  int16_t splits;
  int8_t nbuf;           // LDS tile buffers of this entry (nbuf - 1 tiles in flight)
  int8_t qk_c0;          // first 64-field chunk of the row that enters Q.K (the
                         // fields before it are values only: grouped-query rows
                         // [V || K]); 0 for latent rows
};

// The entry, layer and group-layer arrays sit in the launch arguments for one
// table; for several tables they sit in device memory (plan != nullptr).
struct DevicePlan {
  const EntryArg* entries;
  const LayerArg* layers;
  const uint16_t* group_layers;
};

struct DecodeArgs {
  const void* q_lat;
  const void* q_rope;
  float* out;
  float* ws;
  const int32_t* seq_lens;
  DevicePlan plan;                    // entries == nullptr: the arrays below
  int32_t batch, heads, r, d_rope, t_cap;
  int32_t n_entries, total_items;
  int32_t q_is_f32;
  int32_t seq_div;                    // sequence s reads seq_lens[s / seq_div] (grouped-query: n_kv)
  int32_t merge_parts;                // merge workgroups per (entry, sequence, row chunk), feature ranges
  uint16_t group_layers[kMaxLayers];  // layers ordered by group
  LayerArg layers[kMaxLayers];
  EntryArg entries[kMaxEntries];
};

// Partial slot of one work item in the workspace (float offsets):
//   [0, 32d)        O/l as fp16 [64 rows][d], in units of the slot scale
//   32d + [0, 64)   m, the row max (log2 domain)
//   32d + [64, 128) l, the row sum of 2^(z - m)
//   32d + 128       the slot scale 2^(E+6) (E bounds the item's token scales)
__host__ __device__ inline int64_t partial_slot_floats(int d) { return 32 * (int64_t)d + 192; }
__host__ __device__ inline int64_t partial_ml_offset(int d) { return 32 * (int64_t)d; }

struct WriteArgs {
  const void* latent;
  const void* rope;
  const int32_t* src_index;
  const int64_t* dst_slot;
  uint8_t* codes;
  float* scales;
  int64_t latent_ld, rope_ld, n_src, n_slots;
  int32_t n_tokens, d, d_rope, bits, row_stride, src_bf16;
};

hipError_t launch_write(const WriteArgs& a, hipStream_t stream);

// Grouped-query writer: one scale per token over its K and V of every KV
// head; row (seq * n_kv + g) * t_cap + pos holds [V_g || K_g].
struct GqaWriteArgs {
  const void* k;             // [n_src][n_kv][d_h]
  const void* v;
  const int32_t* src_index;
  const int64_t* dst_slot;   // seq * t_cap + pos
  uint8_t* codes;
  float* scales;
  int64_t n_src, n_slots;
  int32_t n_tokens, n_kv, d_head, bits, row_stride, t_cap, src_bf16;
};
hipError_t launch_gqa_write(const GqaWriteArgs& a, hipStream_t stream);

// Append of one token per sequence to every anchor cache (see kk_append_decode).
struct AppendAnchor {
  uint8_t* codes;
  float* scales;
  int32_t layer, d, bits, row_stride;
};
struct AppendArgs {
  const void* latent;        // [n_layers][batch][latent_ld]
  const void* rope;          // [n_layers][batch][rope_ld]
  const int32_t* seq_lens;   // lengths after the append
  int64_t latent_ld, rope_ld;
  int32_t n_anchors, batch, t_cap, d_rope, src_bf16;
  AppendAnchor anchors[kMaxLayers];
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// Latent epilogue: batched skinny products Y[b][n] = sum_k X[b][k] W[n][k]
// (X fp32 [batch][ldx], W bf16 [N][ldw], Y fp32 [batch][ldy]), one problem
// per layer, `heads` copies per problem at the given element strides.  Each
// wave computes 64 rows n of one copy for the whole batch.
struct GemmProblem {
  const float* x;
  const uint16_t* w;
  float* y;
  int64_t ldx, ldw, ldy;
  int64_t x_hs, w_hs, y_hs;      // strides between the heads' copies
  int32_t n, k, heads;
  int32_t n_tiles;               // ceil(n / 64)
  int32_t wave_base;             // first wave of this problem
};
struct EpiArgs {
  int32_t n_probs, total_waves, batch, pad_;
  GemmProblem p[kMaxLayers];
};
hipError_t launch_epilogue_gemm(const EpiArgs& a, hipStream_t stream);
// Single-copy problems (heads == 1): workgroups of 256 rows sharing the
// activations through LDS; wave_base / total_waves count workgroups
// (n_tiles = ceil(n / 256)).
hipError_t launch_epilogue_gemm_wide(const EpiArgs& a, hipStream_t stream);

// One decode launch covers every work item of the step (all bit widths).
struct DecodeLaunch {
  int items;
  int lds_bytes;         // dynamic LDS per workgroup: the largest entry's need
  int row_blocks;        // 16-row MFMA blocks per item (1..3), uniform for the step
  int merge_blocks;
  int merge_parts = 1;   // merge workgroups per (entry, sequence, row chunk)
  int variant = kFull;   // kernel variant (kGqa: row_blocks <= 2)
};

// ---- LDS map of the decode kernel (bytes of dynamic shared memory) ----------------
//  [0, nbuf*buf)  tile buffers: codes of token block 0 [| block 1] | slack | scales
//  pbuf           P' fragments [tile parity][row block][64 lanes] 8 B per 16 tokens
//  alpha[2][64] flags[2][4] ml[64][2] misc[16]
constexpr int kMiscBytes = 2 * 64 * 4 + 2 * 4 * 4 + 64 * 8 + 64;
__host__ __device__ inline int pbuf_bytes(int rb, int tile_blocks) { return 2 * rb * 64 * 8 * tile_blocks; }

__host__ __device__ inline int nseg_of(int row_stride) { return row_stride >> 4; }
// 16-byte segments a tile row needs for the Q.K reads: latent chunks read 64
// fields from field 0, RoPE chunks 64 fields from field d, so reads reach field
// F = max(64 * latent chunks, d + 64 * RoPE chunks) (past the row's own fields
// they meet zero query values); b = 16 reads both byte planes (low plane at K).
__host__ __device__ inline int nsegpad_of(int d, int d_rope, int bits) {
  const int fl = ((d + 63) >> 6) * 64, fr = d + ((d_rope + 63) >> 6) * 64;
  const int F = fl > fr ? fl : fr;
  return bits == 16 ? (d + d_rope + F + 15) >> 4 : (F * bits / 8 + 15) >> 4;
}
// 16-token blocks per tile: 32 tokens of b <= 8 codes, 16 tokens of b = 16 codes
__host__ __device__ inline int tile_blocks_of(int bits) { return bits == 16 ? 1 : 2; }
// Tile buffer: all but the last token block at full pitch, the last one padded
// for whole-chunk Q.K reads, then the tile's fp32 scales (4 bytes per token).
__host__ __device__ inline int tilebuf_bytes(int row_stride, int d, int d_rope, int bits) {
  const int nseg = nseg_of(row_stride), pad = nsegpad_of(d, d_rope, bits), tb = tile_blocks_of(bits);
  return ((tb - 1) * nseg + (pad > nseg ? pad : nseg)) * 256 + 64 * tb;
}
// Tile buffers of an entry: as many as fit in the LDS share of one workgroup
// (160 KiB per CU over the variant's workgroups), 3 to 12.
inline int decode_nbuf(int row_stride, int d, int d_rope, int bits, int row_blocks, int variant) {
  const int budget =
      160 * 1024 / decode_wg_per_cu(variant) - pbuf_bytes(row_blocks, tile_blocks_of(bits)) - kMiscBytes;
  const int n = budget / tilebuf_bytes(row_stride, d, d_rope, bits);
  return n < 3 ? 3 : (n > 12 ? 12 : n);
}
inline int decode_lds_bytes(int row_stride, int d, int d_rope, int bits, int row_blocks, int variant) {
  return decode_nbuf(row_stride, d, d_rope, bits, row_blocks, variant) * tilebuf_bytes(row_stride, d, d_rope, bits) +
         pbuf_bytes(row_blocks, tile_blocks_of(bits)) + kMiscBytes;
}
hipError_t launch_decode(const DecodeArgs& a, const DecodeLaunch& L, hipStream_t stream);
// One decode kernel variant (RB row blocks, register budget V).
template <int RB, int V>
hipError_t launch_decode_items(const DecodeArgs& a, int n, int lds, hipStream_t stream);

// Copies `words` 32-bit words from host memory to device memory `dst` by
// kernel launches whose arguments carry the data (stream-ordered, no host
// memory has to outlive the call).
hipError_t launch_store(uint32_t* dst, const uint32_t* words, int64_t n_words, hipStream_t stream);

}  // namespace kk
