// Host side of the C ABI: validation, per-layer table resolution, the work
// plan of one decode step, and kernel launches.  Nothing here allocates
// device memory, synchronizes or keeps state between calls (plans live in
// host memory local to the call).
//
// Table semantics follow the KV-Kaizen summary page (picx.dev): "Action Space
// and Cost Model" (actions {inherit} U {(d, b)}, b in {2, 4, 8, 16}) and
// "Three Non-Eviction Compression Axes" (inheriting layers read an anchor's
// cache; the cache keeps the first d latent coordinates plus the RoPE key).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "kk.h"
#include "kk_internal.h"

static_assert(kk::kMaxK == KK_MAX_K && kk::kMaxLayers == KK_MAX_LAYERS, "ABI limits and kernel limits differ");

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_bits(int b) { return b == 2 || b == 4 || b == 8 || b == 16; }

// Layer table rules.  INVALID: breaks the method's rules; UNSUPPORTED: outside
// this library's limits.
kk_status check_model(const kk_model_cfg* c) {
  if (!c || !c->layers) return KK_ERR_INVALID_ARGUMENT;
  if (c->n_layers < 1 || c->n_heads < 1 || c->r < 1 || c->d_rope < 1) return KK_ERR_INVALID_ARGUMENT;
  if (c->n_layers > KK_MAX_LAYERS) return KK_ERR_UNSUPPORTED;
  if (c->r % 8 != 0 || c->d_rope % 16 != 0 || c->d_rope > 128) return KK_ERR_UNSUPPORTED;
  if (c->n_heads > 4096) return KK_ERR_UNSUPPORTED;
  for (int l = 0; l < c->n_layers; ++l) {
    const kk_layer_cfg& L = c->layers[l];
    if (!std::isfinite(L.sm_scale)) return KK_ERR_INVALID_ARGUMENT;
    if (L.anchor == l) {
      if (!valid_bits(L.bits) || L.d < 1 || L.d > c->r) return KK_ERR_INVALID_ARGUMENT;
      if (L.d % 16 != 0 || L.d > KK_MAX_D || L.d + c->d_rope > KK_MAX_K) return KK_ERR_UNSUPPORTED;
      if (kk::qk_chunks_of(L.d, c->d_rope) > kk::kMaxQkChunks) return KK_ERR_UNSUPPORTED;
    } else {
      if (l == 0 || L.anchor < 0 || L.anchor > l) return KK_ERR_INVALID_ARGUMENT;
      if (c->layers[L.anchor].anchor != L.anchor) return KK_ERR_INVALID_ARGUMENT;
    }
  }
  return KK_OK;
}

size_t stride_of(int d, int dr, int bits) {
  if (!valid_bits(bits) || d < 1 || dr < 0) return 0;
  const int64_t bitsum = (int64_t)(d + dr) * bits;
  if (bitsum % 8) return 0;
  return (size_t)((bitsum / 8 + 15) / 16 * 16);
}

// Compute units the automatic split choice plans for: those of the device that
// runs `stream` (the current device for a null stream).  Only automatic splits
// (split_tokens == 0) over a non-empty step depend on it; otherwise no device
// is queried.
kk_status plan_cus(hipStream_t stream, int split_tokens, int max_len, int* cus) {
  *cus = 1;
  if (split_tokens > 0 || max_len <= 0) return KK_OK;
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess) return KK_ERR_DEVICE;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || *cus < 1)
    return KK_ERR_DEVICE;
  return KK_OK;
}

// One table of the step: its layers, its caches and the sequences that use it.
struct TableRef {
  const kk_model_cfg* cfg;
  const kk_cache* caches;   // host [n_layers]; null while only sizes are planned
  int n_seq, seq_base;      // sequences [seq_base, seq_base + n_seq) of the batch
  int layer_base;           // first slot of the table's layers in the layer array
  int64_t out_base;         // float offset of the table's output block
  int qk_c0 = 0;            // first Q.K chunk of a row (grouped-query rows skip their values)
};

struct Plan {
  kk::DecodeArgs args;                 // one table: the arrays travel in here
  kk::DecodeLaunch launch;
  std::vector<kk::EntryArg> ents;
  std::vector<int> entry_anchor, entry_table;
  std::vector<kk::LayerArg> layers;    // slot = layer_base + layer
  std::vector<uint16_t> group_layers;
  int64_t ws_floats = 0;
};

int bits_class(int bits) { return bits == 2 ? 0 : bits == 4 ? 1 : bits == 8 ? 2 : 3; }

// Relative time of one 32-token tile of one work item: about equal for 2-, 4-
// and 8-bit codes (fixed per-tile work dominates), up to 1.7x for 16-bit codes,
// which stream 2-8x the bytes (measured on MI355X).
int64_t tile_cost(int bits, int d) { return 10 + (bits == 16 ? (7 * d + 511) / 512 : 0); }
constexpr int kItemWaves = 4;       // waves of items over the resident slots (mixed tables), at most
constexpr int kMergeBlocksPerCU = 4; // merge workgroups per compute unit below which merges are cut up
constexpr int kMinItemTiles = 96;   // ... fewer when items would average fewer tiles than this
constexpr int kMinSplitTiles = 8;   // no split shorter than 8 tiles (256 tokens)
constexpr int64_t kTailPercent = 15;  // share of the work (last dispatched) cut twice as fine
constexpr int64_t kItemOverhead = 40;   // per-item fixed cost (query setup, pipeline fill, stores)

// Work plan of one decode step.  Groups: an anchor and the layers inheriting
// its cache, per table.  Each group's query rows (layer-major, head-minor)
// form entries of <= 8 chunks of <= 64 rows; an item is (chunk, seq, split).
// Splits are chosen so that items carry similar byte counts; entries are
// ordered by bytes per item, largest first.  The tables share n_layers,
// n_heads, r and d_rope (checked by the callers).
kk_status make_plan(const std::vector<TableRef>& tabs, int max_len, int split_tokens, int n_cus, Plan& P) {
  const kk_model_cfg* c0 = tabs[0].cfg;
  const int H = c0->n_heads, L = c0->n_layers;
  P.layers.assign((size_t)tabs.size() * L, kk::LayerArg{});
  P.group_layers.clear();
  struct Ent {
    kk::EntryArg e;
    int anchor, table;
    int64_t cost_tile;     // relative time of one 32-token tile of one item
    int key_num, key_den;  // position of the entry in its bit width's order
  };
  std::vector<Ent> ents;
  // Row chunks: RB <= 3 blocks of 16 rows per item, RB fixed by the head
  // count; when a layer's heads fit in one item, chunks hold whole layers
  // (least padding), otherwise 48-row chunks run across layer boundaries.
  // (Four row blocks need more registers than a wave has: with their spills,
  // 64- and 128-head tables ran 1.1-2x slower than with 48-row chunks.)
  const int RB = std::min(kk::kMaxRowBlocks, (std::min(H, 64) + 15) / 16);
  const int chunk_rows = H <= 16 * RB ? H * ((16 * RB) / H) : 16 * RB;
  const int kEntryRows = 8 * chunk_rows;
  P.launch.row_blocks = RB;
  for (size_t ti = 0; ti < tabs.size(); ++ti) {
    const TableRef& T = tabs[ti];
    const kk_model_cfg* c = T.cfg;
    int64_t off = T.out_base;
    for (int l = 0; l < L; ++l) {
      const int a = c->layers[l].anchor;
      kk::LayerArg& la = P.layers[(size_t)T.layer_base + l];
      la.sm_scale = c->layers[l].sm_scale;
      la.d_eff = c->layers[a].d;
      la.out_off = off;
      off += (int64_t)T.n_seq * H * c->layers[a].d;
    }
    for (int a = 0; a < L; ++a) {
      if (c->layers[a].anchor != a) continue;
      const int begin = (int)P.group_layers.size();
      for (int l = a; l < L; ++l)
        if (c->layers[l].anchor == a) P.group_layers.push_back((uint16_t)(T.layer_base + l));
      const int rows = ((int)P.group_layers.size() - begin) * H;
      for (int rb = 0; rb < rows; rb += kEntryRows) {
        Ent E;
        std::memset(&E.e, 0, sizeof(E.e));
        E.e.d = (int16_t)c->layers[a].d;
        E.e.bits = (int16_t)c->layers[a].bits;
        E.e.row_stride = (int32_t)stride_of(c->layers[a].d, c->d_rope, c->layers[a].bits);
        E.e.row_begin = rb;
        E.e.row_end = std::min(rows, rb + kEntryRows);
        const int n = E.e.row_end - E.e.row_begin;
        E.e.nrc = (int16_t)((n + chunk_rows - 1) / chunk_rows);
        E.e.chunk_rows = (int16_t)chunk_rows;
        E.e.lay_begin = begin;
        E.e.layer_base = T.layer_base;
        E.e.seq_base = T.seq_base;
        E.e.n_seq = T.n_seq;
        E.e.qk_c0 = (int8_t)T.qk_c0;
        E.anchor = a;
        E.table = (int)ti;
        E.cost_tile = tile_cost(E.e.bits, E.e.d);
        ents.push_back(E);
      }
    }
  }

  // Splits: one launch runs every item, so items are sized by estimated time:
  // about kItemWaves waves of items over the resident workgroup slots, each at
  // least kMinSplitTiles tiles long.  Unsplit items need no merge pass.
  const int max_tiles = std::max(1, (max_len + kk::kTile - 1) / kk::kTile);
  int64_t total_cost = 0;
  for (auto& E : ents) total_cost += E.cost_tile * max_tiles * E.e.nrc * E.e.n_seq;
  // kernel variant: grouped-query rows, or every anchor narrow enough for the
  // lean register budget (items of <= 2 row blocks), or the full one
  int variant = tabs[0].qk_c0 > 0 ? kk::kGqa : RB <= 2 ? kk::kLean : kk::kFull;
  if (variant == kk::kLean)
    for (auto& T : tabs)
      for (int a = 0; a < L; ++a)
        if (T.cfg->layers[a].anchor == a &&
            (T.cfg->layers[a].d > kk::kLeanMaxD ||
             kk::qk_chunks_of(T.cfg->layers[a].d, T.cfg->d_rope) > kk::kLeanMaxChunks))
          variant = kk::kFull;
  P.launch.variant = variant;
  const int64_t slots = (int64_t)std::max(n_cus, 1) * kk::decode_wg_per_cu(variant);
  auto split_of = [&](const Ent& E, int waves) {
    const int64_t target = std::max<int64_t>(1, total_cost / (waves * slots));
    int64_t sp;
    if (split_tokens > 0) sp = (max_len + split_tokens - 1) / split_tokens;
    else sp = (E.cost_tile * max_tiles + target - 1) / target;
    if (split_tokens <= 0) sp = std::min<int64_t>(sp, std::max(1, max_tiles / kMinSplitTiles));
    sp = std::max<int64_t>(1, std::min<int64_t>(sp, max_tiles));
    return std::min<int64_t>(sp, kk::kMaxMergeSplits);
  };
  // Mixed tables: longest-first order leaves short items for the end, so few,
  // long items are best: kItemWaves waves, or fewer (down to 2) while the
  // average item would be shorter than kMinItemTiles (small batches, where the
  // per-item fixed cost and the split merges would weigh more).  When every
  // entry is alike, all items are equal and the last wave of items decides:
  // pick the wave count whose items fill whole waves best, i.e. the least
  // (waves of items) x (item time).
  int waves = kItemWaves;
  if (split_tokens <= 0) {
    for (; waves > 2; --waves) {
      int64_t work = 0, pieces = 0;
      for (auto& E : ents) {
        work += (int64_t)E.e.nrc * E.e.n_seq * max_tiles;
        pieces += (int64_t)E.e.nrc * E.e.n_seq * split_of(E, waves);
      }
      if (pieces == 0 || work >= kMinItemTiles * pieces) break;
    }
  }
  bool alike = split_tokens <= 0 && !ents.empty();
  for (auto& E : ents)
    alike = alike && E.e.bits == ents[0].e.bits && E.e.d == ents[0].e.d && E.e.nrc == ents[0].e.nrc;
  if (alike) {
    int64_t n_items_per_split = 0;
    for (auto& E : ents) n_items_per_split += (int64_t)E.e.nrc * E.e.n_seq;
    int64_t best = -1;
    for (int w = 4; w <= 8; ++w) {
      const int64_t sp = split_of(ents[0], w);
      const int64_t n = sp * n_items_per_split;
      const int64_t t = ((n + slots - 1) / slots) * (((max_tiles + sp - 1) / sp) * ents[0].cost_tile + kItemOverhead);
      if (best < 0 || t < best) { best = t; waves = w; }
    }
  }
  for (auto& E : ents) E.e.splits = (int16_t)split_of(E, waves);
  // Order: within a bit width, longest items first; the widths are interleaved
  // in proportion to their entry counts, so that the workgroups resident at
  // any time mix bandwidth-bound and arithmetic-bound items.
  std::stable_sort(ents.begin(), ents.end(), [](const Ent& x, const Ent& y) {
    if (x.e.bits != y.e.bits) return x.e.bits < y.e.bits;
    return x.cost_tile * y.e.splits > y.cost_tile * x.e.splits;
  });
  {
    int count[4] = {0, 0, 0, 0}, seen[4] = {0, 0, 0, 0};
    for (auto& E : ents) ++count[bits_class(E.e.bits)];
    for (auto& E : ents) {
      const int cl = bits_class(E.e.bits);
      E.key_num = 2 * seen[cl]++ + 1;
      E.key_den = 2 * count[cl];
    }
    std::stable_sort(ents.begin(), ents.end(), [](const Ent& x, const Ent& y) {
      return (int64_t)x.key_num * y.key_den < (int64_t)y.key_num * x.key_den;
    });
  }
  // Tail: the last items dispatched decide how evenly the slots finish, so the
  // entries holding the last kTailPercent of the work are cut twice as fine.
  if (!alike && split_tokens <= 0) {
    int64_t acc = 0;
    const int64_t tail_from = total_cost - total_cost * kTailPercent / 100;
    for (auto& E : ents) {
      if (acc >= tail_from)
        E.e.splits = (int16_t)std::min<int64_t>({2 * (int64_t)E.e.splits, std::max(1, max_tiles / kMinSplitTiles),
                                                 (int64_t)kk::kMaxMergeSplits});
      acc += E.cost_tile * max_tiles * E.e.nrc * E.e.n_seq;
    }
  }
  int64_t items = 0, ws = 0, merges = 0;
  kk::DecodeLaunch& Lc = P.launch;
  Lc.items = 0;
  Lc.lds_bytes = 0;
  P.ents.resize(ents.size());
  P.entry_anchor.resize(ents.size());
  P.entry_table.resize(ents.size());
  for (size_t i = 0; i < ents.size(); ++i) {
    kk::EntryArg& e = ents[i].e;
    e.codes = nullptr;
    e.scales = nullptr;
    e.item_base = (int32_t)std::min<int64_t>(items, 0x7fffffff);
    e.merge_base = (int32_t)std::min<int64_t>(merges, 0x7fffffff);
    items += (int64_t)e.nrc * e.n_seq * e.splits;
    if (e.splits > 1) {
      e.ws_off = ws;
      ws += (int64_t)e.nrc * e.n_seq * e.splits * kk::partial_slot_floats(e.d);
      merges += (int64_t)e.nrc * e.n_seq;
    }
    e.nbuf = (int8_t)kk::decode_nbuf(e.row_stride, e.d, c0->d_rope, e.bits, RB, variant);
    Lc.lds_bytes = std::max(Lc.lds_bytes, kk::decode_lds_bytes(e.row_stride, e.d, c0->d_rope, e.bits, RB, variant));
    if (Lc.lds_bytes > 160 * 1024 / kk::decode_wg_per_cu(variant)) return KK_ERR_UNSUPPORTED;
    P.ents[i] = e;
    P.entry_anchor[i] = ents[i].anchor;
    P.entry_table[i] = ents[i].table;
  }
  // A merge is a short chain of dependent loads.  When there are too few of
  // them to give every compute unit kMergeBlocksPerCU workgroups, each is cut
  // into feature ranges (the per-row weights are recomputed by every part).
  int parts = 1;
  if (merges > 0)
    parts = (int)std::min<int64_t>(kk::kMaxMergeParts,
                                   std::max<int64_t>(1, (kMergeBlocksPerCU * (int64_t)std::max(n_cus, 1) + merges - 1) / merges));
  if (items > 0x7fffffff || merges * parts > 0x7fffffff) return KK_ERR_UNSUPPORTED;
  for (auto& e : P.ents) e.merge_base *= parts;   // no overflow: merge_base <= merges
  merges *= parts;
  Lc.items = (int)items;
  Lc.merge_blocks = (int)merges;
  Lc.merge_parts = parts;
  P.ws_floats = ws;
  return KK_OK;
}

// Plan of one table whose arrays travel in the launch arguments.
kk_status make_single_plan(const kk_model_cfg* c, const kk_cache* caches, int batch, int max_len, int split_tokens,
                           int n_cus, Plan& P) {
  std::vector<TableRef> tabs{TableRef{c, caches, batch, 0, 0, 0}};
  const kk_status st = make_plan(tabs, max_len, split_tokens, n_cus, P);
  if (st != KK_OK) return st;
  if (P.ents.size() > (size_t)kk::kMaxEntries) return KK_ERR_UNSUPPORTED;
  kk::DecodeArgs& A = P.args;
  std::memset(&A, 0, sizeof(A));
  for (size_t i = 0; i < P.group_layers.size(); ++i) A.group_layers[i] = P.group_layers[i];
  for (size_t i = 0; i < P.layers.size(); ++i) A.layers[i] = P.layers[i];
  for (size_t i = 0; i < P.ents.size(); ++i) A.entries[i] = P.ents[i];
  A.n_entries = (int32_t)P.ents.size();
  A.total_items = P.launch.items;
  A.merge_parts = P.launch.merge_parts;
  return KK_OK;
}

}  // namespace

extern "C" {

size_t kk_row_stride_bytes(int32_t d, int32_t d_rope, int32_t bits) { return stride_of(d, d_rope, bits); }

kk_status kk_validate_model(const kk_model_cfg* cfg) { return check_model(cfg); }

kk_status kk_cache_bytes(const kk_model_cfg* cfg, int32_t layer, int32_t batch, int32_t t_cap, size_t* codes_bytes,
                         size_t* scales_bytes) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (layer < 0 || layer >= cfg->n_layers || cfg->layers[layer].anchor != layer) return KK_ERR_INVALID_ARGUMENT;
  if (batch < 1 || t_cap < 1 || !codes_bytes || !scales_bytes) return KK_ERR_INVALID_ARGUMENT;
  const kk_layer_cfg& L = cfg->layers[layer];
  *codes_bytes = (size_t)batch * (size_t)t_cap * stride_of(L.d, cfg->d_rope, L.bits);
  *scales_bytes = (size_t)batch * (size_t)t_cap * sizeof(float);
  return KK_OK;
}

kk_status kk_out_offsets(const kk_model_cfg* cfg, int32_t batch, int64_t* offsets) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (batch < 1 || !offsets) return KK_ERR_INVALID_ARGUMENT;
  int64_t off = 0;
  for (int l = 0; l < cfg->n_layers; ++l) {
    offsets[l] = off;
    off += (int64_t)batch * cfg->n_heads * cfg->layers[cfg->layers[l].anchor].d;
  }
  offsets[cfg->n_layers] = off;
  return KK_OK;
}

kk_status kk_quantize_write(const kk_model_cfg* cfg, int32_t layer, const void* latent, const void* rope,
                            kk_dtype src_dtype, int64_t latent_ld, int64_t rope_ld, int64_t n_src, int32_t n_tokens,
                            const int32_t* src_index, const int64_t* dst_slot, kk_cache dst, int32_t batch,
                            int32_t t_cap, hipStream_t stream) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (layer < 0 || layer >= cfg->n_layers || cfg->layers[layer].anchor != layer) return KK_ERR_INVALID_ARGUMENT;
  if (src_dtype != KK_DTYPE_F32 && src_dtype != KK_DTYPE_BF16) return KK_ERR_INVALID_ARGUMENT;
  if (n_tokens < 0 || n_src < 0 || batch < 1 || t_cap < 1) return KK_ERR_INVALID_ARGUMENT;
  const kk_layer_cfg& L = cfg->layers[layer];
  if (latent_ld < L.d || rope_ld < cfg->d_rope) return KK_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) return KK_OK;
  const size_t ea = src_dtype == KK_DTYPE_F32 ? 4 : 2;
  if (!latent || !rope || !dst_slot || !dst.codes || !dst.scales) return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(latent, ea) || !aligned(rope, ea) || !aligned(dst_slot, 8) || (src_index && !aligned(src_index, 4)))
    return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(dst.codes, 16) || !aligned(dst.scales, 16)) return KK_ERR_INVALID_ARGUMENT;
  kk::WriteArgs a;
  a.latent = latent;
  a.rope = rope;
  a.src_index = src_index;
  a.dst_slot = dst_slot;
  a.codes = dst.codes;
  a.scales = dst.scales;
  a.latent_ld = latent_ld;
  a.rope_ld = rope_ld;
  a.n_src = n_src;
  a.n_slots = (int64_t)batch * t_cap;
  a.n_tokens = n_tokens;
  a.d = L.d;
  a.d_rope = cfg->d_rope;
  a.bits = L.bits;
  a.row_stride = (int32_t)stride_of(L.d, cfg->d_rope, L.bits);
  a.src_bf16 = src_dtype == KK_DTYPE_BF16;
  return kk::launch_write(a, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

kk_status kk_decode_workspace_bytes(const kk_model_cfg* cfg, int32_t batch, int32_t max_seq_len,
                                    int32_t split_tokens, size_t* bytes) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (batch < 1 || max_seq_len < 0 || split_tokens < 0 || !bytes) return KK_ERR_INVALID_ARGUMENT;
  if (split_tokens % kk::kTile) return KK_ERR_INVALID_ARGUMENT;
  int cus = 1;
  st = plan_cus(nullptr, split_tokens, max_seq_len, &cus);
  if (st != KK_OK) return st;
  Plan P;
  st = make_single_plan(cfg, nullptr, batch, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  *bytes = (size_t)P.ws_floats * sizeof(float);
  return KK_OK;
}

kk_status kk_decode_plan_info(const kk_model_cfg* cfg, int32_t batch, int32_t max_seq_len, int32_t split_tokens,
                              int32_t n_cus, kk_plan_info* info) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (batch < 1 || max_seq_len < 0 || split_tokens < 0 || split_tokens % kk::kTile || n_cus < 0 || !info)
    return KK_ERR_INVALID_ARGUMENT;
  int cus = n_cus;
  if (cus == 0) {
    st = plan_cus(nullptr, 0, 1, &cus);
    if (st != KK_OK) return st;
  }
  Plan P;
  st = make_single_plan(cfg, nullptr, batch, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  info->n_cus = cus;
  info->work_items = P.launch.items;
  info->merge_blocks = P.launch.merge_blocks;
  info->max_splits = 0;
  for (const auto& e : P.ents) info->max_splits = std::max<int32_t>(info->max_splits, e.splits);
  info->workspace_bytes = (size_t)P.ws_floats * sizeof(float);
  return KK_OK;
}

namespace {
// Argument checks and work plan of one decode step (nothing is enqueued).
kk_status prepare_decode(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                         const int32_t* seq_lens, int32_t max_seq_len, const void* q_lat, const void* q_rope,
                         kk_dtype q_dtype, float* out, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, Plan& P) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (!caches || batch < 1 || t_cap < 1 || max_seq_len < 0 || max_seq_len > t_cap) return KK_ERR_INVALID_ARGUMENT;
  if (split_tokens < 0 || split_tokens % kk::kTile) return KK_ERR_INVALID_ARGUMENT;
  if (q_dtype != KK_DTYPE_F32 && q_dtype != KK_DTYPE_BF16) return KK_ERR_INVALID_ARGUMENT;
  if (!seq_lens || !q_lat || !q_rope || !out) return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(seq_lens, 4) || !aligned(q_lat, 16) || !aligned(q_rope, 16) || !aligned(out, 16))
    return KK_ERR_INVALID_ARGUMENT;
  for (int l = 0; l < cfg->n_layers; ++l) {
    if (cfg->layers[l].anchor != l) continue;
    if (!caches[l].codes || !caches[l].scales) return KK_ERR_INVALID_ARGUMENT;
    if (!aligned(caches[l].codes, 16) || !aligned(caches[l].scales, 16)) return KK_ERR_INVALID_ARGUMENT;
  }
  if ((int64_t)cfg->n_layers * batch * cfg->n_heads > ((int64_t)1 << 31)) return KK_ERR_UNSUPPORTED;
  int cus = 1;
  st = plan_cus(stream, split_tokens, max_seq_len, &cus);
  if (st != KK_OK) return st;
  st = make_single_plan(cfg, caches, batch, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  const size_t need = (size_t)P.ws_floats * sizeof(float);
  if (need > 0) {
    if (!workspace || !aligned(workspace, 256)) return KK_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return KK_ERR_WORKSPACE_TOO_SMALL;
  }
  kk::DecodeArgs& A = P.args;
  for (int i = 0; i < A.n_entries; ++i) {
    const int anchor = P.entry_anchor[i];
    A.entries[i].codes = caches[anchor].codes;
    A.entries[i].scales = caches[anchor].scales;
  }
  A.q_lat = q_lat;
  A.q_rope = q_rope;
  A.out = out;
  A.ws = static_cast<float*>(workspace);
  A.seq_lens = seq_lens;
  A.batch = batch;
  A.heads = cfg->n_heads;
  A.r = cfg->r;
  A.d_rope = cfg->d_rope;
  A.t_cap = t_cap;
  A.q_is_f32 = q_dtype == KK_DTYPE_F32;
  A.seq_div = 1;
  return KK_OK;
}
}  // namespace

namespace {
// Several tables: the tables' checks, their sequence ranges and output bases.
kk_status check_tables(const kk_table_batch* tables, int32_t n_tables, bool need_caches, std::vector<TableRef>& tabs,
                       int64_t* total_batch) {
  if (!tables || n_tables < 1) return KK_ERR_INVALID_ARGUMENT;
  if (n_tables > KK_MAX_TABLES) return KK_ERR_UNSUPPORTED;
  const kk_model_cfg* c0 = tables[0].cfg;
  int64_t seq = 0, out = 0;
  tabs.clear();
  for (int ti = 0; ti < n_tables; ++ti) {
    const kk_model_cfg* c = tables[ti].cfg;
    const kk_status st = check_model(c);
    if (st != KK_OK) return st;
    if (c->n_layers != c0->n_layers || c->n_heads != c0->n_heads || c->r != c0->r || c->d_rope != c0->d_rope)
      return KK_ERR_INVALID_ARGUMENT;
    const int b = tables[ti].batch;
    if (b < 1) return KK_ERR_INVALID_ARGUMENT;
    if (need_caches) {
      const kk_cache* cc = tables[ti].caches;
      if (!cc) return KK_ERR_INVALID_ARGUMENT;
      for (int l = 0; l < c->n_layers; ++l) {
        if (c->layers[l].anchor != l) continue;
        if (!cc[l].codes || !cc[l].scales) return KK_ERR_INVALID_ARGUMENT;
        if (!aligned(cc[l].codes, 16) || !aligned(cc[l].scales, 16)) return KK_ERR_INVALID_ARGUMENT;
      }
    }
    if (seq + b > 0x7fffffff) return KK_ERR_UNSUPPORTED;
    tabs.push_back(TableRef{c, tables[ti].caches, b, (int)seq, ti * c0->n_layers, out});
    seq += b;
    for (int l = 0; l < c->n_layers; ++l) out += (int64_t)b * c->n_heads * c->layers[c->layers[l].anchor].d;
  }
  if ((int64_t)c0->n_layers * seq * c0->n_heads > ((int64_t)1 << 31)) return KK_ERR_UNSUPPORTED;
  *total_batch = seq;
  return KK_OK;
}

// Workspace of a several-table step: the split partials, then the plan arrays
// (entries, layers, group layers), each part 256-byte aligned.
struct MultiLayout {
  size_t plan_off, lay_off, grp_off, total;
};
MultiLayout multi_layout(const Plan& P) {
  auto up = [](size_t x, size_t a) { return (x + a - 1) / a * a; };
  MultiLayout m;
  m.plan_off = up((size_t)P.ws_floats * sizeof(float), 256);
  m.lay_off = up(m.plan_off + P.ents.size() * sizeof(kk::EntryArg), 16);
  m.grp_off = m.lay_off + P.layers.size() * sizeof(kk::LayerArg);
  m.total = up(m.grp_off + P.group_layers.size() * sizeof(uint16_t), 256);
  return m;
}
}  // namespace

kk_status kk_multi_out_offsets(const kk_table_batch* tables, int32_t n_tables, int64_t* offsets) {
  std::vector<TableRef> tabs;
  int64_t total = 0;
  const kk_status st = check_tables(tables, n_tables, false, tabs, &total);
  if (st != KK_OK) return st;
  if (!offsets) return KK_ERR_INVALID_ARGUMENT;
  int64_t off = 0;
  size_t k = 0;
  for (auto& T : tabs)
    for (int l = 0; l < T.cfg->n_layers; ++l) {
      offsets[k++] = off;
      off += (int64_t)T.n_seq * T.cfg->n_heads * T.cfg->layers[T.cfg->layers[l].anchor].d;
    }
  offsets[k] = off;
  return KK_OK;
}

kk_status kk_multi_decode_workspace_bytes(const kk_table_batch* tables, int32_t n_tables, int32_t max_seq_len,
                                          int32_t split_tokens, size_t* bytes) {
  std::vector<TableRef> tabs;
  int64_t total = 0;
  kk_status st = check_tables(tables, n_tables, false, tabs, &total);
  if (st != KK_OK) return st;
  if (max_seq_len < 0 || split_tokens < 0 || split_tokens % kk::kTile || !bytes) return KK_ERR_INVALID_ARGUMENT;
  int cus = 1;
  st = plan_cus(nullptr, split_tokens, max_seq_len, &cus);
  if (st != KK_OK) return st;
  Plan P;
  st = make_plan(tabs, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  *bytes = multi_layout(P).total;
  return KK_OK;
}

kk_status kk_multi_decode_attn(const kk_table_batch* tables, int32_t n_tables, int32_t t_cap, const int32_t* seq_lens,
                               int32_t max_seq_len, const void* q_lat, const void* q_rope, kk_dtype q_dtype,
                               float* out, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  std::vector<TableRef> tabs;
  int64_t batch = 0;
  kk_status st = check_tables(tables, n_tables, true, tabs, &batch);
  if (st != KK_OK) return st;
  if (t_cap < 1 || max_seq_len < 0 || max_seq_len > t_cap) return KK_ERR_INVALID_ARGUMENT;
  if (split_tokens < 0 || split_tokens % kk::kTile) return KK_ERR_INVALID_ARGUMENT;
  if (q_dtype != KK_DTYPE_F32 && q_dtype != KK_DTYPE_BF16) return KK_ERR_INVALID_ARGUMENT;
  if (!seq_lens || !q_lat || !q_rope || !out) return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(seq_lens, 4) || !aligned(q_lat, 16) || !aligned(q_rope, 16) || !aligned(out, 16))
    return KK_ERR_INVALID_ARGUMENT;
  int cus = 1;
  st = plan_cus(stream, split_tokens, max_seq_len, &cus);
  if (st != KK_OK) return st;
  Plan P;
  st = make_plan(tabs, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  const MultiLayout m = multi_layout(P);
  if (!workspace || !aligned(workspace, 256)) return KK_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < m.total) return KK_ERR_WORKSPACE_TOO_SMALL;
  for (size_t i = 0; i < P.ents.size(); ++i) {
    const kk_cache& cc = tabs[P.entry_table[i]].caches[P.entry_anchor[i]];
    P.ents[i].codes = cc.codes;
    P.ents[i].scales = cc.scales;
  }
  // plan image, uploaded into the workspace ahead of the decode launch
  char* ws = static_cast<char*>(workspace);
  std::vector<uint32_t> img((m.total - m.plan_off) / sizeof(uint32_t), 0u);
  char* base = reinterpret_cast<char*>(img.data());
  std::memcpy(base, P.ents.data(), P.ents.size() * sizeof(kk::EntryArg));
  std::memcpy(base + (m.lay_off - m.plan_off), P.layers.data(), P.layers.size() * sizeof(kk::LayerArg));
  std::memcpy(base + (m.grp_off - m.plan_off), P.group_layers.data(), P.group_layers.size() * sizeof(uint16_t));
  kk::DecodeArgs& A = P.args;
  std::memset(&A, 0, sizeof(A));
  A.plan.entries = reinterpret_cast<const kk::EntryArg*>(ws + m.plan_off);
  A.plan.layers = reinterpret_cast<const kk::LayerArg*>(ws + m.lay_off);
  A.plan.group_layers = reinterpret_cast<const uint16_t*>(ws + m.grp_off);
  A.n_entries = (int32_t)P.ents.size();
  A.total_items = P.launch.items;
  A.merge_parts = P.launch.merge_parts;
  A.q_lat = q_lat;
  A.q_rope = q_rope;
  A.out = out;
  A.ws = reinterpret_cast<float*>(ws);
  A.seq_lens = seq_lens;
  A.batch = (int32_t)batch;
  A.heads = tabs[0].cfg->n_heads;
  A.r = tabs[0].cfg->r;
  A.d_rope = tabs[0].cfg->d_rope;
  A.t_cap = t_cap;
  A.q_is_f32 = q_dtype == KK_DTYPE_F32;
  A.seq_div = 1;
  if (A.n_entries == 0 || P.launch.items == 0) return KK_OK;
  if (kk::launch_store(reinterpret_cast<uint32_t*>(ws + m.plan_off), img.data(), (int64_t)img.size(), stream) !=
      hipSuccess)
    return KK_ERR_DEVICE;
  return kk::launch_decode(A, P.launch, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

kk_status kk_decode_attn(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                         const int32_t* seq_lens, int32_t max_seq_len, const void* q_lat, const void* q_rope,
                         kk_dtype q_dtype, float* out, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  Plan P;
  const kk_status st = prepare_decode(cfg, caches, batch, t_cap, seq_lens, max_seq_len, q_lat, q_rope, q_dtype, out,
                                      split_tokens, workspace, workspace_bytes, stream, P);
  if (st != KK_OK) return st;
  return kk::launch_decode(P.args, P.launch, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

kk_status kk_append_decode(const kk_model_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                           const int32_t* seq_lens, int32_t max_seq_len, const void* new_latent,
                           const void* new_rope, kk_dtype src_dtype, const void* q_lat, const void* q_rope,
                           kk_dtype q_dtype, float* out, int32_t split_tokens, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  // every check of both steps runs before anything is enqueued
  Plan P;
  kk_status st = prepare_decode(cfg, caches, batch, t_cap, seq_lens, max_seq_len, q_lat, q_rope, q_dtype, out,
                                split_tokens, workspace, workspace_bytes, stream, P);
  if (st != KK_OK) return st;
  if (src_dtype != KK_DTYPE_F32 && src_dtype != KK_DTYPE_BF16) return KK_ERR_INVALID_ARGUMENT;
  const size_t ea = src_dtype == KK_DTYPE_F32 ? 4 : 2;
  if (!new_latent || !new_rope || !aligned(new_latent, ea) || !aligned(new_rope, ea)) return KK_ERR_INVALID_ARGUMENT;
  kk::AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.latent = new_latent;
  a.rope = new_rope;
  a.seq_lens = seq_lens;
  a.latent_ld = cfg->r;
  a.rope_ld = cfg->d_rope;
  a.batch = batch;
  a.t_cap = t_cap;
  a.d_rope = cfg->d_rope;
  a.src_bf16 = src_dtype == KK_DTYPE_BF16;
  for (int l = 0; l < cfg->n_layers; ++l) {
    if (cfg->layers[l].anchor != l) continue;
    kk::AppendAnchor& x = a.anchors[a.n_anchors++];
    x.codes = caches[l].codes;
    x.scales = caches[l].scales;
    x.layer = l;
    x.d = cfg->layers[l].d;
    x.bits = cfg->layers[l].bits;
    x.row_stride = (int32_t)stride_of(x.d, cfg->d_rope, x.bits);
  }
  if (kk::launch_append(a, stream) != hipSuccess) return KK_ERR_DEVICE;
  return kk::launch_decode(P.args, P.launch, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

namespace {
// Grouped-query tables run on the latent decode path: each (sequence, KV
// head) is one sequence of rows [V_g || K_g] (values = the first d_h fields,
// keys = the d_h fields after them, which alone enter Q.K), and its G = H /
// n_kv query heads are the rows of an item.
struct GqaModel {
  std::vector<kk_layer_cfg> layers;
  kk_model_cfg cfg;
};
kk_status gqa_model(const kk_gqa_cfg* c, GqaModel& m) {
  if (!c || !c->layers) return KK_ERR_INVALID_ARGUMENT;
  if (c->n_layers < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->d_head < 1) return KK_ERR_INVALID_ARGUMENT;
  if (c->n_q_heads % c->n_kv_heads) return KK_ERR_INVALID_ARGUMENT;
  if (c->d_head != 64 && c->d_head != 128) return KK_ERR_UNSUPPORTED;
  if (c->n_q_heads / c->n_kv_heads > 32) return KK_ERR_UNSUPPORTED;   // query rows of one KV head: <= 2 row blocks
  if (c->n_layers > KK_MAX_LAYERS) return KK_ERR_UNSUPPORTED;
  m.layers.resize(c->n_layers);
  for (int l = 0; l < c->n_layers; ++l) {
    m.layers[l] = c->layers[l];
    if (c->layers[l].anchor == l) m.layers[l].d = c->d_head;   // the cache keeps every key and value coordinate
  }
  m.cfg.n_layers = c->n_layers;
  m.cfg.n_heads = c->n_q_heads / c->n_kv_heads;
  m.cfg.r = c->d_head;
  m.cfg.d_rope = c->d_head;
  m.cfg.layers = m.layers.data();
  return check_model(&m.cfg);
}
}  // namespace

kk_status kk_gqa_cache_bytes(const kk_gqa_cfg* cfg, int32_t layer, int32_t batch, int32_t t_cap, size_t* codes_bytes,
                             size_t* scales_bytes) {
  GqaModel m;
  const kk_status st = gqa_model(cfg, m);
  if (st != KK_OK) return st;
  if (layer < 0 || layer >= cfg->n_layers || cfg->layers[layer].anchor != layer) return KK_ERR_INVALID_ARGUMENT;
  if (batch < 1 || t_cap < 1 || !codes_bytes || !scales_bytes) return KK_ERR_INVALID_ARGUMENT;
  const size_t rows = (size_t)batch * cfg->n_kv_heads * (size_t)t_cap;
  *codes_bytes = rows * stride_of(cfg->d_head, cfg->d_head, cfg->layers[layer].bits);
  *scales_bytes = rows * sizeof(float);
  return KK_OK;
}

kk_status kk_gqa_quantize_write(const kk_gqa_cfg* cfg, int32_t layer, const void* k, const void* v, kk_dtype src_dtype,
                                int64_t n_src, int32_t n_tokens, const int32_t* src_index, const int64_t* dst_slot,
                                kk_cache dst, int32_t batch, int32_t t_cap, hipStream_t stream) {
  GqaModel m;
  const kk_status st = gqa_model(cfg, m);
  if (st != KK_OK) return st;
  if (layer < 0 || layer >= cfg->n_layers || cfg->layers[layer].anchor != layer) return KK_ERR_INVALID_ARGUMENT;
  if (src_dtype != KK_DTYPE_F32 && src_dtype != KK_DTYPE_BF16) return KK_ERR_INVALID_ARGUMENT;
  if (n_tokens < 0 || n_src < 0 || batch < 1 || t_cap < 1) return KK_ERR_INVALID_ARGUMENT;
  if (n_tokens == 0) return KK_OK;
  const size_t ea = src_dtype == KK_DTYPE_F32 ? 4 : 2;
  if (!k || !v || !dst_slot || !dst.codes || !dst.scales) return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(k, ea) || !aligned(v, ea) || !aligned(dst_slot, 8) || (src_index && !aligned(src_index, 4)))
    return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(dst.codes, 16) || !aligned(dst.scales, 16)) return KK_ERR_INVALID_ARGUMENT;
  kk::GqaWriteArgs a;
  a.k = k;
  a.v = v;
  a.src_index = src_index;
  a.dst_slot = dst_slot;
  a.codes = dst.codes;
  a.scales = dst.scales;
  a.n_src = n_src;
  a.n_slots = (int64_t)batch * t_cap;
  a.n_tokens = n_tokens;
  a.n_kv = cfg->n_kv_heads;
  a.d_head = cfg->d_head;
  a.bits = cfg->layers[layer].bits;
  a.row_stride = (int32_t)stride_of(cfg->d_head, cfg->d_head, a.bits);
  a.t_cap = t_cap;
  a.src_bf16 = src_dtype == KK_DTYPE_BF16;
  return kk::launch_gqa_write(a, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

kk_status kk_gqa_decode_workspace_bytes(const kk_gqa_cfg* cfg, int32_t batch, int32_t max_seq_len,
                                        int32_t split_tokens, size_t* bytes) {
  GqaModel m;
  kk_status st = gqa_model(cfg, m);
  if (st != KK_OK) return st;
  if (batch < 1 || max_seq_len < 0 || split_tokens < 0 || split_tokens % kk::kTile || !bytes)
    return KK_ERR_INVALID_ARGUMENT;
  if ((int64_t)batch * cfg->n_kv_heads > 0x7fffffff) return KK_ERR_UNSUPPORTED;
  int cus = 1;
  st = plan_cus(nullptr, split_tokens, max_seq_len, &cus);
  if (st != KK_OK) return st;
  Plan P;
  std::vector<TableRef> tabs{TableRef{&m.cfg, nullptr, batch * cfg->n_kv_heads, 0, 0, 0, cfg->d_head / 64}};
  st = make_plan(tabs, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  if (P.ents.size() > (size_t)kk::kMaxEntries) return KK_ERR_UNSUPPORTED;
  *bytes = (size_t)P.ws_floats * sizeof(float);
  return KK_OK;
}

kk_status kk_gqa_decode_attn(const kk_gqa_cfg* cfg, const kk_cache* caches, int32_t batch, int32_t t_cap,
                             const int32_t* seq_lens, int32_t max_seq_len, const void* q, kk_dtype q_dtype, float* out,
                             int32_t split_tokens, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  GqaModel m;
  kk_status st = gqa_model(cfg, m);
  if (st != KK_OK) return st;
  if (!caches || batch < 1 || t_cap < 1 || max_seq_len < 0 || max_seq_len > t_cap) return KK_ERR_INVALID_ARGUMENT;
  if (split_tokens < 0 || split_tokens % kk::kTile) return KK_ERR_INVALID_ARGUMENT;
  if (q_dtype != KK_DTYPE_F32 && q_dtype != KK_DTYPE_BF16) return KK_ERR_INVALID_ARGUMENT;
  if (!seq_lens || !q || !out || !aligned(seq_lens, 4) || !aligned(q, 16) || !aligned(out, 16))
    return KK_ERR_INVALID_ARGUMENT;
  for (int l = 0; l < cfg->n_layers; ++l) {
    if (cfg->layers[l].anchor != l) continue;
    if (!caches[l].codes || !caches[l].scales) return KK_ERR_INVALID_ARGUMENT;
    if (!aligned(caches[l].codes, 16) || !aligned(caches[l].scales, 16)) return KK_ERR_INVALID_ARGUMENT;
  }
  const int64_t nseq = (int64_t)batch * cfg->n_kv_heads;
  if (nseq > 0x7fffffff || (int64_t)cfg->n_layers * batch * cfg->n_q_heads > ((int64_t)1 << 31))
    return KK_ERR_UNSUPPORTED;
  int cus = 1;
  st = plan_cus(stream, split_tokens, max_seq_len, &cus);
  if (st != KK_OK) return st;
  Plan P;
  std::vector<TableRef> tabs{TableRef{&m.cfg, caches, (int)nseq, 0, 0, 0, cfg->d_head / 64}};
  st = make_plan(tabs, max_seq_len, split_tokens, cus, P);
  if (st != KK_OK) return st;
  if (P.ents.size() > (size_t)kk::kMaxEntries) return KK_ERR_UNSUPPORTED;
  const size_t need = (size_t)P.ws_floats * sizeof(float);
  if (need > 0) {
    if (!workspace || !aligned(workspace, 256)) return KK_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return KK_ERR_WORKSPACE_TOO_SMALL;
  }
  kk::DecodeArgs& A = P.args;
  std::memset(&A, 0, sizeof(A));
  for (size_t i = 0; i < P.group_layers.size(); ++i) A.group_layers[i] = P.group_layers[i];
  for (size_t i = 0; i < P.layers.size(); ++i) A.layers[i] = P.layers[i];
  for (size_t i = 0; i < P.ents.size(); ++i) {
    A.entries[i] = P.ents[i];
    A.entries[i].codes = caches[P.entry_anchor[i]].codes;
    A.entries[i].scales = caches[P.entry_anchor[i]].scales;
  }
  A.n_entries = (int32_t)P.ents.size();
  A.total_items = P.launch.items;
  A.merge_parts = P.launch.merge_parts;
  A.q_lat = q;                 // the value chunks are skipped: never read as queries
  A.q_rope = q;                // [L][B][n_kv * G][d_h] = [L][B * n_kv][G][d_h]
  A.out = out;                 // [L][B * n_kv][G][d_h] = [L][B][H][d_h]
  A.ws = static_cast<float*>(workspace);
  A.seq_lens = seq_lens;
  A.batch = (int32_t)nseq;
  A.heads = m.cfg.n_heads;
  A.r = m.cfg.r;
  A.d_rope = m.cfg.d_rope;
  A.t_cap = t_cap;
  A.q_is_f32 = q_dtype == KK_DTYPE_F32;
  A.seq_div = cfg->n_kv_heads;
  return kk::launch_decode(A, P.launch, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

kk_status kk_latent_epilogue(const kk_model_cfg* cfg, int32_t batch, int32_t d_v, int32_t d_model,
                             const float* o_lat, const void* const* w_uv, const void* const* w_o, float* v, float* y,
                             hipStream_t stream) {
  kk_status st = check_model(cfg);
  if (st != KK_OK) return st;
  if (batch < 1 || d_v < 8 || d_model < 8 || d_v % 8 || d_model % 8) return KK_ERR_INVALID_ARGUMENT;
  if (!o_lat || !w_uv || !w_o || !v || !y) return KK_ERR_INVALID_ARGUMENT;
  if (!aligned(o_lat, 16) || !aligned(v, 16) || !aligned(y, 16)) return KK_ERR_INVALID_ARGUMENT;
  const int L = cfg->n_layers, H = cfg->n_heads;
  for (int l = 0; l < L; ++l) {
    if (!w_uv[l] || !w_o[l] || !aligned(w_uv[l], 16) || !aligned(w_o[l], 16)) return KK_ERR_INVALID_ARGUMENT;
  }
  const int64_t hv = (int64_t)H * d_v;
  const int64_t waves1 = (int64_t)L * H * ((d_v + 63) / 64), waves2 = (int64_t)L * ((d_model + 63) / 64);
  if (waves1 > 0x7ffffff || waves2 > 0x7ffffff || hv > 0x7fffffff) return KK_ERR_UNSUPPORTED;
  kk::EpiArgs up, out;
  std::memset(&up, 0, sizeof(up));
  std::memset(&out, 0, sizeof(out));
  up.n_probs = out.n_probs = L;
  up.batch = out.batch = batch;
  int64_t off = 0;
  for (int l = 0; l < L; ++l) {
    const int d = cfg->layers[cfg->layers[l].anchor].d;
    float* vl = v + (int64_t)l * batch * hv;
    kk::GemmProblem& p = up.p[l];              // v_h = W_UV[h][:, :d] o_h
    p.x = o_lat + off;
    p.ldx = (int64_t)H * d;
    p.x_hs = d;
    p.w = static_cast<const uint16_t*>(w_uv[l]);
    p.ldw = cfg->r;
    p.w_hs = (int64_t)d_v * cfg->r;
    p.y = vl;
    p.ldy = hv;
    p.y_hs = d_v;
    p.n = d_v;
    p.k = d;
    p.heads = H;
    p.n_tiles = (d_v + 63) / 64;
    p.wave_base = up.total_waves;
    up.total_waves += p.heads * p.n_tiles;
    kk::GemmProblem& q = out.p[l];             // y = W_O [v_1; ...; v_H]
    q.x = vl;
    q.ldx = hv;
    q.w = static_cast<const uint16_t*>(w_o[l]);
    q.ldw = hv;
    q.y = y + (int64_t)l * batch * d_model;
    q.ldy = d_model;
    q.n = d_model;
    q.k = (int32_t)hv;
    q.heads = 1;
    q.n_tiles = (d_model + 255) / 256;             // 256-row workgroups
    q.wave_base = out.total_waves;
    out.total_waves += q.n_tiles;
    off += (int64_t)batch * H * d;
  }
  if (kk::launch_epilogue_gemm(up, stream) != hipSuccess) return KK_ERR_DEVICE;
  return kk::launch_epilogue_gemm_wide(out, stream) == hipSuccess ? KK_OK : KK_ERR_DEVICE;
}

const char* kk_status_string(kk_status s) {
  switch (s) {
    case KK_OK: return "ok";
    case KK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KK_ERR_UNSUPPORTED: return "unsupported by this library";
    case KK_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KK_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

}  // extern "C"
