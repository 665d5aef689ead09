// Internal declarations shared by the host library (kvc_api.cpp, layout.cpp)
// and the kernels (kernels.hip).  Plain structs passed to kernels by value.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/kvc.h"

namespace kvc {

// Rows per V block: V is stored as [block][d][16 rows] so that a lane can read
// several consecutive keys of one head-dimension element with one load (the
// contraction dimension of P.V is the key axis).
constexpr int kVBlock = 16;
// Row counts are padded to a multiple of the chunk-attention key tile so that
// whole tiles can be loaded without bounds checks.
constexpr int kRowAlign = 32;
// Caps on split-K partial slots per query row.
constexpr int kDecodeSplitCap = 64;
// Keys per decode tile; decode splits are whole tiles.
constexpr int kDecodeTile = 16;
// Fewest tiles a planned decode split takes: short rows (ring layers) are not
// cut into splits so small that the merge costs more than the keys.
constexpr int kDecodeSplitMinTiles = 4;
constexpr int kChunkSplitCap = 16;
// Query rows per chunk-attention workgroup (8 waves x 32 rows).
constexpr int kChunkQTile = 256;

struct LayerLayout {
  int64_t k_off = 0, v_off = 0;           // byte offsets in the device buffer (paged: the pools)
  int32_t joint = -1;                     // partner layer of a joint softmax, or -1
  int32_t paged = 0;                      // full layout from a shared page pool
  int64_t sk_off = -1, sv_off = -1;       // staging (ring layers, max_chunk >= 2)
  int32_t hkv = 0, window = 0, ring = 0;  // ring: 0 < W < max_len and use_ring
  int32_t rows = 0;                       // W (ring) or max_len; scratch = rows
  int32_t rows_alloc = 0;                 // rows + 1 rounded up to kRowAlign
  int32_t stage_rows_alloc = 0;           // max_chunk rounded up to kRowAlign
};

struct Layout {
  std::vector<LayerLayout> layers;
  int64_t rope_off = -1;      // float2 (cos, sin) [max_len][D/2], fp32
  int64_t lens_off = 0;       // int32 [B]
  int64_t nnew_off = 0;       // int32 [B]
  int64_t first_off = 0;      // int32 [B]: left padding per row
  int64_t dml_off = 0;        // float2 (m, l) [B][Hq][kDecodeSplitCap]
  int64_t dout_off = 0;       // float [B][Hq][kDecodeSplitCap][D]
  int64_t cnt_off = 0;        // int32 [B][max Hkv]: split arrivals (fused decode), 0 between launches
  int64_t cnt_bytes = 0;
  int64_t flags_off = 0;      // int32: sticky error bits of static steps
  // paged caches: pages per pool (the zero page and the scratch page follow),
  // block-table entries per row, the int32 block table [B][pages_per_row]
  // and the int32 rows each row may hold without new pages [B]
  int32_t n_pages = 0, pages_per_row = 0;
  int64_t table_off = -1, cap_off = -1;
  int64_t page_bytes = 0;     // per layer and KV head: 16 rows x D x dtype
  int64_t plan_off = 0;       // int32 [n_layer] split keys, then uint16 [n_layer][B] row orders
  int64_t pml_off = -1;       // float2 [B][max_chunk][Hq][kChunkSplitCap]
  int64_t pout_off = -1;      // float [B][max_chunk][Hq][kChunkSplitCap][D]
  int64_t total = 0;
  int64_t kv_bytes = 0;       // the pages' size formula, no scratch rows
};

// Validates cfg and fills *lay.  Returns KVC_OK or a negative status.
int compute_layout(const kvc_config *cfg, Layout *lay);
int dtype_bytes(int dtype);

// ---------------------------------------------------------------------------
// Kernel-side argument blocks
// ---------------------------------------------------------------------------
struct LayerArgs {
  char *k, *v;          // this layer's K and V region (paged: page pools)
  char *sk, *sv;        // staging K and V (nullptr when the layer has none)
  int32_t hkv, rep, window, ring, rows, rows_alloc, stage_rows_alloc;
  // Paged layer: storage row r of row b lives in page table[b * ppr + r / 16]
  // (row r % 16); the scratch row in page scratch_page.  Page pg of KV head g
  // holds 16 K rows (row-major) and one 16-row V block, at
  // ((pg * hkv + g) * 16) * D elements of the pools.
  int32_t paged;
  const int32_t *table;
  int32_t ppr, scratch_page;
};
constexpr int kPageRows = 16;

struct StepArgs {
  const int32_t *lens;    // device [B]
  const int32_t *n_new;   // device [B]
  const int32_t *first;   // device [B]: left padding (keys before it hidden)
  const float *rope;      // device float2 table or nullptr (no rotation)
  int32_t B, C, Hq, D, max_len;
};

// Joint attention (a layer whose softmax also covers a partner layer's
// keys): a query's partial slots hold the layer's own splits first, then the
// partner's.  A SplitRef describes one layer's splits so a kernel can count
// them for a row: decode splits of its span (dec_sk keys each), or for a
// chunk row its key splits (pre_sk keys each; 1 on a ring).
struct SplitRef {
  int32_t on, ring, window, dec_sk, pre_sk;
};

struct PartialArgs {
  float *dml, *dout;      // decode partials
  float *pml, *pout;      // chunk partials
  int32_t max_chunk;
  int32_t dec_split_keys; // keys per decode split (multiple of 32)
  int32_t pre_split_keys; // keys per chunk split (multiple of 32)
  // Decode dispatch: grid (KV heads, items) when dec_transpose, else (items,
  // KV heads); items in the row order dec_order[0..B) when dec_ordered
  // (B <= kDecodeOrderMax), else in row index order.  The host sets both.
  int32_t dec_transpose;
  int32_t dec_ordered;
  uint16_t dec_order[256];
  // A device-planned step (static one-token steps): the split length and the
  // row order come from device memory written by k_static_begin instead of
  // dec_split_keys / dec_order (null: host plan).
  const int32_t *dec_plan;
  const uint16_t *dec_order_dev;
  // 1: chunk rows of <= 128 query rows go to a 4-wave launch; 2: every
  // chunk row does (a ring layer whose 8-wave launch would not fill the CUs)
  int32_t chunk_small;
  // Non-null: every row of the step is a full chunk with one split (a ring
  // layer), and the chunk kernel writes the final outputs [B, C, Hq, D] here
  // instead of partials; no merge launch follows.
  void *direct_out;
  SplitRef base;   // a launch over the partner's keys: its slots follow these splits
  SplitRef joint;  // the combine: the partner's splits follow the layer's own
  // Non-null on a ring layer's chunk launches with staged rows: one counter
  // per (row, KV head), zero between launches; the last q tile of a (row,
  // KV head) to finish commits its staged rows to the ring.
  int32_t *ring_cnt;
  // Non-null (both) on a ring layer's chunk launches from the appending
  // entry: the chunk's own rows are read from the caller's K and V
  // [B, C, hkv, D] and rotated in the kernel instead of staged, and the
  // committing workgroup writes the kept rows to the ring from them, the
  // slot indices (slot_out, when non-null) and the zeroed V rows of a newly
  // entered tile.  Every row holds 2 .. kChunkOwnMax tokens.
  const void *ck, *cv;
  int32_t *slot_out;
};
// Most tokens per row the chunk kernel takes from the caller's K and V
// (two 32-row key tiles).
constexpr int kChunkOwnMax = 64;
constexpr int kDecodeOrderMax = 256;

// Static one-token steps.  Layers that plan alike (same KV heads, window and
// layout) form a class; k_static_begin checks the step's device counts and
// writes every class's split plan, the same one the host planner would make.
struct StaticClass {
  int32_t hkv, window, ring;
  int32_t target;     // waves in one round (resident decode waves x CUs)
  int32_t min_tiles;  // smallest split in tiles
  int32_t fixed_q;    // > 0: fixed split length in tiles (experiment override)
};
constexpr int kStaticClassMax = 16;
// Sticky error bits of static steps (the step is then run with every count 0).
constexpr int32_t kStaticBadCount = KVC_STATIC_BAD_COUNT;  // a count outside {0, 1}
constexpr int32_t kStaticFull = KVC_STATIC_FULL;          // a row would pass max_len
struct StaticBeginArgs {
  const int32_t *n_src;   // the caller's counts [B] (device)
  int32_t *n_new;         // the step's counts [B]
  const int32_t *lens;    // [B]
  const int32_t *first;   // [B]
  const int32_t *cap;     // [B] rows a paged row holds pages for, or null
  int32_t *flags;         // sticky error bits
  int32_t *plan_sk;       // [n_class] keys per split
  uint16_t *plan_order;   // [n_class][B] dispatch order, or null (B > kDecodeOrderMax)
  int32_t B, max_len, n_class;
  StaticClass cls[kStaticClassMax];
};

// The single-token step of one layer whose decode launch also appends (and,
// with the in-launch merge, combines): the new token's K (pre-RoPE) and V,
// the slot report, the output and the per-(row, KV head) split arrival
// counters of the in-launch merge (zero between launches).
struct FusedArgs {
  const void *k = nullptr, *v = nullptr;  // (B, 1, Hkv, D)
  int32_t *slot_out = nullptr;            // (B, 1) or null
  void *out = nullptr;                    // (B, 1, Hq, D)
  int32_t *cnt = nullptr;                 // [B][Hkv]
};

// Where a launch goes: the caller's stream and, when kernel timing is on, a
// pair of events the dispatch itself stamps at its start and end.
struct Launch {
  void *stream = nullptr;
  void *t0 = nullptr, *t1 = nullptr;  // hipEvent_t or null
};

// Launchers (kernels.hip).  Return hipError_t as int (0 = success).
int launch_set_rows(int32_t *dst, const int32_t *vals, int32_t n, void *stream);
// Empties rows: length and left padding 0.
int launch_reset_rows(int32_t *lens, int32_t *first, const int32_t *rows, int32_t n, void *stream);
// first[rows[i]] = vals[i].
int launch_set_first(int32_t *first, const int32_t *rows, const int32_t *vals, int32_t n,
                     void *stream);
// Row copies between two caches of the same layer shapes: per pair j, the
// first `blocks[j]` 16-row blocks of every KV head of row src_row[j] (K rows
// and V blocks, paged or not on either side), into row dst_row[j].
struct CopyPairs {
  int32_t src_row[64], dst_row[64], blocks[64];
};
int launch_copy_rows(const LayerArgs &dst, const LayerArgs &src, int D, int dtype_bytes,
                     const CopyPairs &pairs, int32_t n_pairs, void *stream);
// Paged caches: block-table updates (table[idx[i]] = page[i]) and the zeroing
// of V of newly taken pages (zero[i] >= 0) in every paged layer, whose V
// pools are listed with their KV heads.
struct PageUpdate {
  int32_t idx[64], page[64], zero[64];
};
struct PagedPools {
  char *v[64];
  int32_t hkv[64];
  int32_t n;
};
int launch_page_update(int32_t *table, int32_t *cap, const int32_t *cap_rows, const int32_t *cap_vals,
                       int32_t n_cap, const PageUpdate &u, int32_t n_upd, const PagedPools &pools,
                       int64_t page_bytes, void *stream);
// lens / first of dst_row[j] = those of src_row[j] (device arrays).
int launch_copy_state(int32_t *dst_lens, int32_t *dst_first, const int32_t *src_lens,
                      const int32_t *src_first, const CopyPairs &pairs, int32_t n_pairs,
                      void *stream);
int launch_advance(int32_t *lens, const int32_t *n_new, int32_t B, void *stream);
int launch_static_begin(const StaticBeginArgs &a, void *stream);
int launch_append(int dtype, const StepArgs &st, const LayerArgs &la, const void *k,
                  const void *v, int32_t *slot_out, const Launch &lc);
int launch_commit(int dtype, const StepArgs &st, const LayerArgs &la, const Launch &lc);
int launch_decode(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                  const void *q, int32_t n_items, const Launch &lc);
// Rows with n_new in {0, 1}, C == 1: RoPE + append and decode attention in
// one launch, and with `merge` the split combine too (else the partials are
// left for launch_combine); n_items counts decode splits plus one item per
// idle row.
int launch_decode_fused(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                        const void *q, const FusedArgs &fa, int32_t n_items, bool merge,
                        const Launch &lc);
// One-token steps of a short ring layer: one workgroup
// per (row, KV head), its waves take the row's splits and merge them through
// LDS into `fa.out` (every row: idle rows get zeros), so there are no
// partials and no launch_combine.  fused: also the rotation and store of the
// new key and value (fa.k, fa.v, fa.slot_out), as launch_decode_fused.
int launch_decode_wg(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                     const void *q, const FusedArgs &fa, bool fused, const Launch &lc);
// qw: waves per workgroup (8: 256 query rows per item; 4: 128;
// kChunkKeyHalves: 128, eight waves as two groups of four over alternate key
// tiles, merged in LDS).  With pa.chunk_small, the 4-wave (or key-halves)
// launch takes the rows of at most 128 query rows and the 8-wave launch the
// rest.
constexpr int kChunkKeyHalves = 2;
int launch_prefill(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                   const void *q, int32_t n_items, int qw, const Launch &lc);
int launch_combine(int dtype, const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                   void *out, const Launch &lc);
// lj: the joint partner's layer (lj.k == nullptr: none).
int launch_generic(int dtype, const StepArgs &st, const LayerArgs &la, const LayerArgs &lj,
                   const void *q, void *out, const Launch &lc);
// A fixed device array per GPU holding one layer's split partials for
// kvc_attend_noalloc (callers that cannot allocate); its size, and its
// address on `device`, looked up once per device with that device current
// (nullptr if the lookup failed or the device index is out of range).
constexpr int64_t kNoAllocScratchBytes = KVC_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes == int64_t(128) << 20, "scratch size");
constexpr int kNoAllocMaxDevices = 64;
void *noalloc_scratch(int device);
bool fast_decode_supported(int D, int rep);
// Decode workgroups (one wave each) resident per compute unit; 0 on error.
int decode_waves_per_cu(int D, int rep);
bool fast_prefill_supported(int D, int rep);
// Chunk-attention workgroups of qw waves resident per compute unit; 0 on error.
int chunk_wgs_per_cu(int D, int rep, int qw);

}  // namespace kvc
