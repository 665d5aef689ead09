// Config validation and the device-buffer layout (pure host code).
//
// Cache rows per layer follow the colibri PR "inkling: ring-buffer KV cache
// for sliding-window layers", section "How it works" (kv_ring_rows): a
// sliding layer keeps W rows iff 0 < W < max_len, every other layer keeps
// max_len rows.  tiny_agent "generate.py" KVCache adds one scratch row that
// padded tokens are written to.  The byte count without scratch rows is the
// size formula of "Lab 07 - KV cache and sampling", section 1.
#include <limits>

#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int64_t kAlign = 256;
// Largest (row, KV head) region of K or V the kernels can address.
constexpr int64_t kMaxRegionBytes = int64_t(1) << 31;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Overflow-checked accumulation of a region; returns false on overflow.
bool take(int64_t *cursor, int64_t bytes, int64_t *off) {
  if (bytes < 0) return false;
  int64_t start = align_up(*cursor, kAlign);
  if (start > std::numeric_limits<int64_t>::max() - bytes) return false;
  *off = start;
  *cursor = start + bytes;
  return true;
}

// a*b*c*... with overflow detection (all operands non-negative).
bool mul(int64_t *acc, int64_t x) {
  if (x < 0) return false;
  if (x != 0 && *acc > std::numeric_limits<int64_t>::max() / x) return false;
  *acc *= x;
  return true;
}

}  // namespace

int dtype_bytes(int dtype) {
  switch (dtype) {
    case KVC_F32: return 4;
    case KVC_BF16: return 2;
    default: return 0;
  }
}

int compute_layout(const kvc_config *cfg, Layout *lay) {
  if (!cfg || !lay) return KVC_E_ARG;
  const int s = dtype_bytes(cfg->dtype);
  if (s == 0) return KVC_E_DTYPE;
  if (cfg->n_layer < 1 || cfg->batch < 1 || cfg->n_q_head < 1) return KVC_E_ARG;
  if (cfg->head_dim < 8 || cfg->head_dim > 256 || cfg->head_dim % 8) return KVC_E_ARG;
  if (cfg->max_len < 1 || cfg->max_chunk < 1 || cfg->max_chunk > 1024) return KVC_E_ARG;
  if (!cfg->n_kv_head || !cfg->window) return KVC_E_ARG;
  if (!(cfg->rope_base >= 0.0)) return KVC_E_ARG;  // also rejects NaN
  if (cfg->use_ring != 0 && cfg->use_ring != 1) return KVC_E_ARG;
  if (cfg->n_pages < 0 || cfg->n_pages > (1 << 30)) return KVC_E_ARG;

  const int64_t B = cfg->batch, D = cfg->head_dim, Hq = cfg->n_q_head;
  lay->layers.assign(cfg->n_layer, LayerLayout{});
  int64_t cur = 0, kv_bytes = 0;
  // Paged: a pool of n_pages pages plus a zero page (unassigned block-table
  // entries point at it) and a scratch page (padded tokens land there).
  const int64_t pool_pages = cfg->n_pages > 0 ? (int64_t)cfg->n_pages + 2 : 0;
  lay->n_pages = cfg->n_pages;
  // whole 32-row tiles: the chunk kernel reads rows up to the next multiple of 32
  lay->pages_per_row = cfg->n_pages > 0 ? (cfg->max_len + 2 * kPageRows - 1) / (2 * kPageRows) * 2 : 0;
  lay->page_bytes = (int64_t)kPageRows * D * s;
  for (int l = 0; l < cfg->n_layer; ++l) {
    const int32_t hkv = cfg->n_kv_head[l], w = cfg->window[l];
    if (hkv < 1 || Hq % hkv) return KVC_E_ARG;
    if (w < 0) return KVC_E_ARG;
    LayerLayout &L = lay->layers[l];
    L.hkv = hkv;
    L.window = w;
    L.ring = (cfg->use_ring && w > 0 && w < cfg->max_len) ? 1 : 0;
    L.paged = (!L.ring && cfg->n_pages > 0) ? 1 : 0;
    L.rows = L.ring ? w : cfg->max_len;
    L.rows_alloc = (int32_t)align_up((int64_t)L.rows + 1, kRowAlign);
    // A (row, KV head) region whose size is a multiple of 8 KB gets one more
    // 16-row block: the decode kernel streams many regions side by side, and
    // with such a stride their tiles crowd the same HBM channels.  Measured
    // on decode_b64 (8224 rows of 256 bytes, a multiple of 8 KB), each
    // variant in both process positions on one box: +16 rows 6.26 TB/s,
    // +48 6.28, +80 6.29 against 6.08 without.
    if (!L.paged && ((int64_t)L.rows_alloc * D * s) % 8192 == 0) L.rows_alloc += kVBlock;
    // The attention kernels address one (row, KV head) region of K or V
    // through a buffer descriptor whose size and offsets are 32-bit: such a
    // region (rows_alloc * D * s bytes) must stay below 2^31.  The row
    // offsets themselves are 64-bit.
    if ((int64_t)L.rows_alloc * D * s >= kMaxRegionBytes) return KVC_E_ARG;
    int64_t region = L.paged ? pool_pages * kPageRows : B * (int64_t)L.rows_alloc;
    if (!mul(&region, hkv) || !mul(&region, D) || !mul(&region, s)) return KVC_E_ARG;
    if (!take(&cur, region, &L.k_off) || !take(&cur, region, &L.v_off)) return KVC_E_ARG;
    // the size formula: every row's max_len rows, or the page pool
    int64_t kvl = L.paged ? 2 * (int64_t)cfg->n_pages * kPageRows : 2 * B * (int64_t)L.rows;
    if (!mul(&kvl, hkv) || !mul(&kvl, D) || !mul(&kvl, s)) return KVC_E_ARG;
    if (kv_bytes > std::numeric_limits<int64_t>::max() - kvl) return KVC_E_ARG;
    kv_bytes += kvl;
    if (L.ring && cfg->max_chunk >= 2) {
      L.stage_rows_alloc = (int32_t)align_up(cfg->max_chunk, kRowAlign);
      int64_t st = B * hkv * (int64_t)L.stage_rows_alloc * D * s;
      if (!take(&cur, st, &L.sk_off) || !take(&cur, st, &L.sv_off)) return KVC_E_ARG;
    }
  }
  if (cfg->rope_base > 0.0) {
    int64_t rb = (int64_t)cfg->max_len * (D / 2) * 8;
    if (!take(&cur, rb, &lay->rope_off)) return KVC_E_ARG;
  } else {
    lay->rope_off = -1;
  }
  if (!take(&cur, B * 4, &lay->lens_off) || !take(&cur, B * 4, &lay->nnew_off) ||
      !take(&cur, B * 4, &lay->first_off))
    return KVC_E_ARG;
  const int64_t dq = B * Hq * kDecodeSplitCap;
  if (!take(&cur, dq * 8, &lay->dml_off) || !take(&cur, dq * D * 4, &lay->dout_off))
    return KVC_E_ARG;
  // One counter per (row, KV head); Hq bounds every layer's Hkv.
  lay->cnt_bytes = B * Hq * 4;
  if (!take(&cur, lay->cnt_bytes, &lay->cnt_off)) return KVC_E_ARG;
  if (cfg->n_pages > 0) {
    if (!take(&cur, B * lay->pages_per_row * 4, &lay->table_off) || !take(&cur, B * 4, &lay->cap_off))
      return KVC_E_ARG;
  }
  // Joint partners: an earlier full-layout layer with the same KV heads and
  // no partner of its own.
  for (int l = 0; l < cfg->n_layer; ++l) {
    const int32_t j = cfg->joint ? cfg->joint[l] : -1;
    if (j < -1 || j >= l) return KVC_E_ARG;
    lay->layers[l].joint = j;
    if (j >= 0) {
      const LayerLayout &P = lay->layers[j];
      if (P.ring || P.hkv != lay->layers[l].hkv || (cfg->joint[j] >= 0)) return KVC_E_ARG;
    }
  }
  // Static steps: error bits, and per layer class a split length and a row order.
  if (!take(&cur, 4, &lay->flags_off)) return KVC_E_ARG;
  if (!take(&cur, (int64_t)cfg->n_layer * (4 + 2 * B), &lay->plan_off)) return KVC_E_ARG;
  if (cfg->max_chunk >= 2) {
    const int64_t pq = B * (int64_t)cfg->max_chunk * Hq * kChunkSplitCap;
    if (!take(&cur, pq * 8, &lay->pml_off) || !take(&cur, pq * D * 4, &lay->pout_off))
      return KVC_E_ARG;
  } else {
    lay->pml_off = lay->pout_off = -1;
  }
  lay->total = align_up(cur, kAlign);
  lay->kv_bytes = kv_bytes;
  return KVC_OK;
}

}  // namespace kvc
