// The C ABI: handle, step state machine, host-side planning and launches.
//
// Protocol (pycraft-1 "model/kv_cache.py": update() writes without advancing,
// advance() once after every layer; tinyllm "kv_cache.py": begin/update/end
// step): per step, every layer is appended and then attended, and one
// kvc_advance ends the step.  The capacity check runs on the host before
// anything is enqueued (tiny_agent "generate.py" append; colibri PR "How it
// works", the fail-fast bound check).  Row lengths live on the device and in
// a host mirror, so planning never reads device memory (tiny_agent module
// docstring: no host syncs inside a step).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "kvc_internal.h"

using kvc::Layout;
using kvc::LayerLayout;

struct kvc_cache {
  kvc_config cfg{};
  std::vector<int32_t> n_kv_head, window, joint;
  Layout lay;
  char *base = nullptr;
  size_t bytes = 0;
  int device = 0;
  std::vector<int32_t> lens_host;
  std::vector<int32_t> first_host;  // left padding per row (mirror of the device copy)
  // paged caches: free pages and the pages each row holds, in block order
  std::vector<int32_t> free_pages;
  std::vector<std::vector<int32_t>> row_pages;
  // step state
  bool in_step = false;
  std::vector<int32_t> n_new;
  int32_t C = 0;
  std::vector<uint8_t> appended, attended;
  // layers that are some layer's joint partner: their keys serve that layer's
  // softmax, so they need not be attended on their own
  std::vector<uint8_t> partner_only;
  // decode split planning: compute units, resident decode waves per CU by
  // query heads per KV head (0 = not yet queried), and overrides
  int32_t n_cu = 0;
  int32_t dec_occ[17] = {0};
  // chunk workgroups per CU, 8-wave and 4-wave, by query heads per KV head (0 = not queried)
  int32_t chunk_occ[17][2] = {{0}};
  int32_t dec_split_fixed = 0;    // keys per split (multiple of 16); 0 = planned
  int32_t dec_waves_target = 0;   // waves per decode launch; 0 = resident slots
  int32_t dec_min_tiles = kvc::kDecodeSplitMinTiles;  // smallest planned split, in tiles
  int32_t log_level = 0;          // KVC_LOG: 1 sizes at create, 2 also decode plans
  bool no_fused = false;          // KVC_DECODE_FUSED=0: append + attend in kvc_append_attend
  bool no_chunk_fused = false;    // KVC_CHUNK_FUSED=0: ring chunk steps staged there too
  bool no_key_halves = false;     // KVC_CHUNK_KEY_HALVES=0: 128-row chunk tiles in 4 waves
  bool fused_merge = false;       // KVC_FUSED_MERGE=1: the appending decode merges its splits
  bool no_wg = false;             // KVC_DECODE_WG=0: short windows take the split plan too
  bool chunk_cap_only = false;    // KVC_CHUNK_PLAN=0: chunk splits from the split cap alone
  bool no_direct = false;         // KVC_CHUNK_DIRECT=0: ring chunk steps merge in k_combine
  bool no_ring_small = false;     // KVC_CHUNK_RING_SMALL=0: ring chunk rows by size as others
  bool no_side = false;           // KVC_CHUNK_SIDE=0: both chunk launches on the caller's stream
  // A second stream (default priority) for the 4-wave chunk launch beside the
  // 8-wave one, forked from and joined back to the caller's stream by events;
  // made at create (max_chunk >= 2), so that no step creates anything.
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // The device address of this GPU's fixed scratch array (kvc_attend_noalloc),
  // looked up at create; null if the lookup failed.
  void *scratch = nullptr;
  bool no_chunk_small = false;    // KVC_CHUNK_SMALL=0: every chunk row in 8-wave workgroups
  // static one-token steps (counts in device memory, planned on the device)
  bool step_static = false;           // the current step is one
  bool lens_stale = false;            // a static step advanced the device lengths only
  std::vector<int32_t> layer_class;   // layer -> plan class
  std::vector<kvc::StaticClass> classes;
  // kernel timing
  bool timing = false;
  std::vector<hipEvent_t> ev;      // 2 per launch
  std::vector<int> ev_kind;
  int32_t ev_used = 0;
  int32_t ev_mask = 0;             // kinds (bit per KVC_K_*) whose launches are timed
};

namespace {

// Smallest chunk-attention split (keys) before the split count per row is capped.
constexpr int32_t kChunkSplitMin = 256;
// Price of one chunk-attention split beyond its keys, in keys: staging the
// query tile, writing its partial and merging it.
constexpr int64_t kChunkSplitCost = 384;
// One-token steps of a ring layer of at most this many rows run in the
// workgroup form of the decode kernel (see wg_layer).
constexpr int32_t kWgMaxWindow = 1024;

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }
int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

bool use_device(const kvc_t *h) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return false;
  if (cur == h->device) return true;
  return hipSetDevice(h->device) == hipSuccess;
}

kvc::StepArgs step_args(const kvc_t *h) {
  kvc::StepArgs st{};
  st.lens = reinterpret_cast<const int32_t *>(h->base + h->lay.lens_off);
  st.n_new = reinterpret_cast<const int32_t *>(h->base + h->lay.nnew_off);
  st.first = reinterpret_cast<const int32_t *>(h->base + h->lay.first_off);
  st.rope = h->lay.rope_off >= 0 ? reinterpret_cast<const float *>(h->base + h->lay.rope_off)
                                  : nullptr;
  st.B = h->cfg.batch;
  st.C = h->C;
  st.Hq = h->cfg.n_q_head;
  st.D = h->cfg.head_dim;
  st.max_len = h->cfg.max_len;
  return st;
}

kvc::LayerArgs layer_args(const kvc_t *h, int layer) {
  const LayerLayout &L = h->lay.layers[layer];
  kvc::LayerArgs la{};
  la.k = h->base + L.k_off;
  la.v = h->base + L.v_off;
  la.sk = L.sk_off >= 0 ? h->base + L.sk_off : nullptr;
  la.sv = L.sv_off >= 0 ? h->base + L.sv_off : nullptr;
  la.hkv = L.hkv;
  la.rep = h->cfg.n_q_head / L.hkv;
  la.window = L.window;
  la.ring = L.ring;
  la.rows = L.rows;
  la.rows_alloc = L.rows_alloc;
  la.stage_rows_alloc = L.stage_rows_alloc;
  if (L.paged) {
    la.paged = 1;
    la.table = reinterpret_cast<const int32_t *>(h->base + h->lay.table_off);
    la.ppr = h->lay.pages_per_row;
    la.scratch_page = h->lay.n_pages + 1;
  }
  return la;
}

// -- paged caches: the host page allocator ----------------------------------
// Pages not held by a row sit in a free list; row b holds row_pages[b] in
// block order.  Unassigned block-table entries name the zero page (n_pages),
// so a 32-row tile may read past a row's last page.  A page taken by a row
// gets V zeroed in every paged layer first (the decode tiles read rows past
// a row's end, masked, and need them finite).

int32_t zero_page(const kvc_t *h) { return h->lay.n_pages; }

// Enqueue block-table entries (table index -> page; zero: page to clear or
// -1) and row capacities, in launches of at most 64 entries and 256 rows,
// once per group of up to 64 paged layers.
int push_page_updates(kvc_t *h, const std::vector<int32_t> &idx, const std::vector<int32_t> &page,
                      const std::vector<int32_t> &zero, const std::vector<int32_t> &cap_rows,
                      const std::vector<int32_t> &cap_vals, void *stream) {
  int32_t *table = reinterpret_cast<int32_t *>(h->base + h->lay.table_off);
  int32_t *cap = reinterpret_cast<int32_t *>(h->base + h->lay.cap_off);
  std::vector<kvc::PagedPools> groups(1);
  groups[0].n = 0;
  for (const LayerLayout &L : h->lay.layers) {
    if (!L.paged) continue;
    if (groups.back().n == 64) {
      groups.emplace_back();
      groups.back().n = 0;
    }
    kvc::PagedPools &g = groups.back();
    g.v[g.n] = h->base + L.v_off;
    g.hkv[g.n] = L.hkv;
    ++g.n;
  }
  const size_t nu = idx.size(), nc = cap_rows.size();
  size_t u0 = 0, c0 = 0;
  while (u0 < nu || c0 < nc) {
    kvc::PageUpdate u{};
    const int32_t mu = (int32_t)std::min<size_t>(64, nu - u0);
    const int32_t mc = (int32_t)std::min<size_t>(256, nc - c0);
    for (int32_t i = 0; i < mu; ++i) {
      u.idx[i] = idx[u0 + i];
      u.page[i] = page[u0 + i];
      u.zero[i] = zero[u0 + i];
    }
    // (every group's launch repeats the table writes: the same values)
    for (const kvc::PagedPools &g : groups)
      if (kvc::launch_page_update(table, cap, cap_rows.data() + c0, cap_vals.data() + c0, mc, u, mu,
                                  g, h->lay.page_bytes, stream))
        return KVC_E_HIP;
    u0 += mu;
    c0 += mc;
  }
  return KVC_OK;
}

// Give each row `rows[i]` pages for at least `tokens[i]` positions; all or
// nothing (KVC_E_FULL if the free list is short).
int take_pages(kvc_t *h, const std::vector<int32_t> &rows, const std::vector<int64_t> &tokens,
               void *stream) {
  int64_t want = 0;
  for (size_t i = 0; i < rows.size(); ++i) {
    const int64_t need = (tokens[i] + kvc::kPageRows - 1) / kvc::kPageRows;
    want += std::max<int64_t>(0, need - (int64_t)h->row_pages[rows[i]].size());
  }
  if (want == 0) return KVC_OK;
  if (want > (int64_t)h->free_pages.size()) return KVC_E_FULL;
  std::vector<int32_t> idx, page, zero, cap_rows, cap_vals;
  for (size_t i = 0; i < rows.size(); ++i) {
    const int32_t b = rows[i];
    const int64_t need = (tokens[i] + kvc::kPageRows - 1) / kvc::kPageRows;
    std::vector<int32_t> &held = h->row_pages[b];
    if ((int64_t)held.size() >= need) continue;
    while ((int64_t)held.size() < need) {
      const int32_t pg = h->free_pages.back();
      h->free_pages.pop_back();
      idx.push_back(b * h->lay.pages_per_row + (int32_t)held.size());
      page.push_back(pg);
      zero.push_back(pg);
      held.push_back(pg);
    }
    cap_rows.push_back(b);
    cap_vals.push_back((int32_t)held.size() * kvc::kPageRows);
  }
  return push_page_updates(h, idx, page, zero, cap_rows, cap_vals, stream);
}

// Return rows' pages to the free list; their table entries name the zero page.
int release_pages(kvc_t *h, const int32_t *rows, int32_t n, void *stream) {
  std::vector<int32_t> idx, page, zero, cap_rows, cap_vals;
  for (int32_t i = 0; i < n; ++i) {
    std::vector<int32_t> &held = h->row_pages[rows[i]];
    for (size_t k = 0; k < held.size(); ++k) {
      idx.push_back(rows[i] * h->lay.pages_per_row + (int32_t)k);
      page.push_back(zero_page(h));
      zero.push_back(-1);
      h->free_pages.push_back(held[k]);
    }
    held.clear();
    cap_rows.push_back(rows[i]);
    cap_vals.push_back(0);
  }
  return push_page_updates(h, idx, page, zero, cap_rows, cap_vals, stream);
}

// Where the next launch of `kind` goes.  With kernel timing on it carries a
// fresh pair of events that the dispatch stamps at its own start and end, so
// the measured time is the kernel's alone and no marker packets are added to
// the stream.
kvc::Launch launch_on(kvc_t *h, int kind, void *stream) {
  kvc::Launch lc;
  lc.stream = stream;
  if (!h->timing || !((h->ev_mask >> kind) & 1) || 2 * (h->ev_used + 1) > (int32_t)h->ev.size())
    return lc;
  const int i = h->ev_used++;
  h->ev_kind[i] = kind;
  lc.t0 = h->ev[2 * i];
  lc.t1 = h->ev[2 * i + 1];
  return lc;
}

void decode_span(const kvc::LayerArgs &la, int64_t p, int64_t first, int64_t *base, int64_t *hi);

// Keys per decode split for this layer and step.  The decode launch should be
// one round of equally long waves: the smallest split (in 16-key tiles) whose
// wave count, summed over the decoding rows and KV heads, fits the waves the
// chip holds at once.  A partial second round or a few long waves would leave
// most of the chip idle at the end of the launch.  Each row keeps at most
// kDecodeSplitCap splits.  The idle rows' items of kvc_append_attend's kernel
// take slots too; both entry points plan with them counted, so a step splits
// its rows the same way (and produces the same bits) through either.
int32_t decode_split_keys(kvc_t *h, const kvc::LayerArgs &la, int D,
                          int32_t cap = kvc::kDecodeSplitCap) {
  const int TK = kvc::kDecodeTile;
  std::vector<int64_t> tiles;
  int64_t max_t = 0, extra = 0;
  for (int32_t b = 0; b < h->cfg.batch; ++b) {
    extra += h->n_new[b] == 0 ? la.hkv : 0;
    if (h->n_new[b] != 1) continue;
    int64_t base, hi;
    decode_span(la, h->lens_host[b], h->first_host[b], &base, &hi);
    tiles.push_back((hi - base + TK - 1) / TK);
    max_t = std::max(max_t, tiles.back());
  }
  const int64_t q_cap = std::max<int64_t>(1, (max_t + cap - 1) / cap);
  if (max_t == 0) return TK;
  const int64_t q_min = std::max<int64_t>(q_cap, h->dec_min_tiles);
  if (h->dec_split_fixed > 0)
    return (int32_t)(std::max<int64_t>(h->dec_split_fixed / TK, q_cap) * TK);
  int64_t target = h->dec_waves_target;
  if (target <= 0) {
    int32_t &occ = h->dec_occ[la.rep <= 16 ? la.rep : 0];
    if (occ == 0) occ = std::max(1, kvc::decode_waves_per_cu(D, la.rep));
    target = (int64_t)h->n_cu * occ;
  }
  target = std::max<int64_t>(1, target - extra);
  auto waves = [&](int64_t q) {
    int64_t w = 0;
    for (int64_t t : tiles) w += (t + q - 1) / q;
    return w * la.hkv;
  };
  int64_t lo = q_min, hi = std::max(q_min, max_t);
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (waves(mid) <= target)
      hi = mid;
    else
      lo = mid + 1;
  }
  return (int32_t)(lo * TK);
}

// Dispatch order of the decode items: the KV heads of an item go out
// together, and items of rows with the longest splits first.  Waves
// dispatched earlier are served first on their compute unit (measured: the
// later half of a one-round launch ran about 1.6x slower until the earlier
// half finished), so the longest work goes to them: 2-3 % off the launch.
void decode_order(const kvc_t *h, const kvc::LayerArgs &la, kvc::PartialArgs *pa) {
  pa->dec_ordered = 0;
  const int32_t B = h->cfg.batch;
  if (B > kvc::kDecodeOrderMax) return;
  std::vector<std::pair<double, int>> key(B);
  for (int32_t b = 0; b < B; ++b) {
    double per = 0.0;
    if (h->n_new[b] == 1) {
      int64_t base, hi;
      decode_span(la, h->lens_host[b], h->first_host[b], &base, &hi);
      const int64_t t = (hi - base + kvc::kDecodeTile - 1) / kvc::kDecodeTile;
      const int64_t ns = (hi - base + pa->dec_split_keys - 1) / pa->dec_split_keys;
      per = (double)t / (double)ns;
    }
    key[b] = {-per, b};
  }
  std::stable_sort(key.begin(), key.end());
  for (int32_t b = 0; b < B; ++b) pa->dec_order[b] = (uint16_t)key[b].second;
  pa->dec_ordered = 1;
}

// Key span of a one-token query at p on this layer, in storage rows (the
// rows a decode visits; masking of the rest is the kernel's).  Global layer:
// from the first visible position (the window's, raised to the row's left
// padding `first`; a pad query sees only itself) to p.  Ring layer: the
// visible positions occupy slots [0, min(p + 1, W)).
void decode_span(const kvc::LayerArgs &la, int64_t p, int64_t first, int64_t *base, int64_t *hi) {
  if (la.ring) {
    *base = 0;
    *hi = std::min<int64_t>(p + 1, la.window);
    return;
  }
  int64_t start = la.window > 0 ? std::max<int64_t>(0, p - la.window + 1) : 0;
  start = p < first ? p : std::max(start, first);
  *hi = p + 1;
  *base = start / kvc::kRowAlign * kvc::kRowAlign;
}

// Key span of a chunk of n tokens starting at L on a non-ring layer; left
// padding raises the start to `first` unless the chunk holds pad queries.
void chunk_span(const kvc::LayerArgs &la, int64_t L, int64_t n, int64_t first, int64_t *base,
                int64_t *hi) {
  int64_t lo = la.window > 0 ? std::max<int64_t>(0, L - la.window + 1) : 0;
  lo = std::max(lo, std::min(first, L));
  *hi = L + n;
  *base = lo / kvc::kRowAlign * kvc::kRowAlign;
}

}  // namespace

extern "C" {

const char *kvc_strerror(int code) {
  switch (code) {
    case KVC_OK: return "ok";
    case KVC_E_ARG: return "invalid argument or unsupported shape";
    case KVC_E_FULL: return "KV cache full";
    case KVC_E_DTYPE: return "unknown dtype";
    case KVC_E_STATE: return "call out of step order";
    case KVC_E_HIP: return "HIP runtime error";
    case KVC_E_SCRATCH: return "step needs more than the fixed scratch of kvc_attend_noalloc";
    default: return "unknown status";
  }
}

size_t kvc_nbytes(const kvc_config *cfg, int what) {
  Layout lay;
  if (kvc::compute_layout(cfg, &lay) != KVC_OK) return 0;
  if (what == KVC_NB_KV) return (size_t)lay.kv_bytes;
  if (what == KVC_NB_ALLOC) return (size_t)lay.total;
  return 0;
}

int kvc_create(const kvc_config *cfg, void *dev_buf, size_t buf_bytes, void *stream,
               kvc_t **out) {
  if (!out) return KVC_E_ARG;
  *out = nullptr;
  Layout lay;
  int rc = kvc::compute_layout(cfg, &lay);
  if (rc != KVC_OK) return rc;
  if (!dev_buf || buf_bytes < (size_t)lay.total) return KVC_E_ARG;
  if (reinterpret_cast<uintptr_t>(dev_buf) % 256) return KVC_E_ARG;

  kvc_t *h = new (std::nothrow) kvc_t();
  if (!h) return KVC_E_ARG;
  h->cfg = *cfg;
  h->n_kv_head.assign(cfg->n_kv_head, cfg->n_kv_head + cfg->n_layer);
  h->window.assign(cfg->window, cfg->window + cfg->n_layer);
  h->cfg.n_kv_head = h->n_kv_head.data();
  h->cfg.window = h->window.data();
  if (cfg->joint) {
    h->joint.assign(cfg->joint, cfg->joint + cfg->n_layer);
    h->cfg.joint = h->joint.data();
  }
  h->lay = std::move(lay);
  h->base = static_cast<char *>(dev_buf);
  h->bytes = buf_bytes;
  h->lens_host.assign(cfg->batch, 0);
  h->first_host.assign(cfg->batch, 0);
  h->n_new.assign(cfg->batch, 0);
  h->appended.assign(cfg->n_layer, 0);
  h->attended.assign(cfg->n_layer, 0);
  h->partner_only.assign(cfg->n_layer, 0);
  for (int32_t l = 0; l < cfg->n_layer; ++l)
    if (h->lay.layers[l].joint >= 0) h->partner_only[h->lay.layers[l].joint] = 1;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return KVC_E_HIP;
  }
  h->scratch = kvc::noalloc_scratch(h->device);
  hipStream_t s = (hipStream_t)stream;
  // RoPE table: angle p * base^(-2d/D) in double, cos/sin rounded once to fp32.
  if (h->lay.rope_off >= 0) {
    const int D = cfg->head_dim, half = D / 2;
    std::vector<float> tab((size_t)cfg->max_len * half * 2);
    for (int d = 0; d < half; ++d) {
      const double theta = std::pow(cfg->rope_base, -2.0 * d / D);
      for (int64_t p = 0; p < cfg->max_len; ++p) {
        const double a = (double)p * theta;
        tab[((size_t)p * half + d) * 2 + 0] = (float)std::cos(a);
        tab[((size_t)p * half + d) * 2 + 1] = (float)std::sin(a);
      }
    }
    if (hipMemcpyAsync(h->base + h->lay.rope_off, tab.data(), tab.size() * sizeof(float),
                       hipMemcpyHostToDevice, s) != hipSuccess) {
      delete h;
      return KVC_E_HIP;
    }
    if (hipStreamSynchronize(s) != hipSuccess) {
      delete h;
      return KVC_E_HIP;
    }
  }
  // Row lengths, n_new and the fused decode's split-arrival counters start
  // at zero (the counters return to zero at the end of every fused launch).
  if (hipMemsetAsync(h->base + h->lay.lens_off, 0, (size_t)cfg->batch * 4, s) != hipSuccess ||
      hipMemsetAsync(h->base + h->lay.nnew_off, 0, (size_t)cfg->batch * 4, s) != hipSuccess ||
      hipMemsetAsync(h->base + h->lay.first_off, 0, (size_t)cfg->batch * 4, s) != hipSuccess ||
      hipMemsetAsync(h->base + h->lay.cnt_off, 0, h->lay.cnt_bytes, s) != hipSuccess ||
      hipMemsetAsync(h->base + h->lay.flags_off, 0, 4, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    delete h;
    return KVC_E_HIP;
  }
  // Paged: every block-table entry names the zero page, whose K and V are
  // zero in every paged layer; all pages are free.
  if (cfg->n_pages > 0) {
    std::vector<int32_t> tab((size_t)cfg->batch * h->lay.pages_per_row, cfg->n_pages);
    bool ok = hipMemcpyAsync(h->base + h->lay.table_off, tab.data(), tab.size() * 4,
                             hipMemcpyHostToDevice, s) == hipSuccess &&
              hipMemsetAsync(h->base + h->lay.cap_off, 0, (size_t)cfg->batch * 4, s) == hipSuccess;
    for (const LayerLayout &L : h->lay.layers) {
      if (!L.paged) continue;
      const size_t bytes = (size_t)h->lay.page_bytes * L.hkv;
      const size_t off = (size_t)cfg->n_pages * bytes;
      ok = ok && hipMemsetAsync(h->base + L.k_off + off, 0, bytes, s) == hipSuccess &&
           hipMemsetAsync(h->base + L.v_off + off, 0, bytes, s) == hipSuccess;
    }
    if (!ok || hipStreamSynchronize(s) != hipSuccess) {
      delete h;
      return KVC_E_HIP;
    }
    h->free_pages.resize(cfg->n_pages);
    for (int32_t i = 0; i < cfg->n_pages; ++i) h->free_pages[i] = cfg->n_pages - 1 - i;
  }
  h->row_pages.assign(cfg->batch, {});
  if (hipDeviceGetAttribute(&h->n_cu, hipDeviceAttributeMultiprocessorCount, h->device) !=
          hipSuccess ||
      h->n_cu <= 0) {
    delete h;
    return KVC_E_HIP;
  }
  // Tuning overrides (documented at kvc_create in kvc.h).
  if (const char *e = std::getenv("KVC_DECODE_SPLIT")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= kvc::kDecodeTile && v <= (1 << 20) && v % kvc::kDecodeTile == 0)
      h->dec_split_fixed = (int32_t)v;
  }
  if (const char *e = std::getenv("KVC_DECODE_WAVES")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v <= (1 << 24)) h->dec_waves_target = (int32_t)v;
  }
  if (const char *e = std::getenv("KVC_DECODE_MIN_TILES")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v <= 4096) h->dec_min_tiles = (int32_t)v;
  }
  if (const char *e = std::getenv("KVC_DECODE_FUSED")) h->no_fused = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_FUSED")) h->no_chunk_fused = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_KEY_HALVES")) h->no_key_halves = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_FUSED_MERGE")) h->fused_merge = std::atoi(e) != 0;
  if (const char *e = std::getenv("KVC_DECODE_WG")) h->no_wg = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_PLAN")) h->chunk_cap_only = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_DIRECT")) h->no_direct = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_RING_SMALL")) h->no_ring_small = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_SIDE")) h->no_side = std::atoi(e) == 0;
  if (const char *e = std::getenv("KVC_CHUNK_SMALL")) h->no_chunk_small = std::atoi(e) == 0;
  if (cfg->max_chunk >= 2 && !h->no_side &&
      (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
       hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) != hipSuccess ||
       hipEventCreateWithFlags(&h->join, hipEventDisableTiming) != hipSuccess)) {
    kvc_destroy(h);
    return KVC_E_HIP;
  }
  // Plan classes of static steps: layers with the same KV heads, window and layout.
  for (int32_t l = 0; l < cfg->n_layer; ++l) {
    const LayerLayout &L = h->lay.layers[l];
    int32_t c = 0;
    while (c < (int32_t)h->classes.size() &&
           !(h->classes[c].hkv == L.hkv && h->classes[c].window == L.window &&
             h->classes[c].ring == L.ring))
      ++c;
    if (c == (int32_t)h->classes.size()) {
      kvc::StaticClass sc{};
      sc.hkv = L.hkv;
      sc.window = L.window;
      sc.ring = L.ring;
      h->classes.push_back(sc);
    }
    h->layer_class.push_back(c);
  }
  if (const char *e = std::getenv("KVC_LOG")) {
    h->log_level = std::atoi(e);
    if (h->log_level >= 1)
      std::fprintf(stderr, "[kvc] %d layers, B %d, KV %.1f MiB (formula), buffer %.1f MiB\n",
                   cfg->n_layer, cfg->batch, h->lay.kv_bytes / 1048576.0,
                   h->lay.total / 1048576.0);
  }
  *out = h;
  return KVC_OK;
}

void kvc_destroy(kvc_t *h) {
  if (!h) return;
  for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
  if (h->fork) (void)hipEventDestroy(h->fork);
  if (h->join) (void)hipEventDestroy(h->join);
  if (h->side) (void)hipStreamDestroy(h->side);
  delete h;
}

int kvc_reset(kvc_t *h, const int32_t *rows_host, int32_t n_rows, void *stream) {
  if (!h || n_rows < 0 || (n_rows > 0 && !rows_host)) return KVC_E_ARG;
  if (h->in_step || h->lens_stale) return KVC_E_STATE;
  for (int32_t i = 0; i < n_rows; ++i)
    if (rows_host[i] < 0 || rows_host[i] >= h->cfg.batch) return KVC_E_ARG;
  if (n_rows == 0) return KVC_OK;
  if (!use_device(h)) return KVC_E_HIP;
  int32_t *lens = reinterpret_cast<int32_t *>(h->base + h->lay.lens_off);
  int32_t *first = reinterpret_cast<int32_t *>(h->base + h->lay.first_off);
  int err = kvc::launch_reset_rows(lens, first, rows_host, n_rows, stream);
  if (err) return KVC_E_HIP;
  if (h->lay.n_pages > 0 && release_pages(h, rows_host, n_rows, stream) != KVC_OK) return KVC_E_HIP;
  for (int32_t i = 0; i < n_rows; ++i) {
    h->lens_host[rows_host[i]] = 0;
    h->first_host[rows_host[i]] = 0;
  }
  return KVC_OK;
}

int kvc_set_first(kvc_t *h, const int32_t *rows_host, const int32_t *first_host, int32_t n_rows,
                  void *stream) {
  if (!h || n_rows < 0 || (n_rows > 0 && (!rows_host || !first_host))) return KVC_E_ARG;
  if (h->in_step) return KVC_E_STATE;
  for (int32_t i = 0; i < n_rows; ++i)
    if (rows_host[i] < 0 || rows_host[i] >= h->cfg.batch || first_host[i] < 0 ||
        first_host[i] > h->cfg.max_len)
      return KVC_E_ARG;
  if (n_rows == 0) return KVC_OK;
  if (!use_device(h)) return KVC_E_HIP;
  int32_t *first = reinterpret_cast<int32_t *>(h->base + h->lay.first_off);
  if (kvc::launch_set_first(first, rows_host, first_host, n_rows, stream)) return KVC_E_HIP;
  for (int32_t i = 0; i < n_rows; ++i) h->first_host[rows_host[i]] = first_host[i];
  return KVC_OK;
}

int kvc_admit(kvc_t *dst, const int32_t *dst_rows, const kvc_t *src, const int32_t *src_rows,
              int32_t n_rows, void *stream) {
  if (!dst || !src || n_rows < 0 || (n_rows > 0 && (!dst_rows || !src_rows))) return KVC_E_ARG;
  if (dst->in_step || src->in_step || dst->lens_stale || src->lens_stale) return KVC_E_STATE;
  const kvc_config &a = dst->cfg, &b = src->cfg;
  if (a.n_layer != b.n_layer || a.head_dim != b.head_dim || a.dtype != b.dtype ||
      a.n_q_head != b.n_q_head || dst->device != src->device)
    return KVC_E_ARG;
  for (int32_t l = 0; l < a.n_layer; ++l) {
    const LayerLayout &x = dst->lay.layers[l], &y = src->lay.layers[l];
    if (x.hkv != y.hkv || x.window != y.window || x.ring != y.ring || x.joint != y.joint)
      return KVC_E_ARG;
  }
  std::vector<uint8_t> seen(a.batch, 0);
  for (int32_t i = 0; i < n_rows; ++i) {
    const int32_t d = dst_rows[i], r = src_rows[i];
    if (d < 0 || d >= a.batch || r < 0 || r >= b.batch || seen[d]) return KVC_E_ARG;
    seen[d] = 1;
    if (src->lens_host[r] > a.max_len) return KVC_E_FULL;
  }
  if (dst == src)  // a row must not be both read and written
    for (int32_t i = 0; i < n_rows; ++i)
      if (seen[src_rows[i]]) return KVC_E_ARG;
  if (n_rows == 0) return KVC_OK;
  if (!use_device(dst)) return KVC_E_HIP;
  if (dst->lay.n_pages > 0) {
    // the admitted rows' old pages go back first; pages for the copies, all
    // or nothing
    int64_t want = 0, back = 0;
    for (int32_t i = 0; i < n_rows; ++i) {
      want += (src->lens_host[src_rows[i]] + kvc::kPageRows - 1) / kvc::kPageRows;
      back += (int64_t)dst->row_pages[dst_rows[i]].size();
    }
    if (want > (int64_t)dst->free_pages.size() + back) return KVC_E_FULL;
    if (release_pages(dst, dst_rows, n_rows, stream) != KVC_OK) return KVC_E_HIP;
    std::vector<int32_t> rows(dst_rows, dst_rows + n_rows);
    std::vector<int64_t> tokens;
    for (int32_t i = 0; i < n_rows; ++i) tokens.push_back(src->lens_host[src_rows[i]]);
    if (take_pages(dst, rows, tokens, stream) != KVC_OK) return KVC_E_HIP;
  }
  const int s = kvc::dtype_bytes(a.dtype);
  for (int32_t off = 0; off < n_rows; off += 64) {
    kvc::CopyPairs pairs{};
    const int32_t m = std::min<int32_t>(64, n_rows - off);
    for (int32_t l = 0; l < a.n_layer; ++l) {
      const kvc::LayerArgs dl = layer_args(dst, l), sl = layer_args(src, l);
      for (int32_t j = 0; j < m; ++j) {
        pairs.src_row[j] = src_rows[off + j];
        pairs.dst_row[j] = dst_rows[off + j];
        // the rows held; a full-layout destination also takes the rest of
        // the last 32-row tile (zero V past the row's end)
        const int64_t top = std::min<int64_t>(src->lens_host[src_rows[off + j]], sl.rows);
        const int64_t rows = dl.paged ? top : round_up(top, kvc::kRowAlign);
        pairs.blocks[j] = (int32_t)((rows + kvc::kPageRows - 1) / kvc::kPageRows);
      }
      if (kvc::launch_copy_rows(dl, sl, a.head_dim, s, pairs, m, stream)) return KVC_E_HIP;
    }
    if (kvc::launch_copy_state(reinterpret_cast<int32_t *>(dst->base + dst->lay.lens_off),
                               reinterpret_cast<int32_t *>(dst->base + dst->lay.first_off),
                               reinterpret_cast<const int32_t *>(src->base + src->lay.lens_off),
                               reinterpret_cast<const int32_t *>(src->base + src->lay.first_off),
                               pairs, m, stream))
      return KVC_E_HIP;
  }
  for (int32_t i = 0; i < n_rows; ++i) {
    dst->lens_host[dst_rows[i]] = src->lens_host[src_rows[i]];
    dst->first_host[dst_rows[i]] = src->first_host[src_rows[i]];
  }
  return KVC_OK;
}

namespace {

// The checks of an append (argument ranges, capacity on the step's first
// append, the same n_new and C on every other one, one append per layer) and,
// on the step's first append, latching n_new and C and uploading n_new.
int begin_append(kvc_t *h, int32_t layer, const int32_t *n_new_host, int32_t C, void *stream) {
  if (layer < 0 || layer >= h->cfg.n_layer) return KVC_E_ARG;
  if (C < 1 || C > h->cfg.max_chunk) return KVC_E_ARG;
  const int32_t B = h->cfg.batch;
  if (h->step_static) {  // the counts are on the device; no host copy of them
    if (n_new_host || C != 1) return KVC_E_ARG;
    if (h->appended[layer]) return KVC_E_STATE;
    return use_device(h) ? KVC_OK : KVC_E_HIP;
  }
  if (!n_new_host) return KVC_E_ARG;
  if (h->lens_stale) return KVC_E_STATE;
  if (!h->in_step) {
    for (int32_t b = 0; b < B; ++b)
      if (n_new_host[b] < 0 || n_new_host[b] > C) return KVC_E_ARG;
    for (int32_t b = 0; b < B; ++b)
      if ((int64_t)h->lens_host[b] + n_new_host[b] > h->cfg.max_len) return KVC_E_FULL;
    if (h->lay.n_pages > 0) {  // pages for the new positions, all or nothing
      if (!use_device(h)) return KVC_E_HIP;
      std::vector<int32_t> rows;
      std::vector<int64_t> tokens;
      for (int32_t b = 0; b < B; ++b)
        if (n_new_host[b] > 0) {
          rows.push_back(b);
          tokens.push_back((int64_t)h->lens_host[b] + n_new_host[b]);
        }
      const int rc = take_pages(h, rows, tokens, stream);
      if (rc != KVC_OK) return rc;
    }
  } else {
    if (C != h->C) return KVC_E_STATE;
    for (int32_t b = 0; b < B; ++b)
      if (n_new_host[b] != h->n_new[b]) return KVC_E_STATE;
    if (h->appended[layer]) return KVC_E_STATE;
  }
  if (!use_device(h)) return KVC_E_HIP;
  if (!h->in_step) {
    int32_t *nn = reinterpret_cast<int32_t *>(h->base + h->lay.nnew_off);
    if (kvc::launch_set_rows(nn, n_new_host, B, stream)) return KVC_E_HIP;
    std::copy(n_new_host, n_new_host + B, h->n_new.begin());
    h->C = C;
    h->in_step = true;
    std::fill(h->appended.begin(), h->appended.end(), 0);
    std::fill(h->attended.begin(), h->attended.end(), 0);
  }
  return KVC_OK;
}

kvc::PartialArgs partial_args(const kvc_t *h) {
  kvc::PartialArgs pa{};
  pa.dec_transpose = 1;
  pa.dml = reinterpret_cast<float *>(h->base + h->lay.dml_off);
  pa.dout = reinterpret_cast<float *>(h->base + h->lay.dout_off);
  pa.pml = h->lay.pml_off >= 0 ? reinterpret_cast<float *>(h->base + h->lay.pml_off) : nullptr;
  pa.pout = h->lay.pout_off >= 0 ? reinterpret_cast<float *>(h->base + h->lay.pout_off) : nullptr;
  pa.max_chunk = h->cfg.max_chunk;
  return pa;
}

// A ring layer of at most kWgMaxWindow rows spends a one-token step mostly on
// fixed latencies: launch, prologue, a few tiles, the partials' round trip
// through HBM and a merge launch.  Its one-token steps take the workgroup
// form instead: one workgroup per (row, KV head) whose waves take the splits
// and merge through LDS.  (A window mask over a full-length layout keeps the
// split plan, which its paged form shares, so that the two give the same
// bits; joint layers keep it too.  REP 8 and 16 run the form on the matrix
// cores, REP 1 to 4 on the vector units.)
bool wg_layer(const kvc_t *h, int32_t layer, const kvc::LayerArgs &la) {
  return !h->no_wg && la.ring && la.window <= kWgMaxWindow && !la.paged &&
         (la.rep <= 8 || la.rep == 16) &&
         h->lay.layers[layer].joint < 0 && h->cfg.dtype == KVC_BF16 &&
         kvc::fast_decode_supported(h->cfg.head_dim, la.rep);
}

// Target waves of one decode round for a layer: resident decode waves per CU
// (queried once per query-heads-per-KV-head) times the CUs, unless overridden.
int64_t decode_wave_target(kvc_t *h, const kvc::LayerArgs &la, int D) {
  if (h->dec_waves_target > 0) return h->dec_waves_target;
  int32_t &occ = h->dec_occ[la.rep <= 16 ? la.rep : 0];
  if (occ == 0) occ = std::max(1, kvc::decode_waves_per_cu(D, la.rep));
  return (int64_t)h->n_cu * occ;
}

// A static step's decode plan for a layer: the class's split length and row
// order from the device table, and a grid that bounds the items any counts
// and lengths can produce.  The plan is a split count per row whose waves
// plus the idle rows' items fit one round, or one split per row when none
// does (then at most B items), and never more than kDecodeSplitCap splits
// per row.
int32_t static_plan(const kvc_t *h, int32_t layer, kvc::PartialArgs *pa) {
  const int32_t c = h->layer_class[layer];
  const kvc::StaticClass &cl = h->classes[c];
  pa->dec_plan = reinterpret_cast<const int32_t *>(h->base + h->lay.plan_off) + c;
  pa->dec_order_dev =
      h->cfg.batch <= kvc::kDecodeOrderMax
          ? reinterpret_cast<const uint16_t *>(h->base + h->lay.plan_off + 4 * h->cfg.n_layer) +
                (int64_t)c * h->cfg.batch
          : nullptr;
  pa->dec_ordered = 0;
  const int64_t B = h->cfg.batch;
  int64_t items = cl.fixed_q > 0 ? B * kvc::kDecodeSplitCap
                                 : std::max<int64_t>((cl.target + cl.hkv - 1) / cl.hkv, B);
  return (int32_t)std::min<int64_t>(items, B * kvc::kDecodeSplitCap);
}

}  // namespace

int kvc_append(kvc_t *h, int32_t layer, const void *k, const void *v,
               const int32_t *n_new_host, int32_t C, int32_t *slot_out_dev, void *stream) {
  if (!h || !k || !v) return KVC_E_ARG;
  const int rc = begin_append(h, layer, n_new_host, C, stream);
  if (rc != KVC_OK) return rc;
  const kvc::StepArgs st = step_args(h);
  const kvc::LayerArgs la = layer_args(h, layer);
  int err = kvc::launch_append(h->cfg.dtype, st, la, k, v, slot_out_dev, launch_on(h, KVC_K_APPEND, stream));
  if (err) return KVC_E_HIP;
  h->appended[layer] = 1;
  return KVC_OK;
}

}  // extern "C"

namespace {

// Bytes of the split partials a step of this handle writes in one layer's
// attention, laid out as kvc_attend_noalloc places them in the fixed
// scratch: decode (m, l) and o per (row, head, split slot), then, when the
// step has chunk rows, the same per (row, token, head, split slot) with the
// step's chunk width C as the token stride.
struct ScratchPlan {
  int64_t dml = 0, dout = 0, pml = 0, pout = 0, total = 0;
};
ScratchPlan scratch_plan(const kvc_t *h) {
  const int64_t B = h->cfg.batch, Hq = h->cfg.n_q_head, D = h->cfg.head_dim;
  const int64_t dq = B * Hq * kvc::kDecodeSplitCap;
  ScratchPlan p;
  int64_t cur = 0;
  p.dml = cur;
  cur = round_up(cur + dq * 8, 256);
  p.dout = cur;
  cur = round_up(cur + dq * D * 4, 256);
  bool chunk = false;
  if (!h->step_static)
    for (int32_t b = 0; b < h->cfg.batch; ++b) chunk |= h->n_new[b] >= 2;
  if (chunk) {
    const int64_t pq = B * (int64_t)h->C * Hq * kvc::kChunkSplitCap;
    p.pml = cur;
    cur = round_up(cur + pq * 8, 256);
    p.pout = cur;
    cur = round_up(cur + pq * D * 4, 256);
  } else {
    p.pml = p.pout = -1;
  }
  p.total = cur;
  return p;
}

// One layer's attention (kvc_attend).  `scratch`: the split partials go to
// this device array, laid out by scratch_plan, instead of the handle's buffer.
// `ck`, `cv` (kvc_append_attend on a ring layer whose rows all hold 2 ..
// kChunkOwnMax tokens; the layer is marked appended but nothing was staged):
// the chunk kernel takes the chunk's rows from the caller's K and V and
// commits them, with the slot indices to `slot_out`.
int attend_layer(kvc_t *h, int32_t layer, const void *q, void *out, void *stream,
                 char *scratch, const void *ck = nullptr, const void *cv = nullptr,
                 int32_t *slot_out = nullptr) {
  if (!h || !q || !out) return KVC_E_ARG;
  if (layer < 0 || layer >= h->cfg.n_layer) return KVC_E_ARG;
  if (!h->in_step || !h->appended[layer] || h->attended[layer]) return KVC_E_STATE;
  const int32_t jl = h->lay.layers[layer].joint;
  const bool joint = jl >= 0;
  if (joint && !h->appended[jl]) return KVC_E_STATE;  // the partner's keys of this step first
  ScratchPlan sp;
  if (scratch) {
    sp = scratch_plan(h);
    if (sp.total > kvc::kNoAllocScratchBytes) return KVC_E_SCRATCH;
  }
  // Where this call's split partials live.
  auto parts = [&]() {
    kvc::PartialArgs pa = partial_args(h);
    if (scratch) {
      pa.dml = reinterpret_cast<float *>(scratch + sp.dml);
      pa.dout = reinterpret_cast<float *>(scratch + sp.dout);
      pa.pml = sp.pml >= 0 ? reinterpret_cast<float *>(scratch + sp.pml) : nullptr;
      pa.pout = sp.pout >= 0 ? reinterpret_cast<float *>(scratch + sp.pout) : nullptr;
      pa.max_chunk = h->C;
    }
    return pa;
  };
  if (!use_device(h)) return KVC_E_HIP;
  const kvc::StepArgs st = step_args(h);
  const kvc::LayerArgs la = layer_args(h, layer);
  const kvc::LayerArgs lj = joint ? layer_args(h, jl) : kvc::LayerArgs{};
  const int32_t B = h->cfg.batch, D = h->cfg.head_dim;
  bool staged = false;
  if (!h->step_static)
    for (int32_t b = 0; b < B; ++b) staged |= (h->n_new[b] >= 2);
  staged = staged && la.ring && la.sk;

  const bool fast = h->cfg.dtype == KVC_BF16 && kvc::fast_decode_supported(D, la.rep) &&
                    kvc::fast_prefill_supported(D, la.rep);
  int err = 0;
  bool committed = false;  // the chunk launches committed the staged ring rows
  if (fast && h->C == 1 && wg_layer(h, layer, la)) {
    // a one-token step over a short window: the workgroup form writes every
    // row's output (static steps too: its grid is one workgroup per row)
    kvc::PartialArgs pa = parts();
    kvc::FusedArgs fa;
    fa.out = out;
    if (kvc::launch_decode_wg(st, la, pa, q, fa, false, launch_on(h, KVC_K_DECODE, stream)))
      return KVC_E_HIP;
  } else if (fast && h->step_static) {
    // one-token rows only; the plan is on the device
    kvc::PartialArgs pa = parts();
    const int32_t items = static_plan(h, layer, &pa);
    err = kvc::launch_decode(st, la, pa, q, items, launch_on(h, KVC_K_DECODE, stream));
    if (err) return KVC_E_HIP;
    err = kvc::launch_combine(h->cfg.dtype, st, la, pa, out, launch_on(h, KVC_K_COMBINE, stream));
    if (err) return KVC_E_HIP;
  } else if (!fast) {
    err = kvc::launch_generic(h->cfg.dtype, st, la, lj, q, out, launch_on(h, KVC_K_GENERIC, stream));
    if (err) return KVC_E_HIP;
  } else {
    // A joint layer's own splits and its partner's share a query's partial
    // slots: each side is planned within half the caps.
    const int32_t dcap = joint ? kvc::kDecodeSplitCap / 2 : kvc::kDecodeSplitCap;
    const int32_t ccap = joint ? kvc::kChunkSplitCap / 2 : kvc::kChunkSplitCap;
    // Plan one layer's keys: decode rows (one token) and chunk rows (two or
    // more tokens); launch its decode and chunk kernels.
    auto run = [&](const kvc::LayerArgs &lx, kvc::PartialArgs *pa) -> int {
      int64_t max_chunk_span = 0;
      for (int32_t b = 0; b < B; ++b) {
        const int64_t L = h->lens_host[b], n = h->n_new[b];
        int64_t base, hi;
        if (n >= 2 && !lx.ring) {
          chunk_span(lx, L, n, h->first_host[b], &base, &hi);
          max_chunk_span = std::max(max_chunk_span, hi - base);
        }
      }
      pa->dec_split_keys = decode_split_keys(h, lx, D, dcap);
      decode_order(h, lx, pa);
      // Chunk rows of at most 128 query rows (a 4-wave workgroup's tile) go
      // to a 4-wave launch, two of whose workgroups share a CU, instead of
      // leaving half of an 8-wave workgroup idle.
      pa->chunk_small = h->no_chunk_small ? 0 : 1;
      // A ring layer's chunk rows are one split each, so a small batch gives
      // its 8-wave launch fewer workgroups than CUs; then every chunk row
      // goes to the 4-wave launch, twice the workgroups for the same work.
      if (pa->chunk_small && lx.ring && !h->no_ring_small) {
        int64_t wg8 = 0;
        for (int32_t b = 0; b < B; ++b) {
          const int64_t n = h->n_new[b];
          if (n >= 2 && n * lx.rep > kvc::kChunkQTile / 2)
            wg8 += ceil_div(n * lx.rep, kvc::kChunkQTile) * lx.hkv;
        }
        if (wg8 > 0 && wg8 < h->n_cu) pa->chunk_small = 2;
      }
      // Chunk split length.  Each launch (8-wave and 4-wave workgroups) is
      // priced as a list schedule over its resident slots (the workgroups of
      // each kind a CU holds at once, from the occupancy query): the larger of its total work over the
      // slots and its longest item, where an item costs its keys plus a fixed
      // kChunkSplitCost (staging the query tile, writing and merging a
      // partial).  The split count per row (1 .. ccap, never under
      // kChunkSplitMin keys) with the lowest sum wins, ties to more splits.
      // Uniform long rows (a batched prefill) come out at fewer splits than
      // the cap; rows of mixed lengths, whose longest item sets the time,
      // keep the cap.
      {
        int32_t *occ = h->chunk_occ[lx.rep <= 16 ? lx.rep : 0];
        if (occ[0] == 0) occ[0] = std::max(1, kvc::chunk_wgs_per_cu(D, lx.rep, 8));
        if (occ[1] == 0) occ[1] = std::max(1, kvc::chunk_wgs_per_cu(D, lx.rep, 4));
        const int64_t slots8 = occ[0] * (int64_t)h->n_cu, slots4 = occ[1] * (int64_t)h->n_cu;
        auto cost = [&](int64_t sk) {
          int64_t sum8 = 0, sum4 = 0, top8 = 0, top4 = 0;
          for (int32_t b = 0; b < B; ++b) {
            const int64_t L = h->lens_host[b], n = h->n_new[b];
            if (n < 2 || lx.ring) continue;
            const bool small =
                pa->chunk_small == 2 || (pa->chunk_small && n * lx.rep <= kvc::kChunkQTile / 2);
            const int64_t nqt =
                ceil_div(n * lx.rep, small ? kvc::kChunkQTile / 2 : kvc::kChunkQTile);
            int64_t base, span_hi;
            chunk_span(lx, L, n, h->first_host[b], &base, &span_hi);
            const int64_t span = span_hi - base;
            const int64_t w = nqt * lx.hkv * (span + ceil_div(span, sk) * kChunkSplitCost);
            (small ? sum4 : sum8) += w;
            int64_t &top = small ? top4 : top8;
            top = std::max(top, std::min(span, sk) + kChunkSplitCost);
          }
          return std::max((sum8 + slots8 - 1) / slots8, top8) +
                 std::max((sum4 + slots4 - 1) / slots4, top4);
        };
        auto keys_for = [&](int64_t k) {
          return std::max<int64_t>(kChunkSplitMin,
                                   round_up(ceil_div(max_chunk_span, k), kvc::kRowAlign));
        };
        int64_t best = keys_for(ccap);
        if (!h->chunk_cap_only && max_chunk_span > 0) {
          int64_t best_cost = cost(best);
          for (int64_t k = ccap - 1; k >= 1; --k) {
            const int64_t sk = keys_for(k);
            if (sk == best) continue;
            const int64_t c = cost(sk);
            if (c < best_cost) best = sk, best_cost = c;
          }
        }
        pa->pre_split_keys = (int32_t)std::min<int64_t>(best, 1 << 30);
      }
      if (h->log_level >= 2 && layer == 0 && max_chunk_span > 0)
        std::fprintf(stderr, "[kvc] chunk plan: %d keys per split (longest span %lld)\n",
                     pa->pre_split_keys, (long long)max_chunk_span);
      int64_t dec_items = 0, pre_items = 0, small_items = 0;
      for (int32_t b = 0; b < B; ++b) {
        const int64_t L = h->lens_host[b], n = h->n_new[b];
        int64_t base, hi;
        if (n == 1) {
          decode_span(lx, L, h->first_host[b], &base, &hi);
          dec_items += ceil_div(hi - base, pa->dec_split_keys);
        } else if (n >= 2) {
          const bool small =
              pa->chunk_small == 2 || (pa->chunk_small && n * lx.rep <= kvc::kChunkQTile / 2);
          const int64_t nqt = ceil_div(n * lx.rep, small ? kvc::kChunkQTile / 2 : kvc::kChunkQTile);
          int64_t nks = 1;
          if (!lx.ring) {
            chunk_span(lx, L, n, h->first_host[b], &base, &hi);
            nks = ceil_div(hi - base, pa->pre_split_keys);
          }
          (small ? small_items : pre_items) += nqt * nks;
        }
      }
      if (h->log_level >= 2 && layer == 0 && dec_items > 0)
        std::fprintf(stderr, "[kvc] decode plan: %d keys per split, %lld waves\n",
                     pa->dec_split_keys, (long long)dec_items * lx.hkv);
      // (Running the decode launch on a second stream beside the chunk
      // launches measured 4 % slower on mixed steps: they take CUs from each
      // other, so they stay in order on one stream.)
      if (dec_items > 0 &&
          kvc::launch_decode(st, lx, *pa, q, (int32_t)dec_items, launch_on(h, KVC_K_DECODE, stream)))
        return KVC_E_HIP;
      // With rows of both sizes, neither chunk launch fills the chip alone:
      // the 4-wave one runs on the side stream beside the 8-wave one (they
      // write disjoint partial slots), joined back before the merge.  Once
      // forked, the join is enqueued whatever the launches return.
      void *s4 = stream;
      if (pre_items > 0 && small_items > 0 && h->side) {
        if (hipEventRecord(h->fork, static_cast<hipStream_t>(stream)) != hipSuccess ||
            hipStreamWaitEvent(h->side, h->fork, 0) != hipSuccess)
          return KVC_E_HIP;
        s4 = h->side;
      }
      // The 128-row query tiles run in the key-halves form: eight waves, each
      // group of four over every other key tile, so a tile's keys take half
      // the steps (a ring layer's small batch: two waves per SIMD instead of
      // one, ring layer-step 35.3 -> 32.1 us; the mixed step 16.86 -> 16.66
      // ms).  Paged and contiguous layers take the same form, so that they
      // give the same bits.
      const int small_qw = !h->no_key_halves ? kvc::kChunkKeyHalves : 4;
      int rc = KVC_OK;
      if (pre_items > 0 && kvc::launch_prefill(st, lx, *pa, q, (int32_t)pre_items, 8,
                                               launch_on(h, KVC_K_PREFILL, stream)))
        rc = KVC_E_HIP;
      if (rc == KVC_OK && small_items > 0 &&
          kvc::launch_prefill(st, lx, *pa, q, (int32_t)small_items, small_qw,
                              launch_on(h, KVC_K_PREFILL, s4)))
        rc = KVC_E_HIP;
      if (s4 != stream && (hipEventRecord(h->join, h->side) != hipSuccess ||
                           hipStreamWaitEvent(static_cast<hipStream_t>(stream), h->join, 0) !=
                               hipSuccess))
        rc = KVC_E_HIP;
      if (rc != KVC_OK) return rc;
      return KVC_OK;
    };
    kvc::PartialArgs pa = parts();
    // A ring layer's chunk rows are one split each; when every row is a full
    // chunk (no decode rows, no padded queries, no idle rows) the chunk
    // kernel writes the outputs itself and the merge launch is skipped.
    bool direct = la.ring && !joint && h->C >= 2 && !h->no_direct;
    for (int32_t b = 0; b < B && direct; ++b) direct = h->n_new[b] == h->C;
    if (direct) pa.direct_out = out;
    // staged ring rows: the chunk launches commit them after scoring
    if (staged) pa.ring_cnt = reinterpret_cast<int32_t *>(h->base + h->lay.cnt_off);
    if (staged && ck) {
      pa.ck = ck;
      pa.cv = cv;
      pa.slot_out = slot_out;
    }
    if (run(la, &pa) != KVC_OK) return KVC_E_HIP;
    committed = staged;
    if (joint) {
      kvc::PartialArgs pj = parts();
      pj.base = kvc::SplitRef{1, la.ring, la.window, pa.dec_split_keys, pa.pre_split_keys};
      if (run(lj, &pj) != KVC_OK) return KVC_E_HIP;
      pa.joint = kvc::SplitRef{1, lj.ring, lj.window, pj.dec_split_keys, pj.pre_split_keys};
    }
    if (!direct) {
      err = kvc::launch_combine(h->cfg.dtype, st, la, pa, out, launch_on(h, KVC_K_COMBINE, stream));
      if (err) return KVC_E_HIP;
    }
  }
  if (staged && !committed) {
    err = kvc::launch_commit(h->cfg.dtype, st, la, launch_on(h, KVC_K_COMMIT, stream));
    if (err) return KVC_E_HIP;
  }
  h->attended[layer] = 1;
  return KVC_OK;
}

}  // namespace

extern "C" {

int kvc_attend(kvc_t *h, int32_t layer, const void *q, void *out, void *stream) {
  return attend_layer(h, layer, q, out, stream, nullptr);
}

int kvc_attend_noalloc(kvc_t *h, int32_t layer, const void *q, void *out, void *stream) {
  if (!h) return KVC_E_ARG;
  if (!h->scratch) return KVC_E_HIP;  // the device array's address was never found
  return attend_layer(h, layer, q, out, stream, static_cast<char *>(h->scratch));
}

int kvc_append_attend(kvc_t *h, int32_t layer, const void *q, const void *k, const void *v,
                      const int32_t *n_new_host, int32_t C, int32_t *slot_out_dev, void *out,
                      void *stream) {
  if (!h || !q || !k || !v || !out) return KVC_E_ARG;
  if (layer < 0 || layer >= h->cfg.n_layer) return KVC_E_ARG;
  const kvc::LayerArgs la = layer_args(h, layer);
  const int32_t B = h->cfg.batch, D = h->cfg.head_dim;
  const bool fused = C == 1 && !h->no_fused && h->cfg.dtype == KVC_BF16 &&
                     kvc::fast_decode_supported(D, la.rep) && h->lay.layers[layer].joint < 0;
  // A ring layer's chunk step: when every row holds 2 .. kChunkOwnMax tokens
  // the chunk kernel reads them from k and v, scores them and commits them
  // to the ring (no staging, no append launch).  A joint layer's partner
  // keeps staging: the joint layer reads its staged rows.
  const bool ring_chunk = C >= 2 && C <= kvc::kChunkOwnMax && !h->no_chunk_fused && la.ring &&
                          la.sk && !la.paged && h->cfg.dtype == KVC_BF16 &&
                          kvc::fast_decode_supported(D, la.rep) &&
                          kvc::fast_prefill_supported(D, la.rep) &&
                          h->lay.layers[layer].joint < 0 && !h->partner_only[layer];
  if (ring_chunk) {
    const int rc = begin_append(h, layer, n_new_host, C, stream);
    if (rc != KVC_OK) return rc;
    bool all = true;
    for (int32_t b = 0; b < B; ++b) all = all && h->n_new[b] >= 2;
    if (all) {
      h->appended[layer] = 1;
      return attend_layer(h, layer, q, out, stream, nullptr, k, v, slot_out_dev);
    }
  }
  if (!fused) {
    const int rc = kvc_append(h, layer, k, v, n_new_host, C, slot_out_dev, stream);
    if (rc != KVC_OK) return rc;
    return kvc_attend(h, layer, q, out, stream);
  }
  const int rc = begin_append(h, layer, n_new_host, C, stream);
  if (rc != KVC_OK) return rc;
  const kvc::StepArgs st = step_args(h);
  kvc::PartialArgs pa = partial_args(h);
  if (wg_layer(h, layer, la)) {  // the workgroup form, appending too
    kvc::FusedArgs fa;
    fa.k = k;
    fa.v = v;
    fa.slot_out = slot_out_dev;
    fa.out = out;
    if (kvc::launch_decode_wg(st, la, pa, q, fa, true, launch_on(h, KVC_K_FUSED, stream)))
      return KVC_E_HIP;
    h->appended[layer] = 1;
    h->attended[layer] = 1;
    return KVC_OK;
  }
  int64_t items = 0;
  if (h->step_static) {
    items = static_plan(h, layer, &pa);
  } else {
    pa.dec_split_keys = decode_split_keys(h, la, D);
    decode_order(h, la, &pa);
    for (int32_t b = 0; b < B; ++b) {
      if (h->n_new[b] == 1) {
        int64_t base, hi;
        decode_span(la, h->lens_host[b], h->first_host[b], &base, &hi);
        items += ceil_div(hi - base, pa.dec_split_keys);
      } else {
        items += 1;  // idle row: its padded token and zero outputs
      }
    }
    if (h->log_level >= 2 && layer == 0)
      std::fprintf(stderr, "[kvc] fused decode plan: %d keys per split, %lld waves\n",
                   pa.dec_split_keys, (long long)items * la.hkv);
  }
  kvc::FusedArgs fa;
  fa.k = k;
  fa.v = v;
  fa.slot_out = slot_out_dev;
  fa.out = out;
  fa.cnt = reinterpret_cast<int32_t *>(h->base + h->lay.cnt_off);
  if (kvc::launch_decode_fused(st, la, pa, q, fa, (int32_t)items, h->fused_merge,
                               launch_on(h, KVC_K_FUSED, stream)))
    return KVC_E_HIP;
  if (!h->fused_merge &&
      kvc::launch_combine(h->cfg.dtype, st, la, pa, out, launch_on(h, KVC_K_COMBINE, stream)))
    return KVC_E_HIP;
  h->appended[layer] = 1;
  h->attended[layer] = 1;
  return KVC_OK;
}

int kvc_advance(kvc_t *h, void *stream) {
  if (!h) return KVC_E_ARG;
  if (!h->in_step) return KVC_E_STATE;
  for (int32_t l = 0; l < h->cfg.n_layer; ++l)
    if (!h->appended[l] || (!h->attended[l] && !h->partner_only[l])) return KVC_E_STATE;
  if (!use_device(h)) return KVC_E_HIP;
  int32_t *lens = reinterpret_cast<int32_t *>(h->base + h->lay.lens_off);
  const int32_t *nn = reinterpret_cast<const int32_t *>(h->base + h->lay.nnew_off);
  if (kvc::launch_advance(lens, nn, h->cfg.batch, stream)) return KVC_E_HIP;
  if (h->step_static) {
    h->lens_stale = true;  // the counts never reached the host
  } else {
    for (int32_t b = 0; b < h->cfg.batch; ++b) h->lens_host[b] += h->n_new[b];
  }
  h->in_step = false;
  h->step_static = false;
  return KVC_OK;
}

int kvc_lens(const kvc_t *h, int32_t *lens_host) {
  if (!h || !lens_host) return KVC_E_ARG;
  if (h->lens_stale) return KVC_E_STATE;
  std::copy(h->lens_host.begin(), h->lens_host.end(), lens_host);
  return KVC_OK;
}

int kvc_page_stats(const kvc_t *h, int64_t *used, int64_t *allocated, int64_t *reserved) {
  if (!h || !used || !allocated || !reserved) return KVC_E_ARG;
  if (h->lens_stale) return KVC_E_STATE;
  int64_t u = 0, held = 0;
  for (int32_t b = 0; b < h->cfg.batch; ++b) {
    u += h->lens_host[b];
    held += (int64_t)h->row_pages[b].size();
  }
  *used = u;
  if (h->lay.n_pages > 0) {
    *allocated = held * kvc::kPageRows;
    *reserved = (int64_t)h->lay.n_pages * kvc::kPageRows;
  } else {
    *allocated = *reserved = (int64_t)h->cfg.batch * h->cfg.max_len;
  }
  return KVC_OK;
}

int kvc_reserve(kvc_t *h, const int32_t *rows_host, const int32_t *tokens_host, int32_t n_rows,
                void *stream) {
  if (!h || n_rows < 0 || (n_rows > 0 && (!rows_host || !tokens_host))) return KVC_E_ARG;
  if (h->in_step) return KVC_E_STATE;
  for (int32_t i = 0; i < n_rows; ++i)
    if (rows_host[i] < 0 || rows_host[i] >= h->cfg.batch || tokens_host[i] < 0) return KVC_E_ARG;
  for (int32_t i = 0; i < n_rows; ++i)
    if (tokens_host[i] > h->cfg.max_len) return KVC_E_FULL;
  if (h->lay.n_pages == 0 || n_rows == 0) return KVC_OK;
  if (!use_device(h)) return KVC_E_HIP;
  std::vector<int32_t> rows(rows_host, rows_host + n_rows);
  std::vector<int64_t> tokens(tokens_host, tokens_host + n_rows);
  return take_pages(h, rows, tokens, stream);
}

int kvc_static_begin(kvc_t *h, const int32_t *n_new_dev, void *stream) {
  if (!h || !n_new_dev) return KVC_E_ARG;
  if (h->in_step) return KVC_E_STATE;
  if ((int32_t)h->classes.size() > kvc::kStaticClassMax) return KVC_E_ARG;
  for (const LayerLayout &L : h->lay.layers)
    if (L.joint >= 0) return KVC_E_ARG;  // joint layers plan on the host
  if (!use_device(h)) return KVC_E_HIP;
  kvc::StaticBeginArgs a{};
  a.n_src = n_new_dev;
  a.n_new = reinterpret_cast<int32_t *>(h->base + h->lay.nnew_off);
  a.lens = reinterpret_cast<const int32_t *>(h->base + h->lay.lens_off);
  a.first = reinterpret_cast<const int32_t *>(h->base + h->lay.first_off);
  a.cap = h->lay.n_pages > 0 ? reinterpret_cast<const int32_t *>(h->base + h->lay.cap_off)
                             : nullptr;
  a.flags = reinterpret_cast<int32_t *>(h->base + h->lay.flags_off);
  a.plan_sk = reinterpret_cast<int32_t *>(h->base + h->lay.plan_off);
  a.plan_order = h->cfg.batch <= kvc::kDecodeOrderMax
                     ? reinterpret_cast<uint16_t *>(h->base + h->lay.plan_off + 4 * h->cfg.n_layer)
                     : nullptr;
  a.B = h->cfg.batch;
  a.max_len = h->cfg.max_len;
  a.n_class = (int32_t)h->classes.size();
  for (int32_t c = 0; c < a.n_class; ++c) {
    kvc::StaticClass &cl = h->classes[c];
    kvc::LayerArgs la{};
    la.hkv = cl.hkv;
    la.rep = h->cfg.n_q_head / cl.hkv;
    cl.target = (int32_t)std::min<int64_t>(decode_wave_target(h, la, h->cfg.head_dim), 1 << 30);
    cl.min_tiles = h->dec_min_tiles;
    cl.fixed_q = h->dec_split_fixed > 0 ? h->dec_split_fixed / kvc::kDecodeTile : 0;
    a.cls[c] = cl;
  }
  if (kvc::launch_static_begin(a, stream)) return KVC_E_HIP;
  h->C = 1;
  h->in_step = true;
  h->step_static = true;
  std::fill(h->appended.begin(), h->appended.end(), 0);
  std::fill(h->attended.begin(), h->attended.end(), 0);
  return KVC_OK;
}

int kvc_static_status(kvc_t *h, int32_t *flags_host, void *stream) {
  if (!h || !flags_host) return KVC_E_ARG;
  if (h->in_step) return KVC_E_STATE;
  if (!use_device(h)) return KVC_E_HIP;
  int32_t *flags = reinterpret_cast<int32_t *>(h->base + h->lay.flags_off);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, flags, 4, hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return KVC_E_HIP;
  const int32_t zero = 0;
  if (kvc::launch_set_rows(flags, &zero, 1, stream)) return KVC_E_HIP;
  *flags_host = v;
  return KVC_OK;
}

int kvc_sync_lens(kvc_t *h, void *stream) {
  if (!h) return KVC_E_ARG;
  if (h->in_step) return KVC_E_STATE;
  if (!use_device(h)) return KVC_E_HIP;
  const int32_t *lens = reinterpret_cast<const int32_t *>(h->base + h->lay.lens_off);
  if (hipMemcpyAsync(h->lens_host.data(), lens, (size_t)h->cfg.batch * 4, hipMemcpyDeviceToHost,
                     (hipStream_t)stream) != hipSuccess ||
      hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return KVC_E_HIP;
  h->lens_stale = false;
  return KVC_OK;
}

int kvc_layer_layout(const kvc_t *h, int32_t layer, kvc_layer_info *info) {
  if (!h || !info || layer < 0 || layer >= h->cfg.n_layer) return KVC_E_ARG;
  const LayerLayout &L = h->lay.layers[layer];
  info->k_offset = L.k_off;
  info->v_offset = L.v_off;
  info->stage_k_offset = L.sk_off;
  info->stage_v_offset = L.sv_off;
  info->n_kv_head = L.hkv;
  info->window = L.window;
  info->is_ring = L.ring;
  info->rows = L.rows;
  info->rows_alloc = L.rows_alloc;
  info->stage_rows_alloc = L.stage_rows_alloc;
  return KVC_OK;
}

int kvc_buffer_info(const kvc_t *h, kvc_buffer_info_t *info) {
  if (!h || !info) return KVC_E_ARG;
  info->total_bytes = h->lay.total;
  info->kv_bytes = h->lay.kv_bytes;
  info->lens_offset = h->lay.lens_off;
  info->n_new_offset = h->lay.nnew_off;
  info->rope_offset = h->lay.rope_off;
  return KVC_OK;
}

int kvc_timing_begin(kvc_t *h, int32_t max_launches) {
  return kvc_timing_begin_kinds(h, max_launches, (1 << KVC_K_NKINDS) - 1);
}

int kvc_timing_begin_kinds(kvc_t *h, int32_t max_launches, int32_t kind_mask) {
  if (!h || max_launches < 1 || (kind_mask & ~((1 << KVC_K_NKINDS) - 1)) != 0) return KVC_E_ARG;
  if ((int32_t)h->ev.size() < 2 * max_launches) {
    while ((int32_t)h->ev.size() < 2 * max_launches) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return KVC_E_HIP;
      h->ev.push_back(e);
    }
  }
  h->ev_kind.assign(max_launches, 0);
  h->ev_used = 0;
  h->ev_mask = kind_mask;
  h->timing = true;
  return KVC_OK;
}

int kvc_timing_spans(kvc_t *h, int32_t cap, int32_t *kinds, double *start_ms, double *end_ms) {
  if (!h || cap < 0 || (cap > 0 && (!kinds || !start_ms || !end_ms))) return KVC_E_ARG;
  if (!h->timing) return KVC_E_STATE;
  const int32_t n = std::min(cap, h->ev_used);
  for (int32_t i = 0; i < n; ++i) {
    float a = 0.f, b = 0.f;
    if (hipEventSynchronize(h->ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&a, h->ev[0], h->ev[2 * i]) != hipSuccess ||
        hipEventElapsedTime(&b, h->ev[0], h->ev[2 * i + 1]) != hipSuccess)
      return KVC_E_HIP;
    kinds[i] = h->ev_kind[i];
    start_ms[i] = a;
    end_ms[i] = b;
  }
  return n;
}

int kvc_timing_end(kvc_t *h, double *ms_per_kind, int32_t *launches_per_kind) {
  if (!h || !ms_per_kind || !launches_per_kind) return KVC_E_ARG;
  if (!h->timing) return KVC_E_STATE;
  for (int k = 0; k < KVC_K_NKINDS; ++k) {
    ms_per_kind[k] = 0.0;
    launches_per_kind[k] = 0;
  }
  int rc = KVC_OK;
  for (int32_t i = 0; i < h->ev_used; ++i) {
    if (hipEventSynchronize(h->ev[2 * i + 1]) != hipSuccess) {
      rc = KVC_E_HIP;
      break;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, h->ev[2 * i], h->ev[2 * i + 1]) != hipSuccess) {
      rc = KVC_E_HIP;
      break;
    }
    ms_per_kind[h->ev_kind[i]] += ms;
    launches_per_kind[h->ev_kind[i]] += 1;
  }
  h->timing = false;
  h->ev_used = 0;
  return rc;
}

}  // extern "C"
