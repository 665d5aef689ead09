// Drives the library's host code (config validation, layout, step protocol,
// split planning, page allocator, static steps, admits, timing) through its
// C ABI over host memory, with the HIP runtime and the kernel launchers
// replaced by hip_host_stub.cpp.  Built with -fsanitize=address,undefined,
// so any out-of-bounds access, use after free, leak or undefined arithmetic
// in that code aborts the run.  Prints "ok" and exits 0 when every check
// holds.
//
// The protocol checked is the pages' (pycraft-1 "model/kv_cache.py": update
// per layer, advance once; tiny_agent "generate.py" append: "KV cache full"
// before anything is written).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../../include/kvc.h"

extern "C" void stub_register(const void *p, size_t n);
extern "C" void stub_unregister(const void *p);
extern "C" void stub_clear();
extern "C" long stub_launches();

namespace {

int g_checks = 0;

#define CHECK(cond)                                                               \
  do {                                                                            \
    ++g_checks;                                                                   \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
      std::exit(1);                                                               \
    }                                                                             \
  } while (0)

struct Buf {
  void *p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
    CHECK(p != nullptr);
    std::memset(p, 0xA5, n);
    stub_register(p, n);
  }
  ~Buf() {
    stub_unregister(p);
    std::free(p);
  }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
};

struct Cfg {
  std::vector<int32_t> hkv, win, joint;
  kvc_config c{};
  Cfg(int L, int B, int hq, int D, int max_len, int max_chunk, int dtype,
      std::vector<int32_t> hkv_, std::vector<int32_t> win_, int n_pages = 0,
      std::vector<int32_t> joint_ = {})
      : hkv(std::move(hkv_)), win(std::move(win_)), joint(std::move(joint_)) {
    c.n_layer = L;
    c.batch = B;
    c.n_q_head = hq;
    c.head_dim = D;
    c.max_len = max_len;
    c.max_chunk = max_chunk;
    c.dtype = dtype;
    c.n_kv_head = hkv.data();
    c.window = win.data();
    c.use_ring = 1;
    c.rope_base = 10000.0;
    c.n_pages = n_pages;
    c.joint = joint.empty() ? nullptr : joint.data();
  }
};

// A cache over a host buffer plus "device" q/k/v/out big enough for any step.
struct Run {
  Cfg &cfg;
  Buf buf;
  Buf io;
  kvc_t *h = nullptr;
  std::vector<int32_t> lens;
  explicit Run(Cfg &c)
      : cfg(c), buf(kvc_nbytes(&c.c, KVC_NB_ALLOC)),
        io((size_t)c.c.batch * c.c.max_chunk * c.c.n_q_head * c.c.head_dim * 4 * 4 + 4096) {
    CHECK(buf.n > 0);
    CHECK(kvc_nbytes(&c.c, KVC_NB_KV) > 0 && kvc_nbytes(&c.c, KVC_NB_KV) < buf.n);
    CHECK(kvc_create(&c.c, buf.p, buf.n - 1, nullptr, &h) == KVC_E_ARG && h == nullptr);
    CHECK(kvc_create(&c.c, buf.p, buf.n, nullptr, &h) == KVC_OK && h != nullptr);
    lens.assign(c.c.batch, 0);
  }
  ~Run() { kvc_destroy(h); }
  char *q() { return static_cast<char *>(io.p); }
  char *k() { return static_cast<char *>(io.p) + io.n / 4; }
  char *v() { return static_cast<char *>(io.p) + io.n / 2; }
  char *out() { return static_cast<char *>(io.p) + 3 * (io.n / 4); }
  void check_lens() {
    std::vector<int32_t> got(cfg.c.batch);
    CHECK(kvc_lens(h, got.data()) == KVC_OK);
    CHECK(got == lens);
    kvc_buffer_info_t bi{};
    CHECK(kvc_buffer_info(h, &bi) == KVC_OK);
    const int32_t *dev = reinterpret_cast<const int32_t *>(static_cast<char *>(buf.p) + bi.lens_offset);
    for (int b = 0; b < cfg.c.batch; ++b) CHECK(dev[b] == lens[b]);
  }
  // One step: every layer appended then attended (some layers through the
  // one-call entry point), then advance.
  void step(const std::vector<int32_t> &n, int C, std::mt19937 &g) {
    const int L = cfg.c.n_layer;
    std::vector<int> order;
    for (int l = 0; l < L; ++l) {
      const bool one_call = (g() % 2) == 0 && (cfg.joint.empty());
      if (one_call) {
        CHECK(kvc_append_attend(h, l, q(), k(), v(), n.data(), C, nullptr, out(), nullptr) == KVC_OK);
      } else {
        CHECK(kvc_append(h, l, k(), v(), n.data(), C, nullptr, nullptr) == KVC_OK);
        order.push_back(l);
      }
    }
    // out-of-order checks inside the step
    CHECK(kvc_advance(h, nullptr) == (order.empty() ? KVC_OK : KVC_E_STATE));
    if (order.empty()) {
      for (int b = 0; b < cfg.c.batch; ++b) lens[b] += n[b];
      return;
    }
    CHECK(kvc_reset(h, std::vector<int32_t>{0}.data(), 1, nullptr) == KVC_E_STATE);
    CHECK(kvc_append(h, order[0], k(), v(), n.data(), C, nullptr, nullptr) == KVC_E_STATE);
    // every other layer through the fixed-scratch entry point, which
    // refuses a step whose partials would not fit it
    bool chunk = false;
    for (int32_t x : n) chunk |= x >= 2;
    const int64_t B = cfg.c.batch, Hq = cfg.c.n_q_head, D = cfg.c.head_dim;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    int64_t need = up(B * Hq * 64 * 8) + up(B * Hq * 64 * D * 4);
    if (chunk) need += up(B * C * Hq * 16 * 8) + up(B * C * Hq * 16 * D * 4);
    for (int l : order) {
      if (l % 2) {
        const int rc = kvc_attend_noalloc(h, l, q(), out(), nullptr);
        CHECK(rc == (need <= (int64_t)KVC_NOALLOC_SCRATCH_BYTES ? KVC_OK : KVC_E_SCRATCH));
        if (rc == KVC_OK) continue;
      }
      CHECK(kvc_attend(h, l, q(), out(), nullptr) == KVC_OK);
    }
    CHECK(kvc_attend(h, order[0], q(), out(), nullptr) == KVC_E_STATE);
    CHECK(kvc_advance(h, nullptr) == KVC_OK);
    for (int b = 0; b < cfg.c.batch; ++b) lens[b] += n[b];
  }
};

std::vector<int32_t> draw_counts(std::mt19937 &g, const std::vector<int32_t> &lens, int C,
                                 int max_len, int mode) {
  std::vector<int32_t> n(lens.size());
  for (size_t b = 0; b < lens.size(); ++b) {
    int x;
    if (mode == 0) x = (int)(g() % 2);                      // decode / idle
    else if (mode == 1) x = (g() % 2) ? 1 : (int)(g() % (C + 1));  // mixed
    else x = C;                                             // full chunks
    if (lens[b] + x > max_len) x = max_len - lens[b];
    n[b] = x;
  }
  return n;
}

void exercise(Cfg &cfg, int steps, unsigned seed, bool chunks) {
  Run r(cfg);
  std::mt19937 g(seed);
  r.check_lens();
  const int max_len = cfg.c.max_len;
  for (int s = 0; s < steps; ++s) {
    const int C = chunks && (s % 3 != 2) ? 1 + (int)(g() % cfg.c.max_chunk) : 1;
    const int mode = C == 1 ? 0 : (s % 3 == 1 ? 2 : 1);
    std::vector<int32_t> n = draw_counts(g, r.lens, C, max_len, mode);
    r.step(n, C, g);
    r.check_lens();
  }
  // guards: a count past C, a C past max_chunk, a full row, a bad layer
  {
    std::vector<int32_t> n(cfg.c.batch, 0);
    n[0] = 2;
    CHECK(kvc_append(r.h, 0, r.k(), r.v(), n.data(), 1, nullptr, nullptr) == KVC_E_ARG);
    CHECK(kvc_append(r.h, 0, r.k(), r.v(), n.data(), cfg.c.max_chunk + 1, nullptr, nullptr) ==
          KVC_E_ARG);
    CHECK(kvc_append(r.h, cfg.c.n_layer, r.k(), r.v(), n.data(), 2, nullptr, nullptr) == KVC_E_ARG);
    CHECK(kvc_attend(r.h, 0, r.q(), r.out(), nullptr) == KVC_E_STATE);
    CHECK(kvc_advance(r.h, nullptr) == KVC_E_STATE);
    // fill row 0 to max_len, then one more token is "KV cache full"
    const int gap = max_len - r.lens[0];
    if (gap > 0 && gap <= cfg.c.max_chunk) {
      std::vector<int32_t> m(cfg.c.batch, 0);
      m[0] = gap;
      r.step(m, gap, g);
      r.check_lens();
    }
    if (r.lens[0] == max_len) {
      std::vector<int32_t> m(cfg.c.batch, 0);
      m[0] = 1;
      CHECK(kvc_append(r.h, 0, r.k(), r.v(), m.data(), 1, nullptr, nullptr) == KVC_E_FULL);
      r.check_lens();
    }
  }
  // reset some rows, left padding, then more steps
  {
    std::vector<int32_t> rows;
    for (int b = 0; b < cfg.c.batch; b += 3) rows.push_back(b);
    CHECK(kvc_reset(r.h, rows.data(), (int32_t)rows.size(), nullptr) == KVC_OK);
    for (int b : rows) r.lens[b] = 0;
    std::vector<int32_t> first(rows.size(), 2);
    CHECK(kvc_set_first(r.h, rows.data(), first.data(), (int32_t)rows.size(), nullptr) == KVC_OK);
    std::vector<int32_t> bad_first(rows.size(), max_len + 1);
    CHECK(kvc_set_first(r.h, rows.data(), bad_first.data(), (int32_t)rows.size(), nullptr) ==
          KVC_E_ARG);
    r.check_lens();
    for (int s = 0; s < 3; ++s) {
      std::vector<int32_t> n = draw_counts(g, r.lens, 1, max_len, 0);
      r.step(n, 1, g);
      r.check_lens();
    }
  }
  // page statistics and reservations
  {
    int64_t used = 0, alloc = 0, res = 0;
    CHECK(kvc_page_stats(r.h, &used, &alloc, &res) == KVC_OK);
    int64_t want = 0;
    for (int32_t x : r.lens) want += x;
    CHECK(used == want && alloc >= used && res >= alloc);
    std::vector<int32_t> rows{0}, toks{max_len + 1};
    CHECK(kvc_reserve(r.h, rows.data(), toks.data(), 1, nullptr) == KVC_E_FULL);
    toks[0] = r.lens[0];
    CHECK(kvc_reserve(r.h, rows.data(), toks.data(), 1, nullptr) == KVC_OK);
  }
  // timing on a few steps
  {
    CHECK(kvc_timing_begin_kinds(r.h, 4, 1 << KVC_K_NKINDS) == KVC_E_ARG);
    CHECK(kvc_timing_begin(r.h, 64) == KVC_OK);
    std::vector<int32_t> n = draw_counts(g, r.lens, 1, max_len, 0);
    r.step(n, 1, g);
    double ms[KVC_K_NKINDS];
    int32_t cnt[KVC_K_NKINDS];
    int32_t kinds[8];
    double t0[8], t1[8];
    const int ns = kvc_timing_spans(r.h, 8, kinds, t0, t1);
    CHECK(ns >= 1 && ns <= 8);
    for (int i = 0; i < ns; ++i) CHECK(kinds[i] >= 0 && kinds[i] < KVC_K_NKINDS && t1[i] >= t0[i]);
    CHECK(kvc_timing_end(r.h, ms, cnt) == KVC_OK);
    CHECK(kvc_timing_spans(r.h, 8, kinds, t0, t1) == KVC_E_STATE);
    CHECK(kvc_timing_end(r.h, ms, cnt) == KVC_E_STATE);
    r.check_lens();
  }
  // a static one-token step (counts in "device" memory), unless joint layers
  if (cfg.joint.empty()) {
    Buf nn(4 * (size_t)cfg.c.batch);
    std::vector<int32_t> n = draw_counts(g, r.lens, 1, max_len, 0);
    std::memcpy(nn.p, n.data(), 4 * n.size());
    CHECK(kvc_static_begin(r.h, static_cast<const int32_t *>(nn.p), nullptr) == KVC_OK);
    for (int l = 0; l < cfg.c.n_layer; ++l)
      CHECK(kvc_append_attend(r.h, l, r.q(), r.k(), r.v(), nullptr, 1, nullptr, r.out(), nullptr) ==
            KVC_OK);
    CHECK(kvc_advance(r.h, nullptr) == KVC_OK);
    std::vector<int32_t> tmp(cfg.c.batch);
    CHECK(kvc_lens(r.h, tmp.data()) == KVC_E_STATE);
    CHECK(kvc_sync_lens(r.h, nullptr) == KVC_OK);
    for (int b = 0; b < cfg.c.batch; ++b) r.lens[b] += n[b];
    r.check_lens();
    int32_t flags = -1;
    CHECK(kvc_static_status(r.h, &flags, nullptr) == KVC_OK);
  }
  // admit rows into a second cache of the same shapes
  {
    Run d(cfg);
    const int m = cfg.c.batch < 4 ? cfg.c.batch : 4;
    std::vector<int32_t> dst, src;
    for (int i = 0; i < m; ++i) {
      dst.push_back(cfg.c.batch - 1 - i);
      src.push_back(i);
    }
    CHECK(kvc_admit(d.h, dst.data(), r.h, src.data(), m, nullptr) == KVC_OK);
    for (int i = 0; i < m; ++i) d.lens[dst[i]] = r.lens[src[i]];
    d.check_lens();
    std::vector<int32_t> dup(2, 0);
    if (cfg.c.batch >= 2) CHECK(kvc_admit(d.h, dup.data(), r.h, src.data(), 2, nullptr) == KVC_E_ARG);
  }
  // layouts are inside the buffer
  for (int l = 0; l < cfg.c.n_layer; ++l) {
    kvc_layer_info li{};
    CHECK(kvc_layer_layout(r.h, l, &li) == KVC_OK);
    CHECK(li.k_offset >= 0 && (size_t)li.v_offset < r.buf.n && li.rows_alloc > li.rows);
  }
}

void validation() {
  // invalid and overflowing configurations are refused, not wrapped
  Cfg ok(2, 2, 8, 64, 64, 8, KVC_BF16, {2, 2}, {0, 0});
  CHECK(kvc_nbytes(&ok.c, KVC_NB_ALLOC) > 0);
  CHECK(kvc_nbytes(&ok.c, 7) == 0);
  CHECK(kvc_nbytes(nullptr, KVC_NB_KV) == 0);
  Cfg huge(1, 1 << 30, 1 << 20, 256, 1 << 30, 1024, KVC_F32, {1 << 20}, {0});
  CHECK(kvc_nbytes(&huge.c, KVC_NB_ALLOC) == 0);
  Cfg wide(1, 1 << 20, 256, 256, 1 << 22, 1024, KVC_BF16, {256}, {0});
  CHECK(kvc_nbytes(&wide.c, KVC_NB_ALLOC) == 0);
  Cfg region(1, 2, 8, 128, 8388576, 1, KVC_BF16, {2}, {0});
  CHECK(kvc_nbytes(&region.c, KVC_NB_ALLOC) == 0);
  region.c.max_len = 8388575;
  CHECK(kvc_nbytes(&region.c, KVC_NB_ALLOC) > 0);
  Cfg neg(1, 2, 8, 64, 64, 8, KVC_BF16, {2}, {-1});
  CHECK(kvc_nbytes(&neg.c, KVC_NB_KV) == 0);
  Cfg pages(1, 2, 8, 64, 64, 8, KVC_BF16, {2}, {0}, (1 << 30) + 1);
  CHECK(kvc_nbytes(&pages.c, KVC_NB_KV) == 0);
  Cfg joint(3, 2, 8, 64, 64, 8, KVC_BF16, {2, 2, 2}, {0, 16, 0}, 0, {-1, 2, -1});
  CHECK(kvc_nbytes(&joint.c, KVC_NB_KV) == 0);
  kvc_t *h = reinterpret_cast<kvc_t *>(1);
  CHECK(kvc_create(&ok.c, nullptr, 1 << 20, nullptr, &h) == KVC_E_ARG && h == nullptr);
  CHECK(kvc_create(&ok.c, reinterpret_cast<void *>(100), 1u << 30, nullptr, &h) == KVC_E_ARG);
  CHECK(std::strcmp(kvc_strerror(KVC_E_FULL), "KV cache full") == 0);
  kvc_destroy(nullptr);
}

}  // namespace

int main() {
  validation();
  // decode rows of a full-cache stack (B 64, Hq 32 / Hkv 8, D 128)
  Cfg dec(3, 64, 32, 128, 512, 1, KVC_BF16, {8, 8, 8}, {0, 0, 0});
  exercise(dec, 12, 1, false);
  // rings and a global layer, chunked prefill over wrapping rings
  Cfg ring(8, 4, 8, 64, 64, 48, KVC_BF16, {2, 2, 2, 2, 2, 2, 2, 2}, {8, 8, 8, 8, 8, 8, 8, 0});
  exercise(ring, 14, 2, true);
  // mixed chunk and decode rows, 4-wave and 8-wave chunk launches
  Cfg mixed(2, 32, 32, 128, 1024, 64, KVC_BF16, {8, 8}, {0, 0});
  exercise(mixed, 10, 3, true);
  // a paged cache beside a ring
  Cfg paged(3, 6, 16, 128, 256, 32, KVC_BF16, {4, 4, 4}, {0, 64, 0}, 96);
  exercise(paged, 12, 4, true);
  // hybrid layer groups (joint partners)
  Cfg hybrid(5, 4, 8, 64, 128, 16, KVC_BF16, {2, 2, 2, 2, 2}, {0, 16, 8, 0, 16}, 0,
             {-1, 0, 0, -1, 3});
  exercise(hybrid, 8, 5, true);
  // fp32 (generic kernel) and a window mask over a full layout
  Cfg f32(2, 3, 8, 64, 96, 16, KVC_F32, {2, 4}, {0, 24});
  f32.c.use_ring = 0;
  exercise(f32, 10, 6, true);
  // more rows than the decode order table holds
  Cfg wide(2, 300, 8, 64, 64, 4, KVC_BF16, {2, 2}, {0, 16});
  exercise(wide, 6, 7, true);
  stub_clear();
  std::printf("ok: %d checks, %ld launches\n", g_checks, stub_launches());
  return 0;
}
