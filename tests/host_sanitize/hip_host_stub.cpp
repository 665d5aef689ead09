// Host stand-ins for the HIP runtime calls and the kernel launchers that the
// library's host code (kvc_api.cpp, layout.cpp) uses, so that code can run
// without a GPU under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// "Device" memory is host memory here.  The runtime stand-ins copy and fill
// it for real; the small bookkeeping launchers (row lengths, left padding,
// n_new, block tables, advance) do what their kernels do, so the state the
// driver checks stays consistent; the attention launchers do no arithmetic
// but check that every pointer they receive lies inside the buffer the
// driver registered and that the split plans fit the partial-slot caps.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../kv_cached_gqa_append_amd/csrc/kvc_internal.h"

namespace stub {

struct Range {
  const char *lo, *hi;
};
std::vector<Range> g_ranges;
int g_cu = 256;
long g_launches = 0;

}  // namespace stub

extern "C" void stub_register(const void *p, size_t n) {
  stub::g_ranges.push_back({static_cast<const char *>(p), static_cast<const char *>(p) + n});
}
extern "C" void stub_unregister(const void *p) {
  for (size_t i = 0; i < stub::g_ranges.size(); ++i)
    if (stub::g_ranges[i].lo == static_cast<const char *>(p)) {
      stub::g_ranges.erase(stub::g_ranges.begin() + (long)i);
      return;
    }
}
extern "C" void stub_clear() { stub::g_ranges.clear(); }
extern "C" long stub_launches() { return stub::g_launches; }

namespace {

[[noreturn]] void fail(const char *what) {
  std::fprintf(stderr, "host stub: %s\n", what);
  std::abort();
}

// p .. p + n must sit inside one registered buffer (p may be null when allowed).
void inside(const void *p, size_t n, const char *what, bool may_be_null = false) {
  if (!p) {
    if (may_be_null) return;
    fail(what);
  }
  const char *c = static_cast<const char *>(p);
  for (const stub::Range &r : stub::g_ranges)
    if (c >= r.lo && c + n <= r.hi) return;
  fail(what);
}

struct Ev {
  int recorded = 0;
};
struct St {
  int dummy = 0;
};

}  // namespace

// ---------------------------------------------------------------------------
// HIP runtime stand-ins
// ---------------------------------------------------------------------------
hipError_t hipGetDevice(int *d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int d) { return d == 0 ? hipSuccess : hipErrorInvalidDevice; }
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int) {
  *v = stub::g_cu;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemsetAsync(void *dst, int value, size_t n, hipStream_t) {
  inside(dst, n, "hipMemsetAsync outside the buffer");
  std::memset(dst, value, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t *s, unsigned int) {
  *s = reinterpret_cast<hipStream_t>(new St());
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  delete reinterpret_cast<St *>(s);
  return hipSuccess;
}
hipError_t hipEventCreate(hipEvent_t *e) {
  *e = reinterpret_cast<hipEvent_t>(new Ev());
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t *e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<Ev *>(e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  reinterpret_cast<Ev *>(e)->recorded = 1;
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned int) {
  if (!reinterpret_cast<Ev *>(e)->recorded) fail("wait on an event never recorded");
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t) {
  *ms = 0.001f;
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launcher stand-ins (the kernels' host entry points)
// ---------------------------------------------------------------------------
namespace kvc {

namespace {

void check_step(const StepArgs &st) {
  inside(st.lens, sizeof(int32_t) * st.B, "lens");
  inside(st.n_new, sizeof(int32_t) * st.B, "n_new");
  inside(st.first, sizeof(int32_t) * st.B, "first");
  if (st.rope) inside(st.rope, sizeof(float) * 2 * st.max_len * (st.D / 2), "rope table");
  if (st.C < 1 || st.B < 1) fail("step shape");
}

void check_layer(const StepArgs &st, const LayerArgs &la) {
  if (la.hkv < 1 || la.rep < 1 || la.hkv * la.rep != st.Hq) fail("layer heads");
  if (la.paged) {
    inside(la.table, sizeof(int32_t) * st.B * la.ppr, "block table");
    inside(la.k, 1, "paged K pool");
    inside(la.v, 1, "paged V pool");
  } else {
    const size_t region = (size_t)st.B * la.hkv * la.rows_alloc * st.D;  // elements
    inside(la.k, region, "K region (bytes >= elements)");
    inside(la.v, region, "V region (bytes >= elements)");
    if (la.rows_alloc < la.rows + 1 || la.rows_alloc % kRowAlign % kVBlock) fail("rows_alloc");
  }
  if (la.sk) {
    inside(la.sk, (size_t)st.B * la.hkv * la.stage_rows_alloc * st.D, "stage K");
    inside(la.sv, (size_t)st.B * la.hkv * la.stage_rows_alloc * st.D, "stage V");
    if (la.stage_rows_alloc < st.C) fail("stage rows below the chunk");
  }
}

// The split plan of a decode launch: every decoding row's splits fit its
// partial slots.  The span is the layer's key range for a query at lens[b].
void check_decode_plan(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                       int32_t n_items, bool idle_items) {
  if (pa.dec_plan) {  // a static step: the plan is on the device
    inside(pa.dec_plan, 4, "static plan");
    return;
  }
  const int64_t sk = pa.dec_split_keys;
  if (sk < kDecodeTile || sk % kDecodeTile) fail("decode split keys");
  int64_t items = 0;
  for (int b = 0; b < st.B; ++b) {
    const int n = st.n_new[b];
    if (n != 1) {
      items += idle_items ? 1 : 0;
      continue;
    }
    const int64_t p = st.lens[b];
    int64_t lo = 0, hi;
    if (la.ring) {
      hi = p + 1 < la.window ? p + 1 : la.window;
    } else {
      hi = p + 1;
      lo = la.window > 0 && p - la.window + 1 > 0 ? p - la.window + 1 : 0;
      lo = p < st.first[b] ? p : (lo > st.first[b] ? lo : st.first[b]);
      lo = lo / kRowAlign * kRowAlign;
    }
    const int64_t ns = (hi - lo + sk - 1) / sk;
    if (ns > kDecodeSplitCap) fail("decode splits past the slot cap");
    items += ns;
  }
  if (pa.joint.on == 0 && pa.base.on == 0 && items != n_items) fail("decode item count");
}

}  // namespace

int launch_set_rows(int32_t *dst, const int32_t *vals, int32_t n, void *) {
  inside(dst, sizeof(int32_t) * n, "set_rows");
  std::memcpy(dst, vals, sizeof(int32_t) * n);
  ++stub::g_launches;
  return 0;
}
int launch_reset_rows(int32_t *lens, int32_t *first, const int32_t *rows, int32_t n, void *) {
  for (int32_t i = 0; i < n; ++i) {
    inside(lens + rows[i], 4, "reset lens");
    inside(first + rows[i], 4, "reset first");
    lens[rows[i]] = 0;
    first[rows[i]] = 0;
  }
  ++stub::g_launches;
  return 0;
}
int launch_set_first(int32_t *first, const int32_t *rows, const int32_t *vals, int32_t n, void *) {
  for (int32_t i = 0; i < n; ++i) {
    inside(first + rows[i], 4, "set_first");
    first[rows[i]] = vals[i];
  }
  ++stub::g_launches;
  return 0;
}
int launch_copy_rows(const LayerArgs &dst, const LayerArgs &src, int, int, const CopyPairs &,
                     int32_t n_pairs, void *) {
  if (n_pairs < 1 || n_pairs > 64 || dst.hkv != src.hkv) return (int)hipErrorInvalidValue;
  inside(dst.k, 1, "copy dst");
  inside(src.k, 1, "copy src");
  ++stub::g_launches;
  return 0;
}
int launch_page_update(int32_t *table, int32_t *cap, const int32_t *cap_rows, const int32_t *cap_vals,
                       int32_t n_cap, const PageUpdate &u, int32_t n_upd, const PagedPools &pools,
                       int64_t page_bytes, void *) {
  if (n_cap < 0 || n_cap > 256 || n_upd < 0 || n_upd > 64) return (int)hipErrorInvalidValue;
  for (int32_t i = 0; i < n_upd; ++i) {
    inside(table + u.idx[i], 4, "block table entry");
    table[u.idx[i]] = u.page[i];
    for (int l = 0; l < pools.n; ++l)
      if (u.zero[i] >= 0)
        inside(pools.v[l] + (int64_t)u.zero[i] * page_bytes * pools.hkv[l],
               (size_t)(page_bytes * pools.hkv[l]), "zeroed page");
  }
  for (int32_t i = 0; i < n_cap; ++i) {
    inside(cap + cap_rows[i], 4, "row capacity");
    cap[cap_rows[i]] = cap_vals[i];
  }
  ++stub::g_launches;
  return 0;
}
int launch_copy_state(int32_t *dst_lens, int32_t *dst_first, const int32_t *src_lens,
                      const int32_t *src_first, const CopyPairs &pairs, int32_t n_pairs, void *) {
  if (n_pairs < 1 || n_pairs > 64) return (int)hipErrorInvalidValue;
  for (int32_t j = 0; j < n_pairs; ++j) {
    dst_lens[pairs.dst_row[j]] = src_lens[pairs.src_row[j]];
    dst_first[pairs.dst_row[j]] = src_first[pairs.src_row[j]];
  }
  ++stub::g_launches;
  return 0;
}
int launch_advance(int32_t *lens, const int32_t *n_new, int32_t B, void *) {
  inside(lens, 4 * (size_t)B, "advance lens");
  for (int32_t b = 0; b < B; ++b) lens[b] += n_new[b];
  ++stub::g_launches;
  return 0;
}
int launch_static_begin(const StaticBeginArgs &a, void *) {
  if (a.n_class < 1 || a.n_class > kStaticClassMax) return (int)hipErrorInvalidValue;
  inside(a.n_src, 4 * (size_t)a.B, "static counts");
  inside(a.plan_sk, 4 * (size_t)a.n_class, "static plan");
  // the counts become the step's (every count valid in the driver's use)
  std::memcpy(a.n_new, a.n_src, 4 * (size_t)a.B);
  ++stub::g_launches;
  return 0;
}
int launch_append(int, const StepArgs &st, const LayerArgs &la, const void *k, const void *v,
                  int32_t *slot_out, const Launch &) {
  check_step(st);
  check_layer(st, la);
  if (!k || !v) fail("append inputs");
  (void)slot_out;
  ++stub::g_launches;
  return 0;
}
int launch_commit(int, const StepArgs &st, const LayerArgs &la, const Launch &) {
  check_step(st);
  check_layer(st, la);
  if (!la.ring || !la.sk) fail("commit on a layer without staging");
  ++stub::g_launches;
  return 0;
}
int launch_decode(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, const void *q,
                  int32_t n_items, const Launch &) {
  check_step(st);
  check_layer(st, la);
  if (!q || n_items < 1) fail("decode launch");
  check_decode_plan(st, la, pa, n_items, false);
  inside(pa.dml, 8, "decode partials");
  ++stub::g_launches;
  return 0;
}
int launch_decode_fused(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                        const void *q, const FusedArgs &fa, int32_t n_items, bool, const Launch &) {
  if (st.C != 1) return (int)hipErrorInvalidValue;
  check_step(st);
  check_layer(st, la);
  if (!q || !fa.k || !fa.v || !fa.out || n_items < 1) fail("fused decode launch");
  inside(fa.cnt, 4 * (size_t)st.B * la.hkv, "split counters");
  check_decode_plan(st, la, pa, n_items, true);
  ++stub::g_launches;
  return 0;
}
int launch_decode_wg(const StepArgs &st, const LayerArgs &la, const PartialArgs &, const void *q,
                     const FusedArgs &fa, bool fused, const Launch &) {
  if (st.C != 1 || la.paged || (la.rep > 8 && la.rep != 16)) return (int)hipErrorInvalidValue;
  check_step(st);
  check_layer(st, la);
  if (!q || !fa.out || (fused && (!fa.k || !fa.v))) fail("workgroup decode launch");
  ++stub::g_launches;
  return 0;
}
int launch_prefill(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, const void *q,
                   int32_t n_items, int qw, const Launch &) {
  check_step(st);
  check_layer(st, la);
  if (!q || n_items < 1 || (qw != 4 && qw != 8 && qw != kChunkKeyHalves)) fail("chunk launch");
  if (qw == kChunkKeyHalves && !pa.chunk_small) fail("key-halves chunk launch");
  if (pa.pre_split_keys < kRowAlign || pa.pre_split_keys % kRowAlign) fail("chunk split keys");
  if (!pa.direct_out) inside(pa.pml, 8, "chunk partials");
  if ((pa.ck != nullptr) != (pa.cv != nullptr)) fail("chunk rows from k without v");
  if (pa.ck && (!la.ring || la.paged || !pa.ring_cnt || st.C < 2 || st.C > kChunkOwnMax))
    fail("chunk rows from the caller's k, v outside a ring layer's chunk step");
  ++stub::g_launches;
  return 0;
}
int launch_combine(int, const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, void *out,
                   const Launch &) {
  check_step(st);
  check_layer(st, la);
  if (!out) fail("combine output");
  inside(pa.dml, 8, "combine partials");
  ++stub::g_launches;
  return 0;
}
int launch_generic(int, const StepArgs &st, const LayerArgs &la, const LayerArgs &lj, const void *q,
                   void *out, const Launch &) {
  check_step(st);
  check_layer(st, la);
  if (lj.k) check_layer(st, lj);
  if (!q || !out) fail("generic launch");
  ++stub::g_launches;
  return 0;
}
void *noalloc_scratch(int device) {
  // a host stand-in for the device array, registered like the buffers
  static char *mem = nullptr;
  if (device != 0) return nullptr;
  if (!mem) {
    mem = static_cast<char *>(std::aligned_alloc(256, (size_t)kNoAllocScratchBytes));
    stub_register(mem, (size_t)kNoAllocScratchBytes);
  }
  return mem;
}
bool fast_decode_supported(int D, int rep) {
  return (D == 64 || D == 128) && (rep == 1 || rep == 2 || rep == 4 || rep == 8 || rep == 16);
}
int decode_waves_per_cu(int D, int rep) { return fast_decode_supported(D, rep) ? 8 : 0; }
bool fast_prefill_supported(int D, int rep) { return (D == 64 || D == 128) && rep >= 1; }
int chunk_wgs_per_cu(int D, int rep, int qw) { return fast_prefill_supported(D, rep) ? (qw == 4 ? 2 : 1) : 0; }

}  // namespace kvc
