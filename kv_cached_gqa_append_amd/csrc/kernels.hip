// HIP kernels for gfx950 (CDNA4): cached GQA attention with append.
//
// Cache layout per layer (all offsets int64):
//   K: [b][g][row][d]                row-major rows (the QK contraction runs
//                                    over d, contiguous)
//   V: [b][g][row/16][d][row%16]     16-row blocks stored transposed (the PV
//                                    contraction runs over rows, contiguous)
// rows = max_len (full layer) or W (ring layer), plus one scratch row at index
// `rows`, padded to a multiple of 32.  Ring layers with max_chunk >= 2 also
// own a staging area with the same two layouts for the rows of a multi-token
// chunk, which is scored from staging and committed to the ring afterwards.
//
// Sources (page titles and sections):
//  - tiny_agent "generate.py", _append_chunk: positions lens + i, padding to
//    the scratch index, ring keep rule (the last W real tokens), grouped query
//    heads h -> KV head h / rep, float32 softmax, P cast to the cache dtype
//    before P.V; _rope_pos: half-split rotation at absolute positions.
//  - colibri PR "inkling: ring-buffer KV cache for sliding-window layers",
//    "What this does": the W-key clamp qpos - W + 1 .. qpos; "How it works":
//    score the chunk from its own new rows, append after scoring.
//  - "Lab 07 - KV cache and sampling", section 2: query i at pos + i sees key
//    j iff j <= pos + i.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {

// ---------------------------------------------------------------------------
// The fixed scratch of kvc_attend_noalloc: one array per GPU, alive until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not device memory): noalloc_scratch() looks up
// its device address once per device and every launch takes that address.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
std::once_flag g_scratch_once[kNoAllocMaxDevices];
void *g_scratch_ptr[kNoAllocMaxDevices];
}  // namespace

void *noalloc_scratch(int device) {
  if (device < 0 || device >= kNoAllocMaxDevices) return nullptr;
  std::call_once(g_scratch_once[device], [device] {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != device) return;
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[device] = ptr;
  });
  return g_scratch_ptr[device];
}

typedef __bf16 bf16;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// RoPE of one (d, d + D/2) pair by (cos, sin), with the multiply-adds spelled
// out so every kernel rounds it identically.
__device__ __forceinline__ void rope_pair(float x1, float x2, float c, float sn, float *y1,
                                          float *y2) {
  *y1 = fmaf(x1, c, -(x2 * sn));
  *y2 = fmaf(x1, sn, x2 * c);
}

// DPP moves within a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;   // lane i <- 15 - i within the row
constexpr int kRowHalfMirror = 0x141;  // lane i <- 7 - i within each half-row

// Sum over aligned groups of G lanes (G in {1,2,4,8,16}); every lane of a
// group ends with the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if (G >= 2) x += dpp<kQuadXor1>(x);
  if (G >= 4) x += dpp<kQuadXor2>(x);
  if (G >= 8) x += dpp<kRowHalfMirror>(x);
  if (G >= 16) x += dpp<kRowMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch on lc's stream.  With timing events the dispatch itself stamps them
// (hipExtLaunchKernel); without, a plain launch, which stream capture records
// as a kernel node of the graph.
template <typename... KArgs, typename... Args>
static void launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, const Launch &lc,
                          Args... args) {
  if (lc.t0 || lc.t1)
    hipExtLaunchKernelGGL(kern, grid, block, 0, (hipStream_t)lc.stream, (hipEvent_t)lc.t0,
                          (hipEvent_t)lc.t1, 0, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, 0, (hipStream_t)lc.stream, args...);
}

// Element pointers.
template <typename T>
__device__ __forceinline__ T *k_row(char *base, int64_t bg, int rows_alloc, int64_t r, int D) {
  return reinterpret_cast<T *>(base) + (bg * rows_alloc + r) * D;
}
// Start of V block `blk` of head (b, g): D x 16 elements.
template <typename T>
__device__ __forceinline__ T *v_block(char *base, int64_t bg, int rows_alloc, int64_t blk, int D) {
  return reinterpret_cast<T *>(base) + ((bg * (rows_alloc / kVBlock) + blk) * D) * kVBlock;
}
template <typename T>
__device__ __forceinline__ T *v_elem(char *base, int64_t bg, int rows_alloc, int64_t r, int d, int D) {
  return v_block<T>(base, bg, rows_alloc, r / kVBlock, D) + d * kVBlock + (r % kVBlock);
}

// Element offset of the 16-row block holding storage row r of KV head g of
// row b in a layer's K or V region (r == rows: the scratch row).  Both
// layouts keep a block's 16 K rows, and its V block, contiguous; a paged
// layer finds the block's page in the block table (the scratch row in the
// scratch page), a full one at its place in the head's region.
__device__ __forceinline__ int64_t row_block_elem(const LayerArgs &la, int b, int g, int64_t r,
                                                  int D) {
  if (la.paged) {
    const int64_t pg = r < la.rows ? la.table[(int64_t)b * la.ppr + r / kPageRows]
                                   : (int64_t)la.scratch_page;
    return (pg * la.hkv + g) * kPageRows * D;
  }
  return (((int64_t)b * la.hkv + g) * la.rows_alloc + r / kPageRows * kPageRows) * D;
}
template <typename T>
__device__ __forceinline__ T *krow_ptr(const LayerArgs &la, int b, int g, int64_t r, int D) {
  return reinterpret_cast<T *>(la.k) + row_block_elem(la, b, g, r, D) + (r % kPageRows) * D;
}
// V element (r, d) of the head is at vcol_ptr(...)[d * kVBlock].
template <typename T>
__device__ __forceinline__ T *vcol_ptr(const LayerArgs &la, int b, int g, int64_t r, int D) {
  return reinterpret_cast<T *>(la.v) + row_block_elem(la, b, g, r, D) + (r % kPageRows);
}

// Position held by ring slot s before this step's commit, L = tokens so far:
// the latest t < L with t % W == s (negative: the slot is empty).
__device__ __forceinline__ int64_t ring_slot_pos(int64_t s, int64_t L, int W) {
  const int64_t r = L % W;
  return s < r ? (L - r + s) : (L - r - W + s);
}

// Keys of a one-token query at position p on this layer, for a row whose
// first `first` positions are left padding (identical spans to the host
// planner).  The first visible position is the window's (W > 0) or 0,
// raised to `first`; a pad query (p < first) sees only itself.  Storage rows
// [base, hi) are visited; row r there is visible iff r < hi and r - va,
// taken mod vwrap on a ring (vwrap = W; 0 on a full layer), lies in [0, vn).
// On a ring the visible positions fill slots [0, min(p + 1, W)) and the
// padding visible in the window is a run of consecutive slots mod W.
struct DecodeSpan {
  int64_t base, hi, va, vn;
  int32_t vwrap;
};
__device__ __forceinline__ DecodeSpan decode_span_dev(const LayerArgs &la, int64_t p,
                                                      int64_t first) {
  int64_t start = la.window > 0 ? (p - la.window + 1 > 0 ? p - la.window + 1 : 0) : 0;
  start = p < first ? p : (start > first ? start : first);
  DecodeSpan s;
  s.vn = p + 1 - start;
  if (la.ring) {
    s.base = 0;
    s.hi = p + 1 < la.window ? p + 1 : la.window;
    s.va = start % la.window;
    s.vwrap = la.window;
  } else {
    s.base = start / kRowAlign * kRowAlign;
    s.hi = p + 1;
    s.va = start;
    s.vwrap = 0;
  }
  return s;
}
// Key span of a chunk of n tokens from position L on a full layer: rows
// [lo, hi), visited from base.  Left padding raises lo to `first` unless the
// chunk holds pad queries (L < first), which see their own rows (>= L).
__device__ __forceinline__ void chunk_span_dev(const LayerArgs &la, int64_t L, int64_t n,
                                               int64_t first, int64_t *base, int64_t *lo,
                                               int64_t *hi) {
  *lo = la.window > 0 ? (L - la.window + 1 > 0 ? L - la.window + 1 : 0) : 0;
  const int64_t f = first < L ? first : L;
  if (f > *lo) *lo = f;
  *hi = L + n;
  *base = *lo / kRowAlign * kRowAlign;
}

// Splits of one layer for a row (see SplitRef): decode splits of a one-token
// row's span, or the key splits of a chunk row.
__device__ __forceinline__ int ref_splits(const SplitRef &r, int64_t L, int n, int64_t first) {
  LayerArgs la{};
  la.ring = r.ring;
  la.window = r.window;
  if (n == 1) {
    const DecodeSpan sp = decode_span_dev(la, L, first);
    return (int)cdiv(sp.hi - sp.base, r.dec_sk);
  }
  if (r.ring) return 1;
  int64_t base, lo, hi;
  chunk_span_dev(la, L, n, first, &base, &lo, &hi);
  return (int)cdiv(hi - base, r.pre_sk);
}

// ---------------------------------------------------------------------------
// tiny state kernels (values arrive as kernel arguments: no host staging)
// ---------------------------------------------------------------------------
struct I32Chunk {
  int32_t v[256];
};

__global__ void k_set_rows(int32_t *dst, I32Chunk c, int32_t n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = c.v[i];
}

__global__ void k_reset_rows(int32_t *lens, int32_t *first, I32Chunk rows, int32_t n) {
  const int i = threadIdx.x;
  if (i < n) {
    lens[rows.v[i]] = 0;
    first[rows.v[i]] = 0;
  }
}

__global__ void k_set_first(int32_t *first, I32Chunk rows, I32Chunk vals, int32_t n) {
  const int i = threadIdx.x;
  if (i < n) first[rows.v[i]] = vals.v[i];
}

// Grid (pairs x KV heads, 2 (K, V), blocks): one 16-row block (K rows or V
// block, contiguous in either layout) of one head of one pair per workgroup.
__global__ __launch_bounds__(256) void k_copy_rows(LayerArgs dst, LayerArgs src, int32_t D,
                                                   int32_t row_bytes, CopyPairs pr) {
  const int j = blockIdx.x / src.hkv, g = blockIdx.x % src.hkv;
  const int64_t blk = blockIdx.z;
  if (blk >= pr.blocks[j]) return;
  const int64_t r = blk * kPageRows;
  const int es = row_bytes / D;  // element size
  const char *sb = (blockIdx.y ? src.v : src.k) + row_block_elem(src, pr.src_row[j], g, r, D) * es;
  char *db = (blockIdx.y ? dst.v : dst.k) + row_block_elem(dst, pr.dst_row[j], g, r, D) * es;
  const int units = kPageRows * row_bytes / 16;
  for (int u = threadIdx.x; u < units; u += blockDim.x)
    reinterpret_cast<uint4 *>(db)[u] = reinterpret_cast<const uint4 *>(sb)[u];
}

// Block-table and capacity updates (workgroup 0) and the zeroing of V of
// newly taken pages, one page per further workgroup, in every paged layer.
__global__ __launch_bounds__(256) void k_page_update(int32_t *table, int32_t *cap, I32Chunk cap_rows,
                                                     I32Chunk cap_vals, int32_t n_cap, PageUpdate u,
                                                     int32_t n_upd, PagedPools pools,
                                                     int64_t page_bytes) {
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < n_upd; i += blockDim.x) table[u.idx[i]] = u.page[i];
    for (int i = threadIdx.x; i < n_cap; i += blockDim.x) cap[cap_rows.v[i]] = cap_vals.v[i];
    return;
  }
  const int k = blockIdx.x - 1;
  if (k >= n_upd || u.zero[k] < 0) return;
  const int64_t pg = u.zero[k];
  for (int l = 0; l < pools.n; ++l) {
    const int64_t bytes = page_bytes * pools.hkv[l];
    uint4 *dst = reinterpret_cast<uint4 *>(pools.v[l] + pg * bytes);
    for (int64_t e = threadIdx.x; e < bytes / 16; e += blockDim.x) dst[e] = make_uint4(0, 0, 0, 0);
  }
}

__global__ void k_copy_state(int32_t *dst_lens, int32_t *dst_first, const int32_t *src_lens,
                             const int32_t *src_first, CopyPairs pr, int32_t n) {
  const int j = threadIdx.x;
  if (j < n) {
    dst_lens[pr.dst_row[j]] = src_lens[pr.src_row[j]];
    dst_first[pr.dst_row[j]] = src_first[pr.src_row[j]];
  }
}

__global__ void k_advance(int32_t *lens, const int32_t *n_new, int32_t B) {
  for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x)
    lens[b] += n_new[b];
}

int launch_set_rows(int32_t *dst, const int32_t *vals, int32_t n, void *stream) {
  for (int32_t off = 0; off < n; off += 256) {
    I32Chunk c;
    const int32_t m = n - off < 256 ? n - off : 256;
    std::memset(&c, 0, sizeof(c));
    std::memcpy(c.v, vals + off, sizeof(int32_t) * m);
    hipLaunchKernelGGL(k_set_rows, dim3(1), dim3(256), 0, (hipStream_t)stream, dst + off, c, m);
  }
  return (int)hipGetLastError();
}

int launch_reset_rows(int32_t *lens, int32_t *first, const int32_t *rows, int32_t n,
                      void *stream) {
  for (int32_t off = 0; off < n; off += 256) {
    I32Chunk c;
    const int32_t m = n - off < 256 ? n - off : 256;
    std::memset(&c, 0, sizeof(c));
    std::memcpy(c.v, rows + off, sizeof(int32_t) * m);
    hipLaunchKernelGGL(k_reset_rows, dim3(1), dim3(256), 0, (hipStream_t)stream, lens, first, c,
                       m);
  }
  return (int)hipGetLastError();
}

int launch_set_first(int32_t *first, const int32_t *rows, const int32_t *vals, int32_t n,
                     void *stream) {
  for (int32_t off = 0; off < n; off += 256) {
    I32Chunk r, v;
    const int32_t m = n - off < 256 ? n - off : 256;
    std::memset(&r, 0, sizeof(r));
    std::memset(&v, 0, sizeof(v));
    std::memcpy(r.v, rows + off, sizeof(int32_t) * m);
    std::memcpy(v.v, vals + off, sizeof(int32_t) * m);
    hipLaunchKernelGGL(k_set_first, dim3(1), dim3(256), 0, (hipStream_t)stream, first, r, v, m);
  }
  return (int)hipGetLastError();
}

int launch_copy_rows(const LayerArgs &dst, const LayerArgs &src, int D, int dtype_bytes,
                     const CopyPairs &pairs, int32_t n_pairs, void *stream) {
  if (n_pairs < 1 || n_pairs > 64 || dst.hkv != src.hkv) return (int)hipErrorInvalidValue;
  int32_t most = 0;
  for (int32_t j = 0; j < n_pairs; ++j) {
    const int64_t rows = (int64_t)pairs.blocks[j] * kPageRows;
    if (pairs.blocks[j] < 0 || (!src.paged && rows > src.rows_alloc) ||
        (!dst.paged && rows > dst.rows_alloc) || (src.paged && rows > (int64_t)src.ppr * kPageRows) ||
        (dst.paged && rows > (int64_t)dst.ppr * kPageRows))
      return (int)hipErrorInvalidValue;
    most = pairs.blocks[j] > most ? pairs.blocks[j] : most;
  }
  if (most == 0) return 0;
  hipLaunchKernelGGL(k_copy_rows, dim3((unsigned)(n_pairs * src.hkv), 2, (unsigned)most), dim3(256),
                     0, (hipStream_t)stream, dst, src, (int32_t)D, (int32_t)(D * dtype_bytes), pairs);
  return (int)hipGetLastError();
}

int launch_page_update(int32_t *table, int32_t *cap, const int32_t *cap_rows, const int32_t *cap_vals,
                       int32_t n_cap, const PageUpdate &u, int32_t n_upd, const PagedPools &pools,
                       int64_t page_bytes, void *stream) {
  if (n_cap < 0 || n_cap > 256 || n_upd < 0 || n_upd > 64) return (int)hipErrorInvalidValue;
  I32Chunk cr, cv;
  std::memset(&cr, 0, sizeof(cr));
  std::memset(&cv, 0, sizeof(cv));
  if (n_cap) {
    std::memcpy(cr.v, cap_rows, sizeof(int32_t) * n_cap);
    std::memcpy(cv.v, cap_vals, sizeof(int32_t) * n_cap);
  }
  hipLaunchKernelGGL(k_page_update, dim3((unsigned)(1 + n_upd)), dim3(256), 0, (hipStream_t)stream,
                     table, cap, cr, cv, n_cap, u, n_upd, pools, page_bytes);
  return (int)hipGetLastError();
}

int launch_copy_state(int32_t *dst_lens, int32_t *dst_first, const int32_t *src_lens,
                      const int32_t *src_first, const CopyPairs &pairs, int32_t n_pairs,
                      void *stream) {
  if (n_pairs < 1 || n_pairs > 64) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy_state, dim3(1), dim3(64), 0, (hipStream_t)stream, dst_lens, dst_first,
                     src_lens, src_first, pairs, n_pairs);
  return (int)hipGetLastError();
}

int launch_advance(int32_t *lens, const int32_t *n_new, int32_t B, void *stream) {
  const int blocks = (int)cdiv(B, 256);
  hipLaunchKernelGGL(k_advance, dim3(blocks), dim3(256), 0, (hipStream_t)stream, lens, n_new, B);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static one-token step prologue: one wave per layer class.  Every wave
// checks the caller's counts against the device lengths (a count outside
// {0, 1} or a row that would pass max_len rejects the whole step: every
// count becomes 0, so nothing is appended and every output is zero, and the
// reason is or-ed into the sticky flags); wave 0 publishes the counts.  Each
// wave then plans its class's decode splits from the device lengths, exactly
// as the host planner does for an eager step (smallest split in tiles, not
// below the class's floor nor below 1/64 of the longest row, whose waves plus
// the idle rows' items fit one round), and the dispatch order (rows by tiles
// per split, descending; ties by row).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
  for (int o = 32; o >= 1; o >>= 1) {
    const int y = __shfl_xor(x, o);
    x = y > x ? y : x;
  }
  return x;
}
__device__ __forceinline__ int wave_or_i(int x) {
  for (int o = 32; o >= 1; o >>= 1) x |= __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(64) void k_static_begin(StaticBeginArgs a) {
  __shared__ int32_t tl[kDecodeOrderMax], nsl[kDecodeOrderMax];
  const int lane = threadIdx.x, c = blockIdx.x;
  const StaticClass cl = a.cls[c];
  int bad = 0;
  for (int b = lane; b < a.B; b += 64) {
    const int n = a.n_src[b];
    if (n < 0 || n > 1)
      bad |= kStaticBadCount;
    else if ((int64_t)a.lens[b] + n > a.max_len || (a.cap && a.lens[b] + n > a.cap[b]))
      bad |= kStaticFull;
  }
  bad = __builtin_amdgcn_readfirstlane(wave_or_i(bad));
  if (c == 0) {
    for (int b = lane; b < a.B; b += 64) a.n_new[b] = bad ? 0 : a.n_src[b];
    if (lane == 0 && bad) a.flags[0] = a.flags[0] | bad;
  }
  LayerArgs la{};
  la.window = cl.window;
  la.ring = cl.ring;
  auto tiles = [&](int b) -> int {  // tiles of a decoding row, 0 for an idle one
    if (bad || a.n_src[b] != 1) return 0;
    const DecodeSpan sp = decode_span_dev(la, a.lens[b], a.first[b]);
    return (int)cdiv(sp.hi - sp.base, kDecodeTile);
  };
  int max_t = 0, idle = 0;
  for (int b = lane; b < a.B; b += 64) {
    const int t = tiles(b);
    max_t = t > max_t ? t : max_t;
    idle += (bad || a.n_src[b] != 1) ? 1 : 0;
  }
  max_t = __builtin_amdgcn_readfirstlane(wave_max_i(max_t));
  idle = __builtin_amdgcn_readfirstlane((int)wave_sum_i64(idle));
  int q = 1;
  if (max_t > 0) {
    const int q_cap = (int)cdiv(max_t, kDecodeSplitCap);
    if (cl.fixed_q > 0) {
      q = cl.fixed_q > q_cap ? cl.fixed_q : q_cap;
    } else {
      int64_t target = (int64_t)cl.target - (int64_t)idle * cl.hkv;
      if (target < 1) target = 1;
      int lo = q_cap > cl.min_tiles ? q_cap : cl.min_tiles;
      int hi = lo > max_t ? lo : max_t;
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        int64_t w = 0;
        for (int b = lane; b < a.B; b += 64) w += cdiv(tiles(b), mid);
        w = wave_sum_i64(w) * cl.hkv;
        if (__builtin_amdgcn_readfirstlane((int)(w <= target)))
          hi = mid;
        else
          lo = mid + 1;
      }
      q = lo;
    }
  }
  if (lane == 0) a.plan_sk[c] = q * kDecodeTile;
  if (a.plan_order && a.B <= kDecodeOrderMax) {
    // per = tiles / splits (0 for idle rows); rank = rows with a larger per,
    // plus rows before this one with an equal per
    for (int b = lane; b < a.B; b += 64) {
      const int t = tiles(b);
      tl[b] = t;
      nsl[b] = t > 0 ? (int)cdiv(t, q) : 1;
    }
    __syncthreads();
    for (int b = lane; b < a.B; b += 64) {
      const int64_t t = tl[b], ns = nsl[b];
      int rank = 0;
      for (int o = 0; o < a.B; ++o) {
        const int64_t lhs = (int64_t)tl[o] * ns, rhs = t * nsl[o];
        rank += (lhs > rhs || (lhs == rhs && o < b)) ? 1 : 0;
      }
      a.plan_order[(int64_t)c * a.B + rank] = (uint16_t)b;
    }
  }
}

int launch_static_begin(const StaticBeginArgs &a, void *stream) {
  if (a.n_class < 1 || a.n_class > kStaticClassMax) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_static_begin, dim3((unsigned)a.n_class), dim3(64), 0, (hipStream_t)stream,
                     a);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// fused RoPE + append: one wave per (row b, token i, KV head g)
// ---------------------------------------------------------------------------

// Zero V rows [lo, end) of one head's region (end at most one 32-row tile
// past lo).  In the V layout each (16-row block, d) pair holds its 16 rows
// contiguously, so a block's rows from lo on are one run per d: element
// stores up to an 8-byte boundary, then 8-byte stores.  Lane l takes
// d = l, l + 64, ...
template <typename T>
__device__ __forceinline__ void zero_v_rows(char *base, int64_t bg, int rows_alloc, int64_t lo,
                                            int64_t end, int D, int lane) {
  constexpr int G = 8 / (int)sizeof(T);  // elements per 8-byte store
  for (int64_t blk = lo / kVBlock; blk * kVBlock < end; ++blk) {
    const int k0 = lo > blk * kVBlock ? (int)(lo - blk * kVBlock) : 0;
    const int k1 = end < (blk + 1) * kVBlock ? (int)(end - blk * kVBlock) : kVBlock;
    for (int d = lane; d < D; d += 64) {
      T *run = v_elem<T>(base, bg, rows_alloc, blk * kVBlock, d, D);
      int k = k0;
      for (; k < k1 && (k % G != 0 || k + G > k1); ++k) run[k] = from_f<T>(0.f);
      for (; k + G <= k1; k += G) *reinterpret_cast<uint2 *>(run + k) = make_uint2(0u, 0u);
      for (; k < k1; ++k) run[k] = from_f<T>(0.f);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(64) void k_append(StepArgs st, LayerArgs la, const T *__restrict__ k,
                                               const T *__restrict__ v, int32_t *slot_out) {
  const int64_t row = blockIdx.x;  // (b * C + i) * hkv + g
  const int g = (int)(row % la.hkv);
  const int64_t bi = row / la.hkv;
  const int i = (int)(bi % st.C);
  const int b = (int)(bi / st.C);
  const int64_t L = st.lens[b];
  const int n = st.n_new[b];
  const int64_t p = L + i;
  const bool valid = i < n;
  const int D = st.D, half = D / 2;
  const bool staged = la.ring && n >= 2 && la.sk != nullptr;

  if (slot_out && g == 0 && threadIdx.x == 0) {
    int64_t s;
    if (la.ring)
      s = (valid && p >= L + n - la.window) ? p % la.window : la.window;
    else
      s = valid ? p : la.rows;
    slot_out[(int64_t)b * st.C + i] = (int32_t)s;
  }
  // Rows past a row's end inside its current 32-row tile are read (and
  // masked) by the decode kernel; keep their V finite: when an append enters
  // a new tile, zero V in the rest of that tile.  The rows zeroed here are
  // beyond every row this append writes (only the scratch row may coincide,
  // and both writes are finite).
  // (A paged layer's pages have V zeroed when a row takes them.)
  if (i == 0 && n >= 1 && !la.paged) {
    const int64_t W = la.window;
    const int64_t old_top = la.ring ? (L < W ? L : W) : L;
    const int64_t new_top = la.ring ? (L + n < W ? L + n : W) : L + n;
    if (old_top == 0 || (new_top - 1) / kRowAlign != (old_top - 1) / kRowAlign) {
      int64_t end = (new_top + kRowAlign - 1) / kRowAlign * kRowAlign;
      if (end > la.rows_alloc) end = la.rows_alloc;
      zero_v_rows<T>(la.v, (int64_t)b * la.hkv + g, la.rows_alloc, new_top, end, st.D,
                     (int)threadIdx.x);
    }
  }
  const int64_t bg = (int64_t)b * la.hkv + g;
  // Staging: V rows past the chunk's n rows, to the end of their 32-row tile,
  // are zero (the chunk kernel reads whole tiles and masks those rows).
  if (staged && i == 0) {
    int64_t end = ((int64_t)n + kRowAlign - 1) / kRowAlign * kRowAlign;
    if (end > la.stage_rows_alloc) end = la.stage_rows_alloc;
    zero_v_rows<T>(la.sv, bg, la.stage_rows_alloc, n, end, st.D, (int)threadIdx.x);
  }
  T *kd, *vd;
  if (staged) {
    if (!valid) return;  // staging rows of padding are never read
    kd = k_row<T>(la.sk, bg, la.stage_rows_alloc, i, D);
    vd = v_elem<T>(la.sv, bg, la.stage_rows_alloc, i, 0, D);
  } else {
    int64_t r;
    if (la.ring)
      r = valid ? p % la.window : la.window;
    else
      r = valid ? p : la.rows;
    kd = krow_ptr<T>(la, b, g, r, D);
    vd = vcol_ptr<T>(la, b, g, r, D);
  }
  const T *ks = k + row * D;
  const T *vs = v + row * D;
  const bool rot = st.rope != nullptr && valid;
  for (int e = threadIdx.x; e < half; e += 64) {
    const float x1 = to_f(ks[e]), x2 = to_f(ks[e + half]);
    float y1 = x1, y2 = x2;
    if (rot) rope_pair(x1, x2, st.rope[(p * half + e) * 2 + 0], st.rope[(p * half + e) * 2 + 1],
                       &y1, &y2);
    kd[e] = from_f<T>(y1);
    kd[e + half] = from_f<T>(y2);
    // A padded token's V goes to the scratch row as zeros: the row can sit
    // inside a tile the decode kernel reads, and whatever the caller left in
    // padded positions must not reach an output through p = 0.
    vd[e * kVBlock] = valid ? vs[e] : from_f<T>(0.f);
    vd[(e + half) * kVBlock] = valid ? vs[e + half] : from_f<T>(0.f);
  }
}

int launch_append(int dtype, const StepArgs &st, const LayerArgs &la, const void *k,
                  const void *v, int32_t *slot_out, const Launch &lc) {
  const int64_t rows = (int64_t)st.B * st.C * la.hkv;
  if (dtype == KVC_F32)
    launch_kernel(k_append<float>, dim3((unsigned)rows), dim3(64), lc, st, la, (const float *)k, (const float *)v, slot_out);
  else
    launch_kernel(k_append<bf16>, dim3((unsigned)rows), dim3(64), lc, st, la, (const bf16 *)k, (const bf16 *)v, slot_out);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// ring commit: staged chunk rows -> ring slots, after the chunk was scored.
// Keep rule: only positions p >= L + n - W survive (the last W real tokens).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_commit(StepArgs st, LayerArgs la) {
  const int64_t row = blockIdx.x;
  const int g = (int)(row % la.hkv);
  const int64_t bi = row / la.hkv;
  const int i = (int)(bi % st.C);
  const int b = (int)(bi / st.C);
  const int64_t L = st.lens[b];
  const int n = st.n_new[b];
  if (n < 2 || i >= n) return;
  const int64_t p = L + i;
  if (p < L + n - la.window) return;
  const int64_t slot = p % la.window;
  const int D = st.D;
  const int64_t bg = (int64_t)b * la.hkv + g;
  const T *ks = k_row<T>(la.sk, bg, la.stage_rows_alloc, i, D);
  T *kd = k_row<T>(la.k, bg, la.rows_alloc, slot, D);
  const T *vs = v_elem<T>(la.sv, bg, la.stage_rows_alloc, i, 0, D);
  T *vd = v_elem<T>(la.v, bg, la.rows_alloc, slot, 0, D);
  for (int d = threadIdx.x; d < D; d += 64) {
    kd[d] = ks[d];
    vd[d * kVBlock] = vs[d * kVBlock];
  }
}

int launch_commit(int dtype, const StepArgs &st, const LayerArgs &la, const Launch &lc) {
  const int64_t rows = (int64_t)st.B * st.C * la.hkv;
  if (dtype == KVC_F32)
    launch_kernel(k_commit<float>, dim3((unsigned)rows), dim3(64), lc, st, la);
  else
    launch_kernel(k_commit<bf16>, dim3((unsigned)rows), dim3(64), lc, st, la);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// generic attention: one wave per query row (b, i, h), any dtype and shape.
// Sequential online softmax over the visible keys; writes the output itself.
// ---------------------------------------------------------------------------
template <typename T>
struct GenericState {
  float q[4], acc[4], m, l;
};

template <typename T>
__device__ __forceinline__ void generic_key(GenericState<T> &S, const T *krow, const T *vcol,
                                            int D, float scale) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d = lane + 64 * t;
    if (d < D) s += S.q[t] * to_f(krow[d]);
  }
  s = wave_sum(s) * scale;
  const float mn = fmaxf(S.m, s);
  const float alpha = __expf(S.m - mn);
  const float pe = __expf(s - mn);
  S.l = S.l * alpha + pe;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d = lane + 64 * t;
    if (d < D) S.acc[t] = S.acc[t] * alpha + pe * to_f(vcol[d * kVBlock]);
  }
  S.m = mn;
}

template <typename T>
__global__ __launch_bounds__(64) void k_generic(StepArgs st, LayerArgs la, LayerArgs lj,
                                                const T *__restrict__ q, T *__restrict__ out) {
  __shared__ float qs[256];
  const int64_t row = blockIdx.x;  // (b * C + i) * Hq + h
  const int h = (int)(row % st.Hq);
  const int64_t bi = row / st.Hq;
  const int i = (int)(bi % st.C);
  const int b = (int)(bi / st.C);
  const int lane = threadIdx.x;
  const int D = st.D, half = D / 2;
  T *o = out + row * D;
  const int64_t L = st.lens[b];
  const int n = st.n_new[b];
  if (i >= n) {
    for (int d = lane; d < D; d += 64) o[d] = from_f<T>(0.f);
    return;
  }
  const int64_t p = L + i;
  const int g = h / la.rep;
  const int64_t bg = (int64_t)b * la.hkv + g;
  const T *qr = q + row * D;
  for (int e = lane; e < half; e += 64) {
    const float x1 = to_f(qr[e]), x2 = to_f(qr[e + half]);
    float y1 = x1, y2 = x2;
    if (st.rope) {
      const float c = st.rope[(p * half + e) * 2 + 0];
      const float s = st.rope[(p * half + e) * 2 + 1];
      y1 = x1 * c - x2 * s;
      y2 = x1 * s + x2 * c;
    }
    qs[e] = y1;
    qs[e + half] = y2;
  }
  __syncthreads();
  GenericState<T> S;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d = lane + 64 * t;
    S.q[t] = d < D ? qs[d] : 0.f;
    S.acc[t] = 0.f;
  }
  S.m = -INFINITY;
  S.l = 0.f;
  const float scale = rsqrtf((float)D);
  const int W = la.window;
  // left padding: keys before `first` are hidden, except the query's own
  const int64_t first = st.first[b];
  auto hidden = [&](int64_t pos) { return pos < first && pos != p; };
  // a joint partner's keys (a full layout) join the same softmax first
  if (lj.k != nullptr) {
    const int Wj = lj.window;
    const int64_t lo = Wj > 0 ? (p - Wj + 1 > 0 ? p - Wj + 1 : 0) : 0;
    for (int64_t t = lo; t <= p; ++t) {
      if (hidden(t)) continue;
      generic_key(S, krow_ptr<T>(lj, b, g, t, D), vcol_ptr<T>(lj, b, g, t, D), D, scale);
    }
  }
  if (la.ring && n >= 2 && la.sk) {
    // history from the ring (slots holding positions within the window) ...
    const int64_t nh = L < W ? L : W;
    for (int64_t s = 0; s < nh; ++s) {
      const int64_t pos = ring_slot_pos(s, L, W);
      if (pos < 0 || p - pos >= W || hidden(pos)) continue;
      generic_key(S, krow_ptr<T>(la, b, g, s, D), vcol_ptr<T>(la, b, g, s, D), D, scale);
    }
    // ... and the chunk's own rows from staging
    for (int j = 0; j <= i; ++j) {
      if (i - j >= W || hidden(L + j)) continue;
      generic_key(S, k_row<T>(la.sk, bg, la.stage_rows_alloc, j, D),
                  v_elem<T>(la.sv, bg, la.stage_rows_alloc, j, 0, D), D, scale);
    }
  } else if (la.ring) {
    // one-token step: the visible positions fill slots [0, min(p + 1, W));
    // slot s holds the latest position <= p congruent to s mod W
    const int64_t hi = p + 1 < W ? p + 1 : W;
    for (int64_t s = 0; s < hi; ++s) {
      if (hidden(p - (p - s) % W)) continue;
      generic_key(S, krow_ptr<T>(la, b, g, s, D), vcol_ptr<T>(la, b, g, s, D), D, scale);
    }
  } else {
    const int64_t lo = W > 0 ? (p - W + 1 > 0 ? p - W + 1 : 0) : 0;
    for (int64_t t = lo; t <= p; ++t) {
      if (hidden(t)) continue;
      generic_key(S, krow_ptr<T>(la, b, g, t, D), vcol_ptr<T>(la, b, g, t, D), D, scale);
    }
  }
  const float inv = 1.f / S.l;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d = lane + 64 * t;
    if (d < D) o[d] = from_f<T>(S.acc[t] * inv);
  }
}

int launch_generic(int dtype, const StepArgs &st, const LayerArgs &la, const LayerArgs &lj,
                   const void *q, void *out, const Launch &lc) {
  const int64_t rows = (int64_t)st.B * st.C * st.Hq;
  if (dtype == KVC_F32)
    launch_kernel(k_generic<float>, dim3((unsigned)rows), dim3(64), lc, st, la, lj, (const float *)q,
                  (float *)out);
  else
    launch_kernel(k_generic<bf16>, dim3((unsigned)rows), dim3(64), lc, st, la, lj, (const bf16 *)q,
                  (bf16 *)out);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Work-item lookup: item `it` of the rows selected by `count(b)`, rows scanned
// 64 at a time by the whole wave.  Returns the row and the index inside it.
// ---------------------------------------------------------------------------
template <typename CountFn>
__device__ __forceinline__ void find_item(int B, int64_t it, CountFn count, int *row_out,
                                          int64_t *local_out) {
  const int lane = threadIdx.x & 63;
  int rem = (int)it;
  int row = -1, local = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < B ? count(b) : 0;
    const int incl = wave_incl_scan(c);
    // every value that steers control flow is made wave-uniform explicitly
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (rem < total) {
      const int excl = incl - c;
      const uint64_t ball = __ballot(rem >= excl && rem < incl);
      const int src = (int)__builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)ball) - 1);
      row = b0 + src;
      local = rem - __builtin_amdgcn_readlane(excl, src);
      break;
    }
    rem -= total;
  }
  *row_out = __builtin_amdgcn_readfirstlane(row);
  *local_out = __builtin_amdgcn_readfirstlane(local);
}

// ---------------------------------------------------------------------------
// Decode attention (rows with one new token), bf16.  One wave per
// (row, KV head, key split).  QK: LK lanes per key, each holding D/LK
// elements of all REP rotated queries in registers (<= 32 VGPRs for the
// common shapes); scores reduced with DPP inside a 16-lane row.  PV: each lane
// owns D/32 head-dim elements for 8 of the 16 keys of a V block and
// accumulates with bf16 dot2 over key pairs.  Online softmax in the exp2
// domain with one running max per query head (cross-row reductions with the
// gfx950 permlane swaps).  K/V tiles are double-buffered in registers.
// Fused mode (one-token steps): the last split block of a (row, KV head)
// merges the partials and writes the output; idle rows are zeroed.
// ---------------------------------------------------------------------------
// (the max of a lane and its partner in one instruction: fmaxf on values the
// compiler cannot prove canonical, as a swap's results are, first quiets
// both inputs, two instructions more; the values here are never NaN)
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// max(x, -FLT_MAX) in one instruction (fmaxf would first quiet x)
__device__ __forceinline__ float max_lowest(float x) {
  float r;
  asm("v_max_f32 %0, 0xff7fffff, %1" : "=v"(r) : "v"(x));
  return r;
}
// Maxima of a and of b over the wave's four 16-lane rows, into every lane
// of a and b.  A row-16 exchange of the pair sets rows (a0, b0, a2, b2)
// against (a1, b1, a3, b3), so one maximum reduces both to row pairs; a
// row-32 exchange and a second maximum leave (A, B, A, B), and a last
// row-16 exchange spreads A and B over whole registers.
__device__ __forceinline__ void rows_max_pair(float &a, float &b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float x = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float z = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Input uniform within aligned groups of G lanes; result: reduction over the
// whole wave, in every lane.
template <int G>
__device__ __forceinline__ float groups_max(float x) {
  if (G <= 4) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if (G <= 8) x = fmaxf(x, dpp<kRowMirror>(x));
  return swap32_max(swap16_max(x));
}
template <int G>
__device__ __forceinline__ float groups_sum(float x) {
  if (G <= 4) x += dpp<kRowHalfMirror>(x);
  if (G <= 8) x += dpp<kRowMirror>(x);
  return swap32_sum(swap16_sum(x));
}

template <int D, int REP>
struct DecodeShape {
  // lanes per key: enough that one lane's share of the REP queries fits in 32
  // VGPRs (bf16 pairs), at least 4 and at most D/8 (one 16-byte chunk)
  static constexpr int LKQ = REP * D / 64;
  static constexpr int LK0 = LKQ < 4 ? 4 : (LKQ > 16 ? 16 : LKQ);
  static constexpr int LK = LK0 > D / 8 ? D / 8 : LK0;
  static constexpr int KR = 64 / LK;            // keys per QK round
  static constexpr int TK = kDecodeTile;        // keys per tile (one V block)
  static_assert(TK == kVBlock, "a decode tile is one V block");
  static constexpr int NR = TK / KR;            // QK rounds per tile
  static constexpr int NCH = D / 8 / LK;        // 16-byte chunks per lane per key
  static constexpr int VT = D / 32;             // V head-dim rows per lane
  static constexpr int HPL = REP >= LK ? REP / LK : 1;   // heads whose scores a lane owns
  // Register tile ring and occupancy target per SIMD.  Shapes with
  // REP * D < 1024 keep one tile in flight beside the one in use and run
  // three waves per SIMD (136 VGPRs at D 128, REP 4): more independent
  // streams per CU measured 3 % faster than two waves with two tiles in
  // flight each (the same bytes in flight).  REP 16 keeps one tile in flight
  // at two waves (D 64) or, holding 64 accumulators and 64 query registers
  // per lane at D 128, at one wave with the full register file rather than
  // spill.
  // REP * D = 1024 with REP <= 8 (D 128, REP 8) keeps four tiles in flight
  // at one wave per SIMD, in both kernels: on 32k-key rows (B 8) the decode
  // kernel measured 182 -> 174 us per layer against two waves with two
  // tiles in flight, and the in-launch merge form 210 -> 177 us (half the
  // waves, so half the splits for the last split of a row to merge).  Five
  // tiles at one wave did not help REP 4 (about 4k-key rows), and six or
  // eight tiles at REP 4 were slower or did not fit.
  static constexpr bool BIG = REP * D >= 2048;
  static constexpr bool SMALL = REP * D < 1024;
  static constexpr bool DEEP = REP * D == 1024 && REP <= 8;
  static constexpr int NBUF = SMALL ? 2 : DEEP ? 5 : 2;
  static constexpr int WAVES = SMALL ? 3 : DEEP ? 1 : (BIG ? 1 : 2);
  // the in-launch merge form (it also holds the merge's registers: two waves)
  static constexpr int FNBUF = DEEP ? 5 : REP <= 8 ? 3 : 2;
  static constexpr int FWAVES = DEEP ? 1 : BIG ? 1 : 2;
  static_assert(NCH >= 1 && NR >= 1 && D % 32 == 0, "unsupported decode shape");
};

constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes) in scalar registers: no stride,
// raw 32-bit records, so out-of-range offsets read zero.
__device__ __forceinline__ i32x4 sgpr_rsrc(const void *base, int bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kRsrcWord3;
  return r;
}

// One of two descriptors, chosen by a wave-uniform condition, element by
// element (a select between two objects would go through memory), kept in
// scalar registers.
__device__ __forceinline__ i32x4 rsrc_sel(bool c, i32x4 a, i32x4 b) {
  i32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = __builtin_amdgcn_readfirstlane(c ? a[e] : b[e]);
  return u;
}

// Streaming tile loads are issued from inline assembly and their waits are
// placed by hand.  The compiler's own wait insertion cannot follow a ring of
// loads that stays in flight across a loop's back edge: it waits for every
// outstanding load at the first use in the loop, which leaves one tile in
// flight.  Each wait names the registers it covers ("+v"), so no use of a
// tile can be scheduled before its wait; the build scans the generated
// assembly for any other instruction touching a register between its load
// and its wait.  The loads are non-temporal (nt): every K and V byte is read
// once per step, and streaming them past the caches measured about 9 %
// faster on the decode launch than cached loads.
template <int OFF>
__device__ __forceinline__ void tile_load(u32x4 &x, i32x4 rsrc, int voff, int soff) {
  static_assert(OFF >= 0 && OFF < 4096, "buffer immediate offsets are 12 bits");
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4 nt ; tile load"
               : "=v"(x)
               : "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF));
}
// The same load through the caches (no nt): for loads that take only part of
// each cache line, the rest going to a neighbouring load instruction.
template <int OFF>
__device__ __forceinline__ void tile_load_cached(u32x4 &x, i32x4 rsrc, int voff, int soff) {
  static_assert(OFF >= 0 && OFF < 4096, "buffer immediate offsets are 12 bits");
  asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4 ; tile load"
               : "=v"(x)
               : "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF));
}
// A load of 64 16-byte chunks straight into LDS: lane L's chunk (at voff +
// soff of the buffer) lands at LDS byte m0 + 16 L.  The compiler does not
// see the LDS write, so the waits for it are placed by hand (lds_wait) and
// an LDS read of the data follows a barrier.  Non-temporal like the tile
// loads.
// (m0 is the compiler's: its value is kept in a scratch register around
// the load.)
__device__ __forceinline__ void lds_load(uint32_t m0, int voff, i32x4 rsrc, int soff) {
  int keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\t"
               "buffer_load_dwordx4 %2, %3, %4 offen nt lds ; lds slab load\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(keep)
               : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory");
}
template <int N>
__device__ __forceinline__ void lds_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0) ; lds slab wait" : : "n"(N) : "memory");
}
// Wait until at most N tile loads are outstanding (loads complete in order).
template <int N>
__device__ __forceinline__ void tile_wait(u32x4 &x) {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%1) ; tile wait %0" : "+v"(x) : "n"(N));
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
constexpr int kRowRor4 = 0x124;         // lane i <- (i - 4) mod 16 within the row
constexpr int kRowRor8 = 0x128;         // lane i <- (i - 8) mod 16 within the row

// One butterfly stage over the lanes of a key (partner selected by CTRL).
template <int CTRL>
__device__ __forceinline__ float dpp_stage(float x) { return dpp<CTRL>(x); }

// Reduce-scatter of per-head partial dot products over the LK lanes of a key.
// Stages pair lanes i/15-i (LK = 16), i/7-i (LK >= 8), then xor 2 and xor 1;
// while a lane holds more than one head the upper lane of each pair keeps the
// upper half of the heads.  Each lane ends with the full sums of HPL heads,
// starting at the returned head index; with REP < LK several lanes end with
// the same head.
template <int LK, int REP, int HPL>
__device__ __forceinline__ int key_reduce_scatter(const float (&a)[REP], int lane,
                                                  float (&o)[HPL]) {
  float v[REP];
#pragma unroll
  for (int h = 0; h < REP; ++h) v[h] = a[h];
  int hbase = 0;
  int H = REP;
  auto stage = [&](auto ctrl_tag, bool upper) {
    constexpr int CTRL = decltype(ctrl_tag)::value;
    if (H > 1) {
      const int half = H / 2;
#pragma unroll
      for (int i = 0; i < REP / 2; ++i) {
        if (i < half) {
          const float keep = upper ? v[half + i] : v[i];
          const float send = upper ? v[i] : v[half + i];
          v[i] = keep + dpp_stage<CTRL>(send);
        }
      }
      if (upper) hbase += half;
      H = half;
    } else {
      v[0] += dpp_stage<CTRL>(v[0]);
    }
  };
  if constexpr (LK >= 16) stage(std::integral_constant<int, kRowMirror>{}, (lane & 15) >= 8);
  if constexpr (LK >= 8) stage(std::integral_constant<int, kRowHalfMirror>{}, (lane & 7) >= 4);
  stage(std::integral_constant<int, kQuadXor2>{}, (lane & 2) != 0);
  stage(std::integral_constant<int, kQuadXor1>{}, (lane & 1) != 0);
#pragma unroll
  for (int u = 0; u < HPL; ++u) o[u] = v[u];
  return hbase;
}

// Lane (within a key's LK lanes) that owns head h after key_reduce_scatter,
// and the slot u of that head in the lane's owned list.
template <int LK, int REP>
__host__ __device__ constexpr int owner_lane(int h, int *u) {
  const int bits[4] = {LK >= 16 ? 8 : 0, LK >= 8 ? 4 : 0, 2, 1};
  int H = REP, rel = h, ln = 0;
  for (int s = 0; s < 4; ++s) {
    if (bits[s] == 0) continue;
    if (H > 1) {
      const int half = H / 2;
      if (rel >= half) {
        ln |= bits[s];
        rel -= half;
      }
      H = half;
    }
  }
  *u = rel;
  return ln;
}

// Max / sum over the KR key groups (lanes that own the same heads).
template <int LK>
__device__ __forceinline__ float keys_max(float x) {
  if constexpr (LK <= 4) x = fmaxf(x, dpp<kRowRor4>(x));
  if constexpr (LK <= 8) x = fmaxf(x, dpp<kRowRor8>(x));
  return swap32_max(swap16_max(x));
}
template <int LK>
__device__ __forceinline__ float keys_sum(float x) {
  if constexpr (LK <= 4) x += dpp<kRowRor4>(x);
  if constexpr (LK <= 8) x += dpp<kRowRor8>(x);
  return swap32_sum(swap16_sum(x));
}

// NBUF: register tiles in the ring (NBUF - 1 in flight); WAVES: occupancy the
// register allocator must meet.
// Stores of one token of a single-token step (C == 1) for (row b, KV head
// g), the same stores k_append makes: lane e < D/2 holds the pair (e, e +
// D/2) of the (rotated) key, y1 and y2, and of the value, v1 and v2.  A real
// token (valid) at position p goes to its slot (full layout: p, ring: p % W);
// a padded one to the scratch row with its value zeroed.  Also the slot
// report and, for a real token entering a new 32-row tile, the zeroing of V
// past the row's end in that tile (the decode tiles read those rows masked).
template <int D>
__device__ __forceinline__ void store_token_row(const LayerArgs &la, const FusedArgs &fa, int b,
                                                int g, int64_t p, bool valid, float y1, float y2,
                                                bf16 v1, bf16 v2, int lane, bool store_v = true) {
  static_assert(D / 2 <= 64, "one (d, d + D/2) pair per lane");
  const int64_t bg = (int64_t)b * la.hkv + g;
  const int64_t r = la.ring ? (valid ? p % la.window : (int64_t)la.window)
                            : (valid ? p : (int64_t)la.rows);
  constexpr int half = D / 2;
  if (lane < half) {
    bf16 *kd = krow_ptr<bf16>(la, b, g, r, D);
    kd[lane] = (bf16)y1;
    kd[lane + half] = (bf16)y2;
    if (store_v) {
      bf16 *vd = vcol_ptr<bf16>(la, b, g, r, D);
      vd[lane * kVBlock] = valid ? v1 : (bf16)0.f;
      vd[(lane + half) * kVBlock] = valid ? v2 : (bf16)0.f;
    }
  }
  if (fa.slot_out && g == 0 && lane == 0) fa.slot_out[b] = (int32_t)r;
  if (valid && !la.paged) {  // (pages have V zeroed when taken)
    const int64_t W = la.window;
    const int64_t old_top = la.ring ? (p < W ? p : W) : p;
    const int64_t new_top = la.ring ? (p + 1 < W ? p + 1 : W) : p + 1;
    if (old_top == 0 || (new_top - 1) / kRowAlign != (old_top - 1) / kRowAlign) {
      int64_t end = (new_top + kRowAlign - 1) / kRowAlign * kRowAlign;
      if (end > la.rows_alloc) end = la.rows_alloc;
      zero_v_rows<bf16>(la.v, bg, la.rows_alloc, new_top, end, D, lane);
    }
  }
}

// The padded token of an idle row (n_new == 0) of a single-token step: its
// key as given and a zero value go to the scratch row.
template <int D>
__device__ __forceinline__ void store_idle_token(const LayerArgs &la, const FusedArgs &fa, int b,
                                                 int g, int64_t p, int lane) {
  const int64_t bg = (int64_t)b * la.hkv + g;
  const bf16 *ks = static_cast<const bf16 *>(fa.k) + bg * D;
  float y1 = 0.f, y2 = 0.f;
  if (lane < D / 2) {
    y1 = (float)ks[lane];
    y2 = (float)ks[lane + D / 2];
  }
  store_token_row<D>(la, fa, b, g, p, false, y1, y2, (bf16)0.f, (bf16)0.f, lane);
}

// One term of a split merge: a + w * x, skipping splits of weight 0 (a split
// that saw no visible key never wrote its slot).  Shared by both merges so
// they round identically.
__device__ __forceinline__ float combine_acc(float a, float w, float x) {
  return w != 0.f ? fmaf(w, x, a) : a;
}
__device__ __forceinline__ float combine_tree(const float (&a)[8]) {
  return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// Merge of the ns decode splits of the REP heads h0.. of row b into the
// output o (REP x D) by one wave, with the same arithmetic in the same order
// as k_combine.  The partials are read with agent-scope loads (served from
// the device's point of coherence, past this XCD's L2).  Each lane owns D/64
// consecutive elements.  The first 8 splits of the first 4 heads are loaded
// together with every head's (m, l), so a merge of up to 8 splits of up to
// 4 heads costs one round trip to memory; later splits and heads load 8
// splits of 4 heads at a time.  wts: REP * 64 floats of LDS.
template <int D, int REP>
__device__ __forceinline__ void combine_group(const PartialArgs &pa, const StepArgs &st, int b,
                                              int h0, int ns, float *wts, bf16 *o, int lane) {
  auto ld = [](const float *ptr) {
    return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  constexpr int DPL = D / 64;                 // elements per lane
  constexpr int HG = REP < 4 ? REP : 4;       // heads per load round
  const int64_t cap = kDecodeSplitCap;
  const int d0 = lane * DPL;
  auto part = [&](int h, int sp) {
    return pa.dout + (((int64_t)b * st.Hq + h0 + h) * cap + sp) * D + d0;
  };
  float lv[REP], mv[REP];
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    const float *ml = pa.dml + ((int64_t)b * st.Hq + h0 + h) * cap * 2;
    lv[h] = lane < ns ? ld(ml + 2 * lane + 1) : 0.f;
    mv[h] = lane < ns ? ld(ml + 2 * lane) : -INFINITY;
  }
  float first[HG][8][DPL];
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < DPL; ++e) first[h][u][e] = u < ns ? ld(part(h, u) + e) : 0.f;
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    const float ms = (lane < ns && lv[h] > 0.f) ? mv[h] : -INFINITY;
    const float M = wave_max(ms);
    const float w = lv[h] > 0.f ? exp2f(ms - M) : 0.f;
    const float Lt = wave_sum(w * lv[h]);
    wts[h * 64 + lane] = w / Lt;
  }
  __syncthreads();
#pragma unroll
  for (int hg = 0; hg < REP; hg += HG) {
    float a[HG][DPL][8];
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int u = 0; u < 8; ++u) a[h][e][u] = 0.f;
    // x[h][u][e]: splits s0 .. s0 + 7 (those below ns) of heads hg ..
    float x[HG][8][DPL];
    auto fetch = [&](int s0) {
      if (hg == 0 && s0 == 0) {
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < DPL; ++e) x[h][u][e] = first[h][u][e];
      } else {
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < DPL; ++e)
              x[h][u][e] = s0 + u < ns ? ld(part(hg + h, s0 + u) + e) : 0.f;
      }
    };
    int s = 0;
    for (; s + 8 <= ns; s += 8) {
      fetch(s);
#pragma unroll
      for (int h = 0; h < HG; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = wts[(hg + h) * 64 + s + u];
#pragma unroll
          for (int e = 0; e < DPL; ++e) a[h][e][u] = combine_acc(a[h][e][u], w, x[h][u][e]);
        }
    }
    if (s < ns) {  // the last ns % 8 splits, summed in order into slot 0
      fetch(s);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s + u < ns) {
#pragma unroll
          for (int h = 0; h < HG; ++h) {
            const float w = wts[(hg + h) * 64 + s + u];
#pragma unroll
            for (int e = 0; e < DPL; ++e) a[h][e][0] = combine_acc(a[h][e][0], w, x[h][u][e]);
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[(hg + h) * D + d0 + e] = (bf16)combine_tree(a[h][e]);
  }
}

// FUSED: the single-token step of a layer (C == 1) appends in the same
// launch: the wave whose split holds the new key's row first appends it
// (RoPE, K row, V column, slot report); rows with n_new == 0 get one item
// that writes their padded token to the scratch row.  MERGE: the last split
// of a (row, KV head) to finish also combines the splits into the output
// (and idle rows' items write zero outputs); else the partials are left for
// k_combine, as the plain kernel leaves them.
// PAGED: a paged full layer; each 16-row tile is one page, found in the
// block table when the tile's loads are issued.
template <int D, int REP, bool FUSED = false, bool PAGED = false,
          int NBUF = FUSED ? DecodeShape<D, REP>::FNBUF : DecodeShape<D, REP>::NBUF,
          int WAVES = FUSED ? DecodeShape<D, REP>::FWAVES : DecodeShape<D, REP>::WAVES,
          bool MERGE = FUSED, int NW = 1>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WAVES)))
void k_decode(StepArgs st, LayerArgs la, PartialArgs pa, const bf16 *__restrict__ q,
              FusedArgs fa, const int32_t *__restrict__ ptab) {
  using S = DecodeShape<D, REP>;
  constexpr int LK = S::LK, KR = S::KR, TK = S::TK, NR = S::NR, NCH = S::NCH, VT = S::VT;
  constexpr int HPL = S::HPL;
  // NW > 1: one workgroup per (row, KV head) whose NW waves take the row's
  // splits and merge them through LDS (short rows: a windowed layer), no
  // partials in HBM and no merge launch.
  static_assert(NW == 1 || (!MERGE && !PAGED && NW <= 16), "workgroup merge form");
  __shared__ __align__(16) float qs_all[NW][REP * D];           // rotated q staging
  __shared__ __align__(16) uint16_t pls_all[NW][2][REP][TK];   // p of a tile, bf16

  const int lane = threadIdx.x & 63;
  const int wv = NW > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
  float *qs = qs_all[wv];
  auto &pls = pls_all[wv];
  const int g = pa.dec_transpose ? blockIdx.x : blockIdx.y;
  const int item = pa.dec_transpose ? blockIdx.y : blockIdx.x;
  int b;
  int64_t split64 = 0;
  int nn_b;
  int64_t p_b, first_b;
  if constexpr (NW > 1) {
    // One workgroup per row: a one-token step's counts are all 0 or 1, so
    // the row is the grid index.  Its count, length and first visible
    // position are loaded together.
    b = __builtin_amdgcn_readfirstlane(item);
    nn_b = st.n_new[b];
    p_b = st.lens[b];
    first_b = st.first[b];
  } else {
    const int SK = __builtin_amdgcn_readfirstlane(pa.dec_plan ? pa.dec_plan[0] : pa.dec_split_keys);
    auto row_at = [&](int r) {
      return pa.dec_order_dev ? (int)pa.dec_order_dev[r] : pa.dec_ordered ? (int)pa.dec_order[r] : r;
    };
    find_item(
        st.B, item,
        [&](int r0) -> int {
          const int r = row_at(r0);
          const int nr = st.n_new[r];
          if (nr != 1) return (FUSED && nr == 0) ? 1 : 0;
          const DecodeSpan sp = decode_span_dev(la, st.lens[r], st.first[r]);
          return (int)cdiv(sp.hi - sp.base, SK);
        },
        &b, &split64);
    if (b < 0) return;
    b = __builtin_amdgcn_readfirstlane(row_at(b));
    nn_b = FUSED ? st.n_new[b] : 1;
    p_b = st.lens[b];
    first_b = st.first[b];
  }
  const int h0 = g * REP;
  const int64_t bg = (int64_t)b * la.hkv + g;
  const int split = NW > 1 ? wv : (int)split64;
  // The row's 16-key tiles are dealt round-robin to its splits: split s
  // takes tiles s, s + nsplit, s + 2 nsplit, ... (counts differ by at most
  // one).  The splits of a row then sweep its K and V regions side by side,
  // so the waves in flight read from far fewer places in HBM than if each
  // split streamed its own contiguous run.  SK is a multiple of TK, so the
  // split count cdiv(hi - base, SK) is also cdiv(tiles, SK / TK) and every
  // split gets a tile.  The workgroup form takes nsplit = min(tiles, NW)
  // with one split per wave: wave w reads tiles w, w + NW, ... from slot 0
  // (a ring layer's span starts there; a row of fewer than NW tiles gives
  // wave w at most tile w).
  int t_begin, t_stride;
  if constexpr (NW > 1) {
    t_begin = split * TK;
    t_stride = NW * TK;
  }

  const int kr = lane / LK, j = lane % LK;          // QK: key in round, chunk group
  const int half = lane >> 5, mm = lane & 31;       // PV: key half, head-dim row

  // -- buffer resources over this head's K and V ------------------------------
  const int64_t region = (int64_t)la.rows_alloc * D * 2;  // bytes per (b, g)
  const i32x4 rk = sgpr_rsrc(la.k + bg * region, (int)region);
  const i32x4 rv = sgpr_rsrc(la.v + bg * region, (int)region);
  // Loads past a split's last tile (the ring keeps its loads in flight in
  // whole groups) go through descriptors of zero records: every lane is out
  // of range, so they return zeros without a memory access.
  const i32x4 rk_none = sgpr_rsrc(la.k + bg * region, 0);
  const i32x4 rv_none = sgpr_rsrc(la.v + bg * region, 0);
  const int koff = (kr * D + j * 8) * 2;
  const int voff = (mm * kVBlock + half * 8) * 2;

  struct Tile {
    u32x4 k[NR][NCH];
    u32x4 v[VT];
  };
  constexpr int LPT = NR * NCH + VT;  // loads per tile
  constexpr int page_b = kPageRows * D * 2;  // bytes of one head's page (K or V)
  int n_iter = 0;  // tiles of this split (loads past them: zero descriptors)
  auto load = [&](int it, Tile &T) {
    const bool live = it < n_iter;
    const int t0 = t_begin + (live ? it : 0) * t_stride;
    i32x4 ka, va;
    int so;
    if constexpr (PAGED) {
      // the tile's page (a scalar load: the table is read-only here); its K
      // rows and V block start the page's head slice
      const int pg = ptab[(int64_t)b * la.ppr + t0 / kPageRows];
      const int64_t off = ((int64_t)pg * la.hkv + g) * page_b;
      ka = live ? sgpr_rsrc(la.k + off, page_b) : rk_none;
      va = live ? sgpr_rsrc(la.v + off, page_b) : rv_none;
      so = 0;
    } else {
      ka = live ? rk : rk_none;
      va = live ? rv : rv_none;
      // K rows and V blocks advance by the same bytes per row
      so = __builtin_amdgcn_readfirstlane(t0 * D * 2);
    }
    static_for<0, NR>([&](auto r) {
      static_for<0, NCH>([&](auto t) {
        constexpr int off = decltype(r)::value * KR * D * 2 + decltype(t)::value * LK * 16;
        tile_load<off>(T.k[decltype(r)::value][decltype(t)::value], ka, koff, so);
      });
    });
    static_for<0, VT>([&](auto t) {
      tile_load<decltype(t)::value * 32 * kVBlock * 2>(T.v[decltype(t)::value], va, voff, so);
    });
  };
  // Wait for tile T when AFTER tiles were issued after it.
  auto wait_tile = [&](Tile &T, auto after) {
    constexpr int N = decltype(after)::value * LPT;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < NCH; ++t) tile_wait<N>(T.k[r][t]);
#pragma unroll
    for (int t = 0; t < VT; ++t) tile_wait<N>(T.v[t]);
  };

  // -- queries: REP heads of token 0 rotated at p; each lane keeps its share --
  // Lane l holds elements l + 64 i, all at head-dim index d = l + 64 i mod D,
  // so it needs one rotation entry (frequency l mod D/2); the partner of an
  // element (d + D/2 mod D) is its own element i ^ 1 at D 128 and lane
  // l ^ 32's element i at D 64.  bf16 values stay as loaded bits.
  constexpr int QE = REP * D / 64;                  // query elements per lane
  static_assert(D == 64 || D == 128, "query staging covers head_dim 64 and 128");
  const uint16_t *qraw = reinterpret_cast<const uint16_t *>(q + ((int64_t)b * st.C * st.Hq + h0) * D);
  uint16_t qx[QE];
  Tile T[NBUF];
  if constexpr (FUSED || NW > 1) {
    if (nn_b == 0) {  // idle row: its padded token (and zero outputs)
      if (FUSED && wv == 0) store_idle_token<D>(la, fa, b, g, p_b, lane);
      if constexpr (MERGE || NW > 1) {  // (else the merge kernel writes them)
        bf16 *o = static_cast<bf16 *>(fa.out) + ((int64_t)b * st.Hq + g * REP) * D;
        for (int e = wv * 64 + lane; e < REP * D; e += 64 * NW) o[e] = (bf16)0.f;
      }
      return;
    }
  }
  const int64_t p = p_b;
  const DecodeSpan span = decode_span_dev(la, p, first_b);
  const int64_t base64 = span.base, hi64 = span.hi;
  // Row indices fit in 32 bits (rows <= max_len < 2^31).
  const int hi = (int)hi64, va = (int)span.va, vn = (int)span.vn, vwrap = span.vwrap;
  const int ntile = (hi - (int)base64 + TK - 1) / TK;
  int nsplit;
  if constexpr (NW > 1) {
    // (waves past the row's splits compute nothing and hold empty partials)
    nsplit = ntile < NW ? ntile : NW;
    n_iter = __builtin_amdgcn_readfirstlane((ntile - split + NW - 1) / NW);
  } else {
    const int SK = __builtin_amdgcn_readfirstlane(pa.dec_plan ? pa.dec_plan[0] : pa.dec_split_keys);
    nsplit = (hi - (int)base64 + SK - 1) / SK;
    // (uniform values; readfirstlane keeps them in scalar registers, where
    // the tile loads take their offsets)
    t_begin = __builtin_amdgcn_readfirstlane((int)base64 + split * TK);
    t_stride = __builtin_amdgcn_readfirstlane(nsplit * TK);
    n_iter = __builtin_amdgcn_readfirstlane((ntile - split + nsplit - 1) / nsplit);
  }
  // Fused: the new key's storage row (full layout: p; ring: p % W) lies in
  // exactly one split.  That wave loads the token's key, value and rotation
  // here, ahead of the queries' loads, and stores the rotated row before its
  // tile loads.
  bool appender = false;
  float ax1 = 0.f, ax2 = 0.f, arc = 1.f, ars = 0.f;
  bf16 av1 = (bf16)0.f, av2 = (bf16)0.f;
  if constexpr (FUSED) {
    const int r_new = la.ring ? (int)(p % la.window) : (int)p;
    appender = (r_new - (int)base64) / TK % nsplit == split;
    if (appender && lane < D / 2) {
      const bf16 *ks = static_cast<const bf16 *>(fa.k) + bg * D;
      const bf16 *vs = static_cast<const bf16 *>(fa.v) + bg * D;
      ax1 = (float)ks[lane];
      ax2 = (float)ks[lane + D / 2];
      av1 = vs[lane];
      av2 = vs[lane + D / 2];
      if (st.rope) {
        arc = st.rope[(p * (D / 2) + lane) * 2 + 0];
        ars = st.rope[(p * (D / 2) + lane) * 2 + 1];
      }
    }
  }

  // The loads of the queries and their rotation go out first, then the
  // first tiles, before any of them is waited for, so the queries' round
  // trip and the first tiles' overlap.  In the appending kernel the wave
  // whose split holds the new row stores it before its tile loads.  No
  // branch around the rotation's load: without a table it reads the query
  // row (16-byte aligned) and is not used.
  const bool rot = st.rope != nullptr;
#pragma unroll
  for (int i = 0; i < QE; ++i) qx[i] = qraw[lane + 64 * i];
  const float2 qcs = *reinterpret_cast<const float2 *>(
      rot ? st.rope + (p * (D / 2) + lane % (D / 2)) * 2 : reinterpret_cast<const float *>(qraw));
  const float qc = qcs.x, qsn = qcs.y;
  // Where the register tiles leave room for it (all shapes but the one
  // wave of four-deep tiles, whose checked wait placement the extra branch
  // would break), the new row's V reaches memory only after every tile load
  // of the launch (below): it is one 2-byte store into each head-dim row's
  // 32-byte run of its block, and ahead of the wave's tile loads it cost the
  // decode_b64 step about 3 %.  The appending wave's own tile, loaded before
  // that store, then takes the new values in registers: lane (half, mm)
  // holds keys 8 half .. 8 half + 7 of head-dim row mm + 32 t in V register
  // t, so the lanes of the new key's half get the element of their rows
  // (from lane d of av1 below D/2, lane d - D/2 of av2 above).
  constexpr bool kLateV = FUSED && !S::DEEP;
  if constexpr (FUSED) {
    if (appender) {
      float y1 = ax1, y2 = ax2;
      if (st.rope) rope_pair(ax1, ax2, arc, ars, &y1, &y2);
      store_token_row<D>(la, fa, b, g, p, true, y1, y2, av1, av2, lane, !kLateV);
    }
  }
  // (the new key's row in its tile and the tile's first row, uniform; the
  // lane's two values packed in one register until the store)
  int vkk = 0, vnew_t0 = -1;
  const uint32_t avpk = (uint32_t)__builtin_bit_cast(uint16_t, av1) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, av2) << 16);
  if constexpr (kLateV) {
    if (appender) {
      const int r_new = la.ring ? (int)(p % la.window) : (int)p;
      vkk = __builtin_amdgcn_readfirstlane((r_new - (int)base64) % TK);
      vnew_t0 = __builtin_amdgcn_readfirstlane(r_new - vkk);
    }
  }
  auto patch_v = [&](Tile &T) {
    const bool own = half == vkk / 8;
    const int word = (vkk % 8) / 2;
    const bool hi = (vkk & 1) != 0;
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      const bool upper = 32 * t >= D / 2;  // (the same for every lane of t)
      const int src = mm + 32 * t - (upper ? D / 2 : 0);
      const uint32_t nv = (uint32_t)__shfl((int)avpk, src);
      const uint32_t bits = upper ? nv >> 16 : nv & 0xffffu;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t old = T.v[t][w];
        const uint32_t upd = hi ? ((old & 0xffffu) | (bits << 16)) : ((old & 0xffff0000u) | bits);
        T.v[t][w] = own && w == word ? upd : old;
      }
    }
  };
  // The barrier keeps the compiler from moving the loads and stores above
  // past the tile loads: every vector memory access of the wave is then
  // older than the tiles, as the hand-placed tile waits require, and the
  // appending wave's tiles come after its store (the memory pipeline keeps
  // one wave's accesses to one address in order).
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) load(i, T[i]);
  // Nothing below moves above the tile loads: the compiler computes nothing
  // from the query values, and so waits for none of them, before they are out.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < QE; ++i) {
    const int e = lane + 64 * i, d = e % D;
    const uint32_t xb = qx[i];
    const uint32_t ob = D == 128 ? (uint32_t)qx[i ^ 1] : (uint32_t)__shfl_xor((int)xb, 32);
    const float x = __builtin_bit_cast(float, xb << 16);
    const float o = __builtin_bit_cast(float, ob << 16);
    const float xr = d < D / 2 ? x * qc - o * qsn : o * qsn + x * qc;
    qs[e] = rot ? xr : x;
  }
  // One wave: its LDS accesses execute in order, so the reads below see the
  // writes above without a barrier (which would also wait for the tiles).
  __builtin_amdgcn_wave_barrier();
  uint32_t qp[REP][NCH][4];
#pragma unroll
  for (int h = 0; h < REP; ++h)
#pragma unroll
    for (int t = 0; t < NCH; ++t)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int d = (j + LK * t) * 8 + 2 * e2;
        qp[h][t][e2] = pack_bf16(qs[h * D + d], qs[h * D + d + 1]);
      }

  const float scale = kLog2e * rsqrtf((float)D);
  float m[HPL], lsum[HPL], acc[REP][VT];
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    m[u] = -INFINITY;
    lsum[u] = 0.f;
  }
#pragma unroll
  for (int h = 0; h < REP; ++h)
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[h][t] = 0.f;
  int hbase = 0;     // first head this lane owns (set by the reduce-scatter)
  bool writer = true;  // one lane per (key, head) publishes p

  // One tile: QK, online softmax, P.V.  Rows of the tile that are not
  // visible (outside the span, left padding) are masked in the scores; their
  // V is finite (rows past a row's end are zeroed when the append enters a
  // new 32-row tile), so p = 0 cancels them.
  auto step = [&](int it, Tile &T) {
    const int t0 = t_begin + it * t_stride;
    const int par = it & 1;
    float a[NR][REP];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        float x = 0.f;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
          x = dot2_bf16(qp[h][t][0], T.k[r][t].x, x);
          x = dot2_bf16(qp[h][t][1], T.k[r][t].y, x);
          x = dot2_bf16(qp[h][t][2], T.k[r][t].z, x);
          x = dot2_bf16(qp[h][t][3], T.k[r][t].w, x);
        }
        a[r][h] = x;
      }
    float s[NR][HPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      key_reduce_scatter<LK, REP, HPL>(a[r], lane, s[r]);
      const int key = t0 + r * KR + kr;
      const int d = key - va + (key < va ? vwrap : 0);
      const bool ok = key < hi && (unsigned)d < (unsigned)vn;
#pragma unroll
      for (int u = 0; u < HPL; ++u) s[r][u] = ok ? s[r][u] : -INFINITY;
    }
    float alpha[HPL];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      float tm = s[0][u];
#pragma unroll
      for (int r = 1; r < NR; ++r) tm = fmaxf(tm, s[r][u]);
      tm = keys_max<LK>(tm);
      // A tile can be entirely masked (a windowed span starting past the
      // tile's first 16 rows); then mn stays -inf and the subtraction uses 0.
      const float mn = fmaxf(m[u], tm * scale);
      const float ms = mn == -INFINITY ? 0.f : mn;
      alpha[u] = __builtin_amdgcn_exp2f(m[u] - ms);
      m[u] = mn;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(s[r][u], scale, -ms));
        ps += pe;
        if (writer) {
          const bf16 pb = (bf16)pe;
          pls[par][hbase + u][r * KR + kr] = __builtin_bit_cast(uint16_t, pb);
        }
      }
      lsum[u] = lsum[u] * alpha[u] + ps;
    }
    // The workgroup is one wave and its LDS operations execute in order, so
    // the p reads below see the writes above.  (__syncthreads would also wait
    // for every outstanding global load, draining the tiles in flight.)
    __builtin_amdgcn_wave_barrier();
    bool moved = false;
#pragma unroll
    for (int u = 0; u < HPL; ++u) moved |= alpha[u] != 1.f;
    if (__ballot(moved) != 0) {
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        int u = 0;
        const int src = owner_lane<LK, REP>(h, &u);  // a lane owning head h
        const float al = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha[u]), src));
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[h][t] *= al;
      }
    }
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      const uint4 pp = *reinterpret_cast<const uint4 *>(&pls[par][h][half * 8]);
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        float x = acc[h][t];
        x = dot2_bf16(T.v[t].x, pp.x, x);
        x = dot2_bf16(T.v[t].y, pp.y, x);
        x = dot2_bf16(T.v[t].z, pp.z, x);
        x = dot2_bf16(T.v[t].w, pp.w, x);
        acc[h][t] = x;
      }
    }
  };

  // Which lanes publish p: with REP < LK the last log2(LK/REP) stages
  // all-reduce (the low lane bits), and only the lane with those bits clear
  // writes; hbase is fixed per lane, computed once here.
  {
    float zin[REP], zout[HPL];
#pragma unroll
    for (int h = 0; h < REP; ++h) zin[h] = 0.f;
    hbase = key_reduce_scatter<LK, REP, HPL>(zin, lane, zout);
    if (REP < LK) writer = (j & (LK / REP - 1)) == 0;
  }

  // Ring of NBUF register tiles (the first NBUF - 1 issued above); NBUF - 1
  // tiles are in flight while one computes.  Unrolled by NBUF so buffer indices are compile-time.  Loads
  // and waits run for whole groups (loads past the end read nothing and
  // return zeros) and only the compute is skipped past the end, so the
  // loop has one back edge and always the same loads in flight.
  for (int it = 0; it < n_iter; it += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      load(it + u + NBUF - 1, T[(u + NBUF - 1) % NBUF]);
      wait_tile(T[u], std::integral_constant<int, NBUF - 1>{});
      if constexpr (kLateV) {
        if (t_begin + (it + u) * t_stride == vnew_t0) patch_v(T[u]);
      }
      if (it + u < n_iter) step(it + u, T[u]);
    }
  }
  // Retire the loads still in flight before their registers are reused.
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int t = 0; t < NCH; ++t) tile_wait<0>(T[i].k[r][t]);
#pragma unroll
    for (int t = 0; t < VT; ++t) tile_wait<0>(T[i].v[t]);
  }
  if constexpr (kLateV) {
    // the new row's V, after the tile loads (see above)
    if (appender && lane < D / 2) {
      const int64_t r = la.ring ? p % la.window : p;
      uint16_t *vd = reinterpret_cast<uint16_t *>(vcol_ptr<bf16>(la, b, g, r, D));
      vd[lane * kVBlock] = (uint16_t)(avpk & 0xffffu);
      vd[(lane + D / 2) * kVBlock] = (uint16_t)(avpk >> 16);
    }
  }

  // ---- partials of this split ----
  const int64_t cap = kDecodeSplitCap;
  float lh[HPL];
#pragma unroll
  for (int u = 0; u < HPL; ++u) lh[u] = keys_sum<LK>(lsum[u]);
  if constexpr (NW > 1) {
    // The workgroup form: each wave's partial to LDS, then wave w merges
    // heads w, w + NW, ... with the weights and the order of k_combine.
    __shared__ float wml[NW][REP][2];
    __shared__ __align__(16) float wout[NW][REP][D];
#pragma unroll
    for (int u = 0; u < HPL; ++u) {
      if (kr == 0 && writer) {
        wml[wv][hbase + u][0] = m[u];
        wml[wv][hbase + u][1] = lh[u];
      }
    }
#pragma unroll
    for (int h = 0; h < REP; ++h)
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        const float o = swap32_sum(acc[h][t]);
        if (half == 0) wout[wv][h][mm + 32 * t] = o;
      }
    __syncthreads();
    bf16 *ob = static_cast<bf16 *>(fa.out) + ((int64_t)b * st.Hq + h0) * D;
    for (int h = wv; h < REP; h += NW) {
      // split weights 2^(m_s - M) / L (a split with no visible key: l == 0)
      const float ls = lane < nsplit ? wml[lane][h][1] : 0.f;
      const float ms = (lane < nsplit && ls > 0.f) ? wml[lane][h][0] : -INFINITY;
      const float M = wave_max(ms);
      const float w = ls > 0.f ? exp2f(ms - M) : 0.f;
      const float Lt = wave_sum(w * ls);
      const int wt = __builtin_bit_cast(int, w / Lt);
      auto wt_of = [&](int sp) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(wt, sp)); };
      for (int d = lane; d < D; d += 64) {
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int sp = 0;
        for (; sp + 8 <= nsplit; sp += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) a[u] = combine_acc(a[u], wt_of(sp + u), wout[sp + u][h][d]);
        }
        for (; sp < nsplit; ++sp) a[0] = combine_acc(a[0], wt_of(sp), wout[sp][h][d]);
        ob[h * D + d] = (bf16)combine_tree(a);
      }
    }
    return;
  }
  if constexpr (MERGE) {
    if (nsplit == 1) {
      // One split: the output is o / l, rounded as the merge rounds a
      // single split (weight 1 / l times o, then the sum with zeros).
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        int u = 0;
        const int src = owner_lane<LK, REP>(h, &u);
        const float l = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lh[u]), src));
        const float w = 1.f / l;
        bf16 *o = static_cast<bf16 *>(fa.out) + ((int64_t)b * st.Hq + h0 + h) * D;
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          const float x = swap32_sum(acc[h][t]);
          if (half == 0) o[mm + 32 * t] = (bf16)(combine_acc(0.f, w, x) + 0.f);
        }
      }
      return;
    }
  }
  // Partials (m, l, o) of this split.  The fused kernel writes them with
  // agent-scope stores (written through to the device's point of coherence,
  // which every XCD reads).
  auto put = [&](float *ptr, float val) {
    if constexpr (MERGE)
      __hip_atomic_store(ptr, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *ptr = val;
  };
  // (over a joint partner's keys, after the layer's own splits)
  const int sbase = pa.base.on ? ref_splits(pa.base, p, 1, st.first[b]) : 0;
#pragma unroll
  for (int u = 0; u < HPL; ++u) {
    if (kr == 0 && writer) {
      const int64_t slot = ((int64_t)b * st.Hq + h0 + hbase + u) * cap + sbase + split;
      put(pa.dml + slot * 2 + 0, m[u]);
      put(pa.dml + slot * 2 + 1, lh[u]);
    }
  }
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    const int64_t slot = ((int64_t)b * st.Hq + h0 + h) * cap + sbase + split;
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      const float o = swap32_sum(acc[h][t]);
      if (half == 0) put(pa.dout + slot * D + mm + 32 * t, o);
    }
  }
  if constexpr (MERGE) {
    // Count this split's arrival once its partials are complete: the wait
    // retires every store of the wave (acknowledged at the point of
    // coherence) before lane 0's agent-scope increment.  The split that reads
    // nsplit - 1 arrives last; it issues its agent-scope loads of the other
    // splits' partials only after that read returned, so it sees them all.
    // This is the order an agent-scope release / acquire pair would give,
    // without the write-back and invalidation of the whole L2 that such
    // fences cost on this chip (they would run once per wave).  The counter
    // goes back to zero for the next launch.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(fa.cnt + bg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != nsplit - 1) return;
    combine_group<D, REP>(pa, st, b, h0, nsplit, qs,
                          static_cast<bf16 *>(fa.out) + ((int64_t)b * st.Hq + h0) * D, lane);
    if (lane == 0) __hip_atomic_store(fa.cnt + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

bool fast_decode_supported(int D, int rep) {
  return (D == 64 || D == 128) && (rep == 1 || rep == 2 || rep == 4 || rep == 8 || rep == 16);
}

template <int D, int REP>
static void launch_decode_t(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                            const void *q, int32_t n_items, const Launch &lc) {
  const dim3 grid = pa.dec_transpose ? dim3((unsigned)la.hkv, (unsigned)n_items)
                                     : dim3((unsigned)n_items, (unsigned)la.hkv);
  if (la.paged)
    launch_kernel((k_decode<D, REP, false, true>), grid, dim3(64), lc, st, la, pa, (const bf16 *)q,
                  FusedArgs{}, la.table);
  else
    launch_kernel((k_decode<D, REP>), grid, dim3(64), lc, st, la, pa, (const bf16 *)q, FusedArgs{},
                  la.table);
}

template <int D, int REP>
static void launch_decode_fused_t(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                                  const void *q, const FusedArgs &fa, int32_t n_items,
                                  bool merge, const Launch &lc) {
  using S = DecodeShape<D, REP>;
  const dim3 grid = pa.dec_transpose ? dim3((unsigned)la.hkv, (unsigned)n_items)
                                     : dim3((unsigned)n_items, (unsigned)la.hkv);
  // without the merge: the plain kernel's register ring and occupancy
  if (merge) {
    if (la.paged)
      launch_kernel((k_decode<D, REP, true, true>), grid, dim3(64), lc, st, la, pa,
                    (const bf16 *)q, fa, la.table);
    else
      launch_kernel((k_decode<D, REP, true>), grid, dim3(64), lc, st, la, pa, (const bf16 *)q, fa,
                    la.table);
  } else {
    if (la.paged)
      launch_kernel((k_decode<D, REP, true, true, S::NBUF, S::WAVES, false>), grid, dim3(64), lc,
                    st, la, pa, (const bf16 *)q, fa, la.table);
    else
      launch_kernel((k_decode<D, REP, true, false, S::NBUF, S::WAVES, false>), grid, dim3(64), lc,
                    st, la, pa, (const bf16 *)q, fa, la.table);
  }
}

// The workgroup form (NW waves per (row, KV head), merged through LDS):
// three register tiles, two waves per SIMD so that a workgroup's eight waves
// share one CU.
constexpr int kDecodeWgWaves = 8;

// The workgroup form on the matrix cores (REP 8 and 16): one workgroup of
// NW waves per (row, KV head), as above, but the rep query heads form one
// 16-column block of v_mfma_f32_16x16x32_bf16 (REP 8 leaves 8 columns
// empty).  Per 32-key tile a wave computes S^T = K Q^T (2 x D/32 products)
// and O^T += V^T P^T (D/16 products), its K and V operands loaded from HBM
// straight into registers in operand order: lane (q4, nl) takes 16 bytes of
// key 8 (nl / 4) + 4 kb + nl % 4 (so its scores are keys 8 q4 .. 8 q4 + 7,
// the P^T operand it then holds) and the 8 keys 8 q4 .. 8 q4 + 7 of head-dim
// row 16 db + nl of the tile's V blocks.  The vector form spends about
// REP x D / 64 dot2 instructions per key and lane, which at REP 8 and only
// one workgroup per (row, KV head) is the larger part of its time.  Wave w
// takes tiles w, w + NW, ... from slot 0 (at most one per tile below NW
// tiles); the waves' partials merge through LDS with k_combine's weights
// and order.  Rows of a tile outside the span are masked in the scores;
// their V is finite (the append zeroes V to the end of the 32-row tile it
// enters).
template <int D, int REP, bool FUSED>
__global__ __launch_bounds__(64 * kDecodeWgWaves) __attribute__((amdgpu_waves_per_eu(2)))
void k_decode_wgm(StepArgs st, LayerArgs la, PartialArgs pa, const bf16 *__restrict__ q,
                  FusedArgs fa) {
  constexpr int NW = kDecodeWgWaves;
  constexpr int NDS = D / 32;  // 32-wide d steps (QK contraction)
  constexpr int NDB = D / 16;  // 16-wide d blocks (PV output)
  constexpr int HS = NDS / 2;  // the partner d + D/2 sits HS steps later
  constexpr int TT = 32;       // keys per tile
  static_assert(REP == 8 || REP == 16, "one 16-column query block");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  __shared__ __align__(16) float wout[NW][REP][D];
  __shared__ float wml[NW][REP][2];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int q4 = lane >> 4, nl = lane & 15;
  const int g = pa.dec_transpose ? blockIdx.x : blockIdx.y;
  // One workgroup per row (a one-token step's counts are all 0 or 1).  No
  // branch until the tiles are out: each branch around a load makes the
  // compiler wait for it at the join, and the prologue would become a chain
  // of round trips.  An idle row (n_new == 0) runs with no splits: no tile
  // is computed and the merge writes zero outputs.
  const int b = __builtin_amdgcn_readfirstlane(pa.dec_transpose ? (int)blockIdx.y : (int)blockIdx.x);
  const int nn_b = st.n_new[b];
  const int p32 = st.lens[b];
  const int first32 = st.first[b];
  // (the row's three counters and the layer's arguments in one batch of
  // scalar loads, waited for once, rather than one round trip after another)
  asm volatile("" ::"s"(nn_b), "s"(p32), "s"(first32), "s"(la.window), "s"(la.rows_alloc),
               "s"(la.hkv), "s"(la.ring), "s"(la.k), "s"(la.v), "s"(st.rope), "s"(st.Hq));
  const int64_t p = p32;
  const bool idle = nn_b == 0;
  const int h0 = g * REP;
  bf16 *ob = static_cast<bf16 *>(fa.out) + ((int64_t)b * st.Hq + h0) * D;
  // A ring layer (the span of decode_span_dev, in 32 bits: positions stay
  // below 2^31): the visible positions [start, p] sit in slots [0, hi) from
  // slot 0, the oldest at slot va; vwrap = W.
  const int W = la.window;
  int start = p32 - W + 1 > 0 ? p32 - W + 1 : 0;
  start = p32 < first32 ? p32 : (start > first32 ? start : first32);
  const int vn = p32 + 1 - start, hi = p32 + 1 < W ? p32 + 1 : W;
  const int va = start % W, vwrap = W;
  const int ntile = idle ? 0 : (hi + TT - 1) / TT;
  const int nsplit = ntile < NW ? ntile : NW;
  const int n_iter = __builtin_amdgcn_readfirstlane((ntile - wv + NW - 1) / NW);
  const int64_t bg = (int64_t)b * la.hkv + g;
  // (an idle row's length may be max_len: no rotation entry is read for it)
  const bool rot = st.rope != nullptr && !idle;

  const bool qrow = nl < REP;
  const float *rbase = st.rope != nullptr ? st.rope : reinterpret_cast<const float *>(q);
  const int64_t rrow = rot ? p : 0;

  // Appending form: the wave whose tiles hold the new row's slot p mod W
  // stores the rotated row before its tile loads (one wave's accesses to one
  // address keep their order); an idle row's wave 0 stores its padded token.
  bool appender = false;
  if constexpr (FUSED) {
    const int r_new = p32 % W;
    appender = !idle && (r_new / TT) % NW == wv;
    const int e = lane & (D / 2 - 1);
    const bf16 *ks = static_cast<const bf16 *>(fa.k) + bg * D;
    const bf16 *vs = static_cast<const bf16 *>(fa.v) + bg * D;
    const float ax1 = (float)ks[e], ax2 = (float)ks[e + D / 2];
    const bf16 av1 = vs[e], av2 = vs[e + D / 2];
    const float2 acs = *reinterpret_cast<const float2 *>(rbase + (rrow * (D / 2) + e) * 2);
    if (appender) {
      float y1 = ax1, y2 = ax2;
      if (rot) rope_pair(ax1, ax2, acs.x, acs.y, &y1, &y2);
      store_token_row<D>(la, fa, b, g, p, true, y1, y2, av1, av2, lane);
    } else if (idle && wv == 0) {
      store_token_row<D>(la, fa, b, g, p, false, ax1, ax2, (bf16)0.f, (bf16)0.f, lane);
    }
  }

  // -- the query block: lane (q4, nl) holds head nl's d = 32 ds + 8 q4 .. + 7
  // (rotated at p), the Q^T operand of each d step; heads past REP are zero.
  // Every lane loads (heads past REP read head 0; without a table the
  // rotation's loads read the start of q, at least REP * D elements, and go
  // unused) and selects afterwards.  These loads go out through the same
  // hand-waited path as the tiles, ahead of them, so that the compiler
  // neither sinks them below the tiles nor waits for the tiles with them.
  // (the appending wave's loads and stores above stay above these loads)
  asm volatile("" ::: "memory");
  const i32x4 rq = sgpr_rsrc(q + ((int64_t)b * st.C * st.Hq + h0) * D, REP * D * 2);
  const i32x4 rr = sgpr_rsrc(rbase + rrow * D, D * 4);  // one position's D/2 (cos, sin)
  u32x4 qv[NDS];
  u32x4 rp[HS][4];  // (cos, sin) of the 8 consecutive frequencies of a step
  {
    const int qoff = (qrow ? nl : 0) * D * 2 + q4 * 16;
    static_for<0, NDS>([&](auto ds) {
      tile_load<decltype(ds)::value * 64>(qv[decltype(ds)::value], rq, qoff, 0);
    });
    static_for<0, HS>([&](auto ds) {
      static_for<0, 4>([&](auto u) {
        tile_load<decltype(ds)::value * 256 + decltype(u)::value * 16>(
            rp[decltype(ds)::value][decltype(u)::value], rr, q4 * 64, 0);
      });
    });
  }
  constexpr int QLD = NDS + 4 * HS;  // the query block's loads

  // -- tiles: K and V operands straight from HBM ------------------------------
  // An operand load takes 64 of each K row's 256 bytes (16 rows per load);
  // through the caches the row's other pieces, loaded next, hit the line
  // the first one brought in (W = 512 rings: 12.5 -> 10.3 us per layer
  // against non-temporal loads).
  const int64_t region = (int64_t)la.rows_alloc * D * 2;  // bytes per (b, g)
  const i32x4 rk = sgpr_rsrc(la.k + bg * region, (int)region);
  const i32x4 rv = sgpr_rsrc(la.v + bg * region, (int)region);
  const i32x4 rnone = sgpr_rsrc(la.k + bg * region, 0);  // zero records: no access
  const int koff = ((8 * (nl >> 2) + (nl & 3)) * D + q4 * 8) * 2;
  const int voff = ((q4 >> 1) * 16 * D + nl * 16 + (q4 & 1) * 8) * 2;
  struct Tile {
    u32x4 k[2][NDS];
    u32x4 v[NDB];
  };
  constexpr int LPT = 2 * NDS + NDB;  // loads per tile
  auto load = [&](int it, Tile &T) {
    const bool live = it < n_iter;
    const int t0 = (wv + (live ? it : 0) * NW) * TT;
    const i32x4 ka = live ? rk : rnone, va_ = live ? rv : rnone;
    // K rows and V blocks advance by the same bytes per row
    const int so = __builtin_amdgcn_readfirstlane(t0 * D * 2);
    static_for<0, 2>([&](auto kb) {
      static_for<0, NDS>([&](auto ds) {
        constexpr int off = decltype(kb)::value * 4 * D * 2 + decltype(ds)::value * 64;
        tile_load_cached<off>(T.k[decltype(kb)::value][decltype(ds)::value], ka, koff, so);
      });
    });
    static_for<0, NDB>([&](auto db) {
      tile_load_cached<decltype(db)::value * 16 * 32>(T.v[decltype(db)::value], va_, voff, so);
    });
  };
  auto wait_tile = [&](Tile &T, auto after) {
    constexpr int N = decltype(after)::value * LPT;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) tile_wait<N>(T.k[kb][ds]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) tile_wait<N>(T.v[db]);
  };
  // (the loads and stores above are older than every tile load, as the
  // hand-placed waits require)
  asm volatile("" ::: "memory");
  Tile T[2];
  load(0, T[0]);
  load(1, T[1]);
  __builtin_amdgcn_sched_barrier(0);

  // the query block's loads are older than both tiles': wait for them only
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) tile_wait<2 * LPT>(qv[ds]);
#pragma unroll
  for (int ds = 0; ds < HS; ++ds)
#pragma unroll
    for (int u = 0; u < 4; ++u) tile_wait<2 * LPT>(rp[ds][u]);
  static_assert(2 * LPT < 64, "vmcnt is 6 bits");
  (void)QLD;
  bf16x8_t qf[NDS];
  {
    float raw[NDS][8];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const uint32_t w[4] = {qv[ds].x, qv[ds].y, qv[ds].z, qv[ds].w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        raw[ds][2 * e2] = bf_lo(w[e2]);
        raw[ds][2 * e2 + 1] = bf_hi(w[e2]);
      }
    }
#pragma unroll
    for (int ds = 0; ds < HS; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const u32x4 cs = rp[ds][e / 2];
        const float c = __uint_as_float((e & 1) ? cs.z : cs.x);
        const float sn = __uint_as_float((e & 1) ? cs.w : cs.y);
        const float x1 = raw[ds][e], x2 = raw[ds + HS][e];
        const float y1 = x1 * c - x2 * sn, y2 = x1 * sn + x2 * c;
        raw[ds][e] = rot ? y1 : x1;
        raw[ds + HS][e] = rot ? y2 : x2;
      }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ds][e] = (bf16)(qrow ? raw[ds][e] : 0.f);
  }

  const float scale = kLog2e * rsqrtf((float)D);
  float mrun = -INFINITY, lrun = 0.f;  // this lane's column (head nl), scaled log2 domain
  floatx4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int it, Tile &T) __attribute__((always_inline)) {
    const int t0 = (wv + it * NW) * TT;
    floatx4 sacc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, T.k[kb][ds]), qf[ds], sacc[kb], 0, 0, 0);
    // sacc[kb][jj]: key t0 + 8 q4 + 4 kb + jj, head nl
    float sv[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int key = t0 + 8 * q4 + 4 * kb + jj;
        const int d = key - va + (key < va ? vwrap : 0);
        const bool ok = key < hi && (unsigned)d < (unsigned)vn;
        const float x = ok ? sacc[kb][jj] : -INFINITY;
        sv[kb][jj] = x;
        tmax = fmaxf(tmax, x);
      }
    // the column's max over the tile: its 4 lane groups hold 8 keys each
    const float mn = fmaxf(mrun, swap32_max(swap16_max(tmax)) * scale);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(mrun - ms);
    mrun = mn;
    float ps = 0.f;
    bf16x8_t pf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sv[kb][jj], scale, -ms));
        ps += pe;
        pf[kb * 4 + jj] = (bf16)pe;
      }
    lrun = lrun * alpha + ps;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      oacc[db] *= alpha;
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, T.v[db]),
                                                        pf, oacc[db], 0, 0, 0);
    }
  };
  // Two register tiles: one tile's loads are out while the other computes.
  for (int it = 0; it < n_iter; it += 2) {
    wait_tile(T[0], std::integral_constant<int, 1>{});
    step(it, T[0]);
    load(it + 2, T[0]);
    wait_tile(T[1], std::integral_constant<int, 1>{});
    if (it + 1 < n_iter) step(it + 1, T[1]);
    load(it + 3, T[1]);
  }
  // retire the loads still in flight before their registers are reused
#pragma unroll
  for (int i = 0; i < 2; ++i) wait_tile(T[i], std::integral_constant<int, 0>{});

  // -- this wave's partial to LDS, then wave w merges heads w, w + NW, ... ------
  if (wv < nsplit) {
    const float lt = swap32_sum(swap16_sum(lrun));
    if (qrow) {
      if (q4 == 0) {
        wml[wv][nl][0] = lt > 0.f ? mrun : -INFINITY;
        wml[wv][nl][1] = lt;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) wout[wv][nl][db * 16 + 4 * q4 + jj] = oacc[db][jj];
    }
  }
  __syncthreads();
  for (int h = wv; h < REP; h += NW) {
    // split weights 2^(m_s - M) / L (a split with no visible key: l == 0)
    const float ls = lane < nsplit ? wml[lane][h][1] : 0.f;
    const float msv = (lane < nsplit && ls > 0.f) ? wml[lane][h][0] : -INFINITY;
    const float M = wave_max(msv);
    const float w = ls > 0.f ? exp2f(msv - M) : 0.f;
    const float Lt = wave_sum(w * ls);
    const int wt = __builtin_bit_cast(int, w / Lt);
    auto wt_of = [&](int sp) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(wt, sp));
    };
    for (int d = lane; d < D; d += 64) {
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int sp = 0;
      for (; sp + 8 <= nsplit; sp += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = combine_acc(a[u], wt_of(sp + u), wout[sp + u][h][d]);
      }
      for (; sp < nsplit; ++sp) a[0] = combine_acc(a[0], wt_of(sp), wout[sp][h][d]);
      ob[h * D + d] = (bf16)combine_tree(a);
    }
  }
}

template <int D, int REP>
static void launch_decode_wg_t(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                               const void *q, const FusedArgs &fa, bool fused,
                               const Launch &lc) {
  const dim3 grid = pa.dec_transpose ? dim3((unsigned)la.hkv, (unsigned)st.B)
                                     : dim3((unsigned)st.B, (unsigned)la.hkv);
  const dim3 block(64 * kDecodeWgWaves);
  if constexpr (REP == 8 || REP == 16) {
    if (fused)
      launch_kernel((k_decode_wgm<D, REP, true>), grid, block, lc, st, la, pa, (const bf16 *)q, fa);
    else
      launch_kernel((k_decode_wgm<D, REP, false>), grid, block, lc, st, la, pa, (const bf16 *)q, fa);
  } else {
    if (fused)
      launch_kernel((k_decode<D, REP, true, false, 3, 2, false, kDecodeWgWaves>), grid, block, lc,
                    st, la, pa, (const bf16 *)q, fa, la.table);
    else
      launch_kernel((k_decode<D, REP, false, false, 3, 2, false, kDecodeWgWaves>), grid, block, lc,
                    st, la, pa, (const bf16 *)q, fa, la.table);
  }
}

int launch_decode_wg(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                     const void *q, const FusedArgs &fa, bool fused, const Launch &lc) {
  if (st.C != 1 || la.paged || (la.rep > 8 && la.rep != 16)) return (int)hipErrorInvalidValue;
#define KVC_DEC(DD, RR)                                                  \
  if (st.D == DD && la.rep == RR) {                                      \
    launch_decode_wg_t<DD, RR>(st, la, pa, q, fa, fused, lc);           \
    return (int)hipGetLastError();                                       \
  }
  KVC_DEC(128, 1) KVC_DEC(128, 2) KVC_DEC(128, 4) KVC_DEC(128, 8) KVC_DEC(128, 16)
  KVC_DEC(64, 1) KVC_DEC(64, 2) KVC_DEC(64, 4) KVC_DEC(64, 8) KVC_DEC(64, 16)
#undef KVC_DEC
  return (int)hipErrorInvalidValue;
}

template <int D, int REP>
static int decode_waves_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_decode<D, REP>, 64, 0) != hipSuccess)
    return 0;
  return n;
}

int decode_waves_per_cu(int D, int rep) {
#define KVC_OCC(DD, RR) \
  if (D == DD && rep == RR) return decode_waves_t<DD, RR>();
  KVC_OCC(128, 1) KVC_OCC(128, 2) KVC_OCC(128, 4) KVC_OCC(128, 8) KVC_OCC(128, 16)
  KVC_OCC(64, 1) KVC_OCC(64, 2) KVC_OCC(64, 4) KVC_OCC(64, 8) KVC_OCC(64, 16)
#undef KVC_OCC
  return 0;
}

int launch_decode_fused(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                        const void *q, const FusedArgs &fa, int32_t n_items, bool merge,
                        const Launch &lc) {
  if (st.C != 1) return (int)hipErrorInvalidValue;
#define KVC_DEC(DD, RR)                                                  \
  if (st.D == DD && la.rep == RR) {                                      \
    launch_decode_fused_t<DD, RR>(st, la, pa, q, fa, n_items, merge, lc); \
    return (int)hipGetLastError();                                       \
  }
  KVC_DEC(128, 1) KVC_DEC(128, 2) KVC_DEC(128, 4) KVC_DEC(128, 8) KVC_DEC(128, 16)
  KVC_DEC(64, 1) KVC_DEC(64, 2) KVC_DEC(64, 4) KVC_DEC(64, 8) KVC_DEC(64, 16)
#undef KVC_DEC
  return (int)hipErrorInvalidValue;
}

int launch_decode(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, const void *q,
                  int32_t n_items, const Launch &lc) {
#define KVC_DEC(DD, RR)                                         \
  if (st.D == DD && la.rep == RR) {                             \
    launch_decode_t<DD, RR>(st, la, pa, q, n_items, lc);    \
    return (int)hipGetLastError();                              \
  }
  KVC_DEC(128, 1) KVC_DEC(128, 2) KVC_DEC(128, 4) KVC_DEC(128, 8) KVC_DEC(128, 16)
  KVC_DEC(64, 1) KVC_DEC(64, 2) KVC_DEC(64, 4) KVC_DEC(64, 8) KVC_DEC(64, 16)
#undef KVC_DEC
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Chunk attention (rows with two or more new tokens), bf16, MFMA.
// Workgroup = 8 waves = up to 256 query rows of one (row b, KV head g), so
// each key tile is read from HBM once for all of them; query row
// r = i * REP + hl (token-major), wave w holds rows w*32 .. w*32+31 as two
// 16-row blocks.  Key tiles of 32 rows pass through a ring of LDS stages
// (8 for the 8-wave workgroup, 4 for the 4-wave one): buffer loads with the
// lds bit move each tile from HBM straight into its stage (no registers on
// the way; K chunks at swizzled positions, V in the cache's own
// [d][16 keys] block order), waits for them are placed by hand, and one
// barrier per tile publishes the stage.  Per wave and tile:
//   S^T (32 keys x 16 queries) = K . Q^T   with v_mfma_f32_16x16x32_bf16
//   O^T (D x 16 queries)     += V^T . P^T  with the same instruction,
// each K and V operand one 16-byte LDS read, used for both query blocks;
// the score accumulator already has the layout P^T needs as an operand.
// Masks apply only on tiles at the diagonal or an edge.
// ---------------------------------------------------------------------------
// PAGED: a paged full layer; a 32-row tile spans two pages, and the chunks
// each wave loads lie in one of them.
// QW: waves per workgroup, 32 query rows each (8: 256-row query tiles, the
// only workgroup on its CU; 4: 128-row tiles for short chunks, two per CU).
// KH (with QW 8): the eight waves are two groups of four over one 128-row
// query tile, group h computing the key tiles i with i % 2 == h; the groups'
// softmax states merge in LDS at the end.  The form of the 128-row query
// tiles: a tile's keys take half the steps, and where the 4-wave form would
// leave one wave per SIMD (a ring layer's chunk step over a small batch)
// there are two.
template <int D, int REP, bool PAGED = false, int QW = 8, bool KH = false>
__global__ __launch_bounds__(QW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void k_chunk(StepArgs st, LayerArgs la, PartialArgs pa,
                                                   const bf16 *__restrict__ q,
                                                   const int32_t *__restrict__ ptab) {
  constexpr int NDS = D / 32;              // 32-wide d steps (QK contraction)
  constexpr int NDB = D / 16;              // 16-wide d blocks (PV output)
  constexpr int CPR = D / 8;               // 16-byte chunks of a K row
  constexpr int KCH = 32 * D / 8;          // 16-byte chunks of a K tile (= of a V tile)
  constexpr int NT = QW * 64;              // threads
  static_assert(!KH || QW == 8, "key halves: two groups of four waves");
  constexpr int QT = KH ? 128 : QW * 32;   // query rows per workgroup
  // Tiles go from memory straight to LDS (buffer loads with the lds bit):
  // one load instruction fills a 1 KB slab of 64 chunks, lane L writing
  // chunk L.  A tile is NSL slabs (K, then V), each wave loading SPW of them.
  constexpr int NSL = 2 * KCH / 64;
  constexpr int SPW = NSL / QW;
  // LDS stages: NSTAGE - 1 tiles are in flight while one is computed.  The
  // eight-wave workgroup is alone on its CU; two four-wave ones share one.
  constexpr int NSTAGE = QW == 8 ? 8 : 4;
  constexpr int STAGE_B = 2 * KCH * 16;    // bytes of a stage: K, then V
  static_assert(SPW >= 1 && NSL % QW == 0, "chunk mapping");
  // Stage layout.  K: 32 rows of CPR chunks, chunk c of row r at position
  // r * CPR + (c ^ swz(r)): the 16 rows an operand read takes (see qk) land
  // in distinct banks.  V: the cache's own layout, two 16-row blocks of
  // [d][16 keys], chunk (d, half) of a block at position 2 d + (half ^ bit 3
  // of d): the 16 d of an operand read land in distinct banks.
  __shared__ __align__(16) char ltile[NSTAGE][STAGE_B];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qwave = KH ? (wave & 3) : wave;  // this wave's 32 query rows of the tile
  const int khalf = KH ? (wave >> 2) : 0;    // (KH) its half of the key tiles
  const int q4 = lane >> 4, nl = lane & 15;
  const int g = blockIdx.y;
  const int SKP = pa.pre_split_keys;

  int b;
  int64_t local;
  find_item(
      st.B, blockIdx.x,
      [&](int r) -> int {
        const int n = st.n_new[r];
        if (n < 2) return 0;
        // with chunk_small 1, rows of at most 128 query rows go to the
        // 4-wave launch and the rest to the 8-wave one; with 2, every row
        // goes to the 4-wave launch
        const bool small = pa.chunk_small == 2 || n * REP <= 4 * 32;
        if (pa.chunk_small && small != (QW == 4 || KH)) return 0;
        const int nqt = (int)cdiv((int64_t)n * REP, QT);
        if (la.ring) return nqt;
        int64_t base, lo, hi;
        chunk_span_dev(la, st.lens[r], n, st.first[r], &base, &lo, &hi);
        return nqt * (int)cdiv(hi - base, SKP);
      },
      &b, &local);
  if (b < 0) return;
  // (the row's three counts in one round trip, before the query and tile
  // loads: a count read later would wait for those too)
  const int64_t L = st.lens[b];
  const int n = st.n_new[b];
  const int first_i = st.first[b];  // left padding: keys before it are hidden
  int nks = 1;
  int64_t cbase = 0, clo = 0, chi = 0;
  if (!la.ring) {
    chunk_span_dev(la, L, n, first_i, &cbase, &clo, &chi);
    nks = (int)cdiv(chi - cbase, SKP);
  }
  const int qt = (int)(local / nks), ks = (int)(local % nks);
  const int64_t bg = (int64_t)b * la.hkv + g;
  const int W = la.window;

  // -- this wave's two 16-row query blocks; lane (q4, nl) holds row nl --------
  // Their loads (and those of their rotation) go out here; the rotation runs
  // after the first key tiles' loads are issued, so the two round trips
  // overlap instead of following one another.
  constexpr int HS = NDS / 2;  // partner d + D/2 sits HS steps later
  int rq[2], qi[2], hl[2];
  bool rvalid[2];
  int64_t qpos[2];
  uint4 qv[2][NDS];
  float4 rp[2][HS][4];  // (cos, sin) of the 8 consecutive frequencies of a step, 4 per load
  const bool rot = st.rope != nullptr;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    rq[blk] = qt * QT + qwave * 32 + blk * 16 + nl;
    rvalid[blk] = rq[blk] < n * REP;
    // A row past the tile's queries computes with the last query row (its
    // output is never written): every lane loads, so no load sits under a
    // lane mask (whose results the compiler copies, waiting for them).
    const int rqc = rvalid[blk] ? rq[blk] : n * REP - 1;
    qi[blk] = rqc / REP;
    hl[blk] = rqc % REP;
    qpos[blk] = L + qi[blk];
    const bf16 *qsrc = q + (((int64_t)b * st.C + qi[blk]) * st.Hq + g * REP + hl[blk]) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qv[blk][ds] = *reinterpret_cast<const uint4 *>(qsrc + ds * 32 + q4 * 8);
#pragma unroll
    for (int ds = 0; ds < HS; ++ds) {
      const float4 *rsrc =
          reinterpret_cast<const float4 *>(st.rope + (qpos[blk] * (D / 2) + ds * 32 + q4 * 8) * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        rp[blk][ds][u] = rot ? rsrc[u] : make_float4(1.f, 0.f, 1.f, 0.f);
    }
  }
  // -- the chunk's own rows from the caller's K and V (the appending entry) ----
  // Rows 0 .. 63 of this (row, KV head): K as pairs of 16-byte chunks (c,
  // c + CPR / 2) with the (cos, sin) of their 8 frequencies, V as 16-byte
  // chunks; rows past n hold zeros.  own_store rotates K
  // (the append's arithmetic, so the bits match a staged row) and writes
  // both into the stage layout, tile t of the rows into stage t.
  const bool fz = !PAGED && la.ring && pa.ck != nullptr;
  constexpr int OKP = kChunkOwnMax * (CPR / 2), OVC = kChunkOwnMax * CPR;
  constexpr int KPT = (OKP + NT - 1) / NT, VPT = (OVC + NT - 1) / NT;
  uint4 okx[KPT][2], ovx[VPT];
  float4 ocs[KPT][4];
  auto own_load = [&]() __attribute__((always_inline)) {
    const bf16 *ckb = static_cast<const bf16 *>(pa.ck);
    const bf16 *cvb = static_cast<const bf16 *>(pa.cv);
    // (every lane loads: items past the end and rows past n read the last
    // row, and own_store writes zeros for them)
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int it = min(tid + u * NT, OKP - 1), c = it % (CPR / 2);
      const int rr = min(it / (CPR / 2), n - 1);
      const bf16 *src = ckb + (((int64_t)b * st.C + rr) * la.hkv + g) * D + c * 8;
      okx[u][0] = *reinterpret_cast<const uint4 *>(src);
      okx[u][1] = *reinterpret_cast<const uint4 *>(src + D / 2);
      const float4 *rs = reinterpret_cast<const float4 *>(st.rope + ((L + rr) * (D / 2) + c * 8) * 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) ocs[u][w] = rot ? rs[w] : make_float4(1.f, 0.f, 1.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int it = min(tid + u * NT, OVC - 1), c = it % CPR;
      const int rr = min(it / CPR, n - 1);
      ovx[u] = *reinterpret_cast<const uint4 *>(cvb + (((int64_t)b * st.C + rr) * la.hkv + g) * D +
                                                 c * 8);
    }
  };
  auto own_store = [&](int ntile) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int it = tid + u * NT, rr = it / (CPR / 2), c = it % (CPR / 2);
      if (it < OKP && rr < ntile * 32) {
        const bool live = rr < n;
        const uint32_t w0[4] = {okx[u][0].x, okx[u][0].y, okx[u][0].z, okx[u][0].w};
        const uint32_t w1[4] = {okx[u][1].x, okx[u][1].y, okx[u][1].z, okx[u][1].w};
        uint32_t y0[4], y1[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float a[2], bb[2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const float x1 = h2 ? bf_hi(w0[e2]) : bf_lo(w0[e2]);
            const float x2 = h2 ? bf_hi(w1[e2]) : bf_lo(w1[e2]);
            const float4 cs = ocs[u][e2];
            a[h2] = x1;
            bb[h2] = x2;
            if (rot) rope_pair(x1, x2, h2 ? cs.z : cs.x, h2 ? cs.w : cs.y, &a[h2], &bb[h2]);
          }
          y0[e2] = live ? pack_bf16(a[0], a[1]) : 0u;
          y1[e2] = live ? pack_bf16(bb[0], bb[1]) : 0u;
        }
        const int r = rr % 32;
        const int swz = ((r & 3) | (((r >> 3) & 3) << 2)) & (CPR - 1);
        char *kt = &ltile[rr / 32][0];
        *reinterpret_cast<uint4 *>(kt + (r * CPR + (c ^ swz)) * 16) =
            make_uint4(y0[0], y0[1], y0[2], y0[3]);
        *reinterpret_cast<uint4 *>(kt + (r * CPR + ((c + CPR / 2) ^ swz)) * 16) =
            make_uint4(y1[0], y1[1], y1[2], y1[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int it = tid + u * NT, rr = it / CPR, c = it % CPR;
      if (it < OVC && rr < ntile * 32) {
        const int r = rr % 32, blk = r / 16, half = (r % 16) / 8;
        const bool live = rr < n;
        const uint32_t w[4] = {live ? ovx[u].x : 0u, live ? ovx[u].y : 0u, live ? ovx[u].z : 0u,
                               live ? ovx[u].w : 0u};
        char *vt = &ltile[rr / 32][KCH * 16] + (r % 8) * 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = c * 8 + e;
          *reinterpret_cast<uint16_t *>(vt + (blk * 2 * D + ((2 * d + half) ^ ((d >> 3) & 1))) * 16) =
              (uint16_t)((e & 1) ? w[e / 2] >> 16 : w[e / 2] & 0xffffu);
        }
      }
    }
  };
  if (fz) own_load();
  // (the loads above are issued before anything below: the hand-placed tile
  // waits count only the tile loads that follow them)
  asm volatile("" ::: "memory");
  bf16x8_t qf[2][NDS];
  auto make_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      float raw[NDS][8];
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const uint32_t w[4] = {qv[blk][ds].x, qv[blk][ds].y, qv[blk][ds].z, qv[blk][ds].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          raw[ds][2 * e2] = bf_lo(w[e2]);
          raw[ds][2 * e2 + 1] = bf_hi(w[e2]);
        }
      }
      // (rows past the tile's queries unrotated: their outputs are never
      // written, and the branch measured a tighter main loop than without)
      if (rot && rvalid[blk]) {
#pragma unroll
        for (int ds = 0; ds < HS; ++ds)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float4 cs = rp[blk][ds][e / 2];
            const float c = (e & 1) ? cs.z : cs.x;
            const float sn = (e & 1) ? cs.w : cs.y;
            const float x1 = raw[ds][e], x2 = raw[ds + HS][e];
            raw[ds][e] = x1 * c - x2 * sn;
            raw[ds + HS][e] = x1 * sn + x2 * c;
          }
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[blk][ds][e] = (bf16)raw[ds][e];
    }
  };
  const bool wave_live = __builtin_amdgcn_readfirstlane((int)(__ballot(rvalid[0]) != 0)) != 0;

  // -- key runs ------------------------------------------------------------------
  // At most two runs of storage rows, visited in order: a full layer's cache
  // rows (run 0 only), or a ring layer's history slots (run 0) and then the
  // chunk's own rows in staging (run 1).  Per run, as 32-bit scalars: the
  // first row (a multiple of 32), the rows holding this sequence's data
  // [vlo, vhi), and the position of row t, t + (t < psplit ? poff_a : poff_b):
  // a full layer's row is its position; ring slot t holds t + L - L mod W
  // below L mod W (the slot the next token takes) and t + L - L mod W - W
  // from there on; staging row t holds L + t.  (Positions fit in 32 bits:
  // max_len < 2^31.)
  // Positions of the whole q-tile span [pmin, pmax].
  const int rlast = (qt + 1) * QT - 1 < n * REP - 1 ? (qt + 1) * QT - 1 : n * REP - 1;
  const int64_t pmin = L + (int64_t)(qt * QT) / REP;
  const int64_t pmax = L + rlast / REP;
  const int Li = (int)L, pmin_i = (int)pmin, pmax_i = (int)pmax;
  int f0, e0, vlo0, vhi0, psplit0 = 0, pa0 = 0, pb0 = 0;
  if (!la.ring) {
    int64_t a = cbase + (int64_t)ks * SKP;
    int64_t e = a + SKP < chi ? a + SKP : chi;
    if (e > pmax + 1) e = pmax + 1;
    if (W > 0) {
      const int64_t wlo = (pmin - W + 1) / 32 * 32;
      if (a < wlo) a = wlo;
    }
    f0 = (int)a;
    e0 = (int)(e > a ? e : a);
    vlo0 = (int)clo;
    vhi0 = (int)chi;
  } else {
    const int nh = L < W ? Li : W;
    f0 = 0;
    e0 = nh;
    vlo0 = 0;
    vhi0 = nh;
    psplit0 = (int)(L % W);
    pa0 = Li - psplit0;
    pb0 = Li - psplit0 - W;
  }
  const int n0 = __builtin_amdgcn_readfirstlane((e0 - f0 + 31) / 32);
  const int n1 = __builtin_amdgcn_readfirstlane(la.ring ? (n + 31) / 32 : 0);
  const int ntiles = n0 + n1;

  // -- buffer resources: this head's K and V in each run, and an empty one
  const int64_t reg0 = (int64_t)la.rows_alloc * D * 2;
  const i32x4 dk0 = sgpr_rsrc(la.k + bg * reg0, (int)reg0);
  const i32x4 dv0 = sgpr_rsrc(la.v + bg * reg0, (int)reg0);
  const int64_t reg1 = la.ring ? (int64_t)la.stage_rows_alloc * D * 2 : 0;
  const i32x4 dk1 = la.ring ? sgpr_rsrc(la.sk + bg * reg1, (int)reg1) : dk0;
  const i32x4 dv1 = la.ring ? sgpr_rsrc(la.sv + bg * reg1, (int)reg1) : dv0;
  const i32x4 dnone = sgpr_rsrc(la.k, 0);
  // This wave's slabs: j = wave + QW e (e < SPW); slab j < KCH / 64 holds K
  // chunks, the rest V chunks.  Per lane: the byte offset of the chunk it
  // fetches within the tile, and the slab's byte offset within a stage.
  constexpr int KSL = KCH / 64;            // K slabs per tile
  int soff_lane[SPW];                      // source offset within the tile (bytes)
#pragma unroll
  for (int e = 0; e < SPW; ++e) {
    const int j = wave + QW * e;
    const int pos = (j < KSL ? j : j - KSL) * 64 + lane;  // chunk position in the LDS region
    if (j < KSL) {
      const int r = pos / CPR, pc = pos % CPR;
      const int swz = ((r & 3) | (((r >> 3) & 3) << 2)) & (CPR - 1);
      soff_lane[e] = (r * CPR + (pc ^ swz)) * 16;
    } else {
      const int blk = pos / (2 * D), qq = pos % (2 * D), d = qq >> 1;
      soff_lane[e] = (blk * 2 * D + (qq ^ ((d >> 3) & 1))) * 16;
    }
  }
  // paged: the 16-row page of slab j within a tile (a slab is 64 chunks: K
  // rows of one page, or part of one V block), the same for every lane
  auto slab_page = [](int j) __attribute__((always_inline)) {
    return j < KSL ? (j * 64 / CPR) / kPageRows : ((j - KSL) * 64) / (2 * D);
  };
  // paged: bytes of one head's page (16 K rows, or one V block)
  constexpr int page_b = kPageRows * D * 2;
  // The chunk's own rows (run 1) are tiles [own0, own0 + n1): after the
  // history, or first when they come from the caller's K and V (written to
  // their stages by own_store before the first barrier, no loads issued).
  const int own0 = fz ? 0 : n0, hist0 = fz ? n1 : 0;
  auto own = [=](int i) __attribute__((always_inline)) {
    return (unsigned)(i - own0) < (unsigned)n1;
  };
  // First storage row of tile i (run 0 from f0, run 1 from row 0).
  auto tile_row = [=](int i) __attribute__((always_inline)) {
    return own(i) ? (i - own0) * 32 : f0 + (i - hist0) * 32;
  };
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)&ltile[0][0];
  // Issue the loads of tile i into stage st_ (zeros and no memory access
  // past the last tile).
  auto issue = [&](int i, int st_) __attribute__((always_inline)) {
    const bool live = i < ntiles;
    const bool second = own(i);
    const int t0 = tile_row(live ? i : 0);
    // (the tile's two sources picked once; when the K slabs are a whole
    // number of rounds of the waves, slab e of every wave is K or V alike,
    // known at compile time)
    const i32x4 rk = PAGED ? dnone : rsrc_sel(live, rsrc_sel(second, dk1, dk0), dnone);
    const i32x4 rv = PAGED ? dnone : rsrc_sel(live, rsrc_sel(second, dv1, dv0), dnone);
#pragma unroll
    for (int e = 0; e < SPW; ++e) {
      const int j = wave + QW * e;
      const bool isv = KSL % QW == 0 ? QW * e >= KSL : j >= KSL;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(
          lds0 + st_ * STAGE_B + (isv ? KCH * 16 + (j - KSL) * 1024 : j * 1024));
      if constexpr (PAGED) {
        // a slab lies in one page: K rows of one block, or one V block
        const int sp = slab_page(j);
        const int idx = live ? t0 / kPageRows + sp : 0;
        const int pg = ptab[(int64_t)b * la.ppr + idx];
        const int64_t off = ((int64_t)pg * la.hkv + g) * page_b;
        const i32x4 rs = rsrc_sel(live, sgpr_rsrc((isv ? la.v : la.k) + off, page_b), dnone);
        lds_load(m0, soff_lane[e] - sp * page_b, rs, 0);
      } else {
        // K rows and V blocks advance by the same bytes per row
        lds_load(m0, soff_lane[e], isv ? rv : rk, __builtin_amdgcn_readfirstlane(t0 * D * 2));
      }
    }
  };

  const float scale = kLog2e * rsqrtf((float)D);
  // Reference-max slack (log2 units): p < 2^8 keeps P well inside bf16 and
  // l, O inside fp32.
  constexpr float kLazyRescale = 8.f;
  // Lowest position each query block row may see besides its own: the
  // window's and the left padding's bound (a pad query sees only itself).
  int qp32[2], lowq[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    qp32[blk] = (int)qpos[blk];
    const int wl = W > 0 ? qp32[blk] - W + 1 : 0;
    lowq[blk] = wl > first_i ? wl : first_i;
  }
  // Tiles whose keys every query of the q tile sees (data rows below the
  // tile's first position and, on a windowed layer, inside its last
  // position's window) need no mask: only those at the diagonal and the
  // edges do.  Within a stretch of storage rows whose position is row + po,
  // a tile starting at row t0 is such a tile iff lo <= t0 <= hi, so the
  // full tiles are index ranges, found once here: the run-0 rows below
  // psplit (po = pa0: a ring's newer slots) and from psplit on (po = pb0;
  // a full layer has psplit 0), and the run-1 rows (po = L).  A ring tile
  // across psplit is in neither.
  auto full_tiles = [&](int po, int vlo, int vhi, int rlo, int rhi, int base, int *klo, int *khi) {
    int lo = max(max(vlo, first_i - po), rlo);
    if (W > 0) lo = max(lo, pmax_i - W + 1 - po);
    const int hi = min(min(vhi - 32, pmin_i - 31 - po), rhi);
    *klo = lo <= base ? 0 : (lo - base + 31) / 32;
    *khi = hi < base ? -1 : (hi - base) / 32;
  };
  int fa0, fa1, fb0, fb1, fo0, fo1;
  full_tiles(pa0, vlo0, vhi0, f0, psplit0 - 32, f0, &fa0, &fa1);
  full_tiles(pb0, vlo0, vhi0, psplit0, 1 << 30, f0, &fb0, &fb1);
  full_tiles(Li, 0, n, 0, 1 << 30, 0, &fo0, &fo1);
  fa0 = __builtin_amdgcn_readfirstlane(fa0);
  fa1 = __builtin_amdgcn_readfirstlane(fa1);
  fb0 = __builtin_amdgcn_readfirstlane(fb0);
  fb1 = __builtin_amdgcn_readfirstlane(fb1);
  fo0 = __builtin_amdgcn_readfirstlane(fo0);
  fo1 = __builtin_amdgcn_readfirstlane(fo1);
  // (as absolute tile indices, each range clipped to its run)
  const int fa_lo = hist0 + fa0, fa_hi = hist0 + min(fa1, n0 - 1);
  const int fb_lo = hist0 + fb0, fb_hi = hist0 + min(fb1, n0 - 1);
  const int fo_lo = own0 + fo0, fo_hi = own0 + min(fo1, n1 - 1);
  // Per block: the reference max m (scaled log2 domain), the exponent
  // offset mu = max(m, -FLT_MAX) and the threshold m + kLazyRescale past
  // which a tile moves m; all three change only on the rare moving tiles.
  float mrun[2] = {-INFINITY, -INFINITY}, mu[2] = {-FLT_MAX, -FLT_MAX},
        thr[2] = {-INFINITY, -INFINITY};
  floatx4 oacc[2][NDB];
  // The rows' sums of P on the matrix cores: a product with a ones operand
  // gives, in every row of its output, the column sums of the tile's P^T
  // (the query's sum over the tile's 32 keys), so no lane sums its 8
  // probabilities and no cross-lane sum is left for the end.
  floatx4 lacc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  bf16x8_t ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.f;
  // held in registers through the loop rather than rebuilt for every tile
  asm volatile("" : "+v"(ones));
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[blk][db] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int i, int s) __attribute__((always_inline)) {
    // S^T = K Q^T for both query blocks, each K operand read once
    floatx4 sacc[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[blk][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8_t ka[2][NDS];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        // A row i of this product is key 8 (i / 4) + 4 kb + i % 4, so lane
        // (q4, nl) ends with keys 8 q4 .. 8 q4 + 7 of the tile, the P^T
        // operand order of P.V
        const int r = 8 * (nl >> 2) + 4 * kb + (nl & 3), c = ds * 4 + q4;
        const int swz = ((r & 3) | (((r >> 3) & 3) << 2)) & (CPR - 1);
        ka[kb][ds] = *reinterpret_cast<const bf16x8_t *>(&ltile[s][(r * CPR + (c ^ swz)) * 16]);
      }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          sacc[blk][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb][ds], qf[blk][ds],
                                                                  sacc[blk][kb], 0, 0, 0);
    // Every K operand read goes out before the first product (left to
    // itself the scheduler may read one operand, wait for it and reuse its
    // registers for the next).
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NDS, 1);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * NDS, 1);  // MFMA
    // mask + scale + online softmax per block; sacc[blk][kb][jj] is key row
    // t0 + 8 q4 + 4 kb + jj, query row nl of the block; unmasked on the full
    // tiles found above
    const bool full = (i >= fa_lo && i <= fa_hi) || (i >= fb_lo && i <= fb_hi) ||
                      (i >= fo_lo && i <= fo_hi);
    // Both blocks' masks and maxima first, then one (rarely taken) branch
    // for the accumulators' rescale, so that the exponentials and the P.V
    // products of the two blocks share one basic block and the scheduler can
    // run one block's exponentials beside the other's matrix products.
    float sv[2][2][4];  // raw scores q.k (the scale enters with the exponent)
    float tmax[2] = {-INFINITY, -INFINITY};
    if (full) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            sv[blk][kb][jj] = sacc[blk][kb][jj];
            tmax[blk] = fmaxf(tmax[blk], sv[blk][kb][jj]);
          }
    } else {
      // (the tile's run: its first row, data rows and positions)
      const bool second = own(i);
      const int t0 = tile_row(i);
      const int vlo = second ? 0 : vlo0, vhi = second ? n : vhi0;
      const int psplit = second ? 0 : psplit0;
      const int poa = second ? Li : pa0, pob = second ? Li : pb0;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int t = t0 + 8 * q4 + 4 * kb + jj;
            const int pos = t + (t < psplit ? poa : pob);
            const bool ok = (unsigned)(t - vlo) < (unsigned)(vhi - vlo) && pos <= qp32[blk] &&
                            (pos >= lowq[blk] || pos == qp32[blk]);
            const float x = ok ? sacc[blk][kb][jj] : -INFINITY;
            sv[blk][kb][jj] = x;
            tmax[blk] = fmaxf(tmax[blk], x);
          }
      }
    }
    // Reference max, in the scaled log2 domain, moved only when the tile's
    // max passes it by more than kLazyRescale: p = 2^(s*scale - m) then
    // stays below 2^kLazyRescale, and the accumulators are rescaled on rare
    // tiles instead of whenever some row's max grows.
    // the row's max over the tile: its 4 lane groups hold 8 keys each
    rows_max_pair(tmax[0], tmax[1]);
    float tm[2];
    bool move[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      tm[blk] = tmax[blk] * scale;
      move[blk] = tm[blk] > thr[blk];
    }
    if (__ballot(move[0] || move[1]) != 0) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float mn = move[blk] ? tm[blk] : mrun[blk];
        const float alpha = move[blk] ? __builtin_amdgcn_exp2f(mrun[blk] - mn) : 1.f;
        // mn = -inf only where every score of the row is -inf so far, and
        // then s * scale - mu stays -inf with any finite mu
        mu[blk] = max_lowest(mn);
        thr[blk] = mn + kLazyRescale;
        mrun[blk] = mn;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[blk][db] *= alpha;
        lacc[blk] *= alpha;
      }
    }
    // O^T += V^T P^T; k-slot 8 q4 + e <-> key 8 q4 + e: 16 bytes of block
    // q4 / 2 at (d, half q4 % 2).  Each V operand (head-dim row db * 16 + nl)
    // serves both blocks.
    bf16x8_t pf[2];
    // Row d = 16 db + nl sits at chunk 2 d + q4 % 2, bit 0 flipped by bit 3
    // of d (= bit 3 of nl): every db adds the same 32 chunks, so one lane
    // address serves all NDB reads through the immediate offset.
    const char *vrow = &ltile[s][KCH * 16 + ((q4 >> 1) * 2 * D + ((2 * nl + (q4 & 1)) ^ ((nl >> 3) & 1))) * 16];
    uint4 av[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) av[db] = *reinterpret_cast<const uint4 *>(vrow + db * 32 * 16);
    auto probs = [&](int blk) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sv[blk][kb][jj], scale, -mu[blk]));
          pf[blk][kb * 4 + jj] = (bf16)pe;
        }
    };
    probs(0);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      oacc[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, av[db]), pf[0], oacc[0][db], 0, 0, 0);
    lacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[0], lacc[0], 0, 0, 0);
    probs(1);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      oacc[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, av[db]), pf[1], oacc[1][db], 0, 0, 0);
    lacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[1], lacc[1], 0, 0, 0);
    // Instruction order for the scheduler: the V operand reads, block 0's
    // probabilities, then block 0's products each followed by a share of
    // block 1's vector work (its exponentials run while the matrix core
    // works), then block 1's products.  Measured on the 32k prefill of the
    // long-context workload: 620 -> 671 TFLOP/s with the softmax
    // restructured into one basic block, 648 of that without this order.
    __builtin_amdgcn_sched_group_barrier(0x100, NDB, 0);     // DS read
    __builtin_amdgcn_sched_group_barrier(0x002, 30, 0);      // VALU (block 0)
#pragma unroll
    for (int k = 0; k < NDB + 1; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);     // VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NDB + 1, 0); // MFMA
  };

  // Pipeline, TP tiles per barrier (the 8-wave workgroup takes two: one
  // barrier of all eight waves per 64 keys; 808 -> 843 TFLOP/s on the
  // long-context prefill and 17.9 -> 17.2 ms per mixed step; four tiles and
  // two tiles in the 4-wave workgroup measured no better).  Tiles 0 ..
  // NSTAGE - TP - 1 go out first, into stages of their own index.  Step i
  // (i a multiple of TP): this wave waits for its own loads of tiles i ..
  // i + TP - 1 (the NSTAGE - 2 TP tiles issued after them stay in flight),
  // every wave meets at the barrier (those tiles are then in LDS, and every
  // wave is done with tiles i - TP .. i - 1), tiles i + NSTAGE - TP ..
  // i + NSTAGE - 1 go out into the stages those used, and tiles i ..
  // i + TP - 1 are computed.  Loads past the last tile read nothing and
  // write zeros.  The queries' loads above are older than every tile load,
  // so the tile waits retire them too.
  constexpr int TP = QW == 8 ? 2 : 1;
  static_assert(NSTAGE >= 2 * TP, "tiles in flight beside the ones computed");
  static_assert(NSTAGE - TP >= kChunkOwnMax / 32, "own_store tiles all in the prologue");
  // (Tiles written by own_store issue no loads.  They are the first ones, so
  // every wait below still finds its tiles' loads older than the count it
  // leaves in flight.)
  const int skip = fz ? n1 : 0;
  for (int t = 0; t < NSTAGE - TP; ++t)
    if (t >= skip) issue(t, t);
  // Nothing below moves above the tile loads: the queries are rotated while
  // the first tiles are in flight.
  __builtin_amdgcn_sched_barrier(0);
  if (fz) own_store(n1);
  make_q();
  for (int i = 0; i < ntiles; i += TP) {
    lds_wait<SPW * (NSTAGE - 2 * TP)>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int u = 0; u < TP; ++u) issue(i + NSTAGE - TP + u, (i + NSTAGE - TP + u) % NSTAGE);
    if (wave_live) {
      if constexpr (KH) {
        if (i + khalf < ntiles) compute(i + khalf, (i + khalf) % NSTAGE);
      } else {
#pragma unroll
        for (int u = 0; u < TP; ++u)
          if (u == 0 || i + u < ntiles) compute(i + u, (i + u) % NSTAGE);
      }
    }
  }
  // the loads of tiles past the end land before the LDS is released
  lds_wait<0>();
  float lrun[2] = {lacc[0][0], lacc[1][0]};  // each row's sum of P (any of the 4 rows)
  if constexpr (KH) {
    // Merge the key halves: the second group leaves its state (per lane:
    // reference max, partial sum and O^T accumulators of both blocks) in the
    // stages, the first takes it in.  Lanes of waves w and w + 4 hold the
    // same query rows and head-dim columns.
    static_assert(4 * 64 * (4 + 8 * NDB) * 4 <= NSTAGE * STAGE_B, "merge area");
    // (16-byte slots, slot k of the 64 lanes of a wave contiguous: one
    // conflict-free 1 KB LDS access per slot; slot 0 holds the two blocks'
    // maxima and sums, slot 1 + blk * NDB + db their accumulators)
    constexpr int XS = 1 + 2 * NDB;  // slots per lane
    float4 *xs = reinterpret_cast<float4 *>(&ltile[0][0]) + qwave * XS * 64 + lane;
    __syncthreads();
    if (khalf == 1) {
      xs[0] = make_float4(mrun[0], mrun[1], lrun[0], lrun[1]);
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          xs[(1 + blk * NDB + db) * 64] = make_float4(oacc[blk][db][0], oacc[blk][db][1],
                                                      oacc[blk][db][2], oacc[blk][db][3]);
    }
    __syncthreads();
    if (khalf == 0) {
      const float4 ml = xs[0];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float m1 = blk ? ml.y : ml.x, l1 = blk ? ml.w : ml.z;
        const float mm = fmaxf(mrun[blk], m1);
        const float a0 = mrun[blk] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[blk] - mm);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        lrun[blk] = lrun[blk] * a0 + l1 * a1;
        mrun[blk] = mm;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float4 o1 = xs[(1 + blk * NDB + db) * 64];
          oacc[blk][db][0] = oacc[blk][db][0] * a0 + o1.x * a1;
          oacc[blk][db][1] = oacc[blk][db][1] * a0 + o1.y * a1;
          oacc[blk][db][2] = oacc[blk][db][2] * a0 + o1.z * a1;
          oacc[blk][db][3] = oacc[blk][db][3] * a0 + o1.w * a1;
        }
      }
    }
  }

  // -- partials for this split (over a joint partner's keys: after the
  // layer's own splits) ------------------------------------------------------------
  const int sbase = pa.base.on ? ref_splits(pa.base, L, n, first_i) : 0;
#pragma unroll
  for (int blk = 0; blk < 2 && khalf == 0; ++blk) {
    const float lt = lrun[blk];
    if (pa.direct_out) {
      // The row's only split: its final output, with the arithmetic of the
      // merge of one split (weight 1 / l, one fused term, then the merge's
      // additions of zeros), so it has the bits the merge launch would write.
      if (rvalid[blk]) {
        const float inv = 1.f / lt;
        bf16 *o = static_cast<bf16 *>(pa.direct_out) +
                  (((int64_t)b * st.C + qi[blk]) * st.Hq + g * REP + hl[blk]) * D;
        // (four consecutive elements per lane and d block: one 8-byte store)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          float y[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) y[jj] = fmaf(inv, oacc[blk][db][jj], 0.f) + 0.f;
          *reinterpret_cast<uint2 *>(o + db * 16 + q4 * 4) =
              make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]));
        }
      }
      continue;
    }
    if (rvalid[blk]) {
      const int64_t slot =
          (((int64_t)b * pa.max_chunk + qi[blk]) * st.Hq + g * REP + hl[blk]) * kChunkSplitCap +
          sbase + ks;
      if (q4 == 0) {
        pa.pml[slot * 2 + 0] = lt > 0.f ? mrun[blk] : -INFINITY;
        pa.pml[slot * 2 + 1] = lt;
      }
      if (lt > 0.f) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            pa.pout[slot * D + db * 16 + q4 * 4 + jj] = oacc[blk][db][jj];
      }
    }
  }

  // -- ring commit (colibri PR "How it works": append after scoring) ---------------
  // A ring layer's chunk rows were scored from the ring and from staging;
  // once every q tile of this (row, KV head) has read them, the staged rows
  // that survive the keep rule (positions >= L + n - W) go to their slots
  // p mod W.  Each workgroup counts its finish; the last one commits.  Every
  // other workgroup's loads have returned before its count (its waves
  // waited for all of them), so no read of a slot can follow its overwrite.
  if (pa.ring_cnt != nullptr) {
    // (the flag of the last workgroup goes through the first word of the
    // stages, free once every wave has passed the barrier below)
    int *commit_last = reinterpret_cast<int *>(&ltile[0][0]);
    __syncthreads();
    if (tid == 0) {
      const int nqt = (int)cdiv((int64_t)n * REP, QT);
      const int prev =
          __hip_atomic_fetch_add(pa.ring_cnt + bg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *commit_last = prev == nqt - 1;
    }
    __syncthreads();
    if (*commit_last && fz) {
      // Kept rows from the caller's K and V: staged in LDS again by
      // own_load / own_store (the flag's word is rewritten, so every wave
      // reads it first), then copied out in 16-byte chunks.
      const int i0 = n > W ? n - W : 0;  // first kept row
      __syncthreads();
      own_load();
      own_store(n1);
      __syncthreads();
      constexpr int KC = D / 8;
      for (int c = tid; c < (n - i0) * KC; c += NT) {
        const int rr = i0 + c / KC, ch = c % KC, r = rr % 32;
        const int swz = ((r & 3) | (((r >> 3) & 3) << 2)) & (CPR - 1);
        *reinterpret_cast<uint4 *>(k_row<bf16>(la.k, bg, la.rows_alloc, (Li + rr) % W, D) + ch * 8) =
            *reinterpret_cast<const uint4 *>(&ltile[rr / 32][(r * CPR + (ch ^ swz)) * 16]);
      }
      // V: runs of 8 rows that start at a multiple of 8 on both sides (one
      // 16-byte chunk per d), the rest element by element
      const int a8 = (Li % 8 == 0 && W % 8 == 0) ? (i0 + 7) / 8 * 8 : n;
      const int e8 = a8 < n ? a8 + (n - a8) / 8 * 8 : a8;
      auto vsrc = [&](int rr, int d) __attribute__((always_inline)) {
        const int r = rr % 32, blk = r / 16, half = (r % 16) / 8;
        return &ltile[rr / 32][KCH * 16 + (blk * 2 * D + ((2 * d + half) ^ ((d >> 3) & 1))) * 16] +
               (r % 8) * 2;
      };
      for (int c = tid; c < (e8 - a8) / 8 * D; c += NT) {
        const int rr = a8 + c / D * 8, d = c % D;
        *reinterpret_cast<uint4 *>(v_elem<bf16>(la.v, bg, la.rows_alloc, (Li + rr) % W, d, D)) =
            *reinterpret_cast<const uint4 *>(vsrc(rr, d));
      }
      const int nrest = (n - i0) - (e8 - a8);
      for (int e = tid; e < nrest * D; e += NT) {
        const int k = e / D, d = e % D;
        const int rr = i0 + k < a8 ? i0 + k : e8 + (k - (a8 - i0));
        *v_elem<bf16>(la.v, bg, la.rows_alloc, (Li + rr) % W, d, D) =
            *reinterpret_cast<const bf16 *>(vsrc(rr, d));
      }
      // the step's slot indices (first KV head), and V zeroed past the new
      // top in a tile the ring enters (the append's rule)
      if (pa.slot_out && g == 0)
        for (int i = tid; i < st.C; i += NT)
          pa.slot_out[(int64_t)b * st.C + i] = i < n && i >= i0 ? (Li + i) % W : W;
      if (wave == 0) {
        const int64_t old_top = L < W ? L : W, new_top = L + n < W ? L + n : W;
        if (old_top == 0 || (new_top - 1) / kRowAlign != (old_top - 1) / kRowAlign) {
          int64_t end = (new_top + kRowAlign - 1) / kRowAlign * kRowAlign;
          if (end > la.rows_alloc) end = la.rows_alloc;
          zero_v_rows<bf16>(la.v, bg, la.rows_alloc, new_top, end, D, lane);
        }
      }
      if (tid == 0) __hip_atomic_store(pa.ring_cnt + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (*commit_last) {
      const int i0 = n > W ? n - W : 0;  // first kept staged row
      // Copies of n_items 16-byte chunks, four per thread in flight: every
      // load is issued (past the end the last chunk again) before the stores.
      auto copy4 = [&](int n_items, auto src_of, auto dst_of) __attribute__((always_inline)) {
        for (int c0 = tid; c0 < n_items; c0 += 4 * NT) {
          const int c1 = c0 + NT, c2 = c0 + 2 * NT, c3 = c0 + 3 * NT;
          const uint4 x0 = *src_of(c0);
          const uint4 x1 = *src_of(c1 < n_items ? c1 : n_items - 1);
          const uint4 x2 = *src_of(c2 < n_items ? c2 : n_items - 1);
          const uint4 x3 = *src_of(c3 < n_items ? c3 : n_items - 1);
          *dst_of(c0) = x0;
          if (c1 < n_items) *dst_of(c1) = x1;
          if (c2 < n_items) *dst_of(c2) = x2;
          if (c3 < n_items) *dst_of(c3) = x3;
        }
      };
      // K: row-major on both sides, 16-byte chunks
      constexpr int KC = D / 8;
      copy4(
          (n - i0) * KC,
          [&](int c) {
            return reinterpret_cast<const uint4 *>(
                k_row<bf16>(la.sk, bg, la.stage_rows_alloc, i0 + c / KC, D) + (c % KC) * 8);
          },
          [&](int c) {
            return reinterpret_cast<uint4 *>(
                k_row<bf16>(la.k, bg, la.rows_alloc, (Li + i0 + c / KC) % W, D) + (c % KC) * 8);
          });
      // V: 16-row blocks stored transposed on both sides.  When the kept rows
      // start a block on both sides (and W is whole blocks), each whole block
      // is one contiguous run of D x 16 elements; the rest goes element by
      // element.
      int iv = i0;
      if ((Li + i0) % kVBlock == 0 && i0 % kVBlock == 0 && W % kVBlock == 0) {
        constexpr int BC = D * kVBlock / 8;  // 16-byte chunks per block
        const int nb = (n - i0) / kVBlock;
        copy4(
            nb * BC,
            [&](int c) {
              return reinterpret_cast<const uint4 *>(
                  v_block<bf16>(la.sv, bg, la.stage_rows_alloc, i0 / kVBlock + c / BC, D) +
                  (c % BC) * 8);
            },
            [&](int c) {
              return reinterpret_cast<uint4 *>(
                  v_block<bf16>(la.v, bg, la.rows_alloc,
                                ((Li + i0) / kVBlock + c / BC) % (W / kVBlock), D) +
                  (c % BC) * 8);
            });
        iv = i0 + nb * kVBlock;
      }
      // (the rest: rows that do not start a block, element by element)
      const int nv = (n - iv) * D;
      for (int e = tid; e < nv; e += NT)
        *v_elem<bf16>(la.v, bg, la.rows_alloc, (Li + iv + e / D) % W, e % D, D) =
            *v_elem<bf16>(la.sv, bg, la.stage_rows_alloc, iv + e / D, e % D, D);
      if (tid == 0) __hip_atomic_store(pa.ring_cnt + bg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

bool fast_prefill_supported(int D, int rep) { return (D == 64 || D == 128) && rep >= 1; }

template <int D, int REP, int QW>
static int chunk_wgs_t() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_chunk<D, REP, false, QW>, QW * 64, 0) !=
      hipSuccess)
    return 0;
  return n;
}

int chunk_wgs_per_cu(int D, int rep, int qw) {
#define KVC_OCC(DD, RR)                                                              \
  if (D == DD && rep == RR) return qw == 4 ? chunk_wgs_t<DD, RR, 4>() : chunk_wgs_t<DD, RR, 8>();
  KVC_OCC(128, 1) KVC_OCC(128, 2) KVC_OCC(128, 4) KVC_OCC(128, 8) KVC_OCC(128, 16)
  KVC_OCC(64, 1) KVC_OCC(64, 2) KVC_OCC(64, 4) KVC_OCC(64, 8) KVC_OCC(64, 16)
#undef KVC_OCC
  return 0;
}

template <int D, int REP>
static void launch_chunk_t(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                           const void *q, int32_t n_items, int qw, const Launch &lc) {
  const dim3 grid((unsigned)n_items, (unsigned)la.hkv);
  if (qw == kChunkKeyHalves) {
    if (la.paged)
      launch_kernel((k_chunk<D, REP, true, 8, true>), grid, dim3(512), lc, st, la, pa,
                    (const bf16 *)q, la.table);
    else
      launch_kernel((k_chunk<D, REP, false, 8, true>), grid, dim3(512), lc, st, la, pa,
                    (const bf16 *)q, la.table);
  } else if (qw == 4) {
    if (la.paged)
      launch_kernel((k_chunk<D, REP, true, 4>), grid, dim3(256), lc, st, la, pa, (const bf16 *)q,
                    la.table);
    else
      launch_kernel((k_chunk<D, REP, false, 4>), grid, dim3(256), lc, st, la, pa, (const bf16 *)q,
                    la.table);
  } else if (la.paged) {
    launch_kernel((k_chunk<D, REP, true>), grid, dim3(512), lc, st, la, pa, (const bf16 *)q,
                  la.table);
  } else {
    launch_kernel((k_chunk<D, REP>), grid, dim3(512), lc, st, la, pa, (const bf16 *)q, la.table);
  }
}

int launch_prefill(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, const void *q,
                   int32_t n_items, int qw, const Launch &lc) {
#define KVC_CHK(DD, RR)                                         \
  if (st.D == DD && la.rep == RR) {                             \
    launch_chunk_t<DD, RR>(st, la, pa, q, n_items, qw, lc);     \
    return (int)hipGetLastError();                              \
  }
  KVC_CHK(128, 1) KVC_CHK(128, 2) KVC_CHK(128, 4) KVC_CHK(128, 8) KVC_CHK(128, 16)
  KVC_CHK(64, 1) KVC_CHK(64, 2) KVC_CHK(64, 4) KVC_CHK(64, 8) KVC_CHK(64, 16)
#undef KVC_CHK
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Split combine: one wave per output row (b, i, h).  Log-sum-exp merge of the
// split partials; padded queries and idle rows get exact zeros.  (Four rows
// per workgroup measured slower: 24.6 against 22.4 us on the mixed step's
// merges.)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_combine(StepArgs st, LayerArgs la, PartialArgs pa,
                                                T *__restrict__ out) {
  // (32-bit index and span arithmetic: rows, positions and split counts
  // stay far below 2^31, and a 64-bit division by a runtime value costs
  // hundreds of instructions)
  // (b * C + i) * Hq + h
  const int row = (int)blockIdx.x;
  const int h = row % st.Hq;
  const int bi = row / st.Hq;
  const int i = bi % st.C;
  const int b = bi / st.C;
  const int lane = threadIdx.x;
  const int D = st.D;
  T *o = out + (int64_t)row * D;
  // (the row's three counts in one round trip: the empty asm takes all
  // three, so none is sunk past the branch into a load of its own)
  const int n = st.n_new[b];
  const int L = st.lens[b];
  const int first = st.first[b];
  asm volatile("" ::"s"(n), "s"(L), "s"(first));
  if (i >= n) {
    for (int d = lane; d < D; d += 64) o[d] = from_f<T>(0.f);
    return;
  }
  // Splits of one layer for this row: the decode splits of a one-token
  // row's key span, or the key splits of a chunk row (one on a ring layer);
  // the spans of decode_span_dev and chunk_span_dev.
  auto splits = [&](int ring, int W, int dec_sk, int pre_sk) {
    if (n == 1) {
      int start = W > 0 ? (L - W + 1 > 0 ? L - W + 1 : 0) : 0;
      start = L < first ? L : (start > first ? start : first);
      const int base = ring ? 0 : start / kRowAlign * kRowAlign;
      const int hi = ring ? (L + 1 < W ? L + 1 : W) : L + 1;
      return (hi - base + dec_sk - 1) / dec_sk;
    }
    if (ring) return 1;
    int lo = W > 0 ? (L - W + 1 > 0 ? L - W + 1 : 0) : 0;
    const int f = first < L ? first : L;
    if (f > lo) lo = f;
    const int base = lo / kRowAlign * kRowAlign;
    return (L + n - base + pre_sk - 1) / pre_sk;
  };
  // a joint partner's splits follow the layer's own
  const int nj =
      pa.joint.on ? splits(pa.joint.ring, pa.joint.window, pa.joint.dec_sk, pa.joint.pre_sk) : 0;
  const float *ml;
  const float *os;
  const int ns =
      splits(la.ring, la.window, pa.dec_plan ? pa.dec_plan[0] : pa.dec_split_keys,
             pa.pre_split_keys) + nj;
  if (n == 1) {
    const int64_t s0 = ((int64_t)b * st.Hq + h) * kDecodeSplitCap;
    ml = pa.dml + s0 * 2;
    os = pa.dout + s0 * D;
  } else {
    const int64_t s0 = (((int64_t)b * pa.max_chunk + i) * st.Hq + h) * kChunkSplitCap;
    ml = pa.pml + s0 * 2;
    os = pa.pout + s0 * D;
  }
  // split weights 2^(m_s - M) / L (splits with no visible key have l == 0)
  if (D == 64 || D == 128) {
    // Every load of a merge of up to 8 splits goes out at once: this lane's
    // (m, l) and its D/64 consecutive elements of the first 8 splits (one
    // round trip instead of one per split and element); later splits load
    // 8 at a time.  The sums are those of the loop below, in its order.
    const int dpl = D / 64, d0 = lane * dpl;
    const float lsr = lane < ns ? ml[2 * lane + 1] : 0.f;
    const float msr = lane < ns ? ml[2 * lane] : 0.f;
    float x0[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        x0[u][e] = (u < ns && e < dpl) ? os[(int64_t)u * D + d0 + e] : 0.f;
    const float ms = (lane < ns && lsr > 0.f) ? msr : -INFINITY;
    const float M = wave_max(ms);
    const float w = lsr > 0.f ? exp2f(ms - M) : 0.f;
    const float Lt = wave_sum(w * lsr);
    // (split s's weight from lane s)
    const int wt = __builtin_bit_cast(int, w / Lt);
    auto wts = [&](int sp) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(wt, sp)); };
    float a[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int u = 0; u < 8; ++u) a[e][u] = 0.f;
    int s = 0;
    for (; s + 8 <= ns; s += 8) {
      float x[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          x[u][e] = s == 0 ? x0[u][e] : (e < dpl ? os[(int64_t)(s + u) * D + d0 + e] : 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = wts(s + u);
#pragma unroll
        for (int e = 0; e < 2; ++e) a[e][u] = combine_acc(a[e][u], wu, x[u][e]);
      }
    }
    if (s < ns) {  // the last ns % 8 splits, summed in order into slot 0
      float x[8][2];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          x[u][e] = s == 0 ? x0[u][e]
                           : ((s + u < ns && e < dpl) ? os[(int64_t)(s + u) * D + d0 + e] : 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s + u < ns) {
          const float wu = wts(s + u);
#pragma unroll
          for (int e = 0; e < 2; ++e) a[e][0] = combine_acc(a[e][0], wu, x[u][e]);
        }
      }
    }
    for (int e = 0; e < dpl; ++e) o[d0 + e] = from_f<T>(combine_tree(a[e]));
    return;
  }
  const float ls = lane < ns ? ml[2 * lane + 1] : 0.f;
  const float ms = (lane < ns && ls > 0.f) ? ml[2 * lane] : -INFINITY;
  const float M = wave_max(ms);
  const float w = ls > 0.f ? exp2f(ms - M) : 0.f;
  const float Lt = wave_sum(w * ls);
  const int wt = __builtin_bit_cast(int, w / Lt);
  auto wts = [&](int sp) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(wt, sp)); };
  for (int d = lane; d < D; d += 64) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= ns; s += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = wts(s + u);
        const float x = os[(int64_t)(s + u) * D + d];
        a[u] = combine_acc(a[u], w, x);  // splits without keys: slot never written
      }
    }
    for (; s < ns; ++s) {
      const float w = wts(s);
      const float x = os[(int64_t)s * D + d];
      a[0] = combine_acc(a[0], w, x);
    }
    o[d] = from_f<T>(combine_tree(a));
  }
}

int launch_combine(int dtype, const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                   void *out, const Launch &lc) {
  const int64_t rows = (int64_t)st.B * st.C * st.Hq;
  if (dtype == KVC_F32)
    launch_kernel(k_combine<float>, dim3((unsigned)rows), dim3(64), lc, st, la, pa, (float *)out);
  else
    launch_kernel(k_combine<bf16>, dim3((unsigned)rows), dim3(64), lc, st, la, pa, (bf16 *)out);
  return (int)hipGetLastError();
}

}  // namespace kvc
