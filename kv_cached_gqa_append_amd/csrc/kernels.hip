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
#include <hip/hip_runtime.h>

#include <cstring>

#include "kvc_internal.h"

namespace kvc {

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

// Reduce across groups: input uniform within aligned groups of G lanes; the
// result is the reduction over the whole wave, in every lane.
template <int G>
__device__ __forceinline__ float across_groups_max(float x) {
  if (G <= 4) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if (G <= 8) x = fmaxf(x, dpp<kRowMirror>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
template <int G>
__device__ __forceinline__ float across_groups_sum(float x) {
  if (G <= 4) x += dpp<kRowHalfMirror>(x);
  if (G <= 8) x += dpp<kRowMirror>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
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

// Position held by ring slot s before this step's commit, L = tokens so far:
// the latest t < L with t % W == s (negative: the slot is empty).
__device__ __forceinline__ int64_t ring_slot_pos(int64_t s, int64_t L, int W) {
  const int64_t r = L % W;
  return s < r ? (L - r + s) : (L - r - W + s);
}

// Decode key span in storage rows (identical to the host planner).
__device__ __forceinline__ void decode_span_dev(const LayerArgs &la, int64_t p, int64_t *base,
                                                int64_t *lo, int64_t *hi) {
  if (la.ring) {
    *lo = 0;
    *hi = p + 1 < la.window ? p + 1 : la.window;
  } else {
    *lo = la.window > 0 ? (p - la.window + 1 > 0 ? p - la.window + 1 : 0) : 0;
    *hi = p + 1;
  }
  *base = *lo / kVBlock * kVBlock;
}
__device__ __forceinline__ void chunk_span_dev(const LayerArgs &la, int64_t L, int64_t n,
                                               int64_t *base, int64_t *lo, int64_t *hi) {
  *lo = la.window > 0 ? (L - la.window + 1 > 0 ? L - la.window + 1 : 0) : 0;
  *hi = L + n;
  *base = *lo / kRowAlign * kRowAlign;
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

__global__ void k_reset_rows(int32_t *lens, I32Chunk rows, int32_t n) {
  const int i = threadIdx.x;
  if (i < n) lens[rows.v[i]] = 0;
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

int launch_reset_rows(int32_t *lens, const int32_t *rows, int32_t n, void *stream) {
  for (int32_t off = 0; off < n; off += 256) {
    I32Chunk c;
    const int32_t m = n - off < 256 ? n - off : 256;
    std::memset(&c, 0, sizeof(c));
    std::memcpy(c.v, rows + off, sizeof(int32_t) * m);
    hipLaunchKernelGGL(k_reset_rows, dim3(1), dim3(256), 0, (hipStream_t)stream, lens, c, m);
  }
  return (int)hipGetLastError();
}

int launch_advance(int32_t *lens, const int32_t *n_new, int32_t B, void *stream) {
  const int blocks = (int)cdiv(B, 256);
  hipLaunchKernelGGL(k_advance, dim3(blocks), dim3(256), 0, (hipStream_t)stream, lens, n_new, B);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// fused RoPE + append: one wave per (row b, token i, KV head g)
// ---------------------------------------------------------------------------
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
  int64_t r;
  char *kreg, *vreg;
  int ralloc;
  if (staged) {
    if (!valid) return;  // staging rows of padding are never read
    r = i;
    kreg = la.sk;
    vreg = la.sv;
    ralloc = la.stage_rows_alloc;
  } else {
    if (la.ring)
      r = valid ? p % la.window : la.window;
    else
      r = valid ? p : la.rows;
    kreg = la.k;
    vreg = la.v;
    ralloc = la.rows_alloc;
  }
  const int64_t bg = (int64_t)b * la.hkv + g;
  T *kd = k_row<T>(kreg, bg, ralloc, r, D);
  T *vd = v_elem<T>(vreg, bg, ralloc, r, 0, D);
  const T *ks = k + row * D;
  const T *vs = v + row * D;
  const bool rot = st.rope != nullptr && valid;
  for (int e = threadIdx.x; e < half; e += 64) {
    const float x1 = to_f(ks[e]), x2 = to_f(ks[e + half]);
    float y1 = x1, y2 = x2;
    if (rot) {
      const float c = st.rope[(p * half + e) * 2 + 0];
      const float s = st.rope[(p * half + e) * 2 + 1];
      y1 = x1 * c - x2 * s;
      y2 = x1 * s + x2 * c;
    }
    kd[e] = from_f<T>(y1);
    kd[e + half] = from_f<T>(y2);
    vd[e * kVBlock] = vs[e];
    vd[(e + half) * kVBlock] = vs[e + half];
  }
}

int launch_append(int dtype, const StepArgs &st, const LayerArgs &la, const void *k,
                  const void *v, int32_t *slot_out, void *stream) {
  const int64_t rows = (int64_t)st.B * st.C * la.hkv;
  if (dtype == KVC_F32)
    hipLaunchKernelGGL(k_append<float>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream,
                       st, la, (const float *)k, (const float *)v, slot_out);
  else
    hipLaunchKernelGGL(k_append<bf16>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream, st,
                       la, (const bf16 *)k, (const bf16 *)v, slot_out);
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

int launch_commit(int dtype, const StepArgs &st, const LayerArgs &la, void *stream) {
  const int64_t rows = (int64_t)st.B * st.C * la.hkv;
  if (dtype == KVC_F32)
    hipLaunchKernelGGL(k_commit<float>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream,
                       st, la);
  else
    hipLaunchKernelGGL(k_commit<bf16>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream, st,
                       la);
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
__global__ __launch_bounds__(64) void k_generic(StepArgs st, LayerArgs la, const T *__restrict__ q,
                                                T *__restrict__ out) {
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
  if (la.ring && n >= 2 && la.sk) {
    // history from the ring (slots holding positions within the window) ...
    const int64_t nh = L < W ? L : W;
    for (int64_t s = 0; s < nh; ++s) {
      const int64_t pos = ring_slot_pos(s, L, W);
      if (pos < 0 || p - pos >= W) continue;
      generic_key(S, k_row<T>(la.k, bg, la.rows_alloc, s, D),
                  v_elem<T>(la.v, bg, la.rows_alloc, s, 0, D), D, scale);
    }
    // ... and the chunk's own rows from staging
    for (int j = 0; j <= i; ++j) {
      if (i - j >= W) continue;
      generic_key(S, k_row<T>(la.sk, bg, la.stage_rows_alloc, j, D),
                  v_elem<T>(la.sv, bg, la.stage_rows_alloc, j, 0, D), D, scale);
    }
  } else if (la.ring) {
    // one-token step: the visible positions fill slots [0, min(p + 1, W))
    const int64_t hi = p + 1 < W ? p + 1 : W;
    for (int64_t s = 0; s < hi; ++s)
      generic_key(S, k_row<T>(la.k, bg, la.rows_alloc, s, D),
                  v_elem<T>(la.v, bg, la.rows_alloc, s, 0, D), D, scale);
  } else {
    const int64_t lo = W > 0 ? (p - W + 1 > 0 ? p - W + 1 : 0) : 0;
    for (int64_t t = lo; t <= p; ++t)
      generic_key(S, k_row<T>(la.k, bg, la.rows_alloc, t, D),
                  v_elem<T>(la.v, bg, la.rows_alloc, t, 0, D), D, scale);
  }
  const float inv = 1.f / S.l;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int d = lane + 64 * t;
    if (d < D) o[d] = from_f<T>(S.acc[t] * inv);
  }
}

int launch_generic(int dtype, const StepArgs &st, const LayerArgs &la, const void *q, void *out,
                   void *stream) {
  const int64_t rows = (int64_t)st.B * st.C * st.Hq;
  if (dtype == KVC_F32)
    hipLaunchKernelGGL(k_generic<float>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream,
                       st, la, (const float *)q, (float *)out);
  else
    hipLaunchKernelGGL(k_generic<bf16>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream,
                       st, la, (const bf16 *)q, (bf16 *)out);
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
  int64_t rem = it;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int c = b < B ? count(b) : 0;
    const int incl = wave_incl_scan(c);
    const int total = __shfl(incl, 63);
    if (rem < total) {
      const int excl = incl - c;
      const bool mine = rem >= excl && rem < incl;
      const uint64_t ball = __ballot(mine);
      const int src = __ffsll((unsigned long long)ball) - 1;
      *row_out = b0 + src;
      *local_out = rem - __shfl(excl, src);
      return;
    }
    rem -= total;
  }
  *row_out = -1;
  *local_out = 0;
}

// ---------------------------------------------------------------------------
// Decode attention (rows with one new token), bf16.  One wave per
// (row, KV head, key split).  QK: LK lanes per key, each holding D/LK
// elements of all REP rotated queries in registers; scores reduced with DPP.
// PV: each lane owns D/32 head-dim elements for 8 of the 16 keys of a V block
// and accumulates with bf16 dot2 over key pairs.  Online softmax in the exp2
// domain with one running max per query head; partials (m, l, o) per split.
// ---------------------------------------------------------------------------
template <int D, int REP>
struct DecodeShape {
  static constexpr int LK0 = REP * D / 128;
  static constexpr int LK = LK0 > 4 ? LK0 : 4;   // lanes per key (QK)
  static constexpr int KR = 64 / LK;             // keys per QK round
  static constexpr int NR = 16 / KR;             // rounds per 16-key tile
  static constexpr int NCH = D / 8 / LK;         // 16-byte chunks per lane
  static constexpr int VT = D / 32;              // V head-dim rows per lane
  static_assert(LK <= 16 && NCH >= 1, "unsupported decode shape");
};

template <int D, int REP>
__global__ __launch_bounds__(64) void k_decode(StepArgs st, LayerArgs la, PartialArgs pa,
                                               const bf16 *__restrict__ q) {
  using S = DecodeShape<D, REP>;
  constexpr int LK = S::LK, KR = S::KR, NR = S::NR, NCH = S::NCH, VT = S::VT;
  __shared__ float qs[REP * D];
  __shared__ __align__(16) uint16_t pls[2][REP][16];

  const int lane = threadIdx.x;
  const int g = blockIdx.y;
  const int SK = pa.dec_split_keys;
  int b;
  int64_t split;
  find_item(
      st.B, blockIdx.x,
      [&](int r) -> int {
        if (st.n_new[r] != 1) return 0;
        int64_t base, lo, hi;
        decode_span_dev(la, st.lens[r], &base, &lo, &hi);
        return (int)cdiv(hi - base, SK);
      },
      &b, &split);
  if (b < 0) return;
  const int64_t p = st.lens[b];
  int64_t base, lo, hi;
  decode_span_dev(la, p, &base, &lo, &hi);
  const int64_t t_begin = base + split * SK;
  const int64_t t_end = t_begin + SK < hi ? t_begin + SK : hi;
  const int64_t bg = (int64_t)b * la.hkv + g;

  // -- queries: load REP heads, rotate at p, keep as bf16 pairs ----------------
  const int h0 = g * REP;
  const bf16 *qsrc = q + ((int64_t)b * st.C * st.Hq + h0) * D;  // token 0 of row b
  for (int e = lane; e < REP * D; e += 64) qs[e] = (float)qsrc[e];
  __syncthreads();
  const int kr = lane / LK, j = lane % LK;
  uint32_t qp[REP][NCH][4];
#pragma unroll
  for (int h = 0; h < REP; ++h)
#pragma unroll
    for (int t = 0; t < NCH; ++t)
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int d = (j + LK * t) * 8 + 2 * e2 + u;
          const float x = qs[h * D + d];
          if (st.rope) {
            const int dd = d < D / 2 ? d : d - D / 2;
            const float c = st.rope[(p * (D / 2) + dd) * 2 + 0];
            const float sn = st.rope[(p * (D / 2) + dd) * 2 + 1];
            y[u] = d < D / 2 ? x * c - qs[h * D + d + D / 2] * sn
                             : qs[h * D + d - D / 2] * sn + x * c;
          } else {
            y[u] = x;
          }
        }
        qp[h][t][e2] = pack_bf16(y[0], y[1]);
      }

  const float scale = kLog2e * rsqrtf((float)D);
  float m[REP], lsum[REP], acc[REP][VT];
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int t = 0; t < VT; ++t) acc[h][t] = 0.f;
  }
  const int half = lane >> 5, mm = lane & 31;
  const bf16 *kbase = reinterpret_cast<const bf16 *>(la.k) + (bg * la.rows_alloc) * D;

  int par = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 16, par ^= 1) {
    // ---- loads: K rows of this lane's keys, V block d-rows of this lane ----
    uint4 kv[NR][NCH];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const bf16 *kr_ptr = kbase + (t0 + r * KR + kr) * D;
#pragma unroll
      for (int t = 0; t < NCH; ++t)
        kv[r][t] = *reinterpret_cast<const uint4 *>(kr_ptr + (j + LK * t) * 8);
    }
    const bf16 *vb = v_block<bf16>(la.v, bg, la.rows_alloc, t0 / kVBlock, D);
    uint4 vv[VT];
#pragma unroll
    for (int t = 0; t < VT; ++t)
      vv[t] = *reinterpret_cast<const uint4 *>(vb + (mm + 32 * t) * kVBlock + half * 8);

    // ---- scores ----
    float s[NR][REP];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int64_t key = t0 + r * KR + kr;
      const bool ok = key >= lo && key < hi;
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        float a = 0.f;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
          a = dot2_bf16(qp[h][t][0], kv[r][t].x, a);
          a = dot2_bf16(qp[h][t][1], kv[r][t].y, a);
          a = dot2_bf16(qp[h][t][2], kv[r][t].z, a);
          a = dot2_bf16(qp[h][t][3], kv[r][t].w, a);
        }
        a = group_sum<LK>(a);
        s[r][h] = ok ? a * scale : -INFINITY;
      }
    }
    // ---- online softmax (one running max per head, uniform over the wave) ----
    float alpha[REP];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      float tm = s[0][h];
#pragma unroll
      for (int r = 1; r < NR; ++r) tm = fmaxf(tm, s[r][h]);
      tm = across_groups_max<LK>(tm);
      const float mn = fmaxf(m[h], tm);
      alpha[h] = exp2f(m[h] - mn);
      rescale |= (mn != m[h]);
      m[h] = mn;
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float pe = exp2f(s[r][h] - mn);
        ps += pe;
        if (j == 0) {
          bf16 pb = (bf16)pe;
          pls[par][h][r * KR + kr] = __builtin_bit_cast(uint16_t, pb);
        }
      }
      lsum[h] = lsum[h] * alpha[h] + ps;
    }
    __syncthreads();
    // ---- zero V of keys outside [lo, hi) on edge tiles (stale rows may hold
    //      anything, and 0 * NaN would leak) ----
    if (t0 < lo || t0 + 16 > hi) {
      uint32_t keep[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int64_t k0 = t0 + half * 8 + 2 * e2;
        keep[e2] = ((k0 >= lo && k0 < hi) ? 0x0000ffffu : 0u) |
                   ((k0 + 1 >= lo && k0 + 1 < hi) ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        vv[t].x &= keep[0];
        vv[t].y &= keep[1];
        vv[t].z &= keep[2];
        vv[t].w &= keep[3];
      }
    }
    // ---- P.V ----
    if (__builtin_expect(rescale, 0)) {
#pragma unroll
      for (int h = 0; h < REP; ++h)
#pragma unroll
        for (int t = 0; t < VT; ++t) acc[h][t] *= alpha[h];
    }
#pragma unroll
    for (int h = 0; h < REP; ++h) {
      const uint4 pp = *reinterpret_cast<const uint4 *>(&pls[par][h][half * 8]);
#pragma unroll
      for (int t = 0; t < VT; ++t) {
        float a = acc[h][t];
        a = dot2_bf16(vv[t].x, pp.x, a);
        a = dot2_bf16(vv[t].y, pp.y, a);
        a = dot2_bf16(vv[t].z, pp.z, a);
        a = dot2_bf16(vv[t].w, pp.w, a);
        acc[h][t] = a;
      }
    }
  }

  // ---- partials: (m, l) and unnormalised o for this split ----
  const int64_t cap = kDecodeSplitCap;
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    const float l = across_groups_sum<LK>(lsum[h]);
    const int64_t slot = ((int64_t)b * st.Hq + h0 + h) * cap + split;
    if (lane == 0) {
      pa.dml[slot * 2 + 0] = m[h];
      pa.dml[slot * 2 + 1] = l;
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      const float o = acc[h][t] + __shfl_xor(acc[h][t], 32);
      if (half == 0) pa.dout[slot * D + mm + 32 * t] = o;
    }
  }
}

bool fast_decode_supported(int D, int rep) {
  return (D == 64 || D == 128) && (rep == 1 || rep == 2 || rep == 4 || rep == 8 || rep == 16);
}

template <int D, int REP>
static void launch_decode_t(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                            const void *q, int32_t n_items, void *stream) {
  hipLaunchKernelGGL((k_decode<D, REP>), dim3((unsigned)n_items, (unsigned)la.hkv), dim3(64), 0,
                     (hipStream_t)stream, st, la, pa, (const bf16 *)q);
}

int launch_decode(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, const void *q,
                  int32_t n_items, void *stream) {
#define KVC_DEC(DD, RR)                                         \
  if (st.D == DD && la.rep == RR) {                             \
    launch_decode_t<DD, RR>(st, la, pa, q, n_items, stream);    \
    return (int)hipGetLastError();                              \
  }
  KVC_DEC(128, 1) KVC_DEC(128, 2) KVC_DEC(128, 4) KVC_DEC(128, 8) KVC_DEC(128, 16)
  KVC_DEC(64, 1) KVC_DEC(64, 2) KVC_DEC(64, 4) KVC_DEC(64, 8) KVC_DEC(64, 16)
#undef KVC_DEC
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Chunk attention (rows with two or more new tokens), bf16, MFMA.
// Workgroup = 4 waves = 64 query rows of one (row b, KV head g); query row
// r = i * REP + hl (token-major).  Key tiles of 32 rows are staged in LDS:
// K row-major (padded rows), V as two transposed 16-row blocks.  Per wave:
//   S^T (32 keys x 16 queries) = K . Q^T   with v_mfma_f32_16x16x32_bf16
//   O^T (D x 16 queries)     += V^T . P^T  with the same instruction,
// so the score accumulator already has the layout P^T needs as an operand.
// Mask per (key, query) only matters on edge tiles but is applied uniformly.
// ---------------------------------------------------------------------------
template <int D>
struct ChunkLds {
  static constexpr int KSTR = D + 8;                 // padded K row (elements)
  bf16 k[32 * KSTR];
  bf16 v[2 * D * kVBlock];
};

struct KeySeg {
  const char *kreg, *vreg;  // region bases
  int ralloc;               // rows per head in the region
  int64_t first, end;       // storage rows [first, end) to visit (first % 32 == 0)
  int64_t vlo, vhi;         // rows holding data of this sequence
  int kind;                 // 0: position = row; 1: ring history; 2: staging (pos = L + row)
};

template <int D>
__device__ __forceinline__ void chunk_load_tile(ChunkLds<D> &lds, const KeySeg &sg, int64_t bg,
                                                int64_t t0) {
  const int tid = threadIdx.x;
  constexpr int KCH = 32 * D / 8;        // 16-byte chunks of the K tile
  constexpr int VCH = 2 * D * kVBlock / 8;
  const bf16 *ksrc = reinterpret_cast<const bf16 *>(sg.kreg) + (bg * sg.ralloc + t0) * D;
  for (int c = tid; c < KCH; c += 256) {
    const int rr = c / (D / 8), cc = c % (D / 8);
    const uint4 x = *reinterpret_cast<const uint4 *>(ksrc + rr * D + cc * 8);
    *reinterpret_cast<uint4 *>(&lds.k[rr * ChunkLds<D>::KSTR + cc * 8]) = x;
  }
  const bf16 *vsrc = reinterpret_cast<const bf16 *>(sg.vreg) +
                     ((bg * (sg.ralloc / kVBlock) + t0 / kVBlock) * D) * kVBlock;
  const bool edge = t0 < sg.vlo || t0 + 32 > sg.vhi;
  for (int c = tid; c < VCH; c += 256) {
    uint4 x = *reinterpret_cast<const uint4 *>(vsrc + c * 8);
    if (edge) {
      // chunk c covers rows (c / (2D)) * 16 + (c % 2) * 8 + 0..7 of the tile
      const int64_t r0 = t0 + (c / (2 * D)) * 16 + (c % 2) * 8;
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int64_t ra = r0 + 2 * e2, rb = ra + 1;
        const uint32_t keep = ((ra >= sg.vlo && ra < sg.vhi) ? 0x0000ffffu : 0u) |
                              ((rb >= sg.vlo && rb < sg.vhi) ? 0xffff0000u : 0u);
        w[e2] &= keep;
      }
      x = make_uint4(w[0], w[1], w[2], w[3]);
    }
    *reinterpret_cast<uint4 *>(&lds.v[c * 8]) = x;
  }
}

template <int D, int REP>
__global__ __launch_bounds__(256) void k_chunk(StepArgs st, LayerArgs la, PartialArgs pa,
                                               const bf16 *__restrict__ q) {
  __shared__ ChunkLds<D> lds;
  constexpr int NDS = D / 32;  // 32-wide d steps (QK contraction)
  constexpr int NDB = D / 16;  // 16-wide d blocks (PV output)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
        const int nqt = (int)cdiv((int64_t)n * REP, kChunkQTile);
        if (la.ring) return nqt;
        int64_t base, lo, hi;
        chunk_span_dev(la, st.lens[r], n, &base, &lo, &hi);
        return nqt * (int)cdiv(hi - base, SKP);
      },
      &b, &local);
  if (b < 0) return;
  const int64_t L = st.lens[b];
  const int n = st.n_new[b];
  int nks = 1;
  int64_t cbase = 0, clo = 0, chi = 0;
  if (!la.ring) {
    chunk_span_dev(la, L, n, &cbase, &clo, &chi);
    nks = (int)cdiv(chi - cbase, SKP);
  }
  const int qt = (int)(local / nks), ks = (int)(local % nks);
  const int64_t bg = (int64_t)b * la.hkv + g;
  const int W = la.window;

  // -- this wave's 16 query rows; lane (q4, nl) holds query row nl ------------
  const int r = qt * kChunkQTile + wave * 16 + nl;
  const bool rvalid = r < n * REP;
  const int qi = r / REP, hl = r % REP;
  const int64_t qpos = L + qi;
  bf16x8_t qf[NDS];
  {
    float raw[NDS][8];
    const bf16 *qsrc = q + (((int64_t)b * st.C + qi) * st.Hq + g * REP + hl) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (rvalid) {
        const uint4 x = *reinterpret_cast<const uint4 *>(qsrc + ds * 32 + q4 * 8);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          raw[ds][2 * e2] = bf_lo(w[e2]);
          raw[ds][2 * e2 + 1] = bf_hi(w[e2]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) raw[ds][e] = 0.f;
      }
    }
    if (st.rope && rvalid) {
      constexpr int HS = NDS / 2;  // partner d + D/2 sits HS steps later
#pragma unroll
      for (int ds = 0; ds < HS; ++ds)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = ds * 32 + q4 * 8 + e;
          const float c = st.rope[(qpos * (D / 2) + d) * 2 + 0];
          const float sn = st.rope[(qpos * (D / 2) + d) * 2 + 1];
          const float x1 = raw[ds][e], x2 = raw[ds + HS][e];
          raw[ds][e] = x1 * c - x2 * sn;
          raw[ds + HS][e] = x1 * sn + x2 * c;
        }
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ds][e] = (bf16)raw[ds][e];
  }

  // -- key segments -------------------------------------------------------------
  // Positions of the whole q-tile span [pmin, pmax].
  const int rlast = (qt + 1) * kChunkQTile - 1 < n * REP - 1 ? (qt + 1) * kChunkQTile - 1
                                                              : n * REP - 1;
  const int64_t pmin = L + (int64_t)(qt * kChunkQTile) / REP;
  const int64_t pmax = L + rlast / REP;
  KeySeg seg0{}, seg1{};
  bool has0 = false, has1 = false;
  if (!la.ring) {
    seg0.kreg = la.k;
    seg0.vreg = la.v;
    seg0.ralloc = la.rows_alloc;
    int64_t a = cbase + (int64_t)ks * SKP;
    int64_t e = a + SKP < chi ? a + SKP : chi;
    if (e > pmax + 1) e = pmax + 1;
    if (W > 0) {
      const int64_t wlo = (pmin - W + 1) / 32 * 32;
      if (a < wlo) a = wlo;
    }
    seg0.first = a;
    seg0.end = e;
    seg0.vlo = clo;
    seg0.vhi = chi;
    seg0.kind = 0;
    has0 = seg0.first < seg0.end;
  } else {
    const int64_t nh = L < W ? L : W;
    seg0.kreg = la.k;
    seg0.vreg = la.v;
    seg0.ralloc = la.rows_alloc;
    seg0.first = 0;
    seg0.end = nh;
    seg0.vlo = 0;
    seg0.vhi = nh;
    seg0.kind = 1;
    has0 = nh > 0;
    seg1.kreg = la.sk;
    seg1.vreg = la.sv;
    seg1.ralloc = la.stage_rows_alloc;
    seg1.first = 0;
    seg1.end = n;
    seg1.vlo = 0;
    seg1.vhi = n;
    seg1.kind = 2;
    has1 = true;
  }

  const float scale = kLog2e * rsqrtf((float)D);
  float mrun = -INFINITY, lrun = 0.f;
  floatx4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto run_segment = [&](const KeySeg &sg) {
    for (int64_t t0 = sg.first; t0 < sg.end; t0 += 32) {
      __syncthreads();
      chunk_load_tile<D>(lds, sg, bg, t0);
      __syncthreads();
      // S^T = K Q^T
      floatx4 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(
              &lds.k[(kb * 16 + nl) * ChunkLds<D>::KSTR + ds * 32 + q4 * 8]);
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ds], sacc[kb], 0, 0, 0);
        }
      }
      // mask + scale; sacc[kb][jj] is key row t0 + kb*16 + 4*q4 + jj, query nl
      float sv[2][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int64_t t = t0 + kb * 16 + q4 * 4 + jj;
          int64_t pos;
          if (sg.kind == 0)
            pos = t;
          else if (sg.kind == 1)
            pos = ring_slot_pos(t, L, W);
          else
            pos = L + t;
          bool ok = rvalid && t >= sg.vlo && t < sg.vhi && pos >= 0 && pos <= qpos;
          if (W > 0) ok = ok && (qpos - pos < W);
          const float x = ok ? sacc[kb][jj] * scale : -INFINITY;
          sv[kb][jj] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(mrun, tmax);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(mrun - mu);
      bf16x8_t pf;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float pe = exp2f(sv[kb][jj] - mu);
          ps += pe;
          pf[kb * 4 + jj] = (bf16)pe;
        }
      lrun = lrun * alpha + ps;
      mrun = mn;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      // O^T += V^T P^T; k-slot 8*q4 + e <-> key (e < 4 ? 4*q4 + e : 16 + 4*q4 + e - 4)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + nl;
        const uint2 lo8 = *reinterpret_cast<const uint2 *>(&lds.v[(0 * D + d) * kVBlock + q4 * 4]);
        const uint2 hi8 = *reinterpret_cast<const uint2 *>(&lds.v[(1 * D + d) * kVBlock + q4 * 4]);
        const uint4 av = make_uint4(lo8.x, lo8.y, hi8.x, hi8.y);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), pf,
                                                           oacc[db], 0, 0, 0);
      }
    }
  };
  if (has0) run_segment(seg0);
  if (has1) run_segment(seg1);

  // -- partials for this split ---------------------------------------------------
  float lt = lrun + __shfl_xor(lrun, 16);
  lt += __shfl_xor(lt, 32);
  if (rvalid) {
    const int64_t slot = (((int64_t)b * pa.max_chunk + qi) * st.Hq + g * REP + hl) * kChunkSplitCap + ks;
    if (q4 == 0) {
      pa.pml[slot * 2 + 0] = lt > 0.f ? mrun : -INFINITY;
      pa.pml[slot * 2 + 1] = lt;
    }
    if (lt > 0.f) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pa.pout[slot * D + db * 16 + q4 * 4 + jj] = oacc[db][jj];
    }
  }
}

bool fast_prefill_supported(int D, int rep) { return (D == 64 || D == 128) && rep >= 1; }

template <int D, int REP>
static void launch_chunk_t(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                           const void *q, int32_t n_items, void *stream) {
  hipLaunchKernelGGL((k_chunk<D, REP>), dim3((unsigned)n_items, (unsigned)la.hkv), dim3(256), 0,
                     (hipStream_t)stream, st, la, pa, (const bf16 *)q);
}

int launch_prefill(const StepArgs &st, const LayerArgs &la, const PartialArgs &pa, const void *q,
                   int32_t n_items, void *stream) {
#define KVC_CHK(DD, RR)                                         \
  if (st.D == DD && la.rep == RR) {                             \
    launch_chunk_t<DD, RR>(st, la, pa, q, n_items, stream);     \
    return (int)hipGetLastError();                              \
  }
  KVC_CHK(128, 1) KVC_CHK(128, 2) KVC_CHK(128, 4) KVC_CHK(128, 8) KVC_CHK(128, 16)
  KVC_CHK(64, 1) KVC_CHK(64, 2) KVC_CHK(64, 4) KVC_CHK(64, 8) KVC_CHK(64, 16)
#undef KVC_CHK
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Split combine: one wave per output row (b, i, h).  Log-sum-exp merge of the
// split partials; padded queries and idle rows get exact zeros.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void k_combine(StepArgs st, LayerArgs la, PartialArgs pa,
                                                T *__restrict__ out) {
  const int64_t row = blockIdx.x;  // (b * C + i) * Hq + h
  const int h = (int)(row % st.Hq);
  const int64_t bi = row / st.Hq;
  const int i = (int)(bi % st.C);
  const int b = (int)(bi / st.C);
  const int lane = threadIdx.x;
  const int D = st.D;
  T *o = out + row * D;
  const int n = st.n_new[b];
  if (i >= n) {
    for (int d = lane; d < D; d += 64) o[d] = from_f<T>(0.f);
    return;
  }
  const int64_t L = st.lens[b];
  const float *ml;
  const float *os;
  int ns;
  if (n == 1) {
    int64_t base, lo, hi;
    decode_span_dev(la, L, &base, &lo, &hi);
    ns = (int)cdiv(hi - base, pa.dec_split_keys);
    const int64_t s0 = ((int64_t)b * st.Hq + h) * kDecodeSplitCap;
    ml = pa.dml + s0 * 2;
    os = pa.dout + s0 * D;
  } else {
    ns = 1;
    if (!la.ring) {
      int64_t base, lo, hi;
      chunk_span_dev(la, L, n, &base, &lo, &hi);
      ns = (int)cdiv(hi - base, pa.pre_split_keys);
    }
    const int64_t s0 = (((int64_t)b * pa.max_chunk + i) * st.Hq + h) * kChunkSplitCap;
    ml = pa.pml + s0 * 2;
    os = pa.pout + s0 * D;
  }
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) {
    if (ml[2 * s + 1] > 0.f) mx = fmaxf(mx, ml[2 * s]);
  }
  mx = wave_max(mx);
  float lt = 0.f;
  for (int s = lane; s < ns; s += 64) {
    const float l = ml[2 * s + 1];
    if (l > 0.f) lt += l * exp2f(ml[2 * s] - mx);
  }
  lt = wave_sum(lt);
  const float inv = 1.f / lt;
  for (int d = lane; d < D; d += 64) {
    float a = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float l = ml[2 * s + 1];
      if (l > 0.f) a += os[(int64_t)s * D + d] * exp2f(ml[2 * s] - mx);
    }
    o[d] = from_f<T>(a * inv);
  }
}

int launch_combine(int dtype, const StepArgs &st, const LayerArgs &la, const PartialArgs &pa,
                   void *out, void *stream) {
  const int64_t rows = (int64_t)st.B * st.C * st.Hq;
  if (dtype == KVC_F32)
    hipLaunchKernelGGL(k_combine<float>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream,
                       st, la, pa, (float *)out);
  else
    hipLaunchKernelGGL(k_combine<bf16>, dim3((unsigned)rows), dim3(64), 0, (hipStream_t)stream,
                       st, la, pa, (bf16 *)out);
  return (int)hipGetLastError();
}

}  // namespace kvc
