/*
 * kvc.h - cached GQA attention with append on AMD Instinct MI355X (gfx950).
 *
 * One handle holds the per-layer key/value cache of B rows (sequences).  Each
 * row has its own length.  A step appends a right-padded chunk of new tokens
 * to every layer and attends the chunk's queries against the cache:
 *
 *     for each layer l:  kvc_append(h, l, k, v, n_new, C, ...);
 *                        kvc_attend(h, l, q, out, ...);
 *     kvc_advance(h, ...);                  (once, after every layer)
 *
 * Sources for the operation (page titles and sections of the study pages):
 *   - tiny_agent "generate.py": KVCache (global cache with a scratch slot,
 *     sliding rings with a scratch slot, per-row lengths mirrored on the host),
 *     _rope_pos (RoPE at per-row absolute positions), append (host-side
 *     capacity check, right-padded chunks), _append_chunk (slot addressing,
 *     grouped-query attention straight against the cache, float32 softmax).
 *   - tinyllm "kv_cache.py": the begin/update/end step protocol; per-slot
 *     lengths with a device copy and a host copy.
 *   - pycraft-1 "model/kv_cache.py": preallocated pre-expansion cache of
 *     post-RoPE keys; update() does not advance, advance() runs once after all
 *     layers; overflow / dtype / batch guards; reset without zeroing; the
 *     bottom-right aligned mask (build_attn_mask).
 *   - colibri PR "inkling: ring-buffer KV cache for sliding-window layers":
 *     "What this does" (W-key clamp), "How it works" (ring iff 0 < W < max_len;
 *     score the chunk from its own new rows and append after scoring; keep
 *     only the last W rows of a chunk; fail-fast bound check).
 *   - "Lab 07 - KV cache and sampling": section 1 (bytes per token), section 2
 *     (the offset mask: query i at pos+i sees key j iff j <= pos+i), section 3
 *     (chunked prefill equals one prefill).
 *
 * Conventions for every call
 *   - Device memory is owned by the caller.  The library never allocates
 *     device memory and never synchronises the host with the device inside a
 *     step.  All device pointers must be 16-byte aligned and contiguous.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it; all calls of one step must be on one stream (or ordered).
 *   - Every check happens on the host before anything is enqueued: a call
 *     that returns an error has changed nothing.  The one exception is
 *     KVC_E_HIP, the runtime refusing a launch or call part way: work the
 *     call enqueued before it stays enqueued (a forked side stream is still
 *     joined back) and the step cannot be completed; treat it as fatal for
 *     the handle.  Asynchronous device faults surface at the caller's next
 *     synchronisation, not here.
 *   - A handle is not thread-safe.
 *   - Integer status codes: KVC_OK (0) or a negative KVC_E_* value.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvc_cache kvc_t;

enum {
  KVC_OK = 0,
  KVC_E_ARG = -1,     /* bad argument or unsupported shape                    */
  KVC_E_FULL = -2,    /* "KV cache full": some row would pass max_len         */
  KVC_E_DTYPE = -3,   /* unknown dtype                                        */
  KVC_E_STATE = -4,   /* call out of the step protocol's order                */
  KVC_E_HIP = -5,     /* the HIP runtime reported an error while enqueueing   */
  KVC_E_SCRATCH = -6  /* kvc_attend_noalloc: the step's split partials need
                         more than its fixed scratch (KVC_NOALLOC_SCRATCH_BYTES) */
};

enum { KVC_F32 = 0, KVC_BF16 = 1 };

/* kvc_nbytes selectors */
enum {
  KVC_NB_KV = 0,      /* sum over layers of 2*B*Hkv_l*rows_l*D*bytes, the
                         size formula of Lab 07 section 1 with ring rows
                         (colibri PR, kv_ring_rows); no scratch rows          */
  KVC_NB_ALLOC = 1    /* bytes of device memory kvc_create needs             */
};

typedef struct {
  int32_t n_layer;          /* >= 1                                             */
  int32_t batch;            /* B rows, >= 1                                     */
  int32_t n_q_head;         /* Hq                                               */
  int32_t head_dim;         /* D: a multiple of 8 in [8, 256]                    */
  int32_t max_len;          /* positions per row, >= 1; one row's keys of one
                               KV head (max_len + 1 rows rounded up to 32, or
                               W + 1 on a ring, times D x dtype bytes) must
                               take under 2^31 bytes, else KVC_E_ARG: the
                               kernels address that region with 32-bit
                               offsets (bf16 D 128: max_len up to 8,388,575) */
  int32_t max_chunk;        /* largest C accepted by kvc_append, in [1, 1024]    */
  int32_t dtype;            /* KVC_F32 or KVC_BF16: cache, q, k, v and out      */
  const int32_t *n_kv_head; /* [n_layer] Hkv_l, Hq % Hkv_l == 0 (host memory)   */
  const int32_t *window;    /* [n_layer] 0 = global layer; W > 0 = sliding
                               layer whose queries see the W most recent keys
                               including their own (host memory)                */
  int32_t use_ring;         /* 1: a sliding layer with 0 < W < max_len keeps a
                               W-row ring; 0: every layer keeps max_len rows and
                               the window is applied as a mask only           */
  double rope_base;         /* > 0: RoPE with theta_d = base^(-2d/D), half-split
                               pairs (d, d+D/2); 0: q and k arrive rotated      */
  int32_t n_pages;          /* 0: every row keeps max_len rows per full layer.
                               > 0: paged cache ("Lab 07 - KV cache and
                               sampling", Stretch: fixed 16-token blocks and a
                               per-sequence block table): the full-layout
                               layers (all but rings) share a pool of n_pages
                               16-row pages, handed to rows as they grow and
                               returned by kvc_reset; one block table per row
                               serves every such layer                          */
  const int32_t *joint;     /* NULL, or [n_layer]: joint[l] = j >= 0 makes layer
                               l's softmax also cover layer j's keys (under
                               layer j's rules: all positions up to the query
                               for a global layer) together with its own, one
                               softmax over both (tiny_agent "generate.py"
                               module docstring and _append_chunk: hybrid layer
                               groups, a group-global K/V written by the
                               group's full layer plus a ring per layer).  j <
                               l, layer j full-layout (not a ring) with the
                               same KV heads and no partner of its own; -1 =
                               none.  Layer j is appended before layer l is
                               attended in a step (else KVC_E_STATE) and need
                               not be attended itself.  Joint layers run
                               append + attend (no single-kernel step) and
                               not in static steps (KVC_E_ARG)              */
} kvc_config;

/* Rows per page of a paged cache. */
enum { KVC_PAGE_ROWS = 16 };

/* Size in bytes for `what` (KVC_NB_KV or KVC_NB_ALLOC); 0 if cfg is invalid.
 * KVC_NB_KV is the size formula of "Lab 07 - KV cache and sampling" section
 * 1 (2 x layers x KV heads x head_dim x bytes per token and row) with W rows
 * for ring layers (colibri PR "Expected memory savings").  Pure host
 * computation. */
size_t kvc_nbytes(const kvc_config *cfg, int what);

/* Create a handle over caller-owned device memory `dev_buf` of `buf_bytes`
 * (>= kvc_nbytes(cfg, KVC_NB_ALLOC)) on the current HIP device: the
 * preallocated cache of pycraft-1 "model/kv_cache.py" (KVCache.__init__:
 * every buffer sized once for max_len, keys stored before the GQA
 * expansion) and tiny_agent "generate.py" KVCache (a global cache with one
 * scratch row, a W-row ring per sliding layer).  Copies cfg
 * (the arrays too).  Enqueues the RoPE table upload and the zeroing of the
 * row lengths on `stream` and waits for them (create is not part of a step).
 * All rows start empty.  On error *out is NULL and nothing was enqueued.
 *
 * Tuning read from the environment at create (none changes results beyond
 * the split order's rounding; out-of-range values are ignored):
 *   KVC_DECODE_WAVES=n      decode split plan for n waves per launch instead
 *                           of the waves the chip holds at once;
 *   KVC_DECODE_SPLIT=k      a fixed decode split of k keys (a multiple of 16);
 *   KVC_DECODE_MIN_TILES=t  shortest decode split, in 16-key tiles (default 4);
 *   KVC_DECODE_FUSED=0      kvc_append_attend enqueues kvc_append + kvc_attend;
 *   KVC_FUSED_MERGE=1       kvc_append_attend merges in its decode launch;
 *   KVC_CHUNK_FUSED=0       kvc_append_attend stages ring layers' chunk
 *                           steps as kvc_append does (then their outputs
 *                           are bit for bit those of the two calls);
 *   KVC_CHUNK_SMALL=0       every chunk row in 8-wave workgroups;
 *   KVC_CHUNK_PLAN=0        chunk splits at the cap (16 per longest row)
 *                           instead of the cost-model plan;
 *   KVC_CHUNK_DIRECT=0      ring layers' full-chunk steps merge in the
 *                           merge kernel too;
 *   KVC_CHUNK_RING_SMALL=0  ring layers' chunk rows take 8-wave workgroups
 *                           by size, as other layers' do, even when that
 *                           launch would hold fewer workgroups than CUs;
 *   KVC_CHUNK_KEY_HALVES=0  chunk rows of 128-row query tiles in 4-wave
 *                           workgroups instead of 8-wave ones whose two
 *                           halves take alternate key tiles;
 *   KVC_CHUNK_SIDE=0        both chunk launches on the caller's stream
 *                           (default: with rows of both sizes, the 4-wave
 *                           launch runs on a second stream of the handle,
 *                           forked from and joined back to the caller's by
 *                           events, so a capture of the caller's stream
 *                           takes it in; the stream and its two events are
 *                           created here when max_chunk >= 2, never inside
 *                           a step, and a failure to create them returns
 *                           KVC_E_HIP);
 *   KVC_DECODE_WG=0         one-token steps of short ring layers (at most
 *                           1024 rows) take the split plan and the merge
 *                           kernel instead of one workgroup per row;
 *   KVC_LOG=1 or 2          sizes at create (2: also decode plans) on stderr. */
int kvc_create(const kvc_config *cfg, void *dev_buf, size_t buf_bytes,
               void *stream, kvc_t **out);

/* Free the host handle and the side stream and events made at create.  The
 * device buffer stays the caller's (pycraft-1 "model/kv_cache.py": the cache
 * memory is the model's, reset only rewinds lengths). */
void kvc_destroy(kvc_t *h);

/* Empty `n_rows` rows (host array of row indices): their length and left
 * padding drop to 0.
 * Nothing is zeroed: stale keys and values stay in memory and are never read
 * again (pycraft-1 reset; tiny_agent KVCache.reset).  Not allowed inside a
 * step (KVC_E_STATE). */
int kvc_reset(kvc_t *h, const int32_t *rows_host, int32_t n_rows, void *stream);

/* Left padding: rows rows_host[i] start with first_host[i] pad positions
 * (0 <= first <= max_len; 0 = none).  Keys at positions below first[b] are
 * hidden from every query of row b, except that a pad query (position below
 * first) sees its own key, so that no query has an empty softmax (tinyllm
 * "kv_cache.py": padded_causal_mask and the KVCache pad_lens; a left-padded
 * batched prefill).  RoPE positions are unchanged: pads take positions
 * 0 .. first - 1.  kvc_reset clears it.  Not inside a step. */
int kvc_set_first(kvc_t *h, const int32_t *rows_host, const int32_t *first_host,
                  int32_t n_rows, void *stream);

/* Admit rows of another cache (tinyllm "kv_cache.py", SlotKVCache.admit: a
 * finished batched prefill's rows become decode slots): row dst_rows[i] of
 * `dst` becomes a copy of row src_rows[i] of `src` (every layer's keys and
 * values, its length and its left padding); the source rows are unchanged.
 * The two caches must have the same layers (KV heads, windows, layouts),
 * head_dim, Hq and dtype, live on one device, and be outside a step with
 * fresh host mirrors (else KVC_E_ARG / KVC_E_STATE); a source row longer
 * than dst's max_len gives KVC_E_FULL; dst rows must be distinct and, when
 * src == dst, not among the source rows.  Device-to-device copies of the
 * rows' stored blocks, enqueued on `stream` after any earlier work there.
 * Release a slot with kvc_reset. */
int kvc_admit(kvc_t *dst, const int32_t *dst_rows, const kvc_t *src,
              const int32_t *src_rows, int32_t n_rows, void *stream);

/* Append layer `layer`'s new keys and values: tiny_agent "generate.py"
 * _append_chunk (key rotated at its absolute position lens[b] + i, then
 * written with the value to slot pos on a global layer or pos % W on a ring,
 * padding to the scratch row), pycraft-1 "model/kv_cache.py" update (writes
 * without advancing) and its overflow guard; on a ring with C >= 2 the rows
 * are staged and committed only after the layer's attention (colibri PR
 * "inkling: ring-buffer KV cache", "How it works": append after scoring,
 * keep the last W rows of the chunk).
 *   k, v          device, (B, C, Hkv_l, D) in the cache dtype; k is pre-RoPE
 *                 (rotated here at position lens[b]+i) unless rope_base == 0.
 *   n_new_host    host, [B]: real tokens of row b, 0 <= n_new[b] <= C; tokens
 *                 i >= n_new[b] are padding (written to the scratch row).
 *   C             chunk width, 1 <= C <= max_chunk.
 *   slot_out_dev  device int32 (B, C) or NULL: the cache row each token lands
 *                 in (full layer: pos or max_len for padding; ring layer:
 *                 pos % W for the last W real tokens, else W).
 * The first append of a step checks capacity (lens[b] + n_new[b] <= max_len
 * for every row, and on a paged cache enough free pages for the rows' new
 * positions, else KVC_E_FULL with nothing taken) and latches n_new and C
 * (and takes the pages); every other append
 * of the step must pass the same values (else KVC_E_STATE).  Each layer is
 * appended once per step. */
int kvc_append(kvc_t *h, int32_t layer, const void *k, const void *v,
               const int32_t *n_new_host, int32_t C, int32_t *slot_out_dev,
               void *stream);

/* Attend layer `layer`'s queries (tiny_agent "generate.py" _append_chunk:
 * grouped-query attention straight against the cache under the offset
 * causal mask of "Lab 07 - KV cache and sampling" section 2, clamped to the
 * window on a sliding layer as in the colibri PR "What this does"): q device
 * (B, C, Hq, D) pre-RoPE (unless rope_base == 0); out device (B, C, Hq, D);
 * C is the step's chunk width latched by its first append (q and out must
 * hold exactly that many tokens per row).  Query i of row b sits at
 * p = lens[b] + i and sees cached key j iff j <= p and, on a sliding layer,
 * p - j < W.  Query head h reads KV head h / (Hq / Hkv_l).  Scores are
 * q.k / sqrt(D) in float32, softmax in float32.  Outputs of padded queries
 * (i >= n_new[b]) and of rows with n_new[b] == 0 are exactly zero.  Must
 * follow this layer's kvc_append in the same step (else KVC_E_STATE).
 * Launches: the split attention kernels, then a merge of the splits; on a
 * ring layer whose step has every row a full chunk (n_new[b] == C >= 2) the
 * chunk kernel writes `out` itself (one split per row) and no merge runs. */
int kvc_attend(kvc_t *h, int32_t layer, const void *q, void *out, void *stream);

/* For callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, checks, launches and results as kvc_attend (the same
 * kernels and split plan, so the same bits), except that the split-K
 * partials live in a fixed array of KVC_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU for the life of the process, instead of the
 * handle's buffer.  Nothing is allocated, freed or cleared by the call
 * (every partial slot the merge reads is written by the same call first).
 * The step's partials take
 *     round_up(B*Hq*64*8, 256) + round_up(B*Hq*64*D*4, 256)
 *   + (a step with a chunk row: round_up(B*C*Hq*16*8, 256) + round_up(B*C*Hq*16*D*4, 256))
 * bytes (a B 64, Hq 32, D 128 decode step: 65 MiB); a step needing more
 * returns KVC_E_SCRATCH with nothing enqueued and the layer still
 * unattended (kvc_attend can then take it).  KVC_E_HIP if the array's
 * device address could not be looked up at kvc_create.  Every handle on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (other
 * streams, other threads, other handles) race and must be ordered by the
 * caller. */
#define KVC_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int kvc_attend_noalloc(kvc_t *h, int32_t layer, const void *q, void *out, void *stream);

/* kvc_append followed by kvc_attend for one layer, in one call: same
 * arguments (q and out as for kvc_attend), same checks, same stored rows and
 * slot indices, same step protocol (the layer counts as appended and
 * attended), and the same outputs (bit for bit, except the chunk steps of
 * ring layers below, whose outputs agree within the attention's rounding:
 * they visit the keys in another order).  A one-token
 * step (C == 1) in bf16 with a decode-kernel head shape (D in {64, 128},
 * Hq / Hkv_l in {1, 2, 4, 8, 16}) runs the rotation and store of each row's
 * new key and value and the decode attention over its key splits as one
 * kernel (tiny_agent "generate.py" _append_chunk writes a token and attends
 * over it in one pass), then the merge of the splits as a second (a ring
 * layer of at most 1024 rows: one launch whose workgroups merge).  With
 * KVC_FUSED_MERGE=1 (see kvc_create), the first kernel
 * merges too (the last split of a row and KV head to finish merges them):
 * one launch per layer, for callers whose launch rate bounds them; it reads
 * the partials back at the end of the launch, so a GPU-bound step is faster
 * without it.  A chunk step of a sliding-window ring layer in bf16 whose
 * rows all hold 2 .. 64 tokens (C <= 64; not a joint layer or a joint
 * layer's partner) stages nothing: the chunk-attention kernel reads the new
 * rows from k and v, rotates them, scores them, and the last workgroup of
 * each (row, KV head) writes the kept ones to their ring slots (colibri PR
 * "How it works": append after scoring), so no append launch runs
 * (KVC_CHUNK_FUSED=0 turns this off).  Other steps enqueue the two calls'
 * work.  While a merging
 * launch runs, no other launch of the same handle may run concurrently (they
 * share split counters in the buffer).
 * Errors as for kvc_append; KVC_E_HIP if a launch fails after the append's
 * work was enqueued. */
int kvc_append_attend(kvc_t *h, int32_t layer, const void *q, const void *k,
                      const void *v, const int32_t *n_new_host, int32_t C,
                      int32_t *slot_out_dev, void *out, void *stream);

/* End the step: lens[b] += n_new[b] on the device and in the host mirror
 * (pycraft-1 "model/kv_cache.py" advance, run once after every layer;
 * tinyllm "kv_cache.py" end_step; "Lab 07 - KV cache and sampling" section 3:
 * the cache length grows by the chunk's real tokens).  Every layer must have
 * been appended and attended (else KVC_E_STATE). */
int kvc_advance(kvc_t *h, void *stream);

/* Paged caches: page use in tokens (tinyllm "kv_cache.py" SlotKVCache:
 * used_tokens / allocated_tokens / reserved_tokens).  used = sum of the row
 * lengths; allocated = pages held by rows x 16; reserved = n_pages x 16 (an
 * unpaged cache reports B x max_len for both allocated and reserved).
 * Host mirrors only (KVC_E_STATE while the lengths mirror is stale). */
int kvc_page_stats(const kvc_t *h, int64_t *used, int64_t *allocated, int64_t *reserved);

/* Paged caches: give rows rows_host[i] pages for at least tokens_host[i]
 * positions (pages are otherwise taken by the appends that need them), so
 * that later static steps, which cannot take pages, have room; a static step
 * rejects a row without a page for its token (KVC_STATIC_FULL).  KVC_E_FULL
 * (nothing taken) if the pool runs short or a count passes max_len.  Not
 * inside a step; a no-op on an unpaged cache. */
int kvc_reserve(kvc_t *h, const int32_t *rows_host, const int32_t *tokens_host, int32_t n_rows,
                void *stream);

/* Copy the host mirror of the row lengths into lens_host[B] (tiny_agent
 * "generate.py" KVCache keeps the lengths on the host as well, so that no
 * step reads the device; tinyllm "kv_cache.py" keeps a host copy of the
 * per-slot positions).  KVC_E_STATE while the mirror is behind the device
 * (after a static step, until kvc_sync_lens). */
int kvc_lens(const kvc_t *h, int32_t *lens_host);

/* Static one-token steps: a step whose work does not depend on anything the
 * host reads, so that it can be captured once in a HIP graph and replayed
 * (tinyllm "kv_cache.py", SlotKVCache: fixed shapes for a CUDA-graph decode
 * step; its end_step splits into the device update a replay runs and a host
 * update the caller runs after each replay).
 *
 *     kvc_static_begin(h, n_new_dev, s);
 *     for each layer l: kvc_append_attend(h, l, q, k, v, NULL, 1, slot, out, s);
 *                       (or kvc_append(.., NULL, 1, ..) + kvc_attend)
 *     kvc_advance(h, s);
 *
 * kvc_static_begin enqueues one small kernel that reads the step's token
 * counts from device memory (n_new_dev: int32 [B], each 0 or 1, read when the
 * kernel runs, so a replay uses the values there at that time), checks them
 * against the device row lengths, and plans every layer's decode splits on
 * the device: the plan is the one the host makes for an eager step, so a
 * static step gives the same bits.  Launch grids are fixed bounds; waves
 * past the planned work exit at once.  If any count is outside {0, 1}
 * (KVC_STATIC_BAD_COUNT) or any row would pass max_len (KVC_STATIC_FULL), the
 * whole step runs with every count 0 (nothing appended, every output zero,
 * lengths unchanged) and the reason is or-ed into sticky device flags.
 * Within the step, appends pass n_new_host = NULL and C = 1; kvc_advance
 * updates the device lengths only and leaves the host mirror stale: eager
 * appends, kvc_reset and kvc_lens return KVC_E_STATE until kvc_sync_lens.
 * Kernel timing must be off while a step is being captured.  No call of a
 * static step allocates, frees, synchronises or copies through host memory;
 * all of them are safe under stream capture. */
enum { KVC_STATIC_BAD_COUNT = 1, KVC_STATIC_FULL = 2 };
int kvc_static_begin(kvc_t *h, const int32_t *n_new_dev, void *stream);

/* Read and clear the sticky flags of static steps (bits KVC_STATIC_*):
 * copies them to *flags_host, waits for `stream`, then enqueues their
 * clearing.  Not inside a step. */
int kvc_static_status(kvc_t *h, int32_t *flags_host, void *stream);

/* Refresh the host mirror of the row lengths from the device (waits for
 * `stream`).  Not inside a step. */
int kvc_sync_lens(kvc_t *h, void *stream);

/* Where layer `layer` lives inside the device buffer (for inspection).
 * K rows are row-major: byte offset k_offset + ((b*Hkv + g)*rows_alloc + r)*D*s.
 * V is stored transposed in blocks of 16 rows: element (b, g, r, d) sits at
 * v_offset + ((((b*Hkv + g)*rows_alloc/16 + r/16)*D + d)*16 + r%16)*s.
 * rows excludes the scratch row (index `rows`); rows_alloc = rows + 1 rounded
 * up to 32, plus 16 on a contiguous (not paged) layer where that many rows
 * would take a multiple of 8 KB (rows_alloc*D*s), so that no two (row, KV
 * head) regions start a multiple of 8 KB apart.  Staging (ring layers, max_chunk >= 2) uses the same two layouts
 * with stage_rows_alloc rows; stage offsets are -1 when there is none. */
typedef struct {
  int64_t k_offset, v_offset, stage_k_offset, stage_v_offset;
  int32_t n_kv_head, window, is_ring, rows, rows_alloc, stage_rows_alloc;
} kvc_layer_info;
int kvc_layer_layout(const kvc_t *h, int32_t layer, kvc_layer_info *info);

/* Where the handle's own state lives inside the device buffer (inspection):
 * the int32 row lengths [B] (device copy of the host mirror), the int32 n_new
 * [B] of the current step, and the float (cos, sin) RoPE table
 * [max_len][D/2][2] (-1 when rope_base == 0). */
typedef struct {
  int64_t total_bytes, kv_bytes, lens_offset, n_new_offset, rope_offset;
} kvc_buffer_info_t;
int kvc_buffer_info(const kvc_t *h, kvc_buffer_info_t *info);

/* Kernel timing (diagnostics): every launch of a timed kind carries a pair of
 * HIP events that the dispatch itself stamps when the kernel starts and ends
 * (hipExtLaunchKernel), so a measurement is the kernel's own duration and no
 * extra packets enter the stream.
 *   kvc_timing_begin: allocate a pool for `max_launches` launches and start
 *                     recording (KVC_E_HIP if events cannot be created).
 *   kvc_timing_begin_kinds: the same for the kinds whose bit (1 << kind) is
 *                     set in `kind_mask` only; other launches carry no
 *                     events (KVC_E_ARG for bits past the last kind).  A
 *                     dispatch that stamps events leaves a longer gap before
 *                     the next dependent dispatch, so timing fewer kinds
 *                     disturbs a timed sequence less.
 *   kvc_timing_end:   wait for the recorded events, write the summed kernel
 *                     time in ms and the launch count per kind, stop.
 * Kinds: 0 append, 1 decode attention, 2 chunk attention, 3 split combine,
 * 4 ring commit, 5 generic attention, 6 single-kernel append + decode +
 * merge (kvc_append_attend). */
enum { KVC_K_APPEND = 0, KVC_K_DECODE = 1, KVC_K_PREFILL = 2, KVC_K_COMBINE = 3,
       KVC_K_COMMIT = 4, KVC_K_GENERIC = 5, KVC_K_FUSED = 6, KVC_K_NKINDS = 7 };
int kvc_timing_begin(kvc_t *h, int32_t max_launches);
int kvc_timing_begin_kinds(kvc_t *h, int32_t max_launches, int32_t kind_mask);
int kvc_timing_end(kvc_t *h, double *ms_per_kind, int32_t *launches_per_kind);
/* While timing: the first min(cap, launches so far) timed launches, in
 * launch order: kind, start and end in ms from the first timed launch's
 * start (waits for them).  Returns that count, or a negative status
 * (KVC_E_STATE when timing is off).  Launches on two streams overlap; the
 * union of their spans is the time the kernels kept the GPU busy. */
int kvc_timing_spans(kvc_t *h, int32_t cap, int32_t *kinds, double *start_ms, double *end_ms);

/* Static text for a status code; KVC_E_FULL reads "KV cache full", the
 * message of tiny_agent "generate.py" append and pycraft-1 update. */
const char *kvc_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
