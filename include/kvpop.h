/*
 * kvpop.h - C ABI of a per-KV-head fixed-budget sparse KV cache (KVpop) for
 * AMD Instinct MI355X (gfx950).
 *
 * What the cache holds.  Every (layer, sequence, KV head) keeps at most
 * budget = n_sink + n_scored + n_recent rows of K and V: the first n_sink
 * positions (sinks), the n_recent newest positions (the protected recent
 * window, which includes the token just decoded), and n_scored older tokens
 * chosen by score ("Qwen3-8B-KVpop-4x" model card, intro: a bounded sink +
 * scored top-k + recent-window cache of 4 + 3,772 + 256 = 4,032 entries per
 * head; aiweekly French article, second paragraph: per-head sinks, protected
 * recent window, learned top-k of older tokens).
 *
 * Delayed scoring.  A token's long-range score is supplied only when the
 * token leaves the window, n_recent steps after it was decoded (model card,
 * "Delayed scoring"; KVpop abstract: scoring deferred by a fixed number of
 * steps).  The score is an input: the learned scorer is not part of this
 * library.  The leaving token then either takes a scored slot or is dropped
 * for good (KVpop abstract: a fixed-budget keep-or-drop eviction policy).
 *
 * Order of importance: key = (score, position) compared lexicographically,
 * so on an equal score the newer token is kept; the lower score, then the
 * older token, is evicted first.  The pages fix no tie order; this is the
 * library's reading.  While fewer than n_scored tokens hold scored slots, a
 * leaving token is admitted without comparison.  Scores are float32; -0 and
 * +0 are equal, infinities order normally, NaN is a caller error (recorded
 * in kvpop_state.flags; the kept set is then unspecified).
 *
 * Because scores never change once assigned and evicted tokens never
 * return, after position n the kept set of a head equals
 *   {0..min(s,n+1)-1}  U  {max(s,n-W+1)..n}  U  top-n_scored of {s..n-W} by key.
 *
 * Decode attention: query head h attends to KV head floor(h*Hkv/Hq) over the
 * kept rows with softmax(scale * q.k) v, bf16 inputs, fp32 accumulation,
 * bf16 output (round to nearest even).
 *
 * Conventions for every call:
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Device pointers are borrowed for the stream-ordered duration of the
 *     call; the caller keeps them alive until the stream has passed it.  No
 *     pointer is retained after a call returns.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).
 *   - Return value: KVPOP_OK (0) or a negative KVPOP_E* code.  Arguments are
 *     validated before anything is enqueued, so a call that fails validation
 *     changes nothing.  A HIP error after enqueueing poisons the cache: every
 *     later call returns KVPOP_ESTATE.
 *   - A cache object is not thread-safe; drive it from one host thread and
 *     one stream (calls on one cache share a device workspace).
 */
#ifndef KVPOP_H_
#define KVPOP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define KVPOP_API __attribute__((visibility("default")))
#else
#define KVPOP_API
#endif

#define KVPOP_OK 0
#define KVPOP_EINVAL (-1) /* bad argument, shape or NULL pointer           */
#define KVPOP_ENOMEM (-2) /* device allocation failed or arena too small    */
#define KVPOP_EHIP (-3)   /* HIP runtime or launch error (cache poisoned)   */
#define KVPOP_ESTATE (-4) /* call out of order, cache poisoned, or position
                             limit reached                                   */
#define KVPOP_ERANGE (-5) /* input larger than the static workspace of a
                             no-allocation entry point                       */

/* kvpop_state.flags bits */
#define KVPOP_FLAG_NAN_SCORE 1 /* a NaN score reached the cache */

typedef struct kvpop_cache kvpop_cache;

typedef struct kvpop_config {
  int32_t n_layers;      /* >= 1 */
  int32_t batch;         /* sequences per layer, >= 1 */
  int32_t n_q_heads;     /* Hq, a multiple of n_kv_heads; Hq/Hkv in {1,2,4,8} */
  int32_t n_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t n_sink;        /* s >= 0 */
  int32_t n_scored;      /* k >= 0 */
  int32_t n_recent;      /* W >= 1 */
  int32_t max_positions; /* positions 0 .. max_positions-1 per sequence;
                            1 .. 2^30 */
  int32_t decode_splits; /* slot ranges per head in decode attention;
                            0 = chosen by the library, else 1 .. 256 */
  float softmax_scale;   /* <= 0: 1/sqrt(head_dim) */
  int32_t prune_interval; /* cache backend ("Qwen3-8B-KVpop-4x" model card,
                            "Cache backends"; when to prune is not given
                            there, this is the reading taken):
                            0 = Static: fixed buffers of n_sink + n_scored +
                                n_recent rows, the leaving token replaces the
                                least important scored one or is dropped;
                            P in 1 .. 4096 = Dynamic: n_scored + P scored
                                rows; every token leaving the window is held,
                                and after every P-th decode step of a layer
                                each of its heads is pruned back to its top
                                n_scored (also on demand, kvpop_cache_prune).
                            Both hold the same rows right after a prune. */
  int32_t decode_finish; /* how a decode step merges a head's splits (no
                            effect with one split):
                            0 = the library's default: 1 for
                                kvpop_decode_step, 2 for
                                kvpop_decode_step_layers;
                            1 = the last split's workgroup, in the same launch;
                            2 = a second launch, one workgroup per head.
                            The outputs and cache updates are identical. */
} kvpop_config;

typedef struct kvpop_state {
  int32_t n;     /* newest processed position of the sequence; -1 when empty */
  int32_t flags; /* KVPOP_FLAG_* bits, OR over the KV heads */
} kvpop_state;

/* Rows per KV head, the "capacity" below: n_sink + n_scored + n_recent +
 * prune_interval. */

/* Device bytes the cache needs for `cfg` (K/V rows, slot metadata and the
 * decode workspace), or 0 if `cfg` is invalid.  Pure host arithmetic. */
KVPOP_API size_t kvpop_cache_required_bytes(const kvpop_config* cfg);

/* Create a cache on the current HIP device; every (layer, sequence) starts
 * empty.  If `device_arena` is NULL the library allocates with hipMalloc and
 * frees in kvpop_cache_destroy; otherwise it uses the caller's device memory
 * (256-byte aligned, at least kvpop_cache_required_bytes(cfg) bytes), which
 * must outlive the cache.  Initialisation runs on the legacy default stream
 * and is complete when the call returns.  *out receives the handle.
 * Errors: KVPOP_EINVAL (NULL pointer, invalid config, misaligned arena),
 * KVPOP_ENOMEM (allocation failed or arena too small), KVPOP_EHIP (no usable
 * device or a runtime error). */
KVPOP_API int kvpop_cache_create(const kvpop_config* cfg, void* device_arena, size_t arena_bytes,
                       kvpop_cache** out);

/* Release the cache and the memory it allocated.  Waits for the device to
 * finish using it.  NULL is a no-op. */
KVPOP_API void kvpop_cache_destroy(kvpop_cache* cache);

/* Mark (layer, seq) empty again (n = -1).  Nothing is enqueued and `stream`
 * is unused: a following non-empty prefill of the sequence writes its control
 * blocks anyway, and any other call that reads them (decode of the layer,
 * prune, state) first re-initialises them on its own stream.  The rows are
 * not cleared; they are unreachable until refilled.  Errors: KVPOP_EINVAL
 * (bad indices), KVPOP_ESTATE (poisoned). */
KVPOP_API int kvpop_cache_reset(kvpop_cache* cache, int32_t layer, int32_t seq, void* stream);

/* Prefill compaction: fill the empty (layer, seq) from an n_tokens-long
 * prompt.  k, v: device [Hkv][n_tokens][D] bf16.  scores: device
 * [Hkv][n_tokens] float32, of which only positions n_sink .. n_tokens-n_recent-1
 * are read (window positions are scored later, when they leave the window).
 * Afterwards n = n_tokens-1 and each head keeps its sinks, its last n_recent
 * positions, and the n_scored candidates with the largest keys.
 * n_tokens == 0 is a no-op.  Errors: KVPOP_EINVAL (NULL pointers, bad
 * indices, n_tokens < 0), KVPOP_ESTATE (not empty, poisoned, or n_tokens >
 * max_positions). */
KVPOP_API int kvpop_prefill_compact(kvpop_cache* cache, int32_t layer, int32_t seq, int32_t n_tokens,
                          const uint16_t* k, const uint16_t* v, const float* scores,
                          void* stream);

/* Prefill compaction of several prompts at once: items[i] fills the empty
 * (layer, seq) it names exactly as kvpop_prefill_compact would (same
 * layouts for k, v and scores; n_tokens == 0 leaves it empty).  The prompts
 * share kernel launches (up to 64 per launch, grouped by how they select;
 * only prompts too long for two-level selection run one at a time), which is
 * how a serving batch, or every layer of one prompt, is compacted without
 * one launch pair per prompt.  Stream-ordered and asynchronous; `items` is read during the call
 * only; the device buffers it points to must stay alive until the stream
 * passes the call.  Every item is checked before anything is enqueued.
 * Errors: KVPOP_EINVAL (NULL pointers, bad indices, n_tokens < 0, the same
 * (layer, seq) twice), KVPOP_ESTATE (an item's (layer, seq) is not empty,
 * n_tokens > max_positions, or the cache is poisoned), KVPOP_EHIP. */
typedef struct kvpop_prefill_item {
  int32_t layer;
  int32_t seq;
  int32_t n_tokens;
  int32_t pad;          /* unused */
  const uint16_t* k;    /* device [Hkv][n_tokens][D] bf16 */
  const uint16_t* v;    /* device [Hkv][n_tokens][D] bf16 */
  const float* scores;  /* device [Hkv][n_tokens] float32 */
} kvpop_prefill_item;
KVPOP_API int kvpop_prefill_compact_batch(kvpop_cache* cache, int32_t n_items,
                                          const kvpop_prefill_item* items, void* stream);

/* One decode step of every sequence of `layer`: sequence b processes position
 * n_b + 1 (position 0 if empty).
 *   q            device [batch][Hq][D] bf16, the query of the new token
 *   k_new, v_new device [batch][Hkv][D] bf16, K/V of the new token
 *   score_leaving device [batch][Hkv] float32, the score of position
 *                n_b + 1 - n_recent (the token leaving the window); read only
 *                when that position is >= n_sink
 *   out          device [batch][Hq][D] bf16, attention over the kept rows
 *                (the new token included)
 * The new token enters the window; the leaving token takes a scored slot
 * (free, or the least important one's, which is evicted) or is dropped.
 * Dynamic backend: the leaving token is held while the scored region has
 * fewer than n_scored + prune_interval tokens, and after every
 * prune_interval-th call for this layer (counted since the cache was
 * created; resets do not restart the count) the call also prunes every head
 * of the layer, as kvpop_cache_prune does.
 * Errors: KVPOP_EINVAL (NULL pointers, bad layer), KVPOP_ESTATE (poisoned or
 * a sequence would reach max_positions), KVPOP_EHIP (launch failed). */
KVPOP_API int kvpop_decode_step(kvpop_cache* cache, int32_t layer, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, const float* score_leaving, uint16_t* out,
                      void* stream);

/* One decode step of `n_layers` consecutive layers (layer0 .. layer0 +
 * n_layers - 1) in a single launch: exactly what n_layers calls of
 * kvpop_decode_step, one per layer in order, would do, with every per-layer
 * tensor given a leading layer dimension:
 *   q            device [n_layers][batch][Hq][D] bf16
 *   k_new, v_new device [n_layers][batch][Hkv][D] bf16
 *   score_leaving device [n_layers][batch][Hkv] float32
 *   out          device [n_layers][batch][Hq][D] bf16
 * Valid only when no layer's inputs depend on another layer's output of the
 * same step: independent per-layer streams, as in the synthetic multi-layer
 * benchmarks.  In a transformer, layer l+1's query comes from layer l's
 * output, so a model decodes one layer at a time with kvpop_decode_step.
 * Every (layer, sequence, KV head) keeps its own bounded cache ("Qwen3-8B-
 * KVpop-4x" model card, intro), so the layers' heads are independent and
 * share one grid; with many heads the launch keeps every compute unit busy
 * where one layer at batch 1 (8 KV heads) cannot.  The Dynamic backend's
 * prune runs for each layer whose step count reaches the interval.
 * Errors: KVPOP_EINVAL (NULL pointers, layer range outside the cache),
 * KVPOP_ESTATE (poisoned, or a sequence of one of the layers would reach
 * max_positions), KVPOP_EHIP (launch failed). */
KVPOP_API int kvpop_decode_step_layers(kvpop_cache* cache, int32_t layer0, int32_t n_layers,
                                       const uint16_t* q, const uint16_t* k_new,
                                       const uint16_t* v_new, const float* score_leaving,
                                       uint16_t* out, void* stream);

/* Dynamic backend: prune every sequence's heads of `layer` now.  A head whose
 * scored region holds more than n_scored tokens keeps its n_scored most
 * important ones (by score, then position: the newer wins a tie) and evicts
 * the rest for good; its rows are compacted into [0, count).  Afterwards
 * every head holds exactly the rows the Static backend would keep.
 * Stream-ordered.  A no-op for the Static backend.  Errors: KVPOP_EINVAL
 * (NULL cache, bad layer), KVPOP_ESTATE (poisoned), KVPOP_EHIP. */
KVPOP_API int kvpop_cache_prune(kvpop_cache* cache, int32_t layer, void* stream);

/* Read back the state of (layer, seq).  Synchronises `stream` first.
 *   st        host, receives n and flags
 *   counts    host [Hkv] or NULL: kept rows per KV head
 *   kept_pos  host [Hkv][capacity] or NULL: kept positions of each head in
 *             ascending order, padded with -1
 * The caller owns the host buffers.  Errors: KVPOP_EINVAL, KVPOP_EHIP. */
KVPOP_API int kvpop_cache_state(kvpop_cache* cache, int32_t layer, int32_t seq, kvpop_state* st,
                      int32_t* counts, int32_t* kept_pos, void* stream);

/* Prefix top-k thresholds of a prompt (the "prefix top-k thresholds" kernel
 * that the "Qwen3-8B-KVpop-4x" model card lists among its cache backends;
 * the exact contract there is not given, this is the reading taken).  With
 * the cache's geometry (n_kv_heads, n_sink, n_scored, n_recent) and no
 * access to its state:
 *   scores  device [Hkv][n_tokens] float32, the score of every position
 *   thr     device [Hkv][n_tokens] uint64 (output): for position n, the key
 *           ((order code of the score) << 32 | position) of the n_scored-th
 *           most important candidate among positions n_sink .. n-n_recent;
 *           0 while there are fewer than n_scored of them, and ~0 when
 *           n_scored == 0.
 * The kept set after position n is then the sinks, the window and the
 * candidates whose key is >= thr[g][n]: the set a cache streamed through
 * position n holds.  Stream-ordered and asynchronous; the caller owns both
 * buffers.  Errors: KVPOP_EINVAL (NULL pointers, n_tokens < 0, n_scored >
 * 4096), KVPOP_ESTATE (n_tokens > max_positions), KVPOP_EHIP. */
KVPOP_API int kvpop_prefix_thresholds(kvpop_cache* cache, int32_t n_tokens, const float* scores,
                                      uint64_t* thr, void* stream);

/* Future-attention target of one sequence: the attention mass each key
 * receives from queries that come after it has left the protected recent
 * window (the target the scorer is trained against: English and French
 * aiweekly articles, KVpop abstract; computed, as they describe, by a
 * transposed-attention pass that never materialises the attention map).
 * With the cache's geometry and softmax scale c, and no access to its state:
 *   q    device [Hq][n_tokens][D] bf16, the queries of every position
 *   k    device [Hkv][n_tokens][D] bf16, the keys of every position
 *   work device [2][Hq][n_tokens] float32 workspace: work[0][h][i]
 *        receives query i of head h's causal log-sum-exp in log2 units,
 *        work[1][h][j] head h's share of y[g][j]
 *   y    device [Hkv][n_tokens] float32 (output):
 *        y[g][j] = sum over the query heads h of g's group and the queries
 *        i >= j + n_recent of softmax over j' <= i of c <q_h,i, k_g,j'>, at
 *        j' = j.  Summed over the group's query heads, not normalised (the
 *        pages leave both open; this is the reading taken).
 * Stream-ordered and asynchronous; the caller owns every buffer.  Errors:
 * KVPOP_EINVAL (NULL pointers, n_tokens < 0), KVPOP_ESTATE (n_tokens >
 * max_positions or poisoned), KVPOP_EHIP. */
KVPOP_API int kvpop_future_attention_target(kvpop_cache* cache, int32_t n_tokens, const uint16_t* q,
                                            const uint16_t* k, float* work, float* y, void* stream);

/* kvpop_future_attention_target without the workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same inputs, output,
 * kernels and result as kvpop_future_attention_target, bit for bit; the
 * [2][Hq][n_tokens] float32 workspace is a static device array of 32 MiB
 * that the library holds on every device it runs on until the process
 * ends, so 2 * Hq * n_tokens * 4 bytes must not exceed 32 MiB (Hq = 32:
 * n_tokens <= 131,072).  The call allocates nothing.  Every call on one
 * device shares that device's array: calls that overlap on one device (two
 * streams, or two host threads) race and give undefined results; order
 * them on one stream.  Nothing in the array needs clearing between calls
 * (every element read is written first by the same call).  Errors: as
 * kvpop_future_attention_target, plus KVPOP_ERANGE when the workspace would
 * exceed the array (checked before anything is enqueued) and KVPOP_EHIP
 * when the array's device address could not be obtained at cache creation. */
KVPOP_API int kvpop_future_attention_target_noalloc(kvpop_cache* cache, int32_t n_tokens,
                                                    const uint16_t* q, const uint16_t* k,
                                                    float* y, void* stream);

/* Static description of a return code. */
KVPOP_API const char* kvpop_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* KVPOP_H_ */
