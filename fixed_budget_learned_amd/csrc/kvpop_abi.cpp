// C-ABI host side of the fixed-budget cache: argument validation, the device
// memory layout, a host mirror of every sequence's position, and kernel
// launches.  No call throws; every failure maps to a KVPOP_E* code.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "kvpop.h"
#include "kvpop_internal.h"

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  size_t kc, vc, keys, pos, ring, ctl, sel, slice_keys, slice_meta, slice_tau, part_acc, part_ml, part_min,
      tickets, total;
  int32_t nsplit, rows_per_split, threads, rows_per_thread, finish_apart;
  int32_t sel_items;    // prompts one batched prefill launch can select at once
  int32_t slice_items;  // long prompts one batched two-level select can hold
};

bool mul_ok(size_t a, size_t b, size_t* r) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *r = a * b;
  return true;
}

// Rows per head: the budget plus the Dynamic backend's growth room.
int64_t capacity_of(const kvpop_config& c) {
  return int64_t(c.n_sink) + c.n_scored + c.n_recent + c.prune_interval;
}

bool config_valid(const kvpop_config* c) {
  if (c == nullptr) return false;
  if (c->n_layers < 1 || c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1) return false;
  if (c->n_q_heads % c->n_kv_heads != 0) return false;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->n_sink < 0 || c->n_scored < 0 || c->n_recent < 1) return false;
  if (c->prune_interval < 0 || c->prune_interval > kvpop::PRUNE_SLACK_MAX) return false;
  if (capacity_of(*c) > (1 << 20)) return false;
  if (c->max_positions < 1 || c->max_positions > (1 << 30)) return false;
  if (c->decode_splits < 0 || c->decode_splits > kvpop::decode_max_splits()) return false;
  if (c->decode_finish < 0 || c->decode_finish > 2) return false;
  if (std::isnan(c->softmax_scale) || std::isinf(c->softmax_scale)) return false;
  return true;
}

// Decode launch shape.  Each KV head's slots are split over `nsplit`
// workgroups of 256 threads, each thread holding 2 rows per pass.  With 256
// or more heads (batched serving) each head is one workgroup: the step needs
// no cross-workgroup merge at all.  With fewer heads the splits fill the
// 256 compute units at most once (one workgroup per unit), with at most 32
// splits per head and at least 64 slots per split.  Measured at batch 1:
//   * 4,032 slots, 8 KV heads: 32 splits of 128 slots 8.3 us; 64 splits of
//     64 slots (two workgroups per unit) 10.3 us;
//   * 2,048 slots, 8 KV heads: 32 splits of 64 slots (one pass of the
//     workgroup) 7.5 us; 16 or 20 splits of 128 slots 8.3 us;
//   * 4,032 slots, one KV head: 32 splits 8.2 us, 48 splits 9.3 us, 64
//     splits 8.7 us: beyond 32 the finishing workgroup's merge of the
//     partials costs more than the shorter splits save.
//
// Split heads are merged by the last split's workgroup, in the same launch,
// unless the configuration asks for the second launch: with each head's
// ticket on its own cache line the in-launch merge measured faster on every
// shape from 1 to 24 sequences (4x layer at batch 1: 10.7 against 12.4 us).
//
// A launch over several layers (kvpop_decode_step_layers) has many heads and
// is bound by bandwidth, not latency: there each head gets about 1,440 /
// heads splits (5 for 36 layers of 8 heads: 1,440 workgroups, 2.8 per
// compute unit), merged in a second launch.  Measured on 36 layers at batch
// 1, 4,032 slots: 1 split 121.6 us, 2 108.2, 4 102.3, 5 (second launch)
// 100.0, 6 (second launch) 98.7, 16 107.0; 2,048 slots: 1 split 65.2, 3
// 57.9, 5 (second launch) 56.2, 6 (second launch) 56.5, 8 (second launch)
// 60.9 (bf16 probabilities; with fp32 ones 5 splits take 101.7 and 58.3
// us).  In-launch tickets cost each workgroup a store acknowledgement and an
// atomic round trip while it holds its slot (6 splits: 102.0 against 98.7
// us).
int64_t decode_splits_for(const kvpop_config& c, int64_t heads, bool layers) {
  const int64_t budget = capacity_of(c);
  int64_t ns = c.decode_splits;
  if (ns == 0) {
    ns = layers ? (1440 + heads - 1) / heads : std::min<int64_t>(256 / heads, 32);
    ns = std::min<int64_t>(ns, (budget + 63) / 64);
    ns = std::min<int64_t>(ns, kvpop::decode_max_splits());
    ns = std::max<int64_t>(ns, 1);
  }
  return ns;
}

int32_t rows_per_split_for(const kvpop_config& c, int64_t ns) {
  const int64_t rpp = 256 / (c.head_dim / 16);  // rows per pass of a workgroup
  int64_t rows = (capacity_of(c) + ns - 1) / ns;
  return int32_t((rows + rpp - 1) / rpp * rpp);
}

void choose_decode_shape(const kvpop_config& c, int32_t* nsplit, int32_t* rows_per_split,
                         int32_t* threads, int32_t* rows_per_thread, int32_t* finish_apart) {
  const int64_t ns = decode_splits_for(c, int64_t(c.batch) * c.n_kv_heads, false);
  *nsplit = int32_t(ns);
  *rows_per_split = rows_per_split_for(c, ns);
  *threads = 256;
  *rows_per_thread = 2;
  *finish_apart = (c.decode_finish == 2) ? 1 : 0;
}

// Partial-result entries the decode workspace needs: the largest of one
// layer's launch and every launch over 1 .. n_layers layers.
size_t decode_parts(const kvpop_config& c) {
  const int64_t heads = int64_t(c.batch) * c.n_kv_heads;
  int64_t parts = heads * decode_splits_for(c, heads, false);
  for (int64_t n = 2; n <= c.n_layers; ++n)
    parts = std::max(parts, n * heads * decode_splits_for(c, n * heads, true));
  return size_t(parts);
}

bool compute_layout(const kvpop_config& c, Layout* L) {
  const size_t budget = size_t(capacity_of(c));
  const size_t heads_all = size_t(c.n_layers) * c.batch * c.n_kv_heads;
  const size_t G = size_t(c.n_q_heads / c.n_kv_heads);
  choose_decode_shape(c, &L->nsplit, &L->rows_per_split, &L->threads, &L->rows_per_thread,
                      &L->finish_apart);
  size_t rows, kvb, tmp;
  if (!mul_ok(heads_all, budget, &rows)) return false;
  if (!mul_ok(rows, size_t(c.head_dim) * 2, &kvb)) return false;
  size_t off = 0;
  auto take = [&](size_t bytes, size_t* at) -> bool {
    *at = off;
    const size_t a = align_up(bytes);
    if (a < bytes || off > SIZE_MAX - a) return false;
    off += a;
    return true;
  };
  bool ok = take(kvb, &L->kc) && take(kvb, &L->vc);
  ok = ok && mul_ok(rows, 8, &tmp) && take(tmp, &L->keys);
  ok = ok && mul_ok(rows, 4, &tmp) && take(tmp, &L->pos);
  ok = ok && mul_ok(heads_all, size_t(c.n_recent) * 4, &tmp) && take(tmp, &L->ring);
  ok = ok && mul_ok(heads_all, sizeof(kvpop::HeadCtl), &tmp) && take(tmp, &L->ctl);
  // selection buffer: up to PREFILL_NB prompts per launch, within 16 MiB
  const size_t sel_one = size_t(c.n_kv_heads) * size_t(std::max(c.n_scored, 1)) * 4;
  L->sel_items = int32_t(std::max<size_t>(1, std::min<size_t>(kvpop::PREFILL_NB,
                                                              (size_t(16) << 20) / sel_one)));
  ok = ok && take(sel_one * size_t(L->sel_items), &L->sel);
  // first-level keys of long prompts: up to PREFILL_NB prompts, within 128 MiB
  // (all 36 layers of a 131k-token prompt at k = 1,788 take 66 MB)
  const size_t slice_one = size_t(c.n_kv_heads) * kvpop::SLICE_MAX *
                           size_t(kvpop::slice_stride(c.n_scored)) * 8;
  L->slice_items = int32_t(std::max<size_t>(1, std::min<size_t>(kvpop::PREFILL_NB,
                                                                (size_t(128) << 20) / slice_one)));
  ok = ok && take(slice_one * size_t(L->slice_items), &L->slice_keys);
  ok = ok && take(size_t(L->slice_items) * c.n_kv_heads * kvpop::SLICE_MAX *
                       sizeof(kvpop::SliceMeta), &L->slice_meta);
  ok = ok && take(size_t(L->slice_items) * c.n_kv_heads * 4, &L->slice_tau);
  const size_t parts = decode_parts(c);
  ok = ok && mul_ok(parts, G * size_t(c.head_dim) * 4, &tmp) && take(tmp, &L->part_acc);
  ok = ok && mul_ok(parts, G * 2 * 4, &tmp) && take(tmp, &L->part_ml);
  ok = ok && mul_ok(parts, sizeof(kvpop::MinPart), &tmp) && take(tmp, &L->part_min);
  // tickets: every head of the cache (a launch over all layers)
  ok = ok && take(heads_all * 4 * kvpop::TICKET_STRIDE, &L->tickets);
  L->total = off;
  return ok;
}

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) return;
    ok = (prev == dev) || (hipSetDevice(dev) == hipSuccess);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct kvpop_cache {
  kvpop_config cfg;
  Layout lay;
  int device = -1;
  bool owns = false;
  bool poisoned = false;
  char* base = nullptr;
  float scale_log2e = 0.f;
  float* scratch = nullptr;     // this device's static future-target workspace
  std::vector<int32_t> n_host;  // [L][B], newest processed position
  // [L][B]: reset since the control blocks were last written.  A reset
  // enqueues nothing: a non-empty prefill overwrites the blocks anyway, and
  // every other call that reads them first initialises the stale ones
  // (flush_resets) on its own stream.
  std::vector<uint8_t> stale;
  int64_t n_stale = 0;
  std::vector<int64_t> steps;   // [L] decode steps taken (the Dynamic backend's prune clock)

  kvpop::Geometry geo() const {
    kvpop::Geometry g;
    g.batch = cfg.batch;
    g.n_q_heads = cfg.n_q_heads;
    g.n_kv_heads = cfg.n_kv_heads;
    g.head_dim = cfg.head_dim;
    g.n_sink = cfg.n_sink;
    g.n_scored = cfg.n_scored;
    g.n_recent = cfg.n_recent;
    g.slack = cfg.prune_interval;
    g.budget = int32_t(capacity_of(cfg));
    return g;
  }
  kvpop::LayerView layer(int32_t l) const {
    const size_t heads = size_t(cfg.batch) * cfg.n_kv_heads;
    const size_t budget = size_t(capacity_of(cfg));
    const size_t h0 = size_t(l) * heads;
    kvpop::LayerView v;
    v.kc = reinterpret_cast<uint16_t*>(base + lay.kc) + h0 * budget * cfg.head_dim;
    v.vc = reinterpret_cast<uint16_t*>(base + lay.vc) + h0 * budget * cfg.head_dim;
    v.keys = reinterpret_cast<uint64_t*>(base + lay.keys) + h0 * budget;
    v.pos = reinterpret_cast<int32_t*>(base + lay.pos) + h0 * budget;
    v.ring = reinterpret_cast<int32_t*>(base + lay.ring) + h0 * cfg.n_recent;
    v.ctl = reinterpret_cast<kvpop::HeadCtl*>(base + lay.ctl) + h0;
    return v;
  }
  // cache-wide index of the first KV head of (layer, seq)
  int64_t head0(int32_t l, int32_t s) const {
    return (int64_t(l) * cfg.batch + s) * cfg.n_kv_heads;
  }
  kvpop::PrefillWork prefill_work() const {
    kvpop::PrefillWork pw;
    pw.sel = reinterpret_cast<int32_t*>(base + lay.sel);
    pw.sel_items = lay.sel_items;
    pw.slice_keys = reinterpret_cast<uint64_t*>(base + lay.slice_keys);
    pw.slice_meta = reinterpret_cast<kvpop::SliceMeta*>(base + lay.slice_meta);
    pw.slice_tau = reinterpret_cast<uint32_t*>(base + lay.slice_tau);
    pw.slice_items = lay.slice_items;
    return pw;
  }
  kvpop::DecodeWork work() const {
    kvpop::DecodeWork w;
    w.part_acc = reinterpret_cast<float*>(base + lay.part_acc);
    w.part_ml = reinterpret_cast<float*>(base + lay.part_ml);
    w.part_min = reinterpret_cast<kvpop::MinPart*>(base + lay.part_min);
    w.tickets = reinterpret_cast<uint32_t*>(base + lay.tickets);
    w.nsplit = lay.nsplit;
    w.rows_per_split = lay.rows_per_split;
    w.threads = lay.threads;
    w.rows_per_thread = lay.rows_per_thread;
    w.finish_apart = lay.finish_apart;
    return w;
  }
};

namespace {

// Initialise the control blocks of the reset sequences among layers
// [l0, l1) x sequences [s0, s1): one launch per run of adjacent ones.
int flush_resets(kvpop_cache* cache, int32_t l0, int32_t l1, int32_t s0, int32_t s1,
                 hipStream_t stream) {
  if (cache->n_stale == 0) return KVPOP_OK;
  const int32_t B = cache->cfg.batch, Hkv = cache->cfg.n_kv_heads;
  for (int32_t l = l0; l < l1; ++l) {
    for (int32_t b = s0; b < s1;) {
      const size_t slot = size_t(l) * B + b;
      if (!cache->stale[slot]) {
        ++b;
        continue;
      }
      int32_t e = b;
      while (e < s1 && cache->stale[size_t(l) * B + e]) ++e;
      hipError_t err = kvpop::launch_init_ctl(cache->layer(l).ctl + size_t(b) * Hkv,
                                              int64_t(e - b) * Hkv, nullptr, 0, stream);
      if (err != hipSuccess) {
        cache->poisoned = true;
        return KVPOP_EHIP;
      }
      for (int32_t x = b; x < e; ++x) cache->stale[size_t(l) * B + x] = 0;
      cache->n_stale -= e - b;
      b = e;
    }
  }
  return KVPOP_OK;
}

// A non-empty prefill writes every control block of its sequence.
void mark_written(kvpop_cache* cache, size_t slot) {
  if (cache->stale[slot]) {
    cache->stale[slot] = 0;
    --cache->n_stale;
  }
}

}  // namespace

extern "C" {

size_t kvpop_cache_required_bytes(const kvpop_config* cfg) {
  if (!config_valid(cfg)) return 0;
  Layout L;
  if (!compute_layout(*cfg, &L)) return 0;
  return L.total;
}

int kvpop_cache_create(const kvpop_config* cfg, void* device_arena, size_t arena_bytes,
                       kvpop_cache** out) {
  if (out == nullptr) return KVPOP_EINVAL;
  *out = nullptr;
  if (!config_valid(cfg)) return KVPOP_EINVAL;
  Layout L;
  if (!compute_layout(*cfg, &L)) return KVPOP_EINVAL;
  if (device_arena != nullptr) {
    if (reinterpret_cast<uintptr_t>(device_arena) % ALIGN != 0) return KVPOP_EINVAL;
    if (arena_bytes < L.total) return KVPOP_ENOMEM;
  }
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return KVPOP_EHIP;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVPOP_EHIP;

  kvpop_cache* c = new (std::nothrow) kvpop_cache();
  if (c == nullptr) return KVPOP_ENOMEM;
  try {
    c->n_host.assign(size_t(cfg->n_layers) * cfg->batch, -1);
    c->stale.assign(size_t(cfg->n_layers) * cfg->batch, 0);
    c->steps.assign(size_t(cfg->n_layers), 0);
  } catch (...) {
    delete c;
    return KVPOP_ENOMEM;
  }
  c->cfg = *cfg;
  c->lay = L;
  c->device = dev;
  const float scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale
                                                : 1.0f / std::sqrt(float(cfg->head_dim));
  c->scale_log2e = scale * 1.4426950408889634f;
  if (device_arena != nullptr) {
    c->base = static_cast<char*>(device_arena);
    c->owns = false;
  } else {
    void* p = nullptr;
    if (hipMalloc(&p, L.total) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      delete c;
      return KVPOP_ENOMEM;
    }
    c->base = static_cast<char*>(p);
    c->owns = true;
  }
  const size_t heads_all = size_t(cfg->n_layers) * cfg->batch * cfg->n_kv_heads;
  hipError_t e = kvpop::launch_init_ctl(reinterpret_cast<kvpop::HeadCtl*>(c->base + L.ctl),
                                        int64_t(heads_all),
                                        reinterpret_cast<uint32_t*>(c->base + L.tickets),
                                        int64_t(heads_all) * kvpop::TICKET_STRIDE, nullptr);
  if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  if (e != hipSuccess) {
    if (c->owns) (void)hipFree(c->base);
    delete c;
    return KVPOP_EHIP;
  }
  // device address of the static workspace of the no-allocation entry
  // point; without it only that entry point is unavailable
  if (kvpop::future_scratch_address(&c->scratch) != hipSuccess) {
    (void)hipGetLastError();
    c->scratch = nullptr;
  }
  *out = c;
  return KVPOP_OK;
}

void kvpop_cache_destroy(kvpop_cache* cache) {
  if (cache == nullptr) return;
  if (cache->owns && cache->base != nullptr) {
    DeviceGuard dg(cache->device);
    (void)hipDeviceSynchronize();
    (void)hipFree(cache->base);
  }
  delete cache;
}

int kvpop_cache_reset(kvpop_cache* cache, int32_t layer, int32_t seq, void* stream) {
  (void)stream;  // nothing is enqueued here
  if (cache == nullptr) return KVPOP_EINVAL;
  if (layer < 0 || layer >= cache->cfg.n_layers || seq < 0 || seq >= cache->cfg.batch)
    return KVPOP_EINVAL;
  if (cache->poisoned) return KVPOP_ESTATE;
  const size_t slot = size_t(layer) * cache->cfg.batch + seq;
  cache->n_host[slot] = -1;
  if (!cache->stale[slot]) {
    cache->stale[slot] = 1;
    ++cache->n_stale;
  }
  return KVPOP_OK;
}

int kvpop_prefill_compact(kvpop_cache* cache, int32_t layer, int32_t seq, int32_t n_tokens,
                          const uint16_t* k, const uint16_t* v, const float* scores,
                          void* stream) {
  if (cache == nullptr) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (layer < 0 || layer >= c.n_layers || seq < 0 || seq >= c.batch || n_tokens < 0)
    return KVPOP_EINVAL;
  if (cache->poisoned) return KVPOP_ESTATE;
  int32_t& nh = cache->n_host[size_t(layer) * c.batch + seq];
  if (nh != -1) return KVPOP_ESTATE;
  if (n_tokens > c.max_positions) return KVPOP_ESTATE;
  if (n_tokens == 0) return KVPOP_OK;
  if (k == nullptr || v == nullptr || scores == nullptr) return KVPOP_EINVAL;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  kvpop::PrefillItem it;
  it.k = k;
  it.v = v;
  it.scores = scores;
  it.n_tokens = n_tokens;
  it.head0 = cache->head0(layer, seq);
  hipError_t e = kvpop::launch_prefill_batch(cache->geo(), cache->layer(0), &it, 1,
                                             cache->prefill_work(),
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  nh = n_tokens - 1;
  mark_written(cache, size_t(layer) * c.batch + seq);
  return KVPOP_OK;
}

int kvpop_prefill_compact_batch(kvpop_cache* cache, int32_t n_items,
                                const kvpop_prefill_item* items, void* stream) {
  if (cache == nullptr || n_items < 0 || (n_items > 0 && items == nullptr)) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  // validate everything before anything is enqueued
  for (int32_t i = 0; i < n_items; ++i) {
    const kvpop_prefill_item& x = items[i];
    if (x.layer < 0 || x.layer >= c.n_layers || x.seq < 0 || x.seq >= c.batch || x.n_tokens < 0)
      return KVPOP_EINVAL;
    if (x.n_tokens > 0 && (x.k == nullptr || x.v == nullptr || x.scores == nullptr))
      return KVPOP_EINVAL;
  }
  if (cache->poisoned) return KVPOP_ESTATE;
  std::vector<kvpop::PrefillItem> its;
  std::vector<size_t> slots;
  try {
    its.reserve(size_t(n_items));
    slots.reserve(size_t(n_items));
  } catch (...) {
    return KVPOP_ENOMEM;
  }
  for (int32_t i = 0; i < n_items; ++i) {
    const kvpop_prefill_item& x = items[i];
    const size_t slot = size_t(x.layer) * c.batch + x.seq;
    if (cache->n_host[slot] != -1 || x.n_tokens > c.max_positions) return KVPOP_ESTATE;
    if (std::find(slots.begin(), slots.end(), slot) != slots.end()) return KVPOP_EINVAL;
    slots.push_back(slot);
    kvpop::PrefillItem it;
    it.k = x.k;
    it.v = x.v;
    it.scores = x.scores;
    it.n_tokens = x.n_tokens;
    it.head0 = cache->head0(x.layer, x.seq);
    its.push_back(it);
  }
  if (n_items == 0) return KVPOP_OK;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  hipError_t e = kvpop::launch_prefill_batch(cache->geo(), cache->layer(0), its.data(), n_items,
                                             cache->prefill_work(),
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  for (int32_t i = 0; i < n_items; ++i)
    if (items[i].n_tokens > 0) {
      cache->n_host[slots[size_t(i)]] = items[i].n_tokens - 1;
      mark_written(cache, slots[size_t(i)]);
    }
  return KVPOP_OK;
}

int kvpop_prefix_thresholds(kvpop_cache* cache, int32_t n_tokens, const float* scores,
                            uint64_t* thr, void* stream) {
  if (cache == nullptr || n_tokens < 0) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (c.n_scored > kvpop::THR_KMAX) return KVPOP_EINVAL;
  if (cache->poisoned) return KVPOP_ESTATE;
  if (n_tokens > c.max_positions) return KVPOP_ESTATE;
  if (n_tokens == 0) return KVPOP_OK;
  if (scores == nullptr || thr == nullptr) return KVPOP_EINVAL;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  // the first-level prefill buffer (free between calls) holds the segment starts
  const kvpop::PrefillWork pw = cache->prefill_work();
  const int64_t ws_keys = int64_t(pw.slice_items) * c.n_kv_heads * kvpop::SLICE_MAX *
                          kvpop::slice_stride(c.n_scored);
  hipError_t e = kvpop::launch_prefix_thresholds(cache->geo(), n_tokens, scores, thr,
                                                 pw.slice_keys, ws_keys,
                                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  return KVPOP_OK;
}

int kvpop_future_attention_target(kvpop_cache* cache, int32_t n_tokens, const uint16_t* q,
                                  const uint16_t* k, float* work, float* y, void* stream) {
  if (cache == nullptr || n_tokens < 0) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (cache->poisoned) return KVPOP_ESTATE;
  if (n_tokens > c.max_positions) return KVPOP_ESTATE;
  if (n_tokens == 0) return KVPOP_OK;
  if (q == nullptr || k == nullptr || work == nullptr || y == nullptr) return KVPOP_EINVAL;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  hipError_t e = kvpop::launch_future_target(cache->geo(), n_tokens, q, k, cache->scale_log2e,
                                             work, y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  return KVPOP_OK;
}

int kvpop_future_attention_target_noalloc(kvpop_cache* cache, int32_t n_tokens,
                                          const uint16_t* q, const uint16_t* k, float* y,
                                          void* stream) {
  if (cache == nullptr || n_tokens < 0) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (cache->poisoned) return KVPOP_ESTATE;
  if (n_tokens > c.max_positions) return KVPOP_ESTATE;
  if (size_t(2) * size_t(c.n_q_heads) * size_t(n_tokens) * sizeof(float) >
      kvpop::FUTURE_SCRATCH_BYTES)
    return KVPOP_ERANGE;
  if (n_tokens == 0) return KVPOP_OK;
  if (q == nullptr || k == nullptr || y == nullptr) return KVPOP_EINVAL;
  if (cache->scratch == nullptr) return KVPOP_EHIP;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  hipError_t e = kvpop::launch_future_target(cache->geo(), n_tokens, q, k, cache->scale_log2e,
                                             cache->scratch, y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  return KVPOP_OK;
}

int kvpop_decode_step(kvpop_cache* cache, int32_t layer, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, const float* score_leaving, uint16_t* out,
                      void* stream) {
  if (cache == nullptr) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (layer < 0 || layer >= c.n_layers) return KVPOP_EINVAL;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || score_leaving == nullptr ||
      out == nullptr)
    return KVPOP_EINVAL;
  if (cache->poisoned) return KVPOP_ESTATE;
  int32_t* nh = cache->n_host.data() + size_t(layer) * c.batch;
  for (int32_t b = 0; b < c.batch; ++b)
    if (int64_t(nh[b]) + 1 >= c.max_positions) return KVPOP_ESTATE;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  if (int r = flush_resets(cache, layer, layer + 1, 0, c.batch, static_cast<hipStream_t>(stream)))
    return r;
  hipError_t e = kvpop::launch_decode(cache->geo(), cache->layer(layer), cache->work(), 1, q,
                                      k_new, v_new, score_leaving, out, cache->scale_log2e,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  for (int32_t b = 0; b < c.batch; ++b) nh[b] += 1;
  // Dynamic backend: after every prune_interval-th step of the layer, cut
  // every head back to the budget
  if (c.prune_interval > 0 && ++cache->steps[size_t(layer)] % c.prune_interval == 0) {
    e = kvpop::launch_prune(cache->geo(), cache->layer(layer), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
      cache->poisoned = true;
      return KVPOP_EHIP;
    }
  }
  return KVPOP_OK;
}

int kvpop_decode_step_layers(kvpop_cache* cache, int32_t layer0, int32_t n_layers,
                             const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                             const float* score_leaving, uint16_t* out, void* stream) {
  if (cache == nullptr) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (layer0 < 0 || n_layers < 1 || int64_t(layer0) + n_layers > c.n_layers) return KVPOP_EINVAL;
  if (q == nullptr || k_new == nullptr || v_new == nullptr || score_leaving == nullptr ||
      out == nullptr)
    return KVPOP_EINVAL;
  if (cache->poisoned) return KVPOP_ESTATE;
  int32_t* nh = cache->n_host.data() + size_t(layer0) * c.batch;
  for (int64_t i = 0; i < int64_t(n_layers) * c.batch; ++i)
    if (int64_t(nh[i]) + 1 >= c.max_positions) return KVPOP_ESTATE;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  if (int r = flush_resets(cache, layer0, layer0 + n_layers, 0, c.batch,
                           static_cast<hipStream_t>(stream)))
    return r;
  kvpop::DecodeWork w = cache->work();
  const int64_t ns = decode_splits_for(c, int64_t(n_layers) * c.batch * c.n_kv_heads, true);
  w.nsplit = int32_t(ns);
  w.rows_per_split = rows_per_split_for(c, ns);
  w.finish_apart = (c.decode_finish == 1) ? 0 : 1;  // the second launch unless asked
  hipError_t e = kvpop::launch_decode(cache->geo(), cache->layer(layer0), w, n_layers, q, k_new,
                                      v_new, score_leaving, out, cache->scale_log2e,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  for (int64_t i = 0; i < int64_t(n_layers) * c.batch; ++i) nh[i] += 1;
  if (c.prune_interval > 0) {
    for (int32_t l = layer0; l < layer0 + n_layers; ++l) {
      if (++cache->steps[size_t(l)] % c.prune_interval != 0) continue;
      e = kvpop::launch_prune(cache->geo(), cache->layer(l), static_cast<hipStream_t>(stream));
      if (e != hipSuccess) {
        cache->poisoned = true;
        return KVPOP_EHIP;
      }
    }
  }
  return KVPOP_OK;
}

int kvpop_cache_prune(kvpop_cache* cache, int32_t layer, void* stream) {
  if (cache == nullptr) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (layer < 0 || layer >= c.n_layers) return KVPOP_EINVAL;
  if (cache->poisoned) return KVPOP_ESTATE;
  if (c.prune_interval == 0) return KVPOP_OK;  // Static: never above the budget
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  if (int r = flush_resets(cache, layer, layer + 1, 0, c.batch, static_cast<hipStream_t>(stream)))
    return r;
  hipError_t e =
      kvpop::launch_prune(cache->geo(), cache->layer(layer), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  return KVPOP_OK;
}

int kvpop_cache_state(kvpop_cache* cache, int32_t layer, int32_t seq, kvpop_state* st,
                      int32_t* counts, int32_t* kept_pos, void* stream) {
  if (cache == nullptr || st == nullptr) return KVPOP_EINVAL;
  const kvpop_config& c = cache->cfg;
  if (layer < 0 || layer >= c.n_layers || seq < 0 || seq >= c.batch) return KVPOP_EINVAL;
  DeviceGuard dg(cache->device);
  if (!dg.ok) return KVPOP_EHIP;
  if (cache->stale[size_t(layer) * c.batch + seq]) {
    if (cache->poisoned) return KVPOP_ESTATE;
    if (int r = flush_resets(cache, layer, layer + 1, seq, seq + 1,
                             static_cast<hipStream_t>(stream)))
      return r;
  }
  const int32_t Hkv = c.n_kv_heads;
  const size_t budget = size_t(capacity_of(c));
  std::vector<kvpop::HeadCtl> ctl;
  std::vector<int32_t> pos;
  try {
    ctl.resize(Hkv);
    pos.resize(size_t(Hkv) * budget);
  } catch (...) {
    return KVPOP_ENOMEM;
  }
  kvpop::LayerView lv = cache->layer(layer);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(ctl.data(), lv.ctl + size_t(seq) * Hkv,
                                sizeof(kvpop::HeadCtl) * Hkv, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(pos.data(), lv.pos + size_t(seq) * Hkv * budget,
                       sizeof(int32_t) * pos.size(), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    cache->poisoned = true;
    return KVPOP_EHIP;
  }
  st->n = ctl[0].n;
  st->flags = 0;
  for (int32_t g = 0; g < Hkv; ++g) {
    st->flags |= ctl[g].flags;
    const int32_t cnt = std::max(0, std::min<int32_t>(ctl[g].count, int32_t(budget)));
    if (counts != nullptr) counts[g] = cnt;
    if (kept_pos != nullptr) {
      int32_t* dst = kept_pos + size_t(g) * budget;
      std::copy(pos.begin() + size_t(g) * budget, pos.begin() + size_t(g) * budget + cnt, dst);
      std::sort(dst, dst + cnt);
      std::fill(dst + cnt, dst + budget, -1);
    }
  }
  return KVPOP_OK;
}

const char* kvpop_strerror(int code) {
  switch (code) {
    case KVPOP_OK: return "success";
    case KVPOP_EINVAL: return "invalid argument";
    case KVPOP_ENOMEM: return "out of device memory or arena too small";
    case KVPOP_EHIP: return "HIP runtime error";
    case KVPOP_ESTATE: return "call out of order, cache poisoned, or position limit reached";
    case KVPOP_ERANGE: return "input larger than the static workspace of a no-allocation entry point";
    default: return "unknown error";
  }
}

}  // extern "C"
