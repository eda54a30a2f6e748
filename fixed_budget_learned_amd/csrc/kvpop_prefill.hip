// Prefill compaction for gfx950: fill an empty (layer, sequence) of the
// fixed-budget cache from a P-token prompt.
//
// The kept set after position P-1 is the sinks {0..s-1}, the window
// {max(s, P-W)..P-1} and the k candidates of {s..P-W-1} with the largest
// (score, position) keys ("Qwen3-8B-KVpop-4x" model card, intro: sink +
// scored top-k + recent window; the window's scores arrive later, when each
// token leaves it, per the card's "Delayed scoring").
//
// Two kernels per call:
//   select  one 1024-thread workgroup per KV head; each thread owns a
//           contiguous block of candidate positions (kept in registers when
//           it is at most 32 long).  A radix select with 12, 12 and 8-bit
//           digits over the order-preserving score codes (one 4096-bin LDS
//           histogram) finds the threshold code and how many tokens carrying
//           it survive; one workgroup scan of per-thread (greater, equal)
//           counts then places every code above the threshold and the newest
//           of the tied ones, writing the kept positions in ascending order
//           plus the head's control block (count, min key and its slot).
//   gather  many 256-thread workgroups per head copy the kept K/V rows into
//           slots [0, count) with 16-byte coalesced loads/stores and write
//           per-slot position and key, and the window ring.
// A batch of (layer, sequence) prompts shares one select and one gather
// launch: the grid's z is the prompt, each reading its own descriptor from
// the kernel arguments (up to PREFILL_NB = 64 per launch, 3.6 KB of arguments).
// Slot layout after prefill: sinks, then selected candidates in ascending
// position, then the window in ascending position.
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int SEL_THREADS = 1024;
constexpr int GATHER_THREADS = 256;

struct PrefillShape {
  int32_t P;       // prompt length
  int32_t s_eff;   // sinks present: min(s, P)
  int32_t c0, c1;  // candidate positions [c0, c1)
  int32_t kk;      // scored slots filled: min(k, c1 - c0)
  int32_t w0;      // first window position
  int32_t count;   // s_eff + kk + (P - w0)
  int32_t leave;   // slot of position P - W (leaves at the next step) or -1
};

__host__ __device__ inline PrefillShape prefill_shape(int32_t P, int32_t s, int32_t k, int32_t W) {
  PrefillShape r;
  r.P = P;
  r.s_eff = P < s ? P : s;
  r.c0 = s;
  r.c1 = P - W;
  if (r.c1 < r.c0) r.c1 = r.c0;
  int32_t C = r.c1 - r.c0;
  r.kk = k < C ? k : C;
  r.w0 = (P - W) > s ? (P - W) : s;
  if (r.w0 > P) r.w0 = P;
  r.count = r.s_eff + r.kk + (P - r.w0);
  // position P - W, when it is not a sink, is the oldest window token and
  // sits in the first window slot
  r.leave = (P - W >= s) ? r.s_eff + r.kk : -1;
  return r;
}

// Radix digits over the 32-bit code: 12, 12 and 8 bits (4096-bin histogram),
// or 11, 11 and 10 bits (2048 bins) where the smaller histogram lets two
// workgroups share a compute unit's LDS (16 codes per thread, not the list
// mode).
constexpr int NBINS = 4096;
constexpr int TILE_LG = 5;   // streamed compaction: tiles of 32 candidates per thread

// Coalesced load of candidates [0, n) at `sc` into LDS as order codes, laid
// out thread-contiguously: candidate i belongs to thread i >> lg, entry
// i & (2^lg - 1), stored at (i >> lg) * (2^lg + 1) + (i & (2^lg - 1)); the pad
// word keeps the 64 lanes of a wave in distinct banks when each then reads
// its own block.  U loads per thread are in flight at once (U * 1024 >= n
// makes it one round trip).  Returns whether this thread saw a NaN.
template <int U>
__device__ __forceinline__ bool stage_codes(const float* __restrict__ sc, int32_t n, int lg,
                                            uint32_t* stage) {
  const int32_t L = 1 << lg;
  bool nan = false;
  for (int32_t i0 = threadIdx.x; i0 < n; i0 += SEL_THREADS * U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = sc[min(i0 + u * SEL_THREADS, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t i = i0 + u * SEL_THREADS;
      if (i < n) {
        nan |= score_is_nan(x[u]);
        stage[(i >> lg) * (L + 1) + (i & (L - 1))] = score_code(x[u]);
      }
    }
  }
  return nan;
}

// f(code) for every candidate [0, n) at `sc`, read with coalesced loads, U
// per thread in flight (the order of the calls is unspecified).  With
// check_nan, *nan collects NaNs.
template <int U, typename F>
__device__ __forceinline__ void stream_codes(const float* __restrict__ sc, int32_t n, bool check_nan,
                                             bool* nan, F&& f) {
  for (int32_t i0 = threadIdx.x; i0 < n; i0 += SEL_THREADS * U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = sc[min(i0 + u * SEL_THREADS, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * SEL_THREADS < n) {
        if (check_nan) *nan |= score_is_nan(x[u]);
        f(score_code(x[u]));
      }
    }
  }
}

// One radix pass over the codes that match `prefix` under `mask`: histogram
// of the digit (code >> shift) & (nbins - 1), then the bin that holds the
// krem-th largest matching code.  Results land in *s_bin, *s_above (matching
// codes in higher bins) and *s_neq (codes in the bin).  All threads call it.
template <typename Visit>
__device__ __forceinline__ void radix_pass(Visit&& visit, uint32_t prefix, uint32_t mask, int shift,
                                           int nbins, uint32_t krem, uint32_t* hist,
                                           uint32_t* scan_buf, uint32_t* s_bin, uint32_t* s_above,
                                           uint32_t* s_neq) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += SEL_THREADS) hist[i] = 0;
  __syncthreads();
  visit([&](uint32_t o) {
    if ((o & mask) == prefix) atomicAdd(&hist[(o >> shift) & static_cast<uint32_t>(nbins - 1)], 1u);
  });
  __syncthreads();
  // thread t holds bins nbins-1-4t down to nbins-4-4t
  uint32_t hb[4], h = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int bin = nbins - 1 - 4 * tid - q;
    hb[q] = bin >= 0 ? hist[bin] : 0u;
    h += hb[q];
  }
  uint32_t tot;
  uint32_t ex = block_exclusive_scan_u32<SEL_THREADS>(h, scan_buf, &tot);
  if (ex < krem && krem <= ex + h) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (krem <= ex + hb[q]) {
        *s_bin = static_cast<uint32_t>(nbins - 1 - 4 * tid - q);
        *s_above = ex;
        *s_neq = hb[q];
        break;
      }
      ex += hb[q];
    }
  }
  __syncthreads();
}

// Select kernels.  1024 threads per workgroup; MODE:
//   SEL_HEAD   one workgroup per KV head selects from all its candidates.
//              VPT 16 / 32: each thread holds a contiguous block of at most
//              VPT candidate codes in registers (staged through LDS from
//              coalesced loads); VPT 0: the scores are streamed on every pass
//              and compacted in LDS-staged tiles (fallback for any length).
//   SEL_SLICE  first level for long prompts: workgroup (head, slice) selects
//              the top min(k, slice length) of a slice of the candidates and
//              writes their keys, ascending in position, padded with key 0 to
//              k entries.  The global top-k lies in the union of the slices'
//              top-k, since a slice contributes at most k of it.
//   SEL_LIST   second level: one workgroup per head selects the top k of that
//              union (read as keys, in position order) and writes positions
//              and the control block like SEL_HEAD.
constexpr int SEL_HEAD = 0, SEL_SLICE = 1, SEL_LIST = 2;

struct SelectArgs {
  const float* scores;   // [Hkv][P] of this prompt
  PrefillShape sh;
  int32_t k;             // scored slots (stride of the selection buffers)
  int32_t* sel;          // [Hkv][k] kept candidate positions, ascending
  HeadCtl* ctl;          // [Hkv]
  uint64_t* slice_keys;  // [Hkv][SLICE_MAX][k] first-level keys
  int32_t* slice_nan;    // [Hkv][SLICE_MAX] first-level NaN flags
  int32_t n_slices, slice_len;
};

// One prompt of a select launch.  head0: the cache-wide index of its
// (layer, sequence)'s first KV head.
struct SelectItem {
  const float* scores;   // [Hkv][P]
  int32_t* sel;          // [Hkv][k] selection slot of the prompt
  uint64_t* slice_keys;  // [Hkv][SLICE_MAX][k] first-level slot of the prompt
  int32_t* slice_nan;    // [Hkv][SLICE_MAX]
  int64_t head0;
  int32_t P, n_slices, slice_len;
};

// Descriptors of the prompts of one launch (grid z = prompt), with what they
// share; kept small enough for the kernel arguments.
template <int NB>
struct SelectBatch {
  HeadCtl* ctl;          // cache-wide control blocks
  int32_t s, k, W;
  SelectItem item[NB];
};

// Occupancy hint: with 16 codes per thread (and not the list mode, whose
// 64-bit staging allows one workgroup per compute unit) two workgroups share
// a compute unit, 8 waves per SIMD.  They fit that many without the hint, but
// with it the compiler schedules for it: the two-level first level of a
// 131k-token prompt ran 134 -> 89 us in a 36-layer batched launch.
template <int VPT, int MODE, int NB>
__global__ __launch_bounds__(SEL_THREADS)
__attribute__((amdgpu_waves_per_eu(VPT == 16 && MODE != SEL_LIST ? 8 : 1)))
void prefill_select_kernel(SelectBatch<NB> batch) {
  const SelectItem& it = batch.item[blockIdx.z];
  SelectArgs a;
  a.scores = it.scores;
  a.sh = prefill_shape(it.P, batch.s, batch.k, batch.W);
  a.k = batch.k;
  a.sel = it.sel;
  a.ctl = batch.ctl + it.head0;
  a.slice_keys = it.slice_keys;
  a.slice_nan = it.slice_nan;
  a.n_slices = it.n_slices;
  a.slice_len = it.slice_len;
  // a batch launch covers its longest prompt's slices: shorter ones have none here
  if (MODE == SEL_SLICE && static_cast<int32_t>(blockIdx.y) >= a.n_slices) return;
  static_assert(MODE != SEL_LIST || VPT == 16, "list mode stages 64-bit keys: at most 16 per thread");
  static_assert(MODE == SEL_HEAD || VPT > 0, "slice and list modes keep codes in registers");
  constexpr int NWAVE = SEL_THREADS / WAVE;
  constexpr int LMAX = VPT > 0 ? VPT : (1 << TILE_LG);
  constexpr int STAGE_WORDS = (MODE == SEL_LIST ? 2 : 1) * SEL_THREADS * (LMAX + 1);
  constexpr bool NARROW = (VPT == 16 && MODE != SEL_LIST);
  constexpr int HBINS = NARROW ? NBINS / 2 : NBINS;
  constexpr int SH0 = NARROW ? 21 : 20, SH1 = NARROW ? 10 : 8, LAST = NARROW ? 1024 : 256;
  __shared__ uint32_t hist[HBINS];
  __shared__ __align__(16) uint32_t stage[STAGE_WORDS];
  __shared__ uint32_t scan_buf[NWAVE + 1];
  __shared__ uint32_t s_bin, s_above, s_nan, s_neq;
  __shared__ int32_t s_minslot;
  __shared__ uint64_t s_minkey;
  __shared__ uint64_t s_wmk[NWAVE];
  __shared__ int32_t s_wmp[NWAVE];

  const PrefillShape& sh = a.sh;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int wid = tid / WAVE;
  const int32_t kst = a.k > 0 ? a.k : 1;  // stride of the per-head buffers
  int32_t* out = a.sel + static_cast<int64_t>(g) * kst;
  // this workgroup's candidates: [cb, cb + C) of the head's candidate range
  // (SEL_LIST: entries of the head's first-level key list)
  int32_t cb = 0, C = sh.c1 - sh.c0, kk = sh.kk;
  if constexpr (MODE == SEL_SLICE) {
    cb = static_cast<int32_t>(blockIdx.y) * a.slice_len;
    C = min(a.slice_len, sh.c1 - sh.c0 - cb);
    kk = min(a.k, C);
  } else if constexpr (MODE == SEL_LIST) {
    C = a.n_slices * a.k;
  }
  const float* sc = a.scores + static_cast<int64_t>(g) * sh.P + sh.c0 + cb;  // candidate 0
  const int64_t list0 = (static_cast<int64_t>(g) * SLICE_MAX) * a.k;
  uint64_t* outk = a.slice_keys + list0 + static_cast<int64_t>(blockIdx.y) * a.k;

  if (tid == 0) {
    s_nan = 0;
    s_minslot = -1;
    s_minkey = KEY_NONE;
  }
  __syncthreads();
  if constexpr (MODE == SEL_LIST) {
    if (tid < a.n_slices && a.slice_nan[g * SLICE_MAX + tid]) s_nan = 1;
  }

  // smallest (code, position) over the workgroup -> s_minkey and its slot
  auto publish_min = [&](uint64_t mk, int32_t mpos) {
    wave_min_key(mk, mpos);
    if ((tid & (WAVE - 1)) == 0) {
      s_wmk[wid] = mk;
      s_wmp[wid] = mpos;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NWAVE; ++w)
        if (s_wmk[w] < mk) {
          mk = s_wmk[w];
          mpos = s_wmp[w];
        }
      s_minkey = mk;
      s_minslot = sh.s_eff + (mpos - sh.c0);
    }
  };
  // where the kept candidate of rank idx goes
  auto emit = [&](uint32_t idx, int32_t pos, uint32_t code) {
    if constexpr (MODE == SEL_SLICE)
      outk[idx] = make_key(code, pos);
    else
      out[idx] = pos;
  };

  if (kk > 0 && VPT > 0) {
    // ---- codes (and list positions) into registers: thread-contiguous
    // blocks of L = 2^lg entries ----------------------------------------------
    int lg = 0;
    while ((SEL_THREADS << lg) < C) ++lg;
    const int32_t L = 1 << lg;
    uint32_t code[LMAX];
    int32_t lpos[MODE == SEL_LIST ? LMAX : 1];
    if constexpr (MODE == SEL_LIST) {
      // coalesced loads of the keys, transposed through LDS like the codes
      uint64_t* st64 = reinterpret_cast<uint64_t*>(stage);
      const uint64_t* lk = a.slice_keys + list0;
      constexpr int U = 16;
      for (int32_t i0 = tid; i0 < C; i0 += SEL_THREADS * U) {
        uint64_t x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = lk[min(i0 + u * SEL_THREADS, C - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int32_t i = i0 + u * SEL_THREADS;
          if (i < C) st64[(i >> lg) * (L + 1) + (i & (L - 1))] = x[u];
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < LMAX; ++j) {
        const uint64_t key = (j < L) ? st64[tid * (L + 1) + j] : 0ull;
        code[j] = static_cast<uint32_t>(key >> 32);
        lpos[j] = static_cast<int32_t>(static_cast<uint32_t>(key));
      }
    } else {
      const bool nan = stage_codes<LMAX>(sc, C, lg, stage);
      if (nan) s_nan = 1;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < LMAX; ++j) code[j] = (j < L) ? stage[tid * (L + 1) + j] : 0u;
    }
    const int32_t lo = min(tid * L, C), hi = min(lo + L, C);  // workgroup-relative
    auto for_each = [&](auto&& f) {
#pragma unroll
      for (int j = 0; j < LMAX; ++j) {
        if (lo + j < hi) {
          int32_t pos;
          if constexpr (MODE == SEL_LIST)
            pos = lpos[j];
          else
            pos = sh.c0 + cb + lo + j;
          f(lo + j, pos, code[j]);
        }
      }
    };

    if (kk == C) {
      // every candidate is kept: positions in order; the least important one
      // is the smallest (code, position)
      uint64_t mk = KEY_NONE;
      int32_t mpos = 0x7FFFFFFF;
      for_each([&](int32_t r, int32_t i, uint32_t o) {
        emit(static_cast<uint32_t>(r), i, o);
        const uint64_t key = make_key(o, i);
        if (key < mk) {
          mk = key;
          mpos = i;
        }
      });
      if constexpr (MODE != SEL_SLICE) publish_min(mk, mpos);
    } else {
      // ---- radix select of the kk-th largest code: three digits --------
      uint32_t prefix = 0, mask = 0, krem = static_cast<uint32_t>(kk);
      auto visit = [&](auto&& f) { for_each([&](int32_t, int32_t, uint32_t o) { f(o); }); };
      const int shifts[3] = {SH0, SH1, 0}, nbins[3] = {HBINS, HBINS, LAST};
#pragma unroll
      for (int ps = 0; ps < 3; ++ps) {
        radix_pass(visit, prefix, mask, shifts[ps], nbins[ps], krem, hist, scan_buf, &s_bin,
                   &s_above, &s_neq);
        krem -= s_above;
        prefix |= s_bin << shifts[ps];
        mask |= static_cast<uint32_t>(nbins[ps] - 1) << shifts[ps];
      }
      // ---- ordered compaction: codes above the threshold, then the newest
      // krem tokens carrying it (ties: the older ones lose) ------------------
      const uint32_t thr = prefix;
      const uint32_t drop = s_neq - krem;
      uint32_t gt = 0, eq = 0;
      for_each([&](int32_t, int32_t, uint32_t o) {
        gt += o > thr;
        eq += o == thr;
      });
      uint32_t tot;
      const uint32_t ex = block_exclusive_scan_u32<SEL_THREADS>((eq << 16) | gt, scan_buf, &tot);
      uint32_t eq_before = ex >> 16, gt_before = ex & 0xFFFFu;
      for_each([&](int32_t, int32_t i, uint32_t o) {
        const bool is_gt = o > thr, is_eq = o == thr;
        if (is_gt || (is_eq && eq_before >= drop)) {
          const uint32_t idx = gt_before + (eq_before > drop ? eq_before - drop : 0u);
          emit(idx, i, o);
          if (is_eq && eq_before == drop) {  // the least important kept token
            s_minslot = sh.s_eff + static_cast<int32_t>(idx);
            s_minkey = make_key(thr, i);
          }
        }
        gt_before += is_gt;
        eq_before += is_eq;
      });
    }
  } else if (kk > 0) {
    // ---- SEL_HEAD, long prompts: stream the scores on every pass -----------
    bool nan = false;
    if (kk == C) {
      uint64_t mk = KEY_NONE;
      int32_t mpos = 0x7FFFFFFF;
      for (int32_t i = tid; i < C; i += SEL_THREADS) {
        const float x = sc[i];
        nan |= score_is_nan(x);
        out[i] = sh.c0 + i;
        const uint64_t key = make_key(score_code(x), sh.c0 + i);
        if (key < mk) {
          mk = key;
          mpos = sh.c0 + i;
        }
      }
      if (nan) s_nan = 1;
      publish_min(mk, mpos);
    } else {
      uint32_t prefix = 0, mask = 0, krem = static_cast<uint32_t>(kk);
      const int shifts[3] = {SH0, SH1, 0}, nbins[3] = {HBINS, HBINS, LAST};
#pragma unroll
      for (int ps = 0; ps < 3; ++ps) {
        auto visit = [&](auto&& f) { stream_codes<16>(sc, C, ps == 0, &nan, f); };
        radix_pass(visit, prefix, mask, shifts[ps], nbins[ps], krem, hist, scan_buf, &s_bin,
                   &s_above, &s_neq);
        krem -= s_above;
        prefix |= s_bin << shifts[ps];
        mask |= static_cast<uint32_t>(nbins[ps] - 1) << shifts[ps];
      }
      if (nan) s_nan = 1;
      const uint32_t thr = prefix;
      const uint32_t drop = s_neq - krem;
      // ordered compaction in tiles of 32 candidates per thread, staged
      // through LDS so that each thread walks a contiguous block
      constexpr int TL = 1 << TILE_LG;
      uint32_t gt_base = 0, eq_base = 0;
      for (int32_t t0 = 0; t0 < C; t0 += SEL_THREADS * TL) {
        const int32_t n = min(SEL_THREADS * TL, C - t0);
        stage_codes<16>(sc + t0, n, TILE_LG, stage);
        __syncthreads();
        uint32_t tcode[TL];
#pragma unroll
        for (int j = 0; j < TL; ++j) tcode[j] = stage[tid * (TL + 1) + j];
        const int32_t lo = min(tid * TL, n), hi = min(lo + TL, n);  // tile-relative
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < TL; ++j)
          if (lo + j < hi) {
            gt += tcode[j] > thr;
            eq += tcode[j] == thr;
          }
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan_u32<SEL_THREADS>((eq << 16) | gt, scan_buf, &tot);
        uint32_t eq_before = eq_base + (ex >> 16), gt_before = gt_base + (ex & 0xFFFFu);
#pragma unroll
        for (int j = 0; j < TL; ++j) {
          if (lo + j < hi) {
            const uint32_t o = tcode[j];
            const int32_t i = sh.c0 + t0 + lo + j;
            const bool is_gt = o > thr, is_eq = o == thr;
            if (is_gt || (is_eq && eq_before >= drop)) {
              const uint32_t idx = gt_before + (eq_before > drop ? eq_before - drop : 0u);
              out[idx] = i;
              if (is_eq && eq_before == drop) {
                s_minslot = sh.s_eff + static_cast<int32_t>(idx);
                s_minkey = make_key(thr, i);
              }
            }
            gt_before += is_gt;
            eq_before += is_eq;
          }
        }
        gt_base += tot & 0xFFFFu;
        eq_base += tot >> 16;
        __syncthreads();  // the stage is refilled by the next tile
      }
    }
  }
  if constexpr (MODE == SEL_SLICE) {
    // pad the slice's list to k entries with the smallest key; record NaNs
    for (int32_t j = kk + tid; j < a.k; j += SEL_THREADS) outk[j] = 0ull;
    __syncthreads();
    if (tid == 0) a.slice_nan[g * SLICE_MAX + blockIdx.y] = s_nan ? 1 : 0;
    return;
  }
  __syncthreads();
  if (tid == 0) {
    HeadCtl c;
    c.n = sh.P - 1;
    c.count = sh.count;
    c.nscored = sh.kk;
    c.minslot = s_minslot;
    c.minkey = s_minkey;
    c.flags = s_nan ? 1 : 0;
    c.leave_slot = sh.leave;
    a.ctl[g] = c;
  }
}

// One prompt of a gather launch: its inputs, selection and destination
// (the cache rows of its (layer, sequence), head 0).
struct GatherItem {
  const uint16_t* k;     // [Hkv][P][D]
  const uint16_t* v;
  const float* scores;   // [Hkv][P]
  const int32_t* sel;    // [Hkv][k] its selection
  int64_t head0;         // cache-wide index of its first KV head
  int32_t P;
};

template <int NB>
struct GatherBatch {
  uint16_t* kc;          // cache-wide rows and slot metadata
  uint16_t* vc;
  uint64_t* keys;
  int32_t* pos;
  int32_t* ring;
  int32_t s, k, W, budget, rows_per_block;
  GatherItem item[NB];
};

// 16-byte loads and stores that do not allocate in the caches: the prompt's
// rows are read once and the cache rows are not read again by this launch.
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load16(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store16(uint4 x, uint4* p) {
  const u32x4_nt v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_nt*>(p));
}

// One gather workgroup: 256 threads, D/8 lanes of 16 bytes per kept row.
template <int D, int NB>
__global__ __launch_bounds__(GATHER_THREADS) void prefill_gather_kernel(GatherBatch<NB> batch) {
  constexpr int LPR = D / 8;                   // lanes per row (16 B each)
  constexpr int RPP = GATHER_THREADS / LPR;    // rows per pass
  const GatherItem& it = batch.item[blockIdx.z];
  const PrefillShape sh = prefill_shape(it.P, batch.s, batch.k, batch.W);
  const int32_t kcap = batch.k > 0 ? batch.k : 1;
  const int32_t budget = batch.budget, W = batch.W, rows_per_block = batch.rows_per_block;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int rg = tid / LPR;
  const int c = tid % LPR;
  const int32_t r0 = blockIdx.x * rows_per_block;
  const int32_t r1 = min(r0 + rows_per_block, sh.count);  // empty past this prompt's rows
  const uint16_t* __restrict__ k = it.k;
  const uint16_t* __restrict__ v = it.v;
  const float* __restrict__ scores = it.scores;
  const int32_t* __restrict__ sel = it.sel;
  const int64_t row0 = it.head0 * budget;
  uint16_t* __restrict__ kc = batch.kc + row0 * D;
  uint16_t* __restrict__ vc = batch.vc + row0 * D;
  uint64_t* __restrict__ keys = batch.keys + row0;
  int32_t* __restrict__ pos = batch.pos + row0;
  int32_t* __restrict__ ring = batch.ring + it.head0 * W;

  const uint4* ksrc = reinterpret_cast<const uint4*>(k + static_cast<int64_t>(g) * sh.P * D);
  const uint4* vsrc = reinterpret_cast<const uint4*>(v + static_cast<int64_t>(g) * sh.P * D);
  uint4* kdst = reinterpret_cast<uint4*>(kc + static_cast<int64_t>(g) * budget * D);
  uint4* vdst = reinterpret_cast<uint4*>(vc + static_cast<int64_t>(g) * budget * D);
  const int32_t* selg = sel + static_cast<int64_t>(g) * kcap;
  const float* scg = scores + static_cast<int64_t>(g) * sh.P;

  constexpr int RPT = 1;  // rows per thread per batch: loads issued before stores
  for (int32_t rb = r0 + rg; rb < r1; rb += RPT * RPP) {
    int32_t pos_r[RPT];
    bool scored_r[RPT];
    uint4 kr[RPT], vr[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) kr[u] = vr[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int32_t r = rb + u * RPP;
      int32_t p = 0;
      bool scored = false;
      if (r < r1) {
        if (r < sh.s_eff) {
          p = r;
        } else if (r < sh.s_eff + sh.kk) {
          p = selg[r - sh.s_eff];
          scored = true;
        } else {
          p = sh.w0 + (r - sh.s_eff - sh.kk);
        }
        kr[u] = nt_load16(&ksrc[static_cast<int64_t>(p) * LPR + c]);
        vr[u] = nt_load16(&vsrc[static_cast<int64_t>(p) * LPR + c]);
      }
      pos_r[u] = p;
      scored_r[u] = scored;
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int32_t r = rb + u * RPP;
      if (r < r1) {
        nt_store16(kr[u], &kdst[static_cast<int64_t>(r) * LPR + c]);
        nt_store16(vr[u], &vdst[static_cast<int64_t>(r) * LPR + c]);
        if (c == 0) {
          const int64_t hs = static_cast<int64_t>(g) * budget + r;
          const int32_t p = pos_r[u];
          pos[hs] = p;
          keys[hs] = scored_r[u] ? make_key(score_code(scg[p]), p) : KEY_NONE;
          if (!scored_r[u] && r >= sh.s_eff) ring[static_cast<int64_t>(g) * W + (p % W)] = r;
        }
      }
    }
  }
}

__global__ void init_ctl_kernel(HeadCtl* __restrict__ ctl, int64_t n_heads,
                                uint32_t* __restrict__ tickets, int64_t n_tickets) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n_heads) {
    HeadCtl c;
    c.n = -1;
    c.count = 0;
    c.nscored = 0;
    c.minslot = -1;
    c.minkey = KEY_NONE;
    c.flags = 0;
    c.leave_slot = -1;
    ctl[i] = c;
  }
  if (tickets != nullptr && i < n_tickets) tickets[i] = 0u;
}

}  // namespace

hipError_t launch_init_ctl(HeadCtl* ctl, int64_t n_heads, uint32_t* tickets, int64_t n_tickets,
                           hipStream_t stream) {
  const int64_t n = n_heads > n_tickets ? n_heads : n_tickets;
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(init_ctl_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(threads), 0,
                     stream, ctl, n_heads, tickets, n_tickets);
  return hipGetLastError();
}

namespace {

SelectItem select_item(const PrefillItem& it, int32_t* sel, const PrefillWork& pw) {
  SelectItem si;
  si.scores = it.scores;
  si.sel = sel;
  si.slice_keys = pw.slice_keys;
  si.slice_nan = pw.slice_nan;
  si.head0 = it.head0;
  si.P = it.n_tokens;
  si.n_slices = 1;
  si.slice_len = 0;
  return si;
}

GatherItem gather_item(const PrefillItem& it, const int32_t* sel) {
  GatherItem g;
  g.k = it.k;
  g.v = it.v;
  g.scores = it.scores;
  g.sel = sel;
  g.head0 = it.head0;
  g.P = it.n_tokens;
  return g;
}

template <int NB>
void fill_shared(SelectBatch<NB>& sb, GatherBatch<NB>& gb, const Geometry& geo,
                 const LayerView& all) {
  sb.ctl = all.ctl;
  sb.s = gb.s = geo.n_sink;
  sb.k = gb.k = geo.n_scored;
  sb.W = gb.W = geo.n_recent;
  gb.kc = all.kc;
  gb.vc = all.vc;
  gb.keys = all.keys;
  gb.pos = all.pos;
  gb.ring = all.ring;
  gb.budget = geo.budget;
}

// Rows per gather workgroup: one pass of its threads, one row per thread
// group (16 rows at D 128).  Smaller workgroups, more of them, measured
// faster than 4 rows per thread (64 rows): batched prefill of 64 prompts
// 0.42 against 0.44 ms.
constexpr int32_t gather_rows(int head_dim) { return GATHER_THREADS / (head_dim / 8); }

// Gather of m prompts whose selections are complete.
template <int NB>
hipError_t launch_gather(const Geometry& geo, GatherBatch<NB>& gb, int32_t m, hipStream_t stream) {
  int32_t maxc = 0;
  for (int32_t i = 0; i < m; ++i) {
    const int32_t c = prefill_shape(gb.item[i].P, geo.n_sink, geo.n_scored, geo.n_recent).count;
    maxc = c > maxc ? c : maxc;
  }
  if (maxc == 0) return hipSuccess;
  const int32_t rows = gather_rows(geo.head_dim);
  gb.rows_per_block = rows;
  const dim3 grid(static_cast<uint32_t>((maxc + rows - 1) / rows),
                  static_cast<uint32_t>(geo.n_kv_heads), static_cast<uint32_t>(m));
  if (geo.head_dim == 128)
    hipLaunchKernelGGL((prefill_gather_kernel<128, NB>), grid, dim3(GATHER_THREADS), 0, stream, gb);
  else
    hipLaunchKernelGGL((prefill_gather_kernel<64, NB>), grid, dim3(GATHER_THREADS), 0, stream, gb);
  return hipGetLastError();
}

// Prompts whose candidates fit VPT per thread, up to NB per launch pair.
template <int VPT, int NB>
hipError_t launch_head_batch(const Geometry& geo, const LayerView& all,
                             const PrefillItem* const* its, int32_t m, const PrefillWork& pw,
                             hipStream_t stream) {
  const int64_t kcap = geo.n_scored > 0 ? geo.n_scored : 1;
  SelectBatch<NB> sb;
  GatherBatch<NB> gb;
  fill_shared(sb, gb, geo, all);
  for (int32_t i = 0; i < m; ++i) {
    int32_t* sel = pw.sel + i * static_cast<int64_t>(geo.n_kv_heads) * kcap;
    sb.item[i] = select_item(*its[i], sel, pw);
    gb.item[i] = gather_item(*its[i], sel);
  }
  const dim3 grid(static_cast<uint32_t>(geo.n_kv_heads), 1u, static_cast<uint32_t>(m));
  hipLaunchKernelGGL((prefill_select_kernel<VPT, SEL_HEAD, NB>), grid, dim3(SEL_THREADS), 0,
                     stream, sb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gather<NB>(geo, gb, m, stream);
}

template <int VPT>
hipError_t launch_head_class(const Geometry& geo, const LayerView& all,
                             const PrefillItem* const* its, int32_t m, const PrefillWork& pw,
                             hipStream_t stream) {
  if (m == 1) return launch_head_batch<VPT, 1>(geo, all, its, 1, pw, stream);
  return launch_head_batch<VPT, PREFILL_NB>(geo, all, its, m, pw, stream);
}

// How a prompt longer than 32 candidates per thread selects: two levels
// with 16k or 32k-candidate slices when the union of its slices' top-k fits
// one workgroup's registers (at most 16 per thread), else (vpt 0) the
// streaming select.
struct LongPlan {
  int vpt;
  int32_t n_slices, slice_len;
};

LongPlan long_plan(const Geometry& geo, const PrefillShape& sh) {
  const int32_t C = sh.c1 - sh.c0;
  const int64_t k64 = geo.n_scored;
  const int32_t ns16 = (C + 16383) / 16384, ns32 = (C + 32767) / 32768;
  if (sh.kk < C && ns16 <= SLICE_MAX && ns16 * k64 <= 16384) return {16, ns16, 16384};
  if (sh.kk < C && ns32 <= SLICE_MAX && ns32 * k64 <= 16384) return {32, ns32, 32768};
  return {0, 1, 0};
}

// Two-level selects of m prompts with the same slice length, then their
// gather; each prompt uses selection and first-level slot i of the workspace.
template <int VPT, int NB>
hipError_t launch_two_level(const Geometry& geo, const LayerView& all,
                            const PrefillItem* const* its, int32_t m, const PrefillWork& pw,
                            hipStream_t stream) {
  const int64_t kcap = geo.n_scored > 0 ? geo.n_scored : 1;
  const int64_t slice_one = static_cast<int64_t>(geo.n_kv_heads) * SLICE_MAX * kcap;
  SelectBatch<NB> sb;
  GatherBatch<NB> gb;
  fill_shared(sb, gb, geo, all);
  int32_t max_slices = 1;
  for (int32_t i = 0; i < m; ++i) {
    int32_t* sel = pw.sel + i * static_cast<int64_t>(geo.n_kv_heads) * kcap;
    SelectItem& si = sb.item[i];
    si = select_item(*its[i], sel, pw);
    const LongPlan lp =
        long_plan(geo, prefill_shape(its[i]->n_tokens, geo.n_sink, geo.n_scored, geo.n_recent));
    si.n_slices = lp.n_slices;
    si.slice_len = lp.slice_len;
    si.slice_keys = pw.slice_keys + i * slice_one;
    si.slice_nan = pw.slice_nan + i * static_cast<int64_t>(geo.n_kv_heads) * SLICE_MAX;
    max_slices = lp.n_slices > max_slices ? lp.n_slices : max_slices;
    gb.item[i] = gather_item(*its[i], sel);
  }
  const dim3 slices(static_cast<uint32_t>(geo.n_kv_heads), static_cast<uint32_t>(max_slices),
                    static_cast<uint32_t>(m));
  hipLaunchKernelGGL((prefill_select_kernel<VPT, SEL_SLICE, NB>), slices, dim3(SEL_THREADS), 0,
                     stream, sb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 heads(static_cast<uint32_t>(geo.n_kv_heads), 1u, static_cast<uint32_t>(m));
  hipLaunchKernelGGL((prefill_select_kernel<16, SEL_LIST, NB>), heads, dim3(SEL_THREADS), 0,
                     stream, sb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gather<NB>(geo, gb, m, stream);
}

template <int VPT>
hipError_t launch_two_level_class(const Geometry& geo, const LayerView& all,
                                  const PrefillItem* const* its, int32_t m,
                                  const PrefillWork& pw, hipStream_t stream) {
  if (m == 1) return launch_two_level<VPT, 1>(geo, all, its, 1, pw, stream);
  return launch_two_level<VPT, PREFILL_NB>(geo, all, its, m, pw, stream);
}

// A prompt for which even two levels do not fit: the streaming select, alone.
hipError_t launch_streaming(const Geometry& geo, const LayerView& all, const PrefillItem& it,
                            const PrefillWork& pw, hipStream_t stream) {
  SelectBatch<1> sb;
  GatherBatch<1> gb;
  fill_shared(sb, gb, geo, all);
  sb.item[0] = select_item(it, pw.sel, pw);
  gb.item[0] = gather_item(it, pw.sel);
  const dim3 heads(static_cast<uint32_t>(geo.n_kv_heads));
  hipLaunchKernelGGL((prefill_select_kernel<0, SEL_HEAD, 1>), heads, dim3(SEL_THREADS), 0, stream,
                     sb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gather<1>(geo, gb, 1, stream);
}

}  // namespace

// Prompts are grouped by how they select (up to 16 or 32 candidates per
// thread; two levels with 16k or 32k slices; streaming) and each group runs
// in launches of up to `chunk` prompts.  Launches share the workspace, which
// is safe because they are ordered on the stream.
hipError_t launch_prefill_batch(const Geometry& geo, const LayerView& all,
                                const PrefillItem* items, int32_t n, const PrefillWork& pw,
                                hipStream_t stream) {
  int32_t chunk = pw.sel_items < PREFILL_NB ? pw.sel_items : PREFILL_NB;
  const int32_t chunk_long = pw.slice_items < chunk ? pw.slice_items : chunk;
  if (chunk < 1 || chunk_long < 1) return hipErrorInvalidValue;
  enum { C16, C32, L16, L32, NCLS };
  const PrefillItem* grp[NCLS][PREFILL_NB];
  int32_t cnt[NCLS] = {0, 0, 0, 0};
  auto flush = [&](int c) -> hipError_t {
    const int32_t m = cnt[c];
    cnt[c] = 0;
    if (m == 0) return hipSuccess;
    switch (c) {
      case C16: return launch_head_class<16>(geo, all, grp[c], m, pw, stream);
      case C32: return launch_head_class<32>(geo, all, grp[c], m, pw, stream);
      case L16: return launch_two_level_class<16>(geo, all, grp[c], m, pw, stream);
      default: return launch_two_level_class<32>(geo, all, grp[c], m, pw, stream);
    }
  };
  for (int32_t i = 0; i < n; ++i) {
    const PrefillItem& it = items[i];
    if (it.n_tokens <= 0) continue;
    const PrefillShape sh = prefill_shape(it.n_tokens, geo.n_sink, geo.n_scored, geo.n_recent);
    const int32_t per_thread = (sh.c1 - sh.c0 + SEL_THREADS - 1) / SEL_THREADS;
    int c;
    if (per_thread <= 16) {
      c = C16;
    } else if (per_thread <= 32) {
      c = C32;
    } else {
      const LongPlan lp = long_plan(geo, sh);
      if (lp.vpt == 0) {
        hipError_t e = launch_streaming(geo, all, it, pw, stream);
        if (e != hipSuccess) return e;
        continue;
      }
      c = lp.vpt == 16 ? L16 : L32;
    }
    grp[c][cnt[c]++] = &it;
    if (cnt[c] == (c >= L16 ? chunk_long : chunk)) {
      hipError_t e = flush(c);
      if (e != hipSuccess) return e;
    }
  }
  for (int c = 0; c < NCLS; ++c) {
    hipError_t e = flush(c);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvpop
