// Prefix top-k thresholds of a prompt for gfx950: for every position n and
// KV head, the key of the k-th most important member of Cand(n) = {s ..
// n - W} (0 while there are fewer than k, KEY_NONE when k = 0), so that the
// kept set at n is the sinks, the window and the candidates whose key
// reaches it.  The "Qwen3-8B-KVpop-4x" model card lists a prefix top-k
// thresholds kernel among its cache backends; the contract is a reading.
//
// Segments.  The candidates of a head are cut into S segments (S = 1 for
// short prompts, up to THR_SEG_MAX), spaced geometrically so that each
// expects about as many entrants (k * ln(end / start) after the first k).
// A first launch finds, for every segment, the exact top-k of all
// candidates before it (for the first segment: the first k): a radix select
// over the prefix (12-, 12- and 8-bit digits of the score code, ties at the
// threshold code resolved by position, the newest kept), a gather of the k
// keys and a sort in LDS.  Long prefixes with a small kept fraction are
// sampled first (two more launches ahead of it): a threshold from 4,096
// sampled codes, then many workgroups keep the candidates that reach it;
// when at least k and at most THR_KMAX do, they hold the top k and the sort
// takes them instead of the select.  The last launch runs one workgroup per
// (segment, head) from the starts.
//
// Within a segment a 1024-thread workgroup sweeps the candidates in chunks,
// keeping the current top-k keys sorted ascending in LDS (R, k <= THR_KMAX;
// in the first segment R starts as k zero keys, below every real key).  A chunk holds about
// THR_ETARGET * m / k candidates after m have been seen (64 to 4,096), so
// that about THR_ETARGET of them beat its threshold.  For a chunk with
// threshold T0 = R[0]:
//   1. entrants: candidates with key > T0, in arrival order (a scan);
//   2. sort the entrants: each one's rank is the number of smaller ones,
//      counted over broadcast LDS reads;
//   3. after the q-th entrant the threshold is the (q+1)-th smallest of R
//      and the first q entrants, so only the e + 1 smallest elements of R
//      and the entrants can be thresholds; they are listed by rank.  For
//      such an element u with c members of R below it, g_u(q) = c - #(the
//      first q entrants not below u) never increases, and u is the
//      threshold from the c-th entrant not below u (or step 0 if c = 0; not
//      before u itself has arrived) up to the step before the (c+1)-th.  One
//      wavefront finds both steps for an element, with ballots over 64
//      arrivals at a time;
//   4. a position's threshold is the one after the entrants up to it;
//   5. R becomes the k largest of R and the entrants: every element's rank
//      (index in its sorted list + binary-search count in the other) gives
//      its place, no sort of the union needed.
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

#include <algorithm>
#include <cmath>

namespace kvpop {
namespace {

constexpr int THR_THREADS = 1024;
constexpr int THR_ARR = 1024;      // entrants one chunk can hold
constexpr int THR_VMAX = 4;        // candidates per thread
constexpr int THR_ETARGET = 256;   // expected entrants per chunk
constexpr int THR_BUCKET = 64;     // segment starts: largest bucket ranked by counting
constexpr int THR_SAMPLE = 4096;   // segment starts: codes read for a sampled threshold
static_assert(THR_SAMPLE <= THR_KMAX, "a prefix read whole fits the key list");
constexpr int THR_FTHREADS = 512;     // sampled starts: threads per filter workgroup
constexpr int THR_FCHUNK = 8 * 1024;   // ... and candidates per filter workgroup

// Segment plan of a prompt: candidate ranges [b[j], b[j+1]) for j < S, and
// for each segment start the rank m of its sampled threshold (0: the start
// takes the exact select).
struct ThrPlan {
  int32_t S;
  int32_t b[THR_SEG_MAX + 1];
  uint32_t m[THR_SEG_MAX];
};

// The filter launch's work: (start, chunk) pairs of the sampled starts.
constexpr int THR_FPAIRS = 512;
struct ThrFilterWork {
  int32_t n;
  uint16_t j[THR_FPAIRS], c[THR_FPAIRS];
};

// A sampled segment start: its threshold, the keys that reach it (counted
// by the filter workgroups, stored up to THR_KMAX) and their largest code.
struct ThrMeta {
  uint32_t tau, count, cmax, pad;
};

// Ascending bitonic sort of a[0, p2) in LDS (p2 a power of two, at most
// 4 * THR_THREADS); called by the whole workgroup.  Thread t handles pairs
// t and t + 1,024, loading both before comparing.  A stage of stride 64 or
// less stays inside the 128 elements of one wavefront (pair i touches
// [2i - i mod stride, + stride], and pairs 64w .. 64w + 63 lie in block w),
// and a wavefront's LDS operations run in order, so two such stages in a
// row need no workgroup barrier between them.
__device__ __forceinline__ void bitonic_sort_lds(uint64_t* a, int32_t p2) {
  const int32_t tid = static_cast<int32_t>(threadIdx.x);
  const int32_t npairs = p2 / 2;
  for (int32_t size = 2; size <= p2; size <<= 1) {
    for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
      int32_t lo[2], hi[2];
      uint64_t x[2], y[2];
      bool live[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int32_t i = tid + u * THR_THREADS;
        live[u] = i < npairs;
        lo[u] = 2 * i - (i & (stride - 1));
        hi[u] = lo[u] + stride;
        if (live[u]) {
          x[u] = a[lo[u]];
          y[u] = a[hi[u]];
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool up = (lo[u] & size) == 0;
        if (live[u] && (x[u] > y[u]) == up) {
          a[lo[u]] = y[u];
          a[hi[u]] = x[u];
        }
      }
      const int32_t next = stride > 1 ? stride >> 1 : (size < p2 ? size : 0);
      if (stride > 64 || next > 64)
        __syncthreads();
      else
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the next stage's loads after these stores
    }
  }
  __syncthreads();
}

// f(i, code) for every candidate i in [0, n) of sc, coalesced, U loads per
// thread in flight.  Every thread runs the same number of rounds, so f is
// also called past the end (i >= n, with the last candidate's code): it
// must test i < n itself.
template <int U, typename F>
__device__ __forceinline__ void stream_scores(const float* __restrict__ sc, int32_t n, F&& f) {
  for (int32_t i0 = threadIdx.x; i0 - static_cast<int32_t>(threadIdx.x) < n;
       i0 += THR_THREADS * U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = sc[min(i0 + u * THR_THREADS, n - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) f(i0 + u * THR_THREADS, score_code(x[u]));
  }
}

// Sampled segment starts, first launch: the threshold of each (start j,
// head g) with plan.m[j] != 0 is the lower edge of the 24-bit bin that holds
// the m-th largest of THR_SAMPLE codes read in 64 runs spread over the
// prefix [0, b[j]) (all of it when b <= THR_SAMPLE).  With m = n + 4 sqrt(n)
// + 8, n = THR_SAMPLE * k / b (about n of the sample are in the top k),
// about m * b / THR_SAMPLE candidates reach it; a prefix read whole takes
// m = k.  The launch also clears the start's count and largest code for
// the filter launch.  Grid (S, Hkv).
__global__ __launch_bounds__(THR_THREADS) void thresholds_tau_kernel(
    const float* __restrict__ scores, int32_t P, int32_t s, ThrPlan plan,
    ThrMeta* __restrict__ meta) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t scan_buf[THR_THREADS / WAVE + 1];
  __shared__ uint32_t s_bin, s_above;
  const int j = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const uint32_t m = plan.m[j];
  ThrMeta* mt = meta + static_cast<int64_t>(g) * plan.S + j;
  if (m == 0) return;
  const int32_t b = plan.b[j];
  const float* __restrict__ sc = scores + static_cast<int64_t>(g) * P + s;
  // a prefix of at most THR_SAMPLE candidates is read whole (the host then
  // asks for m = k: the bin of the k-th largest code); a longer one in runs
  // that do not overlap
  const bool whole = b <= THR_SAMPLE;
  constexpr int TPR = THR_SAMPLE / 64 / 4;  // threads per run (4 codes each)
  const int32_t i0 = whole ? tid * 4
                           : static_cast<int32_t>(static_cast<int64_t>(tid / TPR) * b / 64) +
                                 (tid % TPR) * 4;
  uint32_t code[4];
  bool valid[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    valid[e] = i0 + e < b;
    code[e] = valid[e] ? score_code(sc[i0 + e]) : 0u;
  }
  uint32_t mrem = m, pre = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 20 : 8;
    for (int i = tid; i < 4096; i += THR_THREADS) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (valid[e] && (pass == 0 || (code[e] >> 20) == (pre >> 20)))
        atomicAdd(&hist[(code[e] >> shift) & 4095u], 1u);
    __syncthreads();
    uint32_t h[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = hist[4095 - 4 * tid - q];
      sum += h[q];
    }
    uint32_t tot;
    uint32_t ex = block_exclusive_scan_u32<THR_THREADS>(sum, scan_buf, &tot);
    if (ex < mrem && mrem <= ex + sum) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (mrem <= ex + h[q]) {
          s_bin = static_cast<uint32_t>(4095 - 4 * tid - q);
          s_above = ex;
          break;
        }
        ex += h[q];
      }
    }
    __syncthreads();
    mrem -= s_above;
    pre |= s_bin << shift;
  }
  if (tid == 0) *mt = ThrMeta{pre, 0u, 0u, 0u};  // low 8 bits 0: codes in or above the bin
}

// Sampled segment starts, second launch: every workgroup streams
// THR_FCHUNK candidates of one start's prefix, gathers the keys whose code
// reaches the start's threshold in LDS, then reserves room in the start's
// list with one atomic and copies them there (stores past THR_KMAX are
// dropped: the count still tells), and raises the start's largest code.
// Spreading each prefix over many workgroups matters: one workgroup
// streamed a 114k-candidate prefix in 26-30 us, bound by the loads one
// compute unit keeps in flight.  One global atomic per wavefront instead of
// per workgroup serialised on the start's counter (2x slower overall), and
// so do chunks much smaller than 8,192 candidates (131,072 tokens: 70, 74
// and 93 us per call at 8,192, 4,096 and 2,048; 72 and 79 us at 16,384 and
// 32,768).  512 threads per workgroup: 69.3 us, against 70.4 with 1,024 and
// 70.7 with 256.
// Grid (pairs, Hkv): one workgroup per (start, chunk) pair and head.
__global__ __launch_bounds__(THR_FTHREADS) void thresholds_filter_kernel(
    const float* __restrict__ scores, int32_t P, int32_t s, ThrPlan plan, ThrFilterWork fw,
    ThrMeta* __restrict__ meta, uint64_t* __restrict__ lists) {
  __shared__ uint64_t lk[THR_KMAX];
  __shared__ uint32_t s_cnt, s_cmax, s_base;
  const int j = fw.j[blockIdx.x];
  const int c = fw.c[blockIdx.x];
  const int g = blockIdx.y;
  const int32_t b = plan.b[j];
  const int32_t lo = c * THR_FCHUNK;
  const int32_t hi = min(b, lo + THR_FCHUNK);
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  ThrMeta* mt = meta + static_cast<int64_t>(g) * plan.S + j;
  uint64_t* list = lists + (static_cast<int64_t>(g) * plan.S + j) * THR_KMAX;
  const uint32_t tau = mt->tau;
  const float* __restrict__ sc = scores + static_cast<int64_t>(g) * P + s;
  constexpr int U = THR_FCHUNK / THR_FTHREADS;
  float x[U];
#pragma unroll
  for (int u = 0; u < U; ++u) x[u] = sc[min(lo + u * THR_FTHREADS + tid, hi - 1)];
  if (tid == 0) {
    s_cnt = 0u;
    s_cmax = 0u;
  }
  __syncthreads();
  uint32_t cmax = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int32_t i = lo + u * THR_FTHREADS + tid;
    const uint32_t o = score_code(x[u]);
    const bool keep = i < hi && o >= tau;
    const uint64_t msk = __ballot(keep);
    if (msk != 0ull) {  // wavefront-uniform
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&s_cnt, static_cast<uint32_t>(__popcll(msk)));
      base = __shfl(base, 0, WAVE);
      if (keep) {
        const uint32_t at = base + __builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(msk >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(msk), 0u));
        if (at < static_cast<uint32_t>(THR_KMAX)) lk[at] = make_key(o, s + i);
        cmax = o > cmax ? o : cmax;
      }
    }
  }
#pragma unroll
  for (int d = WAVE / 2; d >= 1; d >>= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_xor(static_cast<int>(cmax), d, WAVE));
    cmax = y > cmax ? y : cmax;
  }
  if (lane == 0 && cmax != 0u) atomicMax(&s_cmax, cmax);
  __syncthreads();
  const uint32_t n = s_cnt;
  if (n == 0u) return;  // uniform
  if (tid == 0) {
    s_base = atomicAdd(&mt->count, n);
    atomicMax(&mt->cmax, s_cmax);
  }
  __syncthreads();
  const uint32_t base = s_base;
  const uint32_t nl = min(n, static_cast<uint32_t>(THR_KMAX));
  for (uint32_t i = tid; i < nl; i += THR_FTHREADS)
    if (base + i < static_cast<uint32_t>(THR_KMAX)) list[base + i] = lk[i];
}

// The exact top-k keys (ascending) of the first b[j] candidates of head g
// (b[0] = k: the first k), the start of segment j, into
// ws[(g * S + j) * k ...].  Grid (S, Hkv).
__global__ __launch_bounds__(THR_THREADS) void thresholds_segment_start_kernel(
    const float* __restrict__ scores, int32_t P, int32_t s, int32_t k, ThrPlan plan,
    uint64_t* __restrict__ ws, const ThrMeta* __restrict__ meta,
    const uint64_t* __restrict__ lists) {
  constexpr int NWAVE = THR_THREADS / WAVE;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t cur[4096];
  __shared__ uint64_t keys[THR_KMAX];
  __shared__ uint64_t keys2[THR_KMAX];
  __shared__ uint32_t scan_buf[NWAVE + 1];
  __shared__ uint32_t s_bin, s_above, s_neq, s_n, s_cmax, s_bmax;
  __shared__ int32_t s_pcut;
  const int j = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int32_t b = plan.b[j];                     // candidates [0, b), b >= k
  const float* __restrict__ sc = scores + static_cast<int64_t>(g) * P + s;
  uint64_t* dst = ws + (static_cast<int64_t>(g) * plan.S + j) * k;
  if (tid == 0) {
    s_n = 0u;
    s_cmax = 0u;
    s_bmax = 0u;
  }

  // ---- a sampled start: when at least k keys reach its threshold and they
  // fit, they hold the top k (every other key is below all of them), which
  // the sort below places.  Otherwise the exact select runs.
  uint32_t t = 0;     // every key of the sort is at or above code t
  int32_t n = k;      // keys to sort; the top k of them are written
  bool sampled = false;
  if (meta != nullptr && plan.m[j] != 0) {
    const ThrMeta mt = meta[g * plan.S + j];
    if (mt.count >= static_cast<uint32_t>(k) && mt.count <= static_cast<uint32_t>(THR_KMAX)) {
      const uint64_t* list = lists + (static_cast<int64_t>(g) * plan.S + j) * THR_KMAX;
      for (int32_t i = tid; i < static_cast<int32_t>(mt.count); i += THR_THREADS) keys[i] = list[i];
      if (tid == 0) s_cmax = mt.cmax;
      __syncthreads();
      sampled = true;
      t = mt.tau;
      n = static_cast<int32_t>(mt.count);
    }
  }

  // the prefix's codes in registers when one round of 16 per thread holds
  // them (the radix passes and the gather then read no memory), in the
  // order stream_scores<16> visits them
  constexpr int RC = 16;
  const bool in_regs = b <= RC * THR_THREADS;
  uint32_t rcode[RC];
  auto codes = [&](auto&& f) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < RC; ++u) f(tid + u * THR_THREADS, rcode[u]);
    } else {
      stream_scores<RC>(sc, b, f);
    }
  };
  if (!sampled) {
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < RC; ++u) rcode[u] = score_code(sc[min(tid + u * THR_THREADS, b - 1)]);
  }
  // ---- radix select of the k-th largest code: 12-, 12- and 8-bit digits.
  // The wide first digit (sign, exponent, 3 mantissa bits) spreads the codes
  // of real-valued scores over many bins; with 8 bits most fell into a few
  // bins and the histogram atomics serialised.
  uint32_t prefix = 0, mask = 0, krem = static_cast<uint32_t>(k);
  const int shifts[3] = {20, 8, 0}, nbins[3] = {4096, 4096, 256};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass], nb = nbins[pass];
    for (int i = tid; i < nb; i += THR_THREADS) hist[i] = 0u;
    __syncthreads();
    codes([&](int32_t i, uint32_t o) {
      if (i < b && (o & mask) == prefix)
        atomicAdd(&hist[(o >> shift) & static_cast<uint32_t>(nb - 1)], 1u);
    });
    __syncthreads();
    // thread t holds bins nb-1-4t down to nb-4-4t, from the top
    uint32_t h[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int bin = nb - 1 - 4 * tid - q;
      h[q] = bin >= 0 ? hist[bin] : 0u;
      sum += h[q];
    }
    uint32_t tot;
    uint32_t ex = block_exclusive_scan_u32<THR_THREADS>(sum, scan_buf, &tot);
    if (ex < krem && krem <= ex + sum) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (krem <= ex + h[q]) {
          s_bin = static_cast<uint32_t>(nb - 1 - 4 * tid - q);
          s_above = ex;
          s_neq = h[q];
          break;
        }
        ex += h[q];
      }
    }
    __syncthreads();
    krem -= s_above;
    prefix |= s_bin << shift;
    mask |= static_cast<uint32_t>(nb - 1) << shift;
  }
  t = prefix;                              // the k-th largest code
  const uint32_t drop = s_neq - krem;      // ties at t that lose (the oldest)

  // ---- the first kept tie, in position order: rank `drop` among ties ------
  if (tid == 0) s_pcut = 0;
  if (drop > 0) {
    const int32_t L = (b + THR_THREADS - 1) / THR_THREADS;  // contiguous run
    const int32_t lo = min(tid * L, b), hi = min(lo + L, b);
    uint32_t cnt = 0;
    for (int32_t i = lo; i < hi; ++i) cnt += score_code(sc[i]) == t ? 1u : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan_u32<THR_THREADS>(cnt, scan_buf, &tot);
    if (ex <= drop && drop < ex + cnt) {
      uint32_t r = ex;
      for (int32_t i = lo; i < hi; ++i) {
        if (score_code(sc[i]) == t) {
          if (r == drop) {
            s_pcut = i;
            break;
          }
          ++r;
        }
      }
    }
  }
  __syncthreads();
  const int32_t pcut = s_pcut;

  // ---- gather the k keys that reach the k-th largest key ------------------
  uint32_t cmax = 0;  // this thread's largest kept code
  codes([&](int32_t i, uint32_t o) {
    const bool keep = i < b && (o > t || (o == t && i >= pcut));
    const uint64_t m = __ballot(keep);
    if (m != 0ull) {  // wavefront-uniform; most rounds keep nothing
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&s_n, static_cast<uint32_t>(__popcll(m)));
      base = __shfl(base, 0, WAVE);
      if (keep) {
        const uint32_t below = __builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
        keys[base + below] = make_key(o, s + i);
        cmax = o > cmax ? o : cmax;
      }
    }
  });
  // the largest kept code: a wave maximum, then one LDS atomic per wave
#pragma unroll
  for (int d = WAVE / 2; d >= 1; d >>= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_xor(static_cast<int>(cmax), d, WAVE));
    cmax = y > cmax ? y : cmax;
  }
  if (lane == 0) atomicMax(&s_cmax, cmax);
  }  // exact select

  // ---- sort the k keys ascending.  Buckets: 4096 equal ranges of the
  // scores from the threshold's up to the largest kept one (of the codes,
  // when either is not finite); a key's place is its bucket's start plus its
  // rank among the (few) keys of its bucket.  A bucket of more than
  // THR_BUCKET keys (many equal scores) sends the sort to a bitonic network.
  for (int i = tid; i < 4096; i += THR_THREADS) hist[i] = 0u;
  __syncthreads();
  const uint32_t cmx = s_cmax;
  const float vlo = code_value(t), vhi = code_value(cmx);
  const float scale = 4096.0f / (vhi - vlo);
  const bool by_value = __builtin_isfinite(vlo) && __builtin_isfinite(vhi) && vhi > vlo &&
                        __builtin_isfinite(scale);
  const uint32_t span = cmx - t;
  const int sh = span >> 12 ? 20 - __builtin_clz(span) : 0;  // (code - t) >> sh < 4096
  // monotone in the code: the order of the buckets is the order of the keys
  auto bucket = [&](uint32_t o) -> uint32_t {
    if (by_value) {
      const float f = (code_value(o) - vlo) * scale;
      return f < 4095.0f ? static_cast<uint32_t>(f) : 4095u;
    }
    return (o - t) >> sh;
  };
  for (int32_t i = tid; i < n; i += THR_THREADS)
    atomicAdd(&hist[bucket(static_cast<uint32_t>(keys[i] >> 32))], 1u);
  __syncthreads();
  {
    // thread t owns buckets 4t .. 4t+3: hist <- starts, cur <- cursors
    uint32_t c[4], sum = 0, mx = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = hist[4 * tid + q];
      sum += c[q];
      mx = c[q] > mx ? c[q] : mx;
    }
    uint32_t tot;
    uint32_t ex = block_exclusive_scan_u32<THR_THREADS>(sum, scan_buf, &tot);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      hist[4 * tid + q] = ex;
      cur[4 * tid + q] = ex;
      ex += c[q];
    }
    atomicMax(&s_bmax, mx);
  }
  __syncthreads();
  // the keys' ranks among all n; the top k (ranks n - k .. n - 1) are written
  const int32_t skip = n - k;
  if (s_bmax <= static_cast<uint32_t>(THR_BUCKET)) {
    for (int32_t i = tid; i < n; i += THR_THREADS) {
      const uint64_t key = keys[i];
      keys2[atomicAdd(&cur[bucket(static_cast<uint32_t>(key >> 32))], 1u)] = key;
    }
    __syncthreads();
    for (int32_t i = tid; i < n; i += THR_THREADS) {
      const uint64_t key = keys2[i];
      const uint32_t d = bucket(static_cast<uint32_t>(key >> 32));
      const uint32_t lo = hist[d], hi = cur[d];  // the bucket, now filled
      uint32_t rank = 0;
      for (uint32_t x = lo; x < hi; ++x) rank += keys2[x] < key ? 1u : 0u;
      const int32_t at = static_cast<int32_t>(lo + rank) - skip;
      if (at >= 0) dst[at] = key;
    }
    return;
  }
  int32_t p2 = 1;
  while (p2 < n) p2 <<= 1;
  for (int32_t i = n + tid; i < p2; i += THR_THREADS) keys[i] = ~0ull;  // sorts past the keys
  __syncthreads();
  bitonic_sort_lds(keys, p2);
  for (int32_t i = tid; i < k; i += THR_THREADS) dst[i] = keys[skip + i];
}

// #(x in a[0..n) with x < v), a sorted ascending
__device__ __forceinline__ int32_t count_below(const uint64_t* a, int32_t n, uint64_t v) {
  int32_t lo = 0, hi = n;
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    if (a[mid] < v)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Index of the n-th (0-based) set bit of a wavefront-uniform 64-bit mask.
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int n, int lane) {
  const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                              __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
  const bool hit = ((mask >> lane) & 1ull) && below == n;
  return __ffsll(static_cast<unsigned long long>(__ballot(hit))) - 1;
}

// One workgroup per (segment, head): grid (S, Hkv).
__global__ __launch_bounds__(THR_THREADS) void prefix_thresholds_kernel(
    const float* __restrict__ scores, int32_t P, int32_t s, int32_t k, int32_t W,
    uint64_t* __restrict__ thr, ThrPlan plan, const uint64_t* __restrict__ ws) {
  constexpr int NWAVE = THR_THREADS / WAVE;
  __shared__ uint64_t Rbuf[2][THR_KMAX];
  __shared__ uint64_t arr[THR_ARR];       // entrant keys in arrival order
  __shared__ uint64_t ak[THR_ARR];        // entrant keys sorted ascending
  __shared__ uint32_t aq[THR_ARR];        // ... and their arrival step (1-based)
  __shared__ uint64_t lu[THR_ARR + 1];    // possible thresholds by rank: key,
  __shared__ int32_t lc[THR_ARR + 1];     // members of R below it,
  __shared__ uint32_t la[THR_ARR + 1];    // first step it is present
  __shared__ uint64_t tq[THR_ARR + 1];    // threshold after q entrants
  __shared__ uint32_t scan_buf[NWAVE + 1];

  const int jseg = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const float* sc = scores + static_cast<int64_t>(g) * P;
  uint64_t* out = thr + static_cast<int64_t>(g) * P;
  const int32_t c1 = P - W;                        // candidates [s, c1)
  const int32_t C = c1 > s ? c1 - s : 0;
  // positions before the first candidate leaves the window
  const int32_t n_first = min(P, s + W);           // positions [0, n_first)
  if (jseg == 0)
    for (int32_t n = tid; n < n_first; n += THR_THREADS) out[n] = 0ull;
  if (C == 0) return;

  uint64_t* R = Rbuf[0];
  uint64_t* R2 = Rbuf[1];
  const int32_t w0 = min(k, C);
  const int32_t cs = plan.b[jseg], ce = plan.b[jseg + 1];  // this segment's candidates
  if (plan.S > 1) {
    // the top-k of every candidate before the segment, from the first launch
    const uint64_t* src = ws + (static_cast<int64_t>(g) * plan.S + jseg) * k;
    for (int32_t i = tid; i < k; i += THR_THREADS) R[i] = src[i];
    __syncthreads();
    if (jseg == 0) {  // the first k candidates: fewer than k after all but the last
      for (int32_t i = tid; i < k - 1; i += THR_THREADS) out[s + W + i] = 0ull;
      if (tid == 0) out[s + W + k - 1] = R[0];
    }
  } else {
    // ---- warm-up: until k candidates have left the window every one is kept
    // (threshold 0); R = the first min(k, C) keys sorted, then zero keys -----
    int32_t p2 = 1;
    while (p2 < k) p2 <<= 1;
    for (int32_t i = tid; i < p2; i += THR_THREADS) {
      uint64_t v = 0ull;
      if (i < w0) {
        const int32_t pos = s + i;
        v = make_key(score_code(sc[pos]), pos);
        if (i < w0 - 1 || w0 < k) out[s + W + i] = 0ull;  // fewer than k after it
      } else if (i >= k) {
        v = ~0ull;                                        // sorts past R
      }
      R2[i] = v;
    }
    __syncthreads();
    bitonic_sort_lds(R2, p2);
    uint64_t* t = R;
    R = R2;
    R2 = t;
    if (w0 == k && tid == 0) out[s + W + k - 1] = R[0];  // the k-th candidate completes R
  }

  // Chunks: each thread takes a run of V = ceil(len / 1024) consecutive
  // candidates.  A chunk whose entrants overflow the arrays (far more than
  // the THR_ETARGET expected) is redone with 1,024 candidates, which cannot.
  auto chunk_len = [&](int32_t m) {
    const int64_t want = static_cast<int64_t>(THR_ETARGET) * m / k;
    return static_cast<int32_t>(min<int64_t>(max<int64_t>(want, 64), THR_THREADS * THR_VMAX));
  };
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;
  float xs[THR_VMAX];  // scores of this thread's run, loaded one chunk ahead
  auto load_run = [&](int32_t c0, int V) {
#pragma unroll
    for (int v = 0; v < THR_VMAX; ++v) {
      const int32_t i = min(c0 + tid * V + v, C - 1);
      xs[v] = (v < V) ? sc[s + i] : 0.f;
    }
  };
  int32_t len = min(chunk_len(cs), ce - cs);
  int V = (len + THR_THREADS - 1) / THR_THREADS;
  if (cs < ce) load_run(cs, V);
  for (int32_t c0 = cs; c0 < ce;) {
    // ---- 1. this thread's candidates and the entrants ---------------------
    const uint64_t T0 = R[0];
    uint64_t key[THR_VMAX];
    uint32_t own;    // entrants in this thread's run
    uint32_t e, before;
    for (;;) {
      own = 0;
#pragma unroll
      for (int v = 0; v < THR_VMAX; ++v) {
        const int32_t i = tid * V + v;  // chunk-relative
        const bool valid = v < V && i < len;
        key[v] = valid ? make_key(score_code(xs[v]), s + c0 + i) : 0ull;
        own += (valid && key[v] > T0) ? 1u : 0u;
      }
      before = block_exclusive_scan_u32<THR_THREADS>(own, scan_buf, &e);
      if (e <= THR_ARR) break;
      len = min(THR_THREADS, ce - c0);  // too many entrants: one per thread
      V = 1;
      load_run(c0, V);
    }
    // next chunk's scores go out now; their latency overlaps this chunk
    const int32_t c_next = c0 + len;
    const int32_t len_next = c_next < ce ? min(chunk_len(c_next), ce - c_next) : 0;
    const int V_next = (len_next + THR_THREADS - 1) / THR_THREADS;
    uint32_t qv[THR_VMAX];  // entrants up to and including each of this run
    {
      uint32_t q = before;
#pragma unroll
      for (int v = 0; v < THR_VMAX; ++v) {
        if (key[v] > T0) arr[q++] = key[v];
        qv[v] = q;
      }
    }
    if (c_next < ce) load_run(c_next, V_next);
    __syncthreads();
    // ---- 2. sort the entrants: rank = #smaller, over broadcast reads ------
    if (tid < static_cast<int>(e)) {
      const uint64_t x = arr[tid];
      uint32_t r = 0;
      uint32_t i = 0;
      for (; i + 4 <= e; i += 4)
        r += (arr[i] < x ? 1u : 0u) + (arr[i + 1] < x ? 1u : 0u) + (arr[i + 2] < x ? 1u : 0u) +
             (arr[i + 3] < x ? 1u : 0u);
      for (; i < e; ++i) r += arr[i] < x ? 1u : 0u;
      ak[r] = x;
      aq[r] = static_cast<uint32_t>(tid) + 1u;
    }
    __syncthreads();
    // ---- 3. the possible thresholds, listed by rank ----------------------
    // R[i] for i <= e (rank i + #(entrants below)), and every entrant (rank
    // j + #(R below)); exactly the e + 1 of rank <= e can be a threshold.
    for (uint32_t u = tid; u < 2 * e + 1; u += THR_THREADS) {
      uint64_t val;
      int32_t below_r;     // #(R below val)
      uint32_t avail;      // first step at which val is present
      int32_t rank;        // rank in R + all entrants
      if (u <= e) {        // R[u]
        if (static_cast<int32_t>(u) >= k) continue;
        val = R[u];
        below_r = static_cast<int32_t>(u);
        avail = 0;
        rank = below_r + count_below(ak, static_cast<int32_t>(e), val);
      } else {             // sorted entrant j
        const uint32_t j = u - e - 1;
        val = ak[j];
        below_r = count_below(R, k, val);
        avail = aq[j];
        rank = static_cast<int32_t>(j) + below_r;
      }
      if (rank > static_cast<int32_t>(e)) continue;
      lu[rank] = val;
      lc[rank] = below_r;
      la[rank] = avail;
    }
    __syncthreads();
    // ---- threshold ranges: one wavefront per possible threshold ----------
    for (int32_t r = wid; r <= static_cast<int32_t>(e); r += NWAVE) {
      const uint64_t u = lu[r];
      const int32_t c = lc[r];
      int32_t seen = 0;                      // arrivals not below u so far
      int32_t q0 = (c == 0) ? 0 : -1;        // first step with g_u = 0
      int32_t q1 = static_cast<int32_t>(e);  // last step with g_u = 0
      for (int32_t base = 0; base < static_cast<int32_t>(e); base += WAVE) {
        const int32_t q = base + lane;
        const bool hit = q < static_cast<int32_t>(e) && !(arr[q] < u);
        const uint64_t mask = __ballot(hit);
        const int32_t pc = __popcll(static_cast<unsigned long long>(mask));
        if (q0 < 0 && seen + pc >= c) q0 = base + nth_set_bit(mask, c - seen - 1, lane) + 1;
        if (seen + pc >= c + 1) {
          q1 = base + nth_set_bit(mask, c - seen, lane);
          break;
        }
        seen += pc;
      }
      if (q0 >= 0)
        for (int32_t q = max(q0, static_cast<int32_t>(la[r])) + lane; q <= q1; q += WAVE)
          tq[q] = u;
    }
    __syncthreads();
    // ---- 4. per-position thresholds ---------------------------------------
#pragma unroll
    for (int v = 0; v < THR_VMAX; ++v) {
      const int32_t i = tid * V + v;
      if (v < V && i < len) out[s + W + c0 + i] = tq[qv[v]];
    }
    // ---- 5. R <- the k largest of R and the entrants ----------------------
    for (int32_t i = tid; i < k; i += THR_THREADS) {
      const uint64_t v = R[i];
      const int32_t r = i + count_below(ak, static_cast<int32_t>(e), v);
      if (r >= static_cast<int32_t>(e)) R2[r - static_cast<int32_t>(e)] = v;
    }
    for (uint32_t j = tid; j < e; j += THR_THREADS) {
      const uint64_t v = ak[j];
      const int32_t r = static_cast<int32_t>(j) + count_below(R, k, v);
      if (r >= static_cast<int32_t>(e)) R2[r - static_cast<int32_t>(e)] = v;
    }
    __syncthreads();
    uint64_t* t = R;
    R = R2;
    R2 = t;
    c0 = c_next;
    len = len_next;
    V = V_next;
  }
}

__global__ void fill_u64_kernel(uint64_t* __restrict__ p, int64_t n, uint64_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_prefix_thresholds(const Geometry& geo, int32_t n_tokens, const float* scores,
                                    uint64_t* thr, uint64_t* ws, int64_t ws_keys,
                                    hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  if (geo.n_scored == 0) {
    const int64_t n = static_cast<int64_t>(geo.n_kv_heads) * n_tokens;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                       0, stream, thr, n, KEY_NONE);
    return hipGetLastError();
  }
  const int32_t k = geo.n_scored;
  if (k > THR_KMAX) return hipErrorInvalidValue;
  // segments: about one per 512 candidates after the first k, at most
  // THR_SEG_MAX and as many as the workspace holds, spaced geometrically
  // from k to C
  const int32_t c1 = n_tokens - geo.n_recent;
  const int32_t C = c1 > geo.n_sink ? c1 - geo.n_sink : 0;
  const int32_t w0 = k < C ? k : C;
  ThrPlan plan;
  plan.S = 1;
  const int64_t fit = ws != nullptr ? ws_keys / (static_cast<int64_t>(geo.n_kv_heads) * k) : 0;
  if (C - w0 >= 4096 && fit >= 2)
    plan.S = static_cast<int32_t>(std::min<int64_t>(std::min<int64_t>(THR_SEG_MAX, fit),
                                                    (C - w0) / 512));
  plan.b[0] = w0;
  for (int j = 1; j < plan.S; ++j) {
    const double f = std::pow(static_cast<double>(C) / w0, static_cast<double>(j) / plan.S);
    const int64_t bj = static_cast<int64_t>(std::floor(w0 * f));
    plan.b[j] = static_cast<int32_t>(std::min<int64_t>(std::max<int64_t>(bj, plan.b[j - 1]), C));
  }
  plan.b[plan.S] = C;
  for (int j = plan.S + 1; j <= THR_SEG_MAX; ++j) plan.b[j] = C;
  for (int j = 0; j < THR_SEG_MAX; ++j) plan.m[j] = 0u;
  if (plan.S > 1) {
    // Sampled starts: prefixes whose expected survivors (m * b / THR_SAMPLE,
    // or at most b for a prefix read whole) fit THR_KMAX with room to spare,
    // when the workspace also holds the starts' lists and records (after the
    // S * Hkv * k start keys) and the filter's pair table has room.  Only
    // when every start qualifies: otherwise the starts that take the exact
    // select set the launch's length and the two extra launches only add to
    // it (16,384-token prompt at k = 3,772: 63 against 53 us per call).
    const int64_t SH = static_cast<int64_t>(plan.S) * geo.n_kv_heads;
    uint64_t* lists = ws + SH * k;
    ThrMeta* meta = reinterpret_cast<ThrMeta*>(lists + SH * THR_KMAX);
    const bool room = ws_keys >= SH * (k + THR_KMAX + 2);
    ThrFilterWork fw;
    fw.n = 0;
    for (int j = 0; j < plan.S && room; ++j) {
      const int32_t b = plan.b[j];
      // a whole prefix (b <= THR_SAMPLE) is its own sample: m = k, and at most
      // b <= THR_KMAX keys can reach the threshold
      const double nf = static_cast<double>(THR_SAMPLE) * k / b;
      const int64_t m = b <= THR_SAMPLE
                            ? k
                            : std::min<int64_t>(
                                  static_cast<int64_t>(std::ceil(nf + 4.0 * std::sqrt(nf) + 8.0)),
                                  THR_SAMPLE);
      const int32_t chunks = (b + THR_FCHUNK - 1) / THR_FCHUNK;
      const bool fits = b <= THR_SAMPLE ||
                        m * b <= static_cast<int64_t>(THR_KMAX) * THR_SAMPLE * 7 / 8;
      if (!fits || fw.n + chunks > THR_FPAIRS) {
        fw.n = 0;
        break;
      }
      plan.m[j] = static_cast<uint32_t>(m);
      for (int32_t q = 0; q < chunks; ++q) {
        fw.j[fw.n] = static_cast<uint16_t>(j);
        fw.c[fw.n] = static_cast<uint16_t>(q);
        ++fw.n;
      }
    }
    if (fw.n == 0)
      for (int j = 0; j < THR_SEG_MAX; ++j) plan.m[j] = 0u;
    const dim3 starts(static_cast<uint32_t>(plan.S), static_cast<uint32_t>(geo.n_kv_heads));
    if (fw.n > 0) {
      hipLaunchKernelGGL(thresholds_tau_kernel, starts, dim3(THR_THREADS), 0, stream, scores,
                         n_tokens, geo.n_sink, plan, meta);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(thresholds_filter_kernel,
                         dim3(static_cast<uint32_t>(fw.n), static_cast<uint32_t>(geo.n_kv_heads)),
                         dim3(THR_FTHREADS), 0, stream, scores, n_tokens, geo.n_sink, plan, fw, meta,
                         lists);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(thresholds_segment_start_kernel, starts, dim3(THR_THREADS), 0, stream,
                       scores, n_tokens, geo.n_sink, k, plan, ws,
                       fw.n > 0 ? meta : static_cast<ThrMeta*>(nullptr), lists);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(prefix_thresholds_kernel,
                     dim3(static_cast<uint32_t>(plan.S), static_cast<uint32_t>(geo.n_kv_heads)),
                     dim3(THR_THREADS), 0, stream, scores, n_tokens, geo.n_sink, k, geo.n_recent,
                     thr, plan, ws);
  return hipGetLastError();
}

}  // namespace kvpop
