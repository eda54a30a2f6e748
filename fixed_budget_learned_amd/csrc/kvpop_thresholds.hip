// Prefix top-k thresholds of a prompt for gfx950: for every position n and
// KV head, the key of the k-th most important member of Cand(n) = {s ..
// n - W} (0 while there are fewer than k, KEY_NONE when k = 0), so that the
// kept set at n is the sinks, the window and the candidates whose key
// reaches it.  The "Qwen3-8B-KVpop-4x" model card lists a prefix top-k
// thresholds kernel among its cache backends; the contract is a reading.
//
// One 1024-thread workgroup per KV head sweeps the candidates in chunks of
// 1024 positions, keeping the current top-k keys sorted ascending in LDS
// (R, k <= THR_KMAX; R starts as k zero keys, below every real key).  For a
// chunk with threshold T0 = R[0]:
//   1. entrants: candidates with key > T0, in arrival order (a scan);
//   2. after the q-th entrant the threshold is the (q+1)-th smallest of R
//      and the first q entrants.  For an element u of R or of the entrants,
//      g_u(q) = #(R below u) + #(entrants 1..q below u) - q never increases
//      with q, so u is the threshold on one contiguous range of steps (where
//      g_u = 0 and u has arrived).  Each of the e + 1 smallest elements of R
//      and the entrants walks the arrival sequence once to find its range;
//   3. a position's threshold is the one after the entrants up to it;
//   4. R becomes the k largest of R and the entrants: every element's rank
//      (index in its sorted list + binary-search count in the other) gives
//      its place, no sort of the union needed.
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int THR_THREADS = 1024;
constexpr int THR_CHUNK = 1024;   // candidates per chunk, one per thread

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

__global__ __launch_bounds__(THR_THREADS) void prefix_thresholds_kernel(
    const float* __restrict__ scores, int32_t P, int32_t s, int32_t k, int32_t W,
    uint64_t* __restrict__ thr) {
  constexpr int NWAVE = THR_THREADS / WAVE;
  __shared__ uint64_t Rbuf[2][THR_KMAX];
  __shared__ uint64_t arr[THR_CHUNK];     // entrant keys in arrival order
  __shared__ uint64_t ak[THR_CHUNK];      // entrant keys sorted ascending
  __shared__ uint32_t aq[THR_CHUNK];      // ... and their arrival step (1-based)
  __shared__ uint64_t tq[THR_CHUNK + 1];  // threshold after q entrants
  __shared__ uint32_t scan_buf[NWAVE + 1];

  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const float* sc = scores + static_cast<int64_t>(g) * P;
  uint64_t* out = thr + static_cast<int64_t>(g) * P;
  const int32_t c1 = P - W;                        // candidates [s, c1)
  const int32_t C = c1 > s ? c1 - s : 0;
  // positions before the first candidate leaves the window
  const int32_t n_first = min(P, s + W);           // positions [0, n_first)
  for (int32_t n = tid; n < n_first; n += THR_THREADS) out[n] = 0ull;
  if (C == 0) return;

  uint64_t* R = Rbuf[0];
  uint64_t* R2 = Rbuf[1];
  // ---- warm-up: until k candidates have left the window every one is kept
  // (threshold 0); R = the first min(k, C) keys sorted, then zero keys ------
  const int32_t w0 = min(k, C);
  {
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
    for (int32_t size = 2; size <= p2; size <<= 1) {
      for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
        for (int32_t i = tid; i < p2 / 2; i += THR_THREADS) {
          const int32_t lo = 2 * i - (i & (stride - 1));
          const int32_t hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = R2[lo], b = R2[hi];
          if ((a > b) == up) {
            R2[lo] = b;
            R2[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    uint64_t* t = R;
    R = R2;
    R2 = t;
    if (w0 == k && tid == 0) out[s + W + k - 1] = R[0];  // the k-th candidate completes R
  }

  // Chunks: each thread takes a run of V consecutive candidates, V = 1, 2 or
  // 4; about 1024 * V * k / m candidates of a chunk beat its threshold after
  // m candidates, so V grows with m while the entrants still fit the
  // arrays (expected 1024 * V * k / m <= 683; a chunk that overflows them
  // is redone with V = 1).
  auto pick_v = [&](int32_t m) { return m >= 6 * k ? 4 : (m >= 3 * k ? 2 : 1); };
  float xs[4];  // scores of this thread's run, loaded one chunk ahead
  auto load_run = [&](int32_t c0, int V) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int32_t i = min(c0 + tid * V + v, C - 1);
      xs[v] = (v < V) ? sc[s + i] : 0.f;
    }
  };
  int V = pick_v(w0);
  if (w0 < C) load_run(w0, V);
  for (int32_t c0 = w0; c0 < C;) {
    // ---- 1. this thread's candidates and the entrants ---------------------
    const uint64_t T0 = R[0];
    uint64_t key[4];
    uint32_t own;    // entrants in this thread's run
    uint32_t e, before;
    int32_t len;
    for (;;) {
      len = min(THR_CHUNK * V, C - c0);
      own = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int32_t i = tid * V + v;  // chunk-relative
        const bool valid = v < V && i < len;
        key[v] = valid ? make_key(score_code(xs[v]), s + c0 + i) : 0ull;
        own += (valid && key[v] > T0) ? 1u : 0u;
      }
      before = block_exclusive_scan_u32<THR_THREADS>(own, scan_buf, &e);
      if (e <= THR_CHUNK) break;
      V = 1;  // too many entrants for the arrays: redo with one per thread
      load_run(c0, V);
    }
    // next chunk's scores go out now; their latency overlaps this chunk
    const int32_t c_next = c0 + len;
    const int V_next = pick_v(c_next);
    uint32_t qv[4];  // entrants up to and including each of this run
    {
      uint32_t q = before;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (key[v] > T0) {
          arr[q] = key[v];
          ak[q] = key[v];
          aq[q] = q + 1;
          ++q;
        }
        qv[v] = q;
      }
    }
    if (c_next < C) load_run(c_next, V_next);
    // pad the sort to a power of two with keys above every real key
    uint32_t p2 = 1;
    while (p2 < e) p2 <<= 1;
    for (uint32_t i = e + tid; i < p2; i += THR_THREADS) {
      ak[i] = ~0ull;
      aq[i] = 0u;
    }
    __syncthreads();
    // ---- sort the entrants ascending (bitonic, pairs) ---------------------
    if (p2 <= WAVE) {
      // one wavefront, in registers: no workgroup barrier per stage
      if (tid < WAVE) {
        const int lane = tid;
        uint64_t kx = ak[lane < static_cast<int>(p2) ? lane : 0];
        uint32_t qx = aq[lane < static_cast<int>(p2) ? lane : 0];
        if (lane >= static_cast<int>(p2)) {
          kx = ~0ull;
          qx = 0u;
        }
        for (uint32_t size = 2; size <= p2; size <<= 1) {
          for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t ko = __shfl_xor(kx, static_cast<int>(stride), WAVE);
            const uint32_t qo = __shfl_xor(qx, static_cast<int>(stride), WAVE);
            const bool up = (lane & size) == 0;
            const bool lower = (lane & stride) == 0;
            const bool take_min = (lower == up);
            const bool other_smaller = ko < kx;
            if (take_min == other_smaller) {
              kx = ko;
              qx = qo;
            }
          }
        }
        if (lane < static_cast<int>(p2)) {
          ak[lane] = kx;
          aq[lane] = qx;
        }
      }
      __syncthreads();
    } else {
      for (uint32_t size = 2; size <= p2; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
          for (uint32_t i = tid; i < p2 / 2; i += THR_THREADS) {
            const uint32_t lo = 2 * i - (i & (stride - 1));
            const uint32_t hi = lo + stride;
            const bool up = (lo & size) == 0;
            const uint64_t a = ak[lo], b = ak[hi];
            if ((a > b) == up) {
              ak[lo] = b;
              ak[hi] = a;
              const uint32_t t = aq[lo];
              aq[lo] = aq[hi];
              aq[hi] = t;
            }
          }
          __syncthreads();
        }
      }
    }
    // ---- 2. threshold after every entrant --------------------------------
    // Candidates: R[i] for i <= e (rank i + #(entrants below)), and every
    // entrant (rank j + #(R below)); the e + 1 of rank <= e are the ones
    // that can be a threshold in this chunk.
    tq[0] = T0;  // written by all threads, same value
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
      // g(q) = below_r + #(arrivals 1..q below val) - q never increases;
      // val is the threshold on the steps q >= avail where g(q) = 0
      int32_t gq = below_r;  // g(0)
      uint32_t q = 0;
      while (gq > 0 && q < e) {
        gq += (arr[q] < val) ? 0 : -1;  // arrival q + 1
        ++q;
      }
      // now g(q) = 0 (or q = e with g > 0: never the threshold)
      if (gq == 0) {
        while (q <= e) {
          if (q >= avail) tq[q] = val;
          if (q == e) break;
          if (!(arr[q] < val)) break;  // g drops below 0 at q + 1
          ++q;
        }
      }
    }
    __syncthreads();
    // ---- 3. per-position thresholds ---------------------------------------
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int32_t i = tid * V + v;
      if (v < V && i < len) out[s + W + c0 + i] = tq[qv[v]];
    }
    // ---- 4. R <- the k largest of R and the entrants ----------------------
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
    V = V_next;
  }
}

__global__ void fill_u64_kernel(uint64_t* __restrict__ p, int64_t n, uint64_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_prefix_thresholds(const Geometry& geo, int32_t n_tokens, const float* scores,
                                    uint64_t* thr, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  if (geo.n_scored == 0) {
    const int64_t n = static_cast<int64_t>(geo.n_kv_heads) * n_tokens;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                       0, stream, thr, n, KEY_NONE);
    return hipGetLastError();
  }
  if (geo.n_scored > THR_KMAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prefix_thresholds_kernel, dim3(geo.n_kv_heads), dim3(THR_THREADS), 0, stream,
                     scores, n_tokens, geo.n_sink, geo.n_scored, geo.n_recent, thr);
  return hipGetLastError();
}

}  // namespace kvpop
