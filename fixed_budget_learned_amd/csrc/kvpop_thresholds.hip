// Prefix top-k thresholds of a prompt for gfx950: for every position n and
// KV head, the key of the k-th most important member of Cand(n) = {s ..
// n - W} (0 while there are fewer than k, KEY_NONE when k = 0), so that the
// kept set at n is the sinks, the window and the candidates whose key
// reaches it.  The "Qwen3-8B-KVpop-4x" model card lists a prefix top-k
// thresholds kernel among its cache backends; the contract is a reading.
//
// One 1024-thread workgroup per KV head sweeps the candidates in chunks,
// keeping the current top-k keys sorted ascending in LDS (R, k <= THR_KMAX;
// R starts as k zero keys, below every real key).  A chunk holds about
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

namespace kvpop {
namespace {

constexpr int THR_THREADS = 1024;
constexpr int THR_ARR = 1024;      // entrants one chunk can hold
constexpr int THR_VMAX = 4;        // candidates per thread
constexpr int THR_ETARGET = 192;   // expected entrants per chunk

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

__global__ __launch_bounds__(THR_THREADS) void prefix_thresholds_kernel(
    const float* __restrict__ scores, int32_t P, int32_t s, int32_t k, int32_t W,
    uint64_t* __restrict__ thr) {
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
  int32_t len = min(chunk_len(w0), C - w0);
  int V = (len + THR_THREADS - 1) / THR_THREADS;
  if (w0 < C) load_run(w0, V);
  for (int32_t c0 = w0; c0 < C;) {
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
      len = min(THR_THREADS, C - c0);  // too many entrants: one per thread
      V = 1;
      load_run(c0, V);
    }
    // next chunk's scores go out now; their latency overlaps this chunk
    const int32_t c_next = c0 + len;
    const int32_t len_next = c_next < C ? min(chunk_len(c_next), C - c_next) : 0;
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
    if (c_next < C) load_run(c_next, V_next);
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
