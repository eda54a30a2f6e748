// Prune of the Dynamic cache backend for gfx950.
//
// The "Qwen3-8B-KVpop-4x" model card ("Cache backends") lists a Dynamic
// backend that grows and then prunes under the same sink + scored top-k +
// window budget as the fixed-buffer one.  Reading taken: between prunes every
// token leaving the window is held (the decode step admits it into the slack
// without a comparison); a prune cuts each head's scored region back to its
// k most important tokens by (score, position) key, and the evicted tokens
// are gone for good.  Right after a prune a head holds exactly what the
// fixed-budget cache keeps.
//
// One 1024-thread workgroup per (sequence, KV head) of the layer; heads whose
// scored region holds no more than k tokens return at once.  With
// E = nscored - k tokens to evict:
//   1. Radix select, 8-bit digits from the top of the 64-bit keys, of the
//      E-th smallest candidate key (slots whose key is not KEY_NONE).  Keys
//      are distinct (the position is their low word), so the walk ends at the
//      latest on the last digit; it ends earlier as soon as a digit's bin
//      holds exactly the tokens still to evict.  Evicted: every candidate
//      whose key, above the final digit, is <= the selected prefix.
//   2. Compaction into [0, count - E): the i-th evicted slot below the new
//      count (a hole) receives the i-th held slot at or above it (a mover),
//      both in slot order; ranks come from one workgroup scan over per-thread
//      blocks of slots.  Sinks (the first slots) and the rows below the new
//      count that are held never move.
//   3. Movers copy their K/V rows (16-byte pieces, one row per D/8 lanes),
//      key and position; a mover in the window updates the ring entry of its
//      position.  Sources (>= new count) and destinations (< new count) are
//      disjoint, so the copies need no ordering among themselves.
//   4. Control block: new count, nscored = k, the least important held key
//      and its (possibly moved) slot, and the moved slot of the next token to
//      leave the window.
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int PR_THREADS = 1024;
constexpr int PR_WAVES = PR_THREADS / WAVE;

struct PruneParams {
  uint16_t* kc;
  uint16_t* vc;
  uint64_t* keys;
  int32_t* pos;
  int32_t* ring;
  HeadCtl* ctl;
  int32_t capacity;   // rows per head
  int32_t n_scored;   // k
  int32_t n_recent;   // W
};

__device__ __forceinline__ bool key_slot_less(uint64_t ka, int32_t sa, uint64_t kb, int32_t sb) {
  return ka < kb || (ka == kb && sa < sb);
}

// Inclusive prefix sum over the wavefront.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, WAVE);
    if (lane >= d) x += y;
  }
  return x;
}

template <int D>
__global__ __launch_bounds__(PR_THREADS) void prune_kernel(PruneParams p) {
  __shared__ uint32_t s_hist[256];
  __shared__ int32_t s_hole[PRUNE_SLACK_MAX];      // slot of the r-th hole
  __shared__ int32_t s_mover[PRUNE_SLACK_MAX];     // old slot of the r-th mover
  __shared__ int32_t s_moved_to[PRUNE_SLACK_MAX];  // new slot of old slot new_count + i
  __shared__ uint32_t s_wsum[PR_WAVES];
  __shared__ uint64_t s_mk[PR_WAVES];
  __shared__ int32_t s_ms[PR_WAVES];
  __shared__ uint64_t s_prefix;
  __shared__ int32_t s_krem, s_done;

  const int head = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
  const HeadCtl c = p.ctl[head];
  const int32_t E = c.nscored - p.n_scored;
  // uniform: nothing above k to evict (or a state no prune can have made)
  if (c.n < 0 || E <= 0 || E > PRUNE_SLACK_MAX || c.count > p.capacity) return;
  const int64_t hrow = static_cast<int64_t>(head) * p.capacity;
  const uint64_t* kyh = p.keys + hrow;
  const int32_t count = c.count;
  const int32_t ca = count - E;  // count after the prune

  // ---- 1. the E-th smallest candidate key, one 8-bit digit per pass -------
  uint64_t prefix = 0;
  int32_t krem = E;
  int shift = 64;
  for (int pass = 0; pass < 8; ++pass) {
    shift -= 8;
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();
    for (int32_t i = tid; i < count; i += PR_THREADS) {
      const uint64_t key = kyh[i];
      if (key == KEY_NONE) continue;
      if (shift < 56 && (key >> (shift + 8)) != (prefix >> (shift + 8))) continue;
      atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      // lane l scans bins 4l .. 4l+3
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = s_hist[4 * lane + j];
      const uint32_t sum4 = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_incl_scan(sum4);
      const uint32_t excl = incl - sum4;
      const uint32_t kr = static_cast<uint32_t>(krem);
      const bool mine = excl < kr && kr <= incl;
      const uint64_t any = __ballot(mine);
      if (mine) {
        uint32_t cum = excl;
        int b = 4 * lane + 3;
        uint32_t hb = h[3];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + h[j] >= kr) {
            b = 4 * lane + j;
            hb = h[j];
            break;
          }
          cum += h[j];
        }
        const uint32_t left = kr - cum;
        s_prefix = prefix | (static_cast<uint64_t>(b) << shift);
        s_krem = static_cast<int32_t>(left);
        s_done = (hb == left || shift == 0) ? 1 : 0;
      }
      if (any == 0 && lane == 0) {  // fewer candidates than nscored says
        s_prefix = prefix | (255ull << shift);
        s_krem = 0;
        s_done = 1;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    const int done = s_done;
    __syncthreads();  // every thread has read the decision before the next pass writes it
    if (done) break;
  }
  const uint64_t cut = prefix >> shift;
  auto evicted = [&](uint64_t key) { return key != KEY_NONE && (key >> shift) <= cut; };

  // ---- 2. holes and movers, ranked in slot order --------------------------
  const int32_t per = (count + PR_THREADS - 1) / PR_THREADS;
  const int32_t b0 = min(count, tid * per), b1 = min(count, b0 + per);
  uint32_t nh = 0, nm = 0;
  uint64_t mk = KEY_NONE;
  int32_t msl = 0x7FFFFFFF;
  for (int32_t i = b0; i < b1; ++i) {
    const uint64_t key = kyh[i];
    const bool ev = evicted(key);
    if (ev && i < ca) ++nh;
    if (!ev && i >= ca) ++nm;
    if (!ev && key != KEY_NONE && key_slot_less(key, i, mk, msl)) {
      mk = key;
      msl = i;
    }
  }
  // counts stay below 2^16 (at most PRUNE_SLACK_MAX each): one scan of both
  const uint32_t packed = nh | (nm << 16);
  const uint32_t wincl = wave_incl_scan(packed);
  if (lane == WAVE - 1) s_wsum[wid] = wincl;
  // least important held candidate of the wave
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) {
    const uint64_t k2 = __shfl_xor(mk, m, WAVE);
    const int32_t s2 = __shfl_xor(msl, m, WAVE);
    if (key_slot_less(k2, s2, mk, msl)) {
      mk = k2;
      msl = s2;
    }
  }
  if (lane == 0) {
    s_mk[wid] = mk;
    s_ms[wid] = msl;
  }
  __syncthreads();
  uint32_t wbase = 0;
  for (int w = 0; w < wid; ++w) wbase += s_wsum[w];
  uint32_t excl = wbase + wincl - packed;
  uint32_t hr = excl & 0xFFFFu, mr = excl >> 16;
  for (int32_t i = b0; i < b1; ++i) {
    const bool ev = evicted(kyh[i]);
    if (ev && i < ca && hr < PRUNE_SLACK_MAX) s_hole[hr++] = i;
    if (!ev && i >= ca && mr < PRUNE_SLACK_MAX) s_mover[mr++] = i;
  }
  uint32_t tot = 0;
  for (int w = 0; w < PR_WAVES; ++w) tot += s_wsum[w];
  // exactly E tokens are evicted, so there are as many holes as movers; the
  // minimum only keeps every index in range should the state say otherwise
  const int32_t nmov = static_cast<int32_t>(min(tot & 0xFFFFu, tot >> 16));
  for (int32_t i = tid; i < E; i += PR_THREADS) s_moved_to[i] = -1;
  __syncthreads();
  for (int32_t r = tid; r < nmov; r += PR_THREADS) s_moved_to[s_mover[r] - ca] = s_hole[r];

  // ---- 3. move the rows ----------------------------------------------------
  constexpr int LPR = D / 8;                  // 16-byte pieces per row
  constexpr int RPI = PR_THREADS / LPR;       // rows per iteration
  const int pc = tid % LPR;
  uint4* kc4 = reinterpret_cast<uint4*>(p.kc) + hrow * LPR;
  uint4* vc4 = reinterpret_cast<uint4*>(p.vc) + hrow * LPR;
  for (int32_t r = tid / LPR; r < nmov; r += RPI) {
    const int32_t x = s_mover[r], y = s_hole[r];
    kc4[static_cast<int64_t>(y) * LPR + pc] = kc4[static_cast<int64_t>(x) * LPR + pc];
    vc4[static_cast<int64_t>(y) * LPR + pc] = vc4[static_cast<int64_t>(x) * LPR + pc];
    if (pc == 0) {
      const uint64_t key = kyh[x];
      const int32_t ps = p.pos[hrow + x];
      p.keys[hrow + y] = key;
      p.pos[hrow + y] = ps;
      if (key == KEY_NONE)  // a window token: its ring entry follows it
        p.ring[static_cast<int64_t>(head) * p.n_recent + ps % p.n_recent] = y;
    }
  }
  __syncthreads();

  // ---- 4. control block -----------------------------------------------------
  if (tid == 0) {
    uint64_t k0 = KEY_NONE;
    int32_t sl0 = 0x7FFFFFFF;
    for (int w = 0; w < PR_WAVES; ++w)
      if (key_slot_less(s_mk[w], s_ms[w], k0, sl0)) {
        k0 = s_mk[w];
        sl0 = s_ms[w];
      }
    // new slot of a held slot (a slot at or above the new count has moved)
    auto moved = [&](int32_t x) {
      const int32_t y = (x >= ca && x < count) ? s_moved_to[x - ca] : x;
      return y >= 0 ? y : x;
    };
    HeadCtl nc = c;
    nc.count = ca;
    nc.nscored = p.n_scored;
    nc.minkey = k0;
    nc.minslot = (k0 == KEY_NONE) ? -1 : moved(sl0);
    nc.leave_slot = moved(c.leave_slot);
    p.ctl[head] = nc;
  }
}

}  // namespace

hipError_t launch_prune(const Geometry& geo, const LayerView& lv, hipStream_t stream) {
  if (geo.slack > PRUNE_SLACK_MAX) return hipErrorInvalidValue;
  PruneParams p;
  p.kc = lv.kc;
  p.vc = lv.vc;
  p.keys = lv.keys;
  p.pos = lv.pos;
  p.ring = lv.ring;
  p.ctl = lv.ctl;
  p.capacity = geo.budget;
  p.n_scored = geo.n_scored;
  p.n_recent = geo.n_recent;
  const dim3 grid(static_cast<uint32_t>(geo.batch * geo.n_kv_heads));
  if (geo.head_dim == 128)
    hipLaunchKernelGGL(prune_kernel<128>, grid, dim3(PR_THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(prune_kernel<64>, grid, dim3(PR_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvpop
