// One decode step of the fixed-budget cache for gfx950, fused into a single
// launch per layer: the delayed-eviction update and split-K GQA decode
// attention over the bounded cache.
//
// What a step does for each (sequence, KV head), token n = previous n + 1:
//   * Token t = n - W leaves the protected window and only now receives its
//     score ("Qwen3-8B-KVpop-4x" model card, "Delayed scoring").  If t is not
//     a sink it competes for a scored slot: admitted while fewer than k are
//     held, else it replaces the least important scored token when its
//     (score, position) key is larger, else it is dropped for good (KVpop
//     abstract: fixed-budget keep-or-drop eviction).
//   * Token n takes the slot that became free: a fresh slot, the evicted
//     token's slot, or the dropped token's own slot.
//   * Attention of the G query heads of the group over all kept rows.
//
// Decomposition.  The grid is (head, split): each workgroup owns a range of
// slots of one KV head.  Every workgroup re-derives the same eviction
// decision from the head's control block, so no workgroup waits for another.
// A workgroup reads K/V of its slots from the cache, except the slot the new
// token takes, whose row it takes from the k_new/v_new inputs.  It writes a
// partial softmax state (running max, sum, unnormalised accumulator) and the
// minimum key over its slots as they will be after this step.  The last
// workgroup of a head to finish (a ticket counter with device-scope
// release/acquire) merges the partials into the bf16 output, reduces the
// next minimum, and only then writes the cache update (new K/V row, keys,
// positions, window ring, control block).  All mutation therefore happens
// after every workgroup of the head has finished reading, so no read in the
// launch races with a write.
//
// Inner loop.  16 lanes share one 256-byte K row (head_dim 128; 8 lanes for
// 64) and each loads 16 bytes, so a wavefront reads 4 whole rows per
// instruction, fully coalesced.  q.k uses v_dot2 on bf16 pairs with fp32
// accumulation and a 16-lane DPP all-reduce; every row group keeps its own
// online-softmax state (exp2 domain, scale * log2(e) folded in), so the loop
// needs no workgroup barrier.  Row groups are merged through LDS at the end.
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int MAX_SPLITS = 256;

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* score_leaving;
  uint16_t* out;
  uint16_t* kc;
  uint16_t* vc;
  uint64_t* keys;
  int32_t* pos;
  int32_t* ring;
  HeadCtl* ctl;
  float* part_acc;
  float* part_ml;
  MinPart* part_min;
  uint32_t* tickets;
  int32_t n_heads;
  int32_t budget, n_sink, n_scored, n_recent;
  int32_t nsplit, rows_per_split;
  float scale_log2e;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP row controls (rows of 16 lanes).
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LPR lanes (LPR = 8 or 16, aligned); result in all lanes.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  x += dpp_f<DPP_HALF_MIRROR>(x);
  if constexpr (LPR == 16) x += dpp_f<DPP_MIRROR>(x);
  return x;
}

__device__ __forceinline__ float safe_exp2_diff(float x, float m) {
  // exp2(x - m) with exp2(-inf - anything) = 0 and m = -inf treated as 0.
  return exp2f(x - m);
}

template <int D, int G, int NP>
__global__ __launch_bounds__(DEC_THREADS) void decode_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;            // lanes per row, 16 bytes each
  constexpr int RPP = DEC_THREADS / LPR;  // rows per pass
  constexpr int CHUNK = NP * RPP;
  constexpr int NWAVE = DEC_THREADS / WAVE;

  __shared__ float s_m[RPP][G];
  __shared__ float s_l[RPP][G];
  __shared__ float s_f[RPP][G];
  __shared__ float s_acc[RPP][G * D];
  __shared__ float s_M[G], s_L[G];
  __shared__ uint64_t s_mk[NWAVE];
  __shared__ int32_t s_ms[NWAVE];
  __shared__ int32_t s_last;
  __shared__ float s_pm[MAX_SPLITS * G];
  __shared__ float s_pl[MAX_SPLITS * G];
  __shared__ float s_pf[MAX_SPLITS * G];

  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;

  // ---- workgroup -> (head, split); all splits of a head on one XCD when
  // the head count allows (workgroups are dealt to the 8 XCDs round robin).
  int head, split;
  {
    const int bid = blockIdx.x;
    if ((p.n_heads & 7) == 0) {
      const int j = bid >> 3;
      head = (bid & 7) + 8 * (j / p.nsplit);
      split = j % p.nsplit;
    } else {
      head = bid / p.nsplit;
      split = bid % p.nsplit;
    }
  }

  // ---- eviction decision, identical in every workgroup of the head -------
  const HeadCtl c = p.ctl[head];
  const int32_t W = p.n_recent;
  const int32_t n = c.n + 1;
  const int32_t t = n - W;
  int32_t newslot = c.count, count_new = c.count, nscored_new = c.nscored, st = -1;
  bool admitted = false, evict = false;
  uint64_t keyt = KEY_NONE;
  int32_t flags = c.flags;
  if (t < p.n_sink) {
    count_new = c.count + 1;                     // sink or window still filling
  } else {
    st = p.ring[static_cast<int64_t>(head) * W + (t % W)];
    const float sg = p.score_leaving[head];
    if (score_is_nan(sg)) flags |= 1;
    keyt = make_key(score_code(sg), t);
    if (c.nscored < p.n_scored) {                // free scored slot
      admitted = true;
      count_new = c.count + 1;
      nscored_new = c.nscored + 1;
    } else if (keyt > c.minkey) {                // replaces the least important
      admitted = true;
      evict = true;
      newslot = c.minslot;
    } else {                                     // dropped for good
      newslot = st;
    }
  }

  // ---- attention over slots [lo, hi) --------------------------------------
  const int32_t lo = split * p.rows_per_split;
  const int32_t hi = min(lo + p.rows_per_split, count_new);
  const int rg = tid / LPR;
  const int cc = tid % LPR;
  const int64_t hrow = static_cast<int64_t>(head) * p.budget;
  const uint4* kb = reinterpret_cast<const uint4*>(p.kc) + hrow * LPR + cc;
  const uint4* vb = reinterpret_cast<const uint4*>(p.vc) + hrow * LPR + cc;
  const uint4 knew = reinterpret_cast<const uint4*>(p.k_new)[static_cast<int64_t>(head) * LPR + cc];
  const uint4 vnew = reinterpret_cast<const uint4*>(p.v_new)[static_cast<int64_t>(head) * LPR + cc];
  uint4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = reinterpret_cast<const uint4*>(p.q)[(static_cast<int64_t>(head) * G + h) * LPR + cc];

  float m_run[G], l_run[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  for (int32_t base = lo; base < hi; base += CHUNK) {
    uint4 kr[NP], vr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int32_t r = base + i * RPP + rg;
      if (r < hi) {
        if (r == newslot) {
          kr[i] = knew;
          vr[i] = vnew;
        } else {
          kr[i] = kb[static_cast<int64_t>(r) * LPR];
          vr[i] = vb[static_cast<int64_t>(r) * LPR];
        }
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
    float x[NP][G];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const bool valid = (base + i * RPP + rg) < hi;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = dot2_bf16(kr[i].x, qv[h].x, 0.f);
        d = dot2_bf16(kr[i].y, qv[h].y, d);
        d = dot2_bf16(kr[i].z, qv[h].z, d);
        d = dot2_bf16(kr[i].w, qv[h].w, d);
        d = group_sum<LPR>(d);
        x[i][h] = valid ? d * p.scale_log2e : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m_run[h];
#pragma unroll
      for (int i = 0; i < NP; ++i) mx = fmaxf(mx, x[i][h]);
      const float ms = (mx == -INFINITY) ? 0.f : mx;
      const float alpha = safe_exp2_diff(m_run[h], ms);
      l_run[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const float pr = safe_exp2_diff(x[i][h], ms);
        l_run[h] += pr;
        acc[h][0] = fmaf(pr, bf16_lo(vr[i].x), acc[h][0]);
        acc[h][1] = fmaf(pr, bf16_hi(vr[i].x), acc[h][1]);
        acc[h][2] = fmaf(pr, bf16_lo(vr[i].y), acc[h][2]);
        acc[h][3] = fmaf(pr, bf16_hi(vr[i].y), acc[h][3]);
        acc[h][4] = fmaf(pr, bf16_lo(vr[i].z), acc[h][4]);
        acc[h][5] = fmaf(pr, bf16_hi(vr[i].z), acc[h][5]);
        acc[h][6] = fmaf(pr, bf16_lo(vr[i].w), acc[h][6]);
        acc[h][7] = fmaf(pr, bf16_hi(vr[i].w), acc[h][7]);
      }
      m_run[h] = mx;
    }
  }

  // ---- minimum key over [lo, hi) as it stands after this step -------------
  uint64_t mk = KEY_NONE;
  int32_t msl = 0x7FFFFFFF;
  for (int32_t r = lo + tid; r < hi; r += DEC_THREADS) {
    uint64_t kv;
    if (r == newslot)
      kv = KEY_NONE;
    else if (admitted && r == st)
      kv = keyt;
    else
      kv = p.keys[hrow + r];
    if (kv < mk) {
      mk = kv;
      msl = r;
    }
  }
  wave_min_key(mk, msl);
  if (lane == 0) {
    s_mk[wid] = mk;
    s_ms[wid] = msl;
  }

  // ---- merge the row groups of this workgroup ------------------------------
  if (cc == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[rg][h] = m_run[h];
      s_l[rg][h] = l_run[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[rg][h * D + cc * 8 + e] = acc[h][e];
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int r = 0; r < RPP; ++r) M = fmaxf(M, s_m[r][tid]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    for (int r = 0; r < RPP; ++r) {
      const float f = safe_exp2_diff(s_m[r][tid], Ms);
      s_f[r][tid] = f;
      L += s_l[r][tid] * f;
    }
    s_M[tid] = M;
    s_L[tid] = L;
  }
  __syncthreads();
  const int64_t pidx = static_cast<int64_t>(head) * p.nsplit + split;
  for (int e = tid; e < G * D; e += DEC_THREADS) {
    const int h = e / D;
    float a = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) a = fmaf(s_acc[r][e], s_f[r][h], a);
    p.part_acc[pidx * (G * D) + e] = a;
  }
  if (tid < G) {
    p.part_ml[(pidx * G + tid) * 2 + 0] = s_M[tid];
    p.part_ml[(pidx * G + tid) * 2 + 1] = s_L[tid];
  }
  if (tid == 0) {
    uint64_t k0 = s_mk[0];
    int32_t sl0 = s_ms[0];
    for (int w = 1; w < NWAVE; ++w) {
      if (s_mk[w] < k0 || (s_mk[w] == k0 && s_ms[w] < sl0)) {
        k0 = s_mk[w];
        sl0 = s_ms[w];
      }
    }
    MinPart mp;
    mp.key = k0;
    mp.slot = sl0;
    mp.pad = 0;
    p.part_min[pidx] = mp;
  }

  // ---- ticket: the last workgroup of the head finishes the step ----------
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&p.tickets[head], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<uint32_t>(p.nsplit - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  const int64_t p0 = static_cast<int64_t>(head) * p.nsplit;
  for (int i = tid; i < p.nsplit * G; i += DEC_THREADS) {
    const float2 ml = reinterpret_cast<const float2*>(p.part_ml)[p0 * G + i];
    s_pm[i] = ml.x;
    s_pl[i] = ml.y;
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int sp = 0; sp < p.nsplit; ++sp) M = fmaxf(M, s_pm[sp * G + tid]);
    s_M[tid] = (M == -INFINITY) ? 0.f : M;
  }
  __syncthreads();
  for (int i = tid; i < p.nsplit * G; i += DEC_THREADS) {
    const int h = i % G;
    s_pf[i] = safe_exp2_diff(s_pm[i], s_M[h]);
  }
  __syncthreads();
  if (tid < G) {
    float L = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp)
      L = fmaf(s_pl[sp * G + tid], s_pf[sp * G + tid], L);
    s_L[tid] = L;
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += DEC_THREADS) {
    const int h = e / D;
    float a = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp)
      a = fmaf(p.part_acc[(p0 + sp) * (G * D) + e], s_pf[sp * G + h], a);
    const float o = a / s_L[h];
    p.out[static_cast<int64_t>(head) * (G * D) + e] = static_cast<uint16_t>(f32_to_bf16_rne(o));
  }

  // next minimum over the head's scored slots
  {
    uint64_t k0 = KEY_NONE;
    int32_t sl0 = 0x7FFFFFFF;
    for (int sp = tid; sp < p.nsplit; sp += DEC_THREADS) {
      const MinPart mp = p.part_min[p0 + sp];
      if (mp.key < k0 || (mp.key == k0 && mp.slot < sl0)) {
        k0 = mp.key;
        sl0 = mp.slot;
      }
    }
    wave_min_key(k0, sl0);
    if (lane == 0) {
      s_mk[wid] = k0;
      s_ms[wid] = sl0;
    }
  }
  __syncthreads();

  // cache update: the new token's row, slot metadata, window ring, control
  uint4* kw = reinterpret_cast<uint4*>(p.kc) + (hrow + newslot) * LPR;
  uint4* vw = reinterpret_cast<uint4*>(p.vc) + (hrow + newslot) * LPR;
  if (tid < LPR) {
    kw[tid] = reinterpret_cast<const uint4*>(p.k_new)[static_cast<int64_t>(head) * LPR + tid];
    vw[tid] = reinterpret_cast<const uint4*>(p.v_new)[static_cast<int64_t>(head) * LPR + tid];
  }
  if (tid == 0) {
    uint64_t k0 = s_mk[0];
    int32_t sl0 = s_ms[0];
    for (int w = 1; w < NWAVE; ++w) {
      if (s_mk[w] < k0 || (s_mk[w] == k0 && s_ms[w] < sl0)) {
        k0 = s_mk[w];
        sl0 = s_ms[w];
      }
    }
    if (admitted) p.keys[hrow + st] = keyt;
    p.keys[hrow + newslot] = KEY_NONE;
    p.pos[hrow + newslot] = n;
    if (n >= p.n_sink) p.ring[static_cast<int64_t>(head) * W + (n % W)] = newslot;
    HeadCtl nc;
    nc.n = n;
    nc.count = count_new;
    nc.nscored = nscored_new;
    nc.minslot = (k0 == KEY_NONE) ? -1 : sl0;
    nc.minkey = k0;
    nc.flags = flags;
    nc.pad = 0;
    p.ctl[head] = nc;
    p.tickets[head] = 0u;
  }
  (void)evict;
}

template <int D, int G>
hipError_t launch_dg(const DecodeParams& prm, int64_t blocks, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<D, G, 4>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(DEC_THREADS), 0, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int G, const DecodeParams& prm, int64_t blocks, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dg<D, 1>(prm, blocks, stream);
    case 2: return launch_dg<D, 2>(prm, blocks, stream);
    case 4: return launch_dg<D, 4>(prm, blocks, stream);
    case 8: return launch_dg<D, 8>(prm, blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_rows_per_pass(int head_dim) { return DEC_THREADS / (head_dim / 8); }
int decode_max_splits() { return MAX_SPLITS; }

hipError_t launch_decode(const Geometry& geo, const LayerView& lv, const DecodeWork& work,
                         const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         const float* score_leaving, uint16_t* out, float scale_log2e,
                         hipStream_t stream) {
  DecodeParams prm;
  prm.q = q;
  prm.k_new = k_new;
  prm.v_new = v_new;
  prm.score_leaving = score_leaving;
  prm.out = out;
  prm.kc = lv.kc;
  prm.vc = lv.vc;
  prm.keys = lv.keys;
  prm.pos = lv.pos;
  prm.ring = lv.ring;
  prm.ctl = lv.ctl;
  prm.part_acc = work.part_acc;
  prm.part_ml = work.part_ml;
  prm.part_min = work.part_min;
  prm.tickets = work.tickets;
  prm.n_heads = geo.batch * geo.n_kv_heads;
  prm.budget = geo.budget;
  prm.n_sink = geo.n_sink;
  prm.n_scored = geo.n_scored;
  prm.n_recent = geo.n_recent;
  prm.nsplit = work.nsplit;
  prm.rows_per_split = work.rows_per_split;
  prm.scale_log2e = scale_log2e;
  const int G = geo.n_q_heads / geo.n_kv_heads;
  const int64_t blocks = static_cast<int64_t>(prm.n_heads) * work.nsplit;
  if (geo.head_dim == 128) return launch_d<128>(G, prm, blocks, stream);
  if (geo.head_dim == 64) return launch_d<64>(G, prm, blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvpop
