// One decode step of the fixed-budget cache for gfx950: the delayed-eviction
// update and split-K GQA decode attention over the bounded cache, fused into
// one launch per layer (two if the configuration asks for a second launch
// to merge split heads).
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
// decision from the head's control block (which also carries the slot of the
// token about to leave the window, so no dependent lookup is needed), so no
// workgroup waits for another.  A workgroup reads K/V of its slots from the
// cache, and substitutes the k_new/v_new row for the slot the new token
// takes.  With one split per head (batched serving) the workgroup then
// writes the output and the cache update (new K/V row, keys, positions,
// window ring, control block) itself.  With several, each writes a partial
// softmax state (max, sum, unnormalised accumulator) and the minimum key
// over its slots as they will be after this step, and the splits are merged
// into the bf16 output, followed by the cache update, in one of two ways:
//   * ticket (the default): each workgroup takes a ticket after publishing,
//     and the last one of the head merges;
//   * second launch: decode_finish_kernel, one workgroup per head, merges
//     after the launch boundary.
// Either way every mutation happens after all reads of the head's slots, so
// nothing races.  The ticket's tail is one atomic round trip and the merge's
// loads; the second launch costs a launch.  Each head's ticket counter sits
// alone in a 256-byte block: atomics on one cache line serialise in L2, and
// with the counters packed the 256 ticket atomics of a batch-1 step queued
// behind one line (12.4 us per step with the second launch, 13.0 with that
// ticket, 10.7 with one counter per block).
//
// Publishing for the ticket without an L2 writeback.  The partial results
// are written with write-through stores (SC1: 16-byte buffer stores for the
// accumulators, agent-scope atomic stores for the rest), which reach the
// device's point of coherence; each workgroup waits until all of its
// stores are acknowledged (vmcnt 0 and a barrier) before its ticket atomic.
// The finishing workgroup invalidates its L2 (agent-scope acquire) before
// it reads them.  A release fence would add a writeback of the whole L2
// (buffer_wbl2), which only ordinary cached stores need: 1.6 us per
// workgroup at batch 1.
//
// Latency.  All loads a workgroup needs (K/V and keys of its first chunk,
// q, the new row, the control block, the score) are issued before anything
// waits, and chunks (K/V rows and their keys) are double-buffered in
// registers; K/V rows are read with non-temporal loads.  The merge issues
// all of its loads at once.
//
// Inner loop.  LPR = D/16 lanes share one row; each lane holds two 16-byte
// pieces (offsets 16*lane and D + 16*lane bytes), so every load instruction
// reads whole 128/64-byte row halves, coalesced.  q.k uses v_dot2 on bf16
// pairs with fp32 accumulation and an LPR-lane DPP all-reduce.  Softmax runs
// in the exp2 domain (scale * log2(e) folded in) with one running max per
// wavefront that moves only when a logit exceeds it by 2^8, so rescaling is
// rare and no barrier is needed.  P.V takes two rows at a time: the bf16
// probabilities of both rows are packed into one register, the two rows' V
// values are interleaved with v_perm, and v_dot2 adds both products into the
// fp32 accumulator (the sum of probabilities uses the same rounded values).
// Row groups are summed with DPP inside each wave and through LDS across
// waves.
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int MAX_SPLITS = 256;

// 16-byte non-temporal load (the K/V stream is read once per step).  On
// batch 64 it raises the step from 5.9 to 6.6 TB/s; batch 1, whose layer
// fits in the last-level cache, is unchanged.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor, last word: 32-bit data format (untyped access).
constexpr int BUF_RSRC_WORD3 = 0x00020000;
// Cache-policy operand of buffer stores: SC1, write through to the device's
// point of coherence (what an agent-scope atomic store uses).
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

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
  int32_t n_heads;
  int32_t budget, n_sink, n_scored, n_recent;
  uint32_t* tickets;
  int32_t nsplit, rows_per_split;
  int32_t finish_apart;  // several splits: merged by decode_finish_kernel
  float scale_log2e;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP row controls (rows of 16 lanes).
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes (LPR = 4 or 8); result in all lanes.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (LPR == 8) x += dpp_f<DPP_HALF_MIRROR>(x);
  return x;
}

__device__ __forceinline__ bool key_less(uint64_t ka, int32_t sa, uint64_t kb, int32_t sb) {
  return ka < kb || (ka == kb && sa < sb);
}

// Full-wavefront reductions: DPP inside each 16-lane row, then two
// cross-row exchanges.  Results land in every lane.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<DPP_QUAD_XOR1>(x));
  x = fmaxf(x, dpp_f<DPP_QUAD_XOR2>(x));
  x = fmaxf(x, dpp_f<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f<DPP_ROW_MIRROR>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  x += dpp_f<DPP_HALF_MIRROR>(x);
  x += dpp_f<DPP_ROW_MIRROR>(x);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  x = fmaxf(x, __shfl_xor(x, 16, WAVE));
  return fmaxf(x, __shfl_xor(x, 32, WAVE));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16, WAVE);
  return x + __shfl_xor(x, 32, WAVE);
}

template <int CTRL>
__device__ __forceinline__ void dpp_min_key_step(uint64_t& key, int32_t& slot) {
  const uint32_t lo = static_cast<uint32_t>(key), hi = static_cast<uint32_t>(key >> 32);
  const uint32_t lo2 = __builtin_amdgcn_update_dpp(0u, lo, CTRL, 0xF, 0xF, false);
  const uint32_t hi2 = __builtin_amdgcn_update_dpp(0u, hi, CTRL, 0xF, 0xF, false);
  const int32_t s2 = __builtin_amdgcn_update_dpp(0, slot, CTRL, 0xF, 0xF, false);
  const uint64_t k2 = (static_cast<uint64_t>(hi2) << 32) | lo2;
  if (key_less(k2, s2, key, slot)) {
    key = k2;
    slot = s2;
  }
}

// Lexicographic minimum of (key, slot) over each 16-lane row, in all lanes.
__device__ __forceinline__ void row16_min_key(uint64_t& key, int32_t& slot) {
  dpp_min_key_step<DPP_QUAD_XOR1>(key, slot);
  dpp_min_key_step<DPP_QUAD_XOR2>(key, slot);
  dpp_min_key_step<DPP_HALF_MIRROR>(key, slot);
  dpp_min_key_step<DPP_ROW_MIRROR>(key, slot);
}

// ... and over the whole wavefront.
__device__ __forceinline__ void wave_min_key_dpp(uint64_t& key, int32_t& slot) {
  row16_min_key(key, slot);
#pragma unroll
  for (int m = 16; m <= 32; m *= 2) {
    const uint64_t k2 = __shfl_xor(key, m, WAVE);
    const int32_t s2 = __shfl_xor(slot, m, WAVE);
    if (key_less(k2, s2, key, slot)) {
      key = k2;
      slot = s2;
    }
  }
}

// Lazy rescaling: the running max only moves when a logit exceeds it by
// more than this many powers of two, so exponentials stay below 2^8 and the
// accumulators are rescaled rarely.
constexpr float RESCALE_SLACK = 8.f;
constexpr uint32_t BF16_ONE_PAIR = 0x3F803F80u;

// 2^x with the hardware instruction; no denormal range fix-up (results below
// 2^-126 flush to zero, which the softmax weights tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float x, int m) { return fmaxf(x, __shfl_xor(x, m, WAVE)); }

// Max over the whole wavefront of a value that is identical within aligned
// groups of LPR lanes.
template <int LPR>
__device__ __forceinline__ float wave_max_groups(float x) {
  if constexpr (LPR <= 4) x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(
                               0, __float_as_int(x), 0x124, 0xF, 0xF, false)));  // row_ror:4
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF,
                                                           false)));  // row_ror:8
  x = xor_max(x, 16);
  x = xor_max(x, 32);
  return x;
}

// Sum over the row groups of one 16-lane DPP row (lanes i, i+8 [, i+4, i+12]).
template <int LPR>
__device__ __forceinline__ float row16_sum_groups(float x) {
  if constexpr (LPR <= 4)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  return x;
}

// The step's eviction decision for one head, derived from its control block
// and the leaving token's score; every workgroup that needs it derives the
// same one.
struct Decision {
  int32_t n;            // the new token's position
  int32_t newslot;      // slot the new token takes
  int32_t count_new, nscored_new;
  int32_t st;           // slot of the leaving token (-1: none leaves)
  int32_t flags;
  bool admitted;        // the leaving token keeps a scored slot
  uint64_t keyt;        // its key
};

__device__ __forceinline__ Decision decide(const HeadCtl& c, float sg, int32_t n_sink,
                                           int32_t n_scored, int32_t W) {
  Decision d;
  d.n = c.n + 1;
  const int32_t t = d.n - W;
  d.newslot = c.count;
  d.count_new = c.count;
  d.nscored_new = c.nscored;
  d.st = -1;
  d.admitted = false;
  d.keyt = KEY_NONE;
  d.flags = c.flags;
  if (t < n_sink) {
    d.count_new = c.count + 1;                   // sink, or window still filling
  } else {
    d.st = c.leave_slot;
    if (score_is_nan(sg)) d.flags |= 1;
    d.keyt = make_key(score_code(sg), t);
    if (c.nscored < n_scored) {                  // free scored slot
      d.admitted = true;
      d.count_new = c.count + 1;
      d.nscored_new = c.nscored + 1;
    } else if (d.keyt > c.minkey) {              // replaces the least important
      d.admitted = true;
      d.newslot = c.minslot;
    } else {                                     // dropped for good
      d.newslot = d.st;
    }
  }
  return d;
}

// Merge the partial results of a head's splits into the bf16 output rows of
// its G query heads, and the splits' key minima into s_mk/s_ms (one entry
// per 16-lane row of the workgroup).  Called by the whole 256-thread
// workgroup.  Every load (accumulators, maxima and sums, key minima) is
// issued before the first wait.
template <int D, int G>
__device__ __forceinline__ void merge_splits(const DecodeParams& p, int head, float* s_buf,
                                             float* s_L, uint64_t* s_mk, int32_t* s_ms) {
  constexpr int NT = 256;
  constexpr int NWAVE = NT / WAVE;
  constexpr int R16 = WAVE / 16;
  constexpr int Q4 = G * D / 4;          // float4s in one split's accumulator
  static_assert(Q4 <= NT && NT % Q4 == 0, "merge layout");
  constexpr int TS = NT / Q4;            // threads per float4 column
  constexpr int MB = MAX_SPLITS / TS < 16 ? MAX_SPLITS / TS : 16;  // loads in flight per thread
  constexpr int SPL = MAX_SPLITS / WAVE;  // splits per lane
  static_assert(MAX_SPLITS <= NT, "one key minimum per thread");
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;
  const int r16 = lane / 16;
  const int ns = p.nsplit;
  const int64_t p0 = static_cast<int64_t>(head) * ns;
  float* s_pf = s_buf;                     // [ns][G] rescale factor
  float* s_red = s_buf + MAX_SPLITS * G;   // [TS][G*D] per-thread-group sums
  const int j4 = tid % Q4;
  const int s0 = tid / Q4;
  const float4* pacc4 = reinterpret_cast<const float4*>(p.part_acc) + j4;
  float4 raw[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int sp = s0 + u * TS;
    raw[u] = (sp < ns) ? pacc4[(p0 + sp) * Q4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  MinPart mp;
  mp.key = KEY_NONE;
  mp.slot = 0x7FFFFFFF;
  if (tid < ns) mp = p.part_min[p0 + tid];
  const float2* pml2 = reinterpret_cast<const float2*>(p.part_ml);
  for (int h = wid; h < G; h += NWAVE) {
    float2 ml[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int sp = lane + u * WAVE;
      ml[u] = (sp < ns) ? pml2[(p0 + sp) * G + h] : make_float2(-INFINITY, 0.f);
    }
    float M = ml[0].x;
#pragma unroll
    for (int u = 1; u < SPL; ++u) M = fmaxf(M, ml[u].x);
    M = wave_max(M);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int sp = lane + u * WAVE;
      const float f = fast_exp2(ml[u].x - Ms);
      if (sp < ns) s_pf[sp * G + h] = f;
      L = fmaf(ml[u].y, f, L);
    }
    L = wave_sum(L);
    if (lane == 0) s_L[h] = L;
  }
  {
    uint64_t k0 = mp.key;
    int32_t sl0 = mp.slot;
    row16_min_key(k0, sl0);
    if (lane % 16 == 0) {
      s_mk[wid * R16 + r16] = k0;
      s_ms[wid * R16 + r16] = sl0;
    }
  }
  __syncthreads();
  const int hq = (j4 * 4) / D;
  float4 a4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int sp = s0 + u * TS;
    const float f = (sp < ns) ? s_pf[sp * G + hq] : 0.f;
    a4.x = fmaf(raw[u].x, f, a4.x);
    a4.y = fmaf(raw[u].y, f, a4.y);
    a4.z = fmaf(raw[u].z, f, a4.z);
    a4.w = fmaf(raw[u].w, f, a4.w);
  }
  for (int sb = s0 + MB * TS; sb < ns; sb += MB * TS) {  // more than MB*TS splits
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int sp = sb + u * TS;
      raw[u] = (sp < ns) ? pacc4[(p0 + sp) * Q4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int sp = sb + u * TS;
      const float f = (sp < ns) ? s_pf[sp * G + hq] : 0.f;
      a4.x = fmaf(raw[u].x, f, a4.x);
      a4.y = fmaf(raw[u].y, f, a4.y);
      a4.z = fmaf(raw[u].z, f, a4.z);
      a4.w = fmaf(raw[u].w, f, a4.w);
    }
  }
  if (TS > 1) reinterpret_cast<float4*>(s_red)[s0 * Q4 + j4] = a4;
  if (TS > 1) __syncthreads();
  if (s0 == 0) {
    float4 o = a4;
    for (int ts = 1; ts < TS; ++ts) {
      const float4 y = reinterpret_cast<const float4*>(s_red)[ts * Q4 + j4];
      o.x += y.x;
      o.y += y.y;
      o.z += y.z;
      o.w += y.w;
    }
    const float invL = 1.f / s_L[hq];
    const uint32_t b0 = f32_to_bf16_rne(o.x * invL), b1 = f32_to_bf16_rne(o.y * invL);
    const uint32_t b2 = f32_to_bf16_rne(o.z * invL), b3 = f32_to_bf16_rne(o.w * invL);
    reinterpret_cast<uint2*>(p.out)[static_cast<int64_t>(head) * Q4 + j4] =
        make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  }
}

// Write the step's cache update for one head: the new K/V row, slot keys
// and position, the window ring and the control block (whose least
// important key is the minimum of the s_mk/s_ms entries).
template <int D, int G>
__device__ __forceinline__ void update_cache(const DecodeParams& p, int head, const Decision& dc,
                                             const uint4 (&knew)[2], const uint4 (&vnew)[2],
                                             int32_t ring_next, const uint64_t* s_mk,
                                             const int32_t* s_ms) {
  constexpr int NWAVE = 256 / WAVE;
  constexpr int R16 = WAVE / 16;
  constexpr int LPR = D / 16;
  constexpr int HALF4 = D / 16;
  constexpr int ROW4 = D / 8;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int64_t hrow = static_cast<int64_t>(head) * p.budget;
  const int32_t W = p.n_recent;
  if (tid < LPR) {  // lane tid holds chunks tid and tid + D/16 of the new row
    uint4* kw = reinterpret_cast<uint4*>(p.kc) + (hrow + dc.newslot) * ROW4 + tid;
    uint4* vw = reinterpret_cast<uint4*>(p.vc) + (hrow + dc.newslot) * ROW4 + tid;
    kw[0] = knew[0];
    kw[HALF4] = knew[1];
    vw[0] = vnew[0];
    vw[HALF4] = vnew[1];
  }
  if (tid < WAVE) {
    uint64_t k0 = KEY_NONE;
    int32_t sl0 = 0x7FFFFFFF;
    if (lane < NWAVE * R16) {
      k0 = s_mk[lane];
      sl0 = s_ms[lane];
    }
    wave_min_key_dpp(k0, sl0);
    if (lane == 0) {
      const int32_t n = dc.n;
      if (dc.admitted) p.keys[hrow + dc.st] = dc.keyt;
      p.keys[hrow + dc.newslot] = KEY_NONE;
      p.pos[hrow + dc.newslot] = n;
      if (n >= p.n_sink) p.ring[static_cast<int64_t>(head) * W + (n % W)] = dc.newslot;
      HeadCtl nc;
      nc.n = n;
      nc.count = dc.count_new;
      nc.nscored = dc.nscored_new;
      nc.minslot = (k0 == KEY_NONE) ? -1 : sl0;
      nc.minkey = k0;
      nc.flags = dc.flags;
      // with a one-token window the next leaving token is the one just added
      nc.leave_slot = (n + 1 - W < p.n_sink) ? -1 : (W == 1 ? dc.newslot : ring_next);
      p.ctl[head] = nc;
      p.tickets[static_cast<int64_t>(head) * TICKET_STRIDE] = 0u;
    }
  }
}

// One workgroup of 256 threads per (KV head, split).  K/V rows stream
// through registers in chunks of 2 rows per thread, double-buffered: the
// loads of the next chunk are in flight while the current one is computed.
// APART: split heads are merged by decode_finish_kernel (else by the last
// split's workgroup, after a ticket).
template <int D, int G, bool APART>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int NT = 256;
  constexpr int NP = 2;                  // rows per thread per chunk
  constexpr int LPR = D / 16;            // lanes per row; 2 x 16 bytes each
  constexpr int HALF4 = D / 16;          // uint4 offset of the second half
  constexpr int RPP = NT / LPR;          // rows per pass
  constexpr int CHUNK = NP * RPP;        // rows per chunk
  static_assert(CHUNK <= NT, "one key per thread per chunk");
  constexpr int NWAVE = NT / WAVE;
  constexpr int R16 = WAVE / 16;         // 16-lane DPP rows per wavefront
  constexpr int ACC = 16;                // accumulators per head per lane
  constexpr int Q4 = G * D / 4;          // float4s in one split's accumulator
  static_assert(Q4 <= NT, "one thread per float4 of the accumulator");
  // LDS: per (wave, DPP row, lane-in-group) the G x 16 accumulators, each
  // block padded by 8 floats so that neighbouring lanes' blocks start in
  // different LDS banks; the finishing workgroup reuses it for the split merge
  constexpr int ACC_STRIDE = G * ACC + 8;
  constexpr int LDS_ROWS = NWAVE * R16 * LPR * ACC_STRIDE;
  constexpr int LDS_MERGE = MAX_SPLITS * G + (NT / Q4) * G * D;
  static_assert(NWAVE * R16 <= WAVE, "key minima of the workgroup fit one wavefront");
  constexpr int LDS_F = LDS_ROWS > LDS_MERGE ? LDS_ROWS : LDS_MERGE;

  __shared__ __align__(16) float s_buf[LDS_F];
  __shared__ float s_wm[NWAVE][G];       // wave max (log2 units)
  __shared__ float s_wl[NWAVE][R16][G];  // per DPP-row sums of p
  __shared__ float s_L[G];
  __shared__ uint64_t s_mk[NWAVE * R16];
  __shared__ int32_t s_ms[NWAVE * R16];
  __shared__ int32_t s_last;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;

  // ---- workgroup -> (head, split); all splits of a head on one XCD when
  // the head count allows (workgroups are dealt to the 8 XCDs round robin),
  // so the head's control block, queries and new row, which every split
  // reads, come from one L2, and its ticket atomics from one XCD.
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

  // ---- issue every independent load first ---------------------------------
  const HeadCtl c = p.ctl[head];
  const float sg = p.score_leaving[head];
  const int32_t W = p.n_recent;
  const int32_t lo = split * p.rows_per_split;
  const int32_t hi_alloc = min(lo + p.rows_per_split, p.budget);
  const int rg = tid / LPR;
  const int cc = tid % LPR;
  const int64_t hrow = static_cast<int64_t>(head) * p.budget;
  constexpr int ROW4 = D / 8;            // uint4 per row
  const uint4* kb = reinterpret_cast<const uint4*>(p.kc) + hrow * ROW4 + cc;
  const uint4* vb = reinterpret_cast<const uint4*>(p.vc) + hrow * ROW4 + cc;
  const uint64_t* kyb = p.keys + hrow;

  // Load the K/V rows and keys of the chunk starting at slot b.  The loads
  // are unconditional (rows past the slot range read slot 0, and compute
  // masks them), so every chunk issues the same number of loads and the
  // compiler can wait for one chunk while the next is still in flight.
  auto load_chunk = [&](uint4 (&kk)[NP][2], uint4 (&vv)[NP][2], uint64_t& key, int32_t b) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      int32_t r = b + i * RPP + rg;
      if (r >= hi_alloc) r = 0;
      kk[i][0] = load_nt(&kb[static_cast<int64_t>(r) * ROW4]);
      kk[i][1] = load_nt(&kb[static_cast<int64_t>(r) * ROW4 + HALF4]);
      vv[i][0] = load_nt(&vb[static_cast<int64_t>(r) * ROW4]);
      vv[i][1] = load_nt(&vb[static_cast<int64_t>(r) * ROW4 + HALF4]);
    }
    const int32_t rk = b + tid % CHUNK;
    key = kyb[rk < hi_alloc ? rk : 0];  // used by threads tid < CHUNK only
  };
  uint4 kA[NP][2], vA[NP][2], kB[NP][2], vB[NP][2];
  uint64_t keyA, keyB;
  load_chunk(kA, vA, keyA, lo);
  const uint4* knp = reinterpret_cast<const uint4*>(p.k_new) + static_cast<int64_t>(head) * ROW4 + cc;
  const uint4* vnp = reinterpret_cast<const uint4*>(p.v_new) + static_cast<int64_t>(head) * ROW4 + cc;
  const uint4 knew0 = knp[0], knew1 = knp[HALF4];
  const uint4 vnew0 = vnp[0], vnew1 = vnp[HALF4];
  uint4 qv[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q) + (static_cast<int64_t>(head) * G + h) * ROW4 + cc;
    qv[h][0] = qp[0];
    qv[h][1] = qp[HALF4];
  }

  // ---- eviction decision, identical in every workgroup of the head -------
  const Decision dc = decide(c, sg, p.n_sink, p.n_scored, W);
  const int32_t newslot = dc.newslot, count_new = dc.count_new, st = dc.st;
  const bool admitted = dc.admitted;
  const uint64_t keyt = dc.keyt;
  // slot of the next token to leave (needed by the cache update)
  const int32_t ring_next = p.ring[static_cast<int64_t>(head) * W + ((dc.n + 1) % W)];

  // ---- attention over slots [lo, hi) --------------------------------------
  const int32_t hi = min(lo + p.rows_per_split, count_new);
  float m_run[G], l_run[G], acc[G][ACC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < ACC; ++e) acc[h][e] = 0.f;
  }
  uint64_t mk = KEY_NONE;
  int32_t msl = 0x7FFFFFFF;

  // one chunk: keys, logits, lazy rescale, P.V
  auto compute_chunk = [&](uint4 (&kk)[NP][2], uint4 (&vv)[NP][2], uint64_t key, int32_t base) {
    const bool full = base + CHUNK <= hi;  // uniform: every row of the chunk is kept
    // keys of this chunk, as they stand after this step
    {
      const int32_t r = base + tid;
      if (tid < CHUNK && r < hi) {
        uint64_t kv = key;
        if (r == newslot)
          kv = KEY_NONE;
        else if (admitted && r == st)
          kv = keyt;
        if (kv < mk) {
          mk = kv;
          msl = r;
        }
      }
    }
    if (newslot >= base && newslot < base + CHUNK) {  // uniform: the new token's row
#pragma unroll
      for (int i = 0; i < NP; ++i)
        if (base + i * RPP + rg == newslot) {
          kk[i][0] = knew0;
          kk[i][1] = knew1;
          vv[i][0] = vnew0;
          vv[i][1] = vnew1;
        }
    }
    if (!full) {  // unwritten slots may hold anything: zero their V
#pragma unroll
      for (int i = 0; i < NP; ++i)
        if (base + i * RPP + rg >= hi) vv[i][0] = vv[i][1] = make_uint4(0, 0, 0, 0);
    }
    float x[NP][G];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d0 = dot2_bf16(kk[i][0].x, qv[h][0].x, 0.f);
        float d1 = dot2_bf16(kk[i][1].x, qv[h][1].x, 0.f);
        d0 = dot2_bf16(kk[i][0].y, qv[h][0].y, d0);
        d1 = dot2_bf16(kk[i][1].y, qv[h][1].y, d1);
        d0 = dot2_bf16(kk[i][0].z, qv[h][0].z, d0);
        d1 = dot2_bf16(kk[i][1].z, qv[h][1].z, d1);
        d0 = dot2_bf16(kk[i][0].w, qv[h][0].w, d0);
        d1 = dot2_bf16(kk[i][1].w, qv[h][1].w, d1);
        x[i][h] = group_sum<LPR>(d0 + d1) * p.scale_log2e;
      }
      if (!full && base + i * RPP + rg >= hi) {
#pragma unroll
        for (int h = 0; h < G; ++h) x[i][h] = -INFINITY;
      }
    }
    // lazy rescale: the wave-shared running max moves only when needed
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = x[0][h];
#pragma unroll
      for (int i = 1; i < NP; ++i) mx = fmaxf(mx, x[i][h]);
      if (__any(mx > m_run[h] + RESCALE_SLACK)) {
        const float mnew = fmaxf(m_run[h], wave_max_groups<LPR>(mx));
        const float alpha = fast_exp2(m_run[h] - mnew);  // 0 while m_run is -inf
        l_run[h] *= alpha;
#pragma unroll
        for (int e = 0; e < ACC; ++e) acc[h][e] *= alpha;
        m_run[h] = mnew;
      }
    }
    // P V on row pairs: bf16 probabilities, v_dot2 over the two rows
#pragma unroll
    for (int i = 0; i < NP; i += 2) {
      uint32_t ph[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ms = (m_run[h] == -INFINITY) ? 0.f : m_run[h];
        float2_t pf = {fast_exp2(x[i][h] - ms), fast_exp2(x[i + 1][h] - ms)};
        ph[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pf, bf16x2v_t));
        l_run[h] = dot2_bf16(ph[h], BF16_ONE_PAIR, l_run[h]);
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t a[4] = {vv[i][hf].x, vv[i][hf].y, vv[i][hf].z, vv[i][hf].w};
        const uint32_t b[4] = {vv[i + 1][hf].x, vv[i + 1][hf].y, vv[i + 1][hf].z, vv[i + 1][hf].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo2 = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
          const uint32_t hi2 = __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][hf * 8 + 2 * j] = dot2_bf16(lo2, ph[h], acc[h][hf * 8 + 2 * j]);
            acc[h][hf * 8 + 2 * j + 1] = dot2_bf16(hi2, ph[h], acc[h][hf * 8 + 2 * j + 1]);
          }
        }
      }
    }
  };

  // ping-pong over chunks: load the next chunk while computing this one
  // (also after the last one, so that the load count never depends on the
  // path taken)
  for (int32_t base = lo; base < hi;) {
    load_chunk(kB, vB, keyB, base + CHUNK);
    compute_chunk(kA, vA, keyA, base);
    base += CHUNK;
    if (base >= hi) break;
    load_chunk(kA, vA, keyA, base + CHUNK);
    compute_chunk(kB, vB, keyB, base);
    base += CHUNK;
  }

  // ---- merge the row groups of the workgroup -----------------------------
  // Key minimum: DPP inside each 16-lane row, one LDS entry per row.
  const int r16 = lane / 16;
  row16_min_key(mk, msl);
  if (lane % 16 == 0) {
    s_mk[wid * R16 + r16] = mk;
    s_ms[wid * R16 + r16] = msl;
  }
  // Accumulators: all row groups of a wave share m_run, so they add plainly;
  // DPP sums the groups of each 16-lane row, LDS takes one copy per row.
  const bool writer = (lane % 16) < LPR;  // first row group of the DPP row
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lsum = row16_sum_groups<LPR>(l_run[h]);
    if (lane % 16 == 0) s_wl[wid][r16][h] = lsum;
    if (lane == 0) s_wm[wid][h] = m_run[h];
#pragma unroll
    for (int e = 0; e < ACC; ++e) acc[h][e] = row16_sum_groups<LPR>(acc[h][e]);
  }
  if (writer) {
    float4* dst = reinterpret_cast<float4*>(&s_buf[((wid * R16 + r16) * LPR + cc) * ACC_STRIDE]);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < ACC; e += 4)
        dst[(h * ACC + e) / 4] = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
  }
  __syncthreads();
  const int64_t pidx = static_cast<int64_t>(head) * p.nsplit + split;
  const bool single = (p.nsplit == 1);  // uniform
  // Each thread forms 4 consecutive outputs (same lane slot, same head):
  // element d of head h sits at lane (d mod D/2)/8, accumulator 8*(2d/D) + d%8.
  for (int o4 = tid; o4 < Q4; o4 += NT) {
    const int h = (o4 * 4) / D;
    const int d = (o4 * 4) % D;
    const int cl = (d % (D / 2)) / 8;
    const int j = (d / (D / 2)) * 8 + d % 8;
    float M = s_wm[0][h];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) M = fmaxf(M, s_wm[w][h]);
    const float Ms = (M == -INFINITY) ? 0.f : M;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const float f = fast_exp2(s_wm[w][h] - Ms);
#pragma unroll
      for (int r = 0; r < R16; ++r) {
        const float4 v = *reinterpret_cast<const float4*>(
            &s_buf[((w * R16 + r) * LPR + cl) * ACC_STRIDE + h * ACC + j]);
        a.x = fmaf(v.x, f, a.x);
        a.y = fmaf(v.y, f, a.y);
        a.z = fmaf(v.z, f, a.z);
        a.w = fmaf(v.w, f, a.w);
        L = fmaf(s_wl[w][r][h], f, L);
      }
    }
    if (single) {  // the only split: normalise and store the output row
      const float invL = 1.f / L;
      const uint32_t b0 = f32_to_bf16_rne(a.x * invL), b1 = f32_to_bf16_rne(a.y * invL);
      const uint32_t b2 = f32_to_bf16_rne(a.z * invL), b3 = f32_to_bf16_rne(a.w * invL);
      reinterpret_cast<uint2*>(p.out)[static_cast<int64_t>(head) * Q4 + o4] =
          make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    } else if (APART) {  // the launch boundary publishes them
      reinterpret_cast<float4*>(p.part_acc)[pidx * Q4 + o4] = a;
      if (d == 0) reinterpret_cast<float2*>(p.part_ml)[pidx * G + h] = make_float2(M, L);
    } else {  // written through to the point of coherence (see the file comment)
      // One 16-byte store per thread with the write-through cache bit, so a
      // wavefront writes whole cache lines (four 4-byte atomic stores wrote
      // each line four times).  The descriptor covers this split's partial.
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          p.part_acc + pidx * Q4 * 4, 0, Q4 * 16, BUF_RSRC_WORD3);
      const u32x4_t v = {__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z),
                         __float_as_uint(a.w)};
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, o4 * 16, 0, CPOL_SC1);
      if (d == 0) {
        float* pm = p.part_ml + (pidx * G + h) * 2;
        __hip_atomic_store(pm + 0, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pm + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // Several splits: publish the partial results; the second launch or the
  // last workgroup of the head to finish merges them.  A single split is
  // complete already.
  if (!single) {
    if (wid == 0) {
      uint64_t k0 = KEY_NONE;
      int32_t sl0 = 0x7FFFFFFF;
      if (lane < NWAVE * R16) {
        k0 = s_mk[lane];
        sl0 = s_ms[lane];
      }
      wave_min_key_dpp(k0, sl0);
      if (lane == 0 && APART) {
        MinPart mp;
        mp.key = k0;
        mp.slot = sl0;
        mp.pad = ring_next;  // read by the finishing launch
        p.part_min[pidx] = mp;
      } else if (lane == 0) {
        __hip_atomic_store(&p.part_min[pidx].key, k0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.part_min[pidx].slot, sl0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (APART) return;

    // ---- ticket: the last workgroup of the head finishes the step ----------
    // Every thread's write-through stores are acknowledged before thread 0
    // takes the ticket; the finisher's acquire invalidates its L2.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev =
          __hip_atomic_fetch_add(&p.tickets[static_cast<int64_t>(head) * TICKET_STRIDE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == static_cast<uint32_t>(p.nsplit - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    merge_splits<D, G>(p, head, s_buf, s_L, s_mk, s_ms);
  }

  // ---- cache update: new row, slot metadata, window ring, control block --
  const uint4 knew[2] = {knew0, knew1}, vnew[2] = {vnew0, vnew1};
  update_cache<D, G>(p, head, dc, knew, vnew, ring_next, s_mk, s_ms);
}

// Second launch of a step with several splits: one workgroup per KV head
// merges the splits' partial results into the output and writes the cache
// update.  The launch boundary orders it after every read of the first
// launch, so no ticket or release is needed.  All of its loads (control
// block, score, new row, partials) are independent and issued together.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_finish_kernel(DecodeParams p) {
  constexpr int NWAVE = 256 / WAVE;
  constexpr int R16 = WAVE / 16;
  constexpr int LPR = D / 16;
  constexpr int HALF4 = D / 16;
  constexpr int ROW4 = D / 8;
  constexpr int TS = 256 / (G * D / 4);
  __shared__ __align__(16) float s_buf[MAX_SPLITS * G + TS * G * D];
  __shared__ float s_L[G];
  __shared__ uint64_t s_mk[NWAVE * R16];
  __shared__ int32_t s_ms[NWAVE * R16];
  const int head = blockIdx.x;
  const int cc = threadIdx.x % LPR;
  const HeadCtl c = p.ctl[head];
  const float sg = p.score_leaving[head];
  const int32_t ring_next = p.part_min[static_cast<int64_t>(head) * p.nsplit].pad;
  const uint4* knp = reinterpret_cast<const uint4*>(p.k_new) + static_cast<int64_t>(head) * ROW4 + cc;
  const uint4* vnp = reinterpret_cast<const uint4*>(p.v_new) + static_cast<int64_t>(head) * ROW4 + cc;
  const uint4 knew[2] = {knp[0], knp[HALF4]};
  const uint4 vnew[2] = {vnp[0], vnp[HALF4]};
  merge_splits<D, G>(p, head, s_buf, s_L, s_mk, s_ms);
  const Decision dc = decide(c, sg, p.n_sink, p.n_scored, p.n_recent);
  update_cache<D, G>(p, head, dc, knew, vnew, ring_next, s_mk, s_ms);
}

template <int D, int G>
hipError_t launch_one(const DecodeParams& prm, int64_t blocks, hipStream_t stream) {
  // The instance with the in-launch merge runs only where it merges; one
  // split per head and the second-launch finish use the one without it.
  if (prm.nsplit > 1 && !prm.finish_apart) {
    hipLaunchKernelGGL((decode_kernel<D, G, false>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(256), 0, stream, prm);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<D, G, true>), dim3(static_cast<uint32_t>(blocks)), dim3(256),
                     0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !prm.finish_apart) return e;
  hipLaunchKernelGGL((decode_finish_kernel<D, G>), dim3(static_cast<uint32_t>(prm.n_heads)),
                     dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int G, const DecodeParams& prm, int64_t blocks, hipStream_t stream) {
  switch (G) {
    case 1: return launch_one<D, 1>(prm, blocks, stream);
    case 2: return launch_one<D, 2>(prm, blocks, stream);
    case 4: return launch_one<D, 4>(prm, blocks, stream);
    case 8: return launch_one<D, 8>(prm, blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_max_splits() { return MAX_SPLITS; }

bool decode_shape_supported(int head_dim, int group, int threads, int rows_per_thread) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8) return false;
  return threads == 256 && rows_per_thread == 2;
}

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
  prm.n_scored = geo.n_scored + geo.slack;  // the Dynamic backend grows into its slack
  prm.n_recent = geo.n_recent;
  prm.nsplit = work.nsplit;
  prm.rows_per_split = work.rows_per_split;
  prm.finish_apart = (work.nsplit > 1 && work.finish_apart) ? 1 : 0;
  prm.scale_log2e = scale_log2e;
  const int G = geo.n_q_heads / geo.n_kv_heads;
  if (work.nsplit < 1 || work.nsplit > MAX_SPLITS ||
      int64_t(work.nsplit) * work.rows_per_split < geo.budget ||
      !decode_shape_supported(geo.head_dim, G, work.threads, work.rows_per_thread))
    return hipErrorInvalidValue;
  const int64_t blocks = static_cast<int64_t>(prm.n_heads) * work.nsplit;
  if (geo.head_dim == 128) return launch_d<128>(G, prm, blocks, stream);
  return launch_d<64>(G, prm, blocks, stream);
}

}  // namespace kvpop
