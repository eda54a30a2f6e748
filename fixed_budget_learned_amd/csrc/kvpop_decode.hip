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
// token about to leave the window), so no workgroup waits for another.  A
// workgroup reads K/V of its slots from the cache and substitutes the
// k_new/v_new row, and the new keys, for the slots that change, so the slot
// contents in memory are never needed for those two slots during the step.
// That lets split 0 write the new row, the two changed keys, the new
// position and the window ring as soon as it has the decision.  Only the
// control block (read by every workgroup at its start) and the output wait
// for the end of the step.  With one split per head (batched serving) the
// workgroup writes them itself.  With several, each writes a partial
// softmax state (max, sum, unnormalised accumulator) and the minimum key of
// its slots as they stand after this step, and the splits are merged into
// the bf16 output and the new control block in one of two ways:
//   * ticket (the default): each workgroup takes a ticket after publishing,
//     and the last one of the head merges;
//   * second launch: decode_finish_kernel, one workgroup per head, merges
//     after the launch boundary.
// Each head's ticket counter sits alone in a 256-byte block: atomics on one
// cache line serialise in L2.
//
// Publishing for the ticket.  The partial results are written with
// write-through stores (cache policy SC1, what an agent-scope atomic store
// uses), which reach the device's point of coherence; each workgroup waits
// until its stores are acknowledged (vmcnt 0) and meets the others at a
// barrier before one thread takes the ticket, so every store of the
// workgroup is performed before its ticket.  The finishing workgroup reads
// the partials with coherent loads (cache policy SC1, what an agent-scope
// atomic load uses), which do not hit stale lines of its L2, so it needs no
// L2 invalidate.  A release fence would add a writeback of the whole L2,
// which only ordinary cached stores need.
//
// Latency.  At batch 1 a step is a chain: the K/V stream, then the
// reduction of a workgroup's 256 threads into one partial state, the
// publishing round trip and the ticket, then the finisher's merge.  With one
// wave per SIMD every instruction of that chain is exposed (about 4 cycles
// per instruction), so the reductions are written to keep the instruction
// count low: DPP folded into the adds, v_permlane32/16_swap transposing
// pairs of accumulators so that each level halves the registers instead of
// duplicating sums, one small LDS exchange across waves, and a finisher in
// which every thread owns a few output columns and takes one load per
// split.  The chunk loop issues no loads past the last chunk, so the
// reduction does not wait for a dummy prefetch.
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
#include <hip/hip_runtime.h>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {
namespace {

constexpr int MAX_SPLITS = 256;
}  // namespace

#ifdef KVPOP_TIMELINE
// Timeline build only (-DKVPOP_TIMELINE): thread 0 of workgroup b records
// the device clock (s_memrealtime, 100 MHz) at point i of the step in
// timeline_stamps[b % TL_SLOTS][i]; kvpop_timeline_read copies them out.
constexpr int TL_SLOTS = 4096, TL_POINTS = 8;
__device__ uint64_t timeline_stamps[TL_SLOTS * TL_POINTS];
#define TL_STAMP(i)                                                                   \
  do {                                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                \
    if (threadIdx.x == 0)                                                             \
      timeline_stamps[(blockIdx.x % TL_SLOTS) * TL_POINTS + (i)] =                    \
          __builtin_amdgcn_s_memrealtime();                                           \
    __builtin_amdgcn_sched_barrier(0);                                                \
  } while (0)
#else
#define TL_STAMP(i) \
  do {              \
  } while (0)
#endif

namespace {

// 16-byte non-temporal load (the K/V stream is read once per step).  On
// batch 64 it raises the step from 5.9 to 6.6 TB/s; batch 1, whose layer
// fits in the last-level cache, is unchanged.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Cache-policy operand of buffer accesses: SC1, coherent at agent scope
// (stores write through to the device's point of coherence; loads do not
// hit stale L2 lines).
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
  float* part_acc;    // [heads][nsplit][G*D]
  float* part_ml;     // [heads][nsplit][G][2]  (max in log2 units, sum)
  MinPart* part_min;  // [heads][nsplit]
  uint32_t* tickets;
  int32_t n_heads;
  int32_t budget, n_sink, n_scored, n_recent;
  int32_t nsplit, rows_per_split;
  float scale_log2e;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP controls (rows of 16 lanes).
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_ROR8 = 0x128;    // lane i reads lane i^8 of its row

// x read from another lane; every lane has a valid source, so bound_ctrl
// lets the compiler fold the move into the consuming add.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR lanes (LPR = 4 or 8); result in all lanes.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  if constexpr (LPR == 8) x += dpp_f<DPP_HALF_MIRROR>(x);
  return x;
}

// Full-wavefront max and sum (every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<DPP_QUAD_XOR1>(x));
  x = fmaxf(x, dpp_f<DPP_QUAD_XOR2>(x));
  x = fmaxf(x, dpp_f<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f<DPP_ROW_MIRROR>(x));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  x += dpp_f<DPP_HALF_MIRROR>(x);
  x += dpp_f<DPP_ROW_MIRROR>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Minimum of a 64-bit key over the wavefront (every lane gets it).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_mov_dpp(static_cast<uint32_t>(x), CTRL, 0xF, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_mov_dpp(static_cast<uint32_t>(x >> 32), CTRL, 0xF, 0xF, true);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return b < a ? b : a; }
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
  x = min_u64(x, dpp_u64<DPP_QUAD_XOR1>(x));
  x = min_u64(x, dpp_u64<DPP_QUAD_XOR2>(x));
  x = min_u64(x, dpp_u64<DPP_HALF_MIRROR>(x));
  x = min_u64(x, dpp_u64<DPP_ROW_MIRROR>(x));
  {
    const uint32_t lo = static_cast<uint32_t>(x), hi = static_cast<uint32_t>(x >> 32);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    x = min_u64((static_cast<uint64_t>(h[0]) << 32) | l[0], (static_cast<uint64_t>(h[1]) << 32) | l[1]);
  }
  {
    const uint32_t lo = static_cast<uint32_t>(x), hi = static_cast<uint32_t>(x >> 32);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    x = min_u64((static_cast<uint64_t>(h[0]) << 32) | l[0], (static_cast<uint64_t>(h[1]) << 32) | l[1]);
  }
  return x;
}

// Transposing pair reductions.  Each takes two per-lane values a and b and
// returns one register in which half of the lanes hold a summed with its
// partner lane and the other half b summed with its partner:
//   swap32: lanes 0-31 a(l) + a(l+32), lanes 32-63 b(l-32) + b(l)
//   swap16: rows 0, 2 a summed over rows (0,1) / (2,3); rows 1, 3 b likewise
//   xor8:   lanes with bit 3 clear a(l) + a(l^8), set b(l) + b(l^8)
//   xor4:   the same on lane bit 2
// so a value needs half an instruction pair per level and no lane holds a
// duplicate.
__device__ __forceinline__ float swap32_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_add(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor8_add(float a, float b, bool hi) {
  const float c = hi ? b : a, d = hi ? a : b;
  return c + dpp_f<DPP_ROW_ROR8>(d);
}
__device__ __forceinline__ float xor4_add(float a, float b, bool hi) {
  const float c = hi ? b : a, d = hi ? a : b;
  return c + __shfl_xor(d, 4, WAVE);
}

// Lazy rescaling: the running max only moves when a logit exceeds it by
// more than this many powers of two, so exponentials stay below 2^8 and the
// accumulators are rescaled rarely.
constexpr float RESCALE_SLACK = 8.f;

// 2^x with the hardware instruction; no denormal range fix-up (results below
// 2^-126 flush to zero, which the softmax weights tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over the whole wavefront of a value that is identical within aligned
// groups of LPR lanes.
template <int LPR>
__device__ __forceinline__ float wave_max_groups(float x) {
  if constexpr (LPR <= 4) x = fmaxf(x, dpp_f<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_f<DPP_ROW_ROR8>(x));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

// Written with selects rather than branches: the leaving token's score is
// then needed on every path, so its load is issued beside the control
// block's instead of after it (a branch would take it into the scoring case
// and make two dependent round trips of the two loads).
__device__ __forceinline__ Decision decide(const HeadCtl& c, float sg, int32_t n_sink,
                                           int32_t n_scored, int32_t W) {
  Decision d;
  d.n = c.n + 1;
  const int32_t t = d.n - W;
  const bool scoring = t >= n_sink;              // else: sink, or window still filling
  const uint64_t key = make_key(score_code(sg), t);
  const bool free_slot = c.nscored < n_scored;   // a scored slot is free
  const bool replace = !free_slot && key > c.minkey;  // replaces the least important
  d.st = scoring ? c.leave_slot : -1;
  d.flags = c.flags | ((scoring && score_is_nan(sg)) ? 1 : 0);
  d.keyt = scoring ? key : KEY_NONE;
  d.admitted = scoring && (free_slot || replace);
  d.count_new = c.count + ((!scoring || free_slot) ? 1 : 0);
  d.nscored_new = c.nscored + ((scoring && free_slot) ? 1 : 0);
  // the new token takes the next free slot, the evicted token's slot, or
  // (dropped for good) the leaving token's own slot
  d.newslot = (!scoring || free_slot) ? c.count : (replace ? c.minslot : c.leave_slot);
  return d;
}

// The slot-side part of the step's cache update: the new K/V row, the keys
// of the two slots that change, the new position and its window ring entry.
// Every workgroup of the step substitutes these values for the slots they
// concern, so they are written as soon as the decision is known (by one
// workgroup of the head).  lane < D/16 holds pieces lane and lane + D/16 of
// the new row.
template <int D>
__device__ __forceinline__ void write_slot_update(const DecodeParams& p, int head,
                                                  const Decision& dc, const uint4& kn0,
                                                  const uint4& kn1, const uint4& vn0,
                                                  const uint4& vn1) {
  constexpr int LPR = D / 16;
  constexpr int HALF4 = D / 16;
  constexpr int ROW4 = D / 8;
  const int tid = threadIdx.x;
  const int64_t hrow = static_cast<int64_t>(head) * p.budget;
  if (tid < LPR) {
    uint4* kw = reinterpret_cast<uint4*>(p.kc) + (hrow + dc.newslot) * ROW4 + tid;
    uint4* vw = reinterpret_cast<uint4*>(p.vc) + (hrow + dc.newslot) * ROW4 + tid;
    kw[0] = kn0;
    kw[HALF4] = kn1;
    vw[0] = vn0;
    vw[HALF4] = vn1;
  }
  if (tid == 0) {
    if (dc.admitted) p.keys[hrow + dc.st] = dc.keyt;
    p.keys[hrow + dc.newslot] = KEY_NONE;
    p.pos[hrow + dc.newslot] = dc.n;
    if (dc.n >= p.n_sink) p.ring[static_cast<int64_t>(head) * p.n_recent + (dc.n % p.n_recent)] =
        dc.newslot;
  }
}

// The fields of the control block that the step's decision fixes (all but
// the least important key and its slot, which need every split's minimum).
struct CtlUpdate {
  int32_t n, count, nscored, flags, leave_slot;
};

// Slot of the next token to leave the window, for the new control block.
__device__ __forceinline__ int32_t next_leave_slot(const Decision& dc, int32_t ring_next,
                                                   int32_t n_sink, int32_t W) {
  // with a one-token window the next leaving token is the one just added
  return (dc.n + 1 - W < n_sink) ? -1 : (W == 1 ? dc.newslot : ring_next);
}

__device__ __forceinline__ CtlUpdate make_update(const Decision& dc, int32_t ring_next,
                                                 int32_t n_sink, int32_t W) {
  return CtlUpdate{dc.n, dc.count_new, dc.nscored_new, dc.flags,
                   next_leave_slot(dc, ring_next, n_sink, W)};
}

// The control block after the step.  Thread 0 writes every field but
// minslot; minslot is written by the thread that holds the least important
// key (-1 by thread 0 when no scored token is held).
__device__ __forceinline__ void write_ctl(const DecodeParams& p, int head, const CtlUpdate& u,
                                          uint64_t minkey, bool zero_thread, bool holds_min,
                                          int32_t minslot) {
  HeadCtl* c = p.ctl + head;
  if (zero_thread) {
    c->n = u.n;
    c->count = u.count;
    c->nscored = u.nscored;
    c->minkey = minkey;
    c->flags = u.flags;
    c->leave_slot = u.leave_slot;
    if (minkey == KEY_NONE) c->minslot = -1;
  }
  if (holds_min && minkey != KEY_NONE) c->minslot = minslot;
}

// Window ring entry of the token that leaves at the next step (read by the
// workgroup that writes the control block).
__device__ __forceinline__ int32_t read_ring_next(const DecodeParams& p, int head,
                                                  const Decision& dc) {
  const int32_t W = p.n_recent;
  if (W == 1 || dc.n + 1 - W < p.n_sink) return -1;
  return p.ring[static_cast<int64_t>(head) * W + ((dc.n + 1) % W)];
}

// LDS of the split merge.
struct FinishLds {
  float f[8][MAX_SPLITS];  // [head of the group][split] rescale factor (0 past nsplit)
  float L[8];              // [head] merged softmax sum
  uint64_t wmin[4];        // [wave] least important key of the splits it read
};

// Merge the nsplit partial states of `head` into its bf16 output rows and
// write the new control block.  Called by all 256 threads of one workgroup.
// COHERENT: read the partials with SC1 loads (in-launch ticket; the second
// launch reads after the launch boundary).  Every thread owns FPT
// consecutive output columns and issues one load per split for them, all
// before the first wait; loads past the last split fall outside the buffer
// descriptors' ranges and read 0, so no load needs a branch.  The splits'
// (max, sum) pairs are turned into per-split factors by one wavefront per
// query head.  get_update() yields the step's control-block fields; it is
// called only after every load has been issued, so a merge that reads them
// from memory waits for them together with the partials.
template <int D, int G, bool COHERENT, class GetUpdate>
__device__ __forceinline__ void finish_head(const DecodeParams& p, int head,
                                            GetUpdate get_update, FinishLds& fl) {
  constexpr int NT = 256;
  constexpr int NWAVE = NT / WAVE;
  constexpr int GD = G * D;
  constexpr int FPT = GD >= NT ? GD / NT : 1;
  constexpr int NACT = GD / FPT;
  constexpr int MB = 32;                 // splits loaded per batch
  constexpr int SPL = MAX_SPLITS / WAVE;
  constexpr int HPW = (G + NWAVE - 1) / NWAVE;  // query heads per wave
  constexpr int CP = COHERENT ? CPOL_SC1 : 0;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;
  const int ns = p.nsplit;
  const int64_t p0 = static_cast<int64_t>(head) * ns;

  const __amdgpu_buffer_rsrc_t r_acc = __builtin_amdgcn_make_buffer_rsrc(
      p.part_acc + p0 * GD, 0, ns * GD * 4, BUF_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t r_ml = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + p0 * G * 2, 0, ns * G * 8, BUF_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t r_min = __builtin_amdgcn_make_buffer_rsrc(
      p.part_min + p0, 0, ns * 16, BUF_RSRC_WORD3);

  // ---- issue the loads: key minima, (max, sum) pairs, the first batch of
  // accumulators, and the ring entry of the next leaving token
  const u32x2_t kraw = __builtin_amdgcn_raw_buffer_load_b64(r_min, tid * 16, 0, CP);
  const uint32_t sraw = __builtin_amdgcn_raw_buffer_load_b32(r_min, tid * 16 + 8, 0, CP);
  u32x2_t ml[HPW][SPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = wid + hh * NWAVE;
    if (h < G) {  // uniform
#pragma unroll
      for (int u = 0; u < SPL; ++u)
        ml[hh][u] = __builtin_amdgcn_raw_buffer_load_b64(r_ml, ((lane + u * WAVE) * G + h) * 8, 0, CP);
    }
  }
  float raw[MB][FPT];
  auto load_batch = [&](int sb) {
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const uint32_t off = static_cast<uint32_t>(((sb + u) * GD + tid * FPT) * 4);
      if constexpr (FPT == 4) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r_acc, off, 0, CP);
        raw[u][0] = __uint_as_float(v.x);
        raw[u][1] = __uint_as_float(v.y);
        raw[u][2] = __uint_as_float(v.z);
        raw[u][3] = __uint_as_float(v.w);
      } else if constexpr (FPT == 2) {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r_acc, off, 0, CP);
        raw[u][0] = __uint_as_float(v.x);
        raw[u][1] = __uint_as_float(v.y);
      } else {
        raw[u][0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_acc, off, 0, CP));
      }
    }
  };
  load_batch(0);

  // ---- per query head: M = max of the splits' maxima, factor 2^(m_s - M)
  // (0 past the last split), merged sum
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = wid + hh * NWAVE;
    if (h < G) {  // uniform
      float mv[SPL];
      float M = -INFINITY;
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        mv[u] = (lane + u * WAVE < ns) ? __uint_as_float(ml[hh][u].x) : -INFINITY;
        M = fmaxf(M, mv[u]);
      }
      M = wave_max(M);
      const float Ms = (M == -INFINITY) ? 0.f : M;
      float Lsum = 0.f;
#pragma unroll
      for (int u = 0; u < SPL; ++u) {
        const float f = fast_exp2(mv[u] - Ms);
        fl.f[h][lane + u * WAVE] = f;
        Lsum = fmaf(__uint_as_float(ml[hh][u].y), f, Lsum);
      }
      Lsum = wave_sum(Lsum);
      if (lane == 0) fl.L[h] = Lsum;
    }
  }
  // ---- the least important key over the splits (keys are unique)
  const uint64_t mkey = tid < ns ? (static_cast<uint64_t>(kraw.y) << 32) | kraw.x : KEY_NONE;
  {
    const uint64_t wm = wave_min_u64(mkey);
    if (lane == 0) fl.wmin[wid] = wm;
  }
  __syncthreads();
  TL_STAMP(6);  // finisher: split factors and barrier

  // ---- accumulate this thread's columns over the splits
  const bool act = tid < NACT;
  const int hq = act ? (tid * FPT) / D : 0;
  float a[FPT];
#pragma unroll
  for (int j = 0; j < FPT; ++j) a[j] = 0.f;
  for (int sb = 0; sb < ns; sb += MB) {
    if (sb > 0) load_batch(sb);
#pragma unroll
    for (int u = 0; u < MB; u += 4) {
      const float4 f4 = *reinterpret_cast<const float4*>(&fl.f[hq][sb + u]);
      const float fu[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int j = 0; j < FPT; ++j) a[j] = fmaf(raw[u + k][j], fu[k], a[j]);
    }
  }
  if (act) {
    const float invL = 1.f / fl.L[hq];
    uint16_t* o = p.out + static_cast<int64_t>(head) * GD + tid * FPT;
    if constexpr (FPT == 1) {
      *o = static_cast<uint16_t>(f32_to_bf16_rne(a[0] * invL));
    } else {
      uint32_t w[FPT / 2];
#pragma unroll
      for (int j = 0; j < FPT / 2; ++j)
        w[j] = f32_to_bf16_rne(a[2 * j] * invL) | (f32_to_bf16_rne(a[2 * j + 1] * invL) << 16);
      if constexpr (FPT == 2) *reinterpret_cast<uint32_t*>(o) = w[0];
      else *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
    }
  }
  const uint64_t minkey = min_u64(min_u64(fl.wmin[0], fl.wmin[1]), min_u64(fl.wmin[2], fl.wmin[3]));
  write_ctl(p, head, get_update(), minkey, tid == 0, mkey == minkey, static_cast<int32_t>(sraw));
  if (tid == 0) p.tickets[static_cast<int64_t>(head) * TICKET_STRIDE] = 0u;
#ifdef KVPOP_TIMELINE
  __builtin_amdgcn_s_waitcnt(0);
#endif
  TL_STAMP(7);  // finisher done, its stores acknowledged
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
  constexpr int ACC = 16;                // accumulators per head per lane
  constexpr int NV = G * ACC;            // accumulators per lane
  constexpr int RGW = WAVE / LPR;        // row groups per wavefront (8 or 16)
  constexpr int NVF = NV / RGW;          // accumulators per lane after the wave reduction
  constexpr int GD = G * D;
  constexpr int FPT = GD >= NT ? GD / NT : 1;  // output columns per thread in the combine
  constexpr int NACT = GD / FPT;
  constexpr int ROW4 = D / 8;            // uint4 per row

  __shared__ __align__(16) float s_wacc[NWAVE][GD];   // each wave's accumulators
  __shared__ float2 s_wml[NWAVE][G];                  // each wave's (max, sum)
  __shared__ uint64_t s_wmin[NWAVE];                  // each wave's least important key
  __shared__ int32_t s_last;
  __shared__ __align__(16) FinishLds s_fin;
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;
  TL_STAMP(0);

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
  const uint4* kb = reinterpret_cast<const uint4*>(p.kc) + hrow * ROW4 + cc;
  const uint4* vb = reinterpret_cast<const uint4*>(p.vc) + hrow * ROW4 + cc;
  const uint64_t* kyb = p.keys + hrow;

  // Load the K/V rows and keys of the chunk starting at slot b.  Rows past
  // the slot range read slot 0 (compute masks them).
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
  if (split == 0) write_slot_update<D>(p, head, dc, knew0, knew1, vnew0, vnew1);
  // the next leaving token's slot (for the control block), read while the
  // K/V loads are in flight; only the workgroup that finishes uses it
  const int32_t ring_next = read_ring_next(p, head, dc);

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
    // P V in fp32: each V element widened from bf16 (exact) and multiplied
    // by the fp32 probability; the sum of probabilities adds the same values
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      float pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ms = (m_run[h] == -INFINITY) ? 0.f : m_run[h];
        pr[h] = fast_exp2(x[i][h] - ms);
        l_run[h] += pr[h];
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const uint32_t a[4] = {vv[i][hf].x, vv[i][hf].y, vv[i][hf].z, vv[i][hf].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = bf16_lo(a[j]), hi = bf16_hi(a[j]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][hf * 8 + 2 * j] = fmaf(lo, pr[h], acc[h][hf * 8 + 2 * j]);
            acc[h][hf * 8 + 2 * j + 1] = fmaf(hi, pr[h], acc[h][hf * 8 + 2 * j + 1]);
          }
        }
      }
    }
  };

  // Chunks.  A split of one chunk loads nothing more; a split of two
  // (batch 1) requests both at once and computes them in order, so no load
  // is left in flight after the last one.  Longer splits ping-pong: the next chunk's loads are issued
  // before the current one is computed (and after the last, whose loads
  // read slot 0), so the load count never depends on the path taken and
  // the compiler's wait for the current chunk counts exactly the loads
  // issued after it.
  const int32_t nch = hi > lo ? (hi - lo + CHUNK - 1) / CHUNK : 0;
  if (nch == 2) {
    load_chunk(kB, vB, keyB, lo + CHUNK);
    compute_chunk(kA, vA, keyA, lo);
    compute_chunk(kB, vB, keyB, lo + CHUNK);
  } else if (nch < 2) {  // one chunk (or none): nothing more to load
    if (nch > 0) compute_chunk(kA, vA, keyA, lo);
  } else {
    for (int32_t base = lo; base < hi;) {
      load_chunk(kB, vB, keyB, base + CHUNK);
      compute_chunk(kA, vA, keyA, base);
      base += CHUNK;
      if (base >= hi) break;
      load_chunk(kA, vA, keyA, base + CHUNK);
      compute_chunk(kB, vB, keyB, base);
      base += CHUNK;
    }
  }

  TL_STAMP(1);  // wave 0's chunk loop done
  // ---- reduce the workgroup to one softmax state ---------------------------
  // Inside each wave: the row groups share m_run, so their accumulators add
  // plainly.  The transposing pair reductions leave lane l with NVF
  // consecutive accumulator indices [NVF * (l / LPR), +NVF) of its column
  // slot cc, summed over all row groups of the wave.
  {
    float v[NV];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < ACC; ++e) v[h * ACC + e] = acc[h][e];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) v[i] = swap32_add(v[i], v[i + NV / 2]);
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) v[i] = swap16_add(v[i], v[i + NV / 4]);
    const bool b3 = (lane >> 3) & 1;
#pragma unroll
    for (int i = 0; i < NV / 8; ++i) v[i] = xor8_add(v[i], v[i + NV / 8], b3);
    if constexpr (LPR == 4) {
      const bool b2 = (lane >> 2) & 1;
#pragma unroll
      for (int i = 0; i < NV / 16; ++i) v[i] = xor4_add(v[i], v[i + NV / 16], b2);
    }
    // accumulator index vi = h * 16 + e holds column (e / 8) * D/2 + 8 cc + e % 8
    const int vb = NVF * (lane / LPR);
#pragma unroll
    for (int i = 0; i < NVF; i += (NVF >= 4 ? 4 : NVF)) {
      const int vi = vb + i;
      const int h = vi / ACC, e = vi % ACC;
      float* dst = &s_wacc[wid][h * D + (e / 8) * (D / 2) + 8 * cc + e % 8];
      if constexpr (NVF >= 4) *reinterpret_cast<float4*>(dst) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
      else if constexpr (NVF == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[i], v[i + 1]);
      else *dst = v[i];
    }
    // each wave's sum of p: l_run is the same in the LPR lanes of a row group
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float l = swap32_add(l_run[h], l_run[h]);
      l = swap16_add(l, l);
      l += dpp_f<DPP_ROW_ROR8>(l);
      if constexpr (LPR == 4) l += __shfl_xor(l, 4, WAVE);
      if (lane == 0) s_wml[wid][h] = make_float2(m_run[h], l);
    }
  }
  {
    const uint64_t wm = wave_min_u64(mk);
    if (lane == 0) s_wmin[wid] = wm;
  }
  __syncthreads();
  TL_STAMP(2);

  // ---- combine the waves: thread t owns columns [t * FPT, +FPT) ------------
  const uint64_t wg_minkey = min_u64(min_u64(s_wmin[0], s_wmin[1]), min_u64(s_wmin[2], s_wmin[3]));
  const bool holds_min = (mk == wg_minkey);  // only meaningful for a real key
  const bool act = tid < NACT;
  const int hq = (tid * FPT) / D;
  float a[FPT];
  float M = -INFINITY, Lsum = 0.f;
  {
    float2 wml[NWAVE];
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      wml[w] = s_wml[w][act ? hq : 0];
      M = fmaxf(M, wml[w].x);
    }
    const float Ms = (M == -INFINITY) ? 0.f : M;
#pragma unroll
    for (int j = 0; j < FPT; ++j) a[j] = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const float f = fast_exp2(wml[w].x - Ms);
      Lsum = fmaf(wml[w].y, f, Lsum);
      const float* src = &s_wacc[w][act ? tid * FPT : 0];
      float xs[FPT];
      if constexpr (FPT == 4) {
        const float4 t4 = *reinterpret_cast<const float4*>(src);
        xs[0] = t4.x; xs[1] = t4.y; xs[2] = t4.z; xs[3] = t4.w;
      } else if constexpr (FPT == 2) {
        const float2 t2 = *reinterpret_cast<const float2*>(src);
        xs[0] = t2.x; xs[1] = t2.y;
      } else {
        xs[0] = *src;
      }
#pragma unroll
      for (int j = 0; j < FPT; ++j) a[j] = fmaf(xs[j], f, a[j]);
    }
  }

  if (p.nsplit == 1) {  // uniform: the only split; output and control block here
    if (act) {
      const float invL = 1.f / Lsum;
      uint16_t* o = p.out + static_cast<int64_t>(head) * GD + tid * FPT;
      if constexpr (FPT == 1) {
        *o = static_cast<uint16_t>(f32_to_bf16_rne(a[0] * invL));
      } else {
        uint32_t w[FPT / 2];
#pragma unroll
        for (int j = 0; j < FPT / 2; ++j)
          w[j] = f32_to_bf16_rne(a[2 * j] * invL) | (f32_to_bf16_rne(a[2 * j + 1] * invL) << 16);
        if constexpr (FPT == 2) *reinterpret_cast<uint32_t*>(o) = w[0];
        else *reinterpret_cast<uint2*>(o) = make_uint2(w[0], w[1]);
      }
    }
    write_ctl(p, head, make_update(dc, ring_next, p.n_sink, W), wg_minkey, tid == 0, holds_min,
              msl);
    return;
  }

  // ---- several splits: publish this split's partial state -----------------
  const int64_t pidx = static_cast<int64_t>(head) * p.nsplit + split;
  {
    constexpr int CP = APART ? 0 : CPOL_SC1;  // the launch boundary publishes for APART
    const __amdgpu_buffer_rsrc_t r_acc =
        __builtin_amdgcn_make_buffer_rsrc(p.part_acc + pidx * GD, 0, GD * 4, BUF_RSRC_WORD3);
    if (act) {
      const uint32_t off = static_cast<uint32_t>(tid * FPT * 4);
      if constexpr (FPT == 4)
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                    __float_as_uint(a[3])}, r_acc, off, 0, CP);
      else if constexpr (FPT == 2)
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(a[0]), __float_as_uint(a[1])},
                                              r_acc, off, 0, CP);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a[0]), r_acc, off, 0, CP);
      if ((tid * FPT) % D == 0) {
        const __amdgpu_buffer_rsrc_t r_ml =
            __builtin_amdgcn_make_buffer_rsrc(p.part_ml + pidx * G * 2, 0, G * 8, BUF_RSRC_WORD3);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(M), __float_as_uint(Lsum)},
                                              r_ml, hq * 8, 0, CP);
      }
    }
    // key minimum of the split: key by thread 0, slot by the thread holding it
    const __amdgpu_buffer_rsrc_t r_min =
        __builtin_amdgcn_make_buffer_rsrc(p.part_min + pidx, 0, 16, BUF_RSRC_WORD3);
    if (tid == 0)
      __builtin_amdgcn_raw_buffer_store_b64(
          u32x2_t{static_cast<uint32_t>(wg_minkey), static_cast<uint32_t>(wg_minkey >> 32)}, r_min, 0,
          0, CP);
    if (holds_min && wg_minkey != KEY_NONE)
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(msl), r_min, 8, 0, CP);
    // the second launch takes the step's control-block fields from here, so
    // its loads need neither the control block nor a decision of their own
    if (APART && split == 0 && tid == 0) {
      const CtlUpdate u = make_update(dc, ring_next, p.n_sink, W);
      const __amdgpu_buffer_rsrc_t r_u = __builtin_amdgcn_make_buffer_rsrc(
          p.tickets + static_cast<int64_t>(head) * TICKET_STRIDE + UPDATE_WORD, 0, 32,
          BUF_RSRC_WORD3);
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4_t{static_cast<uint32_t>(u.n), static_cast<uint32_t>(u.count),
                  static_cast<uint32_t>(u.nscored), static_cast<uint32_t>(u.flags)},
          r_u, 0, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(u.leave_slot), r_u, 16, 0, 0);
    }
  }
  TL_STAMP(3);  // partial state stored (issued)
  if (APART) return;

  // ---- ticket: the last workgroup of the head finishes the step ------------
  // Every thread's write-through stores are acknowledged before thread 0
  // takes the ticket.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  TL_STAMP(4);  // every store of the workgroup acknowledged
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(
        &p.tickets[static_cast<int64_t>(head) * TICKET_STRIDE], 1u, __ATOMIC_RELAXED,
        __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<uint32_t>(p.nsplit - 1)) ? 1 : 0;
  }
  __syncthreads();
  TL_STAMP(5);  // ticket returned
  if (!s_last) return;
  finish_head<D, G, true>(p, head, [&] { return make_update(dc, ring_next, p.n_sink, W); },
                          s_fin);
}

// Second launch of a step with several splits: one workgroup per KV head
// merges the splits' partial results into the output and writes the control
// block.  The launch boundary orders it after every access of the first
// launch, so no ticket is needed.  The control-block fields come from split
// 0's record in the head's ticket block; they are loaded with the partials,
// so the merge waits for one round of loads.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_finish_kernel(DecodeParams p) {
  __shared__ __align__(16) FinishLds s_fin;
  const int head = blockIdx.x;
  const __amdgpu_buffer_rsrc_t r_u = __builtin_amdgcn_make_buffer_rsrc(
      p.tickets + static_cast<int64_t>(head) * TICKET_STRIDE + UPDATE_WORD, 0, 32,
      BUF_RSRC_WORD3);
  const u32x4_t u4 = __builtin_amdgcn_raw_buffer_load_b128(r_u, 0, 0, 0);
  const uint32_t u5 = __builtin_amdgcn_raw_buffer_load_b32(r_u, 16, 0, 0);
  finish_head<D, G, false>(
      p, head,
      [&] {
        return CtlUpdate{static_cast<int32_t>(__builtin_amdgcn_readfirstlane(u4.x)),
                         static_cast<int32_t>(__builtin_amdgcn_readfirstlane(u4.y)),
                         static_cast<int32_t>(__builtin_amdgcn_readfirstlane(u4.z)),
                         static_cast<int32_t>(__builtin_amdgcn_readfirstlane(u4.w)),
                         static_cast<int32_t>(__builtin_amdgcn_readfirstlane(u5))};
      },
      s_fin);
}

template <int D, int G>
hipError_t launch_one(const DecodeParams& prm, bool apart, int64_t blocks, hipStream_t stream) {
  // The instance with the in-launch merge runs only where it merges; one
  // split per head and the second-launch finish use the one without it.
  if (prm.nsplit > 1 && !apart) {
    hipLaunchKernelGGL((decode_kernel<D, G, false>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(256), 0, stream, prm);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<D, G, true>), dim3(static_cast<uint32_t>(blocks)), dim3(256),
                     0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.nsplit == 1) return e;
  hipLaunchKernelGGL((decode_finish_kernel<D, G>), dim3(static_cast<uint32_t>(prm.n_heads)),
                     dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(int G, const DecodeParams& prm, bool apart, int64_t blocks,
                    hipStream_t stream) {
  switch (G) {
    case 1: return launch_one<D, 1>(prm, apart, blocks, stream);
    case 2: return launch_one<D, 2>(prm, apart, blocks, stream);
    case 4: return launch_one<D, 4>(prm, apart, blocks, stream);
    case 8: return launch_one<D, 8>(prm, apart, blocks, stream);
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
                         int32_t n_layers, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, const float* score_leaving, uint16_t* out,
                         float scale_log2e, hipStream_t stream) {
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
  prm.n_heads = n_layers * geo.batch * geo.n_kv_heads;
  prm.budget = geo.budget;
  prm.n_sink = geo.n_sink;
  prm.n_scored = geo.n_scored + geo.slack;  // the Dynamic backend grows into its slack
  prm.n_recent = geo.n_recent;
  prm.nsplit = work.nsplit;
  prm.rows_per_split = work.rows_per_split;
  prm.scale_log2e = scale_log2e;
  const int G = geo.n_q_heads / geo.n_kv_heads;
  if (n_layers < 1 || work.nsplit < 1 || work.nsplit > MAX_SPLITS ||
      int64_t(work.nsplit) * work.rows_per_split < geo.budget ||
      !decode_shape_supported(geo.head_dim, G, work.threads, work.rows_per_thread))
    return hipErrorInvalidValue;
  const bool apart = work.nsplit > 1 && work.finish_apart;
  const int64_t blocks = static_cast<int64_t>(prm.n_heads) * work.nsplit;
  if (geo.head_dim == 128) return launch_d<128>(G, prm, apart, blocks, stream);
  return launch_d<64>(G, prm, apart, blocks, stream);
}

}  // namespace kvpop

#ifdef KVPOP_TIMELINE
// Timeline build only: copy the first n_slots workgroups' stamps
// ([n_slots][8] device-clock ticks, 0 where a point was not reached) to
// host memory, or zero them on the device.
extern "C" __attribute__((visibility("default"))) int kvpop_timeline_read(uint64_t* host,
                                                                         int n_slots) {
  if (n_slots < 0 || n_slots > kvpop::TL_SLOTS) return -1;
  return static_cast<int>(hipMemcpyFromSymbol(host, HIP_SYMBOL(kvpop::timeline_stamps),
                                              size_t(n_slots) * kvpop::TL_POINTS * 8, 0,
                                              hipMemcpyDeviceToHost));
}
extern "C" __attribute__((visibility("default"))) int kvpop_timeline_clear() {
  static const uint64_t zero[kvpop::TL_SLOTS * kvpop::TL_POINTS] = {};
  return static_cast<int>(hipMemcpyToSymbol(HIP_SYMBOL(kvpop::timeline_stamps), zero,
                                            sizeof(zero), 0, hipMemcpyHostToDevice));
}
#endif
