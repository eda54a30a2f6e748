// Internal layout and launcher declarations shared by the C-ABI host code
// (kvpop_abi.cpp) and the HIP kernels (kvpop_*.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kvpop {

// Importance key of a scored token: (score, position) compared
// lexicographically, packed so that unsigned integer order equals key order.
// The high word is the float32 score mapped to an order-preserving unsigned
// code (-0 folded onto +0); the low word is the position.  KEY_NONE is larger
// than every real key (positions stay below 2^31) and marks slots that are
// not scored (sinks, window) so a minimum over a slot range skips them.
constexpr uint64_t KEY_NONE = ~0ull;

// Per (layer, sequence, KV head) control block, 32 bytes.
struct HeadCtl {
  int32_t n;        // newest processed position, -1 when empty
  int32_t count;    // occupied slots are [0, count)
  int32_t nscored;  // slots holding scored tokens
  int32_t minslot;  // slot of the least important scored token (-1: none)
  uint64_t minkey;  // its key, KEY_NONE when nscored == 0
  int32_t flags;    // KVPOP_FLAG_* bits
  int32_t leave_slot;  // slot of position n + 1 - W (the next token to leave
                       // the window); meaningful only when that is >= s
};
static_assert(sizeof(HeadCtl) == 32, "HeadCtl layout");

// Partial minimum of one split of a head's slot range (pad: unused, keeps
// the record at 16 bytes).
struct MinPart {
  uint64_t key;
  int32_t slot;
  int32_t pad;
};
static_assert(sizeof(MinPart) == 16, "MinPart layout");

// Device views of one layer of the cache.  Head index = seq * Hkv + g.
// `budget` below is the row capacity of a head (Geometry::budget).
struct LayerView {
  uint16_t* kc;     // [B][Hkv][budget][D] bf16
  uint16_t* vc;     // [B][Hkv][budget][D] bf16
  uint64_t* keys;   // [B][Hkv][budget]
  int32_t* pos;     // [B][Hkv][budget]
  int32_t* ring;    // [B][Hkv][W]  slot of window position p at p % W
  HeadCtl* ctl;     // [B][Hkv]
};

// n_scored is k, the scored top-k the cache keeps.  slack is the growth room
// of the Dynamic backend (0: Static): its scored region holds up to
// k + slack tokens between prunes.  budget is the row capacity of a head,
// n_sink + n_scored + n_recent + slack.
struct Geometry {
  int32_t batch, n_q_heads, n_kv_heads, head_dim;
  int32_t n_sink, n_scored, n_recent, budget;
  int32_t slack;
};

// Each head's split ticket sits alone in a 256-byte block: atomics on one
// cache line serialise in L2, so heads sharing a line would queue together.
// Words UPDATE_WORD .. UPDATE_WORD + 4 of the block carry, from split 0 to a
// second-launch merge, the control-block fields the step's decision fixes
// (n, count, nscored, flags, leave_slot).
constexpr int TICKET_STRIDE = 64;
constexpr int UPDATE_WORD = 8;

// Decode workspace, shared by every layer (calls are stream-ordered).
struct DecodeWork {
  float* part_acc;     // [heads][nsplit][G*D] unnormalised accumulators
  float* part_ml;      // [heads][nsplit][G][2]  (running max in log2 units, sum)
  MinPart* part_min;   // [heads][nsplit]  least important key of the split and its slot
  uint32_t* tickets;   // [B*Hkv][TICKET_STRIDE]: element 0 the ticket, zero between calls;
                       // elements UPDATE_WORD.. split 0's control-block fields
  int32_t nsplit;
  int32_t rows_per_split;
  int32_t threads;     // workgroup size of the decode kernel (256)
  int32_t rows_per_thread;  // K/V rows one thread holds per pass (2)
  int32_t finish_apart;     // several splits: merge in a second launch
};

// Launchers: return hipSuccess or the launch error.  All work is enqueued
// on `stream`; nothing is synchronised.
hipError_t launch_init_ctl(HeadCtl* ctl, int64_t n_heads, uint32_t* tickets, int64_t n_tickets,
                           hipStream_t stream);
// Prefill workspace (one per cache; calls are stream-ordered).  Long prompts
// select in two levels: up to SLICE_MAX slices per head first keep a
// superset of their share of the head's top k, then one workgroup per head
// selects from the union.
constexpr int SLICE_MAX = 16;
// A first-level slice keeps at most slice_stride(k) entries: its top k plus
// up to SLICE_SLACK more (whole histogram bins), or every entry at or above
// the head's sampled threshold when there are no more than that.
constexpr int SLICE_SLACK = 64;
constexpr int32_t slice_stride(int32_t k) { return (k > 0 ? k : 1) + SLICE_SLACK; }
// What a first-level slice reports: a NaN seen, the keys it wrote, and how
// many of its entries reach the head's sampled threshold.
struct SliceMeta {
  int32_t nan, n_out, n_ge, pad;
};
// A batch of prompts shares launches, up to PREFILL_NB prompts per launch.
constexpr int PREFILL_NB = 64;
struct PrefillWork {
  int32_t* sel;          // [sel_items][Hkv][k] kept candidate positions
  int32_t sel_items;     // prompts the selection buffer holds (1 .. PREFILL_NB)
  uint64_t* slice_keys;  // [slice_items][Hkv][SLICE_MAX][slice_stride(k)] first-level keys
  SliceMeta* slice_meta; // [slice_items][Hkv][SLICE_MAX]
  uint32_t* slice_tau;   // [slice_items][Hkv] sampled threshold codes
  int32_t slice_items;   // long prompts the first-level buffers hold (1 .. PREFILL_NB)
};
// One prompt to compact into an empty (layer, sequence).
struct PrefillItem {
  const uint16_t* k;      // [Hkv][n_tokens][D]
  const uint16_t* v;
  const float* scores;    // [Hkv][n_tokens]
  int32_t n_tokens;
  int64_t head0;          // cache-wide index of the (layer, sequence)'s first KV head
};
// `all`: views of the whole cache (layer 0 onwards).
hipError_t launch_prefill_batch(const Geometry& geo, const LayerView& all,
                                const PrefillItem* items, int32_t n, const PrefillWork& pw,
                                hipStream_t stream);
// Prefix top-k thresholds of a prompt ([Hkv][n_tokens] keys), n_scored <=
// THR_KMAX.  ws: workspace of ws_keys keys for the segment starts
// ([Hkv][S][n_scored]; the number of segments S is capped to fit it); with
// ws NULL the prompt is one segment per head.
constexpr int THR_KMAX = 4096;
constexpr int THR_SEG_MAX = 32;
hipError_t launch_prefix_thresholds(const Geometry& geo, int32_t n_tokens, const float* scores,
                                    uint64_t* thr, uint64_t* ws, int64_t ws_keys,
                                    hipStream_t stream);
// Future-attention target of one sequence: work [2][Hq][n_tokens] fp32
// (each query's log2-domain log-sum-exp, then each query head's share of the
// target), y [Hkv][n_tokens] fp32 output; scale_log2e: the softmax scale
// times log2(e).
hipError_t launch_future_target(const Geometry& geo, int32_t n_tokens, const uint16_t* q,
                                const uint16_t* k, float scale_log2e, float* work, float* y,
                                hipStream_t stream);
// Static workspace of the no-allocation future-target entry point, in bytes
// ([2][Hq][n_tokens] float32 must fit), and its device address on the
// current device (looked up once per device).
constexpr size_t FUTURE_SCRATCH_BYTES = size_t(32) << 20;
hipError_t future_scratch_address(float** ptr);
// Largest split count the decode kernel accepts, and whether a launch shape
// (head_dim, group size, workgroup size, rows per thread) is compiled.
int decode_max_splits();
bool decode_shape_supported(int head_dim, int group, int threads, int rows_per_thread);

// One decode step of n_layers consecutive layers starting at lv (their heads
// are contiguous in the cache), in one launch; q/k_new/v_new/score_leaving/
// out carry a leading layer dimension.  The workspace must hold
// n_layers * batch * Hkv heads of partials.
hipError_t launch_decode(const Geometry& geo, const LayerView& lv, const DecodeWork& work,
                         int32_t n_layers, const uint16_t* q, const uint16_t* k_new,
                         const uint16_t* v_new, const float* score_leaving, uint16_t* out,
                         float scale_log2e, hipStream_t stream);
// Dynamic backend: cut every head of the layer whose scored region holds
// more than n_scored tokens back to its top n_scored, compacting the rows
// into [0, count).  slack <= PRUNE_SLACK_MAX.
constexpr int PRUNE_SLACK_MAX = 4096;
hipError_t launch_prune(const Geometry& geo, const LayerView& lv, hipStream_t stream);

}  // namespace kvpop
