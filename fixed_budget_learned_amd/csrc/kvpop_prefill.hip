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
//   select  one 1024-thread workgroup per KV head; entry i of the head's
//           candidates sits in thread i % 1024, register i / 1024 (up to 16
//           or 32 per thread).  A radix select with 12, 12 and 8-bit digits
//           over the order-preserving score codes finds the threshold code
//           and how many tokens carrying it survive (the newest); the kept
//           positions get ranks from per-wave ballots, and the head's control
//           block (count, min key and its slot) is written.  Prompts longer
//           than the registers hold select in two levels (slices, then their
//           union) or, failing that, stream the scores on every pass.
//   gather  many 256-thread workgroups per head copy the kept K/V rows into
//           slots [0, count) with 16-byte coalesced loads/stores and write
//           per-slot position and key, and the window ring.
// A batch of (layer, sequence) prompts shares one select and one gather
// launch: the grid's z is the prompt, each reading its own descriptor from
// the kernel arguments (up to PREFILL_NB = 64 per launch, 3.6 KB of arguments).
// Slot layout after prefill: sinks, then the selected candidates in
// ascending position (with at most 64 tied at the threshold code: those
// above it in ascending position, then the kept ties in ascending
// position), then the window in ascending position.
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

// Radix digits over the 32-bit code: 12, 12 and 8 bits.
constexpr int NB0 = 4096, NB1 = 4096, NB2 = 256;
constexpr int SH0 = 20, SH1 = 8;
constexpr int NBINS = NB0;
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
//   SEL_SLICE  first level for long prompts: workgroup (head, slice) writes
//              the keys of a superset of the slice's share of the head's top
//              k, ascending in position, and its SliceMeta.  With a sampled
//              threshold tau for the head (prefill_tau_kernel), a slice whose
//              entries at or above tau number at most slice_stride(k) keeps
//              exactly those.  Otherwise it keeps its own top min(k, slice
//              length), or every entry of the radix bin that holds its k-th
//              largest when that overshoots by at most SLICE_SLACK.  A slice's
//              own top k holds its share of the head's top k (it contributes
//              at most k); the entries at or above tau hold it whenever at
//              least k of the head's entries reach tau, since tau is then at
//              or below the head's k-th largest code.
//   SEL_LIST   second level: one workgroup per head reads the union of its
//              slices' keys (in position order) and selects the top k, writing
//              positions and the control block like SEL_HEAD.  When fewer than
//              k of the head's entries reach tau, the workgroup first has
//              each slice keep its own top k, one after another.
constexpr int SEL_HEAD = 0, SEL_SLICE = 1, SEL_LIST = 2;

// One prompt of a select launch.  head0: the cache-wide index of its
// (layer, sequence)'s first KV head.
struct SelectItem {
  const float* scores;   // [Hkv][P]
  int32_t* sel;          // [Hkv][k] selection slot of the prompt
  uint64_t* slice_keys;  // [Hkv][SLICE_MAX][slice_stride(k)] first-level slot of the prompt
  SliceMeta* meta;       // [Hkv][SLICE_MAX]
  int64_t head0;
  int32_t P, n_slices, slice_len;
};

// Descriptors of the prompts of one launch (grid z = prompt), with what they
// share; kept small enough for the kernel arguments.
// tau: the sampled thresholds of prompt z at tau + z * Hkv, or null (no
// sampling: the slices keep their own top k).
template <int NB>
struct SelectBatch {
  HeadCtl* ctl;          // cache-wide control blocks
  uint32_t* tau;
  int32_t s, k, W;
  SelectItem item[NB];
};

// Wave 0 of a workgroup: the bin of histogram `h` (NB counts, bin order =
// code order) that holds the krem-th largest counted code.  Lane l sums the
// NB/64 bins NB-(l+1)*NB/64 .. NB-l*NB/64-1 (the highest in lane 0, read in a
// lane-rotated order so that the lanes spread over the banks); a prefix sum
// over the lanes finds the lane whose range reaches krem; the wave then reads
// that lane's bins, one per lane from the highest down, and a second prefix
// sum finds the bin.  s_pick receives (bin, counted codes in higher bins,
// codes in the bin).  1 <= krem <= the counted total.
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t* h, uint32_t krem, uint32_t* s_pick) {
  constexpr int PER = NB / WAVE;
  static_assert(PER >= 1 && (PER & (PER - 1)) == 0, "bins per lane: a power of two");
  const int lane = threadIdx.x & (WAVE - 1);
  const int base = NB - (lane + 1) * PER;
  uint32_t sum = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) sum += h[base + ((r + lane) & (PER - 1))];
  const uint32_t incl = wave_inclusive_scan_u32(sum);
  const uint32_t ex = incl - sum;
  const uint64_t hit = __builtin_amdgcn_ballot_w64(ex < krem && krem <= incl);
  const int L = hit ? __builtin_ctzll(hit) : 0;
  const uint32_t exL = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ex), L));
  const int top = NB - L * PER - 1;  // highest bin of lane L
  const uint32_t v = lane < PER ? h[top - lane] : 0u;
  const uint32_t iv = wave_inclusive_scan_u32(v);
  const uint64_t hit2 = __builtin_amdgcn_ballot_w64(lane < PER && exL + iv >= krem);
  const int r = hit2 ? __builtin_ctzll(hit2) : 0;
  if (lane == r) {
    s_pick[0] = static_cast<uint32_t>(top - r);
    s_pick[1] = exL + iv - v;
    s_pick[2] = v;
  }
}

// The same search by the whole workgroup, for NB = 4 x 1024 bins: thread t
// sums its 4 bins NB-4(t+1) .. NB-4t-1 (one 16-byte read) and keeps its
// inclusive prefix within its wave; after a barrier wave 0 finds the wave,
// then the thread, then the bin whose range reaches krem.  All threads call
// it; s_pick is written by wave 0 (read it after a barrier).
template <int NB>
__device__ __forceinline__ void block_find_bin(const uint32_t* h, uint32_t krem, uint32_t* s_pick,
                                               uint32_t* s_wsum, uint32_t* s_lincl) {
  constexpr int PT = NB / SEL_THREADS;
  constexpr int NWAVE = SEL_THREADS / WAVE;
  static_assert(PT == 4, "four bins per thread");
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;
  const uint4 b = *reinterpret_cast<const uint4*>(h + NB - (tid + 1) * PT);
  const uint32_t sum = b.x + b.y + b.z + b.w;
  const uint32_t incl = wave_inclusive_scan_u32(sum);
  s_lincl[tid] = incl;
  if (lane == WAVE - 1) s_wsum[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const uint32_t ws = lane < NWAVE ? s_wsum[lane] : 0u;
    const uint32_t wi = wave_inclusive_scan_u32(ws);
    const uint64_t hw = __builtin_amdgcn_ballot_w64(lane < NWAVE && wi - ws < krem && krem <= wi);
    const int W = hw ? __builtin_ctzll(hw) : 0;
    const uint32_t wbase = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wi - ws), W));
    const uint32_t li = s_lincl[W * WAVE + lane];
    const uint32_t lprev = lane > 0 ? s_lincl[W * WAVE + lane - 1] : 0u;
    const uint64_t hl = __builtin_amdgcn_ballot_w64(wbase + lprev < krem && krem <= wbase + li);
    const int L = hl ? __builtin_ctzll(hl) : 0;
    const uint32_t base = wbase + static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lprev), L));
    const int top = NB - (W * WAVE + L) * PT - 1;  // highest bin of that thread
    const uint32_t v = lane < PT ? h[top - lane] : 0u;
    const uint32_t iv = wave_inclusive_scan_u32(v);
    const uint64_t hb = __builtin_amdgcn_ballot_w64(lane < PT && base + iv >= krem);
    const int r = hb ? __builtin_ctzll(hb) : 0;
    if (lane == r) {
      s_pick[0] = static_cast<uint32_t>(top - r);
      s_pick[1] = base + iv - v;
      s_pick[2] = v;
    }
  }
}

// Lanes below this one whose bit is set in the wave mask m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Register-resident select (VPT = 16 or 32 entries per thread; every mode).
// Entry i of the workgroup lives in thread i % 1024, register i / 1024, so
// the loads go straight from coalesced reads into registers and each wave's
// lanes hold consecutive entries of every register row.  Three radix passes
// (12, 12 and 8-bit digits, histograms in LDS, all cleared once at the
// start; the workgroup locates each pass's bin) find the kk-th largest code
// thr and how many entries carrying it are kept (the newest ones).  The
// ordered compaction then ranks every kept entry in position order from
// wave ballots: per register row, each wave's counts of codes above thr and
// equal to it go into a table whose exclusive prefix (row-major, then wave)
// gives each wave its base, and a lane's rank adds the ballot bits below it.
//
// Occupancy hint: two 1024-thread workgroups per compute unit (8 waves per
// SIMD, at most 64 registers) for 16 entries per thread.
// LDS of one register-select workgroup.
template <int VPT>
struct SelLds {
  static constexpr int NWAVE = SEL_THREADS / WAVE;
  __align__(16) uint32_t hist[NB0 + NB1 + NB2];
  uint32_t tab[VPT * NWAVE];
  uint32_t lincl[SEL_THREADS];
  uint32_t wsum[NWAVE];
  uint32_t pick[3];
  uint32_t nan;
  int32_t tpos[WAVE];  // sparse ties: their positions, unordered
  uint32_t ntie;
  int32_t minslot;
  uint64_t minkey;
  uint64_t wmk[NWAVE];
  int32_t wmp[NWAVE];
  uint32_t total;              // rank table: the workgroup's totals
  int32_t nout[SLICE_MAX];     // SEL_LIST: keys of each slice
  int32_t cum[SLICE_MAX + 1];  // SEL_LIST: keys of the slices before each
};

// One register-select workgroup: KV head g of prompt `it` (SEL_SLICE: its
// slice y).  ctl: the cache-wide control blocks; s, k, W: sinks, scored
// slots, window; tau: the prompt's sampled thresholds or null.  Returns the
// number of entries written (SEL_SLICE: keys; else the kept count).
template <int VPT, int MODE>
__device__ __forceinline__ int32_t select_wg(const SelectItem& it, HeadCtl* __restrict__ ctl,
                                             const uint32_t* tau, int32_t s_sink, int32_t k_sc,
                                             int32_t W_rec, int g, int y, SelLds<VPT>& L) {
  static_assert(VPT == 16 || VPT == 32, "register select: 16 or 32 entries per thread");
  static_assert(MODE != SEL_LIST || VPT == 16, "list mode: at most 16 keys per thread");
  constexpr int NWAVE = SEL_THREADS / WAVE;
  constexpr int HTOT = NB0 + NB1 + NB2;
  constexpr int TAB = VPT * NWAVE;
  uint32_t* hist = L.hist;
  uint32_t* s_tab = L.tab;
  uint32_t* s_lincl = L.lincl;
  uint32_t* s_wsum = L.wsum;
  uint32_t* s_pick = L.pick;
  uint32_t& s_nan = L.nan;
  int32_t* s_tpos = L.tpos;
  uint32_t& s_ntie = L.ntie;
  int32_t& s_minslot = L.minslot;
  uint64_t& s_minkey = L.minkey;
  uint64_t* s_wmk = L.wmk;
  int32_t* s_wmp = L.wmp;

  const PrefillShape sh = prefill_shape(it.P, s_sink, k_sc, W_rec);
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1);
  const int wid = tid / WAVE;
  const int32_t kst = k_sc > 0 ? k_sc : 1;  // stride of the per-head buffers
  int32_t* out = it.sel + static_cast<int64_t>(g) * kst;
  // this workgroup's entries: candidates [cb, cb + C) of the head's range, or
  // (SEL_LIST) the head's first-level key list
  int32_t cb = 0, C = sh.c1 - sh.c0, kk = sh.kk;
  if constexpr (MODE == SEL_SLICE) {
    cb = y * it.slice_len;
    C = min(it.slice_len, sh.c1 - sh.c0 - cb);
    kk = min(k_sc, C);
  }
  const int32_t ks = slice_stride(k_sc);  // entries per slice in the key lists
  const int64_t list0 = (static_cast<int64_t>(g) * SLICE_MAX) * ks;
  uint64_t* outk = it.slice_keys + list0 + static_cast<int64_t>(y) * ks;
  int32_t n_out = kk;  // entries this workgroup emits
  const int32_t pos0 = sh.c0 + cb;  // position of entry 0 (not SEL_LIST)

  // SEL_LIST: the union is slice y's n_out[y] keys at y * ks, for each y.
  // With sampling, the entries of the union are numbered densely (L.cum:
  // keys of the slices before each); slices that kept their own top k
  // padded their lists to ks with key 0, which is read as it stands.
  bool packed = false, any_nan = false;
  if constexpr (MODE == SEL_LIST) {
    const SliceMeta* mh = it.meta + static_cast<int64_t>(g) * SLICE_MAX;
    for (int j = 0; j < it.n_slices; ++j) any_nan |= mh[j].nan != 0;
    // tau is passed only when at least kk of the head's entries reach it
    // (the kernel checks before calling)
    packed = tau != nullptr;
    if (tid < SLICE_MAX) L.nout[tid] = tid < it.n_slices ? mh[tid].n_out : 0;
    if (packed) {
      __syncthreads();
      if (tid == 0) {
        int32_t c = 0;
        for (int j = 0; j < SLICE_MAX; ++j) {
          L.cum[j] = c;
          c += L.nout[j];
        }
        L.cum[SLICE_MAX] = c;
      }
      __syncthreads();
      C = L.cum[SLICE_MAX];
    } else {
      C = it.n_slices * ks;
    }
  }

  // ---- entries into registers (loads first, then the LDS set-up) -----------
  // valid entries of this thread: registers 0 .. nvalid-1
  const int nvalid = C > tid ? min(VPT, (C - tid + SEL_THREADS - 1) / SEL_THREADS) : 0;
  uint32_t code[VPT];
  int32_t lpos[MODE == SEL_LIST ? VPT : 1];
  bool nan = false;
  if (kk > 0) {
    // range-checked buffer loads: entries past C read as 0
    if constexpr (MODE == SEL_LIST) {
      const int32_t nbytes = it.n_slices * ks * 8;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          it.slice_keys + list0, 0, nbytes, BUF_RSRC_WORD3);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      u32x2 key[VPT];
      int q = 0;  // packed: the slice of this thread's current entry
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int32_t e = j * SEL_THREADS + tid;  // entry of the union
        int32_t a = e;                             // its place in the lists
        if (packed && e < C) {
          while (e >= L.cum[q + 1]) ++q;
          a = q * ks + (e - L.cum[q]);
        }
        key[j] = __builtin_amdgcn_raw_buffer_load_b64(r, e < C ? a * 8 : nbytes, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        code[j] = key[j].y;
        lpos[j] = static_cast<int32_t>(key[j].x);
      }
    } else {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(it.scores + static_cast<int64_t>(g) * sh.P + pos0), 0, C * 4,
          BUF_RSRC_WORD3);
      float x[VPT];
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        x[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (j * SEL_THREADS + tid) * 4, 0, 0));
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        code[j] = j < nvalid ? score_code(x[j]) : 0u;
        nan |= score_is_nan(x[j]);  // entries past C read as +0
      }
    }
  }
  // Entries past C carry code 0.  Register rows at or past nrows hold only
  // those and are skipped (a uniform test); in the last row a lane past C
  // counts nothing.
  const int nrows = (C + SEL_THREADS - 1) / SEL_THREADS;
  static_assert(HTOT % 4 == 0, "histograms cleared in 16-byte pieces");
  auto clear_hist = [&]() {
    for (int i = tid; i < HTOT / 4; i += SEL_THREADS)
      reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  };
  // a sampled slice clears them only if it needs the radix passes
  const bool sampled = MODE == SEL_SLICE && VPT == 16 && tau != nullptr;
  if (!sampled) clear_hist();
  if (tid == 0) {
    s_nan = 0;
    s_minslot = -1;
    s_minkey = KEY_NONE;
  }
  __syncthreads();
  if (nan) s_nan = 1;
  if constexpr (MODE == SEL_LIST) {
    if (any_nan) s_nan = 1;
  }
  // SEL_SLICE with a sampled threshold: the slice's entries at or above it
  // (n_ge of them); when no more than a key list holds, the slice keeps
  // exactly those (by_tau).  Lanes past C carry code 0 and reach the
  // threshold only if it is 0.
  uint32_t t_cut = 0, n_ge = 0;
  bool by_tau = false;
  if constexpr (MODE == SEL_SLICE && VPT == 16)
    if (tau != nullptr) t_cut = tau[g];
  auto reaches = [&](int j) { return (t_cut != 0u || j < nvalid) && code[j] >= t_cut; };

  auto pos_of = [&](int j) -> int32_t {
    if constexpr (MODE == SEL_LIST)
      return lpos[j];
    else
      return pos0 + j * SEL_THREADS + tid;
  };
  // where the kept entry of rank idx goes
  auto emit = [&](uint32_t idx, int32_t pos, uint32_t o) {
    if (idx >= static_cast<uint32_t>(n_out)) return;  // never taken: ranks are < n_out
    if constexpr (MODE == SEL_SLICE)
      outk[idx] = make_key(o, pos);
    else
      out[idx] = pos;
  };

  if (kk > 0 && kk == C) {
    // every entry is kept, in order; the least important one is the smallest
    // (code, position)
    if (MODE == SEL_SLICE && VPT == 16 && tau != nullptr) {
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        if (j < nrows && reaches(j)) ++mine;
      const uint32_t incl = wave_inclusive_scan_u32(mine);
      if (lane == WAVE - 1) s_wsum[wid] = incl;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) n_ge += s_wsum[w];
      __syncthreads();
    }
    uint64_t mk = KEY_NONE;
    int32_t mpos = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      if (j < nvalid) {
        const int32_t pos = pos_of(j);
        emit(static_cast<uint32_t>(j * SEL_THREADS + tid), pos, code[j]);
        const uint64_t key = make_key(code[j], pos);
        if (key < mk) {
          mk = key;
          mpos = pos;
        }
      }
    }
    if constexpr (MODE != SEL_SLICE) {
      wave_min_key(mk, mpos);
      if (lane == 0) {
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
        s_minslot = sh.s_eff + (mpos - sh.c0);  // all kept: rank = position - c0
      }
    }
  } else if (kk > 0) {
    // ---- radix select of the kk-th largest code ---------------------------
    uint32_t prefix = 0, mask = 0, krem = static_cast<uint32_t>(kk), neq = 0;
    auto pass = [&](uint32_t* h, int shift, uint32_t nbm1, auto find) {
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        if (j < nrows && j * SEL_THREADS + tid < C && (code[j] & mask) == prefix)
          atomicAdd(&h[(code[j] >> shift) & nbm1], 1u);
      __syncthreads();
      find(h, krem);
      __syncthreads();
      const uint32_t bin = s_pick[0];
      krem -= s_pick[1];
      neq = s_pick[2];
      prefix |= bin << shift;
      mask |= nbm1 << shift;
    };
    // ---- ordered compaction.  Kept: entries `above` the cut, then the
    // newest of those `tied` at it (the oldest `drop` tied entries lose).
    // Ranks in position order: per register row, each wave's counts (16-bit
    // halves: above, tied) go into a table whose exclusive prefix, row-major
    // then wave, is the wave's base; a lane adds the ballot bits below it.
    // rank_table builds the table and returns the workgroup's totals (same
    // packing); emit then places every kept entry.
    auto rank_table = [&](auto above, auto tied) -> uint32_t {
      uint32_t mycnt = 0;  // lane j: row j's counts of this wave
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j >= nrows) break;
        const uint64_t gm = __builtin_amdgcn_ballot_w64(above(j));
        const uint64_t em = __builtin_amdgcn_ballot_w64(tied(j));
        const uint32_t cnt = (static_cast<uint32_t>(__builtin_popcountll(em)) << 16) |
                             static_cast<uint32_t>(__builtin_popcountll(gm));
        mycnt = lane == j ? cnt : mycnt;
      }
      if (lane < VPT) s_tab[lane * NWAVE + wid] = mycnt;
      __syncthreads();
      if (wid == 0) {
        // lane l owns table entries l*E .. l*E+E-1
        constexpr int E = TAB / WAVE;
        uint32_t t[E], sum = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          t[e] = s_tab[lane * E + e];
          sum += t[e];
        }
        const uint32_t incl = wave_inclusive_scan_u32(sum);
        uint32_t ex = incl - sum;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s_tab[lane * E + e] = ex;
          ex += t[e];
        }
        if (lane == WAVE - 1) L.total = incl;
      }
      __syncthreads();
      return L.total;
    };
    auto emit_ranked = [&](auto above, auto tied, uint32_t drop, uint32_t thr) {
      uint32_t base[VPT];  // uniform over the wave: kept in scalar registers
#pragma unroll
      for (int j = 0; j < VPT; ++j)
        base[j] = static_cast<uint32_t>(
            __builtin_amdgcn_readfirstlane(static_cast<int>(s_tab[j * NWAVE + wid])));
      int32_t min_rank = -1, min_pos = 0;  // the least important kept entry, if here
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        if (j >= nrows) break;
        const bool is_gt = above(j), is_eq = tied(j);
        const uint64_t gm = __builtin_amdgcn_ballot_w64(is_gt);
        const uint64_t em = __builtin_amdgcn_ballot_w64(is_eq);
        const uint32_t gt_before = (base[j] & 0xFFFFu) + lanes_below(gm);
        const uint32_t eq_before = (base[j] >> 16) + lanes_below(em);
        if (is_gt || (is_eq && eq_before >= drop)) {
          const uint32_t idx = gt_before + (eq_before > drop ? eq_before - drop : 0u);
          const int32_t pos = pos_of(j);
          emit(idx, pos, code[j]);
          if (is_eq && eq_before == drop) {
            min_rank = static_cast<int32_t>(idx);
            min_pos = pos;
          }
        }
      }
      if (min_rank >= 0) {
        s_minslot = sh.s_eff + min_rank;
        s_minkey = make_key(thr, min_pos);
      }
    };
    auto compact = [&](auto above, auto tied, uint32_t drop, uint32_t thr) {
      rank_table(above, tied);
      emit_ranked(above, tied, drop, thr);
    };
    if constexpr (MODE == SEL_SLICE && VPT == 16) {
      if (tau != nullptr) {
        // at most 16,384 entries: the count fits the low half
        n_ge = rank_table(reaches, [&](int) { return false; }) & 0xFFFFu;
        by_tau = n_ge <= static_cast<uint32_t>(ks);
        if (!by_tau) {
          clear_hist();
          __syncthreads();
        }
      }
    }
    if (by_tau) {
      // every entry at or above the sampled threshold, in position order
      n_out = static_cast<int32_t>(n_ge);
      emit_ranked(reaches, [&](int) { return false; }, 0u, t_cut);
    } else {
      pass(hist, SH0, NB0 - 1, [&](const uint32_t* h, uint32_t kr) {
        block_find_bin<NB0>(h, kr, s_pick, s_wsum, s_lincl);
      });
      pass(hist + NB0, SH1, NB1 - 1, [&](const uint32_t* h, uint32_t kr) {
        block_find_bin<NB1>(h, kr, s_pick, s_wsum, s_lincl);
      });
      // A slice may keep whole bins: every entry whose code reaches the pass-2
      // bin, a superset of its top kk by neq - krem <= SLICE_SLACK entries (the
      // second level selects exactly, in position order, from the union).
      bool superset = false;
      if constexpr (MODE == SEL_SLICE) superset = neq - krem <= static_cast<uint32_t>(SLICE_SLACK);
      if (superset) {
        const uint32_t cut = prefix;  // low 8 bits 0: codes in or above the bin
        n_out = kk - static_cast<int32_t>(krem) + static_cast<int32_t>(neq);
        compact([&](int j) { return (cut != 0u || j < nvalid) && code[j] >= cut; },
                [&](int) { return false; }, 0u, cut);
      } else {
        pass(hist + NB0 + NB1, 0, NB2 - 1,
             [&](const uint32_t* h, uint32_t kr) {
               if (wid == 0) find_bin<NB2>(h, kr, s_pick);
             });
        const uint32_t thr = prefix;
        const uint32_t drop = neq - krem;
        if (MODE != SEL_SLICE && neq <= static_cast<uint32_t>(WAVE) && thr != 0u) {
          // Few ties (and none with the padding): the entries above thr take
          // ranks 0 .. kk-krem-1 in position order, the kept ties the ranks
          // after them, ordered by position by wave 0 from a list of at most
          // 64.  A final selection's ranks (cache slots) only have to be
          // distinct and reproducible; a first-level slice keeps position
          // order, which the second level's tie order relies on.
          if (tid == 0) s_ntie = 0;
          compact([&](int j) { return code[j] > thr; }, [&](int) { return false; }, 0u, thr);
  #pragma unroll
          for (int j = 0; j < VPT; ++j)
            if (j < nrows && code[j] == thr) s_tpos[atomicAdd(&s_ntie, 1u)] = pos_of(j);
          __syncthreads();
          if (wid == 0) {
            const uint32_t n = s_ntie;  // == neq
            const int32_t mine = lane < static_cast<int>(n) ? s_tpos[lane] : 0x7FFFFFFF;
            uint32_t rank = 0;
            for (uint32_t t = 0; t < n; ++t) rank += s_tpos[t] < mine ? 1u : 0u;
            if (lane < static_cast<int>(n) && rank >= drop) {
              const uint32_t idx = static_cast<uint32_t>(kk) - krem + (rank - drop);
              emit(idx, mine, thr);
              if (rank == drop) {  // the least important kept entry
                s_minslot = sh.s_eff + static_cast<int32_t>(idx);
                s_minkey = make_key(thr, mine);
              }
            }
          }
        } else {
          // only a threshold of 0 can tie with the padding
          compact([&](int j) { return code[j] > thr; },
                  [&](int j) { return (thr != 0u || j < nvalid) && code[j] == thr; }, drop, thr);
        }
      }
    }
  }
  if constexpr (MODE == SEL_SLICE) {
    // Without sampling, pad the list to its stride with the smallest key
    // (the second level reads the lists whole); record what the slice did.
    if (tau == nullptr)
      for (int32_t j = n_out + tid; j < ks; j += SEL_THREADS) outk[j] = 0ull;
    __syncthreads();
    if (tid == 0) {
      SliceMeta m;
      m.nan = s_nan ? 1 : 0;
      m.n_out = n_out;
      m.n_ge = static_cast<int32_t>(n_ge);
      m.pad = 0;
      it.meta[static_cast<int64_t>(g) * SLICE_MAX + y] = m;
    }
    return n_out;
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
    (ctl + it.head0)[g] = c;
  }
  return n_out;
}

template <int VPT, int MODE, int NB>
__global__ __launch_bounds__(SEL_THREADS)
__attribute__((amdgpu_waves_per_eu(VPT == 16 ? 8 : 1)))
void prefill_select_kernel(SelectBatch<NB> batch) {
  __shared__ SelLds<VPT> L;
  const SelectItem& it = batch.item[blockIdx.z];
  // a batch launch covers its longest prompt's slices: shorter ones have none here
  if (MODE == SEL_SLICE && static_cast<int32_t>(blockIdx.y) >= it.n_slices) return;
  const int g = static_cast<int>(blockIdx.x);
  const uint32_t* tau = (MODE != SEL_HEAD && batch.tau != nullptr)
                            ? batch.tau + static_cast<int64_t>(blockIdx.z) * gridDim.x
                            : nullptr;
  if constexpr (MODE == SEL_LIST) {
    if (tau != nullptr) {
      // Fewer than kk of the head's entries reaching tau: the slices' keys
      // may miss some of the top kk, so each slice keeps its own top kk
      // (padded list) before the union is read.
      const SliceMeta* mh = it.meta + static_cast<int64_t>(g) * SLICE_MAX;
      int32_t n_ge = 0;
      for (int j = 0; j < it.n_slices; ++j) n_ge += mh[j].n_ge;
      if (n_ge < prefill_shape(it.P, batch.s, batch.k, batch.W).kk) {
        for (int j = 0; j < it.n_slices; ++j) {
          select_wg<VPT, SEL_SLICE>(it, batch.ctl, nullptr, batch.s, batch.k, batch.W, g, j, L);
          __syncthreads();
        }
        tau = nullptr;
      }
    }
  }
  select_wg<VPT, MODE>(it, batch.ctl, tau, batch.s, batch.k, batch.W, g,
                       static_cast<int>(blockIdx.y), L);
}

// Sampled threshold of each KV head of two-level prompts, for the first
// level (one workgroup per head).  The workgroup reads TAU_BLOCKS runs of
// TAU_RUN consecutive candidates spread evenly over the head's range
// (TAU_N = 4,096 codes, 4 per thread) and takes tau as the lower edge of the
// 24-bit radix bin that holds their m-th largest code, m = n + 6 sqrt(n) + 16
// with n = TAU_N * kk / C: the sample holds about n of the head's top kk, so
// m exceeds that count by six standard deviations, and about m * C / TAU_N
// entries of the head reach tau.  Nothing relies on the estimate: the
// slices count the entries that reach tau and the second level checks that
// at least kk do.  Two-level prompts have C > 32,768 candidates, so the runs
// stay inside the range.
constexpr int TAU_BLOCKS = 64, TAU_RUN = 64, TAU_N = TAU_BLOCKS * TAU_RUN;
static_assert(TAU_N == 4 * SEL_THREADS, "four sampled codes per thread");

template <int NB>
__global__ __launch_bounds__(SEL_THREADS) void prefill_tau_kernel(SelectBatch<NB> batch) {
  constexpr int NWAVE = SEL_THREADS / WAVE;
  __shared__ __align__(16) uint32_t hist[NB0 + NB1];
  __shared__ uint32_t s_lincl[SEL_THREADS];
  __shared__ uint32_t s_wsum[NWAVE];
  __shared__ uint32_t s_pick[3];
  const SelectItem& it = batch.item[blockIdx.z];
  const PrefillShape sh = prefill_shape(it.P, batch.s, batch.k, batch.W);
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t C = sh.c1 - sh.c0;
  constexpr int TPR = TAU_RUN / 4;  // threads per run
  const int64_t i0 = sh.c0 + static_cast<int64_t>(tid / TPR) * C / TAU_BLOCKS + (tid % TPR) * 4;
  const float* src = it.scores + static_cast<int64_t>(g) * sh.P + i0;
  float x[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = src[e];
  for (int i = tid; i < NB0 + NB1; i += SEL_THREADS) hist[i] = 0u;
  __syncthreads();
  uint32_t code[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    code[e] = score_code(x[e]);
    atomicAdd(&hist[code[e] >> SH0], 1u);
  }
  const float n = static_cast<float>(TAU_N) * static_cast<float>(sh.kk) / static_cast<float>(C);
  const uint32_t m = min(static_cast<uint32_t>(ceilf(n + 6.f * sqrtf(n) + 16.f)),
                         static_cast<uint32_t>(TAU_N));
  __syncthreads();
  block_find_bin<NB0>(hist, m, s_pick, s_wsum, s_lincl);
  __syncthreads();
  const uint32_t b0 = s_pick[0];
  const uint32_t krem = m - s_pick[1];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if ((code[e] >> SH0) == b0) atomicAdd(&hist[NB0 + ((code[e] >> SH1) & (NB1 - 1))], 1u);
  __syncthreads();
  block_find_bin<NB1>(hist + NB0, krem, s_pick, s_wsum, s_lincl);
  __syncthreads();
  if (tid == 0)
    batch.tau[static_cast<int64_t>(blockIdx.z) * gridDim.x + g] = (b0 << SH0) | (s_pick[0] << SH1);
}

// Streaming select (SEL_HEAD, any prompt length): one workgroup per KV head
// reads the scores again on every radix pass and compacts in LDS-staged
// tiles of 32 candidates per thread, so that each thread walks a contiguous
// block in position order.  The fallback for prompts whose candidates fit
// neither the registers nor two levels.
template <int NB>
__global__ __launch_bounds__(SEL_THREADS) void prefill_select_stream_kernel(SelectBatch<NB> batch) {
  constexpr int NWAVE = SEL_THREADS / WAVE;
  constexpr int TL = 1 << TILE_LG;
  __shared__ uint32_t hist[NBINS];
  __shared__ __align__(16) uint32_t stage[SEL_THREADS * (TL + 1)];
  __shared__ uint32_t scan_buf[NWAVE + 1];
  __shared__ uint32_t s_bin, s_above, s_nan, s_neq;
  __shared__ int32_t s_minslot;
  __shared__ uint64_t s_minkey;
  __shared__ uint64_t s_wmk[NWAVE];
  __shared__ int32_t s_wmp[NWAVE];

  const SelectItem& it = batch.item[blockIdx.z];
  const PrefillShape sh = prefill_shape(it.P, batch.s, batch.k, batch.W);
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int wid = tid / WAVE;
  const int32_t kst = batch.k > 0 ? batch.k : 1;
  int32_t* out = it.sel + static_cast<int64_t>(g) * kst;
  const int32_t C = sh.c1 - sh.c0, kk = sh.kk;
  const float* sc = it.scores + static_cast<int64_t>(g) * sh.P + sh.c0;  // candidate 0

  if (tid == 0) {
    s_nan = 0;
    s_minslot = -1;
    s_minkey = KEY_NONE;
  }
  __syncthreads();
  bool nan = false;
  if (kk > 0 && kk == C) {
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
  } else if (kk > 0) {
    uint32_t prefix = 0, mask = 0, krem = static_cast<uint32_t>(kk);
    const int shifts[3] = {SH0, SH1, 0}, nbins[3] = {NB0, NB1, NB2};
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
    (batch.ctl + it.head0)[g] = c;
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

// Where gathered rows go: the cache-wide rows and slot metadata, and the
// cache geometry.
struct GatherDst {
  uint16_t* kc;
  uint16_t* vc;
  uint64_t* keys;
  int32_t* pos;
  int32_t* ring;
  int32_t s, k, W, budget;
};

template <int NB>
struct GatherBatch {
  GatherDst dst;
  int32_t rows_per_block;
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

// Rows [r0, r1) of KV head g of prompt `it` into its slots, by NT threads
// (D/8 lanes of 16 bytes per row; RPT rows per thread have their loads in
// flight before their stores): K and V, and per slot its position and key;
// window rows also enter the ring.
template <int D, int NT, int RPT>
__device__ __forceinline__ void gather_rows(const GatherItem& it, const GatherDst& d, int g,
                                            int32_t r0, int32_t r1) {
  constexpr int LPR = D / 8;        // lanes per row (16 B each)
  constexpr int RPP = NT / LPR;     // rows per pass
  const PrefillShape sh = prefill_shape(it.P, d.s, d.k, d.W);
  const int32_t kcap = d.k > 0 ? d.k : 1;
  const int32_t budget = d.budget, W = d.W;
  const int tid = threadIdx.x;
  const int rg = tid / LPR;
  const int c = tid % LPR;
  const uint16_t* __restrict__ k = it.k;
  const uint16_t* __restrict__ v = it.v;
  const float* __restrict__ scores = it.scores;
  const int32_t* __restrict__ sel = it.sel;
  const int64_t row0 = it.head0 * budget;
  uint16_t* __restrict__ kc = d.kc + row0 * D;
  uint16_t* __restrict__ vc = d.vc + row0 * D;
  uint64_t* __restrict__ keys = d.keys + row0;
  int32_t* __restrict__ pos = d.pos + row0;
  int32_t* __restrict__ ring = d.ring + it.head0 * W;

  const uint4* ksrc = reinterpret_cast<const uint4*>(k + static_cast<int64_t>(g) * sh.P * D);
  const uint4* vsrc = reinterpret_cast<const uint4*>(v + static_cast<int64_t>(g) * sh.P * D);
  uint4* kdst = reinterpret_cast<uint4*>(kc + static_cast<int64_t>(g) * budget * D);
  uint4* vdst = reinterpret_cast<uint4*>(vc + static_cast<int64_t>(g) * budget * D);
  const int32_t* selg = sel + static_cast<int64_t>(g) * kcap;
  const float* scg = scores + static_cast<int64_t>(g) * sh.P;

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

// One gather workgroup: 256 threads, rows_per_block rows of one head.
template <int D, int NB>
__global__ __launch_bounds__(GATHER_THREADS) void prefill_gather_kernel(GatherBatch<NB> batch) {
  const GatherItem& it = batch.item[blockIdx.z];
  const GatherDst& d = batch.dst;
  const int32_t count = prefill_shape(it.P, d.s, d.k, d.W).count;
  const int32_t r0 = static_cast<int32_t>(blockIdx.x) * batch.rows_per_block;
  const int32_t r1 = min(r0 + batch.rows_per_block, count);  // empty past this prompt's rows
  gather_rows<D, GATHER_THREADS, 1>(it, d, static_cast<int>(blockIdx.y), r0, r1);
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
  si.meta = pw.slice_meta;
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
  sb.tau = nullptr;
  sb.s = gb.dst.s = geo.n_sink;
  sb.k = gb.dst.k = geo.n_scored;
  sb.W = gb.dst.W = geo.n_recent;
  gb.dst.kc = all.kc;
  gb.dst.vc = all.vc;
  gb.dst.keys = all.keys;
  gb.dst.pos = all.pos;
  gb.dst.ring = all.ring;
  gb.dst.budget = geo.budget;
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
  const int64_t k64 = slice_stride(geo.n_scored);  // the second level holds n_slices of these
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
  const int64_t slice_one =
      static_cast<int64_t>(geo.n_kv_heads) * SLICE_MAX * slice_stride(geo.n_scored);
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
    si.meta = pw.slice_meta + i * static_cast<int64_t>(geo.n_kv_heads) * SLICE_MAX;
    max_slices = lp.n_slices > max_slices ? lp.n_slices : max_slices;
    gb.item[i] = gather_item(*its[i], sel);
  }
  const dim3 heads(static_cast<uint32_t>(geo.n_kv_heads), 1u, static_cast<uint32_t>(m));
  hipError_t e;
  if (VPT == 16) {
    // 16k slices filter by a sampled threshold.  The second level's
    // fallback (each slice's own top k) runs on its 16 entries per thread,
    // so 32k slices do not sample.
    sb.tau = pw.slice_tau;
    hipLaunchKernelGGL((prefill_tau_kernel<NB>), heads, dim3(SEL_THREADS), 0, stream, sb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 slices(static_cast<uint32_t>(geo.n_kv_heads), static_cast<uint32_t>(max_slices),
                    static_cast<uint32_t>(m));
  hipLaunchKernelGGL((prefill_select_kernel<VPT, SEL_SLICE, NB>), slices, dim3(SEL_THREADS), 0,
                     stream, sb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
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
  hipLaunchKernelGGL((prefill_select_stream_kernel<1>), heads, dim3(SEL_THREADS), 0, stream, sb);
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
