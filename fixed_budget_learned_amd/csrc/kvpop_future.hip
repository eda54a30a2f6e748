// Future-attention target for gfx950: for every KV head g and key j,
//   y[g][j] = sum over the query heads h of g's group and the queries
//             i >= j + W of the causal softmax weight of query i on key j,
// the attention mass a token receives after it has left the protected
// recent window (English and French aiweekly articles: the scorer's
// training target, computed with a transposed-attention pass so that no
// dense attention map is materialised; summing over the group's query heads,
// unnormalised, is the reading taken).
//
// Two passes, FlashAttention-backward style, on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), and a group sum:
//   pass 1  per (query head, 256-query tile): S^T = K . Q^T over the causal
//           key tiles, online row log-sum-exp in the log2 domain -> lse[h][i].
//   pass 2  per (query head, 256-key tile): for each 64-query tile with
//           queries >= key + W, P = 2^(c S - lse), summed over the queries
//           -> part[h][j].
//   sum     y[g][j] = sum of part[h][j] over the group's heads, in head order.
// Splitting pass 2 by query head rather than by KV head keeps its longest
// workgroup to one head's queries (the first key tile sees every query), and
// the fixed-order group sum keeps the result deterministic.
// Both passes launch the largest tiles (most work) first: the grid's x is the
// head, its y the tile.
// Each wave keeps 64 rows of the stationary operand in registers (queries in
// pass 1, keys in pass 2) as two 32-row MFMA operands, and every 32-row
// operand it reads from the LDS tile feeds two MFMAs.  With 32 rows per wave
// the LDS reads bound both passes (one read per MFMA, 1 KB per 32 cycles of
// matrix core per SIMD); 64 rows halve them for 148 and 160 registers, 3
// waves per SIMD instead of 4 (measured on the 16,384-token layer shape:
// 2.22-2.27 -> 2.07-2.12 ms per call).
// Tiles reach LDS in two ways.  Pass 1 stages its key tiles through
// registers into padded LDS rows.  Pass 2 loads its query tiles (and their
// log-sum-exps) straight from global memory into LDS, XOR-swizzled, which
// needs no staging registers.  Pass 1 was slower with the direct loads.
// S^T puts keys on the MFMA rows and queries on its columns: a lane holds 16
// keys of one query, so the row reductions of pass 1 are in-lane plus one
// swap of wave halves, and pass 2 sums columns in-lane until one final
// reduction.  Operand layouts (checked on the hardware): A row l%32, k
// 8*(l/32)+0..7; B k 8*(l/32)+0..7, column l%32; C column l%32, row
// 8*(r/4) + 4*(l/32) + r%4.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvpop_device.h"
#include "kvpop_internal.h"

namespace kvpop {

// Workspace of kvpop_future_attention_target_noalloc: a static device array
// (every device the library runs on holds its own copy until the process
// ends), for callers that cannot allocate.  Host code never passes its name
// to a kernel: it stands for a host-side shadow, not a device address; the
// device address comes from future_scratch_address().
static __device__ __align__(256) float scratch[FUTURE_SCRATCH_BYTES / sizeof(float)];

hipError_t future_scratch_address(float** ptr) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static float* addr[MAX_DEVICES] = {};
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(a);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int FT_THREADS = 256;   // 4 waves
constexpr int FT_WROWS = 64;      // queries (pass 1) or keys (pass 2) per wave, in registers
constexpr int FT_ROWS = FT_WROWS * FT_THREADS / WAVE;  // ... per workgroup
constexpr int FT_TILE = 64;       // keys (pass 1) or queries (pass 2) per LDS tile

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// One 64-row tile of a [rows][D] bf16 matrix into LDS (row stride D + 8
// elements: neighbouring rows start 4 banks apart).  Rows past `nrows` read
// the last valid row (their results are masked).  Coalesced 16-byte pieces.
template <int D>
struct TileLoader {
  static constexpr int PIECES = D / 8;                       // 16-byte pieces per row
  static constexpr int PER_THREAD = FT_TILE * PIECES / FT_THREADS;
  u32x4_t buf[PER_THREAD];
  __device__ __forceinline__ void load(const uint16_t* src, int32_t row0, int32_t nrows) {
    if (row0 + FT_TILE <= nrows) {  // uniform: one base, per-lane offsets that stay fixed
      const uint16_t* base = src + static_cast<int64_t>(row0) * D;
#pragma unroll
      for (int u = 0; u < PER_THREAD; ++u) {
        const int p = threadIdx.x + u * FT_THREADS;
        buf[u] = *reinterpret_cast<const u32x4_t*>(base + (p / PIECES) * D + (p % PIECES) * 8);
      }
    } else {
#pragma unroll
      for (int u = 0; u < PER_THREAD; ++u) {
        const int p = threadIdx.x + u * FT_THREADS;
        const int32_t r = min(row0 + p / PIECES, nrows - 1);
        buf[u] = reinterpret_cast<const u32x4_t*>(src + static_cast<int64_t>(r) * D)[p % PIECES];
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int u = 0; u < PER_THREAD; ++u) {
      const int p = threadIdx.x + u * FT_THREADS;
      *reinterpret_cast<u32x4_t*>(lds + (p / PIECES) * (D + 8) + (p % PIECES) * 8) = buf[u];
    }
  }
};

// One 64-row tile of a [rows][D] bf16 matrix into LDS by direct global->LDS
// loads (no register staging).  Rows are stored unpadded; the 16-byte chunk
// c of row r sits at chunk position c ^ (r % CPR), so that the 8 lanes served
// together by a 16-byte LDS read (8 rows, one chunk) hit distinct banks.  A
// wave instruction fills 1 KB: lane i writes position i of it, so it loads
// the global chunk that belongs there.  Rows past `nrows` read the last row.
// `wid` is the wave index, uniform.
template <int D>
struct TileDma {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 1024 / (D * 2);        // rows per wave instruction
  static constexpr int INST = FT_TILE / RPI / (FT_THREADS / WAVE);  // per wave
  __device__ __forceinline__ static void issue(const uint16_t* src, int32_t row0, int32_t nrows,
                                               uint16_t* lds, int wid) {
    const int lane = threadIdx.x & (WAVE - 1);
    if (row0 + FT_TILE <= nrows) {  // uniform: one base, per-lane offsets that stay fixed
      const uint16_t* base = src + static_cast<int64_t>(row0) * D;
#pragma unroll
      for (int u = 0; u < INST; ++u) {
        const int blk = u * (FT_THREADS / WAVE) + wid;  // 1 KB block of the tile
        const int r = blk * RPI + lane / CPR;           // tile row of this lane
        const int c = (lane % CPR) ^ (r % CPR);         // global chunk it must fetch
        const uint32_t off = static_cast<uint32_t>((r * D + c * 8) * 2);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(reinterpret_cast<const char*>(base) + off),
            (__attribute__((address_space(3))) void*)(lds + blk * 512), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < INST; ++u) {
        const int blk = u * (FT_THREADS / WAVE) + wid;
        const int r = blk * RPI + lane / CPR;
        const int c = (lane % CPR) ^ (r % CPR);
        const int32_t gr = min(row0 + r, nrows - 1);
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(src + static_cast<int64_t>(gr) * D + c * 8),
            (__attribute__((address_space(3))) void*)(lds + blk * 512), 16, 0, 0);
      }
    }
  }
  // byte offset of (row, chunk) in the tile
  __device__ __forceinline__ static int at(int r, int c) { return r * (D * 2) + ((c ^ (r % CPR)) * 16); }
};

// The 32-row operand of one wave held in registers: lane l keeps row
// row0 + l%32, elements 16*ks + 8*(l/32) .. +7 for every k-step ks.
template <int D>
__device__ __forceinline__ void load_operand_rows(const uint16_t* src, int32_t row0, int32_t nrows,
                                                  u32x4_t (&op)[D / 16]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int32_t r = min(row0 + (lane & 31), nrows - 1);
  const uint16_t* p = src + static_cast<int64_t>(r) * D + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) op[ks] = *reinterpret_cast<const u32x4_t*>(p + 16 * ks);
}

// An empty register-to-register statement that reads and rewrites the
// operand: the compiler completes its loads here and can neither sink them
// into the main loop nor count them among that loop's outstanding loads
// (whose waits would then also hold back the next tile's prefetch).
template <int N>
__device__ __forceinline__ void settle(u32x4_t (&op)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(op[i]));
}

// ---- pass 1: log2-domain log-sum-exp of every query row --------------------
// A wave holds 64 queries as two register operands, so every 32-key operand
// it reads from LDS feeds two MFMAs (one per query block).
template <int D>
__global__ __launch_bounds__(FT_THREADS) void future_lse_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int32_t T, int32_t Hq,
    int32_t Hkv, float c2, float* __restrict__ lse) {
  __shared__ __align__(16) uint16_t ktile[2][FT_TILE * (D + 8)];
  const int h = blockIdx.x;
  const int g = (h * Hkv) / Hq;
  // largest tiles (most keys) first
  const int32_t i0 = (static_cast<int32_t>(gridDim.y - 1 - blockIdx.y)) * FT_ROWS;
  // the wave index is uniform across the wave: said so, the per-wave tests
  // below become scalar branches instead of per-lane masks
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const uint16_t* qh = q + static_cast<int64_t>(h) * T * D;
  const uint16_t* kg = k + static_cast<int64_t>(g) * T * D;
  const int32_t iw = i0 + FT_WROWS * wid;    // this wave's first query
  const int32_t my_q = iw + (lane & 31);     // this lane's queries: my_q and my_q + 32
  u32x4_t qreg[2][D / 16];
  load_operand_rows<D>(qh, iw, T, qreg[0]);
  load_operand_rows<D>(qh, iw + 32, T, qreg[1]);
  __builtin_amdgcn_sched_barrier(0);
  const int32_t ilast = min(i0 + FT_ROWS, T) - 1;
  const int ntile = ilast / FT_TILE + 1;      // key tiles 0 .. ilast/64
  TileLoader<D> ld;
  ld.load(kg, 0, T);
  ld.store(ktile[0]);
  settle(qreg[0]);
  settle(qreg[1]);
  __syncthreads();
  // Per query: m is an anchor, the running maximum of the scaled logits when
  // it last moved.  A key block adds 2^(c2 x - m) over its keys; when that
  // passes 2^64 (some logit above m + 64) or no anchor is set yet, m moves to
  // the running maximum and the block is summed again.  The sum is the same
  // up to rounding; most blocks skip the maximum.  The two lanes of a query
  // (l and l ^ 32) hold the same m and part, so they branch together.
  float m[2] = {-INFINITY, -INFINITY}, ssum[2] = {0.f, 0.f};
  auto add_block = [&](const f32x16_t& x, float& mq, float& sq) {
    float part = 0.f;
    if (mq != -INFINITY) {
#pragma unroll
      for (int r = 0; r < 16; ++r) part += __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], c2, -mq));
      part += __shfl_xor(part, 32, WAVE);
    }
    if (mq != -INFINITY && part <= 0x1p64f) {
      sq += part;
    } else {
      // the scale is positive: the largest scaled logit is the scaled maximum
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE)) * c2;
      const float mnew = fmaxf(mq, mx);
      if (mnew != -INFINITY) {
        part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          part += __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], c2, -mnew));
        part += __shfl_xor(part, 32, WAVE);
        sq = sq * __builtin_amdgcn_exp2f(mq - mnew) + part;
        mq = mnew;
      }
    }
  };
  for (int t = 0; t < ntile; ++t) {
    if (t + 1 < ntile) ld.load(kg, (t + 1) * FT_TILE, T);
    // keep the next tile's LDS stores after this tile's math, so that its
    // loads stay in flight meanwhile
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* kt = ktile[t & 1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int32_t kf = t * FT_TILE + 32 * kb;  // the key block's first key
      if (iw <= ilast && kf <= iw + FT_WROWS - 1) {  // some pair of the block is causal
        // the key operand read once per k-step, for both query blocks
        f32x16_t acc0 = {}, acc1 = {};
        const uint16_t* a = kt + (32 * kb + (lane & 31)) * (D + 8) + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4_t av = *reinterpret_cast<const u32x4_t*>(a + 16 * ks);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(qreg[0][ks]),
                                                         acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(qreg[1][ks]),
                                                         acc1, 0, 0, 0);
        }
        // keys of the block past the wave's first query need the causal mask
        if (kf + 31 > iw || kf + 32 > T) {
          const int32_t key0 = kf + 4 * (lane >> 5);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int32_t key = key0 + 8 * (r >> 2) + (r & 3);
            acc0[r] = (key <= my_q && key < T) ? acc0[r] : -INFINITY;
            acc1[r] = (key <= my_q + 32 && key < T) ? acc1[r] : -INFINITY;
          }
        }
        add_block(acc0, m[0], ssum[0]);
        add_block(acc1, m[1], ssum[1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < ntile) {
      ld.store(ktile[(t + 1) & 1]);
    }
    __syncthreads();
  }
  if (lane < 32) {
    float* lh = lse + static_cast<int64_t>(h) * T;
    if (my_q < T) lh[my_q] = m[0] + __log2f(ssum[0]);
    if (my_q + 32 < T) lh[my_q + 32] = m[1] + __log2f(ssum[1]);
  }
}

// ---- pass 2: column sums of the probabilities of queries past the window --
// A wave holds 64 keys as two register operands, so every 32-query operand
// it reads from LDS feeds two MFMAs (one per key block).
template <int D>
__global__ __launch_bounds__(FT_THREADS) void future_colsum_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ lse,
    int32_t T, int32_t Hq, int32_t Hkv, int32_t W, float c2, float* __restrict__ part) {
  __shared__ __align__(16) uint16_t qtile[2][FT_TILE * D];
  __shared__ float ltile[2][FT_TILE];
  const int h = blockIdx.x;
  const int g = (h * Hkv) / Hq;
  const int32_t j0 = static_cast<int32_t>(blockIdx.y) * FT_ROWS;  // earliest keys: most queries
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const uint16_t* kg = k + static_cast<int64_t>(g) * T * D;
  const int32_t jw = j0 + FT_WROWS * wid;    // this wave's first key
  u32x4_t kreg[2][D / 16];
  load_operand_rows<D>(kg, jw, T, kreg[0]);
  load_operand_rows<D>(kg, jw + 32, T, kreg[1]);
  __builtin_amdgcn_sched_barrier(0);
  // this lane's 32 keys: jw + 32*b + 8*(r/4) + 4*(lane/32) + r%4
  float col[2][16];
#pragma unroll
  for (int r = 0; r < 16; ++r) col[0][r] = col[1][r] = 0.f;
  const int32_t qfirst = j0 + W;              // first query any key of the tile counts
  const int t0 = qfirst / FT_TILE;
  const int nsteps = (qfirst < T) ? (T - 1) / FT_TILE + 1 - t0 : 0;  // query tiles
  const uint16_t* qh = q + static_cast<int64_t>(h) * T * D;
  const float* lh = lse + static_cast<int64_t>(h) * T;
  // the query tile and its 64 log-sum-exps, straight into LDS
  auto fetch = [&](int step, int b) {
    const int32_t qrow0 = (t0 + step) * FT_TILE;
    TileDma<D>::issue(qh, qrow0, T, qtile[b], wid);
    if (wid == 0)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(qrow0 + FT_TILE <= T
                                                              ? lh + qrow0 + lane
                                                              : lh + min(qrow0 + lane, T - 1)),
          (__attribute__((address_space(3))) void*)(ltile[b]), 4, 0, 0);
  };
  if (nsteps > 0) fetch(0, 0);
  settle(kreg[0]);
  settle(kreg[1]);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) fetch(step + 1, buf ^ 1);
    const char* qb8 = reinterpret_cast<const char*>(qtile[buf]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int32_t qs = (t0 + step) * FT_TILE + 32 * qb;  // the query block's first query
      if (jw < T && qs + 31 >= jw + W) {  // some query of the block counts (uniform)
        // the query operand read once per k-step, for both key blocks
        f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int cch = 2 * ks + (lane >> 5);
          const u32x4_t bv =
              *reinterpret_cast<const u32x4_t*>(qb8 + TileDma<D>::at(32 * qb + (lane & 31), cch));
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[0][ks]), as_bf16x8(bv),
                                                         acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[1][ks]), as_bf16x8(bv),
                                                         acc1, 0, 0, 0);
        }
        // every (query, key) pair of the block counts when its first query is
        // at least W past the wave's last key and both lie before T
        const bool full = qs >= jw + FT_WROWS - 1 + W && qs + 32 <= T && jw + FT_WROWS <= T;
        if (!full) {  // uniform: pairs that do not count get a logit of -inf (weight 0)
          // the lane's query qi and keys key0 + o (o = 8*(r/4) + r%4, and
          // o + 32 for the second block): a pair counts when qi < T,
          // o < T - key0 and o <= qi - key0 - W
          const int32_t qi = qs + (lane & 31);
          const int32_t key0 = jw + 4 * (lane >> 5);
          const int32_t d = qi < T ? qi - key0 - W : -1;
          const int32_t e = min(T - key0 - 1, d);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = 8 * (r >> 2) + (r & 3);
            if (o > e) acc0[r] = -INFINITY;
            if (o + 32 > e) acc1[r] = -INFINITY;
          }
        }
        // a multiply-add, an exp2 and an add per pair
        const float l2 = ltile[buf][32 * qb + (lane & 31)];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          col[0][r] += __builtin_amdgcn_exp2f(acc0[r] * c2 - l2);
          col[1][r] += __builtin_amdgcn_exp2f(acc1[r] * c2 - l2);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile has landed
    __syncthreads();
  }
  // every key's sum is spread over the 32 query lanes of its wave half
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v = col[b][r];
      v += __shfl_xor(v, 1, WAVE);
      v += __shfl_xor(v, 2, WAVE);
      v += __shfl_xor(v, 4, WAVE);
      v += __shfl_xor(v, 8, WAVE);
      v += __shfl_xor(v, 16, WAVE);
      col[b][r] = v;
    }
  }
  if ((lane & 31) == 0) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t key = jw + 32 * b + 4 * (lane >> 5) + 8 * (r >> 2) + (r & 3);
        if (key < T) part[static_cast<int64_t>(h) * T + key] = col[b][r];
      }
    }
  }
}

// ---- the group sum: y[g][j] = sum over the group's heads of part[h][j] ------
__global__ __launch_bounds__(256) void future_group_sum_kernel(const float* __restrict__ part,
                                                               int32_t T, int32_t G,
                                                               float* __restrict__ y) {
  const int g = blockIdx.y;
  const int32_t j = static_cast<int32_t>(blockIdx.x) * 256 + static_cast<int32_t>(threadIdx.x);
  if (j >= T) return;
  const float* p = part + static_cast<int64_t>(g) * G * T + j;
  float acc = 0.f;
  for (int u = 0; u < G; ++u) acc += p[static_cast<int64_t>(u) * T];
  y[static_cast<int64_t>(g) * T + j] = acc;
}

template <int D>
hipError_t launch_future_d(int32_t T, int32_t Hq, int32_t Hkv, int32_t W, float c2,
                           const uint16_t* q, const uint16_t* k, float* work, float* y,
                           hipStream_t stream) {
  const uint32_t tiles = static_cast<uint32_t>((T + FT_ROWS - 1) / FT_ROWS);
  float* lse = work;
  float* part = work + static_cast<int64_t>(Hq) * T;
  hipLaunchKernelGGL(future_lse_kernel<D>, dim3(static_cast<uint32_t>(Hq), tiles), dim3(FT_THREADS),
                     0, stream, q, k, T, Hq, Hkv, c2, lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(future_colsum_kernel<D>, dim3(static_cast<uint32_t>(Hq), tiles),
                     dim3(FT_THREADS), 0, stream, q, k, lse, T, Hq, Hkv, W, c2, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(future_group_sum_kernel,
                     dim3(static_cast<uint32_t>((T + 255) / 256), static_cast<uint32_t>(Hkv)),
                     dim3(256), 0, stream, part, T, Hq / Hkv, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_future_target(const Geometry& geo, int32_t n_tokens, const uint16_t* q,
                                const uint16_t* k, float scale_log2e, float* work, float* y,
                                hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const float c2 = scale_log2e;
  if (geo.head_dim == 128)
    return launch_future_d<128>(n_tokens, geo.n_q_heads, geo.n_kv_heads, geo.n_recent, c2, q, k,
                                work, y, stream);
  return launch_future_d<64>(n_tokens, geo.n_q_heads, geo.n_kv_heads, geo.n_recent, c2, q, k,
                             work, y, stream);
}

}  // namespace kvpop
