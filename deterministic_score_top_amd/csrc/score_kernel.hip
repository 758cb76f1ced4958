// Score phase of the DSA indexer top-k scan on gfx950 (CDNA4).
//
// Computes I[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[s, :]) for every causally visible
// (query, key) pair of every segment and writes it to a dense row per query (out[t * ld + j],
// j = segment-local key index): the FP32 score, or for the top-k call its order-preserving
// 32-bit key.  Score definition: the lightning-indexer form the scan of flashinfer PR #8691
// (description; vendoring note) is built on.
//
// Work decomposition.  A work unit is (segment, tile of 8 consecutive queries, chunk of
// keys).  The grid is persistent: every block draws unit numbers from a counter in the
// workspace (the ticket word of the same page's description: blocks that are resident take
// the next unit, so a foreign kernel holding some CUs does not push units into a second
// wave).  Every block derives the same plan from the segment tables: segments longest tile
// first, inside a segment from the last query tile (most visible keys) to the first, so the
// cheapest units run last; whole tiles per unit unless the batch's longest tiles are long
// next to a block's share, then even pieces of at most a quarter of that share.  The counter
// is checked and reset by the select kernel that follows (or, for the scores-only call, by
// the last block to leave), so steady-state calls pay no reset.
//
// Inside a unit (512 threads = 8 waves, one query per wave):
//   * each wave holds the BF16 A operand of its query (64 heads x 128 dims: 2 row blocks of
//     32 rows x 8 K-steps of 16) in VGPRs, loaded once per unit, and the query's head weights;
//   * 64-key tiles of k land in LDS two tiles ahead (three buffers) by buffer loads that
//     write LDS directly, 16-byte chunks XOR-swizzled by key so the B-operand reads are
//     bank-conflict free;
//   * per tile: 2 column blocks of 32 keys x 2 row blocks x 8 K-steps of
//     v_mfma_f32_32x32x16_bf16 (FP32 accumulate, d ascending);
//   * epilogue in registers: lane half hf holds heads 32*rb + 16*hf + i (i = 0..15) of key
//     lane&31; it sums w * ReLU over them in a fixed order (ReLU as one integer max on the
//     float bits), then adds the other half's sum with v_permlane32_swap.  The instruction
//     sequence per (t, s) is the same in every unit, tile position, chunking and grid, so
//     every score is bit-reproducible.
//
// Row mapping of the A operand: row n of row block rb carries head
// 32*rb + 16*((n>>2)&1) + 4*(n>>3) + (n&3), which puts heads 32*rb + 16*hf + 0..15 in the
// accumulator registers 0..15 of lane half hf.

#include "dsa_internal.h"
#include "wave_ops.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKBufBytes = kTileKeys * kDim * 2;  // one staged key tile: 16 KiB
constexpr int kKBufs = 3;                         // LDS tile buffers: tiles land two ahead
// s_waitcnt immediate that waits only on the vector memory counter: OR in the count (< 16);
// expcnt (bits 6:4) and lgkmcnt (bits 11:8) at their maxima do not wait
constexpr int kWaitVm = 0x0F70;
constexpr int kSlotInts = 16;
constexpr int kSegSortMax = 256;     // batches with more segments keep table order
constexpr int kUnitsPerBlock = 4;    // a unit holds at most ~1/4 of a resident block's share
constexpr int kGuidedMin = 32;       // batches of only long tiles: guided chunks down to 1/32 of a share
constexpr int kMinChunkTiles = 2;    // smallest automatic key chunk, in key tiles
constexpr int kMaxChunkSearch = 32;  // candidate chunks tried for small batches
constexpr int kPartEntries = kScoreThreads + 4;
// Buffer resource word 3 for raw (stride 0) 32-bit buffers on gfx9-family parts, and a byte
// offset that is always out of range (dropped store).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kDropOffset = 0x40000000;
constexpr int kStageChunks = kTileKeys * kDim * 2 / 16 / kScoreThreads;  // 16-byte chunks per thread per tile

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// max(x, +0) for finite x, as one integer max on the bits (-0 and negatives map to +0).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Order-preserving map of an FP32 score to 32 bits: unsigned order of the keys is score order
// (negative scores have all bits flipped, non-negative ones the sign bit set).  Sums formed
// here never produce -0 (they start from +0 and add finite terms), so no sign canonicalisation
// is needed.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// x[l] + x[l ^ 32], lower half first in every lane (v_permlane32_swap, no LDS traffic).
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// First index in arr[0..n) whose value exceeds x (arr non-decreasing).
__device__ __forceinline__ int upper_bound_u32(const uint32_t* arr, int n, uint32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (arr[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// In-place exclusive scan of arr[0..n) by the block; arr[n] receives the total.
__device__ void block_scan_excl(uint32_t* arr, int n, uint32_t* part) {
  const int tid = threadIdx.x;
  const int per = (n + kScoreThreads - 1) / kScoreThreads;
  const int beg = min(tid * per, n);
  const int end = min(beg + per, n);
  uint32_t s = 0;
  for (int i = beg; i < end; ++i) s += arr[i];
  part[tid] = s;
  __syncthreads();
  if (tid < 64) {
    constexpr int kPer = kScoreThreads / 64;  // partial sums per lane
    uint32_t a[kPer];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      a[i] = part[kPer * tid + i];
      sum += a[i];
    }
    const uint32_t inc = wave_incl_scan(sum);
    uint32_t ex = inc - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      part[kPer * tid + i] = ex;
      ex += a[i];
    }
    if (tid == 63) part[kScoreThreads] = inc;
  }
  __syncthreads();
  uint32_t run = part[tid];
  for (int i = beg; i < end; ++i) {
    const uint32_t v = arr[i];
    arr[i] = run;
    run += v;
  }
  if (tid == 0) arr[n] = part[kScoreThreads];
  __syncthreads();
}

// Guided chunk (in key tiles) of tile g of ntiles: half of a block's share of the work that
// remains from tile g on (ntiles - g tiles of about `full` key tiles each), between `lo` and
// `full` (a whole tile).
__device__ __forceinline__ uint32_t guided_chunk(int g, int ntiles, uint32_t grid, int full, int lo) {
  const uint32_t rest = (uint32_t)(ntiles - g) * (uint32_t)full;
  const uint32_t c = (rest + 2u * grid - 1u) / (2u * grid);
  return min((uint32_t)full, max((uint32_t)lo, c));
}

// The work decomposition of a batch (every block of a launch derives the same one from the
// segment tables; the plan kernel derives it once for a prepared runner): validates the tables,
// orders segments longest tile first, counts each query tile's key tiles, picks the key chunk
// for a persistent grid of `grid` blocks and builds the unit prefix.  Leaves seg_tp (tile prefix
// per segment in that order), seg_ord and unit_pf (unit prefix per tile) in LDS.
struct PlanInfo {
  uint32_t units;
  int ntiles;
  int chunk_tiles;
  int guided_tiles;  // > 0: tile g's chunk is guided_chunk(g) (see there), else chunk_tiles
  int guided_min;
  bool whole_tiles;  // every tile is exactly one unit
  int flags;         // bit 0: invalid tables, bit 1: a segment longer than Lmax
};

__device__ PlanInfo compute_plan(const ScoreParams& p, uint32_t grid, int* slot, uint32_t* part, uint32_t* seg_tp,
                                 uint32_t* seg_ord, uint32_t* unit_pf) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = p.B;
  if (tid == 0) slot[2] = 0;
  __syncthreads();
  {
    int flags = 0;
    for (int b = tid; b <= B; b += kScoreThreads) {
      const int cq = p.cu_q[b], ck = p.cu_k[b];
      if (b == 0 && (cq != 0 || ck != 0)) flags |= 1;
      if (b == B && (cq != p.T || ck != p.Tkv)) flags |= 1;
      if (b < B) {
        const int lq = p.cu_q[b + 1] - cq, lk = p.cu_k[b + 1] - ck;
        if (lq < 0 || lk < 0) flags |= 1;
        if (lk > p.Lmax) flags |= 2;
        seg_tp[b] = lq > 0 ? (uint32_t)ceil_div(lq, kTileQueries) : 0u;
      }
    }
    if (flags) atomicOr(&slot[2], flags);
  }
  __syncthreads();
  const int plan_flags = slot[2];
  uint32_t units = 0;
  int ntiles = 0;
  int chunk_keys = kTileKeys;
  int guided = 0, guided_min = 1;
  bool whole_tiles = false;
  if (!(plan_flags & 1)) {
    // Segment order: longest tile first (the key is the first tile's key-tile count), ties by
    // segment index, so that the longest work units of the whole batch start first.  Every
    // block derives the same order from the same tables.  Large batches keep table order.
    auto seg_key = [&](int b) -> uint32_t {
      const int cq = p.cu_q[b], lq = p.cu_q[b + 1] - cq;
      const int lk = min(p.cu_k[b + 1] - p.cu_k[b], p.Lmax);
      const int off = p.offs ? p.offs[b] : 0;
      return lq > 0 ? (uint32_t)ceil_div(clampi(off + lq, 0, lk), kTileKeys) : 0u;
    };
    if (B > 1 && B <= kSegSortMax) {
      for (int b = tid; b < B; b += kScoreThreads) unit_pf[b] = seg_key(b);  // scratch
      __syncthreads();
      for (int b = tid; b < B; b += kScoreThreads) {
        const uint32_t kb_ = unit_pf[b];
        int r = 0;
        for (int o = 0; o < B; ++o) {
          const uint32_t ko = unit_pf[o];
          r += (ko > kb_ || (ko == kb_ && o < b)) ? 1 : 0;
        }
        seg_ord[r] = (uint32_t)b;
      }
      __syncthreads();
      // tile counts in that order
      for (int j = tid; j < B; j += kScoreThreads) unit_pf[j] = seg_tp[seg_ord[j]];
      __syncthreads();
      for (int j = tid; j < B; j += kScoreThreads) seg_tp[j] = unit_pf[j];
    } else {
      for (int b = tid; b < B; b += kScoreThreads) seg_ord[b] = (uint32_t)b;
    }
    __syncthreads();
    block_scan_excl(seg_tp, B, part);
    ntiles = (int)seg_tp[B];
    if (ntiles > p.max_tiles) {
      ntiles = 0;  // cannot happen for valid tables: ceil-sum of tiles <= T/8 + B
    }
    // key tiles of every query tile (inside a segment the tile with the most keys comes first)
    // and their total
    if (tid == 0) {
      slot[3] = 0;
      slot[6] = 0;
      slot[10] = -1;
    }
    __syncthreads();
    uint32_t work = 0, kt_max = 0, kt_min = 0xffffffffu;
    for (int g = tid; g < ntiles; g += kScoreThreads) {
      const int j = upper_bound_u32(seg_tp, B + 1, (uint32_t)g) - 1;
      const int b = (int)seg_ord[j];
      const int qb = p.cu_q[b], lq = p.cu_q[b + 1] - qb;
      const int lk = min(p.cu_k[b + 1] - p.cu_k[b], p.Lmax);
      const int off = p.offs ? p.offs[b] : 0;
      const int ntile_b = (int)(seg_tp[j + 1] - seg_tp[j]);
      const int i = ntile_b - 1 - (g - (int)seg_tp[j]);
      const int nq_end = min((i + 1) * kTileQueries, lq);
      const uint32_t kt = (uint32_t)ceil_div(clampi(off + nq_end, 0, lk), kTileKeys);
      unit_pf[g] = kt;
      work += kt;
      kt_max = max(kt_max, kt);
      if (kt) kt_min = min(kt_min, kt);
    }
    // integer sum, max and min: order-free; one LDS atomic per wave
    work = wave_sum(work);
    kt_max = wave_max(kt_max);
    kt_min = wave_min(kt_min);
    if (lane == 0) {
      atomicAdd(reinterpret_cast<uint32_t*>(&slot[3]), work);
      atomicMax(reinterpret_cast<uint32_t*>(&slot[6]), kt_max);
      atomicMin(reinterpret_cast<uint32_t*>(&slot[10]), kt_min);
    }
    __syncthreads();
    // Key chunk per work unit, in key tiles: forced by the caller, else chosen from the batch.
    // Longest-first order balances the blocks as long as the longest tile is small next to a
    // resident block's share of the batch's key tiles; whole tiles are then best (each unit
    // reloads its queries).  When the longest tile exceeds 3/5 of the share (long documents,
    // a few long queries), no unit may exceed a quarter of the share: the longest tile is cut
    // into the fewest even pieces within that bound and their size is the chunk, so tiles near
    // the longest split into pieces of nearly equal size.  (Measured: long-document batches
    // run 15-18 % faster than with whole tiles; causal batches and the CP tail prefer whole
    // tiles by 1-2 %.)
    // When even the shortest tile is long next to the share (every query of the batch sees about
    // as many keys: a CP tail), whole tiles leave each block two or three units of equal size,
    // and a block displaced by foreign work leaves a whole unit for a second round (measured:
    // CP tail 1.32x slower with one CU held).  Then chunks are guided (guided self-scheduling):
    // tile g is cut in pieces of half the per-block share of the work that remains from it on,
    // whole tiles while that is at least a tile, shrinking to 1/32 of a share at the end, so
    // blocks that finish early take the small pieces and the last round is short, while most
    // units stay long (each unit start reloads the query block).
    // Small batches (no more query tiles than blocks) instead take the smallest chunk that
    // still fits the whole batch in one round of units, one per block: each unit start costs
    // a query-block load, so a second round of short units is slower than longer units
    // (measured: 4 queries of 42k keys 19 -> 17 us, N = 1024 causal 32 -> 23 us).
    int chunk_tiles = p.chunk_tiles;
    if (chunk_tiles <= 0) {
      const uint32_t total = (uint32_t)slot[3], longest = max((uint32_t)slot[6], 1u);
      const uint32_t share = total / grid;
      chunk_tiles = (int)longest;
      if (ntiles <= (int)grid) {
        uint32_t c = max((total + grid - 1) / grid, 1u);
        for (int it = 0; it < kMaxChunkSearch && c < longest; ++it, ++c) {
          uint32_t n_units = 0;
          for (int g = tid; g < ntiles; g += kScoreThreads) n_units += (unit_pf[g] + c - 1) / c;
          n_units = wave_sum(n_units);
          __syncthreads();  // every thread has read slot[7] of the previous candidate
          if (tid == 0) slot[7] = 0;
          __syncthreads();
          if (lane == 0) atomicAdd(reinterpret_cast<uint32_t*>(&slot[7]), n_units);
          __syncthreads();
          if ((uint32_t)slot[7] <= grid) break;
        }
        chunk_tiles = (int)min(c, longest);
      } else if (5 * longest > 3 * share) {
        const uint32_t bound = max(share / kUnitsPerBlock, (uint32_t)kMinChunkTiles);
        const uint32_t m = (longest + bound - 1) / bound;
        chunk_tiles = (int)max((longest + m - 1) / m, 1u);
      } else if ((uint32_t)slot[10] > share / 8u) {
        guided = (int)longest;
        guided_min = (int)max(share / kGuidedMin, (uint32_t)kMinChunkTiles);
      }
    }
    chunk_keys = chunk_tiles * kTileKeys;
    if (tid == 0) slot[8] = 0;
    __syncthreads();
    bool one_each = true;  // every tile is exactly one unit (keyless tiles have none)
    for (int g = tid; g < ntiles; g += kScoreThreads) {
      const uint32_t ct = guided ? guided_chunk(g, ntiles, grid, guided, guided_min) : (uint32_t)chunk_tiles;
      const uint32_t nu = (unit_pf[g] + ct - 1) / ct;
      unit_pf[g] = nu;
      one_each &= nu == 1u;
    }
    if (!one_each) atomicOr(&slot[8], 1);
    __syncthreads();
    whole_tiles = slot[8] == 0;
    block_scan_excl(unit_pf, ntiles, part);
    units = unit_pf[ntiles];
  }
  PlanInfo info;
  info.units = units;
  info.ntiles = ntiles;
  info.chunk_tiles = chunk_keys / kTileKeys;
  info.guided_tiles = guided;
  info.guided_min = guided_min;
  info.whole_tiles = whole_tiles;
  info.flags = plan_flags;
  return info;
}

// Header of a prepared plan (u32 words at the plan's start), followed by copies of the segment
// tables the plan was derived from (cu_q[B+1], cu_k[B+1], offsets[B]) and then seg_tp[B+1],
// seg_ord[B], unit_pf[ntiles+1].
constexpr int kPlanUnits = 0, kPlanTiles = 1, kPlanChunk = 2, kPlanWhole = 3, kPlanFlags = 4, kPlanGrid = 5,
              kPlanB = 6, kPlanGuided = 7, kPlanGuidedMin = 8, kPlanHeader = 16;

__device__ __forceinline__ int plan_tables_at(int B) { return kPlanHeader; }
__device__ __forceinline__ int plan_arrays_at(int B) { return kPlanHeader + 3 * B + 2; }

// Prepared path: the plan the prepare step stored, if the tables it was derived from still hold
// the live values and it was made for this grid (else returns false and nothing is loaded).
__device__ bool load_plan(const ScoreParams& p, int* slot, uint32_t* seg_tp, uint32_t* seg_ord, uint32_t* unit_pf,
                          PlanInfo& info) {
  const int tid = threadIdx.x;
  const int B = p.B;
  const uint32_t* const hdr = p.plan;
  const uint32_t* const tab = p.plan + plan_tables_at(B);
  if (tid == 0) slot[9] = (hdr[kPlanGrid] != gridDim.x || hdr[kPlanB] != (uint32_t)B) ? 1 : 0;
  __syncthreads();
  int diff = 0;
  for (int i = tid; i <= B; i += kScoreThreads) {
    diff |= (uint32_t)p.cu_q[i] != tab[i];
    diff |= (uint32_t)p.cu_k[i] != tab[B + 1 + i];
    if (i < B) diff |= (uint32_t)(p.offs ? p.offs[i] : 0) != tab[2 * B + 2 + i];
  }
  if (diff) atomicOr(&slot[9], 1);
  __syncthreads();
  if (slot[9]) return false;
  info.units = hdr[kPlanUnits];
  info.ntiles = (int)hdr[kPlanTiles];
  info.chunk_tiles = (int)hdr[kPlanChunk];
  info.guided_tiles = (int)hdr[kPlanGuided];
  info.guided_min = (int)hdr[kPlanGuidedMin];
  info.whole_tiles = hdr[kPlanWhole] != 0;
  info.flags = (int)hdr[kPlanFlags];
  const uint32_t* const arr = p.plan + plan_arrays_at(B);
  const int nseg = B + 1, nord = B, nunit = (info.flags & 1) ? 0 : info.ntiles + 1;
  for (int i = tid; i < nseg; i += kScoreThreads) seg_tp[i] = arr[i];
  for (int i = tid; i < nord; i += kScoreThreads) seg_ord[i] = arr[nseg + i];
  for (int i = tid; i < nunit; i += kScoreThreads) unit_pf[i] = arr[nseg + nord + i];
  __syncthreads();
  return true;
}

__global__ __launch_bounds__(kScoreThreads, 2) void score_kernel(ScoreParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* const kbuf0 = smem;
  unsigned char* const kbuf1 = smem + kKBufBytes;
  unsigned char* const kbuf2 = smem + 2 * kKBufBytes;
  int* const slot = reinterpret_cast<int*>(smem + kKBufs * kKBufBytes);
  uint32_t* const part = reinterpret_cast<uint32_t*>(slot + kSlotInts);
  uint32_t* const seg_tp = part + kPartEntries;                   // B + 1 entries
  uint32_t* const seg_ord = seg_tp + ((p.B + 1 + 3) & ~3);        // B entries
  uint32_t* const unit_pf = seg_ord + ((p.B + 3) & ~3);           // max_tiles + 1 entries

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index, explicitly wave-uniform so per-wave values (query row, buffer resources) live
  // in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = p.B;

  // ---- per-block plan (the block's first ticket is drawn now; its latency overlaps the plan):
  // the prepared one when it still applies, else derived from the tables here
  if (tid == 0) slot[0] = (int)atomicAdd(p.ctrl + kCtrlTicket, 1u);
  PlanInfo info;
  if (!(p.plan && load_plan(p, slot, seg_tp, seg_ord, unit_pf, info)))
    info = compute_plan(p, gridDim.x, slot, part, seg_tp, seg_ord, unit_pf);
  const int plan_flags = info.flags;
  const uint32_t units = info.units;
  const int ntiles = info.ntiles;
  const int chunk_keys = info.chunk_tiles * kTileKeys;
  const int guided = info.guided_tiles;
  const int guided_min = info.guided_min;
  const bool whole_tiles = info.whole_tiles;
  // this call's verdict on its tables, for the select kernel (always overwritten, so a bad call
  // does not affect later calls on the same workspace)
  if (blockIdx.x == 0 && tid == 0) p.ctrl[kCtrlCallBad] = (plan_flags & 1) ? 1u : 0u;
  if (tid == 0 && plan_flags) {
    uint32_t st = 0;
    if (plan_flags & 1) st |= kStatusBadSegments;
    if (plan_flags & 2) st |= kStatusSeqlenBound;
    atomicOr(p.ctrl + kCtrlStatus, st);
  }

  // ---- ticket loop ------------------------------------------------------------------------
  uint32_t u = (uint32_t)slot[0];
  if (tid == 0 && u >= units + gridDim.x) atomicOr(p.ctrl + kCtrlStatus, kStatusCorruptCounter);
  // With a select kernel to follow, the counter is checked and reset there (stream order puts
  // it after every block of this kernel): record the value it must reach.
  if (p.store_keys && blockIdx.x == 0 && tid == 0) p.ctrl[kCtrlExpected] = units + gridDim.x;

  // lane roles (fixed for the whole kernel): one query per wave; A row / B column n, lane half hf
  const int n = lane & 31;
  const int hf = lane >> 5;
  // head held in A row n of row block rb: 32*rb + 16*((n>>2)&1) + 4*(n>>3) + (n&3), so that the
  // accumulator register i of row block rb in lane half hf holds head 32*rb + 16*hf + i
  const int ha = 16 * ((n >> 2) & 1) + 4 * (n >> 3) + (n & 3);

  int iter = 0;
  while (u < units) {
    if (tid == 0) slot[4 + (iter & 1)] = (int)atomicAdd(p.ctrl + kCtrlTicket, 1u);

    // decode u -> (tile g, chunk c) -> (segment b, tile i)
    // (every lane computes the same values; readfirstlane makes that visible to the compiler so
    // the unit's scalars and buffer resources stay in scalar registers)
    // (one unit per tile, the usual case, needs no search)
    const bool whole = whole_tiles;
    const int g = whole ? (int)u : __builtin_amdgcn_readfirstlane(upper_bound_u32(unit_pf, ntiles + 1, u) - 1);
    const int c = whole ? 0 : __builtin_amdgcn_readfirstlane((int)(u - unit_pf[g]));
    const int j = __builtin_amdgcn_readfirstlane(upper_bound_u32(seg_tp, B + 1, (uint32_t)g) - 1);
    const int b = __builtin_amdgcn_readfirstlane((int)seg_ord[j]);
    const int ntile_b = __builtin_amdgcn_readfirstlane((int)(seg_tp[j + 1] - seg_tp[j]));
    const int ti = ntile_b - 1 - (g - __builtin_amdgcn_readfirstlane((int)seg_tp[j]));

    const int qb = p.cu_q[b];
    const int lq = p.cu_q[b + 1] - qb;
    const int kb = p.cu_k[b];
    const int lk = min(p.cu_k[b + 1] - kb, p.Lmax);
    const int off = p.offs ? p.offs[b] : 0;
    const int tq0 = ti * kTileQueries;
    const int nq = min(kTileQueries, lq - tq0);
    const int nmax = clampi(off + tq0 + nq, 0, lk);
    const int ck = guided ? (int)guided_chunk(g, ntiles, gridDim.x, guided, guided_min) * kTileKeys : chunk_keys;
    const int kbeg = c * ck;
    const int kend = min(kbeg + ck, nmax);

    // this wave's query (tile-local index wv): A operand for both row blocks and all 8 K-steps
    const bool qvalid = wv < nq;
    bf16x8 qf[2][8];
    float wr[32];
    int n_o = 0;
    if (qvalid) {
      const int64_t t = qb + tq0 + wv;
      const uint16_t* qrow = p.q + t * (kHeads * kDim);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          qf[rb][j] = *reinterpret_cast<const bf16x8*>(qrow + (32 * rb + ha) * kDim + 16 * j + 8 * hf);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x4* wrow = reinterpret_cast<const f32x4*>(p.w + t * kHeads + 32 * rb + 16 * hf);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const f32x4 x = wrow[v];
          wr[16 * rb + 4 * v] = x[0];
          wr[16 * rb + 4 * v + 1] = x[1];
          wr[16 * rb + 4 * v + 2] = x[2];
          wr[16 * rb + 4 * v + 3] = x[3];
        }
      }
      n_o = clampi(off + tq0 + wv + 1, 0, lk);
    } else {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j) qf[rb][j] = bf16x8{};
#pragma unroll
      for (int v = 0; v < 32; ++v) wr[v] = 0.f;
    }
    float* const orow = p.out + (int64_t)(qb + tq0 + min(wv, nq - 1)) * p.ld;
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(orow, (short)0, n_o * 4, kRsrcWord3);

    // key tile staging: thread tid moves 16-byte chunks id = r*kScoreThreads + tid; tiles are
    // fetched two ahead of the one being multiplied (two register stages, two LDS buffers)
    // Raw buffer resources with hardware range checks: keys at or past the segment's end read
    // as zero, and score stores past the query's visible count (or from lane half 1, which
    // holds the same sums) are dropped.  The tile loop therefore has no branches around memory
    // operations.
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.k + (int64_t)kb * kDim), (short)0, lk * (kDim * 2), kRsrcWord3);
    // A tile is written to LDS by buffer loads that deposit each lane's 16 bytes directly at
    // LDS base + 16 * lane (no register staging).  Instruction r of wave wv fills the 1 KiB
    // block id = r * kWaves + wv, i.e. key rows 4*id .. 4*id+3; lane l writes chunk position
    // l & 15 of row 4*id + (l >> 4), so it fetches the global 16-byte chunk that the XOR
    // swizzle maps there.
    auto ldsload = [&](unsigned char* buf, int kt0) {
#pragma unroll
      for (int r = 0; r < kStageChunks; ++r) {
        const int id = r * kWaves + wv;
        const int s = 4 * id + (lane >> 4), pos = lane & 15;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            krs, (__attribute__((address_space(3))) void*)(buf + id * 1024), 16,
            (kt0 + s) * (kDim * 2) + ((pos ^ (s & 15)) << 4), 0, 0, 0);
      }
    };
    // One phase = the MFMAs of one 32-key column block (2 row blocks x 8 K-steps) into (n0, n1),
    // interleaved with the epilogue of the previous column block's accumulators (e0, e1), so
    // the VALU work of the epilogue issues between independent MFMAs.  The epilogue sums
    // w * ReLU over this lane's 32 heads (two ascending runs of 16, heads 32*rb + 16*hf + i)
    // and adds the other lane half's sum.  ReLU is an integer max on the float bits: negative
    // values and -0 are negative as int32 and become +0; non-negative values pass unchanged.
    auto phase = [&](const unsigned char* cur, int cb, f32x16& n0, f32x16& n1, const f32x16& e0,
                     const f32x16& e1) -> float {
      n0 = f32x16{};
      n1 = f32x16{};
      float p0 = 0.f, p1 = 0.f;
      const int s = 32 * cb + n;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(cur + s * (kDim * 2) + (((2 * j + hf) ^ (n & 15)) << 4));
        // each MFMA is followed by the epilogue step of the matching row block of the previous
        // column block (whose chain finished at least one MFMA earlier); the schedule groups
        // keep the compiler from bunching the epilogue at the start of the phase
        n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][j], kf, n0, 0, 0, 0);
        p0 = __builtin_fmaf(wr[2 * j], relu_bits(e0[2 * j]), p0);
        p0 = __builtin_fmaf(wr[2 * j + 1], relu_bits(e0[2 * j + 1]), p0);
        n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][j], kf, n1, 0, 0, 0);
        p1 = __builtin_fmaf(wr[16 + 2 * j], relu_bits(e1[2 * j]), p1);
        p1 = __builtin_fmaf(wr[16 + 2 * j + 1], relu_bits(e1[2 * j + 1]), p1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
      }
      return half_swap_sum(p0 + p1);
    };
    // Scores of a tile are stored after the barrier that follows it, so the store latency is
    // covered by the next tile's work instead of by the wait before the next LDS tile write.
    // Column block cb of a tile computes its MFMAs while finishing the epilogue of the block
    // before it: sc[0] is the last block of the previous tile (none when kt_prev < 0: its
    // store is dropped), sc[cb] for cb >= 1 is block cb-1 of this tile.  Accumulator pairs
    // alternate: even blocks in c0, odd blocks in c1.
    const bool keys_out = p.store_keys != 0;
    auto outbits = [&](float v) -> uint32_t { return keys_out ? score_key(v) : __float_as_uint(v); };
    constexpr int kPhases = kTileKeys / 32;
    static_assert(kPhases % 2 == 0, "column blocks alternate between two accumulator pairs");
    constexpr int kStores = kPhases / 2;  // score stores per tile
    static_assert(kStores + kStageChunks < 16, "vector-memory wait counts fit the 4-bit field");
    f32x16 c0a, c0b, c1a = f32x16{}, c1b = f32x16{};
    auto tile = [&](const unsigned char* buf, float (&sc)[kPhases]) {
#pragma unroll
      for (int cb = 0; cb < kPhases; ++cb)
        sc[cb] = (cb & 1) ? phase(buf, cb, c1a, c1b, c0a, c0b) : phase(buf, cb, c0a, c0b, c1a, c1b);
    };
    // Both lane halves hold every column-block sum, so one store covers two blocks: lane half
    // 0 writes block 2i, lane half 1 block 2i+1 (kStores = kPhases / 2 stores per tile).
    auto store_tile = [&](const float (&sc)[kPhases], int kt_prev, int kt0) {
      auto offset = [&](int cb) -> int {
        if (cb == 0) return kt_prev >= 0 ? (kt_prev + 32 * (kPhases - 1) + n) * 4 : kDropOffset;
        return (kt0 + 32 * (cb - 1) + n) * 4;
      };
#pragma unroll
      for (int i = 0; i < kPhases / 2; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(outbits(hf ? sc[2 * i + 1] : sc[2 * i]), ors,
                                              hf ? offset(2 * i + 1) : offset(2 * i), 0, 0);
    };

    const int ntl = kend > kbeg ? ceil_div(kend - kbeg, kTileKeys) : 0;
    if (ntl > 0) ldsload(kbuf0, kbeg);
    if (ntl > 1) ldsload(kbuf1, kbeg + kTileKeys);
    // Everything loaded before the tile loop (query block, weights, first tiles) has landed
    // here; saying so once keeps per-use waits on the query registers out of the loop, where
    // they would also wait for the prefetched tiles and the score stores.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int kt_prev = -1;
    float sc[kPhases];
    // One tile: tile t+2 starts loading into the buffer that tile t-1 used (free since the
    // barrier after it), tile t is multiplied, then this wave waits until its part of tile t+1
    // is in LDS, and the barrier makes all of tile t+1 visible.  Vector memory operations
    // complete in issue order; after tile t+1's loads this wave has issued tile t-1's score
    // stores (kStores) and, when present, tile t+2's loads (kStageChunks), so waiting until at
    // most that many are outstanding covers tile t+1.
    auto step = [&](unsigned char* cur, unsigned char* next2, int t) {
      const int kt0 = kbeg + t * kTileKeys;
      if (t + 2 < ntl) ldsload(next2, kt0 + 2 * kTileKeys);
      tile(cur, sc);
      if (t + 2 < ntl) {
        __builtin_amdgcn_s_waitcnt(kWaitVm | (kStores + kStageChunks));
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm | kStores);
      }
      // A plain barrier: a fenced one would also wait for tile t+2's loads.  The memory
      // clobber keeps the compiler from moving LDS accesses across it; this wave's reads of
      // tile t are complete (their MFMAs have issued), and its part of tile t+1 has landed.
      asm volatile("s_barrier" ::: "memory");
      store_tile(sc, kt_prev, kt0);
      kt_prev = kt0;
    };
    for (int tt = 0; tt < ntl; tt += 3) {
      step(kbuf0, kbuf2, tt);
      if (tt + 1 >= ntl) break;
      step(kbuf1, kbuf0, tt + 1);
      if (tt + 2 >= ntl) break;
      step(kbuf2, kbuf1, tt + 2);
    }
    if (ntl > 0) {  // last column block of the last tile
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p0 = __builtin_fmaf(wr[i], relu_bits(c1a[i]), p0);
        p1 = __builtin_fmaf(wr[16 + i], relu_bits(c1b[i]), p1);
      }
      const float s_last = half_swap_sum(p0 + p1);
      __builtin_amdgcn_raw_buffer_store_b32(outbits(s_last), ors,
                                            hf == 0 ? (kt_prev + 32 * (kPhases - 1) + n) * 4 : kDropOffset, 0, 0);
    }
    u = (uint32_t)slot[4 + (iter & 1)];
    ++iter;
  }

  // ---- exit: without a select kernel to follow, the last block out checks and resets the
  // counters --------------------------------------------------------------------------------
  if (!p.store_keys && tid == 0) {
    __threadfence();
    const uint32_t prev = atomicAdd(p.ctrl + kCtrlDone, 1u);
    if (prev == gridDim.x - 1) {
      const uint32_t tk = atomicAdd(p.ctrl + kCtrlTicket, 0u);
      if (tk != units + gridDim.x) atomicOr(p.ctrl + kCtrlStatus, kStatusCorruptCounter);
      atomicExch(p.ctrl + kCtrlTicket, 0u);
      atomicExch(p.ctrl + kCtrlDone, 0u);
    }
  }
}

__global__ void ctrl_init_kernel(uint32_t* ctrl) {
  if (threadIdx.x < kCtrlBytes / 4) ctrl[threadIdx.x] = 0u;
}

// Prepare step of a runner: one block derives the plan for a launch of `grid` blocks, stores it
// with the tables it came from at `out`, and zeroes the control block (the ticket word is zeroed
// once here; every run leaves it at zero again).
__global__ __launch_bounds__(kScoreThreads) void plan_kernel(ScoreParams p, uint32_t grid, uint32_t* out) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* const slot = reinterpret_cast<int*>(smem);
  uint32_t* const part = reinterpret_cast<uint32_t*>(slot + kSlotInts);
  uint32_t* const seg_tp = part + kPartEntries;
  uint32_t* const seg_ord = seg_tp + ((p.B + 1 + 3) & ~3);
  uint32_t* const unit_pf = seg_ord + ((p.B + 3) & ~3);
  const int tid = threadIdx.x;
  const int B = p.B;
  if (tid < kCtrlBytes / 4) p.ctrl[tid] = 0u;
  const PlanInfo info = compute_plan(p, grid, slot, part, seg_tp, seg_ord, unit_pf);
  if (tid == 0) {
    out[kPlanUnits] = info.units;
    out[kPlanTiles] = (uint32_t)info.ntiles;
    out[kPlanChunk] = (uint32_t)info.chunk_tiles;
    out[kPlanGuided] = (uint32_t)info.guided_tiles;
    out[kPlanGuidedMin] = (uint32_t)info.guided_min;
    out[kPlanWhole] = info.whole_tiles ? 1u : 0u;
    out[kPlanFlags] = (uint32_t)info.flags;
    out[kPlanGrid] = grid;
    out[kPlanB] = (uint32_t)B;
  }
  uint32_t* const tab = out + plan_tables_at(B);
  for (int i = tid; i <= B; i += kScoreThreads) {
    tab[i] = (uint32_t)p.cu_q[i];
    tab[B + 1 + i] = (uint32_t)p.cu_k[i];
    if (i < B) tab[2 * B + 2 + i] = (uint32_t)(p.offs ? p.offs[i] : 0);
  }
  uint32_t* const arr = out + plan_arrays_at(B);
  const int nseg = B + 1, nord = B, nunit = (info.flags & 1) ? 0 : info.ntiles + 1;
  for (int i = tid; i < nseg; i += kScoreThreads) arr[i] = seg_tp[i];
  for (int i = tid; i < nord; i += kScoreThreads) arr[nseg + i] = seg_ord[i];
  for (int i = tid; i < nunit; i += kScoreThreads) arr[nseg + nord + i] = unit_pf[i];
}

}  // namespace

size_t score_smem_bytes(int B, int max_tiles) {
  return (size_t)kKBufs * kKBufBytes + kSlotInts * 4 + kPartEntries * 4 +
         (size_t)((B + 1 + 3) & ~3) * 4 + (size_t)((B + 3) & ~3) * 4 + (size_t)(max_tiles + 1) * 4;
}

size_t score_smem_limit() { return 144 * 1024; }

size_t plan_bytes(int B, int max_tiles) {
  const size_t words = (size_t)kPlanHeader + 3 * (size_t)B + 2 + (size_t)(B + 1) + (size_t)B + (size_t)max_tiles + 1;
  return (words * 4 + 255) / 256 * 256;
}

hipError_t launch_plan(const ScoreParams& p, int grid, uint32_t* out, hipStream_t s) {
  const size_t smem = score_smem_bytes(p.B, p.max_tiles) - (size_t)kKBufs * kKBufBytes;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kScoreThreads), smem, s, p, (uint32_t)grid, out);
  return hipGetLastError();
}

hipError_t score_prepare(size_t max_smem) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_smem);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&plan_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_smem);
}

hipError_t score_occupancy(int* blocks_per_cu, size_t smem) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, score_kernel, kScoreThreads,
                                                      smem);
}

hipError_t launch_score(const ScoreParams& p, int grid, size_t smem, hipStream_t s) {
  hipLaunchKernelGGL(score_kernel, dim3(grid), dim3(kScoreThreads), smem, s, p);
  return hipGetLastError();
}

hipError_t launch_ctrl_init(uint32_t* ctrl, hipStream_t s) {
  hipLaunchKernelGGL(ctrl_init_kernel, dim3(1), dim3(64), 0, s, ctrl);
  return hipGetLastError();
}

}  // namespace dsa
