// Top-k select phase of the DSA indexer scan on gfx950.
//
// Input rows hold order-preserving 32-bit keys of the FP32 scores (written by the score phase):
// unsigned key order is score order.  The result rule of the scan (flashinfer PR #8691,
// description: top-k key ids per query, ties go to the larger id, result independent of
// partitioning) is the total order (key descending, position descending) on the row, and the
// selected keys are written with ids ascending.
//
// Per row (one workgroup of 256 threads, or 1024 when the batch has few rows; workgroups loop
// over rows):
//   A  a sample of the row (1/4 of it, 1/8 for 1024-thread rows) gives a threshold theta =
//      lower edge of the sample histogram bin that holds a rank four standard deviations past
//      k*m/n, so that, with overwhelming probability, theta is below the k-th key while only a
//      few hundred keys more than k are >= theta (the sample is kept in LDS for its histogram
//      when it fits);
//   B  one pass compares every key with theta and copies the survivors (key, position) into
//      per-wave LDS regions in position order (one ballot + mbcnt per key slot, no atomics);
//      the rest of a region's last 256-entry step is filled with key 0, below every survivor,
//      so the passes below read whole steps without masks;
//   C  the exact k-th key T is found over the survivors with range-normalised LDS histograms
//      (1024 bins per pass) until the bin holding rank k has at most 64 keys or one value;
//      one more pass counts, per wave, the keys above that bin and gathers the bin's keys,
//      which one wave ranks directly: T, how many keys equal T, how many of those are left
//      out (the lowest positions), and each wave's count of selected and equal keys;
//   D  the survivors are written in position order: wave w starts at the fixed-order sum of
//      the selected counts of waves 0..w-1, lanes are ranked with ballots and mbcnt; a wave
//      that keeps all or none of its keys equal to T decides each key with one comparison.
// If the sample's guess fails (fewer than k survivors, or a region overflows), an exact
// fallback resolves T with histograms over every key and writes from the whole row.  Results
// never depend on which path ran.
//
// Passes read the row from the workspace rows written by the score phase (L2/MALL-resident
// for rows of moderate length).  A row costs about 1.25 reads when the sample's guess holds.
// Lane l of a wave reads keys 64 apart (positions base + 256*s + 64*c + l), so every load is
// a coalesced 256-byte dword load and the keys of a step are in position order c by c; loads
// are range-checked buffer loads (keys past the row read as 0) issued four steps at a time.
// Wave reductions and scans use DPP lane moves.  Output rows are written through
// range-checked buffer stores.  The first workgroup also checks and resets the work-unit
// counter the score kernel left in the control block.

#include "dsa_internal.h"
#include "wave_ops.h"

namespace dsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kHistBits = 10;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandCap = 3072;    // survivors per row held in LDS (256-thread rows)
constexpr int kCandCapWide = 4096;  // the same for 1024-thread rows (16 waves, 256 each)
constexpr int kSegCache = 256;    // segments whose tables are cached in LDS
constexpr int kSampleStride = 4;  // sample = every key of every 4th step (every 8th for 1024-thread rows)
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, range-checked
constexpr int kRankMax = 64;      // a bin with at most this many keys is ranked directly

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = key ^ (~(uint32_t)((int32_t)key >> 31) | 0x80000000u);
  return __uint_as_float(u);
}

// base + the number of set mask bits below this lane
__device__ __forceinline__ uint32_t ballot_rank(uint64_t mask, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, base));
}

__device__ __forceinline__ uint32_t popc(uint64_t mask) { return (uint32_t)__popcll(mask); }

__device__ __forceinline__ uint32_t sub_sat(uint32_t a, uint32_t b) { return __builtin_elementwise_sub_sat(a, b); }


// Segment tables of batches with at most kSegCache segments, cached in LDS by every block.
struct SegCache {
  int32_t cq[kSegCache + 1];
  int32_t ck[kSegCache + 1];
  int32_t off[kSegCache];
};

template <int NT>
__device__ bool cache_segments(const SelectParams& p, SegCache& sc) {
  const bool cached = p.B <= kSegCache;
  if (cached) {
    for (int i = threadIdx.x; i <= p.B; i += NT) {
      sc.cq[i] = p.cu_q[i];
      sc.ck[i] = p.cu_k[i];
      if (i < p.B) sc.off[i] = p.offs ? p.offs[i] : 0;
    }
  }
  return cached;
}

// Visible key count n and first key id kb of row t (both wave-uniform); n = 0 when the call's
// tables are invalid.  The cached tables are read from LDS and the others from global memory on
// separate paths, each value made scalar on its own path: a read through a pointer that may be
// either would be a flat load, whose wait also waits for this wave's outstanding output stores.
__device__ void row_geometry(const SelectParams& p, const SegCache& sc, bool cached, bool bad, int t,
                             int& n_out, int& kb_out) {
  int n = 0, kb = 0;
  if (!bad) {
    auto geometry = [&](auto get) {
      int lo = 0, hi = p.B + 1;  // first segment start beyond t
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (get(0, mid) <= t) lo = mid + 1; else hi = mid;
      }
      const int b = lo - 1;
      if (b >= 0 && b < p.B) {
        const int qb = get(0, b);
        kb = get(1, b);
        const int lk = min(get(1, b + 1) - kb, p.Lmax);
        const int off = get(2, b);
        n = min(max(off + (t - qb) + 1, 0), max(lk, 0));
      }
    };
    if (cached) {
      geometry([&](int which, int i) {
        const int v = which == 0 ? sc.cq[i] : which == 1 ? sc.ck[i] : sc.off[i];
        return __builtin_amdgcn_readfirstlane(v);
      });
    } else {
      geometry([&](int which, int i) {
        const int v = which == 0 ? p.cu_q[i] : which == 1 ? p.cu_k[i] : (p.offs ? p.offs[i] : 0);
        return __builtin_amdgcn_readfirstlane(v);
      });
    }
  }
  n_out = __builtin_amdgcn_readfirstlane(n);  // the same for every lane: keep it scalar
  kb_out = __builtin_amdgcn_readfirstlane(kb);
}

// A row with at most topk visible keys: every key is kept, the rest of the row is padding.  A
// thread's row loads are issued four at a time before their stores.
template <int NT>
__device__ void copy_row(const uint32_t* row, int n, int kb, int topk, int32_t* oid, float* osc) {
  const int tid = threadIdx.x;
  constexpr int kCopyPer = (kMaxTopk + NT - 1) / NT;
  constexpr int kBatch = kCopyPer < 4 ? kCopyPer : 4;
#pragma unroll
  for (int i0 = 0; i0 < kCopyPer; i0 += kBatch) {
    uint32_t kv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = tid + (i0 + i) * NT;
      kv[i] = j < n ? row[j] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int j = tid + (i0 + i) * NT;
      if (j < n) {
        oid[j] = kb + j;
        osc[j] = key_value(kv[i]);
      } else if (j < topk) {
        oid[j] = -1;
        osc[j] = -__builtin_inff();
      }
    }
  }
}

// Block 0: the score kernel drew units + grid tickets; anything else means the counter was not
// zero when it started.  Reset for the next call (this kernel runs after the score kernel).
__device__ void check_reset_counter(const SelectParams& p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (p.ctrl[kCtrlTicket] != p.ctrl[kCtrlExpected]) atomicOr(p.ctrl + kCtrlStatus, kStatusCorruptCounter);
    p.ctrl[kCtrlTicket] = 0u;
    p.ctrl[kCtrlDone] = 0u;
  }
}

template <int NT>
struct alignas(16) Smem {
  static constexpr int NW = NT / 64;
  static constexpr int R = (NT >= 1024 ? kCandCapWide : kCandCap) / NW;  // survivors per wave region
  static_assert(R % 256 == 0, "wave regions are read in steps of 256 entries");
  uint32_t hist[kHistBins];
  uint32_t ckey[NW][R];
  uint16_t cpos[NW][R];
  // per-wave partials: [0] find_bin, [1..3] fallback statistics, [2..3] selected/equal counts,
  // [4..6] sample statistics, [7..8] compaction count and row maximum
  uint32_t wred[NW][12];
  uint32_t bcast[8];
  SegCache seg;
};

// Locate the bin holding rank krem (1-based, from the top) in hist[0..nb): returns
// (bin, count above it, count in it) through bcast.  Thread tid owns bins
// [nb - (tid+1)*per, nb - tid*per).
template <int NT, class SM>
__device__ void find_bin(SM& sm, int nb, uint32_t krem) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = nb >= NT ? nb / NT : 1;
  const int lo = nb - (tid + 1) * per;
  uint32_t local = 0;
  if (lo >= 0) {
    if (per >= 4) {  // contiguous 16-byte reads: lanes cover consecutive bytes, no bank conflicts
      for (int d = 0; d < per; d += 4) {
        const u32x4 h = *reinterpret_cast<const u32x4*>(&sm.hist[lo + d]);
        local += h[0] + h[1] + h[2] + h[3];
      }
    } else {
      for (int d = 0; d < per; ++d) local += sm.hist[lo + d];
    }
  }
  const uint32_t incl = wave_incl_scan(local);
  if (lane == 63) sm.wred[wv][0] = incl;
  __syncthreads();
  uint32_t above = incl - local;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) above += i < wv ? sm.wred[i][0] : 0u;
  if (lo >= 0 && above < krem && krem <= above + local) {
    for (int d = lo + per - 1; d >= lo; --d) {
      const uint32_t h = sm.hist[d];
      if (krem <= above + h) {
        sm.bcast[0] = (uint32_t)d;
        sm.bcast[1] = above;
        sm.bcast[2] = h;
        break;
      }
      above += h;
    }
  }
  __syncthreads();
}

// Row keys seen by one lane: step s of the wave's span covers positions base + 256*s + 64*c + lane
// (c = 0..3), so that for each c the wave reads 256 contiguous bytes and the four keys of a step
// are in position order when taken c by c.  Loads are dword buffer loads range-checked at n keys:
// positions at or past n read as 0, which is below every real key, so no load sits under a branch
// and a batch of loads can be in flight together.
struct Keys {
  __amdgpu_buffer_rsrc_t rs;
  int base, span;

  // f(step s, position of this lane's c = 0 key, keys[4]) for every `stride`-th step of the span,
  // in order (wave-uniform).  Steps are loaded kBatch at a time before any is used.
  template <int kStride = 1, class F>
  __device__ void each(F&& f) const {
    constexpr int kBatch = 4;
    const int lane = threadIdx.x & 63;
    const int steps = span >> 8;
    for (int s = 0; s < steps; s += kBatch * kStride) {
      uint32_t t[kBatch][4];
      // one lane offset per batch; the step and c offsets are instruction immediates when they fit
      int off = (base + 256 * s + lane) * 4;
      asm("" : "+v"(off));  // keeps the offsets as immediates on this base (no loop-carried end pointer)
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          t[u][c] = __builtin_amdgcn_raw_buffer_load_b32(rs, off + 1024 * kStride * u + 256 * c, 0, 0);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s + u * kStride < steps) f(s + u * kStride, base + 256 * (s + u * kStride) + lane, t[u]);
    }
  }
};

// Exact fallback: T from histograms over all keys of the row; returns T and eq_skip, and the
// per-wave counts of keys > T and == T in wred[wv][2], wred[wv][3].
template <int NT, class KS>
__device__ void resolve_all(Smem<NT>& sm, const KS& ks, int topk, uint32_t& T, uint32_t& eq_skip) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t mn = 0xffffffffu, mx = 0u, cnt = 0;
  ks.each([&](int, int, const uint32_t (&k4)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mn = min(mn, k4[c] - 1u);  // invalid (0) wraps to the top and drops out
      mx = max(mx, k4[c]);
      cnt += k4[c] ? 1u : 0u;
    }
  });
  mn = wave_min(mn);
  mx = wave_max(mx);
  cnt = wave_sum(cnt);
  if (lane == 0) {
    sm.wred[wv][1] = mn;
    sm.wred[wv][2] = mx;
    sm.wred[wv][3] = cnt;
  }
  __syncthreads();
  uint32_t valid = 0;
#pragma unroll
  for (int i = 0; i < Smem<NT>::NW; ++i) {
    mn = min(mn, sm.wred[i][1]);
    mx = max(mx, sm.wred[i][2]);
    valid += sm.wred[i][3];
  }
  const uint32_t kmin = mn + 1u;
  const uint32_t range = mx - kmin;
  int shift = range ? 32 - __clz((int)range) : 0;
  uint32_t prefix = 0, krem = (uint32_t)topk, eq_total = valid;  // all equal if no digit left
  bool first = true;
  __syncthreads();
  while (shift > 0) {
    const int bits = min(kHistBits, shift);
    shift -= bits;
    const uint32_t nb = 1u << bits;
    for (int i = tid; i < (int)nb; i += NT) sm.hist[i] = 0u;
    __syncthreads();
    ks.each([&](int, int, const uint32_t (&k4)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t v = k4[c] - kmin;
        if (k4[c] && (first || (uint32_t)((uint64_t)v >> (shift + bits)) == prefix))
          atomicAdd(&sm.hist[(v >> shift) & (nb - 1u)], 1u);
      }
    });
    __syncthreads();
    find_bin<NT>(sm, (int)nb, krem);
    prefix = (prefix << bits) | sm.bcast[0];
    krem -= sm.bcast[1];
    eq_total = sm.bcast[2];
    first = false;
    __syncthreads();
  }
  T = kmin + prefix;
  eq_skip = eq_total - krem;
  uint32_t gt = 0, eq = 0;
  ks.each([&](int, int, const uint32_t (&k4)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      gt += popc(__ballot(k4[c] > T));  // T >= kmin >= 1: padding keys (0) are neither
      eq += popc(__ballot(k4[c] == T));
    }
  });
  if (lane == 0) {
    sm.wred[wv][2] = gt;
    sm.wred[wv][3] = eq;
  }
  __syncthreads();
}

// Output offsets of this wave: selected keys of waves before it, and equal keys before it.
template <int NT, class SM>
__device__ void wave_bases(SM& sm, uint32_t eq_skip, uint32_t& sel_base, uint32_t& eq_base) {
  const int wv = threadIdx.x >> 6;
  sel_base = 0;
  eq_base = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < wv) {
      const uint32_t g_i = sm.wred[i][2], e_i = sm.wred[i][3];
      const uint32_t take = (eq_base + e_i > eq_skip) ? min(e_i, eq_base + e_i - eq_skip) : 0u;
      sel_base += g_i + take;
      eq_base += e_i;
    }
  }
}

// Output row stores: range-checked at topk entries (a store past them is dropped).
struct OutRow {
  __amdgpu_buffer_rsrc_t ids, scores;
  int kb;
  __device__ void put(uint32_t slot, int pos, uint32_t key) const {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(kb + pos), ids, (int)(slot * 4u), 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(key)), scores, (int)(slot * 4u), 0, 0);
  }
};

template <int NT>
__global__ __launch_bounds__(NT, NT == 256 ? 6 : 1) void select_kernel(SelectParams p) {
  constexpr int NW = NT / 64;
  constexpr int R = Smem<NT>::R;
  __shared__ Smem<NT> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int topk = p.topk;
  const bool bad = p.ctrl[kCtrlCallBad] != 0u;  // this call's tables are invalid: all rows padding
  check_reset_counter(p);
  const bool cached = cache_segments<NT>(p, sm.seg);
  __syncthreads();

  for (int t = blockIdx.x; t < p.T; t += gridDim.x) {
    int n, kb;
    row_geometry(p, sm.seg, cached, bad, t, n, kb);
    const uint32_t* const row = p.keys + (int64_t)t * p.ld;
    int32_t* const oid = p.out_ids + (int64_t)t * topk;
    float* const osc = p.out_scores + (int64_t)t * topk;
    if (n <= topk) {  // every visible key is kept; pad the rest
      copy_row<NT>(row, n, kb, topk, oid, osc);
      continue;
    }

    Keys ks;
    ks.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(row), (short)0, n * 4, kRsrcWord3);
    ks.span = ((n + NW * 256 - 1) / (NW * 256)) * 256;
    ks.base = wv * ks.span;
    const int steps = ks.span >> 8;
    OutRow out;
    out.ids = __builtin_amdgcn_make_buffer_rsrc(oid, (short)0, topk * 4, kRsrcWord3);
    out.scores = __builtin_amdgcn_make_buffer_rsrc(osc, (short)0, topk * 4, kRsrcWord3);
    out.kb = kb;

    // ---- A: threshold from a sample: every key of every 4th step of each wave's span --------
    for (int i = tid; i < kHistBins; i += NT) sm.hist[i] = 0u;  // free since the last row's barriers
    // The wave's sample also goes to its (still unused) survivor region when it fits, so the
    // histogram pass below reads it from LDS instead of from the row again.
    // 1024-thread rows (few-row batches) are latency-bound: a sparser sample shortens the wait for
    // the slowest of 16 waves' sample loads, and their 4096 survivor slots hold the wider margin
    constexpr int kSS = NT >= 1024 ? 2 * kSampleStride : kSampleStride;
    const int sample_steps = (steps + kSS - 1) / kSS;
    const bool staged = sample_steps * 256 <= R;
    uint32_t smin = 0xffffffffu, smax = 0u;
    ks.template each<kSS>([&](int s, int, const uint32_t (&k)[4]) {
      if (staged) {
        uint32_t* const st = &sm.ckey[wv][(s / kSS) * 256 + lane];
#pragma unroll
        for (int c = 0; c < 4; ++c) st[64 * c] = k[c];
      }
      smin = min(smin, min(k[0] - 1u, k[1] - 1u));  // invalid (0) wraps to the top and drops out
      smin = min(smin, min(k[2] - 1u, k[3] - 1u));
      smax = max(smax, max(k[0], k[1]));
      smax = max(smax, max(k[2], k[3]));
    });
    smin = wave_min(smin);
    smax = wave_max(smax);
    if (lane == 0) {
      sm.wred[wv][4] = smin;
      sm.wred[wv][5] = smax;
    }
    // sample size: the sampled positions below n (every key below n is a real key)
    uint32_t m = 0;
    for (int w = 0; w < NW; ++w)
      for (int s = 0; s < steps; s += kSS)
        m += (uint32_t)min(max(n - (w * ks.span + 256 * s), 0), 256);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      smin = min(smin, sm.wred[i][4]);
      smax = max(smax, sm.wred[i][5]);
    }
    smin += 1u;
    // sample rank whose bin edge becomes theta: k*m/n plus 4 standard deviations and a margin
    const float expect = (float)topk * (float)m / (float)n;
    const uint32_t r = (uint32_t)(expect + 4.f * __builtin_sqrtf(expect) + 8.f);
    uint32_t theta = 1u;  // every real key is >= 0x007fffff
    if (m >= 64 && r < m && smax > smin) {
      const uint32_t srange = smax - smin;
      const int sbits = 32 - __clz((int)srange);
      const int sshift = max(sbits - kHistBits, 0);
      // invalid keys (0) saturate into bin 0, the lowest: they cannot move the bin of rank r < m
      auto bin_sample = [&](uint32_t k) { atomicAdd(&sm.hist[sub_sat(k, smin) >> sshift], 1u); };
      if (staged) {
        for (int idx = 0; idx < sample_steps; ++idx) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.ckey[wv][idx * 256 + 4 * lane]);
#pragma unroll
          for (int c = 0; c < 4; ++c) bin_sample(v[c]);
        }
      } else {
        ks.template each<kSS>([&](int, int, const uint32_t (&k)[4]) {
#pragma unroll
          for (int c = 0; c < 4; ++c) bin_sample(k[c]);
        });
      }
      __syncthreads();
      find_bin<NT>(sm, kHistBins, r);  // ends with a barrier: the histogram is free afterwards
      theta = smin + (sm.bcast[0] << sshift);
    }

    // ---- B: keys >= theta into this wave's region, in position order ---------------------------
    // the histogram is free again: clear it for the first digit pass over the survivors
    for (int i = tid; i < kHistBins; i += NT) sm.hist[i] = 0u;
    uint32_t run = 0, rmax = 0;
    ks.each([&](int, int pos, const uint32_t (&k)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool keep = k[c] >= theta;
        const uint64_t km = __ballot(keep);
        const uint32_t slot = ballot_rank(km, run);
        if (keep && slot < (uint32_t)R) {
          sm.ckey[wv][slot] = k[c];
          sm.cpos[wv][slot] = (uint16_t)(pos + 64 * c);
        }
        run += popc(km);
      }
      rmax = max(rmax, max(max(k[0], k[1]), max(k[2], k[3])));
    });
    rmax = wave_max(rmax);
    const uint32_t mine = min(run, (uint32_t)R);
    {  // key 0 (below every survivor) in the rest of the last 256-entry step the passes read
      const uint32_t end = min((mine + 255u) & ~255u, (uint32_t)R);
      for (uint32_t i = mine + lane; i < end; i += 64) sm.ckey[wv][i] = 0u;
    }
    if (lane == 0) {
      sm.wred[wv][7] = run;
      sm.wred[wv][8] = rmax;
    }
    if (tid == 0) sm.bcast[3] = 0u;  // gather counter of the direct ranking below
    __syncthreads();
    uint32_t total = 0, cmax = 0;
    bool overflow = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      total += sm.wred[i][7];
      cmax = max(cmax, sm.wred[i][8]);
      overflow |= sm.wred[i][7] > (uint32_t)R;
    }
    // entries i0 + 64c + lane (c = 0..3) of this wave's region, all four read before any is used
    auto cand4 = [&](uint32_t i0, uint32_t (&kk)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) kk[c] = sm.ckey[wv][i0 + 64 * c + lane];
    };

    uint32_t T, eq_skip, sel_base, eq_base;
    if (!overflow && total >= (uint32_t)topk) {
      // ---- C: exact k-th key among the survivors ---------------------------------------------
      // [lo, top] is the key range holding rank krem (from the top) of the survivors, cnt keys.
      // cmax (the row maximum) is a survivor, so [theta, cmax] holds every survivor.  Each
      // digit pass splits the range into 1024 bins and keeps the bin holding rank krem.
      uint32_t lo = theta, top = cmax, krem = (uint32_t)topk, cnt = total;
      bool first = true;
      while (lo != top && (first || cnt > (uint32_t)kRankMax)) {
        const uint32_t width = top - lo;
        const int shift = max(32 - __clz((int)width) - kHistBits, 0);
        if (!first) {  // the first pass uses the histogram cleared during compaction
          for (int i = tid; i < kHistBins; i += NT) sm.hist[i] = 0u;
          __syncthreads();
        }
        for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
          uint32_t kk[4];
          cand4(i0, kk);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t v = kk[c] - lo;  // keys below lo (and padding) wrap past width
            if (v <= width) atomicAdd(&sm.hist[v >> shift], 1u);
          }
        }
        __syncthreads();
        find_bin<NT>(sm, kHistBins, krem);
        const uint32_t b = sm.bcast[0];
        krem -= sm.bcast[1];
        cnt = sm.bcast[2];
        lo += b << shift;
        const uint64_t bin_top = (uint64_t)lo + ((1ull << shift) - 1ull);
        top = bin_top < (uint64_t)top ? (uint32_t)bin_top : top;
        first = false;
      }
      // One pass: per wave, the keys above the bin and in it; when the bin spans several key
      // values (then it holds at most kRankMax keys) its keys are gathered with their wave.
      const bool rank = lo != top;
      const uint32_t width = top - lo;
      uint32_t gtw = 0, inw = 0;
      for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
        uint32_t kk[4];
        cand4(i0, kk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t am = __ballot(kk[c] > top);
          const bool inb = kk[c] - lo <= width;
          const uint64_t bm = __ballot(inb);
          gtw += popc(am);
          inw += popc(bm);
          if (rank && bm) {
            uint32_t g0 = 0;
            if (lane == 0) g0 = atomicAdd(&sm.bcast[3], popc(bm));
            g0 = (uint32_t)__builtin_amdgcn_readlane((int)g0, 0);
            const uint32_t g = ballot_rank(bm, g0);
            if (inb && g < (uint32_t)kRankMax) {
              sm.hist[g] = kk[c];
              sm.hist[kRankMax + g] = (uint32_t)wv;
            }
          }
        }
      }
      if (lane == 0) {
        sm.wred[wv][2] = gtw;
        sm.wred[wv][3] = inw;
      }
      __syncthreads();
      uint32_t eq_total;
      if (rank) {
        // lane i of wave 0 ranks gathered key i against the others; the lane whose rank range
        // holds krem has T.  Per wave: the bin's keys above T join its count above, and its keys
        // equal to T replace its count in the bin.
        if (wv == 0) {
          const uint32_t c = cnt;
          const uint32_t mykey = (uint32_t)lane < c ? sm.hist[lane] : 0u;
          const uint32_t mywv = (uint32_t)lane < c ? sm.hist[kRankMax + lane] : 0xffffffffu;
          // key 0 (below every gathered key) after the last one, so whole 4-key groups are read
          if ((uint32_t)lane < 4u) sm.hist[c + lane] = 0u;
          uint32_t gt = 0, ge = 0;
          for (uint32_t j = 0; j < c; j += 4) {  // every lane reads the same 16 bytes: a broadcast
            const u32x4 o = *reinterpret_cast<const u32x4*>(&sm.hist[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              gt += o[q] > mykey ? 1u : 0u;
              ge += o[q] >= mykey ? 1u : 0u;
            }
          }
          const uint64_t tm = __ballot((uint32_t)lane < c && gt < krem && krem <= ge);
          const int tl = (int)__builtin_ctzll(tm);
          const uint32_t tv = (uint32_t)__builtin_amdgcn_readlane((int)mykey, tl);
          const uint32_t tgt = (uint32_t)__builtin_amdgcn_readlane((int)gt, tl);
          const uint32_t tge = (uint32_t)__builtin_amdgcn_readlane((int)ge, tl);
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const uint32_t g2 = popc(__ballot(mywv == (uint32_t)w && mykey > tv));
            const uint32_t e2 = popc(__ballot(mywv == (uint32_t)w && mykey == tv));
            if (lane == 0) {
              sm.wred[w][2] += g2;
              sm.wred[w][3] = e2;
            }
          }
          if (lane == 0) {
            sm.bcast[4] = tv;
            sm.bcast[5] = tge - tgt;
            sm.bcast[6] = krem - tgt;
          }
        }
        __syncthreads();
        T = sm.bcast[4];
        eq_total = sm.bcast[5];
        krem = sm.bcast[6];
      } else {
        T = lo;
        eq_total = cnt;
      }
      eq_skip = eq_total - krem;
      wave_bases<NT>(sm, eq_skip, sel_base, eq_base);
      // ---- D: ordered write from the survivors ------------------------------------------------
      const uint32_t eq_w = sm.wred[wv][3];
      uint32_t sel_run = sel_base;
      if (eq_w == 0u || eq_base >= eq_skip || eq_base + eq_w <= eq_skip) {
        // this wave keeps all or none of its keys equal to T: one comparison decides
        const uint32_t tc = (eq_w != 0u && eq_base + eq_w <= eq_skip) ? T : T - 1u;  // T >= theta >= 1
        for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
          uint32_t kk[4];
          int pos[4];
          cand4(i0, kk);
#pragma unroll
          for (int c = 0; c < 4; ++c) pos[c] = sm.cpos[wv][i0 + 64 * c + lane];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool self = kk[c] > tc;
            const uint64_t sm_ = __ballot(self);
            if (self) out.put(ballot_rank(sm_, sel_run), pos[c], kk[c]);
            sel_run += popc(sm_);
          }
        }
      } else {
        // keys > T, and the keys equal to T whose rank among the row's equal keys is >= eq_skip
        uint32_t eq_run = eq_base;
        for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
          uint32_t kk[4];
          int pos[4];
          cand4(i0, kk);
#pragma unroll
          for (int c = 0; c < 4; ++c) pos[c] = sm.cpos[wv][i0 + 64 * c + lane];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool eqf = kk[c] == T;
            const uint64_t em = __ballot(eqf);
            const bool self = kk[c] > T || (eqf && ballot_rank(em, eq_run) >= eq_skip);
            const uint64_t sm_ = __ballot(self);
            if (self) out.put(ballot_rank(sm_, sel_run), pos[c], kk[c]);
            eq_run += popc(em);
            sel_run += popc(sm_);
          }
        }
      }
    } else {
      // ---- exact fallback over every key ------------------------------------------------------
      resolve_all<NT>(sm, ks, topk, T, eq_skip);
      wave_bases<NT>(sm, eq_skip, sel_base, eq_base);
      uint32_t eq_run = eq_base, sel_run = sel_base;
      ks.each([&](int, int pos, const uint32_t (&k)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool eqf = k[c] == T;  // T >= 1: padding keys (0) are never equal to it
          const uint64_t em = __ballot(eqf);
          const bool self = k[c] > T || (eqf && ballot_rank(em, eq_run) >= eq_skip);
          const uint64_t sm_ = __ballot(self);
          if (self) out.put(ballot_rank(sm_, sel_run), pos + 64 * c, k[c]);
          eq_run += popc(em);
          sel_run += popc(sm_);
        }
      });
    }
  }
}

}  // namespace

hipError_t select_occupancy(SelectOccupancy* occ) {
  int a = 0, b = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, select_kernel<256>, 256, 0);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, select_kernel<1024>, 1024, 0);
  if (e != hipSuccess) return e;
  occ->narrow = a < 1 ? 1 : a;
  occ->wide = b < 1 ? 1 : b;
  return hipSuccess;
}

hipError_t launch_select(const SelectParams& p, int cus, const SelectOccupancy& occ, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (4 * p.T <= cus) {
    // Few rows (a split tail, a handful of decode queries) leave most CUs idle: give each row
    // 16 waves instead of 4, so its passes over the keys take a quarter of the steps.
    hipLaunchKernelGGL((select_kernel<1024>), dim3(min(p.T, cus * occ.wide * 4)), dim3(1024), 0, s, p);
  } else {
    hipLaunchKernelGGL((select_kernel<256>), dim3(min(p.T, cus * occ.narrow * 4)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace dsa
