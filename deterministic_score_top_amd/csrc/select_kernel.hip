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
//   A  a sample of the row (1/4 of it) gives a threshold theta = lower edge of the sample
//      histogram bin that holds a rank four standard deviations past k*m/n, so that, with
//      overwhelming probability, theta is below the k-th key while only a few hundred keys
//      more than k are >= theta (the sample is kept in LDS for its histogram when it fits);
//   B  one pass compares every key with theta and copies the survivors (key, position) into
//      per-wave LDS regions in position order (ballots + mbcnt, no atomics);
//   C  the exact k-th key T is found over the survivors with range-normalised LDS histograms
//      (digits of up to 10 bits; once the bin holding rank k has at most 64 keys, one wave
//      ranks them directly), together with how many keys equal T and how many of those are
//      left out (the lowest positions);
//   D  the survivors are written in position order: wave w starts at the fixed-order sum of
//      the selected counts of waves 0..w-1, lanes are ranked with ballots and mbcnt.
// If the sample's guess fails (fewer than k survivors, or a region overflows), an exact
// fallback resolves T with histograms over every key and writes from the whole row.  Results
// never depend on which path ran.
//
// Passes read the row from the workspace rows written by the score phase (L2/MALL-resident
// for rows of moderate length).  A row costs about 1.25 reads when the sample's guess holds.
// Wave reductions and scans use DPP lane moves; row loads are range-checked buffer loads
// issued several steps at a time.  The first workgroup also checks and resets the work-unit
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
constexpr int kSampleStride = 4;  // sample = every key of every 4th step
constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data, range-checked

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = key ^ (~(uint32_t)((int32_t)key >> 31) | 0x80000000u);
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive prefix (over lanes) and total of a per-lane count in 0..7.
__device__ __forceinline__ void wave_prefix3(uint32_t cnt, uint32_t& excl, uint32_t& total) {
  const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u);
  excl = lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
  total = (uint32_t)__popcll(b0) + 2u * (uint32_t)__popcll(b1) + 4u * (uint32_t)__popcll(b2);
}


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
// tables are invalid.
__device__ void row_geometry(const SelectParams& p, const SegCache& sc, bool cached, bool bad, int t,
                             int& n_out, int& kb_out) {
  int n = 0, kb = 0;
  if (!bad) {
    const int32_t* cq = cached ? sc.cq : p.cu_q;
    int lo = 0, hi = p.B + 1;  // first segment start beyond t
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (cq[mid] <= t) lo = mid + 1; else hi = mid;
    }
    const int b = lo - 1;
    if (b >= 0 && b < p.B) {
      const int qb = cq[b];
      kb = cached ? sc.ck[b] : p.cu_k[b];
      const int lk = min((cached ? sc.ck[b + 1] : p.cu_k[b + 1]) - kb, p.Lmax);
      const int off = cached ? sc.off[b] : (p.offs ? p.offs[b] : 0);
      n = min(max(off + (t - qb) + 1, 0), max(lk, 0));
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

// Row keys seen by one lane: positions base + 256*s + 4*lane + c of the wave's span, read from
// the row on every pass (the rows stay L2/MALL-resident between passes).  Loads are buffer loads
// range-checked at round_up(n, 4) keys (the row stride is a multiple of 64 keys, so that bound
// stays inside the row): vectors past it read as zero, keys past n inside the last vector are
// masked, so no load sits under a branch and a batch of loads can be in flight together.
struct Keys {
  __amdgpu_buffer_rsrc_t rs;
  int n, base, span;

  __device__ void load4(int pos, uint32_t (&o)[4]) const {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, pos * 4, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = (pos + c < n) ? (uint32_t)v[c] : 0u;
  }
  // f(position of c=0, keys[4]) for every `stride`-th step of the span, in order (wave-uniform).
  // Steps are loaded kBatch at a time before any is used.
  template <class F>
  __device__ void each(F&& f, int stride = 1) const {
    constexpr int kBatch = 4;
    const int lane = threadIdx.x & 63;
    const int steps = span >> 8;
    for (int s = 0; s < steps; s += kBatch * stride) {
      uint32_t t[kBatch][4];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) load4(base + 256 * (s + u * stride) + 4 * lane, t[u]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s + u * stride < steps) f(base + 256 * (s + u * stride) + 4 * lane, t[u]);
    }
  }
};

// Exact fallback: T from histograms over all keys of the row; returns T and eq_skip, and the
// per-wave counts of keys > T and == T in wred[wv][2], wred[wv][3].
template <int NT, class KS>
__device__ void resolve_all(Smem<NT>& sm, const KS& ks, int topk, uint32_t& T, uint32_t& eq_skip) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t mn = 0xffffffffu, mx = 0u, cnt = 0;
  ks.each([&](int, const uint32_t (&k4)[4]) {
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
    ks.each([&](int, const uint32_t (&k4)[4]) {
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
  ks.each([&](int, const uint32_t (&k4)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      gt += (k4[c] && k4[c] > T) ? 1u : 0u;
      eq += (k4[c] && k4[c] == T) ? 1u : 0u;
    }
  });
  gt = wave_sum(gt);
  eq = wave_sum(eq);
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
    ks.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(row), (short)0, ((n + 3) & ~3) * 4,
                                              kRsrcWord3);
    ks.n = n;
    ks.span = ((n + NW * 256 - 1) / (NW * 256)) * 256;
    ks.base = wv * ks.span;

    // ---- A: threshold from a sample: every key of every 4th step of each wave's span --------
    for (int i = tid; i < kHistBins; i += NT) sm.hist[i] = 0u;  // free since the last row's barriers
    // The wave's sample also goes to its (still unused) survivor region when it fits, so the
    // histogram pass below reads it from LDS instead of from the row again.
    const int sample_steps = ((ks.span >> 8) + kSampleStride - 1) / kSampleStride;
    const bool staged = sample_steps * 256 <= R;
    uint32_t smin = 0xffffffffu, smax = 0u, scnt = 0;
    ks.each([&](int pos, const uint32_t (&k4)[4]) {
      if (staged) {
        const int idx = ((pos - ks.base) >> 8) / kSampleStride;  // sampled step of this lane's keys
        *reinterpret_cast<u32x4*>(&sm.ckey[wv][idx * 256 + 4 * lane]) = u32x4{k4[0], k4[1], k4[2], k4[3]};
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        smin = min(smin, k4[c] - 1u);  // invalid (0) wraps to the top and drops out
        smax = max(smax, k4[c]);
        scnt += k4[c] ? 1u : 0u;
      }
    }, kSampleStride);
    smin = wave_min(smin);
    smax = wave_max(smax);
    scnt = wave_sum(scnt);
    if (lane == 0) {
      sm.wred[wv][4] = smin;
      sm.wred[wv][5] = smax;
      sm.wred[wv][6] = scnt;
    }
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      smin = min(smin, sm.wred[i][4]);
      smax = max(smax, sm.wred[i][5]);
      m += sm.wred[i][6];
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
      auto bin_sample = [&](const uint32_t (&k4)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (k4[c]) atomicAdd(&sm.hist[(k4[c] - smin) >> sshift], 1u);
      };
      if (staged) {
        for (int idx = 0; idx < sample_steps; ++idx) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.ckey[wv][idx * 256 + 4 * lane]);
          const uint32_t k4[4] = {v[0], v[1], v[2], v[3]};
          bin_sample(k4);
        }
      } else {
        ks.each([&](int, const uint32_t (&k4)[4]) { bin_sample(k4); }, kSampleStride);
      }
      __syncthreads();
      find_bin<NT>(sm, kHistBins, r);  // ends with a barrier: the histogram is free afterwards
      theta = smin + (sm.bcast[0] << sshift);
    }

    // ---- B: keys >= theta into this wave's region, in position order ---------------------------
    // the histogram is free again: clear it for the first digit pass over the survivors
    for (int i = tid; i < kHistBins; i += NT) sm.hist[i] = 0u;
    uint32_t run = 0, rmax = 0;
    ks.each([&](int pos, const uint32_t (&k4)[4]) {
      uint32_t cnt = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cnt += k4[c] >= theta ? 1u : 0u;
        rmax = max(rmax, k4[c]);
      }
      uint32_t ex, tot;
      wave_prefix3(cnt, ex, tot);
      if (tot) {
        uint32_t slot = run + ex;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (k4[c] >= theta) {
            if (slot < (uint32_t)R) {
              sm.ckey[wv][slot] = k4[c];
              sm.cpos[wv][slot] = (uint16_t)(pos + c);
            }
            ++slot;
          }
        }
      }
      run += tot;
    });
    rmax = wave_max(rmax);
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
    const uint32_t mine = min(run, (uint32_t)R);
    // entries i0 + 64c + lane (c = 0..3) of this wave's region, all four read before any is
    // used; the region holds a whole number of 256-entry steps, so the reads stay inside it
    // (entries at or past `mine` are stale and masked by the callers)
    auto cand4 = [&](uint32_t i0, uint32_t (&kk)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) kk[c] = sm.ckey[wv][i0 + 64 * c + lane];
    };

    uint32_t T, eq_skip, sel_base, eq_base;
    if (!overflow && total >= (uint32_t)topk) {
      // ---- C: exact k-th key among the survivors ---------------------------------------------
      // cmax (the row maximum) is a survivor, so [theta, cmax] spans every survivor
      const uint32_t range = cmax - theta;
      int shift = range ? 32 - __clz((int)range) : 0;
      uint32_t prefix = 0, krem = (uint32_t)topk, eq_total = total;
      bool first = true;
      while (shift > 0) {
        const int bits = min(kHistBits, shift);
        shift -= bits;
        const uint32_t nb = 1u << bits;
        if (!first) {  // the first pass uses the histogram cleared during compaction
          for (int i = tid; i < (int)nb; i += NT) sm.hist[i] = 0u;
          __syncthreads();
        }
        for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
          uint32_t kk[4];
          cand4(i0, kk);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t v = kk[c] - theta;
            if (i0 + 64 * c + lane < mine && (first || (uint32_t)((uint64_t)v >> (shift + bits)) == prefix))
              atomicAdd(&sm.hist[(v >> shift) & (nb - 1u)], 1u);
          }
        }
        __syncthreads();
        find_bin<NT>(sm, (int)nb, krem);
        prefix = (prefix << bits) | sm.bcast[0];
        krem -= sm.bcast[1];
        eq_total = sm.bcast[2];
        first = false;
        if (shift > 0 && eq_total <= 64u) {
          // Few keys left in the bin: rank them directly.  Gather them (any order) and let lane
          // i of wave 0 count how many are greater / greater-or-equal than key i.
          for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
            uint32_t kk[4];
            cand4(i0, kk);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (i0 + 64 * c + lane < mine && ((kk[c] - theta) >> shift) == prefix)
                sm.hist[atomicAdd(&sm.bcast[3], 1u)] = kk[c];
          }
          __syncthreads();
          if (wv == 0) {
            const uint32_t c = eq_total;
            const uint32_t mykey = (uint32_t)lane < c ? sm.hist[lane] : 0u;
            uint32_t gt = 0, ge = 0;
            for (uint32_t j = 0; j < c; ++j) {
              const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mykey, (int)j);
              gt += o > mykey ? 1u : 0u;
              ge += o >= mykey ? 1u : 0u;
            }
            if ((uint32_t)lane < c && gt < krem && krem <= ge) {  // every such lane holds the same key
              sm.bcast[4] = mykey;
              sm.bcast[5] = gt;
              sm.bcast[6] = ge - gt;
            }
          }
          __syncthreads();
          prefix = sm.bcast[4] - theta;
          krem -= sm.bcast[5];
          eq_total = sm.bcast[6];
          shift = 0;
        }
      }
      T = theta + prefix;
      eq_skip = eq_total - krem;
      uint32_t gt = 0, eq = 0;
      for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
        uint32_t kk[4];
        cand4(i0, kk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool live = i0 + 64 * c + lane < mine;
          gt += live && kk[c] > T ? 1u : 0u;
          eq += live && kk[c] == T ? 1u : 0u;
        }
      }
      gt = wave_sum(gt);
      eq = wave_sum(eq);
      if (lane == 0) {
        sm.wred[wv][2] = gt;
        sm.wred[wv][3] = eq;
      }
      __syncthreads();
      wave_bases<NT>(sm, eq_skip, sel_base, eq_base);
      // ---- D: ordered write from the survivors ------------------------------------------------
      uint32_t eq_run = eq_base, sel_run = sel_base;
      for (uint32_t i0 = 0; i0 < mine; i0 += 256) {
        uint32_t kk[4];
        int pos[4];
        cand4(i0, kk);
#pragma unroll
        for (int c = 0; c < 4; ++c) pos[c] = sm.cpos[wv][i0 + 64 * c + lane];
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // entries i0 + 64c + lane: region order
          const bool live = i0 + 64 * c + lane < mine;
          const bool eqf = live && kk[c] == T;
          const bool gtf = live && kk[c] > T;
          const uint64_t eqm = __ballot(eqf);
          const bool self = gtf || (eqf && eq_run + lanes_below(eqm) >= eq_skip);
          const uint64_t selm = __ballot(self);
          const uint32_t slot = sel_run + lanes_below(selm);
          if (self && slot < (uint32_t)topk) {  // exactly topk are selected; the bound is a guard
            oid[slot] = kb + pos[c];
            osc[slot] = key_value(kk[c]);
          }
          eq_run += (uint32_t)__popcll(eqm);
          sel_run += (uint32_t)__popcll(selm);
        }
      }
    } else {
      // ---- exact fallback over every key ------------------------------------------------------
      resolve_all<NT>(sm, ks, topk, T, eq_skip);
      wave_bases<NT>(sm, eq_skip, sel_base, eq_base);
      uint32_t eq_run = eq_base, sel_run = sel_base;
      ks.each([&](int pos, const uint32_t (&k4)[4]) {
        bool eqf[4], gtf[4];
        uint32_t eqc = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          eqf[c] = k4[c] && k4[c] == T;
          gtf[c] = k4[c] && k4[c] > T;
          eqc += eqf[c] ? 1u : 0u;
        }
        uint32_t eq_ex, eq_tot;
        wave_prefix3(eqc, eq_ex, eq_tot);
        bool self[4];
        uint32_t selc = 0;
        uint32_t er = eq_run + eq_ex;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          self[c] = gtf[c] || (eqf[c] && er >= eq_skip);
          er += eqf[c] ? 1u : 0u;
          selc += self[c] ? 1u : 0u;
        }
        uint32_t sel_ex, sel_tot;
        wave_prefix3(selc, sel_ex, sel_tot);
        uint32_t slot = sel_run + sel_ex;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (self[c] && slot < (uint32_t)topk) {
            oid[slot] = kb + pos + c;
            osc[slot] = key_value(k4[c]);
            ++slot;
          }
        }
        eq_run += eq_tot;
        sel_run += sel_tot;
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
