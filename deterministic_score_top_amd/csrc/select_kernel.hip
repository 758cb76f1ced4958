// Top-k select phase of the DSA indexer scan on gfx950.
//
// One workgroup per query row.  Scores are compared as order-preserving 32-bit keys
//     u = bits(score) with -0 -> +0;  key = (u >> 31) ? ~u : (u | 0x80000000)
// so that unsigned key order is score order.  The result rule of the scan (flashinfer
// PR #8691, description: top-k key ids per query, ties go to the larger id, result independent
// of partitioning) is the total order (key descending, position descending) on the row; the
// k-th element of that order is found exactly:
//   pass 1 (row read): LDS histogram of the top 12 key bits -> bin d1 holding the k-th key;
//   pass 2 (row read): every wave copies the keys of its span that fall in bin d1 into its own
//          LDS region and counts its keys above the bin;
//   LDS: two 10-bit digit histograms over the copied keys give the exact threshold key T, the
//        number of keys equal to T and how many of them are left out (the lowest positions);
//   pass 3 (row read): ordered write.  Wave w owns the contiguous span [w*S, (w+1)*S) of the
//          row; its output offset is the sum of the selected counts of waves 0..w-1, and inside
//          the wave positions are ranked with ballots and mbcnt.  No atomic decides any output
//          position, so the output (ids ascending) is deterministic.
// If a wave's copy region overflows, digits 2 and 3 are found with further row passes instead.
// The row is read from the workspace rows written by the score phase (L2/MALL-resident after
// the first pass).

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBits1 = 12;                 // first digit: key bits 31..20
constexpr int kBins1 = 1 << kBits1;
constexpr int kBits2 = 10;                 // second digit: key bits 19..10
constexpr int kBits3 = 10;                 // third digit: key bits 9..0
constexpr int kRegion = 512;               // copied keys per wave

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
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

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}

__device__ __forceinline__ int find_segment(const int32_t* cu_q, int B, int t) {
  int lo = 0, hi = B + 1;  // first index with cu_q[idx] > t
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= t) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

// Four keys at row positions pos..pos+3 (0 = no element past n).  pos is a multiple of 4 and
// below n; the row stride is a multiple of 64 floats, so the 16-byte load stays inside the row.
__device__ __forceinline__ void load4(const float* row, int pos, int n, uint32_t (&k)[4]) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(row + pos);
#pragma unroll
  for (int c = 0; c < 4; ++c) k[c] = (pos + c < n) ? order_key(v[c]) : 0u;
}

struct Smem {
  uint32_t hist[kBins1];
  uint32_t region[kSelWaves][kRegion];
  uint32_t wsum[kSelWaves][4];
  uint32_t bcast[8];
};

// Locate the bin holding rank `krem` (1-based, counted from the top) in hist[0..nb).
// Writes bcast[0] = bin, bcast[1] = count above the bin, bcast[2] = count in the bin.
__device__ void find_bin(Smem& sm, int nb, uint32_t krem) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  const int hi = nb - tid * per;          // this thread owns bins [lo, hi), from the top down
  const int lo = max(hi - per, 0);
  uint32_t local = 0;
  for (int d = hi - 1; d >= lo; --d) local += sm.hist[d];
  uint32_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sm.wsum[wv][0] = incl;
  __syncthreads();
  uint32_t above = incl - local;
  for (int i = 0; i < wv; ++i) above += sm.wsum[i][0];
  if (hi > 0 && above < krem && krem <= above + local) {
    for (int d = hi - 1; d >= lo; --d) {
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

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int t = blockIdx.x;
  const int topk = p.topk;
  int32_t* const oid = p.out_ids + (int64_t)t * topk;
  float* const osc = p.out_scores + (int64_t)t * topk;

  int n = 0, kb = 0;
  if (!(p.ctrl[kCtrlStatus] & kStatusBadSegments)) {
    const int b = find_segment(p.cu_q, p.B, t);
    if (b >= 0 && b < p.B) {
      const int cq = p.cu_q[b];
      const int lk = min(p.cu_k[b + 1] - p.cu_k[b], p.Lmax);
      const int off = p.offs ? p.offs[b] : 0;
      kb = p.cu_k[b];
      n = min(max(off + (t - cq) + 1, 0), max(lk, 0));
    }
  }
  const float* const row = p.scores + (int64_t)t * p.ld;

  if (n <= topk) {  // every visible key is kept; pad the rest
    for (int j = tid; j < topk; j += kSelThreads) {
      if (j < n) {
        oid[j] = kb + j;
        osc[j] = key_value(order_key(row[j]));
      } else {
        oid[j] = -1;
        osc[j] = -__builtin_inff();
      }
    }
    return;
  }

  // wave spans: [wv*span, wv*span + span), span a multiple of 256, lane owns 4 consecutive
  const int span = ((n + kSelWaves * 256 - 1) / (kSelWaves * 256)) * 256;
  const int base = wv * span;
  const int wend = min(base + span, n);

  // ---- pass 1: histogram of the top 12 key bits ---------------------------------------------
  for (int i = tid; i < kBins1; i += kSelThreads) sm.hist[i] = 0u;
  __syncthreads();
  for (int pos0 = base; pos0 < wend; pos0 += 256) {
    const int pos = pos0 + 4 * lane;
    uint32_t k4[4] = {0u, 0u, 0u, 0u};
    if (pos < n) load4(row, pos, n, k4);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (k4[c]) atomicAdd(&sm.hist[k4[c] >> (32 - kBits1)], 1u);
  }
  __syncthreads();
  find_bin(sm, kBins1, (uint32_t)topk);
  const uint32_t d1 = sm.bcast[0];
  uint32_t krem = (uint32_t)topk - sm.bcast[1];
  const uint32_t in_bin1 = sm.bcast[2];

  // ---- pass 2: copy the keys of bin d1 into this wave's region; count keys above the bin ----
  uint32_t above_w = 0, ncopy = 0;
  for (int pos0 = base; pos0 < wend; pos0 += 256) {
    const int pos = pos0 + 4 * lane;
    uint32_t k4[4] = {0u, 0u, 0u, 0u};
    if (pos < n) load4(row, pos, n, k4);
    uint32_t cnt = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t dg = k4[c] >> (32 - kBits1);
      above_w += (k4[c] && dg > d1) ? 1u : 0u;
      cnt += (k4[c] && dg == d1) ? 1u : 0u;
    }
    uint32_t ex, tot;
    wave_prefix3(cnt, ex, tot);
    uint32_t slot = ncopy + ex;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (k4[c] && (k4[c] >> (32 - kBits1)) == d1) {
        if (slot < (uint32_t)kRegion) sm.region[wv][slot] = k4[c];
        ++slot;
      }
    }
    ncopy += tot;
  }
  above_w = wave_sum(above_w);
  if (lane == 0) sm.wsum[wv][1] = ncopy;
  __syncthreads();
  bool overflow = false;
  for (int i = 0; i < kSelWaves; ++i) overflow |= sm.wsum[i][1] > (uint32_t)kRegion;
  __syncthreads();

  // ---- digits 2 and 3: from the copied keys, or by further row passes on overflow ------------
  uint32_t prefix = d1;
  uint32_t eq_total = in_bin1;
  int shift = 32 - kBits1;
#pragma unroll
  for (int dg = 0; dg < 2; ++dg) {
    const int bits = dg == 0 ? kBits2 : kBits3;
    shift -= bits;
    const uint32_t nb = 1u << bits;
    for (int i = tid; i < (int)nb; i += kSelThreads) sm.hist[i] = 0u;
    __syncthreads();
    if (!overflow) {
      const uint32_t m = min(sm.wsum[wv][1], (uint32_t)kRegion);
      for (uint32_t i = lane; i < m; i += 64) {
        const uint32_t kk = sm.region[wv][i];
        if ((kk >> (shift + bits)) == prefix) atomicAdd(&sm.hist[(kk >> shift) & (nb - 1u)], 1u);
      }
    } else {
      for (int pos = base + 4 * lane; pos < wend; pos += 256) {
        uint32_t k4[4];
        load4(row, pos, n, k4);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (k4[c] && (k4[c] >> (shift + bits)) == prefix)
            atomicAdd(&sm.hist[(k4[c] >> shift) & (nb - 1u)], 1u);
      }
    }
    __syncthreads();
    find_bin(sm, (int)nb, krem);
    prefix = (prefix << bits) | sm.bcast[0];
    krem -= sm.bcast[1];
    eq_total = sm.bcast[2];
    __syncthreads();
  }
  const uint32_t thr = prefix;                 // key of the k-th element
  const uint32_t eq_skip = eq_total - krem;    // keys equal to thr left out (lowest positions)

  // ---- per-wave counts of keys above thr and equal to thr ------------------------------------
  uint32_t gt_w = 0, eq_w = 0;
  if (!overflow) {
    const uint32_t m = sm.wsum[wv][1];
    for (uint32_t i = lane; i < m; i += 64) {
      const uint32_t kk = sm.region[wv][i];
      gt_w += kk > thr ? 1u : 0u;
      eq_w += kk == thr ? 1u : 0u;
    }
    gt_w = wave_sum(gt_w) + above_w;
  } else {
    for (int pos = base + 4 * lane; pos < wend; pos += 256) {
      uint32_t k4[4];
      load4(row, pos, n, k4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        gt_w += (k4[c] && k4[c] > thr) ? 1u : 0u;
        eq_w += (k4[c] && k4[c] == thr) ? 1u : 0u;
      }
    }
    gt_w = wave_sum(gt_w);
  }
  eq_w = wave_sum(eq_w);
  if (lane == 0) {
    sm.wsum[wv][2] = gt_w;
    sm.wsum[wv][3] = eq_w;
  }
  __syncthreads();
  uint32_t eq_base = 0, sel_base = 0;
  for (int i = 0; i < wv; ++i) {
    const uint32_t g_i = sm.wsum[i][2], e_i = sm.wsum[i][3];
    const uint32_t take = (eq_base + e_i > eq_skip) ? min(e_i, eq_base + e_i - eq_skip) : 0u;
    sel_base += g_i + take;
    eq_base += e_i;
  }

  // ---- pass 3: ordered write ----------------------------------------------------------------
  uint32_t eq_run = eq_base, sel_run = sel_base;
  for (int pos0 = base; pos0 < wend; pos0 += 256) {
    const int pos = pos0 + 4 * lane;
    uint32_t k4[4] = {0u, 0u, 0u, 0u};
    if (pos < n) load4(row, pos, n, k4);
    bool eqf[4], gtf[4];
    uint32_t eqc = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      eqf[c] = k4[c] && k4[c] == thr;
      gtf[c] = k4[c] && k4[c] > thr;
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
      if (self[c] && slot < (uint32_t)topk) {  // exactly topk are selected; the bound is a guard
        oid[slot] = kb + pos + c;
        osc[slot] = key_value(k4[c]);
        ++slot;
      }
    }
    eq_run += eq_tot;
    sel_run += sel_tot;
  }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3(p.T), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
