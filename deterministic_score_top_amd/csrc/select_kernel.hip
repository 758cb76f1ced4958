// Top-k select phase of the DSA indexer scan on gfx950.
//
// One workgroup per query row.  The row's visible FP32 scores (written by the score phase)
// are read once into registers as order-preserving 32-bit keys
//     u = bits(score) with -0 -> +0;  key = (u >> 31) ? ~u : (u | 0x80000000)
// so that unsigned key order is score order.  The k-th largest key is found exactly by LDS
// radix-select histograms over the key range [min, max] of the row (11-bit digits, at most 3
// passes); ties at that key are broken toward the larger id, i.e. the later positions of the
// row, as the scan's result rule requires (flashinfer PR #8691, description: ties go to the
// larger id; result independent of partitioning).  Selected keys are gathered in ascending
// id order with wave ballots and mbcnt prefix counts plus per-wave offsets summed in fixed
// wave order -- no atomics decide any output position, so the output is deterministic.
//
// Register layout: wave wv owns row positions [wv*span, (wv+1)*span), span a multiple of 256;
// step m of lane l holds positions wv*span + 256*m + 4*l + 0..3 (one float4 load).

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kHistBins = 2048;
constexpr int kDigitBits = 11;

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

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// Exclusive prefix (over lanes) and total of a per-lane count in 0..7.
__device__ __forceinline__ void wave_prefix3(uint32_t cnt, uint32_t& excl, uint32_t& total) {
  const uint64_t b0 = __ballot(cnt & 1u), b1 = __ballot(cnt & 2u), b2 = __ballot(cnt & 4u);
  excl = lanes_below(b0) + 2u * lanes_below(b1) + 4u * lanes_below(b2);
  total = (uint32_t)__popcll(b0) + 2u * (uint32_t)__popcll(b1) + 4u * (uint32_t)__popcll(b2);
}

__device__ __forceinline__ int find_segment(const int32_t* cu_q, int B, int t) {
  int lo = 0, hi = B + 1;  // first index with cu_q[idx] > t
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (cu_q[mid] <= t) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

template <int NT, int STEPS>
__global__ __launch_bounds__(NT) void select_kernel(SelectParams p) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t wred[NW * 4];
  __shared__ uint32_t bcast[8];

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
    for (int j = tid; j < topk; j += NT) {
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

  // ---- load the row as keys (0 marks "no element": real keys are >= 0x007fffff) -------------
  const int span = ((n + NW * 256 - 1) / (NW * 256)) * 256;
  const int base = wv * span;
  uint32_t key[STEPS][4];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int pos = base + 256 * s + 4 * lane;
    if (256 * s < span && pos < n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + pos);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = (pos + c < n) ? order_key(v[c]) : 0u;
        key[s][c] = kk;
        if (kk) {
          kmin = min(kmin, kk);
          kmax = max(kmax, kk);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) key[s][c] = 0u;
    }
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    wred[wv] = kmin;
    wred[NW + wv] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    kmin = min(kmin, wred[i]);
    kmax = max(kmax, wred[NW + i]);
  }

  // ---- radix select on v = key - kmin over the row's range --------------------------------
  const uint32_t range = kmax - kmin;
  int shift = range ? 32 - __clz((int)range) : 0;  // bits of v still undetermined
  uint32_t prefix = 0;                               // determined high bits of the k-th v
  uint32_t krem = (uint32_t)topk;                    // rank still to find inside the prefix
  uint32_t eq_total = (uint32_t)n;                   // elements equal to the threshold
  while (shift > 0) {
    const int bits = min(kDigitBits, shift);
    shift -= bits;
    const uint32_t nb = 1u << bits;
    for (int i = tid; i < (int)nb; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t kk = key[s][c];
        if (kk) {
          const uint32_t v = kk - kmin;
          if ((uint32_t)((uint64_t)v >> (shift + bits)) == prefix)
            atomicAdd(&hist[(v >> shift) & (nb - 1u)], 1u);
        }
      }
    __syncthreads();
    // suffix counts from the top bin down: thread tid owns bins [hi - per, hi) with hi = nb - tid*per
    const int per = ((int)nb + NT - 1) / NT;
    const int hi = (int)nb - tid * per;
    const int lo = max(hi - per, 0);
    uint32_t local = 0;
    for (int d = hi - 1; d >= lo; --d) local += hist[d];
    uint32_t incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wred[wv] = incl;
    __syncthreads();
    uint32_t above = incl - local;
    for (int i = 0; i < wv; ++i) above += wred[i];
    if (hi > 0 && above < krem && krem <= above + local) {
      for (int d = hi - 1; d >= lo; --d) {
        const uint32_t h = hist[d];
        if (krem <= above + h) {
          bcast[0] = (uint32_t)d;
          bcast[1] = above;
          bcast[2] = h;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
    prefix = (prefix << bits) | bcast[0];
    krem -= bcast[1];
    eq_total = bcast[2];
    __syncthreads();
  }
  const uint32_t thr = kmin + prefix;            // key of the k-th largest element
  const uint32_t eq_skip = eq_total - krem;      // equal elements (lowest ids first) left out

  // ---- per-wave counts: equal to thr, greater than thr ----------------------------------------
  uint32_t eq_w = 0, gt_w = 0;
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kk = key[s][c];
      eq_w += (kk && kk == thr) ? 1u : 0u;
      gt_w += (kk && kk > thr) ? 1u : 0u;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    eq_w += (uint32_t)__shfl_xor((int)eq_w, o, 64);
    gt_w += (uint32_t)__shfl_xor((int)gt_w, o, 64);
  }
  if (lane == 0) {
    wred[2 * NW + wv] = eq_w;
    wred[3 * NW + wv] = gt_w;
  }
  __syncthreads();
  uint32_t eq_base = 0, sel_base = 0;
  for (int i = 0; i < wv; ++i) {
    const uint32_t e_i = wred[2 * NW + i], g_i = wred[3 * NW + i];
    const uint32_t take = (eq_base + e_i > eq_skip) ? min(e_i, eq_base + e_i - eq_skip) : 0u;
    sel_base += g_i + take;
    eq_base += e_i;
  }

  // ---- ordered gather --------------------------------------------------------------------
  uint32_t eq_run = eq_base, sel_run = sel_base;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (256 * s >= span) break;
    uint32_t eqc = 0;
    bool eqf[4], gtf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kk = key[s][c];
      eqf[c] = kk && kk == thr;
      gtf[c] = kk && kk > thr;
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
    const int pos = base + 256 * s + 4 * lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (self[c] && slot < (uint32_t)topk) {  // exactly topk are selected; the bound is a guard
        oid[slot] = kb + pos + c;
        osc[slot] = key_value(key[s][c]);
        ++slot;
      }
    }
    eq_run += eq_tot;
    sel_run += sel_tot;
  }
}

template <int NT, int STEPS>
hipError_t launch_variant(const SelectParams& p, hipStream_t s) {
  hipLaunchKernelGGL((select_kernel<NT, STEPS>), dim3(p.T), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  if (p.Lmax <= 8192) return launch_variant<256, 8>(p, s);
  if (p.Lmax <= 16384) return launch_variant<512, 8>(p, s);
  if (p.Lmax <= 32768) return launch_variant<1024, 8>(p, s);
  return launch_variant<1024, 16>(p, s);
}

}  // namespace dsa
