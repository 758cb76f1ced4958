// Backward of the indexer scores on gfx950 (CDNA4): dq, dk and dw from the upstream gradient
// g[t, j] = dL/dI[t, s] of every visible (query t, key s = first_t + j) pair.
//
// With S[t, h, s] = q[t, h, :] . k[s, :] and the score I[t, s] = sum_h w[t, h] * max(0, S):
//     dw[t, h]    = sum_s g * max(0, S)
//     dq[t, h, :] = w[t, h] * sum_s g * [S > 0] * k[s, :]
//     dk[s, :]    = sum_t sum_h w[t, h] * g * [S > 0] * q[t, h, :]
// (flashinfer PR #8691, the vendoring commit message: the deterministic package carries the
// lightning-indexer logits kernels and their backward, with no floating-point atomics and
// the key-side gradient reduced from FP32 partials in a fixed tree.)  The derivative of the
// ReLU at exactly 0 is 0.
//
// Three kernels, no atomics on any gradient, every sum in a fixed order:
//   * dq/dw kernel, query-major: a unit is 4 consecutive queries of one segment (and, when
//     there are few queries, one of P even shares of their key tiles); wave w takes
//     query w/2 and heads 32*(w%2) .. +31.  Key tiles land in LDS two ahead (three buffers,
//     one barrier per tile).  Per 64-key tile it recomputes S^T = K . Q^T
//     (v_mfma_f32_32x32x16_bf16, K tile from LDS, Q in VGPRs), forms dw partials in FP32 and
//     the BF16 operand G' = g * [S > 0] (w is factored out of the key sum and applied once at
//     the end), and accumulates dq += G' . K with the K operand read key-major from the same
//     LDS tile by ds_read_b64_tr_b16.
//   * dk kernel, key-major: a unit is (a block of 256 keys, one of P parts of the queries that
//     see its first key); wave w owns keys 32*w .. +31 of the block and all 8 waves walk the
//     part's queries together, one query per step.  Per query: S = Q . K^T (K in VGPRs for
//     the whole unit, Q from LDS), the BF16 operand G'' = w * g * [S > 0], and
//     dk^T += Q^T . G'' with the Q^T operand read head-major from LDS by ds_read_b64_tr_b16.
//     A query's 16 KiB q block thus serves 256 keys per load; queries land in LDS two ahead
//     (three separate LDS arrays, so the compiler does not wait for the prefetch before reading
//     the current query), and the unit's sums leave through LDS one 32-dim block at a time as
//     16-byte row stores.  P (1, 2, 4, 8 or 16) depends
//     only on the number of keys: enough parts for about 512 units.  With P = 1 the unit
//     writes dk itself; otherwise it writes an FP32 partial.
//   * reduce kernels (P > 1): dk = the P partials added in a fixed pairwise tree
//     ((P0 + P1) + (P2 + P3)) + ...; likewise dq and dw when few query tiles leave room for
//     splitting each tile's keys over P units (P from the number of queries only; w is applied
//     after the tree).
//
// MFMA layout used throughout (32x32x16 BF16): operand lane l carries row/column l % 32 and
// K elements 8 * (l / 32) .. +7; accumulator register i of lane l holds row
// 8 * (i / 4) + 4 * (l / 32) + i % 4, column l % 32.  An accumulator used as the next MFMA's
// operand therefore contributes, for K step st and lane half hf, the rows
// 16 * st + 4 * hf + {0..3} and 16 * st + 8 + 4 * hf + {0..3}; the transposed LDS reads fetch
// exactly those rows of the other operand, so both sides of each product agree on the K order.
//
// ds_read_b64_tr_b16 (measured lane layout): in each group of 16 lanes, lane 4*j + r points
// at 4 consecutive 16-bit elements; lane 4*r + e receives element e of lanes r, 4+r, 8+r and
// 12+r.  With lane 4*j + r pointing at row k0 + j, columns c0 + 4*r .. +3, lane i of the group
// receives column c0 + i of rows k0 .. k0+3.

#include <type_traits>

#include "dsa_internal.h"
#include "wave_ops.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWavesB = kBwdThreads / 64;
constexpr int kTileBytes = kBwdKeyTile * kDim * 2;  // 16 KiB of keys (or of one query's q)
constexpr int kRowBytes = kDim * 2;                 // one key row / one head row: 256 B
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kWaitVm = 0x0F70;  // s_waitcnt: wait on the vector memory counter only

// dq/dw kernel LDS stage: key tile + one 64-key gradient row segment per wave
constexpr int kDqStageBytes = kTileBytes + kWavesB * 256;
constexpr int kStages = 3;
// dk kernel LDS stage: q of one query, the gradients of the unit's keys, w, and a landing
// area for the waves that have no third load
constexpr int kDkStageBytes = kTileBytes + kDkKeys * 4 + 256 + 256;
constexpr int kScratchInts = 16;
// dk output: per wave and value block of 32 dims, 32 key rows of 36 floats (16-byte aligned rows,
// at most two lanes per bank when a wave writes one dim of its 32 keys)
constexpr int kDkOutRow = 36;
constexpr int kDkOutWave = 32 * kDkOutRow * 4;
constexpr int kDkStageArray = kDkStageBytes > 4 * kDkOutWave ? kDkStageBytes : 4 * kDkOutWave;

static_assert(kBwdThreads == 512 && kBwdKeyTile == 64, "layout assumes 8 waves and 64-key tiles");
template <int V>
using Int = std::integral_constant<int, V>;

// The dk kernel's stages are separate LDS arrays used with compile-time indices (the stage loop
// is unrolled by three): the compiler can then tell that the loads into one stage do not write
// the stage being read, and does not wait for the prefetched query before reading the current
// one.
__shared__ __align__(16) unsigned char g_dk0[kDkStageArray];
__shared__ __align__(16) unsigned char g_dk1[kDkStageArray];
__shared__ __align__(16) unsigned char g_dk2[kDkStageArray];
__shared__ __align__(16) int g_dk_scratch[kScratchInts];
template <int S>
__device__ __forceinline__ unsigned char* dk_stage() {
  return S == 0 ? g_dk0 : S == 1 ? g_dk1 : g_dk2;
}
static_assert(kDkKeys == 32 * kWavesB, "32 keys per wave in the dk kernel");

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }
__device__ __forceinline__ int clampi(int64_t x, int lo, int hi) {
  return (int)(x < lo ? lo : (x > hi ? hi : x));
}
// g where S > 0 (as int32 the bits of a positive float are positive; +0, -0 and negatives are not)
__device__ __forceinline__ float pass_pos(float s, float g) { return __float_as_int(s) > 0 ? g : 0.f; }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_b128(const unsigned char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Two transposed 4-row reads -> one 8-element operand (rows k0..k0+3, then k0+8..k0+11).
__device__ __forceinline__ bf16x8 lds_tr_pair(const unsigned char* p1, const unsigned char* p2) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p1));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p2));
  const i16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Accumulator registers 8*jj .. 8*jj+7 as a BF16 operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int jj) {
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[8 * jj + e];
  return __builtin_convertvector(v, bf16x8);
}

// sched_group_barrier instruction classes
constexpr int kSgMfma = 0x008, kSgValu = 0x002, kSgDsRead = 0x100;
#define DSA_SGB(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, voff, 0, 0, 0);
}

// 16-byte chunk swizzle of a 64-row x 256-byte LDS tile: the chunk index is XORed with the
// row's low 4 bits rotated by two (bits 0-1 to 2-3, bits 2-3 to 0-1).  It is a bijection on
// any 16 consecutive rows, so a 16-byte read of one chunk from 16 rows hits 16 different
// chunk positions (no bank conflict), and the 4 consecutive rows of a transposed read
// (row & 3 = 0..3) move its 4 adjacent chunks into 4 different 64-byte groups.  (Plain
// row & 15 leaves those 4 rows in one group: a 4-way conflict on every transposed read.)
__device__ __forceinline__ int swzbits(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
// Byte offset of 16-byte chunk `chunk` of row `row`.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ swzbits(row)) << 4); }

// Validates the segment tables (every thread of the block gets the flags): bit 0 = bad tables,
// bit 1 = a segment longer than Lmax.  Block 0 records them in the control block.
__device__ int table_flags(const BwdParams& p, int* scratch) {
  const int tid = threadIdx.x;
  if (tid == 0) scratch[10] = 0;
  __syncthreads();
  int flags = 0;
  for (int b = tid; b <= p.B; b += kBwdThreads) {
    const int cq = p.cu_q[b], ck = p.cu_k[b];
    if (b == 0 && (cq != 0 || ck != 0)) flags |= 1;
    if (b == p.B && (cq != p.T || ck != p.Tkv)) flags |= 1;
    if (b < p.B) {
      const int lq = p.cu_q[b + 1] - cq, lk = p.cu_k[b + 1] - ck;
      if (lq < 0 || lk < 0) flags |= 1;
      if (lk > p.Lmax) flags |= 2;
    }
  }
  if (flags) atomicOr(&scratch[10], flags);
  __syncthreads();
  flags = scratch[10];
  if (blockIdx.x == 0 && tid == 0) {
    // this call's verdict for the reduce kernels that follow (always overwritten); the status
    // word is sticky and only reports
    p.ctrl[kCtrlCallBad] = (flags & 1) ? 1u : 0u;
    if (flags)
      atomicOr(p.ctrl + kCtrlStatus, ((flags & 1) ? kStatusBadSegments : 0u) | ((flags & 2) ? kStatusSeqlenBound : 0u));
  }
  return flags;
}

// Segment b and index inside it of unit u, units numbered segment by segment with count(b)
// units in segment b; b = -1 if u is past the last unit.
template <class CountFn>
__device__ int locate_unit(int B, uint32_t u, CountFn count, int* scratch, int* idx) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    scratch[8] = -1;
    scratch[9] = 0;
  }
  uint32_t carry = 0;
  for (int base = 0; base < B; base += kBwdThreads) {
    const int b = base + tid;
    const uint32_t c = b < B ? count(b) : 0u;
    const uint32_t inc = wave_incl_scan(c);
    __syncthreads();
    if (lane == 63) scratch[wv] = (int)inc;
    __syncthreads();
    uint32_t before = carry, total = carry;
#pragma unroll
    for (int i = 0; i < kWavesB; ++i) {
      const uint32_t x = (uint32_t)scratch[i];
      before += i < wv ? x : 0u;
      total += x;
    }
    const uint32_t ex = before + inc - c;
    if (c > 0 && u >= ex && u < ex + c) {
      scratch[8] = b;
      scratch[9] = (int)(u - ex);
    }
    carry = total;
  }
  __syncthreads();
  *idx = scratch[9];
  return scratch[8];
}

// ------------------------------------------------------------------------------------------
// dq / dw
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* const scratch = reinterpret_cast<int*>(smem + kStages * kDqStageBytes);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = wv >> 1, hg = wv & 1;
  const int n = lane & 31, hf = lane >> 5;

  if (table_flags(p, scratch) & 1) return;
  int idx = 0;
  const int parts = p.dq_parts;
  const int b = locate_unit(p.B, blockIdx.x, [&](int s) -> uint32_t {
    const int lq = p.cu_q[s + 1] - p.cu_q[s];
    return (uint32_t)(ceil_div(lq, kDqQueries) * parts);
  }, scratch, &idx);
  if (b < 0) return;

  const int cq = p.cu_q[b], lq = p.cu_q[b + 1] - cq;
  const int ck = p.cu_k[b], lk = min(p.cu_k[b + 1] - ck, p.Lmax);
  const int64_t off = p.offs ? p.offs[b] : 0;
  const int ti = ceil_div(lq, kDqQueries) - 1 - idx / parts;   // most visible keys first
  const int part = idx % parts;
  const int tq0 = ti * kDqQueries;
  const int nq = min(kDqQueries, lq - tq0);
  const int nmax = clampi(off + tq0 + nq, 0, lk);
  // this unit's share of the tile's key tiles: [kt0, kt0 + ntk)
  const int ntk_all = ceil_div(nmax, kBwdKeyTile);
  const int kt0 = (int)((int64_t)part * ntk_all / parts);
  const int ntk = (int)((int64_t)(part + 1) * ntk_all / parts) - kt0;
  const bool qvalid = qi < nq;
  const int64_t t = (int64_t)cq + tq0 + min(qi, nq - 1);
  const int nt = __builtin_amdgcn_readfirstlane(qvalid ? clampi(off + tq0 + qi + 1, 0, lk) : 0);

  // B operand of S^T = K . Q^T: column = head 32*hg + n, K elements d = 16*j + 8*hf .. +7
  bf16x8 qf[8];
  {
    const uint16_t* qrow = p.q + (t * kHeads + 32 * hg + n) * kDim + 8 * hf;
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[j] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * j) : bf16x8{};
  }

  // keys at or past the segment's (bounded) end read as zero; gradients past the query's
  // visible count read as zero, which masks every invisible pair
  const __amdgpu_buffer_rsrc_t krs = rsrc(p.k + (int64_t)ck * kDim, lk * kRowBytes);
  const __amdgpu_buffer_rsrc_t grs = rsrc(p.grad + t * p.ld, nt * 4);
  auto stage = [&](int s) { return smem + s * kDqStageBytes; };
  auto load_tile = [&](int s, int kt) {
    unsigned char* const dst = stage(s);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int id = r * kWavesB + wv;
      const int row = 4 * id + (lane >> 4), pos = lane & 15;
      lds_load16(krs, dst + id * 1024, ((kt0 + kt) * kBwdKeyTile + row) * kRowBytes + ((pos ^ swzbits(row)) << 4));
    }
    lds_load4(grs, dst + kTileBytes + wv * 256, ((kt0 + kt) * kBwdKeyTile + lane) * 4);
  };
  constexpr int kLoadsPerTile = 3;

  // transposed-read offsets of the K operand of dq += G' . K: lane 4*jr + r of 16-lane group
  // G reads rows 4*hf + jr (+8) and columns 32*nb + 16*(G&1) + 4*r .. +3
  int trk1[4], trk2[4];
  {
    const int L = lane & 15, jr = L >> 2, r = L & 3, gs = (lane >> 4) & 1;
    const int row1 = 4 * hf + jr, row2 = 8 + 4 * hf + jr;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int chunk = 4 * nb + 2 * gs + (r >> 1);
      trk1[nb] = swz(row1, chunk) + 8 * (r & 1);
      trk2[nb] = swz(row2, chunk) + 8 * (r & 1);
    }
  }

  // per-lane offsets of the row-major K reads: row n, chunk 2*j + hf (row 32 + n is 8 KiB on)
  int nat[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) nat[j] = swz(n, 2 * j + hf);

  f32x16 dqa[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) dqa[nb] = f32x16{};
  float dwa = 0.f;

  // Epilogue of one S^T row block (16 keys of this lane's head in registers): G' = g where
  // S > 0, else 0; dw += G' * S (equal to g * max(S, 0) bit for bit); G' packed to BF16 as
  // the A operand of two K steps.  Key of register i: 32*rb + 8*(i/4) + 4*hf + i%4.
  auto epilogue = [&](f32x16& sv, const float* gb, int rb, bf16x8& lo, bf16x8& hi) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 gv = *reinterpret_cast<const f32x4*>(gb + 32 * rb + 8 * g4 + 4 * hf);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float e = sv[4 * g4 + c];
        const float gp = pass_pos(e, gv[c]);
        dwa = __builtin_fmaf(gp, e, dwa);
        sv[4 * g4 + c] = gp;
      }
    }
    lo = pack8(sv, 0);
    hi = pack8(sv, 1);
  };

  // One key tile from the LDS stage `kb` (a constant offset after inlining).  Phases: S^T rows
  // 0..31; rows 32..63 with the epilogue of rows 0..31 between the MFMAs; dq K steps 0, 1 with
  // the epilogue of rows 32..63; dq K steps 2, 3.
  auto tile = [&](const unsigned char* kb) {
    const float* const gb = reinterpret_cast<const float*>(kb + kTileBytes + wv * 256);
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int j = 0; j < 8; ++j) s0 = mfma(lds_b128(kb + nat[j]), qf[j], s0);
#pragma unroll
    for (int j = 0; j < 8; ++j) s1 = mfma(lds_b128(kb + nat[j] + 32 * kRowBytes), qf[j], s1);
    bf16x8 ga[4];
    epilogue(s0, gb, 0, ga[0], ga[1]);
    DSA_SGB(kSgDsRead, 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      DSA_SGB(kSgMfma, 1);
      DSA_SGB(kSgValu, 7);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        dqa[nb] = mfma(ga[st], lds_tr_pair(kb + st * 16 * kRowBytes + trk1[nb], kb + st * 16 * kRowBytes + trk2[nb]),
                       dqa[nb]);
    epilogue(s1, gb, 1, ga[2], ga[3]);
    DSA_SGB(kSgDsRead, 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      DSA_SGB(kSgMfma, 1);
      DSA_SGB(kSgValu, 7);
    }
#pragma unroll
    for (int st = 2; st < 4; ++st)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        dqa[nb] = mfma(ga[st], lds_tr_pair(kb + st * 16 * kRowBytes + trk1[nb], kb + st * 16 * kRowBytes + trk2[nb]),
                       dqa[nb]);
  };
  // tile kt from stage c: first the load of tile kt + 2 into the stage every wave finished
  // reading before the last barrier, then the tile, then wait for tile kt + 1 and meet
  auto step = [&](int c, int kt) {
    if (kt + 2 < ntk) load_tile((c + 2) % kStages, kt + 2);
    tile(stage(c));
    if (kt + 2 < ntk) __builtin_amdgcn_s_waitcnt(kWaitVm | kLoadsPerTile);
    else __builtin_amdgcn_s_waitcnt(kWaitVm);
    asm volatile("s_barrier" ::: "memory");
  };

  if (ntk > 0) {
    load_tile(0, 0);
    if (ntk > 1) load_tile(1, 1);
    if (ntk > 1) __builtin_amdgcn_s_waitcnt(kWaitVm | kLoadsPerTile);
    else __builtin_amdgcn_s_waitcnt(kWaitVm);
    asm volatile("s_barrier" ::: "memory");
    for (int kt = 0; kt < ntk; kt += kStages) {
      step(0, kt);
      if (kt + 1 < ntk) step(1, kt + 1);
      if (kt + 2 < ntk) step(2, kt + 2);
    }
  }

  if (!qvalid) return;
  // accumulator register i of dqa[nb]: head 32*hg + 8*(i/4) + 4*hf + i%4, dim 32*nb + n.  One
  // part: dq = w * sum.  Several: the unscaled sum is this part's partial; the reduce kernel adds
  // the parts in a fixed tree and then applies w.
  const int64_t prow = (int64_t)part * p.T + t;
  float* const dqrow = (parts == 1 ? p.dq + t * (kHeads * kDim) : p.part_q + prow * (kHeads * kDim)) +
                       (32 * hg + 4 * hf) * kDim + n;
  const float* const wrow = p.w + t * kHeads + 32 * hg + 4 * hf;
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const f32x4 wv4 = parts == 1 ? *reinterpret_cast<const f32x4*>(wrow + 8 * g4) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        dqrow[(8 * g4 + c) * kDim + 32 * nb] = parts == 1 ? wv4[c] * dqa[nb][4 * g4 + c] : dqa[nb][4 * g4 + c];
    }
  }
  // dw: lanes n and n + 32 hold the same head's sums over disjoint keys
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(dwa), __float_as_uint(dwa), false, false);
  const float dwt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (hf == 0) (parts == 1 ? p.dw + t * kHeads : p.part_w + prow * kHeads)[32 * hg + n] = dwt;
}

// ------------------------------------------------------------------------------------------
// dk (or its partials)
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dk_kernel(BwdParams p) {
  int* const scratch = g_dk_scratch;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;
  const int parts = p.dk_parts;

  if (table_flags(p, scratch) & 1) return;
  int idx = 0;
  const int b = locate_unit(p.B, blockIdx.x, [&](int s) -> uint32_t {
    const int lk = p.cu_k[s + 1] - p.cu_k[s];
    return (uint32_t)(ceil_div(lk, kDkKeys) * parts);
  }, scratch, &idx);
  if (b < 0) return;

  const int cq = p.cu_q[b], lq = p.cu_q[b + 1] - cq;
  const int ck = p.cu_k[b], lk_all = p.cu_k[b + 1] - ck;
  const int lk = min(lk_all, p.Lmax);
  const int64_t off = p.offs ? p.offs[b] : 0;
  const int kb = idx / parts, part = idx % parts;   // first key blocks (most queries) first
  const int j0 = kb * kDkKeys;
  // queries that see key j0 (the block's first key): off + i + 1 > j0
  int i0 = 0, L = 0;
  if (j0 < lk) {
    i0 = clampi((int64_t)j0 - off, 0, lq);
    L = lq - i0;
  }
  const int pbeg = i0 + (int)((int64_t)part * L / parts);
  const int iters = i0 + (int)((int64_t)(part + 1) * L / parts) - pbeg;

  // B operand of S = Q . K^T: column = key j0 + 32*wv + n, K elements d = 16*j + 8*hf .. +7
  bf16x8 kf[8];
  {
    const __amdgpu_buffer_rsrc_t krs = rsrc(p.k + (int64_t)ck * kDim, lk_all * kRowBytes);
    const int voff = (j0 + 32 * wv + n) * kRowBytes + 16 * hf;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      kf[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, voff + 32 * j, 0, 0));
  }

  // stage layout: q (16 KiB) | gradients of the 256 keys | w | landing area
  auto gst = [&](unsigned char* st) { return st + kTileBytes; };
  auto wst = [&](unsigned char* st) { return st + kTileBytes + kDkKeys * 4; };
  auto dst_ = [&](unsigned char* st) { return st + kTileBytes + kDkKeys * 4 + 256; };
  // every wave issues 3 loads per query: 2 x 1 KiB of q, then gradients (waves 0-3), w (wave 4)
  // or nothing useful (a zero-length load into the landing area)
  // Every step issues one query's loads (past the unit's last query through zero-record
  // descriptors), so the count in flight is the same on every path and the waits can name it.
  auto load_query = [&](unsigned char* s, int it) {
    const bool real = it < iters;
    const int i = pbeg + (real ? it : 0);
    const int64_t t = (int64_t)cq + i;
    const int nv = clampi(off + i + 1, 0, lk);
    const __amdgpu_buffer_rsrc_t qrs = rsrc(p.q + t * (kHeads * kDim), real ? kTileBytes : 0);
    unsigned char* const qd = s;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int id = r * kWavesB + wv;
      const int row = 4 * id + (lane >> 4), pos = lane & 15;
      lds_load16(qrs, qd + id * 1024, row * kRowBytes + ((pos ^ swzbits(row)) << 4));
    }
    if (wv < 4) lds_load4(rsrc(p.grad + t * p.ld, real ? nv * 4 : 0), gst(s) + wv * 256, (j0 + 64 * wv + lane) * 4);
    else if (wv == 4) lds_load4(rsrc(p.w + t * kHeads, real ? kHeads * 4 : 0), wst(s), lane * 4);
    else lds_load4(rsrc(p.w, 0), dst_(s), lane * 4);
  };
  constexpr int kLoadsPerQuery = 3;

  // transposed-read offsets of the Q^T operand of dk^T += Q^T . G'': rows (heads) 4*hf + jr
  // (+8), columns (dims) 32*mb + 16*(G&1) + 4*r .. +3
  int trq1[4], trq2[4];
  {
    const int L4 = lane & 15, jr = L4 >> 2, r = L4 & 3, gs = (lane >> 4) & 1;
    const int row1 = 4 * hf + jr, row2 = 8 + 4 * hf + jr;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int chunk = 4 * mb + 2 * gs + (r >> 1);
      trq1[mb] = swz(row1, chunk) + 8 * (r & 1);
      trq2[mb] = swz(row2, chunk) + 8 * (r & 1);
    }
  }

  int nat[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) nat[j] = swz(n, 2 * j + hf);

  f32x16 dka[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) dka[mb] = f32x16{};

  // G'' = w[h] * g[key] where S > 0, packed to BF16 as the B operand of two K steps; head of
  // register i in row block rb: 32*rb + 8*(i/4) + 4*hf + i%4
  auto epilogue = [&](f32x16& sv, const float* wb, float gk, int rb, bf16x8& lo, bf16x8& hi) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 wv4 = *reinterpret_cast<const f32x4*>(wb + 32 * rb + 8 * g4 + 4 * hf);
#pragma unroll
      for (int c = 0; c < 4; ++c) sv[4 * g4 + c] = pass_pos(sv[4 * g4 + c], wv4[c] * gk);
    }
    lo = pack8(sv, 0);
    hi = pack8(sv, 1);
  };
  // One query from the LDS stage `qb`: S rows (heads) 0..31; rows 32..63 with the epilogue of
  // rows 0..31; dk K steps 0, 1 with the epilogue of rows 32..63; dk K steps 2, 3.
  auto query = [&](const unsigned char* qb) {
    const float* const wb = reinterpret_cast<const float*>(qb + kTileBytes + kDkKeys * 4);
    const float gk = reinterpret_cast<const float*>(qb + kTileBytes)[32 * wv + n];
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int j = 0; j < 8; ++j) s0 = mfma(lds_b128(qb + nat[j]), kf[j], s0);
#pragma unroll
    for (int j = 0; j < 8; ++j) s1 = mfma(lds_b128(qb + nat[j] + 32 * kRowBytes), kf[j], s1);
    bf16x8 gb[4];
    epilogue(s0, wb, gk, 0, gb[0], gb[1]);
    DSA_SGB(kSgDsRead, 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      DSA_SGB(kSgMfma, 1);
      DSA_SGB(kSgValu, 7);
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        dka[mb] = mfma(lds_tr_pair(qb + st * 16 * kRowBytes + trq1[mb], qb + st * 16 * kRowBytes + trq2[mb]), gb[st],
                       dka[mb]);
    epilogue(s1, wb, gk, 1, gb[2], gb[3]);
    DSA_SGB(kSgDsRead, 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      DSA_SGB(kSgMfma, 1);
      DSA_SGB(kSgValu, 7);
    }
#pragma unroll
    for (int st = 2; st < 4; ++st)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        dka[mb] = mfma(lds_tr_pair(qb + st * 16 * kRowBytes + trq1[mb], qb + st * 16 * kRowBytes + trq2[mb]), gb[st],
                       dka[mb]);
  };
  auto step = [&](auto C_, int it) {
    constexpr int C = decltype(C_)::value;
    load_query(dk_stage<(C + 2) % kStages>(), it + 2);
    query(dk_stage<C>());
    __builtin_amdgcn_s_waitcnt(kWaitVm | kLoadsPerQuery);   // query it + 1 has landed
    asm volatile("s_barrier" ::: "memory");
  };

  if (iters > 0) {
    load_query(dk_stage<0>(), 0);
    load_query(dk_stage<1>(), 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm | kLoadsPerQuery);
    asm volatile("s_barrier" ::: "memory");
    // whole rounds of three steps without a branch inside, then the remainder
    int it = 0;
    for (; it + kStages <= iters; it += kStages) {
      step(Int<0>{}, it);
      step(Int<1>{}, it + 1);
      step(Int<2>{}, it + 2);
    }
    if (it < iters) step(Int<0>{}, it);
    if (it + 1 < iters) step(Int<1>{}, it + 1);
    // the last steps' loads (zero records) are waited for before the stages are reused
    __builtin_amdgcn_s_waitcnt(kWaitVm);
  }

  // The unit's sums leave through LDS so that rows are written with 16-byte stores, one value
  // block of 32 dims at a time: wave wv puts register i of dka[mb] (dim 32*mb + 8*(i/4) +
  // 4*hf + i%4 of key 32*wv + n) at row n, column dim - 32*mb of its own region (waves 0-3 in
  // stage 0, 4-7 in stage 1), then reads the region back by rows.
  __syncthreads();
  float* const ob = reinterpret_cast<float*>(wv < 4 ? dk_stage<0>() : dk_stage<1>()) + (wv & 3) * 32 * kDkOutRow;
  const int nkeys = min(32, lk_all - j0 - 32 * wv);
  float* const out = (parts == 1 ? p.dk : p.part + (int64_t)part * p.Tkv * kDim) +
                     ((int64_t)ck + j0 + 32 * wv) * kDim;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) ob[n * kDkOutRow + 8 * (i >> 2) + 4 * hf + (i & 3)] = dka[mb][i];
#pragma unroll
    for (int rep = 0; rep < 4; ++rep) {
      const int e = rep * 64 + lane;
      const int key = e >> 3, c4 = e & 7;
      const f32x4 v = *reinterpret_cast<const f32x4*>(ob + key * kDkOutRow + 4 * c4);
      if (key < nkeys) *reinterpret_cast<f32x4*>(out + (int64_t)key * kDim + 32 * mb + 4 * c4) = v;
    }
  }
}

// Sum of the P partials src[i + r * stride], r = 0 .. P-1, as the pairwise tree
// ((r0 + r1) + (r2 + r3)) + ... (P a power of two).
template <int P>
struct Tree {
  __device__ __forceinline__ static f32x4 sum(const f32x4* src, int64_t i, int64_t stride, int r0) {
    return Tree<P / 2>::sum(src, i, stride, r0) + Tree<P / 2>::sum(src, i, stride, r0 + P / 2);
  }
};
template <>
struct Tree<1> {
  __device__ __forceinline__ static f32x4 sum(const f32x4* src, int64_t i, int64_t stride, int r0) {
    return src[i + r0 * stride];
  }
};

// dk = the P partials added in the fixed pairwise tree, four floats per thread, grid-stride.
template <int P>
__global__ __launch_bounds__(256) void bwd_dk_reduce_kernel(const float* __restrict__ part, float* __restrict__ dk,
                                                            int64_t n4, const uint32_t* ctrl) {
  if (ctrl[kCtrlCallBad]) return;  // this call's tables are invalid
  const f32x4* src = reinterpret_cast<const f32x4*>(part);
  f32x4* out = reinterpret_cast<f32x4*>(dk);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    out[i] = Tree<P>::sum(src, i, n4, 0);
}

// dq = w * (the P partial sums added in the fixed pairwise tree); dw = the tree of its partials.
template <int P>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(const float* __restrict__ part_q,
                                                            const float* __restrict__ part_w,
                                                            const float* __restrict__ w, float* __restrict__ dq,
                                                            float* __restrict__ dw, int64_t T, const uint32_t* ctrl) {
  if (ctrl[kCtrlCallBad]) return;  // this call's tables are invalid
  const int64_t nq4 = T * (kHeads * kDim / 4), nw4 = T * (kHeads / 4);
  const f32x4* sq = reinterpret_cast<const f32x4*>(part_q);
  const f32x4* sw = reinterpret_cast<const f32x4*>(part_w);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq4 + nw4; i += (int64_t)gridDim.x * blockDim.x) {
    if (i < nq4) {
      const float wt = w[i / (kDim / 4)];   // row (t, h) of the f32x4 group
      reinterpret_cast<f32x4*>(dq)[i] = wt * Tree<P>::sum(sq, i, nq4, 0);
    } else {
      const int64_t j = i - nq4;
      reinterpret_cast<f32x4*>(dw)[j] = Tree<P>::sum(sw, j, nw4, 0);
    }
  }
}

}  // namespace

size_t bwd_dq_smem_bytes() { return kStages * kDqStageBytes + kScratchInts * 4; }
// the dk kernel uses static LDS only
size_t bwd_dk_smem_bytes() { return 0; }

int bwd_dk_parts(int64_t total_k) {
  const int64_t blocks = (total_k + kDkKeys - 1) / kDkKeys;
  int P = 1;
  while (blocks > 0 && P < kBwdMaxParts && blocks * P < kBwdTargetUnits) P *= 2;
  return P;
}

int bwd_dq_parts(int64_t total_q) {
  const int64_t tiles = (total_q + kDqQueries - 1) / kDqQueries;
  int P = 1;
  // one unit per CU is enough here: splitting a tile's keys costs a pass over the partials
  while (tiles > 0 && P < kBwdMaxParts && tiles * P < kBwdTargetUnits / 2) P *= 2;
  return P;
}

hipError_t bwd_prepare() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_dq_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bwd_dq_smem_bytes());
}

hipError_t launch_backward(const BwdParams& p, int dq_grid, int dk_grid, int cus, hipStream_t s,
                           hipEvent_t between) {
  if (dq_grid > 0) {
    hipLaunchKernelGGL(bwd_dq_kernel, dim3(dq_grid), dim3(kBwdThreads), bwd_dq_smem_bytes(), s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.dq_parts > 1) {
      const int64_t n4 = (int64_t)p.T * (kHeads * kDim / 4 + kHeads / 4);
      const int64_t blocks = (n4 + 255) / 256;
      const int grid = (int)(blocks < (int64_t)cus * 8 ? blocks : (int64_t)cus * 8);
#define DSA_DQ_REDUCE(P)                                                                                      \
  case P:                                                                                                     \
    hipLaunchKernelGGL(bwd_dq_reduce_kernel<P>, dim3(grid), dim3(256), 0, s, p.part_q, p.part_w, p.w, p.dq, \
                       p.dw, (int64_t)p.T, p.ctrl);                                                           \
    break;
      switch (p.dq_parts) {
        DSA_DQ_REDUCE(2) DSA_DQ_REDUCE(4) DSA_DQ_REDUCE(8) DSA_DQ_REDUCE(16) DSA_DQ_REDUCE(32) DSA_DQ_REDUCE(64)
        default: return hipErrorInvalidValue;
      }
#undef DSA_DQ_REDUCE
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (between) {
    hipError_t e = hipEventRecord(between, s);
    if (e != hipSuccess) return e;
  }
  if (dk_grid > 0) {
    hipLaunchKernelGGL(bwd_dk_kernel, dim3(dk_grid), dim3(kBwdThreads), bwd_dk_smem_bytes(), s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.dk_parts > 1) {
      const int64_t n4 = (int64_t)p.Tkv * (kDim / 4);
      const int64_t blocks = (n4 + 255) / 256;
      const int grid = (int)(blocks < (int64_t)cus * 8 ? blocks : (int64_t)cus * 8);
#define DSA_DK_REDUCE(P)                                                                         \
  case P:                                                                                        \
    hipLaunchKernelGGL(bwd_dk_reduce_kernel<P>, dim3(grid), dim3(256), 0, s, p.part, p.dk, n4, p.ctrl); \
    break;
      switch (p.dk_parts) {
        DSA_DK_REDUCE(2) DSA_DK_REDUCE(4) DSA_DK_REDUCE(8) DSA_DK_REDUCE(16) DSA_DK_REDUCE(32) DSA_DK_REDUCE(64)
        default: return hipErrorInvalidValue;
      }
#undef DSA_DK_REDUCE
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace dsa
