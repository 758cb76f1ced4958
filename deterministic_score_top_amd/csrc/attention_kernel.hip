// Sparse attention over the selected ids on gfx950 (CDNA4): the consumer of the selection.
//
// For every query row t and head h (flashinfer PR #4573 and its DeepSeek-V4 sparse-MLA decode
// follow-up: the kernel reads the row's selected key ids, never dereferences -1, gathers those
// rows of the shared latent KV table and serves the value operand from the gathered rows):
//     S[h, j]   = scale * q[t, h, :] . kv[id_j, :]            (valid j: 0 <= id_j < Tkv)
//     o[t, h, :] = sum_j softmax_j(S[h, :]) * kv[id_j, :512]
//     lse[t, h]  = log sum_j exp(S[h, j])
// 128 heads, 576-dim latent rows (the first 512 are the value), any number of ids per row.
//
// Two 256-thread blocks per query row, one per half of the heads; one wave per SIMD, so each
// wave may hold 512 registers.  Tiles of 64 ids.  Wave w = (head group g = w % 2, key half
// c = w / 2) owns heads 64*half + 32*g .. +31:
//   * its Q block (32 heads x 576 dims, 144 registers) for the whole row;
//   * the scores of the tile's keys 32*c .. +31 (S^T = K . Q^T on v_mfma_f32_32x32x16_bf16, K
//     rows from LDS, the 36 K steps in ascending dim order): each score is computed once;
//   * the O block of its heads and value half c (32 heads x 256 dims, 128 accumulator
//     registers) over all 64 keys of the tile, with P of the other key half taken from the
//     partner wave (same heads, other key half) through LDS.
// Per tile the pair agrees on each head's maximum (exchanged through LDS), so both apply the
// same softmax reference; the O rows and the partial sums l of a head stay consistent.
//   * Gathered rows land in LDS by buffer loads that write LDS directly (one 16-byte chunk per
//     lane; an id outside [0, Tkv) becomes an out-of-range offset that reads zeros), two
//     stages: the next tile is in flight while one is multiplied.  The 18 load rounds of the
//     next tile are issued between the MFMAs of the current tile's score product, so their
//     address arithmetic runs while the matrix unit works.
//   * Once every wave has finished its score product, the last 64 dims of the tile's rows
//     (needed only for the scores) hold the P exchange.
//   * Online softmax per lane (head) in the exp2 domain.  The reference maximum of a head only
//     moves when a tile's maximum exceeds it by more than 8 (probabilities stay <= 2^8), so the
//     O rescale is rare; the result is the same softmax, a different but fixed rounding.
//   * P rounded to BF16 is the A operand of O += P . V, whose V operand is read key-major from
//     the gathered tile by ds_read_b64_tr_b16.
//   * The valid ids of a row are packed in order to the front of its list first, so -1 entries
//     (the padding of rows with fewer visible keys than k) take no tiles, and only a row's last
//     tile needs the mask of its -1 entries.
//   * A batch of few rows splits each row's tiles into equal parts over several blocks; each part
//     writes its unnormalised O, reference maximum and sum per head, and a second kernel
//     combines the parts in part order.
//   * Every sum has a fixed order, so results are bit-reproducible.

#include <type_traits>

#include "dsa_internal.h"
#include "wave_ops.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kAttnThreads / 64;                // 4: one per SIMD
constexpr int kRowChunks = kAttnDqk * 2 / 16;            // 72 16-byte chunks per latent row
constexpr int kRowBytes = kAttnDqk * 2;                  // 1152
constexpr int kTileSlots = kAttnTile * kRowChunks;       // 4608 chunks per tile
constexpr int kLoadRounds = kTileSlots / kAttnThreads;   // 18 loads per lane per tile
constexpr int kStageBytes = kTileSlots * 16;             // 72 KiB
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kWaitLgkm = 0xC07F;  // s_waitcnt lgkmcnt(0) (LDS), other counters not waited
constexpr int kDropOffset = 0x7FFFFFF0;  // past any table the host accepts (total_kv * 1152 < 2^31)
constexpr int kQkSteps = kAttnDqk / 16;                  // 36 K steps of the score product
constexpr int kDvBlocks = kAttnDv / 2 / 32;              // 8 value column blocks of 32 dims per wave
constexpr int kXcds = 8;                                 // accelerator dies of the MI355X
constexpr float kLazy = 8.f;                             // log2 slack of the reference maximum
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kAttnThreads == 256 && kAttnTile == 64 && kAttnHeads == 2 * 2 * 32, "4 waves x 32 heads x 2 blocks");
static_assert(kTileSlots % kAttnThreads == 0, "whole load rounds per tile");
static_assert(kRowChunks % 8 == 0, "swizzle works inside 8-chunk groups");
static_assert(kWaves * 64 * 32 <= kAttnTile * (kRowBytes - kAttnDv * 2), "the P exchange fits the rope dims");

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int jj) {
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[8 * jj + e];
  return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ bf16x8 lds_tr_pair(const unsigned char* p1, const unsigned char* p2) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p1));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p2));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// x[l] + x[l ^ 32] with the lower half first in every lane, and the same for max
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Chunk swizzle of a gathered tile (rows of 72 16-byte chunks, 1152 bytes): inside each group
// of 8 chunks, XOR with a 3-bit rotation of (row / 2) % 8.  Rows 1152 bytes apart alternate
// between the two halves of the banks, so 16 consecutive rows reading one chunk hit 16
// different bank groups (row parity x 8 XOR values), and the 8 rows of a transposed read
// (4 consecutive rows per lane half) spread over all four 4-chunk bank groups twice.
__device__ __forceinline__ int tswz(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}
__device__ __forceinline__ int toff(int row, int chunk) {
  return row * (kRowChunks * 16) + (((chunk & ~7) | ((chunk ^ tswz(row)) & 7)) << 4);
}

// The two tile stages are separate LDS arrays used with compile-time indices (the tile loop is
// unrolled by two): the compiler can then tell that a gather into one stage does not write the
// stage being read, and waits for the vector-memory counter only where the code says so
// instead of before every LDS read.
__shared__ __align__(16) unsigned char g_stage0[kStageBytes];
__shared__ __align__(16) unsigned char g_stage1[kStageBytes];
__shared__ __align__(16) int g_ids[kMaxTopk];
__shared__ __align__(16) float g_xchg[kWaves * 32];   // per-head maxima, then partial sums
__shared__ __align__(16) float g_fac[kWaves * 32];    // per-head factors of each wave

template <int S>
__device__ __forceinline__ unsigned char* stage() {
  return S == 0 ? g_stage0 : g_stage1;
}
template <int V>
using Int = std::integral_constant<int, V>;

__global__ __launch_bounds__(kAttnThreads, 1) void attention_kernel(AttnParams p) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wv & 1, kh = wv >> 1, partner = wv ^ 2;
  const int n = lane & 31, hf = lane >> 5;
  // Block -> (row, head half), XCD-aware: blocks are dealt to the 8 XCDs round robin, so block
  // b runs on XCD b % 8.  Both halves of a row (which gather the same rows) run on one XCD, and
  // XCD x takes the rows x, x + 8, x + 16, ...: neighbouring rows' selections overlap, so they
  // share the XCD's L2, and every XCD gets the same mix of long and short rows (a row of n
  // valid ids takes ceil(n / 64) tiles).
  // With a split, consecutive blocks are the parts of one (row, head half).
  const int part = (int)(blockIdx.x % (unsigned)p.split);
  int64_t t;
  int half;
  {
    const int64_t b = blockIdx.x / p.split, per = (int64_t)p.T / kXcds;
    if (b < 2 * per * kXcds) {
      const int64_t slot = b / kXcds;
      t = (slot >> 1) * kXcds + b % kXcds;
      half = (int)(slot & 1);
    } else {   // the rows past the last full round of 8: plain order
      const int64_t r = b - 2 * per * kXcds;
      t = per * kXcds + (r >> 1);
      half = (int)(r & 1);
    }
  }
  const int h0 = 64 * half + 32 * hg;   // first head of this wave
  int* const ids = g_ids;

  // The row's ids and this wave's Q block are loaded with all requests in flight at once.  The
  // valid ids are then packed in their order to the front of the LDS list (ids outside
  // [-1, Tkv) are flagged and treated as -1), so tiles hold only valid ids except at the tail
  // (padded with -1) and a row of n valid ids takes ceil(n / 64) tiles: -1 entries (the
  // padding of rows with fewer visible keys than k) cost nothing.  Wave w packs the entries
  // 512*w .. +511, lane l the 8 entries from 512*w + 8*l.
  constexpr int kIdsPerLane = kMaxTopk / kAttnThreads;
  int idr[kIdsPerLane];
  {
    const int j0 = 512 * wv + kIdsPerLane * lane;
#pragma unroll
    for (int k = 0; k < kIdsPerLane; ++k) idr[k] = j0 + k < p.topk ? p.ids[t * p.topk + j0 + k] : -1;
  }
  // B operand of S^T = K . Q^T: column = head h0 + n, K elements = dims 16*st + 8*hf .. +7
  bf16x8 qf[kQkSteps];
  {
    const uint16_t* qrow = p.q + ((t * kAttnHeads + h0 + n) * kAttnDqk) + 8 * hf;
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st);
  }
  int ntile, total;
  {
    uint32_t cnt = 0;
    int bad = 0;
#pragma unroll
    for (int k = 0; k < kIdsPerLane; ++k) {
      if (idr[k] < -1 || idr[k] >= p.Tkv) {
        bad = 1;
        idr[k] = -1;
      }
      cnt += idr[k] >= 0 ? 1u : 0u;
    }
    if (bad) atomicOr(p.ctrl + kCtrlStatus, kStatusBadIds);
    const uint32_t incl = wave_incl_scan(cnt);
    if (lane == 63) g_xchg[wv] = __uint_as_float(incl);   // the wave's count, as bits
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t c = __float_as_uint(g_xchg[w]);
      before += w < wv ? c : 0u;
      tot += c;
    }
    total = (int)tot;
    int pos = (int)(before + incl - cnt);
#pragma unroll
    for (int k = 0; k < kIdsPerLane; ++k) {
      if (idr[k] >= 0) ids[pos++] = idr[k];
    }
    ntile = (total + kAttnTile - 1) / kAttnTile;
    for (int j = total + tid; j < ntile * kAttnTile; j += kAttnThreads) ids[j] = -1;
  }
  // this block's tiles: part `part` of `split` equal ranges (empty when the row is short)
  const int tper = (ntile + p.split - 1) / p.split;
  const int kbeg = min(ntile, part * tper), kend = min(ntile, kbeg + tper);
  const float c2 = p.scale * kLog2e;   // scores in the exp2 domain
  __syncthreads();

  const __amdgpu_buffer_rsrc_t kvrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), (short)0, p.Tkv * kRowBytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t kvrs_none =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), (short)0, 0, kRsrcWord3);
  // Gather slots: load round r of wave wv fills chunk slots (r*4 + wv)*64 .. +63 of a stage; slot ->
  // (row, position), and the lane fetches the logical chunk the swizzle stores at that position.
  // The rounds of the next tile are issued between the MFMAs of this tile's score product.  The
  // offset of id -1 wraps to a huge value that the clamp turns into the drop offset (a valid
  // offset is below total_kv * 1152 < 2^31 - 16).  A step without a next tile still issues the
  // rounds, through a descriptor of zero records (nothing is read, the free stage gets zeros).
  auto gid = [&](int kt, int r) __attribute__((always_inline)) {
    return ids[kt * kAttnTile + ((r * kWaves + wv) * 64 + lane) / kRowChunks];
  };
  auto gload = [&](unsigned char* base, __amdgpu_buffer_rsrc_t rs, int r, int id) __attribute__((always_inline)) {
    const int slot = (r * kWaves + wv) * 64 + lane;
    const int row = slot / kRowChunks, pos = slot - row * kRowChunks;
    const int col = ((pos & ~7) | ((pos ^ tswz(row)) & 7)) * 16;
    const uint32_t voff = min((uint32_t)(__mul24(id, kRowBytes) + col), (uint32_t)kDropOffset);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(base + (r * kWaves + wv) * 1024),
                                             16, (int)voff, 0, 0, 0);
  };

  // transposed-read offsets of the V operand: rows (keys) 4*hf + jr (+8), columns (dims)
  // 256*kh + 32*nb + 16*(G&1) + 4*r .. +3.  The swizzle only touches the low 3 bits of the
  // chunk index, which repeat every 2 column blocks: blocks nb and nb + 2 are 128 bytes apart.
  int trv1[2], trv2[2];
  {
    const int L4 = lane & 15, jr = L4 >> 2, r = L4 & 3, gs = (lane >> 4) & 1;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int chunk = 4 * nb + 2 * gs + (r >> 1);
      trv1[nb] = toff(4 * hf + jr, chunk) + 8 * (r & 1) + kh * 512;
      trv2[nb] = toff(8 + 4 * hf + jr, chunk) + 8 * (r & 1) + kh * 512;
    }
  }
  // row-major K reads: row 32*kh + n, chunk 2*st + hf; K steps st and st + 4 are 128 bytes apart
  // (row 32*kh + n has the swizzle of row n)
  int kro[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) kro[st] = toff(n, 2 * st + hf) + 32 * kh * kRowBytes;
  // P exchange slots in the rope dims: wave w's lane l at row 16*w + l/4, bytes 1024 + 32*(l%4)
  const int xown = (16 * wv + (lane >> 2)) * kRowBytes + kAttnDv * 2 + 32 * (lane & 3);
  const int xpar = (16 * partner + (lane >> 2)) * kRowBytes + kAttnDv * 2 + 32 * (lane & 3);

  // The per-tile work is scheduled by hand: sched_barrier fences keep the compiler from
  // hoisting every operand read of a tile into registers, while the reads of the next chunk
  // still run one chunk ahead of the MFMAs that use them.
  //
  // S^T of this wave's 32 keys; register i: key 32*kh + 8*(i/4) + 4*hf + i%4, head h0 + n.
  // Nine chunks of four K steps (ascending dims) on one accumulator.
  auto scores = [&](const unsigned char* kb, unsigned char* gb, __amdgpu_buffer_rsrc_t grs, int gkt)
      __attribute__((always_inline)) {
    auto rd = [&](int st) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(kb + kro[st & 3] + (st >> 2) * 128);
    };
    f32x16 sp = f32x16{};
    bf16x8 ka[4], kn[4];
    int gi[2], gn[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) ka[j] = rd(j);
    gi[0] = gid(gkt, 0);
    gi[1] = gid(gkt, 1);
#pragma unroll
    for (int c = 0; c < kQkSteps / 4; ++c) {
      if (c + 1 < kQkSteps / 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) kn[j] = rd(4 * (c + 1) + j);
        gn[0] = gid(gkt, 2 * c + 2);
        gn[1] = gid(gkt, 2 * c + 3);
      }
      __builtin_amdgcn_sched_barrier(0);
      sp = mfma(ka[0], qf[4 * c], sp);
      __builtin_amdgcn_sched_barrier(0);
      gload(gb, grs, 2 * c, gi[0]);
      __builtin_amdgcn_sched_barrier(0);
      sp = mfma(ka[1], qf[4 * c + 1], sp);
      __builtin_amdgcn_sched_barrier(0);
      gload(gb, grs, 2 * c + 1, gi[1]);
      __builtin_amdgcn_sched_barrier(0);
      sp = mfma(ka[2], qf[4 * c + 2], sp);
      sp = mfma(ka[3], qf[4 * c + 3], sp);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) ka[j] = kn[j];
      gi[0] = gn[0];
      gi[1] = gn[1];
    }
    return sp;
  };
  f32x16 oa[kDvBlocks];
#pragma unroll
  for (int nb = 0; nb < kDvBlocks; ++nb) oa[nb] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;   // reference max (exp2 domain) and this lane's partial sum

  // O *= alpha per head row (rows of lane l: heads 8*(i/4) + 4*hf + i%4, whose factors sit in
  // lanes of the other layout), skipped when no head of the wave moved its reference
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) == 0) return;
    if (hf == 0) g_fac[wv * 32 + n] = alpha;
    // the factors are read back by the same wave only (no block barrier needed)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    const f32x4* fv = reinterpret_cast<const f32x4*>(g_fac + wv * 32 + 4 * hf);
    f32x4 a4[4];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) a4[g4] = fv[2 * g4];
    // O stays in the accumulator registers: each element is read, scaled and written back in
    // place.  The compiler does not see into the asm, so the MFMA result hazards are covered by
    // hand: 24 wait states after the last value-product MFMA, 8 before the next MFMA.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int nb = 0; nb < kDvBlocks; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = oa[nb][i], tmp;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(tmp)
                     : "v"(a4[i >> 2][i & 3]));
        oa[nb][i] = x;
      }
    asm volatile("s_nop 7" ::: "memory");
  };

  // Step kt (tile kt in stage kt % 2): wait for tile kt and meet (every wave is past step
  // kt - 1, so the other stage is free) and start gathering tile kt + 1 into it; scores of this
  // wave's keys; meet to exchange the per-head maxima; P of this wave's keys into the rope dims;
  // meet; the value product over all 64 keys with the partner's P.
  auto step = [&](auto S_, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value;
    unsigned char* const kb = stage<S>();
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vector memory counter 0: tile kt has landed
    asm volatile("s_barrier" ::: "memory");
    const bool more = kt + 1 < kend;
    f32x16 sp = scores(kb, stage<1 - S>(), more ? kvrs : kvrs_none, more ? kt + 1 : kt);

    // scale, then the maximum of each head over this wave's keys; only the last tile of a row
    // holds -1 entries (the valid ids are packed to the front), so only it is masked
#pragma unroll
    for (int i = 0; i < 16; ++i) sp[i] *= c2;
    if ((kt + 1) * kAttnTile > total) {
      const i32x4* const idv = reinterpret_cast<const i32x4*>(ids + kt * kAttnTile + 32 * kh);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const i32x4 iv = idv[2 * g4 + hf];   // keys 32*kh + 8*g4 + 4*hf .. +3
#pragma unroll
        for (int c = 0; c < 4; ++c) sp[4 * g4 + c] = iv[c] >= 0 ? sp[4 * g4 + c] : -__builtin_inff();
      }
    }
    float tmax = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sp[i]);
    tmax = half_max(tmax);
    if (hf == 0) g_xchg[wv * 32 + n] = tmax;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    asm volatile("s_barrier" ::: "memory");
    tmax = fmaxf(tmax, g_xchg[partner * 32 + n]);   // the pair's maximum: equal in both waves
    // the reference moves only past the slack (and from -inf to the first valid maximum)
    const float mnew = tmax > m + kLazy ? tmax : m;
    // before the first valid key O and l are 0: nothing to rescale
    const float alpha = (mnew == m || m == -__builtin_inff()) ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    const float mref = m == -__builtin_inff() ? 0.f : m;   // no valid key yet: every P is 0
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sp[i] = __builtin_amdgcn_exp2f(sp[i] - mref);   // exp2(-inf) = 0 for invalid keys
      psum += sp[i];
    }
    l = l * alpha + psum;
    const bf16x8 pa0 = pack8(sp, 0), pa1 = pack8(sp, 1);
    // every wave's score product is done (the maxima were written after it): the rope dims of
    // this stage are free for the P exchange
    *reinterpret_cast<bf16x8*>(kb + xown) = pa0;
    *reinterpret_cast<bf16x8*>(kb + xown + 16) = pa1;
    rescale(alpha);
    // The value product over this wave's own keys needs only its own P: its MFMAs are issued
    // before the pair meets, so the matrix unit works through the barrier and the read of the
    // partner's P.  Each value block sums this wave's keys first, then the partner's: a fixed
    // order in every wave.
    auto vread = [&](int nb, int j) __attribute__((always_inline)) {
      const int o1 = trv1[nb & 1] + (nb >> 1) * 128 + 16 * j * kRowBytes;
      const int o2 = trv2[nb & 1] + (nb >> 1) * 128 + 16 * j * kRowBytes;
      return lds_tr_pair(kb + o1, kb + o2);
    };
    // key half `kc` of every value block: K steps 2*kc and 2*kc + 1
    auto half_product = [&](int kc, const bf16x8& a0, const bf16x8& a1, f32x16 (&acc)[kDvBlocks])
        __attribute__((always_inline)) {
      bf16x8 va[2], vn[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) va[j] = vread(0, 2 * kc + j);
#pragma unroll
      for (int nb = 0; nb < kDvBlocks; ++nb) {
        if (nb + 1 < kDvBlocks) {
#pragma unroll
          for (int j = 0; j < 2; ++j) vn[j] = vread(nb + 1, 2 * kc + j);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc[nb] = mfma(a0, va[0], acc[nb]);
        acc[nb] = mfma(a1, va[1], acc[nb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2; ++j) va[j] = vn[j];
      }
    };
    half_product(kh, pa0, pa1, oa);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    asm volatile("s_barrier" ::: "memory");
    const bf16x8 qa0 = *reinterpret_cast<const bf16x8*>(kb + xpar);
    const bf16x8 qa1 = *reinterpret_cast<const bf16x8*>(kb + xpar + 16);
    half_product(1 - kh, qa0, qa1, oa);
  };
  if (kbeg < kend) {
#pragma unroll
    for (int r = 0; r < kLoadRounds; ++r) gload(stage<0>(), kvrs, r, gid(kbeg, r));
  }
  for (int kt = kbeg; kt < kend; kt += 2) {
    step(Int<0>{}, kt);
    if (kt + 1 >= kend) break;
    step(Int<1>{}, kt + 1);
  }
  // the last step's rounds (zero records) are waited for before the block can end
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // l of each head = the pair's partial sums, key half 0 first; o = O / l (0 for a row with no
  // valid id), lse = (m + log2 l) * ln 2.  Every read of the exchanged maxima happened before
  // the last step's final barrier.
  const float lw = half_sum(l);
  if (hf == 0) g_xchg[wv * 32 + n] = lw;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm);
  __syncthreads();
  const float lp = g_xchg[partner * 32 + n];
  const float lt = kh == 0 ? lw + lp : lp + lw;
  if (p.split > 1) {
    // a part's result: O unnormalised and (reference maximum, l) per head, combined with the
    // other parts by the merge kernel
    const int64_t prow = (t * p.split + part) * kAttnHeads;
    float* const orow = p.part_o + ((prow + h0 + 4 * hf) * kAttnDv) + 256 * kh + n;
#pragma unroll
    for (int nb = 0; nb < kDvBlocks; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) orow[(8 * (i >> 2) + (i & 3)) * kAttnDv + 32 * nb] = oa[nb][i];
    if (hf == 0 && kh == 0) {
      p.part_ml[(prow + h0 + n) * 2] = m;
      p.part_ml[(prow + h0 + n) * 2 + 1] = lt;
    }
    return;
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (hf == 0) g_fac[wv * 32 + n] = inv;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm);
  const f32x4* fv = reinterpret_cast<const f32x4*>(g_fac + wv * 32 + 4 * hf);
  f32x4 a4[4];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) a4[g4] = fv[2 * g4];
  float* const orow = p.out + ((t * kAttnHeads + h0 + 4 * hf) * kAttnDv) + 256 * kh + n;
#pragma unroll
  for (int nb = 0; nb < kDvBlocks; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      orow[(8 * (i >> 2) + (i & 3)) * kAttnDv + 32 * nb] = oa[nb][i] * a4[i >> 2][i & 3];
  if (hf == 0 && kh == 0)
    p.lse[t * kAttnHeads + h0 + n] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -__builtin_inff();
}

// Combine the parts of each (row, head): with M the largest reference maximum of the parts and
// f_s = 2^(m_s - M) (0 for a part without a valid id), l = sum_s f_s l_s and o = sum_s f_s O_s / l,
// summed over s = 0, 1, ... in that order; lse = (M + log2 l) ln 2.  One 128-thread block per
// (row, head), four value dims per thread.
__global__ __launch_bounds__(128) void attention_merge_kernel(AttnParams p) {
  const int64_t rh = blockIdx.x;   // row * 128 + head
  const int64_t t = rh / kAttnHeads, h = rh % kAttnHeads;
  const int S = p.split;
  // the loops run over the largest split count with the parts past S switched off, so every
  // part's loads are in flight together; the sums still run s = 0, 1, ... in order
  float ms[kAttnMaxSplit], ls[kAttnMaxSplit];
  f32x4 os[kAttnMaxSplit];
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s) {
    if (s < S) {
      const int64_t ph = (t * S + s) * kAttnHeads + h;
      ms[s] = p.part_ml[ph * 2];
      ls[s] = p.part_ml[ph * 2 + 1];
      os[s] = *reinterpret_cast<const f32x4*>(p.part_o + ph * kAttnDv + 4 * threadIdx.x);
    }
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s)
    if (s < S) M = fmaxf(M, ms[s]);
  float L = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s) {
    if (s < S) {
      const float f = ms[s] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ms[s] - M);
      L += f * ls[s];
      acc += f * os[s];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<f32x4*>(p.out + rh * kAttnDv + 4 * threadIdx.x) = acc * inv;
  if (threadIdx.x == 0) p.lse[rh] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * kLn2 : -__builtin_inff();
}

}  // namespace

int attn_split(int T, int topk) {
  const int ntile = (topk + kAttnTile - 1) / kAttnTile;
  int s = 1;
  while ((int64_t)2 * T * s < kAttnSplitBlocks && s < kAttnMaxSplit && 2 * s <= ntile) s *= 2;
  return s;
}

size_t attn_partial_bytes(int T, int topk) {
  const int s = attn_split(T, topk);
  if (s == 1) return 0;
  return (size_t)T * s * kAttnHeads * (kAttnDv + 2) * 4u;
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attention_kernel, dim3(2 * p.T * p.split), dim3(kAttnThreads), 0, s, p);
  if (p.split > 1) hipLaunchKernelGGL(attention_merge_kernel, dim3(p.T * kAttnHeads), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
