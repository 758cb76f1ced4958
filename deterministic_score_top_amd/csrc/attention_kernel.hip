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
// Two 512-thread blocks per query row, 64 heads each (so a gathered KV tile serves 64 heads;
// all 128 in one block would need more than the 256 VGPRs of two waves per SIMD).  Wave w
// takes heads 32*(w/4) .. +31 of its block and dim quarter w%4: the score product over dims
// 144*(w%4) .. +143 and the output dims 128*(w%4) .. +127.
//   * Tiles of 32 ids: their 576-dim rows land in LDS by buffer loads that write LDS directly
//     (one 16-byte chunk per lane; an id outside [0, Tkv) becomes an out-of-range offset that
//     reads zeros), the next tile in flight while the current one is multiplied.
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K rows from LDS, Q in VGPRs for the whole
//     row), so that each lane holds one head's scores of 16 keys; the four dim quarters of
//     a head group add their partial sums through LDS in one fixed tree ((0+1)+(2+3)).
//   * Online softmax in the exp2 domain per lane (head), the running maximum shared by the
//     two lane halves; P rounded to BF16 is the A operand of O += P . V, whose V operand is
//     read key-major from the gathered tile by ds_read_b64_tr_b16.  The O rescale is skipped
//     when no head's maximum moved (a multiplication by 1).
//   * Every sum has a fixed order, so results are bit-reproducible.

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = kAttnThreads / 64;
constexpr int kRowChunks = kAttnDqk * 2 / 16;            // 72 16-byte chunks per latent row
constexpr int kTileSlots = kAttnTile * kRowChunks;       // 2304 chunks per tile
constexpr int kLoadRounds = (kTileSlots + kAttnThreads - 1) / kAttnThreads;  // 5 loads per wave
constexpr int kStageBytes = kLoadRounds * kAttnThreads * 16;  // 40 KiB (tail slots land in padding)
constexpr int kStages = 2;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kWaitVm = 0x0F70;    // s_waitcnt: vector memory counter only (OR in the count)
constexpr int kWaitLgkm = 0xC07F;  // s_waitcnt lgkmcnt(0) (LDS), other counters not waited
constexpr int kDropOffset = 0x7FFFFFF0;  // past any table the host accepts (total_kv * 1152 < 2^31)
constexpr int kQkSteps = kAttnDqk / 4 / 16;              // 9 K steps per dim quarter
constexpr int kBlockHeads = 64;                          // heads per block (two blocks per row)
constexpr int kXcds = 8;                                 // accelerator dies of the MI355X
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kAttnThreads == 512 && kAttnTile == 32 && kAttnHeads == 128, "layout assumes 8 waves");
static_assert(kRowChunks % 8 == 0, "swizzle works inside 8-chunk groups");

// LDS layout: stages | ids (padded to whole tiles) | score partials | per-head factors
constexpr int kPartStride = 20;                      // floats per lane: 16 partials + 4 pad
constexpr int kPartWave = 64 * kPartStride;          // floats per wave
constexpr int kPartBytes = kWaves * kPartWave * 4;   // 40 KiB
constexpr int kFacBytes = kWaves * 32 * 4;         // 1 KiB

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

__global__ __launch_bounds__(kAttnThreads, 1) void attention_kernel(AttnParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wv >> 2, dq = wv & 3;
  const int n = lane & 31, hf = lane >> 5;
  // Block -> (row, head half), XCD-aware: blocks are dealt to the 8 XCDs round robin, so block
  // b runs on XCD b % 8.  Both head halves of a row, and the rows t, t + 8, t + 16, ... (whose
  // selections overlap), go to the same XCD and share its L2.
  int64_t t;
  int half;
  {
    const int64_t b = blockIdx.x, grid = gridDim.x;   // grid = 2 * T
    const int64_t x = b % kXcds, slot = b / kXcds;
    const int64_t per = grid / kXcds;                  // full rounds of kXcds blocks
    if (slot < (per & ~(int64_t)1)) {
      half = (int)(slot & 1);
      t = (slot >> 1) * kXcds + x;
    } else {                                           // the tail: plain order
      const int64_t r = b - (per & ~(int64_t)1) * kXcds;
      t = ((per & ~(int64_t)1) >> 1) * kXcds + (r >> 1);
      half = (int)(r & 1);
    }
  }
  const int h0 = half * kBlockHeads + 32 * hg;   // first head of this wave's group
  const int ntile = (p.topk + kAttnTile - 1) / kAttnTile;
  int* const ids = reinterpret_cast<int*>(smem + kStages * kStageBytes);
  float* const part = reinterpret_cast<float*>(smem + kStages * kStageBytes + ntile * kAttnTile * 4);
  float* const fac = part + kPartBytes / 4;

  // the row's ids into LDS (padding past topk = -1); ids outside [-1, Tkv) are flagged and skipped
  {
    int bad = 0;
    for (int j = tid; j < ntile * kAttnTile; j += kAttnThreads) {
      int id = j < p.topk ? p.ids[t * p.topk + j] : -1;
      if (id < -1 || id >= p.Tkv) {
        bad = 1;
        id = -1;
      }
      ids[j] = id;
    }
    if (bad) atomicOr(p.ctrl + kCtrlStatus, kStatusBadIds);
  }

  // B operand of S^T = K . Q^T: column = head h0 + n, K elements = dims 144*dq + 16*st + 8*hf ..
  bf16x8 qf[kQkSteps];
  {
    const uint16_t* qrow = p.q + ((t * kAttnHeads + h0 + n) * kAttnDqk) + 144 * dq + 8 * hf;
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qrow + 16 * st);
  }
  const float c2 = p.scale * kLog2e;   // scores in the exp2 domain
  __syncthreads();

  const __amdgpu_buffer_rsrc_t kvrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), (short)0, p.Tkv * (kAttnDqk * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t nullrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.kv), (short)0, 0, kRsrcWord3);
  // tile kt into stage s: load r of wave wv fills slots (r*8 + wv)*64 .. +63; slot -> (row, chunk)
  auto gather = [&](int s, int kt) {
    unsigned char* const base = smem + s * kStageBytes;
#pragma unroll
    for (int r = 0; r < kLoadRounds; ++r) {
      const int slot = (r * kWaves + wv) * 64 + lane;
      const int row = slot / kRowChunks, pos = slot % kRowChunks;
      const int chunk = (pos & ~7) | ((pos ^ tswz(row)) & 7);   // logical chunk stored at pos
      const bool tail = (r * kWaves + wv) * 64 >= kTileSlots;   // wave-uniform
      const int id = tail ? -1 : ids[kt * kAttnTile + min(row, kAttnTile - 1)];
      const int voff = id >= 0 ? id * (kAttnDqk * 2) + chunk * 16 : kDropOffset;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(tail ? nullrs : kvrs,
                                               (__attribute__((address_space(3))) void*)(base + (r * kWaves + wv) * 1024),
                                               16, voff, 0, 0, 0);
    }
  };

  // transposed-read offsets of the V operand: rows (keys) 4*hf + jr (+8), columns (dims)
  // 128*dq + 32*nb + 16*(G&1) + 4*r .. +3.  The swizzle only touches the low 3 bits of the
  // chunk index, which repeat every 2 column blocks: blocks nb and nb + 2 are 128 bytes apart.
  int trv1[2], trv2[2];
  {
    const int L4 = lane & 15, jr = L4 >> 2, r = L4 & 3, gs = (lane >> 4) & 1;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int chunk = 16 * dq + 4 * nb + 2 * gs + (r >> 1);
      trv1[nb] = toff(4 * hf + jr, chunk) + 8 * (r & 1);
      trv2[nb] = toff(8 + 4 * hf + jr, chunk) + 8 * (r & 1);
    }
  }
  // row-major K reads: row n, chunk 18*dq + 2*st + hf; K steps st and st + 4 are 128 bytes apart
  int kro[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) kro[st] = toff(n, 18 * dq + 2 * st + hf);

  f32x16 oa[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) oa[nb] = f32x16{};
  float m = -__builtin_inff(), l = 0.f;   // running max (exp2 domain) and sum of this lane's head

  if (ntile > 0) gather(0, 0);
  for (int kt = 0; kt < ntile; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntile) {
      gather(cur ^ 1, kt + 1);
      __builtin_amdgcn_s_waitcnt(kWaitVm | kLoadRounds);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm);
    }
    asm volatile("s_barrier" ::: "memory");
    const unsigned char* const kb = smem + cur * kStageBytes;

    // partial S^T over this wave's dim quarter; register i: key 8*(i/4) + 4*hf + i%4, head n
    f32x16 sp = f32x16{};
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st)
      sp = mfma(*reinterpret_cast<const bf16x8*>(kb + kro[st & 3] + (st >> 2) * 128), qf[st], sp);
    // lane l's 16 partials at floats l*20 .. l*20+15 of the wave's region: 16-byte accesses,
    // 16 consecutive lanes on 16 different 4-bank groups
    f32x4* const mine = reinterpret_cast<f32x4*>(part + wv * kPartWave + lane * kPartStride);
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) mine[g4] = f32x4{sp[4 * g4], sp[4 * g4 + 1], sp[4 * g4 + 2], sp[4 * g4 + 3]};
    // LDS writes done, then meet (a fenced __syncthreads would also wait for the next tile's
    // loads, which must stay in flight)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
    asm volatile("s_barrier" ::: "memory");
    // the group's four quarters, this lane's 16 partials of each
    const f32x4* const q0 = reinterpret_cast<const f32x4*>(part + (4 * hg) * kPartWave + lane * kPartStride);
    constexpr int kQ = kPartWave / 4;   // f32x4 stride between the quarters
    // validity of this lane's 16 keys
    const i32x4* const idv = reinterpret_cast<const i32x4*>(ids + kt * kAttnTile);
    // scores in the exp2 domain, -inf for invalid keys (in place of the partial)
    float tmax = -__builtin_inff();
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const i32x4 iv = idv[2 * g4 + hf];   // keys 8*g4 + 4*hf .. +3
      // same fixed tree in all four waves of the group
      const f32x4 sc = (q0[g4] + q0[kQ + g4]) + (q0[2 * kQ + g4] + q0[3 * kQ + g4]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int i = 4 * g4 + c;
        sp[i] = iv[c] >= 0 ? sc[c] * c2 : -__builtin_inff();
        tmax = fmaxf(tmax, sp[i]);
      }
    }
    tmax = half_max(tmax);
    const float mnew = fmaxf(m, tmax);
    const bool moved = mnew != m;
    float psum = 0.f;
    // nothing valid yet: every P is 0 (and m, l stay at -inf, 0)
    const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sp[i] = __builtin_amdgcn_exp2f(sp[i] - mref);   // exp2(-inf) = 0 for invalid keys
      psum += sp[i];
    }
    // O and l scale by 2^(m - mnew): exactly 1 when the maximum did not move, 0 before the
    // first valid key
    const float alpha = !moved ? 1.f : (m == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m - mnew));
    l = l * alpha + half_sum(psum);
    m = mnew;
    // O *= alpha per head row, skipped when no head of the wave moved its maximum
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
      if (hf == 0) fac[wv * 32 + n] = alpha;
      // the factors are read back by the same wave only (no block barrier needed)
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      const f32x4* fv = reinterpret_cast<const f32x4*>(fac + wv * 32 + 4 * hf);
      f32x4 a4[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) a4[g4] = fv[2 * g4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oa[nb][i] *= a4[i >> 2][i & 3];
    }
    // O[h, dv] += P[h, key] . V[key, dv]
    const bf16x8 pa0 = pack8(sp, 0), pa1 = pack8(sp, 1);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int o1 = trv1[nb & 1] + (nb >> 1) * 128, o2 = trv2[nb & 1] + (nb >> 1) * 128;
      oa[nb] = mfma(pa0, lds_tr_pair(kb + o1, kb + o2), oa[nb]);
      oa[nb] = mfma(pa1, lds_tr_pair(kb + 16 * (kRowChunks * 16) + o1, kb + 16 * (kRowChunks * 16) + o2), oa[nb]);
    }
    asm volatile("s_barrier" ::: "memory");
  }

  // o = O / l (0 for a row with no valid id), lse = (m + log2 l) * ln 2
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (hf == 0) fac[wv * 32 + n] = inv;
  __builtin_amdgcn_s_waitcnt(kWaitLgkm);
  const f32x4* fv = reinterpret_cast<const f32x4*>(fac + wv * 32 + 4 * hf);
  f32x4 a4[4];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) a4[g4] = fv[2 * g4];
  float* const orow = p.out + ((t * kAttnHeads + h0 + 4 * hf) * kAttnDv) + 128 * dq + n;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      orow[(8 * (i >> 2) + (i & 3)) * kAttnDv + 32 * nb] = oa[nb][i] * a4[i >> 2][i & 3];
  if (dq == 0 && hf == 0)
    p.lse[t * kAttnHeads + h0 + n] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -__builtin_inff();
}

}  // namespace

size_t attn_smem_bytes(int topk) {
  const int ntile = (topk + kAttnTile - 1) / kAttnTile;
  return (size_t)kStages * kStageBytes + (size_t)ntile * kAttnTile * 4 + kPartBytes + kFacBytes;
}

hipError_t attn_prepare(int max_topk) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(attention_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)attn_smem_bytes(max_topk));
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  hipLaunchKernelGGL(attention_kernel, dim3(2 * p.T), dim3(kAttnThreads), attn_smem_bytes(p.topk), s, p);
  return hipGetLastError();
}

}  // namespace dsa
