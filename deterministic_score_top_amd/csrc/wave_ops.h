// Wave-level primitives shared by the kernels (device code only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Wave-wide reductions and scans with DPP lane moves (no LDS round trips).  update_dpp keeps
// `old` in lanes whose row is masked off or whose source lane lies outside the row, so `old`
// is the operation's identity.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppQuad1032 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;     // lane i of a row of 16 reads lane 15-i
constexpr int kDppRowHalfMirror = 0x141; // lane i of a half row of 8 reads lane 7-i
constexpr int kDppRowBcast15 = 0x142;    // lane 15 of each row feeds the next row
constexpr int kDppRowBcast31 = 0x143;    // lane 31 feeds rows 2 and 3
constexpr int kDppRowShr = 0x110;        // + n: lane i reads lane i-n of its row

// After the six steps lane 63 holds the combination of all 64 lanes.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, uint32_t identity, Op op) {
  v = op(v, dpp<kDppQuad1032>(identity, v));
  v = op(v, dpp<kDppQuad2301>(identity, v));
  v = op(v, dpp<kDppRowHalfMirror>(identity, v));
  v = op(v, dpp<kDppRowMirror>(identity, v));
  v = op(v, dpp<kDppRowBcast15, 0xA>(identity, v));
  v = op(v, dpp<kDppRowBcast31, 0xC>(identity, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_reduce(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_reduce(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<kDppRowShr + 1>(0u, v);
  v += dpp<kDppRowShr + 2>(0u, v);
  v += dpp<kDppRowShr + 4>(0u, v);
  v += dpp<kDppRowShr + 8>(0u, v);
  v += dpp<kDppRowBcast15, 0xA>(0u, v);
  v += dpp<kDppRowBcast31, 0xC>(0u, v);
  return v;
}

}  // namespace dsa
