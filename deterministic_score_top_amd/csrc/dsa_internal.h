// Internal declarations shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr int kHeads = 64;       // indexer heads H
constexpr int kDim = 128;        // head dim D
#ifndef DSA_SCORE_THREADS
#define DSA_SCORE_THREADS 512
#endif
constexpr int kScoreThreads = DSA_SCORE_THREADS;  // one query per wave
constexpr int kWaves = kScoreThreads / 64;
constexpr int kTileQueries = kWaves;                     // one query per wave; queries per unit
#ifndef DSA_TILE_KEYS
#define DSA_TILE_KEYS 64
#endif
constexpr int kTileKeys = DSA_TILE_KEYS;                 // keys per LDS stage (64 or 128)
constexpr int kCtrlBytes = 256;                          // control block at workspace offset 0
constexpr int kMaxTopk = 2048;
constexpr int kMaxSeqlenK = 65536;
constexpr int kRowAlign = 64;                            // score rows padded to 64 floats

// Control block layout (u32 words at workspace offset 0).
constexpr int kCtrlTicket = 0;
constexpr int kCtrlDone = 1;
constexpr int kCtrlStatus = 2;
constexpr int kCtrlExpected = 3;  // final counter value of the score kernel, for the select kernel's check
// Verdict of the current call on its segment tables (1 = invalid), overwritten by the first kernel
// of every call and read by the kernels after it; the status word above is sticky and only reports.
constexpr int kCtrlCallBad = 4;

constexpr uint32_t kStatusCorruptCounter = 0x1u;
constexpr uint32_t kStatusBadSegments = 0x2u;
constexpr uint32_t kStatusSeqlenBound = 0x4u;

struct ScoreParams {
  const uint16_t* q;  // bf16 [T, H, D]
  const uint16_t* k;  // bf16 [Tkv, D]
  const float* w;     // fp32 [T, H]
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* offs;  // may be null
  float* out;           // fp32 rows, stride ld
  int64_t ld;
  uint32_t* ctrl;
  int32_t B, T, Tkv, Lmax;
  int32_t chunk_tiles;  // keys per unit = chunk_tiles * kTileKeys; 0 = chosen by the kernel
  int32_t max_tiles;    // capacity of the LDS tile table
  int32_t store_keys;   // 1: store order-preserving 32-bit keys instead of FP32 scores
  const uint32_t* plan; // prepared plan (from launch_plan for this grid), or null: derive it
};

struct SelectParams {
  const uint32_t* keys;  // order-preserving score keys, rows of stride ld
  int64_t ld;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* offs;
  int32_t* out_ids;
  float* out_scores;
  uint32_t* ctrl;  // block 0 checks and resets the work-unit counter left by the score kernel
  int32_t B, T, Tkv, Lmax, topk;
};

// Backward of the scores (dq, dk, dw).
constexpr int kBwdThreads = 512;
constexpr int kBwdKeyTile = 64;  // keys per LDS tile
constexpr int kDqQueries = 4;    // queries per dq unit (two waves per query, 32 heads each)
constexpr int kDkKeys = 256;     // keys per dk unit (32 per wave)
constexpr int kBwdMaxParts = 64;  // parts per key block (dk) or query tile (dq); fixed trees over them
constexpr int kBwdTargetUnits = 512;

struct BwdParams {
  const uint16_t* q;  // bf16 [T, H, D]
  const uint16_t* k;  // bf16 [Tkv, D]
  const float* w;     // fp32 [T, H]
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* offs;  // may be null
  const float* grad;    // fp32 rows of stride ld: dL/dI of the visible keys
  int64_t ld;
  float* dq;    // fp32 [T, H, D]
  float* dk;    // fp32 [Tkv, D]
  float* dw;    // fp32 [T, H]
  float* part;  // fp32 [dk_parts, Tkv, D] partial key gradients (unused when dk_parts == 1)
  uint32_t* ctrl;
  int32_t B, T, Tkv, Lmax;
  int32_t dk_parts;  // 1, 2, 4, .. 64, from bwd_dk_parts(Tkv)
  int32_t dq_parts;  // 1, 2, 4, .. 64, from bwd_dq_parts(T)
  float* part_q;     // fp32 [dq_parts, T, H, D] unscaled partial dq (dq_parts > 1)
  float* part_w;     // fp32 [dq_parts, T, H] partial dw (dq_parts > 1)
};

size_t bwd_dq_smem_bytes();
// Query parts per dk key block: a function of the number of keys only (about 512 units).
int bwd_dk_parts(int64_t total_k);
// Key-tile parts per dq query tile: a function of the number of queries only.
int bwd_dq_parts(int64_t total_q);
size_t bwd_dk_smem_bytes();
hipError_t bwd_prepare();
// `between` (may be null) is recorded after the dq/dw kernel.
hipError_t launch_backward(const BwdParams& p, int dq_grid, int dk_grid, int cus, hipStream_t s,
                           hipEvent_t between);

// Sparse attention over the selected ids (the selection's consumer).
constexpr int kAttnThreads = 256;
constexpr int kAttnTile = 64;    // ids per LDS tile
constexpr int kAttnHeads = 128;
constexpr int kAttnDqk = 576;    // latent row (key) dims
constexpr int kAttnDv = 512;     // value dims: the leading part of the latent row
constexpr uint32_t kStatusBadIds = 0x8u;

constexpr int kAttnSplitBlocks = 512;   // a batch with fewer blocks splits its rows' ids
constexpr int kAttnMaxSplit = 16;

struct AttnParams {
  const uint16_t* q;   // bf16 [T, 128, 576]
  const uint16_t* kv;  // bf16 [Tkv, 576]
  const int32_t* ids;  // [T, topk], -1 = none
  float* out;          // fp32 [T, 128, 512]
  float* lse;          // fp32 [T, 128]
  uint32_t* ctrl;
  float* part_o;       // split > 1: fp32 [T, split, 128, 512] unnormalised partial outputs
  float* part_ml;      // split > 1: fp32 [T, split, 128, 2] reference maximum (exp2 domain) and sum
  int32_t T, Tkv, topk, split;
  float scale;
};
// Number of parts each row's ids are split into (a function of the row count and topk only).
int attn_split(int T, int topk);
// Workspace bytes past the control block for the partial results (0 when split == 1).
size_t attn_partial_bytes(int T, int topk);
hipError_t launch_attention(const AttnParams& p, hipStream_t s);

// Dynamic LDS bytes of the score kernel for a tile table of `max_tiles` entries.
size_t score_smem_bytes(int B, int max_tiles);
size_t score_smem_limit();
hipError_t score_prepare(size_t max_smem);
hipError_t score_occupancy(int* blocks_per_cu, size_t smem);
hipError_t launch_score(const ScoreParams& p, int grid, size_t smem, hipStream_t s);
// Bytes of a prepared plan for B segments and a tile table of max_tiles entries (a multiple of 256).
size_t plan_bytes(int B, int max_tiles);
// One block: derives the plan of `p` for a score launch of `grid` blocks into `out` and zeroes
// p.ctrl.
hipError_t launch_plan(const ScoreParams& p, int grid, uint32_t* out, hipStream_t s);

// Resident blocks per CU of the select kernel variants (queried once per device).
struct SelectOccupancy {
  int narrow = 1;  // 256-thread rows
  int wide = 1;    // 1024-thread rows (batches with few rows)
};
hipError_t select_occupancy(SelectOccupancy* occ);
hipError_t launch_select(const SelectParams& p, int cus, const SelectOccupancy& occ, hipStream_t s);

hipError_t launch_ctrl_init(uint32_t* ctrl, hipStream_t s);

}  // namespace dsa
