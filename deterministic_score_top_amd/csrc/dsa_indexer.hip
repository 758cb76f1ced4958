// Host side of the C ABI declared in include/dsa_indexer.h.
//
// Argument validation is host-only (it never reads device memory and never synchronises);
// each call enqueues exactly two kernels on the caller's stream -- the persistent score
// kernel and the per-row select kernel -- and nothing else: no allocation, no memset, no
// fill kernel (the eager entry of flashinfer PR #8691 launches only the scan's kernels).

#include "dsa_indexer.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string.h>
#include <vector>

#include "dsa_internal.h"

namespace {

// Fixed device memory of the entry point that allocates nothing (dsa_indexer_topk_noalloc): a
// control block and score rows, like a caller's workspace.  Each device the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device copy: kernels and fills take the per-device address from hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)dsa::kCtrlBytes + ((size_t)64 << 20);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceInfo {
  bool ok = false;
  int cus = 0;
  int score_blocks_per_cu = 0;  // at the smem limit (a lower bound for smaller tables)
  dsa::SelectOccupancy select;  // resident blocks per CU of each select variant
};

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
DeviceInfo g_info[kMaxDevices];
// Per device: the address of its copy of `scratch` (looked up once, with the device current)
// and whether its control block is known to be zero (cleared by the first no-allocation call on
// the device, and again after a call that failed to launch).
std::once_flag g_scratch_once[kMaxDevices];
unsigned char* g_scratch_ptr[kMaxDevices];
std::atomic<bool> g_scratch_clean[kMaxDevices];

unsigned char* scratch_of(int dev) {
  std::call_once(g_scratch_once[dev], [dev]() {
    void* sp = nullptr;
    if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = static_cast<unsigned char*>(sp);
  });
  return g_scratch_ptr[dev];
}

const DeviceInfo* device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev]() {
    DeviceInfo info;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return;
    info.cus = prop.multiProcessorCount;
    if (dsa::score_prepare(dsa::score_smem_limit()) != hipSuccess) return;
    int bpc = 0;
    if (dsa::score_occupancy(&bpc, dsa::score_smem_limit()) != hipSuccess || bpc < 1) return;
    if (dsa::bwd_prepare() != hipSuccess) return;
    if (dsa::select_occupancy(&info.select) != hipSuccess) return;
    info.score_blocks_per_cu = bpc;
    info.ok = true;
    g_info[dev] = info;
  });
  return g_info[dev].ok ? &g_info[dev] : nullptr;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Row length bound: max_seqlen_k, or total_k when it is 0 (check_shape keeps both <= 65536).
int64_t lmax_of(const dsa_indexer_shape* s) {
  int64_t L = s->max_seqlen_k > 0 ? s->max_seqlen_k : s->total_k;
  if (L < 1) L = 1;
  return L;
}

int64_t row_stride(const dsa_indexer_shape* s) {
  return (lmax_of(s) + dsa::kRowAlign - 1) / dsa::kRowAlign * dsa::kRowAlign;
}

int check_shape(const dsa_indexer_shape* s) {
  if (!s) return DSA_ERR_NULL;
  if (s->num_segments < 1 || s->total_q < 0 || s->total_k < 0) return DSA_ERR_SHAPE;
  if (s->num_heads != dsa::kHeads || s->head_dim != dsa::kDim) return DSA_ERR_SHAPE;
  if (s->max_seqlen_k < 0 || s->max_seqlen_k > dsa::kMaxSeqlenK) return DSA_ERR_SHAPE;
  // without a stated bound the bound is total_k, which must then be a supported row length
  // (a longer segment would otherwise be cut without an error)
  if (s->max_seqlen_k == 0 && s->total_k > dsa::kMaxSeqlenK) return DSA_ERR_SHAPE;
  return DSA_OK;
}

int max_tiles_of(const dsa_indexer_shape* s) {
  return (s->total_q + dsa::kTileQueries - 1) / dsa::kTileQueries + s->num_segments;
}

struct Call {
  const dsa_indexer_shape* shape;
  const void* q;
  const void* k;
  const float* w;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* offs;
  float* score_out;
  int64_t ld;
  uint32_t* ctrl;
  const dsa_indexer_tuning* tuning;
  int store_keys;
};

int launch_scores(const Call& c, hipStream_t stream) {
  const DeviceInfo* dev = device_info();
  if (!dev) return DSA_ERR_DEVICE;
  const dsa_indexer_shape* s = c.shape;
  const int max_tiles = max_tiles_of(s);
  const size_t smem = dsa::score_smem_bytes(s->num_segments, max_tiles);
  if (smem > dsa::score_smem_limit()) return DSA_ERR_SHAPE;

  const int64_t L = lmax_of(s);
  const int grid_default = dev->cus * dev->score_blocks_per_cu;
  int grid = grid_default;
  int chunk = 0;
  if (c.tuning) {
    if (c.tuning->grid_blocks < 0 || c.tuning->key_chunk_tiles < 0) return DSA_ERR_SHAPE;
    if (c.tuning->grid_blocks > 0) grid = c.tuning->grid_blocks;
    // the knob counts 64-key tiles; units hold whole kernel tiles
    chunk = (int)(((int64_t)c.tuning->key_chunk_tiles * 64 + dsa::kTileKeys - 1) / dsa::kTileKeys);
  }
  // chunk 0: the kernel picks the key chunk from the batch's total work (it alone reads the
  // segment tables)
  if ((int64_t)chunk * dsa::kTileKeys > (int64_t)1 << 30) return DSA_ERR_SHAPE;

  dsa::ScoreParams p;
  p.q = static_cast<const uint16_t*>(c.q);
  p.k = static_cast<const uint16_t*>(c.k);
  p.w = c.w;
  p.cu_q = c.cu_q;
  p.cu_k = c.cu_k;
  p.offs = c.offs;
  p.out = c.score_out;
  p.ld = c.ld;
  p.ctrl = c.ctrl;
  p.B = s->num_segments;
  p.T = s->total_q;
  p.Tkv = s->total_k;
  p.Lmax = (int32_t)L;
  p.chunk_tiles = chunk;
  p.max_tiles = max_tiles;
  p.store_keys = c.store_keys;
  p.plan = nullptr;
  if (dsa::launch_score(p, grid, smem, stream) != hipSuccess) return DSA_ERR_LAUNCH;
  return DSA_OK;
}

int check_inputs(const dsa_indexer_shape* shape, const void* q, const void* k, const float* w,
                 const int32_t* cu_q, const int32_t* cu_k, const int32_t* offs) {
  int rc = check_shape(shape);
  if (rc) return rc;
  // q and w may be NULL when there are no queries, k when there are no keys
  const bool has_q = shape->total_q > 0, has_k = shape->total_k > 0;
  if ((has_q && (!q || !w)) || (has_k && !k) || !cu_q || !cu_k) return DSA_ERR_NULL;
  if ((q && !aligned16(q)) || (k && !aligned16(k)) || (w && !aligned16(w))) return DSA_ERR_ALIGN;
  if (!aligned4(cu_q) || !aligned4(cu_k) || (offs && !aligned4(offs))) return DSA_ERR_ALIGN;
  return DSA_OK;
}

int check_common(const dsa_indexer_shape* shape, const void* q, const void* k, const float* w,
                 const int32_t* cu_q, const int32_t* cu_k, const int32_t* offs,
                 const void* workspace) {
  int rc = check_inputs(shape, q, k, w, cu_q, cu_k, offs);
  if (rc) return rc;
  if (!workspace) return DSA_ERR_NULL;
  if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  return DSA_OK;
}

int check_outputs(const dsa_indexer_shape* shape, int32_t topk, const int32_t* out_ids,
                  const float* out_scores) {
  if (topk < 1 || topk > dsa::kMaxTopk) return DSA_ERR_SHAPE;
  if (shape->total_q > 0 && (!out_ids || !out_scores)) return DSA_ERR_NULL;
  if ((out_ids && !aligned16(out_ids)) || (out_scores && !aligned16(out_scores))) return DSA_ERR_ALIGN;
  return DSA_OK;
}

}  // namespace

struct dsa_indexer_profiler {
  int capacity = 0;
  int used = 0;
  std::vector<hipEvent_t> ev;  // 3 per slot: before score, between, after select
};

// A prepared runner: both kernels' arguments built once, the plan stored in the workspace.
struct dsa_indexer_runner {
  dsa::ScoreParams score;
  dsa::SelectParams select;
  int grid = 0;
  size_t smem = 0;
  int cus = 0;
  dsa::SelectOccupancy occ;
  int total_q = 0;
};

namespace {

// The two kernels of the scan on a validated call; `ws` is a control block followed by the
// score rows (a caller's workspace or this device's scratch).
int enqueue_topk(const DeviceInfo* dev, const dsa_indexer_shape* shape, const void* q, const void* k,
                 const float* w, const int32_t* cu_q, const int32_t* cu_k, const int32_t* offs,
                 int32_t topk, int32_t* out_ids, float* out_scores, unsigned char* ws,
                 hipStream_t stream, const dsa_indexer_tuning* tuning, dsa_indexer_profiler* profiler) {
  uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws);
  float* scores = reinterpret_cast<float*>(ws + dsa::kCtrlBytes);
  const int64_t ld = row_stride(shape);
  hipEvent_t* ev = profiler ? &profiler->ev[3 * profiler->used] : nullptr;

  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return DSA_ERR_LAUNCH;
  Call c{shape, q, k, w, cu_q, cu_k, offs, scores, ld, ctrl, tuning, 1};
  int rc = launch_scores(c, stream);
  if (rc) return rc;
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return DSA_ERR_LAUNCH;

  dsa::SelectParams sp;
  sp.keys = reinterpret_cast<const uint32_t*>(scores);
  sp.ld = ld;
  sp.cu_q = cu_q;
  sp.cu_k = cu_k;
  sp.offs = offs;
  sp.out_ids = out_ids;
  sp.out_scores = out_scores;
  sp.ctrl = ctrl;
  sp.B = shape->num_segments;
  sp.T = shape->total_q;
  sp.Tkv = shape->total_k;
  sp.Lmax = (int32_t)lmax_of(shape);
  sp.topk = topk;
  if (dsa::launch_select(sp, dev->cus, dev->select, stream) != hipSuccess) return DSA_ERR_LAUNCH;
  if (ev) {
    if (hipEventRecord(ev[2], stream) != hipSuccess) return DSA_ERR_LAUNCH;
    profiler->used++;
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

size_t dsa_indexer_workspace_size(const dsa_indexer_shape* shape) {
  if (check_shape(shape) != DSA_OK) return 0;
  return (size_t)dsa::kCtrlBytes + (size_t)shape->total_q * (size_t)row_stride(shape) * 4u;
}

int dsa_indexer_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return DSA_ERR_NULL;
  if (!aligned16(workspace)) return DSA_ERR_ALIGN;
  if (workspace_bytes < (size_t)dsa::kCtrlBytes) return DSA_ERR_WORKSPACE;
  if (!device_info()) return DSA_ERR_DEVICE;
  if (dsa::launch_ctrl_init(static_cast<uint32_t*>(workspace), stream) != hipSuccess)
    return DSA_ERR_LAUNCH;
  return DSA_OK;
}

int dsa_indexer_topk_ex(const dsa_indexer_shape* shape, const void* q, const void* k,
                        const float* w, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* q_pos_offsets, int32_t topk, int32_t* out_ids,
                        float* out_scores, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, const dsa_indexer_tuning* tuning,
                        dsa_indexer_profiler* profiler) {
  int rc = check_common(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, workspace);
  if (rc) return rc;
  rc = check_outputs(shape, topk, out_ids, out_scores);
  if (rc) return rc;
  if (workspace_bytes < dsa_indexer_workspace_size(shape)) return DSA_ERR_WORKSPACE;
  const DeviceInfo* dev = device_info();
  if (!dev) return DSA_ERR_DEVICE;
  if (profiler && profiler->used >= profiler->capacity) return DSA_ERR_SHAPE;
  if (shape->total_q == 0) return DSA_OK;
  return enqueue_topk(dev, shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, topk, out_ids,
                      out_scores, static_cast<unsigned char*>(workspace), stream, tuning, profiler);
}

int dsa_indexer_topk(const dsa_indexer_shape* shape, const void* q, const void* k, const float* w,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     const int32_t* q_pos_offsets, int32_t topk, int32_t* out_ids,
                     float* out_scores, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  return dsa_indexer_topk_ex(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, topk,
                             out_ids, out_scores, workspace, workspace_bytes, stream, nullptr,
                             nullptr);
}

int dsa_indexer_scores(const dsa_indexer_shape* shape, const void* q, const void* k,
                       const float* w, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       const int32_t* q_pos_offsets, float* out_scores, int64_t ld_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_common(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, workspace);
  if (rc) return rc;
  if (!out_scores) return DSA_ERR_NULL;
  if (!aligned16(out_scores)) return DSA_ERR_ALIGN;
  if (ld_out < lmax_of(shape) || (ld_out & 3)) return DSA_ERR_SHAPE;
  if (workspace_bytes < (size_t)dsa::kCtrlBytes) return DSA_ERR_WORKSPACE;
  if (shape->total_q == 0) return DSA_OK;
  Call c{shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, out_scores, ld_out,
         static_cast<uint32_t*>(workspace), nullptr, 0};
  return launch_scores(c, stream);
}

size_t dsa_indexer_prepared_workspace_size(const dsa_indexer_shape* shape) {
  const size_t base = dsa_indexer_workspace_size(shape);
  if (base == 0) return 0;
  return base + dsa::plan_bytes(shape->num_segments, max_tiles_of(shape));
}

int dsa_indexer_prepare(const dsa_indexer_shape* shape, const void* q, const void* k, const float* w,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* q_pos_offsets, int32_t topk, int32_t* out_ids,
                        float* out_scores, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, dsa_indexer_runner** runner) {
  if (!runner) return DSA_ERR_NULL;
  *runner = nullptr;
  int rc = check_common(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, workspace);
  if (rc) return rc;
  rc = check_outputs(shape, topk, out_ids, out_scores);
  if (rc) return rc;
  if (workspace_bytes < dsa_indexer_prepared_workspace_size(shape)) return DSA_ERR_WORKSPACE;
  const DeviceInfo* dev = device_info();
  if (!dev) return DSA_ERR_DEVICE;
  const int max_tiles = max_tiles_of(shape);
  const size_t smem = dsa::score_smem_bytes(shape->num_segments, max_tiles);
  if (smem > dsa::score_smem_limit()) return DSA_ERR_SHAPE;

  unsigned char* const ws = static_cast<unsigned char*>(workspace);
  const int64_t ld = row_stride(shape);
  uint32_t* const plan = reinterpret_cast<uint32_t*>(ws + dsa_indexer_workspace_size(shape));
  dsa_indexer_runner* r = new dsa_indexer_runner();
  r->grid = dev->cus * dev->score_blocks_per_cu;
  r->smem = smem;
  r->cus = dev->cus;
  r->occ = dev->select;
  r->total_q = shape->total_q;
  dsa::ScoreParams& p = r->score;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.w = w;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.offs = q_pos_offsets;
  p.out = reinterpret_cast<float*>(ws + dsa::kCtrlBytes);
  p.ld = ld;
  p.ctrl = reinterpret_cast<uint32_t*>(ws);
  p.B = shape->num_segments;
  p.T = shape->total_q;
  p.Tkv = shape->total_k;
  p.Lmax = (int32_t)lmax_of(shape);
  p.chunk_tiles = 0;
  p.max_tiles = max_tiles;
  p.store_keys = 1;
  p.plan = plan;
  dsa::SelectParams& sp = r->select;
  sp.keys = reinterpret_cast<const uint32_t*>(p.out);
  sp.ld = ld;
  sp.cu_q = cu_seqlens_q;
  sp.cu_k = cu_seqlens_k;
  sp.offs = q_pos_offsets;
  sp.out_ids = out_ids;
  sp.out_scores = out_scores;
  sp.ctrl = p.ctrl;
  sp.B = shape->num_segments;
  sp.T = shape->total_q;
  sp.Tkv = shape->total_k;
  sp.Lmax = p.Lmax;
  sp.topk = topk;
  if (dsa::launch_plan(p, r->grid, plan, stream) != hipSuccess) {
    delete r;
    return DSA_ERR_LAUNCH;
  }
  *runner = r;
  return DSA_OK;
}

int dsa_indexer_run_ex(dsa_indexer_runner* runner, hipStream_t stream, dsa_indexer_profiler* profiler) {
  if (!runner) return DSA_ERR_NULL;
  if (profiler && profiler->used >= profiler->capacity) return DSA_ERR_SHAPE;
  if (runner->total_q == 0) return DSA_OK;
  hipEvent_t* ev = profiler ? &profiler->ev[3 * profiler->used] : nullptr;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return DSA_ERR_LAUNCH;
  if (dsa::launch_score(runner->score, runner->grid, runner->smem, stream) != hipSuccess) return DSA_ERR_LAUNCH;
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return DSA_ERR_LAUNCH;
  if (dsa::launch_select(runner->select, runner->cus, runner->occ, stream) != hipSuccess) return DSA_ERR_LAUNCH;
  if (ev) {
    if (hipEventRecord(ev[2], stream) != hipSuccess) return DSA_ERR_LAUNCH;
    profiler->used++;
  }
  return DSA_OK;
}

int dsa_indexer_run(dsa_indexer_runner* runner, hipStream_t stream) {
  return dsa_indexer_run_ex(runner, stream, nullptr);
}

int dsa_indexer_runner_destroy(dsa_indexer_runner* runner) {
  if (!runner) return DSA_ERR_NULL;
  delete runner;
  return DSA_OK;
}

size_t dsa_indexer_noalloc_max_bytes(void) { return kScratchBytes; }

int dsa_indexer_topk_noalloc(const dsa_indexer_shape* shape, const void* q, const void* k,
                             const float* w, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, const int32_t* q_pos_offsets,
                             int32_t topk, int32_t* out_ids, float* out_scores, hipStream_t stream) {
  int rc = check_inputs(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets);
  if (rc) return rc;
  rc = check_outputs(shape, topk, out_ids, out_scores);
  if (rc) return rc;
  if (dsa_indexer_workspace_size(shape) > kScratchBytes) return DSA_ERR_SCRATCH;
  int dev_id = 0;
  if (hipGetDevice(&dev_id) != hipSuccess || dev_id < 0 || dev_id >= kMaxDevices) return DSA_ERR_DEVICE;
  const DeviceInfo* dev = device_info();
  if (!dev) return DSA_ERR_DEVICE;
  unsigned char* const ws = scratch_of(dev_id);
  if (!ws) return DSA_ERR_DEVICE;
  if (shape->total_q == 0) return DSA_OK;
  // The counters must be zero at entry: every completed call leaves them so, the first call on
  // the device clears them (a fill kernel on this stream), and so does the call after a failed
  // launch.
  if (!g_scratch_clean[dev_id].load()) {
    if (dsa::launch_ctrl_init(reinterpret_cast<uint32_t*>(ws), stream) != hipSuccess)
      return DSA_ERR_LAUNCH;
    g_scratch_clean[dev_id].store(true);
  }
  rc = enqueue_topk(dev, shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, topk, out_ids,
                    out_scores, ws, stream, nullptr, nullptr);
  if (rc == DSA_ERR_LAUNCH) g_scratch_clean[dev_id].store(false);
  return rc;
}

const char* dsa_indexer_status_string(int code) {
  switch (code) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case DSA_ERR_SHAPE: return "unsupported or inconsistent shape";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_LAUNCH: return "HIP launch failed (re-initialise the workspace)";
    case DSA_ERR_DEVICE: return "current device is not gfx950";
    case DSA_ERR_SCRATCH:
      return "the shape needs more than the fixed scratch of the no-allocation entry point "
             "(dsa_indexer_noalloc_max_bytes)";
    default: return "unknown status";
  }
}

int dsa_indexer_profiler_create(int32_t capacity, dsa_indexer_profiler** out) {
  if (!out) return DSA_ERR_NULL;
  if (capacity < 1) return DSA_ERR_SHAPE;
  dsa_indexer_profiler* p = new dsa_indexer_profiler();
  p->capacity = capacity;
  p->ev.resize((size_t)capacity * 3);
  for (auto& e : p->ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      dsa_indexer_profiler_destroy(p);
      return DSA_ERR_DEVICE;
    }
  }
  *out = p;
  return DSA_OK;
}

int dsa_indexer_profiler_destroy(dsa_indexer_profiler* prof) {
  if (!prof) return DSA_ERR_NULL;
  for (auto& e : prof->ev)
    if (e) (void)hipEventDestroy(e);
  delete prof;
  return DSA_OK;
}

int dsa_indexer_profiler_read_calls(dsa_indexer_profiler* prof, float* score_ms, float* select_ms,
                                    int32_t max_calls, int32_t* calls) {
  if (!prof || !score_ms || !select_ms || !calls) return DSA_ERR_NULL;
  if (prof->used > max_calls) return DSA_ERR_SHAPE;
  for (int i = 0; i < prof->used; ++i) {
    hipEvent_t* e = &prof->ev[3 * i];
    if (hipEventSynchronize(e[2]) != hipSuccess) return DSA_ERR_LAUNCH;
    if (hipEventElapsedTime(&score_ms[i], e[0], e[1]) != hipSuccess) return DSA_ERR_LAUNCH;
    if (hipEventElapsedTime(&select_ms[i], e[1], e[2]) != hipSuccess) return DSA_ERR_LAUNCH;
  }
  *calls = prof->used;
  prof->used = 0;
  return DSA_OK;
}

int dsa_indexer_profiler_read(dsa_indexer_profiler* prof, double* score_ms, double* select_ms,
                              int32_t* calls) {
  if (!prof || !score_ms || !select_ms || !calls) return DSA_ERR_NULL;
  double a = 0.0, b = 0.0;
  for (int i = 0; i < prof->used; ++i) {
    hipEvent_t* e = &prof->ev[3 * i];
    if (hipEventSynchronize(e[2]) != hipSuccess) return DSA_ERR_LAUNCH;
    float x = 0.f, y = 0.f;
    if (hipEventElapsedTime(&x, e[0], e[1]) != hipSuccess) return DSA_ERR_LAUNCH;
    if (hipEventElapsedTime(&y, e[1], e[2]) != hipSuccess) return DSA_ERR_LAUNCH;
    a += x;
    b += y;
  }
  *score_ms = a;
  *select_ms = b;
  *calls = prof->used;
  prof->used = 0;
  return DSA_OK;
}

size_t dsa_indexer_backward_workspace_size(const dsa_indexer_shape* shape) {
  if (check_shape(shape) != DSA_OK) return 0;
  const int pk = dsa::bwd_dk_parts(shape->total_k), pq = dsa::bwd_dq_parts(shape->total_q);
  size_t n = (size_t)dsa::kCtrlBytes;
  if (pk > 1) n += (size_t)pk * (size_t)shape->total_k * dsa::kDim * 4u;
  if (pq > 1) n += (size_t)pq * (size_t)shape->total_q * (dsa::kHeads * dsa::kDim + dsa::kHeads) * 4u;
  return n;
}

int dsa_indexer_backward_ex(const dsa_indexer_shape* shape, const void* q, const void* k,
                            const float* w, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const int32_t* q_pos_offsets,
                            const float* grad_scores, int64_t ld_grad, float* dq, float* dk,
                            float* dw, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            dsa_indexer_profiler* profiler) {
  int rc = check_common(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, workspace);
  if (rc) return rc;
  const bool has_q = shape->total_q > 0, has_k = shape->total_k > 0;
  if ((has_q && (!grad_scores || !dq || !dw)) || (has_k && !dk)) return DSA_ERR_NULL;
  if ((grad_scores && !aligned16(grad_scores)) || (dq && !aligned16(dq)) || (dk && !aligned16(dk)) ||
      (dw && !aligned16(dw)))
    return DSA_ERR_ALIGN;
  if (ld_grad < lmax_of(shape) || (ld_grad & 3)) return DSA_ERR_SHAPE;
  if (workspace_bytes < dsa_indexer_backward_workspace_size(shape)) return DSA_ERR_WORKSPACE;
  const DeviceInfo* dev = device_info();
  if (!dev) return DSA_ERR_DEVICE;
  if (profiler && profiler->used >= profiler->capacity) return DSA_ERR_SHAPE;
  if (!has_q && !has_k) return DSA_OK;

  dsa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.w = w;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.offs = q_pos_offsets;
  p.grad = grad_scores;
  p.ld = ld_grad;
  p.dq = dq;
  p.dk = dk;
  p.dw = dw;
  p.part = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + dsa::kCtrlBytes);
  p.ctrl = static_cast<uint32_t*>(workspace);
  p.B = shape->num_segments;
  p.T = shape->total_q;
  p.Tkv = shape->total_k;
  p.Lmax = (int32_t)lmax_of(shape);
  p.dk_parts = dsa::bwd_dk_parts(shape->total_k);
  p.dq_parts = dsa::bwd_dq_parts(shape->total_q);
  {
    // workspace: control block | dk partials (dk_parts > 1) | dq partials, dw partials (dq_parts > 1)
    float* cur = p.part + (p.dk_parts > 1 ? (int64_t)p.dk_parts * shape->total_k * dsa::kDim : 0);
    p.part_q = cur;
    cur += p.dq_parts > 1 ? (int64_t)p.dq_parts * shape->total_q * dsa::kHeads * dsa::kDim : 0;
    p.part_w = cur;
  }
  // unit counts are at most these bounds; blocks past the last unit leave at once
  const int64_t dq_grid =
      has_q ? ((int64_t)(shape->total_q + dsa::kDqQueries - 1) / dsa::kDqQueries + shape->num_segments) * p.dq_parts : 0;
  const int64_t dk_grid = has_k ? ((int64_t)(shape->total_k + dsa::kDkKeys - 1) / dsa::kDkKeys + shape->num_segments) * p.dk_parts : 0;
  if (dq_grid > INT32_MAX || dk_grid > INT32_MAX) return DSA_ERR_SHAPE;

  hipEvent_t* ev = profiler ? &profiler->ev[3 * profiler->used] : nullptr;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return DSA_ERR_LAUNCH;
  if (dsa::launch_backward(p, (int)dq_grid, (int)dk_grid, dev->cus, stream, ev ? ev[1] : nullptr) != hipSuccess)
    return DSA_ERR_LAUNCH;
  if (ev) {
    if (hipEventRecord(ev[2], stream) != hipSuccess) return DSA_ERR_LAUNCH;
    profiler->used++;
  }
  return DSA_OK;
}

int dsa_indexer_backward(const dsa_indexer_shape* shape, const void* q, const void* k,
                         const float* w, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         const int32_t* q_pos_offsets, const float* grad_scores, int64_t ld_grad,
                         float* dq, float* dk, float* dw, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  return dsa_indexer_backward_ex(shape, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets,
                                 grad_scores, ld_grad, dq, dk, dw, workspace, workspace_bytes,
                                 stream, nullptr);
}

size_t dsa_indexer_sparse_attention_workspace_size(int32_t total_q, int32_t topk) {
  if (total_q < 0 || topk < 1 || topk > dsa::kMaxTopk) return 0;
  return (size_t)dsa::kCtrlBytes + dsa::attn_partial_bytes(total_q, topk);
}

int dsa_indexer_sparse_attention(int32_t total_q, int32_t total_kv, int32_t topk, const void* q,
                                 const void* kv, const int32_t* ids, float scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (total_q < 0 || total_kv < 0 || topk < 1 || topk > dsa::kMaxTopk) return DSA_ERR_SHAPE;
  if ((int64_t)total_kv * dsa::kAttnDqk * 2 > INT32_MAX) return DSA_ERR_SHAPE;
  // two blocks per row (times the split count): the grid must fit a 31-bit block count
  if ((int64_t)total_q * 2 * dsa::attn_split(total_q, topk) > INT32_MAX) return DSA_ERR_SHAPE;
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f) return DSA_ERR_SHAPE;
  if (!workspace || (total_q > 0 && (!q || !ids || !out || !lse)) || (total_kv > 0 && !kv)) return DSA_ERR_NULL;
  if (!aligned16(workspace) || (q && !aligned16(q)) || (kv && !aligned16(kv)) || (out && !aligned16(out)) ||
      (lse && !aligned16(lse)) || (ids && !aligned4(ids)))
    return DSA_ERR_ALIGN;
  if (workspace_bytes < dsa_indexer_sparse_attention_workspace_size(total_q, topk)) return DSA_ERR_WORKSPACE;
  if (!device_info()) return DSA_ERR_DEVICE;
  if (total_q == 0) return DSA_OK;
  dsa::AttnParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.kv = static_cast<const uint16_t*>(kv);
  p.ids = ids;
  p.out = out;
  p.lse = lse;
  p.ctrl = static_cast<uint32_t*>(workspace);
  p.T = total_q;
  p.Tkv = total_kv;
  p.topk = topk;
  p.split = dsa::attn_split(total_q, topk);
  p.scale = scale;
  unsigned char* const part = static_cast<unsigned char*>(workspace) + dsa::kCtrlBytes;
  p.part_o = p.split > 1 ? reinterpret_cast<float*>(part) : nullptr;
  p.part_ml = p.split > 1 ? reinterpret_cast<float*>(part + (size_t)total_q * p.split * dsa::kAttnHeads *
                                                                dsa::kAttnDv * 4u)
                          : nullptr;
  if (dsa::launch_attention(p, stream) != hipSuccess) return DSA_ERR_LAUNCH;
  return DSA_OK;
}

int dsa_indexer_read_status(const void* workspace, hipStream_t stream, uint32_t* status,
                            uint32_t* ticket, uint32_t* done) {
  if (!workspace || !status || !ticket || !done) return DSA_ERR_NULL;
  if (hipStreamSynchronize(stream) != hipSuccess) return DSA_ERR_LAUNCH;
  uint32_t h[4] = {0, 0, 0, 0};
  if (hipMemcpy(h, workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return DSA_ERR_LAUNCH;
  *ticket = h[dsa::kCtrlTicket];
  *done = h[dsa::kCtrlDone];
  *status = h[dsa::kCtrlStatus];
  return DSA_OK;
}

}  // extern "C"
