/*
 * dsa_indexer.h — C ABI of the MI355X (gfx950) deterministic DSA indexer top-k scan.
 *
 * Operation (flashinfer PR #8691, "perf(cake_dsa_indexer_det): ticket scheduling on
 * sm_107a, no fill kernel in eager entry", description): BF16 queries and keys, FP32 head
 * weights and scores; for every query the scan returns the ids of its top-k keys; ids and
 * scores do not depend on how the work is partitioned or chunked; equal scores go to the
 * larger id.  The score itself is the lightning-indexer form (named by that page's
 * vendoring note, formula not printed there and adopted here):
 *
 *     I[t, s] = sum_{h < H} w[t, h] * max(0, sum_{d < D} q[t, h, d] * k[s, d])
 *
 * Segments and causality (same page, eager-entry tables: single causal documents, context
 * parallel tails, zigzag rank shares, split tails; causal query offsets of the eager entry):
 * segment b holds queries cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and keys
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.  Query t of segment b sits at position
 * p = q_pos_offsets[b] + (t - cu_seqlens_q[b]) and sees the first
 * n_t = min(max(p + 1, 0), len_k(b)) keys of its segment.
 *
 * Output row t: out_ids[t, 0 .. m-1] are the global key ids (row indices into k) of the
 * top m = min(topk, n_t) keys under the order (score descending, id descending), written in
 * ascending id order, out_scores[t, j] their FP32 scores (-0 is written as +0); slots
 * m .. topk-1 hold id -1 and score -inf (-1 is the "no key" marker of the sparse-index
 * consumer, flashinfer PR #4573 follow-ups).
 *
 * Determinism: every (t, s) score is computed by the same instruction sequence wherever
 * and in whichever work unit it is computed, and the selection is a pure function of the
 * row's scores, so outputs are bit-identical across runs, grid sizes, key chunkings,
 * query splits and segment packings.
 *
 * Conventions common to every call:
 *   - All data pointers are caller-owned DEVICE memory on the current HIP device.  The
 *     library allocates nothing, frees nothing and never synchronises the stream.
 *   - Tensors are dense row-major; q, k, w, out_* and workspace must be 16-byte aligned.
 *     q, w and out_* may be NULL when total_q is 0, and k when total_k is 0.
 *   - Host-side arguments are validated; device-resident tables (cu_seqlens, offsets) are
 *     validated by the kernel, which then skips the call's work and raises a status bit
 *     in the workspace (read with dsa_indexer_read_status) instead of touching memory out
 *     of bounds.
 *   - Calls are asynchronous on `stream`.  A workspace must not be used by two calls that
 *     can run concurrently.
 *   - Return value: DSA_OK (0) or a negative DSA_ERR_* code; nothing is enqueued on error.
 */
#ifndef DSA_INDEXER_H_
#define DSA_INDEXER_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DSA_OK 0
#define DSA_ERR_NULL (-1)       /* a required pointer is NULL                                  */
#define DSA_ERR_ALIGN (-2)      /* a pointer is not 16-byte aligned                            */
#define DSA_ERR_SHAPE (-3)      /* unsupported or inconsistent shape / topk                     */
#define DSA_ERR_WORKSPACE (-4)  /* workspace_bytes below dsa_indexer_workspace_size()          */
#define DSA_ERR_LAUNCH (-5)     /* a HIP launch failed; re-run dsa_indexer_workspace_init      */
#define DSA_ERR_DEVICE (-6)     /* current device is not gfx950 or cannot be queried           */
#define DSA_ERR_SCRATCH (-7)    /* dsa_indexer_topk_noalloc: the shape needs more than its fixed
                                   scratch (dsa_indexer_noalloc_max_bytes)                      */

/* Device status bits, left in the workspace control block by the kernels.  They are sticky
   (reporting only; cleared by dsa_indexer_workspace_init): whether a call's segment tables are
   valid is decided again by every call, so a call with invalid tables does not affect later
   calls on the same workspace. */
#define DSA_STATUS_CORRUPT_COUNTER 0x1u /* work-unit counter was not zero at entry          */
#define DSA_STATUS_BAD_SEGMENTS 0x2u    /* cu_seqlens not 0-based, non-decreasing, ending at T/Tkv */
#define DSA_STATUS_SEQLEN_BOUND 0x4u    /* a segment has more keys than max_seqlen_k; its
                                           queries see only its first max_seqlen_k keys  */
#define DSA_STATUS_BAD_IDS 0x8u         /* sparse attention: an id outside [-1, total_kv)
                                           (skipped like -1)                              */

/* Supported sizes. */
#define DSA_NUM_HEADS 64
#define DSA_HEAD_DIM 128
#define DSA_MAX_TOPK 2048
#define DSA_MAX_SEQLEN_K 65536

/* Host-side sizes; every field must be known without reading device memory. */
typedef struct dsa_indexer_shape {
  int32_t num_segments; /* B >= 1; cu_seqlens_* hold B+1 entries                              */
  int32_t total_q;      /* T >= 0: rows of q, w, out_ids, out_scores                          */
  int32_t total_k;      /* Tkv >= 0: rows of k                                                */
  int32_t num_heads;    /* H, must be 64                                                      */
  int32_t head_dim;     /* D, must be 128                                                     */
  int32_t max_seqlen_k; /* upper bound on any segment's key count, 1..65536; 0 = Tkv, which
                           must then be <= 65536 (DSA_ERR_SHAPE otherwise: a caller with more
                           keys states the bound)                                           */
} dsa_indexer_shape;

/*
 * Bytes of workspace the top-k call needs for `shape`: a 256-byte control block (work-unit
 * counter, exit counter, status word) followed by the score rows, T rows of
 * round_up(max_seqlen_k, 64) 32-bit words (order-preserving keys of the FP32 scores).
 * Returns 0 if the shape is invalid.
 */
size_t dsa_indexer_workspace_size(const dsa_indexer_shape* shape);

/*
 * Zero the workspace control block, on `stream` (a small fill kernel, no memset, so the call
 * can be captured in a graph).  Needed once per workspace before its first use, and again
 * after any call that returned DSA_ERR_LAUNCH (a kernel that did not run leaves the work-unit
 * counter where it stopped).  Every completed call leaves the counters at zero again, so
 * steady-state calls pay no reset; the sticky status bits are cleared only here.  Initialise and
 * call on the same stream, or order the two streams (the page's stream-ordering note for
 * prepared runners).
 */
int dsa_indexer_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The scan.  Enqueues the score kernel (persistent grid drawing work units from the
 * self-resetting counter in the workspace) and the per-row top-k select kernel on `stream`.
 * Two dispatches, not one fused scan program: the score kernel writes every visible score of a
 * query to a dense row in the workspace (the order-preserving 32-bit key of the FP32 score),
 * and the select kernel takes each row's exact top-k from it.  This is why the workspace holds
 * T rows of round_up(max_seqlen_k, 64) words (1 GiB for 16384 queries of 16384 keys) and why a
 * segment may hold at most 65536 keys; in exchange a query's keys can be split over work units
 * with no partial lists to merge and no waiting between blocks.
 *   q              bf16 [T, 64, 128]
 *   k              bf16 [Tkv, 128]
 *   w              fp32 [T, 64]
 *   cu_seqlens_q   int32 [B+1], 0 = cu[0] <= ... <= cu[B] = T
 *   cu_seqlens_k   int32 [B+1], 0 = cu[0] <= ... <= cu[B] = Tkv
 *   q_pos_offsets  int32 [B] causal position of each segment's first query, or NULL (all 0)
 *   topk           1 .. 2048
 *   out_ids        int32 [T, topk]   (fully overwritten)
 *   out_scores     fp32  [T, topk]   (fully overwritten)
 *   workspace      >= dsa_indexer_workspace_size(shape) bytes, initialised once
 */
int dsa_indexer_topk(const dsa_indexer_shape* shape, const void* q, const void* k, const float* w,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     const int32_t* q_pos_offsets, int32_t topk, int32_t* out_ids,
                     float* out_scores, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * Prepared runner (flashinfer PR #8691, description and commit messages: the prepared call form
 * beside the eager entry; the runner zeroes its ticket word once when it prepares and every
 * run leaves it at zero; a new runner is made when a shape or a tensor binding changes, values
 * may change freely; the prepare-time zero is queued on the prepare stream, so a run on another
 * stream must be ordered after it).
 *
 * dsa_indexer_prepare binds the shape, every tensor pointer, topk and a workspace of at least
 * dsa_indexer_prepared_workspace_size(shape) bytes (the top-k workspace followed by the plan).
 * It validates the arguments like dsa_indexer_topk (same error codes), then enqueues on `stream`
 * one small kernel that zeroes the workspace's control block (no dsa_indexer_workspace_init is
 * needed) and stores the work decomposition derived from the segment tables' current contents,
 * with a copy of those contents.  dsa_indexer_run enqueues only the scan's two kernels with the
 * arguments built at prepare time: no argument checks, no device queries.  Results are exactly
 * those of dsa_indexer_topk on the bound tensors' contents at the time of the run: the score
 * kernel compares the live segment tables with the stored copy and derives the plan itself if
 * they differ, so every value, the tables' included, may change between runs.
 *   - The runner owns no device memory; it must be destroyed with dsa_indexer_runner_destroy
 *     (host memory only).  The bound buffers must outlive it.
 *   - Runs of one runner (or of runners sharing a workspace) must not overlap.  After a run
 *     that returned DSA_ERR_LAUNCH, prepare again.
 *   - dsa_indexer_run_ex times the two kernels like dsa_indexer_topk_ex (profiler may be NULL).
 */
typedef struct dsa_indexer_runner dsa_indexer_runner;
size_t dsa_indexer_prepared_workspace_size(const dsa_indexer_shape* shape);
int dsa_indexer_prepare(const dsa_indexer_shape* shape, const void* q, const void* k, const float* w,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* q_pos_offsets, int32_t topk, int32_t* out_ids,
                        float* out_scores, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, dsa_indexer_runner** runner);
int dsa_indexer_run(dsa_indexer_runner* runner, hipStream_t stream);
int dsa_indexer_runner_destroy(dsa_indexer_runner* runner);

/*
 * dsa_indexer_topk for callers that cannot allocate device memory or own a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as dsa_indexer_topk, without the workspace: the control block and score
 * rows live in a fixed device array inside the library, one copy per GPU, held from the first
 * use of the library on that GPU until the process ends.  Nothing is allocated on any call.
 *   - A shape whose dsa_indexer_workspace_size exceeds dsa_indexer_noalloc_max_bytes()
 *     (256 bytes + 64 MiB: e.g. 4096 queries of up to 4096 keys, or 256 of 65536) returns
 *     DSA_ERR_SCRATCH and enqueues nothing.
 *   - Every call on a GPU uses that GPU's one array: calls that can overlap on one GPU (other
 *     streams, other threads) race and must be serialised by the caller.  The first call on a
 *     GPU, and the call after one that returned DSA_ERR_LAUNCH, also enqueue a small fill kernel
 *     that zeroes the array's counters; every other call enqueues only the scan's two kernels.
 */
int dsa_indexer_topk_noalloc(const dsa_indexer_shape* shape, const void* q, const void* k,
                             const float* w, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, const int32_t* q_pos_offsets,
                             int32_t topk, int32_t* out_ids, float* out_scores, hipStream_t stream);
/* Bytes of the fixed array dsa_indexer_topk_noalloc works in (the largest workspace size it accepts). */
size_t dsa_indexer_noalloc_max_bytes(void);

/*
 * Score phase only ("indexer logits"): writes I[t, cu_seqlens_k[b] + j] to
 * out_scores[t * ld_out + j] for every visible j < n_t and leaves every other element of
 * out_scores untouched.  ld_out >= max_seqlen_k, multiple of 4.  The workspace needs only
 * the 256-byte control block (and its init).
 */
int dsa_indexer_scores(const dsa_indexer_shape* shape, const void* q, const void* k,
                       const float* w, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       const int32_t* q_pos_offsets, float* out_scores, int64_t ld_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of the scores ("indexer logits backward", named beside the logits kernels in the
 * vendoring commit message of flashinfer PR #8691, which also fixes its determinism rules: no
 * floating-point atomics, key-side gradients summed from FP32 partials in a fixed tree).
 * With S[t,h,s] = q[t,h,:] . k[s,:] and g[t,j] = grad_scores[t * ld_grad + j], the upstream
 * gradient of I[t, cu_seqlens_k[b] + j] for the visible j < n_t (other elements are not read):
 *     dw[t,h]    = sum_j g[t,j] * max(0, S[t,h,s])
 *     dq[t,h,:]  = w[t,h] * sum_j g[t,j] * [S[t,h,s] > 0] * k[s,:]
 *     dk[s,:]    = sum over the queries t that see s, sum_h w[t,h] * g[t,j] * [S[t,h,s] > 0] * q[t,h,:]
 * (the ReLU's derivative at 0 is 0).  S is the FP32 product of the forward; the gradient
 * factors entering the matrix cores (g for dq, w * g for dk) are rounded to BF16, all sums
 * are FP32.
 *   grad_scores    fp32 rows of stride ld_grad (>= max_seqlen_k, multiple of 4): the layout
 *                  that dsa_indexer_scores writes
 *   dq             fp32 [T, 64, 128], dk fp32 [Tkv, 128], dw fp32 [T, 64]: fully overwritten
 *                  (keys no query sees and queries that see no key get zeros)
 *   workspace      >= dsa_indexer_backward_workspace_size(shape) bytes, initialised once
 *                  (dsa_indexer_workspace_init); holds the status word and, when total_k
 *                  (total_q) is small enough that key blocks (query tiles) alone cannot fill
 *                  the GPU, P FP32 partial key (query and weight) gradients per key (query),
 *                  P = 2 .. 64 a function of total_k (total_q) only
 * Bit-reproducible: every sum has a fixed order that depends only on the segment tables.
 * Invalid device tables (DSA_STATUS_BAD_SEGMENTS) leave the outputs untouched; a segment
 * longer than max_seqlen_k is flagged (DSA_STATUS_SEQLEN_BOUND) and its keys past the bound
 * get dk = 0, as in the forward.
 */
size_t dsa_indexer_backward_workspace_size(const dsa_indexer_shape* shape);
int dsa_indexer_backward(const dsa_indexer_shape* shape, const void* q, const void* k,
                         const float* w, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         const int32_t* q_pos_offsets, const float* grad_scores, int64_t ld_grad,
                         float* dq, float* dk, float* dw, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * The selection's consumer: sparse attention over each row's selected ids (flashinfer PR #4573
 * and its DeepSeek-V4 sparse-MLA decode follow-up: the kernel reads the selected key ids,
 * never dereferences -1, gathers those rows of the shared latent KV table and serves the value
 * operand from the gathered rows).  For query row t and head h, over the valid ids of row t
 * (0 <= id < total_kv; -1 and padding are skipped):
 *     S[h, j]   = scale * q[t, h, :] . kv[id_j, :]
 *     out[t, h, :] = sum_j softmax_j(S[h, :]) * kv[id_j, 0 .. 511]
 *     lse[t, h] = log sum_j exp(S[h, j])          (natural log)
 * A row without a valid id gets out = 0 and lse = -inf.
 *   q          bf16 [total_q, 128, 576]
 *   kv         bf16 [total_kv, 576]: latent rows, the value is the leading 512 dims
 *   ids        int32 [total_q, topk], 1 <= topk <= 2048 (e.g. out_ids of dsa_indexer_topk);
 *              an id outside [-1, total_kv) is skipped and raises DSA_STATUS_BAD_IDS
 *   out        fp32 [total_q, 128, 512], lse fp32 [total_q, 128]: fully overwritten
 *   workspace  dsa_indexer_sparse_attention_workspace_size(total_q, topk) bytes, 16-byte
 *              aligned, whose first 256 bytes are the control block (dsa_indexer_workspace_init)
 *              for the status word; a smaller workspace returns DSA_ERR_WORKSPACE
 * Scores are FP32 products of BF16 operands; the softmax runs in FP32 in the exp2 domain and
 * the probabilities are rounded to BF16 for the value product (FP32 accumulation).  Every sum
 * has a fixed order: results are bit-reproducible.  total_kv * 1152 and 2 * total_q must fit in
 * 31 bits (DSA_ERR_SHAPE otherwise).
 * A batch with few rows (fewer than 256) splits each row's ids over up to 16 blocks, which
 * write partial results (unnormalised output, reference maximum and sum per head) to the
 * workspace; a second dispatch combines the parts in a fixed order.  The split count is a
 * function of total_q and topk only: the bits of a row do not depend on the other rows' ids
 * but may differ in rounding between batch sizes with different split counts.
 */
#define DSA_ATTN_HEADS 128
#define DSA_ATTN_QK_DIM 576
#define DSA_ATTN_V_DIM 512
/* Workspace bytes for dsa_indexer_sparse_attention (0 for an unsupported topk). */
size_t dsa_indexer_sparse_attention_workspace_size(int32_t total_q, int32_t topk);
int dsa_indexer_sparse_attention(int32_t total_q, int32_t total_kv, int32_t topk, const void* q,
                                 const void* kv, const int32_t* ids, float scale, float* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Text of a DSA_ERR_* code. */
const char* dsa_indexer_status_string(int code);

/*
 * Tuning knobs, for tests and measurement only; results never depend on them.
 *   key_chunk_tiles  keys per work unit in tiles of 64 (0 = chosen from the shape)
 *   grid_blocks      persistent score-kernel grid size (0 = CUs x resident blocks per CU)
 */
typedef struct dsa_indexer_tuning {
  int32_t key_chunk_tiles;
  int32_t grid_blocks;
  int32_t reserved[6];
} dsa_indexer_tuning;

/*
 * Per-kernel timing with HIP events recorded on the call's stream around each kernel.
 * A profiler holds `capacity` call slots; dsa_indexer_profiler_read synchronises on the
 * recorded events, returns the summed durations in milliseconds and the number of calls,
 * and empties the slots.
 */
typedef struct dsa_indexer_profiler dsa_indexer_profiler;
int dsa_indexer_profiler_create(int32_t capacity, dsa_indexer_profiler** out);
int dsa_indexer_profiler_destroy(dsa_indexer_profiler* prof);
int dsa_indexer_profiler_read(dsa_indexer_profiler* prof, double* score_ms, double* select_ms,
                              int32_t* calls);
/*
 * Per-call form of dsa_indexer_profiler_read: synchronises, writes the score-kernel and
 * select-kernel milliseconds of each recorded call (oldest first) to score_ms[i] and
 * select_ms[i] for i < *calls (host arrays of `max_calls` floats; DSA_ERR_SHAPE if the
 * profiler holds more calls than that), and empties the slots.
 */
int dsa_indexer_profiler_read_calls(dsa_indexer_profiler* prof, float* score_ms, float* select_ms,
                                    int32_t max_calls, int32_t* calls);

/* dsa_indexer_topk with optional tuning (NULL = defaults) and optional profiler (NULL = none). */
int dsa_indexer_topk_ex(const dsa_indexer_shape* shape, const void* q, const void* k,
                        const float* w, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* q_pos_offsets, int32_t topk, int32_t* out_ids,
                        float* out_scores, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, const dsa_indexer_tuning* tuning,
                        dsa_indexer_profiler* profiler);

/* dsa_indexer_run with an optional profiler (NULL = none). */
int dsa_indexer_run_ex(dsa_indexer_runner* runner, hipStream_t stream, dsa_indexer_profiler* profiler);

/*
 * dsa_indexer_backward with an optional profiler: for backward calls the two figures a
 * profiler read returns are the dq/dw kernel and the dk kernels (partials + fixed-tree sum).
 */
int dsa_indexer_backward_ex(const dsa_indexer_shape* shape, const void* q, const void* k,
                            const float* w, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const int32_t* q_pos_offsets,
                            const float* grad_scores, int64_t ld_grad, float* dq, float* dk,
                            float* dw, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            dsa_indexer_profiler* profiler);

/*
 * Test helper: synchronise `stream`, then copy the control block's status word and the two
 * counters to the host.  Not for the hot path.
 */
int dsa_indexer_read_status(const void* workspace, hipStream_t stream, uint32_t* status,
                            uint32_t* ticket, uint32_t* done);

#ifdef __cplusplus
}
#endif

#endif /* DSA_INDEXER_H_ */
