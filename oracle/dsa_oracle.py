"""Plain FP64 CPU oracle for the deterministic DSA lightning-indexer top-k scan.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import or run this module.  The product package never
imports it, and it shares no code, table or helper with the HIP path.

Sources ("P1" below is flashinfer PR #8691, "perf(cake_dsa_indexer_det):
ticket scheduling on sm_107a, no fill kernel in eager entry"; "P3" is
flashinfer PR #4573, "feat(cake_sparse_mla): support SM100 and SM103"):

* Types and result (P1, description): queries and keys are BF16, head weights
  and scores FP32; for each query the scan returns the ids of its top-k keys;
  ids and scores must not depend on how the work is partitioned or chunked;
  equal scores are ordered by the larger id.
* What is scored (P1, the vendoring commit message naming the package's job
  as lightning-indexer scores plus deterministic exact top-k).  The pages do
  not print the formula; the oracle adopts the standard lightning-indexer
  definition
        I[t, s] = sum_h  w[t, h] * max(0, sum_d q[t, h, d] * k[s, d])
  with no extra scale (w carries any 1/sqrt(H)).
* Segments and causality (P1, eager-entry tables: "single causal document",
  "CP tail", "CP16 zigzag rank 0", "split tail" rows; and the causal query
  offsets the eager entry takes, commit message on the placeholder offsets):
  segment b holds queries cu_q[b]..cu_q[b+1]-1 and keys cu_k[b]..cu_k[b+1]-1;
  query t at position p = off[b] + (t - cu_q[b]) sees the first
  min(max(p+1, 0), len_k) keys of its segment (inclusive diagonal; positions
  past the segment end see the whole segment).
* Ids are global row indices into k.  Rows with fewer than k visible keys
  are padded with id -1 (the consumer's "no key" marker, P3 follow-up PRs on
  sparse-index consumption), and score -inf.
* Output order within a row: ascending id.

Readings where the pages are silent: the formula above with no extra scale;
an inclusive causal diagonal with positions past a segment's end seeing the
whole segment; one causal offset per segment (absent = 0); ids are global
row indices of k; each row lists its ids in ascending order; padding slots
hold id -1 and score -inf; -0 and +0 are the same score.

Backward of the scores (same package page, the vendoring commit message: the
deterministic package holds lightning-indexer logits kernels and their
backward, with no floating-point atomics and the key-side gradient reduced
from FP32 partials in a fixed tree).  The pages print no formula; the oracle
takes the plain chain rule of the score above.  Given g[t, j] = dL/dI[t, s]
for the visible keys s = first_t + j of query t (the layout of the scores
export: row t, column j):
        dw[t, h]    = sum_j g[t, j] * max(0, S[t, h, j])
        dq[t, h, :] = sum_j g[t, j] * w[t, h] * [S[t, h, j] > 0] * k[s, :]
        dk[s, :]    = sum_{t sees s} sum_h g[t, j] * w[t, h] * [S[t, h, j] > 0] * q[t, h, :]
with S[t, h, j] = q[t, h, :] . k[s, :].  The ReLU's derivative at exactly 0
is taken as 0 (the usual convention; the pages are silent).  Keys no query
sees get dk = 0, queries that see no key get dq = dw = 0.

Consumer of the selection (flashinfer PR #4573, "feat(cake_sparse_mla): support SM100 and
SM103", and its follow-up hardening the DeepSeek-V4 sparse-MLA decode path): for each query
row the attention reads the row's selected key ids, never dereferences -1, gathers those
rows of the shared latent KV table and attends over them; the value operand is served from
the gathered key rows (MLA: the value is the first dv dims of the same row).  The pages
print no formula; the oracle takes standard scaled-dot-product attention over the valid ids
of row t, for every head h:
        S[h, j] = scale * q[t, h, :] . kv[id_j, :]          (valid j: id_j >= 0)
        o[t, h, :] = sum_j softmax_j(S[h, :]) * kv[id_j, :dv]
        lse[t, h] = log sum_j exp(S[h, j])
A row with no valid id has o = 0 and lse = -inf.

Everything here is FP64: BF16 and FP32 inputs convert to FP64 exactly, the
dot products use a library matmul, the head reduction a library
matrix-vector product, and the selection a library lexicographic sort on
(score descending, id descending).  No blocking, fusion or reordering beyond
that.
"""
from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact BF16 -> FP64: a BF16 value is the upper half of an FP32 word."""
    b = np.ascontiguousarray(np.asarray(bits).astype(np.uint16)).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def from_torch(q, k, w):
    """Convert torch CPU tensors (q, k BF16; w FP32) into exact FP64 arrays."""
    import torch  # local: the oracle itself only needs numpy
    qb = q.contiguous().view(torch.int16).numpy().view(np.uint16)
    kb = k.contiguous().view(torch.int16).numpy().view(np.uint16)
    return bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), w.double().numpy()


def segment_of(cu_q: np.ndarray, t: int) -> int:
    """Index b of the segment holding query t (empty segments are skipped)."""
    return int(np.searchsorted(np.asarray(cu_q), t, side="right") - 1)


def visible(cu_q, cu_k, offs, t: int):
    """(first global key id, number of visible keys) for query t."""
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    b = segment_of(cu_q, t)
    o = 0 if offs is None else int(np.asarray(offs)[b])
    p = o + (t - int(cu_q[b]))
    len_k = int(cu_k[b + 1] - cu_k[b])
    n = min(max(p + 1, 0), len_k)
    return int(cu_k[b]), n


def row_scores(q64: np.ndarray, k64: np.ndarray, w64: np.ndarray, t: int, first: int, n: int) -> np.ndarray:
    """I[t, s] for the n keys s = first .. first+n-1, in FP64."""
    if n == 0:
        return np.zeros(0, dtype=np.float64)
    S = q64[t] @ k64[first:first + n].T          # [H, n]: per-head dot products
    return w64[t] @ np.maximum(S, 0.0)           # sum_h w[t,h] * ReLU(S[h, :])


def select_topk(scores: np.ndarray, ids: np.ndarray, topk: int):
    """Top-k under the total order (score desc, id desc); ids returned ascending, padded."""
    n = len(ids)
    m = min(topk, n)
    order = np.lexsort((-ids.astype(np.int64), -scores))   # primary: -score, secondary: -id
    take = order[:m]
    sel_ids = ids[take]
    sel_scores = scores[take]
    asc = np.argsort(sel_ids, kind="stable")
    out_ids = np.full(topk, -1, dtype=np.int64)
    out_scores = np.full(topk, NEG_INF, dtype=np.float64)
    out_ids[:m] = sel_ids[asc]
    out_scores[:m] = sel_scores[asc]
    return out_ids, out_scores


def topk_rows(q64, k64, w64, cu_q, cu_k, offs, topk: int, rows=None):
    """Oracle result for the given query rows (all rows if None).

    Returns (ids int64 [R, topk], scores f64 [R, topk], detail) where detail[r]
    holds the row's full visible score vector and first id, for tolerance checks.
    """
    T = q64.shape[0]
    rows = range(T) if rows is None else rows
    rows = list(rows)
    ids_out = np.full((len(rows), topk), -1, dtype=np.int64)
    sc_out = np.full((len(rows), topk), NEG_INF, dtype=np.float64)
    detail = []
    for r, t in enumerate(rows):
        first, n = visible(cu_q, cu_k, offs, t)
        s = row_scores(q64, k64, w64, t, first, n)
        ids = np.arange(first, first + n, dtype=np.int64)
        ids_out[r], sc_out[r] = select_topk(s, ids, topk)
        detail.append((first, s))
    return ids_out, sc_out, detail


def topk_workload(wl, rows=None):
    """Oracle on a generated workload (torch CPU tensors)."""
    q64, k64, w64 = from_torch(wl.q, wl.k, wl.w)
    cu_q = wl.cu_seqlens_q.numpy()
    cu_k = wl.cu_seqlens_k.numpy()
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    return topk_rows(q64, k64, w64, cu_q, cu_k, offs, wl.topk, rows)


def row_backward(q64, k64, w64, t: int, first: int, n: int, g: np.ndarray):
    """Query t's gradient terms for upstream gradients g[0..n-1] of its n visible scores.

    Returns (dq[t] [H, D], dw[t] [H], its contribution to dk[first .. first+n-1] [n, D]).
    """
    H, D = q64.shape[1], q64.shape[2]
    if n == 0:
        return np.zeros((H, D)), np.zeros(H), np.zeros((0, D))
    K = k64[first:first + n]                      # [n, D]
    S = q64[t] @ K.T                              # [H, n] per-head dot products
    on = S > 0.0                                  # ReLU derivative: 1 above zero, 0 at and below
    dw = np.maximum(S, 0.0) @ g                   # [H]
    G = np.where(on, w64[t][:, None] * g[None, :], 0.0)   # dL/dS [H, n]
    return G @ K, dw, G.T @ q64[t]


def backward_rows(q64, k64, w64, cu_q, cu_k, offs, grad):
    """dq [T, H, D], dk [Tkv, D], dw [T, H] in FP64 for upstream gradients grad[t, j] (j < n_t read)."""
    T, H, D = q64.shape
    dq = np.zeros((T, H, D))
    dw = np.zeros((T, H))
    dk = np.zeros((k64.shape[0], D))
    for t in range(T):
        first, n = visible(cu_q, cu_k, offs, t)
        g = np.asarray(grad[t, :n], dtype=np.float64)
        dq[t], dw[t], part = row_backward(q64, k64, w64, t, first, n, g)
        dk[first:first + n] += part
    return dq, dk, dw


def backward_workload(wl, grad):
    """Oracle backward on a generated workload; grad is a CPU FP32 tensor or array [T, >= n_t]."""
    q64, k64, w64 = from_torch(wl.q, wl.k, wl.w)
    g = grad.double().numpy() if hasattr(grad, "double") else np.asarray(grad, dtype=np.float64)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    return backward_rows(q64, k64, w64, wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy(), offs, g)


def sparse_attention_row(q64_t: np.ndarray, kv64: np.ndarray, ids_row, scale: float, dv: int):
    """o [H, dv] and lse [H] of one query row (q64_t [H, Dqk]) over its valid ids."""
    ids_row = np.asarray(ids_row, dtype=np.int64)
    valid = ids_row[ids_row >= 0]
    H = q64_t.shape[0]
    if valid.size == 0:
        return np.zeros((H, dv)), np.full(H, NEG_INF)
    K = kv64[valid]                                   # [m, Dqk] gathered rows
    S = scale * (q64_t @ K.T)                         # [H, m]
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    den = E.sum(axis=1, keepdims=True)
    o = (E / den) @ K[:, :dv]
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def sparse_attention_rows(q64, kv64, ids, scale: float, dv: int, rows=None):
    """o [R, H, dv], lse [R, H] for the given query rows (all if None); ids int [T, k], -1 = none."""
    T, H = q64.shape[0], q64.shape[1]
    rows = range(T) if rows is None else list(rows)
    rows = list(rows)
    o = np.zeros((len(rows), H, dv))
    lse = np.zeros((len(rows), H))
    for r, t in enumerate(rows):
        o[r], lse[r] = sparse_attention_row(q64[t], kv64, ids[t], scale, dv)
    return o, lse
