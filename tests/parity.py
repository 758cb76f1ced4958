"""Acceptance rule for GPU rows against the FP64 oracle.

For query row t with visible keys V_t (n = |V_t|, m = min(topk, n)):
  tau   = 1e-4 * max_{s in V_t} |I_oracle[t, s]|
  theta = the oracle's m-th score
  (i)   every returned (id, score): |score - I_oracle[t, id]| <= tau
  (ii)  ids unique, inside V_t, exactly m of them, then -1 / -inf padding
  (iii) ids in the symmetric difference with the oracle's set have
        |I_oracle[t, s] - theta| <= tau (only near-ties may swap)
  (iv)  ids ascending
With exact=True (integer-valued inputs whose FP32 arithmetic is exact) the
scores must equal the oracle's bit for bit and the id sets must be identical.
"""
import numpy as np

REL_TOL = 1e-4


def check_rows(gpu_ids, gpu_scores, rows, oracle_ids, oracle_scores, detail, topk, exact=False):
    gpu_ids = np.asarray(gpu_ids)
    gpu_scores = np.asarray(gpu_scores)
    bad = []
    for r, t in enumerate(rows):
        first, s_all = detail[r]
        n = len(s_all)
        m = min(topk, n)
        gi = gpu_ids[t].astype(np.int64)
        gs = gpu_scores[t].astype(np.float64)
        try:
            assert np.all(gi[m:] == -1), "padding ids"
            assert np.all(np.isneginf(gs[m:])), "padding scores"
            ids = gi[:m]
            assert np.all(np.diff(ids) > 0), "ids not strictly ascending"
            assert np.all((ids >= first) & (ids < first + n)), "id outside the visible range"
            if m == 0:
                continue
            ref = s_all[ids - first]
            if exact:
                assert np.array_equal(ids, oracle_ids[r][:m]), "id set differs (exact inputs)"
                assert np.array_equal(gs[:m], ref.astype(np.float32).astype(np.float64)), "scores differ (exact)"
                continue
            tau = REL_TOL * float(np.max(np.abs(s_all)))
            err = np.abs(gs[:m] - ref)
            assert np.all(err <= tau), f"score error {err.max():.3g} > tau {tau:.3g}"
            theta = float(np.min(oracle_scores[r][:m]))
            diff = set(ids.tolist()) ^ set(oracle_ids[r][:m].tolist())
            for s in diff:
                assert abs(s_all[s - first] - theta) <= tau, f"id {s} swapped outside the tie band"
        except AssertionError as e:
            bad.append((t, str(e)))
    assert not bad, f"{len(bad)} bad rows, first: {bad[:3]}"


def backward_row_bounds(q64, k64, w64, g, t, first, n):
    """Error bounds of the GPU backward for query t's row (FP64 arrays, g = the row's n upstream
    gradients): (dq [H, D], dw [H], dk terms [n, D] before the accumulation factor, dk mask-flip
    terms [n, D]).

    The GPU rounds the gradient factor of each product to BF16 (relative error <= 2^-8), sums
    m terms in FP32 (<= m * 2^-24 of the sum of |terms|), and computes S in FP32 from exact
    BF16 products (|error| <= 2^-17 * sum|q k|); where |S| is within 2^-16 * sum|q k| of zero
    the ReLU mask may differ, so those terms enter the bound whole.
    """
    U = 2.0 ** -24
    K = k64[first:first + n]
    ag = np.abs(g)
    aK, aq, aw = np.abs(K), np.abs(q64[t]), np.abs(w64[t])
    S = q64[t] @ K.T
    eps = 2.0 ** -16 * (aq @ aK.T)
    amb = np.abs(S) <= eps
    f = 2.0 ** -8 + (n + 10) * U
    bq = aw[:, None] * (f * (ag @ aK)[None, :] + (amb * ag[None, :]) @ aK)
    bw = eps @ ag + (n + 10) * U * (np.abs(S) @ ag)
    return bq, bw, ag[:, None] * (aw @ aq)[None, :], ag[:, None] * ((amb * aw[:, None]).T @ aq)
