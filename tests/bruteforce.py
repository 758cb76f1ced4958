"""Exact brute force for tiny inputs: rational arithmetic and a full sort.

Independent of the oracle's route: pure-Python loops over (query, key, head,
dim) with fractions.Fraction (no floating point at all), a linear scan for
the segment, and Python's sort over (score, id) tuples in descending order,
which is the total order "score descending, then id descending".
"""
from fractions import Fraction


def exact_values(t):
    """Exact rationals of a CPU torch tensor (BF16/FP32 values are exact in FP64)."""
    return [[Fraction(float(x)) for x in row] for row in t.double().reshape(t.shape[0], -1).tolist()]


def brute_topk(q, k, w, cu_q, cu_k, offs, topk, H, D):
    """q: [T][H*D] Fractions; k: [Tkv][D]; w: [T][H]; returns (ids, scores) lists per row."""
    T = len(q)
    B = len(cu_q) - 1
    out = []
    for t in range(T):
        b = None
        for bb in range(B):
            if cu_q[bb] <= t < cu_q[bb + 1]:
                b = bb
                break
        pos = (0 if offs is None else offs[b]) + t - cu_q[b]
        nk = cu_k[b + 1] - cu_k[b]
        n = pos + 1
        if n > nk:
            n = nk
        if n < 0:
            n = 0
        cand = []
        for j in range(n):
            s = cu_k[b] + j
            total = Fraction(0)
            for h in range(H):
                dot = Fraction(0)
                for d in range(D):
                    dot += q[t][h * D + d] * k[s][d]
                if dot > 0:
                    total += w[t][h] * dot
            cand.append((total, s))
        cand.sort(reverse=True)
        kept = sorted(cand[:topk], key=lambda x: x[1])
        ids = [s for _, s in kept] + [-1] * (topk - len(kept))
        scores = [v for v, _ in kept] + [None] * (topk - len(kept))
        out.append((ids, scores))
    return out


def visible_count(cu_q, cu_k, offs, t):
    """(segment, first key id, visible key count) of query t, by a linear scan."""
    for b in range(len(cu_q) - 1):
        if cu_q[b] <= t < cu_q[b + 1]:
            pos = (0 if offs is None else offs[b]) + t - cu_q[b]
            nk = cu_k[b + 1] - cu_k[b]
            return b, cu_k[b], max(0, min(pos + 1, nk))
    raise ValueError(t)


def exact_dots(q, k, cu_q, cu_k, offs, H, D):
    """Every visible per-head dot product, exactly: {(t, h, s): Fraction}."""
    out = {}
    for t in range(len(q)):
        _, first, n = visible_count(cu_q, cu_k, offs, t)
        for s in range(first, first + n):
            for h in range(H):
                acc = Fraction(0)
                for d in range(D):
                    acc += q[t][h * D + d] * k[s][d]
                out[(t, h, s)] = acc
    return out


def exact_loss(q, k, w, g, cu_q, cu_k, offs, H, D):
    """L = sum_t sum_j g[t][j] * I[t, first_t + j] over the visible keys, exactly."""
    dots = exact_dots(q, k, cu_q, cu_k, offs, H, D)
    total = Fraction(0)
    for (t, h, s), v in dots.items():
        if v > 0:
            _, first, _ = visible_count(cu_q, cu_k, offs, t)
            total += g[t][s - first] * w[t][h] * v
    return total
