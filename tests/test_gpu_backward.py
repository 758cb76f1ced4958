"""GPU parity of the backward of the scores (dq, dk, dw) through the C ABI against the FP64 oracle.

Tolerance (Gaussian inputs), per output element, from the arithmetic of the HIP path:
  * the gradient factor entering the matrix cores is rounded to BF16 (g for dq, w * g for
    dk): 8 significant bits, relative error <= 2^-8 per term;
  * FP32 accumulation of m terms: <= m * 2^-24 of the sum of |terms| (any order);
  * S is the FP32 product of 128 exact BF16 products, |S - S_exact| <= 2^-17 * sum|q k|;
    where |S_exact| is within 2^-16 * sum|q k| of zero the ReLU mask may differ, so those
    terms enter the bound whole.
On top of the elementwise bound, the relative RMS error must stay below 2^-7 (dq, dk) and
1e-5 (dw): a dropped key or head moves it far more.  Integer-valued inputs sized so that
every product and partial sum is exact in FP32 and every BF16 factor is exact must match
the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

from deterministic_score_top_amd import indexer as ix
from deterministic_score_top_amd import workloads as W
from oracle import dsa_oracle as O
from tests.parity import backward_row_bounds as _row_bounds

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _tables(wl):
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    return wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy(), offs


def _ld(wl):
    L = wl.max_seqlen_k if wl.max_seqlen_k > 0 else max(wl.Tkv, 1)
    return (L + 3) // 4 * 4


def _gpu(wl, grad, **kw):
    d = "cuda"
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(d)
    dq, dk, dw = ix.backward(wl.q.to(d), wl.k.to(d), wl.w.to(d), wl.cu_seqlens_q.to(d), wl.cu_seqlens_k.to(d),
                             grad.to(d), offs, max_seqlen_k=wl.max_seqlen_k, **kw)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dw.cpu().numpy()


def _bounds(wl, grad):
    """Elementwise error bounds of dq, dk, dw (see the module docstring)."""
    q64, k64, w64 = O.from_torch(wl.q, wl.k, wl.w)
    g64 = grad.double().numpy()
    cu_q, cu_k, offs = _tables(wl)
    T, H, D = q64.shape
    tq = np.zeros((T, H, D))
    tw = np.zeros((T, H))
    tk_sum = np.zeros((wl.Tkv, D))
    tk_amb = np.zeros((wl.Tkv, D))
    cnt = np.zeros(wl.Tkv)
    for t in range(T):
        first, n = O.visible(cu_q, cu_k, offs, t)
        if n == 0:
            continue
        tq[t], tw[t], a, b = _row_bounds(q64, k64, w64, g64[t, :n], t, first, n)
        tk_sum[first:first + n] += a
        tk_amb[first:first + n] += b
        cnt[first:first + n] += 1
    fk = 2.0 ** -8 + (cnt * H + 10) * U
    return tq, fk[:, None] * tk_sum + tk_amb, tw


def _check_close(wl, grad, got, ref):
    bounds = _bounds(wl, grad)
    for name, g, r, b, rms in zip(("dq", "dk", "dw"), got, ref, bounds, (2.0 ** -7, 2.0 ** -7, 1e-5)):
        err = np.abs(g.astype(np.float64) - r)
        bad = err > b
        assert not bad.any(), f"{name}: {bad.sum()} elements out of bound, worst excess {np.max(err - b)}"
        nr = np.linalg.norm(r)
        if nr > 0:
            assert np.linalg.norm(err) <= rms * nr, f"{name}: relative RMS error {np.linalg.norm(err) / nr}"


def _check_exact(got, ref):
    for name, g, r in zip(("dq", "dk", "dw"), got, ref):
        r32 = r.astype(np.float32)
        assert np.array_equal(r32.astype(np.float64), r), f"{name}: reference not exact in FP32"
        diff = g != r32
        assert not diff.any(), f"{name}: {diff.sum()} elements differ, first at {np.argwhere(diff)[0]}"


# segment tables with ragged query tiles (4) and key tiles (64), offsets before, inside and past
# the segment, an empty segment, a keyless segment and a negative offset
MIXED = ([37, 0, 200, 5, 130, 9], [50, 3, 700, 0, 1500, 70], [13, 0, 500, 2, 1370, -4])


def test_exact_integer_mixed_segments():
    wl = W.integer_valued(*MIXED, topk=8, seed=31, qk_range=2, w_den=8)
    grad = W.draw_grad(wl.T, _ld(wl), seed=31, integer=True)
    got = _gpu(wl, grad)
    _check_exact(got, O.backward_workload(wl, grad))


def test_exact_integer_causal_2048():
    # one causal document: key tiles seen by 2048..1 queries, the 4 query parts of each key tile
    # and the 4 query streams inside each part all in use
    wl = W.integer_valued([2048], [2048], [0], topk=8, seed=32, qk_range=2, w_den=8)
    grad = W.draw_grad(wl.T, _ld(wl), seed=32, integer=True)
    got = _gpu(wl, grad)
    _check_exact(got, O.backward_workload(wl, grad))


def test_exact_integer_tie_heavy_keys():
    wl = W.integer_valued([300, 77], [900, 260], [600, 200], topk=8, seed=33, qk_range=2, w_den=8,
                          distinct_keys=3)
    grad = W.draw_grad(wl.T, _ld(wl), seed=33, integer=True)
    _check_exact(_gpu(wl, grad), O.backward_workload(wl, grad))


def test_gaussian_mixed_segments():
    wl = W.random_segments(*MIXED, topk=8, seed=34)
    grad = W.draw_grad(wl.T, _ld(wl), seed=34)
    _check_close(wl, grad, _gpu(wl, grad), O.backward_workload(wl, grad))


def test_gaussian_causal_1024():
    wl = W.make("causal_n1024")
    grad = W.draw_grad(wl.T, _ld(wl), seed=35)
    _check_close(wl, grad, _gpu(wl, grad), O.backward_workload(wl, grad))


def test_gaussian_split_tail_long_rows():
    # 4 queries over 41 986 keys: 657 key tiles, each seen by the same 4 queries
    wl = W.split_tail()
    grad = W.draw_grad(wl.T, _ld(wl), seed=36)
    _check_close(wl, grad, _gpu(wl, grad), O.backward_workload(wl, grad))


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed):
    rng = np.random.default_rng(3000 + seed)
    B = int(rng.integers(1, 24))
    T_lens = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 160, B)]
    K_lens = [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, 900, B)]
    offs = [int(rng.integers(-40, max(K_lens[b], 1) + 20)) for b in range(B)]
    if sum(T_lens) == 0:
        T_lens[0] = 5
    if seed % 2 == 0:
        wl = W.integer_valued(T_lens, K_lens, offs, topk=8, seed=3000 + seed, qk_range=2, w_den=8)
        grad = W.draw_grad(wl.T, _ld(wl), seed=3000 + seed, integer=True)
        _check_exact(_gpu(wl, grad), O.backward_workload(wl, grad))
    else:
        wl = W.random_segments(T_lens, K_lens, offs, topk=8, seed=3000 + seed)
        grad = W.draw_grad(wl.T, _ld(wl), seed=3000 + seed)
        _check_close(wl, grad, _gpu(wl, grad), O.backward_workload(wl, grad))


def test_bitwise_reproducible():
    wl = W.random_segments(*MIXED, topk=8, seed=37)
    grad = W.draw_grad(wl.T, _ld(wl), seed=37)
    a = _gpu(wl, grad)
    b = _gpu(wl, grad)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_grad_outside_visible_columns_ignored():
    # NaN in every column a row does not see must not reach any gradient
    wl = W.random_segments([40, 20], [130, 90], [10, 100], topk=8, seed=38)
    grad = W.draw_grad(wl.T, _ld(wl), seed=38)
    cu_q, cu_k, offs = _tables(wl)
    poisoned = grad.clone()
    for t in range(wl.T):
        _, n = O.visible(cu_q, cu_k, offs, t)
        poisoned[t, n:] = float("nan")
    a = _gpu(wl, grad)
    b = _gpu(wl, poisoned)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_outputs_fully_overwritten():
    wl = W.random_segments([6, 0, 5], [0, 70, 9], [0, 0, -10], topk=8, seed=39)
    grad = W.draw_grad(wl.T, _ld(wl), seed=39)
    d = "cuda"
    dq = torch.full((wl.T, 64, 128), float("nan"), device=d)
    dk = torch.full((wl.Tkv, 128), float("nan"), device=d)
    dw = torch.full((wl.T, 64), float("nan"), device=d)
    got = _gpu(wl, grad, dq=dq, dk=dk, dw=dw)
    # segment 0 has no keys, segment 1 no queries, segment 2's queries see nothing (offset -10)
    for x in got:
        assert np.all(x == 0)


def test_no_queries_or_no_keys():
    wl = W.random_segments([0, 0], [40, 30], [0, 0], topk=8, seed=40)
    grad = torch.zeros((0, _ld(wl)))
    dq, dk, dw = _gpu(wl, grad)
    assert dq.shape == (0, 64, 128) and dw.shape == (0, 64) and np.all(dk == 0)
    wl = W.random_segments([7, 3], [0, 0], [0, 5], topk=8, seed=41)
    wl.max_seqlen_k = 4
    grad = W.draw_grad(wl.T, 4, seed=41)
    dq, dk, dw = _gpu(wl, grad)
    assert dk.shape == (0, 128) and np.all(dq == 0) and np.all(dw == 0)


def test_seqlen_bound_flagged_and_truncated():
    wl = W.random_segments([30, 12], [200, 50], [170, 40], topk=8, seed=42)
    wl.max_seqlen_k = 100
    grad = W.draw_grad(wl.T, 100, seed=42)
    d = "cuda"
    ws = torch.empty(ix.backward_workspace_size(wl.T, wl.Tkv, wl.B, 100), dtype=torch.uint8, device=d)
    ix.workspace_init(ws)
    got = _gpu(wl, grad, workspace=ws)
    status, _, _ = ix.read_status(ws)
    assert status & ix.STATUS_SEQLEN_BOUND
    # reference: segment 0 truncated to its first 100 keys, the rest of its keys unseen
    tr = W.Workload("trunc", wl.q, torch.cat([wl.k[:100], wl.k[200:]]), wl.w,
                    torch.tensor([0, 30, 42], dtype=torch.int32), torch.tensor([0, 100, 150], dtype=torch.int32),
                    wl.q_pos_offsets, 8, 100)
    dq, dk_t, dw = O.backward_workload(tr, grad)
    dk = np.zeros((wl.Tkv, 128))
    dk[:100] = dk_t[:100]
    dk[200:] = dk_t[100:]
    # elementwise bound from the truncated problem, mapped back to the full key rows
    tq, tk_t, tw = _bounds(tr, grad)
    tk = np.zeros((wl.Tkv, 128))
    tk[:100] = tk_t[:100]
    tk[200:] = tk_t[100:]
    for g, r, b in zip(got, (dq, dk, dw), (tq, tk, tw)):
        assert np.all(np.abs(g.astype(np.float64) - r) <= b)
    assert np.all(got[1][100:200] == 0)


def test_bad_tables_leave_outputs_untouched():
    wl = W.random_segments([10, 10], [64, 64], [0, 0], topk=8, seed=43)
    wl.cu_seqlens_q = torch.tensor([0, 12, 20], dtype=torch.int32)
    wl.cu_seqlens_k = torch.tensor([0, 64, 100], dtype=torch.int32)   # does not end at Tkv = 128
    grad = W.draw_grad(wl.T, _ld(wl), seed=43)
    d = "cuda"
    ws = torch.empty(ix.backward_workspace_size(wl.T, wl.Tkv, wl.B), dtype=torch.uint8, device=d)
    ix.workspace_init(ws)
    dq = torch.full((wl.T, 64, 128), 7.0, device=d)
    dk = torch.full((wl.Tkv, 128), 7.0, device=d)
    dw = torch.full((wl.T, 64), 7.0, device=d)
    got = _gpu(wl, grad, workspace=ws, dq=dq, dk=dk, dw=dw)
    status, _, _ = ix.read_status(ws)
    assert status & ix.STATUS_BAD_SEGMENTS
    for x in got:
        assert np.all(x == 7.0)


def test_bad_tables_then_good_tables_same_workspace():
    # few queries and keys: both reduce kernels run.  After a call with invalid tables the next
    # call with valid tables on the same workspace (not re-initialised) must give exactly what a
    # fresh workspace gives: the reduce kernels gate on this call's verdict, not on the sticky
    # status bit
    wl = W.random_segments([10, 10], [64, 64], [0, 0], topk=8, seed=45)
    grad = W.draw_grad(wl.T, _ld(wl), seed=45)
    d = "cuda"
    ws = torch.empty(ix.backward_workspace_size(wl.T, wl.Tkv, wl.B), dtype=torch.uint8, device=d)
    ix.workspace_init(ws)
    good_q, good_k = wl.cu_seqlens_q, wl.cu_seqlens_k
    wl.cu_seqlens_k = torch.tensor([0, 64, 100], dtype=torch.int32)   # does not end at Tkv = 128
    _gpu(wl, grad, workspace=ws)
    assert ix.read_status(ws)[0] & ix.STATUS_BAD_SEGMENTS
    wl.cu_seqlens_q, wl.cu_seqlens_k = good_q, good_k
    got = _gpu(wl, grad, workspace=ws)
    ref = _gpu(wl, grad)   # fresh workspace
    for g, r in zip(got, ref):
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
    assert np.any(got[1] != 0) and np.any(got[0] != 0)


def test_causal_n8192_sampled_rows_and_keys():
    wl = W.make("causal_n8192")
    grad = W.draw_grad(wl.T, _ld(wl), seed=44)
    dq, dk, dw = _gpu(wl, grad)
    q64, k64, w64 = O.from_torch(wl.q, wl.k, wl.w)
    g64 = grad.double().numpy()
    cu_q, cu_k, offs = _tables(wl)
    rng = np.random.default_rng(44)
    rows = sorted(set([0, 1, 63, 64, 4095, 8190, 8191] + rng.integers(0, wl.T, 9).tolist()))
    for t in rows:
        first, n = O.visible(cu_q, cu_k, offs, t)
        rq, rw, _ = O.row_backward(q64, k64, w64, t, first, n, g64[t, :n])
        bq, bw, _, _ = _row_bounds(q64, k64, w64, g64[t, :n], t, first, n)
        assert np.all(np.abs(dq[t] - rq) <= bq), t
        assert np.all(np.abs(dw[t] - rw) <= bw), t
    keys = sorted(set([0, 1, 4095, 8127, 8191] + rng.integers(0, wl.Tkv, 4).tolist()))
    for s in keys:
        acc = np.zeros(128)
        scale = np.zeros(128)
        flips = np.zeros(128)
        for t in range(s, wl.T):   # causal: queries t >= s see key s
            first, n = O.visible(cu_q, cu_k, offs, t)
            gts = g64[t, s - first: s - first + 1]
            acc += O.row_backward(q64, k64, w64, t, s, 1, gts)[2][0]
            _, _, a, b = _row_bounds(q64, k64, w64, gts, t, s, 1)
            scale += a[0]
            flips += b[0]
        fk = 2.0 ** -8 + (64 * (wl.T - s) + 10) * U
        assert np.all(np.abs(dk[s] - acc) <= fk * scale + flips), s


def test_exact_integer_many_keys_direct_dk():
    # 140 000 keys: enough 256-key blocks that the dk kernel writes dk itself (no partials)
    lens = [35000, 35000, 35000, 35000]
    wl = W.integer_valued([8, 5, 0, 12], lens, [34992, 20000, 0, 34990], topk=8, seed=45, qk_range=2, w_den=8)
    # no dk partials (the 25 queries do get 64 key parts each: dq and dw partials)
    assert ix.backward_workspace_size(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k) == 256 + 64 * wl.T * (64 * 128 + 64) * 4
    grad = W.draw_grad(wl.T, _ld(wl), seed=45, integer=True)
    _check_exact(_gpu(wl, grad), O.backward_workload(wl, grad))
