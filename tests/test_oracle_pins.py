"""Pins of the FP64 oracle against values fixed by the pages and by mathematics.

Each pin is chosen so that a plausible mistake in the oracle fails it:
  * golden files (hand-derived): a dropped ReLU, transposed q or w, the wrong
    tie rule, an exclusive causal diagonal, ignored offsets, segment-local
    ids, a wrong output order or missing -1 padding;
  * exact brute force (rational arithmetic, full sort) on tiny random inputs:
    any arithmetic or selection slip, FP32 instead of FP64;
  * closed forms: equal keys or non-positive dots make every visible score
    equal, so the top-k must be the largest visible ids;
  * invariants: exact power-of-two scaling of w, head permutation on integer
    inputs, splitting a segment's queries into two calls with shifted offsets,
    packing segments versus separate calls.
"""
import glob
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from deterministic_score_top_amd import workloads as W
from tests.bruteforce import brute_topk, exact_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(x):
    return float("-inf") if x == "-inf" else float(x)


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))))
def test_golden(path):
    g = json.load(open(path))
    q = np.asarray(g["q"], dtype=np.float64)
    k = np.asarray(g["k"], dtype=np.float64)
    w = np.asarray(g["w"], dtype=np.float64)
    assert q.shape[1:] == (g["H"], g["D"]) and k.shape[1] == g["D"]
    ids, sc, _ = O.topk_rows(q, k, w, np.asarray(g["cu_seqlens_q"]), np.asarray(g["cu_seqlens_k"]),
                             np.asarray(g["q_pos_offsets"]), g["topk"])
    assert ids.tolist() == g["expected_ids"]
    exp = np.asarray([[_f(x) for x in row] for row in g["expected_scores"]])
    assert np.array_equal(sc, exp)


def _wl_to_f64(wl):
    return O.from_torch(wl.q, wl.k, wl.w)


def _run_oracle(wl):
    q64, k64, w64 = _wl_to_f64(wl)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    return O.topk_rows(q64, k64, w64, wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy(), offs, wl.topk)


def _compare_to_brute(wl, H, D):
    ids, sc, _ = _run_oracle(wl)
    qf = exact_values(wl.q.reshape(wl.T, -1))
    kf = exact_values(wl.k)
    wf = exact_values(wl.w)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.tolist()
    ref = brute_topk(qf, kf, wf, wl.cu_seqlens_q.tolist(), wl.cu_seqlens_k.tolist(), offs, wl.topk, H, D)
    for t, (rids, rsc) in enumerate(ref):
        assert ids[t].tolist() == rids, f"row {t}"
        for j, v in enumerate(rsc):
            if v is None:
                assert sc[t, j] == float("-inf")
            else:
                assert abs(sc[t, j] - float(v)) <= 1e-12 * max(1.0, abs(float(v))), (t, j)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_small_heads(seed):
    # several segments, offsets (incl. past-the-end), an empty segment, topk smaller and larger than rows
    wl = W.random_segments([5, 0, 7, 3, 4], [6, 3, 9, 2, 0], [0, 1, 3, 9, 2], topk=4, H=3, D=2, seed=seed)
    _compare_to_brute(wl, 3, 2)


def test_brute_force_full_heads():
    wl = W.random_segments([3, 2], [5, 4], [2, 0], topk=3, H=64, D=128, seed=7)
    _compare_to_brute(wl, 64, 128)


def test_brute_force_integer_ties():
    # integer inputs from 3 distinct key vectors: many exact ties between keys
    wl = W.integer_valued([6, 5], [9, 7], [3, 1], topk=4, H=3, D=4, seed=3, distinct_keys=3)
    _compare_to_brute(wl, 3, 4)


def _largest_visible(wl, t):
    first, n = O.visible(wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy(),
                         None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy(), t)
    m = min(n, wl.topk)
    return list(range(first + n - m, first + n)) + [-1] * (wl.topk - m)


def test_closed_form_equal_keys():
    wl = W.random_segments([9, 6], [12, 5], [0, 4], topk=5, H=4, D=8, seed=11)
    wl.k[:] = wl.k[0:1]
    ids, sc, _ = _run_oracle(wl)
    for t in range(wl.T):
        assert ids[t].tolist() == _largest_visible(wl, t)
        live = sc[t][ids[t] >= 0]
        assert len(set(live.tolist())) <= 1


def test_closed_form_nonpositive_dots():
    g = torch.Generator().manual_seed(5)
    wl = W.random_segments([8, 4], [10, 6], [2, 0], topk=3, H=4, D=8, seed=5)
    u = torch.randn(8, generator=g)
    a = torch.rand(wl.T, 4, 1, generator=g) + 0.1
    b = torch.rand(wl.Tkv, 1, generator=g) + 0.1
    wl.q = (a * u).to(torch.bfloat16)
    wl.k = (-b * u).to(torch.bfloat16)
    ids, sc, _ = _run_oracle(wl)
    for t in range(wl.T):
        assert ids[t].tolist() == _largest_visible(wl, t)
        assert np.all(sc[t][ids[t] >= 0] == 0.0)


def test_invariant_weight_scaling():
    wl = W.random_segments([7, 5], [9, 6], [1, 3], topk=4, H=8, D=16, seed=2)
    ids0, sc0, _ = _run_oracle(wl)
    wl.w = wl.w * 8.0
    ids1, sc1, _ = _run_oracle(wl)
    assert np.array_equal(ids0, ids1)
    assert np.array_equal(sc0 * 8.0, sc1)


def test_invariant_head_permutation_integer():
    wl = W.integer_valued([6, 4], [8, 7], [0, 2], topk=3, H=8, D=16, seed=4)
    ids0, sc0, _ = _run_oracle(wl)
    perm = torch.randperm(8, generator=torch.Generator().manual_seed(1))
    wl.q = wl.q[:, perm].contiguous()
    wl.w = wl.w[:, perm].contiguous()
    ids1, sc1, _ = _run_oracle(wl)
    assert np.array_equal(ids0, ids1) and np.array_equal(sc0, sc1)


def test_invariant_query_split():
    # one segment's queries in two calls: the second call's offset moves by the first part's length
    wl = W.random_segments([10], [14], [3], topk=4, H=4, D=8, seed=9)
    ids, sc, _ = _run_oracle(wl)
    q64, k64, w64 = _wl_to_f64(wl)
    a_ids, a_sc, _ = O.topk_rows(q64[:6], k64, w64[:6], np.array([0, 6]), np.array([0, 14]), np.array([3]), 4)
    b_ids, b_sc, _ = O.topk_rows(q64[6:], k64, w64[6:], np.array([0, 4]), np.array([0, 14]), np.array([9]), 4)
    assert np.array_equal(np.concatenate([a_ids, b_ids]), ids)
    assert np.array_equal(np.concatenate([a_sc, b_sc]), sc)


def test_invariant_segment_packing():
    wl = W.random_segments([5, 6], [7, 8], [1, 2], topk=3, H=4, D=8, seed=12)
    ids, sc, _ = _run_oracle(wl)
    q64, k64, w64 = _wl_to_f64(wl)
    a_ids, a_sc, _ = O.topk_rows(q64[:5], k64[:7], w64[:5], np.array([0, 5]), np.array([0, 7]), np.array([1]), 3)
    b_ids, b_sc, _ = O.topk_rows(q64[5:], k64[7:], w64[5:], np.array([0, 6]), np.array([0, 8]), np.array([2]), 3)
    b_ids = np.where(b_ids >= 0, b_ids + 7, -1)
    assert np.array_equal(np.concatenate([a_ids, b_ids]), ids)
    assert np.array_equal(np.concatenate([a_sc, b_sc]), sc)


def test_bf16_conversion_exact():
    x = torch.tensor([1.0, -2.5, 3.140625, 1e-3, -0.0, 65280.0]).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_bits_to_f64(bits)
    assert np.array_equal(got, x.double().numpy())
    assert math.copysign(1.0, got[4]) == -1.0


def test_workload_shapes():
    # sizes of the five configurations and the N=16384 perf shape, from the pages' tables
    # (T, Tkv, segments) and the adopted causal rule (visible pairs)
    def pairs(wl):
        cu_q, cu_k = wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy()
        offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
        return sum(O.visible(cu_q, cu_k, offs, t)[1] for t in range(wl.T))
    s, L = W.zigzag_doc_lengths(16)
    assert s == 5333 and int(L.sum()) == 170112
    s8, L8 = W.zigzag_doc_lengths(8)
    assert s8 == 70 and int(L8.sum()) == 169504
    wl = W.split_tail()
    assert (wl.T, wl.Tkv, wl.B, pairs(wl)) == (4, 41986, 1, 167938)
    wl = W.make("causal_n1024")
    assert (wl.T, wl.Tkv, pairs(wl)) == (1024, 1024, 524800)
