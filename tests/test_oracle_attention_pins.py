"""Pins of the FP64 oracle's sparse attention over the selected ids (the selection's consumer).

  * library route: torch's float64 scaled_dot_product_attention over the same gathered rows
    (a masked dense call with -1 entries masked out) must agree to 1e-12;
  * closed forms: one valid id gives o = that row's value part and lse = its score; identical
    key rows give o = the value and lse = score + log(count); scale 0 gives the plain mean;
  * invariants: -1 entries behave as absent, the order of the ids does not matter, a row
    with no valid id gives o = 0 and lse = -inf.
"""
import math

import numpy as np
import torch

from oracle import dsa_oracle as O
from deterministic_score_top_amd import workloads as W

DV = 512


def _setup(T=6, Tkv=40, H=8, k=12, seed=0, dqk=576):
    q, kv = W.draw_attention(T, Tkv, H=H, dqk=dqk, seed=seed)
    q64 = q.double().numpy()
    kv64 = kv.double().numpy()
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(Tkv, k, replace=False) for _ in range(T)]).astype(np.int64)
    return q64, kv64, ids


def test_library_sdpa_float64():
    q64, kv64, ids = _setup(seed=1)
    ids[1, 3:7] = -1
    ids[2, :] = -1
    ids[2, 5] = 17
    scale = 1.0 / math.sqrt(576)
    o, lse = O.sparse_attention_rows(q64, kv64, ids, scale, DV)
    q = torch.from_numpy(q64)
    kv = torch.from_numpy(kv64)
    for t in range(q64.shape[0]):
        safe = torch.from_numpy(np.where(ids[t] >= 0, ids[t], 0))
        K = kv[safe]                                   # [k, dqk]
        mask = torch.from_numpy(ids[t] >= 0)[None, :].expand(q.shape[1], -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[t][:, None, :], K[None].expand(q.shape[1], -1, -1), K[:, :DV][None].expand(q.shape[1], -1, -1),
            attn_mask=mask[:, None, :], scale=scale)[:, 0, :]
        assert np.allclose(o[t], ref.numpy(), rtol=1e-12, atol=1e-12), t
        S = scale * (q[t] @ K.T)
        S = S.masked_fill(~mask, float("-inf"))
        assert np.allclose(lse[t], torch.logsumexp(S, dim=1).numpy(), rtol=1e-12, atol=1e-12), t


def test_single_valid_id():
    q64, kv64, ids = _setup(seed=2)
    ids[:, 1:] = -1
    o, lse = O.sparse_attention_rows(q64, kv64, ids, 0.05, DV)
    for t in range(len(ids)):
        assert np.array_equal(o[t], np.broadcast_to(kv64[ids[t, 0], :DV], o[t].shape))
        assert np.allclose(lse[t], 0.05 * (q64[t] @ kv64[ids[t, 0]]), rtol=1e-14, atol=0)


def test_identical_keys_and_zero_scale():
    q64, kv64, ids = _setup(seed=3)
    kv_same = kv64.copy()
    kv_same[:] = kv64[5]
    o, lse = O.sparse_attention_rows(q64, kv_same, ids, 0.07, DV)
    for t in range(len(ids)):
        assert np.allclose(o[t], kv64[5, :DV][None, :], rtol=1e-14, atol=1e-14)
        assert np.allclose(lse[t], 0.07 * (q64[t] @ kv64[5]) + math.log(ids.shape[1]), rtol=1e-13, atol=0)
    o0, lse0 = O.sparse_attention_rows(q64, kv64, ids, 0.0, DV)
    for t in range(len(ids)):
        assert np.allclose(o0[t], kv64[ids[t], :DV].mean(axis=0)[None, :], rtol=1e-13, atol=1e-14)
        assert np.allclose(lse0[t], math.log(ids.shape[1]))


def test_minus_one_absent_order_free_and_empty():
    q64, kv64, ids = _setup(seed=4)
    o, lse = O.sparse_attention_rows(q64, kv64, ids, 0.04, DV)
    rng = np.random.default_rng(9)
    perm = np.stack([rng.permutation(ids.shape[1]) for _ in range(len(ids))])
    padded = np.concatenate([np.take_along_axis(ids, perm, 1), -np.ones((len(ids), 5), np.int64)], axis=1)
    padded = np.stack([rng.permutation(r) for r in padded])
    o2, lse2 = O.sparse_attention_rows(q64, kv64, padded, 0.04, DV)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13) and np.allclose(lse, lse2, rtol=1e-13, atol=0)
    empty = -np.ones_like(ids)
    o3, lse3 = O.sparse_attention_rows(q64, kv64, empty, 0.04, DV)
    assert not o3.any() and np.all(np.isneginf(lse3))
