"""GPU parity of the sparse attention over the selected ids (through the C ABI) against the FP64 oracle.

Tolerance, from the arithmetic of the HIP path: the probabilities enter the value product as
BF16 (8 significant bits, relative error <= 2^-8 per term), so
    |o_gpu - o| <= 2^-7 * (sum_j p_j |v_jd|) / sum_j p_j  (+ 1e-6 * max|v|)
covers that rounding, the FP32 scores and the hardware exp2/log2; lse within
1e-5 * (1 + |lse|) plus the FP32 score error.  The relative RMS error of o must stay below
2^-8.  Rows with one valid id, and identical keys with a power-of-two count, are exact.
"""
import math

import numpy as np
import pytest
import torch

from deterministic_score_top_amd import indexer as ix
from deterministic_score_top_amd import workloads as W
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu
DV = 512


def _gpu(q, kv, ids, scale, **kw):
    d = "cuda"
    o, lse = ix.sparse_attention(q.to(d), kv.to(d), torch.as_tensor(ids, dtype=torch.int32).to(d), scale, **kw)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _check(q, kv, ids, scale, o, lse):
    q64, kv64 = q.double().numpy(), kv.double().numpy()
    ro, rl = O.sparse_attention_rows(q64, kv64, ids, scale, DV)
    for t in range(len(ids)):
        valid = ids[t][(ids[t] >= 0) & (ids[t] < kv.shape[0])]
        if valid.size == 0:
            assert np.all(o[t] == 0) and np.all(np.isneginf(lse[t])), t
            continue
        K = kv64[valid]
        S = scale * (q64[t] @ K.T)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        bound = 2.0 ** -7 * (P @ np.abs(K[:, :DV])) + 1e-6 * np.abs(K[:, :DV]).max()
        err = np.abs(o[t] - ro[t])
        assert np.all(err <= bound), (t, float(np.max(err - bound)))
        serr = abs(scale) * 2.0 ** -16 * (np.abs(q64[t]) @ np.abs(K).T).max()
        assert np.all(np.abs(lse[t] - rl[t]) <= 1e-5 * (1 + np.abs(rl[t])) + serr), t
    nr = np.linalg.norm(ro)
    if nr > 0:
        assert np.linalg.norm(o - ro) <= 2.0 ** -8 * nr


def _ids(T, Tkv, k, seed, minus=0.0):
    rng = np.random.default_rng(seed)
    ids = np.stack([np.sort(rng.choice(Tkv, k, replace=False)) for _ in range(T)]).astype(np.int32)
    if minus:
        ids[rng.random(ids.shape) < minus] = -1
    return ids


def test_random_rows_with_gaps_and_tail():
    T, Tkv, k = 21, 3000, 100            # 4 tiles of 32 ids, the last one partial
    q, kv = W.draw_attention(T, Tkv, seed=1)
    ids = _ids(T, Tkv, k, 1, minus=0.2)
    ids[3, :] = -1                      # no valid id
    ids[4, 1:] = -1                     # one valid id
    scale = 1.0 / math.sqrt(576)
    o, lse = _gpu(q, kv, ids, scale)
    _check(q, kv, ids, scale, o, lse)


@pytest.mark.parametrize("k,seed", [(1, 2), (31, 3), (32, 4), (33, 11), (63, 12), (64, 13), (65, 14), (127, 15),
                                    (2048, 5)])
def test_topk_widths(k, seed):
    T, Tkv = 9, 5000
    q, kv = W.draw_attention(T, Tkv, seed=seed)
    ids = _ids(T, Tkv, k, seed)
    scale = 0.06
    o, lse = _gpu(q, kv, ids, scale)
    _check(q, kv, ids, scale, o, lse)


def test_one_key_half_empty():
    # ids are handled in tiles of 64, each half scored by another wave: a half with no valid id
    # (the other half full) and the reverse, in the same rows
    T, Tkv, k = 6, 4000, 192
    q, kv = W.draw_attention(T, Tkv, seed=16)
    ids = _ids(T, Tkv, k, 16)
    ids[0::2, 0:32] = -1
    ids[1::2, 96:128] = -1
    ids[:, 160:] = -1
    o, lse = _gpu(q, kv, ids, 0.05)
    _check(q, kv, ids, 0.05, o, lse)


def test_reference_maximum_moves():
    # scale 1 on unit-variance rows: scores spread over hundreds of units, so a head's running
    # maximum grows past the slack between tiles many times (the O rescale path)
    T, Tkv, k = 5, 6000, 1024
    q, kv = W.draw_attention(T, Tkv, seed=17)
    ids = _ids(T, Tkv, k, 17)
    o, lse = _gpu(q, kv, ids, 1.0)
    _check(q, kv, ids, 1.0, o, lse)


def test_single_valid_id_exact():
    T, Tkv = 6, 400
    q, kv = W.draw_attention(T, Tkv, seed=6)
    ids = -np.ones((T, 64), np.int32)
    for t in range(T):
        ids[t, (7 * t) % 64] = 13 * t + 5
    o, _ = _gpu(q, kv, ids, 0.05)
    kvf = kv.float().numpy()
    for t in range(T):
        assert np.array_equal(o[t], np.broadcast_to(kvf[13 * t + 5, :DV], o[t].shape)), t


def test_identical_keys_exact_mean():
    T, Tkv = 4, 300
    q, kv = W.draw_attention(T, Tkv, seed=7)
    kv[:] = kv[11]
    ids = _ids(T, Tkv, 64, 7)                 # 64 equal scores: p = 1 each, o = v exactly
    o, lse = _gpu(q, kv, ids, 0.05)
    v = kv[11].float().numpy()[:DV]
    for t in range(T):
        assert np.array_equal(o[t], np.broadcast_to(v, o[t].shape)), t


def test_ids_from_the_topk_call():
    # the selection's ids feed the attention: causal rows of 600 keys, top-128 of the indexer
    wl = W.random_segments([40], [600], [560], topk=128, seed=8)
    d = "cuda"
    ids, _ = ix.topk(wl.q.to(d), wl.k.to(d), wl.w.to(d), wl.cu_seqlens_q.to(d), wl.cu_seqlens_k.to(d),
                     wl.q_pos_offsets.to(d), topk=wl.topk, max_seqlen_k=wl.max_seqlen_k)
    q, kv = W.draw_attention(wl.T, wl.Tkv, seed=8)
    o, lse = ix.sparse_attention(q.to(d), kv.to(d), ids, 1.0 / math.sqrt(576))
    torch.cuda.synchronize()
    _check(q, kv, ids.cpu().numpy(), 1.0 / math.sqrt(576), o.cpu().numpy(), lse.cpu().numpy())


def test_bad_ids_flagged_and_skipped():
    T, Tkv = 5, 200
    q, kv = W.draw_attention(T, Tkv, seed=9)
    ids = _ids(T, Tkv, 40, 9)
    bad = ids.copy()
    bad[1, 3] = Tkv + 7
    bad[2, 0] = -5
    ws = torch.empty(ix.sparse_attention_workspace_size(T, 40), dtype=torch.uint8, device="cuda")
    ix.workspace_init(ws)
    o, lse = _gpu(q, kv, bad, 0.05, workspace=ws)
    status, _, _ = ix.read_status(ws)
    assert status & ix.STATUS_BAD_IDS
    ref = bad.copy()
    ref[(ref < 0) | (ref >= Tkv)] = -1
    _check(q, kv, ref, 0.05, o, lse)


@pytest.mark.parametrize("T,k,seed", [(1, 2048, 20), (4, 2048, 21), (3, 700, 22), (17, 1024, 23), (100, 300, 24)])
def test_few_rows_split_over_blocks(T, k, seed):
    # fewer than 256 rows: each row's ids are split over several blocks and the partial results
    # merged; short rows leave some parts without a valid id
    Tkv = 50000
    q, kv = W.draw_attention(T, Tkv, seed=seed)
    ids = _ids(T, Tkv, k, seed, minus=0.3)
    ids[0, 100:] = -1                     # a short row: most parts are empty
    if T > 2:
        ids[2, :] = -1                    # a row without a valid id
    assert ix.sparse_attention_workspace_size(T, k) > 256
    o, lse = _gpu(q, kv, ids, 0.05)
    _check(q, kv, ids, 0.05, o, lse)
    o2, lse2 = _gpu(q, kv, ids, 0.05)
    assert np.array_equal(o.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(lse.view(np.uint32), lse2.view(np.uint32))


def test_split_workspace_too_small_is_rejected():
    T, Tkv, k = 4, 1000, 512
    q, kv = W.draw_attention(T, Tkv, seed=25)
    ids = _ids(T, Tkv, k, 25)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    ix.workspace_init(ws)
    with pytest.raises(RuntimeError):
        _gpu(q, kv, ids, 0.05, workspace=ws)


def test_bitwise_reproducible():
    T, Tkv = 11, 2000
    q, kv = W.draw_attention(T, Tkv, seed=10)
    ids = _ids(T, Tkv, 300, 10, minus=0.1)
    a = _gpu(q, kv, ids, 0.04)
    b = _gpu(q, kv, ids, 0.04)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("name,rows", [("causal_n8192", 12), ("zigzag16", 12), ("split_tail", None)])
def test_full_workload_ids_from_topk(name, rows):
    # full-size workloads in the configuration bench.py times: the ids are the indexer's top-k of
    # the workload, the attention runs over every row, seeded sampled rows (every row of the split
    # tail, whose 4 rows are split over blocks) are checked against the oracle
    wl = W.make(name)
    d = "cuda"
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(d)
    ids, _ = ix.topk(wl.q.to(d), wl.k.to(d), wl.w.to(d), wl.cu_seqlens_q.to(d), wl.cu_seqlens_k.to(d), offs,
                     topk=wl.topk, max_seqlen_k=wl.max_seqlen_k)
    q, kv = W.draw_attention(wl.T, wl.Tkv, seed=2)
    scale = 1.0 / math.sqrt(576)
    o, lse = ix.sparse_attention(q.to(d), kv.to(d), ids, scale)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    sel = np.arange(wl.T) if rows is None else np.sort(np.random.default_rng(3).choice(wl.T, rows, replace=False))
    if rows is not None:
        sel[0] = 0                       # the shortest row of the first segment
    _check(q[sel], kv, ids_h[sel], scale, o[sel].cpu().numpy(), lse[sel].cpu().numpy())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_batches(seed):
    # seeded random batches: row counts on both sides of the few-row split, any topk, scattered
    # -1 entries, valid prefixes with a -1 tail, duplicate ids, empty rows, zero and large scales
    rng = np.random.default_rng(100 + seed)
    for case in range(8):
        T = int(rng.choice([1, 2, 3, 5, 13, 64, 100, 255, 256, 300]))
        k = int(rng.integers(1, 2049))
        Tkv = int(rng.integers(1, 20000))
        scale = float(rng.choice([0.0, 0.01, 1.0 / 24, 0.3, 1.0, -0.05, -1.0]))
        q, kv = W.draw_attention(T, Tkv, seed=1000 * seed + case)
        ids = rng.integers(0, Tkv, size=(T, k)).astype(np.int32)
        mode = case % 4
        if mode == 1:
            ids[rng.random(ids.shape) < rng.random()] = -1
        elif mode == 2:
            for t in range(T):
                ids[t, int(rng.integers(0, k + 1)):] = -1
        elif mode == 3:
            ids[:, ::3] = ids[:, :1]
            ids[rng.random(T) < 0.3] = -1
        o, lse = _gpu(q, kv, ids, scale)
        sel = np.arange(T) if T <= 12 else np.sort(rng.choice(T, 12, replace=False))
        _check(q[sel], kv, ids[sel], scale, o[sel], lse[sel])


@pytest.mark.parametrize("T", [4, 300])
def test_graph_capture_replays_match_eager(T):
    # the call enqueues only its kernels (one, or two when a few-row batch splits its ids and
    # merges the parts), with no allocation, memset or host sync, so it can be captured; replays
    # interleaved with eager calls and synchronisation must each match the eager result bit for bit
    Tkv, k = 3000, 700
    q, kv = W.draw_attention(T, Tkv, seed=30 + T)
    ids = _ids(T, Tkv, k, 30 + T, minus=0.2)
    d = "cuda"
    qd, kvd, idd = q.to(d), kv.to(d), torch.as_tensor(ids).to(d)
    ws = torch.empty(ix.sparse_attention_workspace_size(T, k), dtype=torch.uint8, device=d)
    ix.workspace_init(ws)
    o = torch.empty((T, 128, DV), dtype=torch.float32, device=d)
    lse = torch.empty((T, 128), dtype=torch.float32, device=d)
    kw = dict(out=o, lse=lse, workspace=ws)
    ix.sparse_attention(qd, kvd, idd, 0.05, **kw)
    torch.cuda.synchronize()
    ref = (o.cpu().numpy().copy(), lse.cpu().numpy().copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ix.sparse_attention(qd, kvd, idd, 0.05, **kw)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(4):
        o.fill_(7.0)
        lse.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy().view(np.uint32), ref[0].view(np.uint32)), r
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref[1].view(np.uint32)), r
        ix.sparse_attention(qd, kvd, idd, 0.05, **kw)    # eager work between replays
        torch.cuda.synchronize()
    _check(q, kv, ids, 0.05, ref[0], ref[1])


def test_empty_kv_table():
    # no latent rows at all: every id is -1 or out of range (flagged); every row gets o = 0 and
    # lse = -inf, split (3 rows) or not (300 rows)
    for T in (3, 300):
        q, _ = W.draw_attention(T, 1, seed=40)
        kv = torch.empty((0, 576), dtype=torch.bfloat16)
        ids = -np.ones((T, 100), np.int32)
        ids[0, 5] = 0
        ws = torch.empty(ix.sparse_attention_workspace_size(T, 100), dtype=torch.uint8, device="cuda")
        ix.workspace_init(ws)
        o, lse = _gpu(q, kv, ids, 0.05, workspace=ws)
        assert np.all(o == 0) and np.all(np.isneginf(lse))
        status, _, _ = ix.read_status(ws)
        assert status & ix.STATUS_BAD_IDS
