"""The entry point that allocates nothing (dsa_indexer_topk_noalloc) against dsa_indexer_topk.

Both run the same kernels; the no-allocation entry works in the library's fixed per-GPU array
instead of a caller's workspace, so its outputs must equal the workspace entry's bit for bit.
Two calls in a row (the second smaller, so stale rows of the first stay in the array), the
largest accepted shape, and a rejected oversize shape.
"""
import ctypes

import numpy as np
import pytest
import torch

from deterministic_score_top_amd import indexer as ix
from deterministic_score_top_amd import workloads as W
from oracle import dsa_oracle as O
from tests.parity import check_rows

pytestmark = pytest.mark.gpu

ERR_SCRATCH = -7


def _dev(wl):
    d = "cuda"
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(d)
    return (wl.q.to(d), wl.k.to(d), wl.w.to(d), wl.cu_seqlens_q.to(d), wl.cu_seqlens_k.to(d), offs)


def _both(wl):
    args = _dev(wl)
    kw = dict(topk=wl.topk, max_seqlen_k=wl.max_seqlen_k)
    a_ids, a_sc = ix.topk_noalloc(*args, **kw)
    torch.cuda.synchronize()
    a = (a_ids.cpu().numpy(), a_sc.cpu().numpy())
    b_ids, b_sc = ix.topk(*args, **kw)
    torch.cuda.synchronize()
    b = (b_ids.cpu().numpy(), b_sc.cpu().numpy())
    return a, b


def _same(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_noalloc_two_calls_second_smaller():
    big = W.random_segments([300, 0, 170], [3000, 40, 1200], [2800, 0, 1100], topk=256, seed=71)
    small = W.random_segments([37, 12], [500, 90], [480, 20], topk=64, seed=72)
    assert ix.workspace_size(big.T, big.Tkv, big.B, big.max_seqlen_k) <= ix.noalloc_max_bytes()
    a, b = _both(big)
    _same(a, b)
    a, b = _both(small)
    _same(a, b)
    oi, osc, det = O.topk_workload(small)
    check_rows(a[0], a[1], range(small.T), oi, osc, det, small.topk)


def test_noalloc_largest_shape_and_oversize_rejected():
    wl = W.single_causal(4096, 2048, seed=73)     # 4096 rows of 4096 keys: exactly the array
    assert ix.workspace_size(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k) == ix.noalloc_max_bytes()
    a, b = _both(wl)
    _same(a, b)
    # one query more does not fit: rejected on the host, nothing enqueued, outputs untouched
    d = "cuda"
    q = torch.zeros((4097, 64, 128), dtype=torch.bfloat16, device=d)
    w = torch.zeros((4097, 64), dtype=torch.float32, device=d)
    k = torch.zeros((4096, 128), dtype=torch.bfloat16, device=d)
    cq = torch.tensor([0, 4097], dtype=torch.int32, device=d)
    ck = torch.tensor([0, 4096], dtype=torch.int32, device=d)
    oi = torch.full((4097, 8), 5, dtype=torch.int32, device=d)
    osc = torch.full((4097, 8), 5.0, dtype=torch.float32, device=d)
    with pytest.raises(ix.DsaError) as e:
        ix.topk_noalloc(q, k, w, cq, ck, None, topk=8, max_seqlen_k=4096, out_ids=oi, out_scores=osc)
    assert e.value.code == ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((oi == 5).all()) and bool((osc == 5.0).all())
    # and the array still serves the next call
    small = W.random_segments([9], [200], [150], topk=16, seed=74)
    a, b = _both(small)
    _same(a, b)
