"""The C-ABI library loads, exports every declared symbol and validates arguments on the host.

No compute call runs here: each call below is rejected by host-side checks
before the library touches a device.
"""
import ctypes
import os
import re

import pytest
import torch

from deterministic_score_top_amd import indexer as ix

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# Placeholder addresses are used throughout; a call whose arguments all pass would enqueue work
# on them, so such calls are made only where no GPU is present (they stop at the device check).
NO_GPU = not torch.cuda.is_available()
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dsa_indexer_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    L = ix.lib()
    names = _declared()
    assert set(names) == set(ix.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def test_workspace_size():
    # control block + T rows of round_up(max_seqlen_k, 64) floats
    assert ix.workspace_size(8192, 8192, 1, 8192) == 256 + 8192 * 8192 * 4
    assert ix.workspace_size(4, 41986, 1, 41986) == 256 + 4 * 42048 * 4
    assert ix.workspace_size(10, 100, 2, 0) == 256 + 10 * 128 * 4   # 0 -> Tkv
    with pytest.raises(ix.DsaError):
        ix.workspace_size(10, 100, 0, 0)
    with pytest.raises(ix.DsaError):
        ix.workspace_size(10, 100, 1, 70000)
    # no stated bound: the bound is total_k, which must itself be a supported row length (more
    # than 65536 keys without a bound would cut a long segment without an error)
    assert ix.workspace_size(10, 65536, 1, 0) == 256 + 10 * 65536 * 4
    with pytest.raises(ix.DsaError):
        ix.workspace_size(10, 65537, 3, 0)
    assert ix.workspace_size(10, 175428, 32, 65536) == 256 + 10 * 65536 * 4


def test_status_strings():
    L = ix.lib()
    for code in range(0, -8, -1):
        assert L.dsa_indexer_status_string(code)
    assert L.dsa_indexer_status_string(-99) == b"unknown status"


def _call(shape, ptrs, topk=16, ws_bytes=1 << 40):
    L = ix.lib()
    q, k, w, cq, ck, offs, oi, osc, ws = ptrs
    V = ctypes.c_void_p
    return L.dsa_indexer_topk(ctypes.byref(shape), V(q), V(k), V(w), V(cq), V(ck), V(offs), topk,
                              V(oi), V(osc), V(ws), ws_bytes, None)


GOOD = (0x10000, 0x20000, 0x30000, 0x40000, 0x50000, None, 0x60000, 0x70000, 0x80000)


def _with(i, v):
    p = list(GOOD)
    p[i] = v
    return tuple(p)


def test_argument_errors():
    s = ix.make_shape(16, 64, 1, 64)
    assert _call(s, _with(0, None)) == -1          # q NULL
    assert _call(s, _with(8, None)) == -1          # workspace NULL
    assert _call(s, _with(1, 0x20008)) == -2       # k misaligned
    assert _call(s, _with(3, 0x40002)) == -2       # cu_seqlens_q misaligned
    assert _call(s, GOOD, topk=0) == -3
    assert _call(s, GOOD, topk=2049) == -3
    assert _call(s, GOOD, ws_bytes=100) == -4
    bad = ix.make_shape(16, 64, 1, 64)
    bad.num_heads = 32
    assert _call(bad, GOOD) == -3
    bad = ix.make_shape(16, 64, 1, 64)
    bad.head_dim = 64
    assert _call(bad, GOOD) == -3
    bad = ix.make_shape(-1, 64, 1, 64)
    assert _call(bad, GOOD) == -3
    bad = ix.make_shape(16, 64, 0, 64)
    assert _call(bad, GOOD) == -3
    # more than 65536 keys with max_seqlen_k = 0 is rejected before any device work, by every
    # entry point that takes the shape
    unbounded = ix.make_shape(16, 70000, 2, 0)
    assert _call(unbounded, GOOD) == -3
    if NO_GPU:   # with the bound stated the arguments pass; the call then stops at the device check
        assert _call(ix.make_shape(16, 70000, 2, 65536), GOOD) == -6
    L = ix.lib()
    V = ctypes.c_void_p
    q, k, w, cq, ck, _, g, dq, ws = GOOD
    assert L.dsa_indexer_scores(ctypes.byref(unbounded), V(q), V(k), V(w), V(cq), V(ck), None, V(g), 70000,
                                V(ws), 1 << 40, None) == -3
    assert L.dsa_indexer_backward(ctypes.byref(unbounded), V(q), V(k), V(w), V(cq), V(ck), None, V(g), 70000,
                                  V(dq), V(0x90000), V(0xA0000), V(ws), 1 << 40, None) == -3


def test_empty_inputs_may_be_null():
    # no queries: q, w and the outputs may be NULL; no keys: k may be NULL.  With the arguments
    # accepted, the call reaches the device check (-6 on a host without the GPU, 0 on the GPU
    # for T = 0, which enqueues nothing).
    no_q = ix.make_shape(0, 64, 1, 64)
    r = _call(no_q, (None, 0x20000, None, 0x40000, 0x50000, None, None, None, 0x80000))
    assert r in (0, -6)
    no_k = ix.make_shape(16, 0, 1, 64)
    if NO_GPU:   # (on a GPU this call would run on the placeholder addresses)
        r = _call(no_k, (0x10000, None, 0x30000, 0x40000, 0x50000, None, 0x60000, 0x70000, 0x80000))
        assert r == -6
    s = ix.make_shape(16, 64, 1, 64)
    assert _call(s, _with(1, None)) == -1          # k NULL with keys present
    assert _call(s, _with(6, None)) == -1          # out_ids NULL with queries present


def test_scores_argument_errors():
    L = ix.lib()
    s = ix.make_shape(16, 64, 1, 64)
    V = ctypes.c_void_p
    q, k, w, cq, ck, _, _, osc, ws = GOOD
    assert L.dsa_indexer_scores(ctypes.byref(s), V(q), V(k), V(w), V(cq), V(ck), None, V(osc), 60, V(ws),
                                1 << 20, None) == -3                       # ld below max_seqlen_k
    assert L.dsa_indexer_scores(ctypes.byref(s), V(q), V(k), V(w), V(cq), V(ck), None, V(osc), 64, V(ws),
                                16, None) == -4                            # no room for the control block


def test_prepare_argument_errors():
    L = ix.lib()
    V = ctypes.c_void_p
    s = ix.make_shape(16, 64, 1, 64)
    q, k, w, cq, ck, _, oi, osc, ws = GOOD
    h = V()

    def call(shape=s, q_=q, topk=16, wsb=1 << 40, out=ctypes.byref(h)):
        return L.dsa_indexer_prepare(ctypes.byref(shape), V(q_), V(k), V(w), V(cq), V(ck), None, topk, V(oi),
                                     V(osc), V(ws), wsb, None, out)
    assert call(out=None) == -1
    assert call(q_=None) == -1 and not h.value
    assert call(q_=0x10008) == -2
    assert call(topk=0) == -3
    assert call(shape=ix.make_shape(16, 70000, 2, 0)) == -3
    # the prepared workspace adds the plan (header, table copies, tile and unit prefixes) to the
    # top-k workspace; one byte less is rejected
    need = ix.prepared_workspace_size(16, 64, 1, 64)
    assert need > ix.workspace_size(16, 64, 1, 64) and need % 256 == 0
    assert call(wsb=need - 1) == -4
    assert L.dsa_indexer_run(None, None) == -1
    assert L.dsa_indexer_runner_destroy(None) == -1


def test_profiler_argument_errors():
    L = ix.lib()
    h = ctypes.c_void_p()
    assert L.dsa_indexer_profiler_create(0, ctypes.byref(h)) == -3
    assert L.dsa_indexer_profiler_read(None, None, None, None) == -1
    assert L.dsa_indexer_profiler_read_calls(None, None, None, 0, None) == -1


def test_backward_argument_errors():
    L = ix.lib()
    V = ctypes.c_void_p
    s = ix.make_shape(16, 64, 1, 64)
    # 16 queries: 4 query tiles, each split over 64 key parts (dq and dw partials); 64 keys: one
    # 256-key block split over 64 query parts (dk partials)
    dq_part = 64 * 16 * (64 * 128 + 64) * 4
    assert ix.backward_workspace_size(16, 64, 1) == 256 + 64 * 64 * 128 * 4 + dq_part
    # 175 428 keys: 686 key blocks fill the GPU alone, no dk partials
    assert ix.backward_workspace_size(16, 175428, 1, 65536) == 256 + dq_part
    # 8192 queries and keys: 2048 query tiles, 32 key blocks x 16 parts
    assert ix.backward_workspace_size(8192, 8192, 1) == 256 + 16 * 8192 * 128 * 4
    q, k, w, cq, ck, _, g, dq, ws = GOOD
    dk, dw = 0x90000, 0xA0000

    def call(grad=g, ld=64, dq_=dq, dk_=dk, dw_=dw, ws_bytes=1 << 40, shape=s):
        return L.dsa_indexer_backward(ctypes.byref(shape), V(q), V(k), V(w), V(cq), V(ck), None, V(grad), ld,
                                      V(dq_), V(dk_), V(dw_), V(ws), ws_bytes, None)
    assert call(grad=None) == -1
    assert call(dk_=None) == -1
    assert call(dw_=0xA0004) == -2
    assert call(ld=60) == -3                     # below max_seqlen_k
    assert call(ld=66) == -3                     # not a multiple of 4
    assert call(ws_bytes=1000) == -4
    no_k = ix.make_shape(16, 0, 1, 64)
    if NO_GPU:   # no keys: dk may be NULL (the call reaches the device check)
        assert call(dk_=None, shape=no_k) == -6


def test_sparse_attention_argument_errors():
    L = ix.lib()
    V = ctypes.c_void_p
    q, kv, ids, out, lse, ws = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000

    def call(T=4, Tkv=100, k=16, scale=0.1, q_=q, kv_=kv, ids_=ids, out_=out, lse_=lse, ws_=ws, wsb=256):
        return L.dsa_indexer_sparse_attention(T, Tkv, k, V(q_), V(kv_), V(ids_), scale, V(out_), V(lse_), V(ws_),
                                              wsb, None)
    assert call(k=0) == -3 and call(k=2049) == -3 and call(T=-1) == -3
    assert call(Tkv=1864136) == -3                 # 1152-byte rows past 31 bits
    assert call(T=1 << 30) == -3                    # 2 blocks per row past a 31-bit grid
    assert call(scale=float("nan")) == -3
    assert call(ids_=None) == -1 and call(ws_=None) == -1
    assert call(out_=0x40004) == -2 and call(ids_=0x30002) == -2
    assert call(wsb=100) == -4
    assert call(T=0, q_=None, ids_=None, out_=None, lse_=None) in (0, -6)


def test_sparse_attention_workspace_size():
    # few rows split their ids over blocks whose partial results (512 output floats and a
    # (maximum, sum) pair per head) live past the 256-byte control block
    L = ix.lib()
    per_part = 128 * (512 + 2) * 4
    assert L.dsa_indexer_sparse_attention_workspace_size(256, 2048) == 256   # 512 blocks: no split
    assert L.dsa_indexer_sparse_attention_workspace_size(4, 2048) == 256 + 4 * 16 * per_part
    assert L.dsa_indexer_sparse_attention_workspace_size(100, 300) == 256 + 100 * 4 * per_part
    assert L.dsa_indexer_sparse_attention_workspace_size(4, 64) == 256       # one tile: nothing to split
    assert L.dsa_indexer_sparse_attention_workspace_size(4, 0) == 0
    assert L.dsa_indexer_sparse_attention_workspace_size(4, 2049) == 0
    V = ctypes.c_void_p
    rc = L.dsa_indexer_sparse_attention(4, 100, 2048, V(0x10000), V(0x20000), V(0x30000), 0.1, V(0x40000),
                                        V(0x50000), V(0x60000), 256, None)
    assert rc == -4
