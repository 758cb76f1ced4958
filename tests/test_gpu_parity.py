"""GPU parity of the HIP path (through the C ABI) against the FP64 oracle.

Sizes: the small cases span several 8-query tiles and 64-key tiles with ragged
tails; the full configurations are checked on sampled rows against the oracle
and on every row through properties that hold at any size.
"""
import numpy as np
import pytest
import torch

from deterministic_score_top_amd import indexer as ix
from deterministic_score_top_amd import workloads as W
from oracle import dsa_oracle as O
from tests.parity import check_rows

pytestmark = pytest.mark.gpu


def _dev(wl):
    d = "cuda"
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(d)
    return (wl.q.to(d), wl.k.to(d), wl.w.to(d), wl.cu_seqlens_q.to(d), wl.cu_seqlens_k.to(d), offs)


def _run(wl, dev_args=None, **kw):
    q, k, w, cq, ck, offs = dev_args or _dev(wl)
    ids, sc = ix.topk(q, k, w, cq, ck, offs, topk=wl.topk, max_seqlen_k=wl.max_seqlen_k, **kw)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), sc.cpu().numpy()


def _oracle(wl, rows=None):
    return O.topk_workload(wl, rows)


def _check_all(wl, exact=False, **kw):
    ids, sc = _run(wl, **kw)
    oi, osc, det = _oracle(wl)
    check_rows(ids, sc, range(wl.T), oi, osc, det, wl.topk, exact=exact)
    return ids, sc


def _structural(wl, ids, sc):
    """Properties of every row at any size: count, range, order, padding, finite scores."""
    cu_q, cu_k = wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy()
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    for t in range(wl.T):
        first, n = O.visible(cu_q, cu_k, offs, t)
        m = min(n, wl.topk)
        row = ids[t]
        assert np.all(row[m:] == -1) and np.all(np.isneginf(sc[t, m:])), t
        assert np.all(np.diff(row[:m]) > 0), t
        assert m == 0 or (row[0] >= first and row[m - 1] < first + n), t
        assert np.all(np.isfinite(sc[t, :m])), t


def test_causal_n1024_all_rows():
    _check_all(W.make("causal_n1024"))


RAGGED = [
    # q_lens, k_lens, offsets, topk
    ([13, 0, 29, 5, 1], [70, 3, 130, 0, 200], [0, 2, 100, 1, 500], 16),
    ([64, 9], [64, 300], [0, 250], 1),
    ([17, 33], [100, 129], None, 2048),
    ([40], [257], [200], 64),
    ([0, 0, 7], [5, 0, 9], [0, 0, 0], 3),
]


@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_segments(case):
    ql, kl, offs, topk = RAGGED[case]
    _check_all(W.random_segments(ql, kl, offs, topk, seed=case))


def test_many_segments():
    # more segments than the select kernel caches in LDS; empty and keyless segments mixed in
    rng = np.random.default_rng(21)
    B = 1100
    ql = rng.integers(0, 3, B).tolist()
    kl = rng.integers(0, 40, B).tolist()
    offs = rng.integers(0, 50, B).tolist()
    _check_all(W.random_segments(ql, kl, offs, topk=8, seed=21))


@pytest.mark.parametrize("distinct", [None, 16, 2])
def test_integer_inputs_exact(distinct):
    wl = W.integer_valued([37, 20], [300, 129], [100, 5], topk=40, seed=3, distinct_keys=distinct)
    _check_all(wl, exact=True)


@pytest.mark.parametrize("distinct,nk,topk", [(2, 6000, 700), (16, 3000, 333), (None, 20000, 2048), (1, 9000, 2048)])
def test_select_long_rows_exact(distinct, nk, topk):
    # long rows of exact scores: few distinct values force the select kernel's overflow path
    # (the threshold bin holds more keys than a wave's copy region); distinct=None is the
    # ordinary path on a long row
    wl = W.integer_valued([6], [nk], [nk - 6], topk=topk, seed=nk, distinct_keys=distinct)
    _check_all(wl, exact=True)


def test_select_region_overflow_random_rows():
    # Gaussian scores on rows of 3073 to 3330 keys with topk = 2048, 160 rows (the 256-thread
    # select blocks): each wave reads a span of 1024 positions (the last wave only the rest), so
    # about three quarters of a span survive the sampled threshold and the three full waves
    # overflow their 768-entry survivor regions -- these rows take the exact fallback over the
    # whole row, without ties deciding anything
    wl = W.random_segments([80, 80], [3400, 3400], [3072, 3250], topk=2048, seed=77)
    _check_all(wl)


FEW_LONG = [
    # q_lens, k_lens, offsets, topk: at most a quarter as many rows as CUs (the 1024-thread select
    # blocks with their sparser sample) and rows of 16 500 to 65 536 keys
    ([8], [60000], [59992], 2048),
    ([3, 5], [17000, 40000], [16997, 39995], 2048),
    ([6], [30000], [29994], 256),
    ([4], [65536], [65532], 1000),
    ([2, 2, 2], [16500, 33000, 50000], [16498, 32998, 49998], 2048),
]


@pytest.mark.parametrize("case", range(len(FEW_LONG)))
def test_few_long_rows(case):
    ql, kl, offs, topk = FEW_LONG[case]
    _check_all(W.random_segments(ql, kl, offs, topk=topk, seed=500 + case))


@pytest.mark.parametrize("distinct", [None, 16, 2, 1])
@pytest.mark.parametrize("nk", [3000, 6000, 12000])
def test_select_many_long_rows_exact(distinct, nk):
    # 80 rows (more than a quarter of the CUs: the 256-thread select blocks) of 3000 to 12000
    # keys on exact scores; few distinct key vectors give long runs of equal scores across the
    # k-th key (the larger-id rule decides) and push the sampled threshold into its fallback
    wl = W.integer_valued([50, 30], [nk, nk // 2], [nk - 50, nk // 2 - 40], topk=2048 if nk > 3000 else 700,
                          seed=nk + (distinct or 0), distinct_keys=distinct)
    _check_all(wl, exact=True)


def test_scores_export():
    wl = W.random_segments([21, 11], [90, 140], [40, 0], topk=8, seed=5)
    q, k, w, cq, ck, offs = _dev(wl)
    out = ix.scores(q, k, w, cq, ck, offs, max_seqlen_k=wl.max_seqlen_k).cpu().numpy()
    _, _, det = _oracle(wl)
    for t in range(wl.T):
        first, s_all = det[t]
        n = len(s_all)
        tau = 1e-4 * max(1e-30, float(np.max(np.abs(s_all)))) if n else 0.0
        assert np.all(np.abs(out[t, :n] - s_all) <= tau), t
        assert np.all(np.isnan(out[t, n:])), t


def test_run_to_run_bitwise():
    wl = W.make("causal_n1024", seed=1)
    dev = _dev(wl)
    a = _run(wl, dev)
    for _ in range(3):
        b = _run(wl, dev)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


@pytest.mark.parametrize("tuning", [dict(key_chunk_tiles=1), dict(key_chunk_tiles=3),
                                    dict(key_chunk_tiles=16, grid_blocks=1),
                                    dict(key_chunk_tiles=2, grid_blocks=7), dict(grid_blocks=1000)])
def test_chunking_and_grid_bitwise(tuning):
    wl = W.random_segments([300, 77], [700, 1500], [400, 1000], topk=128, seed=8)
    dev = _dev(wl)
    a = _run(wl, dev)
    b = _run(wl, dev, tuning=tuning)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_query_split_bitwise():
    wl = W.random_segments([200], [260], [60], topk=64, seed=9)
    full = _run(wl)
    parts = []
    for lo, hi in ((0, 77), (77, 200)):
        sub = W.Workload("part", wl.q[lo:hi].contiguous(), wl.k, wl.w[lo:hi].contiguous(),
                         torch.tensor([0, hi - lo], dtype=torch.int32), wl.cu_seqlens_k,
                         torch.tensor([60 + lo], dtype=torch.int32), 64, 260)
        parts.append(_run(sub))
    ids = np.concatenate([p[0] for p in parts])
    sc = np.concatenate([p[1] for p in parts])
    assert np.array_equal(full[0], ids) and np.array_equal(full[1].view(np.uint32), sc.view(np.uint32))


def test_segment_packing_bitwise():
    wl = W.random_segments([45, 60], [300, 90], [255, 0], topk=32, seed=10)
    packed = _run(wl)
    a = W.Workload("a", wl.q[:45].contiguous(), wl.k[:300].contiguous(), wl.w[:45].contiguous(),
                   torch.tensor([0, 45], dtype=torch.int32), torch.tensor([0, 300], dtype=torch.int32),
                   torch.tensor([255], dtype=torch.int32), 32, 300)
    b = W.Workload("b", wl.q[45:].contiguous(), wl.k[300:].contiguous(), wl.w[45:].contiguous(),
                   torch.tensor([0, 60], dtype=torch.int32), torch.tensor([0, 90], dtype=torch.int32),
                   torch.tensor([0], dtype=torch.int32), 32, 300)
    ra, rb = _run(a), _run(b)
    ids_b = np.where(rb[0] >= 0, rb[0] + 300, -1)
    assert np.array_equal(packed[0], np.concatenate([ra[0], ids_b]))
    assert np.array_equal(packed[1].view(np.uint32), np.concatenate([ra[1], rb[1]]).view(np.uint32))


def test_tail_rows_equal_full_causal_rows():
    full = W.single_causal(4096, 512, seed=4)
    rf = _run(full)
    tail = W.Workload("tail", full.q[3072:].contiguous(), full.k, full.w[3072:].contiguous(),
                      torch.tensor([0, 1024], dtype=torch.int32), full.cu_seqlens_k,
                      torch.tensor([3072], dtype=torch.int32), 512, 4096)
    rt = _run(tail)
    assert np.array_equal(rf[0][3072:], rt[0])
    assert np.array_equal(rf[1][3072:].view(np.uint32), rt[1].view(np.uint32))


def test_control_block_left_clean():
    wl = W.random_segments([50, 30], [400, 100], [300, 0], topk=64, seed=11)
    q, k, w, cq, ck, offs = _dev(wl)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k)
    for _ in range(3):
        ix.topk(q, k, w, cq, ck, offs, topk=64, workspace=ws, max_seqlen_k=wl.max_seqlen_k)
        assert ix.read_status(ws) == (0, 0, 0)


def test_poisoned_counter_flagged_then_recovered():
    wl = W.random_segments([50, 30], [400, 100], [300, 0], topk=64, seed=12)
    q, k, w, cq, ck, offs = _dev(wl)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k)
    good = _run(wl, (q, k, w, cq, ck, offs), workspace=ws)
    ws[0:4].view(torch.int32).fill_(123456)   # stale ticket word
    ix.topk(q, k, w, cq, ck, offs, topk=64, workspace=ws, max_seqlen_k=wl.max_seqlen_k)
    st, tk, dn = ix.read_status(ws)
    assert st & ix.STATUS_CORRUPT_COUNTER and tk == 0 and dn == 0
    ix.workspace_init(ws)
    again = _run(wl, (q, k, w, cq, ck, offs), workspace=ws)
    assert ix.read_status(ws) == (0, 0, 0)
    assert np.array_equal(good[0], again[0]) and np.array_equal(good[1], again[1])


def test_bad_table_then_good_table_same_workspace():
    # a call with invalid tables writes padding rows and raises the (sticky) status bit; the next
    # call with valid tables on the same workspace, without re-initialising it, is unaffected
    wl = W.random_segments([20, 12], [100, 50], [60, 0], topk=8, seed=14)
    q, k, w, cq, ck, offs = _dev(wl)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k)
    cq_bad = torch.tensor([0, 20, 31], dtype=torch.int32, device="cuda")
    ids, _ = ix.topk(q, k, w, cq_bad, ck, offs, topk=8, workspace=ws, max_seqlen_k=wl.max_seqlen_k)
    torch.cuda.synchronize()
    assert bool((ids == -1).all())
    for _ in range(2):
        ids, sc = ix.topk(q, k, w, cq, ck, offs, topk=8, workspace=ws, max_seqlen_k=wl.max_seqlen_k)
        torch.cuda.synchronize()
        oi, osc, det = _oracle(wl)
        check_rows(ids.cpu().numpy(), sc.cpu().numpy(), range(wl.T), oi, osc, det, 8)
        st, tk, dn = ix.read_status(ws)
        assert st & ix.STATUS_BAD_SEGMENTS and tk == 0 and dn == 0   # sticky report, counters clean


def test_bad_segment_table_is_flagged():
    wl = W.random_segments([20, 12], [100, 50], [0, 0], topk=8, seed=13)
    q, k, w, cq, ck, offs = _dev(wl)
    cq_bad = torch.tensor([0, 20, 31], dtype=torch.int32, device="cuda")  # does not end at T=32
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k)
    ids, sc = ix.topk(q, k, w, cq_bad, ck, offs, topk=8, workspace=ws, max_seqlen_k=wl.max_seqlen_k)
    st, tk, dn = ix.read_status(ws)
    assert st & ix.STATUS_BAD_SEGMENTS and tk == 0 and dn == 0
    assert bool((ids == -1).all())


FULL = ["causal_n8192", "cp_tail", "zigzag16", "zigzag8", "split_tail", "split_tail_tie", "causal_n16384"]
MIN_ORACLE_ROWS = 256


def _sample_rows(wl, nmin=MIN_ORACLE_ROWS, seed=0):
    """Rows compared with the oracle: the first and last query of every segment, the queries whose
    visible count is topk - 1, topk and topk + 1 (the copy / select boundary) in every segment,
    and seeded random rows up to at least `nmin` (every row when there are fewer)."""
    T = wl.T
    if T <= nmin:
        return list(range(T))
    cu_q, cu_k = wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy()
    offs = np.zeros(wl.B, np.int64) if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    rows = set()
    for b in range(wl.B):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        if q1 <= q0:
            continue
        rows |= {q0, q1 - 1}
        for n in (wl.topk - 1, wl.topk, wl.topk + 1):   # visible count n at local position n - 1
            t = q0 + n - 1 - int(offs[b])
            if q0 <= t < q1:
                rows.add(t)
    rng = np.random.default_rng(seed)
    while len(rows) < nmin:
        rows.add(int(rng.integers(0, T)))
    return sorted(rows)


@pytest.mark.parametrize("name", FULL)
def test_full_config_sampled(name):
    wl = W.make(name)
    ids, sc = _run(wl)
    _structural(wl, ids, sc)
    rows = _sample_rows(wl)
    assert len(rows) >= min(MIN_ORACLE_ROWS, wl.T)
    print(f"{name}: {len(rows)} rows against the oracle", flush=True)
    oi, osc, det = _oracle(wl, rows)
    check_rows(ids, sc, rows, oi, osc, det, wl.topk)
    if name == "split_tail_tie":
        # Every key row is one of 16 vectors, so a query's scores take at most 16 values and its
        # top group (about 2600 keys, more than topk) ends the selection: the larger-id rule alone
        # decides which of its keys are kept.  Identical key rows give identical FP32 scores on
        # the GPU, and the groups are separated by far more than FP32 rounding (checked here), so
        # the GPU's id set must be exactly the oracle's: the topk largest ids of the top group.
        for r, t in enumerate(rows):
            first, s_all = det[r]
            vals = np.unique(s_all)[::-1]
            tau = 1e-4 * float(np.max(np.abs(s_all)))
            assert len(vals) >= 2 and vals[0] - vals[1] > 2 * tau, t
            top = np.nonzero(s_all == vals[0])[0] + first
            assert len(top) > wl.topk, t            # the top group alone overflows topk
            assert np.array_equal(ids[t], np.sort(top)[-wl.topk:]), t
            assert np.array_equal(ids[t], oi[r][:wl.topk]), t


@pytest.mark.parametrize("name", ["causal_n8192", "cp_tail", "zigzag16"])
@pytest.mark.parametrize("tuning", [dict(grid_blocks=97), dict(key_chunk_tiles=5), dict(key_chunk_tiles=1, grid_blocks=300)])
def test_full_config_chunking_and_grid_bitwise(name, tuning):
    # the full shapes under other work decompositions: an odd grid (other guided chunks on the CP
    # tail, other chunk sizes on the long-document shares) and forced key chunks give the same bits
    wl = W.make(name)
    dev = _dev(wl)
    a = _run(wl, dev)
    b = _run(wl, dev, tuning=tuning)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_weight_power_of_two_scaling_bitwise():
    # w x 2^j scales every FP32 partial sum by 2^j exactly: scores scale bit-exactly, ids are unchanged
    wl = W.random_segments([40, 9, 77], [300, 50, 1000], [200, 0, 900], topk=64, seed=40)
    q, k, w, cq, ck, offs = _dev(wl)
    base = _run(wl, (q, k, w, cq, ck, offs))
    for j in (-3, 2, 5):
        ids, sc = _run(wl, (q, k, w * (2.0 ** j), cq, ck, offs))
        assert np.array_equal(ids, base[0])
        live = base[0] >= 0
        assert np.array_equal(sc[live], (base[1][live].astype(np.float64) * 2.0 ** j).astype(np.float32))


def test_cp_tail_rows_equal_full_document_rows():
    # the context-parallel tail (queries 61440..65535 of a 65536-key document) returns exactly the
    # rows of the same queries in one causal call over the whole document
    tail = W.make("cp_tail")
    n, nq = tail.Tkv, tail.T
    d = "cuda"
    g = torch.Generator(device=d).manual_seed(7)
    q_full = torch.randn((n, 64, 128), generator=g, device=d).to(torch.bfloat16)
    w_full = torch.rand((n, 64), generator=g, device=d) / 8
    q_full[n - nq:] = tail.q.to(d)
    w_full[n - nq:] = tail.w.to(d)
    k = tail.k.to(d)
    cu = torch.tensor([0, n], dtype=torch.int32, device=d)
    ws = ix.alloc_workspace(n, n, 1, n, d)   # 17 GB of score rows, freed below
    ids_f, sc_f = ix.topk(q_full, k, w_full, cu, cu, None, topk=tail.topk, workspace=ws, max_seqlen_k=n)
    torch.cuda.synchronize()
    ids_f, sc_f = ids_f[n - nq:].cpu().numpy(), sc_f[n - nq:].cpu().numpy()
    del q_full, w_full, ws
    torch.cuda.empty_cache()
    ids_t, sc_t = _run(tail)
    assert np.array_equal(ids_f, ids_t)
    assert np.array_equal(sc_f.view(np.uint32), sc_t.view(np.uint32))


def _holder():
    import ctypes
    import os
    path = os.path.join(os.path.dirname(__file__), "native", "libspinner.so")
    assert os.path.exists(path), "tests/native/libspinner.so is not built (run __graft_entry__.build())"
    h = ctypes.CDLL(path)
    h.spinner_start.argtypes = [ctypes.c_int, ctypes.c_double]
    h.spinner_wait_resident.argtypes = [ctypes.c_double]
    return h


@pytest.mark.parametrize("name", ["causal_n1024", "split_tail"])
@pytest.mark.parametrize("held", [1, 32])
def test_bitwise_while_foreign_kernel_holds_cus(held, name):
    # the score kernel's blocks on held CUs start late; the resident ones take their work units
    # from the ticket counter.  Results are bit-identical and the control block ends clean.  (The
    # split tail's four rows are cut into one round of key-chunk units, one per block, so a
    # displaced block's unit is one that another block must take.)
    wl = W.make(name, seed=3)
    dev = _dev(wl)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k)
    ref = _run(wl, dev, workspace=ws)
    h = _holder()
    for hold_us in (50.0, 400.0):
        torch.cuda.synchronize()
        assert h.spinner_start(held, hold_us) == 0
        assert h.spinner_wait_resident(1000.0) == 0
        got = _run(wl, dev, workspace=ws)
        assert h.spinner_sync() == 0
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1].view(np.uint32), got[1].view(np.uint32))
        assert ix.read_status(ws) == (0, 0, 0)


def test_seqlen_bound_flagged_and_truncated():
    # a segment with more keys than max_seqlen_k: the status bit is raised and its queries see
    # only the segment's first max_seqlen_k keys
    wl = W.random_segments([30], [300], [280], topk=64, seed=50)
    q, k, w, cq, ck, offs = _dev(wl)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, 200)
    ids, sc = ix.topk(q, k, w, cq, ck, offs, topk=64, workspace=ws, max_seqlen_k=200)
    torch.cuda.synchronize()
    st, tk, dn = ix.read_status(ws)
    assert st & ix.STATUS_SEQLEN_BOUND and tk == 0 and dn == 0
    cut = W.Workload("cut", wl.q, wl.k[:200].contiguous(), wl.w, wl.cu_seqlens_q,
                     torch.tensor([0, 200], dtype=torch.int32), wl.q_pos_offsets, 64, 200)
    oi, osc, det = _oracle(cut)
    check_rows(ids.cpu().numpy(), sc.cpu().numpy(), range(cut.T), oi, osc, det, 64)


def test_no_queries_and_no_keys():
    d = "cuda"
    # no queries: nothing is enqueued and empty outputs come back
    q = torch.empty((0, 64, 128), dtype=torch.bfloat16, device=d)
    w = torch.empty((0, 64), dtype=torch.float32, device=d)
    k = torch.randn((50, 128), device=d).to(torch.bfloat16)
    cq = torch.tensor([0, 0], dtype=torch.int32, device=d)
    ck = torch.tensor([0, 50], dtype=torch.int32, device=d)
    ids, sc = ix.topk(q, k, w, cq, ck, None, topk=8, max_seqlen_k=50)
    torch.cuda.synchronize()
    assert ids.shape == (0, 8) and sc.shape == (0, 8)
    # no keys at all: every row is padding
    wl = W.random_segments([5, 7], [0, 0], [3, 0], topk=4, seed=51)
    dq, dk, dw, dcq, dck, doffs = _dev(wl)
    assert dk.shape[0] == 0
    ids, sc = ix.topk(dq, dk, dw, dcq, dck, doffs, topk=4, max_seqlen_k=1)
    torch.cuda.synchronize()
    assert bool((ids == -1).all()) and bool(torch.isneginf(sc).all())


def test_graph_capture_replays_match_eager():
    # the call enqueues only its kernels (no allocation, memset or host sync), so it can be
    # captured; replays interleaved with eager work and synchronisation must each match the
    # eager result bit for bit (the work-unit counter resets itself at the end of every run)
    wl = W.random_segments([100, 37], [900, 300], [800, 100], topk=128, seed=60)
    q, k, w, cq, ck, offs = _dev(wl)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k)
    oi = torch.empty((wl.T, 128), dtype=torch.int32, device="cuda")
    osc = torch.empty((wl.T, 128), dtype=torch.float32, device="cuda")
    kw = dict(topk=128, workspace=ws, max_seqlen_k=wl.max_seqlen_k, out_ids=oi, out_scores=osc)
    ix.topk(q, k, w, cq, ck, offs, **kw)
    torch.cuda.synchronize()
    ref = (oi.cpu().numpy().copy(), osc.cpu().numpy().copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ix.topk(q, k, w, cq, ck, offs, **kw)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(4):
        oi.fill_(7)
        osc.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(oi.cpu().numpy(), ref[0]), r
        assert np.array_equal(osc.cpu().numpy().view(np.uint32), ref[1].view(np.uint32)), r
        ix.topk(q, k, w, cq, ck, offs, **kw)       # eager work between replays
        torch.cuda.synchronize()
        assert ix.read_status(ws) == (0, 0, 0)


@pytest.mark.parametrize("seed", range(12))
def test_random_batches(seed):
    # seeded random segment tables: lengths from empty to a few thousand keys, offsets that put
    # queries before, inside and past their segment's keys, k from 1 to 2048; exercises the
    # plan's segment order and chunk choice and both select widths against the oracle.  (Seed
    # 1008 has as many units as tiles while one tile is split in five and four keyless tiles
    # have none: a unit-to-tile shortcut keyed on the totals alone skipped key columns there.)
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 9))
    ql = rng.integers(0, 40, B).tolist()
    kl = [int(x) for x in rng.choice([0, 5, 64, 300, 1000, 2500], B)]
    offs = [int(rng.integers(-20, k + 40)) for k in kl]
    topk = int(rng.choice([1, 7, 64, 256, 1000, 2048]))
    wl = W.random_segments(ql, kl, offs, topk=topk, seed=1000 + seed)
    _check_all(wl)


def _random_table(rng, max_b=40, max_q=60):
    B = int(rng.integers(1, max_b + 1))
    ql = rng.integers(0, max_q, B).tolist()
    kl = [int(x) for x in rng.choice([0, 1, 31, 64, 65, 200, 777, 2100], B)]
    offs = [int(rng.integers(-30, k + 50)) for k in kl]
    topk = int(rng.choice([1, 3, 16, 100, 512, 2048]))
    return ql, kl, offs, topk


@pytest.mark.parametrize("seed", range(8))
def test_random_integer_batches_exact(seed):
    # exact-arithmetic inputs over random tables, with random key-chunk and grid settings:
    # scores bit-equal to the oracle's and id sets identical (ties resolved by the larger id),
    # few distinct key vectors in half the cases so that long tie runs occur
    rng = np.random.default_rng(2000 + seed)
    ql, kl, offs, topk = _random_table(rng)
    distinct = int(rng.choice([2, 5, 0])) or None
    wl = W.integer_valued(ql, kl, offs, topk=topk, seed=2000 + seed, distinct_keys=distinct)
    tuning = dict(key_chunk_tiles=int(rng.choice([0, 1, 2, 5])), grid_blocks=int(rng.choice([0, 1, 3, 37])))
    _check_all(wl, exact=True, tuning=tuning)
