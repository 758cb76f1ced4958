"""Benchmark of the DSA indexer top-k scan on one MI355X.

One step = one dsa_indexer_topk call (score kernel + select kernel) over the
whole workload, inputs resident in HBM.  Default workload: one causal document
of N=8192 tokens, H=64, D=128, top-k 2048.

Prints ONE JSON line: queries/s for the whole call, the score kernel's
effective BF16 TFLOP/s over visible (query, key) pairs against the MI355X
dense BF16 MFMA peak (measured with HIP events recorded on the call's stream
around each kernel during the timed steps), and the FP64 oracle timed on a
bounded row sample on the host cores.
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
FLOP_PER_PAIR = 2 * 64 * 128   # one 64x128 by 128x1 contraction per visible (query, key) pair
COPY_BYTES = 512 << 20         # plain copy used to calibrate the FETCH_SIZE / WRITE_SIZE counters
CSRC = os.path.join(ROOT, "deterministic_score_top_amd", "csrc")
KERNEL_SRC = {"score": os.path.join(CSRC, "score_kernel.hip"), "attention": os.path.join(CSRC, "attention_kernel.hip")}


def kernel_hash(kernel="score"):
    return hashlib.sha256(open(KERNEL_SRC[kernel], "rb").read()).hexdigest()[:16]


def traffic_file(config, kernel="score"):
    return os.path.join(ROOT, "profiles", f"{kernel}_kernel_traffic_{config}.json")


def load_traffic(config, kernel="score"):
    """HBM bytes per launch of a kernel from committed counter runs, if its source is unchanged."""
    try:
        rec = json.load(open(traffic_file(config, kernel)))
    except (OSError, ValueError):
        return None
    if rec.get(f"{kernel}_kernel_sha256_16") != kernel_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def _pmc_avg(run_dir, counter, kernel_substr):
    vals = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"].lower():
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} samples for {kernel_substr} under {run_dir}")
    return sum(vals) / len(vals)


def ingest_traffic(config, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernel="score"):
    """Write profiles/<kernel>_kernel_traffic_<config>.json from four rocprofv3 --pmc runs."""
    copy_kernel = "copy"
    f_copy = _pmc_avg(copy_fetch_dir, "FETCH_SIZE", copy_kernel)   # KiB per dispatch
    w_copy = _pmc_avg(copy_write_dir, "WRITE_SIZE", copy_kernel)
    f_scale = COPY_BYTES / (f_copy * 1024.0)     # true bytes per counted byte
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    name = f"{kernel}_kernel("                   # the kernel itself, not e.g. attention_merge_kernel
    f = _pmc_avg(fetch_dir, "FETCH_SIZE", name) * 1024.0 * f_scale
    w = _pmc_avg(write_dir, "WRITE_SIZE", name) * 1024.0 * w_scale
    rec = {"config": config, f"{kernel}_kernel_sha256_16": kernel_hash(kernel),
           "fetch_bytes_per_launch": f, "write_bytes_per_launch": w, "bytes_per_launch": f + w,
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": f_copy, "write_kib": w_copy,
                                "fetch_scale": f_scale, "write_scale": w_scale}}
    json.dump(rec, open(traffic_file(config, kernel), "w"), indent=1)
    print(json.dumps(rec))


def _kernel_short(name):
    """Kernel name without namespaces, return type and parameter list (template arguments kept)."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].split("::")[-1]


def trace_summary(trace_dir, pmc_dirs=()):
    """Markdown summary of a rocprofv3 --kernel-trace run of bench.py: per workload phase (a new
    phase starts at each control-block fill, i.e. each workspace the run allocates), per kernel:
    dispatches, mean over all and over the last 20 (the timed calls) in microseconds.  With
    --pmc run directories of the same command (GRBM_GUI_ACTIVE), also the mean shader clock
    (counter cycles / kernel duration of the same dispatch)."""
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        rows += list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    phase, per = 0, {}
    for r in rows:
        name = r["Kernel_Name"]
        if "ctrl_init" in name:
            phase += 1
            continue
        short = _kernel_short(name)
        per.setdefault((phase, short), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| phase | kernel | dispatches | mean (us) | mean of the last 20 (us) |")
    print("|---:|---|---:|---:|---:|")
    for (ph, k), v in sorted(per.items()):
        print(f"| {ph} | {k} | {len(v)} | {sum(v) / len(v):.2f} | {sum(v[-20:]) / len(v[-20:]):.2f} |")
    for d in pmc_dirs:
        recs = []
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            recs += list(csv.DictReader(open(path)))
        by = {}
        for r in recs:
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                by.setdefault(_kernel_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        trace = {}
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                trace.setdefault(_kernel_short(r["Kernel_Name"]), []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        # the counter is summed over the GPU's XCCs, each counting its own engine-clock cycles
        nxcc = 1
        for path in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if r.get("Agent_Type") == "GPU":
                    nxcc = max(nxcc, int(r.get("Num_Xcc") or 1))
        for k, cyc in sorted(by.items()):
            if k in trace and len(trace[k]) == len(cyc):
                clk = [c / nxcc / t / 1e9 for c, t in zip(cyc, trace[k]) if t > 0]
                print(f"\n{os.path.basename(d.rstrip('/'))}: {k}: GRBM_GUI_ACTIVE / {nxcc} XCCs / duration = "
                      f"{sum(clk) / len(clk):.3f} GHz mean over {len(clk)} dispatches "
                      f"(min {min(clk):.3f}, max {max(clk):.3f})")


def copy_calibration(reps=5):
    """A plain device-to-device copy of COPY_BYTES, for counter calibration under rocprofv3."""
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x {reps}", flush=True)


def visible_pairs(wl):
    import numpy as np
    cq = wl.cu_seqlens_q.numpy().astype(np.int64)
    ck = wl.cu_seqlens_k.numpy().astype(np.int64)
    offs = np.zeros(wl.B, np.int64) if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy().astype(np.int64)
    total = 0
    for b in range(wl.B):
        i = np.arange(cq[b + 1] - cq[b], dtype=np.int64)
        total += int(np.clip(offs[b] + i + 1, 0, ck[b + 1] - ck[b]).sum())
    return total


def cpu_baseline(wl, ids, sc, budget_s):
    """FP64 oracle on the workload's rows until the time budget is spent; also checks those rows of the GPU output."""
    import numpy as np
    from oracle import dsa_oracle as O
    from tests.parity import check_rows
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    q64, k64, w64 = O.from_torch(wl.q, wl.k, wl.w)
    cu_q, cu_k = wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy()
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    order = np.random.default_rng(0).permutation(wl.T).tolist()   # every row, in a seeded random order
    done = []
    t0 = time.perf_counter()
    res = ([], [], [])
    for t in order:
        a, b, c = O.topk_rows(q64, k64, w64, cu_q, cu_k, offs, wl.topk, [t])
        res[0].append(a[0]); res[1].append(b[0]); res[2].append(c[0])
        done.append(t)
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    ok = True
    try:
        check_rows(ids, sc, done, np.stack(res[0]), np.stack(res[1]), res[2], wl.topk)
    except AssertionError as e:
        ok = False
        print(f"bench: sampled parity FAILED: {e}", file=sys.stderr)
    what = "all" if len(done) == wl.T else "a seeded random sample of"
    cpu = "unknown cpu"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": len(done) / el, "unit": "queries/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{what} {len(done)} of {wl.T} query rows of the same workload, one oracle call per row, "
                      f"{el:.1f} s, FP64 NumPy, host cpu_count={os.cpu_count()} ({cpu})"}, ok


def cpu_baseline_backward(wl, grad, dq, dw, budget_s):
    """FP64 oracle backward, one query row at a time, until the budget is spent; checks those rows' dq, dw."""
    import numpy as np
    from oracle import dsa_oracle as O
    from tests.parity import backward_row_bounds
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    q64, k64, w64 = O.from_torch(wl.q, wl.k, wl.w)
    cu_q, cu_k = wl.cu_seqlens_q.numpy(), wl.cu_seqlens_k.numpy()
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.numpy()
    order = np.random.default_rng(0).permutation(wl.T).tolist()
    done, ok = 0, True
    t0 = time.perf_counter()
    for t in order:
        first, n = O.visible(cu_q, cu_k, offs, t)
        g = grad[t, :n].astype(np.float64)
        rq, rw, _ = O.row_backward(q64, k64, w64, t, first, n, g)
        if n:
            bq, bw, _, _ = backward_row_bounds(q64, k64, w64, g, t, first, n)
            if (np.abs(dq[t] - rq) > bq).any() or (np.abs(dw[t] - rw) > bw).any():
                ok = False
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    what = "all" if done == wl.T else "a seeded random sample of"
    return {"value": done / el, "unit": "queries/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{what} {done} of {wl.T} query rows, one oracle row_backward call per row (dq, dw and the "
                      f"row's dk terms; the GPU's dq and dw of those rows checked against the derived error "
                      f"bound), {el:.1f} s, FP64 NumPy, host cpu_count={os.cpu_count()}"}, ok


def bench_backward(args):
    """One step = one dsa_indexer_backward call (dq/dw kernel + dk kernels) over the whole workload."""
    import torch
    from deterministic_score_top_amd import indexer as ix
    from deterministic_score_top_amd import workloads as W

    wl = W.make(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = wl.max_seqlen_k if wl.max_seqlen_k > 0 else wl.Tkv
    ld = (L + 3) // 4 * 4
    print(f"bench: backward {args.config} T={wl.T} Tkv={wl.Tkv} B={wl.B}", file=sys.stderr, flush=True)
    grad_h = W.draw_grad(wl.T, ld, seed=1)
    q, k, w = wl.q.to(dev), wl.k.to(dev), wl.w.to(dev)
    cq, ck = wl.cu_seqlens_q.to(dev), wl.cu_seqlens_k.to(dev)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(dev)
    grad = grad_h.to(dev)
    ws = torch.empty(ix.backward_workspace_size(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k), dtype=torch.uint8, device=dev)
    ix.workspace_init(ws)
    dq = torch.empty((wl.T, 64, 128), dtype=torch.float32, device=dev)
    dk = torch.empty((wl.Tkv, 128), dtype=torch.float32, device=dev)
    dw = torch.empty((wl.T, 64), dtype=torch.float32, device=dev)
    call = dict(max_seqlen_k=wl.max_seqlen_k, workspace=ws, dq=dq, dk=dk, dw=dw)
    for _ in range(args.warmup):
        ix.backward(q, k, w, cq, ck, grad, offs, **call)
    prof = ix.Profiler(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        ix.backward(q, k, w, cq, ck, grad, offs, profiler=prof, **call)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    per_q, per_k = prof.read_calls()
    prof.close()
    st = ix.read_status(ws)
    if st[0] != 0:
        print(f"bench: workspace status {st}", file=sys.stderr)
    pairs = visible_pairs(wl)
    ms = el * 1000.0 / args.steps
    q_ms, k_ms = sum(per_q) / len(per_q), sum(per_k) / len(per_k)
    # each kernel recomputes S (2HD per pair) and forms one gradient product (2HD per pair);
    # the call's algorithmic minimum is S once plus the two gradient products
    kern_flop = 2 * FLOP_PER_PAIR * pairs
    call_flop = 3 * FLOP_PER_PAIR * pairs
    dom_name, dom_ms = ("bwd_dq_kernel", q_ms) if q_ms >= k_ms else ("bwd_dk_kernel + reduce", k_ms)
    eff_dom = kern_flop / (dom_ms * 1e-3) / 1e12
    eff_call = call_flop / (ms * 1e-3) / 1e12
    print(f"bench: backward {ms:.4f} ms/call, dq/dw kernel {q_ms:.4f} ms, dk kernels {k_ms:.4f} ms",
          file=sys.stderr, flush=True)
    line = {
        "metric": "indexer backward queries/s + effective TFLOP/s (frac of BF16 MFMA peak)",
        "value": wl.T / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.config, "T": wl.T, "Tkv": wl.Tkv, "segments": wl.B, "heads": 64,
                   "head_dim": 128, "visible_pairs": pairs, "grad": "N(0,1) FP32, seed 1"},
        "effective_tflops_call": eff_call,
        "flop_per_pair_call": 3 * FLOP_PER_PAIR,
        "dq_kernel_ms": q_ms,
        "dk_kernels_ms": k_ms,
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": eff_dom, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": eff_dom / PEAK_BF16_TFLOPS, "flop_per_pair": 2 * FLOP_PER_PAIR,
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["parity_sample_ok"] = cpu_baseline_backward(
            wl, grad_h.numpy(), dq.cpu().numpy(), dw.cpu().numpy(), args.cpu_budget)
    print(json.dumps(line), flush=True)


ATTN_FLOP_PER_ID = 2 * 128 * 576 + 2 * 128 * 512   # scores and value product of one (query, valid id)


def bench_attention(args):
    """One step = one dsa_indexer_sparse_attention call over the workload's rows, with the ids the
    indexer selects for that workload (its top-k call runs once, outside the timed region)."""
    import numpy as np
    import torch
    from deterministic_score_top_amd import indexer as ix
    from deterministic_score_top_amd import workloads as W

    wl = W.make(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: attention {args.config} T={wl.T} Tkv={wl.Tkv} topk={wl.topk}", file=sys.stderr, flush=True)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(dev)
    ids, _ = ix.topk(wl.q.to(dev), wl.k.to(dev), wl.w.to(dev), wl.cu_seqlens_q.to(dev), wl.cu_seqlens_k.to(dev),
                     offs, topk=wl.topk, max_seqlen_k=wl.max_seqlen_k)
    q_h, kv_h = W.draw_attention(wl.T, wl.Tkv, seed=2)
    q, kv = q_h.to(dev), kv_h.to(dev)
    scale = 1.0 / math.sqrt(576)
    ws = torch.empty(ix.sparse_attention_workspace_size(wl.T, wl.topk), dtype=torch.uint8, device=dev)
    ix.workspace_init(ws)
    out = torch.empty((wl.T, 128, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.T, 128), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        ix.sparse_attention(q, kv, ids, scale, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        ix.sparse_attention(q, kv, ids, scale, out=out, lse=lse, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    kern = sorted(a.elapsed_time(b) for a, b in ev)
    k_ms = sum(kern) / len(kern)
    ids_h = ids.cpu().numpy()
    valid = int((ids_h >= 0).sum())
    ms = el * 1000.0 / args.steps
    eff = ATTN_FLOP_PER_ID * valid / (k_ms * 1e-3) / 1e12
    print(f"bench: attention {ms:.4f} ms/call, kernel {k_ms:.4f} ms", file=sys.stderr, flush=True)
    line = {
        "metric": "sparse attention over the selected ids: queries/s + effective TFLOP/s (frac of BF16 MFMA peak)",
        "value": wl.T / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.config, "T": wl.T, "Tkv": wl.Tkv, "topk": wl.topk, "heads": 128,
                   "qk_dim": 576, "v_dim": 512, "valid_ids": valid,
                   "ids": "the indexer's top-k of the same workload"},
        "kernel_ms": k_ms,
        "roofline": {"bound": "mfma", "kernel": "attention_kernel", "achieved": eff, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": eff / PEAK_BF16_TFLOPS, "flop_per_valid_id": ATTN_FLOP_PER_ID,
                     "gather_bytes_per_valid_id": 2 * 1152,
                     "traffic": load_traffic(args.config, "attention")},
    }
    if not args.no_cpu_baseline:
        from oracle import dsa_oracle as O
        q64, kv64 = q_h.double().numpy(), kv_h.double().numpy()
        o_h, l_h = out.cpu().numpy(), lse.cpu().numpy()
        order = np.random.default_rng(0).permutation(wl.T).tolist()
        done, ok = 0, True
        t0 = time.perf_counter()
        for t in order:
            ro, rl = O.sparse_attention_row(q64[t], kv64, ids_h[t], scale, 512)
            if np.linalg.norm(o_h[t] - ro) > 2.0 ** -7 * max(np.linalg.norm(ro), 1e-30):
                ok = False
            done += 1
            if time.perf_counter() - t0 > args.cpu_budget:
                break
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": done / el, "unit": "queries/s", "cores": os.cpu_count(), "kind": "oracle",
                                "sample": f"{done} of {wl.T} query rows in a seeded random order, one oracle "
                                          f"sparse_attention_row call per row, {el:.1f} s, FP64 NumPy"}
        line["parity_sample_ok"] = ok
    print(json.dumps(line), flush=True)


def warm_up(call, calls, min_s):
    """`calls` untimed calls, then more until at least `min_s` seconds of back-to-back calls have run
    (a fresh GPU raises its clock over the first few hundred milliseconds of load)."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while n < calls or time.perf_counter() - t0 < min_s:
        for _ in range(16):
            call()
        n += 16
        torch.cuda.synchronize()
    return n, time.perf_counter() - t0


def _pct(v, f):
    v = sorted(v)
    return v[min(len(v) - 1, int(round(f * (len(v) - 1))))]


def score_kernel_gate(dev, min_warm_s, steps=20, config="causal_n16384", gate=0.5):
    """Score-kernel fraction of the BF16 peak on one causal document of N=16384 (the score phase
    must reach half of the peak there), measured in the calling process after its own warm-up."""
    import torch
    from deterministic_score_top_amd import indexer as ix
    from deterministic_score_top_amd import workloads as W
    wl = W.make(config)
    q, k, w = wl.q.to(dev), wl.k.to(dev), wl.w.to(dev)
    cq, ck = wl.cu_seqlens_q.to(dev), wl.cu_seqlens_k.to(dev)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(dev)
    ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k, dev)
    oi = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=dev)
    osc = torch.empty((wl.T, wl.topk), dtype=torch.float32, device=dev)
    kw = dict(topk=wl.topk, workspace=ws, max_seqlen_k=wl.max_seqlen_k, out_ids=oi, out_scores=osc)
    warm_up(lambda: ix.topk(q, k, w, cq, ck, offs, **kw), 5, min_warm_s)
    prof = ix.Profiler(steps)
    for _ in range(steps):
        ix.topk(q, k, w, cq, ck, offs, profiler=prof, **kw)
    torch.cuda.synchronize()
    per_score, per_select = prof.read_calls()
    prof.close()
    score_ms = sum(per_score) / len(per_score)
    eff = FLOP_PER_PAIR * visible_pairs(wl) / (score_ms * 1e-3) / 1e12
    del ws, oi, osc, q, k, w
    torch.cuda.empty_cache()
    return {"workload": config, "calls": steps, "score_kernel_ms": score_ms,
            "score_kernel_ms_p10_p50_p90": [_pct(per_score, f) for f in (0.1, 0.5, 0.9)],
            "select_kernel_ms": sum(per_select) / len(per_select),
            "achieved_tflops": eff, "frac": eff / PEAK_BF16_TFLOPS, "gate_frac": gate,
            "pass": eff / PEAK_BF16_TFLOPS >= gate}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="causal_n8192")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warmup-s", type=float, default=2.0,
                    help="after the --warmup calls, keep warming up until this many seconds have passed")
    ap.add_argument("--call", choices=("eager", "prepared"), default="eager",
                    help="eager: dsa_indexer_topk per call; prepared: one dsa_indexer_prepare, then dsa_indexer_run")
    ap.add_argument("--no-gate", action="store_true",
                    help="skip the N=16384 score-kernel measurement that the headline run adds")
    ap.add_argument("--hold-cus", type=int, default=0,
                    help="before each timed call, hold this many CUs with a foreign kernel (tests/native "
                         "helper) for --hold-frac of the warm call time")
    ap.add_argument("--hold-frac", type=float, default=0.5)
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 512 MiB buffer between timed calls (L2 and MALL cold); value is then "
                         "T / median per-call GPU time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the scores (dq, dk, dw) instead of the top-k call")
    ap.add_argument("--attention", action="store_true",
                    help="time the sparse attention over the selected ids instead of the top-k call")
    ap.add_argument("--trace-summary", nargs="+", metavar="DIR",
                    help="print a markdown summary of a rocprofv3 --kernel-trace directory (then optional "
                         "--pmc GRBM_GUI_ACTIVE --kernel-trace directories for the shader clock) and exit")
    ap.add_argument("--ingest-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the score-kernel traffic record from rocprofv3 --pmc output directories")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary[0], args.trace_summary[1:])
        return
    if args.ingest_pmc:
        ingest_traffic(args.config, *args.ingest_pmc, kernel="attention" if args.attention else "score")
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the scan shards by queries; a multi-GPU driver is not part of this library)", file=sys.stderr)
        sys.exit(2)

    if args.backward:
        bench_backward(args)
        return
    if args.attention:
        bench_attention(args)
        return

    import torch
    from deterministic_score_top_amd import indexer as ix
    from deterministic_score_top_amd import workloads as W

    wl = W.make(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: {args.config} T={wl.T} Tkv={wl.Tkv} B={wl.B} topk={wl.topk}", file=sys.stderr, flush=True)
    q, k, w = wl.q.to(dev), wl.k.to(dev), wl.w.to(dev)
    cq, ck = wl.cu_seqlens_q.to(dev), wl.cu_seqlens_k.to(dev)
    offs = None if wl.q_pos_offsets is None else wl.q_pos_offsets.to(dev)
    out_ids = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=dev)
    out_sc = torch.empty((wl.T, wl.topk), dtype=torch.float32, device=dev)
    if args.call == "prepared":
        # the prepared runner: arguments bound and the plan stored once; each call only launches
        runner = ix.prepare(q, k, w, cq, ck, offs, topk=wl.topk, max_seqlen_k=wl.max_seqlen_k,
                            out_ids=out_ids, out_scores=out_sc)
        ws = runner.workspace

        def topk_call(profiler=None):
            runner.run(profiler)
    else:
        ws = ix.alloc_workspace(wl.T, wl.Tkv, wl.B, wl.max_seqlen_k, dev)
        call = dict(topk=wl.topk, workspace=ws, max_seqlen_k=wl.max_seqlen_k, out_ids=out_ids, out_scores=out_sc)

        def topk_call(profiler=None):
            ix.topk(q, k, w, cq, ck, offs, profiler=profiler, **call)

    flush = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev) if args.cold else None
    warm_calls, warm_s = warm_up(topk_call, args.warmup, args.warmup_s)
    # host path per call: enqueue cost of back-to-back calls (no synchronisation in between), and
    # the wall time of one synchronised call (host path + GPU + completion), median of 100
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(100):
        topk_call()
    host_us = (time.perf_counter() - t0) * 1e4
    torch.cuda.synchronize()
    sync_wall = []
    for _ in range(100):
        t0 = time.perf_counter()
        topk_call()
        torch.cuda.synchronize()
        sync_wall.append((time.perf_counter() - t0) * 1e3)
    hold = None
    if args.hold_cus > 0:
        import ctypes
        hold = ctypes.CDLL(os.path.join(ROOT, "tests", "native", "libspinner.so"))
        hold.spinner_start.argtypes = [ctypes.c_int, ctypes.c_double]
        hold.spinner_wait_resident.argtypes = [ctypes.c_double]
        wprof = ix.Profiler(20)
        for _ in range(20):
            topk_call(wprof)
        a, b = wprof.read_calls()
        wprof.close()
        hold_us = args.hold_frac * 1000.0 * sorted(x + y for x, y in zip(a, b))[len(a) // 2]
        args.steps = min(args.steps, 50)
    prof = ix.Profiler(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if flush is not None:
            flush.fill_(1.0)
        if hold is not None:
            torch.cuda.synchronize()
            if hold.spinner_start(args.hold_cus, hold_us) != 0 or hold.spinner_wait_resident(1000.0) != 0:
                raise SystemExit("bench: could not start the CU holder")
        topk_call(prof)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    per_score, per_select = prof.read_calls()
    prof.close()
    calls = len(per_score)
    score_ms, select_ms = sum(per_score), sum(per_select)
    per_call = sorted(a + b for a, b in zip(per_score, per_select))
    pct = _pct
    st = ix.read_status(ws)
    if st != (0, 0, 0):
        print(f"bench: workspace status {st}", file=sys.stderr)

    pairs = visible_pairs(wl)
    ms = el * 1000.0 / args.steps
    if args.cold or hold is not None:   # time the calls themselves on the GPU
        ms = pct(per_call, 0.5)
    score_avg_ms = score_ms / calls
    select_avg_ms = select_ms / calls
    eff_call = FLOP_PER_PAIR * pairs / (ms * 1e-3) / 1e12
    eff_score = FLOP_PER_PAIR * pairs / (score_avg_ms * 1e-3) / 1e12
    print(f"bench: {ms:.4f} ms/call, score kernel {score_avg_ms:.4f} ms, select kernel {select_avg_ms:.4f} ms",
          file=sys.stderr, flush=True)

    line = {
        "metric": "indexer queries/s + effective TFLOP/s (frac of BF16 MFMA peak), N=8192 k=2048",
        "value": wl.T / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.config, "T": wl.T, "Tkv": wl.Tkv, "segments": wl.B, "topk": wl.topk,
                   "heads": 64, "head_dim": 128, "visible_pairs": pairs,
                   "structure": wl.meta.get("structure", "")},
        "effective_tflops_call": eff_call,
        "frac_bf16_peak_call": eff_call / PEAK_BF16_TFLOPS,
        "score_kernel_ms": score_avg_ms,
        "select_kernel_ms": select_avg_ms,
        "call": args.call,
        "host_enqueue_us_per_call": host_us,
        "sync_call_wall_ms_p50": _pct(sync_wall, 0.5),
        "warmup_calls_run": warm_calls,
        "warmup_s_run": warm_s,
        "score_kernel_ms_per_call": {"first5": per_score[:5], "last5": per_score[-5:],
                                     "p10": pct(per_score, 0.1), "p50": pct(per_score, 0.5),
                                     "p90": pct(per_score, 0.9)},
        "select_kernel_ms_per_call": {"p10": pct(per_select, 0.1), "p50": pct(per_select, 0.5),
                                      "p90": pct(per_select, 0.9)},
        "call_gpu_ms": {"p10": pct(per_call, 0.1), "p50": pct(per_call, 0.5), "p90": pct(per_call, 0.9),
                        "l2": "cold (512 MiB written between calls)" if args.cold else "warm"},
        "foreign_load": ({"held_cus": args.hold_cus, "held_us": hold_us,
                          "note": "a foreign kernel holds the CUs from just before each call for that long"}
                         if hold is not None else None),
        "roofline": {"bound": "mfma", "kernel": "score_kernel", "achieved": eff_score,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": eff_score / PEAK_BF16_TFLOPS,
                     "traffic": load_traffic(args.config)},
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        ids_h, sc_h = out_ids.cpu().numpy(), out_sc.cpu().numpy()
        line["cpu_baseline"], ok = cpu_baseline(wl, ids_h, sc_h, args.cpu_budget)
        line["parity_sample_ok"] = ok
    if args.config == "causal_n8192" and not args.no_gate and hold is None and not args.cold:
        del ws
        torch.cuda.empty_cache()
        print("bench: score-kernel gate on causal_n16384", file=sys.stderr, flush=True)
        line["score_gate_causal_n16384"] = score_kernel_gate(dev, args.warmup_s)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
