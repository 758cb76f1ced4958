"""Thin ctypes binding of libdsa_indexer.so (the C ABI in include/dsa_indexer.h).

Argument marshalling only: every step of the scan runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.  Tensors are
checked for dtype, device, shape and contiguity and are never copied: a
non-contiguous argument is rejected (a silent copy of an output would lose the
result).  The library is loaded on first use; if it is missing the call
raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_indexer.so")

H = 64
D = 128
MAX_TOPK = 2048
MAX_SEQLEN_K = 65536

OK = 0
STATUS_CORRUPT_COUNTER = 0x1
STATUS_BAD_SEGMENTS = 0x2
STATUS_SEQLEN_BOUND = 0x4

EXPORTED_SYMBOLS = (
    "dsa_indexer_workspace_size",
    "dsa_indexer_workspace_init",
    "dsa_indexer_topk",
    "dsa_indexer_scores",
    "dsa_indexer_status_string",
    "dsa_indexer_profiler_create",
    "dsa_indexer_profiler_destroy",
    "dsa_indexer_profiler_read",
    "dsa_indexer_profiler_read_calls",
    "dsa_indexer_topk_ex",
    "dsa_indexer_read_status",
    "dsa_indexer_backward_workspace_size",
    "dsa_indexer_backward",
    "dsa_indexer_backward_ex",
    "dsa_indexer_sparse_attention",
    "dsa_indexer_sparse_attention_workspace_size",
    "dsa_indexer_topk_noalloc",
    "dsa_indexer_noalloc_max_bytes",
    "dsa_indexer_prepared_workspace_size",
    "dsa_indexer_prepare",
    "dsa_indexer_run",
    "dsa_indexer_run_ex",
    "dsa_indexer_runner_destroy",
)
STATUS_BAD_IDS = 0x8
ATTN_HEADS, ATTN_QK_DIM, ATTN_V_DIM = 128, 576, 512


class Shape(ctypes.Structure):
    _fields_ = [("num_segments", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("total_k", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32)]


class Tuning(ctypes.Structure):
    _fields_ = [("key_chunk_tiles", ctypes.c_int32), ("grid_blocks", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 6)]


class DsaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib().dsa_indexer_status_string(code).decode() if _LIB is not None else str(code)
        super().__init__(f"{where}: {msg} (code {code})")


_LIB = None


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sp = ctypes.POINTER(Shape)
        L.dsa_indexer_workspace_size.argtypes = [sp]
        L.dsa_indexer_workspace_size.restype = sz
        L.dsa_indexer_workspace_init.argtypes = [vp, sz, vp]
        L.dsa_indexer_workspace_init.restype = ctypes.c_int
        L.dsa_indexer_topk.argtypes = [sp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.dsa_indexer_topk.restype = ctypes.c_int
        L.dsa_indexer_topk_ex.argtypes = [sp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp,
                                          ctypes.POINTER(Tuning), vp]
        L.dsa_indexer_topk_ex.restype = ctypes.c_int
        L.dsa_indexer_scores.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i64, vp, sz, vp]
        L.dsa_indexer_scores.restype = ctypes.c_int
        L.dsa_indexer_status_string.argtypes = [ctypes.c_int]
        L.dsa_indexer_status_string.restype = ctypes.c_char_p
        L.dsa_indexer_profiler_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.dsa_indexer_profiler_create.restype = ctypes.c_int
        L.dsa_indexer_profiler_destroy.argtypes = [vp]
        L.dsa_indexer_profiler_destroy.restype = ctypes.c_int
        L.dsa_indexer_profiler_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
        L.dsa_indexer_profiler_read.restype = ctypes.c_int
        L.dsa_indexer_profiler_read_calls.argtypes = [vp, ctypes.POINTER(ctypes.c_float),
                                                      ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32)]
        L.dsa_indexer_profiler_read_calls.restype = ctypes.c_int
        L.dsa_indexer_read_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32),
                                              ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
        L.dsa_indexer_read_status.restype = ctypes.c_int
        L.dsa_indexer_backward_workspace_size.argtypes = [sp]
        L.dsa_indexer_backward_workspace_size.restype = sz
        L.dsa_indexer_backward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
        L.dsa_indexer_backward.restype = ctypes.c_int
        L.dsa_indexer_backward_ex.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp, vp]
        L.dsa_indexer_backward_ex.restype = ctypes.c_int
        L.dsa_indexer_sparse_attention.argtypes = [i32, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp, sz, vp]
        L.dsa_indexer_sparse_attention.restype = ctypes.c_int
        L.dsa_indexer_sparse_attention_workspace_size.argtypes = [i32, i32]
        L.dsa_indexer_sparse_attention_workspace_size.restype = sz
        L.dsa_indexer_topk_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.dsa_indexer_topk_noalloc.restype = ctypes.c_int
        L.dsa_indexer_noalloc_max_bytes.argtypes = []
        L.dsa_indexer_noalloc_max_bytes.restype = sz
        L.dsa_indexer_prepared_workspace_size.argtypes = [sp]
        L.dsa_indexer_prepared_workspace_size.restype = sz
        L.dsa_indexer_prepare.argtypes = [sp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp, ctypes.POINTER(vp)]
        L.dsa_indexer_prepare.restype = ctypes.c_int
        L.dsa_indexer_run.argtypes = [vp, vp]
        L.dsa_indexer_run.restype = ctypes.c_int
        L.dsa_indexer_run_ex.argtypes = [vp, vp, vp]
        L.dsa_indexer_run_ex.restype = ctypes.c_int
        L.dsa_indexer_runner_destroy.argtypes = [vp]
        L.dsa_indexer_runner_destroy.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(code: int, where: str):
    if code != OK:
        raise DsaError(code, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_shape(T: int, Tkv: int, B: int, max_seqlen_k: int = 0) -> Shape:
    return Shape(int(B), int(T), int(Tkv), H, D, int(max_seqlen_k))


def workspace_size(T: int, Tkv: int, B: int, max_seqlen_k: int = 0) -> int:
    s = make_shape(T, Tkv, B, max_seqlen_k)
    n = lib().dsa_indexer_workspace_size(ctypes.byref(s))
    if n == 0:
        raise DsaError(-3, "workspace_size")
    return int(n)


def workspace_init(ws: torch.Tensor):
    _check(lib().dsa_indexer_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(ws.device)),
           "workspace_init")


def alloc_workspace(T: int, Tkv: int, B: int, max_seqlen_k: int = 0, device="cuda") -> torch.Tensor:
    """A fresh, initialised workspace (uint8 tensor)."""
    ws = torch.empty(workspace_size(T, Tkv, B, max_seqlen_k), dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def _require(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (it is never copied)")


def _inputs(q, k, w, cu_q, cu_k, offs):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, Tkv, B = q.shape[0], k.shape[0], cu_q.numel() - 1
    _require(q, "q", torch.bfloat16, (T, H, D), dev)
    _require(k, "k", torch.bfloat16, (Tkv, D), dev)
    _require(w, "w", torch.float32, (T, H), dev)
    _require(cu_q, "cu_seqlens_q", torch.int32, (B + 1,), dev)
    _require(cu_k, "cu_seqlens_k", torch.int32, (B + 1,), dev)
    if offs is not None:
        _require(offs, "q_pos_offsets", torch.int32, (B,), dev)
    return dev, T, Tkv, B


class Profiler:
    """Per-kernel HIP-event timing of topk calls (score kernel, select kernel)."""

    def __init__(self, capacity: int):
        h = ctypes.c_void_p()
        _check(lib().dsa_indexer_profiler_create(int(capacity), ctypes.byref(h)), "profiler_create")
        self.handle = h
        self.capacity = int(capacity)

    def read(self):
        a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
        _check(lib().dsa_indexer_profiler_read(self.handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)),
               "profiler_read")
        return a.value, b.value, n.value

    def read_calls(self):
        """Per-call (score ms, select ms) lists, oldest first; empties the profiler."""
        a = (ctypes.c_float * self.capacity)()
        b = (ctypes.c_float * self.capacity)()
        n = ctypes.c_int32()
        _check(lib().dsa_indexer_profiler_read_calls(self.handle, a, b, self.capacity, ctypes.byref(n)),
               "profiler_read_calls")
        return list(a[:n.value]), list(b[:n.value])

    def close(self):
        if self.handle:
            lib().dsa_indexer_profiler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_WS_CACHE = {}


def _default_workspace(dev, T, Tkv, B, max_seqlen_k):
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    need = workspace_size(T, Tkv, B, max_seqlen_k)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < need:
        ws = alloc_workspace(T, Tkv, B, max_seqlen_k, dev)
        _WS_CACHE[key] = ws
    return ws


def topk(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets=None, topk: int = 2048,
         workspace: Optional[torch.Tensor] = None, max_seqlen_k: int = 0,
         out_ids: Optional[torch.Tensor] = None, out_scores: Optional[torch.Tensor] = None,
         tuning: Optional[dict] = None, profiler: Optional[Profiler] = None):
    """Top-k key ids (int32 [T, topk], ascending, -1 padded) and scores (fp32, -inf padded)."""
    dev, T, Tkv, B = _inputs(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets)
    if out_ids is None:
        out_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if out_scores is None:
        out_scores = torch.empty((T, topk), dtype=torch.float32, device=dev)
    _require(out_ids, "out_ids", torch.int32, (T, topk), dev)
    _require(out_scores, "out_scores", torch.float32, (T, topk), dev)
    if workspace is None:
        workspace = _default_workspace(dev, T, Tkv, B, max_seqlen_k)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    shape = make_shape(T, Tkv, B, max_seqlen_k)
    args = (ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            _ptr(q_pos_offsets), int(topk), _ptr(out_ids), _ptr(out_scores), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(dev))
    if tuning is None and profiler is None:
        rc = lib().dsa_indexer_topk(*args)
    else:
        tn = None
        if tuning is not None:
            tn = Tuning(int(tuning.get("key_chunk_tiles", 0)), int(tuning.get("grid_blocks", 0)))
        rc = lib().dsa_indexer_topk_ex(*args, None if tn is None else ctypes.byref(tn),
                                       None if profiler is None else profiler.handle)
    _check(rc, "dsa_indexer_topk")
    return out_ids, out_scores


def prepared_workspace_size(T: int, Tkv: int, B: int, max_seqlen_k: int = 0) -> int:
    s = make_shape(T, Tkv, B, max_seqlen_k)
    n = lib().dsa_indexer_prepared_workspace_size(ctypes.byref(s))
    if n == 0:
        raise DsaError(-3, "prepared_workspace_size")
    return int(n)


class Runner:
    """A prepared top-k call (dsa_indexer_prepare): bound tensors, plan stored in the workspace.

    run() enqueues the scan's two kernels on the current stream and returns (out_ids, out_scores).
    The tensors stay referenced by the runner; their values may change between runs.
    """

    def __init__(self, q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets=None, topk: int = 2048,
                 max_seqlen_k: int = 0, out_ids: Optional[torch.Tensor] = None,
                 out_scores: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
        dev, T, Tkv, B = _inputs(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets)
        if out_ids is None:
            out_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
        if out_scores is None:
            out_scores = torch.empty((T, topk), dtype=torch.float32, device=dev)
        _require(out_ids, "out_ids", torch.int32, (T, topk), dev)
        _require(out_scores, "out_scores", torch.float32, (T, topk), dev)
        if workspace is None:
            workspace = torch.empty(prepared_workspace_size(T, Tkv, B, max_seqlen_k), dtype=torch.uint8, device=dev)
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        self.handle = None
        self.device = dev
        self.tensors = (q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, out_ids, out_scores, workspace)
        self.out_ids, self.out_scores, self.workspace = out_ids, out_scores, workspace
        shape = make_shape(T, Tkv, B, max_seqlen_k)
        h = ctypes.c_void_p()
        _check(lib().dsa_indexer_prepare(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens_q),
                                         _ptr(cu_seqlens_k), _ptr(q_pos_offsets), int(topk), _ptr(out_ids),
                                         _ptr(out_scores), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(dev),
                                         ctypes.byref(h)), "dsa_indexer_prepare")
        self.handle = h

    def run(self, profiler: Optional["Profiler"] = None):
        if profiler is None:
            rc = lib().dsa_indexer_run(self.handle, _stream(self.device))
        else:
            rc = lib().dsa_indexer_run_ex(self.handle, _stream(self.device), profiler.handle)
        _check(rc, "dsa_indexer_run")
        return self.out_ids, self.out_scores

    def close(self):
        if self.handle:
            lib().dsa_indexer_runner_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prepare(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets=None, topk: int = 2048, **kw) -> Runner:
    return Runner(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets, topk, **kw)


def topk_noalloc(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets=None, topk: int = 2048,
                 max_seqlen_k: int = 0, out_ids: Optional[torch.Tensor] = None,
                 out_scores: Optional[torch.Tensor] = None):
    """topk() through the entry point that allocates nothing (the library's fixed per-GPU array)."""
    dev, T, Tkv, B = _inputs(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets)
    if out_ids is None:
        out_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if out_scores is None:
        out_scores = torch.empty((T, topk), dtype=torch.float32, device=dev)
    _require(out_ids, "out_ids", torch.int32, (T, topk), dev)
    _require(out_scores, "out_scores", torch.float32, (T, topk), dev)
    shape = make_shape(T, Tkv, B, max_seqlen_k)
    rc = lib().dsa_indexer_topk_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens_q),
                                        _ptr(cu_seqlens_k), _ptr(q_pos_offsets), int(topk), _ptr(out_ids),
                                        _ptr(out_scores), _stream(dev))
    _check(rc, "dsa_indexer_topk_noalloc")
    return out_ids, out_scores


def noalloc_max_bytes() -> int:
    return int(lib().dsa_indexer_noalloc_max_bytes())


def scores(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets=None, max_seqlen_k: int = 0,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Score phase only: fp32 [T, ld] with row t holding I[t, first_key + j] at column j < n_t.

    Columns past each row's visible count keep whatever `out` held (NaN if allocated here).
    """
    dev, T, Tkv, B = _inputs(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets)
    L = max_seqlen_k if max_seqlen_k > 0 else max(Tkv, 1)
    ld = (L + 3) // 4 * 4
    if out is None:
        out = torch.full((T, ld), float("nan"), dtype=torch.float32, device=dev)
    if out.dtype != torch.float32 or out.dim() != 2 or out.shape[0] != T or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [T, ld] tensor")
    if workspace is None:
        workspace = _default_workspace(dev, T, Tkv, B, max_seqlen_k)
    shape = make_shape(T, Tkv, B, max_seqlen_k)
    rc = lib().dsa_indexer_scores(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens_q),
                                  _ptr(cu_seqlens_k), _ptr(q_pos_offsets), _ptr(out), int(out.shape[1]),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, "dsa_indexer_scores")
    return out


def backward_workspace_size(T: int, Tkv: int, B: int, max_seqlen_k: int = 0) -> int:
    s = make_shape(T, Tkv, B, max_seqlen_k)
    n = lib().dsa_indexer_backward_workspace_size(ctypes.byref(s))
    if n == 0:
        raise DsaError(-3, "backward_workspace_size")
    return int(n)


def backward(q, k, w, cu_seqlens_q, cu_seqlens_k, grad, q_pos_offsets=None, max_seqlen_k: int = 0,
             workspace: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
             profiler: Optional[Profiler] = None):
    """Gradients (dq fp32 [T,H,D], dk fp32 [Tkv,D], dw fp32 [T,H]) of the scores.

    grad: fp32 [T, ld] in the layout `scores` returns (column j of row t = key first_t + j;
    only the visible columns are read).
    """
    dev, T, Tkv, B = _inputs(q, k, w, cu_seqlens_q, cu_seqlens_k, q_pos_offsets)
    if grad.dtype != torch.float32 or grad.dim() != 2 or grad.shape[0] != T or not grad.is_contiguous() \
            or grad.device != dev:
        raise ValueError("grad must be a contiguous fp32 [T, ld] tensor on the inputs' device")
    if dq is None:
        dq = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((Tkv, D), dtype=torch.float32, device=dev)
    if dw is None:
        dw = torch.empty((T, H), dtype=torch.float32, device=dev)
    _require(dq, "dq", torch.float32, (T, H, D), dev)
    _require(dk, "dk", torch.float32, (Tkv, D), dev)
    _require(dw, "dw", torch.float32, (T, H), dev)
    if workspace is None:
        workspace = torch.empty(backward_workspace_size(T, Tkv, B, max_seqlen_k), dtype=torch.uint8, device=dev)
        workspace_init(workspace)
    shape = make_shape(T, Tkv, B, max_seqlen_k)
    args = (ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
            _ptr(q_pos_offsets), _ptr(grad), int(grad.shape[1]), _ptr(dq), _ptr(dk), _ptr(dw),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    if profiler is None:
        rc = lib().dsa_indexer_backward(*args)
    else:
        rc = lib().dsa_indexer_backward_ex(*args, profiler.handle)
    _check(rc, "dsa_indexer_backward")
    return dq, dk, dw


def sparse_attention_workspace_size(total_q: int, topk: int) -> int:
    """Workspace bytes dsa_indexer_sparse_attention needs for total_q rows of topk ids."""
    n = lib().dsa_indexer_sparse_attention_workspace_size(int(total_q), int(topk))
    if n == 0:
        raise ValueError(f"unsupported topk {topk}")
    return n


def sparse_attention(q, kv, ids, scale: float, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Attention of each query row over its selected ids: out fp32 [T, 128, 512], lse fp32 [T, 128].

    q bf16 [T, 128, 576]; kv bf16 [Tkv, 576] (value = leading 512 dims); ids int32 [T, topk], -1 = none.
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, Tkv = q.shape[0], kv.shape[0]
    if ids.dim() != 2 or ids.shape[0] != T:
        raise ValueError("ids must be [T, topk]")
    k = ids.shape[1]
    _require(q, "q", torch.bfloat16, (T, ATTN_HEADS, ATTN_QK_DIM), dev)
    _require(kv, "kv", torch.bfloat16, (Tkv, ATTN_QK_DIM), dev)
    _require(ids, "ids", torch.int32, (T, k), dev)
    if out is None:
        out = torch.empty((T, ATTN_HEADS, ATTN_V_DIM), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((T, ATTN_HEADS), dtype=torch.float32, device=dev)
    _require(out, "out", torch.float32, (T, ATTN_HEADS, ATTN_V_DIM), dev)
    _require(lse, "lse", torch.float32, (T, ATTN_HEADS), dev)
    if workspace is None:
        workspace = torch.empty(sparse_attention_workspace_size(T, k), dtype=torch.uint8, device=dev)
        workspace_init(workspace)
    rc = lib().dsa_indexer_sparse_attention(int(T), int(Tkv), int(k), _ptr(q), _ptr(kv), _ptr(ids), float(scale),
                                            _ptr(out), _ptr(lse), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, "dsa_indexer_sparse_attention")
    return out, lse


def read_status(workspace: torch.Tensor):
    """(status, ticket, done) of a workspace's control block; synchronises the current stream."""
    st, tk, dn = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
    _check(lib().dsa_indexer_read_status(_ptr(workspace), _stream(workspace.device), ctypes.byref(st),
                                         ctypes.byref(tk), ctypes.byref(dn)), "read_status")
    return st.value, tk.value, dn.value
