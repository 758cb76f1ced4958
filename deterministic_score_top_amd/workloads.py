"""Seeded synthetic inputs for the DSA indexer top-k scan.

This module only draws inputs: queries, keys, head weights and the segment
tables (cu_seqlens, per-segment causal position offsets).  It computes none of
the scan's arithmetic, so the FP64 oracle and the HIP path can both consume it
without sharing any of the method.

Workload shapes follow the eager-entry tables of flashinfer PR #8691
("perf(cake_dsa_indexer_det): ticket scheduling on sm_107a, no fill kernel in
eager entry"), rows S1, S2, C1, Z3cp and A3: single causal documents, a context
parallel tail, a packed zigzag rank share and a four-query split tail.  Those
pages print neither head count nor head dim nor value distributions; the
adopted values are H=64, D=128, q and k ~ N(0,1) rounded to BF16 and
w ~ U(0,1)/sqrt(H) in FP32.

Every tensor is a CPU torch tensor:
  q  bf16  [T, H, D]      row-major
  k  bf16  [Tkv, D]       row-major
  w  fp32  [T, H]
  cu_seqlens_q, cu_seqlens_k  int32 [B+1]
  q_pos_offsets               int32 [B] or None (all zero)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

H_DEFAULT = 64
D_DEFAULT = 128


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    w: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    q_pos_offsets: Optional[torch.Tensor]
    topk: int
    max_seqlen_k: int
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def Tkv(self) -> int:
        return int(self.k.shape[0])

    @property
    def B(self) -> int:
        return int(self.cu_seqlens_q.numel() - 1)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def draw_qkw(g: torch.Generator, T: int, Tkv: int, H: int = H_DEFAULT, D: int = D_DEFAULT):
    """q, k ~ N(0,1) rounded to BF16; w ~ U(0,1)/sqrt(H) in FP32."""
    q = torch.randn((T, H, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((Tkv, D), generator=g, dtype=torch.float32).to(torch.bfloat16)
    w = torch.rand((T, H), generator=g, dtype=torch.float32) / math.sqrt(H)
    return q, k, w


def _i32(xs) -> torch.Tensor:
    return torch.tensor(list(xs), dtype=torch.int32)


def segments(q_lens, k_lens, offsets=None):
    """Build cu_seqlens_q / cu_seqlens_k / offsets tensors from per-segment lengths."""
    cq = np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))])
    ck = np.concatenate([[0], np.cumsum(np.asarray(k_lens, dtype=np.int64))])
    offs = None if offsets is None else _i32(offsets)
    return _i32(cq), _i32(ck), offs


def single_causal(n: int, topk: int, seed: int = 0, name: str = "") -> Workload:
    """One document of n tokens; query i sees keys 0..i (rows S1/S2 of the tables)."""
    g = _gen(seed)
    q, k, w = draw_qkw(g, n, n)
    cq, ck, _ = segments([n], [n])
    return Workload(name or f"causal_n{n}", q, k, w, cq, ck, None, topk, n,
                    {"structure": f"one causal document, T=Tkv={n}"})


def cp_tail(n_keys: int = 65536, n_q: int = 4096, topk: int = 2048, seed: int = 0) -> Workload:
    """Context-parallel tail: the last n_q queries of one n_keys document (row C1)."""
    g = _gen(seed)
    q, k, w = draw_qkw(g, n_q, n_keys)
    cq, ck, offs = segments([n_q], [n_keys], [n_keys - n_q])
    return Workload("cp_tail", q, k, w, cq, ck, offs, topk, n_keys,
                    {"structure": f"one document of {n_keys} keys, queries at positions "
                                  f"{n_keys - n_q}..{n_keys - 1}"})


def zigzag_doc_lengths(n_docs: int, target_keys: int = 169984, tol: float = 0.01):
    """Document lengths log-uniform in [4096, 65536], multiples of 32.

    L = floor(4096 * 16**u / 32) * 32 with u = default_rng(s).random(n_docs);
    s is the first seed >= 0 whose total is within tol of target_keys.  The
    target is the packed row's key count with the per-chunk key segments
    removed (175296 * 32 / 33).
    """
    for s in range(0, 1_000_000):
        u = np.random.default_rng(s).random(n_docs)
        L = (np.floor(4096.0 * 16.0 ** u / 32.0).astype(np.int64) * 32)
        if abs(int(L.sum()) - target_keys) <= tol * target_keys:
            return s, L
    raise RuntimeError("no seed found")


def zigzag_share(n_docs: int = 16, topk: int = 2048, seed: int = 0, chunks: int = 32) -> Workload:
    """Packed varlen share of one context-parallel rank under zigzag assignment (row Z3cp).

    Each document of length L is cut into `chunks` chunks of c = L/chunks
    tokens; this rank holds chunk 0 and chunk chunks-1.  Each held chunk is its
    own segment: chunk 0 sees the document's first c keys at offset 0, the last
    chunk sees all L keys at offset (chunks-1)*c.  Both key segments are copies
    of the same document keys.
    """
    len_seed, L = zigzag_doc_lengths(n_docs)
    g = _gen(seed)
    q_lens, k_lens, offs = [], [], []
    k_parts = []
    for Li in L.tolist():
        c = Li // chunks
        kd = torch.randn((Li, D_DEFAULT), generator=g, dtype=torch.float32).to(torch.bfloat16)
        q_lens += [c, c]
        k_lens += [c, Li]
        offs += [0, (chunks - 1) * c]
        k_parts += [kd[:c], kd]
    T = int(sum(q_lens))
    q = torch.randn((T, H_DEFAULT, D_DEFAULT), generator=g, dtype=torch.float32).to(torch.bfloat16)
    w = torch.rand((T, H_DEFAULT), generator=g, dtype=torch.float32) / math.sqrt(H_DEFAULT)
    k = torch.cat(k_parts, 0).contiguous()
    cq, ck, o = segments(q_lens, k_lens, offs)
    return Workload(f"zigzag{n_docs}", q, k, w, cq, ck, o, topk, int(max(k_lens)),
                    {"structure": f"{n_docs} docs, lengths {L.tolist()}, length seed {len_seed}, "
                                  f"chunks 0 and {chunks - 1} of {chunks}", "doc_lengths": L.tolist(),
                     "length_seed": len_seed})


def split_tail(n_keys: int = 41986, n_q: int = 4, topk: int = 2048, seed: int = 0,
               tie: bool = False, distinct: int = 16) -> Workload:
    """A few queries at the end of one long segment (rows A1-A3).

    With tie=True every key row is one of `distinct` BF16 vectors, so each
    query's scores take at most `distinct` values and the larger-id rule
    decides which keys of the top group are kept.
    """
    g = _gen(seed)
    q, k, w = draw_qkw(g, n_q, n_keys)
    if tie:
        V = torch.randn((distinct, D_DEFAULT), generator=g, dtype=torch.float32).to(torch.bfloat16)
        j = torch.randint(0, distinct, (n_keys,), generator=g)
        k = V[j].contiguous()
    cq, ck, offs = segments([n_q], [n_keys], [n_keys - n_q])
    return Workload("split_tail_tie" if tie else "split_tail", q, k, w, cq, ck, offs, topk, n_keys,
                    {"structure": f"{n_q} queries at positions {n_keys - n_q}..{n_keys - 1} of one "
                                  f"segment of {n_keys} keys" + (f"; keys from {distinct} vectors" if tie else "")})


def integer_valued(T_lens, K_lens, offsets, topk, H=H_DEFAULT, D=D_DEFAULT, seed=0,
                   qk_range=4, w_den=64, distinct_keys: Optional[int] = None) -> Workload:
    """Small-integer BF16 q, k in [-qk_range, qk_range] and dyadic w = m / w_den.

    Every dot product is an integer of modest size and every weighted term is
    a dyadic rational, so FP32 sums of them are exact whatever the order.
    """
    g = _gen(seed)
    T, Tkv = int(sum(T_lens)), int(sum(K_lens))
    q = torch.randint(-qk_range, qk_range + 1, (T, H, D), generator=g).to(torch.bfloat16)
    if distinct_keys:
        V = torch.randint(-qk_range, qk_range + 1, (distinct_keys, D), generator=g).to(torch.bfloat16)
        k = V[torch.randint(0, distinct_keys, (Tkv,), generator=g)].contiguous()
    else:
        k = torch.randint(-qk_range, qk_range + 1, (Tkv, D), generator=g).to(torch.bfloat16)
    w = torch.randint(0, w_den + 1, (T, H), generator=g).to(torch.float32) / float(w_den)
    cq, ck, o = segments(T_lens, K_lens, offsets)
    return Workload("integer", q, k, w, cq, ck, o, topk, int(max(K_lens) if len(K_lens) else 0))


def random_segments(T_lens, K_lens, offsets, topk, H=H_DEFAULT, D=D_DEFAULT, seed=0) -> Workload:
    """Gaussian inputs over an arbitrary segment table."""
    g = _gen(seed)
    q, k, w = draw_qkw(g, int(sum(T_lens)), int(sum(K_lens)), H, D)
    cq, ck, o = segments(T_lens, K_lens, offsets)
    return Workload("random", q, k, w, cq, ck, o, topk, int(max(K_lens) if len(K_lens) else 0))


def draw_grad(T: int, ld: int, seed: int = 0, integer: bool = False) -> torch.Tensor:
    """Upstream gradients of the scores, FP32 [T, ld] in the scores-export row layout.

    Gaussian N(0,1), or with integer=True dyadic values n/16, n in [-7, 7] (three
    significant bits, exact in BF16 and in every FP32 product with the other
    integer-valued inputs).
    """
    g = _gen(seed + 7919)
    if integer:
        return torch.randint(-7, 8, (T, ld), generator=g).to(torch.float32) / 16.0
    return torch.randn((T, ld), generator=g, dtype=torch.float32)


def draw_attention(T: int, Tkv: int, H: int = 128, dqk: int = 576, seed: int = 0):
    """Inputs of the sparse attention that consumes the selection: q bf16 [T, H, dqk] ~ N(0,1)
    and the latent KV table bf16 [Tkv, dqk] ~ N(0,1)."""
    g = _gen(seed + 104729)
    q = torch.randn((T, H, dqk), generator=g, dtype=torch.float32).to(torch.bfloat16)
    kv = torch.randn((Tkv, dqk), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return q, kv


CONFIGS = {
    # name: (builder, description)
    "causal_n1024": lambda seed=0: single_causal(1024, 256, seed, "causal_n1024"),
    "causal_n8192": lambda seed=0: single_causal(8192, 2048, seed, "causal_n8192"),
    "cp_tail": lambda seed=0: cp_tail(seed=seed),
    "zigzag16": lambda seed=0: zigzag_share(16, seed=seed),
    "zigzag8": lambda seed=0: zigzag_share(8, seed=seed),
    "split_tail": lambda seed=0: split_tail(seed=seed),
    "split_tail_tie": lambda seed=0: split_tail(seed=seed, tie=True),
    "causal_n16384": lambda seed=0: single_causal(16384, 2048, seed, "causal_n16384"),
}


def make(name: str, seed: int = 0) -> Workload:
    return CONFIGS[name](seed)
