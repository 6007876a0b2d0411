"""Seeded synthetic inputs for the sparse softmax-L1Norm workloads.

This module only draws inputs. It holds none of the operation's arithmetic
(no scores, no softmax, no reduction): both the HIP path and the CPU oracle
consume what it produces, and neither shares any other code.

Recipe (stated once, used by every caller):

* q, k: ``numpy.random.Generator(PCG64(seed))`` standard normals in float32,
  multiplied by ``sigma`` and rounded to nearest-even to bf16/fp16 by torch.
  Exception: ``dist="uniform2"`` draws uniform [0, 2) values, the way the
  page's single-op example fills q and k.
* sparse_indices, one row at a time in row-major order: the row's candidate
  keys are the causal prefix ``[0, L)`` of its sequence's (compressed) keys
  (``L = S2_b`` without a mask); ``n = min(topk, L)`` distinct keys are drawn
  uniformly without replacement, in random order, and the rest of the row is
  padded with -1. ``topk_length`` holds ``n``.
* For the causal mask the prefix length follows the right-down-causal rule
  with compression, stated as an input recipe: a query at position ``i`` of a
  sequence with ``S1_b`` queries and ``S2_b`` compressed keys (compression
  ratio ``r``, residual ``res``) sits at original position
  ``i + S2_b*r + res - S1_b``; compressed key ``j`` covers original positions
  ``[j*r, (j+1)*r - 1]``; the prefix is every key whose last position is not
  after the query.
* dense workloads (``topk=0``) draw no sparse_indices and no topk_length:
  every key of a row's sequence is an entry (the page's dense case).
* softmax_lse is NOT drawn here for parity work: tests take it from the
  oracle. ``lse_standin`` gives a cheap stand-in with the same shape and a
  realistic magnitude for timing runs, where the values do not change the
  work done.

Sources for the shapes and names: the "SparseFlashMlaSoftmaxL1Norm" article
(CANN ops-transformer), parameter table in section 参数说明 and the single-op
example in section 调用方式二 PyTorch API.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = ["Problem", "Spec", "SPECS", "generate", "lse_standin", "visible_prefix"]

_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclasses.dataclass
class Problem:
    """One set of inputs in the operation's own tensor layouts."""

    name: str
    layout: str                 # "BSND" or "TND" (layout_q == layout_k)
    batch: int                  # B (BSND) or number of sequences (TND)
    seqlen_q: int               # S1 (BSND) or T1 (TND)
    seqlen_k: int               # S2 (BSND) or T2 (TND)
    heads_q: int                # N1
    heads_k: int                # N2
    head_dim: int               # D
    topk: int                   # K
    mask_mode: int              # 0 or 3
    cmp_ratio: int
    softmax_scale: float
    dtype: str                  # "bf16" or "fp16"
    q: torch.Tensor             # (B,S1,N1,D) or (T1,N1,D), CPU
    k: torch.Tensor             # (B,S2,N2,D) or (T2,N2,D), CPU
    sparse_indices: Optional[np.ndarray]  # int32 (B,S1,N2,K) or (T1,N2,K); None: dense
    topk_length: Optional[np.ndarray]      # int32 (B,S1,N2) or (T1,N2)
    cu_seqlens_q: Optional[np.ndarray]     # int32 (B+1,) for TND
    cu_seqlens_k: Optional[np.ndarray]
    cmp_residual_k: Optional[np.ndarray]   # int32 (B,)
    max_seqlen_q: int
    max_seqlen_k: int
    softmax_lse: Optional[np.ndarray] = None  # float32 (B,N2,S1,G) or (N2,T1,G)
    row_entries: Optional[np.ndarray] = None  # int64 (R,): keys drawn, or (dense) visible
    seqused_q: Optional[np.ndarray] = None    # int32 (B,): queries of each batch taking part
    seqused_k: Optional[np.ndarray] = None    # int32 (B,): keys of each batch taking part
    kwide: bool = False                       # output of K columns (entry t -> column t)

    @property
    def groups(self) -> int:
        return self.heads_q // self.heads_k

    @property
    def rows(self) -> int:
        """Query rows R = B*S1 (BSND) or T1 (TND)."""
        return self.batch * self.seqlen_q if self.layout == "BSND" else self.seqlen_q

    @property
    def out_width(self) -> int:
        """Last output dimension: S2 (BSND) or T2 (TND); K-wide: K, or without
        indices S2 (BSND) or max_seqlen_k (TND)."""
        if not self.kwide:
            return self.seqlen_k
        if self.sparse_indices is not None:
            return self.topk
        return self.seqlen_k if self.layout == "BSND" else self.max_seqlen_k

    def out_shape(self):
        if self.layout == "BSND":
            return (self.batch, self.seqlen_q, self.heads_k, self.out_width)
        return (self.seqlen_q, self.heads_k, self.out_width)

    def lse_shape(self):
        if self.layout == "BSND":
            return (self.batch, self.heads_k, self.seqlen_q, self.groups)
        return (self.heads_k, self.seqlen_q, self.groups)

    def valid_pairs(self) -> int:
        """Sum over rows of the keys drawn (sparse) or visible (dense)."""
        return int(self.row_entries.sum())


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    layout: str
    heads_q: int
    topk: int
    dtype: str
    mask_mode: int
    batch: int = 1
    seqlen_q: int = 0            # BSND S1
    seqlen_k: int = 0            # BSND S2 (compressed)
    seqlens_q: Sequence[int] = ()  # TND per-sequence query lengths
    seqlens_k: Sequence[int] = ()  # TND per-sequence key lengths
    cmp_ratio: int = 1
    cmp_residual: Optional[Sequence[int]] = None
    sigma: float = 1.0
    dist: str = "normal"         # "normal" or "uniform2"
    head_dim: int = 512
    seed: int = 0
    softmax_scale: Optional[float] = None  # default 1/sqrt(D)
    with_topk_length: bool = True


# The five workloads, plus the page-example stand-in. Sizes follow the
# benchmark table; all use N2 = 1, D = 512 and scale = 1/sqrt(512).
SPECS = {
    "tiny": Spec("tiny", "BSND", heads_q=4, topk=16, dtype="bf16", mask_mode=0,
                 batch=1, seqlen_q=8, seqlen_k=64, seed=1),
    "bsnd_causal": Spec("bsnd_causal", "BSND", heads_q=16, topk=512, dtype="bf16",
                        mask_mode=3, batch=2, seqlen_q=1024, seqlen_k=4096, seed=2),
    "dsv32": Spec("dsv32", "BSND", heads_q=128, topk=2048, dtype="bf16", mask_mode=3,
                  batch=1, seqlen_q=4096, seqlen_k=4096, seed=3),
    "tnd_varlen": Spec("tnd_varlen", "TND", heads_q=64, topk=2048, dtype="fp16",
                       mask_mode=3, seqlens_q=(1024, 3000, 512, 7000),
                       seqlens_k=(1024, 3000, 512, 7000), sigma=0.5, seed=4),
    "compressed": Spec("compressed", "BSND", heads_q=128, topk=512, dtype="bf16",
                       mask_mode=3, batch=1, seqlen_q=8192, seqlen_k=2048,
                       cmp_ratio=4, cmp_residual=(0,), seed=5),
    # The page's TND example (S1=16, S2=2048, N1=128, cmp_ratio=128, mask 3,
    # uniform [0,2) inputs), given indices so it runs on the sparse path.
    "page_example_sparse": Spec("page_example_sparse", "TND", heads_q=128, topk=2048,
                                dtype="fp16", mask_mode=3, seqlens_q=(16,),
                                seqlens_k=(2048,), cmp_ratio=128, cmp_residual=(0,),
                                dist="uniform2", seed=6),
    # Dense variant (no sparse_indices, every key of the sequence): the page's
    # example itself, and a causal 2048x2048 BSND shape to measure.
    "page_example_dense": Spec("page_example_dense", "TND", heads_q=128, topk=0,
                               dtype="fp16", mask_mode=3, seqlens_q=(16,),
                               seqlens_k=(2048,), cmp_ratio=128, cmp_residual=(0,),
                               dist="uniform2", seed=6),
    "dense_causal": Spec("dense_causal", "BSND", heads_q=128, topk=0, dtype="bf16",
                         mask_mode=3, batch=1, seqlen_q=2048, seqlen_k=2048, seed=7),
}


def visible_prefix(i: int, s1: int, s2: int, mask_mode: int, r: int, res: int) -> int:
    """Number of candidate keys [0, L) that the index recipe draws from."""
    if mask_mode == 0:
        return s2
    # query original position p = i + s2*r + res - s1; key j drawn iff (j+1)*r - 1 <= p
    p1 = i + 1 + s2 * r + res - s1
    if p1 <= 0:
        return 0
    return min(s2, p1 // r)


def _draw_values(rng: np.random.Generator, n: int, spec: Spec) -> np.ndarray:
    if spec.dist == "uniform2":
        return rng.random(n, dtype=np.float32) * np.float32(2.0)
    out = rng.standard_normal(n, dtype=np.float32)
    if spec.sigma != 1.0:
        out *= np.float32(spec.sigma)
    return out


def generate(spec: Spec | str, seed: Optional[int] = None, **overrides) -> Problem:
    """Draw one Problem for ``spec`` (a Spec or a name in SPECS).

    ``overrides`` replace Spec fields (used by tests for small variants).
    """
    if isinstance(spec, str):
        spec = SPECS[spec]
    if overrides:
        spec = dataclasses.replace(spec, **overrides)
    seed = spec.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    D, N1, N2, K = spec.head_dim, spec.heads_q, 1, spec.topk
    r = spec.cmp_ratio

    if spec.layout == "BSND":
        B, S1, S2 = spec.batch, spec.seqlen_q, spec.seqlen_k
        seq_q = [S1] * B
        seq_k = [S2] * B
        T1, T2 = B * S1, B * S2
        cu_q = cu_k = None
    elif spec.layout == "TND":
        seq_q = list(spec.seqlens_q)
        seq_k = list(spec.seqlens_k)
        B = len(seq_q)
        assert len(seq_k) == B
        T1, T2 = sum(seq_q), sum(seq_k)
        cu_q = np.concatenate([[0], np.cumsum(seq_q)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(seq_k)]).astype(np.int32)
    else:
        raise ValueError(spec.layout)

    res = list(spec.cmp_residual) if spec.cmp_residual is not None else None
    if res is not None:
        assert len(res) == B

    tdt = _DTYPES[spec.dtype]
    q32 = _draw_values(rng, T1 * N1 * D, spec)
    k32 = _draw_values(rng, T2 * N2 * D, spec)
    q = torch.from_numpy(q32).to(tdt)
    k = torch.from_numpy(k32).to(tdt)
    del q32, k32

    dense = K == 0
    idx = np.full((T1, K), -1, dtype=np.int32)
    tlen = np.zeros((T1,), dtype=np.int32)
    row = 0
    for b in range(B):
        s1, s2 = seq_q[b], seq_k[b]
        rb = res[b] if res is not None else 0
        for i in range(s1):
            L = visible_prefix(i, s1, s2, spec.mask_mode, r, rb)
            n = L if dense else min(K, L)
            if n > 0 and not dense:
                idx[row, :n] = rng.choice(L, n, replace=False)
            tlen[row] = n
            row += 1
    entries = tlen.astype(np.int64)

    scale = spec.softmax_scale if spec.softmax_scale is not None else 1.0 / math.sqrt(D)
    if spec.layout == "BSND":
        q = q.reshape(B, S1, N1, D)
        k = k.reshape(B, S2, N2, D)
        idx = idx.reshape(B, S1, N2, K)
        tlen = tlen.reshape(B, S1, N2)
        sq, sk = S1, S2
        mq, mk = S1, S2
    else:
        q = q.reshape(T1, N1, D)
        k = k.reshape(T2, N2, D)
        idx = idx.reshape(T1, N2, K)
        tlen = tlen.reshape(T1, N2)
        sq, sk = T1, T2
        mq, mk = max(seq_q), max(seq_k)

    return Problem(
        name=spec.name, layout=spec.layout, batch=B, seqlen_q=sq, seqlen_k=sk,
        heads_q=N1, heads_k=N2, head_dim=D, topk=K, mask_mode=spec.mask_mode,
        cmp_ratio=r, softmax_scale=scale, dtype=spec.dtype, q=q, k=k,
        sparse_indices=None if dense else idx,
        topk_length=tlen if spec.with_topk_length and not dense else None,
        cu_seqlens_q=cu_q, cu_seqlens_k=cu_k,
        cmp_residual_k=np.asarray(res, dtype=np.int32) if res is not None else None,
        max_seqlen_q=mq, max_seqlen_k=mk, row_entries=entries,
    )


def lse_standin(p: Problem) -> np.ndarray:
    """A cheap softmax_lse of the right shape for timing runs.

    For scores that are roughly normal with variance v, log(sum_t exp(s_t))
    is close to log(n) + v/2; v is taken as D*scale^2 (unit-variance q and
    k). The values only keep exp(s - lse) in a realistic range; they do not
    make rows sum to one. Rows with no drawn key get -inf.
    """
    n = p.row_entries.astype(np.float64)
    v = p.head_dim * p.softmax_scale ** 2
    base = np.where(n > 0, np.log(np.maximum(n, 1.0)) + 0.5 * v, -np.inf)
    lse = np.repeat(base[:, None], p.groups, axis=1).astype(np.float32)
    return lse.reshape(p.lse_shape())
