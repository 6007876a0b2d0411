"""The pipelined (65..128-head) kernel at every tile-count boundary, through
the C-ABI binding, against the CPU oracle.

A row of n used entries runs ceil(n / 64) key tiles: tiles with two more after
them take the steady path, the last two or three form their stream state at
the tile boundary, a tile's epilogue finishes two tiles later, and the row end
loads the next row's Q and lse as the tile loop ends. Here every row length
around a multiple of 64 (0 .. 16 tiles) appears, in a shuffled order, and the
work is split over a few workgroups (a caller's core budget), so that each
workgroup walks many rows and meets every transition between row lengths.

Bar: |gpu - oracle| <= 2e-5 per element on every row, and every row with a
used entry sums to 1 within 1e-4 (the derivation is in test_gpu_parity).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests import cases as C

pytestmark = pytest.mark.gpu

TOL = 2e-5
ROWSUM_TOL = 1e-4

# used entries per row: both sides of every multiple of 64 up to 1024
LENGTHS = sorted({0, 1, 2} | {v for m in range(64, 1025, 64) for v in (m - 1, m, m + 1)
                              if v <= 1024} | {700, 1000})


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_attention_02_amd as m
    return m


def _t(a, dev="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def with_lengths(p, seed):
    """p with topk_length set to LENGTHS, repeated over the rows and shuffled."""
    p = C.clone(p)
    rng = np.random.Generator(np.random.PCG64(seed))
    tl = np.resize(np.array(LENGTHS, dtype=np.int32), p.rows)
    rng.shuffle(tl)
    p.topk_length = tl.reshape(p.topk_length.shape)
    return p


def cases():
    cs = []
    cs.append(("bsnd_bf16_g128", with_lengths(
        C.gen("tiny", heads_q=128, batch=1, seqlen_q=3 * len(LENGTHS), seqlen_k=1100,
              topk=1024, mask_mode=0, seed=61), seed=1)))
    cs.append(("tnd_fp16_g96", with_lengths(
        C.gen("tnd_varlen", heads_q=96, topk=1024, mask_mode=0, seqlens_q=(60, 45),
              seqlens_k=(1100, 1030), seed=62), seed=2)))
    # dense rows: row i of a causal square sees i+1 keys (1 .. 10 tiles)
    cs.append(("dense_bsnd_g128_causal", C.gen("tiny", heads_q=128, batch=1, seqlen_q=600,
                                                seqlen_k=600, topk=0, mask_mode=3,
                                                seed=63)))
    return cs


CASES = cases()
BUDGETS = (0, 7, 3)


@pytest.mark.parametrize("budget", BUDGETS, ids=[f"cores{b}" for b in BUDGETS])
@pytest.mark.parametrize("case", range(len(CASES)), ids=[n for n, _ in CASES])
def test_tile_counts(smla, case, budget):
    name, p = CASES[case]
    p = C.clone(p)
    oracle.fill_lse(p)
    e = oracle.l1norm(p)
    md = smla.smla_l1norm_metadata(
        p.heads_q, p.heads_k, p.head_dim,
        cu_seqlens_q=_t(p.cu_seqlens_q, "cpu"), cu_seqlens_k=_t(p.cu_seqlens_k, "cpu"),
        batch_size=p.batch, max_seqlen_q=p.max_seqlen_q, max_seqlen_k=p.max_seqlen_k,
        topk=p.topk, layout_q=p.layout, layout_k=p.layout, mask_mode=p.mask_mode,
        cmp_ratio=p.cmp_ratio, device=0, core_budget=budget)
    print(f"[tiles] {name} layout={p.layout} R={p.rows} G={p.groups} K={p.topk} "
          f"workgroups={int(md[4])}", flush=True)
    o = smla.smla_softmax_l1norm(
        p.q.cuda(), p.k.cuda(), _t(np.asarray(p.softmax_lse, dtype=np.float32)),
        sparse_indices=_t(p.sparse_indices), cu_seqlens_q=_t(p.cu_seqlens_q),
        cu_seqlens_k=_t(p.cu_seqlens_k), topk_length=_t(p.topk_length), metadata=md,
        softmax_scale=p.softmax_scale, max_seqlen_k=p.max_seqlen_k, cmp_ratio=p.cmp_ratio,
        mask_mode=p.mask_mode, layout_q=p.layout, layout_k=p.layout)
    torch.cuda.synchronize()
    o = o.reshape(p.rows, p.out_width).cpu().numpy()
    err = np.abs(o.astype(np.float64) - e.astype(np.float64))
    assert float(err.max()) <= TOL, f"{name}: max |gpu - oracle| = {float(err.max()):.3e}"
    sums = o.astype(np.float64).sum(axis=1)
    live = e.astype(np.float64).sum(axis=1) > 0
    assert np.all(np.abs(sums[live] - 1.0) <= ROWSUM_TOL), f"{name}: row sums"
    assert not o[~live].any(), f"{name}: rows without a used entry must be zero"
