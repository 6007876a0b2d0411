"""The GPU softmax_lse producer against the CPU oracle's lse, through the C ABI.

``smla_softmax_lse`` computes, per row and head, the log-sum-exp of the
scaled scores over the row's used entries (-inf for a row with none): the
softmax_lse input of the main call (the article's parameter table names it
the forward pass's log-sum-exp).

Bar: |gpu - oracle| <= 2e-5 wherever the oracle's lse is finite, and -inf
exactly where it is -inf. An lse error d scales every probability
exp(s - lse) of its head by exp(-d), so this is the same 2e-5 relative bound
the main call's outputs are held to. End to end, the main call fed with the
GPU's lse must give rows that sum to 1 within 1e-4 (every row with a used
entry), and match the oracle's output for that same lse within 2e-5.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import cases as C
from tests.test_gpu_parity import (MEDIUM, ROWSUM_TOL, TINY, TOL, _t, rows_view, run_gpu,
                                   say)

pytestmark = pytest.mark.gpu

TOL_LSE = 2e-5


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_attention_02_amd as m
    return m


def metadata(smla, p, core_budget=0):
    return smla.smla_l1norm_metadata(
        p.heads_q, p.heads_k, p.head_dim,
        cu_seqlens_q=_t(p.cu_seqlens_q, "cpu"), cu_seqlens_k=_t(p.cu_seqlens_k, "cpu"),
        cmp_residual_k=_t(p.cmp_residual_k, "cpu"), batch_size=p.batch,
        max_seqlen_q=p.max_seqlen_q, max_seqlen_k=p.max_seqlen_k, topk=p.topk,
        layout_q=p.layout, layout_k=p.layout, mask_mode=p.mask_mode, cmp_ratio=p.cmp_ratio,
        core_budget=core_budget)


def run_lse(smla, p, core_budget=0):
    """smla_softmax_lse for Problem p; returns (R, G) float32 numpy."""
    md = metadata(smla, p, core_budget)
    lse = smla.smla_softmax_lse(
        p.q.cuda(), p.k.cuda(), sparse_indices=_t(p.sparse_indices),
        cu_seqlens_q=_t(p.cu_seqlens_q), cu_seqlens_k=_t(p.cu_seqlens_k),
        cmp_residual_k=_t(p.cmp_residual_k), topk_length=_t(p.topk_length), metadata=md,
        softmax_scale=p.softmax_scale, max_seqlen_k=p.max_seqlen_k, cmp_ratio=p.cmp_ratio,
        mask_mode=p.mask_mode, layout_q=p.layout, layout_k=p.layout)
    torch.cuda.synchronize()
    assert tuple(lse.shape) == tuple(p.lse_shape())
    return lse.cpu().numpy().reshape(p.rows, p.groups)


def check_lse(name, got, want):
    dead = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), dead), f"{name}: -inf pattern"
    live = ~dead
    assert np.isfinite(got[live]).all(), f"{name}: non-finite lse"
    err = np.abs(got[live].astype(np.float64) - want[live].astype(np.float64))
    worst = float(err.max()) if err.size else 0.0
    say(f"    max |lse gpu - oracle| = {worst:.2e}")
    assert worst <= TOL_LSE, f"{name}: max |lse gpu - oracle| = {worst:.3e}"


def check_end_to_end(name, smla, p, lse_gpu, rows=None):
    """The main call fed with the GPU's lse: rows with a used entry sum to 1;
    on `rows` (all if None) it matches the oracle's output for that lse."""
    o = rows_view(p, run_gpu(smla, p, lse=lse_gpu.reshape(p.lse_shape()))).cpu().numpy()
    live = p.row_entries.reshape(p.rows) > 0
    sums = o.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(sums[live] - 1.0) <= ROWSUM_TOL), f"{name}: row sums with GPU lse"
    assert not o[~live].any(), f"{name}: rows without entries must be zero"
    sel = np.arange(p.rows) if rows is None else rows
    e = oracle.l1norm(p, rows=None if rows is None else rows,
                      softmax_lse=lse_gpu.reshape(p.lse_shape()))
    err = np.abs(o[sel].astype(np.float64) - e.astype(np.float64))
    assert float(err.max()) <= TOL, f"{name}: output with GPU lse vs oracle"


@pytest.mark.parametrize("case", range(len(TINY)), ids=[n for n, _ in TINY])
def test_lse_tiny(smla, case):
    name, p = TINY[case]
    p = C.clone(p)
    say(f"[lse tiny] {name} layout={p.layout} R={p.rows} G={p.groups} K={p.topk}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p)
    check_lse(name, got, want)


@pytest.mark.parametrize("case", range(len(MEDIUM)), ids=[n for n, _ in MEDIUM])
def test_lse_medium(smla, case):
    name, p = MEDIUM[case]
    p = C.clone(p)
    say(f"[lse medium] {name} layout={p.layout} R={p.rows} G={p.groups} K={p.topk} "
        f"dtype={p.dtype}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p)
    check_lse(name, got, want)
    check_end_to_end(name, smla, p, got)


def test_lse_core_budget_split_gives_the_same_bits(smla):
    """With a caller's core budget the rows are split over that many
    workgroups instead of the kernel's co-resident count; each row's value
    does not depend on which workgroup computes it."""
    p = C.gen("tnd_varlen", heads_q=128, topk=300, seqlens_q=(70, 33, 90),
              seqlens_k=(500, 64, 900), seed=61)
    say("[lse] core budget 7 vs device split")
    a = run_lse(smla, p)
    b = run_lse(smla, p, core_budget=7)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_lse_without_keys_is_minus_inf(smla):
    p = C.gen("tnd_varlen", heads_q=16, topk=4, seqlens_q=(3, 5), seqlens_k=(0, 0), seed=62)
    say("[lse] no keys")
    got = run_lse(smla, p)
    assert np.isneginf(got).all()


FULL = ["dsv32", "tnd_varlen", "compressed", "bsnd_causal", "page_example_dense",
        "dense_causal"]


@pytest.mark.parametrize("name", FULL)
def test_lse_full_size(smla, name):
    say(f"[lse full] {name}: generating inputs")
    p = workloads.generate(name)
    say(f"[lse full] {name}: GPU lse (R={p.rows} G={p.groups} K={p.topk})")
    got = run_lse(smla, p)
    say(f"[lse full] {name}: oracle lse on all {p.rows} rows")
    want, _ = oracle.lse(p)
    check_lse(name, got, want)
    say(f"[lse full] {name}: main call with the GPU lse, every row against the oracle")
    check_end_to_end(name, smla, p, got)


@pytest.mark.parametrize("heads", [16, 128])
def test_lse_score_jump(smla, heads):
    """Eight keys scaled by 100 and moved to the end of every row's index
    list: their scores lie far above the base the earlier tiles set (well
    past the range the 16-head kernel's lazy step accepts), so the last tile
    must rebase exactly. Scores are large here, so the bar is relative:
    |d| <= 2e-5 * max(1, |lse|)."""
    p = C.gen("tiny", heads_q=heads, batch=1, seqlen_q=8, seqlen_k=300, topk=256, mask_mode=0,
              seed=63)
    idx = p.sparse_indices.reshape(p.rows, p.topk)
    jump = np.arange(8) * 37
    for r in range(p.rows):
        late = np.isin(idx[r], jump)
        idx[r] = np.concatenate([idx[r][~late], idx[r][late]])
    p.k.reshape(-1, p.head_dim)[torch.from_numpy(jump)] *= 100
    say(f"[lse] score jump, G={heads}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p)
    assert np.isfinite(got).all()
    d = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert (d <= 2e-5 * np.maximum(1.0, np.abs(want))).all(), float(d.max())
    assert np.abs(want).max() > 50  # the jump is really there


@pytest.mark.parametrize("heads", [16, 128])
def test_lse_scores_far_below_zero(smla, heads):
    """Every score about -370 in log2 units (q all ones, every key near all
    minus ones, scale 0.5): far below any fixed starting base, so the sums
    must rebase downwards instead of underflowing to an lse of -inf. The
    bar is relative, as for the score jump: |d| <= 2e-5 * max(1, |lse|)."""
    p = C.gen("tiny", heads_q=heads, batch=1, seqlen_q=8, seqlen_k=300, topk=256, mask_mode=0,
              seed=64)
    p.q.fill_(1.0)
    kk = p.k.reshape(-1, p.head_dim)
    kk.copy_((-1.0 + 0.01 * torch.randn(kk.shape, generator=torch.Generator().manual_seed(5)))
             .to(kk.dtype))
    p.softmax_scale = 0.5
    say(f"[lse] scores far below zero, G={heads}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p)
    assert np.isfinite(want).all() and (want < -200).all()  # the case is really there
    assert np.isfinite(got).all()
    d = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert (d <= 2e-5 * np.maximum(1.0, np.abs(want))).all(), float(d.max())


@pytest.mark.parametrize("layout", ["BSND", "TND"])
def test_lse_holes_in_long_rows(smla, layout):
    """Unused entries inside topk_length in the middle of long rows (128
    heads, 24 tiles of 64 entries): a few -1 pads, a whole tile of -1 pads,
    or half the entries pointing past the sequence. Tiles holding such
    entries are summed with their masks, the full tiles around them without,
    and a tile with no used entry adds nothing."""
    if layout == "BSND":
        p = C.gen("tiny", heads_q=128, batch=1, seqlen_q=48, seqlen_k=3000, topk=1536,
                  mask_mode=0, seed=71)
    else:
        p = C.gen("tnd_varlen", heads_q=128, topk=1536, seqlens_q=(20, 28),
                  seqlens_k=(3000, 2600), mask_mode=0, dtype="bf16", seed=73)
    rng = np.random.Generator(np.random.PCG64(71))
    R, K = p.rows, p.topk
    idx = p.sparse_indices.reshape(R, K)
    for r in range(R):
        kind = r % 4
        if kind == 1:
            idx[r, rng.choice(K, 3, replace=False)] = -1
        elif kind == 2:
            t = int(rng.integers(1, K // 64 - 1))
            idx[r, 64 * t:64 * t + 64] = -1
        elif kind == 3:
            idx[r, rng.choice(K, K // 2, replace=False)] = 5000
    say(f"[lse] holes in long rows, G=128, {layout}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p)
    check_lse("holes", got, want)
    check_end_to_end("holes", smla, p, got)


@pytest.mark.parametrize("heads", [64, 128])
def test_lse_score_jump_mid_row(smla, heads):
    """Eight keys scaled by 100 in tile 9 of rows of 24 full tiles: the tile
    that sums them lies in the steady part of the row and must rebase
    exactly there. The bar is relative: |d| <= 2e-5 * max(1, |lse|)."""
    p = C.gen("tiny", heads_q=heads, batch=1, seqlen_q=8, seqlen_k=3000, topk=1536,
              mask_mode=0, seed=72)
    idx = p.sparse_indices.reshape(p.rows, p.topk)
    jump = np.arange(8) * 301
    for r in range(p.rows):
        late = np.isin(idx[r], jump)
        rest = idx[r][~late]
        idx[r] = np.concatenate([rest[:9 * 64], idx[r][late], rest[9 * 64:]])
    p.k.reshape(-1, p.head_dim)[torch.from_numpy(jump)] *= 100
    say(f"[lse] score jump in the middle of the row, G={heads}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p)
    assert np.isfinite(got).all()
    d = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert (d <= 2e-5 * np.maximum(1.0, np.abs(want))).all(), float(d.max())
    assert np.abs(want).max() > 50  # the jump is really there


# used entries per row: 0, 1, 2 and both sides of every multiple of 64 up to
# 704 (1 .. 12 key tiles), in a shuffled order
LSE_LENGTHS = sorted({0, 1, 2} | {v for m in range(64, 705, 64) for v in (m - 1, m, m + 1)
                                   if v <= 704})


@pytest.mark.parametrize("budget", (3, 7), ids=("cores3", "cores7"))
@pytest.mark.parametrize("heads,layout", [(16, "BSND"), (16, "TND"), (33, "BSND"),
                                           (64, "TND")],
                         ids=["g16_bsnd", "g16_tnd", "g33_bsnd", "g64_tnd"])
def test_lse_rows_of_every_length_few_workgroups(smla, heads, layout, budget):
    """Rows of every tile count, split over a few workgroups, so that each
    workgroup walks many rows and meets every transition between row lengths
    (for up to 16 heads the key-tile stream runs on from row to row, and
    short rows count extra tiles without a used entry); every row's lse
    against the oracle's."""
    rng = np.random.Generator(np.random.PCG64(80 + heads))
    n = len(LSE_LENGTHS)
    if layout == "BSND":
        p = C.gen("tiny", heads_q=heads, batch=1, seqlen_q=2 * n, seqlen_k=800, topk=704,
                  mask_mode=0, seed=81)
    else:
        p = C.gen("tnd_varlen", heads_q=heads, topk=704, mask_mode=0, seqlens_q=(n, n),
                  seqlens_k=(800, 760), dtype="fp16", seed=82)
    p = C.clone(p)
    tl = np.resize(np.array(LSE_LENGTHS, dtype=np.int32), p.rows)
    rng.shuffle(tl)
    p.topk_length = tl.reshape(p.topk_length.shape)
    say(f"[lse lengths] G={heads} {layout} R={p.rows} K={p.topk} cores={budget}")
    want, _ = oracle.lse(p)
    got = run_lse(smla, p, core_budget=budget)
    check_lse(f"lengths g{heads} {layout} cores{budget}", got, want)
