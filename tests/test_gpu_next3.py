"""seqused_q / seqused_k and the K-wide output on the GPU against the oracle.

Both follow readings of the pages that the pages give no example of (their
parity is unpinned by the pages; the oracle's readings are pinned by
relations in ``tests/pins.py``): seqused_q[b] / seqused_k[b] drop queries /
keys past the counts, and the K-wide output (the shape-inference section)
puts entry t's value at column t of a row of K columns (without
sparse_indices: S2, or max_seqlen_k for TND).

Bar: the main call's as in ``test_gpu_parity.py`` (|gpu - oracle| <= 2e-5
per element, rows with a used entry summing to 1 within 1e-4 with the
oracle's lse), the lse call's as in ``test_gpu_lse.py``.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests import cases as C
from tests.test_gpu_lse import TOL_LSE
from tests.test_gpu_parity import ROWSUM_TOL, TOL, _t, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_attention_02_amd as m
    return m


def _args(smla, p):
    md = smla.smla_l1norm_metadata(
        p.heads_q, p.heads_k, p.head_dim,
        cu_seqlens_q=_t(p.cu_seqlens_q, "cpu"), cu_seqlens_k=_t(p.cu_seqlens_k, "cpu"),
        cmp_residual_k=_t(p.cmp_residual_k, "cpu"), batch_size=p.batch,
        max_seqlen_q=p.max_seqlen_q, max_seqlen_k=p.max_seqlen_k, topk=p.topk,
        layout_q=p.layout, layout_k=p.layout, mask_mode=p.mask_mode, cmp_ratio=p.cmp_ratio)
    return dict(
        sparse_indices=_t(p.sparse_indices), cu_seqlens_q=_t(p.cu_seqlens_q),
        cu_seqlens_k=_t(p.cu_seqlens_k), seqused_q=_t(p.seqused_q), seqused_k=_t(p.seqused_k),
        cmp_residual_k=_t(p.cmp_residual_k), topk_length=_t(p.topk_length), metadata=md,
        softmax_scale=p.softmax_scale, max_seqlen_k=p.max_seqlen_k, cmp_ratio=p.cmp_ratio,
        mask_mode=p.mask_mode, layout_q=p.layout, layout_k=p.layout)


def run_main(smla, p, lse):
    o = smla.smla_softmax_l1norm(p.q.cuda(), p.k.cuda(), _t(np.asarray(lse, np.float32)),
                                 kwide=p.kwide, **_args(smla, p))
    torch.cuda.synchronize()
    assert tuple(o.shape) == tuple(p.out_shape())
    return o.cpu().numpy().reshape(p.rows, p.out_width)


def run_lse(smla, p):
    l = smla.smla_softmax_lse(p.q.cuda(), p.k.cuda(), **_args(smla, p))
    torch.cuda.synchronize()
    return l.cpu().numpy().reshape(p.rows, p.groups)


def check(name, smla, p):
    want_l, nused = oracle.lse(p)
    got_l = run_lse(smla, p)
    dead = np.isneginf(want_l)
    assert np.array_equal(np.isneginf(got_l), dead), f"{name}: lse -inf pattern"
    if (~dead).any():
        d = np.abs(got_l[~dead].astype(np.float64) - want_l[~dead])
        assert d.max() <= TOL_LSE, f"{name}: lse {d.max():.3e}"
    p.softmax_lse = want_l.reshape(p.lse_shape())
    e = oracle.l1norm(p)
    o = run_main(smla, p, p.softmax_lse)
    err = np.abs(o.astype(np.float64) - e.astype(np.float64))
    assert err.max() <= TOL, f"{name}: max |gpu - oracle| = {err.max():.3e}"
    sums = o.astype(np.float64).sum(axis=1)
    live = nused > 0
    assert np.all(np.abs(sums[live] - 1.0) <= ROWSUM_TOL), f"{name}: row sums"
    assert not o[~live].any(), f"{name}: rows without a used entry must be zero"
    # where the oracle has a zero the GPU has a zero (entries not used)
    assert not o[e == 0].any(), f"{name}: support"


TINY = C.next3_cases()


@pytest.mark.parametrize("case", range(len(TINY)), ids=[n for n, _ in TINY])
def test_next3_tiny(smla, case):
    name, p = TINY[case]
    p = C.clone(p)
    say(f"[next3 tiny] {name} layout={p.layout} R={p.rows} W={p.out_width} kwide={p.kwide}")
    check(name, smla, p)


def medium_cases():
    cs = []
    # pipelined kernel: K-wide sparse rows (in LDS), seqused on 128 heads
    cs.append(("kw_g128_k1000", C.as_kwide(C.gen("tiny", heads_q=128, batch=1, seqlen_q=64,
                                                  seqlen_k=3000, topk=1000, mask_mode=3,
                                                  seed=71))))
    cs.append(("su_g128_causal", C.with_seqused(
        C.gen("tiny", heads_q=128, batch=2, seqlen_q=40, seqlen_k=3000, topk=700, mask_mode=3,
              seed=72), seqused_q=(30, 40), seqused_k=(1500, 2999))))
    # general kernel (64 heads), TND, both features
    cs.append(("kw_su_tnd_g64", C.as_kwide(C.with_seqused(
        C.gen("tnd_varlen", heads_q=64, topk=200, seqlens_q=(40, 30), seqlens_k=(600, 900),
              seed=73), seqused_q=(30, 30), seqused_k=(500, 100)))))
    # dense TND K-wide: rows of max_seqlen_k in LDS, and wider than LDS holds
    cs.append(("kw_dense_tnd_g128", C.as_kwide(C.gen(
        "tnd_varlen", heads_q=128, topk=0, seqlens_q=(30, 20), seqlens_k=(1000, 2500),
        seed=74))))
    cs.append(("kw_dense_tnd_g100_w5000", C.as_kwide(C.with_seqused(C.gen(
        "tnd_varlen", heads_q=100, topk=0, seqlens_q=(12, 20), seqlens_k=(5000, 300),
        seed=75), seqused_k=(4500, 300)))))
    # general kernel with more than 2048 entries (values stored directly)
    cs.append(("kw_g32_k3000_mask0", C.as_kwide(C.gen(
        "tiny", heads_q=32, batch=1, seqlen_q=20, seqlen_k=4000, topk=3000, mask_mode=0,
        seed=76))))
    return cs


MEDIUM = medium_cases()


@pytest.mark.parametrize("case", range(len(MEDIUM)), ids=[n for n, _ in MEDIUM])
def test_next3_medium(smla, case):
    name, p = MEDIUM[case]
    p = C.clone(p)
    say(f"[next3 medium] {name} layout={p.layout} R={p.rows} W={p.out_width} G={p.groups} "
        f"K={p.topk} kwide={p.kwide}")
    check(name, smla, p)
