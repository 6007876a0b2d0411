"""Every kernel variant at every tile-count boundary, through the C-ABI
binding, against the CPU oracle.

A row of n used entries runs ceil(n / T) key tiles (T = 64 keys for the
pipelined kernels, 32 for the general one): tiles with two more after them
take the steady path, the last two or three form their stream state at the
tile boundary, a tile's epilogue finishes two tiles later, and the row end
loads the next row's Q and lse as the tile loop ends. Here every row length
around a multiple of the tile appears, in a shuffled order, and the work is
split over a few workgroups (a caller's core budget), so that each workgroup
walks many rows and meets every transition between row lengths.

Cases, by the kernel variant they reach (the constraints section of the
article allows any B, S1, S2 and S1 != S2; the three-stage formula is the
same for every head count):

* 65..128 heads, output rows of at most 4096 columns: the pipelined kernel
  with the row assembled in LDS (sparse and dense);
* 65..128 heads, rows wider than 4096 columns: the pipelined kernel that
  zero-fills each row and stores values directly (double-buffered index
  lists; sparse, dense TND, K-wide dense);
* up to 64 heads (16, 33, 64), up to 2048 indices per row, and more than
  2048 (the variant without the LDS row);
* up to 16 heads, whose Q has a place of its own and whose key-tile stream
  runs on across rows (5 heads, sparse; 16 heads, dense causal rows).

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


def lengths(tile, top, extra=()):
    """Both sides of every multiple of `tile` up to `top`, plus 0, 1, 2."""
    return sorted({0, 1, 2} | {v for m in range(tile, top + 1, tile)
                               for v in (m - 1, m, m + 1) if v <= top} | set(extra))


@pytest.fixture(scope="module")
def smla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_attention_02_amd as m
    return m


def _t(a, dev="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def with_lengths(p, seed, lens=LENGTHS):
    """p with topk_length set to `lens`, repeated over the rows and shuffled."""
    p = C.clone(p)
    rng = np.random.Generator(np.random.PCG64(seed))
    tl = np.resize(np.array(lens, dtype=np.int32), p.rows)
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
    # rows wider than 4096 columns: zero-filled rows, values stored directly,
    # the next row's index list loaded into the other buffer
    cs.append(("bsnd_bf16_g128_w5000", with_lengths(
        C.gen("tiny", heads_q=128, batch=1, seqlen_q=2 * len(LENGTHS), seqlen_k=5000,
              topk=1024, mask_mode=0, seed=64), seed=3)))
    l2k = lengths(64, 2048)
    cs.append(("tnd_fp16_g100_w6000_k2048", with_lengths(
        C.gen("tnd_varlen", heads_q=100, topk=2048, mask_mode=0, seqlens_q=(70, 30, 50),
              seqlens_k=(2100, 2500, 1400), seed=65), seed=4, lens=l2k)))
    # dense TND rows of a 4700-column output: sequences of different causal
    # squares, one of them with no visible key for its first rows
    cs.append(("dense_tnd_g128_w4700", C.gen(
        "tnd_varlen", heads_q=128, topk=0, mask_mode=3, seqlens_q=(60, 40, 30),
        seqlens_k=(2000, 2650, 20), cmp_ratio=1, seed=66)))
    # K-wide dense rows of 5000 entries (entry t at column t)
    cs.append(("kw_dense_bsnd_g128_w5000", C.as_kwide(C.gen(
        "tiny", heads_q=128, batch=1, seqlen_q=60, seqlen_k=5000, topk=0, mask_mode=3,
        seed=73))))
    # up to 64 heads: 32-key tiles, rows of up to 2048 indices assembled in
    # LDS, longer rows stored directly
    l32 = lengths(32, 1024, extra=(1500, 2047, 2048))
    cs.append(("bsnd_bf16_g16_k2048", with_lengths(
        C.gen("tiny", heads_q=16, batch=2, seqlen_q=len(l32), seqlen_k=2100, topk=2048,
              mask_mode=0, seed=67), seed=5, lens=l32)))
    cs.append(("tnd_fp16_g33_k2048", with_lengths(
        C.gen("tnd_varlen", heads_q=33, topk=2048, mask_mode=0, seqlens_q=(len(l32), 80),
              seqlens_k=(2200, 3000), dtype="fp16", seed=68), seed=6, lens=l32)))
    cs.append(("bsnd_fp16_g64_k2048", with_lengths(
        C.gen("tiny", heads_q=64, batch=1, seqlen_q=len(l2k), seqlen_k=2048, topk=2048,
              mask_mode=0, dtype="fp16", seed=69), seed=7, lens=l2k)))
    l3k = lengths(32, 2600, extra=(2599, 2600)) [::3] + [2600, 2599, 0]
    cs.append(("bsnd_bf16_g64_k2600", with_lengths(
        C.gen("tiny", heads_q=64, batch=1, seqlen_q=len(l3k), seqlen_k=2700, topk=2600,
              mask_mode=0, seed=70), seed=8, lens=sorted(set(l3k)))))
    cs.append(("tnd_bf16_g16_k3000", with_lengths(
        C.gen("tnd_varlen", heads_q=16, topk=3000, mask_mode=0, seqlens_q=(90, 60),
              seqlens_k=(3100, 3500), seed=71), seed=9,
        lens=lengths(32, 3000)[::4] + [3000])))
    # up to 16 heads (Q in a place of its own, the key-tile stream running on
    # across rows, short rows counting extra tiles): fewer heads than a block
    # of 16, and dense causal rows of 1 .. 5 tiles
    cs.append(("bsnd_fp16_g5_k700", with_lengths(
        C.gen("tiny", heads_q=5, batch=2, seqlen_q=len(LENGTHS[:40]), seqlen_k=760,
              topk=700, mask_mode=0, dtype="fp16", seed=74), seed=11,
        lens=[v for v in LENGTHS if v <= 700])))
    cs.append(("dense_bsnd_g16_causal", C.gen("tiny", heads_q=16, batch=1, seqlen_q=300,
                                               seqlen_k=300, topk=0, mask_mode=3, seed=75)))
    cs.append(("bsnd_bf16_g128_k2600", with_lengths(
        C.gen("tiny", heads_q=128, batch=1, seqlen_q=80, seqlen_k=2700, topk=2600,
              mask_mode=0, seed=72), seed=10, lens=lengths(32, 2600)[::5] + [2600])))
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
          f"W={p.out_width} workgroups={int(md[4])}", flush=True)
    o = smla.smla_softmax_l1norm(
        p.q.cuda(), p.k.cuda(), _t(np.asarray(p.softmax_lse, dtype=np.float32)),
        sparse_indices=_t(p.sparse_indices), cu_seqlens_q=_t(p.cu_seqlens_q),
        cu_seqlens_k=_t(p.cu_seqlens_k), topk_length=_t(p.topk_length), metadata=md,
        softmax_scale=p.softmax_scale, max_seqlen_k=p.max_seqlen_k, cmp_ratio=p.cmp_ratio,
        mask_mode=p.mask_mode, layout_q=p.layout, layout_k=p.layout, kwide=p.kwide)
    torch.cuda.synchronize()
    o = o.reshape(p.rows, p.out_width).cpu().numpy()
    err = np.abs(o.astype(np.float64) - e.astype(np.float64))
    assert float(err.max()) <= TOL, f"{name}: max |gpu - oracle| = {float(err.max()):.3e}"
    sums = o.astype(np.float64).sum(axis=1)
    live = e.astype(np.float64).sum(axis=1) > 0
    assert np.all(np.abs(sums[live] - 1.0) <= ROWSUM_TOL), f"{name}: row sums"
    assert not o[~live].any(), f"{name}: rows without a used entry must be zero"
