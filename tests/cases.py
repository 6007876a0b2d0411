"""Small problem builders and edge-case injections shared by the tests.

Nothing here computes the operation: these helpers only build inputs (via
``workloads``) and reshape them into edge cases.
"""

from __future__ import annotations

import copy
import json
import math
import os

import numpy as np
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gen(name="tiny", **kw):
    return workloads.generate(name, **kw)


def seq_bounds(p):
    """[(b, q_lo, q_hi, k_lo, k_hi)] per batch / sequence (rows of q and k)."""
    out = []
    if p.layout == "BSND":
        for b in range(p.batch):
            out.append((b, b * p.seqlen_q, (b + 1) * p.seqlen_q,
                        b * p.seqlen_k, (b + 1) * p.seqlen_k))
    else:
        cq, ck = p.cu_seqlens_q, p.cu_seqlens_k
        for b in range(p.batch):
            out.append((b, int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])))
    return out


def out_col0(p, b):
    """First output column of batch / sequence b (0 for BSND, cu_k[b] for TND)."""
    return 0 if p.layout == "BSND" else int(p.cu_seqlens_k[b])


def clone(p):
    c = copy.copy(p)
    c.q = p.q.clone()
    c.k = p.k.clone()
    c.sparse_indices = None if p.sparse_indices is None else p.sparse_indices.copy()
    c.topk_length = None if p.topk_length is None else p.topk_length.copy()
    c.softmax_lse = None if p.softmax_lse is None else p.softmax_lse.copy()
    return c


def inject_edges(p, seed=0, invisible=True, out_of_range=True, shorten=True):
    """Return a copy of p with planted edge entries.

    * invisible: where a row has a -1 pad inside topk_length's reach, or
      where the row is shortened, put a key beyond the row's causal prefix;
    * out_of_range: an index >= S2_b or a negative non -1 index;
    * shorten: cut topk_length of some rows by 2 (entries past it are left
      in place and must be ignored);
    * shadow (no topk_length, mask 3): blank the first entry of a row that
      sees fewer than K keys and move its key just past the visible count,
      where the entry count min(K, visible keys) leaves it unused.
    """
    c = clone(p)
    rng = np.random.Generator(np.random.PCG64(seed))
    R, K = c.rows, c.topk
    idx = c.sparse_indices.reshape(R, K)
    tlen = None if c.topk_length is None else c.topk_length.reshape(R)
    for (b, q0, q1, k0, k1) in seq_bounds(c):
        s2 = k1 - k0
        res = 0 if c.cmp_residual_k is None else int(c.cmp_residual_k[b])
        for r in range(q0, q1):
            u = rng.random()
            n = int(tlen[r]) if tlen is not None else K
            pads = np.nonzero(idx[r] < 0)[0]
            # first key past the row's causal prefix (the recipe's rule)
            L = workloads.visible_prefix(r - q0, q1 - q0, s2, c.mask_mode, c.cmp_ratio, res)
            if invisible and c.mask_mode == 3 and u < 0.3 and len(pads) and L < s2:
                # put an invisible key into the first pad and extend
                # topk_length over it
                t = pads[0]
                idx[r, t] = L
                if tlen is not None:
                    tlen[r] = max(n, t + 1)
            elif out_of_range and 0.3 <= u < 0.5 and len(pads):
                t = pads[0]
                idx[r, t] = s2 + int(rng.integers(0, 3)) if rng.random() < 0.5 else -7
                if tlen is not None:
                    tlen[r] = max(n, t + 1)
            elif shorten and 0.5 <= u < 0.7 and tlen is not None and n >= 2:
                tlen[r] = n - 2
            elif (0.7 <= u < 0.9 and tlen is None and c.mask_mode == 3 and 0 < L < K
                  and idx[r, 0] >= 0):
                idx[r, L] = idx[r, 0]
                idx[r, 0] = -1
    return c


def full_selection(p):
    """Copy of p whose every row lists every key of its sequence, in order
    (a dense problem is returned as it is: it already selects every key)."""
    c = clone(p)
    if c.sparse_indices is None:
        return c
    s2max = max(k1 - k0 for (_, _, _, k0, k1) in seq_bounds(c))
    R = c.rows
    idx = np.full((R, s2max), -1, dtype=np.int32)
    for (b, q0, q1, k0, k1) in seq_bounds(c):
        idx[q0:q1, :k1 - k0] = np.arange(k1 - k0, dtype=np.int32)[None, :]
    c.topk = s2max
    shp = c.sparse_indices.shape[:-1] + (s2max,)
    c.sparse_indices = idx.reshape(shp)
    c.topk_length = None
    return c


def tiny_cases():
    """Tiny problems covering every feature the oracle handles."""
    cs = []
    cs.append(("tiny", gen("tiny")))
    cs.append(("bsnd_causal_g3", gen("tiny", heads_q=3, batch=2, seqlen_q=5,
                                      seqlen_k=9, topk=6, mask_mode=3, seed=11)))
    cs.append(("s1_gt_s2_g1", gen("tiny", heads_q=1, batch=1, seqlen_q=9, seqlen_k=5,
                                   topk=4, mask_mode=3, seed=12)))
    cs.append(("cmp4_res_g16", gen("tiny", heads_q=16, batch=2, seqlen_q=12, seqlen_k=5,
                                    topk=4, mask_mode=3, cmp_ratio=4,
                                    cmp_residual=(3, 1), seed=13)))
    cs.append(("cmp128_boundary", gen("tiny", heads_q=2, batch=1, seqlen_q=130,
                                       seqlen_k=2, topk=2, mask_mode=3, cmp_ratio=128,
                                       cmp_residual=(3,), seed=14)))
    cs.append(("tnd3_causal_g4", gen("tnd_varlen", heads_q=4, topk=5,
                                      seqlens_q=(3, 1, 6), seqlens_k=(4, 7, 2),
                                      seed=15)))
    cs.append(("tnd2_mask0_g3", gen("tnd_varlen", heads_q=3, topk=4, mask_mode=0,
                                     seqlens_q=(2, 5), seqlens_k=(6, 3), seed=16)))
    cs.append(("tnd_cmp2", gen("tnd_varlen", heads_q=2, topk=3, cmp_ratio=2,
                                cmp_residual=(1, 0), seqlens_q=(7, 4), seqlens_k=(3, 5),
                                seed=17)))
    cs.append(("no_topk_length", gen("tiny", heads_q=4, seqlen_q=6, seqlen_k=8, topk=8,
                                      mask_mode=3, with_topk_length=False, seed=18)))
    cs.append(("fp16_sigma", gen("tiny", heads_q=5, dtype="fp16", sigma=0.5, seed=19)))
    cs.append(("uniform2", gen("tiny", heads_q=4, dist="uniform2", seed=20)))
    edged = [(n + "+edges", inject_edges(p, seed=i)) for i, (n, p) in enumerate(cs)]
    # the dense case (no sparse_indices: every key of the sequence)
    cs.append(("dense_bsnd_mask0", gen("tiny", heads_q=3, batch=2, seqlen_q=4, seqlen_k=7,
                                        topk=0, mask_mode=0, seed=21)))
    cs.append(("dense_bsnd_causal", gen("tiny", heads_q=4, batch=1, seqlen_q=9,
                                         seqlen_k=6, topk=0, mask_mode=3, seed=22)))
    cs.append(("dense_tnd_cmp4", gen("tnd_varlen", heads_q=2, topk=0, cmp_ratio=4,
                                      cmp_residual=(2, 0, 1), seqlens_q=(6, 1, 9),
                                      seqlens_k=(3, 2, 4), seed=23)))
    return cs + edged


def with_seqused(p, seqused_q=None, seqused_k=None):
    """Copy of p with per-batch seqused_q / seqused_k counts."""
    c = clone(p)
    c.seqused_q = None if seqused_q is None else np.asarray(seqused_q, dtype=np.int32)
    c.seqused_k = None if seqused_k is None else np.asarray(seqused_k, dtype=np.int32)
    return c


def as_kwide(p):
    """Copy of p asking for the K-wide output (entry t at column t)."""
    c = clone(p)
    c.kwide = True
    return c


def next3_cases():
    """Tiny problems for seqused_q / seqused_k and the K-wide output."""
    cs = []
    cs.append(("su_bsnd_causal", with_seqused(
        gen("tiny", heads_q=3, batch=2, seqlen_q=6, seqlen_k=9, topk=6, mask_mode=3,
            seed=31), seqused_q=(4, 6), seqused_k=(5, 9))))
    cs.append(("su_tnd_mask0", with_seqused(
        gen("tnd_varlen", heads_q=4, topk=5, mask_mode=0, seqlens_q=(4, 3),
            seqlens_k=(7, 5), seed=32), seqused_q=(2, 3), seqused_k=(4, 0))))
    cs.append(("su_no_topk_length", with_seqused(
        gen("tiny", heads_q=2, seqlen_q=6, seqlen_k=8, topk=8, mask_mode=3,
            with_topk_length=False, seed=33), seqused_k=(5,))))
    cs.append(("su_dense_tnd_cmp2", with_seqused(
        gen("tnd_varlen", heads_q=2, topk=0, cmp_ratio=2, cmp_residual=(1, 0),
            seqlens_q=(5, 3), seqlens_k=(4, 6), seed=34), seqused_q=(5, 1),
        seqused_k=(2, 6))))
    cs.append(("kw_bsnd_edges", as_kwide(inject_edges(
        gen("tiny", heads_q=4, batch=2, seqlen_q=5, seqlen_k=9, topk=6, mask_mode=3,
            seed=35), seed=5))))
    cs.append(("kw_tnd_edges", as_kwide(inject_edges(
        gen("tnd_varlen", heads_q=3, topk=5, seqlens_q=(3, 4), seqlens_k=(6, 8),
            seed=36), seed=6))))
    cs.append(("kw_dense_tnd", as_kwide(
        gen("tnd_varlen", heads_q=2, topk=0, seqlens_q=(3, 4), seqlens_k=(5, 2),
            seed=37))))
    cs.append(("kw_dense_bsnd_mask0", as_kwide(
        gen("tiny", heads_q=3, batch=1, seqlen_q=4, seqlen_k=6, topk=0, mask_mode=0,
            seed=38))))
    cs.append(("kw_su_tnd", as_kwide(with_seqused(
        gen("tnd_varlen", heads_q=5, topk=4, seqlens_q=(4, 5), seqlens_k=(6, 7),
            seed=39), seqused_q=(3, 5), seqused_k=(6, 3)))))
    return cs


def load_hand_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        doc = json.load(f)
    out = []
    for c in doc["cases"]:
        D, G, K = c["D"], c["N1"], c["topk"]
        q0 = np.asarray(c["q0"], dtype=np.float32)          # (R, G)
        k0 = np.asarray(c["k0"], dtype=np.float32)          # (rows of k,)
        R = q0.shape[0]
        q = torch.zeros(R, G, D)
        q[:, :, 0] = torch.from_numpy(q0)
        k = torch.zeros(len(k0), 1, D)
        k[:, 0, 0] = torch.from_numpy(k0)
        idx = np.asarray(c["sparse_indices"], dtype=np.int32)
        tl = np.asarray(c["topk_length"], dtype=np.int32)
        if c["layout"] == "BSND":
            B, S1, S2 = c["B"], c["S1"], c["S2"]
            p = workloads.Problem(
                name=c["name"], layout="BSND", batch=B, seqlen_q=S1, seqlen_k=S2,
                heads_q=G, heads_k=1, head_dim=D, topk=K, mask_mode=c["mask_mode"],
                cmp_ratio=c["cmp_ratio"], softmax_scale=c["softmax_scale"], dtype="bf16",
                q=q.reshape(B, S1, G, D).bfloat16(), k=k.reshape(B, S2, 1, D).bfloat16(),
                sparse_indices=idx.reshape(B, S1, 1, K), topk_length=tl.reshape(B, S1, 1),
                cu_seqlens_q=None, cu_seqlens_k=None, cmp_residual_k=None,
                max_seqlen_q=S1, max_seqlen_k=S2)
        else:
            cq = np.asarray(c["cu_seqlens_q"], dtype=np.int32)
            ck = np.asarray(c["cu_seqlens_k"], dtype=np.int32)
            p = workloads.Problem(
                name=c["name"], layout="TND", batch=len(cq) - 1, seqlen_q=int(cq[-1]),
                seqlen_k=int(ck[-1]), heads_q=G, heads_k=1, head_dim=D, topk=K,
                mask_mode=c["mask_mode"], cmp_ratio=c["cmp_ratio"],
                softmax_scale=c["softmax_scale"], dtype="bf16", q=q.bfloat16(),
                k=k.bfloat16(), sparse_indices=idx.reshape(R, 1, K),
                topk_length=tl.reshape(R, 1), cu_seqlens_q=cq, cu_seqlens_k=ck,
                cmp_residual_k=None, max_seqlen_q=int(np.diff(cq).max()),
                max_seqlen_k=int(np.diff(ck).max()))
        ns = {"E": math.e, "log": math.log}
        exp_out = np.array([[eval(x, ns) for x in row] for row in c["expected"]])
        exp_lse = np.array([[eval(x, ns) for x in row] for row in c["expected_lse"]])
        out.append((c["name"], p, exp_lse, exp_out))
    return out
