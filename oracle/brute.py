"""Dense brute-force formulation of the Softmax-L1Norm, for tiny inputs.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

This is a second, independent way of writing the three-stage formula of the
"SparseFlashMlaSoftmaxL1Norm" article (section 三阶段计算公式): instead of
walking the selected entries one by one, it builds the full score matrix of
every query against every key of its sequence with one matrix product, turns
the index list into a selection-count matrix, builds the right-down-causal
visibility matrix by broadcasting, and averages ``exp(s - lse)`` over the
heads under those masks. Everything is float64.

The readings it takes are the same as the C oracle's (local TND indices,
entries past ``topk_length`` / out of range / -1 ignored, compressed causal
rule, natural-base exp, repeated indices counted twice). Without
sparse_indices (the dense case, stage 1 selecting the whole K) the
selection-count matrix is all ones. seqused_q / seqused_k remove queries
and keys past their counts from the visibility matrix. The K-wide output
(entry t's value at column t) is built entry by entry from the per-key
values.
"""

from __future__ import annotations

import numpy as np


def _sequences(p):
    """Yield (b, query-row slice, key-row slice, first output column)."""
    if p.layout == "BSND":
        for b in range(p.batch):
            yield (b, slice(b * p.seqlen_q, (b + 1) * p.seqlen_q),
                   slice(b * p.seqlen_k, (b + 1) * p.seqlen_k), 0)
    else:
        cq, ck = p.cu_seqlens_q, p.cu_seqlens_k
        for b in range(p.batch):
            yield (b, slice(int(cq[b]), int(cq[b + 1])),
                   slice(int(ck[b]), int(ck[b + 1])), int(ck[b]))


def _pieces(p, b, qs, ks):
    """(scores (s1,G,s2), selection counts x visibility (s1,s2), visibility
    (s1,s2), entry counts n (s1,) or None, indices (s1,K) or None)."""
    R, G, D, K = p.rows, p.groups, p.head_dim, p.topk
    q = p.q.reshape(R, G, D)[qs].double().numpy()          # (s1, G, D)
    k = p.k.reshape(-1, D)[ks].double().numpy()             # (s2, D)
    s1, s2 = q.shape[0], k.shape[0]
    scale = float(np.float32(p.softmax_scale))
    S = scale * np.einsum("igd,jd->igj", q, k)               # (s1, G, s2)

    if p.mask_mode == 3:
        r = p.cmp_ratio
        res = 0 if p.cmp_residual_k is None else int(p.cmp_residual_k[b])
        qpos1 = np.arange(s1) + 1 + s2 * r + res - s1        # query original pos + 1
        kend = (np.arange(s2) + 1) * r                        # key block last pos + 1
        vis = kend[None, :] <= qpos1[:, None]
    else:
        vis = np.ones((s1, s2), dtype=bool)
    # queries / keys past seqused_q / seqused_k take no part
    qu = s1 if p.seqused_q is None else min(max(int(p.seqused_q[b]), 0), s1)
    ku = s2 if p.seqused_k is None else min(max(int(p.seqused_k[b]), 0), s2)
    vis = vis & (np.arange(s1)[:, None] < qu) & (np.arange(s2)[None, :] < ku)

    if p.sparse_indices is None:
        # dense: every key of the sequence is selected once
        return S, np.ones((s1, s2), dtype=np.float64) * vis, vis, None, None
    idx = p.sparse_indices.reshape(R, K)[qs].astype(np.int64)
    if p.topk_length is None:
        # selectBlockCount without topk_length: K, or (mask 3) no more than
        # the number of keys the row sees
        n = np.full(s1, K, dtype=np.int64)
        if p.mask_mode == 3:
            n = np.minimum(n, vis.sum(axis=1))
    else:
        n = np.clip(p.topk_length.reshape(R)[qs].astype(np.int64), 0, K)
    counts = np.zeros((s1, s2), dtype=np.float64)
    take = (np.arange(K)[None, :] < n[:, None]) & (idx >= 0) & (idx < s2)
    rr, tt = np.nonzero(take)
    np.add.at(counts, (rr, idx[rr, tt]), 1.0)
    return S, counts * vis, vis, n, idx


def lse(p):
    """(R, G) float64 log-sum-exp over the masked selected scores."""
    out = np.full((p.rows, p.groups), -np.inf)
    for b, qs, ks, _ in _sequences(p):
        S, M = _pieces(p, b, qs, ks)[:2]
        W = M[:, None, :]
        m = np.max(np.where(W > 0, S, -np.inf), axis=-1, keepdims=True)
        m_safe = np.where(np.isfinite(m), m, 0.0)
        tot = np.sum(np.where(W > 0, W * np.exp(S - m_safe), 0.0), axis=-1)
        with np.errstate(divide="ignore"):
            out[qs] = np.where(tot > 0, m_safe[..., 0] + np.log(tot), -np.inf)
    return out


def l1norm(p, softmax_lse):
    """(R, W) float64 output for all rows, given lse of shape (R, G)."""
    lse_rg = np.asarray(softmax_lse, dtype=np.float64).reshape(p.rows, p.groups)
    out = np.zeros((p.rows, p.out_width), dtype=np.float64)
    for b, qs, ks, col0 in _sequences(p):
        S, M, vis, n, idx = _pieces(p, b, qs, ks)
        s1, s2 = M.shape
        W = M[:, None, :]
        with np.errstate(over="ignore", invalid="ignore"):
            P = np.where(W > 0, W * np.exp(S - lse_rg[qs][:, :, None]), 0.0)
        if not p.kwide:
            out[qs, col0:col0 + s2] = P.mean(axis=1)
            continue
        # K-wide: the value of the key of each used entry, at the entry's column
        with np.errstate(over="ignore", invalid="ignore"):
            V = np.where(vis, np.exp(S - lse_rg[qs][:, :, None]).mean(axis=1), 0.0)
        blk = np.zeros((s1, p.out_width))
        if idx is None:  # dense: entry t is key t
            blk[:, :s2] = V
        else:
            K = idx.shape[1]
            inr = (idx >= 0) & (idx < s2)
            jj = np.where(inr, idx, 0)
            take = (np.arange(K)[None, :] < n[:, None]) & inr & \
                np.take_along_axis(vis, jj, axis=1)
            blk[:, :K] = np.where(take, np.take_along_axis(V, jj, axis=1), 0.0)
        out[qs] = blk
    return out
