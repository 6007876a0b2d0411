"""Pins of the CPU oracle: checks against things other than the oracle itself.

Every function takes an oracle handle (``oracle.COracle``) so that the same
checks can be run against deliberately broken builds (see
``test_oracle_mutants.py``). Each raises AssertionError on a mismatch.

What fixes each expected value:

* ``pin_brute``          a second, dense formulation (``oracle.brute``).
* ``pin_rowsum``         softmax rows sum to one, so their head mean does too.
* ``pin_support``        non-zeros only at selected, in-range, visible keys;
                         visibility from torch's lower-right causal bias.
* ``pin_torch_softmax``  torch.softmax over the selected keys' scores
                         (scores from torch matmul), averaged over heads.
* ``pin_sdpa_full``      selecting every key reduces the operation to the
                         head mean of attention weights: torch
                         scaled_dot_product_attention with V = identity and
                         the lower-right causal bias mapped to compressed keys.
* ``pin_q_zero``         q = 0 gives 1/|T| on the used keys.
* ``pin_arbitrary_lse``  with an lse shifted by d_g the row sum is the head
                         mean of exp(-d_g).
* ``pin_permutation``    entry order and a joint head permutation do not
                         change the result.
* ``pin_hand``           hand-derived closed forms (tests/golden).

seqused_q / seqused_k and the K-wide output (readings of the pages, which
give no example of either; their parity is unpinned by the pages):

* ``pin_next3_brute``        the dense formulation on seqused / K-wide cases.
* ``pin_seqused_identity``   counts equal to the layout's lengths change
                             nothing, bit for bit.
* ``pin_seqused_k_padding``  a key past seqused_k acts as an index of -1.
* ``pin_seqused_q_rows``     rows past seqused_q are 0 (lse -inf); the other
                             rows are unchanged, bit for bit.
* ``pin_kwide_gather``       the K-wide row is the scatter row read at each
                             used entry's key column, 0 elsewhere.
"""

from __future__ import annotations

import numpy as np
import torch
from torch.nn.attention.bias import causal_lower_right

from oracle import brute
from tests import cases as C


# ----------------------------------------------------------------------------
# independent helpers (library definitions, not the oracle's code)

def library_visibility(s1, s2, r, res, mask_mode):
    """(s1, s2) bool: compressed key j visible to query i.

    torch's lower-right causal bias over the original key positions
    (s2*r + res of them); a compressed key is visible when the last original
    position it covers is.
    """
    if mask_mode == 0:
        return np.ones((s1, s2), dtype=bool)
    L = s2 * r + res
    clr = causal_lower_right(s1, L)._materialize(torch.device("cpu")).numpy()
    last = (np.arange(s2) + 1) * r - 1
    return clr[:, last]


def entry_counts(p):
    """Per row: how many leading entries are looked at (topk_length clamped
    to [0, K]; without it K, or under mask 3 min(K, keys visible to the row))."""
    R, K = p.rows, p.topk
    tl = None if p.topk_length is None else p.topk_length.reshape(R)
    n = np.zeros(R, dtype=np.int64)
    for (b, q0, q1, k0, k1) in C.seq_bounds(p):
        res = 0 if p.cmp_residual_k is None else int(p.cmp_residual_k[b])
        vis = library_visibility(q1 - q0, k1 - k0, p.cmp_ratio, res, p.mask_mode)
        for r in range(q0, q1):
            if p.sparse_indices is None:  # dense: every key of the sequence
                n[r] = k1 - k0
            elif tl is not None:
                n[r] = min(max(int(tl[r]), 0), K)
            else:
                n[r] = K if p.mask_mode == 0 else min(K, int(vis[r - q0].sum()))
    return n


def used_entries(p):
    """Per row: (first k row, first output column, local key ids of the used
    entries in entry order)."""
    R, K = p.rows, p.topk
    dense = p.sparse_indices is None
    idx = None if dense else p.sparse_indices.reshape(R, K)
    tl = None if p.topk_length is None else p.topk_length.reshape(R)
    out = [None] * R
    for (b, q0, q1, k0, k1) in C.seq_bounds(p):
        s2 = k1 - k0
        res = 0 if p.cmp_residual_k is None else int(p.cmp_residual_k[b])
        vis = library_visibility(q1 - q0, s2, p.cmp_ratio, res, p.mask_mode)
        for r in range(q0, q1):
            if dense:  # every key of the sequence, in order
                out[r] = (k0, C.out_col0(p, b), [j for j in range(s2) if vis[r - q0, j]])
                continue
            if tl is not None:
                n = min(max(int(tl[r]), 0), K)
            else:  # mask 3: no more entries than visible keys
                n = K if p.mask_mode == 0 else min(K, int(vis[r - q0].sum()))
            js = []
            for t in range(n):
                j = int(idx[r, t])
                if 0 <= j < s2 and vis[r - q0, j]:
                    js.append(j)
            out[r] = (k0, C.out_col0(p, b), js)
    return out


def _q_k(p):
    R, G, D = p.rows, p.groups, p.head_dim
    return (p.q.reshape(R, G, D).double(), p.k.reshape(-1, D).double())


def _scale32(p):
    return float(np.float32(p.softmax_scale))


# ----------------------------------------------------------------------------
# pins

def pin_brute(orc, problems):
    for name, p in problems:
        p = C.clone(p)
        l32, _ = orc.lse(p)
        lb = brute.lse(p)
        fin = np.isfinite(lb)
        assert np.array_equal(fin, np.isfinite(l32)), name
        np.testing.assert_allclose(l32[fin], lb[fin], rtol=2e-7, atol=1e-7, err_msg=name)
        p.softmax_lse = l32.reshape(p.lse_shape())
        o = orc.l1norm(p)
        ob = brute.l1norm(p, p.softmax_lse)
        np.testing.assert_allclose(o, ob, rtol=2e-7, atol=1e-12, err_msg=name)


def pin_rowsum(orc, problems):
    for name, p in problems:
        p = C.clone(p)
        orc.fill_lse(p)
        o = orc.l1norm(p).astype(np.float64)
        used = used_entries(p)
        for r, (k0, c0, js) in enumerate(used):
            if js:
                assert abs(o[r].sum() - 1.0) <= 2e-6, (name, r, o[r].sum())
            else:
                assert not o[r].any(), (name, r)


def pin_support(orc, problems):
    for name, p in problems:
        p = C.clone(p)
        orc.fill_lse(p)
        o = orc.l1norm(p)
        used = used_entries(p)
        for r, (k0, c0, js) in enumerate(used):
            allowed = np.zeros(p.out_width, dtype=bool)
            allowed[[c0 + j for j in js]] = True
            assert not o[r][~allowed].any(), (name, r)
            assert (o[r][allowed] > 0).all(), (name, r)
            assert (o[r] <= 1.0).all(), (name, r)


def expected_by_torch_softmax(p):
    """(R, W) float64: head mean of torch.softmax over the used keys."""
    qd, kd = _q_k(p)
    sc = _scale32(p)
    out = np.zeros((p.rows, p.out_width))
    for r, (k0, c0, js) in enumerate(used_entries(p)):
        if not js:
            continue
        J = torch.tensor(js, dtype=torch.long)
        s = (qd[r] @ kd[k0 + J].T) * sc                 # (G, |J|)
        w = torch.softmax(s, dim=-1).mean(dim=0).numpy()
        np.add.at(out[r], c0 + np.asarray(js), w)
    return out


def pin_torch_softmax(orc, problems):
    for name, p in problems:
        p = C.clone(p)
        orc.fill_lse(p)
        o = orc.l1norm(p)
        e = expected_by_torch_softmax(p)
        np.testing.assert_allclose(o, e, rtol=3e-6, atol=1e-9, err_msg=name)


def pin_sdpa_full(orc, problems):
    for name, p in problems:
        f = C.full_selection(p)
        orc.fill_lse(f)
        o = orc.l1norm(f)
        qd, kd = _q_k(f)
        sc = _scale32(f)
        for (b, q0, q1, k0, k1) in C.seq_bounds(f):
            s1, s2 = q1 - q0, k1 - k0
            if s1 == 0 or s2 == 0:
                continue
            res = 0 if f.cmp_residual_k is None else int(f.cmp_residual_k[b])
            vis = torch.from_numpy(library_visibility(s1, s2, f.cmp_ratio, res,
                                                      f.mask_mode))
            qq = qd[q0:q1].permute(1, 0, 2).unsqueeze(0)             # (1, G, s1, D)
            kk = kd[k0:k1].expand(f.groups, s2, -1).unsqueeze(0)      # (1, G, s2, D)
            vv = torch.eye(s2, dtype=torch.float64).expand(1, f.groups, s2, s2)
            w = torch.nn.functional.scaled_dot_product_attention(
                qq, kk, vv, attn_mask=vis, scale=sc)                  # (1, G, s1, s2)
            w = w[0].mean(dim=0).numpy()                              # (s1, s2)
            live = vis.any(dim=1).numpy()
            c0 = C.out_col0(f, b)
            np.testing.assert_allclose(o[q0:q1][live, c0:c0 + s2], w[live], rtol=3e-6,
                                       atol=1e-9, err_msg=name)
            assert not o[q0:q1][~live].any(), name


def pin_q_zero(orc, problems):
    for name, p in problems:
        z = C.clone(p)
        z.q = torch.zeros_like(z.q)
        orc.fill_lse(z)
        o = orc.l1norm(z)
        for r, (k0, c0, js) in enumerate(used_entries(z)):
            e = np.zeros(z.out_width)
            if js:
                np.add.at(e, c0 + np.asarray(js), 1.0 / len(js))
            np.testing.assert_allclose(o[r], e, rtol=2e-7, atol=1e-12,
                                       err_msg=f"{name} row {r}")


def pin_arbitrary_lse(orc, problems):
    for i, (name, p) in enumerate(problems):
        a = C.clone(p)
        l32, _ = orc.lse(a)
        rng = np.random.Generator(np.random.PCG64(100 + i))
        d = rng.uniform(-1.0, 1.0, size=l32.shape).astype(np.float32)
        shifted = (l32 + d).astype(np.float32)
        o = orc.l1norm(a, softmax_lse=shifted.reshape(a.lse_shape())).astype(np.float64)
        # exp(lse_true - shifted) with lse_true ~ l32 within half an fp32 ulp
        with np.errstate(invalid="ignore"):
            expect = np.exp(l32.astype(np.float64) - shifted.astype(np.float64)).mean(axis=1)
        for r, (k0, c0, js) in enumerate(used_entries(a)):
            if js:
                assert abs(o[r].sum() - expect[r]) <= 4e-6 * expect[r] + 1e-9, (name, r)


def pin_permutation(orc, problems):
    for i, (name, p) in enumerate(problems):
        a = C.clone(p)
        orc.fill_lse(a)
        o = orc.l1norm(a)
        rng = np.random.Generator(np.random.PCG64(200 + i))
        # entry order within each row's first n entries (a dense problem has
        # no index list to permute)
        if a.sparse_indices is not None:
            b = C.clone(a)
            R, K = b.rows, b.topk
            idx = b.sparse_indices.reshape(R, K)
            for r, n in enumerate(entry_counts(b)):
                idx[r, :n] = idx[r, :n][rng.permutation(n)]
            ob = orc.l1norm(b)
            np.testing.assert_array_equal(o, ob, err_msg=name)
        # joint head permutation of q and lse
        c = C.clone(a)
        perm = torch.from_numpy(rng.permutation(c.groups))
        qf = c.q.reshape(c.rows, c.groups, c.head_dim)[:, perm]
        c.q = qf.reshape(c.q.shape).contiguous()
        lf = c.softmax_lse.reshape(c.rows, c.groups)[:, perm.numpy()]
        c.softmax_lse = np.ascontiguousarray(lf).reshape(c.lse_shape())
        oc = orc.l1norm(c)
        np.testing.assert_allclose(o, oc, rtol=1e-6, atol=1e-12, err_msg=name)


def pin_hand(orc):
    for name, p, exp_lse, exp_out in C.load_hand_examples():
        l32, _ = orc.lse(p)
        np.testing.assert_allclose(l32, exp_lse, rtol=1e-7, err_msg=name)
        p.softmax_lse = l32.reshape(p.lse_shape())
        o = orc.l1norm(p)
        np.testing.assert_allclose(o, exp_out, rtol=1e-6, atol=1e-12, err_msg=name)


# ----------------------------------------------------------------------------
# seqused_q / seqused_k and the K-wide output

def _lengths(p):
    b = C.seq_bounds(p)
    return [q1 - q0 for (_, q0, q1, _, _) in b], [k1 - k0 for (_, _, _, k0, k1) in b]


def _same_bits(a, b):
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def pin_next3_brute(orc, problems):
    pin_brute(orc, C.next3_cases())


def pin_seqused_identity(orc, problems):
    for name, p in problems:
        s1s, s2s = _lengths(p)
        c = C.with_seqused(p, s1s, s2s)
        lp, _ = orc.lse(p)
        lc, _ = orc.lse(c)
        assert _same_bits(lp, lc), name
        p = C.clone(p)
        p.softmax_lse = lp.reshape(p.lse_shape())
        c.softmax_lse = p.softmax_lse
        assert _same_bits(orc.l1norm(p), orc.l1norm(c)), name


def pin_seqused_k_padding(orc, problems):
    for name, p in problems:
        # the entry count must not depend on the keys (mask 3 without
        # topk_length caps it by the keys a row sees)
        if p.sparse_indices is None or (p.topk_length is None and p.mask_mode == 3):
            continue
        _, s2s = _lengths(p)
        su_k = [max(s2 - 2, 0) for s2 in s2s]
        c = C.with_seqused(p, None, su_k)
        d = C.clone(p)
        idx = d.sparse_indices.reshape(d.rows, d.topk)
        for (b, q0, q1, _, _) in C.seq_bounds(d):
            blk = idx[q0:q1]
            blk[blk >= su_k[b]] = -1
        lc, _ = orc.lse(c)
        ld, _ = orc.lse(d)
        assert _same_bits(lc, ld), name
        c.softmax_lse = lc.reshape(c.lse_shape())
        d.softmax_lse = c.softmax_lse
        assert _same_bits(orc.l1norm(c), orc.l1norm(d)), name


def pin_seqused_q_rows(orc, problems):
    for name, p in problems:
        s1s, _ = _lengths(p)
        su_q = [s1 // 2 for s1 in s1s]
        c = C.with_seqused(p, su_q, None)
        lp, _ = orc.lse(p)
        lc, _ = orc.lse(c)
        p = C.clone(p)
        p.softmax_lse = lp.reshape(p.lse_shape())
        c.softmax_lse = p.softmax_lse
        op, oc = orc.l1norm(p), orc.l1norm(c)
        for (b, q0, q1, _, _) in C.seq_bounds(p):
            live = slice(q0, q0 + su_q[b])
            dead = slice(q0 + su_q[b], q1)
            assert np.isneginf(lc[dead]).all() and not oc[dead].any(), name
            assert _same_bits(lc[live], lp[live]) and _same_bits(oc[live], op[live]), name


def pin_kwide_gather(orc, problems):
    for name, p in problems:
        p = C.clone(p)
        orc.fill_lse(p)
        o = orc.l1norm(p)
        c = C.as_kwide(p)
        ok = orc.l1norm(c)
        want = np.zeros((p.rows, c.out_width))
        R, K = p.rows, p.topk
        idx = None if p.sparse_indices is None else p.sparse_indices.reshape(R, K)
        tl = None if p.topk_length is None else p.topk_length.reshape(R)
        for (b, q0, q1, k0, k1) in C.seq_bounds(p):
            s2 = k1 - k0
            c0 = C.out_col0(p, b)
            res = 0 if p.cmp_residual_k is None else int(p.cmp_residual_k[b])
            vis = library_visibility(q1 - q0, s2, p.cmp_ratio, res, p.mask_mode)
            for r in range(q0, q1):
                if idx is None:  # dense: entry t is key t
                    want[r, :s2] = o[r, c0:c0 + s2]
                    continue
                if tl is not None:
                    n = min(max(int(tl[r]), 0), K)
                else:
                    n = K if p.mask_mode == 0 else min(K, int(vis[r - q0].sum()))
                js = [int(idx[r, t]) for t in range(n)]
                for t, j in enumerate(js):
                    if 0 <= j < s2 and vis[r - q0, j] and js.count(j) == 1:
                        want[r, t] = o[r, c0 + j]
        assert _same_bits(ok.astype(np.float32), want.astype(np.float32)), name


ALL_PINS = [pin_brute, pin_rowsum, pin_support, pin_torch_softmax, pin_sdpa_full,
            pin_q_zero, pin_arbitrary_lse, pin_permutation, pin_next3_brute,
            pin_seqused_identity, pin_seqused_k_padding, pin_seqused_q_rows,
            pin_kwide_gather]
