"""The CPU oracle against its pins (no GPU).

Every function of the oracle (``oracle_lse``, ``oracle_l1norm`` and the dense
brute force) is pinned by at least one check that does not reuse its code;
see ``tests/pins.py`` for what fixes each expected value.
"""

import pytest

import oracle
from tests import cases as C
from tests import pins

CASES = C.tiny_cases()


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc, CASES)


def test_hand_examples(orc):
    pins.pin_hand(orc)


def test_sampled_rows_match_full(orc):
    """Row-subset calls give the same rows as a full call."""
    import numpy as np
    p = C.gen("tnd_varlen", heads_q=8, topk=6, seqlens_q=(5, 9, 3), seqlens_k=(6, 2, 11),
              seed=31)
    orc.fill_lse(p)
    full = orc.l1norm(p)
    rows = [12, 0, 16, 5, 5]
    part = orc.l1norm(p, rows=rows)
    np.testing.assert_array_equal(part, full[rows])
    l_full, n_full = orc.lse(p)
    l_part, n_part = orc.lse(p, rows=rows)
    np.testing.assert_array_equal(l_part, l_full[rows])
    np.testing.assert_array_equal(n_part, n_full[rows])


def test_generator_draws_visible_distinct(orc):
    """The input recipe only draws distinct, visible, in-range keys."""
    import numpy as np
    for name, p in CASES[:11]:
        used = pins.used_entries(p)
        R, K = p.rows, p.topk
        idx = p.sparse_indices.reshape(R, K)
        tl = p.topk_length.reshape(R) if p.topk_length is not None else None
        for r in range(R):
            row = idx[r]
            drawn = row[row >= 0]
            assert len(set(drawn.tolist())) == len(drawn), name
            assert len(used[r][2]) == len(drawn), (name, r)
            if tl is not None:
                assert tl[r] == len(drawn)
                assert (row[:tl[r]] >= 0).all() and (row[tl[r]:] == -1).all()
