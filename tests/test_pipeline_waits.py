"""Host-side model of the pipelined kernel's vector-memory wait counts.

Each tile barrier of smla_wide_kernel waits with vmcnt(later): at most
`later` of the wave's own vector-memory instructions may still be in flight.
Vector memory completes in issue order, so the wait covers every instruction
issued more than `later` instructions before it. This test replays one
wave's issue order over rows of random tile counts, in the kernel's order:

  * first row: its index list (8 loads), Q (32), lse (1), the zero-fill of
    its output, a wait for everything, then the gather of tile 0 (16);
  * tile t: barrier; the gather of tile t+1 (16 loads, into a dummy row
    when there is no tile t+1); one value store (always issued: lanes with
    nothing to store point past the row);
  * row end: the value stores of the last two tiles, the zero-fill of the
    next row's output, its index list (8), Q (32) and lse (1), a wait for
    everything, then the gather of its tile 0.

It checks that the kernel's count `later` covers, at every barrier, the
gather of the tile and the zero-fill of the row, that the index list of a
row has landed before its first tile reads it, and that every value the
count takes has a case in the kernel's wait switch (anything else would fall
back to waiting for everything: correct but slow).
"""

import os
import random
import re

KERNEL = os.path.join(os.path.dirname(__file__), os.pardir, "sparse_mla_attention_02_amd",
                      "csrc", "smla_kernels.hip")
ROWS_PER_WAVE = 16   # gathered rows per wave and tile
IDX_OPS = 8          # loads of one index list per wave


def switch_values():
    src = open(KERNEL).read()
    body = src[src.index("void barrier_after_vmcnt(int n)"):]
    body = body[:body.index("asm volatile")]
    return {int(v) for v in re.findall(r"case (\d+): waitcnt_vm_lgkm0", body)}


def later_of(t, nt):
    """The kernel's count after tile t (smla_wide_kernel, tile loop): the
    value store of tile t."""
    return 1


def replay(rows, switch, rng, formula=None):
    formula = formula or later_of
    stream, done = [], 0

    def issue(tag, n=1):
        stream.extend([tag] * n)

    def wait(n):
        nonlocal done
        done = max(done, len(stream) - n)

    def landed(tag):
        return all(i < done for i, x in enumerate(stream) if x == tag)

    issue(("index list", 0), IDX_OPS)
    issue(("q", 0), 32)
    issue(("lse", 0))
    issue(("zero fill", 0), rng.randint(0, 12))
    wait(0)
    if rows[0] > 0:
        issue(("gather", 0, 0), ROWS_PER_WAVE)
    for r, nt in enumerate(rows):
        more = r + 1 < len(rows)
        assert landed(("index list", r)) and landed(("zero fill", r)), (rows, r)
        later = 0
        for t in range(nt):
            wait(later if later in switch else 0)
            assert landed(("gather", r, t)) and landed(("zero fill", r)), (rows, r, t)
            issue(("gather", r, t + 1) if t + 1 < nt else ("dummy", r), ROWS_PER_WAVE)
            issue(("store", r))
            later = formula(t, nt)
        issue(("store", r), min(nt, 2))
        if more:
            issue(("zero fill", r + 1), rng.randint(0, 12))
        issue(("index list", r + 1), IDX_OPS)
        if more:
            issue(("q", r + 1), 32)
            issue(("lse", r + 1))
            wait(0)
            if rows[r + 1] > 0:
                issue(("gather", r + 1, 0), ROWS_PER_WAVE)


def test_switch_has_every_count_the_formula_produces():
    switch = switch_values()
    produced = set()
    for nt in range(0, 70):
        for t in range(nt):
            produced.add(later_of(t, nt))
    assert produced - {0} <= switch, sorted(produced - switch)


def test_waits_cover_each_tiles_loads():
    switch = switch_values()
    rng = random.Random(7)
    for _ in range(3000):
        rows = [rng.choice([0, 1, 2, 3, 4, 5, 6, 9, 17, 19, 32]) for _ in range(rng.randint(1, 5))]
        replay(rows, switch, rng)


def test_model_catches_a_too_lenient_wait():
    # a planted mistake (a wait that lets the last 16 operations stay in
    # flight: the gather of the tile) must be caught by the replay
    def wrong(t, nt):
        return 17
    rng = random.Random(3)
    caught = False
    for _ in range(200):
        try:
            replay([rng.choice([5, 9, 17, 32]), 4], set(range(64)), rng, formula=wrong)
        except AssertionError:
            caught = True
            break
    assert caught
