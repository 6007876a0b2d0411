"""Host-side model of the pipelined kernel's vector-memory wait counts.

Each tile barrier of smla_pipe_kernel waits with vmcnt(later): at most
`later` of the wave's own vector-memory instructions may still be in flight.
Vector memory completes in issue order, so the wait covers every instruction
issued more than `later` instructions before it. This test replays one
wave's issue order over rows of random tile counts, in the kernel's order:

  * row start (end of the previous row): gathers of tiles 0..2 (8 loads each
    while the tile exists), index rows of tiles 3..5 (1 each);
  * tile t: barrier; index row of tile t+6 (1); gather of tile t+3 (8, while
    it exists); after tile pf = (ntiles > 3 ? 2 : ntiles-1) the next row's
    indices of tiles 0..2 (3);
  * row end: stores and loads that the next row's tile-0 wait (vmcnt(0))
    covers.

It checks that the kernel's formula for `later` covers, at every barrier,
the gather of the tile and the index row the tile reads, and that every
value the formula produces has a case in the kernel's wait switch (anything
else would fall back to waiting for everything: correct but slow).
"""

import os
import random
import re

KERNEL = os.path.join(os.path.dirname(__file__), os.pardir, "sparse_mla_attention_02_amd",
                      "csrc", "smla_kernels.hip")
PREFETCH = 3


def switch_values():
    src = open(KERNEL).read()
    body = src[src.index("void barrier_after_vmcnt(int n)"):]
    body = body[:body.index("asm volatile")]
    return {int(v) for v in re.findall(r"case (\d+): waitcnt_vm_lgkm0", body)}


def later_of(tile, nt, pf):
    """The kernel's formula (smla_pipe_kernel, body)."""
    extra = lambda u: PREFETCH if u == pf else 0
    if tile == 0:
        return 0
    if tile < 3:
        return 63
    later = (extra(tile - 3) + 2 + 8 * (tile + 1 < nt) + 8 * (tile + 2 < nt) +
             extra(tile - 2) + extra(tile - 1))
    return min(later, 63)


def replay(rows, switch, rng):
    stream, done = [], 0

    def issue(tag, n=1):
        stream.extend([tag] * n)

    def wait(n):
        nonlocal done
        done = max(done, len(stream) - n)

    def start_row(r, nt):
        for k in range(min(nt, 3)):
            issue(("gather", r, k), 8)
        for k in (3, 4, 5):
            issue(("index", r, k))

    issue(("indices", 0), PREFETCH)
    start_row(0, rows[0])
    for r, nt in enumerate(rows):
        pf = 2 if nt > 3 else nt - 1
        if nt == 0:
            issue(("indices", r + 1), PREFETCH)
        for t in range(nt):
            later = later_of(t, nt, pf)
            wait(later if later in switch else 0)
            need = {("gather", r, t), ("index", r, t + 3)}
            for i, tag in enumerate(stream):
                assert not (tag in need and i >= done), (rows, r, t, tag)
            issue(("index", r, t + 6))
            if t + 3 < nt:
                issue(("gather", r, t + 3), 8)
            if t == pf:
                issue(("indices", r + 1), PREFETCH)
        issue(("row end", r), rng.randint(0, 40))
        if r + 1 < len(rows):
            start_row(r + 1, rows[r + 1])
        issue(("stores", r), rng.randint(0, 12))


def test_switch_has_every_count_the_formula_produces():
    switch = switch_values()
    produced = set()
    for nt in range(0, 70):
        pf = 2 if nt > 3 else nt - 1
        for t in range(nt):
            produced.add(later_of(t, nt, pf))
    assert produced - {0} <= switch, sorted(produced - switch)


def test_waits_cover_each_tiles_loads():
    switch = switch_values()
    rng = random.Random(7)
    for _ in range(3000):
        rows = [rng.choice([0, 1, 2, 3, 4, 5, 6, 7, 9, 17, 64])
                for _ in range(rng.randint(1, 5))]
        replay(rows, switch, rng)


def test_model_catches_a_too_lenient_wait():
    # a planted mistake in the formula (one load too few counted as issued
    # after the gather) must be caught by the replay
    global later_of
    good = later_of
    try:
        later_of = lambda t, nt, pf: good(t, nt, pf) + (1 if t >= 3 else 0)
        switch = set(range(64))
        rng = random.Random(3)
        caught = False
        for _ in range(200):
            try:
                replay([rng.choice([8, 17, 64])], switch, rng)
            except AssertionError:
                caught = True
                break
        assert caught
    finally:
        later_of = good
