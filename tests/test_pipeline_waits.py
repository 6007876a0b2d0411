"""Host-side model of the pipelined kernel's vector-memory wait counts.

smla_wide_kernel waits with vmcnt(n): at most n of the wave's own
vector-memory instructions may still be in flight. Vector memory completes
in issue order, so the wait covers every instruction issued more than n
instructions before it. This test replays one wave's issue order over rows
of random tile counts, in the kernel's order:

  * first row: its index list (8 loads), Q (32), lse (1), the zero-fill of
    its output, a wait for everything;
  * row start: the gather of tile 0 (16 loads) and of rows 0..6 of tile 1
    (7 loads, to a dummy row when there is no tile 1), then a wait that
    leaves the last 7 in flight, and the barrier;
  * tile t, steps 1..9: rows 7..15 of tile t+1 (stream A); step 24: a wait
    for everything and the barrier (after which the operands of tile t+1
    are read); steps 25..31: rows 0..6 of tile t+2 (stream B), then the
    value store of the step sequence;
  * before the last two or three tiles of a row (where the steady tiles
    end): an L2 prefetch of the next row's index list (1 load);
  * row end: as the tile loop ends, the rest of the next row's Q (32 in the
    model) and its lse (1); then the value stores of the last two tiles, the
    zero-fill of the next row's output, its index list (8), a wait for
    everything, then the next row's start.

With rows assembled in LDS (output rows of at most 4096 columns) the values
go to LDS instead: no store in the tile loop and no zero-fill; the row end
writes the whole row out before loading the next row's index list.

It checks that each wait covers the loads of the tile whose operands are read
after it, the zero-fill of the row before its first value store and the
index list before its first read, and that every count the kernel uses has a
case in the kernel's wait switch (anything else would fall back to waiting
for everything: correct but slow).
"""

import os
import random
import re

KERNEL = os.path.join(os.path.dirname(__file__), os.pardir, "sparse_mla_attention_02_amd",
                      "csrc", "smla_device.h")
IDX_OPS = 8          # loads of one index list per wave
ROW_START_LATER = 7  # tile 1's first rows, left in flight at a row start
BAR_STEP = 24


def switch_values():
    src = open(KERNEL).read()
    body = src[src.index("void barrier_after_vmcnt(int n)"):]
    body = body[:body.index("asm volatile")]
    return {int(v) for v in re.findall(r"case (\d+): waitcnt_vm_lgkm0", body)}


def replay(rows, switch, rng, row_start_later=ROW_START_LATER, bar_later=0, rowbuf=False):
    stream, done = [], 0

    def issue(tag, n=1):
        stream.extend([tag] * n)

    def wait(n):
        nonlocal done
        assert n == 0 or n in switch, n
        done = max(done, len(stream) - n)

    def landed(tag):
        return all(i < done for i, x in enumerate(stream) if x == tag)

    def gather(r, t, lo, hi, nt):
        issue(("gather", r, t) if t < nt else ("dummy", r), hi - lo)

    def row_start(r):
        nt = rows[r]
        if nt > 0:
            gather(r, 0, 0, 16, nt)
            gather(r, 1, 0, 7, nt)
        wait(row_start_later)
        assert landed(("gather", r, 0)), (rows, r)

    issue(("index list", 0), IDX_OPS)
    issue(("q", 0), 32)
    issue(("lse", 0))
    if not rowbuf:
        issue(("zero fill", 0), rng.randint(0, 12))
    wait(0)
    row_start(0)
    for r, nt in enumerate(rows):
        more = r + 1 < len(rows)
        assert landed(("index list", r)), (rows, r)
        assert rowbuf or landed(("zero fill", r)), (rows, r)
        # the steady pairs run while tile + 3 < nt; the rest form the tail
        tail = 0
        while tail + 3 < nt:
            tail += 2
        for t in range(nt):
            if t == tail and more:
                issue(("prefetch", r + 1))
            gather(r, t + 1, 7, 16, nt)                  # steps 1..9
            wait(bar_later)                              # step 24
            assert landed(("gather", r, t + 1)), (rows, r, t)
            gather(r, t + 2, 0, 7, nt)                   # steps 25..31
            if not rowbuf:
                issue(("store", r))                      # step 31
        if nt == 0 and more:
            issue(("prefetch", r + 1))
        if more:
            issue(("q", r + 1), 32)
            issue(("lse", r + 1))
        if rowbuf:
            issue(("row", r), rng.randint(1, 4))
        else:
            issue(("store", r), min(nt, 2))
            if more:
                issue(("zero fill", r + 1), rng.randint(0, 12))
        issue(("index list", r + 1), IDX_OPS)
        if more:
            wait(0)
            assert landed(("q", r + 1)) and landed(("lse", r + 1)), (rows, r)
            row_start(r + 1)


def test_switch_has_every_count_the_kernel_uses():
    assert {ROW_START_LATER} <= switch_values()


def test_waits_cover_each_tiles_loads():
    switch = switch_values()
    rng = random.Random(7)
    for _ in range(3000):
        rows = [rng.choice([0, 1, 2, 3, 4, 5, 6, 9, 17, 19, 32]) for _ in range(rng.randint(1, 5))]
        replay(rows, switch, rng, rowbuf=rng.random() < 0.5)


def test_model_catches_a_too_lenient_wait():
    # planted mistakes must be caught: a row start that leaves tile 0's last
    # row in flight, and a tile barrier that leaves stream A's last row in
    # flight
    rng = random.Random(3)
    everything = set(range(64))
    for kwargs in ({"row_start_later": 8}, {"bar_later": 1}):
        caught = False
        for _ in range(50):
            try:
                replay([rng.choice([3, 5, 9, 17, 32]), 4], everything, rng, **kwargs)
            except AssertionError:
                caught = True
                break
        assert caught, kwargs
