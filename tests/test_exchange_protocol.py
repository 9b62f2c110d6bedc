"""A host-side model of the strip exchange's workspace protocol (CPU only).

The GEMM + epilogue kernel exchanges per-row partial statistics between the
workgroups of a row strip (the review's level-3 aggregation, Fig. 4) through a
workspace that is cleared once and then reused by every later launch:

  * header words: epoch, done counter, error flag; then the slots;
  * at its start a workgroup reads the epoch; its tag is epoch + 1;
  * a slot word carries (tag << 32) | value, stored by one atomic 64-bit
    store; a reader accepts a peer's word only when its tag is the current
    one, polls until then or until its spin budget runs out (then it marks
    the error flag and its row's results NaN);
  * merges run in tile order;
  * at its end a workgroup adds 1 to the done counter; the one that brings it
    to the grid size resets it to 0 and stores epoch = tag.

The model runs the workgroups of a launch as coroutines under random
interleavings (one atomic step at a time), with workgroups that start late,
consecutive launches of different shapes on one workspace, stale slots from
earlier launches, and a zero spin budget. It checks that every accepted value
is the current launch's, the merged results are exact, the epoch advances by
one per launch and the done counter returns to 0, and that a timeout always
shows as the error flag plus NaN results. A variant that ignores the tag is
caught by the same checks (the model has teeth)."""
import math
import random

import pytest

MASK32 = (1 << 32) - 1


class Workspace:
    def __init__(self, slots):
        self.epoch = 0
        self.done = 0
        self.error = 0
        self.slots = [0] * slots

    def init(self):
        self.epoch = self.done = self.error = 0
        self.slots = [0] * len(self.slots)


def launch(ws, strips, tiles_n, grid, values, rng, spin_budget=10**9, check_tag=True, delays=None):
    """One launch: `grid` workgroups (a multiple of tiles_n, <= strips*tiles_n)
    process the strips in rounds; tile t = strip * tiles_n + tn publishes
    values[t] and every tile of the strip merges all of them in tile order.
    Returns {tile: merged sum (NaN if a peer was lost)}."""
    tiles = strips * tiles_n
    assert grid % tiles_n == 0 and 0 < grid <= tiles
    results = {}

    def wg(bid):
        yield
        tag = (ws.epoch + 1) & MASK32           # read at the workgroup's start
        yield
        for base in range(0, tiles, grid):
            t = base + bid
            if t >= tiles:
                break
            strip, tn = divmod(t, tiles_n)
            ws.slots[t] = (tag << 32) | values[t]   # publish (one atomic store)
            yield
            acc, lost = 0, False
            for peer in range(tiles_n):             # merge in tile order
                pt = strip * tiles_n + peer
                if peer == tn:
                    acc += values[t]
                    continue
                spins = 0
                while True:
                    w = ws.slots[pt]
                    yield
                    if not check_tag or (w >> 32) == tag:
                        acc += w & MASK32
                        break
                    spins += 1
                    if spins > spin_budget:
                        ws.error = 1
                        lost = True
                        break
            results[t] = math.nan if lost else acc
        prev = ws.done
        ws.done = prev + 1                          # one atomic fetch-add
        yield
        if prev == grid - 1:
            ws.done = 0
            ws.epoch = tag

    delays = delays or {}
    live = {b: wg(b) for b in range(grid)}
    wait = {b: delays.get(b, 0) for b in range(grid)}
    steps = 0
    while live:
        runnable = [b for b in live if wait[b] <= 0]
        for b in live:
            wait[b] -= 1
        if not runnable:
            continue
        b = rng.choice(runnable)
        try:
            next(live[b])
        except StopIteration:
            del live[b]
        steps += 1
        assert steps < 10**7, "launch did not finish"
    return results


def expected(strips, tiles_n, values):
    out = {}
    for s in range(strips):
        tot = sum(values[s * tiles_n + j] for j in range(tiles_n))
        for j in range(tiles_n):
            out[s * tiles_n + j] = tot
    return out


SHAPES = [(4, 16, 32), (2, 8, 16), (6, 4, 8), (3, 16, 16), (1, 32, 32), (8, 2, 16)]   # strips, tiles_n, grid


@pytest.mark.parametrize("seed", range(6))
def test_consecutive_launches_of_different_shapes_are_exact(seed):
    rng = random.Random(seed)
    ws = Workspace(8 * 32)
    for n in range(30):
        strips, tiles_n, grid = SHAPES[rng.randrange(len(SHAPES))]
        tiles = strips * tiles_n
        values = [rng.randrange(1, 1000) for _ in range(tiles)]
        delays = {b: rng.randrange(0, 400) for b in rng.sample(range(grid), max(1, grid // 4))}
        epoch0 = ws.epoch
        res = launch(ws, strips, tiles_n, grid, values, rng, delays=delays)
        assert res == expected(strips, tiles_n, values), f"launch {n}: a stale or foreign value was merged"
        assert ws.epoch == epoch0 + 1 and ws.done == 0 and ws.error == 0


def test_stale_slots_with_the_same_values_layout_never_pass():
    # every slot of the workspace holds a word of the previous epoch with a
    # different value: readers must wait for the current one
    rng = random.Random(7)
    ws = Workspace(64)
    strips, tiles_n, grid = 4, 16, 32
    launch(ws, strips, tiles_n, grid, [1] * 64, rng)
    for _ in range(5):
        values = [rng.randrange(2, 1000) for _ in range(64)]
        assert launch(ws, strips, tiles_n, grid, values, rng) == expected(strips, tiles_n, values)


def test_delayed_workgroup_is_waited_for():
    rng = random.Random(3)
    ws = Workspace(64)
    values = list(range(1, 65))
    # workgroup 5 starts long after its strip's peers have published and polled
    res = launch(ws, 4, 16, 32, values, rng, delays={5: 5000})
    assert res == expected(4, 16, values) and ws.error == 0


def test_zero_spin_budget_reports_and_poisons():
    rng = random.Random(11)
    ws = Workspace(64)
    seen_timeout = False
    for _ in range(20):
        values = [rng.randrange(1, 1000) for _ in range(64)]
        res = launch(ws, 4, 16, 32, values, rng, spin_budget=0, delays={b: rng.randrange(0, 50) for b in range(32)})
        exp = expected(4, 16, values)
        nan = [t for t, v in res.items() if isinstance(v, float) and math.isnan(v)]
        # every result is either exact or NaN, and NaN appears iff the flag is set
        assert all(res[t] == exp[t] for t in res if t not in nan)
        assert bool(nan) == bool(ws.error)
        seen_timeout |= bool(nan)
        assert ws.done == 0
        if ws.error:
            ws.init()        # cf_workspace_init
    assert seen_timeout, "a zero spin budget should time out some waits"
    values = [rng.randrange(1, 1000) for _ in range(64)]
    assert launch(ws, 4, 16, 32, values, rng) == expected(4, 16, values)


def test_ignoring_the_tag_is_caught():
    # negative control: without the tag check a reader takes stale words
    caught = False
    for seed in range(20):
        rng = random.Random(seed)
        ws = Workspace(64)
        launch(ws, 4, 16, 32, [1] * 64, rng)
        values = [rng.randrange(2, 1000) for _ in range(64)]
        res = launch(ws, 4, 16, 32, values, rng, check_tag=False, delays={b: 300 for b in range(0, 32, 3)})
        caught |= res != expected(4, 16, values)
    assert caught
