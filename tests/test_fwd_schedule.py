"""Host-side model of the forward step kernel's shared-tile schedule (csrc/fwd_bf16.hip, the
`shared` branch): two groups of four wavefronts, group B one phase behind group A, a workgroup
barrier between phases, three K and three V slots in LDS, tile t in slot t % 3. Group A loads
the K tiles, group B the V tiles; each group waits for its loads with a vmcnt that leaves its
newest load in flight. V_j is read in both phases of tile j: the matrix phase X_j and, for the
PV products of the tile's last 16 keys, the start of the softmax phase Y_j.

The model replays both groups' program order (loads, waits, LDS reads, barriers) for 0..60 tiles
and checks, for every read of a tile: its load was issued into that slot, completed by the
issuing group's wait and published by a later barrier; and no load of a later tile into the same
slot was issued in or before the read's phase. Both groups pass the same number of barriers.
Planted mistakes (a wrong slot, a wait that leaves one load too many in flight, the softmax
phase's V read from the wrong slot) must fail.
"""
import pytest


def _program(grp, n, bad_slot=False, bad_wait=False, bad_tail=False):
    ev = []
    bar = lambda: ev.append(("bar",))
    if grp == 0:
        if n > 0:
            ev.append(("load", "K", 0, 0))
        if n > 1:
            ev.append(("load", "K", 1, 1))
    elif n > 0:
        ev.append(("load", "V", 0, 0))
    ev.append(("wait", 0))
    bar()
    if grp == 1:
        bar()  # group B runs one phase behind
    if grp == 0 and 2 < n:
        ev.append(("load", "K", 2, 2))
    if grp == 1 and 1 < n:
        ev.append(("load", "V", 1, 1))
    if n > 0:
        ev.append(("read", "K", 0, 0))  # X_{-1}: S_0
    bar()
    keep = 2 if bad_wait else 1

    def tile(j, s):
        bar()
        if grp == 0 and j + 3 < n:
            ev.append(("load", "K", j + 3, s))
        if grp == 1 and j + 2 < n:
            ev.append(("load", "V", j + 2, s if (bad_slot and j > 4) else (2 if s == 0 else s - 1)))
        ev.append(("read", "V", j, s))
        ev.append(("read", "K", j + 1, 0 if s == 2 else s + 1))
        if grp == 1:
            ev.append(("wait", keep if j + 2 < n else 0))
        bar()
        # the PV products of the tile's last 16 keys run at the start of Y_j
        ev.append(("read", "V", j, (s + 1) % 3 if (bad_tail and j > 4) else s))
        if grp == 0:
            ev.append(("wait", keep if j + 3 < n else 0))

    n_body = n - 1
    j = 0
    while j < n_body:
        tile(j, 0)
        if j + 1 < n_body:
            tile(j + 1, 1)
            if j + 2 < n_body:
                tile(j + 2, 2)
        j += 3
    if n > 0:
        bar()
        ev.append(("read", "V", n - 1, (n - 1) % 3))  # X of the last tile: PV alone
        bar()
    if grp == 0:
        bar()  # group A ends one phase earlier
    return ev


def _check(n, **plant):
    loads, reads, n_bar = [], [], []
    for grp in (0, 1):
        phase, queue = 0, []
        for e in _program(grp, n, **plant):
            if e[0] == "bar":
                phase += 1
            elif e[0] == "load":
                queue.append({"kind": e[1], "tile": e[2], "slot": e[3], "issued": phase, "done": None})
                loads.append(queue[-1])
            elif e[0] == "wait":  # loads complete in issue order: all but the newest e[1] tiles
                for x in queue[:len(queue) - e[1]]:
                    x["done"] = phase
                queue = queue[len(queue) - e[1]:]
            else:
                reads.append((e[1], e[2], e[3], phase))
        assert not queue, f"group {grp} ends with loads in flight"
        n_bar.append(phase)
    assert n_bar[0] == n_bar[1], f"barrier counts differ: {n_bar}"
    for kind, tile, slot, phase in reads:
        mine = [x for x in loads if x["kind"] == kind and x["tile"] == tile]
        assert len(mine) == 1 and mine[0]["slot"] == slot, (kind, tile, slot, mine)
        assert mine[0]["done"] is not None and mine[0]["done"] < phase, \
            f"{kind}_{tile} read in phase {phase} before it was published: {mine[0]}"
        for x in loads:
            if x["kind"] == kind and x["slot"] == slot and x["tile"] > tile:
                assert x["issued"] > phase, f"{kind}_{tile} overwritten by {x} while read in {phase}"
    for kind in "KV":
        assert sorted(x["tile"] for x in loads if x["kind"] == kind) == list(range(n))


@pytest.mark.parametrize("n", range(0, 61))
def test_shared_tile_schedule(n):
    _check(n)


@pytest.mark.parametrize("plant", [{"bad_slot": True}, {"bad_wait": True}, {"bad_tail": True}])
def test_planted_schedule_mistakes_fail(plant):
    with pytest.raises(AssertionError):
        for n in range(0, 61):
            _check(n, **plant)
