"""Pins of the reference tile scheduler: hand-worked examples of the page's rule
(tests/golden/schedule_examples.json) and properties any correct deal has."""
import json
import os

import numpy as np
import pytest

import jfa_inputs as J
from oracle import schedule_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_examples.json")


def _per_slot(slot_ptr, tiles):
    return [tiles[slot_ptr[s]:slot_ptr[s + 1]].tolist() for s in range(len(slot_ptr) - 1)]


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_golden(case):
    kind = R.KIND_FWD if case["kind"] == "fwd" else R.KIND_BWD
    for order, key in ((R.ORDER_ZIGZAG, "zigzag"), (R.ORDER_INORDER, "inorder")):
        sp, t = R.schedule(case["lengths"], case["heads"], kind, case["tile_rows"], order,
                           case["slots"], causal=case["causal"])
        assert _per_slot(sp, t) == case[key]
        assert R.slot_loads(sp, t) == case[key + "_loads"]


def _tiles_expected(L, H, kind, rows, causal, lq):
    n = 0
    for x in L:
        if kind == R.KIND_FWD:
            n += H * R.ceil_div(lq if lq else x, rows)
        else:
            n += H * R.ceil_div(x, rows)
    return n


@pytest.mark.parametrize("name", ["tiny", "gem", "gem_causal", "broadcast", "imbalance"])
@pytest.mark.parametrize("kind", [R.KIND_FWD, R.KIND_BWD])
def test_properties(name, kind):
    w = J.standard_workloads()[name]
    L = J.lengths(w)
    H = 2 if name == "imbalance" else w.num_heads   # keep the pure-Python run short
    rows = 128
    S = 256
    sp_z, tz = R.schedule(L, H, kind, rows, R.ORDER_ZIGZAG, S, w.causal, w.lq)
    sp_i, ti = R.schedule(L, H, kind, rows, R.ORDER_INORDER, S, w.causal, w.lq)
    n = _tiles_expected(L, H, kind, rows, w.causal, w.lq)
    assert len(tz) == len(ti) == n
    # every tile exactly once, in both orders
    key = lambda a: sorted(map(tuple, a.tolist()))
    assert key(tz) == key(ti)
    assert len(set(map(tuple, tz[:, :3].tolist()))) == n
    counts = np.diff(sp_z)
    assert counts.max() - counts.min() <= 1
    # zigzag: each slot's list is non-increasing in work
    for s in range(S):
        wk = tz[sp_z[s]:sp_z[s + 1], 3]
        assert np.all(np.diff(wk) <= 0)
    loads = np.array(R.slot_loads(sp_z, tz))
    assert loads.max() <= loads.mean() + tz[:, 3].max()
    # zigzag never has a worse makespan than round-robin on these workloads
    assert loads.max() <= max(R.slot_loads(sp_i, ti))


def test_empty_and_zero_length():
    sp, t = R.schedule([0, 0], 3, R.KIND_FWD, 64, R.ORDER_ZIGZAG, 4)
    assert t.shape == (0, 4) and list(sp) == [0] * 5
    # broadcast-Q forward keeps tiles of empty sequences (they write zeros)
    sp, t = R.schedule([0], 1, R.KIND_FWD, 64, R.ORDER_ZIGZAG, 2, lq=100)
    assert t.tolist() == [[0, 0, 0, 0], [0, 0, 1, 0]]


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["xcd_cases"], ids=lambda c: c["name"])
def test_golden_xcd(case):
    kind = R.KIND_FWD if case["kind"] == "fwd" else R.KIND_BWD
    sp, t = R.schedule(case["lengths"], case["heads"], kind, case["tile_rows"], R.ORDER_XCD_ZIGZAG,
                       case["slots"], causal=case["causal"], groups=case["groups"])
    assert _per_slot(sp, t) == case["schedule"]
    assert R.slot_loads(sp, t) == case["loads"]


@pytest.mark.parametrize("name", ["gem", "gem_causal", "broadcast"])
def test_xcd_properties(name):
    w = J.standard_workloads()[name]
    L = J.lengths(w)
    S, X = 512, 8
    sp, t = R.schedule(L, w.num_heads, R.KIND_FWD, 128, R.ORDER_XCD_ZIGZAG, S, w.causal, w.lq)
    sp0, t0 = R.schedule(L, w.num_heads, R.KIND_FWD, 128, R.ORDER_ZIGZAG, S, w.causal, w.lq)
    key = lambda a: sorted(map(tuple, a.tolist()))
    assert key(t) == key(t0)
    per = S // X
    home = {}
    for s in range(S):
        for b, h, _, _ in t[sp[s]:sp[s + 1]].tolist():
            assert home.setdefault((b, h), s // per) == s // per   # a unit stays on one XCD
        assert np.all(np.diff(t[sp[s]:sp[s + 1], 3]) <= 0)
    group_load = [int(t[sp[x * per]:sp[(x + 1) * per], 3].sum()) for x in range(X)]
    assert max(group_load) <= 1.1 * np.mean(group_load)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["folded_cases"], ids=lambda c: c["name"])
def test_golden_folded(case):
    kind = R.KIND_FWD if case["kind"] == "fwd" else R.KIND_BWD
    sp, t = R.schedule(case["lengths"], case["heads"], kind, case["tile_rows"],
                       R.ORDER_FOLDED_ZIGZAG, case["slots"], causal=case["causal"])
    assert _per_slot(sp, t) == case["schedule"]
    assert R.slot_loads(sp, t) == case["loads"]


@pytest.mark.parametrize("name", ["gem", "gem_causal", "broadcast"])
@pytest.mark.parametrize("kind", [R.KIND_FWD, R.KIND_BWD])
def test_folded_properties(name, kind):
    w = J.standard_workloads()[name]
    L = J.lengths(w)
    S = 512
    sp, t = R.schedule(L, w.num_heads, kind, 128, R.ORDER_FOLDED_ZIGZAG, S, w.causal, w.lq)
    sp0, t0 = R.schedule(L, w.num_heads, kind, 128, R.ORDER_ZIGZAG, S, w.causal, w.lq)
    key = lambda a: sorted(map(tuple, a.tolist()))
    assert key(t) == key(t0)                       # every tile exactly once
    if not w.causal:                              # nothing to fold: plain zigzag
        assert np.array_equal(sp, sp0) and np.array_equal(t, t0)
        return
    # the two tiles of a folded pair sit next to each other in one slot, and
    # their indices sum to n - 1 for the (sequence, head) they belong to
    n_of = {}
    for b, h, i, _ in t0.tolist():
        n_of[(b, h)] = max(n_of.get((b, h), 0), i + 1)
    for s in range(S):
        lst = t[sp[s]:sp[s + 1]].tolist()
        k = 0
        while k < len(lst):
            b, h, i, _ = lst[k]
            n = n_of[(b, h)]
            if 2 * i + 1 == n:                        # middle tile of an odd count
                k += 1
                continue
            assert i < n - 1 - i and lst[k + 1][:3] == [b, h, n - 1 - i]
            k += 2
    loads = np.array(R.slot_loads(sp, t))
    assert loads.max() <= loads.mean() + 2 * t[:, 3].max()
    assert loads.max() / loads.mean() < 1.06


def test_padded_gem_recipe():
    """The padded-dense comparison batch is the gem batch with every sequence as
    long as the longest one (same B, H, D and draw)."""
    wl = J.standard_workloads()
    g, p = wl["gem"], wl["gem_padded"]
    Lg, Lp = J.lengths(g), J.lengths(p)
    assert (g.num_seqs, g.num_heads, g.head_dim) == (p.num_seqs, p.num_heads, p.head_dim)
    assert np.all(Lp == Lg.max()) and Lp.shape == Lg.shape
    assert wl["gem_padded_causal"].causal and not p.causal


def _slots(sp, t):
    return [[tuple(x) for x in t[sp[s]:sp[s + 1]].tolist()] for s in range(len(sp) - 1)]


def test_hand_worked_xcd_inorder():
    """Lengths 300, 100, 200, one head, 128-row forward tiles (work = L each):
    units (0,0) with three tiles of 300, (1,0) with one of 100, (2,0) with two
    of 200.
    16 slots: 8 groups of 2. Unit (0,0) goes to group 0: its tiles to slots 0,
    1, then 0 again (both at 300, the lower slot). Unit (1,0) to group 1 (group
    0 holds 900, the others 0): slot 2. Unit (2,0) to group 2: slots 4 and 5.
    3 slots (not a multiple of 8): one group. Unit (0,0) fills slots 0, 1, 2;
    unit (1,0) goes to slot 0 (all at 300); unit (2,0) to slots 1 and 2 (300
    each, then 500 / 300)."""
    L = [300, 100, 200]
    sp, t = R.schedule(L, 1, R.KIND_FWD, 128, R.ORDER_XCD_INORDER, 16)
    want = [[] for _ in range(16)]
    want[0] = [(0, 0, 0, 300), (0, 0, 2, 300)]
    want[1] = [(0, 0, 1, 300)]
    want[2] = [(1, 0, 0, 100)]
    want[4] = [(2, 0, 0, 200)]
    want[5] = [(2, 0, 1, 200)]
    assert _slots(sp, t) == want
    sp, t = R.schedule(L, 1, R.KIND_FWD, 128, R.ORDER_XCD_INORDER, 3)
    assert _slots(sp, t) == [[(0, 0, 0, 300), (1, 0, 0, 100)],
                             [(0, 0, 1, 300), (2, 0, 0, 200)],
                             [(0, 0, 2, 300), (2, 0, 1, 200)]]


@pytest.mark.parametrize("name", ["gem", "gem_causal", "broadcast"])
@pytest.mark.parametrize("kind", [R.KIND_FWD, R.KIND_BWD])
def test_xcd_inorder_properties(name, kind):
    """Every tile once; a (sequence, head) unit on one group of slots; a slot's
    tiles in generation order; within a group the slot loads differ by at most
    the largest tile's work (each tile went to the least-loaded slot)."""
    w = J.standard_workloads()[name]
    L = J.lengths(w)
    S, X = 512, 8
    sp, t = R.schedule(L, w.num_heads, kind, 128, R.ORDER_XCD_INORDER, S, w.causal, w.lq)
    sp0, t0 = R.schedule(L, w.num_heads, kind, 128, R.ORDER_INORDER, S, w.causal, w.lq)
    key = lambda a: sorted(map(tuple, a.tolist()))
    assert key(t) == key(t0)
    per = S // X
    home = {}
    for s in range(S):
        rows = t[sp[s]:sp[s + 1]].tolist()
        for b, h, _, _ in rows:
            assert home.setdefault((b, h), s // per) == s // per
        gen = [(b, h, tt) for b, h, tt, _ in rows]
        assert gen == sorted(gen)
    big = int(t[:, 3].max())
    for x in range(X):
        loads = [int(t[sp[s]:sp[s + 1], 3].sum()) for s in range(x * per, (x + 1) * per)]
        assert max(loads) - min(loads) <= big
