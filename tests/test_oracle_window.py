"""Pins of the oracle's causal sliding window (query i attends keys j with
i - W < j <= i) against things other than itself: torch fp64 SDPA with a banded
mask and autograd, a pure-Python loop, closed forms (W = 1 gives out = v; a
window covering the sequence gives plain causal attention), finite differences,
and the window's tile work in the reference scheduler against brute-force counts.
CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import jfa_inputs as J
from oracle import attention as A
from oracle import schedule_ref as S

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def case(lengths, H, D, seed):
    w = J.custom(lengths, H, D, sigma=0.5, seed=seed, causal=True)
    c = J.make_case(w)
    f = J.bf16_bits_to_f64
    return f(c.q), f(c.k), f(c.v), f(c.do), c.offsets.astype(np.int64), c.scale


def sdpa_window(q, k, v, do, off, scale, W):
    T = q.shape[0]
    seg = np.searchsorted(off, np.arange(T), side="right") - 1
    pos = np.arange(T) - off[seg]
    keep = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None]) & \
        (pos[None, :] > pos[:, None] - W)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))).requires_grad_()
                  for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                       attn_mask=torch.from_numpy(keep)[None, None], scale=scale)[0]
    o.backward(torch.from_numpy(np.ascontiguousarray(do.transpose(1, 0, 2))))
    return (o.detach().numpy().transpose(1, 0, 2),
            *(t.grad.numpy().transpose(1, 0, 2) for t in (tq, tk, tv)))


@pytest.mark.parametrize("W", [1, 5, 64, 130])
def test_window_matches_torch_sdpa_and_autograd(W):
    q, k, v, do, off, sc = case([200, 0, 1, 77, 129], 2, 32, seed=31)
    out, lse = A.jagged_forward(q, k, v, off, sc, True, W)
    ref, rq, rk, rv = sdpa_window(q, k, v, do, off, sc, W)
    assert np.max(np.abs(out - ref)) <= 1e-12
    dq, dk, dv = A.jagged_backward(q, k, v, do, off, sc, True, W)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-10


def test_window_matches_loops():
    rng = np.random.default_rng(32)
    q, k, v = (rng.standard_normal((9, 4)) for _ in range(3))
    W, sc = 3, 0.7
    out, lse = A.seq_forward(q, k, v, sc, True, W)
    for i in range(9):
        keys = [j for j in range(9) if i - W < j <= i]
        s = [sc * float(q[i] @ k[j]) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        assert abs(lse[i] - (mx + math.log(z))) <= 1e-12
        want = sum(e[t] * v[keys[t]] for t in range(len(keys))) / z
        assert np.max(np.abs(out[i] - want)) <= 1e-12


def test_window_closed_forms():
    q, k, v, do, off, sc = case([50, 3], 1, 16, seed=33)
    # W = 1: every query sees only its own key
    out, lse = A.jagged_forward(q, k, v, off, sc, True, 1)
    assert np.max(np.abs(out - v)) <= 1e-12
    assert np.max(np.abs(lse[0] - sc * np.sum(q[:, 0] * k[:, 0], axis=1))) <= 1e-12
    # a window at least as long as every sequence is plain causal attention
    o1, l1 = A.jagged_forward(q, k, v, off, sc, True, 50)
    o2, l2 = A.jagged_forward(q, k, v, off, sc, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_window_finite_differences():
    q, k, v, do, off, sc = case([23], 1, 8, seed=34)
    W = 4
    dq, dk, dv = A.jagged_backward(q, k, v, do, off, sc, True, W)
    loss = lambda q_, k_, v_: float(np.sum(A.jagged_forward(q_, k_, v_, off, sc, True, W)[0] * do))
    rng = np.random.default_rng(35)
    h = 1e-6
    for _ in range(30):
        t, c, which = int(rng.integers(23)), int(rng.integers(8)), int(rng.integers(3))
        xs = [q, k, v]
        xp = [x.copy() for x in xs]
        xm = [x.copy() for x in xs]
        xp[which][t, 0, c] += h
        xm[which][t, 0, c] -= h
        num = (loss(*xp) - loss(*xm)) / (2 * h)
        g = (dq, dk, dv)[which][t, 0, c]
        assert abs(num - g) <= 1e-6 * max(1.0, abs(num))


@pytest.mark.parametrize("W", [1, 100, 128, 300, 5000])
def test_window_tile_work_brute_force(W):
    L = [1, 127, 128, 129, 700, 2000]
    rows = 128
    for kind in (S.KIND_FWD, S.KIND_BWD):
        tiles = S.enumerate_tiles(L, 1, kind, rows, causal=True, window=W)
        for b, h, t, work in tiles:
            n = L[b]
            lo, hi = t * rows, min(n, (t + 1) * rows)
            if kind == S.KIND_FWD:   # keys in the union of the tile's query windows
                want = len({j for i in range(lo, hi) for j in range(max(0, i - W + 1), i + 1)})
            else:                    # queries whose window holds a key of the tile
                want = len({i for j in range(lo, hi) for i in range(j, min(n, j + W))})
            assert work == want, (kind, b, t, work, want)
