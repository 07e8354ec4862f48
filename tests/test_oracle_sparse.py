"""Pins of the oracle's block-sparse attention (oracle/attention.py) against
sources other than itself: torch's fp64 scaled_dot_product_attention with the
token-level boolean mask the block mask expands to (and autograd for the
gradients), a pure-Python loop over a micro case, reductions to forms pinned
elsewhere (an all-ones mask gives plain attention, a diagonal mask the
block-diagonal mode), rows whose blocks allow no key (dropped from the SDPA
problem, whose other rows and keys must not change), central finite differences,
and the pair count against the expanded mask. CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from tests.test_oracle import case64

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

BLK = 64


def rand_masks(lengths, seed, density=0.4, diag=True, empty_rows=()):
    """One random block mask per sequence; `diag` keeps every query block's own
    key block, `empty_rows` lists (sequence, query block) rows to clear."""
    rng = np.random.default_rng(seed)
    out = []
    for b, L in enumerate(lengths):
        n = -(-L // BLK)
        m = rng.random((n, n)) < density
        if diag:
            m |= np.eye(n, dtype=bool)
        for bb, r in empty_rows:
            if bb == b:
                m[r] = False
        out.append(m)
    return out


def token_mask(offsets, masks):
    """[T, T] boolean: query i may attend key j (same sequence, allowed blocks)."""
    T = int(offsets[-1])
    keep = np.zeros((T, T), dtype=bool)
    for b, m in enumerate(masks):
        s, e = int(offsets[b]), int(offsets[b + 1])
        i = np.arange(e - s)
        keep[s:e, s:e] = m[i[:, None] // BLK, i[None, :] // BLK]
    return keep


def sdpa(q, k, v, do, keep, rows):
    """torch fp64 SDPA of the query rows `rows` against all keys (mask keep[rows]),
    with autograd: out, dq [len(rows)], dk, dv [T]."""
    tq = torch.from_numpy(np.ascontiguousarray(q[rows].transpose(1, 0, 2))).requires_grad_()
    tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))).requires_grad_()
              for x in (k, v))
    mask = torch.from_numpy(keep[rows])
    o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask[None, None],
                                       scale=SC)[0]
    o.backward(torch.from_numpy(np.ascontiguousarray(do[rows].transpose(1, 0, 2))))
    tr = lambda t: t.detach().numpy().transpose(1, 0, 2)
    return tr(o), tr(tq.grad), tr(tk.grad), tr(tv.grad)


SC = 0.3


@pytest.mark.parametrize("seed", [0, 1])
def test_sparse_matches_sdpa(seed):
    lengths = [1, 64, 65, 130, 200]
    q, k, v, do, off, _ = case64(lengths, 2, 16, seed=seed)
    masks = rand_masks(lengths, seed, density=0.4)
    keep = token_mask(off, masks)
    rows = np.arange(int(off[-1]))
    o_ref, dq_ref, dk_ref, dv_ref = sdpa(q, k, v, do, keep, rows)
    out, lse = A.block_sparse_forward(q, k, v, off, SC, masks)
    dq, dk, dv = A.block_sparse_backward(q, k, v, do, off, SC, masks)
    assert np.max(np.abs(out - o_ref)) <= 1e-12
    for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        assert np.max(np.abs(got - ref)) <= 1e-11
    # lse against the log-sum-exp of the masked scores
    s = SC * np.einsum("ihd,jhd->hij", q, k)
    s = np.where(keep[None], s, -np.inf)
    mx = s.max(-1)
    ref_lse = mx + np.log(np.exp(s - mx[..., None]).sum(-1))
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_rows_without_keys():
    """Query blocks whose row of the mask is empty: out = 0, lse = -inf, dq = 0,
    and every other row and every key gradient as in the problem without them."""
    lengths = [130, 70, 64]
    empty = [(0, 1), (1, 0), (2, 0)]
    q, k, v, do, off, _ = case64(lengths, 2, 16, seed=4)
    masks = rand_masks(lengths, 4, density=0.5, empty_rows=empty)
    keep = token_mask(off, masks)
    has = keep.any(axis=1)
    out, lse = A.block_sparse_forward(q, k, v, off, SC, masks)
    dq, dk, dv = A.block_sparse_backward(q, k, v, do, off, SC, masks)
    dead = np.nonzero(~has)[0]
    live = np.nonzero(has)[0]
    assert len(dead) == 3 * 64
    assert np.all(out[dead] == 0) and np.all(np.isneginf(lse[:, dead])) and np.all(dq[dead] == 0)
    o_ref, dq_ref, dk_ref, dv_ref = sdpa(q, k, v, do, keep, live)
    assert np.max(np.abs(out[live] - o_ref)) <= 1e-12
    assert np.max(np.abs(dq[live] - dq_ref)) <= 1e-11
    assert np.max(np.abs(dk - dk_ref)) <= 1e-11
    assert np.max(np.abs(dv - dv_ref)) <= 1e-11


def test_all_ones_mask_is_plain_attention():
    lengths = [1, 63, 64, 65, 190]
    q, k, v, do, off, _ = case64(lengths, 2, 16, seed=5)
    masks = [np.ones((-(-L // BLK),) * 2, dtype=bool) for L in lengths]
    out, lse = A.block_sparse_forward(q, k, v, off, SC, masks)
    o2, l2 = A.jagged_forward(q, k, v, off, SC, False)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    g = A.block_sparse_backward(q, k, v, do, off, SC, masks)
    g2 = A.jagged_backward(q, k, v, do, off, SC, False)
    for a, b in zip(g, g2):
        assert np.array_equal(a, b)


def test_diagonal_mask_is_block_diagonal():
    lengths = [64, 192, 128]
    q, k, v, do, off, _ = case64(lengths, 2, 16, seed=6)
    masks = [np.eye(L // BLK, dtype=bool) for L in lengths]
    out, _ = A.block_sparse_forward(q, k, v, off, SC, masks)
    assert np.max(np.abs(out - A.block_diag_forward(q, k, v, off, SC))) <= 1e-13
    g = A.block_sparse_backward(q, k, v, do, off, SC, masks)
    g2 = A.block_diag_backward(q, k, v, do, off, SC)
    for a, b in zip(g, g2):
        assert np.max(np.abs(a - b)) <= 1e-12


def test_matches_python_loops():
    """A 70-token sequence (two blocks, the second partial) with an asymmetric
    mask, evaluated key by key in plain Python."""
    rng = np.random.default_rng(8)
    L, D = 70, 3
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    bm = np.array([[True, False], [True, True]])
    o, l = A.seq_forward(q, k, v, SC, bmask=bm)
    for i in range(L):
        keys = [j for j in range(L) if bm[i // BLK][j // BLK]]
        s = [SC * sum(q[i][d] * k[j][d] for d in range(D)) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        for n in range(D):
            assert abs(o[i][n] - sum(e[t] * v[keys[t]][n] for t in range(len(keys))) / z) <= 1e-13
        assert abs(l[i] - (mx + math.log(z))) <= 1e-13


def test_gradients_match_finite_differences():
    lengths = [70, 20]
    q, k, v, do, off, _ = case64(lengths, 1, 4, seed=9)
    masks = [np.array([[True, False], [True, True]]), np.array([[True]])]
    dq, dk, dv = A.block_sparse_backward(q, k, v, do, off, SC, masks)
    f = lambda q_, k_, v_: float(np.sum(A.block_sparse_forward(q_, k_, v_, off, SC, masks)[0] * do))
    eps = 1e-6
    rng = np.random.default_rng(10)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            t, d = int(rng.integers(0, 90)), int(rng.integers(0, 4))
            xp, xm = x.copy(), x.copy()
            xp[t, 0, d] += eps
            xm[t, 0, d] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num = (f(*args_p) - f(*args_m)) / (2 * eps)
            assert abs(num - g[t, 0, d]) <= 1e-7 * max(1.0, abs(num)), (name, t, d)


def test_pair_count_is_the_expanded_mask():
    lengths = [1, 64, 65, 130, 0, 200]
    masks = rand_masks(lengths, 11, density=0.3, diag=False)
    off = np.concatenate([[0], np.cumsum(lengths)])
    assert A.pair_count(lengths, masks=masks) == int(token_mask(off, masks).sum())


def test_flat_masks_round_trip():
    lengths = [1, 64, 65, 0, 130]
    masks = rand_masks(lengths, 12)
    flat = np.concatenate([m.astype(np.uint8).ravel() for m in masks])
    off = np.concatenate([[0], np.cumsum(lengths)])
    back = A.sparse_masks(off, flat)
    assert all(np.array_equal(a, b) for a, b in zip(masks, back))
    with pytest.raises(ValueError):
        A.sparse_masks(off, flat[:-1])


def _causal(off, keep):
    T = int(off[-1])
    seg = np.repeat(np.arange(len(off) - 1), np.diff(off))
    pos = np.arange(T) - np.asarray(off)[seg]
    return keep & (pos[None, :] <= pos[:, None])


@pytest.mark.parametrize("seed", [0, 1])
def test_causal_sparse_matches_sdpa(seed):
    """With causal, query i keeps key j iff its block mask allows the pair and
    j <= i (every query block keeps its own block here, so every row has a key)."""
    lengths = [1, 64, 65, 130, 200]
    q, k, v, do, off, _ = case64(lengths, 2, 16, seed=seed + 20)
    masks = rand_masks(lengths, seed + 20, density=0.4)
    keep = _causal(off, token_mask(off, masks))
    rows = np.arange(int(off[-1]))
    o_ref, dq_ref, dk_ref, dv_ref = sdpa(q, k, v, do, keep, rows)
    out, lse = A.block_sparse_forward(q, k, v, off, SC, masks, causal=True)
    dq, dk, dv = A.block_sparse_backward(q, k, v, do, off, SC, masks, causal=True)
    assert np.max(np.abs(out - o_ref)) <= 1e-12
    for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        assert np.max(np.abs(got - ref)) <= 1e-11


def test_causal_all_ones_is_plain_causal():
    lengths = [1, 63, 64, 65, 190]
    q, k, v, do, off, _ = case64(lengths, 2, 16, seed=21)
    masks = [np.ones((-(-L // BLK),) * 2, dtype=bool) for L in lengths]
    out, lse = A.block_sparse_forward(q, k, v, off, SC, masks, causal=True)
    o2, l2 = A.jagged_forward(q, k, v, off, SC, True)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    for a, b in zip(A.block_sparse_backward(q, k, v, do, off, SC, masks, causal=True),
                    A.jagged_backward(q, k, v, do, off, SC, True)):
        assert np.array_equal(a, b)


def test_causal_rows_without_keys():
    """A query block whose own block and every earlier block are masked keeps no
    key under causal (block 0 of a sequence whose mask row 0 is all zero)."""
    lengths = [130]
    q, k, v, do, off, _ = case64(lengths, 1, 8, seed=22)
    bm = np.array([[0, 1, 1], [1, 1, 0], [0, 1, 1]], bool)
    out, lse = A.block_sparse_forward(q, k, v, off, SC, [bm], causal=True)
    dq, _, _ = A.block_sparse_backward(q, k, v, do, off, SC, [bm], causal=True)
    assert np.all(out[:64] == 0) and np.all(np.isneginf(lse[:, :64])) and np.all(dq[:64] == 0)
    assert np.all(np.isfinite(lse[:, 64:]))


def test_causal_pair_count_is_the_expanded_mask():
    lengths = [1, 64, 65, 130, 0, 200]
    masks = rand_masks(lengths, 23, density=0.3, diag=False)
    off = np.concatenate([[0], np.cumsum(lengths)])
    assert A.pair_count(lengths, causal=True, masks=masks) == \
        int(_causal(off, token_mask(off, masks)).sum())
