"""Pins of the rotary oracle (oracle/rotary.py) against things other than itself.

Sources of truth: a worked rotation typed from cos/sin values, the complex-number
form of the rotation (multiplying x1 + i x2 by exp(i pos theta)), identities of
rotations (position 0, inverse, norms, relative positions), torch's fp64
scaled-dot-product attention with autograd over rows rotated in complex form,
and central finite differences of the oracle's own forward. CPU only.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import jfa_inputs as J
from oracle import rotary as R

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def block_case(lengths, H, D, seed=0):
    w = J.custom(lengths, H, D, seed=seed, kind="block")
    c = J.make_case(w)
    f = J.bf16_bits_to_f64
    return f(c.q), f(c.k), f(c.v), f(c.do), c.offsets.astype(np.int64), c.scale


def rope_complex(x, positions, base):
    """The rotation as a complex product: z = x1 + i x2 times exp(i pos theta)."""
    d = x.shape[-1]
    theta = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(
        1j * np.asarray(positions, dtype=np.float64)[:, None, None] * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def test_worked_rotation():
    # D = 4, base 100: theta = (1, 0.1); position 1 rotates the pair (x0, x2) by
    # 1 rad and (x1, x3) by 0.1 rad
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    y = R.rope(x, [1], 100.0)[0, 0]
    want = [-1.9841106485555495, 1.590674663968739, 2.4623779024123156, 4.17968349440576]
    assert np.allclose(y, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("D", [4, 64, 128])
def test_matches_complex_form(D):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, D))
    pos = rng.integers(0, 5000, 50)
    assert np.max(np.abs(R.rope(x, pos, 10000.0) - rope_complex(x, pos, 10000.0))) <= 1e-9


def test_identities():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 2, 64))
    pos = np.arange(40)
    y = R.rope(x, pos, 500.0)
    # position 0 is the identity; the inverse undoes; each column pair keeps its norm
    assert np.array_equal(y[0], x[0])
    assert np.max(np.abs(R.rope(y, pos, 500.0, inverse=True) - x)) <= 1e-12
    n = lambda a: a[..., :32] ** 2 + a[..., 32:] ** 2
    assert np.max(np.abs(n(y) - n(x))) <= 1e-12
    # rotating by p then by p' is rotating by p + p'
    assert np.max(np.abs(R.rope(y, pos[::-1], 500.0) - R.rope(x, np.full(40, 39), 500.0))) <= 1e-11


def test_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((64, 1, 128))
    k = rng.standard_normal((64, 1, 128))
    p = np.arange(64)
    s0 = np.einsum("id,jd->ij", R.rope(q, p, 1e4)[:, 0], R.rope(k, p, 1e4)[:, 0])
    for shift in (1, 63, 64, 1000, 12345):
        s1 = np.einsum("id,jd->ij", R.rope(q, p + shift, 1e4)[:, 0], R.rope(k, p + shift, 1e4)[:, 0])
        assert np.max(np.abs(s1 - s0)) <= 1e-9


def test_token_positions():
    assert R.token_positions([0, 3, 3, 5]).tolist() == [0, 1, 2, 0, 1]


def _sdpa_rope_autograd(q, k, v, do, off, scale, base, mode="block"):
    """torch fp64: rows rotated in complex form, then SDPA with a mask keeping
    pairs of one 64-token block (mode "block"), of one sequence ("jagged") or of
    one sequence with key <= query ("causal"); gradients by autograd."""
    T, H, D = q.shape
    pos_np = R.token_positions(off)
    pos = torch.from_numpy(pos_np).double()
    theta = base ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    rot = torch.polar(torch.ones(T, 1, D // 2, dtype=torch.float64), pos[:, None, None] * theta)
    seg = torch.from_numpy(np.searchsorted(np.asarray(off), np.arange(T), side="right") - 1)
    if mode == "block":
        blk = torch.arange(T) // 64  # every sequence is a whole number of blocks
        keep = blk[:, None] == blk[None, :]
    else:
        keep = seg[:, None] == seg[None, :]
        if mode == "causal":
            p_ = torch.from_numpy(pos_np)
            keep &= p_[None, :] <= p_[:, None]

    def rotate(x):
        z = torch.complex(x[..., : D // 2], x[..., D // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    mask = keep[None, None]
    o = F.scaled_dot_product_attention(rotate(tq).transpose(0, 1)[None], rotate(tk).transpose(0, 1)[None],
                                       tv.transpose(0, 1)[None], attn_mask=mask, scale=scale)[0]
    o = o.transpose(0, 1)
    o.backward(torch.from_numpy(do))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("D", [64, 128])
def test_block_rope_matches_torch_autograd(D):
    q, k, v, do, off, sc = block_case([64, 192, 128], 2, D, seed=4)
    base = 10000.0
    out = R.block_diag_rope_forward(q, k, v, off, sc, base)
    ref, rq, rk, rv = _sdpa_rope_autograd(q, k, v, do, off, sc, base)
    assert np.max(np.abs(out - ref)) <= 1e-12
    dq, dk, dv = R.block_diag_rope_backward(q, k, v, do, off, sc, base)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-10


def test_block_rope_finite_differences():
    q, k, v, do, off, sc = block_case([64, 64], 1, 16, seed=5)
    base = 50.0

    def loss(q_, k_):
        return float(np.sum(R.block_diag_rope_forward(q_, k_, v, off, sc, base) * do))

    dq, dk, _ = R.block_diag_rope_backward(q, k, v, do, off, sc, base)
    rng = np.random.default_rng(6)
    h = 1e-6
    for _ in range(24):
        t, c = int(rng.integers(0, 128)), int(rng.integers(0, 16))
        for x, g, which in ((q, dq, 0), (k, dk, 1)):
            xp, xm = x.copy(), x.copy()
            xp[t, 0, c] += h
            xm[t, 0, c] -= h
            args_p = (xp, k) if which == 0 else (q, xp)
            args_m = (xm, k) if which == 0 else (q, xm)
            num = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(num - g[t, 0, c]) <= 1e-6 * max(1.0, abs(num))


def test_rotation_changes_the_result():
    # the rotation is not a no-op on this data: rotated and plain attention differ
    from oracle import attention as A
    q, k, v, do, off, sc = block_case([128], 2, 64, seed=7)
    a = A.block_diag_forward(q, k, v, off, sc)
    b = R.block_diag_rope_forward(q, k, v, off, sc, 10000.0)
    assert np.max(np.abs(a - b)) > 1e-3


def jagged_case(lengths, H, D, seed=0):
    w = J.custom(lengths, H, D, sigma=0.5, seed=seed)
    c = J.make_case(w)
    f = J.bf16_bits_to_f64
    return f(c.q), f(c.k), f(c.v), f(c.do), c.offsets.astype(np.int64), c.scale


@pytest.mark.parametrize("causal", [False, True])
def test_jagged_rope_matches_torch_autograd(causal):
    q, k, v, do, off, sc = jagged_case([37, 0, 1, 150, 64], 2, 64, seed=8)
    base = 10000.0
    out, lse = R.jagged_rope_forward(q, k, v, off, sc, base, causal)
    ref, rq, rk, rv = _sdpa_rope_autograd(q, k, v, do, off, sc, base,
                                          "causal" if causal else "jagged")
    assert np.max(np.abs(out - ref)) <= 1e-12
    dq, dk, dv = R.jagged_rope_backward(q, k, v, do, off, sc, base, causal)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-10


def test_jagged_rope_long_positions_depend_on_differences_only():
    # a sequence placed after another keeps its result: positions restart at every
    # sequence, and a common shift of all positions would not change the scores
    q, k, v, do, off, sc = jagged_case([300, 1000], 1, 64, seed=9)
    out, lse = R.jagged_rope_forward(q, k, v, off, sc, 500.0, True)
    s = 300
    out1, lse1 = R.jagged_rope_forward(q[s:], k[s:], v[s:], np.array([0, 1000]), sc, 500.0, True)
    assert np.max(np.abs(out[s:] - out1)) <= 1e-12
    assert np.max(np.abs(lse[:, s:] - lse1)) <= 1e-12
