"""Pins of the CPU oracle against things other than itself.

Each check compares oracle/attention.py with an independent source of truth:
torch's fp64 scaled_dot_product_attention and autograd (library routines),
dense padded attention with explicit masks, brute-force loops on micro cases,
the online-softmax recurrence that the block-attention page prints (section 2),
closed forms (length-1 sequences, identical keys), invariances, and central
finite differences. None of these runs on a GPU.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import jfa_inputs as J
from oracle import attention as A

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def case64(lengths, H, D, seed=0, sigma=1.0, kind="jagged", lq=0):
    w = J.custom(lengths, H, D, sigma=sigma, seed=seed, kind=kind, lq=lq)
    c = J.make_case(w)
    f = J.bf16_bits_to_f64
    return f(c.q), f(c.k), f(c.v), f(c.do), c.offsets.astype(np.int64), c.scale


def tiny_case(seed=0):
    w = J.standard_workloads()["tiny"].with_(seed=seed)
    c = J.make_case(w)
    f = J.bf16_bits_to_f64
    return f(c.q), f(c.k), f(c.v), f(c.do), c.offsets.astype(np.int64), c.scale


# ------------------------------------------------------------ independent forms
def sdpa_packed(q, k, v, offsets, scale, causal, grad_do=None, block=0):
    """torch fp64 SDPA over the whole packed token axis with a boolean mask that
    keeps only (query, key) pairs of the same sequence (and the causal / block
    rules). Returns out [T,H,D] (and dq, dk, dv through autograd if grad_do)."""
    T = q.shape[0]
    seg = np.zeros(T, dtype=np.int64)
    for b in range(len(offsets) - 1):
        seg[offsets[b]:offsets[b + 1]] = b
    pos = np.arange(T) - offsets[seg]
    m = seg[:, None] == seg[None, :]
    if causal:
        m &= pos[None, :] <= pos[:, None]
    if block:
        m &= (pos[:, None] // block) == (pos[None, :] // block)
    mask = torch.from_numpy(m)
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2))).requires_grad_()
                  for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask[None, None],
                                       scale=scale)[0]
    out = o.detach().numpy().transpose(1, 0, 2)
    if grad_do is None:
        return out
    o.backward(torch.from_numpy(np.ascontiguousarray(grad_do.transpose(1, 0, 2))))
    g = [t.grad.numpy().transpose(1, 0, 2) for t in (tq, tk, tv)]
    return out, g[0], g[1], g[2]


def padded_dense(q, k, v, offsets, scale, causal):
    """Dense [B,H,Lmax,Lmax] attention with -inf on padded keys (and j > i)."""
    off = offsets
    B = len(off) - 1
    L = np.diff(off)
    Lm = int(L.max())
    H, D = q.shape[1], q.shape[2]
    Qp = np.zeros((B, H, Lm, D)); Kp = np.zeros_like(Qp); Vp = np.zeros_like(Qp)
    for b in range(B):
        s, e = off[b], off[b + 1]
        Qp[b, :, :e - s] = q[s:e].transpose(1, 0, 2)
        Kp[b, :, :e - s] = k[s:e].transpose(1, 0, 2)
        Vp[b, :, :e - s] = v[s:e].transpose(1, 0, 2)
    S = scale * np.einsum("bhid,bhjd->bhij", Qp, Kp)
    i = np.arange(Lm)[:, None]
    j = np.arange(Lm)[None, :]
    for b in range(B):
        keep = j < L[b]
        if causal:
            keep = keep & (j <= i)
        S[b] = np.where(keep[None], S[b], -np.inf)
    mx = S.max(-1, keepdims=True)
    E = np.exp(S - mx)
    Z = E.sum(-1, keepdims=True)
    O = (E / Z) @ Vp
    lse = (mx + np.log(Z))[..., 0]
    out = np.zeros_like(q)
    ls = np.full((H, q.shape[0]), -np.inf)
    for b in range(B):
        s, e = off[b], off[b + 1]
        out[s:e] = O[b, :, :e - s].transpose(1, 0, 2)
        ls[:, s:e] = lse[b, :, :e - s]
    return out, ls


def flash_recurrence(q, k, v, scale, tile=16):
    """The online-softmax loop the block-attention page prints (section 2), run
    in float64 over key tiles: running max m, correction alpha, rescaled O and l,
    final O / l and L = m + log(l)."""
    Lq = q.shape[0]
    m = np.full(Lq, -np.inf)
    l = np.zeros(Lq)
    O = np.zeros((Lq, v.shape[1]))
    for j0 in range(0, k.shape[0], tile):
        S = scale * (q @ k[j0:j0 + tile].T)
        m_new = np.maximum(m, S.max(axis=1))
        alpha = np.exp(m - m_new)
        E = np.exp(S - m_new[:, None])
        O = alpha[:, None] * O + E @ v[j0:j0 + tile]
        l = alpha * l + E.sum(axis=1)
        m = m_new
    return O / l[:, None], m + np.log(l)


def loops_forward(q, k, v, scale, causal):
    """Pure-Python triple loop (micro sizes only)."""
    Lq, D, Lk, Dv = len(q), len(q[0]), len(k), len(v[0])
    out = [[0.0] * Dv for _ in range(Lq)]
    lse = []
    for i in range(Lq):
        keys = [j for j in range(Lk) if (not causal or j <= i)]
        s = [scale * sum(q[i][d] * k[j][d] for d in range(D)) for j in keys]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        for n in range(Dv):
            out[i][n] = sum(e[t] * v[keys[t]][n] for t in range(len(keys))) / z
        lse.append(mx + math.log(z))
    return np.array(out), np.array(lse)


# ------------------------------------------------------------------- forward
@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_torch_sdpa(causal):
    q, k, v, do, off, sc = tiny_case(seed=3)
    out, lse = A.jagged_forward(q, k, v, off, sc, causal)
    ref = sdpa_packed(q, k, v, off, sc, causal)
    assert np.max(np.abs(out - ref)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_padded_dense(causal):
    q, k, v, do, off, sc = case64([37, 1, 64, 5, 20], 3, 16, seed=1)
    out, lse = A.jagged_forward(q, k, v, off, sc, causal)
    o2, l2 = padded_dense(q, k, v, off, sc, causal)
    assert np.max(np.abs(out - o2)) <= 1e-12
    assert np.max(np.abs(lse - l2)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_loops(causal):
    rng = np.random.default_rng(7)
    for L in (1, 2, 5):
        q, k, v = (rng.standard_normal((L, 4)) for _ in range(3))
        o, l = A.seq_forward(q, k, v, 0.37, causal)
        o2, l2 = loops_forward(q.tolist(), k.tolist(), v.tolist(), 0.37, causal)
        assert np.max(np.abs(o - o2)) <= 1e-13
        assert np.max(np.abs(l - l2)) <= 1e-13


def test_forward_matches_flash_recurrence():
    q, k, v, do, off, sc = case64([300], 1, 64, seed=2)
    o, l = A.seq_forward(q[:, 0], k[:, 0], v[:, 0], sc, False)
    o2, l2 = flash_recurrence(q[:, 0], k[:, 0], v[:, 0], sc, tile=16)
    assert np.max(np.abs(o - o2)) <= 1e-13
    assert np.max(np.abs(l - l2)) <= 1e-12


def test_rows_sum_to_one_and_constant_v():
    q, k, v, do, off, sc = case64([50, 7], 2, 32, seed=4)
    ones = np.ones_like(v)
    for causal in (False, True):
        out, _ = A.jagged_forward(q, k, ones, off, sc, causal)
        assert np.max(np.abs(out - 1.0)) <= 1e-14


def test_length_one_returns_v():
    q, k, v, do, off, sc = case64([1, 3, 1], 2, 64, seed=5)
    out, lse = A.jagged_forward(q, k, v, off, sc, False)
    for t in (0, 4):
        assert np.array_equal(out[t], v[t])
        np.testing.assert_allclose(lse[:, t], sc * np.sum(q[t] * k[t], axis=-1), rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    q, k, v, do, off, sc = case64([33], 2, 16, seed=6)
    k[:] = k[0]
    out, lse = A.jagged_forward(q, k, v, off, sc, causal)
    L = 33
    for h in range(2):
        if causal:
            ref = np.cumsum(v[:, h], axis=0) / np.arange(1, L + 1)[:, None]
            cnt = np.arange(1, L + 1)
        else:
            ref = np.broadcast_to(v[:, h].mean(axis=0), (L, 16))
            cnt = np.full(L, L)
        assert np.max(np.abs(out[:, h] - ref)) <= 1e-13
        np.testing.assert_allclose(lse[h], sc * (q[:, h] @ k[0, h]) + np.log(cnt), atol=1e-13)


def test_key_shift_invariance():
    q, k, v, do, off, sc = case64([40, 9], 2, 32, seed=8)
    u = np.random.default_rng(0).standard_normal(32)
    out, lse = A.jagged_forward(q, k, v, off, sc, True)
    out2, lse2 = A.jagged_forward(q, k + u, v, off, sc, True)
    assert np.max(np.abs(out - out2)) <= 1e-12
    np.testing.assert_allclose(lse2 - lse, sc * np.einsum("thd,d->ht", q, u), atol=1e-12)


def test_sequence_permutation_and_kv_row_permutation():
    L = [12, 30, 5]
    q, k, v, do, off, sc = case64(L, 2, 16, seed=9)
    out, lse = A.jagged_forward(q, k, v, off, sc, False)
    # reverse the sequence order
    segs = [(off[b], off[b + 1]) for b in range(3)][::-1]
    perm = np.concatenate([np.arange(s, e) for s, e in segs])
    off2 = np.concatenate([[0], np.cumsum([e - s for s, e in segs])])
    out2, lse2 = A.jagged_forward(q[perm], k[perm], v[perm], off2, sc, False)
    assert np.max(np.abs(out2 - out[perm])) <= 1e-13
    # permute (k, v) rows jointly inside sequence 1 (non-causal)
    p = np.arange(q.shape[0])
    p[12:42] = 12 + np.random.default_rng(1).permutation(30)
    out3, _ = A.jagged_forward(q, k[p], v[p], off, sc, False)
    assert np.max(np.abs(out3 - out)) <= 1e-13


def test_convex_hull():
    q, k, v, do, off, sc = case64([60, 3], 2, 16, seed=10)
    out, _ = A.jagged_forward(q, k, v, off, sc, False)
    for b in range(2):
        s, e = off[b], off[b + 1]
        assert np.all(out[s:e] <= v[s:e].max(axis=0) + 1e-14)
        assert np.all(out[s:e] >= v[s:e].min(axis=0) - 1e-14)


def test_long_sequence_row_blocks_match_single_block(monkeypatch):
    q, k, v, do, off, sc = case64([130], 1, 16, seed=11)
    ref = [A.jagged_forward(q, k, v, off, sc, c) for c in (False, True)]
    refb = [A.jagged_backward(q, k, v, do, off, sc, c) for c in (False, True)]
    monkeypatch.setattr(A, "ROW_BLOCK", 32)
    for c in (0, 1):
        o, l = A.jagged_forward(q, k, v, off, sc, bool(c))
        assert np.max(np.abs(o - ref[c][0])) <= 1e-13
        g = A.jagged_backward(q, k, v, do, off, sc, bool(c))
        for a, b in zip(g, refb[c]):
            assert np.max(np.abs(a - b)) <= 1e-13


# ------------------------------------------------------------------ backward
@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    q, k, v, do, off, sc = tiny_case(seed=12)
    _, rq, rk, rv = sdpa_packed(q, k, v, off, sc, causal, grad_do=do)
    dq, dk, dv = A.jagged_backward(q, k, v, do, off, sc, causal)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-10


def _loss(q, k, v, do, off, sc, causal):
    out, _ = A.jagged_forward(q, k, v, off, sc, causal)
    return float(np.sum(out * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences_exhaustive_micro(causal):
    rng = np.random.default_rng(13)
    L = [3, 1, 4]
    off = np.array([0, 3, 4, 8])
    q, k, v, do = (rng.standard_normal((8, 1, 4)) for _ in range(4))
    sc = 0.5
    g = A.jagged_backward(q, k, v, do, off, sc, causal)
    eps = 1e-6
    for ti, x in enumerate((q, k, v)):
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + eps
            fp = _loss(q, k, v, do, off, sc, causal)
            x[idx] = x0 - eps
            fm = _loss(q, k, v, do, off, sc, causal)
            x[idx] = x0
            fd = (fp - fm) / (2 * eps)
            assert abs(fd - g[ti][idx]) <= 1e-6 * max(1.0, abs(g[ti][idx])), (ti, idx)


def test_backward_finite_differences_sampled_tiny():
    q, k, v, do, off, sc = tiny_case(seed=14)
    g = A.jagged_backward(q, k, v, do, off, sc, False)
    rng = np.random.default_rng(15)
    eps = 1e-6
    seg = np.searchsorted(off, np.arange(q.shape[0]), side="right") - 1
    for ti, x in enumerate((q, k, v)):
        scale_ref = np.max(np.abs(g[ti]))
        for _ in range(200):
            t = int(rng.integers(q.shape[0])); h = int(rng.integers(x.shape[1]))
            d = int(rng.integers(x.shape[2]))
            b = seg[t]
            s, e = off[b], off[b + 1]
            sl = [y[s:e, h:h + 1].copy() for y in (q, k, v, do)]
            o1 = np.array([0, e - s])

            def f(delta):
                z = [y.copy() for y in sl[:3]]
                z[ti][t - s, 0, d] += delta
                return _loss(z[0], z[1], z[2], sl[3], o1, sc, False)

            fd = (f(eps) - f(-eps)) / (2 * eps)
            assert abs(fd - g[ti][t, h, d]) <= 1e-6 * max(1.0, scale_ref)


def test_backward_length_one_and_identical_keys():
    q, k, v, do, off, sc = case64([1, 20], 2, 16, seed=16)
    k[1:21] = k[1]
    dq, dk, dv = A.jagged_backward(q, k, v, do, off, sc, False)
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0)
    assert np.array_equal(dv[0], do[0])
    assert np.max(np.abs(dq[1:21])) <= 1e-13        # identical keys: dS rows sum to 0


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    q, k, v, do, off, sc = case64([70, 2, 33], 2, 32, seed=17)
    dq, dk, dv = A.jagged_backward(q, k, v, do, off, sc, causal)
    for b in range(3):
        s, e = off[b], off[b + 1]
        assert np.max(np.abs(dk[s:e].sum(axis=0))) <= 1e-12
        assert np.max(np.abs(dv[s:e].sum(axis=0) - do[s:e].sum(axis=0))) <= 1e-12


# ---------------------------------------------------------------- broadcast-Q
def test_broadcast_matches_torch_sdpa_and_autograd():
    L = [9, 40, 1, 17]
    Lq = 24
    q, k, v, do, off, sc = case64(L, 2, 16, seed=18, kind="broadcast", lq=Lq)
    out, lse = A.broadcast_forward(q, k, v, off, sc)
    dq, dk, dv = A.broadcast_backward(q, k, v, do, off, sc)
    tq = torch.from_numpy(q.transpose(1, 0, 2).copy()).requires_grad_()
    tk = torch.from_numpy(k.transpose(1, 0, 2).copy()).requires_grad_()
    tv = torch.from_numpy(v.transpose(1, 0, 2).copy()).requires_grad_()
    loss = 0
    for b in range(len(L)):
        s, e = off[b], off[b + 1]
        o = F.scaled_dot_product_attention(tq, tk[:, s:e], tv[:, s:e], scale=sc)
        assert np.max(np.abs(o.detach().numpy().transpose(1, 0, 2) - out[b])) <= 1e-12
        ref_lse = torch.logsumexp(sc * tq @ tk[:, s:e].transpose(1, 2), dim=-1)
        assert np.max(np.abs(ref_lse.detach().numpy() - lse[b])) <= 1e-12
        loss = loss + (o * torch.from_numpy(do[b].transpose(1, 0, 2).copy())).sum()
    loss.backward()
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(a - t.grad.numpy().transpose(1, 0, 2))) <= 1e-10


def test_broadcast_identical_copies():
    Lq, Lk, B = 16, 11, 5
    q, k, v, do, off, sc = case64([Lk], 2, 16, seed=19, kind="broadcast", lq=Lq)
    k5 = np.concatenate([k] * B)
    v5 = np.concatenate([v] * B)
    do5 = np.concatenate([do] * B)
    off5 = np.arange(B + 1) * Lk
    out1, _ = A.broadcast_forward(q, k, v, off, sc)
    out5, _ = A.broadcast_forward(q, k5, v5, off5, sc)
    dq1, _, _ = A.broadcast_backward(q, k, v, do, off, sc)
    dq5, _, _ = A.broadcast_backward(q, k5, v5, do5, off5, sc)
    for b in range(B):
        assert np.array_equal(out5[b], out1[0])
    assert np.max(np.abs(dq5 - B * dq1)) <= 1e-12


def test_broadcast_single_sequence_is_cross_attention():
    q, k, v, do, off, sc = case64([21], 1, 8, seed=20, kind="broadcast", lq=13)
    out, lse = A.broadcast_forward(q, k, v, off, sc)
    S = sc * q[:, 0] @ k[:, 0].T
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    assert np.max(np.abs(out[0, :, 0] - P @ v[:, 0])) <= 1e-13


def test_broadcast_empty_sequence_convention():
    q, k, v, do, off, sc = case64([0, 5], 1, 8, seed=21, kind="broadcast", lq=4)
    out, lse = A.broadcast_forward(q, k, v, off, sc)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    dq, dk, dv = A.broadcast_backward(q, k, v, do, off, sc)
    dq1, _, _ = A.broadcast_backward(q, k, v, do[1:], np.array([0, 5]), sc)
    assert np.array_equal(dq, dq1)


# -------------------------------------------------------------- block-diagonal
def test_block_diag_matches_masked_sdpa():
    L = [64, 192, 128]
    q, k, v, do, off, sc = case64(L, 2, 16, seed=22)
    out = A.block_diag_forward(q, k, v, off, sc)
    ref, rq, rk, rv = sdpa_packed(q, k, v, off, sc, False, grad_do=do, block=64)
    assert np.max(np.abs(out - ref)) <= 1e-12
    dq, dk, dv = A.block_diag_backward(q, k, v, do, off, sc)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-10


@pytest.mark.parametrize("bs", [32, 128, 256])
def test_other_block_sizes_match_masked_sdpa(bs):
    L = [bs, 3 * bs, 0, 2 * bs]
    q, k, v, do, off, sc = case64(L, 2, 16, seed=23)
    out = A.block_diag_forward(q, k, v, off, sc, block=bs)
    ref, rq, rk, rv = sdpa_packed(q, k, v, off, sc, False, grad_do=do, block=bs)
    assert np.max(np.abs(out - ref)) <= 1e-12
    dq, dk, dv = A.block_diag_backward(q, k, v, do, off, sc, block=bs)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) <= 1e-10


def test_block_diag_rejects_partial_blocks():
    with pytest.raises(ValueError):
        A.refine_offsets(np.array([0, 64, 100]))


def test_pair_count_brute_force():
    L = [5, 1, 0, 9]
    assert A.pair_count(L) == sum(sum(1 for i in range(n) for j in range(n)) for n in L)
    assert A.pair_count(L, causal=True) == sum(sum(1 for i in range(n) for j in range(i + 1))
                                               for n in L)
    assert A.pair_count(L, lq=7) == 7 * sum(L)
    assert A.pair_count([64, 128], block=64) == 64 * 64 + 2 * 64 * 64


def test_block_attention_arithmetic_intensity():
    # The block-attention page gives an intensity of about 33 FLOP per byte for
    # 64-token blocks at head dim 128 (roofline context); counting 4*64*64*128
    # FLOPs over Q, K, V and out (64x128 bf16 each) gives exactly 32.
    flops = 4 * A.pair_count([64], block=64) * 128
    bytes_ = 4 * 64 * 128 * 2
    assert flops / bytes_ == 32.0
    assert abs(flops / bytes_ - 33) / 33 < 0.05
