"""Plant plausible mistakes in the oracle (CPU only) and check that the pins in
test_oracle.py catch every one of them: a dropped term, a wrong sign or index, a
wrong operand."""
import numpy as np
import pytest

from oracle import attention as A
from tests import test_oracle as T


def _mut_probs_causal_off_by_one(q_blk, k, scale, causal, r0, window=0, bmask=None):
    s = scale * (q_blk @ k.T)
    if causal:
        i = np.arange(r0, r0 + q_blk.shape[0])[:, None]
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j < i, s, -np.inf)
        s[:, 0] = np.where(np.isneginf(s[:, 0]), scale * (q_blk @ k[0]), s[:, 0])
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def _mut_probs_no_scale(q_blk, k, scale, causal, r0, window=0, bmask=None):
    return _orig_probs(q_blk, k, 1.0, causal, r0, window, bmask)


def _mut_forward_lse_without_log(q, k, v, scale, causal=False, window=0, bmask=None):
    out, lse = _orig_seq_forward(q, k, v, scale, causal, window, bmask)
    # drop the log-sum term: lse = m only
    for r0, r1 in A._row_blocks(q.shape[0]):
        if k.shape[0]:
            _, m, _ = A._probs(q[r0:r1], k, scale, causal, r0)
            lse[r0:r1] = m
    return out, lse


def _make_bwd_mutant(kind):
    def bwd(q, k, v, do, scale, causal=False, window=0, bmask=None):
        dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
        if q.shape[0] == 0 or k.shape[0] == 0:
            return dq, dk, dv
        for r0, r1 in A._row_blocks(q.shape[0]):
            p, _, _ = A._probs(q[r0:r1], k, scale, causal, r0)
            o = p @ v
            d_o = do[r0:r1]
            di = np.sum(d_o * o, axis=1)
            dv += p.T @ d_o
            dp = d_o @ v.T
            ds = p * dp if kind == "no_di" else p * (dp - di[:, None])
            if kind == "sign_di":
                ds = p * (dp + di[:, None])
            dq[r0:r1] = (ds @ k) if kind == "no_scale_dq" else scale * (ds @ k)
            if kind == "dk_wrong_operand":
                dk += scale * (ds.T @ d_o)
            elif kind == "dk_transposed_p":
                dk += scale * (p.T @ q[r0:r1])
            else:
                dk += scale * (ds.T @ q[r0:r1])
        return dq, dk, dv
    return bwd


_orig_probs = A._probs
_orig_seq_forward = A.seq_forward


def _caught(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except AssertionError:
        return True
    return False


def test_causal_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(A, "_probs", _mut_probs_causal_off_by_one)
    assert _caught(T.test_forward_matches_torch_sdpa, causal=True)


def test_missing_scale_is_caught(monkeypatch):
    monkeypatch.setattr(A, "_probs", _mut_probs_no_scale)
    assert _caught(T.test_forward_matches_torch_sdpa, causal=False)
    assert _caught(T.test_length_one_returns_v)


def test_lse_without_log_is_caught(monkeypatch):
    monkeypatch.setattr(A, "seq_forward", _mut_forward_lse_without_log)
    assert _caught(T.test_forward_matches_padded_dense, causal=False)
    assert _caught(T.test_identical_keys_give_mean_of_v, causal=False)


@pytest.mark.parametrize("kind", ["no_di", "sign_di", "no_scale_dq", "dk_wrong_operand",
                                  "dk_transposed_p"])
def test_backward_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(A, "seq_backward", _make_bwd_mutant(kind))
    assert _caught(T.test_backward_matches_torch_autograd, causal=False)
    assert _caught(T.test_backward_finite_differences_exhaustive_micro, causal=True)


# ------------------------------------------------------------------ rotary
from oracle import rotary as R  # noqa: E402
from tests import test_oracle_rotary as TR  # noqa: E402

_orig_rope = R.rope


def _mut_rope(kind):
    def rope(x, positions, base, inverse=False):
        d = x.shape[-1]
        if kind == "sin_sign":
            return _orig_rope(x, positions, base, inverse=not inverse)
        if kind == "interleaved":
            perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
            y = _orig_rope(x[..., perm], positions, base, inverse)
            out = np.empty_like(y)
            out[..., perm] = y
            return out
        if kind == "freq_exponent":
            return _orig_rope(x, np.asarray(positions, dtype=np.float64), base ** 0.5, inverse)
        if kind == "no_inverse":
            return _orig_rope(x, positions, base, False)
        raise ValueError(kind)
    return rope


@pytest.mark.parametrize("kind", ["sin_sign", "interleaved", "freq_exponent", "no_inverse"])
def test_rotary_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(R, "rope", _mut_rope(kind))
    # every mutant fails the autograd comparison; the forward-only mutants also
    # fail the worked value or the complex form, the backward one the finite
    # differences
    assert _caught(TR.test_block_rope_matches_torch_autograd, D=64)
    if kind == "no_inverse":
        assert _caught(TR.test_block_rope_finite_differences)
    else:
        assert _caught(TR.test_worked_rotation) or _caught(TR.test_matches_complex_form, D=64)


def test_rotary_backward_without_inverse_rotation_is_caught(monkeypatch):
    def bwd(q, k, v, do, offsets, scale, base, block=64):
        pos = R.token_positions(offsets)
        return R.block_diag_backward(R.rope(q, pos, base), R.rope(k, pos, base), v, do, offsets,
                                     scale, block)
    monkeypatch.setattr(R, "block_diag_rope_backward", bwd)
    assert _caught(TR.test_block_rope_matches_torch_autograd, D=64)
    assert _caught(TR.test_block_rope_finite_differences)


# ------------------------------------------------------------------ window
from tests import test_oracle_window as TW  # noqa: E402


def _mut_probs_window_off_by_one(q_blk, k, scale, causal, r0, window=0, bmask=None):
    s = scale * (q_blk @ k.T)
    if causal:
        i = np.arange(r0, r0 + q_blk.shape[0])[:, None]
        j = np.arange(k.shape[0])[None, :]
        keep = j <= i
        if window:
            keep &= j >= i - window
        s = np.where(keep, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def test_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(A, "_probs", _mut_probs_window_off_by_one)
    assert _caught(TW.test_window_closed_forms)
    assert _caught(TW.test_window_matches_torch_sdpa_and_autograd, W=5)
    assert _caught(TW.test_window_matches_loops)


def test_window_work_mistake_is_caught(monkeypatch):
    orig = TW.S.enumerate_tiles

    def mutated(*a, **kw):
        # query tiles credited with the whole causal prefix despite the window
        kw = dict(kw, window=0) if a[2] == TW.S.KIND_FWD else kw
        return orig(*a, **kw)
    monkeypatch.setattr(TW.S, "enumerate_tiles", mutated)
    assert _caught(TW.test_window_tile_work_brute_force, W=100)


# ------------------------------------------------------------------ block-sparse
from tests import test_oracle_sparse as TS  # noqa: E402


def _mut_probs_sparse(kind):
    def probs(q_blk, k, scale, causal, r0, window=0, bmask=None):
        if bmask is not None:
            if kind == "transposed":
                bmask = bmask.T
            elif kind == "block_off_by_one":
                # a query takes the block of the next row (i + 1) // 64
                n = q_blk.shape[0]
                out = [_orig_probs(q_blk[r:r + 1], k, scale, causal, r0 + r + 1, window, bmask)
                       if (r0 + r + 1) // 64 < bmask.shape[0] else
                       _orig_probs(q_blk[r:r + 1], k, scale, causal, r0 + r, window, bmask)
                       for r in range(n)]
                return (np.concatenate([o[0] for o in out]), np.concatenate([o[1] for o in out]),
                        np.concatenate([o[2] for o in out]))
        return _orig_probs(q_blk, k, scale, causal, r0, window, bmask)
    return probs


@pytest.mark.parametrize("kind", ["transposed", "block_off_by_one"])
def test_sparse_mask_mutants_are_caught(monkeypatch, kind):
    monkeypatch.setattr(A, "_probs", _mut_probs_sparse(kind))
    assert _caught(TS.test_sparse_matches_sdpa, seed=0)
    assert _caught(TS.test_matches_python_loops)
