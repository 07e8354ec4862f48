"""Plant plausible mistakes in the oracle (CPU only) and check that the pins in
test_oracle.py catch every one of them: a dropped term, a wrong sign or index, a
wrong operand."""
import numpy as np
import pytest

from oracle import attention as A
from tests import test_oracle as T


def _mut_probs_causal_off_by_one(q_blk, k, scale, causal, r0):
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


def _mut_probs_no_scale(q_blk, k, scale, causal, r0):
    return _orig_probs(q_blk, k, 1.0, causal, r0)


def _mut_forward_lse_without_log(q, k, v, scale, causal=False):
    out, lse = _orig_seq_forward(q, k, v, scale, causal)
    # drop the log-sum term: lse = m only
    for r0, r1 in A._row_blocks(q.shape[0]):
        if k.shape[0]:
            _, m, _ = A._probs(q[r0:r1], k, scale, causal, r0)
            lse[r0:r1] = m
    return out, lse


def _make_bwd_mutant(kind):
    def bwd(q, k, v, do, scale, causal=False):
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
