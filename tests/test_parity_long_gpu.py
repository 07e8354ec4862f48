"""GPU parity on sequences whose rows span more than 4 GiB.

The kernels load tiles through buffer resources with 32-bit sizes. A tile of one
head is addressed from its first row; the rows from there to the end of a long
sequence may span more than 2^32 bytes (here one sequence of 2^20 + 1000 tokens
at H = 16, D = 128: about 4.3 GB per tensor), and must not wrap the size. The
sliding-window case runs the jagged forward, dQ and dK/dV kernels over the whole
sequence; the broadcast-Q case streams the same long K/V sequence past a dense Q.
Inputs are seeded normal values drawn on the GPU (torch's generator); the slices
the oracle needs are copied to the host, and the oracle (fp64) recomputes sampled
rows near the start, the middle and the end of the sequence, and around key
LONG - 1 - 2^20 = 999: a step of keys starting there is the one whose resource
size, taken over the rest of the sequence, crosses 2^32 bytes (rows from 999 on
would read as zeros if it wrapped). In the broadcast case the keys around it are
made to hold a large share of every query's softmax, so that a key lost there
would change out, lse and the gradients by far more than the tolerances.
"""
import numpy as np
import pytest

import variable_length_flash_jaggedfa_amd as jfa
from oracle import attention as A
from tests.gpu_common import GRAD_TOL, LSE_TOL, OUT_TOL, bf16_to_f64, log, max_abs

pytestmark = pytest.mark.gpu

H, D = 16, 128
LONG = (1 << 20) + 1000
SCALE = float(np.float32(1.0) / np.sqrt(np.float32(D)))


def _randn(shape, seed, dev):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * 0.5).to(
        torch.bfloat16)


def _rel(got, ref):
    m = float(np.abs(ref).max())
    return max_abs(got, ref) / m if m > 0 else max_abs(got, ref)


def test_long_sequence_sliding_window(gpu):
    """Causal window of 256 keys over a 2^20 + 1000 token sequence (after a short
    one, so the long sequence starts at a non-zero row)."""
    import torch
    W = 256
    lengths = [37, LONG]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(off[-1])
    assert (LONG - 1) * H * D * 2 >= 1 << 32
    log(f"long window case: T={T} H={H} D={D} W={W}")
    q, k, v, do = (_randn((T, H, D), s, gpu) for s in (101, 102, 103, 104))
    plan = jfa.Plan(off, H, D, SCALE, jfa.CAUSAL, window=W, device=gpu)
    out, lse = plan.forward(q, k, v)
    dq, dk, dv = plan.backward(q, k, v, out, do, lse)
    torch.cuda.synchronize()
    s0 = int(off[1])
    n = 200
    worst = {"out": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    for r0 in (0, 900, LONG // 2, LONG - n):
        for h in (0, H - 1):
            # rows [r0, r0+n) of the long sequence need keys from r0 - W + 1; their
            # keys' gradients need queries up to r0 + n + W - 2
            a, e = max(0, r0 - W + 1), min(LONG, r0 + n + W - 1)
            sl = slice(s0 + a, s0 + e)
            q_, k_, v_, do_ = (bf16_to_f64(x[sl, h]) for x in (q, k, v, do))
            o_ref, l_ref = A.seq_forward(q_, k_, v_, SCALE, True, W)
            g_ref = A.seq_backward(q_, k_, v_, do_, SCALE, True, W)
            rows = slice(r0 - a, r0 - a + n)
            got = slice(s0 + r0, s0 + r0 + n)
            worst["out"] = max(worst["out"], max_abs(bf16_to_f64(out[got, h]), o_ref[rows]))
            worst["lse"] = max(worst["lse"], max_abs(lse[h, got].cpu().numpy(), l_ref[rows]))
            for name, t, r in (("dq", dq, g_ref[0]), ("dk", dk, g_ref[1]), ("dv", dv, g_ref[2])):
                worst[name] = max(worst[name], _rel(bf16_to_f64(t[got, h]), r[rows]))
    log("  " + " ".join(f"{k} {v:.3e}" for k, v in worst.items()))
    assert worst["out"] <= OUT_TOL and worst["lse"] <= LSE_TOL
    for name in ("dq", "dk", "dv"):
        assert worst[name] <= GRAD_TOL, name


def test_long_sequence_broadcast(gpu):
    """A dense Q of 64 rows against a short and a 2^20 + 1000 token K/V sequence:
    every query row of the long sequence against the oracle for one head, its
    keys' gradients near the start and the end, and dQ summed over both."""
    import torch
    lq = 64
    lengths = [5, LONG]
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(off[-1])
    log(f"long broadcast case: T={T} H={H} D={D} lq={lq}")
    k, v = (_randn((T, H, D), s, gpu) for s in (111, 112))
    q = _randn((lq, H, D), 113, gpu)
    # keys 950..1049 of the long sequence become 4 x the query rows (cycling): each
    # query's own one or two keys there score about 4 |q|^2 scale = 9..13.5 above
    # the rest and hold up to about half of its softmax over the million keys (not
    # all of it: with P near one, dS = P (dP - Di) cancels, and the rounding of the
    # bf16 out inside Di would swamp it)
    hot = slice(int(off[1]) + 950, int(off[1]) + 1050)
    k[hot] = (q[torch.arange(100, device=gpu) % lq].float() * 4.0).to(torch.bfloat16)
    do = _randn((2, lq, H, D), 114, gpu)
    plan = jfa.Plan(off, H, D, SCALE, jfa.BROADCAST_Q, lq=lq, device=gpu)
    out, lse = plan.forward(q, k, v)
    dq, dk, dv = plan.backward(q, k, v, out, do, lse)
    torch.cuda.synchronize()
    h = H - 1
    q_ = bf16_to_f64(q[:, h])
    dq_ref = np.zeros_like(q_)
    errs = {}
    for b in (0, 1):
        sl = slice(int(off[b]), int(off[b + 1]))
        k_, v_ = bf16_to_f64(k[sl, h]), bf16_to_f64(v[sl, h])
        do_ = bf16_to_f64(do[b, :, h])
        o_ref, l_ref = A.seq_forward(q_, k_, v_, SCALE)
        g_ref = A.seq_backward(q_, k_, v_, do_, SCALE)
        dq_ref += g_ref[0]
        errs[f"out{b}"] = max_abs(bf16_to_f64(out[b, :, h]), o_ref)
        errs[f"lse{b}"] = max_abs(lse[b, h].cpu().numpy(), l_ref)
        L = lengths[b]
        for name, t, r in (("dk", dk, g_ref[1]), ("dv", dv, g_ref[2])):
            for r0 in sorted({0, min(900, max(0, L - 300)), max(0, L - 300)}):
                rows = slice(r0, min(L, r0 + 300))
                got = t[int(off[b]) + rows.start:int(off[b]) + rows.stop, h]
                errs[f"{name}{b}@{r0}"] = _rel(bf16_to_f64(got), r[rows])
        del k_, v_, g_ref
    errs["dq"] = _rel(bf16_to_f64(dq[:, h]), dq_ref)
    log("  " + " ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    for key, e in errs.items():
        tol = OUT_TOL if key.startswith("out") else LSE_TOL if key.startswith("lse") else GRAD_TOL
        assert e <= tol, (key, e)
