"""The allocation-free backward (jfa_bwd_noalloc, the library's static scratch
array as workspace) against the backward with a caller-allocated workspace
(jfa_bwd), through the C ABI, on two calls in a row: a larger problem, then a
smaller one that reuses the scratch array left by the first. Each is also held to
the oracle's tolerances against the fp64 oracle."""
import numpy as np
import pytest

import jfa_inputs as J
import variable_length_flash_jaggedfa_amd as jfa
from tests.gpu_common import (GpuRun, assert_grad, bf16_to_f64, log, oracle_full, rel_err,
                              GRAD_TOL)

pytestmark = pytest.mark.gpu


def _compare(w, dev):
    log(f"noalloc case {w.name} kind={w.kind} causal={w.causal} H={w.num_heads} "
        f"D={w.head_dim} lq={w.lq} lengths={J.lengths(w)[:10].tolist()}")
    import torch
    case = J.make_case(w)
    run = GpuRun(case, dev)
    need = jfa.bwd_workspace_bytes(run.plan.p)
    assert 0 < need <= jfa.NOALLOC_SCRATCH_BYTES, need
    out, lse = run.forward()
    dq, dk, dv = run.backward()  # jfa_bwd with the plan's workspace
    dq2, dk2, dv2 = (torch.full_like(t, float("nan")) for t in (dq, dk, dv))
    run.plan.backward_noalloc(run.q, run.k, run.v, out, run.do, lse, dq2, dk2, dv2)
    torch.cuda.synchronize()
    ref = oracle_full(case)
    for name, a, b, r in (("dq", dq, dq2, ref[2]), ("dk", dk, dk2, ref[3]),
                          ("dv", dv, dv2, ref[4])):
        ga, gb = bf16_to_f64(a), bf16_to_f64(b)
        assert np.all(np.isfinite(gb)), name
        # the same kernels on the same inputs: to the oracle's bar against jfa_bwd,
        # and in fact bit for bit
        e = rel_err(gb, ga)
        log(f"  {name}: noalloc vs jfa_bwd max err / max|ref| {e:.3e}")
        assert e <= GRAD_TOL
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        assert_grad(gb, r, name)


def test_noalloc_matches_bwd_twice_smaller_second(gpu):
    # first call: a larger jagged problem (several tiles, ragged tails, causal)
    _compare(J.custom([700, 1, 129, 0, 513, 64, 300], 4, 128, sigma=0.5, seed=21, causal=True), gpu)
    # second call, smaller, on the scratch array the first left behind
    _compare(J.custom([90, 3, 200], 2, 64, sigma=0.5, seed=22), gpu)


def test_noalloc_broadcast_then_jagged(gpu):
    _compare(J.custom([50, 0, 300, 1, 129], 2, 128, sigma=0.5, seed=23, kind="broadcast", lq=200),
             gpu)
    _compare(J.custom([40, 7], 1, 64, sigma=0.5, seed=24, causal=True), gpu)


def test_noalloc_rejects_oversized_problem(gpu):
    # H * T * 4 bytes twice (-Di, -lse/scale) beyond the scratch array: refused
    # before anything runs
    T = 5 << 20
    p = jfa.problem(1, 1, 128, T, T, 0.088)
    assert jfa.bwd_workspace_bytes(p) > jfa.NOALLOC_SCRATCH_BYTES
    with pytest.raises(jfa.JfaError) as e:
        jfa.bwd_noalloc(p, None, None, None, None, None, None, None, None, None, 0, None, None, 0,
                        None, None, None)
    assert e.value.status == jfa.ERR_WORKSPACE
