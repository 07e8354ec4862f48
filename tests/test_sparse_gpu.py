"""GPU parity of block-sparse attention (64-token blocks) through the C ABI.

Small cases compare every element of out, lse, dQ, dK and dV with the fp64
oracle: ragged lengths (1-token and empty sequences, partial last blocks,
sequences of several query and key tiles), D = 64 and 128, masks from empty to
full, query blocks that attend nothing (out 0, lse -inf, dQ 0) and key blocks
that nobody attends (dK = dV = 0), each with and without causal masking.
Identities: an all-ones mask gives the plain kernels' results bit for bit, causal
or not (the same steps in the same order); a diagonal mask gives the
block-diagonal mode's results within rounding. The benchmark's batches (B = 1152,
L ~ U{1..4096}, density 0.3, D = 128 and 64, and D = 128 causal), in their launch
configuration, are compared element by element in full against the oracle run
by the worker pool."""
import numpy as np
import pytest

import jfa_inputs as J
from tests.gpu_common import (GRAD_TOL, LSE_TOL, OUT_TOL, GpuRun, bf16_to_f64, log, max_abs,
                              out_excess, out_rel, oracle_full)

pytestmark = pytest.mark.gpu


def _check(case, res, gpu_out):
    out, lse, dq, dk, dv = res
    g_out, g_lse, g_dq, g_dk, g_dv = gpu_out
    o = bf16_to_f64(g_out)
    e_out = out_excess(o, out, out_rel(case.w))
    fin = np.isfinite(lse)
    gl = g_lse.cpu().numpy()
    assert np.array_equal(np.isfinite(gl), fin), "rows without keys must get lse -inf"
    e_lse = max_abs(gl[fin], lse[fin]) if fin.any() else 0.0
    errs = {"out": e_out, "lse": e_lse}
    for nm, g, r in (("dq", g_dq, dq), ("dk", g_dk, dk), ("dv", g_dv, dv)):
        m = float(np.abs(r).max()) if r.size else 0.0
        errs[nm] = max_abs(bf16_to_f64(g), r) / m if m > 0 else max_abs(bf16_to_f64(g), r)
    log("  " + " ".join(f"{k} {v:.3e}" for k, v in errs.items()))
    assert errs["out"] <= OUT_TOL and errs["lse"] <= LSE_TOL
    for nm in ("dq", "dk", "dv"):
        assert errs[nm] <= GRAD_TOL, nm
    # rows without keys: exactly zero out and dQ
    dead = ~fin.any(axis=0) if fin.ndim == 2 else ~fin
    if dead.any():
        assert np.all(o[dead] == 0) and np.all(bf16_to_f64(g_dq)[dead] == 0)


def _run(case, gpu):
    run = GpuRun(case, gpu)
    out, lse = run.forward()
    dq, dk, dv = run.backward()
    return out, lse, dq, dk, dv


def _case_with_mask(lengths, D, seed, mask_fn, causal=False):
    w = J.custom(lengths, 2, D, sigma=1.0, seed=seed, kind="sparse", density=0.3,
                 causal=causal)
    c = J.make_case(w)
    parts, pos = [], 0
    for b, n in enumerate(c.lengths):
        nb = -(-int(n) // 64)
        parts.append(mask_fn(b, nb).astype(np.uint8).ravel())
    c.mask = np.concatenate(parts) if parts else np.zeros(0, np.uint8)
    return c


LENGTHS = [1, 0, 64, 65, 130, 200, 333, 511]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
def test_random_masks(gpu, D, density, causal):
    rng = np.random.default_rng(int(density * 10) + D)
    case = _case_with_mask(LENGTHS, D, 5, lambda b, n: rng.random((n, n)) < density, causal)
    log(f"sparse D={D} density={density} causal={causal}: lengths {LENGTHS}")
    _check(case, oracle_full(case), _run(case, gpu))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_empty_rows_and_columns(gpu, D, causal):
    """Query blocks with no key (out 0, lse -inf, dQ 0) and key blocks nobody
    attends (dK = dV = 0), on top of a random pattern."""
    rng = np.random.default_rng(9)

    def mask(b, n):
        m = rng.random((n, n)) < 0.5
        if n >= 3:
            m[1, :] = False      # query block 1 attends nothing
            m[:, n - 1] = False  # the last key block is attended by nobody
        return m
    case = _case_with_mask([130, 300, 64, 511], D, 6, mask, causal)
    res = oracle_full(case)
    g = _run(case, gpu)
    _check(case, res, g)
    off = case.offsets.astype(np.int64)
    dk, dv = bf16_to_f64(g[3]), bf16_to_f64(g[4])
    for b, n in enumerate(case.lengths):
        nb = -(-int(n) // 64)
        if nb >= 3:
            s = int(off[b]) + 64 * (nb - 1)
            assert np.all(dk[s:int(off[b + 1])] == 0) and np.all(dv[s:int(off[b + 1])] == 0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_lists_longer_than_64_blocks(gpu, D, causal):
    """Sequences of more than 64 blocks (4096 tokens), dense enough that a tile's
    list holds more than 64 entries: the kernels read a tile's entries 64 at a
    time."""
    rng = np.random.default_rng(31)
    L = [4500, 70, 4353]
    case = _case_with_mask(L, D, 11, lambda b, n: rng.random((n, n)) < 0.8, causal)
    log(f"sparse long lists D={D} causal={causal}: lengths {L}")
    _check(case, oracle_full(case), _run(case, gpu))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_slot_counts_do_not_change_results(gpu, D, causal):
    """One workgroup walking every tile in turn (each tile's first loads issued
    behind the previous tile's stores, the two wave pairs of a tile walking lists
    of different lengths) and far more workgroups than tiles give the bits of the
    default slot count."""
    import torch
    rng = np.random.default_rng(41 + D)
    case = _case_with_mask(LENGTHS + [700, 3], D, 12, lambda b, n: rng.random((n, n)) < 0.4,
                           causal)
    a = GpuRun(case, gpu)
    oa, la = a.forward()
    ga = [x.clone() for x in a.backward()]
    for slots in (1, 2048):
        log(f"sparse D={D} causal={causal} slots={slots}")
        b = GpuRun(case, gpu, num_slots=slots)
        ob, lb = b.forward()
        assert torch.equal(oa, ob) and torch.equal(la, lb)
        for x, y in zip(ga, b.backward()):
            assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_orders_do_not_change_results(gpu, causal):
    """Every dealing order gives the bits of the default (balanced in-order)
    order: a tile's results do not depend on its slot or on the tiles before it."""
    import torch
    import variable_length_flash_jaggedfa_amd as jfa
    rng = np.random.default_rng(61)
    case = _case_with_mask(LENGTHS + [900, 5], 128, 13, lambda b, n: rng.random((n, n)) < 0.35,
                           causal)
    a = GpuRun(case, gpu)
    assert a.plan.order == jfa.ORDER_XCD_INORDER
    oa, la = a.forward()
    ga = [x.clone() for x in a.backward()]
    for order in (jfa.ORDER_INORDER, jfa.ORDER_ZIGZAG, jfa.ORDER_XCD_ZIGZAG,
                  jfa.ORDER_FOLDED_ZIGZAG):
        log(f"sparse causal={causal} order={order}")
        b = GpuRun(case, gpu, order=order)
        ob, lb = b.forward()
        assert torch.equal(oa, ob) and torch.equal(la, lb)
        for x, y in zip(ga, b.backward()):
            assert torch.equal(x, y)


def test_validate_checks_the_step_lists(gpu, monkeypatch):
    """With JFA_VALIDATE=1 valid lists give the same bits; lists corrupted on the
    device (a list pointer past its successor, an entry naming a block past its
    sequence, a wrong first unit) are refused before any launch, forward and
    backward."""
    import torch
    import variable_length_flash_jaggedfa_amd as jfa
    rng = np.random.default_rng(71)
    case = _case_with_mask([130, 300, 64, 511], 64, 14, lambda b, n: rng.random((n, n)) < 0.5)
    run = GpuRun(case, gpu)
    out, lse = run.forward()
    grads = [x.clone() for x in run.backward()]
    monkeypatch.setenv("JFA_VALIDATE", "1")
    out2, lse2 = run.plan.forward(run.q, run.k, run.v)
    grads2 = run.plan.backward(run.q, run.k, run.v, out2, run.do, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for a_, b_ in zip(grads, grads2):
        assert torch.equal(a_, b_)
    for kind in (jfa.KIND_FWD, jfa.KIND_BWD):
        sch = run.plan.sched[kind]
        good = sch.lists_dev
        sb, lp, ent = (t.clone() for t in good)
        bad_lp = lp.clone()
        bad_lp[1] = int(lp[2]) + 1
        bad_ent = ent.clone()
        bad_ent[0] = (int(ent[0]) & ~((1 << 28) - 1)) | 9  # block 9 of a 130-token sequence
        bad_sb = sb.clone()
        bad_sb[1] += 1
        for lists in ((sb, bad_lp, ent), (sb, lp, bad_ent), (bad_sb, lp, ent)):
            sch.lists_dev = lists
            try:
                with pytest.raises(jfa.JfaError) as e:
                    if kind == jfa.KIND_FWD:
                        run.plan.forward(run.q, run.k, run.v, out=out2, lse=lse2)
                    else:
                        run.plan.backward(run.q, run.k, run.v, out2, run.do, lse2)
                assert e.value.status == jfa.ERR_INVALID_ARG and "step lists" in str(e.value)
            finally:
                sch.lists_dev = good
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # the refused calls wrote nothing


@pytest.mark.parametrize("lengths", [[0, 0, 0], []], ids=["all-empty", "no-sequences"])
def test_empty_batches(gpu, lengths):
    """A batch of empty sequences and a batch of none: forward and backward run
    (causal or not) and return empty outputs."""
    for causal in (False, True):
        case = _case_with_mask(lengths, 128, 3, lambda b, n: np.ones((n, n), bool), causal)
        out, lse, dq, dk, dv = _run(case, gpu)
        for t in (out, dq, dk, dv):
            assert tuple(t.shape) == (0, 2, 128)
        assert lse.numel() == 0


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_is_the_plain_kernels_bitwise(gpu, causal):
    import torch
    case = _case_with_mask(LENGTHS, 128, 7, lambda b, n: np.ones((n, n), bool), causal)
    gs = _run(case, gpu)
    plain = J.custom(LENGTHS, 2, 128, sigma=1.0, seed=7, causal=causal)
    cp = J.make_case(plain)
    assert np.array_equal(cp.q, case.q) and np.array_equal(cp.do, case.do)
    gp = _run(cp, gpu)
    for nm, a, b in zip(("out", "lse", "dq", "dk", "dv"), gs, gp):
        assert torch.equal(a, b), nm


def test_diagonal_mask_is_block_diagonal(gpu):
    import torch
    L = [64, 192, 128, 512]
    case = _case_with_mask(L, 64, 8, lambda b, n: np.eye(n, dtype=bool))
    gs = _run(case, gpu)
    blk = J.make_case(J.custom(L, 2, 64, sigma=1.0, seed=8, kind="block"))
    gb = _run(blk, gpu)
    for nm, i in (("out", 0), ("dq", 2), ("dk", 3), ("dv", 4)):
        a, b = bf16_to_f64(gs[i]), bf16_to_f64(gb[i])
        m = float(np.abs(b).max())
        log(f"  {nm}: sparse vs block-diagonal {max_abs(a, b) / m:.3e}")
        assert max_abs(a, b) <= (OUT_TOL if nm == "out" else GRAD_TOL * m)


@pytest.mark.parametrize("name", ["sparse_d128", "sparse_d64", "sparse_d128_causal"])
def test_every_element_benchmark_batch(gpu, oracle_pool, result_dir, name):
    """Every element of out, lse, dQ, dK and dV of the benchmark's batch."""
    from tests.test_parity_full_gpu import _bits
    from oracle import pool as OP
    import os
    import time
    w = J.standard_workloads()[name]
    case = J.make_case(w)
    log(f"{name} every element: B={w.num_seqs} T={int(case.offsets[-1])}")
    out, lse, dq, dk, dv = _run(case, gpu)
    rdir = result_dir
    for nm, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.save(os.path.join(rdir, nm + ".npy"), _bits(t))
    np.save(os.path.join(rdir, "lse.npy"), lse.cpu().numpy())
    del out, lse, dq, dk, dv
    t0 = time.perf_counter()
    r = OP.compare(oracle_pool, w, case.scale, case.offsets, rdir, out_rel=out_rel(w))
    log(f"  oracle over {r['tasks']} tasks: {time.perf_counter() - t0:.0f} s wall, "
        f"{r['cpu_seconds']:.0f} s CPU; out {r['out']:.3e} lse {r['lse']:.3e} " +
        " ".join(f"{k} {r[k] / max(r[k + '_ref'], 1e-30):.3e}" for k in ("dq", "dk", "dv")))
    assert r["finite"] and r["lse_inf_match"]
    assert r["out"] <= OUT_TOL and r["lse"] <= LSE_TOL
    for k in ("dq", "dk", "dv"):
        assert r[k] <= GRAD_TOL * r[k + "_ref"], k
