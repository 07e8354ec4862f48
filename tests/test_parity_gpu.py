"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element
by element, on small seeded cases that span several tiles and ragged tails, plus
the edge cases (empty and length-1 sequences, one sequence, lengths at tile
boundaries, broadcast-Q with empty K/V, identical K/V copies)."""
import numpy as np
import pytest

import jfa_inputs as J
import variable_length_flash_jaggedfa_amd as jfa
from oracle import attention as A
from tests.gpu_common import (GpuRun, assert_grad, assert_lse, assert_out, bf16_to_f64, log,
                              lse_tol, oracle_full, out_rel)

pytestmark = pytest.mark.gpu


def check_case(w, dev, order=jfa.ORDER_FOLDED_ZIGZAG, num_slots=None, bwd=True):
    log(f"case {w.name} kind={w.kind} causal={w.causal} H={w.num_heads} D={w.head_dim} "
        f"lq={w.lq} seed={w.seed} lengths={J.lengths(w)[:12].tolist()}")
    case = J.make_case(w)
    run = GpuRun(case, dev, order=order, num_slots=num_slots)
    out, lse = run.forward()
    ref = oracle_full(case)
    assert_out(bf16_to_f64(out), ref[0], rel=out_rel(w))
    if lse is not None:
        assert_lse(lse.cpu().numpy().astype(np.float64), ref[1], lse_tol(w, case))
    if bwd:
        dq, dk, dv = run.backward()
        for name, g, r in (("dq", dq, ref[2]), ("dk", dk, ref[3]), ("dv", dv, ref[4])):
            assert_grad(bf16_to_f64(g), r, name)
    return run


def test_tiny_workload(gpu):
    check_case(J.standard_workloads()["tiny"], gpu)


def test_tiny_workload_causal(gpu):
    check_case(J.standard_workloads()["tiny"].with_(causal=True), gpu)


RAGGED = [300, 1, 129, 64, 0, 257, 17, 128, 2]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_jagged_ragged(gpu, D, causal):
    check_case(J.custom(RAGGED, 3, D, sigma=0.5, seed=5, causal=causal), gpu)


@pytest.mark.parametrize("D", [64, 128])
def test_broadcast_ragged(gpu, D):
    check_case(J.custom([50, 0, 300, 1, 129, 64], 2, D, sigma=0.5, seed=6, kind="broadcast",
                        lq=200), gpu)


def test_broadcast_all_empty(gpu):
    check_case(J.custom([0, 0], 2, 64, seed=7, kind="broadcast", lq=70), gpu)


def test_broadcast_identical_copies(gpu):
    import torch
    w = J.custom([77], 2, 128, sigma=0.5, seed=8, kind="broadcast", lq=130)
    case1 = J.make_case(w)
    B = 6
    w6 = J.custom([77] * B, 2, 128, sigma=0.5, seed=8, kind="broadcast", lq=130)
    case6 = J.Case(w6, np.full(B, 77), J.offsets_from_lengths([77] * B), case1.q,
                   np.concatenate([case1.k] * B), np.concatenate([case1.v] * B),
                   np.concatenate([case1.do] * B), case1.scale)
    r1 = GpuRun(case1, gpu)
    o1, _ = r1.forward()
    dq1, _, _ = r1.backward()
    r6 = GpuRun(case6, gpu)
    o6, _ = r6.forward()
    dq6, _, _ = r6.backward()
    for b in range(B):
        assert torch.equal(o6[b], o1[0])
    ref = B * bf16_to_f64(dq1)
    assert_grad(bf16_to_f64(dq6), ref, "dq(B copies) vs B*dq(1)")


@pytest.mark.parametrize("D", [64, 128])
def test_block_diag(gpu, D):
    check_case(J.custom([64, 192, 128, 64 * 7], 2, D, seed=9, kind="block"), gpu)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("base", [10000.0, 1.5, 1e9])
def test_block_diag_rotary(gpu, D, base):
    # base 1.5 turns every column pair by up to about 10 revolutions; 1e9 leaves the
    # high columns nearly still
    check_case(J.custom([64, 0, 192, 128, 64 * 7], 2, D, seed=9, kind="block",
                        rope_base=base), gpu)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_jagged_rotary(gpu, D, causal):
    check_case(J.custom(RAGGED, 3, D, sigma=0.5, seed=21, causal=causal, rope_base=10000.0), gpu)


@pytest.mark.parametrize("base", [10000.0, 1.5])
def test_jagged_rotary_long_positions(gpu, base):
    # positions up to 4999: the angles of the lowest frequencies reach ~800 turns
    check_case(J.custom([5000, 3, 0, 700], 1, 128, sigma=0.5, seed=22, causal=True,
                        rope_base=base), gpu)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [32, 128, 256])
def test_other_block_sizes(gpu, D, bs):
    # lengths in blocks: 1, 0, 3, 2, 7 (32-token blocks: an odd total, so the last
    # 64-token unit holds a single block)
    check_case(J.custom([bs, 0, 3 * bs, 2 * bs, 7 * bs], 2, D, seed=26, kind="block", block=bs), gpu)


@pytest.mark.parametrize("bs", [32, 128])
def test_other_block_sizes_with_rotary(gpu, bs):
    check_case(J.custom([bs, 3 * bs, 5 * bs], 2, 128, seed=27, kind="block", block=bs,
                        rope_base=10000.0), gpu)


WINDOW_LENGTHS = [300, 1, 129, 64, 0, 700, 17, 128, 2, 1000]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [1, 33, 64, 100, 128, 129, 256, 5000])
def test_jagged_sliding_window(gpu, D, W):
    check_case(J.custom(WINDOW_LENGTHS, 2, D, sigma=0.5, seed=23, causal=True, window=W), gpu)


def test_sliding_window_with_rotary(gpu):
    check_case(J.custom(WINDOW_LENGTHS, 2, 128, sigma=0.5, seed=24, causal=True, window=200,
                        rope_base=10000.0), gpu)


def test_sliding_window_covering_every_sequence_is_causal(gpu):
    # a window at least as long as every sequence gives the bits of plain causal
    import torch
    w = J.custom(WINDOW_LENGTHS, 2, 64, sigma=0.5, seed=25, causal=True)
    ra = GpuRun(J.make_case(w), gpu)
    rb = GpuRun(J.make_case(w.with_(window=1000)), gpu)
    oa, la = ra.forward()
    ob, lb = rb.forward()
    ga, gb = ra.backward(), rb.backward()
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    for x, y in zip(ga, gb):
        assert torch.equal(x, y)


def test_block_diag_rotary_rows_are_not_plain_attention(gpu):
    # the rotation is applied: rotary and plain block attention differ on the GPU
    import torch
    w = J.custom([128], 2, 64, seed=19, kind="block")
    o_plain, _ = GpuRun(J.make_case(w), gpu).forward()
    o_rope, _ = GpuRun(J.make_case(w.with_(rope_base=10000.0)), gpu).forward()
    assert not torch.equal(o_plain, o_rope)


def test_single_long_sequence(gpu):
    check_case(J.custom([1000], 2, 128, sigma=0.5, seed=10), gpu)
    check_case(J.custom([1000], 2, 128, sigma=0.5, seed=10, causal=True), gpu)


def test_tile_boundaries(gpu):
    check_case(J.custom([64, 128, 192, 256, 127, 129, 63, 65], 1, 128, sigma=0.5, seed=11), gpu)
    check_case(J.custom([64, 128, 192, 256, 127, 129, 63, 65], 1, 64, sigma=0.5, seed=11,
                        causal=True), gpu)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_partial_last_tiles(gpu, D, causal):
    # last query tiles that end inside each of the four 32-row waves (and tiles
    # whose later waves hold no row), last key tiles that end inside each
    # 32-key block: causal waves stop at different steps, waves and key blocks
    # with no row do no work
    lengths = [1, 31, 32, 33, 95, 96, 97, 160, 161, 223, 224, 225, 383, 415]
    check_case(J.custom(lengths, 2, D, sigma=0.5, seed=28, causal=causal), gpu)


def test_all_length_one(gpu):
    check_case(J.custom([1] * 40, 2, 64, seed=12), gpu)


def test_empty_problem(gpu):
    import torch
    plan = jfa.Plan(np.array([0, 0, 0], dtype=np.int32), 2, 64, 0.125, device=gpu)
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=gpu)
    out, lse = plan.forward(q, q, q)
    assert out.shape == (0, 2, 64)


def test_identical_keys_give_mean(gpu):
    w = J.custom([200], 2, 128, sigma=0.5, seed=13)
    case = J.make_case(w)
    case.k[:] = case.k[0]
    run = GpuRun(case, gpu)
    out, _ = run.forward()
    ref = J.bf16_bits_to_f64(case.v).mean(axis=0)
    assert np.max(np.abs(bf16_to_f64(out) - ref[None])) <= 1e-2


def test_schedule_order_does_not_change_results(gpu):
    import torch
    w = J.custom(RAGGED, 3, 128, sigma=0.5, seed=14, causal=True)
    case = J.make_case(w)
    a = GpuRun(case, gpu, order=jfa.ORDER_ZIGZAG)
    oa, la = a.forward()
    dqa, dka, dva = (x.clone() for x in a.backward())
    for order, slots in ((jfa.ORDER_INORDER, 7), (jfa.ORDER_XCD_ZIGZAG, None),
                         (jfa.ORDER_FOLDED_ZIGZAG, 5), (jfa.ORDER_FOLDED_ZIGZAG, None)):
        b = GpuRun(case, gpu, order=order, num_slots=slots)
        ob, lb = b.forward()
        assert torch.equal(oa, ob) and torch.equal(la, lb)
        dqb, dkb, dvb = b.backward()
        assert torch.equal(dqa, dqb) and torch.equal(dka, dkb) and torch.equal(dva, dvb)


@pytest.mark.parametrize("D", [64, 128])
def test_slot_counts_do_not_change_results(gpu, D):
    """One workgroup walking every tile (each tile's first stage and key operand
    are loaded while the previous tile's outputs are stored, across sequences
    and heads) and far more workgroups than tiles (most walk none) give the same
    bits as the default slot count, jagged and broadcast-Q."""
    import torch
    for w in (J.custom(RAGGED, 3, D, sigma=0.5, seed=21),
              J.custom([50, 0, 300, 129, 1], 2, D, sigma=0.5, seed=22, kind="broadcast", lq=130)):
        case = J.make_case(w)
        a = GpuRun(case, gpu)
        oa, la = a.forward()
        ga = [x.clone() for x in a.backward()]
        for slots in (1, 2048):
            log(f"D={D} {w.kind} slots={slots}")
            b = GpuRun(case, gpu, num_slots=slots)
            ob, lb = b.forward()
            assert torch.equal(oa, ob) and torch.equal(la, lb)
            for x, y in zip(ga, b.backward()):
                assert torch.equal(x, y)


def test_run_to_run_bitwise(gpu):
    import torch
    for w in (J.custom(RAGGED, 2, 128, sigma=0.5, seed=15),
              J.custom([50, 0, 300, 129], 2, 128, sigma=0.5, seed=15, kind="broadcast", lq=130)):
        run = GpuRun(J.make_case(w), gpu)
        o1, l1 = (x.clone() for x in run.forward())
        dq1, dk1, dv1 = (x.clone() for x in run.backward())
        for _ in range(3):
            o2, l2 = run.forward()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)
            dq2, dk2, dv2 = run.backward()
            assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


def test_block_diag_matches_jagged_path_on_refined_offsets(gpu):
    w = J.custom([64, 256, 128], 2, 128, seed=16, kind="block")
    case = J.make_case(w)
    blk = GpuRun(case, gpu)
    ob, _ = blk.forward()
    dqb, dkb, dvb = blk.backward()
    ref_off = A.refine_offsets(case.offsets, 64).astype(np.int32)
    L = np.diff(ref_off)
    wj = J.custom(L.tolist(), 2, 128, seed=16)
    cj = J.Case(wj, L, ref_off, case.q, case.k, case.v, case.do, case.scale)
    jag = GpuRun(cj, gpu)
    oj, _ = jag.forward()
    dqj, dkj, dvj = jag.backward()
    assert_out(bf16_to_f64(ob), bf16_to_f64(oj), "block vs jagged out")
    for n, a_, b_ in (("dq", dqb, dqj), ("dk", dkb, dkj), ("dv", dvb, dvj)):
        assert_grad(bf16_to_f64(a_), bf16_to_f64(b_), n + " block vs jagged")


def test_backward_passes_match_fused_call(gpu):
    """jfa_bwd_passes(DQ) then (DKDV) gives the bits of one jfa_bwd call."""
    import torch
    for w in (J.custom(RAGGED, 2, 128, sigma=0.5, seed=17, causal=True),
              J.custom([50, 0, 300, 129], 2, 64, sigma=0.5, seed=17, kind="broadcast", lq=130),
              # rotary: the dK/dV pass reads the rotated rows the dQ pass left behind
              J.custom(RAGGED, 2, 64, sigma=0.5, seed=17, rope_base=10000.0),
              J.custom(RAGGED, 2, 128, sigma=0.5, seed=17, causal=True, window=100)):
        log(f"case passes {w.kind} causal={w.causal} D={w.head_dim}")
        run = GpuRun(J.make_case(w), gpu)
        run.forward()
        dq1, dk1, dv1 = (x.clone() for x in run.backward())
        plan = run.plan
        q, k, v, out, do, lse = run.q, run.k, run.v, run.out_dev, run.do, run.lse_dev
        dq2, dk2, dv2 = (torch.full_like(x, float("nan")) for x in (dq1, dk1, dv1))
        plan.backward(q, k, v, out, do, lse, dq=dq2, dk=dk2, dv=dv2, passes=jfa.PASS_DQ)
        plan.backward(q, k, v, out, do, lse, dq=dq2, dk=dk2, dv=dv2, passes=jfa.PASS_DKDV)
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)


@pytest.mark.parametrize("D", [64, 128])
def test_block128_single_kernel_matches_jagged_passes(gpu, D):
    """128-token blocks: the single-tile backward (one call) and the two jagged
    passes called apart agree, and both match the oracle (checked by
    test_other_block_sizes for the single call)."""
    import torch
    w = J.custom([128, 0, 3 * 128, 7 * 128, 2 * 128], 2, D, seed=29, kind="block", block=128)
    log(f"case block128 passes D={D}")
    run = GpuRun(J.make_case(w), gpu)
    run.forward()
    dq1, dk1, dv1 = (x.clone() for x in run.backward())
    plan = run.plan
    q, k, v, out, do, lse = run.q, run.k, run.v, run.out_dev, run.do, run.lse_dev
    dq2, dk2, dv2 = (torch.full_like(x, float("nan")) for x in (dq1, dk1, dv1))
    plan.backward(q, k, v, out, do, lse, dq=dq2, dk=dk2, dv=dv2, passes=jfa.PASS_DQ)
    plan.backward(q, k, v, out, do, lse, dq=dq2, dk=dk2, dv=dv2, passes=jfa.PASS_DKDV)
    torch.cuda.synchronize()
    for n, a_, b_ in (("dq", dq1, dq2), ("dk", dk1, dk2), ("dv", dv1, dv2)):
        assert_grad(bf16_to_f64(a_), bf16_to_f64(b_), n + " single kernel vs passes")


@pytest.mark.parametrize("D,L", [(128, 129), (64, 300), (128, 128)])
def test_broadcast_one_sequence_matches_jagged(gpu, D, L):
    """Broadcast-Q with one sequence and Lq = L is jagged self-attention on the same
    tensors: both paths must agree with the oracle, on repeated runs, at lengths
    that stream several LDS stages (a hazard in the global->LDS copies once made
    the broadcast dQ pass read stale tiles there)."""
    import torch
    wb = J.custom([L], 1, D, sigma=0.5, seed=18, kind="broadcast", lq=L)
    cb = J.make_case(wb)
    ref = oracle_full(cb)
    wj = J.custom([L], 1, D, sigma=0.5, seed=18)
    cj = J.Case(wj, np.array([L]), cb.offsets, cb.q, cb.k, cb.v, cb.do[0], cb.scale)
    rj = GpuRun(cj, gpu)
    rj.forward()
    dqj, _, _ = rj.backward()
    assert_grad(bf16_to_f64(dqj), ref[2], "jagged dq")
    first = None
    for _ in range(3):
        rb = GpuRun(cb, gpu)
        rb.forward()
        dqb, dkb, dvb = (x.clone() for x in rb.backward())
        assert_grad(bf16_to_f64(dqb), ref[2], "broadcast dq")
        assert_grad(bf16_to_f64(dkb), ref[3], "broadcast dk")
        if first is None:
            first = dqb
        assert torch.equal(first, dqb)


def test_validate_env_checks_device_schedule(gpu, monkeypatch):
    """JFA_VALIDATE=1: a consistent call gives the same bits as without it; device
    offsets that do not match the schedule are refused before anything runs."""
    import torch
    w = J.custom([300, 1, 129, 0, 64], 2, 128, sigma=0.5, seed=29, causal=True)
    run = GpuRun(J.make_case(w), gpu)
    out, lse = run.forward()
    dq, dk, dv = run.backward()
    monkeypatch.setenv("JFA_VALIDATE", "1")
    out2, lse2 = run.plan.forward(run.q, run.k, run.v)
    grads2 = run.plan.backward(run.q, run.k, run.v, out2, run.do, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for a, b in zip((dq, dk, dv), grads2):
        assert torch.equal(a, b)
    # sequence 0 shortened on the device only: its tiles no longer match
    bad = run.plan.offsets_dev.clone()
    bad[1] = 100
    good = run.plan.offsets_dev
    run.plan.offsets_dev = bad
    try:
        with pytest.raises(jfa.JfaError) as e:
            run.plan.forward(run.q, run.k, run.v, out=out2, lse=lse2)
        assert e.value.status == jfa.ERR_INVALID_ARG and "JFA_VALIDATE" in str(e.value)
        with pytest.raises(jfa.JfaError):
            run.plan.backward(run.q, run.k, run.v, out2, run.do, lse2)
    finally:
        run.plan.offsets_dev = good
    torch.cuda.synchronize()
    assert torch.equal(out, out2)  # the refused calls wrote nothing
