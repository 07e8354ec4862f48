"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default slot count, folded zigzag schedule).

The GEM-like batch (causal and not), the broadcast-Q batch and the
block-diagonal batches (64-token blocks at D = 64 and 128, the other block sizes
and rotary blocks) and the rotary and sliding-window variants of the GEM batch
are compared element by element in full: every output row of every (sequence,
head), lse, and dQ/dK/dV, against the fp64 oracle run over the whole batch by a
pool of worker processes (broadcast-Q: dQ summed over all 1024 sequences for
every head). On the imbalance
workload (4.6e14 FLOPs) every short sequence is compared in full, plus seeded
long slices and identities that hold at any size, checked over the whole output
on the GPU."""
import os
import time

import numpy as np
import pytest

import jfa_inputs as J
import variable_length_flash_jaggedfa_amd as jfa
from oracle import attention as A
from oracle import rotary as R
from tests.gpu_common import (GRAD_TOL, LSE_TOL, OUT_TOL, GpuRun, bf16_to_f64, log, lse_tol,
                              max_abs, out_excess, out_rel)

pytestmark = pytest.mark.gpu


def _pick(L, n_random, rng):
    order = np.argsort(L)
    pick = {int(order[-1]), int(order[0])}
    while len(pick) < min(len(L), 2 + n_random):
        pick.add(int(rng.integers(len(L))))
    return sorted(pick)


def _seq_slice(x, off, b, h):
    return J.bf16_bits_to_f64(x[off[b]:off[b + 1], h])


def l_ref_blocks(q_, k_, scale, bs):
    """lse of each block as its own sequence (128- and 256-token blocks keep one)."""
    return np.concatenate([A.seq_forward(q_[s:s + bs], k_[s:s + bs], k_[s:s + bs, :1], scale)[1]
                           for s in range(0, len(q_), bs)] or [np.zeros(0)])


def run_sampled(name, gpu, n_random=2, heads=None, long_heads=None):
    w = J.standard_workloads()[name]
    log(f"workload {name}: generating inputs")
    case = J.make_case(w)
    log(f"  B={w.num_seqs} T={int(case.offsets[-1])} H={w.num_heads} D={w.head_dim}")
    run = GpuRun(case, gpu)
    out, lse = run.forward()
    dq, dk, dv = run.backward()
    import torch
    log("  GPU fwd+bwd done")
    for name, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    off = case.offsets.astype(np.int64)
    rng = np.random.default_rng(123)
    seqs = _pick(case.lengths, n_random, rng)
    H = w.num_heads
    errs = {"out": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    refmax = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in seqs:
        hs = range(H) if heads is None else heads
        if long_heads is not None and case.lengths[b] > 4096:
            hs = long_heads
        for h in hs:
            k_ = _seq_slice(case.k, off, b, h)
            v_ = _seq_slice(case.v, off, b, h)
            if w.kind == "broadcast":
                q_ = J.bf16_bits_to_f64(case.q[:, h])
                do_ = J.bf16_bits_to_f64(case.do[b, :, h])
                got_o, got_l = bf16_to_f64(out[b, :, h]), lse[b, h].cpu().numpy()
            else:
                q_ = _seq_slice(case.q, off, b, h)
                do_ = _seq_slice(case.do, off, b, h)
                got_o = bf16_to_f64(out[off[b]:off[b + 1], h])
                got_l = lse[h, off[b]:off[b + 1]].cpu().numpy() if lse is not None else None
            # rotary: rows rotated by their index in the sequence, gradients turned
            # back afterwards
            pos = np.arange(len(k_))
            rot = (lambda x, inv=False: R.rope(x[:, None], pos, w.rope_base, inv)[:, 0]) \
                if w.rope_base else (lambda x, inv=False: x)
            if w.kind == "block":
                qr, kr = rot(q_), rot(k_)
                o_ref = np.zeros_like(q_)
                gq, gk, gv = np.zeros_like(q_), np.zeros_like(k_), np.zeros_like(v_)
                for s0 in range(0, len(q_), w.block):
                    sl = slice(s0, s0 + w.block)
                    o_ref[sl], _ = A.seq_forward(qr[sl], kr[sl], v_[sl], case.scale)
                    gq[sl], gk[sl], gv[sl] = A.seq_backward(qr[sl], kr[sl], v_[sl], do_[sl], case.scale)
                gq, gk = rot(gq, True), rot(gk, True)
                l_ref = None if w.block <= 64 else l_ref_blocks(qr, kr, case.scale, w.block)
            elif w.rope_base:
                o_ref, l_ref = A.seq_forward(rot(q_), rot(k_), v_, case.scale, w.causal, w.window)
                gq, gk, gv = A.seq_backward(rot(q_), rot(k_), v_, do_, case.scale, w.causal,
                                            w.window)
                gq, gk = rot(gq, True), rot(gk, True)
            else:
                o_ref, l_ref = A.seq_forward(q_, k_, v_, case.scale, w.causal, w.window)
                gq, gk, gv = A.seq_backward(q_, k_, v_, do_, case.scale, w.causal, w.window)
            errs["out"] = max(errs["out"], out_excess(got_o, o_ref, out_rel(w)))
            if l_ref is not None:
                errs["lse"] = max(errs["lse"], max_abs(got_l, l_ref))
            errs["dk"] = max(errs["dk"], max_abs(bf16_to_f64(dk[off[b]:off[b + 1], h]), gk))
            errs["dv"] = max(errs["dv"], max_abs(bf16_to_f64(dv[off[b]:off[b + 1], h]), gv))
            refmax["dk"] = max(refmax["dk"], float(np.abs(gk).max()))
            refmax["dv"] = max(refmax["dv"], float(np.abs(gv).max()))
            if w.kind != "broadcast":
                errs["dq"] = max(errs["dq"], max_abs(bf16_to_f64(dq[off[b]:off[b + 1], h]), gq))
                refmax["dq"] = max(refmax["dq"], float(np.abs(gq).max()))
    if w.kind == "broadcast":
        # dQ of one whole head: the sum over every sequence
        h = 0
        q_ = J.bf16_bits_to_f64(case.q[:, h])
        acc = np.zeros_like(q_)
        for b in range(w.num_seqs):
            gq, _, _ = A.seq_backward(q_, _seq_slice(case.k, off, b, h), _seq_slice(case.v, off, b, h),
                                      J.bf16_bits_to_f64(case.do[b, :, h]), case.scale)
            acc += gq
        errs["dq"] = max_abs(bf16_to_f64(dq[:, h]), acc)
        refmax["dq"] = float(np.abs(acc).max())
    log(f"  sampled sequences {seqs}")
    log(f"  out {errs['out']:.3e} lse {errs['lse']:.3e} "
        + " ".join(f"{k} {errs[k] / refmax[k]:.3e}" for k in ("dq", "dk", "dv")))
    assert errs["out"] <= OUT_TOL
    assert errs["lse"] <= lse_tol(w, case)
    for k in ("dq", "dk", "dv"):
        assert errs[k] <= GRAD_TOL * refmax[k], k


def _bits(t):
    """torch bf16 device tensor -> uint16 bit pattern (numpy)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_full(name, gpu, pool, rdir):
    """Every element of the workload's GPU results against the oracle."""
    from oracle import pool as OP
    w = J.standard_workloads()[name]
    log(f"workload {name} (every element): generating inputs")
    case = J.make_case(w)
    log(f"  B={w.num_seqs} T={int(case.offsets[-1])} H={w.num_heads} D={w.head_dim}")
    run = GpuRun(case, gpu)
    out, lse = run.forward()
    dq, dk, dv = run.backward()
    for nm, t in (("out", out), ("dq", dq), ("dk", dk), ("dv", dv)):
        np.save(os.path.join(rdir, nm + ".npy"), _bits(t))
    if lse is not None:
        np.save(os.path.join(rdir, "lse.npy"), lse.cpu().numpy())
    del run
    t0 = time.perf_counter()
    r = OP.compare(pool, w, case.scale, case.offsets, rdir, out_rel=out_rel(w))
    log(f"  oracle over {r['tasks']} tasks: {time.perf_counter() - t0:.1f} s wall, "
        f"{r['cpu_seconds']:.1f} s CPU")
    if w.kind == "broadcast":
        ref = r["dq_sum"]
        got = bf16_to_f64(dq)
        r["dq"], r["dq_ref"] = max_abs(got, ref), float(np.abs(ref).max())
        assert np.all(np.isfinite(got))
    log(f"  worst out element: reference {r.get('out_at', (0, 0))[0]:.5f}, "
        f"result {r.get('out_at', (0, 0))[1]:.5f} (bound 1e-2 + 2^-8 |reference|)")
    log(f"  out {r['out']:.3e} lse {r['lse']:.3e} " + " ".join(
        f"{k} {r[k] / max(r[k + '_ref'], 1e-30):.3e}" for k in ("dq", "dk", "dv")))
    assert r["finite"] and r["lse_inf_match"]
    assert r["out"] <= OUT_TOL
    assert r["lse"] <= lse_tol(w, case)
    for k in ("dq", "dk", "dv"):
        assert r[k] <= GRAD_TOL * r[k + "_ref"], k


@pytest.mark.parametrize("name", ["gem", "gem_causal", "broadcast", "block64_d64",
                                  "block64_d128", "block32_d128", "block128_d128",
                                  "block256_d128", "block64_rope_d64", "block64_rope_d128",
                                  "gem_rope", "gem_rope_causal", "gem_window"])
def test_every_element(gpu, oracle_pool, result_dir, name):
    run_full(name, gpu, oracle_pool, result_dir)


def test_imbalance(gpu):
    run_sampled("imbalance", gpu, n_random=6, long_heads=[3])


def test_imbalance_all_short_and_invariants(gpu):
    """Every short sequence x head against the oracle; six seeded long (sequence,
    head) pairs including the longest sequence; and over every (sequence, head):
    sum_j dK_j = 0, sum_j dV_j = sum_i dO_i (rows of P sum to one) and each out
    row inside the per-column range of its V rows (a convex combination)."""
    import torch
    w = J.standard_workloads()["imbalance"]
    log("workload imbalance: generating inputs")
    case = J.make_case(w)
    run = GpuRun(case, gpu)
    out, lse = run.forward()
    dq, dk, dv = run.backward()
    off = case.offsets.astype(np.int64)
    L = case.lengths
    H = w.num_heads
    # --- full-tensor identities, per (sequence, head), on the GPU in float32
    T = int(off[-1])
    seg = torch.repeat_interleave(torch.arange(len(L), device=gpu),
                                  torch.as_tensor(L, device=gpu))
    def seg_sum(x):
        return torch.zeros((len(L), H, w.head_dim), dtype=torch.float32,
                           device=gpu).index_add_(0, seg, x.float())
    sdk, sdv, sdo = seg_sum(dk), seg_sum(dv), seg_sum(run.do)
    sabs_dk = seg_sum(dk.abs())
    e_dk = float(((sdk.abs()) / (sabs_dk + 1e-30)).max())
    e_dv = float(((sdv - sdo).abs().max() / sdo.abs().max()))
    log(f"  sum dK / sum |dK| max {e_dk:.3e}; |sum dV - sum dO| / max|sum dO| {e_dv:.3e}")
    assert e_dk <= 2e-2
    assert e_dv <= 2e-2
    idx = seg.view(T, 1, 1).expand(T, H, w.head_dim)
    vmin = torch.full((len(L), H, w.head_dim), float("inf"), device=gpu).scatter_reduce(
        0, idx, run.v.float(), "amin")
    vmax = torch.full((len(L), H, w.head_dim), float("-inf"), device=gpu).scatter_reduce(
        0, idx, run.v.float(), "amax")
    # bf16 P and bf16 out put a row up to a few bf16 ulps of |v| outside the range
    o = out.float()
    tol = 3e-2
    lo_ok = (o >= vmin[seg] - tol).all()
    hi_ok = (o <= vmax[seg] + tol).all()
    assert bool(lo_ok) and bool(hi_ok)
    # --- every short sequence, every head
    short = [b for b in range(len(L)) if L[b] <= 64]
    rng = np.random.default_rng(7)
    long_ = [b for b in range(len(L)) if L[b] > 64]
    longest = int(np.argmax(L))
    pairs = [(longest, 0)] + [(int(b), int(rng.integers(H)))
                              for b in rng.choice([b for b in long_ if b != longest], 5, replace=False)]
    out_h, dq_h, dk_h, dv_h = (bf16_to_f64(x) for x in (out, dq, dk, dv))
    lse_h = lse.cpu().numpy()
    worst = {"out": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    ref = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    todo = [(b, h) for b in short for h in range(H)] + pairs
    log(f"  comparing {len(todo)} (sequence, head) slices ({len(short)} short sequences, "
        f"long pairs {pairs})")
    for b, h in todo:
        s, e = int(off[b]), int(off[b + 1])
        q_, k_, v_, do_ = (J.bf16_bits_to_f64(x[s:e, h]) for x in (case.q, case.k, case.v, case.do))
        o_ref, l_ref = A.seq_forward(q_, k_, v_, case.scale)
        gq, gk, gv = A.seq_backward(q_, k_, v_, do_, case.scale)
        worst["out"] = max(worst["out"], max_abs(out_h[s:e, h], o_ref))
        worst["lse"] = max(worst["lse"], max_abs(lse_h[h, s:e], l_ref))
        for k, got, r in (("dq", dq_h[s:e, h], gq), ("dk", dk_h[s:e, h], gk), ("dv", dv_h[s:e, h], gv)):
            worst[k] = max(worst[k], max_abs(got, r))
            ref[k] = max(ref[k], float(np.abs(r).max()))
    log("  " + " ".join(f"{k} {v:.3e}" for k, v in worst.items()))
    assert worst["out"] <= OUT_TOL and worst["lse"] <= LSE_TOL
    for k in ("dq", "dk", "dv"):
        assert worst[k] <= GRAD_TOL * ref[k], k
