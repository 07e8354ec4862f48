"""The oracle run over a whole workload by a pool of worker processes.

TEST INFRASTRUCTURE ONLY. The GPU parity tests, the smoke check and the
benchmark's CPU-baseline leg use it; the library never does.

The attention oracle treats every sequence on its own (and, for broadcast-Q,
sums the per-sequence dQ), so a workload splits into tasks of contiguous
sequences. A task rebuilds its sequences' inputs from the seeded per-sequence
streams of jfa_inputs (the same values the whole-workload draw holds), runs the
oracle's own whole-batch functions (attention.py, rotary.py) on that sub-batch,
and, when results under test are given, compares them element by element and
returns the worst errors; broadcast-Q tasks also return their partial dQ sum.
Workers run single-threaded BLAS, one per core.

Workers are forked from a forkserver process: call start_server() before the
calling process touches the GPU, so that no worker is a copy of a process that
has opened the device.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from . import attention as A
from . import rotary as R

_LIMITED = False


def workers() -> int:
    """Cores the pool uses: the affinity mask, capped at 16 (a GPU machine's CPU share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def affinity_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def start_server():
    """Start the forkserver (before the GPU is initialised in this process)."""
    ctx = mp.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle.attention", "oracle.rotary", "jfa_inputs"])
    from multiprocessing import forkserver
    forkserver.ensure_running()
    return ctx


def make_pool(n=None):
    return start_server().Pool(n or workers(), initializer=_init_worker)


def _init_worker():
    global _LIMITED
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except Exception:
        pass
    _LIMITED = True


def _sub_inputs(w, off, b0, b1):
    """Inputs of sequences [b0, b1) as float64, with their local offsets."""
    import jfa_inputs as J
    f = J.bf16_bits_to_f64
    L = np.diff(np.asarray(off[b0:b1 + 1], dtype=np.int64))
    loff = np.zeros(len(L) + 1, dtype=np.int64)
    np.cumsum(L, out=loff[1:])

    def packed(stream, rows=None):
        parts = [J.seq_values(w, stream, b, int(rows if rows is not None else L[b - b0]))
                 for b in range(b0, b1)]
        parts = [p for p in parts if p.shape[0]]
        if not parts:
            return np.zeros((0, w.num_heads, w.head_dim))
        return f(np.concatenate(parts, axis=0))

    k, v = packed(J.S_K), packed(J.S_V)
    if w.kind == "broadcast":
        q = f(J.seq_values(w, J.S_QDENSE, 0, w.lq))
        do = packed(J.S_DO, w.lq).reshape(b1 - b0, w.lq, w.num_heads, w.head_dim)
    else:
        q, do = packed(J.S_Q), packed(J.S_DO)
    if w.kind == "sparse":
        masks = [J.sparse_mask_seq(w, b, int(L[b - b0])).astype(bool) for b in range(b0, b1)]
        return q, k, v, do, loff, masks
    return q, k, v, do, loff


def oracle_sub(w, scale, q, k, v, do, loff, masks=None):
    """The oracle on one sub-batch: (out, lse or None, dq, dk, dv), as the oracle's
    whole-workload functions define them."""
    if w.kind == "sparse":
        out, lse = A.block_sparse_forward(q, k, v, loff, scale, masks, w.causal)
        dq, dk, dv = A.block_sparse_backward(q, k, v, do, loff, scale, masks, w.causal)
    elif w.kind == "broadcast":
        out, lse = A.broadcast_forward(q, k, v, loff, scale)
        dq, dk, dv = A.broadcast_backward(q, k, v, do, loff, scale)
    elif w.kind == "block" and w.rope_base:
        out = R.block_diag_rope_forward(q, k, v, loff, scale, w.rope_base, w.block)
        dq, dk, dv = R.block_diag_rope_backward(q, k, v, do, loff, scale, w.rope_base, w.block)
        lse = (R.jagged_rope_forward(q, k, v, A.refine_offsets(loff, w.block), scale,
                                     w.rope_base)[1] if w.block > 64 else None)
    elif w.kind == "block":
        out = A.block_diag_forward(q, k, v, loff, scale, w.block)
        dq, dk, dv = A.block_diag_backward(q, k, v, do, loff, scale, w.block)
        lse = (A.jagged_forward(q, k, v, A.refine_offsets(loff, w.block), scale)[1]
               if w.block > 64 else None)
    elif w.rope_base:
        out, lse = R.jagged_rope_forward(q, k, v, loff, scale, w.rope_base, w.causal, w.window)
        dq, dk, dv = R.jagged_rope_backward(q, k, v, do, loff, scale, w.rope_base, w.causal,
                                            w.window)
    else:
        out, lse = A.jagged_forward(q, k, v, loff, scale, w.causal, w.window)
        dq, dk, dv = A.jagged_backward(q, k, v, do, loff, scale, w.causal, w.window)
    return out, lse, dq, dk, dv


_MAPS = {}


def _result(rdir, name):
    """The stored result `name` of rdir, memory-mapped once per file: the key holds
    the file's identity (inode, size, modification time), so a directory removed
    and made again under the same path, or a file written anew, is mapped afresh."""
    path = os.path.join(rdir, name + ".npy")
    try:
        st = os.stat(path)
    except FileNotFoundError:
        return None
    key = (path, st.st_ino, st.st_size, st.st_mtime_ns)
    if key not in _MAPS:
        for old in [k for k in _MAPS if k[0] == path]:
            del _MAPS[old]
        _MAPS[key] = np.load(path, mmap_mode="r")
    return _MAPS[key]


def _bits64(x):
    import jfa_inputs as J
    return J.bf16_bits_to_f64(np.asarray(x))


def _task(args):
    """One task: the oracle over sequences [b0, b1) and, with rdir, the comparison
    with the results stored there. Returns a dict of worst errors (and the task's
    partial dQ for broadcast-Q)."""
    w, scale, off, b0, b1, rdir, out_rel = args
    t0 = time.perf_counter()
    out, lse, dq, dk, dv = oracle_sub(w, scale, *_sub_inputs(w, off, b0, b1))
    res = {"b0": b0, "b1": b1, "seconds": time.perf_counter() - t0}
    if rdir is None:
        return res
    s, e = int(off[b0]), int(off[b1])
    if w.kind == "broadcast":
        g_out = _bits64(_result(rdir, "out")[b0:b1])
        g_lse = np.asarray(_result(rdir, "lse")[b0:b1], dtype=np.float64)
        res["dq_part"] = dq
    else:
        g_out = _bits64(_result(rdir, "out")[s:e])
        lz = _result(rdir, "lse")
        g_lse = None if lz is None else np.asarray(lz[:, s:e], dtype=np.float64)
    g_dk, g_dv = _bits64(_result(rdir, "dk")[s:e]), _bits64(_result(rdir, "dv")[s:e])
    res["finite"] = bool(np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_dk))
                         and np.all(np.isfinite(g_dv)))
    if out.size:
        ex = np.abs(g_out - out) - out_rel * np.abs(out)
        i = int(np.argmax(ex))
        res["out"] = float(ex.flat[i])
        res["out_at"] = (float(out.flat[i]), float(g_out.flat[i]))  # reference, result
    else:
        res["out"] = 0.0
    if lse is not None and g_lse is not None:
        fin = np.isfinite(lse)
        res["lse_inf_match"] = bool(np.array_equal(np.isfinite(g_lse), fin))
        res["lse"] = float(np.max(np.abs(g_lse[fin] - lse[fin]))) if fin.any() else 0.0
    for name, got, ref in (("dk", g_dk, dk), ("dv", g_dv, dv)):
        res[name] = float(np.max(np.abs(got - ref))) if ref.size else 0.0
        res[name + "_ref"] = float(np.max(np.abs(ref))) if ref.size else 0.0
    if w.kind != "broadcast":
        g_dq = _bits64(_result(rdir, "dq")[s:e])
        res["finite"] = res["finite"] and bool(np.all(np.isfinite(g_dq)))
        res["dq"] = float(np.max(np.abs(g_dq - dq))) if dq.size else 0.0
        res["dq_ref"] = float(np.max(np.abs(dq))) if dq.size else 0.0
    return res


def tasks_of(w, off, per_task=None):
    """Contiguous sequence ranges: one sequence per task for self-attention (the
    longest first, for balance), `per_task` (default 8 or 16) for broadcast-Q and
    block-diagonal workloads."""
    B = len(off) - 1
    L = np.diff(np.asarray(off, dtype=np.int64))
    if per_task is None:
        per_task = 1 if w.kind in ("jagged", "sparse") else (8 if w.kind == "broadcast" else 16)
    ranges = [(b, min(B, b + per_task)) for b in range(0, B, per_task)]
    if per_task == 1:
        ranges.sort(key=lambda r: -int(L[r[0]]))
    return ranges


def compare(pool, w, scale, off, rdir, out_rel=0.0, per_task=None):
    """Every element of the results in `rdir` against the oracle. Returns the
    worst errors over the workload: out (absolute, less out_rel * |ref|), lse
    (absolute), dq/dk/dv (absolute, with the largest |ref| of each tensor), and for
    broadcast-Q the oracle's dQ summed over every sequence (float64)."""
    off = np.asarray(off, dtype=np.int64)
    args = [(w, scale, off, b0, b1, rdir, out_rel) for b0, b1 in tasks_of(w, off, per_task)]
    worst = {"out": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0,
             "dq_ref": 0.0, "dk_ref": 0.0, "dv_ref": 0.0, "finite": True, "lse_inf_match": True,
             "tasks": len(args), "cpu_seconds": 0.0}
    parts = {}
    for r in pool.imap_unordered(_task, args):
        if r.get("out", -np.inf) > worst["out"] or "out_at" not in worst:
            if "out_at" in r:
                worst["out_at"] = r["out_at"]
        for key in ("out", "lse", "dq", "dk", "dv", "dq_ref", "dk_ref", "dv_ref"):
            if key in r:
                worst[key] = max(worst[key], r[key])
        worst["finite"] = worst["finite"] and r.get("finite", True)
        worst["lse_inf_match"] = worst["lse_inf_match"] and r.get("lse_inf_match", True)
        worst["cpu_seconds"] += r["seconds"]
        if "dq_part" in r:
            parts[r["b0"]] = r["dq_part"]
    if parts:
        # partial sums added in sequence order
        worst["dq_sum"] = sum(parts[b] for b in sorted(parts))
    return worst


def time_sample(pool, w, scale, off, budget_s, seed=0):
    """The oracle's forward and backward over random single sequences (all heads)
    until `budget_s` of wall time has passed; tasks still running then are
    dropped. Returns (sequences done, seconds until the last one finished)."""
    off = np.asarray(off, dtype=np.int64)
    B = len(off) - 1
    order = np.random.default_rng(seed).permutation(B)
    args = [(w, scale, off, int(b), int(b) + 1, None, 0.0) for b in order]
    done, t0, last = [], time.perf_counter(), 0.0
    it = pool.imap_unordered(_task, args)
    for r in it:
        done.append(r["b0"])
        last = time.perf_counter() - t0
        if last > budget_s:
            break
    return done, last
