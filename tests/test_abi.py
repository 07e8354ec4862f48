"""CPU tests of the C ABI: the library loads, exports every symbol include/jfa.h
declares, rejects bad arguments on the host (before any HIP call), and its C++
scheduler equals the independent Python reference bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import jfa_inputs as J
import variable_length_flash_jaggedfa_amd as jfa
from oracle import schedule_ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "jfa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jfa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = jfa.lib()
    syms = declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings():
    L = jfa.lib()
    for s in range(5):
        assert L.jfa_status_string(s)


def _p(**kw):
    base = dict(num_seqs=2, num_heads=2, head_dim=64, max_len=10, total_kv=15, scale=0.125,
                flags=0, lq=0)
    base.update(kw)
    return jfa.problem(**base)


OFF = np.array([0, 10, 15], dtype=np.int32)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), jfa.ERR_UNSUPPORTED),
    (dict(num_heads=0), jfa.ERR_INVALID_ARG),
    (dict(scale=0.0), jfa.ERR_INVALID_ARG),
    (dict(scale=float("nan")), jfa.ERR_INVALID_ARG),
    (dict(flags=64), jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.BLOCK_DIAG, block=48, total_kv=96, max_len=96), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.BLOCK_DIAG64, block=128, total_kv=128, max_len=128), jfa.ERR_INVALID_ARG),
    (dict(block=64), jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.BLOCK_DIAG | jfa.CAUSAL, block=128, total_kv=128, max_len=128),
     jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.BLOCK_DIAG, block=128, total_kv=192, max_len=192), jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.ROTARY | jfa.BROADCAST_Q, lq=4, rope_base=10000.0), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.ROTARY), jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.BLOCK_DIAG64 | jfa.ROTARY, total_kv=128, max_len=64), jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.BLOCK_DIAG64 | jfa.ROTARY, total_kv=128, max_len=64, rope_base=1.0),
     jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.BLOCK_DIAG64 | jfa.ROTARY, total_kv=128, max_len=64,
          rope_base=float("inf")), jfa.ERR_INVALID_ARG),
    (dict(rope_base=10000.0), jfa.ERR_INVALID_ARG),
    (dict(window=-1, flags=jfa.CAUSAL), jfa.ERR_INVALID_ARG),
    (dict(window=8), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.CAUSAL | jfa.BROADCAST_Q, lq=4), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.BLOCK_DIAG64 | jfa.CAUSAL), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.BROADCAST_Q, lq=0), jfa.ERR_INVALID_ARG),
    (dict(lq=3), jfa.ERR_INVALID_ARG),
    (dict(max_len=9), jfa.ERR_INVALID_ARG),
    (dict(total_kv=16), jfa.ERR_INVALID_ARG),
])
def test_schedule_count_rejects(kw, status):
    with pytest.raises(jfa.JfaError) as e:
        jfa.schedule_count(_p(**kw), OFF, jfa.KIND_FWD)
    assert e.value.status == status


@pytest.mark.parametrize("bs", [32, 128, 256])
def test_other_block_sizes(bs):
    L = np.array([bs, 3 * bs, 0, 2 * bs])
    off = J.offsets_from_lengths(L)
    p = _p(num_seqs=4, flags=jfa.BLOCK_DIAG, block=bs, total_kv=int(off[-1]), max_len=3 * bs)
    with pytest.raises(jfa.JfaError):  # a length that is not a multiple of the block
        jfa.schedule_count(p, np.array([0, bs + 1, 3 * bs, 3 * bs, int(off[-1])], dtype=np.int32),
                           jfa.KIND_FWD)
    n = jfa.schedule_count(p, off, jfa.KIND_FWD)
    r256 = lambda x: (x + 255) // 256 * 256
    if bs <= 64:   # 64-token units of the single-tile kernels, no schedule
        assert n == -(-int(off[-1]) // 64) * 2
        with pytest.raises(jfa.JfaError):
            jfa.schedule(p, off, jfa.KIND_FWD, jfa.ORDER_ZIGZAG, 8)
        assert jfa.fwd_workspace_bytes(p) == 0 and jfa.bwd_workspace_bytes(p) == 0
        return
    # the jagged tiles of the blocks, dealt as the reference deals blocks as sequences
    nb = int(off[-1]) // bs
    for kind in (jfa.KIND_FWD, jfa.KIND_BWD):
        rows = jfa.tile_rows(kind, 64, jfa.BLOCK_DIAG)
        assert jfa.schedule_count(p, off, kind) == nb * 2 * -(-bs // rows)
        for order in (jfa.ORDER_INORDER, jfa.ORDER_ZIGZAG, jfa.ORDER_FOLDED_ZIGZAG):
            sp, tl = jfa.schedule(p, off, kind, order, 8)
            sp2, tl2 = R.schedule([bs] * nb, 2, kind, rows, order, 8)
            assert np.array_equal(sp, sp2) and np.array_equal(tl, tl2)
    T = int(off[-1])
    assert jfa.fwd_workspace_bytes(p) == r256((nb + 1) * 4)
    assert jfa.bwd_workspace_bytes(p) == 2 * r256(2 * T * 4) + r256((nb + 1) * 4)


def test_addressing_limits():
    """The kernels address one tile (at most 256 token rows of one head) through
    32-bit buffer resources: 256 rows of all heads must span < 2^31 bytes, so
    H * D * 2 * 256 >= 2^31 is rejected before anything runs. A long sequence
    itself is fine: the resource covers only the tile being loaded, not the rest
    of the sequence (whose span may exceed 4 GiB, e.g. L >= 2^20 at H = 16,
    D = 128, or L >= 2^18 at H = 64)."""
    # largest accepted head count at D = 128: 2^22 / 128 - 1 = 32767
    for H, ok in ((32767, True), (32768, False), (16, True)):
        p = _p(num_seqs=1, num_heads=H, head_dim=128, max_len=8, total_kv=8)
        if ok:
            assert jfa.schedule_count(p, np.array([0, 8], dtype=np.int32), jfa.KIND_FWD) == H
        else:
            with pytest.raises(jfa.JfaError) as e:
                jfa.schedule_count(p, np.array([0, 8], dtype=np.int32), jfa.KIND_FWD)
            assert e.value.status == jfa.ERR_UNSUPPORTED
            assert jfa.bwd_workspace_bytes(p) == 0 and jfa.fwd_workspace_bytes(p) == 0
    # one sequence whose rows of one head span more than 4 GiB: accepted (the tile
    # count is exact; nothing is allocated here)
    for H, L in ((16, (1 << 20) + 1), (64, (1 << 18) + 1), (64, (1 << 21) + 77)):
        p = _p(num_seqs=1, num_heads=H, head_dim=128, max_len=L, total_kv=L)
        assert ((L - 1) * H + 1) * 128 * 2 > 1 << 32
        off = np.array([0, L], dtype=np.int32)
        assert jfa.schedule_count(p, off, jfa.KIND_FWD) == H * -(-L // 128)
        assert jfa.schedule_count(p, off, jfa.KIND_BWD) == H * -(-L // 128)
    # broadcast-Q out rows B * Lq * H * D past the element bound
    p = _p(num_seqs=1 << 20, num_heads=64, head_dim=128, lq=1 << 20, flags=jfa.BROADCAST_Q,
           max_len=0, total_kv=0)
    with pytest.raises(jfa.JfaError):
        jfa.schedule_count(p, np.zeros((1 << 20) + 1, dtype=np.int32), jfa.KIND_FWD)


def test_rotary_block_problem_accepted():
    p = _p(flags=jfa.BLOCK_DIAG64 | jfa.ROTARY, total_kv=128, max_len=64, rope_base=10000.0)
    assert jfa.schedule_count(p, np.array([0, 64, 128], dtype=np.int32), jfa.KIND_FWD) == 2 * 2
    assert jfa.bwd_workspace_bytes(p) == 0


def test_offsets_checks():
    with pytest.raises(jfa.JfaError):
        jfa.schedule_count(_p(), np.array([1, 10, 15], dtype=np.int32), jfa.KIND_FWD)
    with pytest.raises(jfa.JfaError):
        jfa.schedule_count(_p(), np.array([0, 10, 9], dtype=np.int32), jfa.KIND_FWD)
    # block-diagonal needs multiples of 64
    p = _p(flags=jfa.BLOCK_DIAG64, total_kv=128, max_len=100)
    with pytest.raises(jfa.JfaError):
        jfa.schedule_count(p, np.array([0, 28, 128], dtype=np.int32), jfa.KIND_FWD)
    assert jfa.schedule_count(p, np.array([0, 64, 128], dtype=np.int32), jfa.KIND_FWD) == 2 * 2


def test_fwd_bwd_reject_bad_pointers_before_any_hip_call():
    L = jfa.lib()
    p = _p()
    nul = None
    fake = 4096  # aligned non-null fake address: never dereferenced on these paths
    # NULL q
    s = L.jfa_fwd(ctypes.byref(p), nul, fake, fake, fake, fake, fake, 4, fake, fake, nul, 0, None)
    assert s == jfa.ERR_INVALID_ARG
    # misaligned k
    s = L.jfa_fwd(ctypes.byref(p), fake, fake + 2, fake, fake, fake, fake, 4, fake, fake, nul, 0, None)
    assert s == jfa.ERR_INVALID_ARG and b"aligned" in L.jfa_last_error()
    # missing lse
    s = L.jfa_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, 4, fake, nul, nul, 0, None)
    assert s == jfa.ERR_INVALID_ARG
    # zero slots
    s = L.jfa_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, 0, fake, fake, nul, 0, None)
    assert s == jfa.ERR_INVALID_ARG
    # jagged rotary without its workspace
    pr = _p(flags=jfa.ROTARY, rope_base=10000.0)
    s = L.jfa_fwd(ctypes.byref(pr), fake, fake, fake, fake, fake, fake, 4, fake, fake, nul, 0, None)
    assert s == jfa.ERR_WORKSPACE
    s = L.jfa_fwd(ctypes.byref(pr), fake, fake, fake, fake, fake, fake, 4, fake, fake, fake + 16,
                  1 << 20, None)
    assert s == jfa.ERR_INVALID_ARG and b"256-byte" in L.jfa_last_error()
    # block-diagonal with an lse pointer
    pb = _p(flags=jfa.BLOCK_DIAG64, total_kv=128, max_len=64)
    s = L.jfa_fwd(ctypes.byref(pb), fake, fake, fake, nul, nul, nul, 0, fake, fake, nul, 0, None)
    assert s == jfa.ERR_INVALID_ARG
    # backward: workspace too small
    s = L.jfa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake, 4,
                  fake, fake, 4, fake, fake, fake, fake, 16, None)
    assert s == jfa.ERR_WORKSPACE
    # backward: NULL dout
    s = L.jfa_bwd(ctypes.byref(p), fake, fake, fake, fake, nul, fake, fake, fake, fake, 4,
                  fake, fake, 4, fake, fake, fake, fake, 1 << 20, None)
    assert s == jfa.ERR_INVALID_ARG
    # backward: missing query-tile schedule for the dQ pass
    s = L.jfa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, nul, nul, 0,
                  fake, fake, 4, fake, fake, fake, fake, 1 << 20, None)
    assert s == jfa.ERR_INVALID_ARG
    # backward passes: an empty or unknown mask, and a single pass of the fused block path
    for bad in (0, 4, 7):
        s = L.jfa_bwd_passes(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake,
                             4, fake, fake, 4, fake, fake, fake, fake, 1 << 20, bad, None)
        assert s == jfa.ERR_INVALID_ARG and b"passes" in L.jfa_last_error()
    s = L.jfa_bwd_passes(ctypes.byref(pb), fake, fake, fake, fake, fake, nul, fake, nul, nul, 0,
                         nul, nul, 0, fake, fake, fake, nul, 0, jfa.PASS_DQ, None)
    assert s == jfa.ERR_INVALID_ARG and b"fused backward" in L.jfa_last_error()
    # empty problems are no-ops that touch nothing
    p0 = _p(num_seqs=0, total_kv=0, max_len=0)
    assert L.jfa_fwd(ctypes.byref(p0), nul, nul, nul, nul, nul, nul, 0, nul, nul, nul, 0, None) == jfa.OK


def test_workspace_bytes():
    r256 = lambda n: (n + 255) // 256 * 256
    # jagged: -Di and -lse/scale, each [H, T]
    assert jfa.bwd_workspace_bytes(_p()) == 2 * r256(2 * 15 * 4)
    # broadcast: two [B, H, Lq] vectors + min(B, 128) partials of [Lq, H, D]
    assert jfa.bwd_workspace_bytes(_p(flags=jfa.BROADCAST_Q, lq=7)) == \
        2 * r256(2 * 2 * 7 * 4) + 2 * 7 * 2 * 64 * 4
    assert jfa.bwd_workspace_bytes(_p(flags=jfa.BLOCK_DIAG64, total_kv=128, max_len=64)) == 0
    # jagged rotary: two rotated bf16 [T, H, D] copies (q and k) in both workspaces
    pr = _p(flags=jfa.ROTARY, rope_base=10000.0)
    rot = r256(15 * 2 * 64 * 2)
    assert jfa.fwd_workspace_bytes(pr) == 2 * rot
    assert jfa.bwd_workspace_bytes(pr) == 2 * r256(2 * 15 * 4) + 2 * rot
    assert jfa.fwd_workspace_bytes(_p()) == 0
    pbr = _p(flags=jfa.BLOCK_DIAG64 | jfa.ROTARY, total_kv=128, max_len=64, rope_base=10000.0)
    assert jfa.fwd_workspace_bytes(pbr) == 0 and jfa.bwd_workspace_bytes(pbr) == 0


def test_tile_rows():
    assert jfa.tile_rows(jfa.KIND_FWD, 128) > 0
    assert jfa.tile_rows(jfa.KIND_BWD, 64) > 0
    assert jfa.tile_rows(jfa.KIND_FWD, 80) == -1
    assert jfa.tile_rows(jfa.KIND_FWD, 128, jfa.BLOCK_DIAG64) == 64


@pytest.mark.parametrize("name", ["tiny", "gem", "gem_causal", "broadcast", "imbalance"])
@pytest.mark.parametrize("kind", [jfa.KIND_FWD, jfa.KIND_BWD])
@pytest.mark.parametrize("order", [jfa.ORDER_INORDER, jfa.ORDER_ZIGZAG, jfa.ORDER_XCD_ZIGZAG,
                                   jfa.ORDER_FOLDED_ZIGZAG, jfa.ORDER_XCD_INORDER])
def test_cpp_schedule_equals_reference(name, kind, order):
    w = J.standard_workloads()[name]
    L = J.lengths(w)
    off = J.offsets_from_lengths(L)
    H = w.num_heads if name != "imbalance" else 4
    flags = (jfa.CAUSAL if w.causal else 0) | (jfa.BROADCAST_Q if w.kind == "broadcast" else 0)
    p = jfa.problem(len(L), H, w.head_dim, int(L.max()), int(off[-1]), 0.1, flags, w.lq)
    S = 512
    sp, tl = jfa.schedule(p, off, kind, order, S)
    rows = jfa.tile_rows(kind, w.head_dim, flags)
    sp2, tl2 = R.schedule(L, H, kind, rows, order, S, w.causal, w.lq)
    assert np.array_equal(sp, sp2)
    assert np.array_equal(tl, tl2)


@pytest.mark.parametrize("W", [1, 100, 512, 5000])
@pytest.mark.parametrize("kind", [jfa.KIND_FWD, jfa.KIND_BWD])
@pytest.mark.parametrize("order", [jfa.ORDER_INORDER, jfa.ORDER_ZIGZAG, jfa.ORDER_XCD_ZIGZAG,
                                   jfa.ORDER_FOLDED_ZIGZAG, jfa.ORDER_XCD_INORDER])
def test_cpp_schedule_equals_reference_with_window(W, kind, order):
    w = J.standard_workloads()["gem_window"]
    L = J.lengths(w)
    off = J.offsets_from_lengths(L)
    p = jfa.problem(len(L), w.num_heads, w.head_dim, int(L.max()), int(off[-1]), 0.1, jfa.CAUSAL,
                    window=W)
    sp, tl = jfa.schedule(p, off, kind, order, 512)
    rows = jfa.tile_rows(kind, w.head_dim, jfa.CAUSAL)
    sp2, tl2 = R.schedule(L, w.num_heads, kind, rows, order, 512, True, window=W)
    assert np.array_equal(sp, sp2)
    assert np.array_equal(tl, tl2)


def test_cpp_schedule_golden():
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "schedule_examples.json")))["cases"]
    for c in cases:
        kind = jfa.KIND_FWD if c["kind"] == "fwd" else jfa.KIND_BWD
        rows = jfa.tile_rows(kind, 64, 0)
        if rows != c["tile_rows"]:
            # the library's tile height differs from the hand example: scale lengths
            f = rows // c["tile_rows"] if rows % c["tile_rows"] == 0 else None
            if f is None:
                continue
            lengths = [x * f for x in c["lengths"]]
        else:
            f, lengths = 1, c["lengths"]
        off = J.offsets_from_lengths(lengths)
        p = jfa.problem(len(lengths), c["heads"], 64, max(lengths), int(off[-1]), 0.1,
                        jfa.CAUSAL if c["causal"] else 0)
        for order, key in ((jfa.ORDER_ZIGZAG, "zigzag"), (jfa.ORDER_INORDER, "inorder")):
            sp, tl = jfa.schedule(p, off, kind, order, c["slots"])
            got = [[[t[0], t[1], t[2], t[3] // f] for t in tl[sp[s]:sp[s + 1]].tolist()]
                   for s in range(c["slots"])]
            assert got == c[key], (c["name"], key)


def test_cpp_schedule_golden_folded():
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "schedule_examples.json")))
    for c in cases["folded_cases"]:
        kind = jfa.KIND_FWD if c["kind"] == "fwd" else jfa.KIND_BWD
        rows = jfa.tile_rows(kind, 64, jfa.CAUSAL)
        assert rows % c["tile_rows"] == 0
        f = rows // c["tile_rows"]          # scale the hand example to the library's tiles
        lengths = [x * f for x in c["lengths"]]
        off = J.offsets_from_lengths(lengths)
        p = jfa.problem(len(lengths), c["heads"], 64, max(lengths), int(off[-1]), 0.1, jfa.CAUSAL)
        sp, tl = jfa.schedule(p, off, kind, jfa.ORDER_FOLDED_ZIGZAG, c["slots"])
        got = [[[t[0], t[1], t[2], t[3] // f] for t in tl[sp[s]:sp[s + 1]].tolist()]
               for s in range(c["slots"])]
        assert got == c["schedule"], c["name"]


def test_schedule_rejects_block_mode_and_small_capacity():
    L = jfa.lib()
    p = _p()
    sp = np.zeros(5, dtype=np.int32)
    tl = np.zeros((2, 4), dtype=np.int32)
    s = L.jfa_schedule(ctypes.byref(p), OFF.ctypes.data, jfa.KIND_FWD, jfa.ORDER_ZIGZAG, 4,
                       sp.ctypes.data, tl.ctypes.data, 1)
    assert s == jfa.ERR_INVALID_ARG
    pb = _p(flags=jfa.BLOCK_DIAG64, total_kv=128, max_len=64)
    off = np.array([0, 64, 128], dtype=np.int32)
    s = L.jfa_schedule(ctypes.byref(pb), off.ctypes.data, jfa.KIND_FWD, jfa.ORDER_ZIGZAG, 4,
                       sp.ctypes.data, tl.ctypes.data, 8)
    assert s == jfa.ERR_UNSUPPORTED


def test_probe_rejects_bad_arguments_before_any_hip_call():
    L = jfa.lib()
    ok = ctypes.c_void_p(256)  # never dereferenced: every call below fails its host checks
    for iters, wgs, sink, clocks in ((0, 1, ok, ok), (1 << 25, 1, ok, ok), (1, 0, ok, ok),
                                     (1, 70000, ok, ok), (1, 1, None, ok), (1, 1, ok, None),
                                     (1, 1, ctypes.c_void_p(258), ok),
                                     (1, 1, ok, ctypes.c_void_p(260))):
        assert L.jfa_probe_mfma(iters, wgs, sink, clocks, None) == jfa.ERR_INVALID_ARG


def test_noalloc_rejects_oversized_problem_on_host():
    """jfa_bwd_noalloc refuses a problem whose workspace exceeds its static scratch
    array before any HIP call (so this runs without a GPU)."""
    import ctypes
    L = jfa.lib()
    T = 5 << 20
    p = jfa.problem(1, 1, 128, T, T, 0.088)
    assert jfa.bwd_workspace_bytes(p) > jfa.NOALLOC_SCRATCH_BYTES
    st = L.jfa_bwd_noalloc(ctypes.byref(p), *([None] * 9), 0, None, None, 0, None, None, None,
                           None)
    assert st == jfa.ERR_WORKSPACE
    assert b"static scratch" in L.jfa_last_error()
    p = jfa.problem(1, 1, 96, 8, 8, 0.1)  # an invalid problem: the usual error first
    st = L.jfa_bwd_noalloc(ctypes.byref(p), *([None] * 9), 0, None, None, 0, None, None, None,
                           None)
    assert st == jfa.ERR_UNSUPPORTED
