"""CPU tests of the block-sparse part of the C ABI: the step lists and the
sparse schedule equal the Python reference (oracle/schedule_ref.py) bit for bit
and a hand-worked example, and bad arguments are rejected on the host before
any HIP call."""
import ctypes

import numpy as np
import pytest

import jfa_inputs as J
import variable_length_flash_jaggedfa_amd as jfa
from oracle import schedule_ref as R

B28, B29 = 1 << 28, 1 << 29


def _problem(L, D=128, flags=jfa.BLOCK_SPARSE, block=64, H=2):
    L = np.asarray(L, dtype=np.int64)
    off = J.offsets_from_lengths(L)
    return jfa.problem(len(L), H, D, int(L.max()) if len(L) else 0, int(off[-1]), 0.1, flags,
                       block=block), off


def _masks(L, seed, density=0.35):
    rng = np.random.default_rng(seed)
    return [(rng.random((-(-int(n) // 64),) * 2) < density) for n in L]


def _flat(masks):
    parts = [m.astype(np.uint8).ravel() for m in masks]
    return np.concatenate(parts) if parts else np.zeros(0, np.uint8)


def test_hand_worked_lists():
    """Two sequences: 130 tokens (blocks 0, 1, 2; block 2 partial) with mask
    [[1,0,1],[0,0,0],[1,1,0]], and 64 tokens with mask [[1]]."""
    L = [130, 64]
    masks = [np.array([[1, 0, 1], [0, 0, 0], [1, 1, 0]], bool), np.array([[1]], bool)]
    p, off = _problem(L)
    # forward units (query tiles): (0,0) = query blocks 0,1; (0,1) = block 2; (1,0)
    fwd = ([0, 2, 3], [0, 2, 4, 5], [0 | B28, 2 | B28, 0 | B28, 1 | B28, 0 | B28])
    # backward units (key tiles): (0,0) = key blocks 0,1; (0,1) = block 2; (1,0)
    bwd = ([0, 2, 3], [0, 2, 3, 4], [0 | B28, 2 | B28 | B29, 0 | B28, 0 | B28])
    for kind, want in ((jfa.KIND_FWD, fwd), (jfa.KIND_BWD, bwd)):
        got = jfa.sparse_lists(p, off, _flat(masks), kind)
        ref = R.sparse_lists(L, masks, kind)
        for g, r, w in zip(got, ref, want):
            assert list(g) == list(r) == w, kind


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("kind", [jfa.KIND_FWD, jfa.KIND_BWD])
def test_lists_equal_reference(seed, kind):
    rng = np.random.default_rng(100 + seed)
    L = rng.integers(0, 700, size=40)
    L[3] = 0
    L[5] = 64
    L[7] = 65
    masks = _masks(L, seed, density=[0.0, 0.3, 1.0][seed])
    p, off = _problem(L)
    got = jfa.sparse_lists(p, off, _flat(masks), kind)
    ref = R.sparse_lists(L, masks, kind)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("kind", [jfa.KIND_FWD, jfa.KIND_BWD])
@pytest.mark.parametrize("order", [jfa.ORDER_INORDER, jfa.ORDER_ZIGZAG, jfa.ORDER_XCD_ZIGZAG,
                                   jfa.ORDER_FOLDED_ZIGZAG, jfa.ORDER_XCD_INORDER])
def test_sparse_schedule_equals_reference(kind, order):
    w = J.standard_workloads()["sparse_d128"].with_(num_seqs=300)
    L = J.lengths(w)
    masks = [J.sparse_mask_seq(w, b, int(n)).astype(bool) for b, n in enumerate(L)]
    p, off = _problem(L, H=w.num_heads)
    sb, lp, ent = jfa.sparse_lists(p, off, _flat(masks), kind)
    sp, tl = jfa.schedule_sparse(p, off, lp, ent, kind, order, 512)
    sp2, tl2 = R.schedule(L, w.num_heads, kind, 128, order, 512, sparse_list_ptr=lp,
                          sparse_entries=ent)
    assert np.array_equal(sp, sp2) and np.array_equal(tl, tl2)
    # the same tiles as plain attention; a key tile is worth 64 x its list's
    # length, a query tile 64 x the longer of its two blocks' lists
    assert len(tl) == jfa.schedule_count(p, off, kind)
    if kind == jfa.KIND_BWD:
        assert tl[:, 3].sum() == w.num_heads * 64 * len(ent)
    else:
        longer = [max(int(((ent[a:b] >> 28) & 1).sum()), int(((ent[a:b] >> 29) & 1).sum()))
                  for a, b in zip(lp[:-1], lp[1:])]
        assert tl[:, 3].sum() == w.num_heads * 64 * sum(longer)


def test_workload_masks_match_flat_draw():
    w = J.custom([1, 64, 200, 0, 65], 2, 64, kind="sparse", density=0.5, seed=4)
    c = J.make_case(w)
    parts = [J.sparse_mask_seq(w, b, int(n)).ravel() for b, n in enumerate(c.lengths)]
    assert np.array_equal(c.mask, np.concatenate(parts))
    # the diagonal is always kept
    pos = 0
    for n in c.lengths:
        nb = -(-int(n) // 64)
        m = c.mask[pos:pos + nb * nb].reshape(nb, nb)
        assert np.all(np.diag(m) == 1)
        pos += nb * nb


def test_hand_worked_causal_lists():
    """The 130-token sequence of the hand-worked case with causal masking: the
    forward drops key block 2 of query tile 0 (it lies after query block 0) and
    the backward drops query block 0 of key tile 1 (it lies before key block 2),
    which leaves that key tile an empty list."""
    L = [130, 64]
    masks = [np.array([[1, 0, 1], [0, 0, 0], [1, 1, 0]], bool), np.array([[1]], bool)]
    p, off = _problem(L, flags=jfa.BLOCK_SPARSE | jfa.CAUSAL)
    fwd = ([0, 2, 3], [0, 1, 3, 4], [0 | B28, 0 | B28, 1 | B28, 0 | B28])
    bwd = ([0, 2, 3], [0, 2, 2, 3], [0 | B28, 2 | B28 | B29, 0 | B28])
    for kind, want in ((jfa.KIND_FWD, fwd), (jfa.KIND_BWD, bwd)):
        got = jfa.sparse_lists(p, off, _flat(masks), kind)
        ref = R.sparse_lists(L, masks, kind, causal=True)
        for g, r, w in zip(got, ref, want):
            assert list(g) == list(r) == w, kind


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("kind", [jfa.KIND_FWD, jfa.KIND_BWD])
def test_causal_lists_are_the_lower_triangle(seed, kind):
    """Causal lists equal the plain lists of the mask with the block pairs above
    the diagonal cleared, and the reference's."""
    rng = np.random.default_rng(200 + seed)
    L = rng.integers(0, 900, size=30)
    L[2] = 0
    masks = _masks(L, 10 + seed, density=[0.4, 1.0][seed])
    p, off = _problem(L, flags=jfa.BLOCK_SPARSE | jfa.CAUSAL)
    got = jfa.sparse_lists(p, off, _flat(masks), kind)
    ref = R.sparse_lists(L, masks, kind, causal=True)
    tril = [np.tril(m) for m in masks]
    pl, _ = _problem(L)
    via = jfa.sparse_lists(pl, off, _flat(tril), kind)
    for g, r, v in zip(got, ref, via):
        assert np.array_equal(g, r) and np.array_equal(g, v)


@pytest.mark.parametrize("kind", [jfa.KIND_FWD, jfa.KIND_BWD])
def test_causal_sparse_schedule_equals_reference(kind):
    w = J.standard_workloads()["sparse_d128_causal"].with_(num_seqs=300)
    L = J.lengths(w)
    masks = [J.sparse_mask_seq(w, b, int(n)).astype(bool) for b, n in enumerate(L)]
    p, off = _problem(L, H=w.num_heads, flags=jfa.BLOCK_SPARSE | jfa.CAUSAL)
    sb, lp, ent = jfa.sparse_lists(p, off, _flat(masks), kind)
    for order in (jfa.ORDER_INORDER, jfa.ORDER_FOLDED_ZIGZAG, jfa.ORDER_XCD_INORDER):
        sp, tl = jfa.schedule_sparse(p, off, lp, ent, kind, order, 512)
        sp2, tl2 = R.schedule(L, w.num_heads, kind, 128, order, 512, sparse_list_ptr=lp,
                              sparse_entries=ent, causal=True)
        assert np.array_equal(sp, sp2) and np.array_equal(tl, tl2)


@pytest.mark.parametrize("kw,status", [
    (dict(flags=jfa.BLOCK_SPARSE | jfa.ROTARY), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.BLOCK_SPARSE | jfa.BROADCAST_Q), jfa.ERR_UNSUPPORTED),
    (dict(flags=jfa.BLOCK_SPARSE, block=0), jfa.ERR_INVALID_ARG),
    (dict(flags=jfa.BLOCK_SPARSE, block=128), jfa.ERR_INVALID_ARG),
])
def test_problem_rejects(kw, status):
    p, off = _problem([100, 30], **kw)
    with pytest.raises(jfa.JfaError) as e:
        jfa.schedule_count(p, off, jfa.KIND_FWD)
    assert e.value.status == status


def test_host_calls_reject_bad_arguments():
    L = [130, 64]
    p, off = _problem(L)
    m = _flat(_masks(L, 7))
    with pytest.raises(jfa.JfaError) as e:  # one byte short
        jfa.sparse_lists(p, off, m[:-1], jfa.KIND_FWD)
    assert e.value.status == jfa.ERR_INVALID_ARG and "mask_bytes" in str(e.value)
    with pytest.raises(jfa.JfaError) as e:  # plain schedule of a sparse problem
        jfa.schedule(p, off, jfa.KIND_FWD, jfa.ORDER_ZIGZAG, 8)
    assert e.value.status == jfa.ERR_INVALID_ARG
    pd, _ = _problem(L, flags=0, block=0)
    with pytest.raises(jfa.JfaError) as e:  # lists of a problem that is not sparse
        jfa.sparse_lists(pd, off, m, jfa.KIND_FWD)
    assert e.value.status == jfa.ERR_INVALID_ARG
    sb, lp, ent = jfa.sparse_lists(p, off, m, jfa.KIND_FWD)
    bad = lp.copy()
    bad[1], bad[2] = bad[2], bad[1] - 1  # a decreasing list pointer
    with pytest.raises(jfa.JfaError) as e:
        jfa.schedule_sparse(p, off, bad, ent, jfa.KIND_FWD, jfa.ORDER_INORDER, 8)
    assert e.value.status == jfa.ERR_INVALID_ARG and "list_ptr" in str(e.value)
    long_ = lp.copy()
    long_[1:] += 50  # the first list longer than its sequence has blocks
    with pytest.raises(jfa.JfaError) as e:
        jfa.schedule_sparse(p, off, long_, ent, jfa.KIND_FWD, jfa.ORDER_INORDER, 8)
    assert e.value.status == jfa.ERR_INVALID_ARG and "longer" in str(e.value)


def test_device_calls_reject_missing_lists_before_any_hip_call():
    Lb = jfa.lib()
    p, _ = _problem([130, 64])
    pd, _ = _problem([130, 64], flags=0, block=0)
    fake, nul = 4096, None
    lists = jfa.SparseListsDev(fake, fake, fake)
    # the plain forward of a sparse problem has no lists
    s = Lb.jfa_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, 4, fake, fake, nul, 0, None)
    assert s == jfa.ERR_INVALID_ARG and b"BLOCK_SPARSE" in Lb.jfa_last_error()
    # the sparse forward of a plain problem
    s = Lb.jfa_fwd_sparse(ctypes.byref(pd), fake, fake, fake, fake, ctypes.byref(lists), fake,
                          fake, 4, fake, fake, None)
    assert s == jfa.ERR_INVALID_ARG
    # a list pointer missing
    bad = jfa.SparseListsDev(fake, nul, fake)
    s = Lb.jfa_fwd_sparse(ctypes.byref(p), fake, fake, fake, fake, ctypes.byref(bad), fake, fake,
                          4, fake, fake, None)
    assert s == jfa.ERR_INVALID_ARG and b"list_ptr" in Lb.jfa_last_error()
    # backward without its key-tile lists
    s = Lb.jfa_bwd_sparse(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake,
                          ctypes.byref(lists), fake, fake, 4, nul, fake, fake, 4, fake, fake,
                          fake, fake, 1 << 20, jfa.PASS_ALL, None)
    assert s == jfa.ERR_INVALID_ARG
    # the plain backward of a sparse problem
    s = Lb.jfa_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake, fake, 4,
                   fake, fake, 4, fake, fake, fake, fake, 1 << 20, None)
    assert s == jfa.ERR_INVALID_ARG and b"BLOCK_SPARSE" in Lb.jfa_last_error()


@pytest.mark.parametrize("sparse", [False, True])
def test_plan_packs_its_device_arrays(sparse):
    """A plan sends the offsets, both schedules and (block-sparse) both kinds of
    step lists in one copy: each view holds its host array exactly, starts on a
    256-byte boundary of the packed buffer, and an empty array still gets one
    element (a valid pointer). Built with CPU tensors and an explicit slot count,
    so no device is needed."""
    L = np.array([130, 0, 64, 700, 1, 257])
    off = J.offsets_from_lengths(L)
    flags = jfa.BLOCK_SPARSE | jfa.CAUSAL if sparse else jfa.CAUSAL
    masks = _flat(_masks(L, 5, density=0.5)) if sparse else None
    plan = jfa.Plan(off, 2, 128, 0.1, flags, num_slots=24, device="cpu", block_mask=masks)
    base = plan.offsets_dev.data_ptr()
    views = [(plan.offsets_dev, off)]
    p = plan.p
    for kind, sch in plan.sched.items():
        if sparse:
            sb, lp, ent = jfa.sparse_lists(p, off, masks, kind)
            sp, tl = jfa.schedule_sparse(p, off, lp, ent, kind, plan.order, 24)
            for dev, host in zip(sch.lists_dev, (sb, lp, ent)):
                views.append((dev, host if host.size else np.zeros(1, np.int32)))
        else:
            sp, tl = jfa.schedule(p, off, kind, plan.order, 24)
        views.append((sch.slot_ptr_dev, sp))
        views.append((sch.tiles_dev, tl))
        assert tuple(sch.tiles_dev.shape) == (len(tl), 4)
    for dev, host in views:
        assert np.array_equal(dev.numpy().reshape(-1), np.asarray(host).reshape(-1))
        assert (dev.data_ptr() - base) % 256 == 0


def test_schedule_sparse_entries_argument():
    """Key-tile schedules need no entries (NULL is accepted); query-tile schedules
    read them for their work and reject NULL when the lists are not empty."""
    L = [130, 64]
    p, off = _problem(L)
    m = _flat(_masks(L, 7))
    Lb = jfa.lib()
    S = 8
    sp = np.zeros(S + 1, np.int32)
    for kind in (jfa.KIND_BWD, jfa.KIND_FWD):
        _, lp, ent = jfa.sparse_lists(p, off, m, kind)
        n = jfa.schedule_count(p, off, kind)
        tl = np.zeros((n, 4), np.int32)
        s = Lb.jfa_schedule_sparse(ctypes.byref(p), off.ctypes.data, lp.ctypes.data, None, kind,
                                   jfa.ORDER_XCD_INORDER, S, sp.ctypes.data, tl.ctypes.data, n)
        if kind == jfa.KIND_BWD:
            assert s == jfa.OK
            want = jfa.schedule_sparse(p, off, lp, ent, kind, jfa.ORDER_XCD_INORDER, S)
            assert np.array_equal(sp, want[0]) and np.array_equal(tl, want[1])
        else:
            assert s == jfa.ERR_INVALID_ARG and b"entries_host" in Lb.jfa_last_error()
