"""The benchmark credits FLOPs from its count of attended (query, key) pairs
(forward 4*N*H*D, backward 10*N*H*D). The count is pinned here against explicit
attention masks, built per sequence from the mask definitions the oracle
applies: causal keeps j <= i, a window W also keeps only j > i - W, block
diagonal keeps i and j in the same block, broadcast attends Lq dense queries to
every key."""
import os

import numpy as np
import pytest

import bench
from oracle import attention as A


def masked_pairs(L, causal=False, lq=0, block=0, window=0):
    n = 0
    for l in L:
        if lq:
            n += int(np.ones((lq, l), dtype=bool).sum())
            continue
        i = np.arange(l)[:, None]
        j = np.arange(l)[None, :]
        keep = np.ones((l, l), dtype=bool)
        if block:
            keep &= (i // block) == (j // block)
        if causal:
            keep &= j <= i
        if window:
            keep &= j > i - window
        n += int(keep.sum())
    return n


LENGTHS = [0, 1, 2, 31, 64, 65, 127, 128, 129, 300, 511]


@pytest.mark.parametrize("causal", [False, True])
def test_self_attention_pairs(causal):
    rng = np.random.default_rng(3)
    L = LENGTHS + list(rng.integers(0, 400, size=8))
    assert bench.pairs_of(L, causal=causal) == masked_pairs(L, causal=causal)
    assert bench.pairs_of(L, causal=causal) == A.pair_count(L, causal=causal)


@pytest.mark.parametrize("W", [1, 2, 33, 128, 129, 5000])
def test_causal_window_pairs(W):
    assert bench.pairs_of(LENGTHS, causal=True, window=W) == masked_pairs(LENGTHS, causal=True, window=W)


def test_window_covering_every_sequence_is_causal():
    assert bench.pairs_of(LENGTHS, causal=True, window=max(LENGTHS)) == masked_pairs(LENGTHS, causal=True)


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_block_diagonal_pairs(bs):
    L = [bs, 0, 3 * bs, 7 * bs, 2 * bs]
    assert bench.pairs_of(L, block=bs) == masked_pairs(L, block=bs)


def test_broadcast_pairs():
    L = [0, 1, 50, 300]
    assert bench.pairs_of(L, lq=256) == masked_pairs(L, lq=256)


def test_padding_ratio_counts_padded_pairs():
    # every sequence padded to the longest: B * Lmax^2 (causal: B * Lmax(Lmax+1)/2)
    class Case:
        lengths = np.array([3, 5, 8])
    g = bench.variants_of("gem")
    assert [w.causal for w in g] == [False, True]
    r_nc = bench.padded_ratio(Case, g[0])
    r_c = bench.padded_ratio(Case, g[1])
    assert r_nc == pytest.approx(3 * 64 / masked_pairs([3, 5, 8]))
    assert r_c == pytest.approx(3 * 36 / masked_pairs([3, 5, 8], causal=True))


def test_block_sparse_pairs():
    """Block-sparse: the pairs of the token mask each block mask expands to."""
    rng = np.random.default_rng(3)
    L = LENGTHS
    masks = [rng.random((-(-l // 64),) * 2) < 0.4 for l in L]
    flat = np.concatenate([m.astype(np.uint8).ravel() for m in masks])
    want = 0
    for l, m in zip(L, masks):
        i = np.arange(l)
        want += int(m[i[:, None] // 64, i[None, :] // 64].sum())
    assert bench.sparse_pairs(L, flat) == want == A.pair_count(L, masks=masks)


def test_causal_block_sparse_pairs():
    rng = np.random.default_rng(4)
    L = LENGTHS
    masks = [rng.random((-(-l // 64),) * 2) < 0.4 for l in L]
    flat = np.concatenate([m.astype(np.uint8).ravel() for m in masks])
    want = 0
    for l, m in zip(L, masks):
        i = np.arange(l)
        keep = m[i[:, None] // 64, i[None, :] // 64] & (i[None, :] <= i[:, None])
        want += int(keep.sum())
    assert bench.sparse_pairs(L, flat, causal=True) == want == \
        A.pair_count(L, causal=True, masks=masks)


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: asked for more it says so and exits with status 2
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_predicted_balance_of_a_hand_dealt_schedule():
    """Busiest slot over the mean slot, from the tiles' work column: slots hold
    works (3, 1), (2) and () -> loads 4, 2, 0, mean 2, ratio 2; a kind without
    tiles is left out."""
    from types import SimpleNamespace

    import variable_length_flash_jaggedfa_amd as jfa
    tiles = np.array([[0, 0, 0, 3], [0, 0, 1, 1], [1, 0, 0, 2]], dtype=np.int32)
    fwd = jfa.Schedule(np.array([0, 2, 3, 3], dtype=np.int32), tiles, 3)
    bwd = jfa.Schedule(np.array([0, 0], dtype=np.int32), np.zeros((0, 4), np.int32), 1)
    plan = SimpleNamespace(sched={jfa.KIND_FWD: fwd, jfa.KIND_BWD: bwd})
    assert bench.predicted_balance(plan, jfa) == {"fwd": 2.0}
    assert bench.predicted_balance(SimpleNamespace(sched={}), jfa) == {}
