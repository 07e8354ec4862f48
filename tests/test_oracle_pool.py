"""The oracle's worker pool (oracle/pool.py) against the oracle run in one piece:
a whole workload split into sub-batches of sequences gives the same outputs, the
comparison finds a planted error, and broadcast-Q partial dQ sums add up to the
whole dQ. CPU only."""
import os

import numpy as np
import pytest

import jfa_inputs as J
from oracle import pool as P
from tests.gpu_common import oracle_full


@pytest.fixture(scope="module")
def workers():
    p = P.make_pool(4)
    yield p
    p.terminate()
    p.join()


def _store(tmp, case, res, w):
    out, lse, dq, dk, dv = res
    bits = J.f32_to_bf16_bits
    np.save(os.path.join(tmp, "out.npy"), bits(out.astype(np.float32)))
    if lse is not None:
        np.save(os.path.join(tmp, "lse.npy"), lse.astype(np.float32))
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.save(os.path.join(tmp, name + ".npy"), bits(x.astype(np.float32)))


CASES = [
    J.custom([70, 1, 0, 200, 33], 2, 64, sigma=0.5, seed=31, causal=True),
    J.custom([70, 1, 0, 200, 33], 2, 64, sigma=0.5, seed=32, causal=True, window=20),
    J.custom([70, 1, 0, 200, 33], 2, 128, sigma=0.5, seed=33, rope_base=100.0),
    J.custom([50, 0, 130, 1], 2, 64, sigma=0.5, seed=34, kind="broadcast", lq=70),
    J.custom([64, 192, 0, 128], 2, 64, seed=35, kind="block"),
    J.custom([128, 256, 0], 2, 64, seed=36, kind="block", block=128),
    J.custom([70, 1, 0, 200, 130], 2, 64, sigma=0.5, seed=37, kind="sparse", density=0.4),
    J.custom([70, 1, 0, 200, 130], 2, 64, sigma=0.5, seed=38, kind="sparse", density=0.4,
             causal=True),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"{w.kind}-c{int(w.causal)}-w{w.window}"
                         f"-r{int(bool(w.rope_base))}-b{w.block}")
def test_pool_matches_whole_oracle(workers, tmp_path, w):
    case = J.make_case(w)
    res = oracle_full(case)
    _store(str(tmp_path), case, res, w)
    r = P.compare(workers, w, case.scale, case.offsets, str(tmp_path), per_task=1)
    # the stored results are the oracle's own, rounded to bf16: errors are at most
    # half a bf16 step of each value
    assert r["finite"] and r["lse_inf_match"]
    for name, ref in (("out", res[0]), ("dk", res[3]), ("dv", res[4])):
        assert r[name] <= 2.0 ** -8 * max(1e-30, float(np.abs(ref).max())) + 1e-12, name
    if res[1] is not None:
        assert r["lse"] <= 1e-6 * max(1.0, float(np.abs(res[1][np.isfinite(res[1])]).max()))
    if w.kind == "broadcast":
        assert np.allclose(r["dq_sum"], res[2], rtol=0, atol=1e-12)
    else:
        assert r["dq"] <= 2.0 ** -8 * float(np.abs(res[2]).max()) + 1e-12
        assert abs(r["dq_ref"] - float(np.abs(res[2]).max())) <= 1e-12


def test_pool_finds_planted_error(workers, tmp_path):
    w = CASES[0]
    case = J.make_case(w)
    res = oracle_full(case)
    _store(str(tmp_path), case, res, w)
    dk = np.load(os.path.join(str(tmp_path), "dk.npy"))
    t, h, d = int(case.offsets[3]) + 5, 1, 17  # a row of the 200-token sequence
    x = J.bf16_bits_to_f32(dk[t, h, d:d + 1]) + np.float32(0.25)
    dk[t, h, d] = J.f32_to_bf16_bits(x)[0]
    np.save(os.path.join(str(tmp_path), "dk.npy"), dk)
    r = P.compare(workers, w, case.scale, case.offsets, str(tmp_path))
    assert r["dk"] >= 0.24
    assert r["dv"] < 0.01


def test_pool_flags_nonfinite(workers, tmp_path):
    w = CASES[4]
    case = J.make_case(w)
    res = oracle_full(case)
    _store(str(tmp_path), case, res, w)
    out = np.load(os.path.join(str(tmp_path), "out.npy"))
    out[3, 0, 0] = 0x7FC0  # a NaN
    np.save(os.path.join(str(tmp_path), "out.npy"), out)
    r = P.compare(workers, w, case.scale, case.offsets, str(tmp_path))
    assert not r["finite"]


def test_pool_maps_a_remade_directory_afresh(workers, tmp_path):
    """Results of one workload stored, compared, the directory removed and made
    again under the same path with another workload's results (another head
    dimension): the workers must read the new files, not their maps of the old."""
    import shutil
    rdir = str(tmp_path / "res")
    for w in (CASES[0].with_(head_dim=64), CASES[0].with_(head_dim=128, seed=41)):
        os.makedirs(rdir)
        case = J.make_case(w)
        res = oracle_full(case)
        _store(rdir, case, res, w)
        for _ in range(2):  # every worker sees this directory at least once
            r = P.compare(workers, w, case.scale, case.offsets, rdir, per_task=1)
            assert r["finite"] and r["dk"] <= 2.0 ** -8 * float(np.abs(res[3]).max()) + 1e-12
        shutil.rmtree(rdir)
