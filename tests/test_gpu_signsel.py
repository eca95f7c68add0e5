"""One-time sign-pattern selection on the GPU (kvq_select_signs) against the oracle.

Each candidate's error is sum |o_c - o|^2 / sum |o|^2 (o exact attention, o_c attention over the keys
encoded with candidate c).  The decode's outputs agree with the oracle within tau = 2e-3 relative L2, so
an error computed on the GPU may differ from the oracle's by at most 2 sqrt(e) tau + tau^2; the chosen
candidate must be the oracle's best or within twice that of it.
"""
import os

import numpy as np
import pytest

import workloads as W
from helpers import log, make_hlm_case, scale_of, torch_dev

pytestmark = pytest.mark.gpu

TAU = 2e-3
HERE = os.path.dirname(os.path.abspath(__file__))


def err_bound(e):
    return 2.0 * np.sqrt(np.asarray(e)) * TAU + TAU * TAU


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import quantized_kv_cache_encode_amd.kvq as kvq
    return kvq


def _check(got_e, got_best, ref_e):
    got_e = np.asarray(got_e, dtype=np.float64)
    diff = np.abs(got_e - ref_e)
    log("  errors %.4g..%.4g, max |gpu - oracle| %.3g (bound %.3g), best %d (oracle %d)"
        % (ref_e.min(), ref_e.max(), diff.max(), err_bound(ref_e).max(), got_best, int(np.argmin(ref_e))))
    assert np.all(diff <= err_bound(ref_e))
    assert got_best == int(np.argmin(got_e))
    assert ref_e[got_best] <= ref_e.min() + 2 * err_bound(ref_e.min())


SMALL = [
    # name, shape, number of candidates
    ("signsel_small", W.scaled(W.SIGNSEL, B=2, Hq=8, Hkv=2, T=300), 12),
    ("fp32_d64_b2", W.scaled(W.SIGNSEL, B=3, Hq=4, Hkv=4, d=64, b=2, T=129, dtype="f32"), 9),
    ("d256_b3_G4", W.scaled(W.SIGNSEL, B=1, Hq=8, Hkv=2, d=256, b=3, T=77), 5),
    ("d16_b1_T1", W.scaled(W.SIGNSEL, B=2, Hq=2, Hkv=1, d=16, b=1, T=1), 4),
    ("d32_T8192", W.scaled(W.SIGNSEL, B=1, Hq=2, Hkv=1, d=32, b=4, T=8192), 3),
]


@pytest.mark.parametrize("name,shape,C", SMALL, ids=[c[0] for c in SMALL])
def test_select_signs_vs_oracle(K, oracle_mod, name, shape, C):
    case = make_hlm_case(shape)
    cands = W.sign_candidates(shape, C)
    log("signsel", name, case["keys"].shape, "C", C)
    lv, th = oracle_mod.codebook(shape.d, shape.b)
    ref_e, _ = oracle_mod.sign_errors(lv, th, cands, case["q"], case["keys"], case["v"], scale_of(shape.d))
    cb = K.kvq_build_codebook(shape.d, shape.b)
    got_e, got_best = K.kvq_select_signs(cb, cands, torch_dev(case["q"]), torch_dev(case["keys"]),
                                         torch_dev(case["v"]), scale=scale_of(shape.d))
    _check(got_e, got_best, ref_e)


def test_select_signs_full_size(K):
    """8 calibration samples, 32/8 heads, d=128, 512 keys, 200 candidates against the stored oracle errors."""
    sh = W.SIGNSEL
    path = os.path.join(HERE, "golden", "signsel_errors.txt")
    rows = [ln.split() for ln in open(path) if not ln.startswith("#")]
    ref_best = int(rows[0][1])
    ref_e = np.array([float(r[1]) for r in rows[1:]])
    assert len(ref_e) == W.SIGN_CANDIDATES and ref_best == int(np.argmin(ref_e))
    case = make_hlm_case(sh)
    cb = K.kvq_build_codebook(sh.d, sh.b)
    log("signsel full", case["keys"].shape, "C", len(ref_e))
    got_e, got_best = K.kvq_select_signs(cb, W.sign_candidates(sh), torch_dev(case["q"]), torch_dev(case["keys"]),
                                         torch_dev(case["v"]), scale=scale_of(sh.d))
    _check(got_e, got_best, ref_e)


def test_select_signs_repeatable_and_workspace_reuse(K):
    """Two calls sharing a dirty workspace give identical errors."""
    import torch
    sh = W.scaled(W.SIGNSEL, B=2, Hq=8, Hkv=2, T=2000)
    case = make_hlm_case(sh)
    cands = W.sign_candidates(sh, 6)
    cb = K.kvq_build_codebook(sh.d, sh.b)
    need = K.kvq_select_signs_workspace(cb, 2, 8, 2, 2000, 6)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda:0")
    args = (torch_dev(case["q"]), torch_dev(case["keys"]), torch_dev(case["v"]))
    e1, b1 = K.kvq_select_signs(cb, cands, *args, workspace=ws)
    e2, b2 = K.kvq_select_signs(cb, cands, *args, workspace=ws)
    assert b1 == b2 and np.array_equal(e1, e2)
