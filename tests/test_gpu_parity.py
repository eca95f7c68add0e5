"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs.

Bars: codes bit-exact except coordinates within 1e-6 of a threshold (the
GPU decides in fp32, the oracle in fp64; such codes may differ by one level
and are counted), scores within 1e-4*|q|*|k_t|, attention outputs within 2e-3
relative L2 per (batch, head) row.  Score and attention parity are checked on
the oracle's own codes and norms, uploaded, so both sides read identical
caches; GPU encode followed by GPU attention is checked separately.
"""
import math

import numpy as np
import pytest

import workloads as W
from helpers import (log, make_hlm_case, oracle_cache, rel_l2_rows, scale_of, score_tolerance, torch_dev)

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import quantized_kv_cache_encode_amd.kvq as kvq
    return kvq


def _gpu_encode(K, cb, signs, keys, T_cap=None, t0=0, write_pos=None):
    import torch
    B, H, T, d = keys.shape
    T_cap = T if T_cap is None else T_cap
    codes = torch.zeros((B, H, T_cap, cb.bytes_per_key), dtype=torch.uint8, device="cuda:0")
    norms = torch.zeros((B, H, T_cap), dtype=torch.float32, device="cuda:0")
    K.kvq_encode_keys(cb, signs, torch_dev(keys), codes, norms, t0=t0, write_pos=write_pos)
    torch.cuda.synchronize()
    return codes, norms


def _check_codes(oracle_mod, shape, got_codes, got_norms, ref_codes, ref_norms, tie):
    d, b = shape.d, shape.b
    gi = oracle_mod.unpack_codes(got_codes, d, b)
    ri = oracle_mod.unpack_codes(ref_codes, d, b)
    diff = gi != ri
    n_diff, n_tie = int(diff.sum()), int(tie.sum())
    assert not np.any(diff & ~tie), "code mismatch outside the tie band: %d" % int((diff & ~tie).sum())
    assert np.all(np.abs(gi[diff] - ri[diff]) == 1)
    # rows without any tie are byte-identical
    row_has_tie = tie.any(axis=-1)
    np.testing.assert_array_equal(got_codes[~row_has_tie], ref_codes[~row_has_tie])
    np.testing.assert_allclose(got_norms, ref_norms, rtol=1e-5, atol=0)
    return n_diff, n_tie


ENCODE_CASES = [
    ("tiny", W.TINY, None, None),
    ("llama8b", W.LLAMA8B, None, None),
    ("longctx_b0_b7", W.LONGCTX, [0, 7], None),
    ("sweep_b2", W.sweep(2, 1), None, None),
    ("sweep_b3", W.sweep(3, 1), None, None),
    ("sweep_b4", W.sweep(4, 1), None, None),
    ("sweep_b3_B64_sample", W.sweep(3, 64), [5, 63], 2000),
    ("d32_b1_ragged", W.scaled(W.LLAMA8B, d=32, b=1, Hq=4, Hkv=2, T=1000), None, None),
    ("d256_b3_ragged", W.scaled(W.LONGCTX, d=256, b=3, B=2, Hq=2, Hkv=2, T=333), None, None),
    ("d16_b4_fp16", W.scaled(W.TINY, b=4, dtype="f16", B=3, Hq=2, Hkv=2, T=77), None, None),
]


@pytest.mark.parametrize("name,shape,batches,T", ENCODE_CASES, ids=[c[0] for c in ENCODE_CASES])
def test_encode_parity(K, oracle_mod, name, shape, batches, T):
    case = make_hlm_case(shape, batches=batches, T=T)
    log("encode", name, case["keys"].shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    codes, norms = _gpu_encode(K, cb, case["signs"], case["keys"])
    ref_codes, ref_norms, tie = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    n_diff, n_tie = _check_codes(oracle_mod, shape, codes.cpu().numpy(), norms.cpu().numpy(), ref_codes,
                                 ref_norms, tie)
    log("  codes differing %d, tie-band coordinates %d of %d" % (n_diff, n_tie, tie.size))


def test_encode_extreme_scales_and_non_finite_keys(K, oracle_mod):
    """fp32 keys scaled far from 1 take the correctly rounded norm and scale (sums of squares outside
    [2^-100, 2^100]) and still match the oracle.  Keys whose fp32 sum of squares overflows are encoded from
    their exact unit vector (the norm is +inf only where |k| itself exceeds fp32), and a key with an
    infinite or NaN coordinate gets the zero vector's codes and the norm its sum gives (+inf or NaN): the
    oracle's reading for keys the pages leave undefined.  The fused append encodes every such key the same
    way as the encode kernel."""
    import torch
    shape = W.scaled(W.LLAMA8B, B=2, Hq=8, Hkv=2, T=96, dtype="f32")
    case = make_hlm_case(shape)
    keys = case["keys"].astype(np.float32)
    keys[0, 0] *= np.float32(1e-18)   # sums of squares near 1e-34
    keys[0, 1] *= np.float32(1e17)    # sums of squares near 1e36
    keys[1, 0, :48] *= np.float32(2e-19)
    keys[1, 1, :40] *= np.float32(1e19)  # sums of squares near 1e40: past fp32, the norms are not
    cb = K.kvq_build_codebook(shape.d, shape.b)
    codes, norms = _gpu_encode(K, cb, case["signs"], keys)
    ref_codes, ref_norms, tie = oracle_cache(oracle_mod, shape, keys, case["signs"])
    assert np.all(np.isfinite(ref_norms))
    _check_codes(oracle_mod, shape, codes.cpu().numpy(), norms.cpu().numpy(), ref_codes, ref_norms, tie)

    bad = np.array(keys[:1, :1, :7])
    bad[0, 0, 0, 5] = np.inf
    bad[0, 0, 1, 9] = np.nan
    bad[0, 0, 2, :] = np.float32(3e38)  # sum and norm both overflow fp32: norm +inf, codes of the unit vector
    bad[0, 0, 3, 0] = -np.inf
    bad[0, 0, 4] = bad[0, 0, 4] * np.float32(3e18)  # the sum of squares overflows fp32, the norm does not
    bad[0, 0, 5, 3], bad[0, 0, 5, 4] = np.inf, np.nan
    bad[0, 0, 6, 100] = np.float32(-3.4e38)  # one huge coordinate among ordinary ones
    c_bad, n_bad = _gpu_encode(K, cb, case["signs"], bad)
    with np.errstate(over="ignore"):
        rc, rn, rtie = oracle_cache(oracle_mod, shape, bad, case["signs"])
    gc, gn = c_bad.cpu().numpy(), n_bad.cpu().numpy()
    n_diff, n_tie = _check_codes(oracle_mod, shape, gc, gn, rc, rn, rtie)
    log("  extreme keys: codes differing %d, tie-band coordinates %d" % (n_diff, n_tie))
    nb = gn[0, 0]
    assert np.isinf(nb[0]) and np.isnan(nb[1]) and np.isinf(nb[2]) and np.isinf(nb[3]) and np.isnan(nb[5])
    assert np.isfinite(nb[4]) and np.isfinite(nb[6])
    middle = oracle_mod.unpack_codes(gc[0, 0, [0, 1, 3, 5]], shape.d, shape.b)
    assert np.all(middle == 1 << (shape.b - 1))
    # the fused append encodes the same keys to the same codes and norms
    q = torch_dev(case["q"][:1, :4])
    cache_c = torch.zeros((1, 1, 8, cb.bytes_per_key), dtype=torch.uint8, device="cuda:0")
    cache_n = torch.zeros((1, 1, 8), dtype=torch.float32, device="cuda:0")
    v = torch.zeros((1, 1, 8, shape.d), dtype=torch.float16, device="cuda:0")
    for r in range(bad.shape[2]):
        nk = torch_dev(np.ascontiguousarray(bad[:, :, r, :]))
        K.kvq_decode_attn_append(cb, case["signs"], nk, q, cache_c, cache_n, v, seq_lens=torch.tensor(
            [r + 1], dtype=torch.int32, device="cuda:0"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cache_c[0, 0, :7].cpu().numpy(), gc[0, 0])
    np.testing.assert_array_equal(cache_n[0, 0, :7].cpu().numpy(), nb)


def test_encode_write_positions(K, oracle_mod):
    """Append at per-batch positions into a larger cache; rows outside the cache are skipped."""
    import torch
    shape = W.scaled(W.LLAMA8B, B=3, Hq=8, Hkv=2, T=5)
    case = make_hlm_case(shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    T_cap = 40
    pos = torch.tensor([0, 17, 37], dtype=torch.int32, device="cuda:0")  # the last one runs past T_cap
    codes, norms = _gpu_encode(K, cb, case["signs"], case["keys"], T_cap=T_cap, write_pos=pos)
    ref_codes, ref_norms, tie = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    for bi, p0 in enumerate([0, 17, 37]):
        n = min(5, T_cap - p0)
        _check_codes(oracle_mod, shape, gc[bi, :, p0:p0 + n], gn[bi, :, p0:p0 + n], ref_codes[bi, :, :n],
                     ref_norms[bi, :, :n], tie[bi, :, :n])
        untouched = np.ones(T_cap, bool)
        untouched[p0:p0 + n] = False
        assert np.all(gc[bi][:, untouched] == 0) and np.all(gn[bi][:, untouched] == 0)
    # one scalar position for every batch
    codes2, norms2 = _gpu_encode(K, cb, case["signs"], case["keys"], T_cap=T_cap, t0=35)
    gc2, gn2 = codes2.cpu().numpy(), norms2.cpu().numpy()
    _check_codes(oracle_mod, shape, gc2[:, :, 35:], gn2[:, :, 35:], ref_codes, ref_norms, tie)
    assert np.all(gc2[:, :, :35] == 0)
    # an empty append writes nothing
    empty = np.zeros((3, 2, 0, shape.d), dtype=np.float16)
    c3, n3 = _gpu_encode(K, cb, case["signs"], empty, T_cap=T_cap)
    assert int(c3.sum()) == 0 and float(n3.abs().sum()) == 0.0


def test_encode_zero_key(K, oracle_mod):
    shape = W.scaled(W.LONGCTX, B=1, Hq=1, Hkv=1, T=3)
    keys = np.zeros((1, 1, 3, 64), dtype=np.float16)
    keys[0, 0, 1] = 1.0
    cb = K.kvq_build_codebook(64, 4)
    s = W.signs(shape)
    codes, norms = _gpu_encode(K, cb, s, keys)
    ref_codes, ref_norms, tie = oracle_cache(oracle_mod, shape, keys, s)
    _check_codes(oracle_mod, shape, codes.cpu().numpy(), norms.cpu().numpy(), ref_codes, ref_norms, tie)
    assert float(norms[0, 0, 0]) == 0.0
    assert np.all(oracle_mod.unpack_codes(codes.cpu().numpy()[0, 0, 0], 64, 4) == 8)


SCORE_CASES = [
    ("tiny", W.TINY, None, None, None),
    ("llama8b", W.LLAMA8B, None, None, None),
    ("longctx_2b_T4000_ragged", W.LONGCTX, [1, 6], 4000, [4000, 1234]),
    ("sweep_b2", W.sweep(2, 1), None, 3000, None),
    ("sweep_b3_ragged_lens", W.scaled(W.sweep(3, 16), B=3), None, 700, [700, 0, 65]),
    ("d256_b1_G2", W.scaled(W.LLAMA8B, d=256, b=1, Hq=4, Hkv=2, T=500), None, None, None),
    ("d32_b3_G1", W.scaled(W.LLAMA8B, d=32, b=3, Hq=3, Hkv=3, T=129), None, None, None),
    ("d64_G6", W.scaled(W.LONGCTX, B=1, Hq=12, Hkv=2, T=300), None, None, None),
    ("d128_G16", W.scaled(W.LLAMA8B, Hq=32, Hkv=2, T=200), None, None, None),
    # query layouts of the read prologue below one wave per query (16 and 32 lanes per query), with the table
    # rows written by the prologue (b = 3, 4) at one, two and four heads per table entry
    ("d16_b4_G4", W.scaled(W.TINY, b=4, B=2, Hq=8, Hkv=2, T=150), None, None, None),
    ("d32_b4_G8", W.scaled(W.LLAMA8B, d=32, b=4, B=2, Hq=16, Hkv=2, T=260), None, None, None),
    ("d32_b3_G2", W.scaled(W.LLAMA8B, d=32, b=3, B=1, Hq=4, Hkv=2, T=130), None, None, None),
]


def _upload_cache(ref_codes, ref_norms):
    return torch_dev(ref_codes), torch_dev(ref_norms)


@pytest.mark.parametrize("name,shape,batches,T,lens", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_score_parity(K, oracle_mod, name, shape, batches, T, lens):
    import torch
    case = make_hlm_case(shape, batches=batches, T=T)
    log("score", name, case["keys"].shape)
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    codes, norms = _upload_cache(ref_codes, ref_norms)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    got = K.kvq_score(cb, case["signs"], torch_dev(case["q"]), codes, norms, seq_lens=sl)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    lv, _ = oracle_mod.codebook(shape.d, shape.b)
    ref = oracle_mod.scores(lv, case["signs"], case["q"], ref_codes, ref_norms, seq_lens=lens)
    G = shape.Hq // shape.Hkv
    tol = score_tolerance(case["q"], ref_norms, G)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(np.isneginf(got), np.isneginf(ref))
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= tol[fin]), "max excess %g" % float(np.max(err - tol[fin]))
    log("  max |ds|/(|q||k|) = %.3g" % float(np.max(err / (tol[fin] / 1e-4 + 1e-30))))


def test_score_heads_of_very_different_norms(K, oracle_mod):
    """Each query head's table has its own fixed-point scale: heads whose norms span 1e-4 .. 1e4 (fp32
    queries) and an all-zero head must each meet the per-head score bar; the zero head scores exactly 0."""
    import torch
    shape = W.scaled(W.LONGCTX, B=1, T=700)
    case = make_hlm_case(shape)
    q = case["q"].astype(np.float32)
    hs = np.logspace(-4, 4, shape.Hq).astype(np.float32)
    hs[5] = 0.0
    q = q * hs[None, :, None]
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    codes, norms = _upload_cache(ref_codes, ref_norms)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    got = K.kvq_score(cb, case["signs"], torch_dev(q), codes, norms)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    lv, _ = oracle_mod.codebook(shape.d, shape.b)
    ref = oracle_mod.scores(lv, case["signs"], q, ref_codes, ref_norms)
    tol = score_tolerance(q, ref_norms, shape.Hq // shape.Hkv)
    assert np.all(got[0, 5] == 0.0)
    err = np.abs(got - ref)
    assert np.all(err <= tol), "max excess %g" % float(np.max(err - tol))
    ratio = err / np.maximum(tol / 1e-4, 1e-30)
    log("  max |ds|/(|q||k|) over heads with norms 1e-4..1e4: %.3g" % float(ratio.max()))


DECODE_CASES = [
    # name, shape, batches, T, seq_lens, n_splits, out dtype
    ("tiny", W.TINY, None, None, None, 0, "f32"),
    ("tiny_split4", W.TINY, None, None, None, 4, "f32"),
    ("llama8b", W.LLAMA8B, None, None, None, 0, "f16"),
    ("llama8b_1split", W.LLAMA8B, None, None, None, 1, "f32"),
    ("longctx_2b_T5000", W.LONGCTX, [2, 3], 5000, None, 0, "f16"),
    ("longctx_ragged_lens", W.LONGCTX, [0, 1, 2], 3000, [3000, 0, 1], 7, "f16"),
    ("sweep_b2_T2000", W.sweep(2, 1), None, 2000, None, 0, "f16"),
    ("sweep_b3_T1111", W.sweep(3, 1), None, 1111, None, 3, "f16"),
    ("sweep_b4_B16_sample", W.sweep(4, 16), [4, 15], 1500, [1500, 999], 0, "f16"),
    ("d256_b2_G4", W.scaled(W.LLAMA8B, d=256, b=2, Hq=8, Hkv=2, T=700), None, None, None, 0, "f16"),
    ("d32_b1_G1_fp32v", W.scaled(W.TINY, d=32, b=1, B=2, Hq=2, Hkv=2, T=333), None, None, None, 0, "f32"),
    ("d64_G6", W.scaled(W.LONGCTX, B=1, Hq=12, Hkv=2, T=600), None, None, None, 0, "f16"),
    ("d128_G16", W.scaled(W.LLAMA8B, Hq=32, Hkv=2, T=300), None, None, None, 0, "f32"),
    ("d16_b4_G4", W.scaled(W.TINY, b=4, B=2, Hq=8, Hkv=2, T=150), None, None, None, 2, "f16"),
    ("d32_b4_G8", W.scaled(W.LLAMA8B, d=32, b=4, B=2, Hq=16, Hkv=2, T=260), None, None, [260, 77], 0, "f16"),
    ("d32_b3_G2_fp32v", W.scaled(W.TINY, d=32, b=3, B=1, Hq=4, Hkv=2, T=130), None, None, None, 0, "f32"),
]


@pytest.mark.parametrize("name,shape,batches,T,lens,n_splits,odt", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(K, oracle_mod, name, shape, batches, T, lens, n_splits, odt):
    import torch
    case = make_hlm_case(shape, batches=batches, T=T)
    log("decode", name, case["keys"].shape, "splits", n_splits)
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    codes, norms = _upload_cache(ref_codes, ref_norms)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    out_dtype = torch.float16 if odt == "f16" else torch.float32
    got = K.kvq_decode_attn(cb, case["signs"], torch_dev(case["q"]), codes, norms, torch_dev(case["v"]),
                            scale=scale_of(shape.d), seq_lens=sl, out_dtype=out_dtype, n_splits=n_splits)
    torch.cuda.synchronize()
    got = got.float().cpu().numpy()
    lv, _ = oracle_mod.codebook(shape.d, shape.b)
    ref = oracle_mod.decode_attn(lv, case["signs"], case["q"], ref_codes, ref_norms, case["v"], scale_of(shape.d),
                                 seq_lens=lens)
    err = rel_l2_rows(got, ref)
    log("  max rel L2 %.3g" % float(err.max()))
    assert np.all(err <= OUT_TOL)
    if lens is not None:
        for bi, n in enumerate(lens):
            if n == 0:
                assert np.all(got[bi] == 0)


def test_decode_same_result_for_every_split_count(K, oracle_mod):
    import torch
    shape = W.scaled(W.LONGCTX, B=1, T=8192)
    case = make_hlm_case(shape)
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    codes, norms = _upload_cache(ref_codes, ref_norms)
    cb = K.kvq_build_codebook(64, 4)
    outs = []
    # up to 128 splits of 64 tokens: the merging workgroup reads the partials in tiles of 32 splits
    for ns in (1, 2, 3, 8, 32, 33, 100, 128):
        outs.append(K.kvq_decode_attn(cb, case["signs"], torch_dev(case["q"]), codes, norms, torch_dev(case["v"]),
                                      out_dtype=torch.float32, n_splits=ns).cpu().numpy())
    # the probabilities enter the matrix cores as fp16 relative to each split's running maximum, so split
    # counts agree to fp16 rounding (~2^-11 relative), well inside the 2e-3 bar against the oracle
    for o in outs[1:]:
        assert np.max(rel_l2_rows(o, outs[0])) < 1e-3
    lv, _ = oracle_mod.codebook(64, 4)
    ref = oracle_mod.decode_attn(lv, case["signs"], case["q"], ref_codes, ref_norms, case["v"], scale_of(64))
    assert np.max(rel_l2_rows(outs[-1], ref)) <= OUT_TOL


def test_decode_twelve_wave_workgroups(K, oracle_mod):
    """Splits of 4096 tokens or more at d = 64 with fp16 V run 12-wave workgroups (three waves per SIMD): the
    same result as 8-wave workgroups (shorter splits) to fp16 rounding of the probabilities, and the oracle's."""
    import torch
    shape = W.LONGCTX
    case = make_hlm_case(shape, batches=[0, 6], T=8192)
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    codes, norms = _upload_cache(ref_codes, ref_norms)
    cb = K.kvq_build_codebook(64, 4)
    lens = [8192, 6001]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    outs = {}
    for ns in (2, 4):  # split_len 4096 (12 waves) and 2048 (8 waves)
        outs[ns] = K.kvq_decode_attn(cb, case["signs"], torch_dev(case["q"]), codes, norms, torch_dev(case["v"]),
                                     seq_lens=sl, out_dtype=torch.float32, n_splits=ns).cpu().numpy()
    assert np.max(rel_l2_rows(outs[2], outs[4])) < 1e-3
    lv, _ = oracle_mod.codebook(64, 4)
    ref = oracle_mod.decode_attn(lv, case["signs"], case["q"], ref_codes, ref_norms, case["v"], scale_of(64),
                                 seq_lens=lens)
    err = rel_l2_rows(outs[2], ref)
    log("  12-wave max rel L2 %.3g" % float(err.max()))
    assert np.all(err <= OUT_TOL)


def test_longctx_full_size_sampled(K, oracle_mod):
    """The bench workload at full size (B=8, T=32768) in the bench's launch configuration; sampled batches
    carry the oracle's codes and are compared against the oracle row by row."""
    import torch
    shape = W.LONGCTX
    log("longctx full size: generating")
    signs = W.signs(shape)
    q = W.queries(shape)
    keys = W.keys(shape)
    v = W.values(shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    codes, norms = _gpu_encode(K, cb, signs, keys)
    sample = [0, 5]
    lv, _ = oracle_mod.codebook(shape.d, shape.b)
    refs = {}
    for bi in sample:
        rc, rn, tie = oracle_cache(oracle_mod, shape, keys[bi:bi + 1], signs)
        # the GPU's own encode of this batch, against the oracle
        _check_codes(oracle_mod, shape, codes[bi:bi + 1].cpu().numpy(), norms[bi:bi + 1].cpu().numpy(), rc, rn, tie)
        codes[bi] = torch_dev(rc[0])
        norms[bi] = torch_dev(rn[0])
        refs[bi] = oracle_mod.decode_attn(lv, signs, q[bi:bi + 1], rc, rn, v[bi:bi + 1], scale_of(shape.d))
    vd = torch_dev(v)
    out = K.kvq_decode_attn(cb, signs, torch_dev(q), codes, norms, vd, out_dtype=torch.float16)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    for bi in sample:
        err = rel_l2_rows(out[bi:bi + 1], refs[bi])
        log("  batch %d max rel L2 %.3g" % (bi, float(err.max())))
        assert np.all(err <= OUT_TOL)
    assert np.all(np.isfinite(out))


def test_end_to_end_gpu_encode_then_attend(K, oracle_mod):
    """GPU encode -> GPU attention.  The GPU's codes match the oracle's outside the tie band, and its
    attention over those codes matches the oracle's attention over the same codes and norms within the
    2e-3 output bar (a tie-band code is a valid code; the oracle then attends over exactly what the GPU
    stored).  The distance to the oracle's own end-to-end result is logged."""
    import torch
    shape = W.scaled(W.LLAMA8B, T=2048)
    case = make_hlm_case(shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    codes, norms = _gpu_encode(K, cb, case["signs"], case["keys"])
    out = K.kvq_decode_attn(cb, case["signs"], torch_dev(case["q"]), codes, norms, torch_dev(case["v"]),
                            out_dtype=torch.float32).cpu().numpy()
    gc, gn = codes.cpu().numpy(), norms.cpu().numpy()
    ref_codes, ref_norms, tie = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    n_diff, n_tie = _check_codes(oracle_mod, shape, gc, gn, ref_codes, ref_norms, tie)
    lv, _ = oracle_mod.codebook(shape.d, shape.b)
    ref = oracle_mod.decode_attn(lv, case["signs"], case["q"], gc, gn, case["v"], scale_of(shape.d))
    err = rel_l2_rows(out, ref)
    ref_own = oracle_mod.decode_attn(lv, case["signs"], case["q"], ref_codes, ref_norms, case["v"], scale_of(shape.d))
    log("  end-to-end: %d tie-band codes differ; max rel L2 %.3g on the GPU's codes, %.3g against the oracle's "
        "own encode" % (n_diff, float(err.max()), float(rel_l2_rows(out, ref_own).max())))
    assert np.all(err <= OUT_TOL)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_sweep_batch64_full_geometry_sampled(K, oracle_mod, b):
    """The bit-width sweep's largest read: B=64, Hq=32, Hkv=8, d=128, T=8192 in the library's launch
    configuration for it (512 units, one split of 8192 keys each).  Batches 0, 31 and 63 hold the
    workload's seeded keys (the GPU's encode, checked against the oracle, then the oracle's codes) and
    values; the other batches hold random bytes.  Sampled batches are compared with the oracle row by row."""
    import torch
    shape = W.sweep(b, 64)
    assert (shape.B, shape.Hq, shape.Hkv, shape.d, shape.T) == (64, 32, 8, 128, 8192)
    sample = [0, 31, 63]
    log("sweep b=%d B=64 T=8192: generating sampled batches" % b)
    case = make_hlm_case(shape, batches=sample)
    cb = K.kvq_build_codebook(shape.d, b)
    assert K.kvq_decode_attn_workspace(cb, shape.B, shape.Hq, shape.Hkv, shape.T, 0) == 0  # one split
    g = torch.Generator(device="cuda:0")
    g.manual_seed(64 + b)
    dev = "cuda:0"
    codes = torch.randint(0, 256, (shape.B, shape.Hkv, shape.T, cb.bytes_per_key), dtype=torch.uint8, device=dev,
                          generator=g)
    norms = torch.rand((shape.B, shape.Hkv, shape.T), device=dev, generator=g) * 20
    v = torch.randn((shape.B, shape.Hkv, shape.T, shape.d), device=dev, generator=g).half()
    q = torch.randn((shape.B, shape.Hq, shape.d), device=dev, generator=g).half()
    gc, gn = _gpu_encode(K, cb, case["signs"], case["keys"])
    lv, _ = oracle_mod.codebook(shape.d, b)
    refs = {}
    for i, bi in enumerate(sample):
        rc, rn, tie = oracle_cache(oracle_mod, shape, case["keys"][i:i + 1], case["signs"])
        _check_codes(oracle_mod, shape, gc[i:i + 1].cpu().numpy(), gn[i:i + 1].cpu().numpy(), rc, rn, tie)
        codes[bi] = torch_dev(rc[0])
        norms[bi] = torch_dev(rn[0])
        v[bi] = torch_dev(case["v"][i])
        q[bi] = torch_dev(case["q"][i])
        refs[bi] = oracle_mod.decode_attn(lv, case["signs"], case["q"][i:i + 1], rc, rn, case["v"][i:i + 1],
                                          scale_of(shape.d))
    out = K.kvq_decode_attn(cb, case["signs"], q, codes, norms, v, out_dtype=torch.float16)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    assert np.all(np.isfinite(out))
    for bi in sample:
        err = rel_l2_rows(out[bi:bi + 1], refs[bi])
        log("  batch %d max rel L2 %.3g" % (bi, float(err.max())))
        assert np.all(err <= OUT_TOL)


# ------------------------------------------------------------------------------------------------
# Product quantization (LOOKAT-style ADC)
# ------------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def pq_case(oracle_mod):
    shape = W.PQ_GPT2
    train = W.pq_training(shape)
    start = W.pq_start_rows(shape)
    ds = shape.d // shape.m
    cent = np.zeros((shape.Hkv, shape.m, shape.K, ds))
    for h in range(shape.Hkv):
        for s in range(shape.m):
            cent[h, s], _ = oracle_mod.kmeans(train[h][:, s * ds:(s + 1) * ds], shape.K, 10, start[h, s])
    cent32 = cent.astype(np.float32)
    q = W.queries(shape)
    keys = W.keys(shape)
    v = W.values(shape)
    codes = np.zeros((shape.B, shape.Hkv, shape.T, shape.m), dtype=np.uint8)
    gaps = np.zeros((shape.B, shape.Hkv, shape.T, shape.m))
    for h in range(shape.Hkv):
        codes[:, h], gaps[:, h] = oracle_mod.pq_encode(cent32[h].astype(np.float64), keys[:, h])
    return dict(shape=shape, cent=cent32, q=q, keys=keys, v=v, codes=codes, gaps=gaps)


def _check_pq_codes(case, got, ref):
    """PQ codes [B][H][T][m] (one index per subspace) against the oracle's.  Tie band: the oracle's best two
    squared distances differ by less than 1e-6 |k_s|^2 (the GPU compares in fp32, the oracle in fp64).  Every
    differing code must lie in the band and be as near as the oracle's within it; the band is counted."""
    sh = case["shape"]
    ds = sh.d // sh.m
    k64 = case["keys"].astype(np.float64).reshape(got.shape[:3] + (sh.m, ds))
    band = 1e-6 * (k64 ** 2).sum(-1)
    in_band = case["gaps"] < band
    diff = np.argwhere(got != ref)
    log("  PQ codes differing: %d of %d; tie-band codes %d" % (len(diff), got.size, int(in_band.sum())))
    for b, h, t, s in diff:
        assert in_band[b, h, t, s], "PQ code outside the tie band differs at %s" % ((b, h, t, s),)
        c = case["cent"][h, s].astype(np.float64)
        dist = ((k64[b, h, t, s][None, :] - c) ** 2).sum(-1)
        assert dist[got[b, h, t, s]] - dist[ref[b, h, t, s]] <= band[b, h, t, s]


def test_pq_encode_parity(K, oracle_mod, pq_case):
    import torch
    sh = pq_case["shape"]
    cb = K.kvq_codebook_pq(sh.d, sh.m, sh.K, sh.Hkv, torch_dev(pq_case["cent"]))
    codes = torch.zeros((sh.B, sh.Hkv, sh.T, sh.m), dtype=torch.uint8, device="cuda:0")
    K.kvq_encode_keys(cb, None, torch_dev(pq_case["keys"]), codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    ref = pq_case["codes"]
    _check_pq_codes(pq_case, got, ref)


def test_pq_score_and_decode_parity(K, oracle_mod, pq_case):
    import torch
    sh = pq_case["shape"]
    cb = K.kvq_codebook_pq(sh.d, sh.m, sh.K, sh.Hkv, torch_dev(pq_case["cent"]))
    codes = torch_dev(pq_case["codes"])
    qd = torch_dev(pq_case["q"])
    cent64 = pq_case["cent"].astype(np.float64)
    got = K.kvq_score(cb, None, qd, codes).cpu().numpy()
    ref = oracle_mod.pq_scores(cent64, pq_case["q"], pq_case["codes"])
    # |q . k_hat| error bound: 1e-4 * |q| * |k_hat|
    khat_norm = np.zeros(pq_case["codes"].shape[:3])
    for h in range(sh.Hkv):
        for s in range(sh.m):
            khat_norm[:, h] += (cent64[h, s][pq_case["codes"][:, h, :, s]] ** 2).sum(-1)
    tol = 1e-4 * np.linalg.norm(pq_case["q"].astype(np.float64), axis=-1)[:, :, None] * np.sqrt(khat_norm)
    assert np.all(np.abs(got - ref) <= tol)
    lens = [1024, 0, 513, 64]
    refo = oracle_mod.pq_decode_attn(cent64, pq_case["q"], pq_case["codes"], pq_case["v"], scale_of(sh.d),
                                     seq_lens=lens)
    # the library's choice (one split at this length) and three splits (the split merge)
    for ns in (0, 3):
        out = K.kvq_decode_attn(cb, None, qd, codes, None, torch_dev(pq_case["v"]), scale=scale_of(sh.d),
                                seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                                out_dtype=torch.float32, n_splits=ns).cpu().numpy()
        err = rel_l2_rows(out, refo)
        log("  PQ decode (n_splits %d) max rel L2 %.3g" % (ns, float(err.max())))
        assert np.all(err <= OUT_TOL)
        assert np.all(out[1] == 0)


@pytest.fixture(scope="module", params=[W.PQ4_GPT2_32X, W.PQ4_GPT2_64X], ids=["pq4_32x", "pq4_64x"])
def pq4_case(request, oracle_mod):
    """4-bit centroid indices (K = 16), two subspaces per byte: centroids from the oracle's k-means, codes
    from the oracle's encode."""
    shape = request.param
    train = W.pq_training(shape)
    start = W.pq_start_rows(shape)
    ds = shape.d // shape.m
    cent = np.zeros((shape.Hkv, shape.m, shape.K, ds))
    for h in range(shape.Hkv):
        for s in range(shape.m):
            cent[h, s], _ = oracle_mod.kmeans(train[h][:, s * ds:(s + 1) * ds], shape.K, 10, start[h, s])
    cent32 = cent.astype(np.float32)
    keys = W.keys(shape)
    codes = np.zeros((shape.B, shape.Hkv, shape.T, shape.m // 2), dtype=np.uint8)
    gaps = np.zeros((shape.B, shape.Hkv, shape.T, shape.m))
    for h in range(shape.Hkv):
        codes[:, h], gaps[:, h] = oracle_mod.pq_encode(cent32[h].astype(np.float64), keys[:, h], bits=4)
    return dict(shape=shape, cent=cent32, q=W.queries(shape), keys=keys, v=W.values(shape), codes=codes, gaps=gaps)


def test_pq4_encode_parity(K, oracle_mod, pq4_case):
    import torch
    sh = pq4_case["shape"]
    cb = K.kvq_codebook_pq(sh.d, sh.m, sh.K, sh.Hkv, torch_dev(pq4_case["cent"]))
    assert cb.b == 4 and cb.bytes_per_key == sh.m // 2
    codes = torch.zeros((sh.B, sh.Hkv, sh.T, sh.m // 2), dtype=torch.uint8, device="cuda:0")
    K.kvq_encode_keys(cb, None, torch_dev(pq4_case["keys"]), codes)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    gi = np.stack([got & 15, got >> 4], axis=-1).reshape(got.shape[:3] + (sh.m,))
    ref = pq4_case["codes"]
    ri = np.stack([ref & 15, ref >> 4], axis=-1).reshape(ref.shape[:3] + (sh.m,))
    _check_pq_codes(pq4_case, gi, ri)


def test_pq4_score_and_decode_parity(K, oracle_mod, pq4_case):
    import torch
    sh = pq4_case["shape"]
    cb = K.kvq_codebook_pq(sh.d, sh.m, sh.K, sh.Hkv, torch_dev(pq4_case["cent"]))
    codes = torch_dev(pq4_case["codes"])
    qd = torch_dev(pq4_case["q"])
    cent64 = pq4_case["cent"].astype(np.float64)
    got = K.kvq_score(cb, None, qd, codes).cpu().numpy()
    ref = oracle_mod.pq_scores(cent64, pq4_case["q"], pq4_case["codes"], bits=4)
    c = pq4_case["codes"]
    idx = np.stack([c & 15, c >> 4], axis=-1).reshape(c.shape[:3] + (sh.m,))
    khat_norm = np.zeros(c.shape[:3])
    for h in range(sh.Hkv):
        for s in range(sh.m):
            khat_norm[:, h] += (cent64[h, s][idx[:, h, :, s]] ** 2).sum(-1)
    tol = 1e-4 * np.linalg.norm(pq4_case["q"].astype(np.float64), axis=-1)[:, :, None] * np.sqrt(khat_norm)
    assert np.all(np.abs(got - ref) <= tol)
    lens = [1024, 0, 700, 1]
    refo = oracle_mod.pq_decode_attn(cent64, pq4_case["q"], pq4_case["codes"], pq4_case["v"], scale_of(sh.d),
                                     seq_lens=lens, bits=4)
    for ns in (0, 2):  # the library's choice (one split) and two splits (the split merge)
        out = K.kvq_decode_attn(cb, None, qd, codes, None, torch_dev(pq4_case["v"]), scale=scale_of(sh.d),
                                seq_lens=torch.tensor(lens, dtype=torch.int32, device="cuda:0"),
                                out_dtype=torch.float32, n_splits=ns).cpu().numpy()
        err = rel_l2_rows(out, refo)
        log("  4-bit PQ decode (n_splits %d) max rel L2 %.3g" % (ns, float(err.max())))
        assert np.all(err <= OUT_TOL)
        assert np.all(out[1] == 0)
