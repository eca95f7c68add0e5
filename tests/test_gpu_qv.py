"""Decode attention with quantized values (kvq_decode_attn_qv) against the oracle.

Keys and values are both encoded by the oracle (the same codes feed both sides), so the test isolates the
read path: scores on the matrix cores from fp16 code levels against a hi/lo-split rotated query, the
rotated-domain weighted sum of the value levels, the split merge and the single inverse transform per head.
Bar: 2e-3 relative L2 per output row, as for kvq_decode_attn.
"""
import numpy as np
import pytest

import workloads as W
from helpers import log, make_hlm_case, oracle_cache, rel_l2_rows, scale_of, torch_dev

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import quantized_kv_cache_encode_amd.kvq as kvq
    return kvq


CASES = [
    # name, shape, batches, T, seq_lens, n_splits, out dtype
    ("tiny_fp32", W.TINY, None, None, None, 0, "f32"),
    ("tiny_split3", W.TINY, None, None, None, 3, "f32"),
    ("llama8b_T1500", W.LLAMA8B, None, 1500, None, 0, "f16"),
    ("longctx_ragged", W.LONGCTX, [0, 4, 7], 3000, [3000, 1, 1777], 0, "f16"),
    ("longctx_len0_and_1split", W.LONGCTX, [1, 2], 700, [0, 700], 1, "f32"),
    ("sweep_b3", W.sweep(3, 1), None, 1111, None, 0, "f16"),
    ("sweep_b2_lens", W.scaled(W.sweep(2, 16), B=2), None, 900, [900, 64], 5, "f16"),
    ("d64_b2_G6", W.scaled(W.LONGCTX, b=2, B=2, Hq=12, Hkv=2, T=600), None, None, [600, 333], 0, "f16"),
    ("d64_b1_G2", W.scaled(W.LONGCTX, b=1, B=2, Hq=4, Hkv=2, T=500), None, None, [500, 77], 0, "f32"),
    ("d64_b3", W.scaled(W.LONGCTX, b=3, B=1, Hq=8, Hkv=1, T=450), None, None, None, 2, "f16"),
    ("d128_b1", W.scaled(W.LLAMA8B, b=1, T=300), None, None, None, 0, "f16"),
    ("d256_b3", W.scaled(W.LONGCTX, d=256, b=3, B=2, Hq=4, Hkv=2, T=300), None, None, [300, 129], 0, "f16"),
    ("d256_b4", W.scaled(W.LONGCTX, d=256, b=4, B=1, Hq=8, Hkv=1, T=520), None, None, None, 0, "f32"),
    ("d32_b1_G1", W.scaled(W.TINY, d=32, b=1, B=2, Hq=2, Hkv=2, T=200, dtype="f16"), None, None, None, 0, "f16"),
    ("d32_b4", W.scaled(W.TINY, d=32, b=4, B=1, Hq=4, Hkv=4, T=130, dtype="f16"), None, None, None, 0, "f16"),
    ("d16_b3", W.scaled(W.TINY, d=16, b=3, B=1, Hq=2, Hkv=1, T=100), None, None, None, 0, "f32"),
    ("d16_b1_G4", W.scaled(W.TINY, d=16, b=1, B=2, Hq=8, Hkv=2, T=333), None, None, [333, 200], 2, "f32"),
    ("d16_b4", W.scaled(W.TINY, d=16, b=4, B=1, Hq=1, Hkv=1, T=77), None, None, None, 0, "f16"),
]


def _value_cache(oracle_mod, shape, v, signs):
    lv, th = oracle_mod.codebook(shape.d, shape.b)
    vc, vn, _, _ = oracle_mod.encode_keys(th, signs, v, shape.b)
    return vc, vn.astype(np.float32)


@pytest.mark.parametrize("name,shape,batches,T,lens,n_splits,odt", CASES, ids=[c[0] for c in CASES])
def test_decode_qv_vs_oracle(K, oracle_mod, name, shape, batches, T, lens, n_splits, odt):
    import torch
    case = make_hlm_case(shape, batches=batches, T=T)
    B, Hkv, T_cap, d = case["keys"].shape
    log("qv", name, case["keys"].shape, "Hq", shape.Hq, "b", shape.b, "lens", lens, "splits", n_splits)
    codes, norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    vcodes, vnorms = _value_cache(oracle_mod, shape, case["v"], case["signs"])
    cb = K.kvq_build_codebook(d, shape.b)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    out = K.kvq_decode_attn_qv(cb, case["signs"], torch_dev(case["q"]), torch_dev(codes), torch_dev(norms),
                               torch_dev(vcodes), torch_dev(vnorms), scale=scale_of(d), seq_lens=sl,
                               out_dtype=torch.float16 if odt == "f16" else torch.float32, n_splits=n_splits)
    torch.cuda.synchronize()
    lv, _ = oracle_mod.codebook(d, shape.b)
    ref = oracle_mod.decode_attn_qv(lv, case["signs"], case["q"], codes, norms, vcodes, vnorms, scale_of(d),
                                    seq_lens=lens)
    got = out.float().cpu().numpy()
    err = rel_l2_rows(got, ref)
    log("  max rel L2 vs oracle %.3g" % float(err.max()))
    assert np.all(np.isfinite(got))
    assert np.all(err <= OUT_TOL)
    if lens is not None:
        for bi, n in enumerate(lens):
            if n == 0:
                assert np.all(got[bi] == 0.0)


def test_decode_qv_split_invariance(K, oracle_mod):
    """The same cache with 1, 7 and the library's number of splits: outputs agree to the fp16 P rounding."""
    import torch
    shape = W.scaled(W.LONGCTX, B=2, T=5000)
    case = make_hlm_case(shape)
    codes, norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    vcodes, vnorms = _value_cache(oracle_mod, shape, case["v"], case["signs"])
    cb = K.kvq_build_codebook(shape.d, shape.b)
    args = (torch_dev(case["q"]), torch_dev(codes), torch_dev(norms), torch_dev(vcodes), torch_dev(vnorms))
    outs = [K.kvq_decode_attn_qv(cb, case["signs"], *args, out_dtype=torch.float32, n_splits=s).cpu().numpy()
            for s in (1, 7, 0)]
    for o in outs[1:]:
        assert np.all(rel_l2_rows(o, outs[0]) <= 1e-3)


def test_decode_qv_full_longctx_sampled(K, oracle_mod):
    """The full long-context cache (B=8, T=32768) in the library's launch configuration; the oracle checks
    every head of two sampled batches (its own encode of those batches' keys and values)."""
    import torch
    shape = W.LONGCTX
    signs = W.signs(shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    B, Hkv, T, d = shape.B, shape.Hkv, shape.T, shape.d
    codes = torch.empty((B, Hkv, T, cb.bytes_per_key), dtype=torch.uint8, device="cuda:0")
    norms = torch.empty((B, Hkv, T), dtype=torch.float32, device="cuda:0")
    vcodes, vnorms = torch.empty_like(codes), torch.empty_like(norms)
    for bi in range(B):  # GPU encode of keys and values, one batch at a time
        kb = torch_dev(W.keys(shape, batches=[bi]))
        vb = torch_dev(W.values(shape, batches=[bi]))
        K.kvq_encode_keys(cb, signs, kb, codes[bi:bi + 1], norms[bi:bi + 1])
        K.kvq_encode_keys(cb, signs, vb, vcodes[bi:bi + 1], vnorms[bi:bi + 1])
    q = W.queries(shape)
    out = K.kvq_decode_attn_qv(cb, signs, torch_dev(q), codes, norms, vcodes, vnorms, out_dtype=torch.float16)
    torch.cuda.synchronize()
    lv, _ = oracle_mod.codebook(d, shape.b)
    for bi in (3, 6):
        ref = oracle_mod.decode_attn_qv(lv, signs, q[bi:bi + 1], codes[bi:bi + 1].cpu().numpy(),
                                        norms[bi:bi + 1].cpu().numpy(), vcodes[bi:bi + 1].cpu().numpy(),
                                        vnorms[bi:bi + 1].cpu().numpy(), scale_of(d))
        err = rel_l2_rows(out[bi:bi + 1].float().cpu().numpy(), ref)
        log("  batch %d: max rel L2 %.3g" % (bi, float(err.max())))
        assert np.all(err <= OUT_TOL)


def test_decode_qv_graph_replays(K, oracle_mod):
    """Captured in a HIP graph: every replay (with eager work between) equals the eager call."""
    import torch
    shape = W.scaled(W.LONGCTX, B=2, T=2500)
    case = make_hlm_case(shape)
    codes, norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    vcodes, vnorms = _value_cache(oracle_mod, shape, case["v"], case["signs"])
    cb = K.kvq_build_codebook(shape.d, shape.b)
    B, Hq, Hkv, T = shape.B, shape.Hq, shape.Hkv, shape.T
    ws = torch.zeros(max(K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, 0), 16), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, Hq, shape.d), dtype=torch.float16, device="cuda:0")
    args = (torch_dev(case["q"]), torch_dev(codes), torch_dev(norms), torch_dev(vcodes), torch_dev(vnorms))

    def step():
        K.kvq_decode_attn_qv(cb, case["signs"], *args, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda:0").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("replay %d: junk %.3f" % (r, float(junk)))
        assert torch.equal(out, eager)
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0
