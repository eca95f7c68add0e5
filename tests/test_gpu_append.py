"""The fused decode step (kvq_decode_attn_append): encode one new key per (batch, kv head) at position
len-1 and attend over [0, len) in one launch.

It must equal, bit for bit, the two-call sequence kvq_encode_keys(write_pos = len-1) + kvq_decode_attn
(same codes, same norms, same outputs), and agree with the oracle (codes outside the tie band, outputs
within 2e-3 relative L2 per row).
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
    ("d64_G6_two_groups", W.scaled(W.LONGCTX, B=2, Hq=12, Hkv=2, T=600), None, None, [600, 333], 0, "f16"),
    ("d256_b3", W.scaled(W.LONGCTX, d=256, b=3, B=2, Hq=4, Hkv=2, T=300), None, None, [300, 129], 0, "f16"),
    ("d32_b1_G1", W.scaled(W.TINY, d=32, b=1, B=2, Hq=2, Hkv=2, T=200, dtype="f16"), None, None, None, 0, "f16"),
    # the new key's codes packed by the whole wave (rows of whole words), and a row shorter than a word
    ("d16_b4_G4", W.scaled(W.TINY, b=4, B=2, Hq=8, Hkv=2, T=150), None, None, [150, 3], 0, "f32"),
    ("d128_b1_G4", W.scaled(W.LLAMA8B, b=1, B=2, T=700), None, None, [700, 65], 0, "f16"),
    ("d16_b1_short_row", W.scaled(W.TINY, b=1, B=2, Hq=2, Hkv=2, T=90), None, None, None, 0, "f32"),
    # splits of 4096 tokens: 12-wave workgroups
    ("longctx_long_splits", W.LONGCTX, [0, 5], 8192, [8192, 6001], 2, "f16"),
]


@pytest.mark.parametrize("name,shape,batches,T,lens,n_splits,odt", CASES, ids=[c[0] for c in CASES])
def test_append_equals_encode_then_attend(K, oracle_mod, name, shape, batches, T, lens, n_splits, odt):
    import torch
    case = make_hlm_case(shape, batches=batches, T=T)
    B, Hkv, T_cap, d = case["keys"].shape
    bsel = list(range(shape.B)) if batches is None else list(batches)
    newk = W.new_keys(shape)[bsel][:, :, 0, :]  # [B][Hkv][d]
    log("append", name, case["keys"].shape, "lens", lens, "splits", n_splits)
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    cb = K.kvq_build_codebook(d, shape.b)
    out_dtype = torch.float16 if odt == "f16" else torch.float32
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    lens_np = np.full(B, T_cap) if lens is None else np.array(lens)
    q, v, nk = torch_dev(case["q"]), torch_dev(case["v"]), torch_dev(newk)

    # two calls: encode at len-1 (skipped where len = 0), then attend
    codes_a, norms_a = torch_dev(ref_codes), torch_dev(ref_norms)
    wp = torch.tensor(lens_np - 1, dtype=torch.int32, device="cuda:0")
    K.kvq_encode_keys(cb, case["signs"], nk.unsqueeze(2).contiguous(), codes_a, norms_a, write_pos=wp)
    out_a = K.kvq_decode_attn(cb, case["signs"], q, codes_a, norms_a, v, scale=scale_of(d), seq_lens=sl,
                              out_dtype=out_dtype, n_splits=n_splits)
    # one fused call
    codes_b, norms_b = torch_dev(ref_codes), torch_dev(ref_norms)
    out_b = K.kvq_decode_attn_append(cb, case["signs"], nk, q, codes_b, norms_b, v, scale=scale_of(d), seq_lens=sl,
                                     out_dtype=out_dtype, n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(codes_a, codes_b), "fused append wrote different codes"
    assert torch.equal(norms_a, norms_b), "fused append wrote different norms"
    assert torch.equal(out_a, out_b), "fused append attends differently from encode + decode"

    # against the oracle: its own encode of the new keys at the same rows
    lv, th = oracle_mod.codebook(d, shape.b)
    nc, nn, _, ntie = oracle_mod.encode_keys(th, case["signs"], newk[:, :, None, :], shape.b)
    exp_codes, exp_norms = ref_codes.copy(), ref_norms.copy()
    got_codes = codes_b.cpu().numpy()
    for bi in range(B):
        if lens_np[bi] == 0:
            continue
        pos = min(int(lens_np[bi]), T_cap) - 1
        exp_codes[bi, :, pos] = nc[bi, :, 0]
        exp_norms[bi, :, pos] = nn[bi, :, 0].astype(np.float32)
        gi = oracle_mod.unpack_codes(got_codes[bi, :, pos], d, shape.b)
        ri = oracle_mod.unpack_codes(nc[bi, :, 0], d, shape.b)
        assert not np.any((gi != ri) & ~ntie[bi, :, 0]), "new-key codes differ from the oracle outside the tie band"
        np.testing.assert_allclose(norms_b.cpu().numpy()[bi, :, pos], nn[bi, :, 0], rtol=1e-5)
    # use the GPU's new-key codes (they may differ in the tie band) for the reference attention
    for bi in range(B):
        if lens_np[bi] > 0:
            pos = min(int(lens_np[bi]), T_cap) - 1
            exp_codes[bi, :, pos] = got_codes[bi, :, pos]
    ref = oracle_mod.decode_attn(lv, case["signs"], case["q"], exp_codes, exp_norms, case["v"], scale_of(d),
                                 seq_lens=lens)
    err = rel_l2_rows(out_b.float().cpu().numpy(), ref)
    log("  max rel L2 vs oracle %.3g" % float(err.max()))
    assert np.all(err <= OUT_TOL)
    # rows other than the new ones are untouched
    untouched = np.ones((B, Hkv, T_cap), dtype=bool)
    for bi in range(B):
        if lens_np[bi] > 0:
            untouched[bi, :, min(int(lens_np[bi]), T_cap) - 1] = False
    np.testing.assert_array_equal(got_codes[untouched], ref_codes[untouched])


@pytest.mark.parametrize("T,n_splits", [(2500, 0), (8192, 2)], ids=["8_waves", "12_waves"])
def test_append_graph_replays(K, oracle_mod, T, n_splits):
    """The fused step captured in a HIP graph: every replay (with eager work between) equals the eager call."""
    import torch
    shape = W.scaled(W.LONGCTX, B=2, T=T)
    case = make_hlm_case(shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    ref_codes, ref_norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    codes, norms = torch_dev(ref_codes), torch_dev(ref_norms)
    q, v = torch_dev(case["q"]), torch_dev(case["v"])
    nk = torch_dev(W.new_keys(shape)[:, :, 0, :])
    B, Hq, Hkv, T = shape.B, shape.Hq, shape.Hkv, shape.T
    ws = torch.zeros(max(K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, n_splits), 16), dtype=torch.uint8,
                     device="cuda:0")
    out = torch.empty((B, Hq, shape.d), dtype=torch.float16, device="cuda:0")

    def step():
        K.kvq_decode_attn_append(cb, case["signs"], nk, q, codes, norms, v, out=out, workspace=ws, n_splits=n_splits)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager, eager_codes = out.clone(), codes.clone()
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
        assert torch.equal(codes, eager_codes)
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0


POT_CASES = [
    # name, shape, batches, T, b, mantissa, seq_lens, n_splits, key dtype
    ("longctx_b4_ragged", W.LONGCTX, [0, 4, 7], 3000, 4, 0, [3000, 1, 1777], 0, np.float16),
    ("llama8b_b4_mant", W.LLAMA8B, None, 1500, 4, 1, None, 0, np.float16),
    ("d32_b3_fp32_len0", W.scaled(W.TINY, d=32, B=2, Hq=2, Hkv=2, T=200), None, None, 3, 1, [0, 200], 3, np.float32),
    ("d256_b2", W.scaled(W.LONGCTX, d=256, B=2, Hq=4, Hkv=2, T=300), None, None, 2, 0, [300, 129], 0, np.float16),
    ("longctx_long_splits", W.LONGCTX, [3, 4], 8192, 4, 1, [8192, 7000], 2, np.float16),
]


@pytest.mark.parametrize("name,shape,batches,T,b,mant,lens,n_splits,kdt", POT_CASES, ids=[c[0] for c in POT_CASES])
def test_pot_append_equals_encode_then_attend(K, oracle_mod, name, shape, batches, T, b, mant, lens, n_splits, kdt):
    """The fused step with power-of-two key codes: bit-identical to encode + decode, and the new keys' codes
    and scales are the oracle's."""
    import torch
    T = shape.T if T is None else T
    bsel = list(range(shape.B)) if batches is None else list(batches)
    keys = W.keys(shape, batches=bsel, T=T).astype(kdt)
    q, v = W.queries(shape)[bsel], W.values(shape, batches=bsel, T=T)
    newk = W.new_keys(shape)[bsel][:, :, 0, :].astype(kdt)
    B, Hkv, T_cap, d = keys.shape
    cb = K.kvq_build_codebook_pot(d, b, mant)
    ref_c, ref_s, _ = oracle_mod.pot_encode(keys, b, mant)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    lens_np = np.full(B, T_cap) if lens is None else np.array(lens)
    log("pot append", name, keys.shape, "b", b, "mantissa", mant, "lens", lens)
    qd, vd, nk = torch_dev(q), torch_dev(v), torch_dev(newk)
    codes_a, sc_a = torch_dev(ref_c), torch_dev(ref_s.astype(np.float32))
    wp = torch.tensor(lens_np - 1, dtype=torch.int32, device="cuda:0")
    K.kvq_encode_keys(cb, None, nk.unsqueeze(2).contiguous(), codes_a, sc_a, write_pos=wp)
    out_a = K.kvq_decode_attn(cb, None, qd, codes_a, sc_a, vd, seq_lens=sl, out_dtype=torch.float32, n_splits=n_splits)
    codes_b, sc_b = torch_dev(ref_c), torch_dev(ref_s.astype(np.float32))
    out_b = K.kvq_decode_attn_append(cb, None, nk, qd, codes_b, sc_b, vd, seq_lens=sl, out_dtype=torch.float32,
                                     n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(codes_a, codes_b) and torch.equal(sc_a, sc_b) and torch.equal(out_a, out_b)
    nc, ns, ntie = oracle_mod.pot_encode(newk[:, :, None, :], b, mant)
    got_c, got_s = codes_b.cpu().numpy(), sc_b.cpu().numpy()
    exp_c, exp_s = ref_c.copy(), ref_s.astype(np.float32)
    for bi in range(B):
        if lens_np[bi] == 0:
            continue
        pos = int(lens_np[bi]) - 1
        gi = oracle_mod.unpack_codes(got_c[bi, :, pos], d, b)
        ri = oracle_mod.unpack_codes(nc[bi, :, 0], d, b)
        assert not np.any((gi != ri) & ~ntie[bi, :, 0])
        np.testing.assert_array_equal(got_s[bi, :, pos], ns[bi, :, 0].astype(np.float32))
        exp_c[bi, :, pos] = got_c[bi, :, pos]
        exp_s[bi, :, pos] = got_s[bi, :, pos]
    ref = oracle_mod.pot_decode_attn(q, exp_c, exp_s, v, b, mant, scale_of(d), seq_lens=lens)
    err = rel_l2_rows(out_b.cpu().numpy(), ref)
    log("  max rel L2 vs oracle %.3g" % float(err.max()))
    assert np.all(err <= OUT_TOL)
