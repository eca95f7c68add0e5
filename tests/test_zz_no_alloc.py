"""The decode entry point that allocates nothing (kvq_decode_attn_noalloc, for callers that cannot allocate
device memory) against kvq_decode_attn with a caller workspace: same kernels and split choice, so the
outputs must agree bit for bit.  Two calls in a row, the second with a smaller input, then a shape whose
split partials exceed the static array (rejected before any launch), then one more call that must still be
right."""
import numpy as np
import pytest

import workloads as W
from helpers import log, make_hlm_case, oracle_cache, rel_l2_rows, scale_of, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import quantized_kv_cache_encode_amd.kvq as kvq
    return kvq


def _case(oracle_mod, shape, batches, T):
    case = make_hlm_case(shape, batches=batches, T=T)
    codes, norms, _ = oracle_cache(oracle_mod, shape, case["keys"], case["signs"])
    return case, codes, norms


def _both(K, cb, shape, case, codes, norms, lens, odt):
    import torch
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    q, c, n, v = torch_dev(case["q"]), torch_dev(codes), torch_dev(norms), torch_dev(case["v"])
    B, Hq = case["q"].shape[:2]
    out_na = torch.full((B, Hq, shape.d), float("nan"), dtype=odt, device="cuda:0")
    K.kvq_decode_attn_noalloc(cb, case["signs"], q, c, n, v, out_na, scale=scale_of(shape.d), seq_lens=sl)
    ref = K.kvq_decode_attn(cb, case["signs"], q, c, n, v, scale=scale_of(shape.d), seq_lens=sl, out_dtype=odt)
    torch.cuda.synchronize()
    return out_na.float().cpu().numpy(), ref.float().cpu().numpy()


def test_noalloc_matches_decode_attn_on_two_calls(K, oracle_mod):
    import torch
    lv, _ = oracle_mod.codebook(64, 4)
    cb = K.kvq_build_codebook(64, 4)
    # first call: 4 batches x 4 kv heads x 8 query heads each, T = 6000 (several splits per unit)
    sh1 = W.LONGCTX
    case1, codes1, norms1 = _case(oracle_mod, sh1, [0, 1, 2, 3], 6000)
    ws_need = K.kvq_decode_attn_workspace(cb, 4, sh1.Hq, sh1.Hkv, 6000, 0)
    log("noalloc call 1: B=4 T=6000, workspace the shape needs %d bytes" % ws_need)
    assert ws_need > 0
    got, ref = _both(K, cb, sh1, case1, codes1, norms1, None, torch.float16)
    np.testing.assert_array_equal(got, ref)
    o1 = oracle_mod.decode_attn(lv, case1["signs"], case1["q"], codes1, norms1, case1["v"], scale_of(64))
    assert np.max(rel_l2_rows(got, o1)) <= 2e-3
    # second call, smaller: 2 batches, T = 1000 with ragged lengths (one empty), fp32 output
    case2, codes2, norms2 = _case(oracle_mod, sh1, [4, 5], 1000)
    lens = [777, 0]
    log("noalloc call 2: B=2 T=1000 lens", lens)
    got2, ref2 = _both(K, cb, sh1, case2, codes2, norms2, lens, torch.float32)
    np.testing.assert_array_equal(got2, ref2)
    assert np.all(got2[1] == 0)
    o2 = oracle_mod.decode_attn(lv, case2["signs"], case2["q"], codes2, norms2, case2["v"], scale_of(64),
                                seq_lens=lens)
    assert np.max(rel_l2_rows(got2[:1], o2[:1])) <= 2e-3


def test_noalloc_rejects_shapes_beyond_its_scratch(K, oracle_mod):
    import torch
    cb = K.kvq_build_codebook(64, 4)
    # 256 splits of 64 tokens for 64 x 32 query heads: 64*32*256*68*4 bytes of partials, far above 4 MiB
    B, Hq, Hkv, T = 64, 32, 4, 256 * 64
    need = K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, 256)
    log("oversized shape needs %d bytes" % need)
    assert need > (4 << 20)
    q = torch.zeros((B, Hq, 64), dtype=torch.float16, device="cuda:0")
    codes = torch.zeros((1, 1, 1, 32), dtype=torch.uint8, device="cuda:0")  # never read: validation fails first
    out = torch.zeros((B, Hq, 64), dtype=torch.float16, device="cuda:0")
    import ctypes
    st = K._lib.kvq_decode_attn_noalloc(ctypes.byref(cb), W.signs(W.LONGCTX).ctypes.data_as(ctypes.c_void_p),
                                        ctypes.c_void_p(q.data_ptr()), K.KVQ_F16, ctypes.c_void_p(codes.data_ptr()),
                                        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(codes.data_ptr()),
                                        K.KVQ_F16, B, Hq, Hkv, T, None, 0.125, ctypes.c_void_p(out.data_ptr()),
                                        K.KVQ_F16, 256, None)
    assert st == K.KVQ_ERR_WORKSPACE
    assert "scratch" in K.kvq_last_error()
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    # the library's array is still usable afterwards
    sh = W.LONGCTX
    case, codes_np, norms_np = _case(oracle_mod, sh, [7], 3000)
    got, ref = _both(K, cb, sh, case, codes_np, norms_np, [2999], torch.float16)
    np.testing.assert_array_equal(got, ref)
