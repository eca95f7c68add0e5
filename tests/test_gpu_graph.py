"""The write + read path captured in a HIP graph and replayed: every replay must equal the eager result.

Replays are interleaved with the program's own eager work and synchronizations, and the split-merge
arrival counters (which each call leaves at zero) are exercised across replays.
"""
import numpy as np
import pytest

import workloads as W
from helpers import log, torch_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    import quantized_kv_cache_encode_amd.kvq as K

    shape = W.scaled(W.LONGCTX, B=2, T=3000)  # several splits per (b, kv head) and a ragged tail
    signs = W.signs(shape)
    cb = K.kvq_build_codebook(shape.d, shape.b)
    keys = torch_dev(W.keys(shape))
    q = torch_dev(W.queries(shape))
    v = torch_dev(W.values(shape))
    newk = torch_dev(W.new_keys(shape))
    B, Hq, Hkv, d, T = shape.B, shape.Hq, shape.Hkv, shape.d, shape.T
    codes = torch.zeros((B, Hkv, T, cb.bytes_per_key), dtype=torch.uint8, device="cuda:0")
    norms = torch.zeros((B, Hkv, T), dtype=torch.float32, device="cuda:0")
    K.kvq_encode_keys(cb, signs, keys, codes, norms)
    ws = torch.zeros(K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, 0), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, Hq, d), dtype=torch.float16, device="cuda:0")

    def step():
        K.kvq_encode_keys(cb, signs, newk, codes, norms, t0=T - 1)
        K.kvq_decode_attn(cb, signs, q, codes, norms, v, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    eager_codes = codes.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda:0").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("replay %d: junk %.3f" % (r, float(junk)))
        assert torch.equal(out, eager), "replay %d differs from the eager result" % r
        assert torch.equal(codes, eager_codes)
    assert int(ws[:256].view(torch.int32).abs().sum()) == 0, "arrival counters not left at zero"


@pytest.mark.parametrize("codec", ["pot", "pq4", "pq8"])
def test_graph_replays_match_eager_other_codecs(codec):
    """The power-of-two, 4-bit PQ and byte-code PQ paths (encode of the step's key + decode) replayed from a
    graph; the byte-code encode of one key runs the matrix-core kernel with one valid key in its workgroup."""
    import torch
    import quantized_kv_cache_encode_amd.kvq as K

    dev = "cuda:0"
    if codec == "pot":
        shape = W.scaled(W.LONGCTX, B=2, T=3000)
        cb = K.kvq_build_codebook_pot(shape.d, 4, 1)
    else:
        shape = W.scaled(W.PQ4_GPT2_32X if codec == "pq4" else W.PQ_GPT2, B=2, T=2000)
        g0 = torch.Generator(device=dev)
        g0.manual_seed(4)
        cent = torch.randn((shape.Hkv, shape.m, shape.K, shape.d // shape.m), device=dev, generator=g0)
        cb = K.kvq_codebook_pq(shape.d, shape.m, shape.K, shape.Hkv, cent)
    B, Hq, Hkv, d, T = shape.B, shape.Hq, shape.Hkv, shape.d, shape.T
    keys = torch_dev(W.keys(shape))
    q = torch_dev(W.queries(shape))
    v = torch_dev(W.values(shape))
    newk = keys[:, :, -1:, :].contiguous() * 0.5
    codes = torch.zeros((B, Hkv, T, cb.bytes_per_key), dtype=torch.uint8, device=dev)
    norms = torch.zeros((B, Hkv, T), dtype=torch.float32, device=dev) if codec == "pot" else None
    K.kvq_encode_keys(cb, None, keys, codes, norms)
    ws = torch.zeros(max(16, K.kvq_decode_attn_workspace(cb, B, Hq, Hkv, T, 0)), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)

    def step():
        K.kvq_encode_keys(cb, None, newk, codes, norms, t0=T - 1)
        K.kvq_decode_attn(cb, None, q, codes, norms, v, out=out, workspace=ws)

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
    for r in range(3):
        out.zero_()
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("%s replay %d: junk %.3f" % (codec, r, float(junk)))
        assert torch.equal(out, eager), "replay %d differs from the eager result" % r
