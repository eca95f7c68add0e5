"""kvq_stream_read, the plain read of a decode cache that measures the decode step's streaming ceiling.

It computes nothing of the method; the checks are that it runs on the shapes it is built for (including a
ragged token count and more splits than chunks), that it writes nothing (the caches and the guard regions
around them stay unchanged), and that it leaves the sink alone (it stores a checksum only if the checksum
equals one fixed value).
"""
import pytest

from helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,Hkv,d,T,n_splits", [(2, 2, 64, 4096, 8), (1, 3, 64, 1000, 4), (2, 1, 128, 777, 16),
                                                (1, 1, 64, 64, 256)])
def test_stream_read_runs_in_bounds(B, Hkv, d, T, n_splits):
    import torch
    import quantized_kv_cache_encode_amd.kvq as K

    dev = torch.device("cuda:0")
    bpk = d // 2
    g = torch.Generator(device=dev)
    g.manual_seed(B * 1000 + T)
    guard = 4096
    # one allocation per buffer with guard regions around the part the call is given
    cbuf = torch.randint(0, 256, (guard + B * Hkv * T * bpk + guard,), dtype=torch.uint8, device=dev, generator=g)
    nbuf = torch.rand((guard + B * Hkv * T + guard,), device=dev, generator=g)
    vbuf = torch.randn((guard + B * Hkv * T * d + guard,), device=dev, generator=g).half()
    cref, nref, vref = cbuf.clone(), nbuf.clone(), vbuf.clone()
    codes = cbuf[guard:guard + B * Hkv * T * bpk].view(B, Hkv, T, bpk)
    norms = nbuf[guard:guard + B * Hkv * T].view(B, Hkv, T)
    v = vbuf[guard:guard + B * Hkv * T * d].view(B, Hkv, T, d)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    log("stream read B=%d Hkv=%d d=%d T=%d splits=%d" % (B, Hkv, d, T, n_splits))
    for _ in range(3):
        K.kvq_stream_read(codes, norms, v, n_splits, sink)
    torch.cuda.synchronize()
    assert torch.equal(cbuf, cref) and torch.equal(nbuf, nref) and torch.equal(vbuf, vref)  # a read only
    assert int(sink.abs().sum()) == 0
