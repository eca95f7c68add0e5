"""CPU checks of the library's host side: it loads, exports every symbol the
header declares, builds the same codebooks as the oracle, and rejects bad
arguments before launching anything (fake, never-dereferenced pointers are
used only where validation must fail first)."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    from quantized_kv_cache_encode_amd import build
    if build.is_stale():
        build.build()
    import quantized_kv_cache_encode_amd.kvq as kvq
    return kvq


def test_exports_every_declared_symbol(K):
    import glob
    hdr = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kvq_[a-z_0-9]+)\s*\(", hdr, flags=re.M))
    assert declared >= {"kvq_build_codebook", "kvq_encode_keys", "kvq_score", "kvq_decode_attn"}
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(K.EXPORTS)


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_codebook_matches_oracle(K, oracle_mod, d, b):
    cb = K.kvq_build_codebook(d, b)
    lv, th = oracle_mod.codebook(d, b)
    np.testing.assert_array_equal(cb.levels_array(), lv.astype(np.float32))
    np.testing.assert_array_equal(cb.thresholds_array(), th.astype(np.float32))
    assert cb.kind == K.KVQ_HADAMARD_LM and cb.d == d and cb.b == b


def test_pq_kmeans_matches_oracle(K, oracle_mod):
    sh = W.scaled(W.PQ_GPT2, Hkv=2, Hq=2, K=64)
    train = W.pq_training(sh, n_train=1024)
    start = W.pq_start_rows(sh, n_train=1024)
    cent = K.kvq_build_codebook_pq(train, sh.m, sh.K, 10, start)
    ds = sh.d // sh.m
    for h in range(sh.Hkv):
        for s in range(sh.m):
            ref, _ = oracle_mod.kmeans(train[h][:, s * ds:(s + 1) * ds], sh.K, 10, start[h, s])
            np.testing.assert_allclose(cent[h, s], ref, rtol=1e-6, atol=1e-6)


def test_version_and_last_error(K):
    assert K.kvq_version() >= 100
    with pytest.raises(K.KvqError) as e:
        K.kvq_build_codebook(48, 4)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG
    assert "d=48" in K.kvq_last_error()
    K.kvq_build_codebook(64, 4)
    assert K.kvq_last_error() == ""


@pytest.mark.parametrize("d,b", [(8, 2), (24, 2), (512, 4), (64, 0), (64, 5)])
def test_codebook_rejects(K, d, b):
    with pytest.raises(K.KvqError) as e:
        K.kvq_build_codebook(d, b)
    assert e.value.status == K.KVQ_ERR_INVALID_ARG


FAKE = 0x100000  # aligned, never dereferenced: every call below must fail validation first


def _raw(K):
    return ctypes.CDLL(K.LIB_PATH)


def _call_encode(K, cb, signs, keys=FAKE, kdt=1, B=1, H=1, T_new=4, codes=FAKE, norms=FAKE, T_cap=64, t0=0, wp=None):
    lib = K._lib
    s = None if signs is None else np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
    return lib.kvq_encode_keys(ctypes.byref(cb), None if s is None else s.ctypes.data_as(ctypes.c_void_p),
                               ctypes.c_void_p(keys), kdt, B, H, T_new, ctypes.c_void_p(codes),
                               None if norms is None else ctypes.c_void_p(norms), T_cap, t0,
                               None if wp is None else ctypes.c_void_p(wp), None)


def test_encode_validation(K):
    cb = K.kvq_build_codebook(16, 2)
    ok_signs = np.ones(16, dtype=np.int8)
    bad = np.ones(16, dtype=np.int8)
    bad[3] = 0
    assert _call_encode(K, cb, bad) == K.KVQ_ERR_INVALID_ARG
    assert "signs[3]" in K.kvq_last_error()
    assert _call_encode(K, cb, None) == K.KVQ_ERR_INVALID_ARG
    assert _call_encode(K, cb, ok_signs, keys=FAKE + 2) == K.KVQ_ERR_INVALID_ARG          # misaligned
    assert _call_encode(K, cb, ok_signs, codes=0) == K.KVQ_ERR_INVALID_ARG                # NULL codes
    assert _call_encode(K, cb, ok_signs, norms=None) == K.KVQ_ERR_INVALID_ARG             # NULL norms
    assert _call_encode(K, cb, ok_signs, kdt=7) == K.KVQ_ERR_INVALID_ARG                  # dtype
    assert _call_encode(K, cb, ok_signs, T_cap=0) == K.KVQ_ERR_INVALID_ARG
    assert _call_encode(K, cb, ok_signs, t0=62, T_new=4) == K.KVQ_ERR_INVALID_ARG         # does not fit
    assert _call_encode(K, cb, ok_signs, t0=-1) == K.KVQ_ERR_INVALID_ARG
    assert _call_encode(K, cb, ok_signs, B=0) == K.KVQ_ERR_INVALID_ARG
    bad_cb = K.kvq_build_codebook(16, 2)
    bad_cb.b = 5
    assert _call_encode(K, bad_cb, ok_signs) == K.KVQ_ERR_INVALID_ARG
    bad_cb.b, bad_cb.d = 2, 20
    assert _call_encode(K, bad_cb, ok_signs) == K.KVQ_ERR_INVALID_ARG
    bad_cb.kind = 9
    assert _call_encode(K, bad_cb, ok_signs) == K.KVQ_ERR_INVALID_ARG


def _call_decode(K, cb, signs, B=1, Hq=4, Hkv=2, T_cap=4096, ws=FAKE, ws_bytes=0, n_splits=0, q=FAKE, scale=0.25,
                 vdt=1, odt=1):
    lib = K._lib
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.int8))
    P = ctypes.c_void_p
    return lib.kvq_decode_attn(ctypes.byref(cb), s.ctypes.data_as(P), P(q), 1, P(FAKE), P(FAKE), P(FAKE), vdt, B,
                               Hq, Hkv, T_cap, None, scale, P(FAKE), odt, None if ws is None else P(ws), ws_bytes,
                               n_splits, None)


def test_decode_validation_and_workspace(K):
    cb = K.kvq_build_codebook(64, 4)
    s = np.ones(64, dtype=np.int8)
    assert _call_decode(K, cb, s, Hq=3, Hkv=2) == K.KVQ_ERR_INVALID_ARG       # Hq % Hkv
    assert _call_decode(K, cb, s, T_cap=0) == K.KVQ_ERR_INVALID_ARG
    assert _call_decode(K, cb, s, q=FAKE + 8) == K.KVQ_ERR_INVALID_ARG
    assert _call_decode(K, cb, s, vdt=5) == K.KVQ_ERR_INVALID_ARG
    assert _call_decode(K, cb, s, n_splits=-1) == K.KVQ_ERR_INVALID_ARG
    assert _call_decode(K, cb, s, scale=float("nan")) == K.KVQ_ERR_INVALID_ARG
    need = K.kvq_decode_attn_workspace(cb, 1, 4, 2, 4096, 0)
    assert need > 0
    assert _call_decode(K, cb, s, ws=None, ws_bytes=0) == K.KVQ_ERR_WORKSPACE
    assert _call_decode(K, cb, s, ws_bytes=need - 1) == K.KVQ_ERR_WORKSPACE
    assert "workspace" in K.kvq_last_error()
    # one split needs no workspace
    assert K.kvq_decode_attn_workspace(cb, 1, 4, 2, 64, 0) == 0
    assert K.kvq_decode_attn_workspace(cb, 1, 4, 2, 4096, 1) == 0
    # workspace grows with the requested split count, and is 0 for invalid shapes
    assert K.kvq_decode_attn_workspace(cb, 1, 4, 2, 4096, 64) == 256 + 1 * 4 * 64 * (64 + 4) * 4  # counters + partials
    assert K.kvq_decode_attn_workspace(cb, 1, 3, 2, 4096, 0) == 0


def test_score_validation(K):
    cb = K.kvq_build_codebook(64, 4)
    s = np.ones(64, dtype=np.int8)
    P = ctypes.c_void_p
    lib = K._lib
    # NULL scores
    assert lib.kvq_score(ctypes.byref(cb), s.ctypes.data_as(P), P(FAKE), 1, P(FAKE), P(FAKE), 1, 4, 2, 128, None,
                         None, None) == K.KVQ_ERR_INVALID_ARG
    # NULL norms for the Hadamard codec
    assert lib.kvq_score(ctypes.byref(cb), s.ctypes.data_as(P), P(FAKE), 1, P(FAKE), None, 1, 4, 2, 128, None,
                         P(FAKE), None) == K.KVQ_ERR_INVALID_ARG


def test_pq_codebook_validation(K):
    with pytest.raises(K.KvqError):
        K._check(K._lib.kvq_codebook_pq(64, 7, 256, 12, ctypes.c_void_p(FAKE), ctypes.byref(K.kvq_codebook())))
    with pytest.raises(K.KvqError):
        K._check(K._lib.kvq_codebook_pq(64, 8, 300, 12, ctypes.c_void_p(FAKE), ctypes.byref(K.kvq_codebook())))
    with pytest.raises(K.KvqError):
        K.kvq_build_codebook_pq(np.zeros((1, 10, 8), np.float32), 2, 4, 3, np.full((1, 2, 4), 11))


def test_append_validation(K):
    import ctypes
    P = ctypes.c_void_p
    cb = K.kvq_build_codebook(64, 4)
    s = np.ones(64, dtype=np.int8)
    lib = K._lib

    def call(cbx, new_keys=FAKE, kdt=1):
        return lib.kvq_decode_attn_append(ctypes.byref(cbx), s.ctypes.data_as(P), None if new_keys is None else P(new_keys),
                                          kdt, P(FAKE), 1, P(FAKE), P(FAKE), P(FAKE), 1, 1, 4, 2, 64, None, 0.125,
                                          P(FAKE), 1, None, 0, 0, None)
    assert call(cb, new_keys=None) == K.KVQ_ERR_INVALID_ARG
    assert "new_keys" in K.kvq_last_error()
    assert call(cb, new_keys=FAKE + 4) == K.KVQ_ERR_INVALID_ARG
    assert call(cb, kdt=3) == K.KVQ_ERR_INVALID_ARG
    pq = K.kvq_codebook()
    K._check(lib.kvq_codebook_pq(64, 8, 256, 2, P(FAKE), ctypes.byref(pq)))
    assert call(pq) == K.KVQ_ERR_UNSUPPORTED
    assert "scalar codecs" in K.kvq_last_error()


def test_pq_decode_split_rule(K):
    """PQ decode splits the token axis less than the scalar codecs (every split rebuilds the head's whole
    table): at least 2048 tokens per split and no extra splits to fill the device.  Checked through the
    workspace query, which sizes the split merge for the same choice the launch makes (no workspace for one
    split)."""
    pq = K.kvq_codebook()
    K._check(K._lib.kvq_codebook_pq(64, 8, 256, 12, ctypes.c_void_p(FAKE), ctypes.byref(pq)))
    ws = lambda T, ns: K.kvq_decode_attn_workspace(pq, 4, 12, 12, T, ns)
    assert ws(1024, 0) == ws(1024, 1) == 0
    assert ws(2048, 0) == 0
    assert ws(4096, 0) == ws(4096, 2) > 0
    assert ws(1024, 4) > 0  # an explicit request still splits
    # the Hadamard codec still splits a short cache over the device
    hlm = K.kvq_build_codebook(128, 4)
    assert K.kvq_decode_attn_workspace(hlm, 4, 32, 8, 1024, 0) > 0


def test_offset_limit(K):
    """T_cap beyond the kernels' 32-bit offsets is rejected before any launch."""
    cb = K.kvq_build_codebook(256, 4)
    s = np.ones(256, dtype=np.int8)
    assert _call_decode(K, cb, s, T_cap=(1 << 31) // (4 * 256)) == K.KVQ_ERR_UNSUPPORTED
    assert "32-bit" in K.kvq_last_error()


def test_select_signs_validation_and_workspace(K):
    P = ctypes.c_void_p
    cb = K.kvq_build_codebook(64, 4)
    lib = K._lib
    cands = np.ones((3, 64), dtype=np.int8)
    errs = np.zeros(3, dtype=np.float32)
    best = ctypes.c_int(-7)
    need = K.kvq_select_signs_workspace(cb, 2, 4, 2, 100, 3)
    # exact + decoded outputs, errors, codes, norms (each padded to 256 bytes); one split needs no decode workspace
    assert need == 2 * 2048 + 256 + 12800 + 1792
    assert K.kvq_select_signs_workspace(cb, 2, 3, 2, 100, 3) == 0

    def call(cbx=cb, c=cands, C=3, T=100, ws=FAKE, ws_bytes=need, qdt=1, e=errs):
        return lib.kvq_select_signs(ctypes.byref(cbx), c.ctypes.data_as(P), C, P(FAKE), qdt, P(FAKE), 1, P(FAKE), 1,
                                    2, 4, 2, T, 0.125, None if e is None else e.ctypes.data_as(P), ctypes.byref(best),
                                    P(ws), ws_bytes, None)
    bad = cands.copy()
    bad[2, 5] = 0
    assert call(c=bad) == K.KVQ_ERR_INVALID_ARG
    assert "candidate 2" in K.kvq_last_error()
    assert call(C=0) == K.KVQ_ERR_INVALID_ARG
    assert call(e=None) == K.KVQ_ERR_INVALID_ARG
    assert call(qdt=9) == K.KVQ_ERR_INVALID_ARG
    assert call(T=0) == K.KVQ_ERR_UNSUPPORTED
    assert call(T=8193) == K.KVQ_ERR_UNSUPPORTED
    assert call(ws_bytes=need - 1) == K.KVQ_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == K.KVQ_ERR_INVALID_ARG
    assert "256-byte" in K.kvq_last_error()
    pq = K.kvq_codebook()
    K._check(lib.kvq_codebook_pq(64, 8, 256, 2, P(FAKE), ctypes.byref(pq)))
    assert call(cbx=pq) == K.KVQ_ERR_UNSUPPORTED
    assert best.value == -7  # nothing written on failure


def test_decode_qv_validation(K):
    P = ctypes.c_void_p
    cb = K.kvq_build_codebook(64, 4)
    s = np.ones(64, dtype=np.int8)
    lib = K._lib

    def call(cbx=cb, vcodes=FAKE, vnorms=FAKE, odt=1, n_splits=0, T_cap=64):
        return lib.kvq_decode_attn_qv(ctypes.byref(cbx), s.ctypes.data_as(P), P(FAKE), 1, P(FAKE), P(FAKE),
                                      None if vcodes is None else P(vcodes), None if vnorms is None else P(vnorms),
                                      1, 4, 2, T_cap, None, 0.125, P(FAKE), odt, None, 0, n_splits, None)
    assert call(vcodes=None) == K.KVQ_ERR_INVALID_ARG
    assert "vcodes" in K.kvq_last_error()
    assert call(vnorms=None) == K.KVQ_ERR_INVALID_ARG
    assert call(vnorms=FAKE + 4) == K.KVQ_ERR_INVALID_ARG
    assert call(odt=4) == K.KVQ_ERR_INVALID_ARG
    assert call(n_splits=-2) == K.KVQ_ERR_INVALID_ARG
    assert call(T_cap=4096, n_splits=8) == K.KVQ_ERR_WORKSPACE
    pq = K.kvq_codebook()
    K._check(lib.kvq_codebook_pq(64, 8, 256, 2, P(FAKE), ctypes.byref(pq)))
    assert call(cbx=pq) == K.KVQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("mant", [0, 1])
def test_pot_codebook_matches_oracle(K, oracle_mod, b, mant):
    """The power-of-two codebook: signed level per code value (sign in the top bit) and the midpoints of the
    magnitudes, equal to the oracle's (all exact in fp32)."""
    cb = K.kvq_build_codebook_pot(64, b, mant)
    assert cb.kind == K.KVQ_POT and cb.b == b and cb.m == mant and cb.bytes_per_key == 64 * b // 8
    mags, thr = oracle_mod.pot_levels(b, mant)
    np.testing.assert_array_equal(cb.levels_array(), np.concatenate([mags, -mags]).astype(np.float32))
    np.testing.assert_array_equal(cb.thresholds_array(), thr.astype(np.float32))


def test_pot_validation(K):
    for d, b, m in [(48, 4, 0), (512, 4, 0), (64, 1, 0), (64, 5, 0), (64, 4, 2)]:
        with pytest.raises(K.KvqError) as e:
            K.kvq_build_codebook_pot(d, b, m)
        assert e.value.status == K.KVQ_ERR_INVALID_ARG
    cb = K.kvq_build_codebook_pot(64, 4, 1)
    # no sign pattern needed; scales (norms) are required
    assert _call_encode(K, cb, None, norms=None) == K.KVQ_ERR_INVALID_ARG
    assert "scales" in K.kvq_last_error()
    bad = K.kvq_build_codebook_pot(64, 4, 1)
    bad.m = 3
    assert _call_encode(K, bad, None) == K.KVQ_ERR_INVALID_ARG
    # the kernels rely on the canonical levels and midpoints: anything else is rejected
    for field, idx in (("thresholds", 2), ("levels", 9)):
        odd = K.kvq_build_codebook_pot(64, 4, 0)
        getattr(odd, field)[idx] *= 1.01
        assert _call_encode(K, odd, None) == K.KVQ_ERR_INVALID_ARG
        assert "canonical" in K.kvq_last_error()
    P = ctypes.c_void_p
    lib = K._lib
    assert lib.kvq_score(ctypes.byref(cb), None, P(FAKE), 1, P(FAKE), None, 1, 4, 2, 128, None, P(FAKE),
                         None) == K.KVQ_ERR_INVALID_ARG
    # quantized values belong to the Hadamard codec
    assert lib.kvq_decode_attn_qv(ctypes.byref(cb), None, P(FAKE), 1, P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1, 4, 2,
                                  128, None, 0.125, P(FAKE), 1, P(FAKE), 1 << 20, 0, None) == K.KVQ_ERR_UNSUPPORTED


def test_pq_code_width(K):
    P = ctypes.c_void_p
    cb = K.kvq_codebook()
    K._check(K._lib.kvq_codebook_pq(64, 8, 16, 2, P(FAKE), ctypes.byref(cb)))
    assert cb.b == 4 and cb.bytes_per_key == 4
    K._check(K._lib.kvq_codebook_pq(64, 8, 17, 2, P(FAKE), ctypes.byref(cb)))
    assert cb.b == 8 and cb.bytes_per_key == 8
    K._check(K._lib.kvq_codebook_pq(64, 4, 16, 2, P(FAKE), ctypes.byref(cb)))
    assert cb.b == 4 and cb.bytes_per_key == 2
    cb.K = 32  # 4-bit codes cannot index 32 centroids
    assert _call_encode(K, cb, None, norms=None) == K.KVQ_ERR_INVALID_ARG
    assert "code width" in K.kvq_last_error()


def test_stream_read_validation(K):
    """kvq_stream_read (the streaming-ceiling read) rejects bad arguments before launching."""
    P = ctypes.c_void_p
    lib = K._lib
    sink = P(FAKE)

    def call(codes=FAKE, norms=FAKE, v=FAKE, B=2, Hkv=2, T_cap=4096, d=64, bpk=32, n_splits=8):
        return lib.kvq_stream_read(P(codes) if codes else None, P(norms) if norms else None, P(v) if v else None,
                                   B, Hkv, T_cap, d, bpk, n_splits, sink, None)

    assert call(codes=0) == K.KVQ_ERR_INVALID_ARG
    assert call(v=0) == K.KVQ_ERR_INVALID_ARG
    assert call(norms=FAKE + 4) == K.KVQ_ERR_INVALID_ARG          # misaligned
    assert call(B=0) == K.KVQ_ERR_INVALID_ARG
    assert call(n_splits=0) == K.KVQ_ERR_INVALID_ARG
    assert call(n_splits=257) == K.KVQ_ERR_INVALID_ARG
    assert call(B=300, Hkv=300) == K.KVQ_ERR_INVALID_ARG          # B*Hkv > 65535
    assert call(T_cap=1 << 23) == K.KVQ_ERR_UNSUPPORTED            # 32-bit offsets
    assert call(d=32, bpk=16) == K.KVQ_ERR_UNSUPPORTED             # instantiated for d = 64 and 128 only
    assert call(d=64, bpk=24) == K.KVQ_ERR_UNSUPPORTED
    assert "kvq_stream_read" in K.kvq_last_error()
