"""Byte-code PQ encode (nearest centroid per subspace, LOOKAT page, Abstract) against the oracle on every
head dimension / subspace count the library builds (4 to 32 dimensions per subspace), centroid counts that
are not a multiple of the kernel's tiles, fp16 and fp32 keys, ragged key counts, write offsets and per-batch
write positions.

The kernel takes the nearest centroid from fp32 matrix products where its lead over the runner-up is beyond
a rounding bound and scans the plain distances otherwise; planted keys make the second branch run: keys on
the midpoint of two centroids (an exact or near tie), keys equal to a centroid, zero keys, and keys scaled
by 1e-12 and 1e12.  The bar is the oracle's: every code equal to the oracle's except in its tie band (best
two squared distances within 1e-6 |k_s|^2), where the code must still be among the nearest within the band.
"""
import numpy as np
import pytest

from helpers import log, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    import torch
    assert torch.cuda.is_available(), "no GPU"
    import quantized_kv_cache_encode_amd.kvq as kvq
    return kvq


def _planted_keys(rng, cent, B, T, d, m, scale_rows):
    """Keys [B][H][T][d] ~ N(0,1) with planted sub-vectors in the first rows of every (batch, head)."""
    H, _, Kc, ds = cent.shape
    keys = rng.standard_normal((B, H, T, d))
    for b in range(B):
        for h in range(H):
            for s in range(m):
                sl = slice(s * ds, (s + 1) * ds)
                i, j = rng.choice(Kc, 2, replace=False)
                keys[b, h, 0, sl] = 0.5 * (cent[h, s, i] + cent[h, s, j])  # midpoint: a tie up to rounding
                keys[b, h, 1, sl] = cent[h, s, i]                            # on a centroid
                keys[b, h, 2, sl] = 0.0                                      # zero sub-vector
                a, c = rng.choice(Kc, 2, replace=False)
                w = 0.5 + 1e-7 * rng.standard_normal()
                keys[b, h, 3, sl] = w * cent[h, s, a] + (1 - w) * cent[h, s, c]  # a near tie
    for r, f in scale_rows:
        if r < T:
            keys[:, :, r] *= f
    return keys


def _check(oracle_mod, cent, keys, got):
    """got [B][H][T][m] against the oracle, with the tie band."""
    H, m, _, ds = cent.shape
    B, _, T, d = keys.shape
    k64 = keys.astype(np.float64)
    ref = np.zeros((B, H, T, m), dtype=np.uint8)
    gaps = np.zeros((B, H, T, m))
    for h in range(H):
        ref[:, h], gaps[:, h] = oracle_mod.pq_encode(cent[h].astype(np.float64), k64[:, h])
    ks = k64.reshape(B, H, T, m, ds)
    band = 1e-6 * (ks ** 2).sum(-1)
    in_band = gaps < band
    diff = np.argwhere(got != ref)
    log("  codes differing %d of %d; tie-band codes %d" % (len(diff), got.size, int(in_band.sum())))
    for b, h, t, s in diff:
        assert in_band[b, h, t, s], "code outside the tie band differs at %s: got %d, oracle %d" % (
            (b, h, t, s), got[b, h, t, s], ref[b, h, t, s])
        c = cent[h, s].astype(np.float64)
        dist = ((ks[b, h, t, s][None, :] - c) ** 2).sum(-1)
        assert dist[got[b, h, t, s]] - dist[ref[b, h, t, s]] <= band[b, h, t, s]


# (d, m, K, key dtype, B, H, T_new)
SHAPES = [
    (64, 16, 256, "f16", 2, 3, 1000),   # 4 dimensions per subspace
    (64, 8, 256, "f32", 2, 2, 777),     # 8
    (128, 8, 200, "f32", 1, 3, 513),    # 16, K not a multiple of 32
    (128, 4, 33, "f16", 2, 2, 300),     # 32, K just past a tile pair
    (64, 8, 17, "f32", 1, 2, 64),       # the fewest centroids that take byte codes
    (64, 4, 256, "f16", 3, 1, 40),      # 16, fewer keys than one workgroup
]


@pytest.mark.parametrize("d,m,Kc,dt,B,H,T", SHAPES)
def test_pq_byte_encode_matches_oracle(K, oracle_mod, d, m, Kc, dt, B, H, T):
    import torch
    rng = np.random.default_rng(1000 * d + 10 * m + Kc)
    ds = d // m
    cent = rng.standard_normal((H, m, Kc, ds)).astype(np.float32)
    keys = _planted_keys(rng, cent, B, T, d, m, [(4, 1e-12), (5, 1e12)])
    keys = keys.astype(np.float16 if dt == "f16" else np.float32)
    if dt == "f16":
        keys = np.nan_to_num(keys, posinf=6e4, neginf=-6e4)  # rows scaled past the fp16 range saturate
    log("PQ byte encode d=%d m=%d K=%d %s B=%d H=%d T=%d" % (d, m, Kc, dt, B, H, T))
    cb = K.kvq_codebook_pq(d, m, Kc, H, torch_dev(cent))
    assert cb.b == 8 and cb.bytes_per_key == m
    codes = torch.zeros((B, H, T, m), dtype=torch.uint8, device="cuda:0")
    K.kvq_encode_keys(cb, None, torch_dev(keys), codes)
    torch.cuda.synchronize()
    _check(oracle_mod, cent, keys, codes.cpu().numpy())


def test_pq_byte_encode_write_positions(K, oracle_mod):
    """New keys written at per-batch positions of a longer cache (one batch past the end: nothing written),
    and at a fixed offset t0; rows outside stay untouched."""
    import torch
    d, m, Kc, H, B, T_new, T_cap = 64, 8, 256, 2, 3, 100, 400
    rng = np.random.default_rng(4242)
    cent = rng.standard_normal((H, m, Kc, d // m)).astype(np.float32)
    keys = _planted_keys(rng, cent, B, T_new, d, m, []).astype(np.float16)
    cb = K.kvq_codebook_pq(d, m, Kc, H, torch_dev(cent))
    wp = np.array([0, 250, 390], dtype=np.int32)
    codes = torch.full((B, H, T_cap, m), 0xAB, dtype=torch.uint8, device="cuda:0")
    K.kvq_encode_keys(cb, None, torch_dev(keys), codes, write_pos=torch.tensor(wp, device="cuda:0"))
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    for b in range(B):
        n = max(0, min(T_new, T_cap - wp[b]))
        _check(oracle_mod, cent, keys[b:b + 1, :, :n], got[b:b + 1, :, wp[b]:wp[b] + n])
        rest = np.ones(T_cap, bool)
        rest[wp[b]:wp[b] + n] = False
        assert np.all(got[b, :, rest] == 0xAB)
    codes = torch.full((B, H, T_cap, m), 0xAB, dtype=torch.uint8, device="cuda:0")
    K.kvq_encode_keys(cb, None, torch_dev(keys), codes, t0=123)
    torch.cuda.synchronize()
    got = codes.cpu().numpy()
    _check(oracle_mod, cent, keys, got[:, :, 123:123 + T_new])
    assert np.all(got[:, :, :123] == 0xAB) and np.all(got[:, :, 123 + T_new:] == 0xAB)
