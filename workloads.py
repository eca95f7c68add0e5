"""Seeded synthetic workloads for attention from quantized key codes.

This module only draws random inputs; it holds none of the method's
arithmetic.  The same arrays feed the GPU library and the CPU oracle.

Every tensor gets its own child of ``numpy.random.SeedSequence(seed)``, and
the per-batch slices of the large caches get one child each, so any subset of
batches can be regenerated bit-for-bit without drawing the rest.

Workloads (shapes of the pages' workloads; synthetic data stands in for the
models and datasets the pages measure on):

* ``tiny``       d=16, b=2, T=64, one head, one query; q, k, v ~ N(0,1) fp32.
* ``llama8b``    one decode layer with Llama-3.1-8B-like shapes: Hq=32, Hkv=8,
                 d=128, b=4, B=1, T=4096; keys and values N(0,1) times a
                 per-(kv head, channel) scale ~ LogNormal(0,1) (independent for
                 K and V); q, k, v fp16.
* ``longctx``    batched long-context decode with 1.1B-Llama-like shapes: Hq=32,
                 Hkv=4, d=64, b=4, B=8, T=32768; k_t = sigma_t z_t with
                 z ~ N(0, I) and sigma_t ~ LogNormal(0, 0.5) per key; q, v ~ N(0,1);
                 all fp16.
* ``sweep``      llama8b shapes with b in {2,3,4}, B in {1,16,64}, T=8192.
* ``signsel``    sign-pattern selection: 200 candidate patterns (+-1 with
                 probability 1/2 each) scored on 8 calibration samples of
                 llama8b-like shapes (Hq=32, Hkv=8, d=128, b=4) with T=512 keys
                 each; keys and values N(0,1) times per-(kv head, channel)
                 LogNormal(0,1) scales, the channel-norm heterogeneity under
                 which the sign pattern matters; fp16.
* ``pq_gpt2``    PQ-ADC with GPT-2-small-like shapes: H=12 (Hq=Hkv), d=64, m=8,
                 K=256, B=4, T=1024; q, k, v ~ N(0,1) fp16; k-means training set
                 4096 fresh N(0,1) keys per head, start rows = first K entries of
                 a seeded permutation per (head, subspace).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 1000


@dataclass(frozen=True)
class Shape:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    T: int
    b: int = 4            # bits per coordinate (Hadamard + Lloyd-Max codec)
    dtype: str = "f16"    # dtype of q, k, v
    key_scale: str = "none"   # "none" | "channel_lognormal" | "token_lognormal"
    v_scale: str = "none"     # "none" | "channel_lognormal"
    m: int = 0            # PQ subspaces (0 = not PQ)
    K: int = 0            # PQ centroids per subspace
    seed: int = SEED_BASE
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


TINY = Shape("tiny", B=1, Hq=1, Hkv=1, d=16, T=64, b=2, dtype="f32", seed=SEED_BASE + 0)
LLAMA8B = Shape("llama8b", B=1, Hq=32, Hkv=8, d=128, T=4096, b=4, key_scale="channel_lognormal",
                v_scale="channel_lognormal", seed=SEED_BASE + 1)
LONGCTX = Shape("longctx", B=8, Hq=32, Hkv=4, d=64, T=32768, b=4, key_scale="token_lognormal",
                seed=SEED_BASE + 2)
PQ_GPT2 = Shape("pq_gpt2", B=4, Hq=12, Hkv=12, d=64, T=1024, m=8, K=256, seed=SEED_BASE + 4)
# 4-bit centroid indices (K = 16) at the same shapes: 4 B per key (m = 8, 32x smaller than fp16 keys) and
# 2 B per key (m = 4, 64x), the two compressions LOOKAT's abstract reports
PQ4_GPT2_32X = Shape("pq4_gpt2_32x", B=4, Hq=12, Hkv=12, d=64, T=1024, m=8, K=16, seed=SEED_BASE + 4)
PQ4_GPT2_64X = Shape("pq4_gpt2_64x", B=4, Hq=12, Hkv=12, d=64, T=1024, m=4, K=16, seed=SEED_BASE + 4)
SIGNSEL = Shape("signsel", B=8, Hq=32, Hkv=8, d=128, T=512, b=4, key_scale="channel_lognormal",
                v_scale="channel_lognormal", seed=SEED_BASE + 5)
SIGN_CANDIDATES = 200


def sweep(b: int, B: int) -> Shape:
    return Shape(f"sweep_b{b}_B{B}", B=B, Hq=32, Hkv=8, d=128, T=8192, b=b, key_scale="channel_lognormal",
                 v_scale="channel_lognormal", seed=SEED_BASE + 3)


SWEEP = [sweep(b, B) for b in (2, 3, 4) for B in (1, 16, 64)]


def _np_dtype(s: str):
    return {"f16": np.float16, "f32": np.float32}[s]


def _children(seed: int, n: int):
    return np.random.SeedSequence(seed).spawn(n)


# child slots: 0 signs, 1 q, 2 key scales, 3 keys (per batch), 4 value scales, 5 values (per batch),
#              6 PQ training set, 7 PQ start rows, 8 new keys for the write path (per batch),
#              9 candidate sign patterns
_SLOTS = 10


def signs(shape: Shape) -> np.ndarray:
    """The +-1 sign pattern D, each entry +1 or -1 with probability 1/2."""
    rng = np.random.default_rng(_children(shape.seed, _SLOTS)[0])
    return (rng.integers(0, 2, size=shape.d, dtype=np.int8) * 2 - 1).astype(np.int8)


def sign_candidates(shape: Shape, C: int = SIGN_CANDIDATES) -> np.ndarray:
    """C candidate sign patterns [C, d], each entry +1 or -1 with probability 1/2."""
    rng = np.random.default_rng(_children(shape.seed, _SLOTS)[9])
    return (rng.integers(0, 2, size=(C, shape.d), dtype=np.int8) * 2 - 1).astype(np.int8)


def queries(shape: Shape) -> np.ndarray:
    rng = np.random.default_rng(_children(shape.seed, _SLOTS)[1])
    return rng.standard_normal((shape.B, shape.Hq, shape.d), dtype=np.float32).astype(_np_dtype(shape.dtype))


def _channel_scales(shape: Shape, slot: int) -> np.ndarray:
    rng = np.random.default_rng(_children(shape.seed, _SLOTS)[slot])
    return rng.lognormal(0.0, 1.0, size=(shape.Hkv, shape.d)).astype(np.float32)


def keys(shape: Shape, batches=None, T: int | None = None, slot: int = 3) -> np.ndarray:
    """Keys [len(batches), Hkv, T, d] in the workload dtype."""
    T = shape.T if T is None else T
    batches = range(shape.B) if batches is None else batches
    kids = _children(shape.seed, _SLOTS)
    per_b = kids[slot].spawn(max(shape.B, 1))
    scales = _channel_scales(shape, 2) if shape.key_scale == "channel_lognormal" else None
    out = np.empty((len(batches), shape.Hkv, T, shape.d), dtype=_np_dtype(shape.dtype))
    for n, bi in enumerate(batches):
        rng = np.random.default_rng(per_b[bi])
        z = rng.standard_normal((shape.Hkv, T, shape.d), dtype=np.float32)
        if shape.key_scale == "channel_lognormal":
            z *= scales[:, None, :]
        elif shape.key_scale == "token_lognormal":
            sigma = rng.lognormal(0.0, 0.5, size=(shape.Hkv, T)).astype(np.float32)
            z *= sigma[:, :, None]
        out[n] = z.astype(out.dtype)
    return out


def new_keys(shape: Shape, T_new: int = 1) -> np.ndarray:
    """Keys of the tokens appended on a decode step, [B, Hkv, T_new, d]."""
    return keys(shape, T=T_new, slot=8)


def values(shape: Shape, batches=None, T: int | None = None) -> np.ndarray:
    """Values [len(batches), Hkv, T, d] in the workload dtype."""
    T = shape.T if T is None else T
    batches = range(shape.B) if batches is None else batches
    kids = _children(shape.seed, _SLOTS)
    per_b = kids[5].spawn(max(shape.B, 1))
    scales = _channel_scales(shape, 4) if shape.v_scale == "channel_lognormal" else None
    out = np.empty((len(batches), shape.Hkv, T, shape.d), dtype=_np_dtype(shape.dtype))
    for n, bi in enumerate(batches):
        rng = np.random.default_rng(per_b[bi])
        z = rng.standard_normal((shape.Hkv, T, shape.d), dtype=np.float32)
        if scales is not None:
            z *= scales[:, None, :]
        out[n] = z.astype(out.dtype)
    return out


def pq_training(shape: Shape, n_train: int = 4096) -> np.ndarray:
    """k-means training keys [Hkv, n_train, d], fresh N(0,1) draws (fp32)."""
    rng = np.random.default_rng(_children(shape.seed, _SLOTS)[6])
    return rng.standard_normal((shape.Hkv, n_train, shape.d), dtype=np.float32)


def pq_start_rows(shape: Shape, n_train: int = 4096) -> np.ndarray:
    """k-means starting rows [Hkv, m, K]: the first K entries of a seeded permutation."""
    rng = np.random.default_rng(_children(shape.seed, _SLOTS)[7])
    out = np.empty((shape.Hkv, shape.m, shape.K), dtype=np.int64)
    for h in range(shape.Hkv):
        for s in range(shape.m):
            out[h, s] = rng.permutation(n_train)[: shape.K]
    return out


def seq_lens_ragged(B: int, T: int, seed: int) -> np.ndarray:
    """A ragged mix of sequence lengths in [0, T], including the empty and the full length."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, T + 1, size=B).astype(np.int32)
    if B >= 2:
        lens[0] = T
    if B >= 3:
        lens[1] = 0
    return lens


def scaled(shape: Shape, **kw) -> Shape:
    """A smaller copy of a workload (same distributions and seed) for tests the oracle finishes quickly."""
    fields = dict(shape.__dict__)
    fields.pop("extra", None)
    fields.update(kw)
    return Shape(**fields)
