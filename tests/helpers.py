"""Shared helpers for the parity tests: build a case from the seeded workloads,
run the oracle on it, and compare with the GPU library."""
from __future__ import annotations

import math
import sys

import numpy as np

import workloads as W


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error of every row (last axis)."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def torch_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda:0")


def make_hlm_case(shape: W.Shape, batches=None, T: int | None = None):
    """Seeded inputs of one Hadamard/Lloyd-Max workload (optionally fewer batches / tokens)."""
    T = shape.T if T is None else T
    bsel = list(range(shape.B)) if batches is None else list(batches)
    q_all = W.queries(shape)
    return dict(
        signs=W.signs(shape),
        q=q_all[bsel],
        keys=W.keys(shape, batches=bsel, T=T),
        v=W.values(shape, batches=bsel, T=T),
    )


def oracle_cache(oracle, shape: W.Shape, keys: np.ndarray, signs: np.ndarray):
    """Oracle encode of keys [B][Hkv][T][d] -> (codes uint8, norms as fp32, tie flags)."""
    lv, th = oracle.codebook(shape.d, shape.b)
    codes, norms, _, tie = oracle.encode_keys(th, signs, keys, shape.b)
    return codes, norms.astype(np.float32), tie


def score_tolerance(q: np.ndarray, norms: np.ndarray, G: int) -> np.ndarray:
    """1e-4 * |q| * |k_t| for every (b, h, t)."""
    qn = np.linalg.norm(q.astype(np.float64), axis=-1)  # [B, Hq]
    kn = np.repeat(norms.astype(np.float64), G, axis=1)  # [B, Hq, T]
    return 1e-4 * qn[:, :, None] * kn


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)
