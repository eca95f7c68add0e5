"""fp64 CPU oracle for attention from quantized key-cache codes.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product library never imports,
links or calls anything here, and nothing here imports the product package.

The arithmetic lives in ``kvq_oracle.c`` (plain C, fp64, explicit loops, one
thread); this module only builds it with gcc and converts numpy arrays.  Each
function names the page passage it follows; see the C file for the readings
taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile kvq_oracle.c into libkvq_oracle.so with gcc (IEEE fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = ctypes.CDLL(_LIB_PATH)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _signs(s):
    s = np.ascontiguousarray(np.asarray(s, dtype=np.int8))
    if not np.all(np.abs(s) == 1):
        raise ValueError("signs must be +-1")
    return s


def _lens(seq_lens, B):
    if seq_lens is None:
        return None
    s = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    assert s.shape == (B,)
    return s


# --------------------------------------------------------------------------
# Codebook (AXELRAM abstract: fixed codebook for N(0,1/d), depends on d and b only)
# --------------------------------------------------------------------------

def lloyd_max_unit(b: int):
    """Lloyd-Max levels/thresholds for N(0,1) with 2^b levels; returns (c, t, iterations)."""
    L = 1 << b
    c = np.zeros(L)
    t = np.zeros(L - 1)
    it = _load().ora_lloyd_max_unit(ctypes.c_int(b), _p(c), _p(t))
    return c, t, it


def codebook(d: int, b: int):
    """Levels and thresholds of the N(0,1/d) Lloyd-Max codebook (unit quantizer / sqrt(d))."""
    L = 1 << b
    c = np.zeros(L)
    t = np.zeros(L - 1)
    _load().ora_codebook(ctypes.c_int(d), ctypes.c_int(b), _p(c), _p(t))
    return c, t


def quantizer_mse_unit(b: int, c, t) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) under levels c and thresholds t (closed-form cell integrals)."""
    lib = _load()
    lib.ora_quantizer_mse_unit.restype = ctypes.c_double
    c = _f64(c)
    t = _f64(t)
    return float(lib.ora_quantizer_mse_unit(ctypes.c_int(b), _p(c), _p(t)))


# --------------------------------------------------------------------------
# Transform (AXELRAM key points/abstract: orthogonal transform with a sign pattern)
# --------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    H = np.zeros((d, d))
    _load().ora_hadamard(ctypes.c_int(d), _p(H))
    return H


def rotate_query(signs, q) -> np.ndarray:
    """q' = H D q for a single query vector."""
    signs = _signs(signs)
    q = _f64(q)
    d = q.shape[-1]
    out = np.zeros(d)
    _load().ora_rotate_query(ctypes.c_int(d), _p(signs), _p(q), _p(out))
    return out


# --------------------------------------------------------------------------
# Write path (AXELRAM abstract: transform on write, store indices)
# --------------------------------------------------------------------------

def encode_keys(thresholds, signs, keys, b: int, tie_eps: float = 1e-6):
    """Encode keys [..., d]: returns (codes [..., d*b/8] uint8, norms [...], y [..., d], tie [..., d] bool)."""
    signs = _signs(signs)
    keys = _f64(keys)
    d = keys.shape[-1]
    lead = keys.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    thr = _f64(thresholds)
    assert thr.shape == ((1 << b) - 1,)
    bpk = d * b // 8
    codes = np.zeros((n, bpk), dtype=np.uint8)
    norms = np.zeros(n)
    y = np.zeros((n, d))
    tie = np.zeros((n, d), dtype=np.uint8)
    _load().ora_encode_keys(ctypes.c_int(d), ctypes.c_int(b), _p(thr), _p(signs), _p(keys),
                            ctypes.c_int64(n), _p(codes), _p(norms), _p(y), _p(tie),
                            ctypes.c_double(tie_eps))
    return (codes.reshape(lead + (bpk,)), norms.reshape(lead), y.reshape(lead + (d,)),
            tie.reshape(lead + (d,)).astype(bool))


def unpack_codes(codes, d: int, b: int) -> np.ndarray:
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    lead = codes.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    idx = np.zeros((n, d), dtype=np.int32)
    _load().ora_unpack_codes(ctypes.c_int(d), ctypes.c_int(b), _p(codes), ctypes.c_int64(n), _p(idx))
    return idx.reshape(lead + (d,))


# --------------------------------------------------------------------------
# Read path (AXELRAM abstract: table lookup on read, no inverse transform)
# --------------------------------------------------------------------------

def build_lut(levels, qrot) -> np.ndarray:
    levels = _f64(levels)
    qrot = _f64(qrot)
    d = qrot.shape[0]
    L = levels.shape[0]
    b = L.bit_length() - 1
    lut = np.zeros((d, L))
    _load().ora_build_lut(ctypes.c_int(d), ctypes.c_int(b), _p(levels), _p(qrot), _p(lut))
    return lut


def scores(levels, signs, q, codes, norms, seq_lens=None) -> np.ndarray:
    """Raw scores [B, Hq, T] from q [B, Hq, d], codes [B, Hkv, T, bpk], norms [B, Hkv, T]."""
    levels = _f64(levels)
    signs = _signs(signs)
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    _, Hkv, T, bpk = codes.shape
    b = levels.shape[0].bit_length() - 1
    assert bpk == d * b // 8
    norms = _f64(norms)
    assert norms.shape == (B, Hkv, T)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, T))
    _load().ora_scores(ctypes.c_int(d), ctypes.c_int(b), _p(levels), _p(signs), _p(q), _p(codes),
                       _p(norms), ctypes.c_int(B), ctypes.c_int(Hq), ctypes.c_int(Hkv),
                       ctypes.c_int64(T), None if lens is None else _p(lens), _p(out))
    return out


def softmax_row(s, scale: float) -> np.ndarray:
    s = _f64(s)
    p = np.zeros_like(s)
    _load().ora_softmax_row(_p(s), ctypes.c_int64(s.shape[0]), ctypes.c_double(scale), _p(p))
    return p


def decode_attn(levels, signs, q, codes, norms, v, scale: float, seq_lens=None) -> np.ndarray:
    """Attention output [B, Hq, d] = softmax(scale * scores) V, V [B, Hkv, T, d]."""
    levels = _f64(levels)
    signs = _signs(signs)
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    _, Hkv, T, bpk = codes.shape
    b = levels.shape[0].bit_length() - 1
    assert bpk == d * b // 8
    norms = _f64(norms)
    v = _f64(v)
    assert v.shape == (B, Hkv, T, d)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, d))
    _load().ora_decode_attn(ctypes.c_int(d), ctypes.c_int(b), _p(levels), _p(signs), _p(q), _p(codes),
                            _p(norms), _p(v), ctypes.c_int(B), ctypes.c_int(Hq), ctypes.c_int(Hkv),
                            ctypes.c_int64(T), None if lens is None else _p(lens),
                            ctypes.c_double(scale), _p(out))
    return out


# --------------------------------------------------------------------------
# Values quantized with the key codec (a reading: the value row is encoded as a
# key is, and attention uses v_hat = |v| D H^T c_hat)
# --------------------------------------------------------------------------

def dequant(levels, signs, codes, norms) -> np.ndarray:
    """Rows [..., d] = norm * D H^T c_hat of code rows [..., bpk] with norms [...]."""
    levels = _f64(levels)
    signs = _signs(signs)
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    lead = codes.shape[:-1]
    b = levels.shape[0].bit_length() - 1
    d = codes.shape[-1] * 8 // b
    norms = _f64(norms)
    assert norms.shape == lead
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (d,))
    _load().ora_dequant_rows(ctypes.c_int(d), ctypes.c_int(b), _p(levels), _p(signs), _p(codes), _p(norms),
                             ctypes.c_int64(n), _p(out))
    return out


def decode_attn_qv(levels, signs, q, codes, norms, vcodes, vnorms, scale: float, seq_lens=None) -> np.ndarray:
    """Attention output [B, Hq, d] with keys and values both as codes + norms [B, Hkv, T, ...]."""
    levels = _f64(levels)
    signs = _signs(signs)
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    vcodes = np.ascontiguousarray(np.asarray(vcodes, dtype=np.uint8))
    _, Hkv, T, bpk = codes.shape
    b = levels.shape[0].bit_length() - 1
    assert bpk == d * b // 8 and vcodes.shape == codes.shape
    norms, vnorms = _f64(norms), _f64(vnorms)
    assert norms.shape == (B, Hkv, T) and vnorms.shape == (B, Hkv, T)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, d))
    _load().ora_decode_attn_qv(ctypes.c_int(d), ctypes.c_int(b), _p(levels), _p(signs), _p(q), _p(codes),
                               _p(norms), _p(vcodes), _p(vnorms), ctypes.c_int(B), ctypes.c_int(Hq),
                               ctypes.c_int(Hkv), ctypes.c_int64(T), None if lens is None else _p(lens),
                               ctypes.c_double(scale), _p(out))
    return out


# --------------------------------------------------------------------------
# Sign-pattern selection (AXELRAM key points/abstract: one-time, gradient-free
# choice among candidate sign patterns on calibration samples)
# --------------------------------------------------------------------------

def exact_attn(q, keys, v, scale: float) -> np.ndarray:
    """Unquantized attention [n, Hq, d] = softmax(scale * q.k) V over all T keys."""
    q, keys, v = _f64(q), _f64(keys), _f64(v)
    n, Hq, d = q.shape
    _, Hkv, T, _ = keys.shape
    out = np.zeros((n, Hq, d))
    _load().ora_exact_attn(ctypes.c_int(d), _p(q), _p(keys), _p(v), ctypes.c_int(n), ctypes.c_int(Hq),
                           ctypes.c_int(Hkv), ctypes.c_int64(T), ctypes.c_double(scale), _p(out))
    return out


def sign_errors(levels, thresholds, cands, q, keys, v, scale: float):
    """Attention-output error of every candidate sign pattern cands [C, d]; returns (errors [C], best)."""
    levels, thr = _f64(levels), _f64(thresholds)
    cands = np.ascontiguousarray(np.asarray(cands, dtype=np.int8))
    if not np.all(np.abs(cands) == 1):
        raise ValueError("candidates must be +-1")
    q, keys, v = _f64(q), _f64(keys), _f64(v)
    n, Hq, d = q.shape
    _, Hkv, T, _ = keys.shape
    C = cands.shape[0]
    b = levels.shape[0].bit_length() - 1
    errors = np.zeros(C)
    best = _load().ora_sign_errors(ctypes.c_int(d), ctypes.c_int(b), _p(levels), _p(thr), _p(cands), ctypes.c_int(C),
                                   _p(q), _p(keys), _p(v), ctypes.c_int(n), ctypes.c_int(Hq), ctypes.c_int(Hkv),
                                   ctypes.c_int64(T), ctypes.c_double(scale), _p(errors))
    return errors, int(best)


# --------------------------------------------------------------------------
# Product quantization + ADC (LOOKAT summary/abstract)
# --------------------------------------------------------------------------

def kmeans(train, K: int, iters: int, init_rows):
    """Lloyd k-means on train [n, ds] from the given starting rows; returns (centroids [K, ds], objective [iters+1])."""
    train = _f64(train)
    n, ds = train.shape
    init = np.ascontiguousarray(np.asarray(init_rows, dtype=np.int64))
    assert init.shape == (K,)
    cent = np.zeros((K, ds))
    obj = np.zeros(iters + 1)
    _load().ora_kmeans(_p(train), ctypes.c_int64(n), ctypes.c_int(ds), ctypes.c_int(K), ctypes.c_int(iters),
                       _p(init), _p(cent), _p(obj))
    return cent, obj


def pq_encode(cent, keys, bits: int = 8):
    """PQ codes [..., m*bits/8] of keys [..., d] for one head's centroids [m, K, d/m]; returns (codes, gap [..., m]).
    bits = 8: one byte per subspace; bits = 4 (K <= 16): two subspaces per byte, the even one low."""
    cent = _f64(cent)
    m, K, ds = cent.shape
    assert bits == 8 or (bits == 4 and K <= 16 and m % 2 == 0)
    keys = _f64(keys)
    d = keys.shape[-1]
    assert d == m * ds
    lead = keys.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    bpk = m * bits // 8
    codes = np.zeros((n, bpk), dtype=np.uint8)
    gap = np.zeros((n, m))
    _load().ora_pq_encode(ctypes.c_int(d), ctypes.c_int(m), ctypes.c_int(K), ctypes.c_int(bits), _p(cent), _p(keys),
                          ctypes.c_int64(n), _p(codes), _p(gap))
    return codes.reshape(lead + (bpk,)), gap.reshape(lead + (m,))


def pq_scores(cent, q, codes, seq_lens=None, bits: int = 8) -> np.ndarray:
    """PQ-ADC scores [B, Hq, T]; cent [Hkv, m, K, d/m], q [B, Hq, d], codes [B, Hkv, T, m*bits/8]."""
    cent = _f64(cent)
    Hkv, m, K, ds = cent.shape
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    T = codes.shape[2]
    assert codes.shape == (B, Hkv, T, m * bits // 8)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, T))
    _load().ora_pq_scores(ctypes.c_int(d), ctypes.c_int(m), ctypes.c_int(K), ctypes.c_int(bits), _p(cent), _p(q),
                          _p(codes), ctypes.c_int(B), ctypes.c_int(Hq), ctypes.c_int(Hkv), ctypes.c_int64(T),
                          None if lens is None else _p(lens), _p(out))
    return out


def pq_decode_attn(cent, q, codes, v, scale: float, seq_lens=None, bits: int = 8) -> np.ndarray:
    cent = _f64(cent)
    Hkv, m, K, ds = cent.shape
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    T = codes.shape[2]
    assert codes.shape == (B, Hkv, T, m * bits // 8)
    v = _f64(v)
    assert v.shape == (B, Hkv, T, d)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, d))
    _load().ora_pq_decode_attn(ctypes.c_int(d), ctypes.c_int(m), ctypes.c_int(K), ctypes.c_int(bits), _p(cent),
                               _p(q), _p(codes), _p(v), ctypes.c_int(B), ctypes.c_int(Hq), ctypes.c_int(Hkv),
                               ctypes.c_int64(T), None if lens is None else _p(lens), ctypes.c_double(scale), _p(out))
    return out


# --------------------------------------------------------------------------
# Power-of-two key codec (shift-accumulate attention page, English abstract):
# sign + index of a magnitude 2^-j (or, with the mantissa term, a sum of two
# neighbouring powers of two) per element, times a per-key scale max |k_i|
# --------------------------------------------------------------------------

def pot_levels(b: int, mantissa: int):
    """(magnitudes [2^(b-1)] descending, midpoints [2^(b-1) - 1])."""
    n = 1 << (b - 1)
    mags = np.zeros(8)
    thr = np.zeros(7)
    _load().ora_pot_levels(ctypes.c_int(b), ctypes.c_int(int(mantissa)), _p(mags), _p(thr))
    return mags[:n].copy(), thr[:n - 1].copy()


def pot_encode(keys, b: int, mantissa: int, tie_eps: float = 1e-6):
    """Encode keys [..., d]: (codes [..., d*b/8] uint8, scales [...] = max |k_i|, tie [..., d] bool)."""
    keys = _f64(keys)
    d = keys.shape[-1]
    lead = keys.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    bpk = d * b // 8
    codes = np.zeros((n, bpk), dtype=np.uint8)
    scales = np.zeros(n)
    tie = np.zeros((n, d), dtype=np.uint8)
    _load().ora_pot_encode(ctypes.c_int(d), ctypes.c_int(b), ctypes.c_int(int(mantissa)), _p(keys),
                           ctypes.c_int64(n), _p(codes), _p(scales), _p(tie), ctypes.c_double(tie_eps))
    return codes.reshape(lead + (bpk,)), scales.reshape(lead), tie.reshape(lead + (d,)).astype(bool)


def pot_dequant(codes, scales, d: int, b: int, mantissa: int) -> np.ndarray:
    """Rows [..., d] = scale * (-1)^sign * magnitude(index)."""
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    lead = codes.shape[:-1]
    assert codes.shape[-1] == d * b // 8
    scales = _f64(scales)
    assert scales.shape == lead
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (d,))
    _load().ora_pot_dequant(ctypes.c_int(d), ctypes.c_int(b), ctypes.c_int(int(mantissa)), _p(codes), _p(scales),
                            ctypes.c_int64(n), _p(out))
    return out


def pot_scores(q, codes, scales, b: int, mantissa: int, seq_lens=None) -> np.ndarray:
    """Raw scores [B, Hq, T]: scale_t * sum_i of q_i sign-flipped and shifted by the code's shift amounts."""
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    _, Hkv, T, bpk = codes.shape
    assert bpk == d * b // 8
    scales = _f64(scales)
    assert scales.shape == (B, Hkv, T)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, T))
    _load().ora_pot_scores(ctypes.c_int(d), ctypes.c_int(b), ctypes.c_int(int(mantissa)), _p(q), _p(codes),
                           _p(scales), ctypes.c_int(B), ctypes.c_int(Hq), ctypes.c_int(Hkv), ctypes.c_int64(T),
                           None if lens is None else _p(lens), _p(out))
    return out


def pot_decode_attn(q, codes, scales, v, b: int, mantissa: int, scale: float, seq_lens=None) -> np.ndarray:
    """Attention output [B, Hq, d] = softmax(scale * pot_scores) V, V [B, Hkv, T, d]."""
    q = _f64(q)
    B, Hq, d = q.shape
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    _, Hkv, T, bpk = codes.shape
    assert bpk == d * b // 8
    scales = _f64(scales)
    v = _f64(v)
    assert v.shape == (B, Hkv, T, d)
    lens = _lens(seq_lens, B)
    out = np.zeros((B, Hq, d))
    _load().ora_pot_decode_attn(ctypes.c_int(d), ctypes.c_int(b), ctypes.c_int(int(mantissa)), _p(q), _p(codes),
                                _p(scales), _p(v), ctypes.c_int(B), ctypes.c_int(Hq), ctypes.c_int(Hkv),
                                ctypes.c_int64(T), None if lens is None else _p(lens), ctypes.c_double(scale),
                                _p(out))
    return out
