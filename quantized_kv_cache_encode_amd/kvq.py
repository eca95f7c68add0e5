"""Python binding of libkvq (include/kvq.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
PyTorch tensors: device buffers must live on the GPU, host arguments (sign
pattern, k-means training data) on the CPU.  Work is enqueued on the current
PyTorch stream unless a stream is given.  All arithmetic runs in the HIP
library; nothing here computes any part of the method, and there is no CPU
fallback: if libkvq.so is missing the import of this module fails.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_DEVICE = range(5)
KVQ_F32, KVQ_F16 = 0, 1
KVQ_HADAMARD_LM, KVQ_PQ, KVQ_POT = 0, 1, 2

_STATUS = {1: "KVQ_ERR_INVALID_ARG", 2: "KVQ_ERR_UNSUPPORTED", 3: "KVQ_ERR_WORKSPACE", 4: "KVQ_ERR_DEVICE"}


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), msg))
        self.status = status


class kvq_codebook(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("b", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("K", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("levels", ctypes.c_float * 16),
        ("thresholds", ctypes.c_float * 15),
        ("pq_centroids", ctypes.c_void_p),
    ]

    def levels_array(self) -> np.ndarray:
        return np.array(self.levels[: 1 << self.b], dtype=np.float32)

    def thresholds_array(self) -> np.ndarray:
        n = (1 << (self.b - 1)) - 1 if self.kind == KVQ_POT else (1 << self.b) - 1
        return np.array(self.thresholds[:n], dtype=np.float32)

    @property
    def bytes_per_key(self) -> int:
        return self.m * self.b // 8 if self.kind == KVQ_PQ else self.d * self.b // 8


if not os.path.exists(LIB_PATH):
    raise ImportError("libkvq.so is not built (run: python -m quantized_kv_cache_encode_amd.build)")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_i32, _i64, _f32, _sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_CB = ctypes.POINTER(kvq_codebook)

_lib.kvq_version.restype = ctypes.c_int
_lib.kvq_last_error.restype = ctypes.c_char_p
_lib.kvq_build_codebook.argtypes = [_i32, _i32, _CB]
_lib.kvq_build_codebook_pot.argtypes = [_i32, _i32, _i32, _CB]
_lib.kvq_build_codebook_pq.argtypes = [_P, _i32, _i64, _i32, _i32, _i32, _i32, _P, _P]
_lib.kvq_codebook_pq.argtypes = [_i32, _i32, _i32, _i32, _P, _CB]
_lib.kvq_encode_keys.argtypes = [_CB, _P, _P, _i32, _i32, _i32, _i64, _P, _P, _i64, _i64, _P, _P]
_lib.kvq_score.argtypes = [_CB, _P, _P, _i32, _P, _P, _i32, _i32, _i32, _i64, _P, _P, _P]
_lib.kvq_decode_attn_workspace.argtypes = [_CB, _i32, _i32, _i32, _i64, _i32]
_lib.kvq_decode_attn_workspace.restype = _sz
_lib.kvq_decode_attn.argtypes = [_CB, _P, _P, _i32, _P, _P, _P, _i32, _i32, _i32, _i32, _i64, _P, _f32,
                                 _P, _i32, _P, _sz, _i32, _P]
_lib.kvq_decode_attn_append.argtypes = [_CB, _P, _P, _i32, _P, _i32, _P, _P, _P, _i32, _i32, _i32, _i32, _i64, _P,
                                        _f32, _P, _i32, _P, _sz, _i32, _P]
_lib.kvq_decode_attn_noalloc.argtypes = [_CB, _P, _P, _i32, _P, _P, _P, _i32, _i32, _i32, _i32, _i64, _P, _f32,
                                         _P, _i32, _i32, _P]
_lib.kvq_stream_read.argtypes = [_P, _P, _P, _i32, _i32, _i64, _i32, _i32, _i32, _P, _P]
_lib.kvq_decode_attn_qv.argtypes = [_CB, _P, _P, _i32, _P, _P, _P, _P, _i32, _i32, _i32, _i64, _P, _f32, _P, _i32,
                                    _P, _sz, _i32, _P]
_lib.kvq_select_signs_workspace.argtypes = [_CB, _i32, _i32, _i32, _i64, _i32]
_lib.kvq_select_signs_workspace.restype = _sz
_lib.kvq_select_signs.argtypes = [_CB, _P, _i32, _P, _i32, _P, _i32, _P, _i32, _i32, _i32, _i32, _i64, _f32, _P, _P,
                                  _P, _sz, _P]
for _f in ("kvq_build_codebook", "kvq_build_codebook_pot", "kvq_build_codebook_pq", "kvq_codebook_pq", "kvq_encode_keys", "kvq_score",
           "kvq_decode_attn", "kvq_decode_attn_noalloc", "kvq_decode_attn_append", "kvq_decode_attn_qv",
           "kvq_select_signs", "kvq_stream_read"):
    getattr(_lib, _f).restype = ctypes.c_int

EXPORTS = ("kvq_version", "kvq_last_error", "kvq_build_codebook", "kvq_build_codebook_pot", "kvq_build_codebook_pq", "kvq_codebook_pq",
           "kvq_encode_keys", "kvq_score", "kvq_decode_attn_workspace", "kvq_decode_attn", "kvq_decode_attn_noalloc",
           "kvq_decode_attn_append",
           "kvq_decode_attn_qv", "kvq_select_signs_workspace", "kvq_select_signs", "kvq_stream_read")


def _check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, _lib.kvq_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError("unsupported dtype %s (fp16 or fp32)" % t.dtype)


def _dev(t, name, dtype=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _signs_host(signs, d):
    if signs is None:
        return None, None
    s = np.ascontiguousarray(np.asarray(signs.cpu() if isinstance(signs, torch.Tensor) else signs, dtype=np.int8))
    if s.shape != (d,):
        raise ValueError("signs must have shape (%d,)" % d)
    return s, s.ctypes.data_as(ctypes.c_void_p)


def kvq_version() -> int:
    return int(_lib.kvq_version())


def kvq_last_error() -> str:
    return _lib.kvq_last_error().decode()


def kvq_build_codebook(d: int, b: int) -> kvq_codebook:
    cb = kvq_codebook()
    _check(_lib.kvq_build_codebook(d, b, ctypes.byref(cb)))
    return cb


def kvq_build_codebook_pot(d: int, b: int, mantissa: int = 0) -> kvq_codebook:
    cb = kvq_codebook()
    _check(_lib.kvq_build_codebook_pot(d, b, int(mantissa), ctypes.byref(cb)))
    return cb


def kvq_build_codebook_pq(train, m: int, K: int, iters: int, start_rows) -> np.ndarray:
    """train: host [H][n][d] fp32; start_rows: host [H][m][K] int64 -> centroids host [H][m][K][d/m] fp32."""
    tr = np.ascontiguousarray(np.asarray(train, dtype=np.float32))
    H, n, d = tr.shape
    st = np.ascontiguousarray(np.asarray(start_rows, dtype=np.int64))
    if st.shape != (H, m, K):
        raise ValueError("start_rows must have shape (%d, %d, %d)" % (H, m, K))
    cent = np.zeros((H, m, K, d // m), dtype=np.float32)
    _check(_lib.kvq_build_codebook_pq(tr.ctypes.data_as(_P), H, n, d, m, K, iters, st.ctypes.data_as(_P),
                                      cent.ctypes.data_as(_P)))
    return cent


def kvq_codebook_pq(d: int, m: int, K: int, n_heads: int, centroids: torch.Tensor) -> kvq_codebook:
    """A PQ codebook referring to device centroids [n_heads][m][K][d/m] fp32 (kept alive by the object)."""
    cb = kvq_codebook()
    _check(_lib.kvq_codebook_pq(d, m, K, n_heads, _dev(centroids, "centroids", torch.float32), ctypes.byref(cb)))
    cb._centroids = centroids
    return cb


def kvq_encode_keys(cb: kvq_codebook, signs, keys: torch.Tensor, codes: torch.Tensor, norms=None, t0: int = 0,
                    write_pos=None, stream=None):
    """Encode keys [B][Hkv][T_new][d] into codes [B][Hkv][T_cap][bpk] (and norms [B][Hkv][T_cap])."""
    B, Hkv, T_new, d = keys.shape
    if codes.dim() != 4 or tuple(codes.shape[:2]) != (B, Hkv) or codes.shape[3] != cb.bytes_per_key:
        raise ValueError("codes must have shape (B, Hkv, T_cap, %d)" % cb.bytes_per_key)
    T_cap = codes.shape[2]
    s_np, s_ptr = _signs_host(signs, d)
    _check(_lib.kvq_encode_keys(ctypes.byref(cb), s_ptr, _dev(keys, "keys"), _dt(keys), B, Hkv, T_new,
                                _dev(codes, "codes", torch.uint8), _dev(norms, "norms", torch.float32, optional=True),
                                T_cap, t0, _dev(write_pos, "write_pos", torch.int32, optional=True), _stream(stream)))
    return codes, norms


def kvq_score(cb: kvq_codebook, signs, q: torch.Tensor, codes: torch.Tensor, norms=None, seq_lens=None, scores=None,
              stream=None) -> torch.Tensor:
    """Raw scores [B][Hq][T_cap] fp32 (-inf past each sequence's length)."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = codes.shape
    if scores is None:
        scores = torch.empty((B, Hq, T_cap), dtype=torch.float32, device=q.device)
    s_np, s_ptr = _signs_host(signs, d)
    _check(_lib.kvq_score(ctypes.byref(cb), s_ptr, _dev(q, "q"), _dt(q), _dev(codes, "codes", torch.uint8),
                          _dev(norms, "norms", torch.float32, optional=True), B, Hq, Hkv, T_cap,
                          _dev(seq_lens, "seq_lens", torch.int32, optional=True),
                          _dev(scores, "scores", torch.float32), _stream(stream)))
    return scores


def kvq_decode_attn_workspace(cb: kvq_codebook, B: int, Hq: int, Hkv: int, T_cap: int, n_splits: int = 0) -> int:
    return int(_lib.kvq_decode_attn_workspace(ctypes.byref(cb), B, Hq, Hkv, T_cap, n_splits))


def kvq_decode_attn(cb: kvq_codebook, signs, q: torch.Tensor, codes: torch.Tensor, norms, v: torch.Tensor,
                    scale: float | None = None, seq_lens=None, out=None, out_dtype=None, workspace=None,
                    n_splits: int = 0, stream=None) -> torch.Tensor:
    """Attention output [B][Hq][d] = softmax(scale * scores) V from codes (fp16 or fp32 V)."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = codes.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or v.dtype, device=q.device)
    need = kvq_decode_attn_workspace(cb, B, Hq, Hkv, T_cap, n_splits)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)  # counters start at zero
    ws_ptr = _dev(workspace, "workspace", optional=True)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    s_np, s_ptr = _signs_host(signs, d)
    _check(_lib.kvq_decode_attn(ctypes.byref(cb), s_ptr, _dev(q, "q"), _dt(q), _dev(codes, "codes", torch.uint8),
                                _dev(norms, "norms", torch.float32, optional=True), _dev(v, "v"), _dt(v), B, Hq, Hkv,
                                T_cap, _dev(seq_lens, "seq_lens", torch.int32, optional=True), float(scale),
                                _dev(out, "out"), _dt(out), ws_ptr, ws_bytes, n_splits, _stream(stream)))
    return out


def kvq_decode_attn_noalloc(cb: kvq_codebook, signs, q: torch.Tensor, codes: torch.Tensor, norms, v: torch.Tensor,
                            out: torch.Tensor, scale: float | None = None, seq_lens=None, n_splits: int = 0,
                            stream=None) -> torch.Tensor:
    """kvq_decode_attn with the library's static scratch array as its workspace: nothing is allocated here or
    in the library, so `out` [B][Hq][d] must be given."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = codes.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_np, s_ptr = _signs_host(signs, d)
    _check(_lib.kvq_decode_attn_noalloc(ctypes.byref(cb), s_ptr, _dev(q, "q"), _dt(q),
                                        _dev(codes, "codes", torch.uint8),
                                        _dev(norms, "norms", torch.float32, optional=True), _dev(v, "v"), _dt(v), B,
                                        Hq, Hkv, T_cap, _dev(seq_lens, "seq_lens", torch.int32, optional=True),
                                        float(scale), _dev(out, "out"), _dt(out), n_splits, _stream(stream)))
    return out


def kvq_decode_attn_qv(cb: kvq_codebook, signs, q: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor,
                       vcodes: torch.Tensor, vnorms: torch.Tensor, scale: float | None = None, seq_lens=None,
                       out=None, out_dtype=torch.float16, workspace=None, n_splits: int = 0,
                       stream=None) -> torch.Tensor:
    """Attention output [B][Hq][d] with the values stored as codes + norms of the same codec."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = codes.shape
    if tuple(vcodes.shape) != tuple(codes.shape) or tuple(vnorms.shape) != (B, Hkv, T_cap):
        raise ValueError("vcodes / vnorms must have the shapes of codes / norms")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype, device=q.device)
    need = kvq_decode_attn_workspace(cb, B, Hq, Hkv, T_cap, n_splits)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)  # counters start at zero
    ws_ptr = _dev(workspace, "workspace", optional=True)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    s_np, s_ptr = _signs_host(signs, d)
    _check(_lib.kvq_decode_attn_qv(ctypes.byref(cb), s_ptr, _dev(q, "q"), _dt(q), _dev(codes, "codes", torch.uint8),
                                   _dev(norms, "norms", torch.float32), _dev(vcodes, "vcodes", torch.uint8),
                                   _dev(vnorms, "vnorms", torch.float32), B, Hq, Hkv, T_cap,
                                   _dev(seq_lens, "seq_lens", torch.int32, optional=True), float(scale),
                                   _dev(out, "out"), _dt(out), ws_ptr, ws_bytes, n_splits, _stream(stream)))
    return out


def kvq_decode_attn_append(cb: kvq_codebook, signs, new_keys: torch.Tensor, q: torch.Tensor, codes: torch.Tensor,
                           norms: torch.Tensor, v: torch.Tensor, scale: float | None = None, seq_lens=None, out=None,
                           out_dtype=None, workspace=None, n_splits: int = 0, stream=None) -> torch.Tensor:
    """Encode new_keys [B][Hkv][d] at position len-1 of the cache, then attention as kvq_decode_attn."""
    B, Hq, d = q.shape
    _, Hkv, T_cap, _ = codes.shape
    if tuple(new_keys.shape) != (B, Hkv, d):
        raise ValueError("new_keys must have shape (%d, %d, %d)" % (B, Hkv, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or v.dtype, device=q.device)
    need = kvq_decode_attn_workspace(cb, B, Hq, Hkv, T_cap, n_splits)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)  # counters start at zero
    ws_ptr = _dev(workspace, "workspace", optional=True)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    s_np, s_ptr = _signs_host(signs, d)
    _check(_lib.kvq_decode_attn_append(ctypes.byref(cb), s_ptr, _dev(new_keys, "new_keys"), _dt(new_keys), _dev(q, "q"),
                                       _dt(q), _dev(codes, "codes", torch.uint8),
                                       _dev(norms, "norms", torch.float32), _dev(v, "v"), _dt(v), B, Hq, Hkv, T_cap,
                                       _dev(seq_lens, "seq_lens", torch.int32, optional=True), float(scale),
                                       _dev(out, "out"), _dt(out), ws_ptr, ws_bytes, n_splits, _stream(stream)))
    return out


def kvq_stream_read(codes: torch.Tensor, norms: torch.Tensor, v: torch.Tensor, n_splits: int, sink: torch.Tensor,
                    stream=None):
    """Plain read of a decode cache (codes [B][Hkv][T_cap][bpk], norms, fp16 v [B][Hkv][T_cap][d]) with the decode
    kernel's access pattern: the streaming ceiling of kvq_decode_attn on it."""
    B, Hkv, T_cap, bpk = codes.shape
    d = v.shape[-1]
    _check(_lib.kvq_stream_read(_dev(codes, "codes", torch.uint8), _dev(norms, "norms", torch.float32),
                                _dev(v, "v", torch.float16), B, Hkv, T_cap, d, bpk, n_splits, _dev(sink, "sink"),
                                _stream(stream)))


def kvq_select_signs_workspace(cb: kvq_codebook, n_cal: int, Hq: int, Hkv: int, T: int, C: int) -> int:
    return int(_lib.kvq_select_signs_workspace(ctypes.byref(cb), n_cal, Hq, Hkv, T, C))


def kvq_select_signs(cb: kvq_codebook, candidates, q: torch.Tensor, keys: torch.Tensor, v: torch.Tensor,
                     scale: float | None = None, workspace=None, stream=None):
    """Rank candidate sign patterns [C][d] on calibration q [n][Hq][d], keys/v [n][Hkv][T][d]: (errors, best)."""
    n, Hq, d = q.shape
    _, Hkv, T, _ = keys.shape
    cand = np.ascontiguousarray(np.asarray(candidates.cpu() if isinstance(candidates, torch.Tensor) else candidates,
                                           dtype=np.int8))
    if cand.ndim != 2 or cand.shape[1] != d:
        raise ValueError("candidates must have shape (C, %d)" % d)
    C = cand.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = kvq_select_signs_workspace(cb, n, Hq, Hkv, T, C)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    errors = np.zeros(C, dtype=np.float32)
    best = ctypes.c_int(-1)
    _check(_lib.kvq_select_signs(ctypes.byref(cb), cand.ctypes.data_as(_P), C, _dev(q, "q"), _dt(q),
                                 _dev(keys, "keys"), _dt(keys), _dev(v, "v"), _dt(v), n, Hq, Hkv, T, float(scale),
                                 errors.ctypes.data_as(_P), ctypes.byref(best), _dev(workspace, "workspace"),
                                 workspace.numel(), _stream(stream)))
    return errors, int(best.value)
