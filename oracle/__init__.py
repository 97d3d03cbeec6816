"""CPU oracle for SimHash-sampled decode attention (MagicPIG, arXiv 2410.16179v2).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use this package; the product path never does.
It wraps ``mp_oracle.c`` (plain C, fp64) with numpy-friendly functions.  It
shares no code with the HIP library.

Each wrapper names the step of the method it follows; the C file states the
readings taken where the pages leave a step open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mp_oracle.c")
_LIB = os.path.join(_HERE, "libmp_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.orc_set_threads.argtypes = [_int]
        L.orc_set_threads.restype = None
        L.orc_bf16.argtypes = [ctypes.c_float]
        L.orc_bf16.restype = ctypes.c_float
        L.orc_key_mean.argtypes = [_f32p, _i64, _int, _i64, _f32p]
        L.orc_key_mean.restype = None
        L.orc_encode.argtypes = [_f32p, _i64, _int, _i64, _vp, _i64, _f32p, _int, _int, _u16p, _i64, _i64, _vp]
        L.orc_encode.restype = None
        L.orc_table_collision_prob.argtypes = [ctypes.c_double, _int]
        L.orc_table_collision_prob.restype = ctypes.c_double
        L.orc_sampling_prob_p.argtypes = [ctypes.c_double, _int]
        L.orc_sampling_prob_p.restype = ctypes.c_double
        L.orc_sampling_prob.argtypes = [ctypes.c_double, _int, _int]
        L.orc_sampling_prob.restype = ctypes.c_double
        L.orc_sampling_prob_pt.argtypes = [ctypes.c_double, _int, _int]
        L.orc_sampling_prob_pt.restype = ctypes.c_double
        L.orc_sampling_prob_t.argtypes = [ctypes.c_double, _int, _int, _int]
        L.orc_sampling_prob_t.restype = ctypes.c_double
        L.orc_scan_t.argtypes = [_u16p, _i64, _i64, _int, _int, _u16p, _i64, _i64, _vp, _vp]
        L.orc_scan_t.restype = _i64
        L.orc_attend_t.argtypes = [_f32p, _f32p, _f32p, _i64, _int, _vp, _int, _int, _int, _i32p, _vp, _i64,
                                   _f64p, _f64p, _vp]
        L.orc_attend_t.restype = None
        L.orc_build.argtypes = [_f32p, _i64, _i64, _i64, _int, _f32p, _int, _int, _f32p, _u16p, _vp]
        L.orc_build.restype = None
        L.orc_decode_t.argtypes = [_f32p, _f32p, _f32p, _u16p, _f32p, _f32p, _vp, _int, _int, _int, _i64, _i64,
                                   _int, _int, _int, _int, _i64, _i64, _vp, _f32p, _f32p, _vp, _i32p]
        L.orc_decode_t.restype = None
        L.orc_lift_radius.argtypes = [_f32p, _i64, _int, _i64, _f32p]
        L.orc_lift_radius.restype = ctypes.c_float
        L.orc_encode_lifted.argtypes = [_f32p, _i64, _int, _i64, _vp, _i64, _int, ctypes.c_float, _f32p, _int, _int,
                                        _u16p, _i64, _i64, _vp]
        L.orc_encode_lifted.restype = None
        L.orc_attend_lt.argtypes = [_f32p, _f32p, _f32p, _i64, _int, _vp, ctypes.c_float, _int, _int, _int, _i32p,
                                    _vp, _i64, _f64p, _f64p, _vp]
        L.orc_attend_lt.restype = None
        L.orc_decode_lt.argtypes = [_f32p, _f32p, _f32p, _u16p, _f32p, _vp, _f32p, _vp, _int, _int, _int, _i64, _i64,
                                    _int, _int, _int, _int, _i64, _i64, _vp, _f32p, _f32p, _vp, _i32p]
        L.orc_decode_lt.restype = None
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (timing only)."""
    lib().orc_set_threads(int(n))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def bf16(x) -> np.ndarray:
    """bf16 round-to-nearest-even of fp32 values (returned as fp32)."""
    x = _f32(x)
    f = lib().orc_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.float32).reshape(x.shape)


def key_mean(keys) -> np.ndarray:
    """Key mean k_avg (Section 4.3 'Data pre-processing'): fp64 sum, one fp32 rounding."""
    keys = _f32(keys)
    n, d = keys.shape
    mu = np.empty(d, np.float32)
    lib().orc_key_mean(keys, n, d, d, mu)
    return mu


def encode(rows, W, K: int, L: int, mu=None, with_margin: bool = False):
    """SimHash codes ``[nrows][L]`` of ``rows`` (centred by ``mu`` when given:
    one mean ``[d]`` for every row, or one per row ``[nrows][d]``).

    Section 2.2 and Section 4.3 'Hash function selection'.  With
    ``with_margin`` also returns, per (row, projection column j = l*K + b),
    the relative projection size |z_j|/(|x||w_j|) (+inf where that norm
    product is 0: the projection is exactly 0 and the bit exactly 0).
    """
    rows = _f32(rows)
    if rows.ndim == 1:
        rows = rows[None]
    nrows, d = rows.shape
    W = _f32(W)
    assert W.shape == (d, K * L)
    codes = np.zeros((nrows, L), np.uint16)
    margin = np.zeros((nrows, K * L), np.float32) if with_margin else None
    mu_a = None if mu is None else _f32(mu)
    mu_stride = 0
    if mu_a is not None and mu_a.ndim == 2:
        assert mu_a.shape == (nrows, d)
        mu_stride = d
    lib().orc_encode(rows, nrows, d, d, _ptr(mu_a), mu_stride, W, K, L, codes, L, 1, _ptr(margin))
    return (codes, margin) if with_margin else codes


def lift_radius(keys, mu) -> float:
    """Lift radius of Section 4.2, Equation 8: the largest |bf16(k - mu)| (fp64 sums, one fp32 rounding)."""
    keys = _f32(keys)
    n, d = keys.shape
    return float(lib().orc_lift_radius(keys, n, d, d, _f32(mu)))


def encode_lifted(rows, W, K: int, L: int, mu=None, R: float = 0.0, lift: bool = True, with_margin: bool = False):
    """SimHash codes of lifted rows (Section 4.2, Equation 8): ``W`` is
    ``[d + 1][K*L]``; keys (``lift``) get the extra coordinate
    bf16(sqrt(R^2 - |x|^2)), queries (``lift=False``) get 0.  ``mu`` is one
    mean ``[d]`` or one per row ``[nrows][d]``.  With ``with_margin`` also the
    per-column margins ``[nrows][K*L]``."""
    rows = _f32(rows)
    if rows.ndim == 1:
        rows = rows[None]
    nrows, d = rows.shape
    W = _f32(W)
    assert W.shape == (d + 1, K * L)
    codes = np.zeros((nrows, L), np.uint16)
    margin = np.zeros((nrows, K * L), np.float32) if with_margin else None
    mu_a = None if mu is None else _f32(mu)
    mu_stride = d if (mu_a is not None and mu_a.ndim == 2) else 0
    lib().orc_encode_lifted(rows, nrows, d, d, _ptr(mu_a), mu_stride, int(bool(lift)), float(R), W, K, L, codes, L,
                            1, _ptr(margin))
    return (codes, margin) if with_margin else codes


def build_codes_lifted(keys, n: int, W, K: int, L: int, with_margin: bool = False):
    """Lifted code-store build of one layer: per unit the key mean, the lift
    radius and the codes of the lifted centred keys.  ``keys`` ``[U][cap][d]``,
    ``W`` ``[d + 1][K*L]``.  Returns kmean ``[U][d]``, rlift ``[U]``, codes
    ``[U][L][cap]`` and, with ``with_margin``, margins ``[U][n][K*L]``."""
    keys = _f32(keys)
    U, cap, d = keys.shape
    kmean = np.zeros((U, d), np.float32)
    rlift = np.zeros(U, np.float32)
    codes = np.zeros((U, L, cap), np.uint16)
    margin = np.zeros((U, n, K * L), np.float32) if with_margin else None
    for u in range(U):
        kmean[u] = key_mean(keys[u, :n])
        rlift[u] = lift_radius(keys[u, :n], kmean[u])
        c, m = encode_lifted(keys[u, :n], W, K, L, mu=kmean[u], R=rlift[u], with_margin=True)
        codes[u][:, :n] = c.T
        if with_margin:
            margin[u] = m
    return (kmean, rlift, codes, margin) if with_margin else (kmean, rlift, codes)


def table_collision_prob(cos_qk: float, K: int) -> float:
    """(1 - theta/pi)^K: one table's collision probability (Section 2.2)."""
    return lib().orc_table_collision_prob(float(cos_qk), int(K))


def sampling_prob_p(p: float, L: int, T: int = 2) -> float:
    """P(at least T of L tables collide) for per-table probability p (Equation 10 for T = 2)."""
    return lib().orc_sampling_prob_pt(float(p), int(L), int(T))


def sampling_prob(cos_qk: float, K: int, L: int, T: int = 2) -> float:
    """Sampling probability of a key at cosine ``cos_qk`` from the query (Equation 10 for T = 2)."""
    return lib().orc_sampling_prob_t(float(cos_qk), int(K), int(L), int(T))


def scan(codes_tn, qcode, n_static_head: int = 0, n_static_tail: int = 0, T: int = 2):
    """Sampled set of one query head: ascending indices and forced flags.

    ``codes_tn`` is table-major ``[L][n]``; Section 4.3 (at least T tables,
    the pages' T = 2).
    """
    codes_tn = np.ascontiguousarray(codes_tn, dtype=np.uint16)
    L, n = codes_tn.shape
    qcode = np.ascontiguousarray(qcode, dtype=np.uint16)
    idx = np.zeros(max(n, 1), np.int32)
    forced = np.zeros(max(n, 1), np.uint8)
    cnt = lib().orc_scan_t(codes_tn, n, n, L, T, qcode, n_static_head, n_static_tail, _ptr(idx), _ptr(forced))
    return idx[:cnt].copy(), forced[:cnt].astype(bool)


def attend(q, keys, vals, idx, forced, K: int, L: int, mu=None, with_logw: bool = False, T: int = 2,
           rlift: float = 0.0):
    """Estimator of one head over its sampled set (Equations 9 and 11).

    Returns ``(out[d] fp64, lse)`` (and the per-sample log-weights).  With
    ``rlift`` > 0 the keys were hashed lifted (Equation 8) and the sampling
    angle uses the lifted key's norm ``rlift``.
    """
    q, keys, vals = _f32(q), _f32(keys), _f32(vals)
    n, d = keys.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    cnt = idx.shape[0]
    forced_a = None if forced is None else np.ascontiguousarray(forced, dtype=np.uint8)
    out = np.zeros(d, np.float64)
    lse = np.zeros(1, np.float64)
    logw = np.zeros(max(cnt, 1), np.float64) if with_logw else None
    mu_a = None if mu is None else _f32(mu)
    lib().orc_attend_lt(q, keys, vals, d, d, _ptr(mu_a), float(rlift), K, L, T,
                        idx if cnt else np.zeros(1, np.int32), _ptr(forced_a), cnt, out, lse, _ptr(logw))
    if with_logw:
        return out, float(lse[0]), logw[:cnt]
    return out, float(lse[0])


def build_codes(keys, n: int, W, K: int, L: int, with_margin: bool = False):
    """Code-store build of one layer.  ``keys`` is ``[U][cap][d]`` (any float dtype).

    Returns ``kmean [U][d]``, ``codes [U][L][cap]`` (columns >= n zero) and,
    with ``with_margin``, ``margin [U][n][K*L]`` (per key and projection column).
    """
    keys = _f32(keys)
    U, cap, d = keys.shape
    W = _f32(W)
    kmean = np.zeros((U, d), np.float32)
    codes = np.zeros((U, L, cap), np.uint16)
    margin = np.zeros((U, n, K * L), np.float32) if with_margin else None
    lib().orc_build(keys, U, n, cap, d, W, K, L, kmean, codes, _ptr(margin))
    return (kmean, codes, margin) if with_margin else (kmean, codes)


def decode(q, keys, vals, codes, kmean, W, K: int, L: int, n: int, qcodes=None, n_static_head: int = 0,
           n_static_tail: int = 0, want_idx: bool = False, T: int = 2, rlift=None):
    """Decode of one layer (Algorithm 1 for every query head; a key is sampled
    when it collides in at least T tables, the pages' T = 2).

    Shapes: q ``[B][Hq][d]``, keys/vals ``[B][Hkv][cap][d]``, codes
    ``[B][Hkv][L][cap]``, kmean ``[B][Hkv][d]``, qcodes ``[B][Hq][L]`` or None.
    ``rlift`` (``[B][Hkv]``, optional) gives the units' lift radii when the
    keys were hashed lifted (Equation 8).
    Returns a dict with out, lse, count, qcodes and (optionally) idx lists.
    """
    q, keys, vals = _f32(q), _f32(keys), _f32(vals)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = keys.shape
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    kmean = _f32(kmean)
    W = _f32(W)
    qc_in = None if qcodes is None else np.ascontiguousarray(qcodes, dtype=np.uint16)
    qc_out = np.zeros((B, Hq, L), np.uint16)
    out = np.zeros((B, Hq, d), np.float32)
    lse = np.zeros((B, Hq), np.float32)
    count = np.zeros((B, Hq), np.int32)
    idx = np.full((B, Hq, cap), -1, np.int32) if want_idx else None
    rl = None if rlift is None else _f32(np.asarray(rlift).reshape(B, Hkv))
    lib().orc_decode_lt(q, keys, vals, codes, kmean, _ptr(rl), W, _ptr(qc_in), B, Hq, Hkv, n, cap, d, K, L, T,
                        n_static_head, n_static_tail, _ptr(qc_out), out, lse, _ptr(idx), count)
    res = {"out": out, "lse": lse, "count": count, "qcodes": qc_out}
    if want_idx:
        res["idx"] = [[idx[b, h, :count[b, h]].copy() for h in range(Hq)] for b in range(B)]
    return res
