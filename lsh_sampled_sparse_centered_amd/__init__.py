"""Python binding of libmagicpig.so, the gfx950 SimHash-sampled decode-attention library.

Every function here has the name of the C entry point it calls and only
marshals arguments: it checks tensor devices, dtypes, shapes and contiguity,
passes raw device pointers and the current HIP stream, and raises
:class:`MPError` on a non-zero status.  All computation runs in the HIP
kernels.  torch is used for device memory and streams only.

The method is MagicPIG (arXiv 2410.16179v2); see ``include/magicpig.h`` for
what each call computes, with citations.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmagicpig.so")

MP_BF16 = 0
MP_F32 = 1
D = 128

_c_int, _c_i64, _c_sz, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "mp_strerror": ([_c_int], ctypes.c_char_p),
    "mp_version": ([], _c_int),
    "mp_proj_bytes": ([_c_int, _c_int, _c_int], _c_sz),
    "mp_proj_pack": ([_vp, _c_int, _c_int, _c_int, _vp, _vp], _c_int),
    "mp_build_ws_bytes": ([_c_i64, _c_i64, _c_int], _c_sz),
    "mp_build_codes": ([_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp, _c_sz, _vp],
                       _c_int),
    "mp_append": ([_vp, _vp, _vp, _vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _c_int, _c_int, _vp, _vp],
                  _c_int),
    "mp_encode_queries": ([_vp, _c_int, _c_i64, _c_int, _vp, _c_int, _c_int, _vp, _vp], _c_int),
    "mp_decode_ws_bytes": ([_c_int, _c_int, _c_int, _c_i64, _c_int, _c_int], _c_sz),
    "mp_planes_bytes": ([_c_i64, _c_i64, _c_int, _c_int], _c_sz),
    "mp_build_planes": ([_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _vp, _vp], _c_int),
    "mp_proj_bytes_lift": ([_c_int, _c_int, _c_int], _c_sz),
    "mp_proj_pack_lift": ([_vp, _c_int, _c_int, _c_int, _vp, _vp], _c_int),
    "mp_build_codes_lift": ([_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp,
                             _c_sz, _vp], _c_int),
    "mp_append_lift": ([_vp, _vp, _vp, _vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _vp, _c_int, _c_int,
                        _vp, _vp], _c_int),
    "mp_decode_attn_lift": ([_vp, _vp, _vp, _c_int, _vp, _vp, _c_i64, _vp, _c_i64, _vp, _vp, _vp, _c_int, _c_int,
                             _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, _c_sz, _vp], _c_int),
    "mp_buckets_bytes": ([_c_i64, _c_i64, _c_int, _c_int], _c_sz),
    "mp_build_buckets": ([_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_int, _vp, _c_sz, _vp], _c_int),
    "mp_decode_attn": ([_vp, _vp, _vp, _c_int, _vp, _vp, _c_i64, _vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_int, _c_i64,
                        _c_i64, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                        _c_sz, _vp], _c_int),
    "mp_decode_sample": ([_vp, _vp, _vp, _c_int, _vp, _vp, _c_i64, _vp, _c_i64, _vp, _vp, _c_int, _c_int, _c_int,
                          _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_int, _vp, _c_sz, _vp],
                         _c_int),
    "mp_decode_merge": ([_c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_i64, _vp, _vp, _vp,
                         _vp, _vp, _c_sz, _vp],
                        _c_int),
    "mp_decode_step": ([_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_i64, _vp, _c_i64, _vp, _vp, _c_int, _c_int,
                        _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _vp, _vp, _vp, _vp,
                        _vp, _c_sz, _vp, _vp], _c_int),
    "mp_decode_step_static": ([_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _c_i64, _vp, _c_i64, _vp, _vp, _c_int,
                               _c_int, _c_int, _c_i64, _c_i64, _c_int, _c_int, _c_int, _c_int, _c_i64, _c_i64, _vp,
                               _vp, _vp, _vp, _vp, _vp], _c_int),
}

MP_STATIC_SCRATCH_BYTES = 32 << 20  # size of the library's static scratch (include/magicpig.h)
MP_BUCKET_CHUNK = 8192  # keys per chunk of the bucketed tables (magicpig.h)

_lib = None


class MPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, strerror(status), status))
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded native library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmagicpig.so is not built (expected at %s); run "
                               "`python -m lsh_sampled_sparse_centered_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def strerror(status: int) -> str:
    return lib().mp_strerror(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MPError(fn, status)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _event_pair(events):
    """ctypes array of the two raw hipEvent_t handles of torch events (None: no timing)."""
    if events is None:
        return None
    handles = [int(e.cuda_event) for e in events]
    if len(handles) != 2 or not all(handles):
        raise ValueError("sample_events needs two torch.cuda.Event objects that were recorded once")
    return ctypes.cast((ctypes.c_void_p * 2)(*handles), ctypes.c_void_p)


def _kv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MP_BF16
    if t.dtype == torch.float32:
        return MP_F32
    raise ValueError("keys/values/queries must be bfloat16 or float32, got %s" % t.dtype)


def _need(t: torch.Tensor, dtype: torch.dtype, shape, name: str):
    if t.dtype != dtype:
        raise ValueError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


# ----------------------------------------------------------------------------- projections
def mp_proj_bytes(d: int, K: int, L: int) -> int:
    return lib().mp_proj_bytes(d, K, L)


def mp_proj_pack(W: torch.Tensor, K: int, L: int, Wp: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pack W[d][K*L] fp32 into the encoder's bf16 tile order; returns the uint8 buffer."""
    d = W.shape[0]
    _need(W, torch.float32, (d, K * L), "W")
    nb = mp_proj_bytes(d, K, L)
    if Wp is None:
        Wp = torch.empty(max(nb, 16), dtype=torch.uint8, device=W.device)
    _check("mp_proj_pack", lib().mp_proj_pack(_p(W), d, K, L, _p(Wp), _stream(stream)))
    return Wp


# ----------------------------------------------------------------------------- build / append
def mp_build_ws_bytes(U: int, n: int, d: int = D) -> int:
    return lib().mp_build_ws_bytes(U, n, d)


def mp_build_codes(Kc: torch.Tensor, n: int, Wp: torch.Tensor, K: int, L: int, kmean: Optional[torch.Tensor] = None,
                   codes: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Key means and the table-major code store of ``Kc`` ([U][cap][d]) for its first n rows."""
    U, cap, d = Kc.shape
    if kmean is None:
        kmean = torch.empty(U, d, dtype=torch.float32, device=Kc.device)
    if codes is None:
        codes = torch.zeros(U, L, cap, dtype=torch.uint16, device=Kc.device)
    _need(kmean, torch.float32, (U, d), "kmean")
    _need(codes, torch.uint16, (U, L, cap), "codes")
    nb = mp_build_ws_bytes(U, max(n, 1), d)
    if ws is None:
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=Kc.device)
    _check("mp_build_codes", lib().mp_build_codes(_p(Kc), _kv_dtype(Kc), U, n, cap, d, _p(Wp), K, L, _p(kmean),
                                                  _p(codes), _p(ws), ws.numel() * ws.element_size(),
                                                  _stream(stream)))
    return kmean, codes


def mp_append(k_new: torch.Tensor, v_new: torch.Tensor, Kc: torch.Tensor, Vc: torch.Tensor, n: int,
              kmean: torch.Tensor, Wp: torch.Tensor, K: int, L: int, codes: torch.Tensor, stream=None) -> None:
    """Write row n of the caches and its codes (frozen mean)."""
    U, cap, d = Kc.shape
    _need(k_new, Kc.dtype, (U, d), "k_new")
    _need(v_new, Kc.dtype, (U, d), "v_new")
    _need(Vc, Kc.dtype, (U, cap, d), "Vc")
    _need(codes, torch.uint16, (U, L, cap), "codes")
    _check("mp_append", lib().mp_append(_p(k_new), _p(v_new), _p(Kc), _p(Vc), _kv_dtype(Kc), U, n, cap, d, _p(kmean),
                                        _p(Wp), K, L, _p(codes), _stream(stream)))


def mp_encode_queries(q: torch.Tensor, Wp: torch.Tensor, K: int, L: int, qcodes: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """SimHash codes of queries ``q`` ([..., d], uncentred); returns uint16 [..., L]."""
    d = q.shape[-1]
    nq = q.numel() // d
    if qcodes is None:
        qcodes = torch.empty(*q.shape[:-1], L, dtype=torch.uint16, device=q.device)
    _check("mp_encode_queries", lib().mp_encode_queries(_p(q), _kv_dtype(q), nq, d, _p(Wp), K, L, _p(qcodes),
                                                        _stream(stream)))
    return qcodes


# ----------------------------------------------------------------------------- lift (Equation 8)
def mp_proj_bytes_lift(d: int, K: int, L: int) -> int:
    return lib().mp_proj_bytes_lift(d, K, L)


def mp_proj_pack_lift(W: torch.Tensor, K: int, L: int, Wp: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Pack W[d + 1][K*L] fp32 (the lifted projections); returns the uint8 buffer."""
    d = W.shape[0] - 1
    _need(W, torch.float32, (d + 1, K * L), "W")
    nb = mp_proj_bytes_lift(d, K, L)
    if nb == 0:
        raise MPError("mp_proj_bytes_lift", -2)
    if Wp is None:
        Wp = torch.empty(nb, dtype=torch.uint8, device=W.device)
    _check("mp_proj_pack_lift", lib().mp_proj_pack_lift(_p(W), d, K, L, _p(Wp), _stream(stream)))
    return Wp


def mp_build_codes_lift(Kc: torch.Tensor, n: int, Wp: torch.Tensor, K: int, L: int, stream=None):
    """Key means, lift radii and codes of the lifted centred keys; returns (kmean, rlift, codes)."""
    U, cap, d = Kc.shape
    kmean = torch.empty(U, d, dtype=torch.float32, device=Kc.device)
    rlift = torch.empty(U, dtype=torch.float32, device=Kc.device)
    codes = torch.zeros(U, L, cap, dtype=torch.uint16, device=Kc.device)
    nb = mp_build_ws_bytes(U, max(n, 1), d)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=Kc.device)
    _check("mp_build_codes_lift", lib().mp_build_codes_lift(_p(Kc), _kv_dtype(Kc), U, n, cap, d, _p(Wp), K, L,
                                                            _p(kmean), _p(rlift), _p(codes), _p(ws), ws.numel(),
                                                            _stream(stream)))
    return kmean, rlift, codes


def mp_append_lift(k_new, v_new, Kc, Vc, n: int, kmean, rlift, Wp, K: int, L: int, codes, stream=None) -> None:
    """Write row n of the caches and its lifted codes (frozen mean and radius)."""
    U, cap, d = Kc.shape
    _need(k_new, Kc.dtype, (U, d), "k_new")
    _need(v_new, Kc.dtype, (U, d), "v_new")
    _need(rlift, torch.float32, (U,), "rlift")
    _need(codes, torch.uint16, (U, L, cap), "codes")
    _check("mp_append_lift", lib().mp_append_lift(_p(k_new), _p(v_new), _p(Kc), _p(Vc), _kv_dtype(Kc), U, n, cap, d,
                                                  _p(kmean), _p(rlift), _p(Wp), K, L, _p(codes), _stream(stream)))


def mp_planes_bytes(U: int, cap: int, K: int, L: int) -> int:
    return lib().mp_planes_bytes(U, cap, K, L)


def mp_build_planes(codes: torch.Tensor, K: int, n1: int, n0: int = 0, planes: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Bit-plane index of ``codes`` ([U][L][cap] uint16) for keys [n0, n1) (multiples of 512).

    Returns (or fills) ``planes``: uint32 [U][ceil(cap/512)][K][L][16]."""
    U, L, cap = codes.shape
    shape = (U, (cap + 511) // 512, K, L, 16)
    if planes is None:
        planes = torch.empty(shape, dtype=torch.int32, device=codes.device)
    _need(planes, torch.int32, shape, "planes")
    _check("mp_build_planes", lib().mp_build_planes(_p(codes), U, n0, n1, cap, K, L, _p(planes), _stream(stream)))
    return planes


def mp_buckets_bytes(U: int, cap: int, K: int, L: int) -> int:
    return lib().mp_buckets_bytes(U, cap, K, L)


def mp_build_buckets(codes: torch.Tensor, K: int, n1: int, n0: int = 0, buckets: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Bucketed hash tables of ``codes`` ([U][L][cap] uint16) for the chunks
    of MP_BUCKET_CHUNK keys from n0 (a multiple of MP_BUCKET_CHUNK) up to n1 (a multiple of 512).

    Returns (or fills) ``buckets``: a uint8 buffer of mp_buckets_bytes bytes."""
    U, L, cap = codes.shape
    nb = mp_buckets_bytes(U, cap, K, L)
    if nb == 0:
        raise MPError("mp_buckets_bytes", -2)
    if buckets is None:
        buckets = torch.empty(nb, dtype=torch.uint8, device=codes.device)
    if buckets.dtype != torch.uint8 or buckets.dim() != 1:
        raise ValueError("buckets: expected a 1-D uint8 buffer")
    _check("mp_build_buckets", lib().mp_build_buckets(_p(codes), U, n0, n1, cap, K, L, _p(buckets), buckets.numel(),
                                                      _stream(stream)))
    return buckets


# ----------------------------------------------------------------------------- decode
def mp_decode_ws_bytes(B: int, Hq: int, Hkv: int, cap: int, L: int, d: int = D) -> int:
    return lib().mp_decode_ws_bytes(B, Hq, Hkv, cap, d, L)


def decode_workspace(B: int, Hq: int, Hkv: int, cap: int, L: int, device) -> torch.Tensor:
    nb = mp_decode_ws_bytes(B, Hq, Hkv, cap, L)
    if nb == 0:
        raise MPError("mp_decode_ws_bytes", -2)
    return torch.empty(nb, dtype=torch.uint8, device=device)


def _decode_shapes(q, Kc, Vc, codes, kmean, Hkv):
    B, Hq, d = q.shape
    U, cap, _ = Kc.shape
    if U != B * Hkv:
        raise ValueError("Kc has %d units, expected B*Hkv = %d" % (U, B * Hkv))
    _need(Vc, Kc.dtype, Kc.shape, "Vc")
    if q.dtype != Kc.dtype:
        raise ValueError("q and the caches must share a dtype")
    L = codes.shape[1]
    _need(codes, torch.uint16, (U, L, cap), "codes")
    _need(kmean, torch.float32, (U, d), "kmean")
    return B, Hq, d, U, cap, L


def _planes_ok(planes, codes, K, buckets=None):
    U, L, cap = codes.shape
    if planes is not None:
        _need(planes, torch.int32, (U, (cap + 511) // 512, K, L, 16), "planes")
    if buckets is not None:
        nb = mp_buckets_bytes(U, cap, K, L)
        if buckets.dtype != torch.uint8 or buckets.dim() != 1 or buckets.numel() < nb:
            raise ValueError("buckets: expected a 1-D uint8 buffer of at least %d bytes" % nb)


def mp_decode_attn(q: torch.Tensor, Kc: torch.Tensor, Vc: torch.Tensor, codes: torch.Tensor, kmean: torch.Tensor,
                   Wp: Optional[torch.Tensor], Hkv: int, n: int, K: int, n_static_head: int = 0,
                   n_static_tail: int = 0, qcodes_in: Optional[torch.Tensor] = None,
                   qcodes_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                   count: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None,
                   T: int = 2, planes: Optional[torch.Tensor] = None, n_planes: int = 0,
                   buckets: Optional[torch.Tensor] = None, n_buckets: int = 0):
    """Sampled decode attention of one layer.  q [B][Hq][d]; caches [B*Hkv][cap][d].

    ``T`` is the collision threshold (a key is sampled when it collides with
    the query in at least T of the L tables; the pages use 2).  ``planes``
    (from mp_build_planes, valid below ``n_planes``) lets the T = 2 scan read
    the bit-plane index for those tiles; ``buckets`` (from mp_build_buckets,
    valid below ``n_buckets``) replaces the T = 2 scan of those tiles by a
    lookup of the query's buckets."""
    B, Hq, d, U, cap, L = _decode_shapes(q, Kc, Vc, codes, kmean, Hkv)
    dev = q.device
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    _need(out, torch.float32, (B, Hq, d), "out")
    if lse is not None:
        _need(lse, torch.float32, (B, Hq), "lse")
    if count is not None:
        _need(count, torch.int32, (B, Hq), "count")
    if idx is not None:
        _need(idx, torch.int32, (B, Hq, cap), "idx")
    for name, t in (("qcodes_in", qcodes_in), ("qcodes_out", qcodes_out)):
        if t is not None:
            _need(t, torch.uint16, (B, Hq, L), name)
    if ws is None:
        ws = decode_workspace(B, Hq, Hkv, cap, L, dev)
    _planes_ok(planes, codes, K, buckets)
    st = lib().mp_decode_attn(_p(q), _p(Kc), _p(Vc), _kv_dtype(Kc), _p(codes), _p(planes), n_planes, _p(buckets),
                              n_buckets, _p(kmean), _p(Wp),
                              B, Hq, Hkv, n, cap,
                              d, K, L, T, n_static_head, n_static_tail, _p(qcodes_in), _p(qcodes_out), _p(out), _p(lse),
                              _p(idx), _p(count), _p(ws), ws.numel(), _stream(stream))
    _check("mp_decode_attn", st)
    return out


def mp_decode_attn_lift(q, Kc, Vc, codes, kmean, rlift, Wp, Hkv: int, n: int, K: int, qcodes_in=None, out=None,
                        lse=None, idx=None, count=None, ws=None, stream=None, T: int = 2, n_static_head: int = 0,
                        n_static_tail: int = 0, buckets=None, n_buckets: int = 0, planes=None, n_planes: int = 0):
    """mp_decode_attn for keys hashed lifted (Equation 8), with the units' radii ``rlift`` [B*Hkv]."""
    B, Hq, d, U, cap, L = _decode_shapes(q, Kc, Vc, codes, kmean, Hkv)
    _need(rlift, torch.float32, (U,), "rlift")
    dev = q.device
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    _need(out, torch.float32, (B, Hq, d), "out")
    if lse is not None:
        _need(lse, torch.float32, (B, Hq), "lse")
    if count is not None:
        _need(count, torch.int32, (B, Hq), "count")
    if idx is not None:
        _need(idx, torch.int32, (B, Hq, cap), "idx")
    if qcodes_in is not None:
        _need(qcodes_in, torch.uint16, (B, Hq, L), "qcodes_in")
    if ws is None:
        ws = decode_workspace(B, Hq, Hkv, cap, L, dev)
    _planes_ok(planes, codes, K, buckets)
    st = lib().mp_decode_attn_lift(_p(q), _p(Kc), _p(Vc), _kv_dtype(Kc), _p(codes), _p(planes), n_planes,
                                   _p(buckets), n_buckets, _p(kmean), _p(rlift), _p(Wp), B, Hq, Hkv, n, cap, d, K, L,
                                   T, n_static_head, n_static_tail, _p(qcodes_in), None, _p(out), _p(lse), _p(idx),
                                   _p(count), _p(ws), ws.numel(), _stream(stream))
    _check("mp_decode_attn_lift", st)
    return out


def mp_decode_sample(q, Kc, Vc, codes, kmean, qcodes, Hkv: int, n: int, K: int, ws: torch.Tensor,
                     n_static_head: int = 0, n_static_tail: int = 0, want_idx: bool = False, stream=None,
                     T: int = 2, planes: Optional[torch.Tensor] = None, n_planes: int = 0,
                     buckets: Optional[torch.Tensor] = None, n_buckets: int = 0) -> None:
    """Scan (or bucket lookup) + weighting + split attention into the workspace (first stage of mp_decode_attn)."""
    B, Hq, d, U, cap, L = _decode_shapes(q, Kc, Vc, codes, kmean, Hkv)
    _need(qcodes, torch.uint16, (B, Hq, L), "qcodes")
    _planes_ok(planes, codes, K, buckets)
    st = lib().mp_decode_sample(_p(q), _p(Kc), _p(Vc), _kv_dtype(Kc), _p(codes), _p(planes), n_planes, _p(buckets),
                                n_buckets, _p(kmean),
                                _p(qcodes), B, Hq, Hkv,
                                n, cap, d, K, L, T, n_static_head, n_static_tail, int(bool(want_idx)), _p(ws), ws.numel(),
                                _stream(stream))
    _check("mp_decode_sample", st)


def mp_decode_merge(B: int, Hq: int, Hkv: int, n: int, cap: int, L: int, out: torch.Tensor, ws: torch.Tensor,
                    lse: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    count: Optional[torch.Tensor] = None, d: int = D, stream=None,
                    kv_dtype: torch.dtype = torch.bfloat16, T: int = 2, n_buckets: int = 0) -> None:
    """Log-sum-exp merge of the sampled partials (second stage of mp_decode_attn); ``kv_dtype``, ``T``
    and ``n_buckets`` as the sampling stage had them (0 without buckets)."""
    _need(out, torch.float32, (B, Hq, d), "out")
    code = MP_BF16 if kv_dtype == torch.bfloat16 else MP_F32 if kv_dtype == torch.float32 else -1
    st = lib().mp_decode_merge(code, B, Hq, Hkv, n, cap, d, L, T, n_buckets, _p(out), _p(lse), _p(idx), _p(count),
                               _p(ws), ws.numel(), _stream(stream))
    _check("mp_decode_merge", st)


def _step_args(k_new, v_new, q, Kc, Vc, codes, kmean, Hkv, K, out, lse, idx, count, planes, buckets):
    B, Hq, d, U, cap, L = _decode_shapes(q, Kc, Vc, codes, kmean, Hkv)
    if k_new is not None:
        _need(k_new, Kc.dtype, (U, d), "k_new")
        _need(v_new, Kc.dtype, (U, d), "v_new")
    if out is None:
        out = torch.empty(B, Hq, d, dtype=torch.float32, device=q.device)
    _need(out, torch.float32, (B, Hq, d), "out")
    if lse is not None:
        _need(lse, torch.float32, (B, Hq), "lse")
    if count is not None:
        _need(count, torch.int32, (B, Hq), "count")
    if idx is not None:
        _need(idx, torch.int32, (B, Hq, cap), "idx")
    _planes_ok(planes, codes, K, buckets)
    return B, Hq, d, cap, L, out


def mp_decode_step_static(k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor], q: torch.Tensor,
                          Kc: torch.Tensor, Vc: torch.Tensor, codes: torch.Tensor, kmean: torch.Tensor,
                          Wp: torch.Tensor, Hkv: int, n: int, K: int, out: torch.Tensor,
                          lse: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                          count: Optional[torch.Tensor] = None, n_static_head: int = 0, n_static_tail: int = 0,
                          sample_events=None, stream=None, T: int = 2, planes: Optional[torch.Tensor] = None,
                          n_planes: int = 0, buckets: Optional[torch.Tensor] = None,
                          n_buckets: int = 0) -> torch.Tensor:
    """mp_decode_step with the library's static scratch as its workspace: the
    native call allocates nothing (``out`` must be given, so this wrapper
    allocates nothing either).  Calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("mp_decode_step_static: out must be given")
    B, Hq, d, cap, L, out = _step_args(k_new, v_new, q, Kc, Vc, codes, kmean, Hkv, K, out, lse, idx, count, planes,
                                       buckets)
    st = lib().mp_decode_step_static(_p(k_new), _p(v_new), _p(q), _p(Kc), _p(Vc), _kv_dtype(Kc), _p(codes),
                                     _p(planes), n_planes, _p(buckets), n_buckets, _p(kmean), _p(Wp), B, Hq, Hkv, n,
                                     cap, d, K, L, T,
                                     n_static_head, n_static_tail, _p(out), _p(lse), _p(idx), _p(count),
                                     _event_pair(sample_events), _stream(stream))
    _check("mp_decode_step_static", st)
    return out


def mp_decode_step(k_new: Optional[torch.Tensor], v_new: Optional[torch.Tensor], q: torch.Tensor, Kc: torch.Tensor,
                   Vc: torch.Tensor, codes: torch.Tensor, kmean: torch.Tensor, Wp: torch.Tensor, Hkv: int, n: int,
                   K: int, ws: torch.Tensor, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None, n_static_head: int = 0,
                   n_static_tail: int = 0, sample_events=None, stream=None, T: int = 2,
                   planes: Optional[torch.Tensor] = None, n_planes: int = 0, buckets: Optional[torch.Tensor] = None,
                   n_buckets: int = 0) -> torch.Tensor:
    """Append (k_new, v_new) at row n (unless None), encode q, sample and merge over the keys.

    ``sample_events``: optional pair of torch.cuda.Event objects (created with
    timing and recorded once, so that their handles exist); they are attached
    to the sampling kernel's dispatch and record its start and end."""
    B, Hq, d, cap, L, out = _step_args(k_new, v_new, q, Kc, Vc, codes, kmean, Hkv, K, out, lse, idx, count, planes,
                                       buckets)
    st = lib().mp_decode_step(_p(k_new), _p(v_new), _p(q), _p(Kc), _p(Vc), _kv_dtype(Kc), _p(codes), _p(planes),
                              n_planes, _p(buckets), n_buckets, _p(kmean), _p(Wp),
                              B, Hq, Hkv, n, cap, d, K, L, T, n_static_head, n_static_tail, _p(out), _p(lse), _p(idx),
                              _p(count), _p(ws), ws.numel(), _event_pair(sample_events), _stream(stream))
    _check("mp_decode_step", st)
    return out
