"""Host-only checks of the C ABI: the library loads, exports every declared
entry point, and rejects invalid arguments with the documented status
before anything is enqueued (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import lsh_sampled_sparse_centered_amd as mp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "magicpig.h")

pytestmark = pytest.mark.skipif(not os.path.exists(mp.LIB_PATH), reason="libmagicpig.so not built")

FAKE = 0x10000  # never dereferenced: every call below fails validation first
OK, ARG, UNSUP, CAP, WS = 0, -1, -2, -3, -4


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(mp_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(mp.exported_symbols())


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mp.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_strerror_and_version():
    for code in (OK, ARG, UNSUP, CAP, WS, -5):
        assert len(mp.strerror(code)) > 5
    assert mp.strerror(12345) == "unknown status"
    assert mp.lib().mp_version() == 3


def test_size_queries():
    assert mp.mp_proj_bytes(128, 10, 150) == 50 * 8 * 64 * 16  # 3 tables of 10 bits per 32-column tile
    assert mp.mp_proj_bytes(128, 8, 75) == 19 * 8 * 64 * 16
    assert mp.mp_proj_bytes(64, 8, 75) == 0
    assert mp.mp_proj_bytes(128, 17, 75) == 0
    assert mp.mp_proj_bytes(128, 10, 1) == 0
    assert mp.mp_build_ws_bytes(8, 16384) == 8 * (16384 // 512) * 128 * 8  # fp64 partial sums per 512 keys
    a = mp.mp_decode_ws_bytes(1, 32, 8, 98368, 150)
    b = mp.mp_decode_ws_bytes(1, 32, 8, 2 * 98368, 150)
    assert 0 < a < b
    assert mp.mp_decode_ws_bytes(1, 32, 7, 1024, 150) == 0  # Hq % Hkv
    assert mp.mp_decode_ws_bytes(1, 32, 2, 1024, 150) == 0  # G = 16 > 8


def _build(**kw):
    a = dict(Kc=FAKE, dt=0, U=8, n=100, cap=128, d=128, Wp=FAKE, K=8, L=75, km=FAKE, codes=FAKE, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return mp.lib().mp_build_codes(a["Kc"], a["dt"], a["U"], a["n"], a["cap"], a["d"], a["Wp"], a["K"], a["L"],
                                   a["km"], a["codes"], a["ws"], a["wsb"], None)


def test_build_rejects_invalid_arguments():
    assert _build(d=64) == UNSUP
    assert _build(K=17) == UNSUP
    assert _build(L=1) == UNSUP
    assert _build(K=16, L=300) == UNSUP
    assert _build(dt=7) == ARG
    assert _build(Kc=None) == ARG
    assert _build(codes=None) == ARG
    assert _build(cap=100) == ARG  # not a multiple of 8
    assert _build(n=0) == CAP
    assert _build(n=129) == CAP
    assert _build(ws=None) == WS
    assert _build(wsb=16) == WS
    for arg in ("Kc", "Wp", "km", "codes", "ws"):  # 16-byte vector loads and stores
        assert _build(**{arg: FAKE + 8}) == ARG, arg


def _append(**kw):
    a = dict(k=FAKE, v=FAKE, Kc=FAKE, Vc=FAKE, dt=0, U=8, n=100, cap=128, d=128, km=FAKE, Wp=FAKE, K=8, L=75,
             codes=FAKE)
    a.update(kw)
    return mp.lib().mp_append(a["k"], a["v"], a["Kc"], a["Vc"], a["dt"], a["U"], a["n"], a["cap"], a["d"], a["km"],
                              a["Wp"], a["K"], a["L"], a["codes"], None)


def test_append_rejects_invalid_arguments():
    assert _append(n=128) == CAP
    assert _append(n=500) == CAP
    assert _append(n=-1) == ARG
    assert _append(v=None) == ARG
    assert _append(d=256) == UNSUP
    assert _append(cap=129) == ARG
    for arg in ("k", "v", "Kc", "Vc", "km", "Wp", "codes"):
        assert _append(**{arg: FAKE + 4}) == ARG, arg


def _decode(**kw):
    a = dict(q=FAKE, Kc=FAKE, Vc=FAKE, dt=0, codes=FAKE, planes=None, np=0, bk=None, nb=0, km=FAKE, Wp=FAKE, B=1,
             Hq=32, Hkv=8, n=100, cap=128, d=128, K=8, L=75, T=2, nsh=0, nst=0, qin=None, qout=None, out=FAKE,
             lse=None, idx=None, cnt=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return mp.lib().mp_decode_attn(a["q"], a["Kc"], a["Vc"], a["dt"], a["codes"], a["planes"], a["np"], a["bk"],
                                   a["nb"], a["km"],
                                   a["Wp"], a["B"], a["Hq"],
                                   a["Hkv"], a["n"], a["cap"], a["d"], a["K"], a["L"], a["T"], a["nsh"], a["nst"], a["qin"],
                                   a["qout"], a["out"], a["lse"], a["idx"], a["cnt"], a["ws"], a["wsb"], None)


def test_decode_rejects_invalid_arguments():
    assert _decode(Hkv=7) == ARG
    assert _decode(Hkv=2) == UNSUP  # 16 query heads per KV head
    assert _decode(B=0) == ARG
    assert _decode(n=129) == CAP
    assert _decode(n=-1) == CAP
    assert _decode(nsh=-1) == ARG
    assert _decode(out=None) == ARG
    assert _decode(Wp=None) == ARG  # needed to encode q when no qcodes_in
    assert _decode(ws=None) == WS
    assert _decode(wsb=100) == WS
    assert _decode(d=96) == UNSUP
    assert _decode(B=70000, Hq=8, Hkv=8) == UNSUP
    assert _decode(cap=1 << 26) == UNSUP  # a scan batch's row offsets must fit 32 bits
    assert _decode(T=0) == UNSUP  # collision threshold outside [1, L]
    assert _decode(T=76) == UNSUP
    for arg in ("q", "Kc", "Vc", "codes", "km", "Wp", "out", "ws"):
        assert _decode(**{arg: FAKE + 2}) == ARG, arg
    # bit-plane index: whole 512-key tiles at or below n, 16-byte aligned
    assert _decode(planes=FAKE, np=100, n=1000, cap=1024) == ARG
    assert _decode(planes=FAKE, np=1024, n=1000, cap=1024) == ARG
    assert _decode(planes=FAKE + 4, np=512, n=1000, cap=1024) == ARG
    assert _decode(planes=FAKE, np=-512, n=1000, cap=1024) == ARG
    # bucketed tables: whole 512-key tiles at or below n, 16-byte aligned, a K they can exist for
    assert _decode(bk=FAKE, nb=100, n=1000, cap=1024) == ARG
    assert _decode(bk=FAKE, nb=1024, n=1000, cap=1024) == ARG
    assert _decode(bk=FAKE + 4, nb=512, n=1000, cap=1024) == ARG
    assert _decode(bk=FAKE, nb=512, n=1000, cap=1024, K=13) == ARG


def test_build_planes_rejects_invalid_arguments():
    L = mp.lib()
    assert L.mp_planes_bytes(8, 98304, 10, 150) == 8 * 192 * 10 * 150 * 64
    assert L.mp_planes_bytes(2, 1000, 8, 75) == 2 * 2 * 8 * 75 * 64  # the last tile is partial
    assert L.mp_planes_bytes(2, 1024, 0, 75) == 0
    ok = dict(codes=FAKE, U=2, n0=0, n1=1024, cap=1024, K=8, L=75, planes=FAKE)

    def b(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mp_build_planes(a["codes"], a["U"], a["n0"], a["n1"], a["cap"], a["K"], a["L"], a["planes"], None)

    assert b(codes=None) == ARG
    assert b(planes=None) == ARG
    assert b(planes=FAKE + 4) == ARG
    assert b(n0=100) == ARG
    assert b(n1=1000) == ARG
    assert b(n1=1536) == ARG  # past cap
    assert b(n0=1024, n1=512) == ARG
    assert b(K=0) == ARG
    assert b(L=513) == UNSUP
    assert b(cap=1020) == ARG
    assert b(n0=512, n1=512) == OK  # nothing to do


def test_build_buckets_rejects_invalid_arguments():
    L = mp.lib()
    # offsets: one 4-byte word per (unit, table, bucket, 8192-key chunk), then the keys, each part
    # 256-byte aligned
    off = 8 * 150 * 1024 * 13 * 4
    assert L.mp_buckets_bytes(8, 98368, 10, 150) == (off + 255) // 256 * 256 + 8 * 150 * 98368 * 2
    assert L.mp_buckets_bytes(2, 1024, 0, 75) == 0
    assert L.mp_buckets_bytes(2, 1024, 13, 75) == 0
    ok = dict(codes=FAKE, U=2, n0=0, n1=1024, cap=1024, K=8, L=75, bk=FAKE, nb=1 << 30)

    def b(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mp_build_buckets(a["codes"], a["U"], a["n0"], a["n1"], a["cap"], a["K"], a["L"], a["bk"], a["nb"],
                                  None)

    assert b(codes=None) == ARG
    assert b(bk=None) == ARG
    assert b(bk=FAKE + 4) == ARG
    assert b(n0=512) == ARG  # chunk starts are multiples of 8192
    assert b(n0=4096, n1=4096, cap=8192) == ARG
    assert b(n1=1000) == ARG
    assert b(n1=1536) == ARG  # past cap
    assert b(K=0) == UNSUP
    assert b(K=13) == UNSUP
    assert b(L=513) == UNSUP
    assert b(cap=1020) == ARG
    assert b(nb=100) == WS
    assert b(n0=0, n1=0) == OK  # nothing to do


def test_decode_stages_reject_invalid_arguments():
    L = mp.lib()
    assert L.mp_decode_sample(FAKE, FAKE, FAKE, 0, FAKE, None, 0, None, 0, FAKE, None, 1, 32, 8, 100, 128, 128, 8, 75,
                              2, 0, 0, 0, FAKE, 1 << 30, None) == ARG  # qcodes required
    assert L.mp_decode_sample(FAKE, FAKE, FAKE, 0, FAKE, None, 0, None, 0, FAKE, FAKE, 1, 32, 8, 100, 128, 128, 8, 75,
                              0, 0, 0, 0, FAKE, 1 << 30, None) == UNSUP  # threshold 0
    assert L.mp_decode_sample(FAKE, FAKE, FAKE, 0, FAKE, FAKE, 512, None, 0, FAKE, FAKE, 1, 32, 8, 100, 128, 128, 8,
                              75, 2, 0, 0, 0, FAKE, 1 << 30, None) == ARG  # planes past n
    assert L.mp_decode_sample(FAKE, FAKE, FAKE, 0, FAKE, None, 0, FAKE, 512, FAKE, FAKE, 1, 32, 8, 100, 128, 128, 8,
                              75, 2, 0, 0, 0, FAKE, 1 << 30, None) == ARG  # buckets past n
    assert L.mp_decode_merge(0, 1, 32, 8, 100, 128, 128, 75, 2, 0, None, None, None, None, FAKE, 1 << 30, None) == ARG
    assert L.mp_decode_merge(0, 1, 32, 8, 100, 128, 128, 75, 2, 0, FAKE, None, None, None, FAKE, 10, None) == WS
    assert L.mp_decode_merge(0, 1, 32, 8, 100, 128, 128, 75, 2, 512, FAKE, None, None, None, FAKE, 1 << 30,
                             None) == ARG  # buckets past n
    assert L.mp_decode_merge(0, 1, 32, 8, 100, 128, 128, 75, 0, 0, FAKE, None, None, None, FAKE, 1 << 30,
                             None) == UNSUP  # threshold 0
    assert L.mp_decode_merge(7, 1, 32, 8, 100, 128, 128, 75, 2, 0, FAKE, None, None, None, FAKE, 1 << 30,
                             None) != OK  # no such dtype


def test_encode_queries_rejects_invalid_arguments():
    L = mp.lib()
    assert L.mp_encode_queries(FAKE, 0, 0, 128, FAKE, 8, 75, FAKE, None) == ARG
    assert L.mp_encode_queries(FAKE, 3, 4, 128, FAKE, 8, 75, FAKE, None) == ARG
    assert L.mp_encode_queries(FAKE, 0, 4, 128, FAKE, 8, 513, FAKE, None) == UNSUP
    assert L.mp_proj_pack(None, 128, 8, 75, FAKE, None) == ARG
    assert L.mp_proj_pack(FAKE, 128, 8, 75, FAKE + 8, None) == ARG
    assert L.mp_encode_queries(FAKE + 8, 0, 4, 128, FAKE, 8, 75, FAKE, None) == ARG


def _step(**kw):
    a = dict(k=FAKE, v=FAKE, q=FAKE, Kc=FAKE, Vc=FAKE, dt=0, codes=FAKE, planes=None, np=0, bk=None, nb=0, km=FAKE,
             Wp=FAKE, B=1, Hq=32, Hkv=8, n=100, cap=128, d=128, K=8, L=75, T=2, nsh=0, nst=0, out=FAKE, lse=None,
             idx=None, cnt=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return mp.lib().mp_decode_step(a["k"], a["v"], a["q"], a["Kc"], a["Vc"], a["dt"], a["codes"], a["planes"],
                                   a["np"], a["bk"], a["nb"], a["km"], a["Wp"],
                                   a["B"], a["Hq"], a["Hkv"], a["n"], a["cap"], a["d"], a["K"], a["L"], a["T"], a["nsh"],
                                   a["nst"], a["out"], a["lse"], a["idx"], a["cnt"], a["ws"], a["wsb"], None, None)


def test_step_rejects_invalid_arguments():
    assert _step(v=None) == ARG
    assert _step(n=128) == CAP  # no room for the appended row
    assert _step(n=-1) == CAP
    assert _step(Wp=None) == ARG
    assert _step(out=None) == ARG
    assert _step(Hkv=3) == ARG
    assert _step(ws=None) == WS
    assert _step(T=0) == UNSUP
    assert _step(planes=FAKE, np=512, n=511, cap=1024) == ARG  # the appended key is not in the index
    assert _step(bk=FAKE, nb=512, n=511, cap=1024) == ARG  # nor in the buckets
    for arg in ("k", "v", "q", "Kc", "Vc", "codes", "km", "Wp", "out", "ws"):
        assert _step(**{arg: FAKE + 4}) == ARG, arg


def _static(**kw):
    a = dict(k=FAKE, v=FAKE, q=FAKE, Kc=FAKE, Vc=FAKE, dt=0, codes=FAKE, planes=None, np=0, bk=None, nb=0, km=FAKE,
             Wp=FAKE, B=1, Hq=32, Hkv=8, n=100, cap=128, d=128, K=8, L=75, T=2, nsh=0, nst=0, out=FAKE, lse=None,
             idx=None, cnt=None)
    a.update(kw)
    return mp.lib().mp_decode_step_static(a["k"], a["v"], a["q"], a["Kc"], a["Vc"], a["dt"], a["codes"],
                                          a["planes"], a["np"], a["bk"], a["nb"], a["km"], a["Wp"], a["B"], a["Hq"],
                                          a["Hkv"], a["n"],
                                          a["cap"], a["d"], a["K"], a["L"], a["T"], a["nsh"], a["nst"], a["out"],
                                          a["lse"], a["idx"], a["cnt"], None, None)


def test_static_step_rejects_invalid_arguments_and_oversized_shapes():
    """The allocation-free step validates like mp_decode_step (no workspace
    argument) and rejects a shape whose workspace exceeds its static scratch
    with MP_ERR_SCRATCH, all before any HIP call."""
    SCRATCH = -6
    assert len(mp.strerror(SCRATCH)) > 5
    assert _static(v=None) == ARG
    assert _static(n=128) == CAP
    assert _static(Wp=None) == ARG
    assert _static(out=None) == ARG
    assert _static(Hkv=3) == ARG
    assert _static(T=0) == UNSUP
    for arg in ("k", "v", "q", "Kc", "Vc", "codes", "km", "Wp", "out"):
        assert _static(**{arg: FAKE + 4}) == ARG, arg
    # the CodeLlama-13B-shaped batch of 16 MHA sequences needs far more than the scratch
    big = dict(B=16, Hq=40, Hkv=40, n=16384, cap=16448, K=9, L=120)
    assert mp.mp_decode_ws_bytes(16, 40, 40, 16448, 120) > mp.MP_STATIC_SCRATCH_BYTES
    assert _static(**big) == SCRATCH
    assert mp.mp_decode_ws_bytes(1, 32, 8, 98368, 150) <= mp.MP_STATIC_SCRATCH_BYTES  # the 96K layer fits


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="these arguments pass validation and would launch kernels on fake pointers")
def test_valid_arguments_pass_validation():
    """Arguments at the documented limits pass validation (the calls then
    fail to launch: there is no GPU here)."""
    assert _decode(cap=(1 << 26) - 8, wsb=1 << 40) not in (ARG, UNSUP, CAP, WS)
    assert _decode(T=1) not in (ARG, UNSUP) and _decode(T=75) not in (ARG, UNSUP)
    assert _decode(planes=None, np=12345) not in (ARG, UNSUP)  # ignored without planes
    assert _step(planes=FAKE, np=512, n=512, cap=1024) not in (ARG, UNSUP, CAP, WS)


def test_lift_entry_points_reject_invalid_arguments():
    L = mp.lib()
    assert L.mp_proj_bytes_lift(128, 10, 150) == L.mp_proj_bytes(128, 10, 150) + 50 * 32 * 2
    assert L.mp_proj_bytes_lift(128, 0, 150) == 0
    assert L.mp_proj_pack_lift(None, 128, 8, 75, FAKE, None) == ARG
    assert L.mp_proj_pack_lift(FAKE, 128, 0, 75, FAKE, None) == UNSUP
    assert L.mp_build_codes_lift(FAKE, 0, 8, 100, 128, 128, FAKE, 8, 75, FAKE, None, FAKE, FAKE, 1 << 30,
                                 None) == ARG  # rlift required
    assert L.mp_build_codes_lift(FAKE, 0, 8, 100, 128, 128, FAKE, 0, 75, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                 None) == UNSUP
    assert L.mp_build_codes_lift(FAKE, 0, 8, 100, 128, 128, FAKE, 8, 75, FAKE, FAKE, FAKE, FAKE, 10, None) == WS
    assert L.mp_append_lift(FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 128, 128, FAKE, FAKE, FAKE, 8, 75, FAKE, None) == CAP
    assert L.mp_append_lift(FAKE, FAKE, FAKE, FAKE, 0, 8, 10, 128, 128, FAKE, None, FAKE, 8, 75, FAKE, None) == ARG
    assert L.mp_decode_attn_lift(FAKE, FAKE, FAKE, 0, FAKE, None, 0, None, 0, FAKE, None, FAKE, 1, 32, 8, 100, 128,
                                 128, 8, 75, 2, 0, 0, None, None, FAKE, None, None, None, FAKE, 1 << 30,
                                 None) == ARG  # rlift required
