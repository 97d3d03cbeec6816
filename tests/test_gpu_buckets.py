"""GPU parity of the bucketed hash tables (mp_build_buckets) and of the
decode that looks the query's buckets up instead of scanning.

A key sits in bucket c of table l exactly when its code of table l is c, so:
(1) unpacked on the host, every bucket of every (unit, table, 8192-key
chunk) holds exactly the keys whose code is that bucket's; (2) a decode that
takes the tiles below n_buckets from the buckets gives the same sampled index
lists, counts and outputs as the decode that scans the codes, bit for bit,
and therefore meets the oracle's bars; (3) across appends, with the newest
chunk rebuilt whenever a 512-key tile fills, the step stays equal to the
scan and to the oracle.
"""
import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
import oracle
import synth
from tests.common import layer, oracle_decode, variant
from tests.test_gpu_parity import CASES, _compare, _inject, case, gpu_build

pytestmark = pytest.mark.gpu

CHUNK = mp.MP_BUCKET_CHUNK


def unpack_buckets(buf: np.ndarray, U: int, L: int, cap: int, K: int):
    """Host view of the layout: words [U][L][2^K][chunks] (start | count << 16), keys [U][L][cap]
    (uint16).  Returns the bucket offsets as [U][L][chunks][2^K + 1] (bucket c of chunk r: entries
    off[c] .. off[c+1] - 1), checking that each bucket starts where the one before it ends."""
    nb = 1 << K
    chunks = (cap + CHUNK - 1) // CHUNK
    noff = U * L * nb * chunks
    off_bytes = (4 * noff + 255) // 256 * 256
    words = buf[:4 * noff].view(np.uint32).reshape(U, L, nb, chunks).transpose(0, 1, 3, 2).astype(np.int64)
    start, count = words & 0xffff, words >> 16
    off = np.concatenate([start, (start[..., -1:] + count[..., -1:])], axis=3)
    keys = buf[off_bytes:off_bytes + 2 * U * L * cap].view(np.uint16).reshape(U, L, cap)
    return off, keys, start, count


def check_buckets_hold_their_codes(buf, codes, K, n1, n0=0):
    """Every bucket of the chunks [n0/CHUNK, ceil(n1/CHUNK)) holds exactly the keys with its code."""
    U, L, cap = codes.shape
    off, keys, start, count = unpack_buckets(buf, U, L, cap, K)
    nb = 1 << K
    for ci in range(n0 // CHUNK, (n1 + CHUNK - 1) // CHUNK):
        r0, r1 = ci * CHUNK, min((ci + 1) * CHUNK, n1)
        o = off[:, :, ci].astype(np.int64)  # [U][L][nb + 1]
        assert np.all(o[:, :, 0] == 0) and np.all(o[:, :, nb] == r1 - r0)
        assert np.array_equal(start[:, :, ci, 1:], start[:, :, ci, :-1] + count[:, :, ci, :-1])  # contiguous
        assert np.all(np.diff(o, axis=2) >= 0)
        c = codes[:, :, r0:r1].astype(np.int64)
        k = keys[:, :, r0:r1].astype(np.int64)  # entries of the chunk, ordered by bucket
        assert np.all(k < r1 - r0)
        # entry j lies in the bucket whose range contains j; its key's code must be that bucket
        for u in range(U):
            for l in range(L):
                bucket_of_entry = np.repeat(np.arange(nb), np.diff(o[u, l]))
                assert np.array_equal(c[u, l, k[u, l]], bucket_of_entry), (u, l, ci)
                assert np.array_equal(np.sort(k[u, l]), np.arange(r1 - r0)), (u, l, ci)  # each key once


@pytest.mark.parametrize("name", ["llama8b_layer", "g8_ragged", "mha_b3", "g2_small", "g4_f32", "tiny", "l512_g2"])
def test_buckets_hold_their_codes(name):
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    n1 = (lay["n"] // 512) * 512
    buf = mp.mp_build_buckets(gcodes, w.K, n1)
    torch.cuda.synchronize()
    check_buckets_hold_their_codes(buf.cpu().numpy(), codes, w.K, n1)


def _decode(w, lay, kmean, gcodes, qcodes, buckets=None, n_buckets=0, nsh=0, nst=0, T=2, planes=None, n_planes=0):
    B, Hq, cap = w.batch, w.hq, lay["cap"]
    out = torch.empty(B, Hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, Hq, dtype=torch.int32, device="cuda")
    mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, None, w.hkv, lay["n"], w.K, nsh, nst,
                      qcodes_in=qcodes, out=out, lse=lse, idx=idx, count=cnt, T=T, buckets=buckets,
                      n_buckets=n_buckets, planes=planes, n_planes=n_planes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("name,nsh,nst,part", [
    ("llama8b_layer", 0, 0, 1.0),
    ("llama8b_layer", 4, 64, 1.0),   # forced ranges inside bucket tiles
    ("llama8b_layer", 0, 0, 0.3),    # the first tiles from the buckets, the rest scanned
    ("g8_ragged", 0, 0, 1.0),
    ("g8_ragged", 4, 64, 1.0),
    ("mha_b3", 0, 0, 1.0),
    ("g2_small", 0, 0, 1.0),
    ("g4_f32", 0, 0, 1.0),
    ("g5_f32", 0, 0, 1.0),
    ("g6_bf16", 0, 0, 1.0),
    ("g7_bf16", 0, 0, 1.0),
    ("tiny", 0, 0, 1.0),
    ("l512_g2", 0, 0, 1.0),
    ("l512_g8", 4, 64, 1.0),
])
def test_decode_with_buckets(name, nsh, nst, part):
    """Sets, counts, outputs and lse bit-identical to the code scan, and within the oracle's bars."""
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    n1 = (lay["n"] // 512) * 512
    buf = mp.mp_build_buckets(gcodes, w.K, n1)
    nb = max(512, int(n1 * part) // 512 * 512)
    got = _decode(w, lay, kmean, gcodes, qcodes, buf, nb, nsh, nst)
    base = _decode(w, lay, kmean, gcodes, qcodes, None, 0, nsh, nst)
    for a, b, what in zip(got, base, ("out", "lse", "idx", "count")):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (name, what)
    ref = oracle_decode(w, lay, km, codes, qc, nsh=nsh, nst=nst)
    _compare(w, ref, *got, "%s buckets<%d nsh=%d nst=%d" % (name, nb, nsh, nst))


def test_buckets_with_other_thresholds_scan_the_codes():
    """The buckets serve threshold 2; with T = 3 they are ignored and the decode scans."""
    w, lay, km, codes, margin, qc = case("llama8b_layer")
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    n1 = (lay["n"] // 512) * 512
    buf = mp.mp_build_buckets(gcodes, w.K, n1)
    got = _decode(w, lay, kmean, gcodes, qcodes, buf, n1, T=3)
    base = _decode(w, lay, kmean, gcodes, qcodes, None, 0, T=3)
    for a, b in zip(got, base):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_buckets_and_planes_together():
    """Buckets below 2048 keys, bit planes from there to the last whole tile, codes above."""
    w, lay, km, codes, margin, qc = case("llama8b_layer")
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    n1 = (lay["n"] // 512) * 512
    buf = mp.mp_build_buckets(gcodes, w.K, 2048)
    planes = mp.mp_build_planes(gcodes, w.K, n1)
    got = _decode(w, lay, kmean, gcodes, qcodes, buf, 2048, planes=planes, n_planes=n1)
    base = _decode(w, lay, kmean, gcodes, qcodes)
    for a, b in zip(got, base):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("name", ["llama8b_layer", "g8_small"])
def test_index_maintenance_across_tile_boundaries(name):
    """A long appending decode with both indexes kept up to date by the
    caller's rule: whenever a 512-key tile fills, its plane tile and its
    bucket chunk are rebuilt (the appended keys are scanned until then).
    The step with buckets, the step with planes and the plain scan stay
    bit-identical at every step, and the oracle (decoding the GPU's own codes)
    agrees at the first step, on both sides of each rebuild and at the last."""
    w = variant("llama8b_layer", n=3500, steps=700) if name == "llama8b_layer" else \
        variant("codellama34b_b4", layers=1, batch=1, n=3900, steps=700)
    lay = layer(w, seed=808)
    Wp, kmean, codes = gpu_build(w, lay)
    U, cap, G = w.batch * w.hkv, lay["cap"], w.group
    n = lay["n"]
    runs = {}
    for mode in ("scan", "planes", "buckets"):
        runs[mode] = dict(Kc=lay["Kc"].clone(), Vc=lay["Vc"].clone(), codes=codes.clone(),
                          ws=mp.decode_workspace(w.batch, w.hq, w.hkv, cap, w.L, "cuda"))
    r = runs["planes"]
    r["planes"] = mp.mp_build_planes(r["codes"], w.K, (n // 512) * 512)
    r = runs["buckets"]
    r["buckets"] = mp.mp_build_buckets(r["codes"], w.K, (n // 512) * 512)
    n_idx = (n // 512) * 512
    steps = w.steps
    checks = {1, steps}
    rebuilds = 0
    for s in range(1, steps + 1):
        kn = torch.stack([synth.step_kv(808, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=s)[0]
                          for u in range(U)]).cuda()
        vn = torch.stack([synth.step_kv(808, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=s)[1]
                          for u in range(U)]).cuda()
        q = torch.stack([synth.unit_queries(808, 0, u // w.hkv, u % w.hkv, G, w.d, w.torch_dtype, step=s)
                         for u in range(U)]).reshape(w.batch, w.hq, w.d).cuda()
        res = {}
        for mode, r in runs.items():
            out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
            lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
            cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
            idx = torch.full((w.batch, w.hq, cap), -1, dtype=torch.int32, device="cuda")
            kw = {}
            if mode == "planes":
                kw = dict(planes=r["planes"], n_planes=n_idx)
            elif mode == "buckets":
                kw = dict(buckets=r["buckets"], n_buckets=n_idx)
            mp.mp_decode_step(kn, vn, q, r["Kc"], r["Vc"], r["codes"], kmean, Wp, w.hkv, n, w.K, r["ws"], out=out,
                              lse=lse, idx=idx, count=cnt, **kw)
            res[mode] = [t.cpu().numpy() for t in (out, lse, idx, cnt)]
        torch.cuda.synchronize()
        for mode in ("planes", "buckets"):
            for a, b in zip(res[mode], res["scan"]):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (s, mode)
        n += 1
        if n % 512 == 0:  # a tile filled: rebuild its plane tile and its bucket chunk
            mp.mp_build_planes(runs["planes"]["codes"], w.K, n, n0=n - 512, planes=runs["planes"]["planes"])
            mp.mp_build_buckets(runs["buckets"]["codes"], w.K, n, n0=(n - 512) // CHUNK * CHUNK,
                                buckets=runs["buckets"]["buckets"])
            n_idx = n
            rebuilds += 1
            checks |= {s, s + 1}
        if s in checks:
            gc = runs["scan"]["codes"]
            torch.cuda.synchronize()
            Kh = runs["scan"]["Kc"].float().cpu().numpy().reshape(w.batch, w.hkv, cap, w.d)
            Vh = runs["scan"]["Vc"].float().cpu().numpy().reshape(w.batch, w.hkv, cap, w.d)
            qh = q.float().cpu().numpy()
            qc = mp.mp_encode_queries(q, Wp, w.K, w.L).cpu().numpy()
            import oracle
            ref = oracle.decode(qh, Kh, Vh, gc.cpu().numpy().reshape(w.batch, w.hkv, w.L, cap),
                                kmean.cpu().numpy().reshape(w.batch, w.hkv, w.d), lay["host"]["W"], w.K, w.L, n,
                                qcodes=qc, want_idx=True)
            out, lse, idx, cnt = res["buckets"]
            _compare(w, ref, out, lse, idx, cnt, "%s step %d n=%d index<%d" % (name, s, n, n_idx))
    assert rebuilds >= 1
    # the rebuilt buckets hold their codes
    buf = runs["buckets"]["buckets"].cpu().numpy()
    check_buckets_hold_their_codes(buf, runs["buckets"]["codes"].cpu().numpy(), w.K, n_idx)


# One or two query heads per KV head and at least 4 x 256 x 7 = 7,168 one-tile
# sampling blocks: the sampling kernel takes the bitmap tiles four per block
# (the record in the first tile's slot, empty records in the others).
SPAN_CASES = {
    # one query head per KV head: 224 units x 33 tiles
    "mha_span": variant("codellama13b_b16", layers=1, batch=16, hq=14, hkv=14, n=16600, K=8, L=75),
    # two query heads per KV head: 224 units x 33 tiles
    "g2_span": variant("llama8b_layer", batch=28, hq=16, hkv=8, n=16600, K=8, L=75),
    # whole tiles only: 224 units x 32 tiles, every tile from the buckets (no tile scans)
    "mha_span_whole": variant("codellama13b_b16", layers=1, batch=16, hq=14, hkv=14, n=16384, K=8, L=75),
}
_span_cache = {}


def span_case(name):
    """Seeded keys, values and queries; the oracle's key means and query codes and seeded uniform
    codes for every unit (the same on both sides), injected into the device's stores."""
    if name not in _span_cache:
        w = SPAN_CASES[name]
        U = w.batch * w.hkv
        print("[gpu parity] span case %s: B=%d Hq=%d Hkv=%d n=%d K=%d L=%d" % (name, w.batch, w.hq, w.hkv, w.n,
                                                                             w.K, w.L), flush=True)
        lay = layer(w, seed=4321)
        cap, n = lay["cap"], lay["n"]
        h = lay["host"]
        keys = h["K"].reshape(U, cap, w.d)
        km = np.stack([oracle.key_mean(keys[u, :n]) for u in range(U)])
        codes = np.stack([synth.unit_codes(4321, 0, u // w.hkv, u % w.hkv, w.K, w.L, cap).numpy().astype(np.uint16)
                          for u in range(U)])
        qc = oracle.encode(h["q"].reshape(-1, w.d), h["W"], w.K, w.L).reshape(w.batch, w.hq, w.L)
        _span_cache[name] = (w, lay, km, codes, qc)
    return _span_cache[name]


@pytest.mark.parametrize("name,nb_tiles,nsh,nst,pl_tiles", [
    ("mha_span", 32, 0, 0, 0),    # eight blocks of four bitmap tiles; the short last tile scanned
    ("mha_span", 31, 4, 64, 0),   # a last block of three bitmap tiles, two tiles scanned; forced ranges
    ("mha_span", 17, 0, 0, 32),   # bitmap tiles below 17 (a last block of one), planes to 32, codes above
    ("g2_span", 30, 0, 0, 0),
    ("mha_span_whole", 32, 0, 0, 0),  # every tile from the bitmaps
])
def test_bitmap_tiles_shared_by_sampling_blocks(name, nb_tiles, nsh, nst, pl_tiles):
    """Index lists and counts equal the code scan's (one tile per block) and
    the oracle's; outputs and lse within the oracle's bars and within
    rounding of the scan's; the merge without index lists, and the two stages
    called apart, give the same bits."""
    w, lay, km, codes, qc = span_case(name)
    U = w.batch * w.hkv
    assert w.group <= 2 and U * ((lay["n"] + 511) // 512) >= 4 * 256 * 7
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    nb, npl = nb_tiles * 512, pl_tiles * 512
    buf = mp.mp_build_buckets(gcodes, w.K, nb)
    planes = mp.mp_build_planes(gcodes, w.K, npl) if npl else None
    got = _decode(w, lay, kmean, gcodes, qcodes, buf, nb, nsh, nst, planes=planes, n_planes=npl)
    base = _decode(w, lay, kmean, gcodes, qcodes, None, 0, nsh, nst)
    assert np.array_equal(got[2], base[2]) and np.array_equal(got[3], base[3])
    assert np.allclose(got[0], base[0], rtol=1e-5, atol=1e-6)
    fin = np.isfinite(base[1])
    assert np.array_equal(fin, np.isfinite(got[1])) and np.allclose(got[1][fin], base[1][fin], rtol=0, atol=1e-5)
    # the merge without index lists (four heads or fewer per unit: the wider merge) gives the same bits
    out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
    cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
    mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, None, w.hkv, lay["n"], w.K, nsh, nst,
                      qcodes_in=qcodes, out=out, lse=lse, count=cnt, buckets=buf, n_buckets=nb, planes=planes,
                      n_planes=npl)
    torch.cuda.synchronize()
    for a, b in zip((out, lse, cnt), got[:2] + got[3:]):
        assert np.array_equal(a.cpu().numpy().view(np.uint8), b.view(np.uint8))
    # the two stages called apart, the merge told the sampling stage's bucket bound: the same bits
    ws = mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda")
    mp.mp_decode_sample(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, qcodes, w.hkv, lay["n"], w.K, ws,
                        n_static_head=nsh, n_static_tail=nst, want_idx=True, buckets=buf, n_buckets=nb,
                        planes=planes, n_planes=npl)
    idx = torch.full((w.batch, w.hq, lay["cap"]), -7, dtype=torch.int32, device="cuda")
    mp.mp_decode_merge(w.batch, w.hq, w.hkv, lay["n"], lay["cap"], w.L, out, ws, lse=lse, idx=idx, count=cnt,
                       n_buckets=nb)
    torch.cuda.synchronize()
    for a, b in zip((out, lse, idx, cnt), got):
        assert np.array_equal(a.cpu().numpy().view(np.uint8), b.view(np.uint8))
    ref = oracle_decode(w, lay, km, codes, qc, nsh=nsh, nst=nst)
    _compare(w, ref, *got, "%s buckets<%d planes<%d nsh=%d nst=%d (four tiles per block)" % (name, nb, npl, nsh, nst))
