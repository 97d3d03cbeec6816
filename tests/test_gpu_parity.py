"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bars (floating point is bf16-in / fp32-accumulate on the GPU, fp64 in the
oracle):
  * key means: bitwise equal;
  * codes: equal bit for bit, except bits whose own projection is within
    the rounding band |z| < 1e-5 |x| |w| (the oracle reports |z|/(|x||w|)
    per projection column);
  * with the oracle's codes injected: sampled index lists and counts equal
    exactly; outputs within 2e-3 max-abs; lse within 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
import oracle
import synth
from tests.common import BAND, code_mismatches_outside_band, host_f32, layer, oracle_codes, oracle_decode, variant

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3

CASES = {
    # fp32 keys, one head, (8, 75)
    "tiny": variant("tiny"),
    # Llama-3.1-8B-shaped layer: 32 q heads over 8 KV heads, (8, 75)
    "llama8b_layer": variant("llama8b_layer"),
    # 8 query heads per KV head, (10, 240), ragged n (not a multiple of 512)
    "g8_ragged": variant("codellama34b_b4", layers=1, batch=1, n=5000, steps=0),
    # MHA with batch 3, (9, 120)
    "mha_b3": variant("codellama13b_b16", layers=1, batch=3, hq=4, hkv=4, n=3000),
    # 2 query heads per KV head, odd K and L, short n
    "g2_small": variant("llama8b_layer", hq=4, hkv=2, n=777, K=6, L=33),
    # 3 query heads per KV head (not a power of two), K = 16
    "g3_k16": variant("llama8b_layer", hq=6, hkv=2, n=1500, K=16, L=20),
    # fp32 caches with 4 query heads per KV head
    "g4_f32": variant("llama8b_layer", hq=8, hkv=2, n=2500, dtype="f32"),
    # 5, 6 and 7 query heads per KV head: the eight-head kernel with heads unused
    "g5_f32": variant("llama8b_layer", hq=10, hkv=2, n=1800, dtype="f32"),
    "g6_bf16": variant("codellama34b_b4", layers=1, batch=2, hq=12, hkv=2, n=3000, steps=0),
    "g7_bf16": variant("codellama13b_b16", layers=1, batch=1, hq=7, hkv=1, n=2100),
    # the merges' two phase counts: 64 partial records per head (the most merged in 8 phases) and 65
    # (the fewest merged in 32)
    "mha_64rec": variant("codellama13b_b16", layers=1, batch=1, hq=2, hkv=2, n=64 * 512),
    "g4_65rec": variant("llama8b_layer", hq=4, hkv=1, n=64 * 512 + 232),
    # the most tables (L = 512, K * L = 4096): two tables per lookup thread, the largest query-code tables
    "l512_g2": variant("llama8b_layer", hq=4, hkv=2, n=3000, K=8, L=512),
    "l512_g8": variant("codellama34b_b4", layers=1, batch=1, n=1100, K=8, L=512, steps=0),
}

_cache = {}


def case(name):
    if name not in _cache:
        w = CASES[name]
        print("[gpu parity] case %s: B=%d Hq=%d Hkv=%d n=%d K=%d L=%d %s" % (name, w.batch, w.hq, w.hkv, w.n, w.K,
                                                                           w.L, w.dtype), flush=True)
        lay = layer(w, seed=1234)
        km, codes, margin, qc = oracle_codes(w, lay)
        _cache[name] = (w, lay, km, codes, margin, qc)
    return _cache[name]


def gpu_build(w, lay):
    Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
    kmean, codes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, w.K, w.L)
    return Wp, kmean, codes


@pytest.mark.parametrize("name", list(CASES))
def test_key_mean_and_codes(name):
    w, lay, km, codes, margin, qc = case(name)
    Wp, kmean, gcodes = gpu_build(w, lay)
    torch.cuda.synchronize()
    gk = kmean.cpu().numpy()
    assert np.array_equal(gk.view(np.uint32), km.view(np.uint32)), "key means differ in %d elements" % int(
        (gk != km).sum())
    n = lay["n"]
    g = gcodes.cpu().numpy()[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    r = codes[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    ndiff, nbad = code_mismatches_outside_band(g, r, margin.reshape(-1, w.K * w.L))
    print("[gpu parity] %s: %d of %d codes differ, all inside the band" % (name, ndiff, g.size))
    assert nbad == 0
    # columns >= n are untouched
    assert int(gcodes[:, :, n:].cpu().numpy().astype(np.int64).sum()) == 0


@pytest.mark.parametrize("name", list(CASES))
def test_query_codes(name):
    w, lay, km, codes, margin, qc = case(name)
    Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
    gq = mp.mp_encode_queries(lay["q"], Wp, w.K, w.L).cpu().numpy().reshape(-1, w.L)
    h = lay["host"]
    ref, mg = oracle.encode(h["q"].reshape(-1, w.d), h["W"], w.K, w.L, with_margin=True)
    ndiff, nbad = code_mismatches_outside_band(gq, ref, mg)
    assert nbad == 0


@pytest.mark.parametrize("K", [1, 2, 3, 4, 5, 6, 7, 8, 11, 12, 15, 16])
def test_codes_every_table_width(K):
    """Codes of every table width the encoders handle differently: a 32-bit
    tile word holds floor(32/K) tables (32 for K = 1 down to 2 for K >= 11).
    In the build encoder, 2 to 4 tables per tile (K = 7 to 16) take the path
    whose lanes store their codes directly with a fixed number of buffer
    stores per stage (dropped past the row or table range); 5 to 8 tables
    (K = 4 to 6) transpose a stage's codes through LDS; K <= 3 store each
    code from its lane.  L = 37 leaves a partial last tile; n = 700 a ragged
    last row block.  Build (large encoder), 8 query rows and one append
    (small encoder), all against the oracle."""
    w = variant("llama8b_layer", hq=4, hkv=2, n=700, K=K, L=37)
    lay = layer(w, seed=40 + K)
    km, codes, margin, qc = oracle_codes(w, lay)
    Wp, kmean, gcodes = gpu_build(w, lay)
    n = lay["n"]
    torch.cuda.synchronize()
    assert np.array_equal(kmean.cpu().numpy().view(np.uint32), km.view(np.uint32))
    g = gcodes.cpu().numpy()[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    r = codes[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    assert code_mismatches_outside_band(g, r, margin.reshape(-1, w.K * w.L))[1] == 0
    assert int(gcodes[:, :, n:].cpu().numpy().astype(np.int64).sum()) == 0  # columns >= n untouched
    h = lay["host"]
    q = lay["q"].reshape(-1, w.d)[:8]
    gq = mp.mp_encode_queries(q, Wp, w.K, w.L).cpu().numpy().reshape(-1, w.L)
    ref, mg = oracle.encode(h["q"].reshape(-1, w.d)[:8], h["W"], w.K, w.L, with_margin=True)
    assert code_mismatches_outside_band(gq, ref, mg)[1] == 0
    kn = lay["Kc"][:, n - 1].clone()
    mp.mp_append(kn, torch.zeros_like(kn), lay["Kc"], lay["Vc"], n, kmean, Wp, w.K, w.L, gcodes)
    torch.cuda.synchronize()
    got = gcodes.cpu().numpy()[:, :, n]
    U = w.batch * w.hkv
    for u in range(U):
        ref, mg = oracle.encode(host_f32(kn)[u][None], h["W"], w.K, w.L, mu=km[u], with_margin=True)
        assert code_mismatches_outside_band(got[u][None], ref, mg)[1] == 0, u


@pytest.mark.parametrize("rows", [5, 100])
def test_zero_rows_encode_to_zero_codes(rows):
    """A zero row projects to exactly 0 in every column, and (z > 0) is false:
    all its codes are 0 (the oracle agrees), for the small-job (<= 64 rows)
    and the large encoder alike.  An appended key equal to the frozen mean
    (fp32 cache) is such a row after centring."""
    w = variant("tiny", K=10, L=30)
    lay = layer(w, seed=5)
    Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
    q = torch.randn(1, rows, w.d, generator=torch.Generator().manual_seed(3)).cuda()
    q[0, 1] = 0.0
    q[0, rows - 1] = -0.0
    got = mp.mp_encode_queries(q, Wp, w.K, w.L).cpu().numpy().reshape(rows, w.L)
    ref = oracle.encode(host_f32(q).reshape(rows, w.d), lay["host"]["W"], w.K, w.L)
    assert np.all(ref[1] == 0) and np.all(ref[rows - 1] == 0)
    assert np.all(got[1] == 0) and np.all(got[rows - 1] == 0)
    _, nbad = code_mismatches_outside_band(got, ref, oracle.encode(host_f32(q).reshape(rows, w.d), lay["host"]["W"],
                                                                   w.K, w.L, with_margin=True)[1])
    assert nbad == 0
    # append a key equal to the frozen mean: centred row = 0 -> codes 0
    kmean, gcodes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, w.K, w.L)
    n = lay["n"]
    kn = kmean.clone()
    mp.mp_append(kn, torch.zeros_like(kn), lay["Kc"], lay["Vc"], n, kmean, Wp, w.K, w.L, gcodes)
    torch.cuda.synchronize()
    assert int(np.abs(gcodes.view(torch.int16)[0, :, n].cpu().numpy().astype(np.int64)).sum()) == 0


def test_zero_projection_column_encodes_bit_zero():
    """A zero projection column projects every row to exactly 0, and
    (z > 0) is false: that bit is 0 in every code of the build, the
    queries and an append, as in the oracle (whose margin for that column is
    infinite, so any difference would be outside the band)."""
    w = variant("llama8b_layer", hq=4, hkv=2, n=900, K=10, L=30)
    lay = layer(w, seed=17)
    W = lay["W"].clone()
    j = 7 * w.K + 4  # table 7, bit 4
    W[:, j] = 0.0
    Wh = W.cpu().numpy()
    Wp = mp.mp_proj_pack(W, w.K, w.L)
    kmean, gcodes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, w.K, w.L)
    gq = mp.mp_encode_queries(lay["q"], Wp, w.K, w.L)
    n, U = lay["n"], w.batch * w.hkv
    kn = lay["Kc"][:, 3].clone()
    mp.mp_append(kn, torch.zeros_like(kn), lay["Kc"], lay["Vc"], n, kmean, Wp, w.K, w.L, gcodes)
    torch.cuda.synchronize()
    g = gcodes.cpu().numpy()
    assert np.all((g[:, 7, :n + 1] >> 4) & 1 == 0)
    assert np.all((gq.cpu().numpy()[..., 7] >> 4) & 1 == 0)
    h = lay["host"]
    km, codes, margin = oracle.build_codes(h["K"].reshape(U, lay["cap"], w.d), n, Wh, w.K, w.L, with_margin=True)
    assert np.all(np.isinf(margin[:, :, j]))
    r = codes[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    assert code_mismatches_outside_band(g[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L), r,
                                        margin.reshape(-1, w.K * w.L))[1] == 0
    qref, qmg = oracle.encode(h["q"].reshape(-1, w.d), Wh, w.K, w.L, with_margin=True)
    assert code_mismatches_outside_band(gq.cpu().numpy().reshape(-1, w.L), qref, qmg)[1] == 0
    aref, amg = oracle.encode(host_f32(kn), Wh, w.K, w.L, mu=km, with_margin=True)
    assert code_mismatches_outside_band(g[:, :, n], aref, amg)[1] == 0


def _inject(w, lay, km, codes, qc):
    U = w.batch * w.hkv
    kmean = torch.from_numpy(km).cuda()
    gcodes = torch.from_numpy(codes).cuda()
    qcodes = torch.from_numpy(qc).cuda()
    assert gcodes.shape == (U, w.L, lay["cap"])
    return kmean, gcodes, qcodes


def _run_decode(w, lay, kmean, gcodes, qcodes, n=None, nsh=0, nst=0, Wp=None, T=2):
    n = lay["n"] if n is None else n
    B, Hq, cap = w.batch, w.hq, lay["cap"]
    out = torch.empty(B, Hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, Hq, dtype=torch.int32, device="cuda")
    mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, Wp, w.hkv, n, w.K, nsh, nst, qcodes_in=qcodes,
                      out=out, lse=lse, idx=idx, count=cnt, T=T)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


def _compare(w, ref, out, lse, idx, cnt, label):
    worst = 0.0
    for b in range(w.batch):
        for h in range(w.hq):
            c = int(cnt[b, h])
            assert c == int(ref["count"][b, h]), (label, b, h, c, int(ref["count"][b, h]))
            assert np.array_equal(idx[b, h, :c], ref["idx"][b][h]), (label, b, h)
            if c == 0:
                assert np.all(out[b, h] == 0) and lse[b, h] == -np.inf
                continue
            err = float(np.max(np.abs(out[b, h] - ref["out"][b, h])))
            worst = max(worst, err)
            assert err <= OUT_TOL, (label, b, h, err)
            assert abs(float(lse[b, h]) - float(ref["lse"][b, h])) <= LSE_TOL, (label, b, h)
    print("[gpu parity] %s: worst |out - oracle| = %.3g, mean |S| = %.1f" % (label, worst, np.mean(ref["count"])))
    return worst


@pytest.mark.parametrize("name", list(CASES))
def test_decode_with_oracle_codes(name):
    """Identical codes (injected from the oracle) give identical sets and outputs within tolerance."""
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    out, lse, idx, cnt = _run_decode(w, lay, kmean, gcodes, qcodes)
    ref = oracle_decode(w, lay, km, codes, qc)
    _compare(w, ref, out, lse, idx, cnt, name)


@pytest.mark.parametrize("name,T", [("llama8b_layer", 1), ("llama8b_layer", 3), ("llama8b_layer", 5),
                                    ("g8_ragged", 1), ("g8_ragged", 3), ("tiny", 4), ("tiny", 75)])
def test_decode_collision_threshold(name, T):
    """Collision threshold T other than the pages' 2 (a key is sampled in at
    least T of L tables, P the binomial tail from T): with the oracle's codes
    injected, sets and counts are equal and outputs within tolerance.  T = 1
    takes the complement of the tail wherever L p > 1, T = L leaves only keys
    that collide everywhere (often none: out = 0, lse = -inf)."""
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    out, lse, idx, cnt = _run_decode(w, lay, kmean, gcodes, qcodes, T=T)
    ref = oracle_decode(w, lay, km, codes, qc, T=T)
    _compare(w, ref, out, lse, idx, cnt, "%s T=%d" % (name, T))
    if T == 1:
        ref2 = oracle_decode(w, lay, km, codes, qc)
        assert np.all(ref["count"] >= ref2["count"])  # T = 1 samples a superset of T = 2


@pytest.mark.parametrize("name", ["llama8b_layer", "g8_ragged"])
def test_decode_static_ranges(name):
    """Forced head/tail ranges (probability 1) on top of the sampled set."""
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    out, lse, idx, cnt = _run_decode(w, lay, kmean, gcodes, qcodes, nsh=4, nst=64)
    ref = oracle_decode(w, lay, km, codes, qc, nsh=4, nst=64)
    _compare(w, ref, out, lse, idx, cnt, name + "+static")


@pytest.mark.parametrize("n", [0, 1, 7, 511, 512, 513, 1023, 1024, 1025, 1535, 2047])
def test_decode_short_and_ragged_n(n):
    """Edge lengths: empty cache, a single key, tails around the 512-key scan tile."""
    w, lay, km, codes, margin, qc = case("llama8b_layer")
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    out, lse, idx, cnt = _run_decode(w, lay, kmean, gcodes, qcodes, n=n)
    ref = oracle_decode(w, lay, km, codes, qc, n=n)
    _compare(w, ref, out, lse, idx, cnt, "n=%d" % n)
    if n == 0:
        assert np.all(cnt == 0) and np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("name,tail,T,static", [
    ("tiny", 1, 2, False), ("tiny", 65, 3, True), ("llama8b_layer", 8, 2, False), ("llama8b_layer", 9, 2, True),
    ("llama8b_layer", 64, 2, False), ("llama8b_layer", 129, 3, False), ("llama8b_layer", 256, 2, True),
    ("llama8b_layer", 257, 2, False), ("g8_ragged", 33, 2, True), ("g8_ragged", 200, 1, False),
    ("g3_k16", 100, 2, False), ("g2_small", 250, 2, True), ("g4_f32", 17, 2, False), ("g7_bf16", 5, 2, False)])
def test_decode_narrow_last_tile(name, tail, T, static):
    """A last tile of at most 256 keys is scanned with several table rows per
    load (a key group's lanes spread over the tables and add their counts):
    tails of 1 to 257 keys, thresholds 1 to 3, forced ranges reaching into
    the tail, every head count."""
    w, lay, km, codes, margin, qc = case(name)
    n = (lay["n"] - tail) // 512 * 512 + tail
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    nsh, nst = (4, 64) if static else (0, 0)
    out, lse, idx, cnt = _run_decode(w, lay, kmean, gcodes, qcodes, n=n, nsh=nsh, nst=nst, T=T)
    ref = oracle_decode(w, lay, km, codes, qc, n=n, nsh=nsh, nst=nst, T=T)
    _compare(w, ref, out, lse, idx, cnt, "%s n=%d T=%d static=%s" % (name, n, T, static))


def _dense_oracle(w, q, K, V, n):
    """The oracle's decode with K = 0 (every key sampled with P = 1), which
    the oracle's pins reduce to Equation 1; codes and query codes are 0."""
    U, cap = K.shape[0], K.shape[1]
    return oracle.decode(q.reshape(w.batch, w.hq, w.d), K.reshape(w.batch, w.hkv, cap, w.d),
                         V.reshape(w.batch, w.hkv, cap, w.d), np.zeros((w.batch, w.hkv, w.L, cap), np.uint16),
                         np.zeros((w.batch, w.hkv, w.d), np.float32), np.zeros((w.d, 0), np.float32), 0, w.L, n,
                         qcodes=np.zeros((w.batch, w.hq, w.L), np.uint16), want_idx=True)


def test_decode_K0_is_exact_attention():
    """K = 0: empty codes collide everywhere, P = 1, the estimate is Equation 1
    (the oracle's decode at K = 0, pinned to Equation 1 on the CPU)."""
    w = variant("tiny", K=0, L=4, n=2000)
    lay = layer(w, seed=77)
    Wp = mp.mp_proj_pack(lay["W"], 0, w.L)
    kmean, gcodes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, 0, w.L)
    idx = torch.full((1, 1, lay["cap"]), -1, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, 1, dtype=torch.int32, device="cuda")
    lse = torch.empty(1, 1, dtype=torch.float32, device="cuda")
    out = mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, Wp, w.hkv, w.n, 0, idx=idx, count=cnt,
                            lse=lse)
    torch.cuda.synchronize()
    h = lay["host"]
    ref = _dense_oracle(w, h["q"], h["K"].reshape(1, lay["cap"], w.d), h["V"].reshape(1, lay["cap"], w.d), w.n)
    assert int(ref["count"][0, 0]) == w.n
    _compare(w, ref, out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), "K=0")
    assert np.array_equal(idx.cpu().numpy()[0, 0, :w.n], np.arange(w.n))  # every key, ascending


def test_dense_layer_step_is_exact_attention():
    """A dense layer of the pages' policy runs as K = 0 (one 0-bit code per
    table, every key sampled with P = 1) through mp_decode_step: append, then
    exact softmax attention over all n + 1 keys for every query head,
    against the oracle's K = 0 decode."""
    w = variant("llama8b_layer", K=0, L=2, n=3000)
    lay = layer(w, seed=91)
    Wp = mp.mp_proj_pack(lay["W"], 0, w.L)
    kmean, gcodes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, 0, w.L)
    n, U = lay["n"], w.batch * w.hkv
    kn = torch.randn(U, w.d, generator=torch.Generator().manual_seed(5)).to(w.torch_dtype).cuda()
    vn = torch.randn(U, w.d, generator=torch.Generator().manual_seed(6)).to(w.torch_dtype).cuda()
    ws = mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda")
    out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
    cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
    idx = torch.full((w.batch, w.hq, lay["cap"]), -1, dtype=torch.int32, device="cuda")
    mp.mp_decode_step(kn, vn, lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, Wp, w.hkv, n, 0, ws, out=out, lse=lse,
                      count=cnt, idx=idx)
    torch.cuda.synchronize()
    assert torch.equal(lay["Kc"][:, n], kn) and torch.equal(lay["Vc"][:, n], vn)
    ref = _dense_oracle(w, lay["host"]["q"], host_f32(lay["Kc"]), host_f32(lay["Vc"]), n + 1)
    assert np.all(ref["count"] == n + 1)
    _compare(w, ref, out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), "dense step")


@pytest.mark.parametrize("name", ["llama8b_layer", "g8_ragged", "g3_k16"])
def test_end_to_end_gpu_codes(name):
    """The whole GPU path with its own means, codes and query codes.  The
    codes meet the per-bit band against the oracle's; then every unit is
    decoded by the oracle on the GPU's own codes and query codes, and the
    sets must be identical and the outputs within the bars."""
    w, lay, km, codes, margin, qc = case(name)
    Wp, kmean, gcodes = gpu_build(w, lay)
    qout = torch.empty(w.batch, w.hq, w.L, dtype=torch.uint16, device="cuda")
    cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
    lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
    idx = torch.full((w.batch, w.hq, lay["cap"]), -1, dtype=torch.int32, device="cuda")
    out = mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, Wp, w.hkv, lay["n"], w.K, qcodes_out=qout,
                            idx=idx, count=cnt, lse=lse)
    torch.cuda.synchronize()
    n = lay["n"]
    g = gcodes.cpu().numpy()
    gq = qout.cpu().numpy()
    gk = kmean.cpu().numpy()
    assert np.array_equal(gk.view(np.uint32), km.view(np.uint32))
    assert code_mismatches_outside_band(g[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L),
                                        codes[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L),
                                        margin.reshape(-1, w.K * w.L))[1] == 0
    ref = oracle_decode(w, lay, gk, g, gq)
    worst = _compare(w, ref, out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
                     name + " end-to-end")
    G = w.group
    same = sum(int(np.array_equal(g[u], codes[u]) and
                   np.array_equal(gq[u // w.hkv, (u % w.hkv) * G:(u % w.hkv + 1) * G],
                                  qc[u // w.hkv, (u % w.hkv) * G:(u % w.hkv + 1) * G]))
               for u in range(w.batch * w.hkv))
    print("[gpu parity] %s end-to-end: all %d units decoded by the oracle on the GPU's codes (worst %.3g); "
          "%d have codes identical to the oracle's" % (name, w.batch * w.hkv, worst, same))


def test_decode_stages_equal_composite_and_are_deterministic():
    w, lay, km, codes, margin, qc = case("g8_ragged")
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    a = _run_decode(w, lay, kmean, gcodes, qcodes)
    b = _run_decode(w, lay, kmean, gcodes, qcodes)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
    ws = mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda")
    mp.mp_decode_sample(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, qcodes, w.hkv, lay["n"], w.K, ws,
                        want_idx=True)
    out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
    idx = torch.full((w.batch, w.hq, lay["cap"]), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
    mp.mp_decode_merge(w.batch, w.hq, w.hkv, lay["n"], lay["cap"], w.L, out, ws, lse=lse, idx=idx, count=cnt)
    torch.cuda.synchronize()
    for x, y in zip(a, (out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy())):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("name", ["g8_ragged", "llama8b_layer", "tiny", "g6_bf16", "g4_f32", "mha_b3", "g2_small",
                                  "g3_k16", "mha_64rec", "g4_65rec"])
def test_merge_without_index_lists_equals_merge_with_them(name):
    """The merge runs as a wider kernel when no index lists are asked for
    (up to four heads per KV head); both fold the per-tile partial records in
    the same order, so the output, log-sum-exp and counts agree bit for bit."""
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    a = _run_decode(w, lay, kmean, gcodes, qcodes)
    out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
    cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
    mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, None, w.hkv, lay["n"], w.K, 0, 0,
                      qcodes_in=qcodes, out=out, lse=lse, count=cnt)
    torch.cuda.synchronize()
    for x, y in zip((a[0], a[1], a[3]), (out.cpu().numpy(), lse.cpu().numpy(), cnt.cpu().numpy())):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("name", ["llama8b_layer", "tiny"])
def test_append_then_decode(name):
    """Append a decoded token per unit (frozen mean): cache rows copied exactly,
    its codes equal the oracle's encoding (up to the band), and a decode over
    n + 1 keys matches the oracle."""
    w = CASES[name]
    lay = layer(w, seed=99)
    Wp, kmean, gcodes = gpu_build(w, lay)
    U, n, cap = w.batch * w.hkv, lay["n"], lay["cap"]
    kn = torch.stack([synth.step_kv(99, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=1)[0] for u in range(U)])
    vn = torch.stack([synth.step_kv(99, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=1)[1] for u in range(U)])
    kn, vn = kn.cuda(), vn.cuda()
    mp.mp_append(kn, vn, lay["Kc"], lay["Vc"], n, kmean, Wp, w.K, w.L, gcodes)
    torch.cuda.synchronize()
    assert torch.equal(lay["Kc"][:, n], kn) and torch.equal(lay["Vc"][:, n], vn)
    km = kmean.cpu().numpy()
    h = lay["host"]
    knh = host_f32(kn)
    for u in range(U):
        ref, mg = oracle.encode(knh[u], h["W"], w.K, w.L, mu=km[u], with_margin=True)
        got = gcodes[u, :, n].cpu().numpy()[None]
        assert code_mismatches_outside_band(got, ref, mg)[1] == 0
    # decode over n + 1 keys with the oracle's codes for the whole store
    keys = host_f32(lay["Kc"]).reshape(w.batch, w.hkv, cap, w.d)
    vals = host_f32(lay["Vc"]).reshape(w.batch, w.hkv, cap, w.d)
    codes_o = np.zeros((U, w.L, cap), np.uint16)
    for u in range(U):
        codes_o[u][:, :n + 1] = oracle.encode(keys.reshape(U, cap, w.d)[u, :n + 1], h["W"], w.K, w.L, mu=km[u]).T
    qc = oracle.encode(h["q"].reshape(-1, w.d), h["W"], w.K, w.L).reshape(w.batch, w.hq, w.L)
    lay2 = dict(lay)
    lay2["host"] = dict(h, K=keys, V=vals)
    lay2["n"] = n + 1
    kmean_t, gcodes_t, qcodes = _inject(w, lay2, km, codes_o, qc)
    out, lse, idx, cnt = _run_decode(w, lay2, kmean_t, gcodes_t, qcodes)
    ref = oracle_decode(w, lay2, km, codes_o, qc)
    _compare(w, ref, out, lse, idx, cnt, name + "+append")


@pytest.mark.parametrize("name", ["llama8b_layer", "g8_ragged", "tiny"])
def test_decode_step_equals_separate_calls(name):
    """mp_decode_step (append + query encode in one launch, sample, merge)
    gives bit-identical caches, codes and outputs to mp_append +
    mp_encode_queries + mp_decode_attn."""
    w = CASES[name]
    outs = []
    for fused in (False, True):
        lay = layer(w, seed=321)
        Wp, kmean, gcodes = gpu_build(w, lay)
        U, n, cap = w.batch * w.hkv, lay["n"], lay["cap"]
        kn = torch.stack([synth.step_kv(321, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=1)[0]
                          for u in range(U)]).cuda()
        vn = torch.stack([synth.step_kv(321, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=1)[1]
                          for u in range(U)]).cuda()
        out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
        lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
        cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
        idx = torch.full((w.batch, w.hq, cap), -3, dtype=torch.int32, device="cuda")
        ws = mp.decode_workspace(w.batch, w.hq, w.hkv, cap, w.L, "cuda")
        if fused:
            ev = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for e in ev:
                e.record()
            mp.mp_decode_step(kn, vn, lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, Wp, w.hkv, n, w.K, ws, out=out,
                              lse=lse, idx=idx, count=cnt, n_static_head=2, sample_events=ev)
            torch.cuda.synchronize()
            assert ev[0].elapsed_time(ev[1]) >= 0.0
        else:
            mp.mp_append(kn, vn, lay["Kc"], lay["Vc"], n, kmean, Wp, w.K, w.L, gcodes)
            mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, Wp, w.hkv, n + 1, w.K, 2, 0, out=out,
                              lse=lse, idx=idx, count=cnt, ws=ws)
            torch.cuda.synchronize()
        outs.append([t.detach().cpu().contiguous().view(torch.uint8).numpy()
                     for t in (lay["Kc"], lay["Vc"], gcodes, out, lse, idx, cnt)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_two_streams_with_own_workspaces_match_sequential():
    """The library keeps no state: two decodes enqueued on two streams at
    once, each with its own workspace, give the bytes of running them one
    after the other."""
    runs = []
    for name in ("llama8b_layer", "g8_ragged"):
        w, lay, km, codes, margin, qc = case(name)
        kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
        runs.append((w, lay, kmean, gcodes, qcodes))

    def launch(w, lay, kmean, gcodes, qcodes, stream):
        out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
        cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
        idx = torch.full((w.batch, w.hq, lay["cap"]), -1, dtype=torch.int32, device="cuda")
        ws = mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda")
        torch.cuda.synchronize()
        mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, None, w.hkv, lay["n"], w.K,
                          qcodes_in=qcodes, out=out, idx=idx, count=cnt, ws=ws, stream=stream)
        return out, idx, cnt, ws  # ws stays referenced until the streams are synchronised

    seq = []
    for r in runs:
        seq.append(launch(*r, stream=torch.cuda.current_stream()))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    par = [launch(*r, stream=st) for r, st in zip(runs, streams)]
    torch.cuda.synchronize()
    for a, b in zip(seq, par):
        for x, y in zip(a[:3], b[:3]):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
