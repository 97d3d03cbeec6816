"""GPU parity of the lift of Section 4.2, Equation 8 (an option the pages do
not use): the lifted code-store build, appends and decode, through the C ABI,
against the oracle's lifted functions (which the CPU pins check against an
independent brute force, Monte-Carlo inclusion frequencies and the
monotonicity in the inner product).

Bars as for the unlifted path: key means bitwise; lift radii bitwise (fp64
sums of exact bf16 squares, one rounding); code bits equal except where
their own projection is inside the rounding band; with the oracle's codes
injected, sampled sets exact and outputs within 2e-3 (lse 1e-3).
"""
import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
import oracle
from tests.common import code_mismatches_outside_band, host_f32, layer, variant
from tests.test_gpu_parity import _compare

pytestmark = pytest.mark.gpu

CASES = {
    "llama8b_k8": variant("llama8b_layer", n=6000),                              # 4 tables per tile
    "k10_l150_ragged": variant("llama8b_96k", layers=1, n=5000, steps=1),        # 3 tables per tile
    "k4_small": variant("llama8b_layer", hq=4, hkv=2, n=777, K=4, L=33),         # 8 tables per tile
    "k16_g3": variant("llama8b_layer", hq=6, hkv=2, n=1500, K=16, L=20),         # 2 tables per tile
    "tiny_f32": variant("tiny", n=3000),
}

_cache = {}


def lifted_case(name):
    if name not in _cache:
        w = CASES[name]
        lay = layer(w, seed=515)
        g = torch.Generator().manual_seed(516)
        W = torch.randn(w.d + 1, w.K * w.L, generator=g)  # the extra row of the lift
        U = w.batch * w.hkv
        keys = lay["host"]["K"].reshape(U, lay["cap"], w.d)
        km, rl, codes, margin = oracle.build_codes_lifted(keys, lay["n"], W.numpy(), w.K, w.L, with_margin=True)
        qc = oracle.encode_lifted(lay["host"]["q"].reshape(-1, w.d), W.numpy(), w.K, w.L, lift=False)
        _cache[name] = (w, lay, W, km, rl, codes, margin, qc.reshape(w.batch, w.hq, w.L))
        print("[gpu lift] case %s: n=%d K=%d L=%d G=%d %s; radii %s" % (name, w.n, w.K, w.L, w.group, w.dtype,
                                                                        np.round(rl, 3)), flush=True)
    return _cache[name]


@pytest.mark.parametrize("name", list(CASES))
def test_lifted_build(name):
    w, lay, W, km, rl, codes, margin, qc = lifted_case(name)
    Wp = mp.mp_proj_pack_lift(W.cuda(), w.K, w.L)
    kmean, rlift, gcodes = mp.mp_build_codes_lift(lay["Kc"], lay["n"], Wp, w.K, w.L)
    torch.cuda.synchronize()
    assert np.array_equal(kmean.cpu().numpy().view(np.uint32), km.view(np.uint32))
    assert np.array_equal(rlift.cpu().numpy().view(np.uint32), rl.view(np.uint32)), (rlift.cpu().numpy(), rl)
    n = lay["n"]
    g = gcodes.cpu().numpy()[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    r = codes[:, :, :n].transpose(0, 2, 1).reshape(-1, w.L)
    ndiff, nbad = code_mismatches_outside_band(g, r, margin.reshape(-1, w.K * w.L))
    print("[gpu lift] %s: %d of %d code bits differ, all inside the band" % (name, ndiff, g.size * w.K))
    assert nbad == 0
    assert int(gcodes[:, :, n:].cpu().numpy().astype(np.int64).sum()) == 0
    # queries: the extra coordinate is 0, so the lifted packing encodes them as the first d rows do
    gq = mp.mp_encode_queries(lay["q"], Wp, w.K, w.L).cpu().numpy()
    Wp0 = mp.mp_proj_pack(W[:w.d].contiguous().cuda(), w.K, w.L)
    gq0 = mp.mp_encode_queries(lay["q"], Wp0, w.K, w.L).cpu().numpy()
    assert np.array_equal(gq, gq0)
    qref, qmg = oracle.encode_lifted(lay["host"]["q"].reshape(-1, w.d), W.numpy(), w.K, w.L, lift=False,
                                     with_margin=True)
    assert code_mismatches_outside_band(gq.reshape(-1, w.L), qref, qmg)[1] == 0


@pytest.mark.parametrize("name", ["llama8b_k8", "k10_l150_ragged", "tiny_f32"])
def test_lifted_append(name):
    """An appended key is lifted with the frozen mean and radius; one longer
    than the radius gets the extra coordinate 0."""
    w, lay, W, km, rl, codes, margin, qc = lifted_case(name)
    Wp = mp.mp_proj_pack_lift(W.cuda(), w.K, w.L)
    Kc, Vc = lay["Kc"].clone(), lay["Vc"].clone()
    kmean, rlift, gcodes = mp.mp_build_codes_lift(Kc, lay["n"], Wp, w.K, w.L)
    U, n = w.batch * w.hkv, lay["n"]
    g = torch.Generator().manual_seed(517)
    kn = (torch.randn(U, w.d, generator=g) * 2.0).to(w.torch_dtype)
    kn[0] = kn[0] * 50.0  # far outside the radius
    kn = kn.cuda()
    vn = torch.randn(U, w.d, generator=g).to(w.torch_dtype).cuda()
    mp.mp_append_lift(kn, vn, Kc, Vc, n, kmean, rlift, Wp, w.K, w.L, gcodes)
    torch.cuda.synchronize()
    assert torch.equal(Kc[:, n], kn) and torch.equal(Vc[:, n], vn)
    got = gcodes.cpu().numpy()[:, :, n]
    knh = host_f32(kn)
    for u in range(U):
        ref, mg = oracle.encode_lifted(knh[u], W.numpy(), w.K, w.L, mu=km[u], R=rl[u], with_margin=True)
        assert code_mismatches_outside_band(got[u][None], ref, mg)[1] == 0, u


@pytest.mark.parametrize("name,nsh,nst,index", [("llama8b_k8", 0, 0, None), ("llama8b_k8", 4, 64, "buckets"),
                                                ("k10_l150_ragged", 0, 0, "planes"), ("k4_small", 0, 0, None),
                                                ("k16_g3", 0, 0, None), ("tiny_f32", 0, 0, None)])
def test_lifted_decode(name, nsh, nst, index):
    """With the oracle's lifted codes and radii injected: sets exact and
    outputs within the bars, also through the bucketed tables or the planes."""
    w, lay, W, km, rl, codes, margin, qc = lifted_case(name)
    kmean = torch.from_numpy(km).cuda()
    rlift = torch.from_numpy(rl).cuda()
    gcodes = torch.from_numpy(codes).cuda()
    qcodes = torch.from_numpy(qc).cuda()
    B, Hq, cap, n = w.batch, w.hq, lay["cap"], lay["n"]
    out = torch.empty(B, Hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, Hq, dtype=torch.int32, device="cuda")
    kw = {}
    n_idx = (n // 512) * 512
    if index == "buckets":
        kw = dict(buckets=mp.mp_build_buckets(gcodes, w.K, n_idx), n_buckets=n_idx)
    elif index == "planes":
        kw = dict(planes=mp.mp_build_planes(gcodes, w.K, n_idx), n_planes=n_idx)
    mp.mp_decode_attn_lift(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, rlift, None, w.hkv, n, w.K,
                           qcodes_in=qcodes, out=out, lse=lse, idx=idx, count=cnt, n_static_head=nsh,
                           n_static_tail=nst, **kw)
    torch.cuda.synchronize()
    h = lay["host"]
    ref = oracle.decode(h["q"], h["K"], h["V"], codes.reshape(w.batch, w.hkv, w.L, cap),
                        km.reshape(w.batch, w.hkv, w.d), W.numpy(), w.K, w.L, n, qcodes=qc, n_static_head=nsh,
                        n_static_tail=nst, want_idx=True, rlift=rl.reshape(w.batch, w.hkv))
    _compare(w, ref, out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(),
             "%s lifted %s" % (name, index))
    # the lift changes the probabilities: the unlifted oracle gives other outputs on the same sets
    # (K = 16 leaves the lifted sets empty: nothing to compare there)
    if int(ref["count"].sum()) == 0:
        return
    ref0 = oracle.decode(h["q"], h["K"], h["V"], codes.reshape(w.batch, w.hkv, w.L, cap),
                         km.reshape(w.batch, w.hkv, w.d), W.numpy(), w.K, w.L, n, qcodes=qc, n_static_head=nsh,
                         n_static_tail=nst)
    assert np.max(np.abs(ref0["out"] - ref["out"])) > 1e-3
