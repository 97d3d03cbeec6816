"""GPU parity of the bit-plane index of the code store (mp_build_planes) and
of the decode that scans it.

The index holds the same codes as the 16-bit store, K bits per key and table,
so: (1) unpacking it on the host gives back the oracle's codes bit for bit;
(2) a decode that scans it for the tiles below n_planes (and the 16-bit codes
above) gives the same sampled index lists, counts and outputs as the decode
from the codes alone (bit for bit: the lists are the same, so is the
arithmetic), and therefore meets the oracle's bars.
"""
import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
from tests.common import oracle_decode
from tests.test_gpu_parity import CASES, _compare, _inject, case, gpu_build

pytestmark = pytest.mark.gpu

PREFILL = 0x5A5A5A5A


def planes_to_codes(planes, K, L):
    """Host unpacking: int32 [U][T][K][L][16] -> uint32 codes [U][L][T*512]."""
    p = planes.view(np.uint32)
    U, T = p.shape[:2]
    codes = np.zeros((U, L, T * 512), dtype=np.uint32)
    e = np.arange(32, dtype=np.uint32)
    for b in range(K):
        bits = ((p[:, :, b, :, :, None] >> e) & 1).astype(np.uint32)  # [U][T][L][16][32]: key 32 j + e
        codes |= bits.transpose(0, 2, 1, 3, 4).reshape(U, L, T * 512) << np.uint32(b)
    return codes


def _planes(gcodes, K, n1, n0=0, planes=None):
    U, L, cap = gcodes.shape
    if planes is None:
        planes = torch.full((U, (cap + 511) // 512, K, L, 16), PREFILL, dtype=torch.int32, device="cuda")
    mp.mp_build_planes(gcodes, K, n1, n0=n0, planes=planes)
    return planes


@pytest.mark.parametrize("name", list(CASES))
def test_planes_are_the_codes(name):
    """Unpacked on the host, the index equals the codes for every whole tile;
    tiles past n1 are not written; building in two parts gives the same words."""
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    n1 = (lay["n"] // 512) * 512
    assert n1 >= 512
    planes = _planes(gcodes, w.K, n1)
    torch.cuda.synchronize()
    hp = planes.cpu().numpy()
    back = planes_to_codes(hp[:, : n1 // 512], w.K, w.L)
    assert np.array_equal(back, codes[:, :, :n1].astype(np.uint32)), name
    assert np.all(hp[:, n1 // 512:].view(np.uint32) == PREFILL)
    two = _planes(gcodes, w.K, 512)
    _planes(gcodes, w.K, n1, n0=512, planes=two)
    torch.cuda.synchronize()
    assert torch.equal(two, planes)
    print("[gpu planes] %s: %d tiles per unit unpack to the codes" % (name, n1 // 512))


def _decode(w, lay, kmean, gcodes, qcodes, planes=None, n_planes=0, nsh=0, nst=0, T=2):
    B, Hq, cap = w.batch, w.hq, lay["cap"]
    out = torch.empty(B, Hq, w.d, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    idx = torch.full((B, Hq, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, Hq, dtype=torch.int32, device="cuda")
    mp.mp_decode_attn(lay["q"], lay["Kc"], lay["Vc"], gcodes, kmean, None, w.hkv, lay["n"], w.K, nsh, nst,
                      qcodes_in=qcodes, out=out, lse=lse, idx=idx, count=cnt, T=T, planes=planes, n_planes=n_planes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("name,nsh,nst,T,part", [
    ("llama8b_layer", 0, 0, 2, 1.0),
    ("llama8b_layer", 4, 64, 2, 1.0),   # forced ranges inside plane tiles
    ("llama8b_layer", 0, 0, 2, 0.5),    # half of the whole tiles from the index, the rest from the codes
    ("llama8b_layer", 0, 0, 3, 1.0),    # other thresholds scan the codes
    ("g8_ragged", 0, 0, 2, 1.0),
    ("mha_b3", 0, 0, 2, 1.0),
    ("g2_small", 0, 0, 2, 1.0),
    ("g3_k16", 0, 0, 2, 1.0),
    ("tiny", 0, 0, 2, 1.0),
    ("l512_g2", 0, 0, 2, 1.0),
    ("l512_g8", 0, 0, 2, 1.0),
])
def test_decode_scans_planes(name, nsh, nst, T, part):
    w, lay, km, codes, margin, qc = case(name)
    kmean, gcodes, qcodes = _inject(w, lay, km, codes, qc)
    n1 = (lay["n"] // 512) * 512
    planes = _planes(gcodes, w.K, n1)
    n_planes = max(512, int(n1 * part) // 512 * 512)
    got = _decode(w, lay, kmean, gcodes, qcodes, planes, n_planes, nsh, nst, T)
    base = _decode(w, lay, kmean, gcodes, qcodes, None, 0, nsh, nst, T)
    for a, b, what in zip(got, base, ("out", "lse", "idx", "count")):
        assert np.array_equal(a, b), (name, what)
    ref = oracle_decode(w, lay, km, codes, qc, nsh=nsh, nst=nst, T=T)
    _compare(w, ref, *got, "%s planes<%d nsh=%d nst=%d T=%d" % (name, n_planes, nsh, nst, T))


def test_decode_step_with_planes():
    """Append + decode over GPU-built codes: the appended key lies past the
    index (n_planes <= n) and is found through its 16-bit codes."""
    w, lay, km, codes, margin, qc = case("llama8b_layer")
    Wp, kmean, gcodes = gpu_build(w, lay)
    n = lay["n"]
    assert lay["cap"] > n
    n1 = (n // 512) * 512
    planes = _planes(gcodes, w.K, n1)
    U = w.batch * w.hkv
    g = torch.Generator(device="cpu").manual_seed(5)
    # the new key, centred by the frozen mean, is the query of its group's
    # first head (up to bf16 rounding): it collides in nearly every table
    kn = (kmean + lay["q"][:, :: w.hq // w.hkv].reshape(U, w.d).float()).to(lay["Kc"].dtype)
    vn = torch.randn(U, w.d, generator=g).to(lay["Kc"].dtype).cuda()
    outs = []
    for use in (True, False):
        Kc, Vc, cd = lay["Kc"].clone(), lay["Vc"].clone(), gcodes.clone()
        ws = mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda")
        cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
        idx = torch.full((w.batch, w.hq, lay["cap"]), -7, dtype=torch.int32, device="cuda")
        out = mp.mp_decode_step(kn, vn, lay["q"], Kc, Vc, cd, kmean, Wp, w.hkv, n, w.K, ws, idx=idx, count=cnt,
                                planes=planes if use else None, n_planes=n1 if use else 0)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    cnt, idx = outs[0][2], outs[0][1]
    assert any(n in idx[0, h, : cnt[0, h]] for h in range(w.hq)), "appended key never sampled"
