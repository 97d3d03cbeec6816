"""GPU check of mp_decode_step_static, the decode step that allocates
nothing (its workspace is the library's static scratch): called through the C
ABI, it must give the bytes mp_decode_step gives with a caller workspace --
appended cache rows and codes, outputs, lse, index lists and counts -- on two
calls in a row, the second with a smaller input than the first, so the second
reuses scratch the first left behind."""
import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
import synth
from tests.common import layer, variant

pytestmark = pytest.mark.gpu

CASES = [
    # Llama-3.1-8B-shaped layer (32 q / 8 KV heads, K=8, L=75), 16K keys, forced sink/local keys
    ("llama8b_layer", variant("llama8b_layer"), 4, 64),
    # smaller: 8 query heads per KV head, (10, 240), ragged n
    ("g8_small", variant("codellama34b_b4", layers=1, batch=1, n=3000, steps=0), 0, 0),
]


def _run(w, nsh, nst, static):
    lay = layer(w, seed=606)
    Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
    kmean, codes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, w.K, w.L)
    U, n, cap = w.batch * w.hkv, lay["n"], lay["cap"]
    kn = torch.stack([synth.step_kv(606, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=1)[0]
                      for u in range(U)]).cuda()
    vn = torch.stack([synth.step_kv(606, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=1)[1]
                      for u in range(U)]).cuda()
    out = torch.full((w.batch, w.hq, w.d), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, w.hq), 7.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((w.batch, w.hq), -1, dtype=torch.int32, device="cuda")
    idx = torch.full((w.batch, w.hq, cap), -3, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    if static:
        mp.mp_decode_step_static(kn, vn, lay["q"], lay["Kc"], lay["Vc"], codes, kmean, Wp, w.hkv, n, w.K, out,
                                 lse=lse, idx=idx, count=cnt, n_static_head=nsh, n_static_tail=nst)
    else:
        ws = mp.decode_workspace(w.batch, w.hq, w.hkv, cap, w.L, "cuda")
        mp.mp_decode_step(kn, vn, lay["q"], lay["Kc"], lay["Vc"], codes, kmean, Wp, w.hkv, n, w.K, ws, out=out,
                          lse=lse, idx=idx, count=cnt, n_static_head=nsh, n_static_tail=nst)
    torch.cuda.synchronize()
    return [t.detach().cpu().contiguous().view(torch.uint8).numpy()
            for t in (lay["Kc"], lay["Vc"], codes, out, lse, idx, cnt)], cnt.cpu().numpy()


def test_static_step_equals_workspace_step_twice():
    sizes = []
    for name, w, nsh, nst in CASES:
        print("[no-alloc] case %s: B=%d Hq=%d Hkv=%d n=%d K=%d L=%d" % (name, w.batch, w.hq, w.hkv, w.n, w.K, w.L),
              flush=True)
        need = mp.mp_decode_ws_bytes(w.batch, w.hq, w.hkv, w.cap, w.L)
        assert 0 < need <= mp.MP_STATIC_SCRATCH_BYTES
        sizes.append(need)
        ref, cnt = _run(w, nsh, nst, static=False)
        got, _ = _run(w, nsh, nst, static=True)
        for a, b, what in zip(ref, got, ("Kc", "Vc", "codes", "out", "lse", "idx", "count")):
            assert np.array_equal(a, b), (name, what)
        assert np.all(cnt > 0)
    assert sizes[1] < sizes[0]  # the second call works on a smaller part of the scratch
