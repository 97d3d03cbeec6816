"""Checkpoint and resume: the decode state is plain device memory owned by the
caller -- key/value caches, the code store, key means, the bit-plane index
and the bucketed tables -- so saving it with torch and loading it back gives a
decode that continues bit for bit as the uninterrupted one."""
import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
import synth
from tests.common import layer, variant

pytestmark = pytest.mark.gpu


def _steps(w, state, Wp, first, count, seed):
    U, G = w.batch * w.hkv, w.group
    outs = []
    for s in range(first, first + count):
        kn = torch.stack([synth.step_kv(seed, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=s)[0]
                          for u in range(U)]).cuda()
        vn = torch.stack([synth.step_kv(seed, 0, u // w.hkv, u % w.hkv, w.d, w.torch_dtype, step=s)[1]
                          for u in range(U)]).cuda()
        q = torch.stack([synth.unit_queries(seed, 0, u // w.hkv, u % w.hkv, G, w.d, w.torch_dtype, step=s)
                         for u in range(U)]).reshape(w.batch, w.hq, w.d).cuda()
        out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
        lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
        idx = torch.full((w.batch, w.hq, state["Kc"].shape[1]), -1, dtype=torch.int32, device="cuda")
        cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
        n = int(state["n"])
        mp.mp_decode_step(kn, vn, q, state["Kc"], state["Vc"], state["codes"], state["kmean"], Wp, w.hkv, n, w.K,
                          state["ws"], out=out, lse=lse, idx=idx, count=cnt, buckets=state["buckets"],
                          n_buckets=int(state["n_index"]) if state["buckets"] is not None else 0,
                          planes=state["planes"], n_planes=int(state["n_index"]) if state["planes"] is not None else 0)
        state["n"] = n + 1
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().view(np.uint8).copy() for t in (out, lse, idx, cnt)])
    return outs


@pytest.mark.parametrize("index", ["buckets", "planes"])
def test_saved_and_reloaded_state_decodes_identically(tmp_path, index):
    w = variant("llama8b_layer", n=3000, steps=40)
    seed = 909
    lay = layer(w, seed=seed)
    Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
    kmean, codes = mp.mp_build_codes(lay["Kc"], lay["n"], Wp, w.K, w.L)
    n_index = (lay["n"] // 512) * 512
    state = dict(Kc=lay["Kc"], Vc=lay["Vc"], codes=codes, kmean=kmean, n=lay["n"], n_index=n_index,
                 buckets=mp.mp_build_buckets(codes, w.K, n_index) if index == "buckets" else None,
                 planes=mp.mp_build_planes(codes, w.K, n_index) if index == "planes" else None,
                 ws=mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda"))
    _steps(w, state, Wp, 1, 5, seed)
    path = tmp_path / "decode_state.pt"
    torch.save({k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in state.items() if k != "ws"}, path)
    a = _steps(w, state, Wp, 6, 10, seed)
    loaded = torch.load(path, weights_only=True)
    resumed = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in loaded.items()}
    resumed["ws"] = mp.decode_workspace(w.batch, w.hq, w.hkv, lay["cap"], w.L, "cuda")
    assert resumed["n"] == lay["n"] + 5
    b = _steps(w, resumed, Wp, 6, 10, seed)
    for s, (x, y) in enumerate(zip(a, b)):
        for t, (p, r) in enumerate(zip(x, y)):
            assert np.array_equal(p, r), (s, t)
    for k in ("Kc", "Vc", "codes"):
        assert torch.equal(state[k].view(torch.uint8), resumed[k].view(torch.uint8)), k
