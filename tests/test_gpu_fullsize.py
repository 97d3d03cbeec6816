"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one ``mp_decode_step`` per layer: append, query encode,
sample, merge).

The inputs are generated on the device (seeded, by ``synth``); the oracle
recomputes a sample of units one by one from copies of those inputs:

* key means bitwise, codes up to the rounding band (the oracle's margins);
* the appended key's codes, and the query codes, up to the band;
* for every sampled unit whose appended and query codes equal the oracle's,
  the step's own outputs, lse and counts (out within 2e-3, lse within 1e-3,
  counts exact);
* for every sampled unit, a decode with the oracle's query codes injected:
  index lists exact, outputs within 2e-3.

The code store of the sampled units holds the oracle's codes (injected after
the build was compared), so both sides decode the same sets.
"""
import numpy as np
import pytest
import torch

import lsh_sampled_sparse_centered_amd as mp
import oracle
import synth
from tests.common import code_mismatches_outside_band, host_f32

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-3
LSE_TOL = 1e-3
SEED = 2024


def _i16(a: np.ndarray) -> torch.Tensor:
    """uint16 codes as an int16 device tensor (copies and slices of uint16
    tensors go through their int16 view)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def _say(msg):
    print("[gpu fullsize] " + msg, flush=True)


class Store:
    """One layer on the device plus the oracle's copy of the sampled units."""

    def __init__(self, w, layer_idx, units):
        self.w, self.layer_idx, self.units = w, layer_idx, list(units)
        _say("%s layer %d: B=%d Hq=%d Hkv=%d n=%d K=%d L=%d, sampled units %s" %
             (w.name, layer_idx, w.batch, w.hq, w.hkv, w.n, w.K, w.L, self.units))
        lay = synth.layer_inputs(w, SEED, layer_idx, device="cuda")
        self.U, self.cap, self.n = w.batch * w.hkv, lay["cap"], lay["n"]
        self.Kc = lay["K"].view(self.U, self.cap, w.d)
        self.Vc = lay["V"].view(self.U, self.cap, w.d)
        self.q0 = lay["q"]
        self.Wh = lay["W"].cpu().numpy().copy()
        self.Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
        self.kmean, self.codes = mp.mp_build_codes(self.Kc, self.n, self.Wp, w.K, w.L)
        self.c16 = self.codes.view(torch.int16)
        torch.cuda.synchronize()
        # host copies of the sampled units (rows >= n are zero, as on the device)
        self.hK = np.stack([host_f32(self.Kc[u]) for u in self.units])
        self.hV = np.stack([host_f32(self.Vc[u]) for u in self.units])

    def check_build_and_inject(self):
        w = self.w
        km, codes, margin = oracle.build_codes(self.hK, self.n, self.Wh, w.K, w.L, with_margin=True)
        gk = self.kmean[self.units].cpu().numpy()
        assert np.array_equal(gk.view(np.uint32), km.view(np.uint32)), "key means differ"
        g = np.stack([_u16(self.c16[u]) for u in self.units])
        ndiff, nbad = code_mismatches_outside_band(g[:, :, :self.n].transpose(0, 2, 1).reshape(-1, w.L),
                                                   codes[:, :, :self.n].transpose(0, 2, 1).reshape(-1, w.L),
                                                   margin.reshape(-1, w.L))
        _say("build: %d of %d sampled codes differ, %d outside the band" % (ndiff, g[:, :, :self.n].size, nbad))
        assert nbad == 0
        self.km_o, self.codes_o = km, codes
        for i, u in enumerate(self.units):
            self.c16[u].copy_(_i16(codes[i]))

    def step_inputs(self, s):
        """The key/value appended and the queries of decode step s (1-based), on the device."""
        w = self.w
        kn = torch.empty(self.U, w.d, dtype=w.torch_dtype, device="cuda")
        vn = torch.empty_like(kn)
        q = torch.empty(w.batch, w.hq, w.d, dtype=w.torch_dtype, device="cuda")
        G = w.group
        for b in range(w.batch):
            for h in range(w.hkv):
                k1, v1 = synth.step_kv(SEED, self.layer_idx, b, h, w.d, w.torch_dtype, s, device="cuda")
                kn[b * w.hkv + h] = k1
                vn[b * w.hkv + h] = v1
                q[b, h * G:(h + 1) * G] = synth.unit_queries(SEED, self.layer_idx, b, h, G, w.d, w.torch_dtype,
                                                             device="cuda", step=s)
        return kn, vn, q

    def run_step(self, s, ws, check):
        """One decode step through mp_decode_step at row n; checks the sampled units when ``check``."""
        w, G = self.w, self.w.group
        n = self.n
        kn, vn, q = self.step_inputs(s)
        out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
        lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
        cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
        mp.mp_decode_step(kn, vn, q, self.Kc, self.Vc, self.codes, self.kmean, self.Wp, w.hkv, n, w.K, ws, out=out,
                          lse=lse, count=cnt)
        torch.cuda.synchronize()
        # the oracle's side of the append: raw rows and codes with the frozen mean
        same_append = []
        for i, u in enumerate(self.units):
            kh, vh = host_f32(kn[u]), host_f32(vn[u])
            assert torch.equal(self.Kc[u, n], kn[u]) and torch.equal(self.Vc[u, n], vn[u])
            self.hK[i, n], self.hV[i, n] = kh, vh
            ref, mg = oracle.encode(kh[None], self.Wh, w.K, w.L, mu=self.km_o[i], with_margin=True)
            got = _u16(self.c16[u, :, n])[None]
            ndiff, nbad = code_mismatches_outside_band(got, ref, mg)
            assert nbad == 0, (s, u)
            same_append.append(ndiff == 0)
            self.codes_o[i][:, n] = ref[0]
            if ndiff:  # keep both stores identical for later steps
                self.c16[u, :, n] = _i16(ref[0])
        self.n = n + 1
        if not check:
            return
        qh = host_f32(q)
        gq = _u16(mp.mp_encode_queries(q, self.Wp, w.K, w.L).view(torch.int16))
        o_out, o_lse, o_cnt = out.cpu().numpy(), lse.cpu().numpy(), cnt.cpu().numpy()
        qc16 = _i16(gq)
        refs = []
        direct = 0
        for i, u in enumerate(self.units):
            b, h = divmod(u, w.hkv)
            qu = qh[b, h * G:(h + 1) * G]
            qref, qmg = oracle.encode(qu, self.Wh, w.K, w.L, with_margin=True)
            ndiff, nbad = code_mismatches_outside_band(gq[b, h * G:(h + 1) * G], qref, qmg)
            assert nbad == 0, (s, u)
            qc16[b, h * G:(h + 1) * G] = _i16(qref)
            ref = oracle.decode(qu[None], self.hK[i][None, None], self.hV[i][None, None], self.codes_o[i][None, None],
                                self.km_o[i][None, None], self.Wh, w.K, w.L, self.n, qcodes=qref[None],
                                want_idx=True)
            refs.append((b, h, ref))
            if ndiff == 0 and same_append[i]:
                direct += 1
                for g in range(G):
                    hh = h * G + g
                    assert int(o_cnt[b, hh]) == int(ref["count"][0, g]), (s, u, g)
                    if ref["count"][0, g] == 0:
                        continue
                    assert np.max(np.abs(o_out[b, hh] - ref["out"][0, g])) <= OUT_TOL, (s, u, g)
                    assert abs(float(o_lse[b, hh]) - float(ref["lse"][0, g])) <= LSE_TOL, (s, u, g)
        # the same decode with the oracle's query codes, index lists included
        out2 = torch.empty_like(out)
        cnt2 = torch.empty_like(cnt)
        idx = torch.full((w.batch, w.hq, self.cap), -1, dtype=torch.int32, device="cuda")
        mp.mp_decode_attn(q, self.Kc, self.Vc, self.codes, self.kmean, None, w.hkv, self.n, w.K,
                          qcodes_in=qc16.view(torch.uint16), out=out2, idx=idx, count=cnt2, ws=ws)
        torch.cuda.synchronize()
        worst, sizes = 0.0, []
        for b, h, ref in refs:
            for g in range(G):
                hh = h * G + g
                c = int(cnt2[b, hh])
                assert c == int(ref["count"][0, g]), (s, b, hh)
                assert np.array_equal(idx[b, hh, :c].cpu().numpy(), ref["idx"][0][g]), (s, b, hh)
                sizes.append(c)
                if c:
                    err = float(np.max(np.abs(out2[b, hh].cpu().numpy() - ref["out"][0, g])))
                    worst = max(worst, err)
                    assert err <= OUT_TOL, (s, b, hh, err)
        _say("step %d (n=%d): %d/%d units checked on the step's own outputs; sets exact; worst |out - oracle| %.3g; "
             "mean |S| %.0f" % (s, self.n, direct, len(self.units), worst, float(np.mean(sizes))))


def _run(w, layer_idx, units, check_steps):
    st = Store(w, layer_idx, units)
    st.check_build_and_inject()
    ws = mp.decode_workspace(w.batch, w.hq, w.hkv, st.cap, w.L, "cuda")
    for s in range(1, max(check_steps) + 1):
        st.run_step(s, ws, s in check_steps)


def test_llama8b_96k_layer():
    """Llama-3.1-8B shape at 96K context: one layer (32 q / 8 KV heads, K=10, L=150), one step."""
    _run(synth.WORKLOADS["llama8b_96k"], layer_idx=5, units=[0, 3, 7], check_steps=[1])


def test_codellama13b_b16_layer():
    """CodeLlama-13B shape, batch 16, MHA (640 units, K=9, L=120), one step."""
    _run(synth.WORKLOADS["codellama13b_b16"], layer_idx=0, units=[0, 7 * 40 + 23, 15 * 40 + 39], check_steps=[1])


def test_codellama34b_b4_64_steps():
    """CodeLlama-34B shape, batch 4, GQA 8 (K=10, L=240): build, then 64 appending decode steps."""
    _run(synth.WORKLOADS["codellama34b_b4"], layer_idx=0, units=[0, 13, 31], check_steps=[1, 2, 33, 64])
