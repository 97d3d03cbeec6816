"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one ``mp_decode_step`` per layer: append, query encode,
sample, merge).

Inputs are generated on the device by ``synth`` (seeded).  The oracle gets
its own copies of them by regenerating each unit from ``synth``; nothing it
reads comes from memory the HIP path writes.  Checked per layer:

* key means of every unit, bitwise;
* codes of a seeded 5% subset of units against the oracle's, up to the
  rounding band; those units then decode with the oracle's codes, every other
  unit with seeded uniform random codes (the same on both sides);
* every appended key: cache rows exact, codes up to the band;
* every query's codes up to the band;
* outputs, lse and counts of the step itself for every checked unit whose
  appended and query codes equal the oracle's (out within 2e-3, lse within
  1e-3, counts exact);
* a decode with the oracle's query codes injected: index lists exact and
  outputs within 2e-3 for every checked unit.

The prefill keys' whole tiles are found through the bit-plane index or the
bucketed hash tables (the benchmark's default), built from the injected
codes, or by scanning the codes; the appended keys are always scanned.

Which units are checked at which step: every unit at the first and last
step; at the steps in between, the code subset.
"""
import dataclasses

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
BATCH_UNITS = 64  # units per oracle batch (host memory)


def _i16(a: np.ndarray) -> torch.Tensor:
    """uint16 codes as an int16 device tensor (copies and slices of uint16
    tensors go through their int16 view)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def _say(msg):
    print("[gpu fullsize] " + msg, flush=True)


def code_subset(w, layers):
    """Seeded 5% of the units of ``layers`` (at least one): list of (layer, unit)."""
    U = w.batch * w.hkv
    allu = [(l, u) for l in layers for u in range(U)]
    k = max(1, round(0.05 * len(allu)))
    pick = np.random.default_rng([SEED, w.L, len(allu)]).choice(len(allu), size=k, replace=False)
    return sorted(allu[i] for i in pick)


class LayerRun:
    """One layer on the device, decoded step by step, checked against the oracle."""

    def __init__(self, w, layer_idx, code_units, T=2, index=None, nsh=0, nst=0):
        self.w, self.li, self.T, self.nsh, self.nst = w, layer_idx, T, nsh, nst
        self.index, self.planes, self.n_planes, self.buckets, self.n_buckets = index, None, 0, None, 0
        self.code_units = sorted(code_units)
        lay = synth.layer_inputs(w, SEED, layer_idx, device="cuda")
        self.U, self.cap, self.n0 = w.batch * w.hkv, lay["cap"], lay["n"]
        self.n = self.n0
        self.Kc = lay["K"].view(self.U, self.cap, w.d)
        self.Vc = lay["V"].view(self.U, self.cap, w.d)
        self.Wh = lay["W"].cpu().numpy().copy()
        self.Wp = mp.mp_proj_pack(lay["W"], w.K, w.L)
        self.kmean, self.codes = mp.mp_build_codes(self.Kc, self.n0, self.Wp, w.K, w.L)
        self.c16 = self.codes.view(torch.int16)
        torch.cuda.synchronize()
        self.kn_h, self.vn_h, self.app = [], [], []  # per step: [U][d] keys/values, [U][L] oracle codes
        self.oracle_codes = {}  # unit -> oracle codes [L][cap] of the build (code subset)
        self.km_o = np.zeros((self.U, w.d), np.float32)
        self.ws = mp.decode_workspace(w.batch, w.hq, w.hkv, self.cap, w.L, "cuda")
        _say("%s layer %d: B=%d Hq=%d Hkv=%d n=%d K=%d L=%d forced %d+%d; code subset %s" %
             (w.name, layer_idx, w.batch, w.hq, w.hkv, w.n, w.K, w.L, nsh, nst, self.code_units))

    # ------------------------------------------------------------ host inputs
    def host_kv(self, u):
        """Keys and values of unit u as the oracle sees them: regenerated from
        synth, with the appended rows of the steps so far."""
        w = self.w
        b, h = divmod(u, w.hkv)
        k, v = synth.unit_kv(SEED, self.li, b, h, self.n0, w.d, w.torch_dtype, device="cuda")
        K = np.zeros((self.cap, w.d), np.float32)
        V = np.zeros((self.cap, w.d), np.float32)
        K[:self.n0], V[:self.n0] = host_f32(k), host_f32(v)
        for s, (kn, vn) in enumerate(zip(self.kn_h, self.vn_h)):
            K[self.n0 + s], V[self.n0 + s] = kn[u], vn[u]
        return K, V

    def host_codes(self, u):
        """The code store of unit u as the oracle sees it."""
        w = self.w
        if u in self.oracle_codes:
            c = self.oracle_codes[u].copy()
        else:
            b, h = divmod(u, w.hkv)
            c = synth.unit_codes(SEED, self.li, b, h, w.K, w.L, self.cap, device="cuda").cpu().numpy()
            c = c.astype(np.uint16)
        for s, a in enumerate(self.app):
            c[:, self.n0 + s] = a[u]
        return c

    # ------------------------------------------------------------ build checks
    def check_build_and_inject(self):
        w = self.w
        gk = self.kmean.cpu().numpy()
        for u in range(self.U):
            b, h = divmod(u, w.hkv)
            k, _ = synth.unit_kv(SEED, self.li, b, h, self.n0, w.d, w.torch_dtype, device="cuda")
            self.km_o[u] = oracle.key_mean(host_f32(k))
        bad = np.nonzero((gk.view(np.uint32) != self.km_o.view(np.uint32)).any(axis=1))[0]
        assert len(bad) == 0, "key means differ in units %s" % bad[:10]
        ndiff = total = 0
        for u in self.code_units:
            K, _ = self.host_kv(u)
            km, codes, margin = oracle.build_codes(K[None], self.n0, self.Wh, w.K, w.L, with_margin=True)
            assert np.array_equal(km[0].view(np.uint32), self.km_o[u].view(np.uint32))
            g = _u16(self.c16[u])[:, :self.n0]
            nd, nbad = code_mismatches_outside_band(g.T, codes[0][:, :self.n0].T, margin[0])
            assert nbad == 0, (self.li, u, nbad)
            ndiff, total = ndiff + nd, total + g.size
            self.oracle_codes[u] = codes[0]
        for u in range(self.U):
            if u in self.oracle_codes:
                self.c16[u].copy_(_i16(self.oracle_codes[u]))
            else:
                b, h = divmod(u, w.hkv)
                self.c16[u].copy_(synth.unit_codes(SEED, self.li, b, h, w.K, w.L, self.cap, device="cuda"))
        torch.cuda.synchronize()
        _say("layer %d: %d key means bitwise; %d of %d subset codes differ, all inside the band" %
             (self.li, self.U, ndiff, total))

    def build_index(self):
        """The bit-plane index or the bucketed tables of the (injected) codes
        for the prefill keys' whole tiles, as the benchmark builds them;
        appended keys stay past them."""
        nw = (self.n0 // 512) * 512
        if self.index == "planes":
            self.n_planes = nw
            self.planes = mp.mp_build_planes(self.codes, self.w.K, nw)
        elif self.index == "buckets":
            self.n_buckets = nw
            self.buckets = mp.mp_build_buckets(self.codes, self.w.K, nw)
        torch.cuda.synchronize()
        _say("layer %d: %s of keys [0, %d)" % (self.li, self.index, nw))

    def _index_args(self):
        return dict(planes=self.planes, n_planes=self.n_planes, buckets=self.buckets, n_buckets=self.n_buckets)

    # ------------------------------------------------------------ one step
    def step(self, s, check_units):
        w, G = self.w, self.w.group
        n = self.n
        kn = torch.empty(self.U, w.d, dtype=w.torch_dtype, device="cuda")
        vn = torch.empty_like(kn)
        q = torch.empty(w.batch, w.hq, w.d, dtype=w.torch_dtype, device="cuda")
        for b in range(w.batch):
            for h in range(w.hkv):
                kn[b * w.hkv + h], vn[b * w.hkv + h] = synth.step_kv(SEED, self.li, b, h, w.d, w.torch_dtype, s,
                                                                     device="cuda")
                q[b, h * G:(h + 1) * G] = synth.unit_queries(SEED, self.li, b, h, G, w.d, w.torch_dtype,
                                                             device="cuda", step=s)
        out = torch.empty(w.batch, w.hq, w.d, dtype=torch.float32, device="cuda")
        lse = torch.empty(w.batch, w.hq, dtype=torch.float32, device="cuda")
        cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device="cuda")
        mp.mp_decode_step(kn, vn, q, self.Kc, self.Vc, self.codes, self.kmean, self.Wp, w.hkv, n, w.K, self.ws,
                          out=out, lse=lse, count=cnt, T=self.T, n_static_head=self.nsh, n_static_tail=self.nst,
                          **self._index_args())
        torch.cuda.synchronize()
        assert torch.equal(self.Kc[:, n], kn) and torch.equal(self.Vc[:, n], vn)
        # appended codes (frozen means) of every unit
        knh, vnh = host_f32(kn), host_f32(vn)
        got = _u16(self.c16[:, :, n])
        app, amg = oracle.encode(knh, self.Wh, w.K, w.L, mu=self.km_o, with_margin=True)  # one mean per unit
        app_same = np.zeros(self.U, bool)
        for u in range(self.U):
            nd, nbad = code_mismatches_outside_band(got[u][None], app[u][None], amg[u][None])
            assert nbad == 0, (s, u)
            app_same[u] = nd == 0
            if nd:  # keep the stores identical for the later steps
                self.c16[u, :, n] = _i16(app[u])
        self.kn_h.append(knh)
        self.vn_h.append(vnh)
        self.app.append(app)
        self.n = n + 1
        # query codes of every head
        qh = host_f32(q)
        gq = _u16(mp.mp_encode_queries(q, self.Wp, w.K, w.L).view(torch.int16))
        qref, qmg = oracle.encode(qh.reshape(-1, w.d), self.Wh, w.K, w.L, with_margin=True)
        qref = qref.reshape(w.batch, w.hq, w.L)
        nd_q = gq != qref
        assert code_mismatches_outside_band(gq.reshape(-1, w.L), qref.reshape(-1, w.L), qmg)[1] == 0, s
        if not check_units:
            return
        # decode of the checked units with the oracle's query codes, index lists included
        qc16 = _i16(qref)
        out2 = torch.empty_like(out)
        cnt2 = torch.empty_like(cnt)
        idx = torch.full((w.batch, w.hq, self.cap), -1, dtype=torch.int32, device="cuda")
        mp.mp_decode_attn(q, self.Kc, self.Vc, self.codes, self.kmean, None, w.hkv, self.n, w.K, self.nsh, self.nst,
                          qcodes_in=qc16.view(torch.uint16), out=out2, idx=idx, count=cnt2, ws=self.ws, T=self.T,
                          **self._index_args())
        torch.cuda.synchronize()
        o1, l1, c1 = out.cpu().numpy(), lse.cpu().numpy(), cnt.cpu().numpy()
        o2, c2, ix = out2.cpu().numpy(), cnt2.cpu().numpy(), idx.cpu().numpy()
        direct, worst, sizes = 0, 0.0, []
        for i0 in range(0, len(check_units), BATCH_UNITS):
            us = check_units[i0:i0 + BATCH_UNITS]
            kv = [self.host_kv(u) for u in us]
            bh = [divmod(u, w.hkv) for u in us]
            ref = oracle.decode(np.stack([qh[b, h * G:(h + 1) * G] for b, h in bh]),
                                np.stack([k for k, _ in kv])[:, None], np.stack([v for _, v in kv])[:, None],
                                np.stack([self.host_codes(u) for u in us])[:, None], self.km_o[us][:, None],
                                self.Wh, w.K, w.L, self.n, qcodes=np.stack([qref[b, h * G:(h + 1) * G] for b, h in bh]),
                                n_static_head=self.nsh, n_static_tail=self.nst, want_idx=True, T=self.T)
            for j, (u, (b, h)) in enumerate(zip(us, bh)):
                own = app_same[u] and not nd_q[b, h * G:(h + 1) * G].any()
                direct += int(own)
                for g in range(G):
                    hh = h * G + g
                    rc = int(ref["count"][j, g])
                    sizes.append(rc)
                    assert int(c2[b, hh]) == rc, (s, u, g)
                    assert np.array_equal(ix[b, hh, :rc], ref["idx"][j][g]), (s, u, g)
                    if own:
                        assert int(c1[b, hh]) == rc, (s, u, g)
                    if rc == 0:
                        assert np.all(o2[b, hh] == 0)
                        continue
                    err = float(np.max(np.abs(o2[b, hh] - ref["out"][j, g])))
                    worst = max(worst, err)
                    assert err <= OUT_TOL, (s, u, g, err)
                    if own:
                        assert np.max(np.abs(o1[b, hh] - ref["out"][j, g])) <= OUT_TOL, (s, u, g)
                        assert abs(float(l1[b, hh]) - float(ref["lse"][j, g])) <= LSE_TOL, (s, u, g)
        _say("layer %d step %d (n=%d, K=%d, T=%d, forced %d+%d, %s below %d): %d units checked (%d on the step's "
             "own outputs); sets exact; worst |out - oracle| %.3g; mean |S| %.0f" %
             (self.li, s, self.n, w.K, self.T, self.nsh, self.nst, self.index, max(self.n_planes, self.n_buckets),
              len(check_units), direct, worst, float(np.mean(sizes))))


def _run_layers(w, layers, steps=1, check_every=None, T=2, index="planes", layer_cfg=None):
    """Each layer: build, check and inject; then ``steps`` appending decode
    steps.  ``index``: "planes", "buckets" or None (scan the codes).
    ``layer_cfg(layer) -> (workload, forced head, forced tail)`` gives a
    layer its own table shape and forced ranges (the pages' policy)."""
    subset = code_subset(w, layers)
    for li in layers:
        wl, nsh, nst = layer_cfg(li) if layer_cfg else (w, 0, 0)
        ix = index if wl.K > 0 else None
        run = LayerRun(wl, li, [u for l, u in subset if l == li], T=T, index=ix, nsh=nsh, nst=nst)
        run.check_build_and_inject()
        if ix:
            run.build_index()
        allu = list(range(run.U))
        sub = run.code_units
        for s in range(1, steps + 1):
            full = s in (1, steps)
            run.step(s, allu if full else (sub if check_every and s % check_every == 0 else []))
        del run
        torch.cuda.empty_cache()


@pytest.mark.parametrize("part", range(4))
def test_llama8b_96k_all_layers(part):
    """Llama-3.1-8B shape at 96K context (32 q / 8 KV heads, K=10, L=150):
    every unit of 8 of the 32 layers, one appending step, the prefill keys
    found through the bucketed tables (the benchmark's default: layers 0-15)
    or the bit-plane index (layers 16-31)."""
    w = synth.WORKLOADS["llama8b_96k"]
    _run_layers(w, list(range(8 * part, 8 * part + 8)), index="buckets" if part < 2 else "planes")


def test_llama8b_96k_codes_only():
    """The 96K layer shape scanning only the 16-bit codes (no index)."""
    _run_layers(synth.WORKLOADS["llama8b_96k"], [7], index=None)


@pytest.mark.parametrize("T", [1, 3])
def test_llama8b_96k_threshold(T):
    """The 96K layer shape with collision thresholds 1 and 3 (the step and the
    index-list decode both take T): every unit of one layer, one appending step."""
    _run_layers(synth.WORKLOADS["llama8b_96k"], [5], T=T)


@pytest.mark.parametrize("layer_idx,index", [(0, "planes"), (39, "buckets"), (20, None)])
def test_codellama13b_b16_layer(layer_idx, index):
    """CodeLlama-13B shape, batch 16, MHA (640 units per layer, K=9, L=120), one appending step; with the
    bucketed tables the sampling blocks take four bitmap tiles each (21,120 tiles per layer)."""
    _run_layers(synth.WORKLOADS["codellama13b_b16"], [layer_idx], index=index)


@pytest.mark.parametrize("part", range(6))
def test_codellama34b_b4_64_steps(part):
    """CodeLlama-34B shape, batch 4, GQA 8 (K=10, L=240), all 48 layers in six
    parts: build, then 64 appending steps; every unit at steps 1 and 64, the
    seeded 5% code subset at every step in between (every appended key and
    every query's codes at every step)."""
    w = synth.WORKLOADS["codellama34b_b4"]
    _run_layers(w, list(range(8 * part, 8 * part + 8)), steps=64, check_every=1,
                index="buckets" if part < 3 else "planes")


@pytest.mark.parametrize("part", range(2))
def test_llama8b_96k_pages_policy(part):
    """The pages' decoding policy at 96K, one appending step over all 32
    layers (two parts): layers 0 and 16 dense (K = 0: every key sampled with
    P = 1), every other layer sampled with 4 sink and 64 local keys forced in
    with P = 1; every unit of every layer against the oracle."""
    w = synth.WORKLOADS["llama8b_96k"]
    dense = dataclasses.replace(w, K=0, L=2)

    def cfg(li):
        return (dense, 0, 0) if li in (0, 16) else (w, 4, 64)

    _run_layers(w, list(range(16 * part, 16 * part + 16)), layer_cfg=cfg)
