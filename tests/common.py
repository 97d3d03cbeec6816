"""Shared helpers of the parity tests: seeded inputs on host and device, and
the oracle's results for them.  Inputs come from ``synth``; expected values
come from ``oracle``; nothing here computes any part of the method."""
import dataclasses

import numpy as np
import torch

import oracle
import synth

BAND = 1e-5  # projections with |z| < BAND * |x| |w| may round either way


def variant(name: str, **kw) -> synth.Workload:
    return dataclasses.replace(synth.WORKLOADS[name], **kw)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).contiguous().numpy()


def layer(w: synth.Workload, seed: int, layer_idx: int = 0, n=None, cap=None, device="cuda"):
    """Seeded inputs of one layer, drawn on the host and copied to ``device``."""
    inp = synth.layer_inputs(w, seed, layer_idx, device="cpu", n=n, cap=cap)
    dev = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    U = w.batch * w.hkv
    dev["Kc"] = dev["K"].reshape(U, dev["cap"], w.d).contiguous()
    dev["Vc"] = dev["V"].reshape(U, dev["cap"], w.d).contiguous()
    dev["host"] = {"K": host_f32(inp["K"]), "V": host_f32(inp["V"]), "q": host_f32(inp["q"]),
                   "W": inp["W"].numpy().copy()}
    return dev


def oracle_codes(w: synth.Workload, lay, with_margin=True):
    """Oracle key means, codes [U][L][cap], margins [U][n][L] and query codes [B][Hq][L]."""
    h = lay["host"]
    U = w.batch * w.hkv
    keys = h["K"].reshape(U, lay["cap"], w.d)
    km, codes, margin = oracle.build_codes(keys, lay["n"], h["W"], w.K, w.L, with_margin=True)
    qc = oracle.encode(h["q"].reshape(-1, w.d), h["W"], w.K, w.L).reshape(w.batch, w.hq, w.L)
    return km, codes, margin, qc


def oracle_decode(w: synth.Workload, lay, km, codes, qc, n=None, nsh=0, nst=0, T=2):
    h = lay["host"]
    return oracle.decode(h["q"], h["K"], h["V"], codes.reshape(w.batch, w.hkv, w.L, lay["cap"]),
                         km.reshape(w.batch, w.hkv, w.d), h["W"], w.K, w.L, lay["n"] if n is None else n,
                         qcodes=qc, n_static_head=nsh, n_static_tail=nst, want_idx=True, T=T)


def code_mismatches_outside_band(gpu_codes: np.ndarray, ref_codes: np.ndarray, margin: np.ndarray):
    """Bit-by-bit comparison of codes against the oracle's.

    gpu/ref codes are ``[rows][L]`` uint16, margin ``[rows][K*L]`` (the
    oracle's |z|/(|x||w|) per projection column j = l*K + b).  A bit may
    differ only where its own projection is inside the rounding band.
    Returns (#differing bits, #differing bits outside the band)."""
    rows, L = ref_codes.shape
    assert gpu_codes.shape == ref_codes.shape and margin.shape[0] == rows and margin.shape[1] % L == 0
    K = margin.shape[1] // L
    diff = (np.asarray(gpu_codes, np.uint16) ^ np.asarray(ref_codes, np.uint16)).astype(np.uint32)
    # bit b of table l -> column l*K + b
    bits = (diff[:, :, None] >> np.arange(K, dtype=np.uint32)[None, None, :]) & 1
    bits = bits.reshape(rows, L * K).astype(bool)
    # codes carry no bits above K
    high = int(np.count_nonzero(diff >> np.uint32(K))) if K < 16 else 0
    return int(bits.sum()) + high, int((bits & (margin >= BAND)).sum()) + high
