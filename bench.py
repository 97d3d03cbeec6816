#!/usr/bin/env python3
"""Benchmark of the SimHash-sampled decode-attention step on one MI355X.

Workload (default): Llama-3.1-8B-shaped decode at 96K context -- 32 layers x
(32 query heads, 8 KV heads, d = 128), n = 98304 bf16 keys/values per KV head,
batch 1, SimHash (K, L) = (10, 150).  Inputs are synthetic (the cone-plus-sink
generator in ``synth``), resident in HBM before timing starts.

One step = for every layer: mp_decode_step, i.e. append the new token's
key/value and codes and encode the 32 queries (one launch), look the queries'
buckets up in the bucketed hash tables of the prefill keys (one launch),
select + weight + split-attend (the sampling kernel) and merge.  The code
store and its index are built once beforehand (mp_build_codes,
mp_build_buckets), timed separately.  By default the same steps are replayed
with the bit-plane index and with a plain scan of the 16-bit codes, reported
under "index_alternatives".

Prints one JSON line.  ``value`` = context keys scanned per second over the
whole step (all layers and KV heads); ``ms_per_step`` = decode-step latency.
``roofline`` describes the dominant kernel (the sampling kernel: scan,
weighting, split attention) against the 8 TB/s HBM peak, its duration taken
from HIP events that mp_decode_step attaches to every launch of it in the
last timed step (32 launches; the events add ~4 us per launch, so the other
timed steps run without them).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSH-sampled decode attn: context keys/s + latency at 96K, % HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sample_kernel_traffic.json")
DECODE_SRC = os.path.join(ROOT, "lsh_sampled_sparse_centered_amd", "csrc", "mp_decode.hip")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def source_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha1(f.read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_96k")
    ap.add_argument("--seed", type=int, default=2024)
    ap.add_argument("--layers", type=int, default=0, help="override the resident layer count (0 = workload's)")
    ap.add_argument("--step-layers", type=int, default=0,
                    help="layer decodes per step (0 = the resident layers); more cycle through the resident layers, "
                         "for a workload whose caches exceed one GPU's memory at the real per-layer shape")
    ap.add_argument("--threshold", type=int, default=2,
                    help="collision threshold T: a key is sampled in at least T of the L tables (the pages' 2)")
    ap.add_argument("--alternatives", choices=("on", "off"), default="on",
                    help="also time the other two index choices on the same built layers (reported as context)")
    ap.add_argument("--index", choices=("planes", "buckets", "codes"), default="buckets",
                    help="planes: build the bit-plane index of the code store at set-up (whole 512-key tiles of the "
                         "prefill keys) and let the threshold-2 scan read it; buckets: build the bucketed hash "
                         "tables and look the query's buckets up instead of scanning; codes: scan the 16-bit codes")
    ap.add_argument("--policy", choices=("sampled", "pages"), default="sampled",
                    help="sampled: every layer sampled; pages: the pages' decoding policy (layers 0 and 16 "
                         "dense, i.e. K = 0, and 4 sink + 64 local keys forced into every sampled layer's set)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-oracle baseline budget (0 = skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration under rocprofv3)")
    ap.add_argument("--trace-stats", metavar="KERNEL_TRACE_CSV",
                    help="print per-kernel statistics of the timed decode steps from a rocprofv3 kernel trace of a "
                         "run with the same --steps/--warmup/--layers/--workload and --alternatives off, and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection.csv files (FETCH_SIZE run, WRITE_SIZE run, both with "
                         "--calib-copy-mib and --alternatives off, and the same --steps/--warmup/--layers as given "
                         "here) into %s and exit" % os.path.relpath(TRAFFIC_FILE, ROOT))
    return ap.parse_args()


def traffic_from_counters(fetch_csv: str, write_csv: str, calib_mib: int, workload: str, index: str,
                          ndecode: int) -> dict:
    """HBM bytes per launch of the sampling kernel (and of the bucket lookup)
    in the decode steps from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for the calibration copy of
    calib_mib MiB (the largest __amd_rocclr_copyBuffer dispatch).  Only the
    first ndecode dispatches of a kernel count: the steps' (warmup + timed)
    launches, not the decodes after timing that measure the sampled sets."""
    import csv

    def per_kernel(path, counter, kernel):
        samp, calib = [], []
        with open(path) as f:
            for r in sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"])):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if kernel in r["Kernel_Name"]:
                    samp.append(v)
                elif "copyBuffer" in r["Kernel_Name"]:
                    calib.append(v)
        if not calib:
            raise SystemExit("%s: no calibration-copy rows for %s" % (path, counter))
        samp = samp[:ndecode]
        return (sum(samp) / len(samp) if samp else None), max(calib), len(samp)

    calib_bytes = calib_mib * (1 << 20)
    res = {"workload": workload, "source_sha": source_sha(DECODE_SRC), "index": index}
    for kernel, key in (("sample_kernel", ""), ("bucket_lookup_kernel", "lookup_")):
        f_s, f_c, nf = per_kernel(fetch_csv, "FETCH_SIZE", kernel)
        w_s, w_c, nw = per_kernel(write_csv, "WRITE_SIZE", kernel)
        if f_s is None or w_s is None:
            if not key:
                raise SystemExit("no sample_kernel rows in the counter files")
            continue
        fetch_scale = calib_bytes / (f_c * 1024.0)
        write_scale = calib_bytes / (w_c * 1024.0)
        fetch_b = f_s * 1024.0 * fetch_scale
        write_b = w_s * 1024.0 * write_scale
        res.update({key + "bytes_per_launch": fetch_b + write_b,
                    key + "fetch_bytes_per_launch": fetch_b, key + "write_bytes_per_launch": write_b,
                    key + "fetch_size_kib_per_launch": f_s, key + "write_size_kib_per_launch": w_s,
                    key + "dispatches": [nf, nw]})
        res["calibration"] = {"copy_mib": calib_mib, "fetch_size_kib": f_c, "write_size_kib": w_c,
                              "fetch_scale": fetch_scale, "write_scale": write_scale}
    return res


def trace_stats(path: str, steps: int, warmup: int, nlayers: int) -> str:
    """Markdown table of the kernels of the timed decode steps in a rocprofv3
    kernel trace: the sampling-kernel dispatches warmup*nlayers ..
    (warmup+steps)*nlayers - 1 (set-up launches none), widened back to the
    launch after the last warmup merge and forward to the merge after the
    last of them."""
    import csv

    with open(path) as f:
        rows = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                       for r in csv.DictReader(f) if r["Kind"] == "KERNEL_DISPATCH"))
    samp = [i for i, r in enumerate(rows) if "sample_kernel" in r[2]]
    if len(samp) < (warmup + steps) * nlayers:
        raise SystemExit("%s: %d sampling-kernel dispatches, expected at least %d" %
                         (path, len(samp), (warmup + steps) * nlayers))
    if warmup < 1:
        raise SystemExit("--trace-stats needs --warmup >= 1 (the window starts after a warmup step's merge)")
    lo, hi = samp[warmup * nlayers], samp[(warmup + steps) * nlayers - 1]
    def is_merge(name):  # the merge with index lists (merge_kernel) or without them (merge_q_kernel)
        return "merge_kernel" in name or "merge_q_kernel" in name

    while lo > 0 and not is_merge(rows[lo - 1][2]):  # back to the previous step's last merge
        lo -= 1
    while hi + 1 < len(rows) and not is_merge(rows[hi][2]):
        hi += 1
    win = rows[lo:hi + 1]
    by = {}
    for s0, e0, name in win:
        short = name.split("(")[0]
        for key in ("encode_small_kernel", "encode_kernel", "bucket_lookup_kernel", "sample_kernel", "merge_q_kernel",
                    "merge_kernel"):
            if key in short:
                short = key
        by.setdefault(short, []).append((e0 - s0) / 1e3)
    span = (win[-1][1] - win[0][0]) / 1e3
    out = ["| kernel | calls | avg us | min us | max us | total us per step |", "|---|---|---|---|---|---|"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append("| %s | %d | %.2f | %.2f | %.2f | %.1f |" % (k, len(v), sum(v) / len(v), min(v), max(v),
                                                              sum(v) / steps))
    out.append("")
    out.append("timed steps: %d; first to last dispatch %.1f us = %.1f us per step; kernel time %.1f us per step"
               % (steps, span, span / steps, sum(sum(v) for v in by.values()) / steps))
    return "\n".join(out)


def main() -> int:
    args = parse()
    if args.trace_stats:
        w = __import__("synth").WORKLOADS[args.workload]
        print(trace_stats(args.trace_stats, args.steps, args.warmup, args.step_layers or args.layers or w.layers))
        return 0
    if args.traffic:
        w = __import__("synth").WORKLOADS[args.workload]
        tr = traffic_from_counters(args.traffic[0], args.traffic[1], args.calib_copy_mib, args.workload,
                                   args.index if args.threshold == 2 else "codes",
                                   (args.steps + args.warmup) * (args.layers or w.layers))
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(tr, f, indent=1)
        print(json.dumps(tr))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the sampled decode shards by (layer, sequence, KV head) with no "
              "exchange, so more GPUs are independent copies of this run; --gpus %d is not supported"
              % max(args.gpus, world), file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import lsh_sampled_sparse_centered_amd as mp
    import synth

    w = synth.WORKLOADS[args.workload]
    nlayers = args.layers or w.layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    U, G, d, K, L, n0 = w.batch * w.hkv, w.group, w.d, w.K, w.L, w.n
    total_steps = args.warmup + args.steps
    cap = (n0 + total_steps + 8 + 63) // 64 * 64
    dt = w.torch_dtype
    log("workload %s: %d layers, B=%d Hq=%d Hkv=%d d=%d n=%d cap=%d (K,L)=(%d,%d) policy %s" %
        (w.name, nlayers, w.batch, w.hq, w.hkv, d, n0, cap, K, L, args.policy))
    # per layer: (K, L, forced head, forced tail); a dense layer has K = 0 (every key collides in
    # every table, P = 1: exact attention) and the smallest table count
    pages = args.policy == "pages"
    lcfg = [((0, 2, 0, 0) if pages and l in (0, 16) else (K, L, 4 if pages else 0, 64 if pages else 0))
            for l in range(nlayers)]
    sampled_layers = [l for l in range(nlayers) if lcfg[l][0] > 0]
    step_layers = args.step_layers or nlayers
    step_lids = [i % nlayers for i in range(step_layers)]  # resident layer of each of a step's layer decodes
    step_sampled = [i for i, l in enumerate(step_lids) if lcfg[l][0] > 0]
    modes = [args.index] + ([m for m in ("buckets", "planes", "codes") if m != args.index]
                            if args.alternatives == "on" else [])
    use_planes = "planes" in modes
    use_buckets = "buckets" in modes
    n_planes = (n0 // 512) * 512  # appended keys stay in the 16-bit codes (tiles past the index)

    # ------------------------------------------------------------------ inputs + code-store build
    layers = []
    build_ms = []
    ws_build = torch.empty(mp.mp_build_ws_bytes(U, n0), dtype=torch.uint8, device=dev)
    for l in range(nlayers):
        Kc = torch.zeros(U, cap, d, dtype=dt, device=dev)
        Vc = torch.zeros(U, cap, d, dtype=dt, device=dev)
        for u in range(U):
            b, h = divmod(u, w.hkv)
            synth.unit_kv(args.seed, l, b, h, n0, d, dt, dev, out_k=Kc[u, :n0], out_v=Vc[u, :n0])
        Kl, Ll = lcfg[l][0], lcfg[l][1]
        W = synth.projections(args.seed, l, d, Kl, Ll, dev)
        Wp = mp.mp_proj_pack(W, Kl, Ll)
        kmean = torch.empty(U, d, dtype=torch.float32, device=dev)
        codes = torch.zeros(U, Ll, cap, dtype=torch.uint16, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mp.mp_build_codes(Kc, n0, Wp, Kl, Ll, kmean=kmean, codes=codes, ws=ws_build)
        e1.record()
        kn = torch.empty(total_steps, U, d, dtype=dt)
        vn = torch.empty(total_steps, U, d, dtype=dt)
        qs = torch.empty(total_steps, w.batch, w.hq, d, dtype=dt)
        for s in range(total_steps):
            for u in range(U):
                b, h = divmod(u, w.hkv)
                kn[s, u], vn[s, u] = synth.step_kv(args.seed, l, b, h, d, dt, step=s + 1)
                qs[s, b, h * G:(h + 1) * G] = synth.unit_queries(args.seed, l, b, h, G, d, dt, step=s + 1)
        kn, vn, qs = kn.to(dev), vn.to(dev), qs.to(dev)
        planes, buckets, pev, bev = None, None, None, None
        if Kl > 0:  # the indexes of the prefill keys' whole tiles
            if use_planes:
                pev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                pev[0].record()
                planes = torch.empty(U, (cap + 511) // 512, Kl, Ll, 16, dtype=torch.int32, device=dev)
                mp.mp_build_planes(codes, Kl, n_planes, planes=planes)
                pev[1].record()
            if use_buckets:
                bev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                bev[0].record()
                buckets = mp.mp_build_buckets(codes, Kl, n_planes)
                bev[1].record()
        layers.append(dict(Kc=Kc, Vc=Vc, Wp=Wp, kmean=kmean, codes=codes, kn=kn, vn=vn, qs=qs, ev=(e0, e1),
                           planes=planes, buckets=buckets, pev=pev, bev=bev))
    torch.cuda.synchronize()
    build_ms = [layers[l]["ev"][0].elapsed_time(layers[l]["ev"][1]) for l in sampled_layers]
    index_ms = {}
    for key, name in (("pev", "planes"), ("bev", "buckets")):
        t = [layers[l][key][0].elapsed_time(layers[l][key][1]) for l in sampled_layers if layers[l][key] is not None]
        if t:
            index_ms[name] = float(np.median(t))
    log("built %d layers; build %.3f ms/layer (median); index builds %s ms/layer" %
        (nlayers, float(np.median(build_ms)), {k: round(v, 3) for k, v in index_ms.items()}))

    ws = mp.decode_workspace(w.batch, w.hq, w.hkv, cap, L, dev)
    outs = [torch.empty(w.batch, w.hq, d, dtype=torch.float32, device=dev) for _ in range(nlayers)]
    lses = [torch.empty(w.batch, w.hq, dtype=torch.float32, device=dev) for _ in range(nlayers)]

    # ------------------------------------------------------------------ decode steps
    # one step = for every layer: mp_decode_step (append + query encode in one
    # launch, [bucket lookup,] the sampling kernel and the merge).  In the last
    # timed step the library attaches HIP events to every sampling-kernel
    # dispatch; they cost about 4 us per launch, so the other timed steps run
    # without them.  Each index choice replays the same steps from n0 (the
    # appended rows and codes are rewritten with the same values).
    def run_steps(mode):
        ev_steps = min(args.steps, 1)
        kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(ev_steps * step_layers)]
        for pair in kev:
            for e in pair:
                e.record()  # create the underlying events before handing them to the library
        n_cur = n0
        t0 = 0.0
        step_ev = [torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
        n_timed = []
        torch.cuda.synchronize()
        for s in range(total_steps):
            if s == args.warmup:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                step_ev[0].record()
            for i, l in enumerate(step_lids):
                lay = layers[l]
                k = s - (total_steps - ev_steps)
                ev = kev[k * step_layers + i] if k >= 0 else None
                pl = lay["planes"] if mode == "planes" else None
                bk = lay["buckets"] if mode == "buckets" else None
                mp.mp_decode_step(lay["kn"][s], lay["vn"][s], lay["qs"][s], lay["Kc"], lay["Vc"], lay["codes"],
                                  lay["kmean"], lay["Wp"], w.hkv, n_cur, lcfg[l][0], ws, n_static_head=lcfg[l][2],
                                  n_static_tail=lcfg[l][3], out=outs[l], lse=lses[l], sample_events=ev,
                                  T=args.threshold, planes=pl, n_planes=n_planes if pl is not None else 0,
                                  buckets=bk, n_buckets=n_planes if bk is not None else 0)
            if s >= args.warmup:
                n_timed.append(n_cur + 1)
            n_cur += 1
        step_ev[1].record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / args.steps
        evms = step_ev[0].elapsed_time(step_ev[1]) / args.steps
        kern = np.array([a.elapsed_time(b) for a, b in kev])[step_sampled]  # the sampled layers' kernel
        log("[%s] step %.3f ms (wall) / %.3f ms (events); sample kernel %.2f us avg over %d launches" %
            (mode, wall, evms, kern.mean() * 1e3, len(kern)))
        return wall, evms, kern, n_timed, n_cur

    timing = {m: run_steps(m) for m in modes}
    wall_ms, ev_ms, kern_ms, n_timed, n_cur = timing[args.index]
    keys_per_step = float(np.mean(n_timed)) * U * step_layers
    value = keys_per_step / (wall_ms * 1e-3)

    # ------------------------------------------------------------------ sampled-set sizes (after timing)
    union_sum = 0
    head_sum = 0
    bucket_entries = 0  # sum over heads and tables of the query's bucket sizes (keys below the index)
    idx = torch.empty(w.batch, w.hq, cap, dtype=torch.int32, device=dev)
    cnt = torch.empty(w.batch, w.hq, dtype=torch.int32, device=dev)
    s_last = total_steps - 1
    for l in sampled_layers:
        lay = layers[l]
        mp.mp_decode_attn(lay["qs"][s_last], lay["Kc"], lay["Vc"], lay["codes"], lay["kmean"], lay["Wp"], w.hkv,
                          n_cur, K, lcfg[l][2], lcfg[l][3], idx=idx, count=cnt, ws=ws, T=args.threshold)
        qc_last = mp.mp_encode_queries(lay["qs"][s_last], lay["Wp"], K, L).view(torch.int16)
        for b in range(w.batch):
            for h in range(w.hkv):
                mask = torch.zeros(n_cur, dtype=torch.bool, device=dev)
                for g in range(G):
                    c = int(cnt[b, h * G + g])
                    mask[idx[b, h * G + g, :c].long()] = True
                    if use_buckets:
                        cu = lay["codes"].view(torch.int16)[b * w.hkv + h, :, :n_planes]
                        bucket_entries += int((cu == qc_last[b, h * G + g][:, None]).sum())
                union_sum += int(mask.sum())
        head_sum += int(cnt.sum())
    union_per_unit = union_sum / (len(sampled_layers) * U)
    head_frac = head_sum / (len(sampled_layers) * w.batch * w.hq * n_cur)
    e = 2 if w.dtype == "bf16" else 4
    n_dec = float(np.mean(n_timed))

    def launch_bytes(mode):
        """Algorithmic bytes of one sampling-kernel launch (one layer): the
        index or codes it reads, each distinct sampled K and V row once, the
        queries, their codes and the key means.  planes: K bits per key and
        table for the tiles the index covers; buckets: the lookup's sampled-key
        words (64 bytes per head and tile) for those tiles; 16-bit codes for
        the rest."""
        T2 = args.threshold == 2
        if mode == "buckets" and T2:
            code = G * 64 * n_planes / 512 + 2 * L * (n_dec - n_planes)
        elif mode == "planes" and T2:
            code = K * L * n_planes / 8 + 2 * L * (n_dec - n_planes)
        else:
            code = 2 * L * n_dec
        return U * (code + 2 * d * e * union_per_unit + G * (d * e + 2 * L) + 4 * d)

    # the bucket lookup kernel (before the sampling kernel): the query's bucket
    # entries (2 bytes each), one 4-byte start/count word per head, table and
    # chunk, the query codes; it writes the sampled-key words
    nbc = (n_planes + mp.MP_BUCKET_CHUNK - 1) // mp.MP_BUCKET_CHUNK
    lookup_bytes = (2 * bucket_entries / max(len(sampled_layers), 1) + U * G * L * (nbc * 4 + 2)
                    + U * G * 64 * n_planes / 512) if use_buckets else None
    bytes_launch = launch_bytes(args.index)
    achieved = bytes_launch / (kern_ms.mean() * 1e-3) / 1e9
    traffic = lookup_traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("source_sha") == source_sha(DECODE_SRC) and tr.get("workload") == w.name and not pages and
                args.threshold == 2 and tr.get("index") == args.index):
            traffic = tr.get("bytes_per_launch")
            lookup_traffic = tr.get("lookup_bytes_per_launch")
    alternatives = {}
    for m in modes[1:]:
        wm, em, km, nt, _ = timing[m]
        bl = launch_bytes(m)
        alternatives[m] = {"ms_per_step": wm, "value": float(np.mean(nt)) * U * step_layers / (wm * 1e-3),
                           "kernel_us": km.mean() * 1e3, "algorithmic_bytes_per_launch": bl,
                           "frac": bl / (km.mean() * 1e-3) / 1e9 / HBM_PEAK_GBS}
    # a dense layer reads its (two-table) codes and every key's K and V row
    dense_bytes = U * (2 * 2 * n_dec + 2 * d * e * n_dec + G * (d * e + 4) + 4 * d)
    step_bytes = len(step_sampled) * bytes_launch + (step_layers - len(step_sampled)) * dense_bytes
    log("|S_h|/n = %.4f, union per unit %.0f keys (%.4f of n); %.1f MB algorithmic per launch%s" %
        (head_frac, union_per_unit, union_per_unit / n_dec, bytes_launch / 1e6,
         "; bucket lookup %.2f MB per launch" % (lookup_bytes / 1e6) if lookup_bytes else ""))

    # ------------------------------------------------------------------ encoder (build) figures
    flops_layer = 2.0 * d * K * L * n0 * U
    enc_tflops = flops_layer / (float(np.median(build_ms)) * 1e-3) / 1e12

    # ------------------------------------------------------------------ calibration copy (profiling runs only)
    if args.calib_copy_mib:
        nb = args.calib_copy_mib * (1 << 20)
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        a.fill_(1)
        flush = torch.empty(2 * nb, dtype=torch.uint8, device=dev)
        flush.fill_(2)  # evicts a from L2 and the last-level cache
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)  # one device-to-device copy of known size
        torch.cuda.synchronize()
        del flush
        log("calibration copy of %d MiB done" % args.calib_copy_mib)

    # ------------------------------------------------------------------ achievable HBM rate (context)
    # a 1 GiB device-to-device copy (reads and writes 1 GiB each), best of 3, sources flushed
    nb = 1 << 30
    src = torch.empty(nb, dtype=torch.uint8, device=dev)
    src.fill_(3)
    dst = torch.empty_like(src)
    flush = torch.empty(nb, dtype=torch.uint8, device=dev)
    copy_ms = []
    for _ in range(3):
        flush.fill_(4)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    copy_gbs = 2.0 * nb / (min(copy_ms) * 1e-3) / 1e9
    del src, dst, flush
    log("device copy: %.0f GB/s (read + write)" % copy_gbs)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.seed, args.cpu_seconds, args.threshold)

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic cone-plus-sink keys/queries, N(0,1) values and projections, resident in HBM",
        "config": {"workload": w.name, "layers": step_layers, "resident_layers": nlayers, "batch": w.batch, "q_heads": w.hq, "kv_heads": w.hkv,
                   "head_dim": d, "context": n0, "K": K, "L": L, "threshold": args.threshold,
                   "code_scan": ("bit-plane index below key %d, 16-bit codes above" % n_planes
                                 if args.index == "planes" and args.threshold == 2
                                 else "bucketed tables below key %d, 16-bit codes above" % n_planes
                                 if args.index == "buckets" and args.threshold == 2
                                 else "16-bit codes"),
                   "parallelism": "single GPU",
                   "policy": ("every layer sampled" if not pages else
                              "pages: layers 0 and 16 dense (K = 0), 4 sink + 64 local keys forced elsewhere")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "sample_kernel (mp_decode_step / mp_decode_sample)", "kernel_us": kern_ms.mean() * 1e3,
                     "algorithmic_bytes_per_launch": bytes_launch, "device_copy_GBs": copy_gbs,
                     "frac_of_device_copy": achieved / copy_gbs,
                     "bucket_lookup_bytes_per_launch": lookup_bytes,
                     "bucket_lookup_traffic_per_launch": lookup_traffic},
        "index_alternatives": alternatives,
        "step": {"latency_ms": wall_ms, "latency_ms_events": ev_ms, "bytes_per_step": step_bytes,
                 "frac_hbm_step": step_bytes / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "sampled_frac_per_head": head_frac, "union_keys_per_unit": union_per_unit},
        "encoder": {"build_ms_per_layer": float(np.median(build_ms)), "tflops": enc_tflops,
                    "frac_mfma_bf16": enc_tflops / BF16_MFMA_PEAK_TFLOPS,
                    "note": "build = key mean + projection GEMM + sign pack, per layer",
                    "index_build_ms_per_layer": index_ms},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline(w, seed: int, budget_s: float, T: int = 2):
    """The CPU oracle timed on the host on a bounded sample of the same workload.

    Sample: KV heads 0..3 of layer 0 (batch 0) at the full context, with their
    query heads; keys/values regenerated on the host from the same recipe.
    The oracle builds its own codes for them (timed once, reported under
    "build" and extrapolated to a whole layer), then its decode over those
    heads is repeated with successive queries until the budget is spent.
    """
    import numpy as np
    import torch

    import oracle
    import synth

    nunits = min(4, w.hkv)
    G, d, n = w.group, w.d, w.n
    cap = (n + 63) // 64 * 64
    keys = np.zeros((1, nunits, cap, d), np.float32)
    vals = np.zeros_like(keys)
    for h in range(nunits):
        k, v = synth.unit_kv(seed, 0, 0, h, n, d, w.torch_dtype, "cpu")
        keys[0, h, :n] = k.float().numpy()
        vals[0, h, :n] = v.float().numpy()
    W = synth.projections(seed, 0, d, w.K, w.L, "cpu").numpy()
    t = time.perf_counter()
    km, codes = oracle.build_codes(keys[0], n, W, w.K, w.L)
    build_s = time.perf_counter() - t
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    reps = 0
    t = time.perf_counter()
    while True:
        q = np.zeros((1, nunits * G, d), np.float32)
        for h in range(nunits):
            q[0, h * G:(h + 1) * G] = synth.unit_queries(seed, 0, 0, h, G, d, w.torch_dtype, "cpu",
                                                         step=reps + 1).float().numpy()
        oracle.decode(q, keys, vals, codes.reshape(1, nunits, w.L, cap), km.reshape(1, nunits, d), W, w.K, w.L, n,
                      T=T)
        reps += 1
        el = time.perf_counter() - t
        if el >= budget_s:
            break
    keys_done = reps * nunits * n
    # the same decode on one thread, on one KV head's query heads, for a quarter of the budget
    oracle.set_threads(1)
    reps1 = 0
    t = time.perf_counter()
    while True:
        q1 = synth.unit_queries(seed, 0, 0, 0, G, d, w.torch_dtype, "cpu", step=reps1 + 1).float().numpy()[None]
        oracle.decode(q1, keys[:, :1], vals[:, :1], codes[:1].reshape(1, 1, w.L, cap), km[:1].reshape(1, 1, d), W,
                      w.K, w.L, n, T=T)
        reps1 += 1
        el1 = time.perf_counter() - t
        if el1 >= budget_s / 4:
            break
    oracle.set_threads(threads)
    return {"value": keys_done / el, "unit": "keys/s", "cores": min(threads, nunits * G), "kind": "oracle",
            "sample": "%d decode passes over %d KV heads x %d keys (%d query heads each), layer 0; "
                      "oracle build of their codes %.1fs (timed once); one-thread figure: %d passes over KV head 0"
                      % (reps, nunits, n, G, build_s, reps1),
            "value_1thread": reps1 * n / el1,
            "build": {"seconds": build_s, "keys": nunits * n,
                      "keys_per_s": nunits * n / build_s if build_s > 0 else None,
                      "per_layer_s_extrapolated": build_s * w.batch * w.hkv / nunits},
            "cpu_model": cpu_model(), "host_threads": threads,
            "seconds": el + el1 + build_s}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


if __name__ == "__main__":
    sys.exit(main())
