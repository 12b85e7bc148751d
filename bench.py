#!/usr/bin/env python3
"""Benchmark of the MapFlow retrieval hot path on one MI355X.

Workload: the 14B->8B-like pair, 24 reuse layers back to back (N = 8192,
B = 64, H_s = 40, H_r = 32, H_kv = 8, d = 128, bf16, p = 0.9), seeded
synthetic structured sender maps, one distinct sender map per layer.

One step = the whole hot path over all 24 layers, inputs resident in HBM:
    block mass -> Top-p selection + BSR build for every layer, then the fused
    head-mapped retrieval of every layer
with no host synchronisation inside the step (BSR capacities are sized in the
untimed warm-up).  Compressing all layers first means that no retrieval reads
tiles that the gather just before it wrote: each layer's compressed state was
last touched 23 layers earlier (about 10 GB of other traffic), so it comes
from HBM and not from the 256 MB Infinity Cache.  `value` is the metric:
fused-retrieval query-tokens/s per layer = 24 * N * steps / (sum of retrieval
kernel times), timed with HIP events on the launch stream.  The line also
carries the roofline of the retrieval kernel, per-kernel times, the same
retrieval timed right after its own gather (the warm, in-pipeline order),
single-layer retrieval legs for the 8B->3B-like and long-context workloads,
and the fp64 CPU oracle timed on a bounded sample of block rows.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--no-cpu]
                    [--no-qk] [--no-varlen] [--no-fanout] [--no-cache] [--no-configs]
                    [--copy-ref-mib M]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=None,
                    help="reuse layers per step (default: the workload's 24)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU work for the oracle leg")
    ap.add_argument("--no-qk", action="store_true",
                    help="skip the compression-without-dense-map leg")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed-batch (varlen) retrieval leg")
    ap.add_argument("--no-fanout", action="store_true",
                    help="skip the one-sender-several-receivers leg")
    ap.add_argument("--no-cache", action="store_true",
                    help="skip the Block Manager (prefix cache) leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the single-layer 8B->3B and long-context retrieval legs")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (reference "
                         "kernel for scaling hardware byte counters)")
    return ap.parse_args()


def launch_stats(us):
    """Median, 10th and 90th percentile of per-launch times (microseconds)."""
    v = np.asarray(us, dtype=np.float64)
    return {"n": int(v.size), "median": float(np.median(v)),
            "p10": float(np.percentile(v, 10)), "p90": float(np.percentile(v, 90))}


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "k_retrieve_pair_pair14b8b_bf16_N8192_traffic.txt")
KERNEL_SRC = os.path.join(HERE, "cross_model_sparse_amd", "csrc", "k_retrieve.hip")


def kernel_source_hash():
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic():
    """HBM bytes per retrieval launch measured with hardware counters (two
    rocprofv3 --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by a plain copy
    of known size), or None when no record exists or the kernel source has
    changed since it was taken."""
    try:
        rec = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    rec[k.strip()] = v.strip()
        if rec.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return {"bytes_per_launch": float(rec["hbm_bytes_per_launch"]),
                "fetch_bytes_per_launch": float(rec["fetch_bytes_per_launch"]),
                "write_bytes_per_launch": float(rec["write_bytes_per_launch"]),
                "source": os.path.relpath(TRAFFIC_FILE, HERE)}
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the retrieval path is built and measured "
              "on a single MI355X (multi-GPU sharding by block rows is design-only). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import cross_model_sparse_amd as mf
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mf.load()
    dev = torch.device("cuda:0")
    w = synth.workload("pair14b8b-bf16")
    L = args.layers or w.layers
    N, B, T = w.N, w.B, w.T
    e = synth.DTYPE_BYTES[w.dtype]

    # ---- inputs (untimed) ---------------------------------------------------
    t0 = time.time()
    layers = []
    for l in range(L):
        g = synth.gen_layer(w, layer=l, device=dev)
        layers.append({"A": g["A"], "W": g["W"].to(dev), "V": g["V"].to(dev),
                       "seed": g["seed"]})
        log(f"generated layer {l} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()

    # ---- capacities from one synchronous pass (untimed) ----------------------
    for x in layers:
        mass = mf.block_mass(x["A"], B)
        rp, ci, vals, nnzb = mf.topp_select_bsr(mass, x["A"], B, w.p)
        x.update(mass=mass, rp=rp, ci=ci, vals=vals, nnzb=nnzb,
                 ws=torch.empty(mf.topp_workspace_bytes(N, B), dtype=torch.uint8, device=dev),
                 O=torch.empty(N, w.H_r, w.d, dtype=synth.torch_dtype(w.dtype), device=dev))
    ws_bm = torch.empty(max(1, mf.block_mass_ws_bytes(w.H_s, N, B)), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(max(1, mf.retrieve_workspace_bytes(N, B, w.H_kv, w.d,
                                                          synth.torch_dtype(w.dtype))),
                       dtype=torch.uint8, device=dev)
    nnzbs = [x["nnzb"] for x in layers]
    log(f"nnzb per layer: min {min(nnzbs)} max {max(nnzbs)} "
        f"density {np.mean(nnzbs) / (T * (T + 1) / 2):.4f}")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    if args.copy_ref_mib > 0:
        # plain copy of known size: the counter-scaling reference
        n = args.copy_ref_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)         # one elementwise kernel: reads n, writes n bytes
        torch.cuda.synchronize()
        log(f"copy reference: {args.copy_ref_mib} MiB read + {args.copy_ref_mib} MiB written per launch")
        del src, dst

    def compress(x, evs=None):
        if evs: evs[0].record(stream)
        mf.block_mass(x["A"], B, out=x["mass"], workspace=ws_bm)
        if evs: evs[1].record(stream)
        mf.topp_select_bsr(x["mass"], x["A"], B, w.p, cap_nnzb=x["nnzb"],
                           row_ptr=x["rp"], col_idx=x["ci"], vals=x["vals"],
                           workspace=x["ws"], sync=False)
        if evs: evs[2].record(stream)

    def retrieve(x, evs=None):
        if evs: evs[2].record(stream)
        mf.retrieve_fused(x["rp"], x["ci"], x["vals"], x["nnzb"], x["W"], x["V"],
                          N, B, out=x["O"], workspace=ws_r)
        if evs: evs[3].record(stream)

    def step(record):
        evs = [[ev(), ev(), ev(), ev(), ev()] if record else None for _ in layers]
        for x, e in zip(layers, evs):
            compress(x, e and e[:3])
        for x, e in zip(layers, evs):
            retrieve(x, e and [None, None, e[3], e[4]])
        if record:
            rec.extend(tuple(e[:2]) + (e[1], e[2], e[3], e[4]) for e in evs)

    rec = []
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - tw0

    # the same retrieval in the warm order: each layer right after its own
    # gather, whose freshly written tiles partly sit in the Infinity Cache
    warm = []
    for _ in range(max(2, args.steps)):
        for x in layers:
            compress(x)
            a, b = ev(), ev()
            a.record(stream)
            mf.retrieve_fused(x["rp"], x["ci"], x["vals"], x["nnzb"], x["W"], x["V"],
                              N, B, out=x["O"], workspace=ws_r)
            b.record(stream)
            warm.append((a, b))
    torch.cuda.synchronize()

    # rec entries: (mass start, mass end, topp start, topp end, retrieve start, retrieve end)
    t_mass = sum(r[0].elapsed_time(r[1]) for r in rec) / 1e3
    t_topp = sum(r[2].elapsed_time(r[3]) for r in rec) / 1e3
    t_retr = sum(r[4].elapsed_time(r[5]) for r in rec) / 1e3
    K = args.steps
    n_retr = K * L
    ms_per_step = wall / K * 1e3

    # algorithmic bytes / flops of one retrieval launch, summed over layers
    def retr_bytes(nz):
        return (nz * w.H_s * B * B * e + N * w.H_kv * w.d * e + N * w.H_r * w.d * e
                + 4 * (T + 1 + nz) + 4 * w.H_r * w.H_s)

    def retr_flops(nz):
        return 2.0 * nz * w.H_r * B * B * (w.H_s + w.d)

    bytes_step = sum(retr_bytes(nz) for nz in nnzbs)
    traffic = recorded_traffic()
    flops_step = sum(retr_flops(nz) for nz in nnzbs)
    achieved_gbs = bytes_step * K / t_retr / 1e9
    achieved_tflops = flops_step * K / t_retr / 1e12
    causal_bytes = sum(w.H_s * B * B * e * (T * (T + 1) // 2) for _ in nnzbs)  # K1 tiles read
    gather_bytes = sum(2 * nz * w.H_s * B * B * e for nz in nnzbs)

    out = {
        "metric": "fused retrieval query-tokens/s per layer + % of HBM/MFMA roofline at N=8192",
        "value": N * n_retr / t_retr,
        "unit": "query-tokens/s per layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "pair14b8b-bf16: 14B->8B-like pair, 24 reuse layers",
                   "N": N, "B": B, "H_s": w.H_s, "H_r": w.H_r, "H_kv": w.H_kv,
                   "d": w.d, "p": w.p, "layers": L, "storage_dtype": "bf16",
                   "compute": "bf16 MFMA (W and mixed map as hi+lo bf16), fp32 accumulate",
                   "maps": "structured: sink + band 512 + 4 stripes/head + N(0,1) noise"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "traffic_detail": traffic,
                     "kernel": "k_retrieve_pair",
                     "bytes_per_launch": bytes_step / L,
                     "mfma_tflops": achieved_tflops,
                     "mfma_frac": achieved_tflops / MFMA_F16_PEAK_TFLOPS},
        "kernels_ms_per_layer": {"block_mass": t_mass / n_retr * 1e3,
                                 "topp_select_bsr": t_topp / n_retr * 1e3,
                                 "retrieve_fused": t_retr / n_retr * 1e3},
        "retrieve_fused_launch_us": launch_stats([r[4].elapsed_time(r[5]) * 1e3 for r in rec]),
        "retrieve_fused_after_own_gather_us": launch_stats([a.elapsed_time(b) * 1e3 for a, b in warm]),
        "roofline_kernels": {
            "block_mass_GBs": causal_bytes * K / t_mass / 1e9,
            "topp_select_bsr_GBs": gather_bytes * K / t_topp / 1e9},
        "e2e_query_tokens_per_s_per_layer": N * n_retr / wall,
        "nnzb_per_layer": {"min": min(nnzbs), "max": max(nnzbs),
                           "mean": float(np.mean(nnzbs))},
        "cpu_baseline": None,
    }

    if not args.no_qk:
        out["compress_without_dense_map"] = qk_leg(dev, args.steps)
    if not args.no_fanout:
        out["fanout"] = fanout_leg(dev, w, layers, max(5, args.steps))
    if not args.no_cache:
        out["prefix_cache"] = cache_leg(dev, w, layers, max(5, args.steps))
    if not args.no_varlen:
        out["varlen_batch"] = varlen_leg(dev, max(5, args.steps))
    if not args.no_configs:
        out["retrieval_configs"] = {name: single_layer_leg(dev, name, max(10, args.steps))
                                    for name in ("pair8b3b-f16", "long32k-f16")}
    out["measured_hbm"] = hbm_leg(dev)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_leg(w, layers, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def scrub(buf):
    """Overwrite a 512 MB buffer: afterwards the 256 MB Infinity Cache holds
    none of the data a timed kernel is about to read."""
    buf.add_(1)


def single_layer_leg(dev, name, reps):
    """Retrieval of one layer of another workload at its full size: the
    8B->3B-like pair (N = 4096, B = 64, H_s = 32, H_r = 24, H_kv = 8, fp16,
    p = 0.95, near-dense maps) or the long-context layer (N = 32768, B = 128,
    H_s = 32, H_r = 32, H_kv = 8, fp16, p = 0.9).  The layer is generated and
    compressed (untimed), its dense map freed, and the retrieval timed with HIP
    events `reps` times, each after a 512 MB scrub; median and spread, and the
    roofline from the same algorithmic bytes as the headline.  Where the
    library splits long block rows (near-dense maps), the retrieval gets the
    workspace for it, and the same layer with rows kept whole is timed beside."""
    import torch
    import cross_model_sparse_amd as mf
    import synth
    w = synth.workload(name)
    N, B, T, e = w.N, w.B, w.T, synth.DTYPE_BYTES[w.dtype]
    t0 = time.time()
    g = synth.gen_layer(w, device=dev)
    A = g["A"]
    W, V = g["W"].to(dev), g["V"].to(dev)
    mass = mf.block_mass(A, B)
    rp, ci, vals, nnzb = mf.topp_select_bsr(mass, A, B, w.p)
    del A, g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"{name}: generated and compressed ({time.time() - t0:.1f}s), nnzb {nnzb}")
    O = torch.empty(N, w.H_r, w.d, dtype=V.dtype, device=dev)
    buf = torch.zeros(512 << 18, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    # a workspace that lets the library split long block rows (0 bytes when
    # splitting does not apply to this layer)
    ws_bytes = mf.retrieve_split_workspace_bytes(nnzb, V.dtype, w.H_s, N, B, w.H_r, w.H_kv, w.d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def timed(workspace):
        mf.retrieve_fused(rp, ci, vals, nnzb, W, V, N, B, out=O, workspace=workspace)
        ts = []
        for _ in range(reps):
            scrub(buf)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            mf.retrieve_fused(rp, ci, vals, nnzb, W, V, N, B, out=O, workspace=workspace)
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return launch_stats(ts)
    st = timed(ws)
    st_whole = timed(None) if ws is not None else None
    alg = (nnzb * w.H_s * B * B * e + N * w.H_kv * w.d * e + N * w.H_r * w.d * e
           + 4 * (T + 1 + nnzb) + 4 * w.H_r * w.H_s)
    flops = 2.0 * nnzb * w.H_r * B * B * (w.H_s + w.d)
    t = st["median"] * 1e-6
    rows = np.diff(rp.cpu().numpy())
    out = {"workload": f"{name}: N={N}, B={B}, H_s={w.H_s}, H_r={w.H_r}, H_kv={w.H_kv}, "
                       f"d={w.d}, {w.dtype}, p={w.p}, {w.maps} maps",
           "kernel": mf.retrieve_kernel(vals, V, W, N, B, out=O),
           "nnzb": nnzb, "density": nnzb / (T * (T + 1) / 2),
           "kept_per_row": {"min": int(rows.min()), "max": int(rows.max()),
                            "mean": float(rows.mean())},
           "retrieve_us": st,
           "split_rows": ws is not None,
           "retrieve_us_rows_whole": st_whole,
           "query_tokens_per_s": N / t,
           "roofline": {"bound": "hbm", "bytes_per_launch": alg, "achieved": alg / t / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": alg / t / 1e9 / HBM_PEAK_GBS,
                        "mfma_tflops": flops / t / 1e12}}
    del rp, ci, vals, O, buf
    torch.cuda.empty_cache()
    return out


def hbm_leg(dev, reps=5):
    """Measured stream-copy rate of a plain library kernel on the same device,
    as context for the 8 TB/s peak the roofline uses: a 2 GiB device-to-device
    copy (4 GiB moved), HIP events, best of `reps`."""
    import torch
    stream = torch.cuda.current_stream()
    n = 2 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_GBs": 2 * n / min(ts) / 1e9, "peak_GBs": HBM_PEAK_GBS,
            "method": "torch copy_ of 2 GiB (2 GiB read + 2 GiB written), HIP events, best of 5"}


def qk_leg(dev, reps):
    """Compression from Q and K without a dense map, on the 8B->3B-like pair's
    first layer (N = 4096, B = 64, H_s = 32, d = 128, fp16, p = 0.95; Q, K from
    the workload's seeded recipe), timed with HIP events next to the dense
    path (block mass + selection/gather over the [H_s][N][N] map built from the
    same Q and K).  Two forms: row_lse then block_mass_qk (two passes over the
    scores), and lse_block_mass_qk (one pass and a small reduction)."""
    import torch
    import cross_model_sparse_amd as mf
    import synth
    w = synth.workload("pair8b3b-f16")
    N, B, H_s, d, p = w.N, w.B, w.H_s, w.d, w.p
    A, Q, K, tau = synth.gen_maps(w, synth.layer_seed(w, 0), device=dev, return_qk=True)
    Qd = Q.to(device=dev, dtype=torch.float16)
    Kd = K.to(device=dev, dtype=torch.float16)
    scale = (1.0 / (d ** 0.5 * tau)).to(device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(3, reps)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    lse = mf.row_lse(Qd, Kd, scale)
    ws = torch.empty(mf.block_mass_qk_workspace_bytes(H_s, N, B), dtype=torch.uint8, device=dev)
    mass = mf.block_mass_qk(Qd, Kd, scale, lse, B, workspace=ws)
    rp, ci, vals, nnzb = mf.topp_select_bsr_qk(mass, Qd, Kd, scale, lse, B, p)
    wsel = torch.empty(mf.topp_workspace_bytes(N, B), dtype=torch.uint8, device=dev)
    t_lse = timed(lambda: mf.row_lse(Qd, Kd, scale, out=lse))
    t_mass = timed(lambda: mf.block_mass_qk(Qd, Kd, scale, lse, B, out=mass, workspace=ws))
    t_sel = timed(lambda: mf.topp_select_bsr_qk(mass, Qd, Kd, scale, lse, B, p, cap_nnzb=nnzb,
                                                row_ptr=rp, col_idx=ci, vals=vals,
                                                workspace=wsel, sync=False))
    # lse and masses in one pass over the scores (mf_lse_block_mass_qk)
    ws1 = torch.empty(mf.lse_block_mass_qk_workspace_bytes(H_s, N, B), dtype=torch.uint8, device=dev)
    lse1, mass1 = mf.lse_block_mass_qk(Qd, Kd, scale, B, workspace=ws1)
    t_one = timed(lambda: mf.lse_block_mass_qk(Qd, Kd, scale, B, lse=lse1, out=mass1, workspace=ws1))
    rp1, ci1, vals1, nnzb1 = mf.topp_select_bsr_qk(mass1, Qd, Kd, scale, lse1, B, p)
    dmass = mf.block_mass(A, B)
    drp, dci, dvals, dnnzb = mf.topp_select_bsr(dmass, A, B, p)
    t_dmass = timed(lambda: mf.block_mass(A, B, out=dmass))
    t_dsel = timed(lambda: mf.topp_select_bsr(dmass, A, B, p, cap_nnzb=dnnzb, row_ptr=drp,
                                              col_idx=dci, vals=dvals, workspace=wsel,
                                              sync=False))
    # one score pass covers the causal pairs (diagonal 32 x 32 tiles computed whole)
    tiles = sum(i + 1 for i in range(-(-N // 32)))
    pass_flops = 2.0 * H_s * tiles * 32 * 32 * d
    gather_flops = 2.0 * nnzb * H_s * B * B * d
    causal_pairs = N * (N + 1) / 2
    total = t_lse + t_mass + t_sel
    return {
        "workload": f"pair8b3b-f16 layer 0: N={N}, B={B}, H_s={H_s}, K heads {K.shape[0]}, d={d}, fp16, p={p}",
        "ms": {"row_lse": t_lse, "block_mass_qk": t_mass, "topp_select_bsr_qk": t_sel, "total": total},
        "one_pass_ms": {"lse_block_mass_qk": t_one, "topp_select_bsr_qk": t_sel,
                        "total": t_one + t_sel, "nnzb": nnzb1},
        "dense_path_ms": {"block_mass": t_dmass, "topp_select_bsr": t_dsel,
                          "total": t_dmass + t_dsel},
        "dense_map_bytes_not_formed": H_s * N * N * 2,
        "nnzb": nnzb, "nnzb_dense_path": dnnzb,
        "mfma_tflops": {"row_lse": pass_flops / t_lse / 1e9, "block_mass_qk": pass_flops / t_mass / 1e9,
                        "lse_block_mass_qk": pass_flops / t_one / 1e9,
                        "topp_select_bsr_qk": gather_flops / t_sel / 1e9},
        "mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS,
        "exp_per_s": {"row_lse": H_s * causal_pairs / t_lse * 1e3,
                      "block_mass_qk": H_s * causal_pairs / t_mass * 1e3},
    }


def fanout_leg(dev, w, layers, reps):
    """One sender state feeding two receivers: the BSR states of the step's
    layers (14B->8B-like sender, N = 8192, B = 64, H_s = 40, bf16) feed the
    8B-like receiver of the workload (H_r = 32, H_kv = 8) and a second,
    1.7B-like receiver (H_r = 16, H_kv = 8; W ~ N(0, 1/H_s), V ~ N(0, 1),
    seeded).  HIP events per layer, medians over `reps` passes over all layers:
    one joint launch (mf_retrieve_fused_multi) against the two receivers'
    launches back to back.  Algorithmic bytes of the pair: the kept tiles once,
    both receivers' V and O, indices and both head maps."""
    import torch
    import cross_model_sparse_amd as mf
    import synth
    wb = w.with_(H_r=16, H_kv=8)
    B, e = w.B, synth.DTYPE_BYTES[w.dtype]
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    recv_b = [(synth.gen_W(wb, 8100 + i).to(dev), synth.gen_V(wb, 8100 + i).to(dev))
              for i in range(len(layers))]
    O_a = torch.empty(w.N, w.H_r, w.d, dtype=synth.torch_dtype(w.dtype), device=dev)
    O_b = torch.empty(w.N, wb.H_r, w.d, dtype=synth.torch_dtype(w.dtype), device=dev)

    def joint(x, rb):
        mf.retrieve_fused_multi(x["rp"], x["ci"], x["vals"], x["nnzb"], [(x["W"], x["V"]), rb],
                                w.N, B, outs=[O_a, O_b])

    def separate(x, rb):
        mf.retrieve_fused(x["rp"], x["ci"], x["vals"], x["nnzb"], x["W"], x["V"], w.N, B, out=O_a)
        mf.retrieve_fused(x["rp"], x["ci"], x["vals"], x["nnzb"], rb[0], rb[1], w.N, B, out=O_b)

    def timed(fn):
        per_rep = []
        for rep in range(reps + 1):
            evs = []
            for x, rb in zip(layers, recv_b):
                a, b = ev(), ev()
                a.record(stream)
                fn(x, rb)
                b.record(stream)
                evs.append((a, b))
            torch.cuda.synchronize()
            if rep:
                per_rep.append(sum(a.elapsed_time(b) for a, b in evs) / len(layers))
        return float(np.median(per_rep))

    t_joint = timed(joint)
    t_sep = timed(separate)
    nz = float(np.mean([x["nnzb"] for x in layers]))
    T = w.T
    alg = (nz * w.H_s * B * B * e + w.N * (w.H_kv + wb.H_kv) * w.d * e
           + w.N * (w.H_r + wb.H_r) * w.d * e + 4 * (T + 1 + nz) + 4 * (w.H_r + wb.H_r) * w.H_s)
    return {
        "workload": f"pair14b8b-bf16 sender states ({len(layers)} layers, N={w.N}, B={B}, H_s={w.H_s}) "
                    f"feeding receivers (H_r={w.H_r}, H_kv={w.H_kv}) and (H_r={wb.H_r}, H_kv={wb.H_kv}), d={w.d}",
        "ms_per_layer": {"joint_launch": t_joint, "two_launches": t_sep},
        "query_tokens_per_s_per_layer_both_receivers": {"joint_launch": w.N / t_joint * 1e3,
                                                        "two_launches": w.N / t_sep * 1e3},
        "roofline_joint": {"bound": "hbm", "bytes": alg, "achieved": alg / t_joint / 1e6,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": alg / t_joint / 1e6 / HBM_PEAK_GBS},
    }


def cache_leg(dev, w, layers, reps):
    """The Block Manager on the step's BSR states: every full block row of all
    layers (N = 8192 tokens, 128 rows per layer, seeded token ids) is inserted
    into one manager over a tile pool sized for them, the tiles are copied into
    their pages (mf_pool_store, HIP events; timed on the pool's first touch and
    again on pages already written once), and the whole prefix is then looked
    up and released for every layer (host wall time per call).  Layer 0 is then
    retrieved from the pool through the block table and from its own BSR
    state (HIP events, medians over `reps`)."""
    import torch
    import cross_model_sparse_amd as mf
    B, N, T = w.B, w.N, w.T
    e = 2
    tokens = np.random.default_rng(17).integers(0, 151_000, size=N).astype(np.int32)
    total = int(sum(x["nnzb"] for x in layers))
    pool = torch.empty(total, w.H_s, B, B, dtype=layers[0]["vals"].dtype, device=dev)
    bm = mf.BlockManager(B, len(layers), total, seed=1)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    host = [(x["rp"].cpu().numpy(), x["ci"][: x["nnzb"]].cpu().numpy()) for x in layers]
    t_ins, t_store, pages_l0, pages_all = 0.0, 0.0, None, []
    for l, (x, (rp, ci)) in enumerate(zip(layers, host)):
        t0 = time.perf_counter()
        pages = bm.insert(l, tokens, 0, rp, ci)
        t_ins += time.perf_counter() - t0
        pg = torch.from_numpy(pages).to(dev)
        a, b = ev(), ev()
        a.record(stream)
        mf.pool_store(x["vals"][: x["nnzb"]], pg, pool)
        b.record(stream)
        b.synchronize()
        t_store += a.elapsed_time(b) / 1e3
        if l == 0:
            pages_l0 = pg
        pages_all.append(pg)
    # the same copies again: pages already touched once (steady state of a
    # pool whose pages are reused after eviction)
    t_store_warm = 0.0
    for x, pg in zip(layers, pages_all):
        a, b = ev(), ev()
        a.record(stream)
        mf.pool_store(x["vals"][: x["nnzb"]], pg, pool)
        b.record(stream)
        b.synchronize()
        t_store_warm += a.elapsed_time(b) / 1e3
    t_look = 0.0
    for l in range(len(layers)):
        t0 = time.perf_counter()
        rp_c, ci_c, pg_c = bm.lookup(l, tokens)
        bm.release(l, tokens, len(rp_c) - 1)
        t_look += time.perf_counter() - t0
        assert len(rp_c) - 1 == T
    rows = T * len(layers)
    x = layers[0]
    cu = torch.tensor([0, N], dtype=torch.int32, device=dev)
    cr = torch.tensor([0, T], dtype=torch.int32, device=dev)
    O = torch.empty_like(x["O"])

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_pool = timed(lambda: mf.retrieve_fused_varlen(cu, cr, x["rp"], x["ci"], pool, x["nnzb"], x["W"],
                                                    x["V"], B, block_table=pages_l0, out=O))
    t_own = timed(lambda: mf.retrieve_fused(x["rp"], x["ci"], x["vals"], x["nnzb"], x["W"], x["V"],
                                            N, B, out=O))
    st = bm.stats()
    bm.close()
    store_bytes = 2 * total * w.H_s * B * B * e
    return {
        "workload": f"pair14b8b-bf16: {len(layers)} layers x {T} block rows of {B} tokens, "
                    f"{total} kept blocks in one pool ({total * w.H_s * B * B * e / 1e9:.2f} GB)",
        "host_us_per_row": {"insert": t_ins / rows * 1e6, "lookup_and_release": t_look / rows * 1e6},
        "pool_store": {"ms_per_layer": t_store_warm / len(layers) * 1e3,
                       "achieved_GBs": store_bytes / t_store_warm / 1e9,
                       "frac_of_hbm_peak": store_bytes / t_store_warm / 1e9 / HBM_PEAK_GBS,
                       "first_touch_ms_per_layer": t_store / len(layers) * 1e3,
                       "first_touch_GBs": store_bytes / t_store / 1e9},
        "retrieve_layer0_ms": {"from_pool_via_block_table": t_pool, "from_own_bsr": t_own},
        "manager_stats": st,
    }


def varlen_leg(dev, reps):
    """The packed varlen batch: 16 sequences, lengths U[1024, 16384] (seeded),
    B = 64, H_s = 32, H_r = 24, H_kv = 8, d = 128, bf16, p = 0.9, structured
    maps.  Each sequence's dense map is generated, compressed (block mass +
    Top-p/BSR into buffers allocated once for the longest sequence, HIP
    events) and freed in turn; the kept tiles of all sequences
    then sit in one pool in a shuffled page order.  Timed with HIP events
    (medians over `reps`): the whole batch's retrieval in one launch through
    the block table, the same over a contiguous pool without a table, and one
    retrieval launch per sequence."""
    import torch
    import cross_model_sparse_amd as mf
    import synth
    w0 = synth.workload("varlen-bf16")
    lens = synth.varlen_lengths(w0)
    B, p, e = w0.B, w0.p, synth.DTYPE_BYTES[w0.dtype]
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # compression buffers sized once for the longest sequence, as a serving
    # loop holds them: workspaces, masses and a BSR of full causal capacity
    Tm = -(-max(lens) // B)
    cap_m = Tm * (Tm + 1) // 2
    ws_bm = torch.empty(mf.block_mass_ws_bytes(w0.H_s, max(lens), B), dtype=torch.uint8, device=dev)
    ws_tp = torch.empty(mf.topp_workspace_bytes(max(lens), B), dtype=torch.uint8, device=dev)
    mass_b = torch.empty(Tm * Tm, dtype=torch.float32, device=dev)
    rp_b = torch.empty(Tm + 1, dtype=torch.int32, device=dev)
    ci_b = torch.empty(cap_m, dtype=torch.int32, device=dev)
    vals_b = torch.empty(cap_m, w0.H_s, B, B, dtype=synth.torch_dtype(w0.dtype), device=dev)
    seqs, W, t_comp = [], None, 0.0
    for s, n in enumerate(lens):
        g = synth.gen_layer(w0.with_(N=n), device=dev, seed=5000 + s)
        if W is None:
            W = g["W"].to(dev)
        A = g["A"]
        T = -(-n // B)
        mass = mass_b[: T * T].view(T, T)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        mf.block_mass(A, B, out=mass, workspace=ws_bm)
        mf.topp_select_bsr(mass, A, B, p, cap_nnzb=T * (T + 1) // 2, row_ptr=rp_b[: T + 1],
                           col_idx=ci_b, vals=vals_b, workspace=ws_tp, sync=False)
        b.record(stream)
        b.synchronize()
        t_comp += a.elapsed_time(b)
        nnzb = int(rp_b[T].item())
        seqs.append(dict(N=n, rp=rp_b[: T + 1].clone(), ci=ci_b[:nnzb].clone(),
                         vals=vals_b[:nnzb].clone(), nnzb=nnzb, V=g["V"].to(dev)))
        del A, g
    del vals_b, ci_b, ws_bm, ws_tp
    torch.cuda.empty_cache()
    S = len(seqs)
    Ts = [-(-n // B) for n in lens]
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    cu, cr = i32(np.cumsum([0] + lens).tolist()), i32(np.cumsum([0] + Ts).tolist())
    offs = np.cumsum([0] + [x["nnzb"] for x in seqs])
    row_ptr = torch.cat([torch.zeros(1, dtype=torch.int32, device=dev)] +
                        [x["rp"][1:] + int(o) for x, o in zip(seqs, offs)])
    col_idx = torch.cat([x["ci"] for x in seqs])
    contig = torch.cat([x["vals"] for x in seqs])
    nnzb = int(offs[-1])
    perm = torch.from_numpy(np.random.default_rng(0).permutation(nnzb)).to(dev)
    pool = torch.empty_like(contig)
    pool[perm] = contig
    table = perm.to(torch.int32)
    V = torch.cat([x["V"] for x in seqs])
    O = torch.empty(V.shape[0], w0.H_r, w0.d, dtype=V.dtype, device=dev)
    Os = [torch.empty(x["N"], w0.H_r, w0.d, dtype=V.dtype, device=dev) for x in seqs]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_tab = timed(lambda: mf.retrieve_fused_varlen(cu, cr, row_ptr, col_idx, pool, nnzb, W, V, B,
                                                   block_table=table, out=O))
    t_con = timed(lambda: mf.retrieve_fused_varlen(cu, cr, row_ptr, col_idx, contig, nnzb, W, V, B,
                                                   out=O))

    def per_seq():
        for x, o in zip(seqs, Os):
            mf.retrieve_fused(x["rp"], x["ci"], x["vals"], x["nnzb"], W, x["V"], x["N"], B, out=o)
    t_seq = timed(per_seq)
    tokens = int(sum(lens))
    alg = sum(x["nnzb"] * w0.H_s * B * B * e + x["N"] * w0.H_kv * w0.d * e
              + x["N"] * w0.H_r * w0.d * e + 4 * (T + 1 + x["nnzb"]) for x, T in zip(seqs, Ts))
    alg += 4 * w0.H_r * w0.H_s + 8 * (S + 1)
    alg_tab = alg + 4 * nnzb
    return {
        "workload": f"varlen-bf16: {S} sequences, lengths U[1024, 16384] (total {tokens} tokens), "
                    f"B={B}, H_s={w0.H_s}, H_r={w0.H_r}, H_kv={w0.H_kv}, d={w0.d}, bf16, p={p}",
        "lengths": lens,
        "nnzb_total": nnzb,
        "ms": {"one_launch_paged_pool": t_tab, "one_launch_contiguous_pool": t_con,
               "one_launch_per_sequence": t_seq, "compress_all_sequences": t_comp},
        "query_tokens_per_s": {"one_launch_paged_pool": tokens / t_tab * 1e3,
                               "one_launch_contiguous_pool": tokens / t_con * 1e3,
                               "one_launch_per_sequence": tokens / t_seq * 1e3,
                               "compress_plus_one_launch": tokens / (t_comp + t_tab) * 1e3},
        "roofline_one_launch_paged": {"bound": "hbm", "bytes": alg_tab,
                                      "achieved": alg_tab / t_tab / 1e6, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": alg_tab / t_tab / 1e6 / HBM_PEAK_GBS},
    }


def cpu_model():
    """The host CPU's model name (lscpu's "Model name", read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_leg(w, layers, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of block rows: every
    block row of layer 0 from the last, then layer 1, ... (the same device
    tensors, copied to the host row by row) until about `budget_s` seconds of
    oracle work.  The rate counts the oracle's retrieval time only, like the
    GPU metric; the compression time is reported beside it."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the visible cores
        blas_threads = os.cpu_count()
    N, B, T = w.N, w.B, w.T
    t_comp = t_retr = 0.0
    rows = blocks = 0
    used_layers = 0
    for layer in layers:
        A = layer["A"]
        W = layer["W"].cpu().numpy()
        V = layer["V"].float().cpu().numpy()

        class RowSlab:
            shape = tuple(A.shape)

            def __getitem__(self, idx):
                return A[idx].float().cpu().numpy()

        view = RowSlab()
        used_layers += 1
        for I in range(T - 1, -1, -1):
            c0 = time.perf_counter()
            m = oracle.block_mass_row(view, B, I)
            kept = oracle.topp_row(oracle.decision_masses(m), w.p)
            tiles = [oracle.bsr_tile(view, B, I, int(J)) for J in kept]
            c1 = time.perf_counter()
            oracle.retrieve_row(I, kept, tiles, W, V, N, B)
            c2 = time.perf_counter()
            t_comp += c1 - c0
            t_retr += c2 - c1
            rows += 1
            blocks += len(kept)
            if t_comp + t_retr > budget_s:
                break
        if t_comp + t_retr > budget_s:
            break
    tokens = rows * B
    return {"value": tokens / t_retr, "unit": "query-tokens/s per layer",
            "cores": int(blas_threads), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": (f"{rows} block rows ({tokens} query tokens, {blocks} kept blocks) from "
                       f"{used_layers} layer(s), last row first; oracle retrieval "
                       f"{t_retr:.1f} s, oracle compression (host copy + block mass + Top-p "
                       f"+ tile gather) {t_comp:.1f} s; host cpu_count {os.cpu_count()}")}


if __name__ == "__main__":
    main()
