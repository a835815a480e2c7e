#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer over the cross-layer LRU slot cache on one MI355X.

Workload (default): Qwen3.6-35B-A3B-shaped decode — 40 MoE layers, 256 routed experts
top-8 plus one shared expert, hidden 2048, expert intermediate 512, MXFP4 experts,
bf16 activations, batch 1, cross-layer LRU pool of 600 of the 10240 (layer, expert)
slots, routing locality p = 0.8, seeded synthetic weights / trace / activations.

A step is one decode token through all 40 layers: per layer moe_route ->
slot_cache_lookup_evict -> mc_fill_slots (misses from pinned host memory over the
host link) -> moe_experts_decode -> mc_finish_bf16, all captured in one hipGraph.
Inputs (router logits, activations, the pinned host expert pool) are resident
before the timed region starts; the fills are part of the path.

Printed: one JSON line (value = decode tokens/s).  ``roofline`` is for the expert
GEMV (moe_experts_decode), timed with HIP events on its own stream over graph
replays of the same calls the steps make; ``cpu_baseline`` times the CPU oracle on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 63.0       # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes, 128b/130b encoding
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic_pmc.txt")
# kernels of each measured entry point and the source file they are built from
TRAFFIC_KERNELS = {
    # one token (the headline pass): the dot-product kernels
    "moe_experts_decode": ("decode.hip", ("gate_up_tok1_kernel", "down_tok1_kernel", "down_tok1b_kernel")),
    # several tokens (the pmc workload's batched pass): the matrix-core kernels
    "moe_experts_decode_batched": ("decode.hip", ("gate_up_kernel", "down_unit_kernel")),
    "moe_experts_prefill": ("prefill.hip", ("sort_count_kernel", "sort_plan_kernel", "sort_scatter_kernel",
                                            "prefill_gemm_kernel", "prefill_combine_kernel")),
}
METRIC = "MoE-layer decode tok/s (bs=1) + prefill tok/s at 8k; HBM GB/s & MFMA % peak"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--cpu-tokens", type=int, default=2, help="decode tokens in the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill part (for profiling); prints its objects alone")
    ap.add_argument("--prefill-resident-only", action="store_true",
                    help="prefill: time only the resident layer (no serialized / double-buffered passes)")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run only the workload the HBM traffic counters are taken on, then exit")
    ap.add_argument("--pmc-batch", type=int, default=16, help="tokens of the counter workload's batched pass")
    ap.add_argument("--pmc-table", metavar="CSV",
                    help="print the per-dispatch average of every counter in a rocprofv3 counter CSV, per "
                         "kernel of the library, then exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic table from two rocprofv3 --pmc counter CSVs, then exit")
    ap.add_argument("--c5-sweep", action="store_true",
                    help="run only the batched Zipf decode sweep (bs 1/4/16 x pools 256..4096 slots, one "
                         "process, the pool resized between points) and print its table")
    ap.add_argument("--c5-steps", type=int, default=48, help="timed steps per sweep point")
    ap.add_argument("--c3", action="store_true",
                    help="DeepSeek-V4-Flash-shaped hybrid decode (43 layers, 1500 slots, pinned pool of "
                         "all 11008 experts): q* splits for B_H/B_P in {1.5, 2, 3} x locality {0.5, 0.9}, "
                         "and the split from this machine's bandwidth profile")
    ap.add_argument("--c3-steps", type=int, default=48, help="timed steps per C3 run")
    ap.add_argument("--c3-layers", type=int, default=16,
                    help="layers of the C3 pool actually built (the box pins at most 64 GiB; the slot "
                         "pool is scaled to the same share of the experts)")
    ap.add_argument("--fill-mode", choices=("copy", "through", "split", "fused"), default="fused",
                    help="how misses reach their slots: copy (mc_fill_slots first), through (the expert "
                         "pass reads the host and writes the slots), split (gate_up through, down banks "
                         "copied on a side stream), fused (gate_up through, down banks copied by "
                         "workgroups of the same launch)")
    return ap.parse_args()


def _src_sha(name):
    """Hash of a kernel source file together with every header of the library's sources."""
    import glob
    import hashlib
    d = os.path.join(HERE, "expert_cache_offloaded_amd", "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(d, name)] + sorted(glob.glob(os.path.join(d, "*.h"))):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes(entry):
    """HBM bytes per call of `entry` from the committed counter table, or None when the
    table is missing or its kernels' source has changed since the counters were taken."""
    src = TRAFFIC_KERNELS[entry][0]
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                p = line.split()
                if len(p) == 6 and p[0] == "traffic" and p[1] == entry:
                    if p[2] != src or p[3] != _src_sha(src):
                        return None
                    return int(p[4].split("=")[1]) + int(p[5].split("=")[1])
    except OSError:
        return None
    return None


def pmc_summary(fetch_csv, write_csv, batch=16):
    """Traffic table from FETCH_SIZE / WRITE_SIZE runs of --pmc-workload.  Each counter
    is scaled by what it reads for the workload's 256 MiB device copy (rocclr copy
    kernel dispatches of known size)."""
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
                acc[name].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    # the commands are printed with the directories the two counter files came from
    dir_f, dir_w = os.path.dirname(fetch_csv) or ".", os.path.dirname(write_csv) or "."
    print("# HBM traffic per dispatch from rocprofv3 counters on MI355X (ROCm 7.2), made by:")
    print("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s -o run -- "
          "python3 -u bench.py --pmc-workload" % dir_f)
    print("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s -o run -- "
          "python3 -u bench.py --pmc-workload" % dir_w)
    print("#   python3 bench.py --pmc-summary %s %s" % (fetch_csv, write_csv))
    print("# 'traffic' lines: calibrated bytes per call of each entry point, keyed by the sha256 "
          "prefix of the kernel source they were taken on (bench.py reports null once it changes).")
    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, _ = per_kernel(write_csv, "WRITE_SIZE")
    copy = "__amd_rocclr_copyBuffer"
    chunk_kib = (256 << 10) / nf[copy] * 3     # 3 copies of 256 MiB over nf dispatches
    f_fac, w_fac = chunk_kib / fetch[copy], chunk_kib / write[copy]
    print("# calibration: 256 MiB device copy in %d dispatches of %.0f KiB: FETCH_SIZE %.1f KiB, "
          "WRITE_SIZE %.1f KiB per dispatch -> factors %.4f (fetch), %.4f (write)"
          % (nf[copy], chunk_kib, fetch[copy], write[copy], f_fac, w_fac))
    print("# %-44s %12s %12s %14s %14s" % ("kernel", "FETCH KiB", "WRITE KiB", "read bytes", "write bytes"))
    rows = {}
    for k in sorted(fetch):
        rb, wb = fetch[k] * 1024 * f_fac, write.get(k, 0.0) * 1024 * w_fac
        rows[k] = (rb, wb)
        print("# %-44s %12.1f %12.1f %14.0f %14.0f" % (k[:44], fetch[k], write.get(k, 0.0), rb, wb))
    algo = pmc_algorithmic(batch)
    print("# batched pass: %d tokens; algorithmic bytes per call (distinct experts + shared, each read once):"
          % batch)
    for entry, (src, kernels) in TRAFFIC_KERNELS.items():
        mine = [k for k in rows if any(k == "mc::" + n or k.startswith("mc::" + n + "<") for n in kernels)]
        rb, wb = sum(rows[k][0] for k in mine), sum(rows[k][1] for k in mine)
        if entry in algo:
            print("#   %-28s algorithmic %12.0f  read %12.0f  read / algorithmic %.3f"
                  % (entry, algo[entry], rb, rb / algo[entry]))
        print("traffic %s %s %s fetch_bytes=%d write_bytes=%d" % (entry, src, _src_sha(src), rb, wb))


def pmc_table(path):
    """Per-dispatch averages of every counter of a rocprofv3 counter CSV, per library
    kernel (and the derived MFMA-busy and wave-occupancy ratios where their counters are
    present)."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
            if not name.startswith("mc::"):
                continue
            acc[name][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[name].add(r["Dispatch_Id"])
    for name in sorted(acc):
        n = len(disp[name])
        c = {k: v / n for k, v in acc[name].items()}
        print("%s  (%d dispatches)" % (name, n))
        for k in sorted(c):
            print("    %-30s %16.1f" % (k, c[k]))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "SQ_BUSY_CU_CYCLES" in c and c["SQ_BUSY_CU_CYCLES"] > 0:
            print("    %-30s %16.4f" % ("MFMA busy / CU busy", c["SQ_VALU_MFMA_BUSY_CYCLES"] / c["SQ_BUSY_CU_CYCLES"]))


def pmc_calls(n, k, T, count=20, seed=0):
    """Slot lists of the counter workload's expert passes: T tokens x k distinct slots of
    n resident experts each (seeded, so the summary recomputes the same lists)."""
    r = np.random.default_rng(seed + T)
    return [np.stack([r.choice(n, k, replace=False) for _ in range(T)]).astype(np.int32) for _ in range(count)]


def pmc_algorithmic(batch):
    """Algorithmic bytes per call of the workload's passes: the distinct experts' weights
    (plus the shared expert), each read once."""
    import synth
    cfg = synth.CONFIGS["qwen_decode"]
    eb = synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)
    out = {}
    for name, T in (("moe_experts_decode", 1), ("moe_experts_decode_batched", batch)):
        calls = pmc_calls(64, cfg.k, T)
        out[name] = float(np.mean([len(np.unique(c)) + 1 for c in calls])) * eb
    return out


def pmc_workload(batch=16):
    """What the traffic counters are taken on: a 256 MiB device copy (calibration), 20
    Qwen-shaped expert passes over resident experts (8 routed + shared) at bs 1 and 20 at
    bs `batch`, and one 8192-token prefill layer (E 256, top-6, H 4096, I 2048)."""
    import torch

    import synth
    from expert_cache_offloaded_amd import _lib as L
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    a.fill_(3)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    cfg = synth.CONFIGS["qwen_decode"]
    n = 64
    pool_np = synth.host_pool(cfg.with_(L=1, E=n))
    pool = {k: torch.from_numpy(v).cuda() for k, v in pool_np.items()}
    sh = {k: torch.from_numpy(v).cuda() for k, v in synth.shared_pool(cfg.with_(L=1)).items()}
    pb, sb = L.make_banks(cfg.fmt, cfg.H, cfg.I, pool), L.make_banks(cfg.fmt, cfg.H, cfg.I, sh)
    for T in (1, batch):
        x = torch.from_numpy(synth.activations(cfg.with_(T=T), 0).view(np.int16)).cuda()
        w = torch.full((T, cfg.k), 0.125, dtype=torch.float32, device="cuda")
        ws = torch.zeros(L.decode_ws_bytes(T, cfg.k, cfg.H, cfg.I), dtype=torch.uint8, device="cuda")
        y = torch.zeros((T, cfg.H), dtype=torch.float32, device="cuda")
        for c in pmc_calls(n, cfg.k, T):
            L.moe_experts_decode(x, torch.from_numpy(c).cuda(), w, None, pb, sb, ws, y, accumulate=1)
        torch.cuda.synchronize()
    del pool
    cfg = synth.CONFIGS["prefill"]
    T, E, k, H, I = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I
    from expert_cache_offloaded_amd.runtime import alloc_banks
    bt = alloc_banks(E, H, I, cfg.fmt, pin=True)
    fill_host_pool(cfg.with_(L=1), bt)
    dev = {k_: v.cuda() for k_, v in bt.items()}
    buf = L.make_banks(cfg.fmt, H, I, dev)
    xp = torch.from_numpy(synth.activations(cfg, 0).view(np.int16)).cuda()
    lg = torch.from_numpy(synth.uniform_logits(cfg)).cuda()
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wp = torch.empty((T, k), dtype=torch.float32, device="cuda")
    L.moe_route(lg, k, 1, ids, wp)
    wsp = torch.empty(L.prefill_ws_bytes(T, k, E, H, I), dtype=torch.uint8, device="cuda")
    yp = torch.empty((T, H), dtype=torch.int16, device="cuda")
    L.moe_experts_prefill(xp, ids, wp, None, E, buf, wsp, yp)
    torch.cuda.synchronize()
    print("pmc workload done", flush=True)


def random_pool(n, H, I, torch, seed=1):
    """n MXFP4 experts of random codes with block scales 2^-9 .. 2^-4 (device), for
    timing passes whose outputs are not checked."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = {"gate_up": torch.randint(0, 256, (n, 2 * I, H // 2), dtype=torch.uint8, device="cuda", generator=g),
         "gate_up_scale": torch.randint(118, 124, (n, 2 * I, H // 32), dtype=torch.uint8, device="cuda", generator=g),
         "down": torch.randint(0, 256, (n, H, I // 2), dtype=torch.uint8, device="cuda", generator=g),
         "down_scale": torch.randint(118, 124, (n, H, I // 32), dtype=torch.uint8, device="cuda", generator=g)}
    return t


def time_pass(torch, L, H, I, k, T, calls, pool, shared, reps=5):
    """Median µs per moe_experts_decode call over graph replays of `calls` (slot arrays
    [T, k]) back to back, HIP events on the replay stream."""
    x = torch.randint(-3000, 3000, (T, H), dtype=torch.int16, device="cuda")
    w = torch.full((T, k), 0.125, dtype=torch.float32, device="cuda")
    ws = torch.zeros(L.decode_ws_bytes(T, k, H, I), dtype=torch.uint8, device="cuda")
    slots = [torch.from_numpy(c).cuda() for c in calls]
    ys = [torch.zeros((T, H), dtype=torch.float32, device="cuda") for _ in calls]
    for c in range(len(calls)):
        L.moe_experts_decode(x, slots[c], w, None, pool, shared, ws, ys[c], accumulate=0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            for c in range(len(calls)):
                L.moe_experts_decode(x, slots[c], w, None, pool, shared, ws, ys[c], accumulate=0)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    st = torch.cuda.current_stream()
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return 1000.0 * float(np.median(ts)) / (reps * len(calls))


def expert_pass_rooflines(torch, L, synth):
    """The expert pass (moe_experts_decode) at the other decode shapes, against 8 TB/s:
    DeepSeek-V4-Flash-shaped bs 1 (6 routed experts of H 4096 x I 2048, no shared) and
    Qwen-shaped bs 4 and bs 16 under Zipf(1.1) routing (8 routed + shared, H 2048 x
    I 512).  Bytes are the distinct experts' weights (each read once)."""
    out = {}
    r = np.random.default_rng(0)
    H, I, k = 4096, 2048, 6
    pt = random_pool(24, H, I, torch)
    pool = L.make_banks("mxfp4", H, I, pt)
    calls = [r.choice(24, k, replace=False).astype(np.int32)[None] for _ in range(40)]
    us = time_pass(torch, L, H, I, k, 1, calls, pool, None)
    b = k * synth.expert_bytes(H, I, "mxfp4")
    out["dsv4_bs1"] = {"us_per_call": round(us, 2), "bytes_per_call": int(b), "gbs": round(b / us * 1e-3, 1),
                       "frac": round(b / us * 1e-3 / HBM_PEAK_GBS, 4), "units": k}
    del pt, pool
    torch.cuda.empty_cache()
    H, I, k = 2048, 512, 8
    pt = random_pool(512, H, I, torch)
    pool = L.make_banks("mxfp4", H, I, pt)
    st = random_pool(1, H, I, torch, seed=2)
    sh = L.make_banks("mxfp4", H, I, st)
    for T in (4, 16):
        calls = []
        for c in range(40):
            ids = synth.zipf_stream(256, k, T, 1.1, r.permutation(256), r)
            calls.append((ids + 256 * (c % 2)).astype(np.int32))
        units = float(np.mean([len(np.unique(c)) + 1 for c in calls]))
        us = time_pass(torch, L, H, I, k, T, calls, pool, sh)
        b = units * synth.expert_bytes(H, I, "mxfp4")
        out["qwen_bs%d" % T] = {"us_per_call": round(us, 2), "bytes_per_call": int(b),
                                "gbs": round(b / us * 1e-3, 1), "frac": round(b / us * 1e-3 / HBM_PEAK_GBS, 4),
                                "units": round(units, 2)}
    del pt, pool
    torch.cuda.empty_cache()
    return out


def tiny_layer(torch, L, synth, steps=64):
    """The tiny MoE layer (E 8 top-2, H 64, I 128, bf16 experts, 4 tokens, LRU pool of 4
    slots, locality 0.7): µs per layer call of the whole path (route + lookup + fill +
    expert pass + bf16 output) over a trace of `steps` calls in one graph."""
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer, alloc_banks
    cfg = synth.CONFIGS["tiny"]
    host_t = alloc_banks(cfg.n_flat, cfg.H, cfg.I, cfg.fmt, pin=True)
    fill_host_pool(cfg, host_t)
    host = BankSet(host_t, cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(cfg.S, cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    cache = CacheState(cfg.L, cfg.E, cfg.S)
    cache.reset()
    tr = synth.trace(cfg, steps=steps)
    lg = torch.from_numpy(np.stack([synth.step_logits(cfg, tr[s], s)[0] for s in range(steps)])).cuda()
    xs = torch.from_numpy(np.stack([synth.activations(cfg, s, 0) for s in range(steps)]).view(np.int16)).cuda()
    # 4 slots for up to 8 distinct experts per call: overflow misses run on the host branch
    workers = L.HostPool(2)
    dl = DecodeLayer(cache, host, pool, None, DecodeBuffers(cfg.T, cfg.k, cfg.H, cfg.I), renorm=cfg.renorm,
                     hybrid=True, host_pool=workers)
    for s_ in range(steps):
        dl(0, lg[s_], xs[s_])
    torch.cuda.synchronize()
    cache.reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s_ in range(steps):
            dl(0, lg[s_], xs[s_])
    cache.reset()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    st = cache.t["stats"].cpu().numpy()
    del g, dl
    workers.close()
    return {"us_per_call": round(1000.0 * e0.elapsed_time(e1) / steps, 2), "calls": steps,
            "hits": int(st[0]), "misses": int(st[1]), "fills": int(st[2]), "host_routes": int(st[3])}


def link_roofline(torch, L, synth, cfg, host, pool, shared_desc, x, calls=20, n_fill=2):
    """The decode step's dominant kernel, the one-token gate_up launch that carries the
    fills, against the host link: graph replays of moe_experts_decode with n_fill experts
    filled in that launch (the rest of the routes resident) and with none; the time the
    fills add, per filled expert, gives the link rate the launch reaches.  The slots the
    fills write are overwritten (pool contents are not used after this point)."""
    rng = np.random.default_rng(7)
    k, dev = cfg.k, "cuda"
    S_e = synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)
    w = torch.full((1, k), 1.0 / k, dtype=torch.float32, device=dev)
    y = torch.empty((1, cfg.H), dtype=torch.float32, device=dev)
    yb = torch.empty((1, cfg.H), dtype=torch.int16, device=dev)
    ws = torch.zeros(L.decode_ws_bytes(1, k, cfg.H, cfg.I) // 4 + 4, dtype=torch.float32, device=dev)
    us = {}
    for n in (0, n_fill):
        keep = []
        for c in range(calls):
            sl = rng.choice(pool.n, k, replace=False).astype(np.int32)
            fl = np.full(k, -1, np.int32)
            fl[:n] = rng.choice(host.n, n, replace=False)
            fs = np.full(k, -1, np.int32)
            fs[:n] = sl[:n]
            ff, fsl = torch.tensor(fl, device=dev), torch.tensor(fs, device=dev)
            nf = torch.tensor([n], dtype=torch.int32, device=dev)
            keep.append((torch.tensor(sl.reshape(1, k), device=dev),
                         L.make_fill_list(host.desc, ff, fsl, nf, mode=L.MC_FILL_WITH_GATE_UP), ff, fsl, nf))

        def run():
            for slots, fill, *_ in keep:
                L.moe_experts_decode(x, slots, w, None, pool.desc, shared_desc, ws, y, 0, yb, fill=fill)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / calls)
        us[n] = float(np.median(times))
        del g
    per_expert = (us[n_fill] - us[0]) / n_fill
    achieved = S_e / (per_expert * 1e-6) / 1e9
    return {"bound": "host link", "kernel": "gate_up_fill_tok1_kernel (moe_experts_decode, MC_FILL_WITH_GATE_UP)",
            "achieved": round(achieved, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / PCIE_PEAK_GBS, 4), "us_per_filled_expert": round(per_expert, 2),
            "bytes_per_filled_expert": S_e, "us_per_call": {str(n): round(v, 2) for n, v in us.items()}}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_env():
    """Host facts for a CPU baseline: the cores this process may run on, the threads
    the oracle's array library actually uses, and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cores": min(cores, threads), "affinity_cores": cores, "cpu_model": model}


def one_core(fn):
    """fn() with the oracle's array library held to one thread; (result, seconds)."""
    t0 = time.perf_counter()
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            r = fn()
    except ImportError:
        r = fn()
    return r, time.perf_counter() - t0


def build_host_pool(cfg, torch):
    """Pinned host expert pool indexed by flat id (the host truth)."""
    import synth
    from expert_cache_offloaded_amd.runtime import alloc_banks
    banks = alloc_banks(cfg.n_flat, cfg.H, cfg.I, cfg.fmt, pin=True)
    fill_host_pool(cfg, banks)
    return banks, {k: v.numpy() for k, v in banks.items()}


def fill_host_pool(cfg, banks):
    import synth
    views = {k: v.numpy() for k, v in banks.items()}
    t0 = time.time()

    def one(f):
        for k, a in synth.expert_weights(cfg, f).items():
            views[k][f] = a if a.dtype != np.uint16 else a.view(np.int16)
        if f % 2048 == 0:
            log("host pool %d/%d experts (%.0f s)" % (f, cfg.n_flat, time.time() - t0))

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(one, range(cfg.n_flat)))
    log("host pool ready (%.0f s)" % (time.time() - t0))


def main():
    args = _parse()
    if args.pmc_table:
        pmc_table(args.pmc_table)
        return
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, batch=args.pmc_batch)
        return
    if args.pmc_workload:
        pmc_workload(args.pmc_batch)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures a single GPU: the method runs on one GPU (its expert pool, slot "
              "cache and host link); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from expert_cache_offloaded_amd import _lib as L
    from expert_cache_offloaded_amd.runtime import (BankSet, CacheState, DecodeBuffers, DecodeLayer,
                                                   alloc_banks)

    L.lib()   # fails loudly if the library is not built
    if args.c5_sweep:
        print(json.dumps({"c5_sweep": c5_sweep(args, torch, L, synth)}), flush=True)
        return
    if args.c3:
        print(json.dumps({"c3_hybrid": c3_runs(args, torch, L, synth)}), flush=True)
        return
    if args.prefill_only:
        pre, roof = bench_prefill(args, torch, L, synth)
        print(json.dumps({"prefill": pre, "roofline_prefill": roof}), flush=True)
        return
    cfg = synth.CONFIGS["qwen_decode"]
    W, K = args.warmup, args.steps
    n_steps = W + K
    dev = "cuda"

    # ------------------------------------------------------------------ inputs
    log("trace / logits / activations for %d steps" % n_steps)
    tr = synth.trace(cfg, steps=n_steps)
    logits = np.stack([synth.step_logits(cfg, tr[s], s) for s in range(n_steps)])     # [S, L, 1, E]
    xs = np.stack([np.stack([synth.activations(cfg, s, l) for l in range(cfg.L)]) for s in range(n_steps)])
    logits_all = torch.from_numpy(logits).to(dev)
    x_all = torch.from_numpy(xs.view(np.int16)).to(dev)
    log("host pool: %d experts x %d B pinned" % (cfg.n_flat, synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)))
    host_t, host_np = build_host_pool(cfg, torch)
    host = BankSet(host_t, cfg.H, cfg.I, cfg.fmt)
    sh_np = synth.shared_pool(cfg)
    shared = BankSet({k: torch.from_numpy(v if v.dtype != np.uint16 else v.view(np.int16)).to(dev)
                      for k, v in sh_np.items()}, cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(cfg.S, cfg.H, cfg.I, cfg.fmt, device=dev), cfg.H, cfg.I, cfg.fmt)
    cache = CacheState(cfg.L, cfg.E, cfg.S)
    cache.reset()
    layers = [DecodeLayer(cache, host, pool, shared, DecodeBuffers(1, cfg.k, cfg.H, cfg.I),
                          frac_q16=1 << 16, renorm=cfg.renorm, fill_mode=args.fill_mode)
              for _ in range(cfg.L)]
    logits_buf = torch.empty_like(logits_all[0])
    x_buf = torch.empty_like(x_all[0])

    def step():
        for l in range(cfg.L):
            layers[l](l, logits_buf[l], x_buf[l])

    # ------------------------------------------------------------------ warmup + capture
    log("warmup (%d steps) and graph capture" % W)
    logits_buf.copy_(logits_all[0])
    x_buf.copy_(x_all[0])
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for s in range(1, W):
        logits_buf.copy_(logits_all[s])
        x_buf.copy_(x_all[s])
        g.replay()
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ timed region
    stats0 = cache.t["stats"].cpu().numpy().copy()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in range(W, n_steps):
        logits_buf.copy_(logits_all[s])
        x_buf.copy_(x_all[s])
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    stats1 = cache.t["stats"].cpu().numpy().copy()
    d = stats1 - stats0
    ms_per_step = ms_total / K
    tok_s = 1000.0 / ms_per_step
    S_e = synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)
    miss_rate = float(d[1]) / max(1.0, float(d[0] + d[1]))
    link_gbs = float(d[2]) * S_e / (ms_total * 1e-3) / 1e9
    log("decode: %.3f ms/token, %.1f tok/s, miss rate %.3f, %.1f fills/token, link %.1f GB/s"
        % (ms_per_step, tok_s, miss_rate, d[2] / K, link_gbs))

    # ------------------------------------------------------------------ expert GEMV timing
    # the same moe_experts_decode calls as the last step (all routes resident), replayed
    # back to back in a graph; HIP events on the replay stream.
    reps = args.kernel_reps
    ys = [torch.zeros((1, cfg.H), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
    gk = torch.cuda.CUDAGraph()
    sh_descs = [shared.entry(l).desc for l in range(cfg.L)]
    with torch.cuda.graph(gk):
        for _ in range(reps):
            for l in range(cfg.L):
                b = layers[l].b
                L.moe_experts_decode(x_buf[l], b.slots, b.w, None, pool.desc, sh_descs[l], b.ws, ys[l],
                                     accumulate=1)
    gk.replay()
    torch.cuda.synchronize()
    times = []
    stream = torch.cuda.current_stream()
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        gk.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    us_per_call = 1000.0 * float(np.median(times)) / (reps * cfg.L)
    units = []
    for l in range(cfg.L):
        sl = layers[l].b.slots.cpu().numpy().ravel()
        units.append(len(set(int(v) for v in sl if v >= 0)) + 1)       # + shared expert
    bytes_per_call = float(np.mean(units)) * S_e
    achieved = bytes_per_call / (us_per_call * 1e-6) / 1e9
    log("expert GEMV: %.2f us/call, %.2f MB/call, %.0f GB/s" % (us_per_call, bytes_per_call / 1e6, achieved))

    out = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "qwen3.6-35b-a3b-shaped decode: 40 MoE layers, E=256 top-8 + 1 shared, "
                               "H=2048, I=512, MXFP4 experts, bf16 activations, bs=1, LRU pool 600 of "
                               "10240 slots, locality p=0.8",
                   "global_batch": 1, "layers": cfg.L, "slots": cfg.S, "locality": cfg.p},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_bytes("moe_experts_decode"),
                     "kernel": "moe_experts_decode", "bytes_per_launch": int(bytes_per_call),
                     "us_per_launch": round(us_per_call, 3)},
        "decode": {"miss_rate": round(miss_rate, 4), "fills_per_token": round(float(d[2]) / K, 2),
                   "host_routes": int(d[3]), "link_gbs": round(link_gbs, 2),
                   "expert_gemv_us_per_token": round(us_per_call * cfg.L, 2),
                   "wall_s": round(wall, 3)},
    }

    # ------------------------------------------------------------------ dominant kernel vs the host link
    out["roofline_link"] = link_roofline(torch, L, synth, cfg, host, pool, shared.entry(0).desc, x_buf[0])
    log("gate_up launch with fills: %.2f us per filled expert -> %.1f GB/s (%.3f of %.0f GB/s)"
        % (out["roofline_link"]["us_per_filled_expert"], out["roofline_link"]["achieved"],
           out["roofline_link"]["frac"], PCIE_PEAK_GBS))

    # ------------------------------------------------------------------ other decode shapes
    log("expert pass at the other decode shapes")
    out["expert_pass"] = expert_pass_rooflines(torch, L, synth)
    for name, v in out["expert_pass"].items():
        log("expert pass %s: %.2f us/call, %.0f GB/s (%.3f of 8 TB/s)" % (name, v["us_per_call"], v["gbs"], v["frac"]))
    out["tiny_layer"] = tiny_layer(torch, L, synth)
    log("tiny layer: %.2f us per layer call" % out["tiny_layer"]["us_per_call"])

    # ------------------------------------------------------------------ bandwidth profile
    # the start-up profile of the two miss paths on this machine (link gather vs host
    # expert kernel, alone and overlapped) -> fetched fraction and backend choice
    workers = L.HostPool(min(16, len(os.sched_getaffinity(0))))
    prof = L.bandwidth_profile(host.desc, pool.desc, workers, 8, seconds=1.0)
    workers.close()
    prof["workers"] = workers.n_threads
    log("bandwidth profile: link %.1f GB/s, host experts %.1f GB/s (overlapped %.1f / %.1f) -> "
        "fetch fraction %.3f, %s" % (prof["pcie_gbs"], prof["cpu_gbs"], prof["pcie_ov_gbs"],
                                     prof["cpu_ov_gbs"], prof["frac_q16"] / 65536.0, prof["backend"]))
    out["bandwidth_profile"] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in prof.items()}

    # ------------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, tr, logits, xs, host_np, sh_np, args.cpu_tokens)

    # ------------------------------------------------------------------ prefill
    if not args.no_prefill:
        del host_t, host_np, host, layers, pool, cache, shared
        torch.cuda.empty_cache()
        pre, roof = bench_prefill(args, torch, L, synth)
        out["prefill"] = pre
        out["roofline_prefill"] = roof
    print(json.dumps(out), flush=True)


def c5_sweep(args, torch, L, synth):
    """Batched decode with skew (40 layers, E=256 top-8, H=2048, I=512, MXFP4, Zipf(1.1)
    expert popularity): bs in {1, 4, 16} x LRU pools of {256, 512, 1024, 2048, 4096} slots
    in one process; between points the pool is resized at a safe point (the cache
    restarts cold) and the same steps are replayed as one captured graph per step."""
    from expert_cache_offloaded_amd.runtime import (BankSet, CacheState, DecodeBuffers, DecodeLayer,
                                                   alloc_banks, resize_pool)
    cfg = synth.CONFIGS["zipf_decode"]
    sizes = (256, 512, 1024, 2048, 4096)
    W, K = 16, args.c5_steps
    log("c5: host pool %d experts" % cfg.n_flat)
    host_t, _ = build_host_pool(cfg, torch)
    host = BankSet(host_t, cfg.H, cfg.I, cfg.fmt)
    S_e = synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)
    out = []
    for bs in (1, 4, 16):
        c = cfg.with_(T=bs)
        tr = synth.trace(c, steps=W + K)
        logits = torch.from_numpy(np.stack([synth.step_logits(c, tr[s], s) for s in range(W + K)])).cuda()
        xs = torch.from_numpy(np.stack([np.stack([synth.activations(c, s, l, T=bs) for l in range(c.L)])
                                        for s in range(W + K)]).view(np.int16)).cuda()
        pool = BankSet(alloc_banks(sizes[0], c.H, c.I, c.fmt, device="cuda"), c.H, c.I, c.fmt)
        cache = CacheState(c.L, c.E, sizes[0])
        cache.reset()
        layers = [DecodeLayer(cache, host, pool, None, DecodeBuffers(bs, c.k, c.H, c.I), renorm=c.renorm)
                  for _ in range(c.L)]
        lg_buf, x_buf = torch.empty_like(logits[0]), torch.empty_like(xs[0])

        def step():
            for l in range(c.L):
                layers[l](l, lg_buf[l], x_buf[l])
        for i, S in enumerate(sizes):
            if i:
                del pool
                cache, pool = resize_pool(layers, S)
            lg_buf.copy_(logits[0])
            x_buf.copy_(xs[0])
            step()                                  # warm-up step 0, eager (also the capture's warm-up)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            for s in range(1, W):
                lg_buf.copy_(logits[s])
                x_buf.copy_(xs[s])
                g.replay()
            torch.cuda.synchronize()
            st0 = cache.t["stats"].cpu().numpy().copy()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for s in range(W, W + K):
                lg_buf.copy_(logits[s])
                x_buf.copy_(xs[s])
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / K
            d = cache.t["stats"].cpu().numpy() - st0
            miss = float(d[1]) / max(1.0, float(d[0] + d[1]))
            row = {"bs": bs, "slots": S, "ms_per_step": round(ms, 3), "tok_s": round(bs * 1000.0 / ms, 1),
                   "miss_rate": round(miss, 4), "unique_per_layer_call": round(float(d[0] + d[1]) / (K * c.L), 2),
                   "fills_per_step": round(float(d[2]) / K, 1),
                   "link_gbs": round(float(d[2]) * S_e / (ms * K * 1e-3) / 1e9, 1)}
            log("c5 bs %2d slots %4d: %.3f ms/step, %.1f tok/s, miss %.3f, %.1f unique/layer, %.0f fills/step"
                % (bs, S, ms, row["tok_s"], miss, row["unique_per_layer_call"], row["fills_per_step"]))
            out.append(row)
            del g
        del layers, cache, pool
        torch.cuda.empty_cache()
    return out


def c3_runs(args, torch, L, synth):
    """DeepSeek-V4-Flash-shaped hybrid decode (E=256 top-6, H=4096, I=2048, MXFP4, bs=1):
    misses split by q* = m * B_P / B_H with at least one fill per call; the rest run on the
    CPU worker pool over the pinned banks while the GPU fills and runs its routes, and the
    merge waits for the slower branch.  The full model (43 layers, 11008 experts, 147 GB
    pinned, 1500 slots) does not fit the 64 GiB of host memory a process can pin here, so
    `--c3-layers` layers are built with the slot pool scaled to the same share of the
    experts (1500 / 11008); the per-token figure is 43 x the measured per-layer time.
    One captured graph per step (the host branch is served from the pinned stage by the
    worker pool's dispatcher, so the step holds kernels only).  The pool holds 64 distinct seeded experts repeated over its entries: the bytes moved are
    those of the real pool, and the values do not change the timing (the split's numerics
    are tested at this expert shape)."""
    from concurrent.futures import ThreadPoolExecutor
    from expert_cache_offloaded_amd.runtime import BankSet, CacheState, DecodeBuffers, DecodeLayer, alloc_banks
    full = synth.CONFIGS["dsv4_hybrid"]
    n_layers = max(1, min(full.L, args.c3_layers))
    cfg = full.with_(L=n_layers, S=max(full.k, round(full.S * n_layers / full.L)))
    W, K = 8, args.c3_steps
    n_distinct = 64
    S_e = synth.expert_bytes(cfg.H, cfg.I, cfg.fmt)
    log("c3: pinned host pool %d experts x %d B (%.1f GB)" % (cfg.n_flat, S_e, cfg.n_flat * S_e / 1e9))
    host_t, host_free = alloc_pinned_exact(cfg.n_flat, cfg.H, cfg.I, cfg.fmt, torch)
    views = {k: v.numpy() for k, v in host_t.items()}
    distinct = [synth.expert_weights(cfg, f) for f in range(n_distinct)]
    t0 = time.time()

    def fill(f0):
        for f in range(f0, min(cfg.n_flat, f0 + 256)):
            for k, a in distinct[f % n_distinct].items():
                views[k][f] = a
        if f0 % 2048 == 0:
            log("c3: host pool %d/%d (%.0f s)" % (f0, cfg.n_flat, time.time() - t0))
    with ThreadPoolExecutor(max_workers=min(16, len(os.sched_getaffinity(0)))) as ex:
        list(ex.map(fill, range(0, cfg.n_flat, 256)))
    log("c3: host pool ready (%.0f s)" % (time.time() - t0))
    host = BankSet(host_t, cfg.H, cfg.I, cfg.fmt)
    pool = BankSet(alloc_banks(cfg.S, cfg.H, cfg.I, cfg.fmt, device="cuda"), cfg.H, cfg.I, cfg.fmt)
    workers = L.HostPool(min(16, len(os.sched_getaffinity(0))))
    prof = L.bandwidth_profile(host.desc, pool.desc, workers, 4, seconds=1.0)
    log("c3: bandwidth profile: link %.1f GB/s, host experts %.1f GB/s -> fetch fraction %.3f, %s"
        % (prof["pcie_gbs"], prof["cpu_gbs"], prof["frac_q16"] / 65536.0, prof["backend"]))
    runs = [(r, p, L.fetch_fraction_q16(1.0, r)) for p in (0.5, 0.9) for r in (1.5, 2.0, 3.0)]
    runs.append(("measured", 0.5, int(prof["frac_q16"])))
    out = {"workload": "deepseek-v4-flash-shaped hybrid decode: E=256 top-6, H=4096, I=2048, MXFP4, bs=1; "
                       "%d of the 43 MoE layers built (pinned pool of %d experts), %d slots (the share "
                       "1500/11008 of the experts); per token = 43 x per layer" % (cfg.L, cfg.n_flat, cfg.S),
           "layers_built": cfg.L, "slots": cfg.S,
           "steps": K, "warmup": W, "host_workers": workers.n_threads,
           "bandwidth_profile": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in prof.items()},
           "runs": []}
    for ratio, p, frac in runs:
        c = cfg.with_(p=p)
        tr = synth.trace(c, steps=W + K)
        logits = torch.from_numpy(np.stack([synth.step_logits(c, tr[s], s) for s in range(W + K)])).cuda()
        xs = torch.from_numpy(np.stack([np.stack([synth.activations(c, s, l) for l in range(c.L)])
                                        for s in range(W + K)]).view(np.int16)).cuda()
        cache = CacheState(c.L, c.E, c.S)
        cache.reset()
        layers = [DecodeLayer(cache, host, pool, None, DecodeBuffers(1, c.k, c.H, c.I), frac_q16=frac,
                              min_fill=1, renorm=c.renorm, hybrid=True, host_pool=workers)
                  for _ in range(c.L)]

        lg_buf, x_buf = torch.empty_like(logits[0]), torch.empty_like(xs[0])

        def step():
            for l in range(c.L):
                layers[l](l, lg_buf[l], x_buf[l])
        lg_buf.copy_(logits[0])
        x_buf.copy_(xs[0])
        step()                                  # eager step 0 (also the capture's warm-up)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for s in range(1, W):
            lg_buf.copy_(logits[s])
            x_buf.copy_(xs[s])
            g.replay()
        torch.cuda.synchronize()
        st0 = cache.t["stats"].cpu().numpy().copy()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(W, W + K):
            lg_buf.copy_(logits[s])
            x_buf.copy_(xs[s])
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        errs = sum(dl.stage.errors() for dl in layers)
        if errs:
            raise RuntimeError("c3: %d merge waits ran out" % errs)
        ms = e0.elapsed_time(e1) / K
        ms_layer = ms / c.L
        d = cache.t["stats"].cpu().numpy() - st0
        row = {"b_h_over_b_p": ratio, "locality": p, "fetch_fraction": round(frac / 65536.0, 4),
               "ms_per_layer": round(ms_layer, 4), "ms_per_token_43": round(ms_layer * full.L, 3),
               "tok_s_43": round(1000.0 / (ms_layer * full.L), 2),
               "miss_rate": round(float(d[1]) / max(1.0, float(d[0] + d[1])), 4),
               "fills_per_layer": round(float(d[2]) / (K * c.L), 3),
               "host_routes_per_layer": round(float(d[3]) / (K * c.L), 3),
               "link_gbs": round(float(d[2]) * S_e / (ms * K * 1e-3) / 1e9, 2),
               "host_gbs": round(float(d[3]) * S_e / (ms * K * 1e-3) / 1e9, 2)}
        log("c3 B_H/B_P %s p %.1f f %.3f: %.3f ms/layer (43 layers: %.2f tok/s), miss %.3f, %.2f fills + "
            "%.2f host routes per layer" % (ratio, p, frac / 65536.0, ms_layer, row["tok_s_43"],
                                            row["miss_rate"], row["fills_per_layer"], row["host_routes_per_layer"]))
        out["runs"].append(row)
        del g
        for dl in layers:
            dl.stage.close()
        del layers, cache, logits, xs
    workers.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_c3(cfg, full.L, views)
    del host, pool, views, host_t
    torch.cuda.synchronize()
    host_free()
    return out


def cpu_baseline_c3(cfg, n_layers_model, views, n_layers=4):
    """The oracle on one decode token through `n_layers` layers of the C3 pool (route, LRU
    lookup, unsplit per-token expert sum in float64); per-token time scaled to the model."""
    from oracle import LruOracle, decode_layer, route
    import synth
    env = cpu_env()
    tr = synth.trace(cfg, steps=1)
    lg = synth.step_logits(cfg, tr[0], 0)

    def run(n):
        o = LruOracle(cfg.L, cfg.E, cfg.S)
        for l in range(n):
            ids, w = route(lg[l], cfg.k, cfg.renorm)
            o.lookup(l, ids, 1 << 16)
            decode_layer(synth.activations(cfg, 0, l), ids, w, views, l, cfg.E, cfg.fmt, cfg.H, cfg.I)

    log("cpu baseline: decode oracle, 1 token x %d layers of the C3 pool" % n_layers)
    t0 = time.perf_counter()
    run(n_layers)
    dt = time.perf_counter() - t0
    _, dt1 = one_core(lambda: run(1))
    return dict({"value": round(1.0 / (dt / n_layers * n_layers_model), 4), "unit": "tok/s", "kind": "oracle",
                 "sample": "1 decode token through %d layers (route, LRU lookup, unsplit float64 expert sum); "
                           "per-token time scaled to %d layers (one core: 1 layer)" % (n_layers, n_layers_model),
                 "seconds": round(dt, 2),
                 "one_core": {"value": round(1.0 / (dt1 * n_layers_model), 4), "seconds": round(dt1, 2)}}, **env)


def alloc_pinned_exact(n, H, I, fmt, torch):
    """Pinned host banks of exactly n entries each, from hipHostMalloc (torch's pinned
    allocator rounds every block up to a power of two: 147 GB of banks would pin ~204 GiB).
    Returns the tensors and a function that frees them."""
    import ctypes as C
    from expert_cache_offloaded_amd.runtime import bank_shapes
    hip = C.CDLL("libamdhip64.so")
    ptrs, out = [], {}
    for name, (shp, dt) in bank_shapes(H, I, fmt).items():
        nbytes = n * int(np.prod(shp)) * torch.empty((), dtype=dt).element_size()
        p = C.c_void_p()
        log("pinning %s: %.1f GB" % (name, nbytes / 1e9))
        rc = hip.hipHostMalloc(C.byref(p), C.c_size_t(nbytes), C.c_uint(0))
        if rc != 0 or not p.value:
            raise MemoryError("hipHostMalloc of %d bytes failed (%d)" % (nbytes, rc))
        ptrs.append(p)
        np_dt = {torch.uint8: np.uint8, torch.int16: np.int16}[dt]
        arr = np.ctypeslib.as_array(C.cast(p, C.POINTER(C.c_uint8)), shape=(nbytes,)).view(np_dt)
        out[name] = torch.from_numpy(arr.reshape((n,) + tuple(shp)))

    def free():
        out.clear()
        for p in ptrs:
            hip.hipHostFree(p)
    return out, free


def bench_prefill(args, torch, L, synth):
    """8192-token prefill over 4 DeepSeek-V4-Flash-shaped MoE layers (E=256 top-6, H=4096,
    I=2048, MXFP4, uniform routing): grouped-GEMM throughput on a resident layer, and the
    whole-layer double buffer streaming each next layer's 256 experts host -> HBM."""
    from expert_cache_offloaded_amd.runtime import alloc_banks
    cfg = synth.CONFIGS["prefill"]
    T, E, k, H, I = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I
    dev = "cuda"
    log("prefill: pinned pool of %d layers x %d experts" % (cfg.L, E))
    host_t = alloc_banks(cfg.n_flat, H, I, cfg.fmt, pin=True)
    fill_host_pool(cfg, host_t)
    host = L.make_banks(cfg.fmt, H, I, host_t)
    bufs_t = [alloc_banks(E, H, I, cfg.fmt, device=dev) for _ in range(2)]
    bufs = [L.make_banks(cfg.fmt, H, I, b) for b in bufs_t]
    x = torch.from_numpy(synth.activations(cfg, 0).view(np.int16)).to(dev)
    logits = [torch.from_numpy(synth.uniform_logits(cfg, layer=l)).to(dev) for l in range(cfg.L)]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws = torch.empty(L.prefill_ws_bytes(T, k, E, H, I), dtype=torch.uint8, device=dev)
    ys = [torch.empty((T, H), dtype=torch.int16, device=dev) for _ in range(cfg.L)]
    layer_bytes = synth.expert_bytes(H, I, cfg.fmt) * E
    flops = 6.0 * H * I * T * k

    def copy_layer(l, b, stream):
        with torch.cuda.stream(stream):
            for name in bufs_t[b]:
                bufs_t[b][name].copy_(host_t[name][l * E:(l + 1) * E], non_blocking=True)

    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()

    # resident layer: route + sort + grouped GEMMs + combine, graph replays timed with events
    copy_layer(0, 0, comp)
    torch.cuda.synchronize()

    def layer_compute(l, b, nxt=None):
        L.moe_route(logits[l], k, 1, ids, w)
        L.moe_experts_prefill(x, ids, w, None, E, bufs[b], ws, ys[l], nxt)

    layer_compute(0, 0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer_compute(0, 0)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(args.prefill_reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        g.replay()
        e1.record(comp)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    t_comp = float(np.median(ts))
    log("prefill compute (resident layer): %.3f ms, %.0f tok/s, %.0f TFLOP/s"
        % (t_comp, T / t_comp * 1e3, flops / t_comp * 1e-9))

    # serialized: copy a layer, then compute it (GPU events; best of two passes, the
    # first pass also pays first-use costs of the host pages)
    def serial_pass():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(comp)
        for l in range(cfg.L):
            copy_layer(l, 0, comp)
            layer_compute(l, 0)
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    # double buffer: layer l computes from buffer l % 2 while l+1 streams into the other
    def pipelined_pass():
        done = [torch.cuda.Event() for _ in range(2)]
        free = [torch.cuda.Event() for _ in range(2)]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(copy)
        copy_layer(0, 0, copy)
        done[0].record(copy)
        for l in range(cfg.L):
            b = l % 2
            comp.wait_event(done[b])
            nxt = None
            if l + 1 < cfg.L:
                copy.wait_event(free[1 - b])
                nxt = L.make_prefetch(host, (l + 1) * E, bufs[1 - b], copy)
            layer_compute(l, b, nxt)
            if nxt is not None:
                done[1 - b].record(copy)
            free[b].record(comp)
        e1.record(comp)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    tflops = flops / t_comp * 1e-9
    roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
            "frac": round(tflops / 2500.0, 4), "traffic": traffic_bytes("moe_experts_prefill"),
            "kernel": "moe_experts_prefill (route + sort + gate_up + down + combine)",
            "flop_per_launch": flops, "ms_per_launch": round(t_comp, 4)}
    pre = {"workload": "8192-token prefill, 4 MoE layers, E=256 top-6 uniform routing, H=4096, I=2048, "
                       "MXFP4 experts, double-buffered 256-expert layer pool",
           "tokens": T, "layers": cfg.L,
           "compute_ms_per_layer": round(t_comp, 4), "compute_tok_s": round(T / t_comp * 1e3, 1)}
    if args.prefill_resident_only:
        return pre, roof
    t_serial = min(serial_pass() for _ in range(2)) / cfg.L
    t_pipe = min(pipelined_pass() for _ in range(2)) / cfg.L
    t_link = t_serial - t_comp
    link_gbs = layer_bytes / (t_link * 1e-3) / 1e9
    ideal = (t_comp + t_link) / max(t_comp, t_link)
    log("prefill serialized %.1f ms/layer, double-buffered %.1f ms/layer (overlap %.3f of ideal %.3f)"
        % (t_serial, t_pipe, t_serial / t_pipe, ideal))
    pre.update({"serial_ms_per_layer": round(t_serial, 3), "pipelined_ms_per_layer": round(t_pipe, 3),
                "pipelined_tok_s": round(T / t_pipe * 1e3, 1), "layer_pool_bytes": int(layer_bytes),
                "link_gbs": round(link_gbs, 2), "overlap_speedup": round(t_serial / t_pipe, 3),
                "overlap_ideal": round(ideal, 3)})
    if not args.no_cpu_baseline:
        pre["cpu_baseline"] = cpu_baseline_prefill(cfg, host_t)
    return pre, roof


def cpu_baseline_prefill(cfg, host_t, n_experts=64):
    """The oracle's grouped prefill (route, stable sort, per-expert float64 FFN, scatter-add)
    on `n_experts` of the 256 experts of layer 0; tok/s scaled to the whole layer."""
    from oracle import prefill_grouped, route
    import synth
    env = cpu_env()
    banks = {k: v[:cfg.E].numpy() for k, v in host_t.items()}
    x = synth.activations(cfg, 0)

    def run(n):
        ids, w = route(synth.uniform_logits(cfg, layer=0), cfg.k, 1)
        prefill_grouped(x, ids, w, banks, cfg.E, cfg.fmt, cfg.H, cfg.I, experts=range(n))

    log("cpu baseline: prefill oracle on %d of %d experts (layer 0)" % (n_experts, cfg.E))
    t0 = time.perf_counter()
    run(n_experts)
    dt = time.perf_counter() - t0
    n1 = max(1, n_experts // 4)
    _, dt1 = one_core(lambda: run(n1))
    return dict({"value": round(cfg.T / (dt * cfg.E / n_experts), 2), "unit": "tok/s", "kind": "oracle",
                 "sample": "%d of the %d experts of one 8192-token layer (their routed tokens), grouped "
                           "per-expert float64 FFN; tok/s scaled to the whole layer (one core: %d experts)"
                           % (n_experts, cfg.E, n1),
                 "seconds": round(dt, 2),
                 "one_core": {"value": round(cfg.T / (dt1 * cfg.E / n1), 2), "seconds": round(dt1, 2)}}, **env)


def cpu_baseline(cfg, tr, logits, xs, host_np, sh_np, n_tokens):
    """The oracle (as it stands) on the host cores: route + LRU + split + per-token expert
    sum; then the same sample held to one core."""
    from oracle import LruOracle, decode_layer, route
    env = cpu_env()
    host = {k: (v.view(np.uint16) if v.dtype == np.int16 else v) for k, v in host_np.items()}

    def run():
        o = LruOracle(cfg.L, cfg.E, cfg.S)
        for s_ in range(n_tokens):
            for l in range(cfg.L):
                ids, w = route(logits[s_, l], cfg.k, cfg.renorm)
                o.lookup(l, ids, 1 << 16)
                decode_layer(xs[s_, l], ids, w, host, l, cfg.E, cfg.fmt, cfg.H, cfg.I, shared=sh_np)

    log("cpu baseline: oracle on %d token(s) x %d layers (%d threads, then 1)" % (n_tokens, cfg.L, env["cores"]))
    t0 = time.perf_counter()
    run()
    dt = time.perf_counter() - t0
    _, dt1 = one_core(run)
    return dict({"value": round(n_tokens / dt, 4), "unit": "tok/s", "kind": "oracle",
                 "sample": "%d decode token(s) x %d layers of the same workload (route, LRU lookup, split, "
                           "unsplit per-token expert sum in float64)" % (n_tokens, cfg.L),
                 "seconds": round(dt, 2), "one_core": {"value": round(n_tokens / dt1, 4), "seconds": round(dt1, 2)}},
                **env)


if __name__ == "__main__":
    main()
