"""Benchmark of the MoE expert path on one MI355X.

Default workload: one MoE layer at hidden 4096, expert intermediate 1024, 512 experts, top-4,
4-bit group-64 affine experts (bf16 scale/bias), router bf16 512 x 4096, one decode token per
step.  A step is one token through the whole path (router, softmax/top-K/renormalise, gate/up
+ SwiGLU for the 4 experts, down + weighted combine), issued as one moe_layer_decode call; the
steps run back to back on one stream (each call is complete before the next starts) and are
captured in HIP graphs.  Tokens rotate through a bank of 4096 distinct seeded activations so
that routing, and the experts read, change every step (3.4 GiB of experts, far beyond the
256 MB last-level cache).  Inputs are synthetic and already resident in HBM.

Prints ONE JSON line on stdout; progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--config {0,1,2,3,4}] [--cpu-seconds S]
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=4096)
    p.add_argument("--warmup", type=int, default=512)
    p.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 3, 4])
    p.add_argument("--tokens", type=int, default=0,
                   help="tokens per call through the batched path (2..4096) instead of the config's own; "
                        "for single-layer configs (small-T multi-token decode)")
    p.add_argument("--graph-steps", type=int, default=0, help="steps per captured graph (0: auto)")
    p.add_argument("--schedule", default="two_launch", choices=["two_launch", "single_launch", "three_kernels"],
                   help="layer schedule of the decode steps: two launches (default), one, or three kernels")
    p.add_argument("--no-graph", action="store_true", help="issue steps eagerly instead of via HIP graphs")
    p.add_argument("--graph", action="store_true",
                   help="replay HIP graphs for batched configs too (by default their steps are issued eagerly; "
                        "both measure the same at 256 tokens, 540 us per batch)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--timing-steps", type=int, default=256, help="steps of the per-kernel timing pass")
    p.add_argument("--quantize", action="store_true",
                   help="measure quantise-from-float (moe_quantize_matrix) instead of the expert path")
    p.add_argument("--retier", action="store_true",
                   help="measure the tiered-store policy (usage over the routed token bank, hot order, "
                        "requantisation of the cold experts) instead of the expert path")
    p.add_argument("--cache-device", action="store_true",
                   help="with --cache: the device-side policy (moe_cache_fetch_device, no host round trip)")
    p.add_argument("--cache", type=int, default=0, metavar="SLOTS",
                   help="decode with the experts in pinned host memory and SLOTS of them cached in device "
                        "memory (moe_cache_fetch before each step's expert FFN)")
    p.add_argument("--small-t", action="store_true",
                   help="expert FFN of 2..16 tokens on config 1, shared-read against per-token kernels, on "
                        "router-chosen, draft-style and identical routings (one JSON line)")
    p.add_argument("--small-t-case", default="", metavar="T:ROUTING",
                   help="with --small-t: only this case (e.g. 16:same), for profiler runs")
    p.add_argument("--small-t-path", default="both", choices=["both", "shared", "per_token"],
                   help="with --small-t: the kernels to time")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run device-to-device copies of 1 GiB (reference for the HBM byte counters)")
    p.add_argument("--traffic-from", metavar="DIR",
                   help="read rocprofv3 --pmc output under DIR/{fetch,write,copy_fetch,copy_write} and write "
                        "profiles/traffic.json for this workload")
    p.add_argument("--traffic-key", default="",
                   help="workload key for --traffic-from (default config<N>; 'quantize' and 'retier' for "
                        "those modes)")
    return p.parse_args()


# The source file that defines each measured kernel; every kernel also includes the shared headers.
KERNEL_SOURCES = {
    "k_layer": "moe_fused.hip",
    "k_route_gateup": "moe_layer.hip",
    "k_router": "moe_decode.hip", "k_gateup": "moe_decode.hip", "k_down": "moe_decode.hip",
    "k_router_mfma": "moe_grouped.hip", "k_group": "moe_grouped.hip", "k_gu_mfma": "moe_grouped.hip",
    "k_dn_mfma": "moe_grouped.hip", "k_dn_res": "moe_grouped.hip",
    "k_gu8": "moe_batched8.hip", "k_dn8": "moe_batched8.hip",
    "k_stage_rows": "moe_shared_gu.hip", "k_gu_sh": "moe_shared_gu.hip", "k_dn_sh": "moe_shared_dn.hip",
    "k_quantize": "moe_quant.hip", "k_requant": "moe_tier.hip",
}
SHARED_HEADERS = ("moe_device.h", "moe_internal.h", "moe_handoff.h", "moe_small.h")


def source_hash(kernel: str = "") -> str:
    """Hash of the sources a kernel is built from (its file and the shared headers); with no kernel,
    of every device source."""
    d = os.path.join(ROOT, "bit_expert_dequant_amd", "csrc")
    if kernel:
        files = sorted({KERNEL_SOURCES[kernel], *SHARED_HEADERS})
    else:
        files = sorted(f for f in os.listdir(d) if f.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload_key: str):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, valid only while the
    kernel's sources (its file and the shared headers) are unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(workload_key, {}).get(kernel)
        if e and e.get("source_hash") == source_hash(kernel):
            return e.get("bytes_per_launch")
    except Exception:
        return None
    return None


COPY_BYTES = 1 << 30
STREAM_BYTES = 4 << 30


def copy_calibration():
    """Plain device-to-device copies of known size: each reads and writes COPY_BYTES."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {COPY_BYTES} bytes 4 times")


def read_counter_csv(d: str, counter: str):
    """{kernel name: [value per dispatch]} from a rocprofv3 counter_collection.csv under d."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic_from(d: str, workload_key: str):
    """HBM bytes per launch of each decode kernel: FETCH_SIZE + WRITE_SIZE (KiB per dispatch), each
    scaled so that the copy kernel reads and writes exactly COPY_BYTES."""
    scale = {}
    for c, sub in (("FETCH_SIZE", "copy_fetch"), ("WRITE_SIZE", "copy_write")):
        vals = [v for k, vs in read_counter_csv(os.path.join(d, sub), c).items() for v in vs
                if "copy" in k.lower() or "elementwise" in k.lower()]
        big = [v for v in vals if v * 1024 > COPY_BYTES / 2]
        if not big:
            raise SystemExit(f"no copy dispatch found for {c}")
        scale[c] = COPY_BYTES / (float(np.median(big)) * 1024)
    fetch = read_counter_csv(os.path.join(d, "fetch"), "FETCH_SIZE")
    write = read_counter_csv(os.path.join(d, "write"), "WRITE_SIZE")
    res = {}
    for short in ("k_route_gateup", "k_router", "k_gateup", "k_down", "k_router_mfma", "k_group", "k_gu_mfma",
                  "k_dn_mfma", "k_dn_res", "k_gu8", "k_dn8", "k_quantize", "k_requant"):
        fk = [k for k in fetch if f"{short}<" in k or f"{short}(" in k]
        wk = [k for k in write if f"{short}<" in k or f"{short}(" in k]
        if not fk or not wk:
            continue
        f = float(np.mean([v for k in fk for v in fetch[k]])) * 1024 * scale["FETCH_SIZE"]
        w = float(np.mean([v for k in wk for v in write[k]])) * 1024 * scale["WRITE_SIZE"]
        res[short] = {"bytes_per_launch": f + w, "fetch_bytes": f, "write_bytes": w,
                      "dispatches": sum(len(fetch[k]) for k in fk), "source_hash": source_hash(short),
                      "scale_fetch": scale["FETCH_SIZE"], "scale_write": scale["WRITE_SIZE"]}
    p = os.path.join(ROOT, "profiles", "traffic.json")
    allp = json.load(open(p)) if os.path.exists(p) else {}
    allp[workload_key] = res
    json.dump(allp, open(p, "w"), indent=1, sort_keys=True)
    log(f"[bench] wrote {p}: {json.dumps(res)}")


def quantize_bench(a):
    """Quantise-from-float: 64 fp32 matrices of 1024 x 4096 (the shape of a 4-bit expert's gate and
    up) into 4-bit packed planes, 16 matrices stacked row-wise per launch (a bulk conversion; a
    single 19 MB matrix per launch is dominated by the launch's ramp), timed with events on the
    launch stream.
    Algorithmic bytes per launch: the weights read once plus the code and (scale, bias) planes
    written once.  Parity: every code and pair of the first matrix against the oracle."""
    import torch
    import bit_expert_dequant_amd as M
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rows, cols, bits, n, per = 1024, 4096, 4, 64, 16
    cb, sbb = M.lib().moe_packed_codes_bytes(rows, cols, bits), M.lib().moe_packed_sb_bytes(rows, cols)
    gen = torch.Generator(device="cuda").manual_seed(0x9A47)
    W = torch.randn(n, rows, cols, device="cuda", dtype=torch.float32, generator=gen) * 0.05
    codes = torch.empty(n, cb, dtype=torch.uint8, device="cuda")
    sb = torch.empty(n, sbb // 2, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    nl = n // per

    def run():
        for i in range(nl):
            M.moe_quantize_matrix(W[i * per:(i + 1) * per].view(per * rows, cols), bits, codes[i * per:(i + 1) * per],
                                  sb[i * per:(i + 1) * per])
    run()
    torch.cuda.synchronize()
    reps = 8
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * nl)
    per_launch = per * (rows * cols * 4 + cb + sbb)
    gbps = per_launch / (us * 1e-6) / 1e9
    # CPU leg (skipped with --no-cpu): the oracle's quantiser on the first matrix, compared code by code
    parity_ok = None
    if not a.no_cpu:
        import oracle
        oc, os_, ob = oracle.quantize(W[0].cpu().numpy(), bits)
        plane = codes[0].cpu().numpy().reshape(rows, cols // 2)
        gc = np.empty((rows, cols), dtype=np.uint8)
        gc[:, 0::2], gc[:, 1::2] = plane & 15, plane >> 4
        gsb = sb[0].cpu().numpy().view(np.uint16).reshape(rows, cols // 64, 2)
        parity_ok = bool(np.array_equal(gc, oc) and np.array_equal(gsb[:, :, 0], os_)
                         and np.array_equal(gsb[:, :, 1], ob))
    line = {"metric": "quantise-from-float GB/s (fp32 weights -> 4-bit packed planes)", "value": round(gbps, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": reps * nl, "warmup": nl, "ms_per_step": round(us * 1e-3, 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"{n} fp32 matrices of {rows} x {cols}, 4-bit, group 64, {per} per launch",
                       "rows": per * rows, "cols": cols, "bits": bits},
            "roofline": {"bound": "hbm", "kernel": "k_quantize", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic("k_quantize", "quantize"),
                         "bytes_per_launch": per_launch, "us_per_launch": round(us, 3),
                         "timing": "HIP events around back-to-back launches on the launch stream"},
            "parity": {"matrices": 1, "bit_exact": parity_ok}}
    print(json.dumps(line), flush=True)


def retier_bench(a):
    """Re-tiering a layer of 512 experts of 4096 x 1024 at 4 bits into hot 4-bit / cold 2-bit (the
    tiered store of the pages): a step is moe_expert_usage over the routing indices of a 4096-token
    stream (routed once beforehand with the Zipf(1.1) prior, 256 tokens per moe_route call), then
    moe_hot_order, then moe_retier with 128 hot experts, the other 384 requantised to 2 bits.
    Algorithmic bytes per step: each cold expert's 4-bit blob read once and its 2-bit blob written
    once.  The requantisation kernel is timed on its own with HIP events around moe_retier (which
    adds one small table kernel).  Parity: the first and last cold experts bit-exact against the
    oracle; the hot set's share of the stream's selections beside that of the prior's hot set."""
    import torch
    import bit_expert_dequant_amd as M
    import synth
    from synth.device import act_tensor, build_layer
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synth.WORKLOADS[4]
    H, I, E, K, n_hot, T, chunk = wl.H, wl.I, wl.E, wl.K, synth.N_HOT, 4096, 256
    d = M.make_dims(H, I, E, K)
    dl = build_layer(wl)
    stream = torch.cuda.current_stream()
    bank = wl.tokens_bank(T)
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, K, dtype=torch.float32, device="cuda")
    ws = M.workspace(M.MOE_OP_ROUTE, d, chunk, 1)
    for c in range(0, T, chunk):
        M.moe_route(d, dl.L, act_tensor(wl, bank[c:c + chunk]), idx[c:c + chunk], wts[c:c + chunk], ws=ws)
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    order = torch.empty(E, dtype=torch.int32, device="cuda")
    cold_bytes = M.lib().moe_packed_expert_bytes(H, I, 2)
    base_bytes = M.lib().moe_packed_expert_bytes(H, I, 4)
    cold = torch.empty((E - n_hot) * cold_bytes, dtype=torch.uint8, device="cuda")
    tiered = torch.zeros_like(dl.table)

    def step():
        counts.zero_()
        M.moe_expert_usage(idx, E, counts)
        M.moe_hot_order(counts, order)
        M.moe_retier(d, dl.table, order, n_hot, 2, cold, tiered)

    steps, warm = max(1, min(a.steps, 16)), max(1, min(a.warmup, 4))
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 2)]
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    step_ms = ev[0].elapsed_time(ev[1]) / steps
    for i in range(steps):
        counts.zero_()
        M.moe_expert_usage(idx, E, counts)
        M.moe_hot_order(counts, order)
        ev[2 + 2 * i].record(stream)
        M.moe_retier(d, dl.table, order, n_hot, 2, cold, tiered)
        ev[3 + 2 * i].record(stream)
    torch.cuda.synchronize()
    rq_ms = [ev[2 + 2 * i].elapsed_time(ev[3 + 2 * i]) for i in range(steps)]
    rq = float(np.median(rq_ms))
    algo = (E - n_hot) * (base_bytes + cold_bytes)
    gbps_step = algo / (step_ms * 1e-3) / 1e9
    gbps_rq = algo / (rq * 1e-3) / 1e9
    c_np = counts.cpu().numpy().astype(np.int64)
    o_np = order.cpu().numpy()
    total = int(c_np.sum())
    share = float(c_np[o_np[:n_hot]].sum()) / total
    prior_share = float(c_np[synth.hot_set(wl.seed, E)].sum()) / total
    # CPU leg (skipped with --no-cpu): the oracle's requantisation of two cold experts (inputs: the
    # seeded base blobs), compared code by code, then its throughput on a bounded sample
    parity_ok = None
    cpu = None
    if not a.no_cpu:
        import oracle
        parity_ok = True
        for r in (n_hot, E - 1):
            e = int(o_np[r])
            slot = r - n_hot
            gpu = cold[slot * cold_bytes:(slot + 1) * cold_bytes].cpu().numpy()
            ref = oracle.requantize_expert(synth.expert_blob(wl.seed, 0, e, H, I, 4), H, I, 4, 2)
            off, _ = synth.blob_layout(H, I, 2)
            sizes = synth.plane_sizes(H, I, 2)
            for m, (rows, cols) in enumerate([(I, H), (I, H), (H, I)]):
                plane = gpu[off[2 * m]:off[2 * m] + sizes[2 * m]].reshape(rows, cols // 4)
                codes = np.empty((rows, cols), dtype=np.uint8)
                for k in range(4):
                    codes[:, k::4] = (plane >> (2 * k)) & 3
                sb = gpu[off[2 * m + 1]:off[2 * m + 1] + sizes[2 * m + 1]].view(np.uint16).reshape(rows, cols // 64, 2)
                parity_ok &= bool(np.array_equal(codes, ref[m][0]) and np.array_equal(sb[:, :, 0], ref[m][1])
                                  and np.array_equal(sb[:, :, 1], ref[m][2]))
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        blob0 = synth.expert_blob(wl.seed, 0, 0, H, I, 4)
        n_cpu, t0 = 0, time.perf_counter()
        while n_cpu < 1 or (time.perf_counter() - t0 < 10.0 and n_cpu < 8):
            oracle.requantize_expert(blob0, H, I, 4, 2)
            n_cpu += 1
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(n_cpu * (base_bytes + cold_bytes) / cpu_s / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle", "sample": f"{n_cpu} experts requantised 4 -> 2 bits (oracle.requantize_expert: "
                                           f"fp32 dequantisation with OpenMP, then the single-threaded quantiser)"}
    line = {"metric": "re-tier GB/s (4-bit base -> hot 4-bit / cold 2-bit store)", "value": round(gbps_step, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": round(step_ms, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"{E} experts H{H} I{I} 4-bit, usage over {T} routed tokens (top-{K}, Zipf(1.1) "
                                   f"prior), {n_hot} hot, {E - n_hot} requantised to 2 bits",
                       "hidden": H, "inter": I, "experts": E, "hot": n_hot, "tokens": T},
            "roofline": {"bound": "hbm", "kernel": "k_requant", "achieved": round(gbps_rq, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps_rq / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic("k_requant", "retier"),
                         "bytes_per_launch": algo, "us_per_launch": round(rq * 1e3, 2),
                         "timing": "HIP events around moe_retier on the launch stream (requantisation + table)"},
            "hot_share": {"measured_hot_set": round(share, 4), "prior_hot_set": round(prior_share, 4),
                          "selections": total},
            "parity": {"experts": 2, "bit_exact": parity_ok}, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def cache_bench(a):
    """Decode with the store in host memory: the 512 experts of a 4096 x 1024 4-bit layer (3.6 GB)
    in pinned host memory, a cache of a.cache slots in device memory, Zipf(1.1)-biased routing (the
    tiered workload's prior).  A step is one token: moe_route, the indices copied to the host,
    moe_cache_fetch (host-to-device copies of the missing experts, table update), moe_expert_ffn
    through the cache's table, moe_combine; steps are dependent (each waits for its indices).
    Reported beside it: the hit rate, the copy rate of the misses, a plain pinned host-to-device copy
    of 64 MiB as the link's reference, and the same steps with every expert resident."""
    import torch
    import bit_expert_dequant_amd as M
    import synth
    from synth.device import act_tensor, build_layer
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = dataclasses.replace(synth.WORKLOADS[4], tokens=1)
    H, I, E, K = wl.H, wl.I, wl.E, wl.K
    d = M.make_dims(H, I, E, K)
    dl = build_layer(wl)
    n_slots = a.cache
    host = torch.empty(dl.store.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.store)
    slots = torch.empty(n_slots * dl.stride, dtype=torch.uint8, device="cuda")
    table = torch.zeros_like(dl.table)
    cache = M.ExpertCache(d, [host.data_ptr() + e * dl.stride for e in range(E)], [4] * E, slots, dl.stride,
                          n_slots, table)
    dev = a.cache_device
    if dev:
        cache.attach_device()
    Lc = M.Layer(dl.router, table, dl.logit_bias, dl.norm_w, wl.norm_eps)
    bank = act_tensor(wl, wl.tokens_bank(4096))
    idx = torch.empty(1, K, dtype=torch.int32, device="cuda")
    w = torch.empty(1, K, dtype=torch.float32, device="cuda")
    y = torch.empty(1, K, H, dtype=torch.float32, device="cuda")
    out = torch.empty(1, H, dtype=torch.float32, device="cuda")
    ws_r = M.workspace(M.MOE_OP_ROUTE, d, 1, 1)
    ws_f = M.workspace(M.MOE_OP_EXPERT_FFN, d, 1, 1)
    idx_h = torch.empty(1, K, dtype=torch.int32, pin_memory=True)
    stream = torch.cuda.current_stream()
    fetch_ev = []                                # (start, stop) events around fetches that copied

    def step(t, cached=True, timed=False):
        x = bank[t % 4096:t % 4096 + 1]
        M.moe_route(d, dl.L, x, idx, w, ws=ws_r)
        if cached and dev:
            # no host step: the policy kernel reads the routing where moe_route left it
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if timed else None
            if ev:
                ev[0].record(stream)
            cache.fetch_device(idx)
            if ev:
                ev[1].record(stream)
                fetch_ev.append(ev)
        elif cached:
            idx_h.copy_(idx)                     # synchronous: the step needs its routing on the host
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if timed else None
            if ev:
                ev[0].record(stream)
            miss = cache.fetch(idx_h.numpy())
            if ev and miss:
                ev[1].record(stream)
                fetch_ev.append(ev)
        M.moe_expert_ffn(d, Lc if cached else dl.L, x, idx, y, ws_f)
        M.moe_combine(y, w, out)

    warm, steps = max(a.warmup, 64), max(min(a.steps, 2048), 64)
    for t in range(warm):
        step(t)
    torch.cuda.synchronize()
    h0, m0, b0 = cache.stats()
    t0 = time.perf_counter()
    for t in range(warm, warm + steps):
        step(t)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    h1, m1, b1 = cache.stats()
    # the copies' own rate: events around each fetch that copied (its copies and table kernel)
    b2 = cache.stats()[2]
    for t in range(warm + steps, warm + 2 * steps):
        step(t, timed=True)
    torch.cuda.synchronize()
    fetch_s = sum(e0.elapsed_time(e1) for e0, e1 in fetch_ev) * 1e-3
    fetch_gbps = (cache.stats()[2] - b2) / fetch_s / 1e9 if fetch_s > 0 else 0.0
    t0 = time.perf_counter()
    for t in range(warm, warm + steps):
        step(t, cached=False)
    torch.cuda.synchronize()
    dt_res = time.perf_counter() - t0
    # the link's reference: pinned host-to-device copies of 64 MiB
    src = torch.empty(64 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(16):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    link = 16 * (64 << 20) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    hits, misses, copied = h1 - h0, m1 - m0, b1 - b0
    copy_gbps = copied / dt / 1e9
    # parity: 16 more tokens through the cache against the resident store (same kernels: bit-exact);
    # in the CPU leg (skipped with --no-cpu) two of them also against the oracle
    from synth.device import act_f64
    exact, errs = True, []
    outs_c = []
    for t in range(warm + 2 * steps, warm + 2 * steps + 16):
        step(t)
        out_c = out.clone()
        idx_c = idx.clone()
        step(t, cached=False)
        torch.cuda.synchronize()
        exact &= bool(torch.equal(out_c, out) and torch.equal(idx_c, idx))
        if len(outs_c) < 2:
            outs_c.append((t, out_c.cpu().numpy()[0].astype(np.float64)))
    if not a.no_cpu:
        import oracle
        ol = oracle.workload_layer(wl)
        bank_np = wl.tokens_bank(4096)
        for t, got in outs_c:
            ref = oracle.layer_token(act_f64(wl, bank_np[t % 4096]), ol, H, I, K)
            errs.append(float(np.abs(got - ref.out).max() / (np.linalg.norm(ref.out) / math.sqrt(H))))
    policy = ("device-side policy (moe_cache_fetch_device: policy kernel + zero-copy copy kernel, no host step)"
              if dev else "host policy (indices copied to the host, moe_cache_fetch: DMA copies + table kernel)")
    line = {"metric": "decode tok/s with the expert store in host memory (device expert cache)",
            "value": round(steps / dt, 1), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warm,
            "ms_per_step": round(dt / steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "i4-dot-i32+f32", "data": "synthetic",
        "dtype_note": ("expert matvecs: 4-bit (or 2-bit) codes times 16-bit fixed-point activation digits per "
                       "32-column slot as exact int32 dot products (v_dot8_i32_i4), scale and bias applied in fp32; "
                       "router: bf16 pairs (hi + lo split when the activation is not bf16) with fp32 accumulation; "
                       "batched busy experts: bf16 MFMA with fp32 accumulation; inputs bf16, outputs fp32"),
            "config": {"workload": f"one layer H{H} I{I} E{E} top-{K} 4-bit (3.6 GB) in pinned host memory, "
                                   f"{n_slots} device slots, Zipf(1.1) routing, 1 token per step",
                       "slots": n_slots, "experts": E},
            "cache": {"hit_rate": round(hits / max(1, hits + misses), 4), "misses_per_token": round(misses / steps, 3),
                      "bytes_copied": copied, "copied_per_second_of_decode_GBps": round(copy_gbps, 2)},
            "policy": policy,
            "roofline": {"bound": "pcie",
                         "kernel": ("k_cache_policy + k_cache_copy (every step's device fetch)" if dev else
                                    "host-to-device copies of missing experts (moe_cache_fetch)"),
                         "achieved": round(fetch_gbps, 2), "peak": round(link, 2), "unit": "GB/s",
                         "frac": round(fetch_gbps / link, 4), "traffic": None,
                         "timing": (f"HIP events around the device fetch of each of {steps} further steps "
                                    "(policy kernel + copy kernel, hits-only steps included)" if dev else
                                    f"HIP events around the {len(fetch_ev)} fetches that copied, in {steps} further "
                                    "steps (copies plus the table kernel)"),
                         "peak_is": "measured pinned host-to-device copy rate (64 MiB copies)"},
            "resident_tok_s": round(steps / dt_res, 1),
            "parity": {"tokens_vs_resident": 16, "bit_exact_vs_resident": exact, "tokens_vs_oracle": len(errs),
                       "max_err_over_rms": max(errs) if errs else None, "tolerance": 2e-3,
                       "ok": bool(exact and (not errs or max(errs) <= 2e-3))}}
    cache.close()
    print(json.dumps(line), flush=True)


def small_t_bench(a):
    """Expert FFN of a few tokens (moe_expert_ffn_path): each call's T tokens with their K experts;
    the shared-read kernels stream every distinct expert once, the per-token kernels every (token,
    expert) pair.  Routing is fixed before the timed region (the FFN alone is timed).  Every path
    replays a HIP graph of 64 calls that cycles through 16 batches of T tokens."""
    import torch
    import bit_expert_dequant_amd as M
    import synth
    from synth.device import build_layer, to_bf16_tensor

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[1]
    H, I, E, K = wl.H, wl.I, wl.E, wl.K
    d = M.make_dims(H, I, E, K)
    dl = build_layer(wl)
    bits = wl.expert_bits()
    blob_bytes = np.array([wl.blob_bytes(int(b)) for b in bits], dtype=np.int64)
    cases = [(T, kind) for T in (2, 4, 8, 16) for kind in ("router", "draft", "same")]
    if a.small_t_case:
        t_s, kind_s = a.small_t_case.split(":")
        cases = [(int(t_s), kind_s)]
    paths = {"both": ["shared", "per_token"], "shared": ["shared"], "per_token": ["per_token"]}[a.small_t_path]
    code = {"shared": M.MOE_FFN_SHARED, "per_token": M.MOE_FFN_PER_TOKEN}
    NB, G = 16, 64
    R = max(1, min(a.steps, 4096) // G)          # replays of the 64-call graph per path
    stream = torch.cuda.current_stream()
    hip = ctypes.CDLL("libamdhip64.so")
    out = []
    for T, kind in cases:
        bank_np = wl.tokens_bank(NB * T)
        x = to_bf16_tensor(bank_np, dev).view(NB, T, H)
        ridx = torch.empty(NB, T, K, dtype=torch.int32, device=dev)
        rw = torch.empty(NB, T, K, dtype=torch.float32, device=dev)
        ws_r = M.workspace(M.MOE_OP_ROUTE, d, T)
        for b in range(NB):
            M.moe_route(d, dl.L, x[b], ridx[b], rw[b], ws=ws_r)
        torch.cuda.synchronize()
        idx_np = np.stack([synth.shared_routing(kind, r, E) for r in ridx.cpu().numpy()])
        idx = torch.from_numpy(idx_np).to(dev)
        distinct = [np.unique(idx_np[b]) for b in range(NB)]
        shared_bytes = float(np.mean([blob_bytes[u].sum() for u in distinct]))
        pair_bytes = float(np.mean([blob_bytes[idx_np[b].reshape(-1)].sum() for b in range(NB)]))
        ws = M.workspace(M.MOE_OP_EXPERT_FFN, d, T)
        y = torch.empty(T, K, H, dtype=torch.float32, device=dev)
        row = {"T": T, "routing": kind, "distinct_experts": float(np.mean([u.size for u in distinct])),
               "distinct_expert_bytes": shared_bytes, "pair_bytes": pair_bytes}
        for path in paths:
            def call(i):
                M.moe_expert_ffn(d, dl.L, x[i % NB], idx[i % NB], y, ws, path=code[path])
            for i in range(max(1, min(a.warmup, 64))):
                call(i)
            torch.cuda.synchronize()
            if a.no_graph:                        # eager issue (for counter runs, one record per launch)
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                for i in range(R * G):
                    call(i)
                ev1.record(stream)
                torch.cuda.synchronize()
                us = ev0.elapsed_time(ev1) * 1e3 / (R * G)
                row[f"{path}_eager_us"] = round(us, 2)
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(G):
                    call(i)
            assert hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()), ctypes.c_void_p(stream.cuda_stream)) == 0
            g.replay()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for _ in range(R):
                g.replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            us = ev0.elapsed_time(ev1) * 1e3 / (R * G)
            row[f"{path}_us"] = round(us, 2)
            row[f"{path}_tok_s"] = round(T / (us * 1e-6), 1)
            del g
        if "shared_us" in row:
            gbps = shared_bytes / (row["shared_us"] * 1e-6) / 1e9
            row["shared_distinct_GBps"] = round(gbps, 1)
            row["shared_frac_of_hbm"] = round(gbps / HBM_PEAK_GBPS, 4)
        if "shared_us" in row and "per_token_us" in row:
            row["speedup_vs_per_token"] = round(row["per_token_us"] / row["shared_us"], 3)
        log(f"[small-t] {row}")
        out.append(row)
    line = {"metric": "expert_ffn_small_t", "unit": "us per call", "higher_is_better": False,
            "data": "synthetic", "steps_per_path": R * G, "dtype": "int4 codes x 16-bit fixed-point activations",
            "config": {"workload": wl.name.split(",")[0], "H": H, "I": I, "E": E, "K": K,
                       "timed": "moe_expert_ffn_path only (routing fixed beforehand)"},
            "cases": out}
    print(json.dumps(line), flush=True)


def main():
    a = parse()
    if a.small_t:
        small_t_bench(a)
        return
    if a.cache:
        cache_bench(a)
        return
    if a.quantize:
        quantize_bench(a)
        return
    if a.retier:
        retier_bench(a)
        return
    if a.copy_calibration:
        copy_calibration()
        return
    if a.traffic_from:
        traffic_from(a.traffic_from, a.traffic_key or f"config{a.config}")
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU (the expert path of one device); multi-GPU runs are not "
              "part of this benchmark: run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_expert_dequant_amd as M
    import synth
    from synth.device import act_f64, build_layer, to_bf16_tensor

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[a.config]
    if a.tokens:
        if wl.n_layers != 1 or not 2 <= a.tokens <= 4096:
            print("--tokens takes 2..4096 and a single-layer config (0, 1, 2 or 4)", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, tokens=a.tokens,
                                 name=f"{wl.name.split(',')[0]}, {a.tokens} tokens per call (batched path)")
    H, I, E, K = wl.H, wl.I, wl.E, wl.K
    d = M.make_dims(H, I, E, K)
    batched = wl.tokens > 1
    log(f"[bench] config {a.config}: {wl.name}")

    t0 = time.time()
    layers = [build_layer(wl, l) for l in range(wl.n_layers)]
    torch.cuda.synchronize()
    log(f"[bench] built {wl.n_layers} layer(s) in {time.time() - t0:.1f}s")
    bits = wl.expert_bits()
    blob_bytes = np.array([wl.blob_bytes(int(b)) for b in bits], dtype=np.int64)
    gu_bytes = np.array([2 * (M.moe_expert_plane_offsets(H, I, int(b))[2]) for b in bits], dtype=np.int64)
    router_bytes = E * H * (2 if wl.router_bf16 else 4)
    norm_bytes = H * 2 if wl.norm else 0

    n_bank = 4096 if not batched else 16 * wl.tokens
    bank_np = wl.tokens_bank(n_bank)
    bank = to_bf16_tensor(bank_np, dev) if wl.x_bf16 else torch.from_numpy(bank_np).to(dev)
    L = [dl.L for dl in layers]

    stream = torch.cuda.current_stream()
    if not batched:
        G = a.graph_steps or (256 if wl.n_layers == 1 else 16)
        ws = M.workspace(M.MOE_OP_LAYER_DECODE, d, 1, wl.n_layers)
        outs = torch.empty(G, H, dtype=torch.float32, device=dev)
        idxs = torch.empty(n_bank, wl.n_layers, K, dtype=torch.int32, device=dev)
        wts = torch.empty(n_bank, wl.n_layers, K, dtype=torch.float32, device=dev)
        residual = wl.norm

        sched = {"separate_kernels": a.schedule == "three_kernels", "single_launch": a.schedule == "single_launch"}

        def step(i, g):
            M.moe_layer_decode(d, L, bank[i % n_bank], outs[g], idxs[i % n_bank], wts[i % n_bank],
                               residual=residual, ws=ws, **sched)
    else:
        T = wl.tokens
        G = a.graph_steps or 1
        ws_r = M.workspace(M.MOE_OP_ROUTE, d, T)
        ws_f = M.workspace(M.MOE_OP_EXPERT_FFN, d, T)
        y = torch.empty(T, K, H, dtype=torch.float32, device=dev)
        outs = torch.empty(T, H, dtype=torch.float32, device=dev)
        idxs = torch.empty(n_bank // T, T, K, dtype=torch.int32, device=dev)
        wts = torch.empty(n_bank // T, T, K, dtype=torch.float32, device=dev)
        bank_b = bank.view(n_bank // T, T, H)

        def step(i, g):
            j = i % (n_bank // T)
            M.moe_route(d, L[0], bank_b[j], idxs[j], wts[j], ws=ws_r)
            M.moe_expert_ffn(d, L[0], bank_b[j], idxs[j], y, ws_f)
            M.moe_combine(y, wts[j], outs)

    # eager warm-up: exactly --warmup steps (at least one, which also sets kernel attributes before
    # any capture); the tokens continue through the bank after the warm-up's
    n_cycle = n_bank if not batched else n_bank // wl.tokens
    for i in range(max(1, a.warmup)):
        step(i, i % G)
    torch.cuda.synchronize()

    # timed region: exactly --steps steps.  Single-token steps replay HIP graphs of G steps (launch
    # bound otherwise), cycling through the bank, plus one graph for the remainder when G does not
    # divide the step count; every graph is uploaded to the device (hipGraphUpload, nothing runs)
    # before the timed region.  Batched steps are issued eagerly unless --graph.
    use_graph = not a.no_graph and (not batched or a.graph)
    graphs = []
    timed_tokens = list(range(a.steps))         # bank position of each timed step (mod the bank)
    if use_graph:
        G = max(1, min(G, a.steps))
        n_full, rem = divmod(a.steps, G)
        n_graphs = max(1, min(n_full, n_cycle // G)) if n_full else 0
        plan = []                                   # graph of each replay, in timed order
        timed_tokens = []
        for gi in range(n_graphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(G):
                    step(gi * G + s, s)
            graphs.append(g)
        for r in range(n_full):
            plan.append(r % n_graphs)
            timed_tokens.extend((r % n_graphs) * G + s for s in range(G))
        if rem:
            timed_tokens.extend(n_full * G + s for s in range(rem))
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(rem):
                    step(n_full * G + s, s)
            graphs.append(g)
            plan.append(len(graphs) - 1)
        hip = ctypes.CDLL("libamdhip64.so")
        for g in graphs:
            rc = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()), ctypes.c_void_p(stream.cuda_stream))
            assert rc == 0, f"hipGraphUpload failed ({rc})"
        torch.cuda.synchronize()
        log(f"[bench] captured {len(graphs)} graph(s): {n_full} replay(s) of {G} step(s)"
            + (f" + one of {rem}" if rem else ""))

    def run():
        if use_graph:
            for gi in plan:
                graphs[gi].replay()
            return a.steps
        for i in range(a.steps):
            step(i, i % G)
        return a.steps

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    w0 = time.perf_counter()
    done = run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / done
    log(f"[bench] timed {done} steps: {ms_per_step * 1e3:.2f} us/step (wall {wall * 1e3:.1f} ms)")

    # exact weight bytes per step from the routing the timed steps used
    idx_h = idxs.cpu().numpy()
    steps_idx = [t % n_cycle for t in timed_tokens]
    if not batched:
        per_tok = {t: float(sum(router_bytes + norm_bytes + blob_bytes[idx_h[t, l]].sum()
                                for l in range(wl.n_layers))) for t in set(steps_idx)}
        bytes_per_step = float(np.mean([per_tok[t] for t in steps_idx]))
        tokens_per_step = 1
    else:
        per_b = {j: float(router_bytes + blob_bytes[np.unique(idx_h[j].reshape(-1))].sum()) for j in set(steps_idx)}
        bytes_per_step = float(np.mean([per_b[j] for j in steps_idx]))
        tokens_per_step = wl.tokens
    tok_s = tokens_per_step / (ms_per_step * 1e-3)
    gbps = bytes_per_step / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] {tok_s:,.0f} tok/s, {gbps:,.1f} GB/s of weights ({gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s)")

    # per-kernel durations: start/stop HIP events that the library's launches stamp with each
    # dispatch's own start and end, on the schedule the timed steps use (router + gate/up, down)
    # and, for the breakdown, on the three-kernel schedule
    roof = None
    kernel_us = {}
    kernel_us_other = {}
    if not batched:
        n_t = min(a.timing_steps, n_bank)

        def timed_pass(schedule):
            names = {"single_launch": ["layer"], "two_launch": ["route_gateup", "down"],
                     "three_kernels": ["router", "gateup", "down"]}[schedule]
            kw = {"separate_kernels": schedule == "three_kernels", "single_launch": schedule == "single_launch"}
            nk = len(names) * wl.n_layers
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nk)] for _ in range(n_t)]
            for row in evs:      # torch creates the HIP event on first record
                for e in row:
                    e.record(stream)
            torch.cuda.synchronize()
            for t in range(n_t):  # ROCm records no event nodes inside captured graphs: eager issue
                M.moe_layer_decode_timed(d, L, bank[t], outs[t % G], evs[t], idxs[t], wts[t], residual=wl.norm,
                                         ws=ws, **kw)
            torch.cuda.synchronize()
            dur = {n: [] for n in names}
            for t in range(n_t):
                for j in range(nk):
                    dur[names[j % len(names)]].append(evs[t][2 * j].elapsed_time(evs[t][2 * j + 1]) * 1e3)
            return {n: float(np.mean(v)) for n, v in dur.items()}

        kernel_us = timed_pass(a.schedule)
        kernel_us_other = {sc: timed_pass(sc) for sc in ("two_launch", "single_launch", "three_kernels") if sc != a.schedule}
        idx_h = idxs.cpu().numpy()          # the timing passes routed tokens 0 .. n_t-1
        if a.schedule == "single_launch":
            # the dominant (only) kernel of a step: router matrix, norm weight and the whole blobs
            # (gate, up and down planes) of the K selected experts
            kb = [router_bytes + norm_bytes + blob_bytes[idx_h[t, l]].sum() for t in range(n_t)
                  for l in range(wl.n_layers)]
            k_us = kernel_us["layer"]
            kname, kdesc = "k_layer", "k_layer (router, top-K, gate/up + SwiGLU, down + combine of the K experts; one launch)"
        else:
            # router + gate/up launch: router matrix, norm weight and the gate and up planes
            kb = [router_bytes + norm_bytes + gu_bytes[idx_h[t, l]].sum() for t in range(n_t)
                  for l in range(wl.n_layers)]
            k_us = kernel_us["route_gateup" if a.schedule == "two_launch" else "gateup"]
            kname, kdesc = "k_route_gateup", "k_route_gateup (router, top-K, gate/up + SwiGLU of the K experts)"
            if a.schedule == "three_kernels":
                kb = [gu_bytes[idx_h[t, l]].sum() for t in range(n_t) for l in range(wl.n_layers)]
                kname, kdesc = "k_gateup", "k_gateup (top-K, gate/up + SwiGLU of the K experts)"
        achieved = float(np.mean(kb)) / (k_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": kdesc,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(kname, f"config{a.config}"),
                "bytes_per_launch": float(np.mean(kb)), "us_per_launch": round(k_us, 3),
                "timing": f"start/stop HIP events of each dispatch (hipExtLaunchKernel), {n_t} eager steps"}
        log(f"[bench] kernel us ({a.schedule}): {kernel_us}; other schedules: {kernel_us_other}; "
            f"{kname} {achieved:,.1f} GB/s")

    if batched:
        # a batch runs several kernels on two streams, so its roofline is the whole batch's: the
        # distinct expert bytes (each read once at best) over the batch time; traffic sums the HBM
        # bytes its kernels read and wrote, from the committed counters
        ks = ("k_router_mfma", "k_group", "k_gu8", "k_dn8", "k_gu_mfma", "k_dn_res")
        tr = [load_traffic(k, f"config{a.config}") for k in ks]
        roof = {"bound": "hbm", "kernel": "whole batch (" + ", ".join(ks) + ", k_combine)",
                "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "traffic": float(sum(tr)) if all(t is not None for t in tr) else None,
                "bytes_per_launch": bytes_per_step, "us_per_launch": round(ms_per_step * 1e3, 3),
                "timing": "HIP events around the timed batches (" + ("graph replays" if use_graph else "eager issue") + ")"}

    # measured read-stream reference: moe_stream_read over 4 GiB (best of 5 after 2 warm-ups)
    sbuf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device=dev)
    sbuf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        M.moe_stream_read(sbuf, sink)
    s_ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        M.moe_stream_read(sbuf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        s_ms.append(e0.elapsed_time(e1))
    del sbuf
    stream_gbps = STREAM_BYTES / (min(s_ms) * 1e-3) / 1e9
    stream = {"GBps": round(stream_gbps, 1), "bytes": STREAM_BYTES, "kernel": "moe_stream_read (16-byte non-temporal "
              "loads from every CU)", "runs_ms": [round(x, 4) for x in s_ms]}
    if roof is not None:
        roof["frac_of_measured_stream"] = round(roof["achieved"] / stream_gbps, 4)
    log(f"[bench] read stream {stream_gbps:,.1f} GB/s over {STREAM_BYTES >> 30} GiB")

    # CPU baseline: the oracle on a bounded sample of the same workload
    cpu = None
    parity = None
    if not a.no_cpu:
        import oracle
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        ols = [oracle.workload_layer(wl, l) for l in range(wl.n_layers)]
        x0 = act_f64(wl, bank_np[0])
        # one token first to size the sample
        t1 = time.perf_counter()
        oracle.stack_token(x0, ols, H, I, K, residual=wl.norm) if wl.n_layers > 1 else \
            oracle.layer_token(x0, ols[0], H, I, K)
        per = time.perf_counter() - t1
        n_s = max(1, min(4096, int(a.cpu_seconds / max(per, 1e-3))))
        if batched:
            n_s = min(n_s, wl.tokens)
        # pre-generate the expert blobs the sample needs, so that only the oracle is timed
        sample = list(range(n_s))
        routed = ({t % n_cycle for t in timed_tokens} | {t % n_cycle for t in range(max(1, a.warmup))}
                  | (set(range(n_t)) if not batched else set()))
        for t in sample:
            if (t if not batched else 0) not in routed:
                continue                     # routing of this token not known yet: generated when used
            for l in range(wl.n_layers):
                for e in (idx_h[t, l] if not batched else idx_h[0, t]):
                    ols[l].blob(int(e))
        t1 = time.perf_counter()
        refs = []
        for t in sample:
            xt = act_f64(wl, bank_np[t])
            if wl.n_layers > 1:
                refs.append(oracle.stack_token(xt, ols, H, I, K, residual=wl.norm)[0])
            else:
                refs.append(oracle.layer_token(xt, ols[0], H, I, K).out)
        cpu_s = time.perf_counter() - t1
        cpu_tok_s = n_s / cpu_s
        cpu = {"value": round(cpu_tok_s, 3), "unit": "tok/s", "cores": cores, "kind": "oracle",
               "sample": f"{n_s} token(s) of this workload through the CPU oracle (fp32 dequant, fp64 "
                         f"accumulation, OpenMP over output rows), timed after host generation of the "
                         f"selected experts; {cpu_s:.1f} s",
               "weight_GBps": round(cpu_tok_s * bytes_per_step / tokens_per_step / 1e9, 4)}
        log(f"[bench] oracle: {cpu_tok_s:.3f} tok/s on {cores} threads ({n_s} tokens, {cpu_s:.1f}s)")
        # parity of the same tokens (GPU eager call vs oracle)
        if not batched:
            errs = []
            o = torch.empty(H, dtype=torch.float32, device=dev)
            for t, ref in zip(sample, refs):
                M.moe_layer_decode(d, L, bank[t], o, residual=wl.norm, ws=ws)
                g = o.cpu().numpy().astype(np.float64)
                errs.append(np.abs(g - ref).max() / (np.linalg.norm(ref) / math.sqrt(ref.size)))
            parity = {"tokens": len(errs), "max_err_over_rms": float(max(errs)), "tolerance": 2e-3,
                      "ok": bool(max(errs) <= 2e-3)}
        else:
            step(0, 0)                       # batch 0 (tokens 0..T-1) through route, grouped FFN, combine
            torch.cuda.synchronize()
            got = outs.cpu().numpy().astype(np.float64)
            errs = [np.abs(got[t] - ref).max() / (np.linalg.norm(ref) / math.sqrt(ref.size))
                    for t, ref in zip(sample, refs)]
            parity = {"tokens": len(errs), "max_err_over_rms": float(max(errs)), "tolerance": 2e-3,
                      "ok": bool(max(errs) <= 2e-3)}

    cfg = {"workload": wl.name, "hidden": H, "intermediate": I, "experts": E, "top_k": K,
           "layers": wl.n_layers, "tokens_per_step": tokens_per_step, "bits": sorted(set(bits.tolist())),
           "group": 64, "graph_steps": G if use_graph else 0, "bank_tokens": n_bank}
    if not batched:
        cfg["schedule"] = a.schedule
    line = {
        "metric": "MoE decode tok/s and weight GB/s (% of HBM peak), 4-bit, 512 experts top-4",
        "value": round(tok_s, 1), "unit": "tok/s", "n_gpus": 1, "steps": done, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i4-dot-i32+f32", "data": "synthetic",
        "dtype_note": ("expert matvecs: 4-bit (or 2-bit) codes times 16-bit fixed-point activation digits per "
                       "32-column slot as exact int32 dot products (v_dot8_i32_i4), scale and bias applied in fp32; "
                       "router: bf16 pairs (hi + lo split when the activation is not bf16) with fp32 accumulation; "
                       "batched busy experts: bf16 MFMA with fp32 accumulation; inputs bf16, outputs fp32"),
        "config": cfg,
        "weight_bytes_per_step": bytes_per_step, "weight_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "stream_frac": round(gbps / stream_gbps, 4), "stream": stream,
        "kernel_us": {k: round(v, 3) for k, v in kernel_us.items()},
        "kernel_us_other_schedules": {sc: {k: round(v, 3) for k, v in ku.items()} for sc, ku in kernel_us_other.items()},
        "roofline": roof, "cpu_baseline": cpu, "parity": parity,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
