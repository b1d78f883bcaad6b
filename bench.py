#!/usr/bin/env python3
"""Benchmark of one key-eviction pass (score + top-B select + compaction) on one MI355X.

A step is one pass over the Qwen3-8B-shaped layer workload (8 KV heads x 32768 bf16 keys,
d = 128, theta = 1e6, offsets 2^0..2^16, B = 2048): one tri_prune_pass call (score with the
fused radix histogram, candidates, then threshold, output slots and row gather in one kernel), on
the current stream. Inputs are resident in HBM; to keep the 256 MB Infinity Cache from serving
them, consecutive steps rotate over ``--rotate`` distinct copies of the inputs and outputs (about
135 MB per copy), and the score kernel alone rotates over at least 8 copies of the keys (67 MB
each): with 4 copies or fewer it runs measurably faster, served in part from the Infinity Cache.

Prints ONE JSON line (rank 0). Extra legs:
  --pmc-copy       only run a plain device copy of known size (for counter calibration)
  --no-cpu         skip the CPU baseline
  --no-large       skip the large device-generated workloads (all layers, ragged batch, chat pass 0)
  --no-steady      skip the chat steady state
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E spec
SCORE_WARMUP = 1000  # untimed launches of the score kernel before its timed ones
METRIC = "cached keys scored+selected/sec and achieved HBM GB/s (% of peak), 32k keys"


def algorithmic_bytes(wl, n_keys_total, n_units):
    """Bytes the method must move per pass: every K row and position read, the kept V rows
    read, the kept K/V rows and positions written."""
    e = wl.elem_bytes
    B = wl.budget
    return {
        "K": n_keys_total * wl.d * e,
        "pos": n_keys_total * 4,
        "V_kept": n_units * B * wl.d * e,
        "writes": n_units * B * (2 * wl.d * e + 4),
    }


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ["score.hip", "score_device.h", "tri_device.h", "tri_internal.h"]:
        with open(os.path.join(ROOT, "rotary_frequency_key_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_hash):
    """HBM traffic per score launch from the committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "score_kernel_c2_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*([0-9a-f]+)", txt)
    m_val = re.search(r"traffic bytes per launch \(scaled\):\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_val or m_hash.group(1) != kernel_hash:
        return None
    return float(m_val.group(1))


def cpu_baseline(wl, P, budget, seconds_target=10.0):
    """The fp64 oracle (folded score + select + gather), unchanged, over the units of the
    workload, one process per unit up to the host cores; repeated until ~seconds_target."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    units = list(range(len(P["row_off"]) - 1))
    cores = max(1, min(len(units), len(os.sched_getaffinity(0)), 16))
    jobs = []
    for i in units:
        a, b = P["row_off"][i], P["row_off"][i + 1]
        jobs.append((P["centers"][i], P["keys"][a:b], P["values"][a:b], P["pos"][a:b],
                     int(P["t"][i]), wl.d, wl.theta, budget))
    passes = 0
    keys = 0
    with ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_job, jobs[:cores]))  # start the workers
        t0 = time.perf_counter()
        while True:
            list(ex.map(_oracle_job, jobs))
            passes += 1
            keys += int(P["row_off"][-1])
            if time.perf_counter() - t0 >= seconds_target or passes >= 50:
                break
        dt = time.perf_counter() - t0
    return {"value": keys / dt, "unit": "keys/s", "cores": cores, "kind": "oracle",
            "sample": f"{passes} full passes over all {len(units)} units ({keys} keys) of the same "
                      f"workload, fp64 NumPy folded score + select + gather, {dt:.1f} s"}


def _oracle_job(args):
    import oracle as O

    center, keys, values, pos, t, d, theta, budget = args
    O.unit_pass(center, keys, values, pos, t, d, theta, O.power_of_two_offsets(), budget)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=6)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--pmc-copy", action="store_true")
    ap.add_argument("--no-steady", action="store_true")
    ap.add_argument("--no-large", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every unit is scored, selected and compacted "
              "independently, so more GPUs would each run this same pass on their own units. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import rotary_frequency_key_amd as tri
    from synthgen import pack_units, workload

    dev = torch.device("cuda:0")

    if args.pmc_copy:
        # plain device copy of a known size for FETCH_SIZE / WRITE_SIZE calibration
        n = 256 << 20
        a = torch.ones(n // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    wl = workload("c2")
    P = pack_units(wl, workers=min(8, len(os.sched_getaffinity(0))))
    U = wl.n_units
    R = int(P["row_off"][-1])
    B = wl.budget
    max_rows = int(np.diff(P["row_off"]).max())
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, np.array([1 << j for j in range(17)]), P["centers"])

    def dev_bf16(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    copies = []
    for _ in range(args.rotate):
        c = {
            "K": dev_bf16(P["keys"]),
            "V": dev_bf16(P["values"]),
            "pos": torch.from_numpy(P["pos"]).to(dev),
            "row_off": torch.from_numpy(P["row_off"]).to(dev),
            "t": torch.from_numpy(P["t"]).to(dev),
            "mu": torch.from_numpy(mu).to(dev),
            "ws": tri.make_workspace(U, max_rows, dev),
            "scores": torch.empty(R, dtype=torch.float32, device=dev),
            "kept_idx": torch.empty((U, B), dtype=torch.int32, device=dev),
            "kept_cnt": torch.empty(U, dtype=torch.int32, device=dev),
            "K_out": torch.empty((U, B, wl.d), dtype=torch.bfloat16, device=dev),
            "V_out": torch.empty((U, B, wl.d), dtype=torch.bfloat16, device=dev),
            "pos_out": torch.empty((U, B), dtype=torch.int32, device=dev),
        }
        c["plan"] = tri.PassPlan(c["K"], c["V"], c["pos"], c["row_off"], max_rows, c["t"], c["mu"],
                                 wl.theta, B, ws=c["ws"], scores=c["scores"], kept_idx=c["kept_idx"],
                                 kept_cnt=c["kept_cnt"], K_out=c["K_out"], V_out=c["V_out"],
                                 pos_out=c["pos_out"])
        copies.append(c)
    plans = [c["plan"] for c in copies]

    def step(i):
        plans[i % len(plans)].run()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole passes
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} passes: {ms * 1e3:.2f} us/pass (host wall {t_wall / args.steps * 1e6:.2f} us)",
          file=sys.stderr, flush=True)

    # score kernel alone (with its histogram, as in the pass): K launches back to back on the
    # launch stream, bracketed by HIP events on that stream; arguments are marshalled once so
    # that the host enqueues faster than the GPU runs. A separate workspace takes the histograms;
    # the keys rotate over at least 8 copies (536 MB), which the Infinity Cache cannot hold.
    ws_score = tri.make_workspace(U, max_rows, dev)
    kcopies = [(c["K"], c["scores"]) for c in copies]
    while len(kcopies) < 8:
        kcopies.append((dev_bf16(P["keys"]), torch.empty(R, dtype=torch.float32, device=dev)))
    splans = [tri.ScorePlan(k, copies[0]["row_off"], max_rows, copies[0]["pos"], copies[0]["t"], copies[0]["mu"],
                            wl.theta, scores=sc, ws=ws_score) for k, sc in kcopies]
    # untimed: at least SCORE_WARMUP launches (a few ms), enough for the launch-to-launch time to
    # settle; with 20-200 it still varied by up to 15% between runs
    for i in range(max(args.warmup, SCORE_WARMUP)):
        splans[i % len(splans)].run()
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record()
    for i in range(args.steps):
        splans[i % len(splans)].run()
    e3.record()
    torch.cuda.synchronize()
    del splans, ws_score, kcopies
    k_score = e2.elapsed_time(e3) * 1e3 / args.steps

    # the same pass with the keys read as stored after the rotary rotation (TRI_KEYS_ROTATED):
    # one coefficient vector per unit, no positions and no trigonometry per key. The key bits
    # are the same copies (their values do not change the work).
    rot = tri.TRI_BANDS_INTERLEAVED | tri.TRI_KEYS_ROTATED
    rplans = [tri.PassPlan(c["K"], c["V"], c["pos"], c["row_off"], max_rows, c["t"], c["mu"], wl.theta, B,
                           ws=c["ws"], scores=c["scores"], kept_idx=c["kept_idx"], kept_cnt=c["kept_cnt"],
                           K_out=c["K_out"], V_out=c["V_out"], pos_out=c["pos_out"], layout=rot)
              for c in copies]
    ws_rs = tri.make_workspace(U, max_rows, dev)
    rsplans = [tri.ScorePlan(c["K"], c["row_off"], max_rows, None, c["t"], c["mu"], wl.theta,
                             scores=c["scores"], ws=ws_rs, layout=rot) for c in copies]
    rot_times = []
    for plist in (rplans, rsplans):
        for i in range(args.warmup):
            plist[i % len(plist)].run()
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        for i in range(args.steps):
            plist[i % len(plist)].run()
        eb.record()
        torch.cuda.synchronize()
        rot_times.append(ea.elapsed_time(eb) * 1e3 / args.steps)
    del rplans, rsplans, ws_rs
    rot_pass_us, rot_score_us = rot_times

    alg = algorithmic_bytes(wl, R, U)
    alg_total = sum(alg.values())
    secs = ms * 1e-3
    keys_per_s = R / secs
    gbps = alg_total / secs / 1e9
    score_bytes = alg["K"] + alg["pos"]
    score_gbps = score_bytes / (k_score * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = read_traffic(khash)

    result = {
        "metric": METRIC,
        "value": keys_per_s,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-shaped layer: 8 KV heads x 32768 keys, d=128, bf16 K/V, "
                        "theta=1e6, D=2^0..2^16, B=2048",
            "units": U, "keys_per_unit": max_rows, "d": wl.d, "kv_dtype": "bf16",
            "budget": B, "theta": wl.theta,
            "cold_cache": f"{args.rotate} rotating input/output copies",
        },
        "hbm_gbps": gbps,
        "hbm_frac_of_peak": gbps / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_pass": alg_total,
        "score_kernel_us": k_score,
        "roofline": {
            "bound": "hbm",
            "kernel": "score_kernel<bf16, interleaved, 128>",
            "achieved": score_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": score_gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": score_bytes,
        },
        "kernel_source_sha256_16": khash,
        "rotated_keys": {
            "note": "same workload, keys read as stored after the rotary rotation",
            "us_per_pass": rot_pass_us,
            "keys_per_s": R / (rot_pass_us * 1e-6),
            "score_kernel_us": rot_score_us,
            "score_kernel_gbps": alg["K"] / (rot_score_us * 1e-6) / 1e9,
        },
    }
    # the max-over-offsets variant on the same workload: centers E[q] (not folded), 17 offsets;
    # the pass as score_max + select + compact, and the score kernel alone (its histograms go to a
    # workspace of their own, as for the averaged score)
    D = np.array([1 << j for j in range(17)], dtype=np.int64)
    centers = torch.from_numpy(np.ascontiguousarray(P["centers"], dtype=np.float32)).to(dev)
    ws_max = tri.make_workspace(U, max_rows, dev)

    def max_plan(c, ws):
        return tri.MaxPassPlan(c["K"], c["V"], c["pos"], c["row_off"], max_rows, c["t"], centers, wl.theta, D, B,
                               ws=ws, scores=c["scores"], kept_idx=c["kept_idx"], kept_cnt=c["kept_cnt"],
                               K_out=c["K_out"], V_out=c["V_out"], pos_out=c["pos_out"])

    mpass = [max_plan(c, c["ws"]) for c in copies]
    mscore = [max_plan(c, ws_max) for c in copies]
    max_times = []
    nsteps = max(10, args.steps // 4)
    for call in ([p.run for p in mpass], [p.score for p in mscore]):
        for i in range(args.warmup):
            call[i % len(call)]()
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        for i in range(nsteps):
            call[i % len(call)]()
        eb.record()
        torch.cuda.synchronize()
        max_times.append(ea.elapsed_time(eb) * 1e3 / nsteps)
    del mpass, mscore, ws_max
    result["max_over_offsets"] = {
        "note": "same workload, maximum over the 17 offsets of the unfolded score; pass = three calls",
        "us_per_pass": max_times[0],
        "keys_per_s": R / (max_times[0] * 1e-6),
        "score_kernel_us": max_times[1],
        "band_offset_evals_per_s": R * (wl.d // 2) * D.size / (max_times[1] * 1e-6),
    }

    # the same passes issued over two streams, as a serving loop that compresses layer after
    # layer may issue them: copy c always runs on stream c % 2 (its workspace and outputs are
    # only ever used on that stream), so one pass's select overlaps the next pass's score.
    # Reported beside the single-stream figure, which stays the headline.
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    oplans = []
    for ci, c in enumerate(copies):
        with torch.cuda.stream(streams[ci % 2]):
            oplans.append(tri.PassPlan(c["K"], c["V"], c["pos"], c["row_off"], max_rows, c["t"], c["mu"],
                                       wl.theta, B, ws=c["ws"], scores=c["scores"], kept_idx=c["kept_idx"],
                                       kept_cnt=c["kept_cnt"], K_out=c["K_out"], V_out=c["V_out"],
                                       pos_out=c["pos_out"]))
    if len(oplans) % 2 == 0:
        torch.cuda.synchronize()
        for i in range(args.warmup):
            oplans[i % len(oplans)].run()
        torch.cuda.synchronize()
        main = torch.cuda.current_stream()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record(main)
        for st in streams:
            st.wait_event(ea)
        for i in range(args.steps):
            oplans[i % len(oplans)].run()
        for st in streams:
            ev = torch.cuda.Event()
            ev.record(st)
            main.wait_event(ev)
        eb.record(main)
        torch.cuda.synchronize()
        ov_us = ea.elapsed_time(eb) * 1e3 / args.steps
        result["two_streams"] = {
            "note": "same passes, consecutive passes on two streams (independent inputs and outputs)",
            "us_per_pass": ov_us,
            "keys_per_s": R / (ov_us * 1e-6),
        }
    del oplans, streams

    # free the pass copies before the larger caches
    del copies, plans
    torch.cuda.empty_cache()
    if not args.no_large:
        for name in LARGE_WORKLOADS:
            result[name] = large_workload(tri, torch, dev, args, name)
            torch.cuda.empty_cache()
    if not args.no_steady:
        result["steady_state"] = steady_state(tri, torch, dev, args)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl, P, B, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# Large workloads, each in one tri_prune_pass call, generated on the device (synthgen.device: the
# host recipe's centers, device-drawn noise). Each moves gigabytes per pass, far beyond the
# 256 MB Infinity Cache, so no copies rotate.
LARGE_WORKLOADS = {
    "all_layers": ("c3", "36 layers x 8 KV heads x 32768 keys (Qwen3-8B shape), bf16, B=2048, "
                         "10% flat heads; 256 units or more: one select workgroup per unit"),
    "ragged_batch": ("c4", "16 sequences x 32 layers x 8 KV heads (Llama-3-8B shape), 8192..65536 keys "
                           "per sequence, bf16, B=2048"),
    "chat_pass0": ("c5", "4 sequences x 64 layers x 8 KV heads (Qwen3-32B shape), 131072 + 1024 keys, "
                         "bf16, B=12000: candidates, resolve and emit"),
}


def large_workload(tri, torch, dev, args, name):
    """One large workload: the pass and the score kernel alone, in keys/s and algorithmic GB/s."""
    from synthgen import workload
    from synthgen.device import device_workload

    wl_name, note = LARGE_WORKLOADS[name]
    wl = workload(wl_name)
    W = device_workload(wl, dev)
    U = wl.n_units
    R = int(W["row_off"][-1])
    B = wl.budget
    max_rows = int(W["lengths"].max())
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, np.array([1 << j for j in range(17)]), W["centers"])
    mu_d = torch.from_numpy(mu).to(dev)
    ws = tri.make_workspace(U, max_rows, dev)
    scores = torch.empty(R, dtype=torch.float32, device=dev)
    outs = dict(kept_idx=torch.empty((U, B), dtype=torch.int32, device=dev),
                kept_cnt=torch.empty(U, dtype=torch.int32, device=dev),
                K_out=torch.empty((U, B, wl.d), dtype=torch.bfloat16, device=dev),
                V_out=torch.empty((U, B, wl.d), dtype=torch.bfloat16, device=dev),
                pos_out=torch.empty((U, B), dtype=torch.int32, device=dev))
    plan = tri.PassPlan(W["K"], W["V"], W["pos"], W["row_off_d"], max_rows, W["t_d"], mu_d, wl.theta, B,
                        ws=ws, scores=scores, **outs)
    ws_s = tri.make_workspace(U, max_rows, dev)
    splan = tri.ScorePlan(W["K"], W["row_off_d"], max_rows, W["pos"], W["t_d"], mu_d, wl.theta, scores=scores,
                          ws=ws_s)
    steps = max(5, min(args.steps, 20))
    times = []
    for run in (plan.run, splan.run):
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        for _ in range(steps):
            run()
        eb.record()
        torch.cuda.synchronize()
        times.append(ea.elapsed_time(eb) * 1e3 / steps)
    alg = algorithmic_bytes(wl, R, U)
    alg_total = sum(alg.values())
    us, score_us = times
    del W, plan, splan, ws, ws_s, scores, outs
    return {"workload": note, "units": U, "keys": R, "us_per_pass": us, "keys_per_s": R / (us * 1e-6),
            "algorithmic_bytes_per_pass": alg_total,
            "hbm_gbps": alg_total / (us * 1e-6) / 1e9,
            "hbm_frac_of_peak": alg_total / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "score_kernel_us": score_us,
            "score_kernel_gbps": (alg["K"] + alg["pos"]) / (score_us * 1e-6) / 1e9,
            "note": "one tri_prune_pass; generated on the device"}


def steady_state(tri, torch, dev, args, base_units=32, replicas=64, chunk=1024):
    """Chat steady state (the 64-layer x 8-head x 4-sequence shape, B = 12000): every unit holds
    the B rows kept by earlier passes, at sparse positions below 131072, and a 1024-row prefill
    chunk at the next positions; tri_prune_inplace prunes the 13024 rows back to B in place.

    The cache is synthetic: base_units units are generated (keys around a center as in every
    workload, B positions drawn without replacement from 0..131071, then 1024 new ones) and
    tiled replicas times on the device, 2048 units in all. Before each timed pass a fresh chunk
    is copied into rows B.. of every unit (untimed, events bracket the pass only)."""
    from synthgen import unit_inputs, workload

    wl = workload("c5")
    B = wl.budget
    C = B + chunk
    t_now = 131072 + chunk
    Ks, Vs, Ps, Cs, pool_k, pool_v = [], [], [], [], [], []
    for u in range(base_units):
        x = unit_inputs(wl, u, C + chunk)  # C rows for the cache, one more chunk for the pool
        rng = np.random.default_rng([wl.seed, 0xC5, u])
        old = np.sort(rng.choice(131072, size=B, replace=False)).astype(np.int32)
        Ks.append(x["keys"][:C]); Vs.append(x["values"][:C]); Cs.append(x["center"])
        Ps.append(np.concatenate([old, np.arange(131072, t_now, dtype=np.int32)]))
        pool_k.append(x["keys"][C:]); pool_v.append(x["values"][C:])

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    U = base_units * replicas
    K = dev16(np.stack(Ks)).repeat(replicas, 1, 1).reshape(U * C, wl.d)
    V = dev16(np.stack(Vs)).repeat(replicas, 1, 1).reshape(U * C, wl.d)
    pos = torch.from_numpy(np.stack(Ps)).to(dev).repeat(replicas, 1).reshape(U * C)
    chunk_k = dev16(np.stack(pool_k)).repeat(replicas, 1, 1)
    chunk_v = dev16(np.stack(pool_v)).repeat(replicas, 1, 1)
    chunk_p = torch.arange(131072, t_now, dtype=torch.int32, device=dev).repeat(U, 1)
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, np.array([1 << j for j in range(17)]), np.stack(Cs))
    mu = torch.from_numpy(mu).to(dev).repeat(replicas, 1, 1).contiguous()
    row_off = torch.arange(0, (U + 1) * C, C, dtype=torch.int64, device=dev)
    t = torch.full((U,), t_now, dtype=torch.int32, device=dev)
    plan = tri.InplacePlan(K, V, pos, row_off, C, t, mu, wl.theta, B,
                           ws=tri.make_inplace_workspace(U, C, B, dev),
                           scores=torch.empty(U * C, dtype=torch.float32, device=dev),
                           kept_cnt=torch.empty(U, dtype=torch.int32, device=dev))
    K3, V3, P2 = K.view(U, C, wl.d), V.view(U, C, wl.d), pos.view(U, C)

    def append():
        K3[:, B:].copy_(chunk_k)
        V3[:, B:].copy_(chunk_v)
        P2[:, B:].copy_(chunk_p)

    steps = max(3, min(args.steps, 20))
    for _ in range(2):
        append()
        plan.run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        append()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        plan.run()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1e3)
    rows = U * C
    # algorithmic bytes: every key row and position read, each moved row's K, V and position
    # read and written (at most one chunk per unit)
    moved_max = U * chunk * (2 * wl.d * 2 + 4) * 2
    return {"units": U, "rows_per_unit": C, "budget": B, "chunk": chunk, "us_per_pass": us,
            "keys_per_s": rows / (us * 1e-6),
            "algorithmic_gbps": (rows * (wl.d * 2 + 4) + moved_max) / (us * 1e-6) / 1e9,
            "note": f"{base_units} generated units tiled {replicas}x; chunk copy untimed"}


if __name__ == "__main__":
    main()
