#!/usr/bin/env python3
"""Benchmark of the TurboQuant compressed-KV hot path on one MI355X.

Workload (default): batched decode, batch 32, 8 KV heads, 32 query heads,
d = 128, 32768 compressed tokens per sequence, bf16 K/V/q with 4 outlier
channels per KV head scaled x10, keys 2-bit Lloyd-Max + 1-bit QJL, values
2-bit min/max in groups of 32, fp32 norms, 128-token bf16 ring.

* Bulk encode of all 32 x 32768 tokens (timed separately): encode tokens/s.
* A step = one decode step: append one token per sequence to the ring, then
  query prep, split scan over the compressed cache, combine with the ring.
  W untimed warm-up steps, then K timed steps (ring lengths 1..K).
* value = effective HBM GB/s of the decode step (algorithmic bytes / time).
* roofline = the split-scan kernel: compressed bytes per launch / its average
  duration, from HIP events recorded around that launch on every 4th of the
  timed steps (--time-every).
* cold = more steps, each timed alone right after a 1 GiB device read that
  evicts the 256 MB MALL (the last-level cache), so no step reads a cache
  that a previous step left in it; the scan launch of each is timed too.
* cpu_baseline = the float64 oracle on a bounded sample, on the host cores.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def _hip():
    import torch  # noqa: F401  (loads the HIP runtime)

    h = ctypes.CDLL("libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return h


class Events:
    """Pairs of raw hipEvents for per-kernel timing through the library hook."""

    def __init__(self, n):
        self.h = _hip()
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.h.hipEventCreate(ctypes.byref(a)) == 0 and self.h.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def ms(self, i):
        a, b = self.pairs[i]
        self.h.hipEventSynchronize(b)
        t = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return float(t.value)

    def close(self):
        for a, b in self.pairs:
            self.h.hipEventDestroy(a)
            self.h.hipEventDestroy(b)


def _source_sha(*names):
    """Hash of the named kernel sources and of the build script (which holds
    their compiler flags): a traffic figure taken on other code is not used."""
    h = hashlib.sha256()
    paths = [os.path.join(ROOT, "compressed_kv_decode_tq_amd", "csrc", n) for n in names]
    for path in paths + [os.path.join(ROOT, "compressed_kv_decode_tq_amd", "build.py")]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


SCAN_KERNEL = "scan_mfma_kernel"


def _traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")


def _traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None
    when absent or taken on a different kernel source."""
    path = _traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha") != sha:
        return None
    return t.get("bytes_per_launch")


def _pmc_rows(d: str, counter: str):
    """(kernel name, value) per dispatch from a rocprofv3 --pmc csv run under d."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = (fn, r["Dispatch_Id"])
                name, val = per.get(key, (r["Kernel_Name"], 0.0))
                per[key] = (name, val + float(r["Counter_Value"]))
    return list(per.values())


def pmc_summary(args):
    """Scale the scan kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what
    the same counters read for the known-size probe (y = -x over M MiB: M MiB
    read, M MiB written), and store bytes per launch under profiles/."""
    fetch_dir, write_dir = args.pmc_summary
    with open(os.path.join(fetch_dir, "bench.json")) as f:
        run = json.loads([l for l in f if l.startswith("{")][-1])
    mib = run["copy_probe_mib"]
    probe_bytes = float(mib) * (1 << 20)
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        probe = [v for n, v in rows if "neg" in n.lower()]
        scan = [v for n, v in rows if SCAN_KERNEL in n]
        if not probe or not scan:
            raise SystemExit(f"{counter}: probe dispatches {len(probe)}, scan dispatches {len(scan)}; kernels seen: "
                             + ", ".join(sorted({n[:60] for n, _ in rows})))
        probe_kib = sorted(probe)[len(probe) // 2]
        factor = probe_bytes / (probe_kib * 1024.0)
        scan_kib = sum(scan) / len(scan)
        out[counter] = {"scan_kib_per_dispatch": scan_kib, "scan_dispatches": len(scan),
                        "probe_kib_per_dispatch": probe_kib, "probe_dispatches": len(probe),
                        "factor": factor, "bytes_per_launch": scan_kib * 1024.0 * factor}
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    alg = run["roofline"]["algorithmic_bytes_per_launch"]
    wname = run["config"]["workload"]
    summary = {"kernel": SCAN_KERNEL, "workload": wname, "source_sha": run["roofline"]["source_sha"],
               "bytes_per_launch": int(total), "algorithmic_bytes_per_launch": alg,
               "traffic_over_algorithmic": round(total / alg, 4), "copy_probe_mib": mib,
               "counters": out, "command": args.pmc_command}
    path = _traffic_path(SCAN_KERNEL, wname)
    with open(path, "w") as f:
        json.dump(summary, f, indent=1)
        f.write("\n")
    print(json.dumps(summary, indent=1))


def _cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's
    processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, seconds_budget: float = 25.0):
    """Time the float64 oracle (encode, then dequantize-then-attend decode) on a
    bounded sample: sequence 0, every KV head, its first n tokens."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from compressed_kv_decode_tq_amd import workloads as wl

    pi, s = wl.params(w)
    cb = oracle.lloyd_max(w.d, w.key_mse_bits)
    hi = oracle.lloyd_max(w.d, w.key_mse_bits + 1) if w.key_half else None
    khi = {"centroids_hi": hi.centroids} if hi else {}
    vcb = oracle.lloyd_max(w.d, w.value_bits) if w.value_kind == "mse" else None
    n = min(w.n_tokens, 32768)
    t_enc = t_dec = 0.0
    seqs = 0
    # whole sequences until the budget is spent (at least one)
    while seqs < w.batch and (seqs == 0 or t_enc + t_dec < seconds_budget):
        b = seqs
        q = wl.query(w)[b:b + 1].double().numpy()
        kd, vd = [[]], [[]]
        for h in range(w.h_kv):
            k = wl.slot_tokens(w, "k", b, h, n).double().numpy()
            v = wl.slot_tokens(w, "v", b, h, n).double().numpy()
            t0 = time.perf_counter()
            kc = oracle.encode_keys(k, pi, s, cb.centroids, cb.thresholds, w.scalar_dtype,
                                    **({"centroids_hi": hi.centroids, "thresholds_hi": hi.thresholds} if hi else {}))
            if vcb is None:
                vc = oracle.encode_values_minmax(v, w.value_bits, w.value_group)
            else:
                vc = oracle.encode_values_mse(v, pi, vcb.centroids, vcb.thresholds, w.scalar_dtype)
            t1 = time.perf_counter()
            kd[0].append(oracle.dequantize_keys(kc, pi, s, cb.centroids, **khi))
            vd[0].append(oracle.dequantize_values_minmax(vc, w.value_group) if vcb is None
                         else oracle.dequantize_values_mse(vc, pi, vcb.centroids))
            t_enc += t1 - t0
            t_dec += time.perf_counter() - t1
        t0 = time.perf_counter()
        oracle.decode_attention(q, kd, vd)
        t_dec += time.perf_counter() - t0
        seqs += 1
    per_th = oracle.bytes_per_token_head(oracle.Layout(
        d=w.d, key_mse_bits=w.key_mse_bits, key_qjl=w.key_qjl, value_kind=w.value_kind,
        value_bits=w.value_bits, value_group=w.value_group, scalar_dtype=w.scalar_dtype,
        key_half=w.key_half))["total"]
    nbytes = per_th * w.h_kv * n * seqs
    pools = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in pools] + [1])
    return {
        "value": round(nbytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "cpu_model": _cpu_model(),
        "blas": [{"library": i.get("internal_api"), "threads": i.get("num_threads")} for i in pools
                 if i.get("user_api") == "blas"],
        "sample": f"{seqs} of {w.batch} sequences, all {w.h_kv} KV heads, {n} tokens each: float64 encode "
                  f"({t_enc:.2f} s) and one dequantize-then-attend decode step for their {w.h_q} query heads "
                  f"({t_dec:.2f} s); value = compressed bytes of the sample / decode time",
        "encode_tokens_per_s": round(seqs * n / t_enc, 1),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batched-b32-hkv8-n32768")
    ap.add_argument("--encode-reps", type=int, default=3)
    ap.add_argument("--queries", type=int, default=1,
                    help="causal queries per sequence and step (multi-query decode: T new tokens are appended, "
                         "then all T attend in one call)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain elementwise kernel (y = -x, fp32) over this many MiB, "
                         "the known-size reference for HBM byte counters")
    ap.add_argument("--achievable-mib", type=int, default=1024,
                    help="after the timed steps, time a plain device copy of this many MiB (0: skip); "
                         "its read + write GB/s is reported as the achievable bandwidth")
    ap.add_argument("--time-every", type=int, default=4,
                    help="record the timing events around the decode scan on every k-th timed step: each event "
                         "pair is a pair of packets in the stream that delays the next kernel, so timing every "
                         "step would slow the steps being measured")
    ap.add_argument("--cold-steps", type=int, default=16,
                    help="after the timed steps, this many more steps each timed alone (events around the "
                         "call), each after a 1 GiB device write that evicts the 256 MB MALL; 0: skip")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) "
                         "made with --copy-probe-mib into the decode scan's traffic summary under profiles/")
    ap.add_argument("--pmc-command", default="", help="the rocprofv3 command line, recorded in the summary")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path shards by KV head or sequence with no communication, but no multi-GPU run is made).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from compressed_kv_decode_tq_amd import tq
    from compressed_kv_decode_tq_amd import workloads as wl

    w = wl.by_name(args.workload)
    dev = "cuda"
    if args.copy_probe_mib:
        x = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y
    lay = tq.Layout(head_dim=w.d, key_mse_bits=w.key_mse_bits, key_qjl=w.key_qjl,
                    value_kind=tq.TQ_V_MINMAX if w.value_kind == "minmax" else tq.TQ_V_MSE,
                    value_bits=w.value_bits, value_group=w.value_group,
                    scalar_dtype=tq.TQ_F32 if w.scalar_dtype == "f32" else tq.TQ_F16, key_half=w.key_half)
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    pi, s = wl.params(w)
    prm = tq.Params(lay, pi, s, device=dev)
    k, v = wl.prefill_kv(w)
    k, v = k.to(dev), v.to(dev)
    total_steps = args.warmup + args.steps + args.cold_steps
    nq = args.queries
    ring = w.ring_cap if w.step_mode == "ring" else 0
    if nq < 1 or (ring and nq > ring):
        print(f"--queries must be in 1..{ring or 'any'}", file=sys.stderr)
        sys.exit(2)
    flushes = (total_steps * nq // ring + 1) if ring else 0
    extra = (total_steps * nq if w.step_mode == "encode" else flushes * ring)
    cap = ((w.n_tokens + extra + 31) // 32) * 32
    cache = tq.Cache(lay, w.batch, w.h_kv, cap, device=dev)
    torch.cuda.synchronize()

    # ---- bulk encode
    print("[bench] bulk encode", file=sys.stderr, flush=True)
    pos0 = [0] * w.batch
    tq.encode_kv(prm, k, v, pos0, cache)  # warm-up (also fills the cache)
    torch.cuda.synchronize()
    ev = Events(args.encode_reps)
    t0 = time.perf_counter()
    for r in range(args.encode_reps):
        a, b = ev.pairs[r]
        tq.time_next_launch(tq.TQ_KERNEL_ENCODE_KEYS, a, b)
        tq.encode_kv(prm, k, v, pos0, cache)
    torch.cuda.synchronize()
    enc_wall = (time.perf_counter() - t0) / args.encode_reps
    enc_key_ms = sum(ev.ms(r) for r in range(args.encode_reps)) / args.encode_reps
    ev.close()
    del k, v
    torch.cuda.empty_cache()
    n_vec = w.batch * w.h_kv * w.n_tokens
    enc_tokens_per_s = w.batch * w.n_tokens / enc_wall
    key_flops = 4.0 * w.d * w.d * n_vec  # Pi rotation + QJL projection, 2 d^2 each
    enc_achieved = key_flops / (enc_key_ms * 1e-3) / 1e12

    # ---- decode steps
    print("[bench] decode steps", file=sys.stderr, flush=True)
    if nq == 1:
        qs = [wl.query(w, i).to(dev) for i in range(total_steps)]
    else:
        qs = [torch.stack([wl.query(w, i * nq + t) for t in range(nq)], dim=1).to(dev).contiguous()
              for i in range(total_steps)]
    news = [tuple(x.to(dev).contiguous() for x in wl.step_kv(w, i)) for i in range(total_steps * nq)]
    rk = torch.zeros((w.batch, max(ring, 1), w.h_kv, w.d), dtype=torch.bfloat16, device=dev)
    rv = torch.zeros_like(rk)
    out = torch.empty(tuple(qs[0].shape), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_workspace_bytes(lay, w.batch, w.h_q, w.h_kv, cap, nq), dtype=torch.uint8, device=dev)
    state = {"n_c": w.n_tokens, "n_r": 0}
    per_th = tq.memory_bytes(lay, 1, 1, 1, 0, tq.TQ_BYTES_DATA)
    qbytes = 2 if w.in_dtype == "bf16" else 4

    def step(i, timed_pair=None):
        if ring and state["n_r"] + nq > ring:  # no room for the step's tokens: flush the ring
            tq.encode_kv(prm, rk[:, :state["n_r"]].contiguous(), rv[:, :state["n_r"]].contiguous(),
                         [state["n_c"]] * w.batch, cache)
            state["n_c"] += state["n_r"]
            state["n_r"] = 0
        fused = ring and nq == 1  # one call appends the token and attends
        for t in range(nq):
            kn, vn = news[i * nq + t]
            if ring and not fused:
                tq.ring_append(kn, vn, rk, rv, [state["n_r"]] * w.batch)
                state["n_r"] += 1
            elif w.step_mode == "encode":
                tq.encode_kv(prm, kn, vn, [state["n_c"]] * w.batch, cache)
                state["n_c"] += 1
        if timed_pair is not None:
            tq.time_next_launch(tq.TQ_KERNEL_DECODE_SCAN, *timed_pair)
        if fused:
            kn, vn = news[i]
            tq.decode_attn_append(prm, qs[i], cache, [state["n_c"]] * w.batch, kn, vn, rk, rv,
                                  [state["n_r"]] * w.batch, out=out, workspace=ws)
            state["n_r"] += 1
        else:
            tq.decode_attn(prm, qs[i], cache, [state["n_c"]] * w.batch, rk if ring else None,
                           rv if ring else None, [state["n_r"]] * w.batch if ring else None,
                           out=out, workspace=ws)
        # algorithmic bytes of this step
        by = per_th * w.batch * w.h_kv * state["n_c"]                       # compressed cache
        by += state["n_r"] * w.batch * w.h_kv * w.d * 2 * 2                 # ring K and V
        by += nq * w.batch * w.h_q * w.d * (qbytes + 4)                     # q in, out
        by += 2 * w.d * w.d * 4                                             # Pi, S
        if ring:
            by += nq * w.batch * w.h_kv * w.d * (qbytes + 2) * 2            # new tokens in, ring writes
        return by, per_th * w.batch * w.h_kv * state["n_c"]

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if ring:  # the timed steps start from an empty ring
        state["n_r"] = 0
    every = max(1, args.time_every)
    timed = list(range(0, args.steps, every))  # steps whose scan launch is timed
    ev = Events(len(timed))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tot_bytes = 0
    scan_bytes = []
    for j in range(args.steps):
        by, sb = step(args.warmup + j, ev.pairs[j // every] if j % every == 0 else None)
        tot_bytes += by
        if j % every == 0:
            scan_bytes.append(sb)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scan_ms = [ev.ms(i) for i in range(len(timed))]
    ev.close()
    ms_per_step = wall / args.steps * 1e3
    gbs = tot_bytes / wall / 1e9
    scan_avg_ms = sum(scan_ms) / len(scan_ms)
    scan_avg_bytes = sum(scan_bytes) / len(scan_bytes)
    scan_gbs = scan_avg_bytes / (scan_avg_ms * 1e-3) / 1e9
    scan_sorted = sorted(scan_ms)
    launch_spread = {"median": round(scan_sorted[len(scan_sorted) // 2], 5), "min": round(scan_sorted[0], 5),
                     "max": round(scan_sorted[-1], 5)}
    cold = None
    if args.cold_steps:
        # cold steps: a read of 1 GiB (four times the MALL) before each,
        # outside the events, so the compressed cache comes from HBM; a read
        # leaves clean lines behind, so the step does not also pay for writing
        # back someone else's dirty data
        if ring:
            state["n_r"] = 0
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cev = Events(args.cold_steps)  # the scan launch of every cold step
        cms, cby, csb = [], [], []
        for j in range(args.cold_steps):
            flushed = flush.amax()  # reads all of it; the result stays on the device
            e0.record()
            by, sb = step(args.warmup + args.steps + j, cev.pairs[j])
            e1.record()
            torch.cuda.synchronize()
            cms.append(e0.elapsed_time(e1))
            cby.append(by)
            csb.append(sb)
        cscan = [cev.ms(i) for i in range(args.cold_steps)]
        cev.close()
        del flush, flushed
        torch.cuda.empty_cache()
        order = sorted(range(len(cms)), key=lambda i: cms[i])
        med = order[len(order) // 2]
        sorder = sorted(range(len(cscan)), key=lambda i: cscan[i])
        smed = sorder[len(sorder) // 2]
        cold_scan_gbs = csb[smed] / (cscan[smed] * 1e-3) / 1e9
        cold = {"steps": args.cold_steps, "flush_mib": 1024,
                "ms_per_step": {"median": round(cms[med], 5), "min": round(cms[order[0]], 5),
                                "max": round(cms[order[-1]], 5)},
                "gbs_at_median": round(cby[med] / (cms[med] * 1e-3) / 1e9, 2),
                "scan_ms": {"median": round(cscan[smed], 5), "min": round(cscan[sorder[0]], 5),
                            "max": round(cscan[sorder[-1]], 5)},
                "scan_gbs_at_median": round(cold_scan_gbs, 1),
                "scan_frac_at_median": round(cold_scan_gbs / HBM_PEAK_GBS, 4),
                "note": "each step timed alone with events around the call, after a 1 GiB device read "
                        "that evicts the 256 MB MALL; scan_ms: the scan launch of the same steps"}
    copy_gbs = None
    if args.achievable_mib:
        # a plain device copy (read and write) on the same device: what HBM
        # delivers to the simplest streaming kernel
        x = torch.ones(args.achievable_mib << 18, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        copy_gbs = 2.0 * x.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del x, y
        torch.cuda.empty_cache()
    sha = _source_sha("tq_decode_mfma.hip", "tq_decode.hip", "tq_common.h", "tq_internal.h")
    generic = os.environ.get("TQ_DECODE_PATH") == "generic"
    # the committed counter summaries are single-query runs
    traffic = None if generic or args.queries != 1 else _traffic(SCAN_KERNEL, w.name, sha)
    scan_kernel_name = ("scan_kernel (VALU split scan over the compressed cache)"
                        if generic
                        else "scan_mfma_kernel (int8-MFMA split scan over the compressed cache)")

    res = {
        "metric": "decode-attn effective HBM GB/s (% peak) and encode tokens/s, 1xMI355X",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8-mfma+f32",
        "data": "synthetic (seeded N(0,1) K/V/q with outlier channels; no dataset, no weights)",
        "config": {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_kv": w.h_kv, "head_dim": w.d,
                   "n_compressed": w.n_tokens, "ring_cap": w.ring_cap,
                   "ring_tokens_in_timed_steps": f"{nq}..{min(args.steps * nq, ring)}" if ring else "none",
                   "queries_per_step": nq,
                   "key_bits": f"{w.key_mse_bits + 0.5 * w.key_half:g}-bit Lloyd-Max + {w.key_qjl}-bit QJL",
                   "value_code": f"{w.value_bits}-bit {w.value_kind}" + (f" g{w.value_group}" if w.value_kind == "minmax" else ""),
                   "scalars": w.scalar_dtype, "bytes_per_token_head": per_th, "parallelism": "single GPU"},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"kernel": scan_kernel_name, "bound": "hbm",
                     "achieved": round(scan_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_ms": round(scan_avg_ms, 5), "launch_ms": launch_spread,
                     "timed_launches": f"{len(scan_ms)} of {args.steps} (every {every})",
                     "algorithmic_bytes_per_launch": int(scan_avg_bytes), "source_sha": sha},
        "cold": cold,
        "achievable": None if copy_gbs is None else {
            "copy_gbs": round(copy_gbs, 1), "copy_mib": args.achievable_mib,
            "scan_over_copy": round(scan_gbs / copy_gbs, 4),
            "note": "device copy y = x (read + write) timed with torch events after the decode steps"},
        "encode": {"tokens_per_s": round(enc_tokens_per_s, 1), "ms_per_bulk_encode": round(enc_wall * 1e3, 3),
                   "tokens": w.batch * w.n_tokens, "key_vectors": n_vec,
                   "roofline": {"kernel": "encode_rot_kernel (keys: Pi and S' rotations)", "bound": "mfma",
                                "achieved": round(enc_achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": round(enc_achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                                "avg_launch_ms": round(enc_key_ms, 4),
                                "note": "algorithmic flops 4 d^2 per key vector; the split-bf16 passes issue 2.5x that"}},
    }
    if args.copy_probe_mib:
        res["copy_probe_mib"] = args.copy_probe_mib
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
