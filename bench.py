#!/usr/bin/env python3
"""KDA chunked forward throughput on one MI355X.

A step is one kda_fwd call (schedule, chunk-local and recurrence kernels:
the whole chunked hot path) over one batch of the dense KDA workload
B=2, T=16384, H=16, K=V=128 with fp32 initial/final state, inputs already
resident in HBM.  Prints ONE JSON line: throughput, per-kernel times, the
dominant kernel's roofline fraction and the oracle's CPU rate.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10]

Only one GPU is used; --gpus above 1 exits with an explanation.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix throughput, published
D, C = 128, 64                 # head dim, chunk length
FLOP_PER_TOKEN_HEAD = 6 * D * D + 5 * C * D   # 139,264 (algorithmic, per token and head)
# the sources each kernel's code is built from: a counter-derived traffic figure is reported only while
# they are unchanged
FORWARD_SOURCES = ["chunked_gated_delta_10_amd/csrc/" + f for f in
                   ("kda_chunk.hip", "kda_chunk_job.h", "kda_fused.hip", "kda_recur.hip", "kda_table.hip",
                    "kda_decode.hip", "kda_device.h", "kda_kernels.h")]
BACKWARD_SOURCES = ["chunked_gated_delta_10_amd/csrc/" + f for f in ("kda_bwd.hip", "kda_bwd_pc.hip",
                                                                     "kda_bwd_common.h", "kda_bwd.h",
                                                                     "kda_device.h", "kda_kernels.h")]


def algorithmic_bytes(w, with_state=True, state_bytes=4):
    """Each input read once and each output written once (bytes), split by kernel."""
    tok = w.B * w.T
    qk = 2 * tok * w.H_qk * D * 2
    g = tok * w.H * (D if w.gate_per_channel else 1) * 2
    beta = tok * w.H * 4 if w.delta else 0
    v = tok * w.H * D * 2
    out = tok * w.H * D * 2
    C_ = w.N if w.N else w.B
    state = C_ * w.H * D * D * state_bytes
    s_in = state if w.state_std is not None else 0
    s_out = state if with_state else 0
    local = qk + g + beta + w.H * 4
    chain = v + out + s_in + s_out
    # the fused kernel does both parts in one launch
    return {"kda_chunk_local": local, "kda_recur": chain, "kda_fused": local + chain}


def backward_bytes(w):
    """The backward operator's own inputs read once and outputs written once (bytes): q, k, v, dout (bf16),
    g_raw (bf16, one or 128 per token-head), beta logits (fp32) in; dq, dk, dv, dg_raw, dbeta (fp32) out.
    The gradient kernel touches all of them.  The recomputed forward, the chunk states and the adjoint's
    records are the method's own intermediates and are not counted."""
    tok = w.B * w.T
    C_ = w.N if w.N else w.B
    gw = D if w.gate_per_channel else 1
    reads = 2 * tok * w.H_qk * D * 2 + 2 * tok * w.H * D * 2 + tok * w.H * (2 * gw + 4)
    writes = 2 * tok * w.H_qk * D * 4 + tok * w.H * D * 4 + tok * w.H * (4 * gw + 4)
    return {"kda_bwd_grad": reads + writes, "total": reads + writes + w.H * 8 + C_ * w.H * D * D * 4}


# Algorithmic FLOP per token-head of the backward: the recomputed forward (FLOP_PER_TOKEN_HEAD) plus the
# chunk form's products per 64-token chunk: seven C x D x D (kn dS', dO' S^T, dV S^T, U dS'^T, kn S, and
# the adjoint's qn^T dO', kn^T Z), ten C x C x D (M^T dO', T^T dU, U, dO' U^T, dU (bR)^T, dP kn, dGm kn,
# dP^T qn, qn kn^T, kn kn^T) and two C x C x C (dA = -T^T dT T^T): 548,864 in all.  The per-channel gate's
# backward is counted the same way (its masked Gram products replace the scalar gate's Gram products one for
# one; the per-block decay factors are elementwise work, not counted).
BWD_FLOP_PER_TOKEN_HEAD = FLOP_PER_TOKEN_HEAD + 2 * (7 * C * D * D + 10 * C * C * D + 2 * C ** 3) // C


def sources_hash(kernel="kda_recur"):
    h = hashlib.sha256()
    for p in (BACKWARD_SOURCES if kernel.startswith("kda_bwd") else FORWARD_SOURCES):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("sources_hash") != sources_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_bandwidth(mib=1024, reps=10):
    """Achieved GB/s (read + write) of a plain 1 GiB device-to-device copy: what
    this HBM delivers in practice, next to the 8 TB/s specification."""
    import torch
    n = mib * 1024 * 1024
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def copy_calibration(mib):
    """A plain device-to-device copy of `mib` MiB, five times: the reference
    kernel whose FETCH_SIZE / WRITE_SIZE counters calibrate HBM byte counts."""
    import torch
    n = mib * 1024 * 1024
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n}), flush=True)


def _counter_rows(directory):
    """(kernel name, counter name, value) from every rocprofv3 counter CSV under `directory`."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""), float(r.get("Counter_Value", 0))))
    return rows


def _per_dispatch_kib(rows, counter, match):
    vals = [v for k, c, v in rows if c == counter and match(k)]
    return sum(vals) / len(vals) if vals else None


def traffic_from(root, copy_bytes, workload="kda_dense"):
    """Turn four rocprofv3 --pmc runs into the `workload` entry of profiles/traffic.json
    (other workloads' entries are kept).

    Expects under `root`: pmc_fetch/ and pmc_write/ (FETCH_SIZE, WRITE_SIZE of
    the bench run; pmc_fetch_<workload>/ and pmc_write_<workload>/ for a
    workload other than kda_dense) and cal_fetch/, cal_write/ (the same
    counters over --copy-calibration).  Each counter is scaled by
    ideal/measured of the copy (a copy of N bytes fetches N and writes N
    bytes)."""
    cal_f = _counter_rows(os.path.join(root, "cal_fetch"))
    cal_w = _counter_rows(os.path.join(root, "cal_write"))
    copy_f = max(v for _, c, v in cal_f if c == "FETCH_SIZE")
    copy_w = max(v for _, c, v in cal_w if c == "WRITE_SIZE")
    kf = copy_bytes / (copy_f * 1024.0)
    kw = copy_bytes / (copy_w * 1024.0)
    sfx = "" if workload == "kda_dense" else "_" + workload
    run_f = _counter_rows(os.path.join(root, "pmc_fetch" + sfx))
    run_w = _counter_rows(os.path.join(root, "pmc_write" + sfx))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    out = {}
    if os.path.exists(path):
        with open(path) as fh:
            out = json.load(fh)
    out["_calibration"] = {"copy_bytes": copy_bytes, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
                           "fetch_factor": kf, "write_factor": kw}
    rec = {}
    for kern, tags in (("kda_chunk_local", ("chunk_local_kernel", "chunk_group_kernel")), ("kda_recur", ("recur_",)),
                       ("kda_table", ("table_kernel",)), ("kda_fused", ("fused_kernel",)),
                       ("kda_bwd_coef", ("bwd_coef",)), ("kda_bwd_chains", ("bwd_chain",)),
                       ("kda_bwd_grad", ("bwd_grad",))):
        f = _per_dispatch_kib(run_f, "FETCH_SIZE", lambda k, t=tags: any(x in k for x in t))
        w = _per_dispatch_kib(run_w, "WRITE_SIZE", lambda k, t=tags: any(x in k for x in t))
        if f is None or w is None:
            continue
        rec[kern] = {"fetch_kib": f, "write_kib": w, "hbm_read_bytes": f * 1024 * kf,
                     "hbm_write_bytes": w * 1024 * kw, "hbm_bytes_per_launch": f * 1024 * kf + w * 1024 * kw,
                     "sources_hash": sources_hash(kern)}
    out[workload] = rec
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, w, tokens, tokens_1t):
    """The fp64 oracle, untuned, on the same workload: all chains over the first
    `tokens` tokens of every row with every allowed thread, and the first
    `tokens_1t` tokens of every row on one thread."""
    import numpy as np
    import oracle
    env_threads = os.environ.get("OMP_NUM_THREADS")
    allowed = int(env_threads) if env_threads and env_threads.isdigit() else (os.cpu_count() or 1)
    cores = max(1, min(allowed, w.B * w.H))   # the oracle is parallel over chains only

    def run(n_tok, threads):
        sub = {n: np.ascontiguousarray(inp[n][:, :n_tok]) for n in ("q", "k", "v", "g_raw", "b")}
        t0 = time.perf_counter()
        oracle.kda_fwd(sub["q"], sub["k"], sub["v"], sub["g_raw"], sub["b"], inp["A_log"], inp["scale"],
                       gate_per_channel=w.gate_per_channel, initial_state=inp["initial_state"], nthreads=threads)
        return time.perf_counter() - t0

    dt = run(tokens, cores)
    dt1 = run(tokens_1t, 1)
    return {"value": w.B * tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%s: all %d chains (B=%d x H=%d), first %d of %d tokens per row, fp32 initial state, "
                      "%d threads; %.1f s" % (w.name, w.B * w.H, w.B, w.H, tokens, w.T, cores, dt),
            "single_thread": {"value": w.B * tokens_1t / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": "all %d chains, first %d tokens per row, 1 thread; %.1f s"
                                        % (w.B * w.H, tokens_1t, dt1)},
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "omp_num_threads": env_threads,
            "build": "gcc -O3 -fopenmp (plain C, fp64, token by token)"}


def device_inputs(inp, state_dtype):
    """Copy one batch of seeded host inputs (bf16 bit patterns, fp32, int32) to the GPU."""
    import numpy as np
    import torch

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    d = {n: bf16(inp[n]) for n in ("q", "k", "v", "g_raw")}
    d["b"] = torch.from_numpy(inp["b"]).cuda()
    d["A_log"] = torch.from_numpy(inp["A_log"]).cuda()
    s0 = inp.get("initial_state")
    d["initial_state"] = None if s0 is None else torch.from_numpy(s0).to(device="cuda", dtype=state_dtype)
    cu = inp.get("cu_seqlens")
    d["cu_seqlens"] = None if cu is None else torch.from_numpy(cu).cuda()
    return d


def time_workload(name, steps, warmup, bf16_state=False):
    """Returns (ms per step, per-kernel {name: avg ms}, inputs, workload, percentiles).  With
    bf16_state the initial and final states are bf16 instead of fp32."""
    import torch
    from chunked_gated_delta_10_amd import kda
    from chunked_gated_delta_10_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS[name]
    inp = workload_inputs(name)
    sdt = torch.bfloat16 if bf16_state else torch.float32
    d = device_inputs(inp, sdt)
    if w.backward:
        from chunked_gated_delta_10_amd.inputs import backward_upstream
        dout_bits, _ = backward_upstream(inp, w.seed + 1000)
        dout = torch.from_numpy(dout_bits.view("int16")).view(torch.bfloat16).cuda()
        ws = torch.empty(kda.bwd_workspace_bytes(w.B, w.T, w.H_qk, w.H, w.N), dtype=torch.uint8, device="cuda")

        if w.N:
            def step():
                kda.bwd_varlen(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], dout, d["cu_seqlens"],
                               scale=inp["scale"], initial_state=d["initial_state"], workspace=ws)
        else:
            def step():
                kda.bwd(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], dout, scale=inp["scale"],
                        initial_state=d["initial_state"], workspace=ws)
    elif w.decode:
        st = d["initial_state"]
        out = torch.empty((w.B, w.H, D), dtype=torch.bfloat16, device="cuda")

        if w.delta:
            def step():
                kda.decode_step(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], st, scale=inp["scale"],
                                out=out)
        else:
            def step():
                kda.la_decode_step(d["q"], d["k"], d["v"], d["g_raw"], d["A_log"], st, scale=inp["scale"], out=out)
    else:
        C_ = w.N if w.N else w.B
        out = torch.empty((w.B, w.T, w.H, D), dtype=torch.bfloat16, device="cuda")
        fin = torch.empty((C_, w.H, D, D), dtype=sdt, device="cuda")
        ws = torch.empty(kda.workspace_bytes(w.B, w.T, w.H_qk, w.H, w.N), dtype=torch.uint8, device="cuda")
        if not w.delta:
            def step():
                if w.N:
                    kda.la_fwd_varlen(d["q"], d["k"], d["v"], d["g_raw"], d["A_log"], d["cu_seqlens"],
                                      scale=inp["scale"], initial_state=d["initial_state"], final_state=fin, out=out,
                                      workspace=ws)
                else:
                    kda.la_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["A_log"], scale=inp["scale"],
                               initial_state=d["initial_state"], final_state=fin, out=out, workspace=ws)
        elif w.N:
            def step():
                kda.fwd_varlen(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], d["cu_seqlens"],
                               scale=inp["scale"], initial_state=d["initial_state"], final_state=fin, out=out,
                               workspace=ws)
        else:
            def step():
                kda.fwd(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], scale=inp["scale"],
                        initial_state=d["initial_state"], final_state=fin, out=out, workspace=ws)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # 1. the timed steps.  The library's per-kernel events (diagnostic: they add ~20 us to a step) bracket
    #    the launches of every 10th step only, so the kernel averages come from the timed region itself.
    kda.kernel_timing(False)
    kda.kernel_timing_read()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        kda.kernel_timing(i % 10 == 0)
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kda.kernel_timing(False)
    kt = kda.kernel_timing_read()
    ms = max(wall * 1000.0, e0.elapsed_time(e1)) / steps
    per_kernel = {k: v[0] / v[1] for k, v in kt.items()}
    # 2. per-step spread, with one event between steps (outside the timed region)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    pct = {"p10": round(per_step[int(0.1 * (steps - 1))], 4), "p50": round(per_step[int(0.5 * (steps - 1))], 4),
           "p90": round(per_step[int(0.9 * (steps - 1))], 4)}
    return ms, per_kernel, inp, w, pct


def run_sweep(steps, warmup):
    """Grouped-value-head sweep: every head shape x sequence pattern of the
    forward table on the FlashQLA H200 results page, timed as packed calls.
    Prints one JSON line with a row per (shape, pattern)."""
    import torch
    from chunked_gated_delta_10_amd import kda
    from chunked_gated_delta_10_amd.inputs import SWEEP_HEAD_SHAPES, SWEEP_PATTERNS, cu_seqlens_from_lengths, \
        sweep_inputs
    rows = []
    for h_qk, h_v in SWEEP_HEAD_SHAPES:
        inp = sweep_inputs(h_qk, h_v)
        d = device_inputs(inp, torch.float32)
        print("shape h_qk=%d h_v=%d" % (h_qk, h_v), file=sys.stderr, flush=True)
        for pname, lens in SWEEP_PATTERNS.items():
            T = sum(lens)
            cu = torch.from_numpy(cu_seqlens_from_lengths(lens)).cuda()
            q, k, v, g, b = (d[n][:, :T] for n in ("q", "k", "v", "g_raw", "b"))
            out = torch.empty((1, T, h_v, D), dtype=torch.bfloat16, device="cuda")
            fin = torch.empty((len(lens), h_v, D, D), dtype=torch.float32, device="cuda")
            ws = torch.empty(kda.workspace_bytes(1, T, h_qk, h_v, len(lens)), dtype=torch.uint8, device="cuda")

            def step():
                kda.fwd_varlen(q, k, v, g, b, d["A_log"], cu, scale=inp["scale"], final_state=fin, out=out,
                               workspace=ws)
            for _ in range(warmup):
                step()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            rows.append({"h_qk": h_qk, "h_v": h_v, "seqlens": pname, "tokens": T, "ms": round(ms, 4),
                         "tokens_per_s": round(T / (ms * 1e-3), 1)})
            del out, fin, ws
        del d
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "grouped value heads, scalar decay, K=V=128, no initial state, fp32 final state",
                      "steps": steps, "warmup": warmup, "rows": rows}), flush=True)


# the backward table of the FlashQLA H200 results page: heads x total tokens, split into 8 equal sequences
BWD_SWEEP_HEADS = (32, 48, 64)
BWD_SWEEP_TOKENS = (16384, 32768, 65536, 131072, 262144)


def run_bwd_sweep(steps, warmup):
    """Backward sweep: every (heads, tokens) row of the backward table, 8 sequences, scalar decay, one
    kda.bwd_varlen call per step.  Inputs are drawn on the device from a seeded generator with the
    workloads' distributions (q, k, v, g_raw, beta logits, dout ~ N(0, 1); A_log = 0): the largest rows hold
    several GB per tensor.  Prints one JSON line with a row per (heads, tokens)."""
    import torch
    from chunked_gated_delta_10_amd import kda
    rows = []
    for H in BWD_SWEEP_HEADS:
        for T in BWD_SWEEP_TOKENS:
            gen = torch.Generator(device="cuda")
            gen.manual_seed(3000 + H * 1000 + T // 1024)

            def draw(*shape):
                return torch.randn(*shape, generator=gen, device="cuda", dtype=torch.float32)
            q, k, v = (draw(1, T, H, D).to(torch.bfloat16) for _ in range(3))
            g = draw(1, T, H).to(torch.bfloat16)
            b = draw(1, T, H)
            dout = draw(1, T, H, D).to(torch.bfloat16)
            a = torch.zeros(H, device="cuda")
            cu = torch.arange(0, T + 1, T // 8, dtype=torch.int32, device="cuda")
            ws = torch.empty(kda.bwd_workspace_bytes(1, T, H, H, 8), dtype=torch.uint8, device="cuda")
            print("backward H=%d T=%d" % (H, T), file=sys.stderr, flush=True)

            def step():
                return kda.bwd_varlen(q, k, v, g, b, a, dout, cu, workspace=ws)
            for _ in range(warmup):
                step()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                step()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            rows.append({"heads": H, "tokens": T, "sequences": 8, "ms": round(ms, 4),
                         "tokens_per_s": round(T / (ms * 1e-3), 1)})
            del q, k, v, g, b, dout, ws
            torch.cuda.empty_cache()
    print(json.dumps({"bwd_sweep": "gated delta rule backward, scalar decay, K=V=128, 8 equal sequences, "
                      "fp32 gradients", "steps": steps, "warmup": warmup, "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-tokens", type=int, default=16384, help="tokens per row in the oracle's all-thread sample")
    ap.add_argument("--cpu-tokens-1t", type=int, default=2048, help="tokens per row in the oracle's one-thread sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 counter runs under DIR (no GPU needed)")
    ap.add_argument("--traffic-workload", default="kda_dense",
                    help="the workload the counter runs of --traffic-from were taken on")
    ap.add_argument("--copy-bytes", type=int, default=1024 * 1024 * 1024,
                    help="size of the calibration copy used with --traffic-from")
    ap.add_argument("--only", metavar="WORKLOAD",
                    help="only time one workload (kda_tiny, kda_dense, kda_varlen, gdn_gva, kda_decode, la_varlen, la_decode, kda_bwd, "
                         "gdn_bwd) and print "
                         "its per-kernel averages; for profiling runs")
    ap.add_argument("--sweep", action="store_true",
                    help="only run the grouped-value-head sweep (head shapes x sequence patterns)")
    ap.add_argument("--bwd-sweep", action="store_true",
                    help="only run the backward sweep (heads 32/48/64 x 16k..256k tokens in 8 sequences)")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from, args.copy_bytes, args.traffic_workload)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the KDA path here is built and measured on a single MI355X "
              "(sharding across GPUs is by batch, sequence and head with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    from chunked_gated_delta_10_amd import kda
    kda.load()
    if args.sweep:
        run_sweep(args.steps, args.warmup)
        return
    if args.bwd_sweep:
        run_bwd_sweep(args.steps, args.warmup)
        return
    if args.only:
        ms, per_kernel, _, w, pct = time_workload(args.only, args.steps, args.warmup)
        print(json.dumps({"workload": args.only, "ms_per_step": round(ms, 4), "step_ms_percentiles": pct,
                          "kernels_avg_ms": {k: round(v, 4) for k, v in per_kernel.items()}}), flush=True)
        return

    name = "kda_dense"
    ms, per_kernel, inp, w, pct = time_workload(name, args.steps, args.warmup)
    tokens = w.B * w.T
    value = tokens / (ms / 1000.0)
    alg = algorithmic_bytes(w)
    alg_total = alg["kda_fused"]
    flops = FLOP_PER_TOKEN_HEAD * tokens * w.H
    kernels = {}
    for k, avg in per_kernel.items():
        b = alg.get(k, 0)
        kernels[k] = {"avg_ms": round(avg, 4), "algorithmic_bytes": b,
                      "hbm_gbs": round(b / (avg * 1e-3) / 1e9, 1) if b else None,
                      "hbm_frac": round(b / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if b else None}
    dom = max((k for k in per_kernel if k in alg), key=lambda k: per_kernel[k])
    dom_gbs = alg[dom] / (per_kernel[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic(dom, name), "kernel": dom,
                "algorithmic_bytes_per_launch": alg[dom], "avg_launch_ms": round(per_kernel[dom], 4),
                "step": {"algorithmic_bytes": alg_total,
                         "hbm_frac": round(alg_total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_flop": flops,
                         "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}}
    result = {
        "metric": "KDA fwd tokens/s (B=2,T=16384,H=16,K=V=128) + % of MFMA/HBM roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "B": w.B, "T": w.T, "H": w.H, "H_qk": w.H_qk, "K": D, "V": D,
                   "state": "fp32 in/out", "seed": w.seed},
        "roofline": roofline,
        "kernels": kernels,
        "step_ms_percentiles": pct,
    }
    if not args.no_extra:
        extra = {}
        # the bf16-state variant of the headline shape first, with the headline's step count, before anything
        # else runs (measured after the copy probe or the decode runs, both of its kernels ran ~10% slower,
        # the chunk-local one included, which never touches the state)
        for other in ("kda_dense_bf16_state", "kda_varlen", "gdn_gva", "kda_decode", "la_varlen", "la_decode",
                      "gdn_bwd", "kda_bwd"):
            bf16_state = other.endswith("_bf16_state")
            osteps = args.steps if bf16_state else max(10, args.steps // 5)
            oms, opk, _, ow, _ = time_workload(other.replace("_bf16_state", ""), osteps, 10, bf16_state=bf16_state)
            ab = algorithmic_bytes(ow, state_bytes=2 if bf16_state else 4)
            tok = ow.B if ow.decode else ow.B * ow.T
            tot = backward_bytes(ow)["total"] if ow.backward else ab["kda_fused"]
            extra[other] = {"ms_per_step": round(oms, 4), "tokens_per_s": round(tok / (oms * 1e-3), 1),
                            "algorithmic_bytes": tot,
                            "hbm_frac": round(tot / (oms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "kernels_avg_ms": {k: round(v, 4) for k, v in opk.items()}}
            if ow.backward and "kda_bwd_grad" in opk:
                gb = backward_bytes(ow)["kda_bwd_grad"]
                ach = gb / (opk["kda_bwd_grad"] * 1e-3) / 1e9
                fl = BWD_FLOP_PER_TOKEN_HEAD * tok * ow.H
                extra[other]["roofline"] = {
                    "bound": "hbm", "kernel": "kda_bwd_grad", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": load_traffic("kda_bwd_grad", other),
                    "algorithmic_bytes_per_launch": gb, "avg_launch_ms": round(opk["kda_bwd_grad"], 4),
                    "step": {"algorithmic_flop": fl,
                             "mfma_frac": round(fl / (oms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)}}
        result["other_workloads"] = extra
    # after every timed workload: the probe's 2 GiB of buffers are allocated and freed last
    result["hbm_copy_gbs"] = copy_bandwidth()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w, min(args.cpu_tokens, w.T), min(args.cpu_tokens_1t, w.T))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
