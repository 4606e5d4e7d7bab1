#!/usr/bin/env python3
"""Benchmark of the KDA forward operator on one MI355X.

    python bench.py [--steps K] [--warmup W] [--decode-steps D] [--no-cpu-baseline]

One step is one kda_chunk_fwd over the 128K-token workload (B=1, H=32,
T=131072, d_k=d_v=128, bf16 q/k/v, fp32 gates, random initial state,
chunk 64), inputs resident in HBM. After the prefill steps, the decode
workload (64 sequences x 32 heads, fp32 state cache, D successive
kda_decode_step calls with fresh inputs per step) is timed the same way.

Prints ONE JSON line: prefill Mtokens/s as `value`, its roofline (HBM bytes
and MFMA FLOPs of the algorithm), the decode us/step with its HBM roofline,
and the fp64 CPU oracle timed on a bounded sample of the same inputs.
Timing uses HIP events recorded on the stream the kernels are launched on.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
C = 64


def prefill_bytes(T, H, K, V, N, in_bytes=2, out_bytes=2, s0=True, sT=True):
    """Algorithmic HBM bytes of one prefill: q, k, v, log_alpha, beta read
    once, o written once, initial state read, final state written."""
    per_tok_head = (2 * K + V) * in_bytes + 4 * K + 4 + V * out_bytes
    return T * H * per_tok_head + N * H * K * V * 4 * (int(s0) + int(sT))


def prefill_flops_per_token_head(K, V, c=C):
    """FLOPs of the chunk algorithm per token-head, counting only triangles
    that exist: K c(c-1) for A (strict lower), 2K c(c+1) for P and the WY
    factor T (K e^G), 2V c(c+1) for T V and P U', c^3/3 for the triangular
    inverse and 6 c K V for the three c x K x V products with the state."""
    return (K * c * (c - 1) + 2 * K * c * (c + 1) + 2 * V * c * (c + 1)
            + c ** 3 / 3 + 6 * c * K * V) / c


def fused_prefill_bytes(T, H, K, V, N, in_bytes=2, out_bytes=2, epilogue=True):
    """Algorithmic bytes of the extended call with gate pre-activations: q, k, v,
    gate_x ([T,H,K]), beta_y ([T,H]) and, with the output epilogue, the output gate
    z ([T,H,V]) read once in the input type, o written once, the d_v norm weight,
    and the initial and final states."""
    per_tok_head = (3 * K + V + 1 + (V if epilogue else 0)) * in_bytes + V * out_bytes
    return T * H * per_tok_head + (4 * V if epilogue else 0) + N * H * K * V * 4 * 2


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def decode_bytes(B, H, K, V, in_bytes=2, out_bytes=2):
    return B * H * (2 * K * V * 4 + 2 * K * in_bytes + K * 4 + 4 + V * in_bytes + V * out_bytes)


ROOT = os.path.dirname(os.path.abspath(__file__))
SOURCES = ("gated_delta_rule_10_amd/csrc/kda_prefill_mfma.hip", "gated_delta_rule_10_amd/csrc/kda_decode.hip",
           "gated_delta_rule_10_amd/csrc/kda_api.cpp")


def source_hash():
    """Hash of the kernel and ABI sources without comments and blank lines, so
    that a profile stays valid across edits that change no code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(profile):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary in
    profiles/<profile>, if it was taken on the kernel sources as they are now
    (same source hash); None otherwise."""
    path = os.path.join(ROOT, "profiles", profile)
    try:
        text = open(path).read()
    except OSError:
        return None
    want = source_hash()
    if f"code sha256 (kda_prefill_mfma.hip, kda_decode.hip, kda_api.cpp; comments stripped): {want}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:"):
            return int(line.split(":")[1])
    return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_threads():
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


def cpu_baseline_prefill(d, target_s=12.0):
    """Time the fp64 oracle on the first tokens of the same 128K sequence, all
    heads; the token count is grown until one run takes at least target_s / 2
    (or covers the whole sequence)."""
    import numpy as np
    import oracle
    threads = _cpu_threads()
    tokens, elapsed = 256, 0.0
    while True:
        sub = {n: d[n][:tokens].float().cpu().numpy() for n in ("q", "k", "v", "log_alpha", "beta")}
        s0 = d["initial_state"].cpu().numpy()
        t0 = time.perf_counter()
        ref = oracle.prefill(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"],
                             np.array([0, tokens], np.int32), 1.0, s0, nthreads=threads)
        elapsed = time.perf_counter() - t0
        if elapsed >= target_s / 2 or tokens >= d["q"].shape[0]:
            break
        tokens = min(d["q"].shape[0], int(tokens * max(2.0, min(16.0, target_s / max(elapsed, 1e-3)))))
    out = dict(value=tokens / elapsed / 1e6, unit="Mtokens/s", cores=threads, cpu=_cpu_model(), kind="oracle",
               sample=f"fp64 oracle, first {tokens} tokens of the 128K sequence, all 32 heads, "
                      f"{elapsed:.2f} s", seconds=elapsed)
    return out, (ref if tokens >= d["q"].shape[0] else None)


def err_over_rms(got, ref, bf16_out):
    """Max-abs error over RMS(ref); for bf16 outputs, the error beyond half a bf16
    ulp of the value (rounding the exact value to bf16 alone costs that much)."""
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    if bf16_out:
        ax = np.maximum(np.abs(ref), np.abs(got))
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
        d = np.maximum(d - np.where(ax > 0, np.exp2(e - 8.0), 0.0), 0.0)
    return float(d.max() / max(float(np.sqrt(np.mean(ref * ref))), 1e-300))


def cpu_baseline_decode(d, target_s=5.0):
    """Time the fp64 oracle on the first decode steps of the same workload: one
    step sets how many run in about target_s (at most the steps drawn)."""
    import numpy as np
    import oracle
    threads = _cpu_threads()
    state = d["state"].cpu().numpy().astype(np.float64)
    avail = d["q"].shape[0]

    def step(s, host):
        oracle.decode(host["q"][s], host["k"][s], host["v"][s], host["log_alpha"][s],
                      host["beta"][s], state, nthreads=threads)

    host = {n: d[n][:1].float().cpu().numpy() for n in ("q", "k", "v", "log_alpha", "beta")}
    t0 = time.perf_counter()
    step(0, host)
    first = time.perf_counter() - t0
    s0 = 1 if avail > 1 else 0  # the timed steps follow the untimed one when there are more
    steps = int(max(1, min(avail - s0, target_s / max(first, 1e-4))))
    host = {n: d[n][s0:s0 + steps].float().cpu().numpy() for n in ("q", "k", "v", "log_alpha", "beta")}
    t0 = time.perf_counter()
    for s in range(steps):
        step(s, host)
    el = time.perf_counter() - t0
    return dict(value=el / steps * 1e6, unit="us/step", cores=threads, cpu=_cpu_model(), kind="oracle",
                sample=f"fp64 oracle, {steps} decode steps of B=64, H=32, d=128 (after one untimed step), "
                       f"{el:.2f} s", seconds=el)


def oracle_sample_parity(d, o, sT, seqs, heads):
    """The CPU baseline on a sample of a workload: the fp64 oracle on sequences `seqs`
    and heads `heads` of the device inputs d (timed, on the host's threads), and the
    error of the GPU outputs o (bf16) and final states sT on the same sample."""
    import numpy as np
    import torch
    import oracle
    threads = _cpu_threads()
    cu = d["cu_seqlens"].cpu().numpy().astype(np.int64)
    tok = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs]).astype(np.int64)
    tok_t = torch.from_numpy(tok).to(d["q"].device)
    hd = torch.tensor(heads, device=d["q"].device)
    sq = torch.tensor(seqs, device=d["q"].device)

    def sub(x):
        return x.index_select(0, tok_t).index_select(1, hd).float().cpu().numpy()

    lens = [int(cu[n + 1] - cu[n]) for n in seqs]
    cu_sub = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    s0 = d["initial_state"]
    s0_sub = None if s0 is None else s0.index_select(0, sq).index_select(1, hd).cpu().numpy()
    t0 = time.perf_counter()
    ro, rs = oracle.prefill(sub(d["q"]), sub(d["k"]), sub(d["v"]), sub(d["log_alpha"]), sub(d["beta"]), cu_sub, 1.0,
                            s0_sub, nthreads=threads)
    elapsed = time.perf_counter() - t0
    go, gs = sub(o), sT.index_select(0, sq).index_select(1, hd).cpu().numpy()
    return {"o_err_over_rms": round(err_over_rms(go, ro, True), 6),
            "final_state_err_over_rms": round(err_over_rms(gs, rs, False), 6), "tol": 2e-2,
            "oracle_seconds": round(elapsed, 2), "cores": threads}


def time_prefill_workload(name, steps, warmup, dev, stream, check=None):
    """Median time of kda_chunk_fwd on a named synthetic workload (inputs resident on the
    device); with check(lengths) -> (sequences, heads, description), also the last timed
    call's outputs on that sample against the fp64 oracle."""
    import torch
    from gated_delta_rule_10_amd import inputs, kda

    torch.cuda.empty_cache()
    w = inputs.WORKLOADS[name]
    d1 = inputs.device_workload_inputs(name, device=dev)
    T1, H1 = d1["q"].shape[0], d1["q"].shape[1]
    K1, V1 = d1["q"].shape[2], d1["v"].shape[2]
    N1 = d1["cu_seqlens"].numel() - 1
    o1 = torch.empty((T1, H1, V1), dtype=torch.bfloat16, device=dev)
    s1 = torch.empty((N1, H1, K1, V1), dtype=torch.float32, device=dev)
    ws1 = torch.empty(kda.kda_chunk_fwd_workspace_size(N1, T1, H1, K1, V1, torch.bfloat16), dtype=torch.uint8,
                      device=dev)

    def call():
        kda.kda_chunk_fwd(d1["q"], d1["k"], d1["v"], d1["log_alpha"], d1["beta"], d1["cu_seqlens"],
                          initial_state=d1["initial_state"], final_state=s1, o=o1, workspace=ws1, stream=stream)

    ms1 = time_calls(call, steps, warmup, stream)
    torch.cuda.synchronize()
    b1 = prefill_bytes(T1, H1, K1, V1, N1, s0=d1["initial_state"] is not None)
    g1 = b1 / (ms1 / 1e3) / 1e9
    lens = d1["cu_seqlens"].diff().tolist()
    par = None
    if check is not None:
        seqs, heads, what = check(lens)
        par = oracle_sample_parity(d1, o1, s1, seqs, heads)
        par["sample"] = what + ": the timed calls' outputs against the fp64 oracle (bf16 o: error beyond half a bf16 ulp)"
    del d1, o1, s1, ws1
    torch.cuda.empty_cache()
    return par, {
        "entry": "kda_chunk_fwd",
        "workload": f"{name}: {N1} sequence(s), {T1} tokens (lengths {min(lens)}-{max(lens)}), H={H1}, "
                    f"d_k={K1}, d_v={V1}, bf16, log alpha = -{w['decay_scale']} softplus(x), "
                    f"initial state {w['init']}",
        "ms_per_step": round(ms1, 3), "value": round(T1 / (ms1 / 1e3) / 1e6, 3), "unit": "Mtokens/s",
        "roofline": {"bound": "hbm", "achieved": round(g1, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(g1 / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": b1}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the extended-entry-point measurements")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this many MiB (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this operator benchmark runs on one GPU only; "
                                   "--gpus must be 1"}))
        sys.exit(2)

    import torch
    from gated_delta_rule_10_amd import inputs, kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load_library()
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---- prefill: the 128K-token workload ----------------------------------
    name = "long_128k"
    w = inputs.WORKLOADS[name]
    d = inputs.device_workload_inputs(name, device=dev)
    T, H, K, V = d["q"].shape[0], w["H"], w["K"], w["V"]
    N = d["cu_seqlens"].shape[0] - 1
    o = torch.empty((T, H, V), dtype=torch.bfloat16, device=dev)
    sT = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)

    def step():
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"],
                          initial_state=d["initial_state"], final_state=sT, o=o, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    # the timed calls' own outputs (later variants reuse the buffers), for the parity check
    gpu_out = None if args.no_cpu_baseline else (o.float().cpu(), sT.cpu())
    total_ms = ev[0].elapsed_time(ev[-1])
    ms = total_ms / args.steps
    mtok = T / (ms / 1e3) / 1e6
    nbytes = prefill_bytes(T, H, K, V, N)
    flops = prefill_flops_per_token_head(K, V) * T * H
    gbs = nbytes / (ms / 1e3) / 1e9
    tflops = flops / (ms / 1e3) / 1e12
    result = {
        "metric": "KDA prefill Mtokens/s (H=32,d=128,T=128K) + decode us/step (B=64)",
        "value": round(mtok, 3),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic (seeded torch draws on the device)",
        "config": {"workload": "long_128k: 1 sequence x 131072 tokens, H=32, d_k=d_v=128, "
                               "bf16 q/k/v, fp32 log_alpha/beta, fp32 initial+final state, "
                               "chunk 64, o bf16",
                   "global_batch": 1, "seq_len": T, "parallelism": "none (one GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("prefill_long_128k.md"),
                     "kernel": "kda_chunk_fwd (one call: offsets, prep, map pass with the outputs of segment 0, prefix, output pass)",
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"achieved_tflops": round(tflops, 2), "peak_tflops": PEAK_BF16_TFLOPS,
                 "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                 "flops_per_launch": flops, "count": "triangular-aware, C=64"},
        "arith": "bf16 q/k/v in; fp16 MFMA operands with fp32 accumulation; fp32 gates, "
                 "decay factors, triangular inverse and state; o rounded to bf16",
        "prefill_ms": {"min": round(min(per), 4), "max": round(max(per), 4),
                       "median": round(sorted(per)[len(per) // 2], 4)},
    }

    # ---- the same workload through kda_chunk_fwd_ex: bf16 gate pre-activations
    # (log alpha = -0.05 softplus(x), beta = sigmoid(y)) and the RMS-norm + sigmoid
    # output-gate epilogue fused into the output pass
    if not args.no_variants:
        gen = torch.Generator(device=dev)
        gen.manual_seed(20)
        gx = torch.randn((T, H, K), generator=gen, device=dev).to(torch.bfloat16)
        by = torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16)
        z = torch.randn((T, H, V), generator=gen, device=dev).to(torch.bfloat16)
        nw = 1 + 0.1 * torch.randn((V,), generator=gen, device=dev)

        def fused():
            kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], d["cu_seqlens"], gate_x=gx, beta_y=by,
                                 gate_scale=0.05, norm=True, norm_eps=1e-6, norm_weight=nw, out_gate=z,
                                 out_gate_act="sigmoid", initial_state=d["initial_state"], final_state=sT,
                                 o=o, stream=stream)

        def gates_only():
            kda.kda_chunk_fwd_ex(d["q"], d["k"], d["v"], d["cu_seqlens"], gate_x=gx, beta_y=by,
                                 gate_scale=0.05, initial_state=d["initial_state"], final_state=sT, o=o,
                                 stream=stream)

        result["variants"] = {}
        for vname, fn, entry, epi in (
                ("fused_gates_norm_gate", fused,
                 "kda_chunk_fwd_ex (gate_x, beta_y bf16; norm + weight; sigmoid output gate)", True),
                ("fused_gates", gates_only, "kda_chunk_fwd_ex (gate_x, beta_y bf16; no epilogue)", False)):
            fms = time_calls(fn, args.steps, args.warmup, stream)
            fb = fused_prefill_bytes(T, H, K, V, N, epilogue=epi)
            fgbs = fb / (fms / 1e3) / 1e9
            result["variants"][vname] = {
                "entry": entry, "workload": name, "ms_per_step": round(fms, 4),
                "value": round(T / (fms / 1e3) / 1e6, 3), "unit": "Mtokens/s",
                "roofline": {"bound": "hbm", "achieved": round(fgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(fgbs / PEAK_HBM_GBS, 4), "algorithmic_bytes_per_launch": fb}}
        del gx, by, z

    cpu_d = None
    if not args.no_cpu_baseline:
        cpu_d = {n: d[n] for n in ("q", "k", "v", "log_alpha", "beta", "initial_state")}
        cpu_d["gpu_o"], cpu_d["gpu_s"] = gpu_out
    del d, o, sT

    # ---- the same operator on the other prefill workloads: one 1,048,576-token
    # sequence (the pages' 1M point), 16 packed sequences of mixed lengths, and
    # 4 x 4,096 tokens at H = 16
    # (with the CPU baseline, each also checked against the oracle on a sample: heads 0
    # and 31 of the 1M-token sequence; the shortest and longest of the 16 sequences on
    # all 32 heads)
    import numpy as np
    checks = {
        "long_1m": lambda lens: ([0], [0, 31], "heads 0 and 31 of the 1,048,576-token sequence"),
        "varlen_512k": lambda lens: (sorted({int(np.argmin(lens)), int(np.argmax(lens))}), list(range(32)),
                                     f"the shortest ({min(lens)} tokens) and longest ({max(lens)} tokens) "
                                     "sequences, all 32 heads"),
    }
    sample_parity = {}
    if not args.no_variants:
        for wname, wsteps, wwarm in (("long_1m", 3, 1), ("varlen_512k", 5, 2), ("mid_4x4k", 20, 3)):
            chk = None if args.no_cpu_baseline else checks.get(wname)
            par, result["variants"][wname] = time_prefill_workload(wname, wsteps, wwarm, dev, stream, chk)
            if par is not None:
                sample_parity[wname] = par

    # ---- decode: 64 sequences x 32 heads, fp32 cache -----------------------
    # The figure of record reads the state from HBM: four independent 128 MiB
    # caches are cycled step by step (512 MiB, twice the 256 MB Infinity Cache),
    # so the state a step reads was last touched three steps (800 MB of traffic)
    # earlier, as it is in a model whose every layer keeps its own cache. The
    # steps on one cache, which can stay in the Infinity Cache, are a variant.
    if not args.prefill_only:
        steps = args.decode_steps
        dd = inputs.device_workload_inputs("decode_b64", device=dev, steps=steps)
        Bd, Hd, Kd, Vd = 64, 32, 128, 128
        state = dd["state"]
        od = torch.empty((Bd, Hd, Vd), dtype=torch.bfloat16, device=dev)
        dbytes = decode_bytes(Bd, Hd, Kd, Vd)
        NCACHE = 4
        caches = [state] + [state.clone() for _ in range(NCACHE - 1)]

        def dsteps(cache_of, n0, n):
            for s in range(n0, n0 + n):
                kda.kda_decode_step(dd["q"][s % steps], dd["k"][s % steps], dd["v"][s % steps],
                                    dd["log_alpha"][s % steps], dd["beta"][s % steps], cache_of(s), o=od,
                                    stream=stream)

        def timed(cache_of):
            dsteps(cache_of, 0, min(args.warmup, steps) + NCACHE)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dsteps(cache_of, 0, steps)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / steps

        us = timed(lambda s: caches[s % NCACHE])
        warm_us = timed(lambda s: state)
        del caches
        # the one-cache steps from a captured HIP graph as well
        Gp = min(steps, 64)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for s in range(Gp):
                kda.kda_decode_step(dd["q"][s], dd["k"][s], dd["v"][s], dd["log_alpha"][s], dd["beta"][s],
                                    state, o=od)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        pgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph):
            for s in range(Gp):
                kda.kda_decode_step(dd["q"][s], dd["k"][s], dd["v"][s], dd["log_alpha"][s], dd["beta"][s],
                                    state, o=od)
        graph_us = time_calls(pgraph.replay, max(1, steps // Gp), 1, stream) * 1e3 / Gp
        del pgraph
        dgbs = dbytes / (us / 1e6) / 1e9
        wgbs = dbytes / (warm_us / 1e6) / 1e9
        result["decode"] = {
            "value": round(us, 3), "unit": "us/step", "steps": steps,
            "workload": "decode_b64: B=64, H=32, d_k=d_v=128, fp32 state cache (128 MiB), bf16 q/k/v/o, "
                        "fresh inputs every step; four caches cycled step by step (512 MiB), so the "
                        "state comes from HBM",
            "roofline": {"bound": "hbm", "achieved": round(dgbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(dgbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_b64.md"),
                         "algorithmic_bytes_per_launch": dbytes},
            "variants": {"mall_resident": {
                "entry": "kda_decode_step, one 128 MiB cache every step (it fits the 256 MB Infinity Cache)",
                "value": round(warm_us, 3), "unit": "us/step", "graph_us_per_step": round(graph_us, 3),
                "achieved_gbs": round(wgbs, 1),
                "note": "not an HBM figure: part of the state may come from the Infinity Cache"}},
        }
        if not args.no_variants:
            gen = torch.Generator(device=dev)
            gen.manual_seed(21)
            dgx = torch.randn((min(steps, 64), Bd, Hd, Kd), generator=gen, device=dev).to(torch.bfloat16)
            dby = torch.randn((min(steps, 64), Bd, Hd), generator=gen, device=dev).to(torch.bfloat16)
            dz = torch.randn((min(steps, 64), Bd, Hd, Vd), generator=gen, device=dev).to(torch.bfloat16)
            dnw = 1 + 0.1 * torch.randn((Vd,), generator=gen, device=dev)
            it = [0]

            def dfused():
                s = it[0] % dgx.shape[0]
                it[0] += 1
                # on the current stream, which is the capture stream while the graph is recorded
                kda.kda_decode_step_ex(dd["q"][s], dd["k"][s], dd["v"][s], state, gate_x=dgx[s], beta_y=dby[s],
                                       gate_scale=0.1, norm=True, norm_weight=dnw, out_gate=dz[s],
                                       out_gate_act="sigmoid", o=od)

            dus = time_calls(dfused, steps, min(args.warmup, steps), stream) * 1e3
            # the same steps from a captured HIP graph (no per-call host work)
            G = dgx.shape[0]
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                it[0] = 0
                for _ in range(G):
                    dfused()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            it[0] = 0
            with torch.cuda.graph(graph):
                for _ in range(G):
                    dfused()
            reps = max(1, steps // G)
            gus = time_calls(graph.replay, reps, 1, stream) * 1e3 / G
            result["decode"]["variants"]["fused_gates_norm_gate"] = {
                "entry": "kda_decode_step_ex (gate_x, beta_y bf16; norm + weight; sigmoid output gate), one cache",
                "value": round(gus, 3), "unit": "us/step", "timing": f"HIP graph of {G} steps, {reps} replays",
                "eager_us_per_step": round(dus, 3)}
            del graph
        if cpu_d is not None:
            result["decode"]["cpu_baseline"] = cpu_baseline_decode(dd)
        del dd, state

    if cpu_d is not None:
        result["cpu_baseline"], ref = cpu_baseline_prefill(cpu_d)
        if ref is not None:
            result["parity"] = {
                "o_err_over_rms": round(err_over_rms(cpu_d["gpu_o"].numpy(), ref[0], True), 6),
                "final_state_err_over_rms": round(err_over_rms(cpu_d["gpu_s"].numpy(), ref[1], False), 6),
                "tol": 2e-2, "sample": "the timed calls' outputs, all 32 heads and 131072 tokens, against the "
                                      "fp64 oracle of the CPU baseline (bf16 o: error beyond half a bf16 ulp)"}
    if sample_parity:
        result.setdefault("parity", {})["workloads"] = sample_parity
    result["source_sha256"] = source_hash()  # the hash the profiles under profiles/ record
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
