"""Benchmark of the gated-delta-rule hot path on one MI355X.

One "step" is one chunked-prefill call of the 27B-shaped workload
(B=1, T=16384, 16 key heads shared 1:3 by 48 value heads, d=128, bf16 q/k/v,
fp32 gates and state, chunk 64).  ``value`` is prefill tokens/s.  The decode
half of the metric (B=64 sequences, same heads, one token per step for 1000
steps, fp32 state updated in place) is timed in the same run and reported
under "decode" as state-update HBM GB/s and tokens/s.  The same prefill call
storing a state checkpoint every 512 tokens (gdn_chunk_prefill_ckpt) is timed
too and reported under "checkpoints", and the call that forms the gates from
raw projections (gdn_chunk_prefill_gated) under "raw_gates", and decode with
4 tokens per call (gdn_decode_multi) under "decode_multi", a packed batch
of 8 sequences of different lengths (gdn_chunk_prefill_varlen) under "varlen",
the 0.8B head shape (T=2048, 16/16 heads) under "prefill_0.8b", and a
131,072-token prompt processed as 256 consecutive 512-token calls carrying the
state from call to call through a bank that keeps the state at every call
boundary, under "long_context".

Inputs are seeded synthetic tensors already resident in HBM when the timed
region starts.  Kernel time comes from HIP events recorded on the stream the
kernels are launched on.  The fp64 oracle (test infrastructure) is timed on
host cores on a bounded sample of the same prefill workload as "cpu_baseline".

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from linear_attention_recurrence_04_amd import inputs as gi  # noqa: E402

METRIC = "GDN prefill tokens/s (Hk16/Hv48, d=128) + decode state-update HBM GB/s"

# MI355X published peaks
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VALU_PEAK_TFLOPS = 157.3

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_recurrence_04_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work (per call), stated once here and in the design notes
# ---------------------------------------------------------------------------


def prefill_useful_flops(p) -> float:
    """Useful flops of the chunked method per call: per token and value head
    6 dk dv (three state products) + C (dk + 2 dv) (triangular halves of the
    intra-chunk products) + 2 C dk / r (the two Gram products, once per key head)."""
    r = p.Hv // p.Hk
    per = 6 * p.dk * p.dv + p.chunk * (p.dk + 2 * p.dv) + 2 * p.chunk * p.dk / r
    return per * p.B * p.T * p.Hv


def prefill_bytes(p, h0: bool = True) -> float:
    """Minimum HBM bytes of one call: read q, k, v, log_g, beta, h0; write o, hT."""
    s = 2 if p.dtype == "bf16" else 4
    per_token = 2 * p.Hk * p.dk * s + p.Hv * p.dv * s + p.Hv * p.dv * s + 8 * p.Hv
    state = p.B * p.Hv * p.dk * p.dv * 4
    return p.B * p.T * per_token + state * (1 + (1 if h0 else 0))


def decode_bytes(d) -> float:
    """Minimum HBM bytes of one decode step: the state read and written once,
    plus q, k, v, o (bf16) and log_g, beta (fp32)."""
    s = 2 if d.dtype == "bf16" else 4
    return 2 * d.B * d.Hv * d.dk * d.dv * 4 + d.B * (2 * d.Hk * d.dk * s + 2 * d.Hv * d.dv * s + 8 * d.Hv)


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_traffic(kernel_key: str, src_hash: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    or None when absent or taken on a different kernel source."""
    path = os.path.join(PROFILES, "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    ent = tab.get(kernel_key)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return float(ent["bytes_per_launch"])


# ---------------------------------------------------------------------------


def time_stream(torch, fn, steps: int):
    """Run fn() `steps` times between two events on the current stream."""
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop)  # ms


def bench_prefill(torch, gdn, p, steps, warmup, ckpt_every: int = 0, raw_gates: bool = False):
    """ms per prefill call; with ckpt_every > 0 the call also stores the state
    every ckpt_every tokens (gdn_chunk_prefill_ckpt); with raw_gates the gates
    are formed in the kernels from raw projections (gdn_chunk_prefill_gated)."""
    log(f"prefill workload {p.name}: generating inputs")
    inp = gi.make_prefill(p, 0)
    dev = {n: torch.from_numpy(inp[n]).cuda() for n in ("q", "k", "v", "log_g", "beta", "h0")}
    for n in ("q", "k", "v"):
        dev[n] = dev[n].to(torch.bfloat16) if p.dtype == "bf16" else dev[n]
    out = torch.empty((p.B, p.T, p.Hv, p.dv), dtype=dev["q"].dtype, device="cuda")
    hT = torch.empty((p.B, p.Hv, p.dk, p.dv), dtype=torch.float32, device="cuda")
    prob = gdn.make_problem(p.B, p.T, p.Hk, p.Hv, p.dk, p.dv, chunk=p.chunk,
                            dtype=gdn.GDN_DTYPE_BF16 if p.dtype == "bf16" else gdn.GDN_DTYPE_F32)
    ws_bytes = gdn.gdn_chunk_prefill_workspace_bytes(prob)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    if raw_gates:
        rg = {n: torch.from_numpy(x).cuda() for n, x in gi.make_raw_gates((p.B, p.T), p.Hv, 0).items()}

        def call():
            gdn.gdn_chunk_prefill_gated(dev["q"], dev["k"], dev["v"], rg["a"], rg["b"], rg["A_log"],
                                        rg["dt_bias"], dev["h0"], chunk=p.chunk, out=out, hT=hT,
                                        workspace=ws)
    elif ckpt_every:
        nck = -(-p.T // ckpt_every)
        ck = torch.empty((p.B, nck, p.Hv, p.dk, p.dv), dtype=torch.float32, device="cuda")

        def call():
            gdn.gdn_chunk_prefill_ckpt(dev["q"], dev["k"], dev["v"], dev["log_g"], dev["beta"],
                                       dev["h0"], ckpt_every=ckpt_every, chunk=p.chunk, out=out,
                                       hT=hT, h_ckpt=ck, workspace=ws)
    else:
        def call():
            gdn.gdn_chunk_prefill(dev["q"], dev["k"], dev["v"], dev["log_g"], dev["beta"],
                                  dev["h0"], chunk=p.chunk, out=out, hT=hT, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    log(f"prefill{' with checkpoints every %d' % ckpt_every if ckpt_every else ''}"
        f"{' with raw gates' if raw_gates else ''}: timing {steps} steps")
    ms = time_stream(torch, call, steps)
    return ms / steps, prob


VARLEN_MIX = [4096, 3000, 2500, 2048, 1800, 1500, 900, 540]   # 16384 tokens, 8 sequences


def bench_prefill_varlen(torch, gdn, p, steps, warmup):
    """ms per packed call of the sequence mix VARLEN_MIX at the 27B head shape."""
    log(f"varlen prefill {VARLEN_MIX}: generating inputs")
    seqs = [gi.make_prefill(p, 100 + i, T=L) for i, L in enumerate(VARLEN_MIX)]
    dev = {n: torch.from_numpy(np.concatenate([s[n][0] for s in seqs], axis=0)).cuda()
           for n in ("q", "k", "v", "log_g", "beta")}
    for n in ("q", "k", "v"):
        dev[n] = dev[n].to(torch.bfloat16)
    h0 = torch.from_numpy(np.concatenate([s["h0"] for s in seqs], axis=0)).cuda()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(VARLEN_MIX)]), dtype=torch.int32, device="cuda")
    total = int(sum(VARLEN_MIX))
    out = torch.empty((total, p.Hv, p.dv), dtype=torch.bfloat16, device="cuda")
    hT = torch.empty_like(h0)
    prob = gdn.make_problem(len(VARLEN_MIX), max(VARLEN_MIX), p.Hk, p.Hv, p.dk, p.dv, chunk=p.chunk)
    ws = torch.empty(max(gdn.gdn_chunk_prefill_workspace_bytes(prob), 1), dtype=torch.uint8,
                     device="cuda")

    def call():
        gdn.gdn_chunk_prefill_varlen(dev["q"], dev["k"], dev["v"], dev["log_g"], dev["beta"], cu,
                                     max(VARLEN_MIX), h0, chunk=p.chunk, out=out, hT=hT,
                                     workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    log(f"varlen prefill: timing {steps} steps")
    return time_stream(torch, call, steps) / steps



LONG_DISTINCT_SEGMENTS = 32   # seeded 512-token segments, cycled over the 256 calls


def bench_long_context(torch, gdn, p, warmup):
    """Long prompt processed as consecutive fixed-size calls carrying the fp32
    state: call c reads its initial state from slot c - 1 of a checkpoint bank
    (zeros for the first call) and writes its final state to slot c, so the
    bank holds the state at every call boundary.  Returns ms for the whole
    prompt."""
    Tc = p.extra["call_tokens"]
    ncalls = p.T // Tc
    log(f"long context {p.name}: generating {LONG_DISTINCT_SEGMENTS} segments")
    segs = []
    for c in range(LONG_DISTINCT_SEGMENTS):
        s = gi.make_long_segment(p, 0, c)
        dv = {n: torch.from_numpy(s[n]).cuda() for n in ("q", "k", "v", "log_g", "beta")}
        for n in ("q", "k", "v"):
            dv[n] = dv[n].to(torch.bfloat16)
        segs.append(dv)
    bank = torch.empty((ncalls, p.B, p.Hv, p.dk, p.dv), dtype=torch.float32, device="cuda")
    out = torch.empty((p.B, Tc, p.Hv, p.dv), dtype=torch.bfloat16, device="cuda")
    prob = gdn.make_problem(p.B, Tc, p.Hk, p.Hv, p.dk, p.dv, chunk=p.chunk)
    ws = torch.empty(max(gdn.gdn_chunk_prefill_workspace_bytes(prob), 1), dtype=torch.uint8,
                     device="cuda")

    def prompt():
        for c in range(ncalls):
            s = segs[c % LONG_DISTINCT_SEGMENTS]
            gdn.gdn_chunk_prefill(s["q"], s["k"], s["v"], s["log_g"], s["beta"],
                                  bank[c - 1] if c else None, chunk=p.chunk, out=out, hT=bank[c],
                                  workspace=ws)

    for _ in range(max(warmup, 1)):
        prompt()
    torch.cuda.synchronize()
    log(f"long context: timing 3 prompts of {ncalls} calls")
    return time_stream(torch, prompt, 3) / 3, ncalls

def measured_peaks(torch):
    """Achievable figures on this GPU, for fractions against measured as well as
    published peaks: a 2 GiB device copy (read + write) and a large bf16 GEMM
    (hipBLASLt through torch)."""
    n = 512 * 1024 * 1024                      # fp32 elements = 2 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = time_stream(torch, lambda: dst.copy_(src), 10) / 10
    copy_gbps = 2 * n * 4 / (ms * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    c = a @ b
    ms = time_stream(torch, lambda: torch.matmul(a, b, out=c), 10) / 10
    gemm_tflops = 2 * m ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(copy_gbps, 1), "bf16_gemm_8192_TFLOPs": round(gemm_tflops, 1),
            "note": "2 GiB device copy (bytes read + written); 8192^3 bf16 torch.matmul"}


def gpu_state():
    """Clock and power readings from rocm-smi, when the tool is present (read only)."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, "-d", "0", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=30)
        data = json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip() else None
    except (OSError, ValueError, subprocess.TimeoutExpired):
        return None
    if not isinstance(data, dict):
        return None
    card = next(iter(data.values()), {})
    return {k: v for k, v in card.items() if isinstance(v, str) and len(v) < 64}


def bench_decode_graph(torch, gdn, d, steps, warmup, chunk_steps: int = 100):
    """ms per decode step when the steps are replayed from captured HIP graphs:
    `chunk_steps` consecutive steps (fixed input pointers) per graph, replayed
    until `steps` steps have run."""
    st = gi.make_decode_steps(d, 0, steps=chunk_steps)
    dv = {n: torch.from_numpy(st[n]).cuda() for n in st}
    for n in ("q", "k", "v"):
        dv[n] = dv[n].to(torch.bfloat16)
    state = torch.from_numpy(gi.make_decode_state(d, 0)).cuda()
    out = torch.empty((d.B, d.Hv, d.dv), dtype=torch.bfloat16, device="cuda")

    def steps_fn():
        for s in range(chunk_steps):
            gdn.gdn_decode_step(dv["q"][s], dv["k"][s], dv["v"][s], dv["log_g"][s], dv["beta"][s],
                                state, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(warmup):
            steps_fn()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps_fn()
    torch.cuda.synchronize()
    reps = max(steps // chunk_steps, 1)
    log(f"decode from HIP graphs: timing {reps} x {chunk_steps} steps")
    ms = time_stream(torch, graph.replay, reps)
    return ms / (reps * chunk_steps)


def bench_decode(torch, gdn, d, steps, warmup):
    log(f"decode workload {d.name}: generating {steps} steps of inputs")
    st = gi.make_decode_steps(d, 0, steps=steps)
    dv = {n: torch.from_numpy(st[n]).cuda() for n in st}
    for n in ("q", "k", "v"):
        dv[n] = dv[n].to(torch.bfloat16)
    state0 = torch.from_numpy(gi.make_decode_state(d, 0)).cuda()
    state = state0.clone()
    out = torch.empty((d.B, d.Hv, d.dv), dtype=torch.bfloat16, device="cuda")
    idx = [0]

    def call():
        s = idx[0]
        gdn.gdn_decode_step(dv["q"][s], dv["k"][s], dv["v"][s], dv["log_g"][s], dv["beta"][s],
                            state, out=out)
        idx[0] = (s + 1) % steps

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    state.copy_(state0)
    idx[0] = 0
    log(f"decode: timing {steps} steps")
    ms = time_stream(torch, call, steps)
    return ms / steps


def bench_decode_multi(torch, gdn, d, steps, warmup, tokens_per_call: int):
    """ms per gdn_decode_multi call of `tokens_per_call` tokens per sequence, over
    the same per-step inputs as the decode leg, grouped in calls."""
    T = tokens_per_call
    calls = max(steps // T, 1)
    st = gi.make_decode_steps(d, 0, steps=calls * T)
    dv = {}
    for n in st:   # [calls*T, B, ...] -> [calls, B, T, ...], contiguous per call
        x = torch.from_numpy(st[n]).cuda()
        x = x.reshape((calls, T) + x.shape[1:]).transpose(1, 2).contiguous()
        dv[n] = x.to(torch.bfloat16) if n in ("q", "k", "v") else x
    state0 = torch.from_numpy(gi.make_decode_state(d, 0)).cuda()
    state = state0.clone()
    out = torch.empty((d.B, T, d.Hv, d.dv), dtype=torch.bfloat16, device="cuda")
    idx = [0]

    def call():
        c = idx[0]
        gdn.gdn_decode_multi(dv["q"][c], dv["k"][c], dv["v"][c], dv["log_g"][c], dv["beta"][c],
                             state, out=out)
        idx[0] = (c + 1) % calls

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    state.copy_(state0)
    idx[0] = 0
    log(f"decode, {T} tokens per call: timing {calls} calls")
    ms = time_stream(torch, call, calls)
    return ms / calls, calls


def cpu_baseline(p, sample_tokens: int, cores=None):
    """The oracle as it stands, on the first `sample_tokens` tokens of the
    prefill workload (all heads), threaded over (b, h) on the host cores."""
    import oracle
    cores = cores or max(1, min(os.cpu_count() or 1, 64))
    inp = gi.make_prefill(p, 0, T=sample_tokens)
    t0 = time.perf_counter()
    oracle.gdn_sequential(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["beta"], inp["h0"],
                          nthreads=cores)
    dt = time.perf_counter() - t0
    return {"value": round(p.B * sample_tokens / dt, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {sample_tokens} of {p.T} tokens of {p.name}, all {p.Hv} value heads, "
                      f"fp64 token-serial oracle, {dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the plain prefill and decode calls (profiling runs, where "
                         "the checkpoint, raw-gate and multi-token legs would mix into the "
                         "same kernels' statistics)")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "copy"], default="all",
                    help="restrict to one half (profiling runs); 'copy' runs only the plain "
                         "copy kernel used to calibrate HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the gated-delta-rule core shards by heads or "
              "sequences with no exchange, so a multi-GPU figure is not produced here "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrence_04_amd as gdn

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    p = gi.QWEN27B_PREFILL
    d = gi.QWEN27B_DECODE

    if args.only == "copy":
        # a plain device copy of known size: FETCH_SIZE / WRITE_SIZE of this
        # kernel calibrate the counters of the gated-delta-rule kernels
        n = 256 * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": max(args.steps, 1)}), flush=True)
        return

    result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16 storage, fp32 accumulate/state",
              "data": "synthetic (seeded numpy PCG64, shapes and distributions of the workload)",
              "config": {"workload": p.name, "B": p.B, "T": p.T, "Hk": p.Hk, "Hv": p.Hv,
                         "dk": p.dk, "dv": p.dv, "chunk": p.chunk,
                         "gate": "log g = -exp(A_log) softplus(dt)", "h0": "N(0, 0.02)"}}

    if args.only in ("all", "prefill"):
        ms, prob = bench_prefill(torch, gdn, p, args.steps, args.warmup)
        flops = prefill_useful_flops(p)
        nbytes = prefill_bytes(p)
        kernel = gdn.selected_prefill_kernel(prob)
        gbps = nbytes / (ms * 1e-3) / 1e9
        tflops = flops / (ms * 1e-3) / 1e12
        src = source_hash(*kernel["sources"])
        result["value"] = round(p.B * p.T / (ms * 1e-3), 1)
        result["ms_per_step"] = round(ms, 4)
        mm_peak = MFMA_BF16_PEAK_TFLOPS if kernel["arith"] == "bf16-mfma" else FP32_VALU_PEAK_TFLOPS
        hbm_floor = nbytes / (HBM_PEAK_GBPS * 1e9)
        mm_floor = flops / (mm_peak * 1e12)
        traffic = pmc_traffic(kernel["name"], src)
        result["roofline"] = {
            "bound": "hbm" if hbm_floor >= mm_floor else "mfma",
            "kernel": kernel["name"],
            "achieved": round(gbps if hbm_floor >= mm_floor else tflops, 3),
            "peak": HBM_PEAK_GBPS if hbm_floor >= mm_floor else mm_peak,
            "unit": "GB/s" if hbm_floor >= mm_floor else "TFLOP/s",
            "frac": round((gbps / HBM_PEAK_GBPS) if hbm_floor >= mm_floor else (tflops / mm_peak), 5),
            "traffic": traffic,
            "algorithmic_bytes": nbytes, "useful_flops": flops,
            "compute": {"achieved_tflops": round(tflops, 3), "peak_tflops": mm_peak,
                        "peak_kind": kernel["arith"], "frac": round(tflops / mm_peak, 5),
                        "frac_of_bf16_mfma": round(tflops / MFMA_BF16_PEAK_TFLOPS, 5)},
            "avg_launch_us": round(ms * 1e3, 2), "source_hash": src,
        }
        log(f"prefill: {ms:.3f} ms/call, {result['value']:.0f} tok/s, {gbps:.1f} GB/s, {tflops:.2f} TFLOP/s")
    if args.only in ("all", "prefill") and not args.no_extras:
        # the same call storing a state checkpoint every 512 tokens (32 slots)
        every = 512
        ms_c, _ = bench_prefill(torch, gdn, p, args.steps, args.warmup, ckpt_every=every)
        nck = -(-p.T // every)
        ck_bytes = p.B * nck * p.Hv * p.dk * p.dv * 4
        result["checkpoints"] = {
            "ckpt_every": every, "slots": nck, "slot_bytes_total": ck_bytes,
            "ms_per_call": round(ms_c, 4), "overhead_ms": round(ms_c - ms, 4),
            "tokens_per_s": round(p.B * p.T / (ms_c * 1e-3), 1),
            "extra_write_GBps_over_overhead": (round(ck_bytes / ((ms_c - ms) * 1e-3) / 1e9, 1)
                                               if ms_c > ms else None),
        }
        log(f"prefill with {nck} checkpoints: {ms_c:.3f} ms/call ({(ms_c - ms) * 1e3:+.1f} us)")
        # the same call forming log g and beta in the kernels from raw projections
        ms_g, _ = bench_prefill(torch, gdn, p, args.steps, args.warmup, raw_gates=True)
        result["raw_gates"] = {
            "ms_per_call": round(ms_g, 4), "delta_ms_vs_precomputed_gates": round(ms_g - ms, 4),
            "tokens_per_s": round(p.B * p.T / (ms_g * 1e-3), 1),
            "gate_tensor_bytes_not_materialised": 2 * p.B * p.T * p.Hv * 4 * 2,
        }
        log(f"prefill with raw gates: {ms_g:.3f} ms/call ({(ms_g - ms) * 1e3:+.1f} us)")
        # a packed batch of 8 sequences of different lengths, 16384 tokens in all
        ms_v = bench_prefill_varlen(torch, gdn, p, args.steps, args.warmup)
        result["varlen"] = {
            "lengths": VARLEN_MIX, "ms_per_call": round(ms_v, 4),
            "tokens_per_s": round(sum(VARLEN_MIX) / (ms_v * 1e-3), 1),
            "vs_one_16384_token_sequence": round(ms / ms_v, 3),
        }
        log(f"varlen prefill: {ms_v:.3f} ms/call, {result['varlen']['tokens_per_s']:.0f} tok/s")
        # the 0.8B head shape (16 key = 16 value heads, 2048 tokens): 64 scan
        # workgroups, a short chain of 32 chunks
        p8 = gi.QWEN08B_PREFILL
        ms_8, _ = bench_prefill(torch, gdn, p8, args.steps, args.warmup)
        result["prefill_0.8b"] = {
            "workload": p8.name, "ms_per_call": round(ms_8, 4),
            "tokens_per_s": round(p8.B * p8.T / (ms_8 * 1e-3), 1),
            "hbm_frac": round(prefill_bytes(p8) / (ms_8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5),
            "bf16_mfma_frac": round(prefill_useful_flops(p8) / (ms_8 * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
        }
        log(f"0.8B prefill: {ms_8 * 1e3:.1f} us/call")
        # the long prompt: 256 consecutive 512-token calls, state carried and checkpointed
        pl = gi.QWEN27B_LONG
        ms_l, ncalls = bench_long_context(torch, gdn, pl, args.warmup)
        result["long_context"] = {
            "workload": pl.name, "calls": ncalls, "tokens_per_call": pl.extra["call_tokens"],
            "distinct_segments": LONG_DISTINCT_SEGMENTS,
            "ms_per_prompt": round(ms_l, 4), "us_per_call": round(ms_l * 1e3 / ncalls, 3),
            "tokens_per_s": round(pl.B * pl.T / (ms_l * 1e-3), 1),
            "state_checkpoint_bank_bytes": ncalls * pl.B * pl.Hv * pl.dk * pl.dv * 4,
        }
        log(f"long context: {ms_l:.3f} ms per prompt, {ms_l * 1e3 / ncalls:.1f} us per call")

    if args.only in ("all", "decode"):
        ms_d = bench_decode(torch, gdn, d, args.decode_steps, min(args.warmup, 10) or 1)
        nb = decode_bytes(d)
        gbps_d = nb / (ms_d * 1e-3) / 1e9
        src_d = source_hash("decode.hip", "gdn_device.h")
        result["decode"] = {
            "workload": d.name, "steps": args.decode_steps,
            "us_per_step": round(ms_d * 1e3, 3),
            "tokens_per_s": round(d.B / (ms_d * 1e-3), 1),
            "state_update_GBps": round(gbps_d, 2),
            "roofline": {"bound": "hbm", "kernel": "decode_step_kernel<128,bf16>",
                         "achieved": round(gbps_d, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps_d / HBM_PEAK_GBPS, 5),
                         "traffic": pmc_traffic("decode_step_kernel<128,bf16>", src_d),
                         "algorithmic_bytes": nb, "source_hash": src_d},
        }
        log(f"decode: {ms_d * 1e3:.2f} us/step, {gbps_d:.1f} GB/s")
        if result["value"] is None:
            result["value"] = result["decode"]["tokens_per_s"]
            result["unit"] = "tokens/s (decode)"
            result["ms_per_step"] = round(ms_d, 5)
    if args.only in ("all", "decode") and not args.no_extras:
        # several tokens per call (speculative verification): the state is read
        # and written once per call
        Tm = 4
        ms_m, calls = bench_decode_multi(torch, gdn, d, args.decode_steps, min(args.warmup, 10) or 1, Tm)
        tok_bytes = d.B * Tm * (2 * d.Hk * d.dk * 2 + 2 * d.Hv * d.dv * 2 + 8 * d.Hv)
        nb_m = 2 * d.B * d.Hv * d.dk * d.dv * 4 + tok_bytes
        result["decode_multi"] = {
            "tokens_per_call": Tm, "calls": calls, "us_per_call": round(ms_m * 1e3, 3),
            "tokens_per_s": round(d.B * Tm / (ms_m * 1e-3), 1),
            "speedup_vs_single_steps": round(Tm * ms_d / ms_m, 3),
            "hbm_GBps": round(nb_m / (ms_m * 1e-3) / 1e9, 2),
            "algorithmic_bytes_per_call": nb_m,
        }
        log(f"decode, {Tm} tokens per call: {ms_m * 1e3:.2f} us/call, "
            f"{result['decode_multi']['tokens_per_s']:.0f} tok/s")
        # the same steps replayed from captured HIP graphs (no per-step launch cost)
        ms_gr = bench_decode_graph(torch, gdn, d, args.decode_steps, min(args.warmup, 10) or 1)
        result["decode_graph"] = {"us_per_step": round(ms_gr * 1e3, 3),
                                  "state_update_GBps": round(nb / (ms_gr * 1e-3) / 1e9, 2),
                                  "vs_stream_launches": round(ms_d / ms_gr, 3)}
        log(f"decode from HIP graphs: {ms_gr * 1e3:.2f} us/step")
        # twice the batch: 402.7 MB of state, more than the 256 MB Infinity Cache
        d2 = gi.DecodeProblem(d.name.replace("B64", "B128"), 2 * d.B, d.Hk, d.Hv, d.dk, d.dv, 200)
        ms_2 = bench_decode(torch, gdn, d2, d2.steps, min(args.warmup, 10) or 1)
        nb2 = decode_bytes(d2)
        result["decode_B128"] = {"workload": d2.name, "steps": d2.steps,
                                 "us_per_step": round(ms_2 * 1e3, 3),
                                 "state_update_GBps": round(nb2 / (ms_2 * 1e-3) / 1e9, 2),
                                 "frac_of_hbm_peak": round(nb2 / (ms_2 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 5)}
        log(f"decode B=128: {ms_2 * 1e3:.2f} us/step, {result['decode_B128']['state_update_GBps']:.1f} GB/s")

    if args.only == "all" and not args.no_extras:
        peaks = measured_peaks(torch)
        result["measured_peaks"] = peaks
        if "roofline" in result:
            r = result["roofline"]
            r["frac_of_measured_peak"] = round(
                r["achieved"] / (peaks["hbm_copy_GBps"] if r["unit"] == "GB/s" else peaks["bf16_gemm_8192_TFLOPs"]), 5)
            r["compute"]["frac_of_measured_bf16_gemm"] = round(
                r["compute"]["achieved_tflops"] / peaks["bf16_gemm_8192_TFLOPs"], 5)
        if "decode" in result:
            dr = result["decode"]["roofline"]
            dr["frac_of_measured_peak"] = round(dr["achieved"] / peaks["hbm_copy_GBps"], 5)
        result["gpu_state"] = gpu_state()

    if not args.no_cpu_baseline and args.only in ("all", "prefill"):
        log("cpu baseline: oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(p, args.cpu_sample_tokens)
        if not args.no_extras:
            log("cpu baseline: one thread, 512 tokens")
            result["cpu_baseline_1thread"] = cpu_baseline(p, 512, cores=1)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
