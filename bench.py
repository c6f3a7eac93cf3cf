"""Benchmark of the gated delta rule core on one MI355X.

One JSON line on stdout.  The timed step is one chunkwise prefill of the headline
workload (B=4 sequences x T=4096 tokens, H=16 heads of d_k = d_v = 128, chunk 64, bf16
q/k/v/beta/log alpha, fp32 state, bf16 outputs, final state out): `value` is Mtok/s
(B*T tokens per second, each token carrying all 16 heads), inputs resident in HBM.
Beside it, with their own timings: the recurrent decode step (256 sequences x 32 heads of
128x128 fp32 states, 100 in-place steps; state GB/s), the long prefill with snapshots
(T = 65536, 32 heads, a snapshot every 8192 tokens) and the KDA prefill.

`roofline` is measured live with HIP events on the stream the kernels run on;
`cpu_baseline` times the fp64 oracle on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib

import numpy as np
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunkwise prefill Mtok/s at H=16,d=128 (MFMA %); decode state GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak


def prefill_flops_per_head_token(C: int, d: int) -> int:
    """Algorithmic flops per head-token of the chunkwise prefill with C x C products counted as
    full tiles: K K^T, Q K^T (2 C d each), W/U-type products T X and P U (2 C d each, 2 of
    them at d_v = d), and the three state-coupled d x d products K S^T, Q S^T, U^T K (2 d^2
    each): 10 C d + 6 d^2."""
    return 10 * C * d + 6 * d * d


def prefill_bytes(B, H, T, d, in_bytes=2, out_bytes=2, n_ckpt=0, kda=False, s0=True) -> int:
    """Compulsory HBM traffic: q, k, v, beta, log alpha in; o out; S0 in, S_final and the
    snapshots out (fp32)."""
    per_tok = (3 * d + 1 + (d if kda else 1)) * in_bytes + d * out_bytes
    state = d * d * 4
    return B * H * (T * per_tok + state * ((1 if s0 else 0) + 1 + n_ckpt))


def _src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_deltanet_state_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel: str, src_files):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("src_sha256_16") != _src_hash(*src_files):
        return None
    return rec.get("bytes_per_launch")


def time_launches(fn, steps: int, warmup: int, torch) -> float:
    """Average ms per call of fn(i) over `steps` calls, HIP events on torch's current stream
    (the stream every launch goes to)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        fn(i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def cpu_model() -> str:
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline_prefill(inp, min_seconds: float = 8.0, max_reps: int = 200, single_seconds: float = 2.0):
    """The fp64 oracle, as it stands, on the whole workload (every (batch, head) stream, all
    tokens) on all host cores, repeated until at least `min_seconds` of wall time; then on one
    thread over the first two streams, repeated until `single_seconds`."""
    import oracle
    oracle.build(force=False)
    B, H, T, d = inp["q"].shape
    args = (inp["q"], inp["k"], inp["v"], inp["beta"], inp["log_alpha"], inp["s0"])
    reps, threads = 0, 0
    t0 = time.perf_counter()
    while True:
        _, _, _, threads = oracle.forward(*args, return_threads=True)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    tokens = reps * B * T  # a token carries all H heads
    # one thread, two (batch, head) streams: head-tokens per second, scaled to tokens of H heads
    sub = tuple(None if x is None else x[:1, :2].contiguous() for x in args)
    reps1 = 0
    t1 = time.perf_counter()
    while True:
        oracle.forward(*sub, nthreads=1)
        reps1 += 1
        dt1 = time.perf_counter() - t1
        if dt1 >= single_seconds or reps1 >= max_reps:
            break
    head_tok_s1 = reps1 * 2 * T / dt1
    return {"value": round(tokens / dt / 1e6, 6), "unit": "Mtok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole workload ({B * H} streams x {T} tokens) repeated {reps} times, fp64 token "
                      f"loop, {dt:.1f} s wall",
            "cpu": cpu_model(),
            "single_thread": {"value": round(head_tok_s1 / H / 1e6, 6), "unit": "Mtok/s", "cores": 1,
                              "sample": f"2 streams x {T} tokens on one thread, repeated {reps1} times, "
                                        f"{dt1:.1f} s wall; scaled to tokens of {H} heads"}}


def cpu_baseline_decode(inp, min_seconds: float = 3.0, max_steps: int = 100):
    """The fp64 oracle's decode step on every (sequence, head) state of the decode workload, on
    all host cores, stepping until `min_seconds` of wall time.  State traffic is counted in
    the oracle's own fp64 bytes (read and write once per step)."""
    import oracle
    oracle.build(force=False)
    st = inp["state"].double().numpy().copy()
    N, H, Dv, Dk = st.shape
    steps = 0
    t0 = time.perf_counter()
    while True:
        t = steps % inp["q"].shape[0]
        oracle.decode_step(st, *(inp[k][t] for k in ("q", "k", "v", "beta", "log_alpha")))
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or steps >= max_steps:
            break
    fp64_bytes = 2 * N * H * Dv * Dk * 8
    return {"value": round(steps * fp64_bytes / dt / 1e9, 3), "unit": "GB/s (fp64 state)",
            "cores": int(oracle.hardware_threads()), "kind": "oracle",
            "us_per_step": round(dt / steps * 1e6, 1),
            "sample": f"{steps} steps over all {N * H} states of {Dv}x{Dk}, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "prefill_ex", "decode", "long", "kda", "serving", "copy", "all"],
                    default="all",
                    help="run a subset (for profiling); the JSON line needs 'all' or 'prefill'")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the (batch, head) streams shard with no exchange, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_state_amd as g
    from gated_deltanet_state_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    out = {}
    extra = {}

    def log(*a):
        print(*a, file=sys.stderr, flush=True)

    # ---------------- headline: chunkwise prefill, B=4 H=16 T=4096 d=128 C=64 ----------------
    if args.only in ("prefill", "all"):
        c = synth.WORKLOADS[1]
        log("prefill: generating inputs")
        sets = [synth.make_workload(1), synth.make_prefill(c.B, c.H, c.T, c.Dk, c.Dv, c.dtype,
                                                             s0_std=c.s0_std, seed=synth.seed_of(1) + 100)]
        dsets = [{k: v.to(dev) for k, v in s.items()} for s in sets]
        outs = [(torch.empty(c.B, c.H, c.T, c.Dv, dtype=torch.bfloat16, device=dev),
                 torch.empty(c.B, c.H, c.Dv, c.Dk, dtype=torch.float32, device=dev)) for _ in dsets]

        def step(i):
            d = dsets[i % 2]
            o, sf = outs[i % 2]
            g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], chunk=c.chunk,
                            o=o, s_final=sf)

        log("prefill: timing")
        ms = time_launches(step, args.steps, args.warmup, torch)
        tokens = c.B * c.T
        mtoks = tokens / (ms * 1e-3) / 1e6
        flops = c.B * c.H * c.T * prefill_flops_per_head_token(c.chunk, c.Dk)
        nbytes = prefill_bytes(c.B, c.H, c.T, c.Dk)
        gbs = nbytes / (ms * 1e-3) / 1e9
        tflops = flops / (ms * 1e-3) / 1e12
        traffic = _traffic("gdn_chunk_mfma", ["gdn_chunk_mfma.hip", "gdn_mfma_common.h"])
        out.update({
            "metric": METRIC, "value": round(mtoks, 3), "unit": "Mtok/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": c.name, "B": c.B, "H": c.H, "T": c.T, "d_k": c.Dk, "d_v": c.Dv,
                       "chunk": c.chunk, "inputs": "bf16", "state": "fp32", "o": "bf16",
                       "global_batch": c.B, "seq_len": c.T, "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "kernel": "gdn_chunk_mfma_kernel", "algorithmic_bytes": nbytes},
            "mfma": {"achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops},
        })
        log(f"prefill: {ms*1e3:.1f} us/step, {mtoks:.1f} Mtok/s, {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")
        if not args.no_cpu_baseline:
            log("cpu baseline: fp64 oracle on the host cores")
            out["cpu_baseline"] = cpu_baseline_prefill(sets[0])
        del dsets, outs, sets
        torch.cuda.empty_cache()

    # ---------------- decode: 256 x 32 states of 128 x 128 fp32, 100 steps ----------------
    if args.only in ("decode", "all"):
        c = synth.WORKLOADS[3]
        log("decode: generating inputs")
        inp = synth.make_workload(3)
        st = inp["state"].to(dev)
        dq = {k: inp[k].to(dev) for k in ("q", "k", "v", "beta", "log_alpha")}
        o = torch.empty(c.N, c.H, c.Dv, dtype=torch.bfloat16, device=dev)

        def dstep(i):
            t = i % c.steps
            g.gdn_decode_step(st, dq["q"][t], dq["k"][t], dq["v"][t], dq["beta"][t], dq["log_alpha"][t], o=o)

        for i in range(3):
            dstep(i)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(c.steps):
            dstep(i)
        e.record()
        torch.cuda.synchronize()
        ms100 = s.elapsed_time(e)
        per = ms100 / c.steps
        state_bytes = 2 * c.N * c.H * c.Dk * c.Dv * 4
        io_bytes = c.N * c.H * ((3 * c.Dk + 2) * 2 + c.Dv * 2)
        gbs = state_bytes / (per * 1e-3) / 1e9
        hbm = (state_bytes + io_bytes) / (per * 1e-3) / 1e9
        extra["decode"] = {
            "workload": c.name, "N": c.N, "H": c.H, "d": c.Dk, "steps": c.steps,
            "ms_total": round(ms100, 4), "us_per_step": round(per * 1e3, 3),
            "state_GBps": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(hbm / HBM_PEAK_GBS, 4),
                         "traffic": _traffic("gdn_decode", ["gdn_decode.hip"]),
                         "kernel": "decode_kernel", "algorithmic_bytes": state_bytes + io_bytes},
        }
        log(f"decode: {per*1e3:.1f} us/step, state {gbs:.0f} GB/s, HBM frac {hbm/HBM_PEAK_GBS:.3f}")
        if not args.no_cpu_baseline and args.only == "all":
            log("cpu baseline: fp64 oracle decode step on the host cores")
            cpu_dec = cpu_baseline_decode(inp)
            if "cpu_baseline" in out:
                out["cpu_baseline"]["decode"] = cpu_dec
        del st, dq, inp
        torch.cuda.empty_cache()

    # ---------------- long prefill with snapshots: H=32, T=65536 ----------------
    if args.only in ("long", "all"):
        c = synth.WORKLOADS[2]
        log("long prefill: generating inputs")
        inp = synth.make_workload(2)
        d = {k: v.to(dev) for k, v in inp.items()}
        del inp
        o = torch.empty(c.B, c.H, c.T, c.Dv, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(c.B, c.H, c.Dv, c.Dk, dtype=torch.float32, device=dev)
        sc = torch.empty(c.B, c.H, c.T // c.ckpt_every, c.Dv, c.Dk, dtype=torch.float32, device=dev)

        def lstep(i):
            g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], chunk=c.chunk,
                            ckpt_every=c.ckpt_every, o=o, s_final=sf, s_ckpt=sc)

        ms = time_launches(lstep, 3, 1, torch)
        nb = prefill_bytes(c.B, c.H, c.T, c.Dk, n_ckpt=c.T // c.ckpt_every)
        fl = c.B * c.H * c.T * prefill_flops_per_head_token(c.chunk, c.Dk)
        extra["long_prefill"] = {
            "workload": c.name, "B": c.B, "H": c.H, "T": c.T, "ckpt_every": c.ckpt_every,
            "ms": round(ms, 4), "Mtok_per_s": round(c.B * c.T / (ms * 1e-3) / 1e6, 3),
            "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        # the same with the snapshots written into pinned host memory by the kernel itself
        sch = torch.empty(sc.shape, dtype=torch.float32, pin_memory=True)

        def lstep_host(i):
            g.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], chunk=c.chunk,
                            ckpt_every=c.ckpt_every, o=o, s_final=sf, s_ckpt=sch)

        ms_h = time_launches(lstep_host, 3, 1, torch)
        extra["long_prefill"]["snapshots_to_host"] = {
            "ms": round(ms_h, 4), "Mtok_per_s": round(c.B * c.T / (ms_h * 1e-3) / 1e6, 3),
            "snapshot_MiB": round(sch.numel() * 4 / 2**20, 1)}
        log(f"long prefill: {ms:.3f} ms; snapshots into pinned host memory: {ms_h:.3f} ms")
        del d, o, sf, sc, sch
        torch.cuda.empty_cache()

    # ---------------- KDA prefill: B=2 H=32 T=8192 ----------------
    if args.only in ("kda", "all"):
        c = synth.WORKLOADS[4]
        log("kda: generating inputs")
        inp = synth.make_workload(4)
        d = {k: v.to(dev) for k, v in inp.items()}
        del inp
        o = torch.empty(c.B, c.H, c.T, c.Dv, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(c.B, c.H, c.Dv, c.Dk, dtype=torch.float32, device=dev)

        # two-kernel form: per-chunk state-independent tiles into the workspace, then the
        # sequential pass (allocated once, outside the timed region)
        ws = torch.empty(g.gdn_chunk_workspace_size(c.B, c.H, c.T, c.Dk, chunk=c.chunk, kda=True),
                         dtype=torch.uint8, device=dev)

        def kstep(i, w=ws):
            g.kda_chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"], chunk=c.chunk,
                            o=o, s_final=sf, workspace=w)

        ms = time_launches(kstep, 3, 1, torch)
        ms_single = time_launches(lambda i: kstep(i, False), 3, 1, torch)
        nb = prefill_bytes(c.B, c.H, c.T, c.Dk, kda=True)
        fl = c.B * c.H * c.T * prefill_flops_per_head_token(c.chunk, c.Dk)
        gb = nb / (ms * 1e-3) / 1e9
        extra["kda_prefill"] = {
            "workload": c.name, "B": c.B, "H": c.H, "T": c.T, "ms": round(ms, 4),
            "Mtok_per_s": round(c.B * c.T / (ms * 1e-3) / 1e6, 3),
            "roofline": {"bound": "hbm", "achieved": round(gb, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gb / HBM_PEAK_GBS, 4),
                         "traffic": _traffic("kda_chunk_mfma", ["kda_chunk_mfma.hip", "gdn_mfma_common.h"]),
                         "kernel": "kda_prep_kernel + kda_chain_kernel", "algorithmic_bytes": nb},
            "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "workspace_MiB": round(ws.numel() / 2**20, 1),
            "single_kernel_ms": round(ms_single, 4)}
        log(f"kda prefill: {ms:.3f} ms (single-kernel form {ms_single:.3f} ms)")
        del ws

    # ---------------- prefill with the layer prologue: 32 value / 16 query-key heads, raw gates ----------------
    if args.only in ("prefill_ex", "all"):
        B, H, Hqk, T, D = 2, 32, 16, 4096, 128
        log("prefill_ex: generating inputs")
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in synth.make_prefill_ex(B, H, Hqk, T, D, raw=True, unit=False, s0_std=0.01, seed=2003).items()}
        o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
        ms = time_launches(lambda i: g.gdn_chunk_fwd_ex(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["s0"],
                                                         A_log=d["A_log"], dt_bias=d["dt_bias"], qk_l2norm=True,
                                                         o=o, s_final=sf),
                           20, 3, torch)
        # q, k once per query/key head; v, b, a, o per value head; s0 and s_final
        nb = B * T * (2 * Hqk * D + H * (D + 2)) * 2 + B * H * T * D * 2 + 2 * B * H * D * D * 4
        fl = B * H * T * prefill_flops_per_head_token(64, D)
        gb = nb / (ms * 1e-3) / 1e9
        extra["prefill_layer_prologue"] = {
            "workload": "gdn_prefill_grouped32x16_rawgates_qknorm_bf16", "B": B, "H": H, "H_qk": Hqk, "T": T, "d": D,
            "us": round(ms * 1e3, 2), "Mtok_per_s": round(B * T / (ms * 1e-3) / 1e6, 3),
            "roofline": {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gb / HBM_PEAK_GBS, 4),
                         "traffic": _traffic("gdn_chunk_mfma_prologue", ["gdn_chunk_mfma.hip", "gdn_mfma_common.h"]),
                         "kernel": "gdn_chunk_mfma_kernel", "algorithmic_bytes": int(nb)},
            "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        log(f"prefill_ex: {ms * 1e3:.1f} us, {gb:.0f} GB/s")
        del d, o, sf
        torch.cuda.empty_cache()

    # ---------------- ragged prefill: 16 prompts of 256..1792 tokens in one call ----------------
    if args.only in ("prefill_ex", "all"):
        H, D = 16, 128
        lens = synth.ragged_lengths(16, 256, 1792, seed=2004)
        seqs = [synth.make_prefill(1, H, n, D, D, seed=3000 + i) for i, n in enumerate(lens)]
        pk = lambda key: torch.cat([x[key][0].reshape(H * x[key].shape[2], *x[key].shape[3:]) for x in seqs], 0).to(dev)
        d = {key: pk(key) for key in ("q", "k", "v", "beta", "log_alpha")}
        s0 = torch.cat([x["s0"] for x in seqs], 0).to(dev)
        cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=dev)
        del seqs
        T = int(sum(lens))
        ms = time_launches(lambda i: g.gdn_chunk_fwd_ragged(d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], cu,
                                                            H=H, s0=s0), 20, 3, torch)
        nb = H * T * ((3 * D + 2) * 2 + D * 2) + 2 * len(lens) * H * D * D * 4
        gb = nb / (ms * 1e-3) / 1e9
        extra["prefill_ragged"] = {
            "workload": "gdn_prefill_ragged16_bf16", "sequences": len(lens), "tokens": T, "H": H, "d": D,
            "lengths": f"uniform 256..1792 (seeded), min {min(lens)}, max {max(lens)}",
            "us": round(ms * 1e3, 2), "Mtok_per_s": round(T / (ms * 1e-3) / 1e6, 3),
            "roofline": {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gb / HBM_PEAK_GBS, 4),
                         "traffic": _traffic("gdn_chunk_mfma_ragged", ["gdn_chunk_mfma.hip", "gdn_mfma_common.h"]),
                         "kernel": "gdn_chunk_mfma_kernel", "algorithmic_bytes": int(nb)}}
        log(f"prefill_ragged: {T} tokens in {ms * 1e3:.1f} us, {T / (ms * 1e-3) / 1e6:.1f} Mtok/s")
        del d, s0, cu
        torch.cuda.empty_cache()

    # ---------------- serving-side decode windows: verify 4 draft tokens, commit, KDA step ----------------
    if args.only in ("serving", "all"):
        cv = synth.SERVING["verify"]
        log("serving: generating inputs")
        inp = synth.make_serving(cv.N, cv.T, cv.H, cv.Hqk, cv.D, cv.P, cv.dtype, raw=True, s_std=cv.s_std,
                                 seed=2001)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        o = torch.empty(cv.N, cv.T, cv.H, cv.D, dtype=torch.bfloat16, device=dev)
        kw = dict(slots=d["slots"], qk_l2norm=True, A_log=d["A_log"], dt_bias=d["dt_bias"])
        state_b = cv.D * cv.D * 4                         # one (sequence, head) state
        tok_in = (2 * cv.Hqk * cv.D + cv.H * cv.D + 2 * cv.H) * 2   # q, k, v, b, a of one token (bf16)
        tok_out = cv.H * cv.D * 2                         # o of one token (bf16)
        ms_v = time_launches(lambda i: g.gdn_decode_verify(d["pool"], d["q"], d["k"], d["v"], d["beta"],
                                                           d["log_alpha"], o=o, **kw), 20, 3, torch)
        nb_v = cv.N * cv.H * state_b + cv.N * cv.T * (tok_in + tok_out) + 2 * cv.H * 4 + cv.N * 4

        def commit(i):  # the same accepted counts each time: the states keep advancing
            g.gdn_decode_commit(d["pool"], d["q"], d["k"], d["v"], d["beta"], d["log_alpha"], d["n_commit"], **kw)

        ms_c = time_launches(commit, 20, 3, torch)
        nc = inp["n_commit"].numpy()
        # a sequence with no accepted token needs neither its state nor its inputs; a commit
        # produces no outputs and so reads no queries
        tok_in_c = tok_in - cv.Hqk * cv.D * 2
        nb_c = int(2 * (nc > 0).sum() * cv.H * state_b + nc.sum() * tok_in_c + 2 * cv.H * 4 + 2 * cv.N * 4)
        del d, o, inp
        torch.cuda.empty_cache()
        ck = synth.SERVING["kda"]
        inp = synth.make_serving(ck.N, ck.T, ck.H, ck.Hqk, ck.D, ck.P, ck.dtype, kda=True, s_std=ck.s_std,
                                 seed=2002)
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        o = torch.empty(ck.N, ck.T, ck.H, ck.D, dtype=torch.bfloat16, device=dev)
        ms_k = time_launches(lambda i: g.gdn_decode_ex(d["pool"], d["q"], d["k"], d["v"], d["beta"],
                                                       d["log_alpha"], kda=True, o=o), 20, 3, torch)
        nb_k = 2 * ck.N * ck.H * ck.D * ck.D * 4 + ck.N * (2 * ck.Hqk * ck.D + 2 * ck.H * ck.D + ck.H
                                                           + ck.H * ck.D) * 2

        def rec(name, cfg, ms, nb, phase, **more):
            gb = nb / (ms * 1e-3) / 1e9
            r = {"workload": cfg.name, "N": cfg.N, "H": cfg.H, "H_qk": cfg.Hqk, "d": cfg.D, "T": cfg.T,
                 "pool_rows": cfg.P, "us": round(ms * 1e3, 2),
                 "roofline": {"bound": "hbm", "achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(gb / HBM_PEAK_GBS, 4),
                              "traffic": _traffic(f"decode_ex_{phase}", ["gdn_decode.hip"]),
                              "kernel": {"verify": "decode_win_mfma_kernel", "commit": "decode_commit128_kernel"}.get(
                                  phase, "decode_ex_kernel"),
                              "algorithmic_bytes": int(nb)}}
            r.update(more)
            log(f"serving {name}: {ms * 1e3:.1f} us, {gb:.0f} GB/s, HBM frac {gb / HBM_PEAK_GBS:.3f}")
            return r

        extra["serving_decode"] = {
            "verify": rec("verify", cv, ms_v, nb_v, "verify", draft_tokens=cv.T,
                          fused="q/k L2 norm, gate activations"),
            "commit": rec("commit", cv, ms_c, nb_c, "commit", accepted_tokens=int(nc.sum()),
                          sequences_committing=int((nc > 0).sum())),
            "kda_step": rec("kda step", ck, ms_k, nb_k, "kda_step"),
        }
        del d, o, inp
        torch.cuda.empty_cache()

    # ---------------- plain device copy of known size: calibrates the HBM byte counters ----------------
    if args.only == "copy":
        n = 1 << 28  # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = time_launches(lambda i: dst.copy_(src), 5, 1, torch)
        extra["copy"] = {"bytes_read": 4 * n, "bytes_written": 4 * n, "ms": round(ms, 4),
                         "GBps": round(8 * n / (ms * 1e-3) / 1e9, 1)}
        log(f"copy: {ms:.3f} ms, {8 * n / (ms * 1e-3) / 1e9:.0f} GB/s (read + write)")
        # a write-only and a read-only kernel of the same size: the two counters in isolation
        ms_f = time_launches(lambda i: dst.fill_(1.5), 3, 1, torch)
        acc = torch.empty((), dtype=torch.float32, device=dev)
        ms_s = time_launches(lambda i: torch.sum(src, out=acc), 3, 1, torch)
        extra["fill"] = {"bytes_written": 4 * n, "ms": round(ms_f, 4)}
        extra["sum"] = {"bytes_read": 4 * n, "ms": round(ms_s, 4), "value": float(acc)}
        log(f"fill: {ms_f:.3f} ms, sum: {ms_s:.3f} ms")

    if "metric" not in out:
        print(json.dumps(extra))
        return
    out.update(extra)
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
