"""Benchmark: fwd+bwd throughput of the chunked causal linear attention on one MI355X.

One step = slim_attn_fwd + slim_attn_bwd over one batch of synthetic inputs
already resident in HBM (every kernel of the path: feature maps, chunk states,
scans, outputs, statistics, dQ, dK/dV).  Default workload: FAVOR+, bf16 I/O with
fp32 state, B=4, H=16, L=16384, d=64, M=256, 32 slices of 512.

Prints ONE JSON line (rank 0): throughput (tokens/s = B*L per step time), the
roofline record of the dominant kernel (timed live with hipEvents on the
launch stream through the library's kernel timer), peak HBM, per-kernel times
and the fp64 CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
  python bench.py --profile-run     # a few steps, for rocprofv3 runs
  python bench.py --copy-calib      # one plain copy kernel of known size (PMC calibration)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal linear-attn fwd+bwd tokens/s & % roofline; peak HBM, L=16K d=64 M=256"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU oracle sample (0 = H)")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    return ap.parse_args()


def make_inputs(w, torch, synth):
    """Seeded synthetic inputs, generated per head on the host and copied to HBM."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")

    def tensor(tid, scale):
        t = torch.empty((w.B, w.H, w.L, w.d), dtype=dt, device=dev)
        for b in range(w.B):
            for h in range(w.H):
                t[b, h].copy_(torch.from_numpy(synth.head_normal(w.seed, tid, b, h, w.L, w.d, scale)).to(dev))
        return t

    q = tensor(synth.TID_Q, w.qkv_scale)
    k = tensor(synth.TID_K, w.qkv_scale)
    v = tensor(synth.TID_V, 1.0)
    dy = tensor(synth.TID_DY, 1.0)
    W = None
    if w.feat == "favor":
        W = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).to(dev).to(dt).contiguous()
    return q, k, v, W, dy


def cpu_baseline(w, synth, heads):
    """The fp64 oracle's linear-time (prefix) form, fwd+bwd, on batch row 0 and
    `heads` heads at full length, one thread per head."""
    import numpy as np

    import oracle

    def head(tid, b, h, s):
        return synth.head_normal(w.seed, tid, b, h, w.L, w.d, s).astype(np.float64)[None, None]

    heads = min(heads, w.H)
    q = np.concatenate([head(synth.TID_Q, 0, h, w.qkv_scale) for h in range(heads)], axis=1)
    k = np.concatenate([head(synth.TID_K, 0, h, w.qkv_scale) for h in range(heads)], axis=1)
    v = np.concatenate([head(synth.TID_V, 0, h, 1.0) for h in range(heads)], axis=1)
    dy = np.concatenate([head(synth.TID_DY, 0, h, 1.0) for h in range(heads)], axis=1)
    W = synth.projection(w.seed, w.M, w.d, w.w_kind).astype(np.float64) if w.feat == "favor" else None
    threads = min(heads, os.cpu_count() or 1)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, W, w.feat, form="prefix", threads=threads)
    oracle.attn_bwd(q, k, v, W, dy, w.feat, form="prefix", threads=threads)
    dt = time.perf_counter() - t0
    # one token needs all H heads: a sample of `heads` heads covers heads/H of L tokens
    tok = w.L * heads / w.H
    return {"value": tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle, iterative prefix-sum form, fwd+bwd of batch row 0, {heads} of {w.H} heads, "
                      f"full L={w.L}, one thread per head ({dt:.1f} s); tokens credited = L*{heads}/{w.H}",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU mode "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from causal_linear_attention_amd import _lib
    from causal_linear_attention_amd import attention as A
    from causal_linear_attention_amd import synth
    from causal_linear_attention_amd.workloads import HEADLINE, WORKLOADS, kernel_flops, survey_flops

    if args.copy_calib:
        # plain device-to-device copy of 1 GiB (reads 1 GiB, writes 1 GiB): the
        # calibration kernel for rocprofv3 FETCH_SIZE / WRITE_SIZE
        x = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0").fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4, "launches": 3}))
        return

    w = WORKLOADS[args.workload or HEADLINE]
    q, k, v, W, dy = make_inputs(w, torch, synth)
    tile = int(_lib.lib().slim_tile_rows(__import__("ctypes").byref(A.make_desc(q, w.M, w.feat, w.chunks))))
    torch.cuda.synchronize()

    def step():
        Y, R, S = A.attn_fwd(q, k, v, W, w.feat, w.chunks)
        if w.backward:
            A.attn_bwd(q, k, v, W, dy, R, S, w.feat, w.chunks)
        return Y

    if args.profile_run:
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": w.name, "steps": args.steps}))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # peak HBM of one step (the page's method: max_memory_allocated)
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()

    _lib.prof_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.prof_enable(False)
    prof = _lib.prof_read()

    ms_step = 1e3 * elapsed / args.steps
    tokens_per_s = w.tokens * args.steps / elapsed
    fl = kernel_flops(w, tile)
    passes = {"state": 2 if w.backward else 1}
    kernels = {}
    for name, (ms, n) in prof.items():
        rec = {"ms_total": round(ms, 4), "launches": n, "ms_avg": round(ms / n, 5),
               "ms_per_step": round(ms / args.steps, 5)}
        if name in fl:
            flop = fl[name] * w.head_tokens * passes.get(name, 1) * args.steps
            rec["tflops"] = round(flop / (ms * 1e-3) / 1e12, 2)
            rec["flop_per_launch"] = flop / n
        kernels[name] = rec
    mfma = {k2: v2 for k2, v2 in kernels.items() if "tflops" in v2}
    dom = max(mfma, key=lambda k2: mfma[k2]["ms_total"])
    d = kernels[dom]
    achieved = d["flop_per_launch"] / (d["ms_avg"] * 1e-3) / 1e12
    peak_t = PEAK_TFLOPS[w.dtype]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak_t,
                "unit": "TFLOP/s", "frac": round(achieved / peak_t, 4), "traffic": None,
                "flop_per_launch": d["flop_per_launch"], "ms_avg": d["ms_avg"]}
    isz = 2 if w.dtype == "bf16" else 4
    # minimum HBM traffic of a step: read Q K V (fwd) and Q K V dY (bwd), write Y dQ dK dV
    io = w.head_tokens * w.d * isz * (11 if w.backward else 4)
    footprint = w.head_tokens * w.d * isz * (9 if w.backward else 4)  # Q K V dY Y dQ dK dV resident
    step_flop = sum(fl[n] * (passes.get(n, 1)) for n in fl) * w.head_tokens
    rec = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "M": w.M, "feat": w.feat,
                   "W": w.w_kind, "chunks": w.chunks, "chunk_len": w.chunk_len, "tile": tile,
                   "window_chunks": int(_lib.lib().slim_window_chunks(
                       __import__("ctypes").byref(A.make_desc(q, w.M, w.feat, w.chunks)))),
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "step_tflops": round(step_flop / (ms_step * 1e-3) / 1e12, 2),
        "step_tflops_unsliced_accounting": round(survey_flops(w) * w.head_tokens / (ms_step * 1e-3) / 1e12, 2),
        "peak_hbm_bytes": peak, "resident_before_step_bytes": base, "step_extra_bytes": peak - base,
        "io_traffic_bytes_per_step": io, "io_gbs": round(io / (ms_step * 1e-3) / 1e9, 1),
        "io_footprint_bytes": footprint,
        "kernels": kernels,
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, synth, args.cpu_heads or w.H)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
