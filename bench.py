"""Benchmark: fwd+bwd throughput of the chunked causal linear attention on one MI355X.

One step = slim_attn_fwd + slim_attn_bwd over one batch of synthetic inputs
already resident in HBM (every kernel of the path: feature maps, chunk states,
scans, outputs, statistics, dQ, dK/dV); the forward keeps its output, per-row
denominator statistics and, where one window holds every slice, the slices'
entry states for the backward, as the autograd function does (the step with the
backward rebuilding all of them is timed too, ms_per_step_stats_recomputed).
Default workload: FAVOR+, bf16 I/O with fp32 state, B=4, H=16, L=16384, d=64,
M=256, 32 slices of 512.

Prints ONE JSON line (rank 0): throughput (tokens/s = B*L per step time, timed
over plain steps), the roofline record of the dominant kernel (its launches
timed with hipEvents on the launch stream through the library's kernel timer,
over the same number of further steps), peak HBM, per-kernel times and the fp64
CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
  python bench.py --profile-run     # a few steps, for rocprofv3 runs
  python bench.py --copy-calib      # one plain copy kernel of known size (PMC calibration)
  python bench.py --pmc-summary DIR # (host only) HBM traffic per kernel from rocprofv3 counter CSVs
  python bench.py --decode [...]    # the recurrent decode step instead (one JSON line of its own)
  python bench.py --chunk-sweep     # time, peak HBM and gradient discrepancy vs slice length (one JSON line)
  python bench.py --algorithm1      # the same for the page's Algorithm 1 on a multi-layer Performer
  python bench.py --dw              # the step with the backward also computing dW (FAVOR+ projection)
  python bench.py --featmap         # the standalone feature map g(Q) with row offsets (one JSON line)

roofline.traffic: HBM bytes per launch of the dominant kernel, FETCH_SIZE and
WRITE_SIZE scaled by what the same counters read for a plain copy of known
size; taken from profiles/traffic_<workload>.md when that summary was made
from the kernel sources as they are now (hash match), else null.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (a few do not let the clocks settle: after 3, 1.52 ms per step at "
                         "the default workload, after 20, 1.46)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-mem-sweep", action="store_true", help="skip the peak-HBM-vs-L rows of the JSON line")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU oracle sample (0 = H)")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--mem-sweep", action="store_true",
                    help="peak HBM of one fwd+bwd step vs L at the 1M-token workload's shape (one JSON line)")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="fwd+bwd time, peak HBM and gradient discrepancy against one unsliced run for slice "
                         "lengths 1, 2, 4, ..., L at the headline head shape (one JSON line)")
    ap.add_argument("--sweep-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--sweep-window", type=int, default=0, help="window_chunks of the swept runs (0 = auto)")
    ap.add_argument("--sweep-cmax", type=int, default=0, help="largest slice length swept (0 = L)")
    ap.add_argument("--algorithm1", action="store_true",
                    help="time, peak HBM and gradient discrepancy of Algorithm 1 on a 4-layer Performer vs the "
                         "slice length C (one JSON line)")
    ap.add_argument("--decode", action="store_true",
                    help="time the recurrent decode step (one token per sequence per step) instead")
    ap.add_argument("--dw", action="store_true",
                    help="the backward of every step also computes dW, the gradient of the FAVOR+ projection")
    ap.add_argument("--featmap", action="store_true",
                    help="time the standalone feature map (slim_featmap with per-row offsets) on the workload's Q")
    ap.add_argument("--pmc-summary", default=None, metavar="DIR",
                    help="DIR holds rocprofv3 counter runs F, W (FETCH_SIZE, WRITE_SIZE of --profile-run; "
                         "DF, DW with --decode; DWF, DWW with --dw) and CF, CW (the same of --copy-calib); prints "
                      "the summary")
    return ap.parse_args()


def kernel_source_hash():
    """sha256 of the kernel sources, the C-ABI header and the build script with its compiler
    flags (what the traffic figures depend on)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "causal_linear_attention_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "slim.h"))
    files.append(os.path.join(ROOT, "causal_linear_attention_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_kernel(name):
    m = re.match(r"void slim::scan_kernel<(\d)(?:, (?:true|false))?>", name)
    if m:
        return ("scan_prefix", "scan_window", "scan_grad", "scan_sum")[int(m.group(1))]
    m = re.match(r"void slim::(\w+?)_kernel<", name) or re.match(r"_ZN4slim\d+(\w+?)_kernel", name)
    if m:
        return m.group(1)
    if "copyBuffer" in name:
        return "copy"
    return None


def read_counter(path, counter):
    """Per short kernel name: list of per-dispatch values of `counter` (KiB)."""
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            k = short_kernel(r["Kernel_Name"])
            if k:
                out.setdefault(k, []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(d, w, bytes_of_copy, runs=("F", "W"), dw=False):
    """HBM bytes per dispatch and kernel from counter runs in d: runs[0] (FETCH_SIZE) and
    runs[1] (WRITE_SIZE) of the workload, CF and CW of the calibration copy.  dw: the
    runs are of the step with dW (its dQ and dK/dV kernels get the _dw names)."""
    fetch = read_counter(glob.glob(os.path.join(d, runs[0], "*counter_collection.csv"))[0], "FETCH_SIZE")
    write = read_counter(glob.glob(os.path.join(d, runs[1], "*counter_collection.csv"))[0], "WRITE_SIZE")
    cf = read_counter(glob.glob(os.path.join(d, "CF", "*counter_collection.csv"))[0], "FETCH_SIZE")["copy"]
    cw = read_counter(glob.glob(os.path.join(d, "CW", "*counter_collection.csv"))[0], "WRITE_SIZE")["copy"]
    # the calibration copy reads and writes bytes_of_copy per launch
    f_fac = bytes_of_copy / (sum(cf) / len(cf) * 1024)
    w_fac = bytes_of_copy / (sum(cw) / len(cw) * 1024)
    rows = {}
    for k in sorted(set(fetch) & set(write)):
        fb = sum(fetch[k]) / len(fetch[k]) * 1024 * f_fac
        wb = sum(write[k]) / len(write[k]) * 1024 * w_fac
        rows[k] = {"dispatches": len(fetch[k]), "fetch_bytes": round(fb), "write_bytes": round(wb),
                   "traffic_bytes": round(fb + wb)}
    if "bwdq" in rows and "gstate" not in rows and "bwdkv" in rows:
        rows["bwdq_gstate"] = rows.pop("bwdq")  # the dQ kernel with the gradient state folded in
    if dw:
        for k in ("bwdq", "bwdq_gstate", "bwdkv"):
            if k in rows:
                rows[k + "_dw"] = rows.pop(k)
        if "sum_rows" in rows:
            rows["dw_sum"] = rows.pop("sum_rows")
    return {"workload": w.name, "source_hash": kernel_source_hash(), "fetch_factor": round(f_fac, 4),
            "write_factor": round(w_fac, 4), "kernels": rows}


def load_traffic(w, kernel):
    """HBM bytes per launch of `kernel` from the committed summaries of this workload (the
    plain step's, or the dW step's), if one lists it and matches these sources."""
    for fn in (f"traffic_{w.name}.md", f"traffic_dw_{w.name}.md"):
        path = os.path.join(ROOT, "profiles", fn)
        if not os.path.exists(path):
            continue
        m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("source_hash") == kernel_source_hash() and kernel in rec.get("kernels", {}):
            return rec["kernels"][kernel]["traffic_bytes"]
    return None


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


def host_cpu():
    """The host's logical CPU count and model name (from /proc/cpuinfo)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


QUAD_SAMPLE_ROWS = 16


def cpu_baseline(w, synth, heads):
    """The fp64 oracle's linear-time (prefix) form, fwd+bwd, on batch row 0 and
    `heads` heads at full length, one thread per head; beside it, the oracle's
    quadratic form (the definition, eq. (2)) timed on QUAD_SAMPLE_ROWS evenly spaced
    rows of one head (its cost per row grows with the row index, so the sample mean
    is the mean over all rows) and extrapolated to the forward of every row."""
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
    rows = (np.arange(QUAD_SAMPLE_ROWS) * w.L) // QUAD_SAMPLE_ROWS + w.L // (2 * QUAD_SAMPLE_ROWS)
    t1 = time.perf_counter()
    oracle.attn_fwd_rows(q[0, 0], k[0, 0], v[0, 0], W, rows, w.feat)
    dq = time.perf_counter() - t1
    quad_fwd_s = dq / QUAD_SAMPLE_ROWS * w.L * w.H  # every row of every head of one batch row, one thread
    ncpu, model = host_cpu()
    return {"value": tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle, iterative prefix-sum form, fwd+bwd of batch row 0, {heads} of {w.H} heads, "
                      f"full L={w.L}, one thread per head ({dt:.1f} s); tokens credited = L*{heads}/{w.H}",
            "seconds": dt, "host_logical_cpus": ncpu, "host_cpu_model": model,
            "quadratic_fwd": {"value": w.L / quad_fwd_s, "unit": "tokens/s", "threads": 1,
                              "sample": f"fp64 oracle, quadratic form (the definition), forward of "
                                        f"{QUAD_SAMPLE_ROWS} evenly spaced rows of one head ({dq:.1f} s), "
                                        f"extrapolated to all {w.L} rows x {w.H} heads of one batch row",
                              "extrapolated": True}}


MEM_SWEEP_WINDOW = 512


def mem_sweep(torch, A, synth, w):
    """Peak HBM of one fwd+bwd step for L = 2^16 .. 2^20 at the shape of workload w
    (B, H, d, M, slice length 512, a fixed window of MEM_SWEEP_WINDOW slices).  Inputs (Q, K, V, dY, W) are
    resident before the step; the step allocates the outputs Y, dQ, dK, dV (4 L d
    bf16 per head), the workspaces and the final state.  'beyond_io' = peak step
    allocation minus those outputs: what the sliced method itself needs."""
    import ctypes
    from causal_linear_attention_amd import _lib
    rows = []
    for lg in range(16, 21):
        L = 1 << lg
        shp = (w.B, w.H, L, w.d)
        q = synth.device_normal(w.seed, synth.TID_Q, shp, w.qkv_scale).to(torch.bfloat16)
        k = synth.device_normal(w.seed, synth.TID_K, shp, w.qkv_scale).to(torch.bfloat16)
        v = synth.device_normal(w.seed, synth.TID_V, shp, 1.0).to(torch.bfloat16)
        dy = synth.device_normal(w.seed, synth.TID_DY, shp, 1.0).to(torch.bfloat16)
        W = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).to(torch.bfloat16).cuda()
        chunks = L // 512
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        P = MEM_SWEEP_WINDOW
        # as the bench step runs it: the forward keeps Y, the row statistics and (where one
        # window holds every slice) the slices' entry states for the backward
        Y, R, S, rs, st = A.attn_fwd(q, k, v, W, w.feat, chunks, window_chunks=P, want_row_stats=True,
                                     want_states=True)
        g = A.attn_bwd(q, k, v, W, dy, w.feat, chunks, window_chunks=P, Y=Y, row_stats=rs, states=st)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        dsc = A.make_desc(q, w.M, w.feat, chunks, P)
        outs = 4 * q.numel() * 2
        rows.append({"L": L, "chunks": chunks, "window_chunks": int(_lib.lib().slim_window_chunks(ctypes.byref(dsc))),
                     "inputs_bytes": 4 * q.numel() * 2, "step_peak_bytes": peak, "outputs_bytes": outs,
                     "beyond_io_bytes": peak - outs,
                     "states_kept_bytes": 0 if st is None else st.numel() * 4,
                     "ws_fwd_bytes": int(A.workspace_bytes(dsc, _lib.SLIM_PASS_FWD, st is not None)),
                     "ws_bwd_bytes": int(A.workspace_bytes(dsc, _lib.SLIM_PASS_BWD, st is not None))})
        del q, k, v, dy, W, Y, R, S, rs, st, g
        torch.cuda.empty_cache()
    return {"mem_sweep": w.name, "B": w.B, "H": w.H, "d": w.d, "M": w.M, "chunk_len": 512, "rows": rows}


def featmap_bench(torch, A, _lib, synth, w, steps, warmup):
    """slim_featmap on the workload's Q ([B, H, L, d] io dtype -> [B, H, L, M] fp32, with
    the per-row offsets): an HBM stream (read the rows, write M fp32 per row)."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = synth.device_normal(w.seed, synth.TID_Q, (w.B, w.H, w.L, w.d), w.qkv_scale).to(dt)
    W = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).to(dt).cuda() if w.feat == "favor" else None
    favor = w.feat == "favor"
    for _ in range(warmup):
        out = A.featmap(q, W, w.feat, row_offset=favor)
    del out
    torch.cuda.synchronize()
    _lib.prof_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        out = A.featmap(q, W, w.feat, row_offset=favor)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    _lib.prof_enable(False)
    prof = _lib.prof_read()
    ms, n = prof["featmap"]
    rows = w.B * w.H * w.L
    isz = 2 if w.dtype == "bf16" else 4
    by = rows * (w.d * isz + w.M * 4 + (4 if favor else 0))  # X in, phi out, row offsets out
    fl = rows * 2 * w.d * w.M if favor else 0
    kern_s = ms / n * 1e-3
    # a plain device copy of the same number of bytes, read + written, for scale
    x = torch.empty(by // 8, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 4 / ((time.perf_counter() - t1) / steps) / 1e9
    return {"featmap": w.name, "rows": rows, "d": w.d, "M": w.M, "dtype": w.dtype, "row_offsets": favor,
            "ms_per_call": round(1e3 * el, 4), "kernel_ms": round(ms / n, 5), "bytes_per_call": by,
            "gbs": round(by / kern_s / 1e9, 1), "tflops": round(fl / kern_s / 1e12, 2),
            "roofline": {"bound": "hbm", "achieved": round(by / kern_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(by / kern_s / 1e9 / PEAK_HBM_GBS, 4)},
            "plain_copy_gbs": round(copy_gbs, 1)}


DECODE_METRIC = "causal linear-attn decode tokens/s (one new token per sequence per step, state in place)"


def decode_cpu_baseline(w, synth, seqs, budget_s=10.0):
    """The fp64 oracle's decode step (its prefix form over one position) on
    `seqs` sequences x H heads, stepped until about budget_s seconds pass."""
    import numpy as np

    import oracle
    W = synth.projection(w.seed, w.M, w.d, w.w_kind).astype(np.float64) if w.feat == "favor" else None
    rng = np.random.default_rng(w.seed)
    R = np.zeros((seqs, w.H, w.d, w.M))
    S = np.zeros((seqs, w.H, w.M))
    steps = 0
    t0 = time.perf_counter()
    while True:
        q, k = (rng.standard_normal((seqs, w.H, w.d)) * w.qkv_scale for _ in range(2))
        v = rng.standard_normal((seqs, w.H, w.d))
        _, R, S = oracle.decode_step(q, k, v, W, w.feat, R, S)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s or steps >= 10000:
            break
    threads = min(seqs * w.H, 32, os.cpu_count() or 1)
    return {"value": seqs * steps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle decode step (prefix form over one position), {seqs} of {w.B} sequences "
                      f"x {w.H} heads, {steps} steps ({dt:.1f} s), one thread per head"}


def decode_main(args, torch, _lib, A, synth):
    from causal_linear_attention_amd.workloads import DECODE_HEADLINE, DECODE_WORKLOADS, decode_bytes_per_head
    w = DECODE_WORKLOADS[args.workload or DECODE_HEADLINE]
    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary, w, 1 << 30, runs=("DF", "DW"))))
        return
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    W = None
    if w.feat == "favor":
        W = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).cuda().to(dt).contiguous()

    def draw(tid, L, scale):
        return synth.device_normal(w.seed, tid, (w.B, w.H, L, w.d), scale).to(dt).contiguous()

    # the state after a prompt of w.prefix tokens (chunked forward), then one token per step
    _, R, S = A.attn_fwd(draw(synth.TID_Q, w.prefix, w.qkv_scale), draw(synth.TID_K, w.prefix, w.qkv_scale),
                         draw(synth.TID_V, w.prefix, 1.0), W, w.feat, 1)
    tok = [draw(tid, 1, sc)[:, :, 0].contiguous()
           for tid, sc in ((synth.TID_Q, w.qkv_scale), (synth.TID_K, w.qkv_scale), (synth.TID_V, 1.0))]
    torch.cuda.synchronize()

    def step():
        return A.decode_step(*tok, W, w.feat, R, S, inplace=True)[0]

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    if args.profile_run:
        for _ in range(max(1, args.steps)):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": w.name, "steps": args.steps}))
        return
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.prof_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    _lib.prof_enable(False)
    ms, n = _lib.prof_read()["decode"]
    isz = 2 if w.dtype == "bf16" else 4
    by = w.heads * decode_bytes_per_head(w) + (w.M * w.d * isz if W is not None else 0)
    avg = ms / n
    achieved = by / (avg * 1e-3) / 1e9
    rec = {
        "metric": DECODE_METRIC, "value": round(w.B * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "d": w.d, "M": w.M, "feat": w.feat, "W": w.w_kind,
                   "prompt": w.prefix, "state_bytes": w.heads * (w.d + 1) * w.M * 4,
                   "global_batch": w.B, "seq_len": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": load_traffic(w, "decode"),
                     "kernel": "decode", "ms_avg": round(avg, 5), "bytes_per_launch": by},
        "kernels": {"decode": {"ms_total": round(ms, 4), "launches": n, "ms_avg": round(avg, 5)}},
    }
    if not args.no_cpu:
        rec["cpu_baseline"] = decode_cpu_baseline(w, synth, min(w.B, 8))
    print(json.dumps(rec))


def chunk_sweep(torch, A, synth, w, dtype, window, cmax):
    """The page's time / memory / precision trade-off at op level (its Figure 2 study,
    for this one operation): for slice lengths c = 1, 2, 4, ..., cmax, one fwd+bwd step's
    time and peak HBM, and the relative discrepancy ||grad_c - grad_L|| / ||grad_L|| of
    (dQ, dK, dV) against the unsliced run; beside each, the time and peak HBM of the
    unsliced computation on an input of length c alone.  `window` = slices whose states
    are held at once (0 = automatic, about 4096 workgroups per launch; 1 = the page's
    order, one slice after another).  Peak HBM is max_memory_allocated over one step
    minus what was allocated before it (inputs resident; outputs and workspaces count)."""
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    shp = (w.B, w.H, w.L, w.d)
    q = synth.device_normal(w.seed, synth.TID_Q, shp, w.qkv_scale).to(dt)
    k = synth.device_normal(w.seed, synth.TID_K, shp, w.qkv_scale).to(dt)
    v = synth.device_normal(w.seed, synth.TID_V, shp, 1.0).to(dt)
    dy = synth.device_normal(w.seed, synth.TID_DY, shp, 1.0).to(dt)
    W = torch.from_numpy(synth.projection(w.seed, w.M, w.d, w.w_kind)).cuda().to(dt).contiguous()

    def step(qq, kk, vv, dd, chunks, win):
        # one slice per workgroup: the sweep measures the page's slice length itself
        A.attn_fwd(qq, kk, vv, W, w.feat, chunks, window_chunks=win, group_slices=1)
        return A.attn_bwd(qq, kk, vv, W, dd, w.feat, chunks, window_chunks=win, group_slices=1)[:3]

    def measure(qq, kk, vv, dd, chunks, win, reps):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        g = step(qq, kk, vv, dd, chunks, win)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        t0 = time.perf_counter()
        for _ in range(reps):
            step(qq, kk, vv, dd, chunks, win)
        torch.cuda.synchronize()
        return g, 1e3 * (time.perf_counter() - t0) / reps, peak

    full, full_ms, full_peak = measure(q, k, v, dy, 1, 0, 3)
    fnorm = sum(float(x.double().pow(2).sum()) for x in full) ** 0.5
    rows = []
    c = 1
    while c <= min(cmax or w.L, w.L):
        chunks = -(-w.L // c)
        reps = 1 if chunks > 4096 else 2 if c < 64 else 5
        g, ms, peak = measure(q, k, v, dy, chunks, window, reps)
        disc = sum(float((a.double() - b.double()).pow(2).sum()) for a, b in zip(g, full)) ** 0.5 / fnorm
        del g
        sl = [x[:, :, :c].contiguous() for x in (q, k, v, dy)]
        g, ms_c, peak_c = measure(*sl, 1, 0, 5)
        del sl, g
        rows.append({"c": c, "chunks": chunks, "ms_per_step": round(ms, 4), "step_peak_bytes": peak,
                     "grad_discrepancy": disc, "full_on_c_ms": round(ms_c, 4), "full_on_c_peak_bytes": peak_c})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        c *= 2
    # the explicit prefix-sum evaluation (eq. (4) materialised) would hold L d M fp32 per head
    return {"chunk_sweep": w.name, "dtype": dtype, "window_chunks": window, "B": w.B, "H": w.H, "L": w.L,
            "d": w.d, "M": w.M, "unsliced_ms": round(full_ms, 4), "unsliced_peak_bytes": full_peak,
            "io_bytes": 4 * q.numel() * q.element_size(),
            "explicit_prefix_state_bytes": w.B * w.H * w.L * w.d * w.M * 4, "rows": rows}


def algorithm1_sweep(torch, synth):
    """The page's Figure-2 study on a randomly initialised Performer (4 layers,
    d_model 256 = 4 heads x 64, M = 64 FAVOR+ features, d_ff 1024, alphabet 256)
    over one random string of L = 16384 tokens: one gradient evaluation by
    Algorithm 1 per slice length C (time, peak HBM, relative gradient discrepancy
    against the whole sequence in one pass), beside the whole-sequence pass and
    the whole-sequence pass on C tokens alone."""
    from causal_linear_attention_amd.performer import Performer
    cfg = dict(vocab=256, d_model=256, heads=4, layers=4, M=64, d_ff=1024)
    L = 16384
    tok = torch.from_numpy(synth.random_tokens(9, 1, L, cfg["vocab"])).cuda()
    model = Performer(**cfg, seed=9)

    def grads():
        return {n: t.grad.detach().clone() for n, t in model.parameters().items()}

    def measure(fn):
        model.zero_grad()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        t0 = time.perf_counter()
        loss = fn()
        torch.cuda.synchronize()
        return loss, 1e3 * (time.perf_counter() - t0), torch.cuda.max_memory_allocated() - base

    def full(t):
        loss = model.loss_full(t)
        loss.backward()
        return float(loss)

    measure(lambda: full(tok))  # warm-up
    lf, ms_f, mem_f = measure(lambda: full(tok))
    gf = grads()
    fnorm = sum(float(g.double().pow(2).sum()) for g in gf.values()) ** 0.5
    rows = []
    for C in (4096, 1024, 256, 64):
        lc, ms, mem = measure(lambda: model.algorithm1(tok, C))
        gc = grads()
        disc = sum(float((gc[n].double() - gf[n].double()).pow(2).sum()) for n in gf) ** 0.5 / fnorm
        _, ms_c, mem_c = measure(lambda: full(tok[:, :C]))
        rows.append({"C": C, "ms": round(ms, 1), "peak_bytes": mem, "grad_discrepancy": disc,
                     "loss_rel_diff": abs(lc - lf) / abs(lf), "full_on_C_ms": round(ms_c, 2),
                     "full_on_C_peak_bytes": mem_c})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    n_param = sum(t.numel() for t in model.parameters().values())
    return {"algorithm1": "performer_4x256_M64_L16384", "config": dict(cfg, L=L, B=1, params=n_param),
            "full_ms": round(ms_f, 1), "full_peak_bytes": mem_f, "rows": rows}


DW_PASS_KERNELS = ("bwdq_dw", "bwdq_gstate_dw", "bwdkv_dw", "dw", "dw_sum")


def kernel_records(w, prof, steps, tile, nwin, group=1):
    """Per-kernel records from the library's hipEvent timings {name: (ms total, launches)}
    over `steps` steps, and the roofline record of the dominant kernel.  Every chunk and
    scan kernel is launched once per window and covers that window's slices, so one
    launch processes head_tokens / (windows of its pass) token-heads; nwin = windows of
    the forward and plain backward, and the dW pass's are counted from its row
    contraction, launched once per window.  group: slices per workgroup (one state
    slot per group)."""
    from causal_linear_attention_amd.workloads import kernel_bytes, kernel_flops
    fl = kernel_flops(w, tile)
    # the row statistics: made by the dQ kernel unless a pass of their own ran
    by = kernel_bytes(w, group, fr="rowstat" not in prof and "stats" not in prof)
    nwin_dw = prof["dw"][1] / steps if "dw" in prof else nwin
    peak_t = PEAK_TFLOPS[w.dtype]
    kernels = {}
    for name, (ms, n) in prof.items():
        rec = {"ms_total": round(ms, 4), "launches": n, "launches_per_step": round(n / steps, 3),
               "ms_avg": round(ms / n, 5), "ms_per_step": round(ms / steps, 5)}
        units = w.head_tokens / (nwin_dw if name in DW_PASS_KERNELS else nwin)  # token-heads per launch
        if name in fl:
            rec["flop_per_launch"] = fl[name] * units
            rec["tflops"] = round(rec["flop_per_launch"] / (rec["ms_avg"] * 1e-3) / 1e12, 2)
        if name in by:
            rec["bytes_per_launch"] = by[name] * units
            rec["gbs"] = round(rec["bytes_per_launch"] / (rec["ms_avg"] * 1e-3) / 1e9, 1)
        kernels[name] = rec
    # dominant kernel: most time in the timed region; its roof is whichever of the MFMA
    # peak (its flops) and the HBM peak (its algorithmic bytes) takes longer
    dom = max(kernels, key=lambda k2: kernels[k2]["ms_total"])
    d = kernels[dom]
    t_mfma = d.get("flop_per_launch", 0.0) / (peak_t * 1e12)
    t_hbm = d.get("bytes_per_launch", 0.0) / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        achieved = d["flop_per_launch"] / (d["ms_avg"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_t, "unit": "TFLOP/s",
                    "frac": round(achieved / peak_t, 4)}
    else:
        achieved = d["bytes_per_launch"] / (d["ms_avg"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roofline.update({"traffic": load_traffic(w, dom), "kernel": dom, "ms_avg": d["ms_avg"],
                     "flop_per_launch": d.get("flop_per_launch"), "bytes_per_launch": d.get("bytes_per_launch"),
                     "mfma_frac": round(t_mfma / (d["ms_avg"] * 1e-3), 4),
                     "hbm_frac": round(t_hbm / (d["ms_avg"] * 1e-3), 4)})
    return kernels, roofline


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
    from causal_linear_attention_amd.workloads import HEADLINE, WORKLOADS, unsliced_flops

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

    if args.decode:
        decode_main(args, torch, _lib, A, synth)
        return

    if args.algorithm1:
        print(json.dumps(algorithm1_sweep(torch, synth)))
        return

    if args.chunk_sweep:
        print(json.dumps(chunk_sweep(torch, A, synth, WORKLOADS[args.workload or HEADLINE], args.sweep_dtype,
                                     args.sweep_window, args.sweep_cmax)))
        return

    if args.featmap:
        print(json.dumps(featmap_bench(torch, A, _lib, synth, WORKLOADS[args.workload or HEADLINE], args.steps,
                                       args.warmup)))
        return

    if args.mem_sweep:
        print(json.dumps(mem_sweep(torch, A, synth, WORKLOADS["favor_bf16_L1048576_d64_M64"])))
        return
    w = WORKLOADS[args.workload or HEADLINE]
    if args.pmc_summary:
        rec = pmc_summary(args.pmc_summary, w, 1 << 30, ("DWF", "DWW") if args.dw else ("F", "W"), dw=args.dw)
        print(json.dumps(rec))
        return
    q, k, v, W, dy = make_inputs(w, torch, synth)
    tile = int(_lib.lib().slim_tile_rows(__import__("ctypes").byref(A.make_desc(q, w.M, w.feat, w.chunks))))
    torch.cuda.synchronize()

    want_dw = bool(args.dw and w.backward and w.feat == "favor")

    def step(keep_stats=True):
        # the forward keeps its output, per-row denominator statistics and (one window)
        # the slices' entry states for the backward, as autograd does; keep_stats=False:
        # the backward rebuilds all of them
        keep = keep_stats and w.backward
        out = A.attn_fwd(q, k, v, W, w.feat, w.chunks, want_row_stats=keep, want_states=keep)
        Y = out[0]
        if w.backward:
            A.attn_bwd(q, k, v, W, dy, w.feat, w.chunks, want_dw=want_dw, Y=Y if keep else None,
                       row_stats=out[3] if keep else None, states=out[4] if keep else None)
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

    # the timed region: plain steps (the kernel timer's event pairs stay out of it)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the same steps with the backward recomputing the row statistics (no state kept
    # from the forward but its inputs), for comparison
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step(keep_stats=False)
    torch.cuda.synchronize()
    elapsed_recompute = time.perf_counter() - t1
    # the forward alone (no row statistics kept), for the forward-only figure
    t2 = time.perf_counter()
    for _ in range(args.steps):
        A.attn_fwd(q, k, v, W, w.feat, w.chunks)
    torch.cuda.synchronize()
    elapsed_fwd = time.perf_counter() - t2
    # per-kernel times: the same number of steps again, each kernel bracketed by hipEvents
    _lib.prof_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    _lib.prof_enable(False)
    prof = _lib.prof_read()

    ms_step = 1e3 * elapsed / args.steps
    tokens_per_s = w.tokens * args.steps / elapsed
    dsc = A.make_desc(q, w.M, w.feat, w.chunks)
    window = int(_lib.lib().slim_window_chunks(__import__("ctypes").byref(dsc)))
    group = int(_lib.lib().slim_group_slices(__import__("ctypes").byref(dsc)))
    nchunks = -(-w.L // -(-w.L // w.chunks))  # slices actually used: ceil(L / ceil(L / chunks))
    nwin = -(-nchunks // window)
    kernels, roofline = kernel_records(w, prof, args.steps, tile, nwin, group)
    isz = 2 if w.dtype == "bf16" else 4
    # minimum HBM traffic of a step: read Q K V (fwd) and Q K V dY (bwd), write Y dQ dK dV
    io = w.head_tokens * w.d * isz * (11 if w.backward else 4)
    footprint = w.head_tokens * w.d * isz * (9 if w.backward else 4)  # Q K V dY Y dQ dK dV resident
    # the work of the kernels the step actually launched (per launch x launches per step)
    step_flop = sum(r.get("flop_per_launch", 0.0) * r["launches"] for r in kernels.values()) / args.steps
    rec = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "ms_per_step_stats_recomputed": round(1e3 * elapsed_recompute / args.steps, 4),
        "ms_forward_only": round(1e3 * elapsed_fwd / args.steps, 4),
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "M": w.M, "feat": w.feat,
                   "W": w.w_kind, "chunks": w.chunks, "chunk_len": w.chunk_len, "tile": tile,
                   "group_slices": group, "window_chunks": window, "windows": nwin,
                   "dW": want_dw, "global_batch": w.B, "seq_len": w.L, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "step_tflops": round(step_flop / (ms_step * 1e-3) / 1e12, 2),
        "step_tflops_unsliced_accounting": round(unsliced_flops(w) * w.head_tokens / (ms_step * 1e-3) / 1e12, 2),
        "peak_hbm_bytes": peak, "resident_before_step_bytes": base, "step_extra_bytes": peak - base,
        "io_traffic_bytes_per_step": io, "io_gbs": round(io / (ms_step * 1e-3) / 1e9, 1),
        "io_footprint_bytes": footprint,
        "kernels": kernels,
    }
    if not args.no_mem_sweep:
        # the sub-linear memory claim, measured in the same run: peak HBM of one fwd+bwd
        # step vs L at the 1M-token workload's shape (fixed window of 512 slices)
        del q, k, v, W, dy
        torch.cuda.empty_cache()
        sw = mem_sweep(torch, A, synth, WORKLOADS["favor_bf16_L1048576_d64_M64"])
        rec["peak_hbm_vs_L"] = {k2: sw[k2] for k2 in ("mem_sweep", "B", "H", "d", "M", "chunk_len")}
        rec["peak_hbm_vs_L"]["window_chunks"] = MEM_SWEEP_WINDOW
        rec["peak_hbm_vs_L"]["rows"] = [{k2: r[k2] for k2 in ("L", "step_peak_bytes", "outputs_bytes",
                                                              "beyond_io_bytes")} for r in sw["rows"]]
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, synth, args.cpu_heads or w.H)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
