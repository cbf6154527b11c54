#!/usr/bin/env python3
"""Benchmark: lightning-indexer score + top-k on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step is the whole hot path over one batch of synthetic input: the fused
score + top-k entry point of the workload's kind.  The timed region is
exactly K steps between two synchronisations: by default the replays of HIP
graphs captured from the K steps' calls, split into (at most) ten batches of
consecutive steps with an event between batches (so the Python binding's
per-call cost is not timed; the last outputs are checked bit for bit against
the same step issued eagerly, and the eager rate is reported beside it), with
--eager the K calls themselves.  ``ms_per_step`` is the whole region over K;
``ms_per_step_median`` the median over the batches.  Inputs are resident in
HBM before it starts, and several copies of them are rotated so that
consecutive steps do not hit the 256 MB Infinity Cache.

Prints ONE JSON line: throughput in visible (token, key) pairs per second,
the roofline of the dominant kernel (its average duration measured with HIP
events on the launch stream over its own timed loop of K launches, replayed
the same way; also the score and top-k kernels on their own), floors of
the launches timed the same way (``floors_ms``: an empty kernel on each
kernel's grid, the top-k's bytes moved without selecting, a plain read of
the paged score's bytes), and the CPU oracle timed on a bounded sample of
the same workload as a baseline.

Workloads (``--config``):
  tiny            16 tokens x 256 keys, 4 heads of 64, top-32
  decode          32 requests x 1 query, 1024..8192 paged keys, 64 heads of 128, top-512
  spec_decode     32 requests x 4 queries, 16384 paged keys, top-2048
  prefill_causal  8192 tokens x 8192 keys, causal f16 mask, top-2048
  long_chunk      1024-token chunk x 131072 keys, causal, top-2048 (default: the
                  largest workload, 2.19 TFLOP of visible pairs per step)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
MALL_BYTES = 256 << 20


CSRC = os.path.join(ROOT, "sparse_attention_lightning_indexer_amd", "csrc")
# sources whose change makes a stored byte count stale, per kernel
KERNEL_SOURCES = {
    "score": ["score_kernel.hip", "device_common.h", "internal.h"],           # contiguous keys
    "score_paged": ["decode_kernel.hip", "device_common.h", "internal.h"],    # paged decode
    "topk": ["topk_kernel.hip", "device_common.h", "internal.h"],
    "stream_score": ["score_kernel.hip", "stream_select.h", "device_common.h", "internal.h"],
    "stream_merge": ["stream_topk.hip", "stream_select.h", "device_common.h", "internal.h"],
    "pool": ["pool_kernel.hip", "device_common.h", "internal.h"],
}
TRAFFIC_MARK = "traffic-record:"


PAGED_CONFIGS = ("decode", "spec_decode")


def source_digest(kernel: str, config: str = "") -> str:
    """Digest of the sources a kernel role is built from (the score role's
    kernels differ between paged and contiguous workloads)."""
    import hashlib
    if kernel == "score" and config in PAGED_CONFIGS:
        kernel = "score_paged"
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def kernel_role(name: str):
    if "pool_keys_kernel" in name:
        return "pool"
    if "stream_merge" in name:
        return "stream_merge"
    if "score_kernel<" in name and name.replace(" ", "").split(">")[0].endswith("true"):
        return "stream_score"  # the streaming instance (last template flag)
    if "stream_pc_kernel" in name or "decode_kernel" in name or "score_kernel" in name:
        return "score"
    if "topk" in name:
        return "topk"
    return None


def traffic_path(config: str) -> str:
    return os.path.join(ROOT, "profiles", f"{config}_hbm_traffic.md")


def stored_traffic(config: str, kernel: str):
    """HBM bytes per launch of `kernel` on workload `config` from the
    committed counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the
    plain copy's reading), or None when there is none or the kernel's
    sources have changed since the counters were taken."""
    try:
        with open(traffic_path(config)) as f:
            lines = [ln for ln in f if ln.strip().startswith(TRAFFIC_MARK)]
    except OSError:
        return None
    for ln in lines:
        rec = json.loads(ln.strip()[len(TRAFFIC_MARK):])
        if rec.get("kernel") == kernel and rec.get("source") == source_digest(kernel, config):
            return rec["bytes_per_launch"]
    return None


def pmc_summary(config: str, fetch_dir: str, write_dir: str, calib_mib: int) -> str:
    """Markdown summary of two rocprofv3 counter runs of this benchmark
    (--pmc FETCH_SIZE, then --pmc WRITE_SIZE, both with --calib-copy-mib):
    per kernel the mean KiB per dispatch, scaled so that the plain copy
    reads and writes exactly the bytes it moves."""
    import csv
    import glob

    def per_kernel(d):
        out = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: (len(v), sum(v) / len(v)) for k, v in out.items()}

    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    calib_kib = calib_mib * 1024.0
    # the copy: writes the calibration size and reads a good part of it
    # (a fill of the same size writes as much but reads almost nothing)
    copy = min((k for k in write if k in fetch and fetch[k][1] > 0.25 * calib_kib),
               key=lambda k: abs(write[k][1] - calib_kib))
    f_scale, w_scale = calib_kib / fetch[copy][1], calib_kib / write[copy][1]
    lines = [f"| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | "
             f"HBM MB/launch (scaled) |", "|---|---|---|---|---|"]
    records = []
    for k in sorted(fetch):
        role = kernel_role(k)
        if role is None and k != copy:
            continue
        n, fk = fetch[k]
        wk = write.get(k, (0, 0.0))[1]
        mb = (fk * f_scale + wk * w_scale) * 1024 / 1e6
        short = k if len(k) < 90 else k[:87] + "..."
        lines.append(f"| `{short}` | {n} | {fk:.1f} | {wk:.1f} | {mb:.3f} |")
        if role is not None:
            records.append({"config": config, "kernel": role, "name": k,
                            "fetch_bytes": fk * f_scale * 1024, "write_bytes": wk * w_scale * 1024,
                            "bytes_per_launch": (fk * f_scale + wk * w_scale) * 1024,
                            "source": source_digest(role, config)})
    txt = "\n".join(lines)
    txt += (f"\n\nCalibration: the plain copy (`{copy[:60]}...`) moves {calib_mib} MiB each way; "
            f"FETCH_SIZE read {fetch[copy][1]:.1f} KiB for it (scale {f_scale:.4f}), "
            f"WRITE_SIZE {write[copy][1]:.1f} KiB (scale {w_scale:.4f}).\n\n")
    txt += "\n".join(TRAFFIC_MARK + " " + json.dumps(r) for r in records) + "\n"
    return txt


def mfma_summary(config: str, counter_dir: str) -> str:
    """Markdown summary of a rocprofv3 --pmc run of this benchmark with the
    MFMA counters (SQ_INSTS_VALU_MFMA_MOPS_F16, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE) and --kernel-trace: per kernel the mean
    per dispatch, the f16 MFMA flops the hardware counted (MOPS x 512), the
    shader clock (SQ busy cycles per shader engine over the dispatch time;
    32 shader engines), the MFMA busy fraction (MFMA busy cycles over those
    cycles x 1024 SIMDs), and GRBM_GUI_ACTIVE per XCD over the dispatch time
    beside it (it reads higher than the shader clock measured inside the
    kernels with s_memtime, so the fractions use SQ_BUSY_CYCLES), and the
    VALU instructions other than MFMAs per MFMA instruction (SQ_INSTS_VALU
    counts the MFMAs too, SQ_INSTS_MFMA only them)."""
    import csv
    import glob

    vals, dur = {}, {}
    for path in glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], r["Counter_Name"])
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
    for path in glob.glob(os.path.join(counter_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                dur.setdefault(r["Kernel_Name"], []).append(
                    (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-9)
    kernels = sorted({k for k, _ in vals if kernel_role(k) == "score"})
    n_simd, n_xcd, n_se = 1024, 8, 32
    out = [f"| kernel | dispatches | MFMA f16 TFLOP counted | dispatch us | shader clock GHz | MFMA busy | "
           f"counted TFLOP/s | of the clock-scaled peak | GRBM clock GHz | other VALU per MFMA |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        def mean(c):
            v = vals.get((k, c))
            return sum(v) / len(v) if v else float("nan")
        mops = mean("SQ_INSTS_VALU_MFMA_MOPS_F16")
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
        sq = mean("SQ_BUSY_CYCLES") / n_se
        act = mean("GRBM_GUI_ACTIVE") / n_xcd
        n = len(vals.get((k, "SQ_VALU_MFMA_BUSY_CYCLES"), []))
        d = dur.get(k)
        us = sum(d) / len(d) * 1e6 if d else float("nan")
        flops = mops * 512
        n_mfma = mean("SQ_INSTS_MFMA")
        other = (mean("SQ_INSTS_VALU") - n_mfma) / n_mfma
        clk = sq / (us * 1e3)
        rate = flops / (us * 1e-6) / 1e12
        scaled = MFMA_F16_PEAK_TFLOPS * clk / 2.4
        short = k if len(k) < 70 else k[:67] + "..."
        out.append(f"| `{short}` | {n} | {flops / 1e12:.3g} | {us:.1f} | {clk:.2f} | {busy / (sq * n_simd):.3f} | "
                   f"{rate:.0f} | {rate / scaled:.3f} | {act / (us * 1e3):.2f} | {other:.2f} |")
    return "\n".join(out) + "\n"


def trace_summary(trace_dir: str) -> str:
    """Markdown table of the kernel statistics of a rocprofv3
    --kernel-trace --stats run (the *kernel_stats.csv it writes)."""
    import csv
    import glob
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    rows = []
    for path in paths:
        with open(path) as f:
            rows += list(csv.DictReader(f))
    out = ["| kernel | calls | average us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"] if len(r["Name"]) < 90 else r["Name"][:87] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="long_chunk",
                    choices=["tiny", "decode", "spec_decode", "prefill_causal", "long_chunk", "pool_keys"])
    ap.add_argument("--path", default="fused", choices=["fused", "stream"],
                    help="contiguous workloads: the fused entry point (score rows in a workspace, then the "
                         "top-k) or the streaming one (candidate lists, no score rows)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out", default=None, help="also append the JSON line to this file")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="print the markdown summary of two rocprofv3 --pmc runs of this benchmark "
                         "(FETCH_SIZE, WRITE_SIZE) for --config and exit; needs no GPU")
    ap.add_argument("--mfma-summary", metavar="COUNTER_DIR", default=None,
                    help="print the markdown summary of a rocprofv3 --pmc run with the MFMA counters "
                         "(and --kernel-trace) for --config and exit; needs no GPU")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR", default=None,
                    help="print the kernel table of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip the measured-peak probes reported beside the published peak, and the "
                         "launch floors (floors_ms)")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps (and kernels) as Python-issued launches instead of one replay of a "
                         "captured HIP graph of them")
    ap.add_argument("--no-kernel-split", action="store_true",
                    help="skip the separate score and top-k timing loops (and the roofline)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before the warmup, run a plain f32 copy kernel (out = in * 1) over this "
                         "many MiB three times: the known-size reference for hardware byte counters")
    return ap.parse_args()


DEFAULT_STEPS = {"tiny": (2000, 200), "decode": (1000, 100), "spec_decode": (300, 30),
                 "prefill_causal": (20, 3), "long_chunk": (10, 2), "pool_keys": (200, 20)}

# pooled-key producer workload: the long-context keys before pooling, four
# raw keys per pooled key (131072 pooled keys of 128 dimensions)
POOL_RAW_KEYS, POOL_SIZE, POOL_DIM = 524288, 4, 128


def visible_pairs_rows(inp) -> np.ndarray:
    """Visible keys per score row (entries the score defines as finite)."""
    if hasattr(inp, "k_cache"):
        R, Q = inp.R, inp.Q
        sl = inp.seq_lens.astype(np.int64)
        vis = np.empty(R * Q, dtype=np.int64)
        for r in range(R):
            for j in range(Q):
                vis[r * Q + j] = min(max(sl[r] - Q + 1 + j, 0), inp.max_seq_len)
        return vis
    T, P = inp.T, inp.P
    if inp.mask is not None:
        return (~np.isneginf(inp.mask.astype(np.float32))).sum(axis=1).astype(np.int64)
    return np.full(T, P, dtype=np.int64)


def score_bytes_decode(inp) -> int:
    """Algorithmic HBM bytes of one paged score launch: every key of every
    request read once (for all heads and all query tokens), q once, the
    weights, the block-table entries used, seq_lens, and the f32 score rows
    written once."""
    H, d, R, Q, bs = inp.H, inp.d, inp.R, inp.Q, inp.block_size
    L = np.minimum(inp.seq_lens.astype(np.int64), inp.max_seq_len)
    keys = int(L.sum()) * d * 2
    qb = R * Q * H * d * 2
    bt = int(np.ceil(L / bs).sum()) * 4
    out = R * Q * inp.max_seq_len * 4
    return keys + qb + H * 4 + bt + R * 4 + out


def main():
    args = parse()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.mfma_summary:
        print(mfma_summary(args.config, args.mfma_summary))
        return
    if args.pmc_summary:
        print(pmc_summary(args.config, args.pmc_summary[0], args.pmc_summary[1], args.calib_copy_mib or 1024))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the indexer has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_lightning_indexer_amd as li
    import workloads as W

    if args.config == "pool_keys":
        bench_pool(args, torch, li)
        return

    steps, warmup = DEFAULT_STEPS[args.config]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = li.load_library()  # raises if the HIP library is missing

    gen = getattr(W, args.config)
    inp = gen(0, poison=False) if args.config in ("decode", "spec_decode") else gen(0)
    paged = hasattr(inp, "k_cache")
    vis_rows = visible_pairs_rows(inp)
    pairs = int(vis_rows.sum())

    # ---- device-resident inputs, rotated copies -----------------------
    def t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if paged:
        base = dict(q=t(inp.q), k=t(inp.k_cache), mask=t(inp.mask))
        shared = dict(bt=t(inp.block_table), sl=t(inp.seq_lens), w=t(inp.w))
        n_rows, n_cols = inp.R * inp.Q, inp.max_seq_len
    else:
        base = dict(q=t(inp.q), k=t(inp.k), mask=t(inp.mask))
        shared = dict(w=t(inp.w), vis=t(inp.vis_len))
        n_rows, n_cols = inp.T, inp.P
    copy_bytes = sum(v.numel() * v.element_size() for v in base.values() if v is not None)
    n_copies = max(1, min(16, math.ceil(2 * MALL_BYTES / max(copy_bytes, 1))))
    copies = [base] + [{k2: (v.clone() if v is not None else None) for k2, v in base.items()}
                       for _ in range(n_copies - 1)]
    k_top = inp.k_top
    score = torch.empty((n_rows, n_cols), dtype=torch.float32, device=dev)
    idx = torch.empty((n_rows, k_top), dtype=torch.int32, device=dev)
    val = torch.empty((n_rows, k_top), dtype=torch.float32, device=dev)
    stream_path = args.path == "stream" and not paged
    op = li.OP_FUSED_DECODE if paged else (li.OP_STREAM_PREFILL if stream_path else li.OP_FUSED_PREFILL)
    ws = torch.empty(li.workspace_bytes(op, n_rows, n_cols, k_top), dtype=torch.uint8, device=dev)

    def run_score(c):
        if paged:
            li.score_decode(c["q"], c["k"], shared["bt"], shared["sl"], inp.Q, inp.max_seq_len,
                            shared["w"], c["mask"], out=score)
        else:
            li.score_prefill(c["q"], c["k"], shared["w"], c["mask"], shared["vis"], out=score)

    def run_topk():
        # as in the fused entry points: a contiguous row's visible prefix
        # is its row length
        li.topk(score, k_top, row_len=None if paged else shared["vis"], idx=idx, val=val)

    def run_fused(c):
        if paged:
            li.score_topk_fused_decode(c["q"], c["k"], shared["bt"], shared["sl"], inp.Q, inp.max_seq_len,
                                       shared["w"], k_top, c["mask"], workspace=ws, idx=idx, val=val)
        elif stream_path:
            li.score_topk_stream_prefill(c["q"], c["k"], shared["w"], k_top, c["mask"], shared["vis"],
                                         workspace=ws, idx=idx, val=val)
        else:
            li.score_topk_fused_prefill(c["q"], c["k"], shared["w"], k_top, c["mask"], shared["vis"],
                                        workspace=ws, idx=idx, val=val)

    # one step: the fused entry point (score kernel into a workspace, then
    # the top-k kernel)
    def step(i):
        run_fused(copies[i % n_copies])

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 18  # f32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # HIP graphs of consecutive launches fn(lo) .. fn(hi-1), captured on a
    # side stream (the library launches on torch's current stream, which
    # capture redirects); the library allocates nothing and records no
    # memset, so replays repeat the same kernels on the same buffers.
    def capture(fn, lo, hi):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(lo, hi):
                    fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g.replay()  # untimed: the first replay uploads the graph
        torch.cuda.synchronize()
        return g

    def batches(n):
        nb = min(10, n)
        edges = [round(i * n / nb) for i in range(nb + 1)]
        return [(edges[i], edges[i + 1]) for i in range(nb)]

    def timed(fn, n, graphs):
        """Exactly n launches fn(0) .. fn(n-1) in batches, an event between
        batches, one synchronisation at the end.  Returns (whole region / n,
        median over batches of the batch time per launch)."""
        parts = batches(n)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
        evs[0].record()
        for b, (lo, hi) in enumerate(parts):
            if graphs is not None:
                graphs[b].replay()
            else:
                for i in range(lo, hi):
                    fn(i)
            evs[b + 1].record()
        torch.cuda.synchronize()
        per = [evs[b].elapsed_time(evs[b + 1]) / (hi - lo) for b, (lo, hi) in enumerate(parts)]
        return evs[0].elapsed_time(evs[-1]) / n, float(np.median(per))

    def graphs_for(fn, n):
        return None if args.eager else [capture(fn, lo, hi) for lo, hi in batches(n)]

    # ---- warmup, then the timed region: exactly `steps` steps --------
    # (replays of graphs holding the K steps' launches, so that the Python
    # binding's per-call cost is not timed; --eager times the calls)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    step_graphs = graphs_for(step, steps)
    t0 = time.perf_counter()
    ms_per_step, ms_per_step_median = timed(step, steps, step_graphs)
    wall = time.perf_counter() - t0
    if step_graphs is not None:
        # the replay's outputs (those of the last step) against the same step
        # issued eagerly, bit for bit
        gi, gv = idx.clone(), val.clone()
        step(steps - 1)
        torch.cuda.synchronize()
        if not (torch.equal(gi, idx) and torch.equal(gv.view(torch.int32), val.view(torch.int32))):
            raise RuntimeError("graph replay and eager step disagree")
        del step_graphs
        ms_per_step_eager, _ = timed(step, steps, None)
    else:
        ms_per_step_eager = ms_per_step

    # check the timed outputs once (cheap sanity: every row's first index is a
    # visible key or -1)
    first = idx[:, 0].cpu().numpy()
    assert np.all((first >= -1) & (first < n_cols))

    # ---- per-kernel average durations (HIP events, same stream, K launches) --
    def avg_ms(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = graphs_for(fn, steps)
        ms = timed(fn, steps, g)
        del g
        return ms

    kernels, kernels_median = {}, {}
    if stream_path and not args.no_kernel_split:
        # the streaming call's two kernels run inside one entry point: timed
        # together, and the roofline is charged on both
        kernels["stream"], kernels_median["stream"] = avg_ms(lambda i: run_fused(copies[i % n_copies]))
    elif not args.no_kernel_split:
        kernels["score"], kernels_median["score"] = avg_ms(lambda i: run_score(copies[i % n_copies]))
        kernels["topk"], kernels_median["topk"] = avg_ms(lambda i: run_topk())

    # ---- floors of the launches, timed the same way ---------------------
    # An empty kernel on the top-k's grid (one 1024-thread workgroup per
    # row) and, for the paged score, on the persistent kernel's (one
    # 512-thread workgroup per compute unit); a kernel that reads each score
    # row's visible prefix, takes one block-wide maximum and writes the k
    # outputs (the top-k's bytes without the selection); a plain streaming
    # read of the paged score's algorithmic bytes, over rotated buffers.
    floors = None
    if not args.no_peak_probe and not stream_path and not args.no_kernel_split:
        from sparse_attention_lightning_indexer_amd import peak_probe as pp
        floors = {"empty_topk_grid": avg_ms(lambda i: pp.empty(n_rows, 1024))[0]}
        if n_cols <= 16384:
            lens = torch.from_numpy(vis_rows.astype(np.int32)).to(dev)
            pv, pi = torch.empty_like(val), torch.empty_like(idx)
            floors["topk_bytes"] = avg_ms(lambda i: pp.rows(score, lens, k_top, pv, pi))[0]
            del pv, pi
        if paged:
            cus = torch.cuda.get_device_properties(dev).multi_processor_count
            floors["empty_score_grid"] = avg_ms(lambda i: pp.empty(cus, 512))[0]
            nb = (score_bytes_decode(inp) + 15) // 16 * 16
            n_rb = max(1, min(16, math.ceil(2 * MALL_BYTES / nb)))
            bufs = [torch.zeros(nb // 4, dtype=torch.float32, device=dev) for _ in range(n_rb)]
            sink = pp.sink_for(dev)
            floors["score_bytes_read"] = avg_ms(lambda i: pp.read(bufs[i % n_rb], sink))[0]
            del bufs

    # ---- roofline of the dominant kernel --------------------------------
    out_bytes = n_rows * k_top * 8
    if "stream" in kernels:
        kern, kms = "stream", kernels["stream"]
        work = 2 * inp.H * inp.d * pairs
        roof = dict(bound="mfma", achieved=work / (kms * 1e-3) / 1e12, peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s")
    elif "score" not in kernels:
        kern, kms, work, roof = None, None, None, None
    elif kernels["score"] >= kernels["topk"]:
        kern, kms = "score", kernels["score"]
        if paged:
            work = score_bytes_decode(inp)
            roof = dict(bound="hbm", achieved=work / (kms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
        else:
            work = 2 * inp.H * inp.d * pairs
            roof = dict(bound="mfma", achieved=work / (kms * 1e-3) / 1e12, peak=MFMA_F16_PEAK_TFLOPS,
                        unit="TFLOP/s")
    else:
        kern, kms = "topk", kernels["topk"]
        work = n_rows * n_cols * 4 + out_bytes
        roof = dict(bound="hbm", achieved=work / (kms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    if roof is not None:
        roof["frac"] = roof["achieved"] / roof["peak"]
        # HBM bytes the hardware counters saw per launch of the same kernel,
        # as a rate over the same average duration (GB/s, comparable to
        # `achieved` for an HBM-bound kernel), and per launch
        tb = None if stream_path else stored_traffic(args.config, kern)
        roof["traffic"] = None if tb is None else tb / (kms * 1e-3) / 1e9
        roof["traffic_unit"] = "GB/s"
        roof["traffic_bytes_per_launch"] = tb
        roof["algorithmic_bytes_per_launch"] = work if roof["bound"] == "hbm" else None
        roof["kernel"] = kern
        roof["kernel_ms"] = kms
        if not args.no_peak_probe:
            # the same kernel against what this device sustains: an LDS-fed
            # f16 MFMA stream, or a 4 GiB streaming read
            from sparse_attention_lightning_indexer_amd.peak_probe import probe_peaks
            peaks = probe_peaks(dev)
            measured = peaks["read_gbs"] if roof["bound"] == "hbm" else peaks["mfma_f16_tflops"]
            roof["measured_peak"] = measured
            roof["frac_of_measured"] = roof["achieved"] / measured
            roof["measured_peak_probe"] = ("streaming read of 4 GiB" if roof["bound"] == "hbm" else
                                           "f16 MFMA 32x32x16, B fragments from LDS, 2 waves per SIMD, random operands")

    line = {
        "metric": "indexer score+top-k: (token,key) pairs/s; % of MFMA or HBM roofline",
        "value": pairs / (ms_per_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": ms_per_step_median,
        "ms_per_step_eager": ms_per_step_eager,
        "timing": ("eager launches" if args.eager else "replays of captured graphs of the K steps") +
                  f", {min(10, steps)} batches; ms_per_step = region / K, median over batches beside it",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": args.config, "rows": n_rows, "keys": n_cols, "heads": inp.H,
                   "head_dim": inp.d, "k_top": k_top, "visible_pairs": pairs,
                   "input_copies": n_copies, "path": "stream" if stream_path else "fused",
                   "workspace_bytes": ws.numel()},
        "roofline": roof,
        "kernels_ms": kernels,
        "kernels_ms_median": kernels_median,
        "floors_ms": floors,
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, vis_rows, args.cpu_seconds)
    text = json.dumps(line)
    print(text, flush=True)
    if args.out:
        with open(args.out, "a") as f:
            f.write(text + "\n")


def bench_pool(args, torch, li):
    """The pooled-key producer alone: K launches of indexer_pool_keys over
    rotated copies of 524288 f16 keys (128 dimensions, N(0,1)), four raw keys
    per pooled key; throughput in raw keys per second, roofline against HBM
    (one read of the raw keys, one write of the pooled keys)."""
    steps, warmup = DEFAULT_STEPS["pool_keys"]
    steps = args.steps if args.steps is not None else steps
    warmup = args.warmup if args.warmup is not None else warmup
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    li.load_library()
    gen = torch.Generator(device=dev).manual_seed(0)
    raw_bytes = POOL_RAW_KEYS * POOL_DIM * 2
    n_copies = max(1, math.ceil(2 * MALL_BYTES / raw_bytes))
    ks = [torch.randn((POOL_RAW_KEYS, POOL_DIM), device=dev, generator=gen).half() for _ in range(n_copies)]
    n_pool = -(-POOL_RAW_KEYS // POOL_SIZE)
    outs = [torch.empty((n_pool, POOL_DIM), dtype=torch.float16, device=dev) for _ in range(n_copies)]

    def step(i):
        li.pool_keys(ks[i % n_copies], POOL_SIZE, out=outs[i % n_copies])

    if args.calib_copy_mib > 0:  # the known-size copy for hardware byte counters
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    work = raw_bytes + n_pool * POOL_DIM * 2
    achieved = work / (ms * 1e-3) / 1e9
    line = {
        "metric": "pooled-key producer: raw keys/s; % of HBM roofline",
        "value": POOL_RAW_KEYS / (ms * 1e-3), "unit": "keys/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms, "timing": "eager launches", "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "pool_keys", "raw_keys": POOL_RAW_KEYS, "pool_size": POOL_SIZE,
                   "head_dim": POOL_DIM, "input_copies": n_copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": work, "kernel": "pool", "kernel_ms": ms},
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(inp, vis_rows, seconds):
    """The CPU oracle (fp64, OpenMP over the host cores) on a bounded sample
    of the same workload: score and top-k of a subset of rows, each timed on
    its own and repeated until about `seconds` of wall time in all; reported
    as visible pairs per second of score + top-k, and of each alone."""
    import oracle
    n_rows = len(vis_rows)
    # rows per repetition: keep one repetition around a second on a few cores
    budget_pairs = 400_000
    order = np.linspace(0, n_rows - 1, num=min(n_rows, 64)).astype(np.int64)
    rows, acc = [], 0
    for r in order:
        rows.append(int(r))
        acc += int(vis_rows[r])
        if acc >= budget_pairs:
            break
    if hasattr(inp, "k_cache"):
        # whole requests: the oracle scores a request's rows together
        reqs = sorted(set(r // inp.Q for r in rows))
        rows = [r * inp.Q + j for r in reqs for j in range(inp.Q)]
    rows = np.array(sorted(set(rows)))
    sample_pairs = int(vis_rows[rows].sum())
    reps, t_score, t_topk = 0, 0.0, 0.0
    while True:
        t0 = time.perf_counter()
        s = oracle.score_rows(inp, rows)
        t1 = time.perf_counter()
        oracle.topk(s, inp.k_top)
        t2 = time.perf_counter()
        t_score += t1 - t0
        t_topk += t2 - t1
        reps += 1
        if t_score + t_topk >= seconds or reps >= 1000:
            break
    el = t_score + t_topk
    return {"value": sample_pairs * reps / el, "unit": "pairs/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "score_pairs_per_s": sample_pairs * reps / t_score,
            "topk_pairs_per_s": sample_pairs * reps / t_topk,
            "sample": f"{len(rows)} of {n_rows} score rows ({sample_pairs} visible pairs), "
                      f"score then top-{inp.k_top} (timed apart: {t_score:.1f} s and {t_topk:.1f} s), "
                      f"repeated {reps}x"}


if __name__ == "__main__":
    main()
