"""Benchmark of the sparse MLA attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]

A step is one forward pass over the whole workload (every token, every
head): one call of the library's entry point, which launches the fused
kernel (plus the split combine for decode plans).  Inputs are resident in HBM
before the timed region.  Before every timed step a 512 MiB scratch buffer is
written and then read back (outside the step's events), so that neither the
L2 nor the 256 MB MALL holds anything of the inputs from the previous step,
and the caches hold only clean lines (a write alone leaves the MALL full of
dirty lines, whose write-back the next step would pay for); the step itself is
bracketed by HIP events on its stream, and the median over the K steps is the
step time.  The K steps with their flushes run between two device
synchronisations.  Prints one JSON line.

Default workload: prefill, 4096 query tokens, h_q 64, topk 2048, d_qk 576,
d_v 512, one shared bf16 KV of 65536 rows, indices uniform without
replacement per token.

``roofline``: algorithmic FLOPs of one launch (2·h_q·(d_qk + d_v) per valid
slot) over the median launch duration, measured with HIP events recorded on
the stream the kernel runs on, against the MI355X dense bf16 MFMA peak; for
the decode workloads (HBM-bound) the algorithmic bytes of one launch over the
same duration against the 8 TB/s HBM peak.
``binding``: the gathered rows (every valid slot's KV row) per launch over the
same duration, against the measured random-row gather ceiling of the memory
system (``profiles/gather_ceiling.json``, from ``bench/micro/gather_ceiling``):
the roof that actually binds a kernel whose rows come at random from the MALL
or HBM.
``cpu_baseline``: the float64 CPU oracle timed on this host over a bounded
sample of the same workload's tokens, with every BLAS thread and with one.
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

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "sparse_mla_attention_fwd_amd", "csrc")
FLUSH_MIB = 512                  # > 2x the 256 MB MALL, > 60x one XCD's 4 MB L2


def gather_ceiling(w):
    """The measured random-row gather ceiling that applies to a workload:
    (GB/s, regime name) from profiles/gather_ceiling.json, or (None, None)."""
    path = os.path.join(ROOT, "profiles", "gather_ceiling.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    if w.seqs == 1:
        key = "bf16_mall"            # one shared KV that fits the MALL
    else:
        key = {"bf16": "bf16_hbm", "fp8": "fp8_hbm", "fp4": "fp8_hbm"}[w.kv_format]
    c = rec.get("ceilings", {}).get(key)
    return (c["gbs"], c["regime"]) if c else (None, None)


def cpu_description():
    """CPU model name and the BLAS library numpy calls."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', 'n/a')})"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return model, ", ".join(blas) or "unknown"


def kernel_hash() -> str:
    """sha256[:16] over the device sources (csrc/*.hip, *.cuh, *.h in name
    order): a traffic summary applies only to the kernels it was taken on."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".cuh", ".h")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, per_launch_flops: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"smla_fwd_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def algorithmic_bytes(w) -> int:
    """HBM bytes one launch must move at least: every valid slot's KV row
    (1152 bytes bf16; 576 (fp8) or 288 (fp4) code bytes + 20 scale bytes) when the rows are
    not reused (decode: each sequence's slots are distinct rows of its own
    cache), else the KV once; plus Q, out, lse, the indices and a block table."""
    row = {"bf16": 1152, "fp8": 576 + 20, "fp4": 288 + 20}[w.kv_format]
    kv = w.valid_slots * row if w.seqs > 1 else w.s_kv * row
    table = w.s_q * (w.rows_per_seq // w.page_size) * 4 if w.page_size else 0
    return kv + w.s_q * w.h_q * (576 + 512) * 2 + w.s_q * w.h_q * 4 + w.s_q * w.topk * 4 + table


def cpu_baseline(x, budget_s: float):
    """The float64 oracle timed on this host: with every BLAS thread for
    budget_s seconds of oracle time, then with one thread for a third of that
    (each on the first tokens of the workload, at least 16)."""
    from threadpoolctl import threadpool_limits
    res = _cpu_oracle_rate(x, budget_s)
    with threadpool_limits(limits=1):
        one = _cpu_oracle_rate(x, budget_s / 3)
    model, blas = cpu_description()
    res["single_thread"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}
    res["cpu_model"] = model
    res["blas"] = blas
    res["logical_cpus"] = os.cpu_count()
    return res


def _cpu_oracle_rate(x, budget_s: float):
    """Time the float64 oracle on the first tokens of the workload until the
    time budget is used (at least 16 tokens)."""
    import numpy as np
    import torch

    import workloads
    from oracle import sparse_mla_fwd_exact

    w = x["workload"]
    idx = x["indices"].numpy()
    done, t_used, chunk = 0, 0.0, 16
    if w.page_size:
        # paged oracle on each token's own pages (float64 copies made outside the timing)
        from oracle import sparse_mla_fwd_paged
        ps, table = w.page_size, x["block_table"].numpy()
        chunk = 2
        while done < w.s_q and (t_used < budget_s or done < 4):
            sl = slice(done, min(w.s_q, done + chunk))
            pages = np.unique(table[sl])
            rows = torch.from_numpy((pages[:, None] * ps + np.arange(ps)[None, :]).reshape(-1))
            kv_pages = workloads.to_f64(x["kv"][rows]).reshape(-1, ps, 576)
            remap = np.searchsorted(pages, table[sl])
            q = workloads.to_f64(x["q"][sl])
            t0 = time.perf_counter()
            sparse_mla_fwd_paged(q, kv_pages, remap, idx[sl], x["sm_scale"], 512)
            t_used += time.perf_counter() - t0
            done = sl.stop
        valid = int((idx[:done] >= 0).sum())
        return _cpu_result(w, valid, t_used, done, "paged float64 numpy")
    from oracle import dequant_fp4_rows, dequant_fp8_rows

    def rows_f64(sel):
        """float64 values of KV rows sel (exact for every format)."""
        if w.kv_format == "bf16":
            return workloads.to_f64(x["kv"][sel])
        dq = dequant_fp8_rows if w.kv_format == "fp8" else dequant_fp4_rows
        return dq(x["kv_codes"][sel].numpy(), x["kv_scales"][sel].numpy())

    if w.seqs > 1:
        # decode: each chunk's referenced rows only (the caches are GBs);
        # float64 copies made outside the timing
        def chunk_inputs(sl):
            ii = idx[sl]
            ok = (ii >= 0) & (ii < w.s_kv)
            rows = np.unique(ii[ok])
            remap = np.full(ii.shape, -1, dtype=np.int64)
            remap[ok] = np.searchsorted(rows, ii[ok])
            return rows_f64(torch.from_numpy(rows)), remap
    else:
        kv_all = rows_f64(torch.arange(w.s_kv))

        def chunk_inputs(sl):
            return kv_all, idx[sl]
    kv0, i0 = chunk_inputs(slice(0, 1))
    sparse_mla_fwd_exact(workloads.to_f64(x["q"][:1]), kv0, i0, x["sm_scale"], 512)  # warm BLAS
    while done < w.s_q and (t_used < budget_s or done < 16):
        sl = slice(done, min(w.s_q, done + chunk))
        q = workloads.to_f64(x["q"][sl])
        kv, ii = chunk_inputs(sl)
        t0 = time.perf_counter()
        sparse_mla_fwd_exact(q, kv, ii, x["sm_scale"], 512)
        t_used += time.perf_counter() - t0
        done = sl.stop
    valid = ((idx[:done] >= 0) & (idx[:done] < w.s_kv)).sum()
    return _cpu_result(w, valid, t_used, done, f"float64 numpy ({w.kv_format} KV values)")


def _cpu_result(w, valid, t_used, done, kind):
    from threadpoolctl import threadpool_info
    flops = 2.0 * w.h_q * (576 + 512) * float(valid)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {done} of {w.s_q} tokens of the {w.name} workload, {kind} "
                      f"(gather + two GEMMs + exact softmax per token), {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--b-topk", type=int, default=0)
    ap.add_argument("--num-splits", type=int, default=-1, help="-1: the workload's own setting")
    ap.add_argument("--schedule", choices=["auto", "grid", "persistent"], default="auto",
                    help="work schedule: the planner's choice, one workgroup per token, or persistent")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time; 0 skips")
    ap.add_argument("--flush-mib", type=int, default=FLUSH_MIB,
                    help="MiB written before every timed step to evict the inputs from L2 and MALL")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(query tokens are independent, so they would shard across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mla_attention_fwd_amd as smla
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A plain copy of known size: under rocprofv3 its FETCH_SIZE / WRITE_SIZE
        # give the factor that turns those counters into bytes.
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    w = workloads.WORKLOADS[args.workload]
    x = workloads.make_inputs(w)
    q = x["q"].to(dev)
    idx = x["indices"].to(dev)
    if w.kv_format == "fp8":
        kv = smla.pack_fp8_kv(x["kv_codes"], x["kv_scales"], dev)
    elif w.kv_format == "fp4":
        kv = smla.pack_fp4_kv(x["kv_codes"], x["kv_scales"], dev)
    else:
        kv = x["kv"].to(dev)
    fmt = w.kv_format
    ns = w.num_splits if args.num_splits < 0 else args.num_splits
    out = torch.empty((w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.s_q, w.h_q), dtype=torch.float32, device=dev)
    p = smla.make_params(q, kv, idx, x["sm_scale"], out, lse,
                         kv_format={"bf16": smla.SMLA_KV_BF16, "fp8": smla.SMLA_KV_FP8_E4M3,
                                    "fp4": smla.SMLA_KV_FP4_E2M1}[fmt],
                         num_splits=ns, b_topk=args.b_topk,
                         schedule={"auto": smla.SMLA_SCHEDULE_AUTO, "grid": smla.SMLA_SCHEDULE_GRID,
                                   "persistent": smla.SMLA_SCHEDULE_PERSISTENT}[args.schedule])
    plan_splits, plan_bt = smla.smla_fwd_plan(p)
    plan_schedule = {smla.SMLA_SCHEDULE_GRID: "grid",
                     smla.SMLA_SCHEDULE_PERSISTENT: "persistent"}[smla.smla_fwd_schedule(p)]
    if w.page_size:
        bt = x["block_table"].to(dev)
        paged = smla.make_paged(bt, w.page_size)
        need = smla.smla_fwd_paged_workspace_size(p, paged)
    else:
        need = smla.smla_fwd_workspace_size(p)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    p.workspace, p.workspace_bytes = ws.data_ptr(), ws.numel()
    stream = torch.cuda.current_stream()

    def step():
        if w.page_size:
            smla.smla_fwd_paged(p, paged, torch.cuda.current_stream().cuda_stream)
        else:
            smla.smla_fwd(p, torch.cuda.current_stream().cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        # one step captured once (torch captures on a side stream) and
        # replayed on the current stream: the host cost of a step becomes one
        # graph launch
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

        def step():
            graph.replay()
        step()
        torch.cuda.synchronize()

    # Per-step durations with events on the launch stream.  Before each step a
    # scratch buffer larger than the MALL is written and read back (outside
    # the events), so the step finds its inputs in HBM, not in a cache warmed
    # by the last step, and no dirty flush lines are left for it to evict.
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib > 0 else None
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
            flush.view(torch.int32).amax()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))
    n = len(launch_ms)
    median_ms = launch_ms[n // 2] if n % 2 else 0.5 * (launch_ms[n // 2 - 1] + launch_ms[n // 2])
    mean_ms = sum(launch_ms) / n
    step_s = median_ms / 1e3

    flops = w.flops
    value = flops / step_s / 1e12
    traffic = load_traffic(w.name, flops)
    row_bytes = {"bf16": 1152, "fp8": 640, "fp4": 320}[fmt]
    gathered = w.valid_slots * row_bytes
    gather_gbs = gathered / step_s / 1e9

    if w.seqs > 1:
        # decode: HBM-bound (arithmetic intensity below the MFMA/HBM ridge)
        alg = algorithmic_bytes(w)
        gbs = alg / step_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes": alg, "tflops": round(value, 2)}
    else:
        roofline = {"bound": "mfma", "achieved": round(value, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": traffic}
    ceiling, regime = gather_ceiling(w)
    binding = {"bound": "gather", "achieved": round(gather_gbs, 1), "unit": "GB/s",
               "ceiling": ceiling, "frac": round(gather_gbs / ceiling, 4) if ceiling else None,
               "ceiling_regime": regime, "source": "profiles/gather_ceiling.md",
               "gathered_bytes_per_launch": gathered}
    res = {
        "metric": "sparse MLA fwd TFLOP/s and % bf16 MFMA peak (h_q=64, topk=2048, d_qk=576)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(median_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "s_q": w.s_q, "h_q": w.h_q, "topk": w.topk, "s_kv": w.s_kv,
                   "d_qk": 576, "d_v": 512, "kv_format": fmt, "num_splits": plan_splits,
                   "page_size": w.page_size or None, "hip_graph": bool(args.graph),
                   "b_topk": plan_bt, "schedule": plan_schedule, "parallelism": "single GPU"},
        "roofline": roofline,
        "binding": binding,
        "timing": {"statistic": f"median of {n} steps, HIP events on the launch stream",
                   "median_ms": round(median_ms, 4), "mean_ms": round(mean_ms, 4),
                   "min_ms": round(launch_ms[0], 4), "max_ms": round(launch_ms[-1], 4),
                   "flush_mib_before_each_step": args.flush_mib,
                   "wall_ms_per_step_with_flush": round(wall / args.steps * 1e3, 4)},
    }
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
