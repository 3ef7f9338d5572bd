"""Paged-decode benchmark on one MI355X.

One step = one ``pa_decode`` call (split-KV attention over the paged cache,
plus the LSE combine when the split count is above 1) over one batch of the
Llama-3-8B decode shape: B=256, Hq=32, Hkv=8, D=128, bf16, 16-token pages,
4096 keys per sequence, K and V caches of exactly 2 GiB each addressed
through a seeded random permutation of all 65,536 pages.  Inputs are
resident in HBM before the timed region starts.

Prints one JSON line: KV-read GB/s (algorithmic K+V bytes per step divided by
the step time), microseconds per step, the roofline entry of the attention
kernel, and the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode KV-read GB/s (% of HBM peak) + µs/step, Llama-3-8B shape, 1 GPU"
METRIC_OTHER_DECODE = "paged decode KV-read GB/s (% of HBM peak) + µs/step, 1 GPU"
TIMING_BATCHES = 5
# parity bar of the output against the f64 oracle: |y - x| <= atol + rtol * |x|
TOLERANCE = {"f32": (1e-5, 1e-5), "f16": (2e-3, 2.0 ** -8), "bf16": (2e-3, 2.0 ** -8)}


def _quantile(sorted_values, q):
    """Linear-interpolation quantile of an ascending list."""
    pos = q * (len(sorted_values) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(sorted_values) - 1)
    return sorted_values[lo] + (pos - lo) * (sorted_values[hi] - sorted_values[lo])
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak, 8 TB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # MI355X dense MFMA peaks
TRAFFIC_FILES = {
    "llama3_8b_decode": os.path.join(ROOT, "profiles", "attn_decode_llama3_8b_traffic.md"),
    "qwen3_235b_decode": os.path.join(ROOT, "profiles", "attn_decode_qwen3_235b_traffic.md"),
    "llama3_8b_decode_int8": os.path.join(ROOT, "profiles", "attn_decode_llama3_8b_int8_traffic.md"),
    "llama3_8b_decode_fp8": os.path.join(ROOT, "profiles", "attn_decode_llama3_8b_fp8_traffic.md"),
    "decode_g32_b256": os.path.join(ROOT, "profiles", "attn_decode_g32_b256_traffic.md"),
}
KERNEL_SOURCES = os.path.join(ROOT, "paged_kv_cache_195_amd", "csrc")
# the sources each workload's kernel is built from (host planning included)
_COMMON = ["device_common.h", "page_table.h", "pa_internal.h", "pa_api.cpp"]
_MFMA = ["attn_mfma.h", "attn_mfma_launch.h"]   # the decode kernel (prefill shares only the file)
TRAFFIC_SOURCES = {
    "llama3_8b_decode": _COMMON + _MFMA + ["attn_mfma_bf16.hip"],
    "qwen3_235b_decode": _COMMON + _MFMA + ["attn_mfma_bf16.hip"],
    "llama3_8b_decode_int8": _COMMON + _MFMA + ["attn_mfma_q_bf16.hip"],
    "llama3_8b_decode_fp8": _COMMON + _MFMA + ["attn_mfma_q_bf16.hip"],
    "decode_g32_b256": _COMMON + _MFMA + ["attn_mfma_rows.h", "attn_mfma_bf16.hip"],
}


def _code_only(text: str) -> str:
    """C/C++ source without comments and whitespace runs, so that a change of
    wording does not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(workload: str) -> str:
    """sha256 over the code (comments and layout stripped) of the sources the
    workload's kernel is built from."""
    h = hashlib.sha256()
    for name in sorted(TRAFFIC_SOURCES[workload]):
        with open(os.path.join(KERNEL_SOURCES, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def measured_traffic(workload: str = "llama3_8b_decode"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    path = TRAFFIC_FILES.get(workload)
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    fields = dict(re.findall(r"^\s*[-*]?\s*`?(\w+)`?\s*[:=]\s*`?([0-9a-f.e+]+)`?\s*$", text, re.M))
    if fields.get("kernel_source_sha256") != kernel_source_hash(workload):
        return None
    try:
        return int(float(fields["fetch_bytes_per_launch"]) + float(fields["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, out_gpu, budget_s: float, threads: int):
    """Time the oracle on whole sequences of the same workload until about
    ``budget_s`` of wall time is spent; also report its agreement with the GPU."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle.paged_attention as O

    ps = w.k_cache.shape[1]
    batch = w.q.shape[0]
    # spread the sample over the batch first, then fill in
    order = []
    for b in list(range(0, batch, max(1, batch // 64))) + list(range(batch)):
        if b not in order:
            order.append(b)

    def host_pages(cache, scales, rows):
        """Host copies of the pages ``rows`` reference.  8-bit pages stay codes
        here; the oracle dequantizes each page when the gather reads it, inside
        the timed work."""
        ids = sorted({int(x) for b in rows for x in w.table_host[b, : -(-w.seq_lens_host[b] // ps)]})
        idx = torch.tensor(ids, device=cache.device)
        if w.kv is None:
            pages = cache.index_select(0, idx).float().cpu().numpy()
            page_scales = None
        else:
            pages = cache.view(torch.uint8).index_select(0, idx).cpu().numpy()
            page_scales = scales.index_select(0, idx).cpu().numpy()
        lut = {pid: i for i, pid in enumerate(ids)}

        class Pages:
            shape = tuple(cache.shape)

            def __getitem__(self, pid):
                i = lut[int(pid)]
                if page_scales is None:
                    return pages[i]
                return O.dequantize_cache(pages[i:i + 1], page_scales[i:i + 1], w.kv)[0]
        return Pages()

    def one(b, kp, vp):
        return O.attention(w.q[b:b + 1].float().cpu().numpy(), kp, vp,
                           w.table_host[b:b + 1].numpy(), np.array(w.seq_lens_host[b:b + 1]),
                           w.scale, w.causal)

    atol, rtol = TOLERANCE[w.spec.dtype]
    done, elapsed, max_err, tokens, pages_read, n_bad = [], 0.0, 0.0, 0, 0, 0
    with threadpool_limits(limits=1):
        while elapsed < budget_s and len(done) < batch:
            rows = order[len(done): len(done) + threads]
            kp, vp = host_pages(w.k_cache, w.k_scale, rows), host_pages(w.v_cache, w.v_scale, rows)
            t0 = time.perf_counter()
            with cf.ThreadPoolExecutor(max_workers=threads) as ex:
                res = list(ex.map(lambda b: one(b, kp, vp), rows))
            elapsed += time.perf_counter() - t0
            for b, (xo, _) in zip(rows, res):
                y = out_gpu[b].double().cpu().numpy()
                err = np.abs(y - xo[0, 0])
                max_err = max(max_err, float(err.max()))
                n_bad += int((~(err <= atol + rtol * np.abs(xo[0, 0]))).sum())
                tokens += w.seq_lens_host[b]
                pages_read += -(-w.seq_lens_host[b] // ps)
            done.extend(rows)
    per_token = 2 * w.k_cache.shape[2] * w.k_cache.shape[3] * w.k_cache.element_size()
    nbytes = tokens * per_token
    if w.kv is not None:   # the K and V scales of every page read
        nbytes += 2 * 4 * w.k_cache.shape[2] * pages_read
    return {
        "value": round(nbytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(done)} of {batch} sequences (whole sequences, all heads), f64 NumPy, "
                  f"{threads} threads x 1 BLAS thread on {len(os.sched_getaffinity(0))} visible "
                  f"host cores, {elapsed:.1f} s wall",
        "max_abs_err_vs_gpu": max_err,
        "parity": {"ok": n_bad == 0, "elements_out_of_tolerance": n_bad,
                   "atol": atol, "rtol": rtol},
    }


def copy_calibration(mib: int, steps: int):
    """A plain copy of a known size: HBM counters read on it give the factor
    between counter units and bytes."""
    import torch

    n = mib * 2 ** 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        dst.copy_(src)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "steps": steps,
                      "ms_per_copy": round(ms, 5), "GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # ~35-70 ms of untimed steps: after input generation the GPU needs some
    # milliseconds of load to reach steady clocks (5 steps: 403 us, 100 steps:
    # 344 us per int8 step)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--splits", type=int, default=0, help="split-KV count (0 = automatic)")
    ap.add_argument("--workload", default="llama3_8b_decode",
                    choices=["llama3_8b_decode", "qwen3_235b_decode", "llama3_70b_decode",
                             "decode_b64_s8192_g8", "ragged_bf16", "tiny_f32",
                             "prefill_b4_s1024", "prefill_b1_s4096", "prefill_f16",
                             "llama3_8b_decode_int8", "llama3_8b_decode_fp8",
                             "prefill_b4_s1024_int8", "decode_g32_b256"],
                    help="decode workload (the metric is quoted on llama3_8b_decode)")
    ap.add_argument("--variant", default=None,
                    help="'contiguous' for an identity page order; 'straddle' (qwen3 only) for "
                         "a 2 GiB + 4 MiB cache")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="keys per sequence for every sequence of a decode workload (default: "
                         "the workload's own; for counter runs at several lengths)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle wall time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and replay it (no host launch cost)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for scaling HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the paged decode path "
              "is single-GPU by design", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_195_amd as pa
    from paged_kv_cache_195_amd.workloads import attention_flops, kv_bytes, make_workload

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    lens = None
    if args.seq_len is not None:
        from paged_kv_cache_195_amd.workloads import WORKLOADS
        lens = [args.seq_len] * WORKLOADS[args.workload].batch
    w = make_workload(args.workload, device="cuda", variant=args.variant, seq_lens=lens)
    shape = pa.make_shape(w.q, w.k_cache, w.v_cache, w.block_table)
    splits = pa.resolve_num_splits(shape, args.splits)
    ws_bytes = pa.workspace_bytes(shape, args.splits)
    workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.q.shape[0], 1, w.q.shape[2], w.v_cache.shape[3]), dtype=w.q.dtype,
                      device="cuda")
    lse = torch.empty(out.shape[:3], dtype=torch.float32, device="cuda")

    prefill = w.q.shape[1] > 1
    if prefill:
        out = torch.empty((w.q.shape[0], w.q.shape[1], w.q.shape[2], w.v_cache.shape[3]),
                          dtype=w.q.dtype, device="cuda")
        lse = torch.empty(out.shape[:3], dtype=torch.float32, device="cuda")

    def step():
        fn = pa.prefill if prefill else pa.decode
        fn(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, w.scale, causal=w.causal,
           num_splits=args.splits, out=out, lse=lse, workspace=workspace, k_scale=w.k_scale,
           v_scale=w.v_scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=side):
                step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
    # One timed region of exactly `steps` steps, bracketed by synchronisations;
    # events between TIMING_BATCHES equal batches (recorded without waiting)
    # give the spread of the per-step time across the region.
    stream = torch.cuda.current_stream()
    n_batches = min(TIMING_BATCHES, args.steps)
    bounds = [round(i * args.steps / n_batches) for i in range(n_batches + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in range(n_batches + 1)]
    torch.cuda.synchronize()
    events[0].record(stream)
    for i in range(n_batches):
        for _ in range(bounds[i + 1] - bounds[i]):
            run()
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = events[0].elapsed_time(events[-1]) / args.steps
    batch_us = sorted(events[i].elapsed_time(events[i + 1]) * 1e3 / (bounds[i + 1] - bounds[i])
                      for i in range(n_batches))
    spread = {"batches": n_batches, "median": round(_quantile(batch_us, 0.5), 2),
              "p10": round(_quantile(batch_us, 0.1), 2), "p90": round(_quantile(batch_us, 0.9), 2)}

    nbytes = kv_bytes(w)
    spec = w.spec
    gbps = nbytes / (ms * 1e-3) / 1e9
    if prefill:
        flops = attention_flops(w)
        tflops = flops / (ms * 1e-3) / 1e12
        line = {
            "metric": "paged causal prefill TFLOP/s (% of bf16 MFMA peak) + us/step",
            "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
            "us_per_step_over_batches": spread,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": spec.dtype, "data": "synthetic: seeded N(0,1) q/k/v, seeded page permutation",
            "config": {"workload": f"{spec.name}: {spec.description}", "num_splits": splits,
                       "flops_per_step": flops, "graph": args.graph},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_PEAK_TFLOPS[spec.dtype], "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_PEAK_TFLOPS[spec.dtype], 4), "traffic": None},
        }
        print(json.dumps(line), flush=True)
        return
    line = {
        "metric": METRIC if spec.name == "llama3_8b_decode" else METRIC_OTHER_DECODE,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "us_per_step_over_batches": spread,
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic: seeded N(0,1) q/k/v, seeded random page permutation",
        "config": {
            "workload": f"{spec.name}: {spec.description}, "
                        f"{w.k_cache.shape[0]:,} pages per cache tensor",
            "batch": w.q.shape[0], "seq_kv": max(w.seq_lens_host),
            "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
            "head_dim": spec.head_dim, "page_size": spec.page_size, "num_splits": splits,
            "page_order": args.variant or "random",
            "kv_cache": (f"{w.kv} codes + float32 scale per (page, kv head)" if w.kv
                         else spec.dtype),
            "kv_bytes_per_step": nbytes,
            "graph": args.graph,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": (measured_traffic(spec.name)
                        if (splits == 1 and not args.variant and args.seq_len is None) else None),
        },
    }
    if splits > 1:
        line["roofline"]["note"] = "step = attention + combine kernels"
    if not args.no_cpu_baseline:
        # at most 16 threads: the host CPU share of one GPU on the measuring box,
        # whatever count of cores the process is allowed to see
        visible = len(os.sched_getaffinity(0))
        threads = max(1, min(visible, 16))
        base = cpu_baseline(w, out[:, 0], args.cpu_budget, threads)
        base["host_cores_visible"] = visible
        base["gpu_over_oracle"] = round(gbps / base["value"], 1) if base["value"] > 0 else None
        line["cpu_baseline"] = base
    print(json.dumps(line), flush=True)
    if "cpu_baseline" in line and not line["cpu_baseline"]["parity"]["ok"]:
        print("bench.py: the GPU output of the timed workload disagrees with the oracle",
              file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
