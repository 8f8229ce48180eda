"""Decode-attention benchmark: one decode step of the paged GQA workload on one GPU.

Workload (the one the >= 70 %-of-HBM target is stated for): batch 32, 64 q heads /
8 kv heads (group 8), head dim 128, bf16 ~ N(0, 1), page size 64, per-sequence
KV length uniform in [512, 32768] (seed 3: 626 521 keys), page table a seeded
random permutation of the page pool, splits chosen per sequence.

A step is one call of decode_attn_splitk_fused on inputs already resident in HBM: the
partition kernel, then the LSE combine, either by each group's last-arriving workgroup
(where that beats a second launch: small sets of partials) or by the combine launch
(--combine separate forces the latter). The K timed steps run one at a time, each after the
Infinity Cache has been flushed (1 GiB read and written outside the step's HIP events),
so that no input is served from the memory-side cache of the step before. Output: one
JSON line with
  value / ms_per_step  KV-read GB/s of the whole step (algorithmic bytes: attended keys
                 x kv heads x (Dqk + Dv) x 2 B) and the step time, both from the median
                 of the K per-step HIP-event times (p10 / p90 in step_us_events_cache_flushed)
  step_us_back_to_back  labelled extra: the same steps issued back to back without a flush
                 (wall clock over K steps, and per-step event times)
  roofline       the partition kernel alone, timed with HIP events on its stream (cache
                 flushed before every launch), against the 8 TB/s HBM peak; traffic from the
                 committed rocprofv3 counter summary when it matches the current source
  cpu_baseline   the fp64 CPU oracle timed on this host's cores
Other workloads can be timed with --workload (not the reported line by default).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_partition_mfma128_paged_gqa.json")
KERNEL_SOURCES = ["partition_mfma.h", "partition_mfma128.hip", "da_device.h", "da_internal.h"]


def kernel_source_hash():
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "lse_combine_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="paged_gqa")
    ap.add_argument("--num-splits", type=int, default=None, help="override the workload's split count")
    ap.add_argument("--kernel", default="auto", choices=["auto", "fma", "mfma"])
    ap.add_argument("--combine", default="auto", choices=["auto", "separate", "fused", "fused-force"],
                    help="auto (= fused): the fused entry point, which folds the partials in each group's "
                         "last-arriving workgroup where that beats a second launch and runs the combine launch "
                         "otherwise; separate: always the combine launch; fused-force: always the fold in pass 1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--probe-gib", type=float, default=2.0, help="streaming-read probe size")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this engine has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    from lse_combine_amd import _lib, api
    from lse_combine_amd.inputs import to_device, workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    overrides = {} if args.num_splits is None else {"num_splits": args.num_splits}
    case = workload(args.workload, **overrides)
    dc = to_device(case, dev)
    kv_bytes = case.kv_bytes()
    tokens = int(case.seq_lens.clamp(min=0).sum())
    print(f"[bench] workload {case.name}: {tokens} keys, KV {kv_bytes / 1e9:.3f} GB", file=sys.stderr, flush=True)

    prob = api.make_problem(dc.q, dc.k_cache, dc.v_cache, dc.page_table, page_size=case.page_size,
                            v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, kernel=args.kernel,
                            k_rope=dc.k_rope)
    chunk, max_splits = api.choose_splits(prob, case.num_splits)
    B, Hq, Dv = prob.batch, prob.num_q_heads, prob.ov_depth
    rows = api.row_shape(prob)   # (B, Hq), or (B, q_len, Hq) with several queries per sequence
    out = torch.empty(rows + (Dv,), dtype=torch.bfloat16, device=dev)
    part_o, part_ml = api.alloc_partials(prob, chunk, max_splits, dev)
    comb = (torch.empty_like(out), torch.empty(rows, dtype=torch.float32, device=dev),
            torch.empty(rows + (Dv,), dtype=torch.float32, device=dev))
    api.check_outputs(prob, *comb)

    plan = api.DecodePlan(dc.q, dc.k_cache, dc.v_cache, dc.page_table, dc.seq_lens, case.scale, case.num_splits,
                          page_size=case.page_size, v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth,
                          kernel=args.kernel, out=out,
                          fused={"separate": False, "auto": True, "fused": True, "fused-force": "force"}[args.combine],
                          k_scale=dc.k_scale, v_scale=dc.v_scale, k_rope=dc.k_rope)
    step = plan.run

    # --- streaming-read probe and a copy of known size (counter calibration) ---
    lib = _lib.load()
    probe = _lib.load_probe()
    import ctypes
    probe_bytes = int(args.probe_gib * (1 << 30)) // 16 * 16
    probe_src = torch.empty(probe_bytes, dtype=torch.uint8, device=dev)
    probe_src.fill_(1)
    sink = torch.zeros(4096, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    probe_times = []
    for i in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if probe.da_read_probe(ctypes.c_void_p(probe_src.data_ptr()), probe_bytes, ctypes.c_void_p(sink.data_ptr()),
                               stream):
            raise RuntimeError("read probe launch failed")
        e1.record()
        torch.cuda.synchronize()
        if i:
            probe_times.append(e0.elapsed_time(e1) / 1e3)
    read_probe_gbps = probe_bytes / statistics.median(probe_times) / 1e9
    copy_bytes = 256 << 20
    copy_dst = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    if probe.da_copy_probe(ctypes.c_void_p(probe_src.data_ptr()), ctypes.c_void_p(copy_dst.data_ptr()), copy_bytes,
                           stream):
        raise RuntimeError("copy probe launch failed")
    torch.cuda.synchronize()
    del probe_src, copy_dst

    # The Infinity Cache (256 MiB) is flushed before every timed step and launch: 1 GiB read
    # and written outside the events, so that a step's inputs are never served from the
    # memory-side cache of the step before.
    flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)

    def summary(us):
        us = sorted(us)
        pick = lambda f: us[min(len(us) - 1, int(f * len(us)))]
        med = statistics.median(us)
        return {"p10": round(pick(0.1), 2), "median": round(med, 2), "p90": round(pick(0.9), 2),
                "kv_GBps_median": round(kv_bytes / (med * 1e-6) / 1e9, 1)}

    # --- warm-up, then EXACTLY `steps` timed steps, each after a flush ---
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e0, e1 in evs:
        flush_buf.add_(1)
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    flushed_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
    step_flushed = summary(flushed_us)
    s_per_step = statistics.median(flushed_us) * 1e-6
    value = kv_bytes / s_per_step / 1e9

    # --- labelled extra: the same steps back to back, with no flush in between ---
    torch.cuda.synchronize()
    b0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    b1 = time.perf_counter()
    hot_wall_s = (b1 - b0) / args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    step_hot = summary([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    step_hot["wall_us_per_step"] = round(hot_wall_s * 1e6, 2)
    step_hot["kv_GBps_wall"] = round(kv_bytes / hot_wall_s / 1e9, 1)

    # --- the partition kernel alone (same kernels, launched pass by pass) ---
    # arguments are marshalled once so the host stays ahead of the GPU and the
    # events bracket only the kernels
    P_ = ctypes.c_void_p

    def ptr(t):
        return None if t is None else P_(t.data_ptr())

    if case.k_rope is not None:
        kv = _lib.DaKv(dc.k_cache.data_ptr(), None if dc.v_cache is None else dc.v_cache.data_ptr(),
                       dc.k_rope.data_ptr(),
                       None if dc.k_scale is None else dc.k_scale.data_ptr(),
                       None if dc.v_scale is None else dc.v_scale.data_ptr())
        part_fn = lib.decode_attn_partition_kv
        part_args = (ctypes.byref(prob), ptr(dc.q), ctypes.byref(kv), ptr(dc.page_table), ptr(dc.seq_lens),
                     float(case.scale), chunk, max_splits, ptr(part_o), ptr(part_ml), stream)
    elif case.kv_fp8:
        part_fn = lib.decode_attn_partition_fp8
        part_args = (ctypes.byref(prob), ptr(dc.q), ptr(dc.k_cache), ptr(dc.v_cache), ptr(dc.k_scale),
                     ptr(dc.v_scale), ptr(dc.page_table), ptr(dc.seq_lens), float(case.scale), chunk, max_splits,
                     ptr(part_o), ptr(part_ml), stream)
    else:
        part_fn = lib.decode_attn_partition
        part_args = (ctypes.byref(prob), ptr(dc.q), ptr(dc.k_cache), ptr(dc.v_cache), ptr(dc.page_table),
                     ptr(dc.seq_lens), float(case.scale), chunk, max_splits, ptr(part_o), ptr(part_ml), stream)
    comb_args = (ctypes.byref(prob), P_(dc.seq_lens.data_ptr()), float(case.scale), chunk, max_splits,
                 P_(part_o.data_ptr()), P_(part_ml.data_ptr()), P_(comb[0].data_ptr()), P_(comb[1].data_ptr()),
                 P_(comb[2].data_ptr()), stream)
    part_ms, comb_ms = [], []
    n_timed = max(args.steps, 10)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_timed)]
    for i in range(n_timed):
        flush_buf.add_(1)
        evs[i][0].record()
        _lib.check(part_fn(*part_args))
        evs[i][1].record()
        _lib.check(lib.decode_attn_combine(*comb_args))
        evs[i][2].record()
    torch.cuda.synchronize()
    del flush_buf
    for e in evs:
        part_ms.append(e[0].elapsed_time(e[1]))
        comb_ms.append(e[1].elapsed_time(e[2]))
    part_s = statistics.mean(part_ms) / 1e3
    achieved = kv_bytes / part_s / 1e9

    traffic = None
    if args.workload == "paged_gqa" and args.kernel == "auto" and os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash() and tr.get("chunk") == chunk:
            traffic = tr.get("hbm_bytes_per_launch")

    result = {
        "metric": "decode attention \u00b5s/step + KV-read GB/s (% of HBM peak), 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s_per_step * 1e3, 4),
        "us_per_step": round(s_per_step * 1e6, 2),
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "timing": "median of the per-step HIP-event times, Infinity Cache flushed before every step",
        "timed_region_wall_s": round(t1 - t0, 4),
        "step_us_events_cache_flushed": step_flushed,
        "step_us_back_to_back": step_hot,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype_name,
        "data": "synthetic (seeded torch.randn" + (", E4M3 K/V with per-token scales" if case.kv_fp8 else "")
                + (", rotary K columns stored apart in bf16" if case.k_rope is not None else "") + ")",
        "config": {
            "workload": case.name,
            "batch": B, "q_len": max(1, prob.q_len), "q_heads": Hq, "kv_heads": prob.num_kv_heads,
            "qk_depth": prob.qk_depth, "ov_depth": Dv, "nope_depth": prob.nope_depth, "page_size": case.page_size,
            "keys": tokens, "max_seq_len": int(case.seq_lens.max()),
            "num_splits": case.num_splits, "chunk_tokens": chunk, "max_splits": max_splits, "kernel": args.kernel,
            "combine": ("fold in pass 1 (last-arriving workgroup)" if args.combine == "fused-force" or
                        (args.combine in ("auto", "fused") and api.fused_applies(prob, case.num_splits))
                        else "combine launch"),
            "kv_bytes": kv_bytes,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "partition (split-K pass 1)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
            "partition_us_mean": round(part_s * 1e6, 2),
            "partition_us_median": round(statistics.median(part_ms) * 1e3, 2),
            "combine_us_mean": round(statistics.mean(comb_ms) * 1e3, 2),
            "read_probe_GBps": round(read_probe_gbps, 1),
            "frac_of_read_probe": round(achieved / read_probe_gbps, 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, kv_bytes, args.cpu_budget_s)
    print(json.dumps(result), flush=True)


def cpu_baseline(case, kv_bytes, budget_s):
    """The fp64 oracle on this host: the full step if it fits the budget, else a prefix of sequences."""
    import numpy as np
    import threadpoolctl

    from oracle import decode_attention_fp64

    lens = case.seq_lens.clamp(min=0).numpy().astype(np.int64)
    q = case.q.float().numpy()
    pt = None if case.page_table is None else case.page_table.numpy()
    # (fp8 caches stay raw E4M3 codes; the oracle decodes them with their scales)
    k = case.k_cache.numpy() if case.kv_fp8 else case.k_cache.float().numpy()
    v = None if case.v_cache is None else (case.v_cache.numpy() if case.kv_fp8 else case.v_cache.float().numpy())
    ks = None if case.k_scale is None else case.k_scale.numpy()
    vs = None if case.v_scale is None else case.v_scale.numpy()
    kr = None if case.k_rope is None else case.k_rope.float().numpy()
    info = threadpoolctl.threadpool_info()
    blas = [i for i in info if i.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else 1
    times = []
    t_start = time.perf_counter()
    while len(times) < 3:
        t0 = time.perf_counter()
        decode_attention_fp64(q, k, v, lens, case.scale, page_table=pt, page_size=case.page_size,
                              v_is_k_prefix=case.v_is_k_prefix, ov_depth=case.ov_depth, k_scale=ks, v_scale=vs,
                              k_rope=kr)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start + times[-1] > budget_s:
            break
    t = statistics.median(times)
    return {
        "value": round(kv_bytes / t / 1e9, 3),
        "unit": "GB/s",
        "us_per_step": round(t * 1e6, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"the full {case.name} step ({int(lens.sum())} keys, {case.batch} sequences), "
                  f"median of {len(times)} run(s); numpy fp64, BLAS {blas[0]['internal_api'] if blas else '?'} "
                  f"with {threads} threads (elementwise numpy is single-threaded); "
                  f"host affinity {len(os.sched_getaffinity(0))} cores",
    }


if __name__ == "__main__":
    main()
