"""Benchmark of the approximate-attention prefill hot path on one MI355X.

One step = one layer of the hot path on the 128K-token Qwen2.5-VL-7B-shaped workload
(28 query / 4 KV heads, head_dim 128, 16 virtual blocks of 8K on 8 ZigZag buckets,
anchor 2048, query block 128, l_p 1024): score_select -> gather_passing ->
approx_attn_prefill, with every input already resident in HBM. Prints one JSON line.
Beside the timed steps it also times the query block's rows (query_forward), each ZigZag
bucket's attention alone, the attention with the last-level cache flushed, the one-call
layer (prefill_layer) on one stream and with the selection of later blocks on a second
stream beside the attention, and one layer for each layout of the bucket sweep (2, 4, 6, 8
buckets) and of the anchor-only baseline.

    python bench.py [--steps K] [--warmup W] [--workload c2] [--no-cpu-baseline]
                    [--profile] [--calib-copy]

``--profile`` shortens the run for rocprofv3 (no CPU baseline); ``--calib-copy`` also runs
a plain 1 GiB device copy so that HBM byte counters can be scaled against a known size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "approx-attn prefill tokens/s per layer at 128K ctx; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
ATTN_SOURCES = ["sequence_approximate_attention_score_amd/csrc/attn.hip",
                "sequence_approximate_attention_score_amd/csrc/attn_pipe.h",
                "sequence_approximate_attention_score_amd/csrc/apbv_device.h",
                "sequence_approximate_attention_score_amd/csrc/apbv_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_c2_traffic.txt")


def attention_flops(block_starts, l_anchor, l_pass, hq, d) -> float:
    """Algorithmic attention FLOPs: 4*d per visible (row, key) pair per query head."""
    pairs = 0
    for v in range(len(block_starts) - 1):
        L = int(block_starts[v + 1] - block_starts[v])
        P = l_anchor + v * l_pass
        pairs += L * P + L * (L + 1) // 2
    return float(pairs) * hq * 4 * d


def gather_bytes(lay, d) -> float:
    """Algorithmic bytes of the gather: K and V prefix rows read once and written once."""
    return 2.0 * 2.0 * lay.hkv * lay.pre_rows * d * 2


def median_ms(fn, reps: int, before=None) -> float:
    """Median duration (HIP events on the current stream) of ``fn`` over ``reps`` calls;
    ``before`` runs ahead of each call, outside its events."""
    import torch
    times = []
    for _ in range(reps):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return float(np.median(times))


def attn_source_sha() -> str:
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, or None
    if it is missing or was taken on a different attention kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != attn_source_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(x, budget_s: float = 15.0):
    """The float64 oracle, as it is, on a bounded sample of the same workload: scores and
    selection of the middle block for every KV head, and the attention of that block for as
    many query heads as fit in about ``budget_s`` seconds (one per KV group first);
    extrapolated to the whole layer by algorithmic work."""
    from oracle import apbv_oracle as orc
    w = x.w
    bs = np.asarray(x.block_starts)
    n = len(bs) - 1
    v = n // 2
    scale = 1.0 / math.sqrt(w.head_dim)
    qq, kc, vc = x.f32("q_query"), x.f32("k_ctx"), x.f32("v_ctx")
    t0 = time.perf_counter()
    s = orc.passing_scores(qq, kc, bs, w.hq, w.hkv, scale, blocks=[v])
    t_score = time.perf_counter() - t0
    # selection of every block is needed for the prefix; blocks other than v keep the top rows
    # of their (unscored) keys by position so that the sample stays bounded
    s32 = np.nan_to_num(s, nan=0.0).astype(np.float32)
    t1 = time.perf_counter()
    sel = orc.select_passing(s32, bs, w.l_pass)
    kp, vp = orc.gather_prefix(x.f32("k_anchor"), x.f32("v_anchor"), kc, vc, sel)
    t_sel = time.perf_counter() - t1
    G = w.hq // w.hkv
    order = [g * G + j for j in range(G) for g in range(w.hkv)]   # one head per group first
    L = int(bs[v + 1] - bs[v])
    rows = np.arange(bs[v], bs[v + 1])
    heads = []
    t2 = time.perf_counter()
    for h in order:                        # add heads until about budget_s of CPU work
        orc.attend(x.f32("q_ctx"), kp, vp, kc, vc, bs, w.l_anchor, w.l_pass, w.hq, w.hkv,
                   scale, rows=rows, heads=[h])
        heads.append(h)
        if time.perf_counter() - t2 >= budget_s:
            break
    t_attn = time.perf_counter() - t2
    P = w.l_anchor + v * w.l_pass
    sample_pairs = (L * P + L * (L + 1) // 2) * len(heads)
    total_pairs = attention_flops(bs, w.l_anchor, w.l_pass, 1, 1) / 4
    est = t_score * n + t_sel + t_attn * (total_pairs / sample_pairs)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    return {"value": x.N / est, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"float64 numpy oracle on block {v} of {n}: scores+selection for all "
                       f"{w.hkv} KV heads ({t_score:.1f}s), gather ({t_sel:.1f}s), attention of "
                       f"{len(heads)} of {w.hq} heads over the block's {L} rows ({t_attn:.1f}s); "
                       f"layer time extrapolated by block count (scores) and by visible "
                       f"(row, key) pairs (attention): {est:.0f}s per layer")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--calib-copy", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the approximate-attention path is built for a single "
              "MI355X (all virtual blocks on one device, no collectives); runs on more than one "
              "GPU are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sequence_approximate_attention_score_amd as apbv
    from synthetic import generate, sweep_layouts, workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w = workload(args.workload)
    print(f"# generating {w.name}: {w.description}", file=sys.stderr, flush=True)
    x = generate(w)
    up = lambda n: torch.from_numpy(x.bits[n].view(np.int16)).to(dev).view(torch.bfloat16)
    d = {n: up(n) for n in ("q_query", "q_ctx", "k_ctx", "v_ctx", "k_anchor", "v_anchor",
                            "k_query", "v_query")}
    lay = apbv.Layout(x.block_starts, l_anchor=w.l_anchor, l_query=w.l_query, l_pass=w.l_pass,
                      hq=w.hq, hkv=w.hkv, head_dim=w.head_dim, zigzag=True)
    ws = torch.empty(max(apbv.score_select_workspace(lay), 256), dtype=torch.uint8, device=dev)
    sel = torch.empty((lay.n_blocks, w.hkv, w.l_pass), dtype=torch.int32, device=dev)
    kp = torch.empty((w.hkv, lay.pre_rows, w.head_dim), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    out = torch.empty((x.N, w.hq, w.head_dim), dtype=torch.bfloat16, device=dev)
    q_ws = torch.empty(max(apbv.query_forward_workspace(lay), 256), dtype=torch.uint8, device=dev)
    q_out = torch.empty((w.l_query, w.hq, w.head_dim), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def attention(rb=0, re=0):
        apbv.approx_attn_prefill(lay, d["q_ctx"], kp, vp, d["k_ctx"], d["v_ctx"], out=out,
                                 range_begin=rb, range_end=re)

    def query_rows():
        apbv.query_forward(lay, d["q_query"], d["k_query"], d["v_query"], d["k_anchor"],
                           d["v_anchor"], d["k_ctx"], d["v_ctx"], out=q_out, workspace=q_ws)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        apbv.score_select(lay, d["q_query"], d["k_ctx"], sel=sel, workspace=ws, want_scores=False)
        if ev is not None:
            ev[1].record()
        apbv.gather_passing(lay, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"], sel,
                            k_pre=kp, v_pre=vp)
        if ev is not None:
            ev[2].record()
        attention()
        if ev is not None:
            ev[3].record()

    steps, warmup = (3, 1) if args.profile else (args.steps, args.warmup)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                    for e in evs])   # ms: score_select, gather, attention
    ms_step = (t1 - t0) * 1e3 / steps
    # beside the timed steps: the query block's rows, each ZigZag bucket alone, and the
    # attention with the 256 MB last-level cache flushed by a 512 MiB write before each call
    # (a profiled run keeps every attention launch whole, so its kernel statistics match)
    q_ms = median_ms(query_rows, 2 if args.profile else 5)
    bucket_ms, cold_ms = None, None
    if not args.profile:
        bucket_ms = [median_ms(lambda b=b: attention(b, b + 1), 3)
                     for b in range(apbv.num_buckets(lay))]
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold_ms = median_ms(attention, 5, before=lambda: flush.fill_(1))
        del flush
    # the one-call layer (apbv_prefill_layer): the three steps in order on one stream, and
    # with the selection and gather of later blocks on a second stream beside the attention
    layer_one_ms = layer_two_ms = None
    if not args.profile:
        aux = torch.cuda.Stream()

        def one_call(aux_s=None):
            apbv.prefill_layer(lay, d["q_query"], d["q_ctx"], d["k_ctx"], d["v_ctx"],
                               d["k_anchor"], d["v_anchor"], aux_stream=aux_s, sel=sel,
                               k_pre=kp, v_pre=vp, out=out, workspace=ws)
        one_call()
        one_call(aux)
        torch.cuda.synchronize()
        layer_one_ms = median_ms(one_call, 9)
        layer_two_ms = median_ms(lambda: one_call(aux), 9)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        plan = apbv.prefill_layer_plan(lay, cus)
    # the bucket-count sweep (2, 4, 6, 8 buckets) and the anchor-only baseline (l_p = 0) on
    # the same context, each as one layer: score_select -> gather_passing -> attention
    sweep = []
    if not args.profile and w.keys == "frame" and w.frame_len > 0:
        for lv in sweep_layouts(w):
            L = apbv.Layout(lv["block_starts"], l_anchor=lv["l_anchor"], l_query=w.l_query,
                            l_pass=lv["l_pass"], hq=w.hq, hkv=w.hkv, head_dim=w.head_dim,
                            zigzag=True)
            ws_v = torch.empty(max(apbv.score_select_workspace(L), 256), dtype=torch.uint8,
                               device=dev)
            sel_v = torch.empty((L.n_blocks, w.hkv, L.l_pass), dtype=torch.int32, device=dev)
            kp_v = torch.empty((w.hkv, max(L.pre_rows, 1), w.head_dim), dtype=torch.bfloat16,
                               device=dev)
            vp_v = torch.empty_like(kp_v)

            def select_gather(L=L, ws_v=ws_v, sel_v=sel_v, kp_v=kp_v, vp_v=vp_v):
                apbv.score_select(L, d["q_query"], d["k_ctx"], sel=sel_v, workspace=ws_v,
                                  want_scores=False)
                apbv.gather_passing(L, d["k_anchor"], d["v_anchor"], d["k_ctx"], d["v_ctx"],
                                    sel_v, k_pre=kp_v, v_pre=vp_v)

            def attend_v(L=L, kp_v=kp_v, vp_v=vp_v):
                apbv.approx_attn_prefill(L, d["q_ctx"], kp_v, vp_v, d["k_ctx"], d["v_ctx"],
                                         out=out)

            select_gather()
            attend_v()
            ms_sg = median_ms(select_gather, 3)
            ms_at = median_ms(attend_v, 3)
            fl = attention_flops(L.block_starts, L.l_anchor, L.l_pass, w.hq, w.head_dim)
            sweep.append({"variant": lv["name"], "virtual_blocks": L.n_blocks,
                          "buckets": apbv.num_buckets(L), "l_pass": L.l_pass,
                          "layer_ms": ms_sg + ms_at, "attention_ms": ms_at,
                          "tokens_per_s": x.N / ((ms_sg + ms_at) * 1e-3),
                          "attention_tflops": fl / (ms_at * 1e-3) / 1e12,
                          "attention_frac_of_peak": fl / (ms_at * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
            del ws_v, sel_v, kp_v, vp_v
    if args.calib_copy:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()

    flops = attention_flops(x.block_starts, w.l_anchor, w.l_pass, w.hq, w.head_dim)
    attn_ms = float(per[:, 2].mean())
    achieved = flops / (attn_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": x.N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: Qwen2.5-VL-7B-shaped layer, {x.N // 1024}K visual tokens",
                   "tokens": x.N, "virtual_blocks": lay.n_blocks, "zigzag_buckets": w.n_buckets,
                   "hq": w.hq, "hkv": w.hkv, "head_dim": w.head_dim, "l_anchor": w.l_anchor,
                   "l_query": w.l_query, "l_pass": w.l_pass},
        "roofline": {"bound": "mfma", "kernel": "attn_kernel (approx_attn_prefill)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": read_traffic(),
                     "algorithmic_flop_per_launch": flops},
        "breakdown_ms": {"score_select": float(per[:, 0].mean()), "gather": float(per[:, 1].mean()),
                         "attention": attn_ms},
        "attention_only_tokens_per_s": x.N / (attn_ms * 1e-3),
        "attention_ms_median_warm": float(np.median(per[:, 2])),
        "attention_ms_median_cold": cold_ms,
        "per_bucket_attention_ms": bucket_ms,
        "bucket_max_over_mean": (max(bucket_ms) / (sum(bucket_ms) / len(bucket_ms))
                                 if bucket_ms else None),
        "query_forward_ms": q_ms,
        "layer_with_query_rows_tokens_per_s": (x.N + w.l_query) / ((ms_step + q_ms) * 1e-3),
        "layer_one_call_ms": layer_one_ms,
        "layer_two_stream_ms": layer_two_ms,
        "layer_two_stream_tokens_per_s": x.N / (layer_two_ms * 1e-3) if layer_two_ms else None,
        "layer_two_stream_plan": ({"late_bucket_begin": plan[0], "early_blocks": plan[1]}
                                  if layer_two_ms else None),
        "gather_GBps": gather_bytes(lay, w.head_dim) / (float(per[:, 1].mean()) * 1e-3) / 1e9,
        "sweep": sweep or None,
        "cpu_baseline": None,
    }
    if not (args.profile or args.no_cpu_baseline):
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
