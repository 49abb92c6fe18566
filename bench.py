"""Benchmark of the MI355X block drafter forward on one GPU.

Workload (FlashMap-shaped flow-map drafter: dim 2048, 16 heads x 128, 6 DiT layers, MLP 8192, 5 taps x 2560,
vocab 151936, random-init bf16 weights, synthetic f32 taps):
  * the timed step is one 16-slot draft block -- fm_draft_block + fm_lm_argmax (anchor slot, 6 DiT layers, head,
    lm_head GEMM fused with the per-slot argmax) -- at position 512 after a 512-row context prefill (L = 513);
  * the same drafter's context prefill of 8192 rows (fm_context_append: fc 12800 -> 2048 on the matrix cores,
    RMSNorm, 12 K/V projections with head-norm + RoPE + f16 cache stores) is timed as a second line item.

Prints one JSON line: draft blocks/s (value), the lm_head+argmax kernel against the HBM roofline (timed live with
HIP events on the stream it runs on), the prefill against the bf16/f16 MFMA roofline, and the float64 oracle timed
on the host cores on a bounded sample of the same draft step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / f16 matrix peak
METRIC = "draft blocks/sec (16-slot forward) + context-prefill tokens/sec; % HBM/MFMA peak"


def _hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_record(kernel_file: str, record: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha") != _hash(os.path.join(ROOT, "block_drafter_forward_amd", "csrc", kernel_file)):
        return None
    return rec.get("traffic_bytes_per_launch")


def draft_step_bytes(cfg, L: int) -> int:
    """Algorithmic HBM bytes of one flow-map draft block: every weight the step reads once (the anchor path, the
    DiT layers, the head, the lm_head table, the modulation table) plus the f16 K/V rows [0, L) cross-attention
    reads. Create-time tensors (fc, hidden_norm, state_norm, x_embed) are not part of the step."""
    D, Ht, F, hd, Lyr, V = cfg["dim"], cfg["target_dim"], cfg["ffn"], cfg["head_dim"], cfg["layers"], cfg["vocab"]
    w = D * Ht + 2 * D + Ht                       # anchor_proj (+bias), anchor_norm, E[anchor]
    w += Lyr * (8 * D * D + 4 * hd + 2 * F * D + F + D)
    w += Ht * D + Ht + V * Ht                     # head (+bias), lm_head
    b = 2 * w + 4 * (3 * Lyr + 1) * 3 * D         # bf16 weights, f32 modulation table
    return b + 2 * Lyr * L * D * 2


def cpu_baseline(cfg, W, budget_s: float):
    """The oracle (float64 NumPy) on the host cores: draft block + lm_head argmax at the same position."""
    from inputs import gen
    from oracle import flowmap
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    o = flowmap.FlowMapOracle(cfg, W)
    n = cfg["ctx_rows"]
    o.context_append(gen.taps(cfg, "prefill", n), 0)
    an = int(gen.anchors(cfg, "bench", 1)[0])
    out, _ = o.draft_block(an, n)       # warm-up: decodes the weights to float64
    o.lm_argmax(out)
    t0 = time.perf_counter()
    k = 0
    while True:
        out, _ = o.draft_block(an, n)
        o.lm_argmax(out)
        k += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": k / dt, "unit": "draft blocks/s", "cores": cores, "kind": "oracle",
            "sample": f"{k} draft blocks (fm_draft_block + fm_lm_argmax) of the same 512-row-context workload, "
                      f"float64 NumPy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--graph", choices=["on", "off"], default="on")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for a rocprofv3 --pmc pass: set up, run fm_lm_argmax 5 times and one elementwise kernel that "
                         "reads 1 GiB and writes 1 GiB (the counters' scale reference), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_drafter_forward_amd import fm
    from inputs import configs, gen

    cfg = configs.get("flashmap")
    lcfg = configs.get("longctx")
    print("[bench] generating weights", file=sys.stderr, flush=True)
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    d = fm.Drafter(cfg, dw)
    n = cfg["ctx_rows"]
    taps = torch.from_numpy(gen.taps(cfg, "prefill", n)).cuda()
    d.fm_context_append(taps, 0)
    T, Ht, V = cfg["block"], cfg["target_dim"], cfg["vocab"]
    anchor = torch.tensor([int(gen.anchors(cfg, "bench", 1)[0])], dtype=torch.int32, device="cuda")
    hidden = torch.empty(T, Ht, dtype=torch.float32, device="cuda")
    tokens = torch.empty(T, dtype=torch.int32, device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step():
        d.fm_draft_block(hidden, anchor=anchor, pos=n)
        d.fm_lm_argmax(hidden, T, tokens)

    if args.pmc_probe:
        step()
        for _ in range(5):
            d.fm_lm_argmax(hidden, T, tokens)
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        src.fill_(1.0)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)   # one elementwise kernel: 1 GiB read, 1 GiB written
        torch.cuda.synchronize()
        print("[bench] pmc probe done: 5 x fm_lm_argmax, one 1 GiB elementwise pass", file=sys.stderr, flush=True)
        return

    stream = torch.cuda.current_stream()
    graph = None
    if args.graph == "on":
        try:
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                step()
            stream.wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
        except Exception as e:   # capture unsupported: plain launches
            print(f"[bench] graph capture failed ({e}); timing plain launches", file=sys.stderr, flush=True)
            graph = None
    run = graph.replay if graph is not None else step

    print("[bench] warm-up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] draft step {ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    # dominant kernel: the lm_head GEMM fused with the argmax, timed alone with events on its stream
    lm_reps = max(20, args.steps // 2)
    for _ in range(3):
        d.fm_lm_argmax(hidden, T, tokens)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(lm_reps):
        d.fm_lm_argmax(hidden, T, tokens)
    ev1.record()
    torch.cuda.synchronize()
    lm_us = ev0.elapsed_time(ev1) / lm_reps * 1e3
    lm_bytes = V * Ht * 2 + T * Ht * 4
    lm_gbs = lm_bytes / (lm_us * 1e-6) / 1e9
    traffic = traffic_record("k_lm.hip", "lm_argmax_flashmap_traffic.json")

    # context prefill: 8192 rows on the long-context shape (same weights)
    print("[bench] prefill", file=sys.stderr, flush=True)
    dl = fm.Drafter(lcfg, dw)
    P = lcfg["ctx_rows"]
    ptaps = torch.from_numpy(gen.taps(lcfg, "prefill", P)).cuda()
    dl.fm_context_append(ptaps, 0)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.prefill_steps):
        dl.fm_context_append(ptaps, 0)
    ev1.record()
    torch.cuda.synchronize()
    pf_ms = ev0.elapsed_time(ev1) / args.prefill_steps
    D, KT = lcfg["dim"], lcfg["n_taps"] * lcfg["target_dim"]
    pf_flop = 2.0 * P * D * (KT + 2 * lcfg["layers"] * D)
    pf_tflops = pf_flop / (pf_ms * 1e-3) / 1e12

    step_bytes = draft_step_bytes(cfg, n + 1)
    res = {
        "metric": METRIC, "value": 1e3 / ms, "unit": "draft blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random-init weights, N(0,1) taps)",
        "config": {"workload": "flashmap draft block: fm_draft_block + fm_lm_argmax, dim 2048, 16x128 heads, "
                               "6 layers, MLP 8192, 16 slots, L=513 cached rows, vocab 151936 (bf16)",
                   "graph": graph is not None, "step_hbm_bytes": step_bytes,
                   "step_hbm_gbs": step_bytes / (ms * 1e-3) / 1e9,
                   "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "roofline": {"kernel": "lm_argmax (lm_head GEMM + fused argmax, V=151936 x 2560 bf16, 16 rows)",
                     "bound": "hbm", "achieved": lm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": lm_gbs / HBM_PEAK_GBS, "traffic": traffic, "us_per_launch": lm_us,
                     "algorithmic_bytes_per_launch": lm_bytes},
        "prefill": {"value": P / (pf_ms * 1e-3), "unit": "tokens/s", "rows": P, "ms": pf_ms,
                    "roofline": {"bound": "mfma", "achieved": pf_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": pf_tflops / MFMA_F16_PEAK_TFLOPS, "flop": pf_flop,
                                 "dtype": "f16 operands, f32 accumulate"}},
    }
    if not args.no_cpu:
        print("[bench] oracle on the host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, W, args.cpu_budget)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
