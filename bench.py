"""Benchmark of the MI355X block drafter forward on one GPU.

Workload (FlashMap-shaped flow-map drafter: dim 2048, 16 heads x 128, 6 DiT layers, MLP 8192, 5 taps x 2560,
vocab 151936, random-init bf16 weights, synthetic f32 taps):
  * the timed step is one 16-slot draft block -- fm_draft_block + fm_lm_argmax (anchor slot, 6 DiT layers, head,
    lm_head GEMM fused with the per-slot argmax) -- at position 512 after a 512-row context prefill (L = 513);
  * the same drafter's context prefill of 8192 rows (fm_context_append: fc 12800 -> 2048 on the matrix cores,
    RMSNorm, 12 K/V projections with head-norm + RoPE + f16 cache stores) is timed as a second line item.

Prints one JSON line: draft blocks/s (value); the skinny weight-streaming GEMM (K1, the step's largest kernel time)
and the lm_head+argmax kernel against the HBM roofline, both timed live with HIP events on the stream they run on;
the prefill against the bf16/f16 MFMA roofline; and the float64 oracle timed on the host cores on a bounded sample
of the same draft step.
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
    reads. Create-time work is not part of the step: fc, hidden_norm, state_norm, x_embed, and layer 0 from the
    zero-noise slot row up to the cross-attention's q (q / k / v, o_proj and the cross q_proj: the same for every
    draft, computed at create; its few small norm and modulation rows, ~41 KB, stay counted)."""
    D, Ht, F, hd, Lyr, V = cfg["dim"], cfg["target_dim"], cfg["ffn"], cfg["head_dim"], cfg["layers"], cfg["vocab"]
    w = D * Ht + 2 * D + Ht                       # anchor_proj (+bias), anchor_norm, E[anchor]
    w += Lyr * (8 * D * D + 4 * hd + 2 * F * D + F + D) - 5 * D * D
    w += Ht * D + Ht + V * Ht                     # head (+bias), lm_head
    b = 2 * w + 4 * (3 * Lyr + 1) * 3 * D         # bf16 weights, f32 modulation table
    return b + 2 * Lyr * L * D * 2


def skinny_step_bytes(cfg) -> int:
    """Algorithmic HBM bytes of the skinny GEMM launches (K1) of one flow-map draft: each launch's bf16 weights and
    biases once, its activation rows once (hi/lo bf16 pairs: 4 bytes an element) and its result once, plus what its
    fused epilogue moves. The launches: anchor_proj (1 row); the 12 cross K / V projections of the anchor row (one
    launch); layer 0 from its cross o_proj (cross o_proj, fc1, fc2); every further layer's q | k | v, self o_proj,
    cross q_proj, cross o_proj, fc1, fc2 (16 rows); the head.
      * residual update (o_proj, cross o_proj, fc2): reads the residual rows x (layer 0's cross o_proj one broadcast
        row), the gate and the next modulation's scale row; writes x, the next product's fragments and x's
        (mean, M2) per 16-column tile;
      * LayerNorm fold (q | k | v, cross q_proj, fc1, head): reads those tile statistics and each matrix's c1 / c2;
      * self-attention in the q | k | v launch: reads the head-norm weights and the slots' RoPE rows, writes o as
        fragments (q, k, v themselves are its f32 result, counted once)."""
    D, Ht, F, Lyr, T, hd = cfg["dim"], cfg["target_dim"], cfg["ffn"], cfg["layers"], cfg["block"], cfg["head_dim"]

    def g(M, K, rows, bias=0, groups=1):   # one launch: `groups` M x K matrices over the same rows
        return groups * (2 * M * K + 2 * bias + 4 * rows * M) + 4 * rows * K

    def resid(M, rows, base_rows):         # x read (base rows) and written, gate + scale rows, tile statistics
        return 4 * base_rows * M + 4 * rows * M + 8 * M + 8 * rows * (M // 16)

    def ln(K, rows, M, groups=1):          # the statistics of the input rows, c1 / c2 of each matrix
        return 8 * rows * (K // 16) + groups * 8 * M

    sa = 2 * 2 * hd + 4 * T * hd + 4 * T * D   # q / k norm weights, RoPE rows, o fragments
    b = g(D, Ht, 1) + g(D, D, 1, groups=2 * Lyr)
    mlp = g(F, D, T, bias=F) + ln(D, T, F) + g(D, F, T, bias=D) + resid(D, T, T)
    b += g(D, D, T) + resid(D, T, 1) + mlp                                   # layer 0
    b += (Lyr - 1) * (g(D, D, T, groups=3) + ln(D, T, D, 3) + sa           # q | k | v + self-attention
                      + g(D, D, T) + resid(D, T, T)                         # o_proj
                      + g(D, D, T) + ln(D, T, D)                            # cross q_proj
                      + g(D, D, T) + resid(D, T, T) + mlp)                  # cross o_proj, MLP
    b += g(Ht, D, T, bias=Ht) + ln(D, T, Ht)
    return b


def weight_bytes(W, names) -> int:
    """Bytes of the named tensors in their storage format (a Q8_0 tensor is its codes plus its f16 scales)."""
    tot = 0
    for n in names:
        v = W[n]
        tot += sum(x.nbytes for x in v) if isinstance(v, tuple) else v.nbytes
    return tot


def _graph_of(torch, fn):
    """fn captured into a HIP graph after one eager run on a side stream; plain fn if capture fails."""
    try:
        cur = torch.cuda.current_stream()
        s = torch.cuda.Stream()
        s.wait_stream(cur)
        with torch.cuda.stream(s):
            fn()
        cur.wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g.replay
    except Exception as e:
        print(f"[bench] graph capture failed ({e}); plain launches", file=sys.stderr, flush=True)
        return fn


def _time_ms(torch, run, warmup: int, reps: int) -> float:
    """Mean ms of run() over reps calls after warmup calls, HIP events on torch's current stream (the stream the
    library launches on)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _hbm_row(what, ms, nbytes, unit="per s"):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"what": what, "value": 1e3 / ms, "unit": unit, "us": ms * 1e3, "algorithmic_bytes": nbytes,
            "achieved_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}


def _mfma_row(what, ms, rows, flop):
    tf = flop / (ms * 1e-3) / 1e12
    return {"what": what, "value": rows / (ms * 1e-3), "unit": "tokens/s", "ms": ms, "flop": flop,
            "achieved_tflops": tf, "mfma_frac": tf / MFMA_F16_PEAK_TFLOPS}


def other_rows(torch, fm, configs, gen, W, d, dl, reps: int):
    """The remaining measured rows of the hot-path table: long-context draft and 16-row append, the 512-row
    prefill, the KV-injection draft and prefill, and the MTP pass at M = 1, 2, 4, 8."""
    rows = {}
    cfg, lcfg = configs.get("flashmap"), configs.get("longctx")
    D, Ht, T, Lyr = cfg["dim"], cfg["target_dim"], cfg["block"], cfg["layers"]
    hid = torch.empty(T, Ht, dtype=torch.float32, device="cuda")
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    an = torch.tensor([int(gen.anchors(cfg, "bench", 1)[0])], dtype=torch.int32, device="cuda")

    # long context: draft at pos = 8192 (L = 8193) after the 8192-row prefill, then 16-row appends at 8192
    P = lcfg["ctx_rows"]

    def lstep():
        dl.fm_draft_block(hid, anchor=an, pos=P)
        dl.fm_lm_argmax(hid, T, tok)
    ms = _time_ms(torch, _graph_of(torch, lstep), 5, reps)
    rows["longctx_draft_L8193"] = _hbm_row("flow-map draft block + lm_head argmax at L = 8193", ms,
                                           draft_step_bytes(lcfg, P + 1), "draft blocks/s")
    t16 = torch.from_numpy(gen.taps(lcfg, "bench-append", 16)).cuda()
    ms = _time_ms(torch, lambda: dl.fm_context_append(t16, P), 5, reps)
    app_w = ["fc.weight", "hidden_norm.weight"] + [f"layers.{l}.cross_attn.{m}" for l in range(Lyr)
                                                    for m in ("k_proj.weight", "v_proj.weight", "k_norm.weight")]
    rows["longctx_append_16"] = _hbm_row("16-row context append (fc, RMSNorm, 12 K/V projections, f16 cache)", ms,
                                         weight_bytes(W, app_w) + t16.numel() * 4 + 2 * Lyr * 16 * D * 2,
                                         "appends/s")
    dl.fm_context_append(t16, P)   # leave the context at 8192 + 16 rows

    # the long-context workload's own schedule after its 8192-row prefill: 64 steps, each a draft block + lm_head
    # argmax at pos_s, then an append of U{1..16} rows at pos_s (the first rewinds the 16 rows above). Every call's
    # arguments are fixed by the schedule, so the 64 steps replay as one graph; a replay rewrites the same rows.
    sched = gen.longctx_schedule(lcfg)
    s_an = torch.tensor([a for a, _, _ in sched], dtype=torch.int32, device="cuda")
    s_taps = [torch.from_numpy(gen.taps(lcfg, f"step{i}", ns)).cuda() for i, (_, _, ns) in enumerate(sched)]

    def sched_run():
        for i, (_, pos, ns) in enumerate(sched):
            dl.fm_draft_block(hid, anchor=s_an[i:i + 1], pos=pos)
            dl.fm_lm_argmax(hid, T, tok)
            dl.fm_context_append(s_taps[i], pos)
    ms = _time_ms(torch, _graph_of(torch, sched_run), 1, 3)
    s_bytes = sum(draft_step_bytes(lcfg, pos + 1) + weight_bytes(W, app_w) + ns * lcfg["n_taps"] * Ht * 4 +
                  2 * Lyr * ns * D * 2 for _, pos, ns in sched)
    r = _hbm_row(f"the long-context schedule: {len(sched)} x (draft block + lm_head argmax at L = {sched[0][1] + 1} .. "
                 f"{sched[-1][1] + 1}, then an append of 1-16 rows)", ms, s_bytes, "schedules/s")
    r["draft_blocks_per_s"] = len(sched) / (ms * 1e-3)
    r["us_per_step"] = ms * 1e3 / len(sched)
    rows["longctx_schedule_64"] = r

    # two FlowMap requests in one pass (fm_draft_batch, 32 rows): each over its own 512-row context, the lm_head
    # argmax over both blocks' rows; the weights and the table stream once for both
    n = cfg["ctx_rows"]
    d2 = fm.Drafter(cfg, d.weights)
    d2.fm_context_append(torch.from_numpy(gen.taps(cfg, "bench-b2", n)).cuda(), 0)
    an2 = torch.tensor([int(gen.anchors(cfg, "bench-b2", 1)[0])], dtype=torch.int32, device="cuda")
    hid2 = torch.empty(2 * T, Ht, dtype=torch.float32, device="cuda")
    tok2 = torch.empty(2 * T, dtype=torch.int32, device="cuda")

    def b2step():
        fm.Drafter.fm_draft_batch([d, d2], [{"anchor": an, "pos": n}, {"anchor": an2, "pos": n}], hid2)
        d.fm_lm_argmax(hid2, 2 * T, tok2)
    ms = _time_ms(torch, _graph_of(torch, b2step), 5, reps)
    row = _hbm_row("two flow-map requests in one pass (fm_draft_batch B = 2, 32 rows, each over its own 512-row "
                   "context) + lm_head argmax over the 32 rows", ms,
                   draft_step_bytes(cfg, n + 1) + 2 * Lyr * (n + 1) * D * 2, "draft blocks/s")
    row["value"] *= 2   # two blocks per pass
    rows["flashmap_batch2"] = row
    del d2

    # the same draft step on the persistent schedule (every phase of the draft in one launch; the automatic schedule
    # is one launch per phase, the faster of the two)
    if d.draft_path == "launches":
        try:
            d.set_draft_path("persistent")
        except fm.FmError:
            pass
    if d.draft_path == "persistent":
        def pstep():
            d.fm_draft_block(hid, anchor=an, pos=n)
            d.fm_lm_argmax(hid, T, tok)
        ms = _time_ms(torch, _graph_of(torch, pstep), 5, reps)
        d.device_status()
        rows["flashmap_draft_persistent"] = _hbm_row("FlashMap draft block + lm_head argmax, the draft as one persistent "
                                                     "launch (fm_set_draft_path 2)", ms, draft_step_bytes(cfg, n + 1),
                                                     "draft blocks/s")
        d.set_draft_path("auto")

    # 512-row prefill on the FlashMap shape
    tp = torch.from_numpy(gen.taps(cfg, "prefill", n)).cuda()
    ms = _time_ms(torch, lambda: d.fm_context_append(tp, 0), 2, 10)
    rows["flashmap_prefill_512"] = _mfma_row("512-row context prefill", ms, n,
                                             2.0 * n * D * (cfg["n_taps"] * Ht + 2 * Lyr * D))

    # time conditioning of the jump 0 -> 1 at the FlashMap shape (time / condition widths 256, scale 1000): the time
    # MLPs and 19 adaLN linears, written into a copy of the modulation table (the other rows keep theirs)
    ct = configs.get("flashmap", time_dim=256, cond_dim=256, time_scale=1000.0)
    tnames = [(nm, sh, k) for nm, sh, k in gen.weight_specs(ct) if "time_embed" in nm or "jump_embed" in nm or "adaln" in nm]
    Wt = {nm: gen.make_tensor(ct, nm, sh, k) for nm, sh, k in tnames}
    dwt = dict(d.weights)
    dwt.update(fm.upload_weights(Wt))
    dwt["mod"] = d.weights["mod"].clone()
    dt = fm.Drafter(ct, dwt)
    ms = _time_ms(torch, _graph_of(torch, lambda: dt.fm_time_condition(0.0, 1.0, 256, 256, 1000.0)), 5, reps)
    rows["flashmap_time_condition"] = _hbm_row("time conditioning of a jump (time MLPs + 19 adaLN linears -> the "
                                               "modulation table)", ms,
                                               weight_bytes(Wt, [nm for nm, _, _ in tnames]) + dwt["mod"].numel() * 4,
                                               "tables/s")
    del dt, dwt

    # KV-injection: 2048-row prefill, then the gamma = 5 draft + lm_head argmax
    kc = configs.get("kvinject")
    print("[bench] KV-injection weights", file=sys.stderr, flush=True)
    Wk = gen.make_weights(kc)
    dwk = fm.upload_weights(Wk)
    dk = fm.Drafter(kc, dwk)
    nk, Dk, Htk, g = kc["ctx_rows"], kc["dim"], kc["target_dim"], kc["block"]
    tk = torch.from_numpy(gen.taps(kc, "prefill", nk)).cuda()
    ms = _time_ms(torch, lambda: dk.fm_context_append(tk, 0), 2, 10)
    rows["kvinject_prefill_2048"] = _mfma_row("2048-row context prefill (KV-injection)", ms, nk,
                                              2.0 * nk * Dk * (kc["n_taps"] * Htk + 2 * kc["layers"] * Dk))
    hk = torch.empty(g, Htk, dtype=torch.float32, device="cuda")
    tkk = torch.empty(g, dtype=torch.int32, device="cuda")
    ak = torch.tensor([int(gen.anchors(kc, "bench", 1)[0])], dtype=torch.int32, device="cuda")

    def kstep():
        dk.fm_draft_block(hk, anchor=ak)
        dk.fm_lm_argmax(hk, g, tkk)
    ms = _time_ms(torch, _graph_of(torch, kstep), 5, reps)
    kw = [nm for nm, _, _ in gen.kvinject_weight_specs(kc)
          if nm not in ("W_c", "ctx_norm") and not nm.startswith(("markov.", "conf."))]
    kbytes = weight_bytes(Wk, kw) + 2 * kc["layers"] * nk * Dk * 4
    rows["kvinject_draft"] = _hbm_row("KV-injection draft (gamma 5) + lm_head argmax", ms, kbytes, "draft blocks/s")
    # the same draft decoded with the DSpark Markov correction and confidence head (fm_markov_argmax): the base
    # logits once (written and read back), then per row the rank x V correction table and the w1 row
    rk, Vk = kc["markov_rank"], kc["vocab"]
    cfk = torch.empty(g, dtype=torch.float32, device="cuda")

    def mkstep():
        dk.fm_draft_block(hk, anchor=ak)
        dk.fm_markov_argmax(hk, g, ak, rk, tkk, cfk)
    ms = _time_ms(torch, _graph_of(torch, mkstep), 5, reps)
    rows["kvinject_draft_markov"] = _hbm_row("KV-injection draft + Markov-corrected greedy decode and confidence "
                                             "(gamma 5, rank 256)", ms,
                                             kbytes + g * (rk * Vk * 2 + 2 * Vk * 4 + rk * 2), "draft blocks/s")
    # the same with confidence pruning that ends the block at position 2 (thresholds 0, 0, 1, 0, 0): the decode
    # steps of the dropped positions do no work
    thr = [0.0, 0.0, 1.0] + [0.0] * (g - 3)
    lenk = torch.zeros(1, dtype=torch.int32, device="cuda")

    def mpstep():
        dk.fm_draft_block(hk, anchor=ak)
        dk.fm_markov_argmax(hk, g, ak, rk, tkk, cfk, thresholds=thr, length=lenk)
    ms = _time_ms(torch, _graph_of(torch, mpstep), 5, reps)
    rows["kvinject_draft_markov_pruned_at_2"] = _hbm_row(
        "KV-injection draft + Markov decode with confidence pruning that keeps 2 of 5 positions (the other steps "
        "skip the correction table)", ms, kbytes + 2 * (rk * Vk * 2 + 2 * Vk * 4 + rk * 2), "draft blocks/s")
    # three requests with their own 2048-row contexts drafted in one pass (fm_draft_batch) + the lm_head over the 15
    # rows: the weights stream once for all three blocks
    Bq = 3
    dks = [dk] + [fm.Drafter(kc, dwk) for _ in range(Bq - 1)]
    for b in range(1, Bq):
        dks[b].fm_context_append(torch.from_numpy(gen.taps(kc, f"prefill-{b}", nk)).cuda(), 0)
    akb = torch.tensor([int(a) for a in gen.anchors(kc, "bench-batch", Bq)], dtype=torch.int32, device="cuda")
    hkb = torch.empty(Bq * g, Htk, dtype=torch.float32, device="cuda")
    tkb = torch.empty(Bq * g, dtype=torch.int32, device="cuda")

    def bstep():
        fm.Drafter.fm_draft_batch(dks, [{"anchor": akb[b:b + 1]} for b in range(Bq)], hkb)
        dk.fm_lm_argmax(hkb, Bq * g, tkb)
    ms = _time_ms(torch, _graph_of(torch, bstep), 5, reps)
    r = _hbm_row(f"{Bq} KV-injection requests (own 2048-row contexts) drafted in one pass + lm_head argmax over "
                 f"{Bq * g} rows", ms, kbytes + (Bq - 1) * 2 * kc["layers"] * nk * Dk * 4, "draft blocks/s")
    r["value"] = Bq * 1e3 / ms   # blocks per second: Bq blocks per pass
    rows["kvinject_batch3"] = r
    del dk, dks, Wk, dwk

    # MTP head: M rows at pos0 = 4096 - M over the 4096-row cache, + the Q8_0 lm_head argmax
    mc = configs.get("mtp")
    print("[bench] MTP weights", file=sys.stderr, flush=True)
    Wm = gen.make_weights(mc)
    dwm = fm.upload_weights(Wm)
    dm = fm.Drafter(mc, dwm)
    H, NKV, HD = mc["dim"], mc["kv_heads"], mc["head_dim"]
    dm.kv_layer(0, 0).normal_()
    dm.kv_layer(0, 1).normal_()
    mw = weight_bytes(Wm, [nm for nm, _, _ in gen.mtp_weight_specs(mc)])
    for M in (1, 2, 4, 8):
        pos0 = mc["max_ctx"] - M
        e, h = gen.mtp_inputs(mc, M)
        e, h = torch.from_numpy(e).cuda(), torch.from_numpy(h).cuda()
        hm = torch.empty(M, H, dtype=torch.float32, device="cuda")
        tm = torch.empty(M, dtype=torch.int32, device="cuda")

        def mstep():
            dm.fm_draft_block(hm, pos=pos0, rows=M, embed_rows=e, prev_hidden=h)
            dm.fm_lm_argmax(hm, M, tm)
        ms = _time_ms(torch, _graph_of(torch, mstep), 5, reps)
        rows[f"mtp_pass_M{M}"] = _hbm_row(f"MTP pass, M = {M} rows + Q8_0 lm_head argmax", ms,
                                          mw + 2 * (pos0 + M) * NKV * HD * 4, "passes/s")
    # four sequences' 2-row passes in one batched pass (fm_draft_batch) + the lm_head over the 8 rows
    Bm, Mb = 4, 2
    dms = [dm] + [fm.Drafter(mc, dwm) for _ in range(Bm - 1)]
    for b in range(1, Bm):
        dms[b].kv_layer(0, 0).normal_()
        dms[b].kv_layer(0, 1).normal_()
    eb, hb = gen.mtp_inputs(mc, Bm * Mb)
    eb, hb = torch.from_numpy(eb).cuda(), torch.from_numpy(hb).cuda()
    posb = mc["max_ctx"] - Mb
    reqs = [dict(rows=Mb, pos=posb, kv_lo=0, embed_rows=eb[b * Mb:(b + 1) * Mb], prev_hidden=hb[b * Mb:(b + 1) * Mb])
            for b in range(Bm)]
    hbm = torch.empty(Bm * Mb, H, dtype=torch.float32, device="cuda")
    tbm = torch.empty(Bm * Mb, dtype=torch.int32, device="cuda")

    def bmstep():
        fm.Drafter.fm_draft_batch(dms, reqs, hbm)
        dm.fm_lm_argmax(hbm, Bm * Mb, tbm)
    ms = _time_ms(torch, _graph_of(torch, bmstep), 5, reps)
    r = _hbm_row(f"{Bm} MTP sequences x {Mb} rows in one pass + Q8_0 lm_head argmax over {Bm * Mb} rows", ms,
                 mw + Bm * 2 * (posb + Mb) * NKV * HD * 4, "passes/s")
    r["value"] = Bm * 1e3 / ms   # sequences' passes per second
    rows["mtp_batch4_M2"] = r
    del dms
    # chained depth: 3 single-row passes, each on the previous draft's table row and h' (fm_mtp_chain)
    steps = 3
    posc = mc["max_ctx"] - steps
    _, h1 = gen.mtp_inputs(mc, 1)
    h1 = torch.from_numpy(h1[0].copy()).cuda()
    tc = torch.tensor([7] + [0] * steps, dtype=torch.int32, device="cuda")
    hc = torch.empty(steps, H, dtype=torch.float32, device="cuda")

    def cstep():
        dm.fm_mtp_chain(tc, h1, steps, posc, 0, hc)
    ms = _time_ms(torch, _graph_of(torch, cstep), 5, reps)
    cbytes = sum(mw + 2 * (posc + i + 1) * NKV * HD * 4 for i in range(steps))
    rows["mtp_chain_3"] = _hbm_row("MTP chained depth: 3 single-row passes (table row gather + pass + Q8_0 lm_head "
                                   "argmax each)", ms, cbytes, "chains/s")
    del dm, Wm, dwm
    return rows


def cpu_baseline(cfg, W):
    """The oracle (float64 NumPy) on the host cores, timed as a fixed protocol: one warm-up, then the median of 3
    timed runs, of (a) the draft block -- fm_draft_block + fm_lm_argmax at the same position as the GPU step -- and
    (b) the 512-row context prefill (fm_context_append)."""
    import statistics
    from inputs import gen
    from oracle import flowmap
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    o = flowmap.FlowMapOracle(cfg, W)
    n = cfg["ctx_rows"]
    taps = gen.taps(cfg, "prefill", n)
    an = int(gen.anchors(cfg, "bench", 1)[0])

    def timed(fn):
        fn()   # warm-up (the first call also decodes the weights to float64)
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    pf_s = timed(lambda: o.context_append(taps, 0))

    def draft():
        out, _ = o.draft_block(an, n)
        o.lm_argmax(out)
    dr_s = timed(draft)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": 1.0 / dr_s, "unit": "draft blocks/s", "cores": cores, "kind": "oracle",
            "prefill_tokens_per_s": n / pf_s, "cpu": cpu,
            "sample": f"median of 3 timed runs after 1 warm-up: the draft block (fm_draft_block + fm_lm_argmax, "
                      f"{dr_s * 1e3:.0f} ms) and the {n}-row context prefill ({pf_s * 1e3:.0f} ms) of the "
                      f"512-row-context FlashMap workload, float64 NumPy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--prefill-warmup", type=int, default=10)
    ap.add_argument("--graph", choices=["on", "off"], default="on")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline, lm_head and 8192-row prefill only")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for a rocprofv3 --pmc pass: set up, run fm_lm_argmax 5 times on the FlashMap and 5 times on "
                         "the MTP head's Q8_0 table, 3 FlashMap draft steps, one 8192-row context prefill, and one "
                         "elementwise kernel that reads 1 GiB and writes 1 GiB (the counters' scale reference), then "
                         "exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
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
        # the MTP head's Q8_0 lm_head (248320 x 5120), 8 rows
        mc = configs.get("mtp")
        dm = fm.Drafter(mc, fm.upload_weights(gen.make_weights(mc)))
        _, hm = gen.mtp_inputs(mc, 8)
        hm = torch.from_numpy(hm).cuda()
        tm = torch.empty(8, dtype=torch.int32, device="cuda")
        for _ in range(5):
            dm.fm_lm_argmax(hm, 8, tm)
        # three draft steps (the skinny GEMM launches) and one 8192-row context prefill (the MFMA GEMMs)
        for _ in range(3):
            step()
        dlp = fm.Drafter(lcfg, dw)
        dlp.fm_context_append(torch.from_numpy(gen.taps(lcfg, "prefill", lcfg["ctx_rows"])).cuda(), 0)
        torch.cuda.synchronize()
        del dlp
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        src.fill_(1.0)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)   # one elementwise kernel: 1 GiB read, 1 GiB written
        torch.cuda.synchronize()
        print("[bench] pmc probe done: 5 x fm_lm_argmax (bf16), 5 x fm_lm_argmax (Q8_0), 3 draft steps, one 8192-row "
              "prefill, one 1 GiB elementwise pass", file=sys.stderr, flush=True)
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

    # dominant kernel by step time: the skinny weight-streaming GEMM (K1); a draft's K1 launches replayed alone,
    # back to back, between HIP events on the stream they run on (fm_profile_draft, 8 passes); median of 5 calls
    prof = sorted((d.profile_draft(hidden, anchor, n, 8) for _ in range(5)), key=lambda r: r[0])
    k1_us, k1_n, k1_draft_us = prof[len(prof) // 2]
    k1_bytes = skinny_step_bytes(cfg)
    k1_gbs = k1_bytes / (k1_us * 1e-6) / 1e9
    k1_traffic = traffic_record("k_skinny.hip", "skinny_flashmap_traffic.json")

    # second kernel: the lm_head GEMM fused with the argmax, timed alone with events on its stream
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
    for _ in range(args.prefill_warmup):   # untimed, as the draft step's warm-up: the clocks settle under the load
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
        "roofline": {"kernel": f"skinny_kernel (K1: the draft's {k1_n} weight-streaming GEMM launches, bf16 "
                               "weights, 1 or 16 activation rows)",
                     "bound": "hbm", "achieved": k1_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": k1_gbs / HBM_PEAK_GBS, "traffic": k1_traffic, "launches_per_step": k1_n,
                     "us_per_step": k1_us, "us_per_launch": k1_us / k1_n,
                     "algorithmic_bytes_per_step": k1_bytes, "algorithmic_bytes_per_launch": k1_bytes / k1_n,
                     "draft_us_profiled": k1_draft_us},
        "roofline_lm_head": {"kernel": "lm_argmax (lm_head GEMM + fused argmax, V=151936 x 2560 bf16, 16 rows)",
                             "bound": "hbm", "achieved": lm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": lm_gbs / HBM_PEAK_GBS, "traffic": traffic, "us_per_launch": lm_us,
                             "algorithmic_bytes_per_launch": lm_bytes},
        "prefill": {"value": P / (pf_ms * 1e-3), "unit": "tokens/s", "rows": P, "ms": pf_ms,
                    "steps": args.prefill_steps, "warmup": args.prefill_warmup,
                    "roofline": {"bound": "mfma", "achieved": pf_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": pf_tflops / MFMA_F16_PEAK_TFLOPS, "flop": pf_flop,
                                 "dtype": "f16 operands, f32 accumulate"}},
    }
    if not args.quick:
        print("[bench] remaining workloads", file=sys.stderr, flush=True)
        res["rows"] = other_rows(torch, fm, configs, gen, W, d, dl, max(20, args.steps // 4))
    if not args.no_cpu:
        print("[bench] oracle on the host cores", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, W)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
