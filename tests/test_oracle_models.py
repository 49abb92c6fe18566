"""Pins of the three drafter oracles: a loop-only second implementation at micro shapes, structural invariants
the pages fix, special cases with closed forms, and the pages' own shape constants."""
import json
import os

import numpy as np
import pytest

from inputs import configs, gen
from oracle import flowmap, kvinject, loops, mtp
from oracle import prims as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))

FM_MICRO = dict(variant="flowmap", dim=16, heads=2, head_dim=8, kv_heads=2, layers=2, ffn=32, block=4, target_dim=12,
                n_taps=2, vocab=20, max_ctx=16, rope="interleaved", rope_dims=8, rope_theta=1e4, ln_eps=1e-6,
                rms_eps=1e-6, qk_eps=1e-5, mlp="gelu_erf", kv_dtype="f16", wtype="bf16", ctx_rows=5, name="fm_micro")
KV_MICRO = dict(variant="kvinject", dim=16, heads=2, head_dim=8, kv_heads=2, layers=2, ffn=24, block=3, target_dim=12,
                n_taps=2, vocab=20, max_ctx=16, rope="none", rope_dims=0, rope_theta=0.0, ln_eps=1e-6, rms_eps=1e-6,
                qk_eps=1e-6, mlp="geglu_tanh", kv_dtype="f32", wtype="bf16", ctx_rows=6, name="kv_micro")
MTP_MICRO = dict(variant="mtp", dim=32, heads=4, head_dim=8, kv_heads=2, layers=1, ffn=64, block=4, target_dim=32,
                 n_taps=2, vocab=20, max_ctx=16, rope="neox", rope_dims=4, rope_theta=1e7, ln_eps=1e-6, rms_eps=1e-6,
                 qk_eps=1e-6, mlp="swiglu", kv_dtype="f32", wtype="q8_0", ctx_rows=16, name="mtp_micro")


def _decoded(cfg, W):
    return {k: P.weight_f64(v) for k, v in W.items()}


def _bump_gates(W, cfg, value=None):
    """A copy of the weights whose modulation gates are all `value` (None: keep)."""
    W = dict(W)
    m = W["mod"].copy().reshape(-1, 3, cfg["dim"])
    if value is not None:
        m[:, 2, :] = value
    W["mod"] = m.reshape(-1)
    return W


# ── flow-map ────────────────────────────────────────────────────────────────────────────────────

def _fm(cfg=FM_MICRO, seed=0):
    W = gen.make_weights(cfg, seed)
    o = flowmap.FlowMapOracle(cfg, W)
    return o, W


def test_flowmap_matches_loop_implementation():
    cfg = FM_MICRO
    o, W = _fm()
    taps = gen.taps(cfg, "micro", cfg["ctx_rows"])
    o.context_append(taps, 0)
    out, _ = o.draft_block(anchor=7, pos=cfg["ctx_rows"])
    tok, z = o.lm_argmax(out)
    ref_out, ref_z = loops.flowmap_forward(cfg, _decoded(cfg, W), taps, 7, cfg["ctx_rows"])
    assert np.allclose(out, ref_out, rtol=1e-11, atol=1e-12)
    assert np.allclose(z, ref_z, rtol=1e-11, atol=1e-12)
    assert list(tok) == [int(np.argmax(r)) for r in ref_z]


def test_flowmap_draft_at_earlier_pos_matches_loops():
    # pos < length: keys are rows [0, pos]; the anchor overwrites row pos
    cfg = FM_MICRO
    o, W = _fm()
    taps = gen.taps(cfg, "micro", cfg["ctx_rows"])
    o.context_append(taps, 0)
    out, _ = o.draft_block(anchor=3, pos=2)
    ref_out, _ = loops.flowmap_forward(cfg, _decoded(cfg, W), taps, 3, 2)
    assert np.allclose(out, ref_out, rtol=1e-11, atol=1e-12)


def test_flowmap_slots_identical_without_rope():
    # Zero noise: every slot starts from the same row; with no positional signal the T slots stay identical.
    cfg = FM_MICRO
    o, _ = _fm()
    o.context_append(gen.taps(cfg, "micro", 5), 0)
    out, xs = o.draft_block(anchor=1, pos=5, rope=False)
    assert np.allclose(out, np.tile(out[:1], (cfg["block"], 1)), atol=1e-13)
    # with RoPE they diverge only through positions: the same position for every slot makes them identical again
    out2, _ = o.draft_block(anchor=1, pos=5, slot_pos=np.full(cfg["block"], 9))
    assert np.allclose(out2, np.tile(out2[:1], (cfg["block"], 1)), atol=1e-13)
    out3, _ = o.draft_block(anchor=1, pos=5)
    assert np.max(np.abs(out3 - out3[:1])) > 1e-6


def test_flowmap_slot_permutation_equivariance():
    # Self-attention is unmasked: permuting the slot positions permutes the outputs.
    cfg = FM_MICRO
    o, _ = _fm()
    o.context_append(gen.taps(cfg, "micro", 5), 0)
    sp = np.array([6, 7, 8, 9])
    perm = np.array([2, 0, 3, 1])
    a, _ = o.draft_block(anchor=4, pos=5, slot_pos=sp)
    b, _ = o.draft_block(anchor=4, pos=5, slot_pos=sp[perm])
    assert np.allclose(b, a[perm], atol=1e-12)


def test_flowmap_zero_gates_reduce_to_head_of_h0():
    # All gates 0: every branch is switched off, the residual stream stays h0, and the output is the head applied to
    # the final modulation of h0 -- independent of context and anchor.
    cfg = FM_MICRO
    W = _bump_gates(gen.make_weights(cfg), cfg, 0.0)
    o = flowmap.FlowMapOracle(cfg, W)
    o.context_append(gen.taps(cfg, "micro", 5), 0)
    out, _ = o.draft_block(anchor=2, pos=5)
    D = cfg["dim"]
    Wd = _decoded(cfg, W)
    E = Wd["lm_head.weight"]
    h0 = P.rmsnorm(E.mean(axis=0)[None], Wd["state_norm.weight"], 1e-6) @ Wd["x_embed.weight"].T + Wd["x_embed.bias"]
    m = Wd["mod"].reshape(-1, 3, D)[-1]
    ref = P.ln_mod(h0, m[0], m[1], 1e-6) @ Wd["head.weight"].T + Wd["head.bias"]
    assert np.allclose(out, np.tile(ref, (cfg["block"], 1)), atol=1e-12)


def test_flowmap_cross_attention_sees_only_rows_up_to_pos():
    cfg = FM_MICRO
    o, W = _fm()
    o.context_append(gen.taps(cfg, "micro", 8), 0)
    a, _ = o.draft_block(anchor=5, pos=4)
    o.K[0][5:8] += 100.0
    o.V[1][6] -= 50.0
    b, _ = o.draft_block(anchor=5, pos=4)
    assert np.array_equal(a, b)


def test_flowmap_append_chunking_and_overwrite():
    cfg = FM_MICRO
    taps = gen.taps(cfg, "chunk", 9)
    o1, W = _fm()
    o1.context_append(taps, 0)
    o2 = flowmap.FlowMapOracle(cfg, W)
    o2.context_append(taps[:4], 0)
    o2.context_append(taps[4:5], 4)
    o2.context_append(taps[5:], 5)
    for l in range(cfg["layers"]):
        assert np.allclose(o1.K[l][:9], o2.K[l][:9], atol=1e-14)
        assert np.allclose(o1.V[l][:9], o2.V[l][:9], atol=1e-14)
    # rewrite from an earlier start (a rewind), then the tail again: the cache equals a fresh append
    o2.context_append(gen.taps(cfg, "other", 3), 2)
    o2.context_append(taps[2:], 2)
    assert o2.length == 9
    for l in range(cfg["layers"]):
        assert np.allclose(o1.K[l][:9], o2.K[l][:9], atol=1e-14)


def test_flowmap_context_full_and_bad_positions():
    cfg = FM_MICRO
    o, _ = _fm()
    with pytest.raises(flowmap.ContextFull):
        o.context_append(gen.taps(cfg, "x", 12), 0)          # 12 + 4 + 1 > 16
    o.context_append(gen.taps(cfg, "x", 3), 0)
    with pytest.raises(ValueError):
        o.context_append(gen.taps(cfg, "x", 1), 5)           # start beyond length
    with pytest.raises(ValueError):
        o.draft_block(anchor=0, pos=4)                         # pos beyond length


def test_flowmap_param_count_matches_page():
    # The page's drafter has 475M parameters (bf16 file of 949,897,866 bytes).  Our flow-map shape replaces the
    # time-conditioning MLPs by a constant table; adding back the per-norm adaLN linears (cond 256 -> 3*dim, 19 norms)
    # and the time / jump embedders (256 -> 256 -> 256, two each) must land within 0.5% of the page's count.
    c = configs.get("flashmap")
    fc = GOLD["flashmap_cfg"]
    assert (c["dim"], c["heads"], c["head_dim"], c["layers"], c["ffn"], c["block"], c["target_dim"], c["n_taps"]) == (
        fc["dim"], fc["heads"], fc["hd"], fc["layers"], fc["ff"], fc["block"], fc["targetDim"], len(fc["taps"]))
    n = sum(int(np.prod(s)) for name, s, k in gen.flowmap_weight_specs(c) if name not in ("mod", "lm_head.weight"))
    cond = fc["cond"]
    n += (3 * c["layers"] + 1) * (cond * 3 * c["dim"] + 3 * c["dim"])
    n += 2 * 2 * (cond * cond + cond)
    assert abs(n - GOLD["flashmap_size"]["params"]) / GOLD["flashmap_size"]["params"] < 0.005
    assert abs(2 * n - GOLD["flashmap_size"]["file_bytes"]) / GOLD["flashmap_size"]["file_bytes"] < 0.005


# ── time conditioning ───────────────────────────────────────────────────────────────────────────

FM_TC = dict(variant="flowmap", dim=8, heads=2, head_dim=4, kv_heads=2, layers=2, ffn=16, block=4, target_dim=8,
             n_taps=2, vocab=12, max_ctx=32, rope="interleaved", rope_dims=4, rope_theta=1e4, ln_eps=1e-6,
             rms_eps=1e-6, qk_eps=1e-5, mlp="gelu_erf", kv_dtype="f16", wtype="bf16", ctx_rows=4, time_dim=8,
             cond_dim=6, time_scale=1000.0, name="fm_tc")


def test_time_conditioning_matches_plain_loops():
    # Brute force of the page's timeConditioning: sinusoid, two-layer time MLPs, SiLU of the sum, one linear per
    # norm, as explicit Python loops over the decoded weights (frequencies and angles rounded to f32 as the page's
    # Math.fround does)
    import math
    cfg = FM_TC
    W = gen.make_weights(cfg)
    o = flowmap.FlowMapOracle(cfg, W)
    dec = {k: P.weight_f64(v) for k, v in W.items()}
    half, cd, D = cfg["time_dim"] // 2, cfg["cond_dim"], cfg["dim"]
    f32 = lambda x: float(np.float32(x))

    def lin(name, x):
        Wm, b = dec[name + ".weight"], dec[name + ".bias"]
        return [b[m] + sum(Wm[m][k] * x[k] for k in range(len(x))) for m in range(Wm.shape[0])]

    silu = lambda v: [u / (1.0 + math.exp(-u)) for u in v]

    def embed(pre, time):
        e = [0.0] * (2 * half)
        for i in range(half):
            fi = f32(math.exp(-math.log(10000.0) * i / half))
            a = f32(f32(time * cfg["time_scale"]) * fi)
            e[i], e[half + i] = math.cos(a), math.sin(a)
        return lin(pre + ".linear_2", silu(lin(pre + ".linear_1", e)))

    for s_, t_ in ((0.0, 1.0), (0.25, 0.75)):
        ts, tj = embed("time_embed", s_), embed("jump_embed", t_)
        cond = silu([ts[i] + tj[i] for i in range(cd)])
        ref = []
        for l in range(cfg["layers"]):
            for n in ("self_attn", "cross_attn", "mlp"):
                ref += lin(f"layers.{l}.{n}_adaln.linear", cond)
        ref += lin("final_adaln.linear", cond)
        assert np.allclose(o.time_conditioning(s_, t_), ref, rtol=1e-12, atol=1e-14)
        assert len(ref) == (3 * cfg["layers"] + 1) * 3 * D


def test_time_conditioning_closed_forms():
    cfg = FM_TC
    W = gen.make_weights(cfg)
    # zero weights everywhere: every linear returns its bias, so the table is the adaLN biases
    Wz = {k: (np.zeros_like(v) if k.endswith(".weight") and ("embed" in k or "adaln" in k) else v) for k, v in W.items()}
    oz = flowmap.FlowMapOracle(cfg, Wz)
    biases = np.concatenate([P.weight_f64(W[f"layers.{l}.{n}_adaln.linear.bias"]) for l in range(cfg["layers"])
                             for n in ("self_attn", "cross_attn", "mlp")] + [P.weight_f64(W["final_adaln.linear.bias"])])
    assert np.array_equal(oz.time_conditioning(0.0, 1.0), biases)
    # at time 0 the sinusoid is [1 .. 1 | 0 .. 0] (cos 0, sin 0), so linear_1 of it is the sum of its first half of
    # columns plus its bias; the jump 0 -> 0 built from that closed form must give the table's final-norm rows
    o = flowmap.FlowMapOracle(cfg, W)
    w1 = P.weight_f64(W["time_embed.linear_1.weight"])
    half = cfg["time_dim"] // 2
    h = w1[:, :half].sum(axis=1) + P.weight_f64(W["time_embed.linear_1.bias"])
    ts = P.weight_f64(W["time_embed.linear_2.weight"]) @ P.silu(h) + P.weight_f64(W["time_embed.linear_2.bias"])
    tab = o.time_conditioning(0.0, 1.0)
    tab00 = o.time_conditioning(0.0, 0.0)
    cond00 = P.silu(ts + (P.weight_f64(W["jump_embed.linear_2.weight"]) @ P.silu(
        P.weight_f64(W["jump_embed.linear_1.weight"])[:, :half].sum(axis=1) + P.weight_f64(W["jump_embed.linear_1.bias"]))
        + P.weight_f64(W["jump_embed.linear_2.bias"])))
    fw, fb = P.weight_f64(W["final_adaln.linear.weight"]), P.weight_f64(W["final_adaln.linear.bias"])
    assert np.allclose(tab00[-3 * cfg["dim"]:], fw @ cond00 + fb, rtol=1e-12, atol=1e-14)
    assert not np.allclose(tab, tab00)


# ── KV-injection ────────────────────────────────────────────────────────────────────────────────

def test_kvinject_matches_loop_implementation():
    cfg = KV_MICRO
    W = gen.make_weights(cfg)
    o = kvinject.KVInjectOracle(cfg, W)
    taps = gen.taps(cfg, "micro", cfg["ctx_rows"])
    o.context_append(taps, 0)
    out, _ = o.draft_block(anchor=11)
    tok, z = o.lm_argmax(out)
    ref_out, ref_z = loops.kvinject_forward(cfg, _decoded(cfg, W), taps, 11)
    assert np.allclose(out, ref_out, rtol=1e-11, atol=1e-12)
    assert np.allclose(z, ref_z, rtol=1e-11, atol=1e-12)


KV_MARKOV = dict(KV_MICRO, markov_rank=4, name="kv_markov")


def _markov_setup(W=None):
    cfg = KV_MARKOV
    W = W if W is not None else gen.make_weights(cfg)
    o = kvinject.KVInjectOracle(cfg, W)
    o.context_append(gen.taps(cfg, "micro", cfg["ctx_rows"]), 0)
    out, _ = o.draft_block(anchor=11)
    return cfg, W, o, out


def test_markov_decode_at_the_page_init_is_the_parallel_argmax():
    # The page initialises w2 and conf.w to zero ("starts as pure parallel DFlash"): the tokens are the plain
    # per-row argmax of the base logits and every confidence is sigmoid(conf.b) (closed form).
    cfg, W, o, _ = _markov_setup()
    W0 = dict(W)
    W0["markov.w2"] = np.zeros_like(W["markov.w2"])
    W0["conf.w"] = np.zeros_like(W["conf.w"])
    cfg, W0, o0, out0 = _markov_setup(W0)
    tok, z = o0.lm_argmax(out0)
    t, sc, conf = o0.markov_decode(o0.block_n, out0, anchor=11)
    assert np.array_equal(t, tok) and np.array_equal(sc, z)
    b = float(P.bf16_to_f64(W["conf.b"])[0])
    assert np.allclose(conf, 1.0 / (1.0 + np.exp(-b)), rtol=1e-15)


def test_markov_decode_matches_plain_loops():
    # Brute force: every score and the confidence dot product as explicit Python loops over the decoded weights.
    cfg, W, o, out = _markov_setup()
    t, sc, conf = o.markov_decode(o.block_n, out, anchor=11)
    E = P.bf16_to_f64(W["lm_head.weight"])
    w1, w2 = P.bf16_to_f64(W["markov.w1"]), P.bf16_to_f64(W["markov.w2"])
    cw, cb = P.bf16_to_f64(W["conf.w"]), P.bf16_to_f64(W["conf.b"])
    V, r, d = cfg["vocab"], cfg["markov_rank"], cfg["dim"]
    prev = 11
    for k in range(cfg["block"]):
        s = []
        for v in range(V):
            zv = sum(out[k][j] * E[v][j] for j in range(cfg["target_dim"]))
            s.append(zv + sum(w1[prev][j] * w2[j][v] for j in range(r)))
        best = max(range(V), key=lambda v: (s[v], -v))
        assert t[k] == best
        assert np.allclose(sc[k], s, rtol=1e-12, atol=1e-14)
        c = cb[0] + sum(o.block_n[k][j] * cw[j][0] for j in range(d)) + sum(w1[prev][j] * cw[d + j][0] for j in range(r))
        assert abs(conf[k] - 1.0 / (1.0 + np.exp(-c))) < 1e-14
        prev = best


def test_markov_decode_identical_rows_remove_the_chain():
    # If every w1 row is the same, the correction no longer depends on the previous token: each row's token is the
    # argmax of its base logits plus one common bias, whatever the other rows chose (and whatever `follow` says).
    cfg, W, o, out = _markov_setup()
    W1 = dict(W)
    W1["markov.w1"] = np.repeat(W["markov.w1"][3:4], cfg["vocab"], axis=0)
    cfg, W1, o1, out1 = _markov_setup(W1)
    t, sc, _ = o1.markov_decode(o1.block_n, out1, anchor=11)
    bias = P.bf16_to_f64(W1["markov.w1"])[0] @ P.bf16_to_f64(W1["markov.w2"])
    _, z = o1.lm_argmax(out1)
    assert np.array_equal(t, np.argmax(z + bias, axis=1))
    t2, sc2, _ = o1.markov_decode(o1.block_n, out1, anchor=11, follow=(t + 1) % cfg["vocab"])
    assert np.array_equal(t2, t) and np.array_equal(sc2, sc)


def test_markov_decode_pruning_cuts_at_the_first_low_confidence():
    # DF forwardRows' pruning only shortens the block: the kept positions are the unpruned decode's first positions,
    # cut at the first k >= 1 whose confidence is below thresholds[k]; position 0 is never cut; thresholds that no
    # sigmoid reaches cut where they stand, thresholds of zero never cut.
    cfg, W, o, out = _markov_setup()
    g = cfg["block"]
    t, sc, conf = o.markov_decode(o.block_n, out, anchor=11)
    assert len(t) == g
    tz, _, _ = o.markov_decode(o.block_n, out, anchor=11, thresholds=[0.0] * g)
    assert np.array_equal(tz, t)
    for j in range(1, g):
        thr = [0.0] * g
        thr[j] = 1.0   # above any sigmoid
        tj, scj, cj = o.markov_decode(o.block_n, out, anchor=11, thresholds=thr)
        assert len(tj) == j and np.array_equal(tj, t[:j]) and np.array_equal(scj, sc[:j]) and np.array_equal(cj, conf[:j])
    t0, _, _ = o.markov_decode(o.block_n, out, anchor=11, thresholds=[1.0] + [0.0] * (g - 1))
    assert len(t0) == g   # a threshold at position 0 is never applied
    for m in sorted(set(conf[1:])):   # a uniform minConf at each confidence value and just above it
        for thrv in (m, np.nextafter(m, 2.0)):
            want = next((k for k in range(1, g) if conf[k] < thrv), g)
            tm, _, _ = o.markov_decode(o.block_n, out, anchor=11, thresholds=[thrv] * g)
            assert len(tm) == want and np.array_equal(tm, t[:want])


def test_kvinject_cached_route_equals_reprojection():
    # The page: the context projection is independent of the block and can be retained.
    cfg = KV_MICRO
    W = gen.make_weights(cfg)
    o = kvinject.KVInjectOracle(cfg, W)
    taps = gen.taps(cfg, "micro", 6)
    o.context_append(taps[:2], 0)
    o.context_append(taps[2:], 2)
    a, _ = o.draft_block(anchor=4)
    b = o.draft_block_reproject(taps, anchor=4)
    assert np.allclose(a, b, atol=1e-13)


def test_kvinject_mask_slot_permutation_equivariance():
    # No positions and no mask: permuting the mask-token slots (1..gamma-1, their block_pos rows with them) permutes
    # those outputs and leaves slot 0 unchanged.
    cfg = KV_MICRO
    W = gen.make_weights(cfg)
    o = kvinject.KVInjectOracle(cfg, W)
    o.context_append(gen.taps(cfg, "micro", 6), 0)
    a, _ = o.draft_block(anchor=4)
    W2 = dict(W)
    W2["mask_emb"] = W["mask_emb"][::-1].copy()
    bp = W["block_pos"].copy()
    bp[1:] = bp[1:][::-1]
    W2["block_pos"] = bp
    o2 = kvinject.KVInjectOracle(cfg, W2)
    o2.context_append(gen.taps(cfg, "micro", 6), 0)
    b, _ = o2.draft_block(anchor=4)
    assert np.allclose(b[0], a[0], atol=1e-13)
    assert np.allclose(b[1:], a[1:][::-1], atol=1e-13)


def test_dflash_defaults_match_page():
    c = configs.get("kvinject")
    d = GOLD["dflash_defaults"]
    assert (c["block"], c["dim"], c["layers"], c["heads"], c["ffn"] // c["dim"], c["n_taps"]) == (
        d["gamma"], d["dDraft"], d["nLayers"], d["nHeads"], d["ffMult"], len(d["tapLayers"]))


# ── MTP ─────────────────────────────────────────────────────────────────────────────────────────

def _mtp(seed=0):
    cfg = MTP_MICRO
    W = gen.make_weights(cfg, seed)
    o = mtp.MTPOracle(cfg, W)
    return cfg, W, o


def test_mtp_matches_loop_implementation():
    cfg, W, o = _mtp()
    pos0, M, kv_lo = 9, 3, 2
    kc, vc = gen.mtp_cache_rows(cfg, pos0)
    o.set_cache_rows(kc, vc)
    e, h = gen.mtp_inputs(cfg, M)
    out = o.forward(e, h, pos0, kv_lo)
    tok, z = o.lm_argmax(out)
    ref_out, ref_z = loops.mtp_forward(cfg, _decoded(cfg, W), e, h, kc, vc, pos0, kv_lo)
    assert np.allclose(out, ref_out, rtol=1e-11, atol=1e-12)
    assert np.allclose(z, ref_z, rtol=1e-11, atol=1e-12)


def test_mtp_rows_at_once_equal_rows_one_by_one():
    # Causal attention over the head's own cache: M rows in one pass equal M single-row passes at consecutive
    # positions (each pass writes its row's K/V before the next reads it).
    cfg, W, o = _mtp()
    pos0, M = 6, 4
    kc, vc = gen.mtp_cache_rows(cfg, pos0)
    o.set_cache_rows(kc, vc)
    e, h = gen.mtp_inputs(cfg, M)
    all_rows = o.forward(e, h, pos0, 0)
    o2 = mtp.MTPOracle(cfg, W)
    o2.set_cache_rows(kc, vc)
    one = np.concatenate([o2.forward(e[m:m + 1], h[m:m + 1], pos0 + m, 0) for m in range(M)])
    assert np.allclose(all_rows, one, atol=1e-13)


def test_mtp_kv_lo_hides_earlier_rows():
    cfg, W, o = _mtp()
    kc, vc = gen.mtp_cache_rows(cfg, 8)
    o.set_cache_rows(kc, vc)
    e, h = gen.mtp_inputs(cfg, 2)
    a = o.forward(e, h, 8, 3)
    kc2 = kc.copy(); kc2[:3] += 10.0
    o.set_cache_rows(kc2, vc)
    b = o.forward(e, h, 8, 3)
    assert np.array_equal(a, b)
    c = o.forward(e, h, 8, 0)
    assert np.max(np.abs(c - a)) > 1e-6


def test_mtp_embed_row_is_scale_times_code():
    # Q8_0: every element of a table row is its block's f16 scale times its int8 code (closed form, element by
    # element, without the oracle's vectorised decode)
    cfg, W, o = _mtp()
    codes, scales = W["lm_head"]
    for tok in (0, 7, cfg["vocab"] - 1):
        row = o.embed_row(tok)
        for k in range(cfg["dim"]):
            d = float(np.frombuffer(np.uint16(scales[tok, k // 32]).tobytes(), dtype=np.float16)[0])
            assert row[k] == d * int(codes[tok, k])


def test_mtp_chain_equals_one_pass_over_the_chained_rows():
    # Chained depth: step i runs at pos + i on (E[token i-1], h'_(i-1)). By causality and the cache rows each step
    # writes, one M = steps pass over those same inputs gives the same rows, so the chain's plumbing (positions,
    # which h and which token feed the next step, the cache rows it leaves) is pinned by the batched forward.
    cfg, W, o = _mtp()
    pos, steps, kv_lo = 7, 3, 1
    kc, vc = gen.mtp_cache_rows(cfg, pos)
    o.set_cache_rows(kc, vc)
    _, h = gen.mtp_inputs(cfg, 1)
    toks, hs, zs = o.chain(5, h[0], steps, pos, kv_lo)
    assert toks.shape == (steps,) and hs.shape == (steps, cfg["dim"]) and zs.shape == (steps, cfg["vocab"])
    assert np.array_equal(toks, np.argmax(zs, axis=1))
    chain_K = o.Kc[pos:pos + steps].copy()
    o2 = mtp.MTPOracle(cfg, W)
    o2.set_cache_rows(kc, vc)
    e_in = np.stack([o2.embed_row(t) for t in [5, *toks[:-1]]])
    h_in = np.concatenate([h[:1], hs[:-1]])
    batch = o2.forward(e_in, h_in, pos, kv_lo)
    assert np.allclose(batch, hs, atol=1e-12)
    assert np.allclose(o2.Kc[pos:pos + steps], chain_K, atol=1e-12)
    # follow: chaining other tokens changes every later step, and re-chaining its own tokens changes nothing
    o3 = mtp.MTPOracle(cfg, W)
    o3.set_cache_rows(kc, vc)
    t3, h3, _ = o3.chain(5, h[0], steps, pos, kv_lo, follow=toks)
    assert np.array_equal(t3, toks) and np.array_equal(h3, hs)
    o4 = mtp.MTPOracle(cfg, W)
    o4.set_cache_rows(kc, vc)
    other = (toks + 1) % cfg["vocab"]
    _, h4, _ = o4.chain(5, h[0], steps, pos, kv_lo, follow=other)
    assert np.array_equal(h4[0], hs[0]) and np.max(np.abs(h4[1] - hs[1])) > 1e-6


def test_mtp_shapes_match_page_tensor_map():
    # The page's tensor map gives [offset, type, ne0 = K, ne1 = N]; a Q8_0 tensor occupies N * K/32 * 34 bytes, and
    # consecutive offsets must agree with those sizes for our [N][K] shapes.
    c = configs.get("mtp")
    mc = GOLD["mcfg"]
    assert (c["dim"], c["ffn"], c["heads"], c["kv_heads"], c["head_dim"], c["rope_dims"], c["rope_theta"],
            c["vocab"], c["block"]) == (mc["H"], mc["I"], mc["NH"], mc["NKV"], mc["HD"], mc["ROT"], mc["THETA"],
                                          mc["VOCAB"], mc["MAXM"])
    t = GOLD["mtp_tensors"]["tensors"]
    ours = {name: shape for name, shape, kind in gen.mtp_weight_specs(c)}
    items = sorted(t.items(), key=lambda kv: kv[1][0])
    end = GOLD["mtp_tensors"]["head_block"][0] + GOLD["mtp_tensors"]["head_block"][1]
    for i, (name, (off, typ, ne0, ne1)) in enumerate(items):
        if name == "output_norm" or off < GOLD["mtp_tensors"]["head_block"][0]:
            continue
        nxt = items[i + 1][1][0] if i + 1 < len(items) else end
        if typ == 8:
            assert ours[name] == (ne1, ne0)
            assert nxt - off == ne1 * ne0 // 32 * 34
        else:
            assert ours[name] == (ne0,)
            assert nxt - off == ne0 * 4
