"""Degenerate cases on the GPU, against the float64 oracle: exact ties in the lm_head argmax (the lowest index wins),
drafts at the last position the cache allows, and an empty append."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import flowmap, kvinject, mtp
from tests.parity import assert_rows_close, assert_tokens_match

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MTP_SMALL = dict(variant="mtp", dim=512, heads=4, head_dim=256, kv_heads=2, layers=1, ffn=1024, block=8,
                 target_dim=512, n_taps=2, vocab=4096, max_ctx=300, rope="neox", rope_dims=64, rope_theta=1e7,
                 ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="swiglu", kv_dtype="f32", wtype="q8_0", ctx_rows=300,
                 name="mtp_small")
KV_SMALL = dict(variant="kvinject", dim=256, heads=2, head_dim=128, kv_heads=2, layers=2, ffn=512, block=5,
                target_dim=512, n_taps=2, vocab=4096, max_ctx=160, rope="none", rope_dims=0, rope_theta=0.0,
                ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="geglu_tanh", kv_dtype="f32", wtype="bf16", ctx_rows=100,
                name="kvinject_small")


def _say(msg):
    print(f"[gpu-edges] {msg}", flush=True)
    sys.stdout.flush()


def _fm():
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return fm


def _tie_sets(V: int, rows: int):
    """Groups of vocabulary rows made identical: neighbours inside a 16-row tile, across a tile boundary, across
    a 64-row boundary, at the end of the table, far apart, a four-way group; then random pairs."""
    fixed = [[0, 1], [15, 16], [63, 64, 65], [V - 2, V - 1], [5, V - 3], [1000, 1001, V // 3, V - 900]]
    used = {v for s in fixed for v in s}
    rng = np.random.default_rng(11)
    sets = fixed[:rows]
    while len(sets) < rows:
        a, b = sorted(int(x) for x in rng.choice(V, 2, replace=False))
        if a not in used and b not in used:
            used |= {a, b}
            sets.append([a, b])
    return sets


def _zero_weights(cfg, keep: dict) -> dict:
    """Every tensor of the drafter as zeros, except those in `keep` (only the lm_head matters to these tests)."""
    W = {}
    for name, shape, kind in gen.weight_specs(cfg):
        if name in keep:
            W[name] = keep[name]
        elif kind == "q8":
            W[name] = (np.zeros(shape, np.int8), np.zeros((shape[0], shape[1] // 32), np.uint16))
        elif kind in ("mod", "nf"):
            W[name] = np.zeros(shape, np.float32)
        else:
            W[name] = np.zeros(shape, np.uint16)
    return W


@pytest.mark.parametrize("name", ["flashmap", "mtp_small"])
def test_lm_argmax_exact_ties(name):
    """Rows of the lm_head table copied onto others, each draft row equal to one group's (decoded) table row: the
    group's logits are the row's unique maximum and equal to each other bit for bit, and the token is the group's
    lowest index (argmax takes the lowest index among maxima)."""
    fm = _fm()
    cfg = configs.get("flashmap") if name == "flashmap" else MTP_SMALL
    V, Ht = cfg["vocab"], cfg["target_dim"]
    rows = 16 if cfg["variant"] == "flowmap" else cfg["block"]
    sets = _tie_sets(V, rows)
    _say(f"{name}: lm_head {V} x {Ht} ({cfg['wtype']}), {rows} rows, groups {[s[:4] for s in sets[:6]]} ...")
    key = "lm_head.weight" if cfg["variant"] == "flowmap" else "lm_head"
    spec = {n: (s, k) for n, s, k in gen.weight_specs(cfg)}[key]
    E = gen.make_tensor(cfg, key, *spec)
    for s in sets:
        if isinstance(E, tuple):
            E[0][s[1:]] = E[0][s[0]]
            E[1][s[1:]] = E[1][s[0]]
        else:
            E[s[1:]] = E[s[0]]
    W = _zero_weights(cfg, {key: E})
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = (flowmap.FlowMapOracle if cfg["variant"] == "flowmap" else mtp.MTPOracle)(cfg, {key: E})
    table = o.w(key)
    h = np.stack([table[s[0]] * (1.0 + 0.25 * i) for i, s in enumerate(sets)]).astype(np.float32)
    hid = torch.from_numpy(h).cuda()
    tok = torch.empty(rows, dtype=torch.int32, device="cuda")
    logits = torch.empty(rows, V, dtype=torch.float32, device="cuda")
    d.fm_lm_argmax(hid, rows, tok, logits)
    torch.cuda.synchronize()
    t, lg = tok.cpu().numpy(), logits.cpu().numpy()
    _, z = o.lm_argmax(h.astype(np.float64))
    assert_rows_close(lg, z, what="logits")
    for r, s in enumerate(sets):
        zs = z[r, s]
        others = np.delete(z[r], s)
        assert np.max(np.abs(zs - zs[0])) <= 1e-12 * abs(zs[0]), f"row {r}: oracle group logits differ"
        assert others.max() < zs[0] - 1e-3 * abs(zs[0]), f"row {r}: the group is not the unique maximum"
        assert np.all(lg[r, s] == lg[r, s[0]]), f"row {r}: device logits of identical rows differ: {lg[r, s]}"
        assert t[r] == min(s), f"row {r}: token {t[r]}, expected the group's lowest index {min(s)}"
    _say(f"{name}: {rows} tied rows resolved to the lowest index")


def test_flowmap_last_position_and_empty_append():
    """tiny flow-map: a context filled to the last length a draft allows (max_ctx - T - 1, the last 47 rows by a
    ragged append), a draft there (slot positions up to max_ctx - 1) against the oracle; one more row is refused
    (context full), an empty append is refused, and neither changes the length."""
    fm = _fm()
    cfg = configs.get("tiny")
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = flowmap.FlowMapOracle(cfg, W)
    n0, last = cfg["ctx_rows"], cfg["max_ctx"] - cfg["block"] - 1
    for start, n, key in ((0, n0, "prefill"), (n0, last - n0, "fill")):
        taps = gen.taps(cfg, key, n)
        o.context_append(taps, start)
        d.fm_context_append(torch.from_numpy(taps).cuda(), start)
    torch.cuda.synchronize()
    assert d.length == last
    _say(f"tiny: context filled to {last} rows; draft at pos {last}")
    a = torch.tensor([4095], dtype=torch.int32, device="cuda")
    hid = torch.empty(cfg["block"], cfg["target_dim"], dtype=torch.float32, device="cuda")
    d.fm_draft_block(hid, anchor=a, pos=last)
    tok = torch.empty(cfg["block"], dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg["block"], cfg["vocab"], dtype=torch.float32, device="cuda")
    d.fm_lm_argmax(hid, cfg["block"], tok, logits)
    torch.cuda.synchronize()
    out, _ = o.draft_block(4095, last)
    _, z = o.lm_argmax(out)
    e = assert_rows_close(hid.cpu().numpy(), out, what="hidden at the last position")
    assert_rows_close(logits.cpu().numpy(), z, what="logits at the last position")
    assert_tokens_match(tok.cpu().numpy(), z)
    one = torch.zeros(1, cfg["n_taps"] * cfg["target_dim"], device="cuda")
    with pytest.raises(fm.FmError) as ex:
        d.fm_context_append(one, last)
    assert ex.value.status == fm.FM_E_CONTEXT_FULL
    with pytest.raises(flowmap.ContextFull):
        o.context_append(np.zeros((1, cfg["n_taps"] * cfg["target_dim"]), np.float32), last)
    with pytest.raises(fm.FmError) as ex:
        d.fm_context_append(one[:0], 0)
    assert ex.value.status == fm.FM_E_INVALID
    with pytest.raises(fm.FmError) as ex:
        d.fm_draft_block(hid, anchor=a, pos=last + 1)
    assert ex.value.status in (fm.FM_E_INVALID, fm.FM_E_CONTEXT_FULL)
    assert d.length == last
    _say(f"tiny: draft at the last position ok, hidden err {e:.2e}; full / empty appends refused")


def test_kvinject_full_context():
    """KV-injection with the context at the longest length a draft allows (max_ctx - gamma - 1 rows, the last 54
    by a ragged append): the block attends over every cached row plus its own; one more row is refused."""
    fm = _fm()
    cfg = KV_SMALL
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = kvinject.KVInjectOracle(cfg, W)
    n0, full = cfg["ctx_rows"], cfg["max_ctx"] - cfg["block"] - 1
    for start, n, key in ((0, n0, "prefill"), (n0, full - n0, "fill")):
        taps = gen.taps(cfg, key, n)
        o.context_append(taps, start)
        d.fm_context_append(torch.from_numpy(taps).cuda(), start)
    torch.cuda.synchronize()
    assert d.length == full
    _say(f"kvinject: context of {full} rows (+{cfg['block']} block rows = {full + cfg['block']} keys)")
    an = 4093
    T = cfg["block"]
    hid = torch.empty(T, cfg["target_dim"], dtype=torch.float32, device="cuda")
    d.fm_draft_block(hid, anchor=torch.tensor([an], dtype=torch.int32, device="cuda"))
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    logits = torch.empty(T, cfg["vocab"], dtype=torch.float32, device="cuda")
    d.fm_lm_argmax(hid, T, tok, logits)
    torch.cuda.synchronize()
    out, _ = o.draft_block(an)
    _, z = o.lm_argmax(out)
    e = assert_rows_close(hid.cpu().numpy(), out, what="hidden over the full context")
    assert_rows_close(logits.cpu().numpy(), z, what="logits over the full context")
    assert_tokens_match(tok.cpu().numpy(), z)
    one = np.zeros((1, cfg["n_taps"] * cfg["target_dim"]), np.float32)
    with pytest.raises(fm.FmError) as ex:
        d.fm_context_append(torch.from_numpy(one).cuda(), full)
    assert ex.value.status == fm.FM_E_CONTEXT_FULL
    with pytest.raises(flowmap.ContextFull):
        o.context_append(one, full)
    assert d.length == full and o.length == full
    _say(f"kvinject: full-context draft ok, hidden err {e:.2e}")


@pytest.mark.parametrize("gamma", [1, 16])
def test_kvinject_block_sizes(gamma):
    """KV-injection blocks of one row (the anchor alone) and of 16 rows (the most a draft takes): hidden rows, logits
    and tokens against the oracle after a ragged prefill."""
    fm = _fm()
    cfg = dict(KV_SMALL, block=gamma, name=f"kvinject_g{gamma}")
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = kvinject.KVInjectOracle(cfg, W)
    n = 77
    taps = gen.taps(cfg, "prefill", n)
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    an = 1234
    _say(f"kvinject: block of {gamma} rows over {n} context rows")
    hid = torch.empty(gamma, cfg["target_dim"], dtype=torch.float32, device="cuda")
    d.fm_draft_block(hid, anchor=torch.tensor([an], dtype=torch.int32, device="cuda"))
    tok = torch.empty(gamma, dtype=torch.int32, device="cuda")
    logits = torch.empty(gamma, cfg["vocab"], dtype=torch.float32, device="cuda")
    d.fm_lm_argmax(hid, gamma, tok, logits)
    torch.cuda.synchronize()
    out, _ = o.draft_block(an)
    _, z = o.lm_argmax(out)
    e = assert_rows_close(hid.cpu().numpy(), out, what=f"hidden, block {gamma}")
    assert_rows_close(logits.cpu().numpy(), z, what=f"logits, block {gamma}")
    k = assert_tokens_match(tok.cpu().numpy(), z)
    _say(f"kvinject: block {gamma} hidden err {e:.2e}, tokens exact on {k}/{gamma}")
