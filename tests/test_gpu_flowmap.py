"""GPU parity of the flow-map drafter (the HIP path through the C ABI) against the float64 oracle."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import flowmap
from tests.parity import assert_rows_close, assert_tokens_match, row_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-flowmap] {msg}", flush=True)
    sys.stdout.flush()


def _setup(cfg, seed=0):
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    W = gen.make_weights(cfg, seed)
    dw = fm.upload_weights(W)
    d = fm.Drafter(cfg, dw)
    o = flowmap.FlowMapOracle(cfg, W)
    return fm, d, o


def _cache_rows(d, l, which, r0, r1):
    return d.kv_layer(l, which)[r0:r1].float().cpu().numpy()


def _check_cache(d, o, cfg, r0, r1, what):
    worst = 0.0
    for l in range(cfg["layers"]):
        worst = max(worst, assert_rows_close(_cache_rows(d, l, 0, r0, r1), o.K[l][r0:r1], what=f"{what} K{l}"))
        worst = max(worst, assert_rows_close(_cache_rows(d, l, 1, r0, r1), o.V[l][r0:r1], what=f"{what} V{l}"))
    return worst


def _draft(fm, d, cfg, anchor, pos, debug=True):
    T, D, Ht = cfg["block"], cfg["dim"], cfg["target_dim"]
    a = torch.tensor([anchor], dtype=torch.int32, device="cuda")
    hid = torch.empty(T, Ht, dtype=torch.float32, device="cuda")
    dbg = torch.empty(cfg["layers"], T, D, dtype=torch.float32, device="cuda") if debug else None
    d.fm_draft_block(hid, anchor=a, pos=pos, debug_layers=dbg)
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    logits = torch.empty(T, cfg["vocab"], dtype=torch.float32, device="cuda")
    d.fm_lm_argmax(hid, T, tok, logits)
    torch.cuda.synchronize()
    return (hid.cpu().numpy(), tok.cpu().numpy(), logits.cpu().numpy(),
            dbg.cpu().numpy() if debug else None)


@pytest.fixture(scope="module")
def tiny():
    cfg = configs.get("tiny")
    _say("tiny: setup")
    fm, d, o = _setup(cfg)
    return cfg, fm, d, o


def test_tiny_prefill_cache(tiny):
    cfg, fm, d, o = tiny
    _say("tiny: 64-row prefill (MFMA path)")
    taps = gen.taps(cfg, "prefill", cfg["ctx_rows"])
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    torch.cuda.synchronize()
    assert d.length == cfg["ctx_rows"]
    w = _check_cache(d, o, cfg, 0, cfg["ctx_rows"], "prefill")
    _say(f"tiny prefill cache worst row err {w:.2e}")


def test_tiny_draft_block(tiny):
    cfg, fm, d, o = tiny
    pos = cfg["ctx_rows"]
    _say(f"tiny: draft at pos {pos}")
    hid, tok, logits, dbg = _draft(fm, d, cfg, anchor=1234, pos=pos)
    out, xs = o.draft_block(1234, pos)
    _, z = o.lm_argmax(out)
    # the anchor slot written at pos
    _check_cache(d, o, cfg, pos, pos + 1, "anchor slot")
    for l in range(cfg["layers"]):
        assert_rows_close(dbg[l], xs[l], what=f"x after layer {l}")
    e = assert_rows_close(hid, out, what="hidden")
    assert_rows_close(logits, z, what="logits")
    n = assert_tokens_match(tok, z)
    _say(f"tiny draft hidden err {e:.2e}, tokens checked exactly on {n}/{cfg['block']} rows")


def test_tiny_small_append_then_draft(tiny):
    # skinny append path (n <= 16) at start = pos (overwrites the anchor slot), then a second draft
    cfg, fm, d, o = tiny
    pos = cfg["ctx_rows"]
    _say("tiny: 7-row append at the anchor position, then draft")
    taps = gen.taps(cfg, "append1", 7)
    o.context_append(taps, pos)
    d.fm_context_append(torch.from_numpy(taps).cuda(), pos)
    torch.cuda.synchronize()
    _check_cache(d, o, cfg, pos, pos + 7, "small append")
    pos2 = pos + 7
    hid, tok, logits, _ = _draft(fm, d, cfg, anchor=77, pos=pos2, debug=False)
    out, _ = o.draft_block(77, pos2)
    _, z = o.lm_argmax(out)
    assert_rows_close(hid, out, what="hidden")
    assert_tokens_match(tok, z)


def test_tiny_draft_is_deterministic(tiny):
    cfg, fm, d, o = tiny
    pos = d.length
    h1, t1, _, _ = _draft(fm, d, cfg, anchor=5, pos=pos, debug=False)
    h2, t2, _, _ = _draft(fm, d, cfg, anchor=5, pos=pos, debug=False)
    assert np.array_equal(h1, h2) and np.array_equal(t1, t2)


def test_tiny_rewind_and_errors(tiny):
    cfg, fm, d, o = tiny
    with pytest.raises(fm.FmError) as e:
        d.fm_context_append(torch.zeros(4, cfg["n_taps"] * cfg["target_dim"], device="cuda"), d.length + 1)
    assert e.value.status == fm.FM_E_INVALID
    with pytest.raises(fm.FmError) as e:
        d.fm_context_append(torch.zeros(cfg["max_ctx"], cfg["n_taps"] * cfg["target_dim"], device="cuda"), 0)
    assert e.value.status == fm.FM_E_CONTEXT_FULL
    hid = torch.empty(cfg["block"], cfg["target_dim"], device="cuda")
    with pytest.raises(fm.FmError) as e:
        d.fm_draft_block(hid, anchor=torch.zeros(1, dtype=torch.int32, device="cuda"), pos=d.length + 1)
    assert e.value.status == fm.FM_E_INVALID


@pytest.fixture(scope="module")
def flashmap():
    cfg = configs.get("flashmap")
    _say("flashmap: generating weights")
    fm, d, o = _setup(cfg)
    return cfg, fm, d, o


def test_flashmap_prefill_and_draft(flashmap):
    cfg, fm, d, o = flashmap
    n = cfg["ctx_rows"]
    _say(f"flashmap: {n}-row prefill")
    taps = gen.taps(cfg, "prefill", n)
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    torch.cuda.synchronize()
    w = _check_cache(d, o, cfg, 0, n, "prefill")
    _say(f"flashmap prefill cache worst row err {w:.2e}")
    an = int(gen.anchors(cfg, "flashmap", 1)[0])
    _say(f"flashmap: draft at pos {n}, anchor {an}")
    hid, tok, logits, dbg = _draft(fm, d, cfg, anchor=an, pos=n)
    out, xs = o.draft_block(an, n)
    _, z = o.lm_argmax(out)
    for l in range(cfg["layers"]):
        assert_rows_close(dbg[l], xs[l], what=f"x after layer {l}")
    e = assert_rows_close(hid, out, what="hidden")
    assert_rows_close(logits, z, what="logits")
    k = assert_tokens_match(tok, z)
    _say(f"flashmap draft hidden err {e:.2e}; tokens exact on {k}/{cfg['block']} rows")


def test_flashmap_ragged_prefill(flashmap):
    """A 1000-row prefill: the fusion GEMM on 128-row tiles, the 12 K/V projections on 256-row tiles whose last
    row block is ragged (1000 = 3 x 256 + 232); then a rewinding append of 600 rows at an unaligned start."""
    from block_drafter_forward_amd import fm as fmod
    cfg, _, _, o0 = flashmap
    d = fmod.Drafter(cfg, fmod.upload_weights(o0.raw))
    o = flowmap.FlowMapOracle(cfg, o0.raw)
    o._w = o0._w
    n = 1000
    _say(f"flashmap: {n}-row ragged prefill")
    taps = gen.taps(cfg, "ragged", n)
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    torch.cuda.synchronize()
    rows = np.r_[0:8, 250:262, 760:776, n - 40:n]
    worst = 0.0
    for l in range(cfg["layers"]):
        worst = max(worst, assert_rows_close(d.kv_layer(l, 0)[rows].float().cpu().numpy(), o.K[l][rows],
                                             what=f"ragged K{l}"))
        worst = max(worst, assert_rows_close(d.kv_layer(l, 1)[rows].float().cpu().numpy(), o.V[l][rows],
                                             what=f"ragged V{l}"))
    assert d.length == n
    _say(f"flashmap ragged prefill worst row err {worst:.2e}")
    # a rewinding 600-row append at start 301 (not a multiple of 4 or 32): the K/V projections still run on
    # 256-row tiles, RoPE positions start at 301, V lands in the 32-position tiles 4 positions at a time only where
    # they are aligned; rows before the start keep their values
    s2, n2 = 301, 600
    _say(f"flashmap: {n2}-row append at start {s2}")
    t2 = gen.taps(cfg, "ragged-rewind", n2)
    o.context_append(t2, s2)
    d.fm_context_append(torch.from_numpy(t2).cuda(), s2)
    torch.cuda.synchronize()
    rows = np.r_[290:312, 316:324, 500:515, s2 + n2 - 24:s2 + n2]
    worst = 0.0
    for l in range(cfg["layers"]):
        worst = max(worst, assert_rows_close(d.kv_layer(l, 0)[rows].float().cpu().numpy(), o.K[l][rows],
                                             what=f"rewind K{l}"))
        worst = max(worst, assert_rows_close(d.kv_layer(l, 1)[rows].float().cpu().numpy(), o.V[l][rows],
                                             what=f"rewind V{l}"))
    assert d.length == s2 + n2
    _say(f"flashmap unaligned append worst row err {worst:.2e}")


def test_longctx_workload(flashmap):
    """8192-row prefill on the MFMA path, then 64 draft steps, each followed by an append of U{1..16} rows at the
    anchor position (the long-context workload's own schedule)."""
    from block_drafter_forward_amd import fm as fmod
    cfg0, _, _, o0 = flashmap
    cfg = configs.get("longctx")
    d = fmod.Drafter(cfg, fmod.upload_weights(o0.raw))
    o = flowmap.FlowMapOracle(cfg, o0.raw)
    o._w = o0._w                      # share the decoded float64 weights
    n = cfg["ctx_rows"]
    _say(f"longctx: {n}-row prefill")
    taps = gen.taps(cfg, "prefill", n)
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    torch.cuda.synchronize()
    for l in (0, cfg["layers"] - 1):
        rows = np.r_[0:64, n - 64:n]
        assert_rows_close(d.kv_layer(l, 0)[rows].float().cpu().numpy(), o.K[l][rows], what=f"prefill K{l}")
        assert_rows_close(d.kv_layer(l, 1)[rows].float().cpu().numpy(), o.V[l][rows], what=f"prefill V{l}")
    # drafts over short prefixes of the cache: one key, a ragged chunk, and both sides of the split kernel's chunk
    # switch (960 keys: 32-key chunks, as 16 heads x 15 64-key chunks would leave CUs idle; 961 keys: 64-key chunks)
    for pos in (0, 16, 959, 960):
        an = 1000 + pos
        hid, tok, _, _ = _draft(fmod, d, cfg, anchor=an, pos=pos, debug=False)
        out, _ = o.draft_block(an, pos)
        _, z = o.lm_argmax(out)
        e = assert_rows_close(hid, out, what=f"draft at pos {pos} hidden")
        assert_tokens_match(tok, z)
        _say(f"longctx: draft over L={pos + 1} keys ok, hidden err {e:.2e}")
    worst = 0.0
    exact = 0
    for s, (an, pos, ns) in enumerate(gen.longctx_schedule(cfg)):
        hid, tok, _, _ = _draft(fmod, d, cfg, anchor=an, pos=pos, debug=False)
        out, _ = o.draft_block(an, pos)
        _, z = o.lm_argmax(out)
        worst = max(worst, assert_rows_close(hid, out, what=f"step {s} hidden"))
        exact += assert_tokens_match(tok, z)
        t2 = gen.taps(cfg, f"step{s}", ns)
        o.context_append(t2, pos)
        d.fm_context_append(torch.from_numpy(t2).cuda(), pos)
        if s % 16 == 0:
            _say(f"longctx: step {s} pos {pos} (L={pos + 1}) ok, worst hidden err so far {worst:.2e}")
    torch.cuda.synchronize()
    assert d.length == o.length
    _say(f"longctx: 64 steps, worst hidden err {worst:.2e}, tokens exact on {exact}/{64 * cfg['block']} rows")


@pytest.mark.parametrize("widths", [(256, 256), (96, 80)])
def test_tiny_time_conditioning(widths):
    """The adaLN table of a jump s -> t from the time MLPs, written into the drafter's modulation table: equal to
    the oracle's (two jumps), then a prefill and a draft that use it, against the oracle drafting with its own
    table. Power-of-two widths take the coalesced kernels, others the one-row-per-thread ones."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("tiny", time_dim=widths[0], cond_dim=widths[1], time_scale=1000.0)
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    d = fm.Drafter(cfg, dw)
    o = flowmap.FlowMapOracle(cfg, W)
    L, D = cfg["layers"], cfg["dim"]
    mod0 = dw["mod"].cpu().numpy()
    tab = torch.empty(3 * L + 1, 3 * D, dtype=torch.float32, device="cuda")
    for s_, t_ in ((0.25, 0.5), (0.0, 1.0)):
        _say(f"tiny: time conditioning {s_} -> {t_}")
        d.fm_time_condition(s_, t_, cfg["time_dim"], cfg["cond_dim"], cfg["time_scale"], table_out=tab)
        torch.cuda.synchronize()
        got = tab.cpu().numpy()
        ref = o.time_conditioning(s_, t_).reshape(3 * L + 1, 3 * D)
        e = assert_rows_close(got, ref, tol=1e-4, what=f"table {s_}->{t_}")
        _say(f"tiny: table err {e:.2e}")
    assert np.array_equal(dw["mod"].cpu().numpy(), mod0), "the caller's modulation table was written"
    o.use_table(ref.reshape(-1))
    taps = gen.taps(cfg, "prefill", cfg["ctx_rows"])
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    pos = cfg["ctx_rows"]
    hid, tok, logits, dbg = _draft(fm, d, cfg, anchor=321, pos=pos)
    out, _ = o.draft_block(321, pos)
    _, z = o.lm_argmax(out)
    e = assert_rows_close(hid, out, what="hidden with the derived table")
    k = assert_tokens_match(tok, z)
    _say(f"tiny: draft with the derived table: hidden err {e:.2e}, tokens exact on {k}/{cfg['block']}")
    with pytest.raises(fm.FmError) as ex:
        d.fm_time_condition(0.0, 1.0, cfg["time_dim"] - 1, cfg["cond_dim"], 1000.0)
    assert ex.value.status == fm.FM_E_INVALID


def test_flashmap_time_conditioning_table():
    """The adaLN table at the FlashMap shape (dim 2048, 6 layers, time and condition widths 256, time scale 1000:
    the page's configuration), for the page's jump 0 -> 1 and one more, against the oracle. Only the time MLPs and
    the 19 adaLN linears take part, so the other weights are zeros."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("flashmap", time_dim=256, cond_dim=256, time_scale=1000.0)
    W = {}
    for name, shape, kind in gen.weight_specs(cfg):
        if "time_embed" in name or "jump_embed" in name or "adaln" in name:
            W[name] = gen.make_tensor(cfg, name, shape, kind)
        else:
            W[name] = np.zeros(shape, np.float32 if kind == "mod" else np.uint16)
    dw = fm.upload_weights(W)
    d = fm.Drafter(cfg, dw)
    o = flowmap.FlowMapOracle(cfg, W)
    L, D = cfg["layers"], cfg["dim"]
    tab = torch.empty(3 * L + 1, 3 * D, dtype=torch.float32, device="cuda")
    for s_, t_ in ((0.0, 1.0), (0.3, 0.85)):
        d.fm_time_condition(s_, t_, cfg["time_dim"], cfg["cond_dim"], cfg["time_scale"], table_out=tab)
        torch.cuda.synchronize()
        got = tab.cpu().numpy()
        ref = o.time_conditioning(s_, t_).reshape(3 * L + 1, 3 * D)
        e = assert_rows_close(got, ref, tol=1e-4, what=f"flashmap table {s_}->{t_}")
        _say(f"flashmap: time conditioning {s_} -> {t_}: table err {e:.2e}")


def test_tiny_handles_sharing_weights_keep_their_own_tables():
    """Two drafters created on the same weight tensors: time conditioning of one changes that handle's modulation
    table only. The other still drafts with the table it was created with, and each matches an oracle drafting
    with its own table."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("tiny", time_dim=256, cond_dim=256, time_scale=1000.0)
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    da, db = fm.Drafter(cfg, dw), fm.Drafter(cfg, dw)
    oa, ob = flowmap.FlowMapOracle(cfg, W), flowmap.FlowMapOracle(cfg, W)
    _say("tiny: two handles on one weight set, time conditioning on the first")
    da.fm_time_condition(0.0, 1.0, cfg["time_dim"], cfg["cond_dim"], cfg["time_scale"])
    oa.use_table(oa.time_conditioning(0.0, 1.0).reshape(-1))
    taps = gen.taps(cfg, "shared", cfg["ctx_rows"])
    pos = cfg["ctx_rows"]
    for d, o, what in ((da, oa, "conditioned handle"), (db, ob, "other handle")):
        o.context_append(taps, 0)
        d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
        hid, tok, _, _ = _draft(fm, d, cfg, anchor=99, pos=pos, debug=False)
        out, _ = o.draft_block(99, pos)
        _, z = o.lm_argmax(out)
        e = assert_rows_close(hid, out, what=what)
        assert_tokens_match(tok, z)
        _say(f"tiny: {what}: hidden err {e:.2e}")


@pytest.mark.parametrize("n", [40, 16, 5])
def test_tiny_taps_over_f16_range(n):
    """Tap rows whose magnitudes span 1e-3 .. 1e6 (rows far outside f16's range and rows near its subnormals, and
    within each row values spread over three decades): an append of more than 16 rows (f16 matrix-core route, rows
    scaled by powers of two) and appends of 16 rows or fewer (hi + lo bf16 route) both match the oracle's cache rows
    and draft, and the two routes agree with each other."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("tiny")
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    rows = 40
    taps = gen.taps(cfg, "wide-range", rows)
    rng = np.random.default_rng(7)
    row_mag = np.logspace(-3, 6, rows)
    rng.shuffle(row_mag)
    taps = (taps * row_mag[:, None] * 10.0 ** rng.uniform(-1.5, 1.5, taps.shape)).astype(np.float32)
    d = fm.Drafter(cfg, dw)
    o = flowmap.FlowMapOracle(cfg, W)
    _say(f"tiny: {rows} wide-range tap rows appended {n} at a time")
    for r0 in range(0, rows, n):
        t = taps[r0:r0 + n]
        o.context_append(t, r0)
        d.fm_context_append(torch.from_numpy(np.ascontiguousarray(t)).cuda(), r0)
    torch.cuda.synchronize()
    w = _check_cache(d, o, cfg, 0, rows, f"wide-range appends of {n}")
    hid, tok, _, _ = _draft(fm, d, cfg, anchor=11, pos=rows, debug=False)
    out, _ = o.draft_block(11, rows)
    _, z = o.lm_argmax(out)
    e = assert_rows_close(hid, out, what="hidden")
    assert_tokens_match(tok, z)
    _say(f"tiny: appends of {n}: cache err {w:.2e}, hidden err {e:.2e}")
    # the other route over the same rows: one append of all 40 (n = 16, 5) or 16-row pieces (n = 40)
    d2 = fm.Drafter(cfg, dw)
    m = 16 if n > 16 else rows
    for r0 in range(0, rows, m):
        d2.fm_context_append(torch.from_numpy(np.ascontiguousarray(taps[r0:r0 + m])).cuda(), r0)
    torch.cuda.synchronize()
    for l in range(cfg["layers"]):
        for which in (0, 1):
            assert_rows_close(_cache_rows(d, l, which, 0, rows), _cache_rows(d2, l, which, 0, rows),
                              what=f"routes agree, layer {l} {'KV'[which]}")
