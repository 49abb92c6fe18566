"""GPU parity of the KV-injection (DFlash) drafter against the float64 oracle."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import kvinject
from tests.parity import assert_rows_close, assert_tokens_match

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SMALL = dict(variant="kvinject", dim=256, heads=2, head_dim=128, kv_heads=2, layers=2, ffn=512, block=5,
             target_dim=512, n_taps=2, vocab=4096, max_ctx=160, rope="none", rope_dims=0, rope_theta=0.0,
             ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="geglu_tanh", kv_dtype="f32", wtype="bf16", ctx_rows=100,
             markov_rank=64, name="kvinject_small")


def _say(msg):
    print(f"[gpu-kvinject] {msg}", flush=True)
    sys.stdout.flush()


def _setup(cfg):
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    return fm, d, kvinject.KVInjectOracle(cfg, W)


def _check_cache(d, o, cfg, r0, r1, what):
    for i in range(cfg["layers"]):
        assert_rows_close(d.kv_layer(i, 0)[r0:r1].cpu().numpy(), o.K[i][r0:r1], what=f"{what} K{i}")
        assert_rows_close(d.kv_layer(i, 1)[r0:r1].cpu().numpy(), o.V[i][r0:r1], what=f"{what} V{i}")


def _draft(d, cfg, anchor):
    T = cfg["block"]
    a = torch.tensor([anchor], dtype=torch.int32, device="cuda")
    hid = torch.empty(T, cfg["target_dim"], dtype=torch.float32, device="cuda")
    dbg = torch.empty(cfg["layers"], T, cfg["dim"], dtype=torch.float32, device="cuda")
    d.fm_draft_block(hid, anchor=a, debug_layers=dbg)
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    logits = torch.empty(T, cfg["vocab"], dtype=torch.float32, device="cuda")
    d.fm_lm_argmax(hid, T, tok, logits)
    torch.cuda.synchronize()
    return hid.cpu().numpy(), tok.cpu().numpy(), logits.cpu().numpy(), dbg.cpu().numpy()


@pytest.mark.parametrize("name", ["small", "kvinject"])
def test_kvinject_prefill_append_draft(name):
    cfg = SMALL if name == "small" else configs.get("kvinject")
    _say(f"{name}: setup")
    fm, d, o = _setup(cfg)
    n = cfg["ctx_rows"]
    taps = gen.taps(cfg, "prefill", n)
    _say(f"{name}: {n}-row prefill")
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    torch.cuda.synchronize()
    _check_cache(d, o, cfg, 0, n, "prefill")
    an = int(gen.anchors(cfg, name, 1)[0])
    _say(f"{name}: draft, anchor {an}")
    hid, tok, logits, dbg = _draft(d, cfg, an)
    out, xs = o.draft_block(an)
    _, z = o.lm_argmax(out)
    for i in range(cfg["layers"]):
        assert_rows_close(dbg[i], xs[i], what=f"block after layer {i}")
    e = assert_rows_close(hid, out, what="hidden")
    assert_rows_close(logits, z, what="logits")
    k = assert_tokens_match(tok, z)
    _say(f"{name}: hidden err {e:.2e}; tokens exact on {k}/{cfg['block']} rows")
    # a short append (skinny path) that rewinds two rows, then a second draft
    taps2 = gen.taps(cfg, "append", 9)
    o.context_append(taps2, n - 2)
    d.fm_context_append(torch.from_numpy(taps2).cuda(), n - 2)
    torch.cuda.synchronize()
    assert d.length == n + 7
    _check_cache(d, o, cfg, n - 2, n + 7, "append")
    hid, tok, logits, _ = _draft(d, cfg, 17)
    out, _ = o.draft_block(17)
    _, z = o.lm_argmax(out)
    assert_rows_close(hid, out, what="hidden after append")
    assert_tokens_match(tok, z)


@pytest.mark.parametrize("name", ["small", "kvinject"])
def test_kvinject_markov_decode(name):
    """DSpark Markov correction + confidence head after a draft: the oracle conditions each step on the device's
    previous token (each checked by the top-2 gap rule on the oracle's scores), so a near-tie cannot make the two
    decodes diverge; scores within the row tolerance, confidences within 1e-4."""
    cfg = SMALL if name == "small" else configs.get("kvinject")
    fm, d, o = _setup(cfg)
    n = cfg["ctx_rows"]
    taps = gen.taps(cfg, "prefill", n)
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    an = int(gen.anchors(cfg, name + "-markov", 1)[0])
    _say(f"{name}: draft + Markov decode, anchor {an}, rank {cfg['markov_rank']}")
    T, V = cfg["block"], cfg["vocab"]
    a = torch.tensor([an], dtype=torch.int32, device="cuda")
    hid = torch.empty(T, cfg["target_dim"], dtype=torch.float32, device="cuda")
    d.fm_draft_block(hid, anchor=a)
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    conf = torch.empty(T, dtype=torch.float32, device="cuda")
    scores = torch.empty(T, V, dtype=torch.float32, device="cuda")
    d.fm_markov_argmax(hid, T, a, cfg["markov_rank"], tok, conf, scores)
    torch.cuda.synchronize()
    gt = tok.cpu().numpy()
    out, _ = o.draft_block(an)
    ot, osc, oconf = o.markov_decode(o.block_n, out, an, follow=gt)
    k = assert_tokens_match(gt, osc)
    e = assert_rows_close(scores.cpu().numpy(), osc, what="Markov scores")
    assert np.max(np.abs(conf.cpu().numpy() - oconf)) < 1e-4, (conf.cpu().numpy(), oconf)
    _say(f"{name}: tokens {gt.tolist()} (exact on {k}/{T}), scores err {e:.2e}, conf {np.round(oconf, 4).tolist()}")
    # the correction acts: the Markov tokens differ from the plain argmax somewhere, or the scores do
    _, z = o.lm_argmax(out)
    assert np.max(np.abs(osc - z)) > 1e-4
    # a second call over the first 3 rows (greedy and sequential, so a prefix of the same decode): every step's key
    # slot starts from zero again, so tokens and confidences repeat exactly
    tok3 = torch.empty(3, dtype=torch.int32, device="cuda")
    conf3 = torch.empty(3, dtype=torch.float32, device="cuda")
    d.fm_markov_argmax(hid, 3, a, cfg["markov_rank"], tok3, conf3)
    torch.cuda.synchronize()
    assert np.array_equal(tok3.cpu().numpy(), gt[:3])
    assert np.array_equal(conf3.cpu().numpy(), conf.cpu().numpy()[:3])
    with pytest.raises(fm.FmError) as ex:
        d.fm_markov_argmax(hid, T + 1, a, cfg["markov_rank"], tok, conf)
    assert ex.value.status == fm.FM_E_INVALID

    # confidence pruning (DF forwardRows' thresholds / minConf), decided on the device: the kept positions are the
    # unpruned decode's prefix; dropped ones read token -1 and confidence 0; the kept count lands in `length`.
    # Thresholds of 0 never cut and 1.0 (above any sigmoid) always cuts where it stands, so the cut does not hinge on
    # rounding; a uniform minConf halfway between two well-separated device confidences cuts where the oracle's
    # confidences (within 1e-4 of the device's) say it does.
    gc = conf.cpu().numpy()
    length = torch.zeros(1, dtype=torch.int32, device="cuda")
    cases = [[0.0] * T] + [[0.0] * j + [1.0] + [0.0] * (T - j - 1) for j in range(1, T)]
    srt = sorted(set(gc[1:].tolist()))
    for lo, hi in zip(srt, srt[1:]):
        if hi - lo > 1e-3:
            cases.append([(lo + hi) / 2] * T)
    for thr in cases:
        tp = torch.full((T,), 7, dtype=torch.int32, device="cuda")
        cp = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
        d.fm_markov_argmax(hid, T, a, cfg["markov_rank"], tp, cp, thresholds=thr, length=length)
        torch.cuda.synchronize()
        ot_p, _, oc_p = o.markov_decode(o.block_n, out, an, follow=gt, thresholds=thr)
        n_keep = int(length.item())
        assert n_keep == len(ot_p), (thr, n_keep, len(ot_p))
        assert np.array_equal(tp.cpu().numpy()[:n_keep], gt[:n_keep])
        assert np.array_equal(cp.cpu().numpy()[:n_keep], gc[:n_keep])
        assert np.all(tp.cpu().numpy()[n_keep:] == -1) and np.all(cp.cpu().numpy()[n_keep:] == 0.0)
    _say(f"{name}: pruning: {len(cases)} threshold sets, kept lengths checked against the oracle")
    # after pruned calls, an unpruned call decodes every position again
    d.fm_markov_argmax(hid, T, a, cfg["markov_rank"], tok, conf, length=length)
    torch.cuda.synchronize()
    assert int(length.item()) == T and np.array_equal(tok.cpu().numpy(), gt)


@pytest.mark.parametrize("name", ["small", "kvinject"])
def test_kvinject_batched_requests(name):
    """Three requests with their own contexts (different lengths) drafted in one pass: each request's rows equal
    its own oracle's block and the same handle's single-request draft; tokens by the top-2 gap rule."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL if name == "small" else configs.get("kvinject")
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    B, G, Ht = 3, cfg["block"], cfg["target_dim"]
    n = cfg["ctx_rows"]
    lens = [n, n - 37, n - 90]
    ds, os_ = [], []
    for b in range(B):
        d = fm.Drafter(cfg, dw)
        o = kvinject.KVInjectOracle(cfg, W)
        taps = gen.taps(cfg, f"batch-{b}", lens[b])
        o.context_append(taps, 0)
        d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
        ds.append(d)
        os_.append(o)
    anchors = [int(a) for a in gen.anchors(cfg, name + "-batch", B)]
    _say(f"{name}: batched draft of {B} requests, contexts {lens}, anchors {anchors}")
    an = torch.tensor(anchors, dtype=torch.int32, device="cuda")
    hid = torch.empty(B * G, Ht, dtype=torch.float32, device="cuda")
    fm.Drafter.fm_draft_batch(ds, [{"anchor": an[b:b + 1]} for b in range(B)], hid)
    tok = torch.empty(B * G, dtype=torch.int32, device="cuda")
    logits = torch.empty(B * G, cfg["vocab"], dtype=torch.float32, device="cuda")
    ds[0].fm_lm_argmax(hid, B * G, tok, logits)
    torch.cuda.synchronize()
    h, t, lg = hid.cpu().numpy(), tok.cpu().numpy(), logits.cpu().numpy()
    for b in range(B):
        out, _ = os_[b].draft_block(anchors[b])
        _, z = os_[b].lm_argmax(out)
        rows = slice(b * G, (b + 1) * G)
        e = assert_rows_close(h[rows], out, what=f"request {b} hidden")
        assert_rows_close(lg[rows], z, what=f"request {b} logits")
        k = assert_tokens_match(t[rows], z)
        single = torch.empty(G, Ht, dtype=torch.float32, device="cuda")
        ds[b].fm_draft_block(single, anchor=an[b:b + 1])
        torch.cuda.synchronize()
        s = single.cpu().numpy()
        assert np.max(np.abs(s - h[rows])) <= 1e-6 * np.max(np.abs(s)), "batched rows differ from the single draft"
        _say(f"{name}: request {b}: hidden err {e:.2e}, tokens exact on {k}/{G}")
    # each request's Markov-corrected decode on its own handle reads that request's normed backbone rows
    if "markov_rank" in cfg:
        rk = cfg["markov_rank"]
        for b in range(B):
            rows = slice(b * G, (b + 1) * G)
            tk = torch.empty(G, dtype=torch.int32, device="cuda")
            cf = torch.empty(G, dtype=torch.float32, device="cuda")
            sc = torch.empty(G, cfg["vocab"], dtype=torch.float32, device="cuda")
            ds[b].fm_markov_argmax(hid[rows], G, an[b:b + 1], rk, tk, cf, sc)
            torch.cuda.synchronize()
            gt = tk.cpu().numpy()
            out, _ = os_[b].draft_block(anchors[b])
            _, osc, oconf = os_[b].markov_decode(os_[b].block_n, out, anchors[b], follow=gt)
            assert_tokens_match(gt, osc)
            assert_rows_close(sc.cpu().numpy(), osc, what=f"request {b} Markov scores")
            assert np.max(np.abs(cf.cpu().numpy() - oconf)) < 1e-4, (b, cf.cpu().numpy(), oconf)
            _say(f"{name}: request {b}: Markov decode on its own handle, conf {np.round(oconf, 4).tolist()}")
    with pytest.raises(fm.FmError) as ex:
        fm.Drafter.fm_draft_batch([ds[0], ds[0]], [{"anchor": an[0:1]}, {"anchor": an[1:2]}], hid)
    assert ex.value.status == fm.FM_E_INVALID
    with pytest.raises(fm.FmError) as ex:
        fm.Drafter.fm_draft_batch(ds * 2, [{"anchor": an[b % B:b % B + 1]} for b in range(6)],
                                  torch.empty(6 * G, Ht, device="cuda"))
    assert ex.value.status == fm.FM_E_INVALID
