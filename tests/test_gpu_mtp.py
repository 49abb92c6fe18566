"""GPU parity of the MTP head (Q8_0 weights, grouped-query causal attention over its own cache) against the
float64 oracle."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import mtp
from tests.parity import assert_rows_close, assert_tokens_match

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SMALL = dict(variant="mtp", dim=512, heads=4, head_dim=256, kv_heads=2, layers=1, ffn=1024, block=8,
             target_dim=512, n_taps=2, vocab=4096, max_ctx=300, rope="neox", rope_dims=64, rope_theta=1e7,
             ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="swiglu", kv_dtype="f32", wtype="q8_0", ctx_rows=300,
             name="mtp_small")


def _say(msg):
    print(f"[gpu-mtp] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["small", "mtp"])
def test_mtp_rows(name):
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL if name == "small" else configs.get("mtp")
    _say(f"{name}: generating Q8_0 weights")
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = mtp.MTPOracle(cfg, W)
    kc, vc = gen.mtp_cache_rows(cfg, cfg["max_ctx"])
    H = cfg["dim"]
    for M in (1, 2, 4, 8):
        pos0 = cfg["max_ctx"] - M
        kv_lo = 0 if M != 4 else pos0 // 3
        _say(f"{name}: M={M} pos0={pos0} kv_lo={kv_lo}")
        o.set_cache_rows(kc[:pos0], vc[:pos0])
        d.kv_layer(0, 0)[:pos0].copy_(torch.from_numpy(kc[:pos0]))
        d.kv_layer(0, 1)[:pos0].copy_(torch.from_numpy(vc[:pos0]))
        e, h = gen.mtp_inputs(cfg, M)
        hid = torch.empty(M, H, dtype=torch.float32, device="cuda")
        dbg = torch.empty(1, M, H, dtype=torch.float32, device="cuda")
        d.fm_draft_block(hid, pos=pos0, rows=M, kv_lo=kv_lo, embed_rows=torch.from_numpy(e).cuda(),
                         prev_hidden=torch.from_numpy(h).cuda(), debug_layers=dbg)
        tok = torch.empty(M, dtype=torch.int32, device="cuda")
        logits = torch.empty(M, cfg["vocab"], dtype=torch.float32, device="cuda")
        d.fm_lm_argmax(hid, M, tok, logits)
        torch.cuda.synchronize()
        out = o.forward(e, h, pos0, kv_lo)
        _, z = o.lm_argmax(out)
        # the rows' own K/V were appended to the cache at pos0 .. pos0 + M - 1
        assert_rows_close(d.kv_layer(0, 0)[pos0:pos0 + M].cpu().numpy(), o.Kc[pos0:pos0 + M], what="new K rows")
        assert_rows_close(d.kv_layer(0, 1)[pos0:pos0 + M].cpu().numpy(), o.Vc[pos0:pos0 + M], what="new V rows")
        err = assert_rows_close(hid.cpu().numpy(), out, what=f"hidden M={M}")
        assert_rows_close(logits.cpu().numpy(), z, what=f"logits M={M}")
        k = assert_tokens_match(tok.cpu().numpy(), z)
        _say(f"{name}: M={M} hidden err {err:.2e}; tokens exact on {k}/{M}")


def test_mtp_bad_rows():
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    e = torch.zeros(9, cfg["dim"], device="cuda")
    hid = torch.empty(9, cfg["dim"], device="cuda")
    for rows, pos, kv_lo, st in [(9, 0, 0, fm.FM_E_INVALID), (0, 0, 0, fm.FM_E_INVALID),
                                 (4, cfg["max_ctx"] - 3, 0, fm.FM_E_CONTEXT_FULL), (2, 5, 6, fm.FM_E_INVALID)]:
        with pytest.raises(fm.FmError) as ex:
            d.fm_draft_block(hid, pos=pos, rows=rows, kv_lo=kv_lo, embed_rows=e, prev_hidden=e)
        assert ex.value.status == st
    with pytest.raises(fm.FmError) as ex:
        d.fm_context_append(e, 0)
    assert ex.value.status == fm.FM_E_INVALID


def test_mtp_misaligned_codes_refused():
    """The create-time copies read Q8_0 codes 8 bytes at a time: a misaligned table is refused on the host."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL
    dev = fm.upload_weights(gen.make_weights(cfg))
    q = dev["lm_head.q"]
    buf = torch.zeros(q.numel() + 16, dtype=q.dtype, device="cuda")
    buf[1:1 + q.numel()].copy_(q.reshape(-1))
    dev["lm_head.q"] = buf[1:1 + q.numel()].view(q.shape)
    assert dev["lm_head.q"].data_ptr() % 8 != 0
    with pytest.raises(fm.FmError) as ex:
        fm.Drafter(cfg, dev)
    assert ex.value.status == fm.FM_E_INVALID and "aligned" in str(ex.value)
    torch.cuda.synchronize()


def test_mtp_lm_head_row_scales():
    """The Q8_0 lm_head alone on rows whose magnitudes span 1e-30 .. 1e30 (each row is brought into the f16 range
    by a power of two inside the library): logits within the row tolerance, tokens by the top-2 gap rule."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = mtp.MTPOracle(cfg, W)
    rng = np.random.default_rng(7)
    scales = np.array([1.0, 1e-30, 1e30, 3e-5, 7e4, 1.0, 0.5, 2.0 ** 20], dtype=np.float64)
    h = (rng.standard_normal((8, cfg["target_dim"])) * scales[:, None]).astype(np.float32)
    h[5, ::7] = 0.0                                   # a row with exact zeros in it
    for M in (8, 3):
        _say(f"lm_head row scales: M={M}")
        hid = torch.from_numpy(h[:M].copy()).cuda()
        tok = torch.empty(M, dtype=torch.int32, device="cuda")
        logits = torch.empty(M, cfg["vocab"], dtype=torch.float32, device="cuda")
        d.fm_lm_argmax(hid, M, tok, logits)
        torch.cuda.synchronize()
        _, z = o.lm_argmax(h[:M].astype(np.float64))
        assert_rows_close(logits.cpu().numpy(), z, what=f"logits M={M}")
        assert_tokens_match(tok.cpu().numpy(), z)


@pytest.mark.parametrize("name", ["small", "mtp"])
def test_mtp_chain(name):
    """Chained depth: 3 single-row passes on the device, each on the previous draft token's table row and the
    previous output h'. The oracle chains the device's tokens (each checked by the top-2 gap rule first), so a
    near-tie cannot make the two chains diverge; hidden rows and the new cache rows within the row tolerance."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL if name == "small" else configs.get("mtp")
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = mtp.MTPOracle(cfg, W)
    steps, H = 3, cfg["dim"]
    pos = cfg["max_ctx"] - steps
    kv_lo = 0 if name == "small" else pos // 4
    kc, vc = gen.mtp_cache_rows(cfg, pos)
    o.set_cache_rows(kc, vc)
    d.kv_layer(0, 0)[:pos].copy_(torch.from_numpy(kc))
    d.kv_layer(0, 1)[:pos].copy_(torch.from_numpy(vc))
    _, h = gen.mtp_inputs(cfg, 1)
    tok0 = 123 % cfg["vocab"]
    _say(f"{name}: chain of {steps} from token {tok0} at pos {pos}, kv_lo {kv_lo}")
    tokens = torch.tensor([tok0] + [0] * steps, dtype=torch.int32, device="cuda")
    hid = torch.empty(steps, H, dtype=torch.float32, device="cuda")
    d.fm_mtp_chain(tokens, torch.from_numpy(h[0].copy()).cuda(), steps, pos, kv_lo, hid)
    torch.cuda.synchronize()
    gt = tokens.cpu().numpy()
    _, oh, oz = o.chain(tok0, h[0], steps, pos, kv_lo, follow=gt[1:])
    for i in range(steps):
        assert_tokens_match(gt[i + 1:i + 2], oz[i:i + 1])
    err = assert_rows_close(hid.cpu().numpy(), oh, what="chained h'")
    assert_rows_close(d.kv_layer(0, 0)[pos:pos + steps].cpu().numpy(), o.Kc[pos:pos + steps], what="chained K rows")
    assert_rows_close(d.kv_layer(0, 1)[pos:pos + steps].cpu().numpy(), o.Vc[pos:pos + steps], what="chained V rows")
    _say(f"{name}: chain tokens {gt[1:].tolist()}, h' err {err:.2e}")
    with pytest.raises(fm.FmError) as ex:
        d.fm_mtp_chain(tokens, hid[0], steps, cfg["max_ctx"] - 1, 0, hid)
    assert ex.value.status == fm.FM_E_CONTEXT_FULL
    with pytest.raises(fm.FmError) as ex:
        d.fm_mtp_chain(tokens, hid[0], 0, 0, 0, hid)
    assert ex.value.status == fm.FM_E_INVALID


@pytest.mark.parametrize("name", ["small", "mtp"])
def test_mtp_batched_requests(name):
    """Three MTP requests (2, 1 and 4 rows, their own caches, positions and kv_lo) in one pass: each request's rows
    and new cache rows equal its own oracle's and the same handle's single-request pass; tokens by the gap rule."""
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = SMALL if name == "small" else configs.get("mtp")
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    H, mc = cfg["dim"], cfg["max_ctx"]
    Ms = [2, 1, 4]
    poss = [mc - 2, mc - 50, mc - 14]
    kvlos = [0, 7, (mc - 14) // 3]
    kc, vc = gen.mtp_cache_rows(cfg, mc)
    e_all, h_all = gen.mtp_inputs(cfg, sum(Ms))
    ds, reqs, outs, oks = [], [], [], []
    r0 = 0
    for b, (M, pos, kvl) in enumerate(zip(Ms, poss, kvlos)):
        d = fm.Drafter(cfg, dw)
        d.kv_layer(0, 0)[:pos].copy_(torch.from_numpy(kc[:pos]))
        d.kv_layer(0, 1)[:pos].copy_(torch.from_numpy(vc[:pos]))
        o = mtp.MTPOracle(cfg, W)
        o.set_cache_rows(kc[:pos], vc[:pos])
        e, h = e_all[r0:r0 + M], h_all[r0:r0 + M]
        outs.append(o.forward(e, h, pos, kvl))
        oks.append(o)
        reqs.append(dict(rows=M, pos=pos, kv_lo=kvl, embed_rows=torch.from_numpy(e.copy()).cuda(),
                         prev_hidden=torch.from_numpy(h.copy()).cuda()))
        ds.append(d)
        r0 += M
    _say(f"{name}: batched pass of {len(Ms)} requests, rows {Ms}, positions {poss}, kv_lo {kvlos}")
    hid = torch.empty(sum(Ms), H, dtype=torch.float32, device="cuda")
    fm.Drafter.fm_draft_batch(ds, reqs, hid)
    tok = torch.empty(sum(Ms), dtype=torch.int32, device="cuda")
    logits = torch.empty(sum(Ms), cfg["vocab"], dtype=torch.float32, device="cuda")
    ds[0].fm_lm_argmax(hid, sum(Ms), tok, logits)
    torch.cuda.synchronize()
    hg, tg, lg = hid.cpu().numpy(), tok.cpu().numpy(), logits.cpu().numpy()
    r0 = 0
    for b, M in enumerate(Ms):
        rows = slice(r0, r0 + M)
        pos = poss[b]
        err = assert_rows_close(hg[rows], outs[b], what=f"request {b} hidden")
        _, z = oks[b].lm_argmax(outs[b])
        assert_rows_close(lg[rows], z, what=f"request {b} logits")
        k = assert_tokens_match(tg[rows], z)
        assert_rows_close(ds[b].kv_layer(0, 0)[pos:pos + M].cpu().numpy(), oks[b].Kc[pos:pos + M], what="new K")
        assert_rows_close(ds[b].kv_layer(0, 1)[pos:pos + M].cpu().numpy(), oks[b].Vc[pos:pos + M], what="new V")
        single = torch.empty(M, H, dtype=torch.float32, device="cuda")
        ds[b].fm_draft_block(single, pos=pos, rows=M, kv_lo=kvlos[b], embed_rows=reqs[b]["embed_rows"],
                             prev_hidden=reqs[b]["prev_hidden"])
        torch.cuda.synchronize()
        s = single.cpu().numpy()
        assert np.max(np.abs(s - hg[rows])) <= 1e-6 * np.max(np.abs(s)), "batched rows differ from the single pass"
        _say(f"{name}: request {b}: hidden err {err:.2e}, tokens exact on {k}/{M}")
        r0 += M
