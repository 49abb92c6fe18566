"""Two flow-map requests drafted in one pass (fm_draft_batch, B = 2: 32 rows, every DiT weight and the lm_head table
streamed once for both): each request's hidden rows, tokens and logits against its own float64 oracle, each over its
own context of its own length, and each anchor slot in its own request's cache. The batch follows the pages' batched
drafting of several anchors at once (forwardRows over anchors[], each with its own context)."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import flowmap
from tests.parity import assert_rows_close, assert_tokens_match

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-fm-batch] {msg}", flush=True)
    sys.stdout.flush()


LENGTHS = (512, 300)   # the two requests' context rows


@pytest.fixture(scope="module")
def pair():
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("flashmap")
    _say("flashmap: generating weights")
    W = gen.make_weights(cfg)
    dw = fm.upload_weights(W)
    ds, os_ = [], []
    for b, n in enumerate(LENGTHS):
        d = fm.Drafter(cfg, dw)
        o = flowmap.FlowMapOracle(cfg, W)
        taps = gen.taps(cfg, f"batch-{b}", n)
        o.context_append(taps, 0)
        d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
        ds.append(d)
        os_.append(o)
    torch.cuda.synchronize()
    return cfg, fm, ds, os_, dw


def _anchor(cfg, tag):
    return torch.tensor([int(gen.anchors(cfg, tag, 1)[0])], dtype=torch.int32, device="cuda")


def test_two_requests_match_their_own_oracles(pair):
    cfg, fm, ds, os_, _ = pair
    T, Ht, V = cfg["block"], cfg["target_dim"], cfg["vocab"]
    anchors = [_anchor(cfg, f"batch-a{b}") for b in range(2)]
    hid = torch.full((2 * T, Ht), float("nan"), dtype=torch.float32, device="cuda")
    fm.Drafter.fm_draft_batch(ds, [{"anchor": anchors[b], "pos": LENGTHS[b]} for b in range(2)], hid)
    tok = torch.empty(2 * T, dtype=torch.int32, device="cuda")
    logits = torch.empty(2 * T, V, dtype=torch.float32, device="cuda")
    ds[0].fm_lm_argmax(hid, 2 * T, tok, logits=logits)
    torch.cuda.synchronize()
    h, tk, lg = hid.cpu().numpy(), tok.cpu().numpy(), logits.cpu().numpy()
    for b in range(2):
        out, _ = os_[b].draft_block(int(anchors[b].item()), LENGTHS[b])
        _, z = os_[b].lm_argmax(out)
        rows = slice(b * T, (b + 1) * T)
        e = assert_rows_close(h[rows], out, what=f"request {b}: hidden")
        el = assert_rows_close(lg[rows], z, what=f"request {b}: logits")
        k = assert_tokens_match(tk[rows], z)
        for l in range(cfg["layers"]):
            for which in (0, 1):
                p = LENGTHS[b]
                got = ds[b].kv_layer(l, which)[p:p + 1].float().cpu().numpy()
                ref = (os_[b].K if which == 0 else os_[b].V)[l][p:p + 1]
                assert_rows_close(got, ref, what=f"request {b}: anchor slot {'KV'[which]}{l}")
        _say(f"request {b} (L = {LENGTHS[b] + 1}): hidden err {e:.2e}, logits err {el:.2e}, tokens exact on {k}/{T}")


def test_batch_equals_single_drafts(pair):
    """The batched pass and two single drafts agree row for row (within rounding: the k-split of a two-block launch
    may differ), and a batch of one is the single draft exactly."""
    cfg, fm, ds, os_, _ = pair
    T, Ht = cfg["block"], cfg["target_dim"]
    anchors = [_anchor(cfg, f"batch-s{b}") for b in range(2)]
    hb = torch.empty(2 * T, Ht, dtype=torch.float32, device="cuda")
    fm.Drafter.fm_draft_batch(ds, [{"anchor": anchors[b], "pos": LENGTHS[b]} for b in range(2)], hb)
    singles = []
    for b in range(2):
        hs = torch.empty(T, Ht, dtype=torch.float32, device="cuda")
        ds[b].fm_draft_block(hs, anchor=anchors[b], pos=LENGTHS[b])
        h1 = torch.empty(T, Ht, dtype=torch.float32, device="cuda")
        fm.Drafter.fm_draft_batch([ds[b]], [{"anchor": anchors[b], "pos": LENGTHS[b]}], h1)
        torch.cuda.synchronize()
        assert torch.equal(hs, h1), f"request {b}: a batch of one differs from fm_draft_block"
        singles.append(hs.cpu().numpy())
    hb = hb.cpu().numpy()
    for b in range(2):
        assert_rows_close(hb[b * T:(b + 1) * T], singles[b], what=f"request {b}: batch vs single")


def test_batch_refusals(pair):
    cfg, fm, ds, os_, dw = pair
    T, Ht = cfg["block"], cfg["target_dim"]
    a = _anchor(cfg, "batch-r")
    hid = torch.empty(3 * T, Ht, dtype=torch.float32, device="cuda")
    extra = fm.Drafter(cfg, dw)
    with pytest.raises(fm.FmError) as e:   # three requests: more than a flow-map batch takes
        fm.Drafter.fm_draft_batch(ds + [extra], [{"anchor": a, "pos": 0}] * 3, hid)
    assert e.value.status == fm.FM_E_UNSUPPORTED
    with pytest.raises(fm.FmError) as e:   # the same handle twice
        fm.Drafter.fm_draft_batch([ds[0], ds[0]], [{"anchor": a, "pos": 0}] * 2, hid)
    assert e.value.status == fm.FM_E_INVALID
    with pytest.raises(fm.FmError) as e:   # a position past the request's own context
        fm.Drafter.fm_draft_batch(ds, [{"anchor": a, "pos": LENGTHS[0]}, {"anchor": a, "pos": LENGTHS[1] + 1}], hid)
    assert e.value.status == fm.FM_E_INVALID
    # a handle whose modulation table was conditioned on another jump
    ct = configs.get("flashmap", time_dim=256, cond_dim=256, time_scale=1000.0)
    tw = {nm: gen.make_tensor(ct, nm, sh, k) for nm, sh, k in gen.weight_specs(ct)
          if "time_embed" in nm or "jump_embed" in nm or "adaln" in nm}
    dwt = dict(dw)
    dwt.update(fm.upload_weights(tw))
    d1, d2 = fm.Drafter(ct, dwt), fm.Drafter(ct, dwt)
    d1.fm_time_condition(0.0, 1.0, 256, 256, 1000.0)
    with pytest.raises(fm.FmError) as e:
        fm.Drafter.fm_draft_batch([d1, d2], [{"anchor": a, "pos": 0}] * 2, hid)
    assert e.value.status == fm.FM_E_INVALID
    d2.fm_time_condition(0.0, 1.0, 256, 256, 1000.0)   # the same jump: the tables agree again
    fm.Drafter.fm_draft_batch([d1, d2], [{"anchor": a, "pos": 0}] * 2, hid[:2 * T])
    torch.cuda.synchronize()
    assert torch.isfinite(hid[:2 * T]).all()
