"""The flow-map draft on its two schedules -- one launch per phase, and the persistent kernel that runs every phase of
the draft in one launch -- each against the float64 oracle at the FlashMap shape, at positions that exercise the
cross-attention's 32-key steps (no context key at all, partial and whole steps) and with the per-layer residuals."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import flowmap
from tests.parity import assert_rows_close, assert_tokens_match

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[gpu-paths] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fmap():
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("flashmap")
    _say("flashmap: generating weights")
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = flowmap.FlowMapOracle(cfg, W)
    n = cfg["ctx_rows"]
    taps = gen.taps(cfg, "paths", n)
    o.context_append(taps, 0)
    d.fm_context_append(torch.from_numpy(taps).cuda(), 0)
    torch.cuda.synchronize()
    return cfg, fm, d, o


def _run(d, cfg, anchor, pos, path, debug=False):
    d.set_draft_path(path)
    T, Ht, D = cfg["block"], cfg["target_dim"], cfg["dim"]
    a = torch.tensor([anchor], dtype=torch.int32, device="cuda")
    hid = torch.full((T, Ht), float("nan"), dtype=torch.float32, device="cuda")
    dbg = torch.full((cfg["layers"], T, D), float("nan"), dtype=torch.float32, device="cuda") if debug else None
    d.fm_draft_block(hid, anchor=a, pos=pos, debug_layers=dbg)
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    d.fm_lm_argmax(hid, T, tok)
    d.device_status()   # synchronises; raises if a persistent launch gave up waiting
    return hid.cpu().numpy(), tok.cpu().numpy(), dbg.cpu().numpy() if debug else None


def test_path_selection_at_the_flashmap_shape(fmap):
    cfg, fm, d, o = fmap
    d.set_draft_path("auto")
    assert d.draft_path == "launches"
    d.set_draft_path("persistent")
    assert d.draft_path == "persistent"
    d.set_draft_path("launches")
    assert d.draft_path == "launches"
    d.set_draft_path("auto")


@pytest.mark.parametrize("pos", [512, 0, 1, 31, 32, 33, 100, 257])
def test_both_paths_match_the_oracle(fmap, pos):
    """pos = 0: the anchor is the only key; 1, 31: one partial 32-key step; 32: one whole step; 33: a whole step
    and a one-key step; 100, 257, 512: several steps and runs. Each draft writes its anchor slot into the cache at
    pos, on the oracle's side too."""
    cfg, fm, d, o = fmap
    an = int(gen.anchors(cfg, f"paths-{pos}", 1)[0])
    out, xs = o.draft_block(an, pos)
    _, z = o.lm_argmax(out)
    res = {}
    for path in ("launches", "persistent"):
        hid, tok, dbg = _run(d, cfg, an, pos, path, debug=True)
        for l in range(cfg["layers"]):
            assert_rows_close(dbg[l], xs[l], what=f"{path}: x after layer {l}")
        e = assert_rows_close(hid, out, what=f"{path}: hidden")
        k = assert_tokens_match(tok, z)
        for l in range(cfg["layers"]):
            for which in (0, 1):
                got = d.kv_layer(l, which)[pos:pos + 1].float().cpu().numpy()
                ref = (o.K if which == 0 else o.V)[l][pos:pos + 1]
                assert_rows_close(got, ref, what=f"{path}: anchor slot {'KV'[which]}{l}")
        res[path] = hid
        _say(f"pos {pos}: {path}: hidden err {e:.2e}, tokens exact on {k}/{cfg['block']}")
    assert_rows_close(res["persistent"], res["launches"], what="the two paths")


def test_persistent_draft_is_deterministic(fmap):
    cfg, fm, d, o = fmap
    pos = cfg["ctx_rows"]
    h1, t1, _ = _run(d, cfg, 4242, pos, "persistent")
    h2, t2, _ = _run(d, cfg, 4242, pos, "persistent")
    assert np.array_equal(h1, h2) and np.array_equal(t1, t2)
    d.set_draft_path("auto")


def test_persistent_path_is_refused_where_it_does_not_apply():
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("tiny")   # 64-wide heads: one launch per phase
    d = fm.Drafter(cfg, fm.upload_weights(gen.make_weights(cfg)))
    assert d.draft_path == "launches"
    with pytest.raises(fm.FmError) as e:
        d.set_draft_path("persistent")
    assert e.value.status == fm.FM_E_UNSUPPORTED
    with pytest.raises(fm.FmError) as e:
        fm.check(d.L.fm_set_draft_path(d.h, 3))
    assert e.value.status == fm.FM_E_INVALID
