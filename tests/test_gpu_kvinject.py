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
             name="kvinject_small")


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
