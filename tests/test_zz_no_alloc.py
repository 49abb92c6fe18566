"""fm_lm_argmax_static (the entry point that allocates nothing: its scratch is the library's static device array)
against fm_lm_argmax (scratch in the handle's workspace), through the C ABI: two calls in a row, the second with
fewer rows, on a bf16 table (the tiny flow-map shape) and a Q8_0 table (a small MTP head). Tokens are integers and
must be equal; both also pass the oracle's top-2 gap rule."""
import sys

import numpy as np
import pytest

from inputs import configs, gen
from oracle import flowmap, mtp
from tests.parity import assert_tokens_match

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

MTP_SMALL = dict(variant="mtp", dim=512, heads=4, head_dim=256, kv_heads=2, layers=1, ffn=1024, block=8,
                 target_dim=512, n_taps=2, vocab=4096, max_ctx=300, rope="neox", rope_dims=64, rope_theta=1e7,
                 ln_eps=1e-6, rms_eps=1e-6, qk_eps=1e-6, mlp="swiglu", kv_dtype="f32", wtype="q8_0", ctx_rows=300,
                 name="mtp_small")


def _say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["tiny", "mtp_small"])
def test_static_scratch_lm_argmax_matches_the_workspace_one(name):
    from block_drafter_forward_amd import fm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = configs.get("tiny") if name == "tiny" else MTP_SMALL
    W = gen.make_weights(cfg)
    d = fm.Drafter(cfg, fm.upload_weights(W))
    o = flowmap.FlowMapOracle(cfg, W) if name == "tiny" else mtp.MTPOracle(cfg, W)
    Ht = cfg["target_dim"]
    rng = np.random.default_rng(3)
    for call, rows in enumerate((16 if name == "tiny" else 8, 5)):
        _say(f"{name}: call {call}: {rows} rows")
        h = rng.standard_normal((rows, Ht)).astype(np.float32)
        hid = torch.from_numpy(h).cuda()
        t_ws = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
        t_st = torch.full((rows,), -2, dtype=torch.int32, device="cuda")
        d.fm_lm_argmax(hid, rows, t_ws)
        d.fm_lm_argmax_static(hid, rows, t_st)
        torch.cuda.synchronize()
        a, b = t_ws.cpu().numpy(), t_st.cpu().numpy()
        assert np.array_equal(a, b), (a, b)
        _, z = o.lm_argmax(h.astype(np.float64))
        k = assert_tokens_match(b, z)
        _say(f"{name}: call {call}: tokens equal to the workspace entry point's, exact vs oracle on {k}/{rows}")
    with pytest.raises(fm.FmError) as ex:
        d.fm_lm_argmax_static(hid, 17, t_st)
    assert ex.value.status == fm.FM_E_INVALID
