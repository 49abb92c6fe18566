"""CPU checks of the C ABI: the library loads, exports every entry point of include/fm.h, and rejects bad arguments
on the host before any device work (no HIP call is reached by these cases)."""
import ctypes
import os
import re

import pytest

from inputs import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
fm = pytest.importorskip("block_drafter_forward_amd.fm")


def _lib():
    if not os.path.exists(fm.LIB_PATH):
        pytest.skip("libfm.so not built")
    return fm.lib()


def test_exports_every_header_symbol():
    L = _lib()
    hdr = open(os.path.join(ROOT, "include", "fm.h")).read()
    names = set(re.findall(r"\b(fm_[a-z_]+)\s*\(", hdr))
    assert {"fm_create", "fm_context_append", "fm_draft_block", "fm_lm_argmax", "fm_destroy"} <= names
    for n in sorted(names):
        assert hasattr(L, n), f"{n} not exported"


@pytest.mark.parametrize("name", configs.ORDER)
def test_sizes_of_the_named_configs(name):
    _lib()
    cfg = configs.get(name)
    kv = fm.kv_bytes(cfg)
    ws = fm.workspace_bytes(cfg)
    assert kv > 0 and ws > 0, fm.last_error()
    if cfg["variant"] == "flowmap":
        assert kv == 2 * cfg["layers"] * cfg["max_ctx"] * cfg["dim"] * 2
    assert ws % 256 == 0


@pytest.mark.parametrize("field,value", [("dim", 0), ("block", 17), ("heads", 3), ("head_dim", 96), ("vocab", 4097),
                                         ("rope", "neox"), ("variant", "mtp")])
def test_invalid_configs_report_zero_size(field, value):
    _lib()
    cfg = configs.get("tiny")
    cfg[field] = value
    assert fm.kv_bytes(cfg) == 0
    assert fm.last_error() != ""


@pytest.mark.parametrize("name", ["flashmap", "kvinject"])
def test_norm_fold_width_limit(name):
    # the LayerNorm / RMSNorm fold reduces at most 256 tiles of 16 columns per row
    _lib()
    cfg = configs.get(name)
    cfg.update(dim=4352, heads=34, kv_heads=34)
    assert fm.kv_bytes(cfg) == 0
    assert "4096" in fm.last_error()


def test_create_rejects_null_and_missing_weights_before_any_launch():
    L = _lib()
    c = fm.make_config(configs.get("tiny"))
    h = ctypes.c_void_p()
    # null kv / workspace
    assert L.fm_create(ctypes.byref(c), 0, None, None, None, None, None, ctypes.byref(h)) == fm.FM_E_INVALID
    # misaligned
    assert L.fm_create(ctypes.byref(c), 0, None, None, 0x1010, 0x2000, None, ctypes.byref(h)) == fm.FM_E_INVALID
    # a table without the required weights (pointers are never dereferenced on this path)
    names = (ctypes.c_char_p * 1)(b"fc.weight")
    ptrs = (ctypes.c_void_p * 1)(0x100000)
    s = L.fm_create(ctypes.byref(c), 1, names, ptrs, 0x200000, 0x300000, None, ctypes.byref(h))
    assert s == fm.FM_E_MISSING_WEIGHT and "missing weight" in fm.last_error()
    assert not h.value
    # a null pointer in the table
    ptrs0 = (ctypes.c_void_p * 1)(None)
    assert L.fm_create(ctypes.byref(c), 1, names, ptrs0, 0x200000, 0x300000, None, ctypes.byref(h)) == fm.FM_E_INVALID


def test_calls_on_a_null_handle():
    L = _lib()
    assert L.fm_context_append(None, 0x1000, 4, 0, None) == fm.FM_E_INVALID
    args = fm.FmBlockArgs()
    assert L.fm_draft_block(None, ctypes.byref(args), 0x1000, None) == fm.FM_E_INVALID
    assert L.fm_lm_argmax(None, 0x1000, 1, 0x2000, None, None) == fm.FM_E_INVALID
    assert L.fm_context_length(None) == -1
    L.fm_destroy(None)


def test_later_entry_points_reject_bad_arguments_on_the_host():
    # chained MTP depth, Markov decode, time conditioning and batched drafts validate before any launch
    L = _lib()
    assert L.fm_mtp_chain(None, 0x1000, 0x2000, 3, 0, 0, 0x3000, None) == fm.FM_E_INVALID
    assert L.fm_markov_argmax(None, 0x1000, 5, 0x2000, 256, 0x3000, 0x4000, None, None, None, None) == fm.FM_E_INVALID
    assert L.fm_time_condition(None, 0.0, 1.0, 256, 256, 1000.0, None, None) == fm.FM_E_INVALID
    assert L.fm_lm_argmax_static(None, 0x1000, 5, 0x2000, None) == fm.FM_E_INVALID
    assert L.fm_set_draft_path(None, 0) == fm.FM_E_INVALID
    assert L.fm_draft_path(None) == -1
    assert L.fm_device_status(None, None) == fm.FM_E_INVALID
    k1, n, tot = ctypes.c_float(), ctypes.c_int32(), ctypes.c_float()
    assert L.fm_profile_draft(None, None, 0x1000, 4, ctypes.byref(k1), ctypes.byref(n), ctypes.byref(tot),
                              None) == fm.FM_E_INVALID
    arr = (ctypes.c_void_p * 1)(None)
    args = (fm.FmBlockArgs * 1)()
    assert L.fm_draft_batch(arr, 1, args, 0x2000, None) == fm.FM_E_INVALID
    assert L.fm_draft_batch(None, 1, args, 0x2000, None) == fm.FM_E_INVALID
    assert L.fm_draft_batch(arr, 0, args, 0x2000, None) == fm.FM_E_INVALID
    assert L.fm_last_error()


def test_bench_refuses_more_than_one_gpu():
    # bench.py measures one GPU; asking for more exits with a message before any GPU work
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
