"""Thin Python binding of libfm (include/fm.h): argument marshalling only.

PyTorch provides device memory and the stream; every step of the drafter runs in the HIP kernels behind the C ABI.
The library must be built (``python -m block_drafter_forward_amd.build``); importing this module without it, or
calling into it without a GPU, raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfm.so")

FM_OK, FM_E_INVALID, FM_E_CONTEXT_FULL, FM_E_HIP, FM_E_UNSUPPORTED, FM_E_MISSING_WEIGHT, FM_E_DEVICE = range(7)
STATUS_NAMES = {0: "FM_OK", 1: "FM_E_INVALID", 2: "FM_E_CONTEXT_FULL", 3: "FM_E_HIP", 4: "FM_E_UNSUPPORTED",
                5: "FM_E_MISSING_WEIGHT", 6: "FM_E_DEVICE"}
DRAFT_PATH = {"auto": 0, "launches": 1, "persistent": 2}
VARIANT = {"flowmap": 0, "kvinject": 1, "mtp": 2}
ROPE = {"none": 0, "interleaved": 1, "neox": 2}
MLP = {"gelu_erf": 0, "geglu_tanh": 1, "swiglu": 2}
KV_DTYPE = {"f16": 0, "f32": 1}
WTYPE = {"bf16": 0, "q8_0": 1}


class FmConfig(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("dim", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("block", ctypes.c_int32), ("target_dim", ctypes.c_int32),
                ("n_taps", ctypes.c_int32), ("vocab", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("rope", ctypes.c_int32), ("rope_dims", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("ln_eps", ctypes.c_float), ("rms_eps", ctypes.c_float), ("qk_eps", ctypes.c_float),
                ("mlp", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("wtype", ctypes.c_int32)]


class FmBlockArgs(ctypes.Structure):
    _fields_ = [("anchor", ctypes.c_void_p), ("pos", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("kv_lo", ctypes.c_int32), ("embed_rows", ctypes.c_void_p), ("prev_hidden", ctypes.c_void_p),
                ("debug_layers", ctypes.c_void_p)]


class FmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfm (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_drafter_forward_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.fm_kv_bytes.argtypes = [ctypes.POINTER(FmConfig)]
        L.fm_kv_bytes.restype = sz
        L.fm_workspace_bytes.argtypes = [ctypes.POINTER(FmConfig)]
        L.fm_workspace_bytes.restype = sz
        L.fm_create.argtypes = [ctypes.POINTER(FmConfig), i32, ctypes.POINTER(ctypes.c_char_p),
                                ctypes.POINTER(vp), vp, vp, vp, ctypes.POINTER(vp)]
        L.fm_create.restype = ctypes.c_int
        L.fm_context_append.argtypes = [vp, vp, i32, i32, vp]
        L.fm_context_append.restype = ctypes.c_int
        L.fm_draft_block.argtypes = [vp, ctypes.POINTER(FmBlockArgs), vp, vp]
        L.fm_draft_block.restype = ctypes.c_int
        L.fm_lm_argmax.argtypes = [vp, vp, i32, vp, vp, vp]
        L.fm_lm_argmax.restype = ctypes.c_int
        L.fm_lm_argmax_static.argtypes = [vp, vp, i32, vp, vp]
        L.fm_lm_argmax_static.restype = ctypes.c_int
        L.fm_mtp_chain.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
        L.fm_mtp_chain.restype = ctypes.c_int
        L.fm_markov_argmax.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, ctypes.POINTER(ctypes.c_float), vp, vp]
        L.fm_markov_argmax.restype = ctypes.c_int
        L.fm_time_condition.argtypes = [vp, ctypes.c_float, ctypes.c_float, i32, i32, ctypes.c_float, vp, vp]
        L.fm_time_condition.restype = ctypes.c_int
        L.fm_draft_batch.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(FmBlockArgs), vp, vp]
        L.fm_draft_batch.restype = ctypes.c_int
        L.fm_set_draft_path.argtypes = [vp, i32]
        L.fm_set_draft_path.restype = ctypes.c_int
        L.fm_draft_path.argtypes = [vp]
        L.fm_draft_path.restype = i32
        L.fm_device_status.argtypes = [vp, vp]
        L.fm_device_status.restype = ctypes.c_int
        L.fm_profile_draft.argtypes = [vp, vp, vp, i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32),
                                       ctypes.POINTER(ctypes.c_float), vp]
        L.fm_profile_draft.restype = ctypes.c_int
        L.fm_context_length.argtypes = [vp]
        L.fm_context_length.restype = i32
        L.fm_destroy.argtypes = [vp]
        L.fm_destroy.restype = None
        L.fm_last_error.argtypes = []
        L.fm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().fm_last_error().decode()


def check(status: int):
    if status != FM_OK:
        raise FmError(status, last_error())


def make_config(cfg: dict) -> FmConfig:
    return FmConfig(VARIANT[cfg["variant"]], cfg["dim"], cfg["heads"], cfg["head_dim"], cfg["kv_heads"],
                    cfg["layers"], cfg["ffn"], cfg["block"], cfg["target_dim"], cfg["n_taps"], cfg["vocab"],
                    cfg["max_ctx"], ROPE[cfg["rope"]], cfg["rope_dims"], float(cfg["rope_theta"]),
                    cfg["ln_eps"], cfg["rms_eps"], cfg["qk_eps"], MLP[cfg["mlp"]], KV_DTYPE[cfg["kv_dtype"]],
                    WTYPE[cfg["wtype"]])


def kv_bytes(cfg: dict) -> int:
    c = make_config(cfg)
    return lib().fm_kv_bytes(ctypes.byref(c))


def workspace_bytes(cfg: dict) -> int:
    c = make_config(cfg)
    return lib().fm_workspace_bytes(ctypes.byref(c))


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _device_tensor(a: np.ndarray, device):
    """Upload one stored tensor (bf16 / f16 bits as uint16, int8 codes, f32) to device memory."""
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_weights(weights: dict, device="cuda") -> dict:
    """name -> device tensor; Q8_0 (codes, scales) pairs become "<name>.q" and "<name>.d"."""
    out = {}
    for name, w in weights.items():
        if isinstance(w, tuple):
            out[name + ".q"] = _device_tensor(w[0], device)
            out[name + ".d"] = _device_tensor(w[1], device)
        else:
            out[name] = _device_tensor(w, device)
    return out


class Drafter:
    """One fm_drafter handle with its caller-owned device memory (weights, K/V cache, workspace)."""

    def __init__(self, cfg: dict, dev_weights: dict, stream=None):
        import torch
        self.cfg = cfg
        self.L = lib()
        self.c = make_config(cfg)
        self.weights = dev_weights
        kvb = self.L.fm_kv_bytes(ctypes.byref(self.c))
        wsb = self.L.fm_workspace_bytes(ctypes.byref(self.c))
        if kvb == 0 or wsb == 0:
            raise FmError(FM_E_INVALID, last_error())
        self.kv = torch.empty(kvb, dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        names = [n for n in dev_weights if dev_weights[n].numel() > 0]   # a tensor with no elements has no memory
        self._names = (ctypes.c_char_p * len(names))(*[n.encode() for n in names])
        self._ptrs = (ctypes.c_void_p * len(names))(*[dev_weights[n].data_ptr() for n in names])
        h = ctypes.c_void_p()
        check(self.L.fm_create(ctypes.byref(self.c), len(names), self._names, self._ptrs, self.kv.data_ptr(),
                               self.ws.data_ptr(), _stream_ptr(stream), ctypes.byref(h)))
        self.h = h

    def __del__(self):
        h = getattr(self, "h", None)
        if h is not None and h.value:
            self.L.fm_destroy(h)
            self.h = None

    @property
    def length(self) -> int:
        return self.L.fm_context_length(self.h)

    def set_draft_path(self, path: str):
        check(self.L.fm_set_draft_path(self.h, DRAFT_PATH[path]))

    @property
    def draft_path(self) -> str:
        return {1: "launches", 2: "persistent"}.get(self.L.fm_draft_path(self.h), "?")

    def device_status(self, stream=None):
        check(self.L.fm_device_status(self.h, _stream_ptr(stream)))

    def fm_context_append(self, taps, start: int, stream=None):
        check(self.L.fm_context_append(self.h, taps.data_ptr(), taps.shape[0], start, _stream_ptr(stream)))

    def fm_draft_block(self, hidden_out, anchor=None, pos: int = 0, rows: int = 0, kv_lo: int = 0, embed_rows=None,
                       prev_hidden=None, debug_layers=None, stream=None):
        a = FmBlockArgs(anchor.data_ptr() if anchor is not None else None, pos, rows, kv_lo,
                        embed_rows.data_ptr() if embed_rows is not None else None,
                        prev_hidden.data_ptr() if prev_hidden is not None else None,
                        debug_layers.data_ptr() if debug_layers is not None else None)
        check(self.L.fm_draft_block(self.h, ctypes.byref(a), hidden_out.data_ptr(), _stream_ptr(stream)))

    def profile_draft(self, hidden_out, anchor, pos: int, reps: int = 8, stream=None):
        """A flow-map draft's skinny GEMM launches timed alone and the draft timed whole, with HIP events:
        (skinny_us per draft, skinny_launches, draft_us)."""
        a = FmBlockArgs(anchor.data_ptr(), pos, 0, 0, None, None, None)
        k1, n, tot = ctypes.c_float(), ctypes.c_int32(), ctypes.c_float()
        check(self.L.fm_profile_draft(self.h, ctypes.byref(a), hidden_out.data_ptr(), reps, ctypes.byref(k1),
                                      ctypes.byref(n), ctypes.byref(tot), _stream_ptr(stream)))
        return k1.value, n.value, tot.value

    def fm_lm_argmax(self, hidden, rows: int, tokens, logits=None, stream=None):
        check(self.L.fm_lm_argmax(self.h, hidden.data_ptr(), rows, tokens.data_ptr(),
                                  logits.data_ptr() if logits is not None else None, _stream_ptr(stream)))

    def fm_lm_argmax_static(self, hidden, rows: int, tokens, stream=None):
        check(self.L.fm_lm_argmax_static(self.h, hidden.data_ptr(), rows, tokens.data_ptr(), _stream_ptr(stream)))

    def fm_mtp_chain(self, tokens, h, steps: int, pos: int, kv_lo: int, hidden_out, stream=None):
        check(self.L.fm_mtp_chain(self.h, tokens.data_ptr(), h.data_ptr(), steps, pos, kv_lo, hidden_out.data_ptr(),
                                  _stream_ptr(stream)))

    def fm_markov_argmax(self, hidden, rows: int, anchor, rank: int, tokens, conf, scores=None, thresholds=None,
                         length=None, stream=None):
        """thresholds: None, or rows floats (host): the minimum confidence to keep each position (pruning);
        length: None, or a device int32 tensor [1] that receives the positions kept."""
        thr = None
        if thresholds is not None:
            thr = (ctypes.c_float * rows)(*[float(v) for v in thresholds])
        check(self.L.fm_markov_argmax(self.h, hidden.data_ptr(), rows, anchor.data_ptr(), rank, tokens.data_ptr(),
                                      conf.data_ptr(), scores.data_ptr() if scores is not None else None,
                                      thr, length.data_ptr() if length is not None else None, _stream_ptr(stream)))

    def fm_time_condition(self, s: float, t: float, time_dim: int, cond_dim: int, time_scale: float, table_out=None,
                          stream=None):
        check(self.L.fm_time_condition(self.h, s, t, time_dim, cond_dim, time_scale,
                                       table_out.data_ptr() if table_out is not None else None, _stream_ptr(stream)))

    @staticmethod
    def fm_draft_batch(drafters, requests, hidden_out, stream=None):
        """One block forward for len(drafters) requests, each drafter holding its own context; requests[b] holds
        fm_draft_block's keyword arguments for request b (anchor; or rows, pos, kv_lo, embed_rows, prev_hidden)."""
        L = lib()
        B = len(drafters)
        arr = (ctypes.c_void_p * B)(*[dr.h for dr in drafters])
        args = (FmBlockArgs * B)()
        for b, r in enumerate(requests):
            ptr = lambda k: r[k].data_ptr() if r.get(k) is not None else None
            args[b] = FmBlockArgs(ptr("anchor"), r.get("pos", 0), r.get("rows", 0), r.get("kv_lo", 0),
                                  ptr("embed_rows"), ptr("prev_hidden"), None)
        check(L.fm_draft_batch(arr, B, args, hidden_out.data_ptr(), _stream_ptr(stream)))

    # views of the caller-owned cache (layout documented in include/fm.h)
    def kv_layer(self, l: int, which: int):
        import torch
        c = self.cfg
        if c["variant"] == "mtp":
            w = c["kv_heads"] * c["head_dim"]
            t = self.kv.view(torch.float32).view(2, c["max_ctx"], w)
            return t[which]
        dt = torch.float16 if c["kv_dtype"] == "f16" else torch.float32
        t = self.kv.view(dt).view(c["layers"], 2, c["max_ctx"] * c["dim"])[l, which]
        if c["kv_dtype"] == "f16" and which == 1:   # the f16 V cache is tiled [pos/32][dim][32]: a [pos][dim] copy
            return t.view(c["max_ctx"] // 32, c["dim"], 32).permute(0, 2, 1).reshape(c["max_ctx"], c["dim"])
        return t.view(c["max_ctx"], c["dim"])
