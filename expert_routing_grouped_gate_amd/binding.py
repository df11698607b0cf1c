"""Thin ctypes binding of libmoe (include/moe.h).

Argument marshalling only: each function checks dtypes, shapes and devices
of torch tensors, passes raw device pointers and torch's current HIP stream
to the C entry point of the same name, and raises on a non-zero status.
Every step of the layer runs in the HIP kernels; there is no CPU path.
torch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libmoe.so")

GATE_SOFTMAX, GATE_SIGMOID = 0, 1
FMT_BF16, FMT_W4A8 = 0, 1
DEV_BAD_EXPERT_ID = 1

_c = ctypes
_vp = _c.c_void_p


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {code} ({text})")
        self.code = code


class MoeFfnWeights(_c.Structure):
    _fields_ = [("H", _c.c_int), ("I", _c.c_int), ("E", _c.c_int), ("fmt", _c.c_int),
                ("w13", _vp), ("w13_scales", _vp), ("w2", _vp), ("w2_scales", _vp),
                ("shared_I", _c.c_int),
                ("shared_w13", _vp), ("shared_w13_scales", _vp),
                ("shared_w2", _vp), ("shared_w2_scales", _vp)]


class MoeLayerDesc(_c.Structure):
    _fields_ = [("H", _c.c_int), ("E", _c.c_int), ("k", _c.c_int), ("gate_mode", _c.c_int),
                ("routed_scale", _c.c_float), ("eps", _c.c_float),
                ("wr", _vp), ("bias", _vp), ("ffn", MoeFfnWeights)]


class MoeLayerBuffers(_c.Structure):
    _fields_ = [("logits", _vp), ("topk_ids", _vp), ("topk_w", _vp), ("counts", _vp),
                ("offsets", _vp), ("sorted_pair", _vp), ("pair_pos", _vp), ("dev_status", _vp),
                ("xq", _vp), ("xq_scales", _vp), ("act", _vp), ("act_scales", _vp), ("y", _vp),
                ("shared_act", _vp), ("shared_act_scales", _vp), ("shared_y", _vp),
                ("workspace", _vp), ("workspace_bytes", _c.c_size_t),
                ("ev_ffn_up_begin", _vp), ("ev_ffn_up_end", _vp)]


# name -> (restype, argtypes); mirrors include/moe.h
_I, _F, _SZ = _c.c_int, _c.c_float, _c.c_size_t
_P = _c.POINTER
SIGNATURES = {
    "moe_status_string": (_c.c_char_p, [_I]),
    "moe_router_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_router_logits": (_I, [_vp, _vp, _I, _I, _I, _vp, _vp, _SZ, _vp]),
    "moe_gate_topk": (_I, [_vp, _vp, _I, _I, _I, _I, _F, _F, _vp, _vp, _vp]),
    "moe_route_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_route": (_I, [_vp, _I, _I, _I, _vp, _vp, _vp, _vp, _vp, _vp, _SZ, _vp]),
    "moe_mx_quantize": (_I, [_vp, _I, _I, _vp, _vp, _vp]),
    "moe_add_rmsnorm": (_I, [_vp, _vp, _vp, _I, _I, _F, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_combine_add_rmsnorm": (_I, [_vp, _vp, _vp, _vp, _I, _I, _I, _vp, _vp, _F, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp]),
    "moe_router_f32_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_router_logits_f32": (_I, [_vp, _vp, _I, _I, _I, _vp, _vp, _SZ, _vp]),
    "moe_mx_packed_scales_bytes": (_SZ, [_I, _I]),
    "moe_mx_pack_weight": (_I, [_vp, _vp, _I, _I, _I, _vp, _vp, _vp]),
    "moe_grouped_ffn_up": (_I, [_P(MoeFfnWeights), _vp, _vp, _I, _I, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_ffn_down": (_I, [_P(MoeFfnWeights), _vp, _vp, _I, _I, _vp, _vp, _vp]),
    "moe_shared_ffn": (_I, [_P(MoeFfnWeights), _vp, _vp, _I, _vp, _vp, _vp, _vp]),
    "moe_grouped_ffn": (_I, [_P(MoeFfnWeights), _vp, _vp, _I, _I, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp]),
    "moe_combine": (_I, [_vp, _vp, _vp, _vp, _I, _I, _I, _vp, _vp]),
    "moe_layer_workspace_size": (_SZ, [_P(MoeLayerDesc), _I]),
    "moe_workspace_size": (_SZ, [_P(MoeLayerDesc), _I]),
    "moe_layer_forward": (_I, [_P(MoeLayerDesc), _vp, _I, _vp, _P(MoeLayerBuffers), _vp]),
    "moe_layer_forward_noalloc": (_I, [_P(MoeLayerDesc), _vp, _I, _vp, _P(MoeLayerBuffers), _vp]),
}
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so into the process (after torch, so that the library
    binds to the HIP runtime torch already loaded).  Raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m expert_routing_grouped_gate_amd.build`")
    lib = _c.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, code: int):
    if code != 0:
        raise MoeError(fn, code, load().moe_status_string(code).decode())


def status_string(code: int) -> str:
    return load().moe_status_string(code).decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libmoe takes device tensors only")
            if not t.is_contiguous():
                raise ValueError("libmoe takes contiguous tensors only")


# --------------------------------------------------------------- calls ----

def router_logits(x: torch.Tensor, wr: torch.Tensor, out: Optional[torch.Tensor] = None):
    _dev(x, wr)
    assert x.dtype == torch.bfloat16 and wr.dtype == torch.float32
    T, H = x.shape
    E = wr.shape[0]
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _dev(out)
    nws = int(load().moe_router_workspace_size(T, H, E))
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=x.device) if nws else None
    _check("moe_router_logits", load().moe_router_logits(_ptr(x), _ptr(wr), T, H, E, _ptr(out),
                                                         _ptr(ws), nws, _stream()))
    return out


def gate_topk(logits: torch.Tensor, k: int, mode: int, bias: Optional[torch.Tensor] = None,
              routed_scale: float = 1.0, eps: float = 1e-20, ids=None, w=None):
    _dev(logits, bias)
    assert logits.dtype == torch.float32
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(ids, w)
    _check("moe_gate_topk", load().moe_gate_topk(_ptr(logits), _ptr(bias), T, E, k, mode,
                                                 float(routed_scale), float(eps), _ptr(ids),
                                                 _ptr(w), _stream()))
    return ids, w


def route_workspace_size(T: int, k: int, E: int) -> int:
    return int(load().moe_route_workspace_size(T, k, E))


def route(ids: torch.Tensor, E: int, dev_status: Optional[torch.Tensor] = None, out=None):
    """Returns (counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k])."""
    _dev(ids, dev_status)
    assert ids.dtype == torch.int32
    T, k = ids.shape
    d = ids.device
    if out is None:
        out = (torch.empty(E, dtype=torch.int32, device=d), torch.empty(E + 1, dtype=torch.int32, device=d),
               torch.empty(T * k, dtype=torch.int32, device=d), torch.empty(T * k, dtype=torch.int32, device=d))
    counts, offsets, sp, pp = out
    ws_bytes = route_workspace_size(T, k, E)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=d)
    _check("moe_route", load().moe_route(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sp),
                                         _ptr(pp), _ptr(dev_status), _ptr(ws), ws_bytes, _stream()))
    return counts, offsets, sp, pp


def mx_quantize(x: torch.Tensor):
    _dev(x)
    assert x.dtype == torch.bfloat16
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=x.device)
    _check("moe_mx_quantize", load().moe_mx_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def combine_add_rmsnorm(y, pair_pos, topk_w, shared_y, weight: torch.Tensor, eps: float,
                        residual: Optional[torch.Tensor] = None, out: bool = False, f32: bool = True,
                        bf16: bool = True, residual_out: bool = True, mx: bool = False):
    """moe_combine_add_rmsnorm: the combine of the layer's expert rows, then
    residual add + RMSNorm of the combined rows.  Returns a dict with the
    requested outputs: "out" [T, H] bf16 (the combined rows), and "f32",
    "bf16", "residual", "mx" as add_rmsnorm."""
    T, k = topk_w.shape
    H = y.shape[1]
    _dev(y, pair_pos, topk_w, shared_y, weight, residual)
    dev = y.device
    res = {}
    if out:
        res["out"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if f32:
        res["f32"] = torch.empty((T, H), dtype=torch.float32, device=dev)
    if bf16:
        res["bf16"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if residual_out:
        res["residual"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if mx:
        res["mx"] = (torch.empty((T, H), dtype=torch.uint8, device=dev),
                     torch.empty((T, H // 32), dtype=torch.uint8, device=dev))
    q, qs = res.get("mx", (None, None))
    _check("moe_combine_add_rmsnorm", load().moe_combine_add_rmsnorm(
        _ptr(y), _ptr(pair_pos), _ptr(topk_w), _ptr(shared_y), T, k, H, _ptr(residual), _ptr(weight),
        float(eps), _ptr(res.get("out")), _ptr(res.get("f32")), _ptr(res.get("bf16")),
        _ptr(res.get("residual")), _ptr(q), _ptr(qs), _stream()))
    return res


def router_logits_f32(x: torch.Tensor, wr: torch.Tensor, out: Optional[torch.Tensor] = None):
    """moe_router_logits_f32: logits [T, E] fp32 from fp32 hidden states."""
    _dev(x, wr)
    assert x.dtype == torch.float32 and wr.dtype == torch.float32
    T, H = x.shape
    E = wr.shape[0]
    lib = load()
    if out is None:
        out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    nbytes = lib.moe_router_f32_workspace_size(T, H, E)
    ws = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=x.device)
    _check("moe_router_logits_f32", lib.moe_router_logits_f32(_ptr(x), _ptr(wr), T, H, E, _ptr(out), _ptr(ws),
                                                            ws.numel(), _stream()))
    return out


def add_rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float, residual: Optional[torch.Tensor] = None,
                f32: bool = True, bf16: bool = True, residual_out: bool = True, mx: bool = False):
    """moe_add_rmsnorm: residual add + RMSNorm.  Returns a dict with the
    requested outputs: "f32" [T, H] fp32, "bf16" [T, H] bf16, "residual"
    [T, H] bf16, "mx" ([T, H] uint8 codes, [T, H/32] uint8 scales)."""
    _dev(x, weight, *(() if residual is None else (residual,)))
    assert x.dtype == torch.bfloat16 and weight.dtype == torch.bfloat16
    T, H = x.shape
    assert weight.shape == (H,) and (residual is None or (residual.shape == (T, H) and residual.dtype == torch.bfloat16))
    out = {}
    if f32:
        out["f32"] = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if bf16:
        out["bf16"] = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if residual_out:
        out["residual"] = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if mx:
        out["mx"] = (torch.empty((T, H), dtype=torch.uint8, device=x.device),
                     torch.empty((T, H // 32), dtype=torch.uint8, device=x.device))
    p = lambda k: _ptr(out[k]) if k in out else None  # noqa: E731
    q, qs = out.get("mx", (None, None))
    _check("moe_add_rmsnorm", load().moe_add_rmsnorm(
        _ptr(x), None if residual is None else _ptr(residual), _ptr(weight), T, H, float(eps),
        p("f32"), p("bf16"), p("residual"), None if q is None else _ptr(q), None if qs is None else _ptr(qs),
        _stream()))
    return out


def mx_pack_weight(codes: torch.Tensor, scales: torch.Tensor):
    """Packed layout of MX weights (moe_mx_pack_weight): codes [G, R, K/2] or
    [R, K/2] and scales [G, R, K/32] -> (packed codes, same shape; packed
    scales, uint8 [G, moe_mx_packed_scales_bytes(R, K)] or [bytes])."""
    _dev(codes, scales)
    flat = codes.dim() == 2
    c3 = codes.unsqueeze(0) if flat else codes
    s3 = scales.unsqueeze(0) if flat else scales
    G, R, K2 = c3.shape
    K = 2 * K2
    assert c3.dtype == torch.uint8 and s3.dtype == torch.uint8 and s3.shape == (G, R, K // 32)
    nbytes = load().moe_mx_packed_scales_bytes(R, K)
    pc = torch.empty_like(c3)
    ps = torch.empty((G, nbytes), dtype=torch.uint8, device=c3.device)
    _check("moe_mx_pack_weight", load().moe_mx_pack_weight(
        _ptr(c3.contiguous()), _ptr(s3.contiguous()), G, R, K, _ptr(pc), _ptr(ps), _stream()))
    return (pc[0], ps[0]) if flat else (pc, ps)


@dataclass
class ExpertWeights:
    """Device weights of one MoE layer (see MoeFfnWeights in include/moe.h).
    W4A8 weights are given in the plain layout (codes [.., R, K/2], scales
    [.., R, K/32]) and packed once here; the packed copies are what the
    library reads."""
    H: int
    I: int
    E: int
    fmt: int
    w13: torch.Tensor
    w2: torch.Tensor
    w13_scales: Optional[torch.Tensor] = None
    w2_scales: Optional[torch.Tensor] = None
    shared_I: int = 0
    shared_w13: Optional[torch.Tensor] = None
    shared_w2: Optional[torch.Tensor] = None
    shared_w13_scales: Optional[torch.Tensor] = None
    shared_w2_scales: Optional[torch.Tensor] = None

    def __post_init__(self):
        self._lib_view = {k: getattr(self, k) for k in _WFIELDS}
        if self.fmt == FMT_W4A8:
            for codes, scales in (("w13", "w13_scales"), ("w2", "w2_scales"),
                                  ("shared_w13", "shared_w13_scales"), ("shared_w2", "shared_w2_scales")):
                c, sc = getattr(self, codes), getattr(self, scales)
                if c is not None:
                    self._lib_view[codes], self._lib_view[scales] = mx_pack_weight(c, sc)

    def c_struct(self) -> MoeFfnWeights:
        v = self._lib_view
        _dev(*(v[k] for k in _WFIELDS))
        return MoeFfnWeights(self.H, self.I, self.E, self.fmt, _ptr(v["w13"]), _ptr(v["w13_scales"]),
                             _ptr(v["w2"]), _ptr(v["w2_scales"]), self.shared_I, _ptr(v["shared_w13"]),
                             _ptr(v["shared_w13_scales"]), _ptr(v["shared_w2"]),
                             _ptr(v["shared_w2_scales"]))


_WFIELDS = ("w13", "w13_scales", "w2", "w2_scales", "shared_w13", "shared_w13_scales", "shared_w2",
            "shared_w2_scales")


def _act_tensors(rows: int, I: int, fmt: int, device):
    if fmt == FMT_W4A8:
        return (torch.empty((rows, I), dtype=torch.uint8, device=device),
                torch.empty((rows, I // 32), dtype=torch.uint8, device=device))
    return torch.empty((rows, I), dtype=torch.bfloat16, device=device), None


def grouped_ffn_up(w: ExpertWeights, x, x_scales, k: int, sorted_pair, offsets, act=None, act_scales=None):
    T = x.shape[0]
    if act is None:
        act, act_scales = _act_tensors(T * k, w.I, w.fmt, x.device)
    _dev(x, x_scales, sorted_pair, offsets, act, act_scales)
    ws = w.c_struct()
    _check("moe_grouped_ffn_up", load().moe_grouped_ffn_up(
        _c.byref(ws), _ptr(x), _ptr(x_scales), T, k, _ptr(sorted_pair), _ptr(offsets), _ptr(act),
        _ptr(act_scales), _stream()))
    return act, act_scales


def grouped_ffn_down(w: ExpertWeights, act, act_scales, T: int, k: int, offsets, y=None):
    if y is None:
        y = torch.empty((T * k, w.H), dtype=torch.bfloat16, device=act.device)
    _dev(act, act_scales, offsets, y)
    ws = w.c_struct()
    _check("moe_grouped_ffn_down", load().moe_grouped_ffn_down(
        _c.byref(ws), _ptr(act), _ptr(act_scales), T, k, _ptr(offsets), _ptr(y), _stream()))
    return y


def shared_ffn(w: ExpertWeights, x, x_scales=None, shared_act=None, shared_act_scales=None, shared_y=None):
    T = x.shape[0]
    if shared_act is None:
        shared_act, shared_act_scales = _act_tensors(T, w.shared_I, w.fmt, x.device)
    if shared_y is None:
        shared_y = torch.empty((T, w.H), dtype=torch.bfloat16, device=x.device)
    _dev(x, x_scales, shared_act, shared_act_scales, shared_y)
    ws = w.c_struct()
    _check("moe_shared_ffn", load().moe_shared_ffn(
        _c.byref(ws), _ptr(x), _ptr(x_scales), T, _ptr(shared_act), _ptr(shared_act_scales),
        _ptr(shared_y), _stream()))
    return shared_act, shared_act_scales, shared_y


def grouped_ffn(w: ExpertWeights, x, x_scales, k: int, sorted_pair, offsets, with_shared: bool = True):
    """moe_grouped_ffn: GEMM1 + SwiGLU, GEMM2 (and the shared expert when the
    weights have one and with_shared).  Returns (act, act_scales, y,
    shared_act, shared_act_scales, shared_y)."""
    T = x.shape[0]
    act, act_scales = _act_tensors(T * k, w.I, w.fmt, x.device)
    y = torch.empty((T * k, w.H), dtype=torch.bfloat16, device=x.device)
    sa = sas = sy = None
    if with_shared and w.shared_I > 0:
        sa, sas = _act_tensors(T, w.shared_I, w.fmt, x.device)
        sy = torch.empty((T, w.H), dtype=torch.bfloat16, device=x.device)
    _dev(x, x_scales, sorted_pair, offsets, act, act_scales, y, sa, sas, sy)
    ws = w.c_struct()
    _check("moe_grouped_ffn", load().moe_grouped_ffn(
        _c.byref(ws), _ptr(x), _ptr(x_scales), T, k, _ptr(sorted_pair), _ptr(offsets), _ptr(act),
        _ptr(act_scales), _ptr(y), _ptr(sa), _ptr(sas), _ptr(sy), _stream()))
    return act, act_scales, y, sa, sas, sy


def combine(y, pair_pos, topk_w, shared_y, out=None):
    T, k = topk_w.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _dev(y, pair_pos, topk_w, shared_y, out)
    _check("moe_combine", load().moe_combine(_ptr(y), _ptr(pair_pos), _ptr(topk_w), _ptr(shared_y),
                                             T, k, H, _ptr(out), _stream()))
    return out


class MoeLayer:
    """A layer's device weights plus caller-owned intermediate buffers for
    a fixed token count; ``forward`` is one moe_layer_forward call."""

    def __init__(self, weights: ExpertWeights, wr: torch.Tensor, k: int, gate_mode: int,
                 bias: Optional[torch.Tensor] = None, routed_scale: float = 1.0, eps: float = 1e-20):
        _dev(wr, bias)
        self.w, self.wr, self.bias, self.k = weights, wr, bias, k
        self.desc = MoeLayerDesc(weights.H, weights.E, k, gate_mode, float(routed_scale), float(eps),
                                 _ptr(wr), _ptr(bias), weights.c_struct())
        self._T = None

    def alloc(self, T: int, device):
        w, k, E = self.w, self.k, self.w.E
        i32 = dict(dtype=torch.int32, device=device)
        b = {}
        b["logits"] = torch.empty((T, E), dtype=torch.float32, device=device)
        b["topk_ids"] = torch.empty((T, k), **i32)
        b["topk_w"] = torch.empty((T, k), dtype=torch.float32, device=device)
        b["counts"] = torch.empty(E, **i32)
        b["offsets"] = torch.empty(E + 1, **i32)
        b["sorted_pair"] = torch.empty(T * k, **i32)
        b["pair_pos"] = torch.empty(T * k, **i32)
        b["dev_status"] = torch.zeros(4, **i32)
        if w.fmt == FMT_W4A8:
            b["xq"] = torch.empty((T, w.H), dtype=torch.uint8, device=device)
            b["xq_scales"] = torch.empty((T, w.H // 32), dtype=torch.uint8, device=device)
        b["act"], b["act_scales"] = _act_tensors(T * k, w.I, w.fmt, device)
        b["y"] = torch.empty((T * k, w.H), dtype=torch.bfloat16, device=device)
        if w.shared_I > 0:
            b["shared_act"], b["shared_act_scales"] = _act_tensors(T, w.shared_I, w.fmt, device)
            b["shared_y"] = torch.empty((T, w.H), dtype=torch.bfloat16, device=device)
        nws = int(load().moe_layer_workspace_size(_c.byref(self.desc), T))
        b["workspace"] = torch.empty(max(nws, 16), dtype=torch.uint8, device=device)
        self.buf = b
        self.cbuf = MoeLayerBuffers(**{n: _ptr(b.get(n)) for n, _ in MoeLayerBuffers._fields_
                                       if n not in ("workspace_bytes", "ev_ffn_up_begin", "ev_ffn_up_end")},
                                    workspace_bytes=nws)
        self._T = T
        return b

    def time_ffn_up(self, begin, end):
        """Have later forward calls record these events around the grouped
        GEMM1 launch: objects whose `cuda_event` is a hipEvent_t handle (a
        torch.cuda.Event recorded once, or a raw HIP event); None, None to
        stop."""
        assert self._T is not None, "call alloc() or forward() first"
        self.cbuf.ev_ffn_up_begin = None if begin is None else begin.cuda_event
        self.cbuf.ev_ffn_up_end = None if end is None else end.cuda_event

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        _dev(x)
        assert x.dtype == torch.bfloat16
        T = x.shape[0]
        if self._T != T:
            self.alloc(T, x.device)
        if out is None:
            out = torch.empty((T, self.w.H), dtype=torch.bfloat16, device=x.device)
        _check("moe_layer_forward", load().moe_layer_forward(
            _c.byref(self.desc), _ptr(x), T, _ptr(out), _c.byref(self.cbuf), _stream()))
        return out

    def forward_noalloc(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """One moe_layer_forward_noalloc call: the same layer with the
        library's static scratch in place of the workspace buffer."""
        _dev(x)
        assert x.dtype == torch.bfloat16
        T = x.shape[0]
        if self._T != T:
            self.alloc(T, x.device)
        if out is None:
            out = torch.empty((T, self.w.H), dtype=torch.bfloat16, device=x.device)
        _check("moe_layer_forward_noalloc", load().moe_layer_forward_noalloc(
            _c.byref(self.desc), _ptr(x), T, _ptr(out), _c.byref(self.cbuf), _stream()))
        return out
