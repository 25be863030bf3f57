"""Thin ctypes binding of libtrellis.so (argument marshalling only).

Every computation runs in the HIP library; this module checks dtypes, devices and
contiguity, allocates outputs and workspaces with torch, and passes raw device pointers
and the current HIP stream.  If the library is not built, loading fails loudly: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Dict, List, Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtrellis.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "trellis.h")

TRELLIS_OP_GEMV, TRELLIS_OP_GEMM, TRELLIS_OP_MOE_GEMV, TRELLIS_OP_GEMM_FP8 = 0, 1, 2, 3
TRELLIS_OP_MOE_MLP = 100  # workspace-cache key only (the C ABI has a dedicated size call)
STATUS = {0: "TRELLIS_OK", -1: "TRELLIS_EINVAL", -2: "TRELLIS_EALIGN", -3: "TRELLIS_EWORKSPACE",
          -4: "TRELLIS_EUNSUPPORTED", -5: "TRELLIS_EHIP"}


class TrellisError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class CLinear(ctypes.Structure):
    """Mirror of ``trellis_linear`` in include/trellis.h."""

    _fields_ = [
        ("code", ctypes.c_void_p),
        ("rin", ctypes.c_void_p),
        ("rout", ctypes.c_void_p),
        ("s_in", ctypes.c_void_p),
        ("s_out", ctypes.c_void_p),
        ("K", ctypes.c_int32),
        ("in_features", ctypes.c_int32),
        ("out_features", ctypes.c_int32),
        ("cb", ctypes.c_int32),
    ]


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libtrellis.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run `python -m trellis_coded_bit_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
            L.trellis_abi_version.restype = i32
            L.trellis_abi_version.argtypes = []
            L.trellis_last_error.restype = ctypes.c_char_p
            L.trellis_last_error.argtypes = []
            L.trellis_decode_tiles.restype = i32
            L.trellis_decode_tiles.argtypes = [vp, i32, i32, i32, vp, vp, vp]
            L.had128_scale.restype = i32
            L.had128_scale.argtypes = [vp, i32, i32, i32, vp, vp, i32, vp, i32, vp]
            L.trellis_workspace_bytes.restype = sz
            L.trellis_workspace_bytes.argtypes = [i32, ctypes.POINTER(CLinear), i32, i32]
            L.trellis_gemv.restype = i32
            L.trellis_gemv.argtypes = [ctypes.POINTER(CLinear), vp, i32, vp, vp, sz, vp]
            L.trellis_gemm.restype = i32
            L.trellis_gemm.argtypes = [ctypes.POINTER(CLinear), vp, i32, vp, vp, sz, vp]
            L.trellis_moe_gemv.restype = i32
            L.trellis_moe_gemv.argtypes = [vp, i32, vp, i32, i32, i32, vp, i32, vp, vp, i32, vp, vp, sz, vp]
            L.trellis_decode_tiles_e4m3.restype = i32
            L.trellis_decode_tiles_e4m3.argtypes = [vp, i32, i32, i32, vp, vp]
            L.trellis_gemm_fp8.restype = i32
            L.trellis_gemm_fp8.argtypes = [ctypes.POINTER(CLinear), vp, i32, vp, vp, sz, vp]
            L.trellis_encode_workspace_bytes.restype = sz
            L.trellis_encode_workspace_bytes.argtypes = [i32]
            L.trellis_encode_tiles.restype = i32
            L.trellis_encode_tiles.argtypes = [vp, i32, i32, i32, vp, vp, vp, sz, vp]
            L.trellis_moe_mlp_workspace_bytes.restype = sz
            L.trellis_moe_mlp_workspace_bytes.argtypes = [i32, i32, i32, i32]
            L.trellis_moe_mlp.restype = i32
            L.trellis_moe_mlp.argtypes = [vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                          sz, vp]
            L.trellis_micro_cus.restype = i32
            L.trellis_micro_cus.argtypes = []
            L.trellis_micro_stream_read.restype = i32
            L.trellis_micro_stream_read.argtypes = [vp, sz, i32, vp, vp]
            L.trellis_micro_valu.restype = i32
            L.trellis_micro_valu.argtypes = [i32, i32, i32, vp, vp, vp, vp]
            L.trellis_micro_mfma.restype = i32
            L.trellis_micro_mfma.argtypes = [i32, i32, i32, vp, vp, vp, vp]
            L.trellis_gemv_list_workspace_bytes.restype = sz
            L.trellis_gemv_list_workspace_bytes.argtypes = [vp, i32, i32]
            L.trellis_gemv_list.restype = i32
            L.trellis_gemv_list.argtypes = [vp, i32, i32, vp, sz, vp]
            L.trellis_gemv_list_noalloc.restype = i32
            L.trellis_gemv_list_noalloc.argtypes = [vp, i32, i32, vp]
            L.trellis_validate_table.restype = i32
            L.trellis_validate_table.argtypes = [ctypes.POINTER(CLinear), i32, i32, i32, i32]
            _lib = L
    return _lib


def header_functions(header: str = HEADER) -> List[str]:
    """Names of the functions a header under include/ declares (default include/trellis.h)."""
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const\s+char\s*\*)\s*\*?\s*(\w+)\s*\(", txt, flags=re.M)


def _check(status: int) -> None:
    if status != 0:
        raise TrellisError(status, lib().trellis_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _req(t: torch.Tensor, dtype: torch.dtype, name: str, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------------------
# Workspaces: zero-filled once, reused by back-to-back calls on one stream.
# ---------------------------------------------------------------------------------------

_ws: Dict[Tuple[int, int], torch.Tensor] = {}


def workspace(nbytes: int, device: torch.device, op: int = 0) -> torch.Tensor:
    """One zero-filled workspace per (device, stream), grown on demand.  Every entry point
    leaves the reserved region at the start of a workspace as it found it, so all of them
    share one buffer (``op`` is accepted for compatibility and ignored)."""
    key = (device.index if device.index is not None else torch.cuda.current_device(), _stream())
    w = _ws.get(key)
    if w is None or w.numel() < nbytes:
        w = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws[key] = w
    return w


def _out(out: Optional[torch.Tensor], shape, device, dtype=torch.float16, name="out") -> torch.Tensor:
    """A new output tensor, or the caller's after checking dtype, device, contiguity and size
    (the kernels write exactly prod(shape) elements through its pointer)."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _req(out, dtype, name, device)
    n = 1
    for d in shape:
        n *= int(d)
    if out.numel() != n:
        raise ValueError(f"{name} has {out.numel()} elements, expected {n} (shape {tuple(shape)})")
    return out


def _ws_arg(ws: Optional[torch.Tensor], nb: int, device) -> torch.Tensor:
    if ws is None:
        return workspace(nb, device)
    _req(ws, torch.uint8, "ws", device)
    if ws.numel() < nb:
        raise ValueError(f"workspace of {ws.numel()} bytes < {nb}")
    return ws


class TrellisLinear:
    """Device tensors of one trellis-coded layer (y = x W, W [in, out])."""

    def __init__(self, code: torch.Tensor, rin: torch.Tensor, rout: torch.Tensor,
                 s_in: Optional[torch.Tensor], s_out: Optional[torch.Tensor], K: int, cb: int = 1):
        self.code, self.rin, self.rout, self.s_in, self.s_out, self.K = code, rin, rout, s_in, s_out, int(K)
        self.cb = int(cb)
        ti, tj, nw = code.shape
        self.in_features, self.out_features = 16 * ti, 16 * tj
        if nw != 16 * self.K:
            raise ValueError(f"code last dim {nw} != 16*K")
        dev = code.device
        _req(code, torch.int16, "code")
        _req(rin, torch.float16, "rin", dev)
        _req(rout, torch.float16, "rout", dev)
        if s_in is not None:
            _req(s_in, torch.float32, "s_in", dev)
        if s_out is not None:
            _req(s_out, torch.float32, "s_out", dev)
        self._c = None
        self._ws_bytes = {}

    @classmethod
    def from_host(cls, lin, device="cuda") -> "TrellisLinear":
        """From a ``synth.Linear`` (numpy arrays)."""
        t = lambda a: torch.from_numpy(a).to(device)
        return cls(t(lin.code), t(lin.rin), t(lin.rout), t(lin.s_in), t(lin.s_out), lin.K, getattr(lin, "cb", 1))

    def c(self) -> CLinear:
        if self._c is None:
            self._c = CLinear(_ptr(self.code), _ptr(self.rin), _ptr(self.rout), _ptr(self.s_in), _ptr(self.s_out),
                              self.K, self.in_features, self.out_features, self.cb)
        return self._c

    def workspace_bytes(self, op: int, batch_or_M: int) -> int:
        key = (op, batch_or_M)
        nb = self._ws_bytes.get(key)
        if nb is None:
            nb = lib().trellis_workspace_bytes(op, ctypes.byref(self.c()), batch_or_M, 0)
            self._ws_bytes[key] = nb
        return nb


# ---------------------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------------------

def trellis_decode_tiles(code: torch.Tensor, K: int, want_states: bool = False):
    """code int16 [in/16, out/16, 16K] -> (w_hat fp16 [in, out], states uint16-as-int16 or None)."""
    _req(code, torch.int16, "code")
    ti, tj, nw = code.shape
    if nw != 16 * K:
        raise ValueError("code last dim must be 16*K")
    w = torch.empty((16 * ti, 16 * tj), dtype=torch.float16, device=code.device)
    st = torch.empty((ti, tj, 256), dtype=torch.int16, device=code.device) if want_states else None
    _check(lib().trellis_decode_tiles(code.data_ptr(), K, 16 * ti, 16 * tj, w.data_ptr(), _ptr(st), _stream()))
    return w, st


def had128_scale(x: torch.Tensor, r: Optional[torch.Tensor] = None, s: Optional[torch.Tensor] = None,
                 post: bool = False, out_dtype: Optional[torch.dtype] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = had(x*r*s) (post=False) or had(x)*r*s (post=True) over 128-blocks of the last axis."""
    if x.dtype not in (torch.float16, torch.float32):
        raise TypeError("x must be float16 or float32")
    _req(x, x.dtype, "x")
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    if r is not None:
        _req(r, torch.float16, "r", x.device)
    if s is not None:
        _req(s, torch.float32, "s", x.device)
    if out is not None and out.dtype not in (torch.float16, torch.float32):
        raise TypeError("out must be float16 or float32")
    out = _out(out, tuple(x.shape), x.device, out.dtype if out is not None else (out_dtype or x.dtype))
    _check(lib().had128_scale(x.data_ptr(), int(x.dtype == torch.float32), rows, n, _ptr(r), _ptr(s), int(post),
                              out.data_ptr(), int(out.dtype == torch.float32), _stream()))
    return out


def trellis_gemv(layer: TrellisLinear, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x fp16 [B, in] (B = 1..8) -> y fp16 [B, out].  ``ws``: optional uint8 workspace tensor
    (at least ``layer.workspace_bytes(TRELLIS_OP_GEMV, B)`` bytes), e.g. for graph capture."""
    _req(x, torch.float16, "x", layer.code.device)
    if x.numel() % layer.in_features:
        raise ValueError(f"x has {x.numel()} elements, not a multiple of in_features={layer.in_features}")
    x2 = x.reshape(-1, layer.in_features)
    B = x2.shape[0]
    out = _out(out, (B, layer.out_features), x.device)
    ws = _ws_arg(ws, layer.workspace_bytes(TRELLIS_OP_GEMV, B), x.device)
    _check(lib().trellis_gemv(ctypes.byref(layer.c()), x2.data_ptr(), B, out.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream()))
    return out


class CGemvItem(ctypes.Structure):
    """Mirror of ``trellis_gemv_item`` in include/trellis.h."""

    _fields_ = [("L", CLinear), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


GEMV_LIST_MAX = 8


def _gemv_items(layers: Sequence[TrellisLinear], xs: Sequence[torch.Tensor], outs: Sequence[torch.Tensor]):
    items = (CGemvItem * len(layers))()
    for i, (l, x, y) in enumerate(zip(layers, xs, outs)):
        items[i].L = l.c()
        items[i].x = x.data_ptr()
        items[i].y = y.data_ptr()
    return items


def trellis_gemv_list_workspace_bytes(layers: Sequence[TrellisLinear], B: int) -> int:
    """Workspace bytes of trellis_gemv_list for these layers at batch B (fake x/y pointers:
    only shapes matter)."""
    items = (CGemvItem * len(layers))()
    for i, l in enumerate(layers):
        items[i].L = l.c()
        items[i].x = 0x1000 * (2 * i + 1) << 32
        items[i].y = 0x1000 * (2 * i + 2) << 32
    nb = lib().trellis_gemv_list_workspace_bytes(items, len(layers), B)
    if nb == 0:
        raise TrellisError(-4, lib().trellis_last_error().decode() or "unsupported list")
    return nb


def trellis_gemv_list(layers: Sequence[TrellisLinear], xs: Sequence[torch.Tensor],
                      outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
                      ws: Optional[torch.Tensor] = None) -> List[torch.Tensor]:
    """One launch for several small-batch products: xs[p] fp16 [B, in_p] -> fp16 [B, out_p],
    the same B (1..8) for every layer."""
    n = len(layers)
    if n < 1 or n > GEMV_LIST_MAX or len(xs) != n:
        raise ValueError(f"1..{GEMV_LIST_MAX} layers with one input each expected")
    dev = layers[0].code.device
    x2s, B = [], None
    for l, x in zip(layers, xs):
        _req(x, torch.float16, "x", dev)
        if x.numel() % l.in_features:
            raise ValueError(f"x has {x.numel()} elements, not a multiple of in_features={l.in_features}")
        x2 = x.reshape(-1, l.in_features)
        if B is None:
            B = x2.shape[0]
        elif x2.shape[0] != B:
            raise ValueError("every input must have the same batch B")
        x2s.append(x2)
    outs = list(outs) if outs is not None else [None] * n
    if len(outs) != n:
        raise ValueError("one output (or None) per layer expected")
    ys = [_out(o, (B, l.out_features), dev) for o, l in zip(outs, layers)]
    items = _gemv_items(layers, x2s, ys)
    nb = lib().trellis_gemv_list_workspace_bytes(items, n, B)
    if nb == 0:
        _check(lib().trellis_gemv_list(items, n, B, None, 0, _stream()))
    ws = _ws_arg(ws, nb, dev)
    _check(lib().trellis_gemv_list(items, n, B, ws.data_ptr(), ws.numel(), _stream()))
    return ys


def trellis_gemm(layer: TrellisLinear, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x fp16 [M, in] -> y fp16 [M, out]."""
    _req(x, torch.float16, "x", layer.code.device)
    if x.dim() != 2 or x.shape[1] != layer.in_features:
        raise ValueError(f"x must be [M, {layer.in_features}]")
    M = x.shape[0]
    out = _out(out, (M, layer.out_features), x.device)
    ws = _ws_arg(ws, layer.workspace_bytes(TRELLIS_OP_GEMM, M), x.device)
    _check(lib().trellis_gemm(ctypes.byref(layer.c()), x.data_ptr(), M, out.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream()))
    return out


def trellis_decode_tiles_e4m3(code: torch.Tensor, K: int) -> torch.Tensor:
    """code int16 [in/16, out/16, 16K] -> E4M3 codes uint8 [in, out] (the cb = 2 weights)."""
    _req(code, torch.int16, "code")
    ti, tj, nw = code.shape
    if nw != 16 * K:
        raise ValueError("code last dim must be 16*K")
    w8 = torch.empty((16 * ti, 16 * tj), dtype=torch.uint8, device=code.device)
    _check(lib().trellis_decode_tiles_e4m3(code.data_ptr(), K, 16 * ti, 16 * tj, w8.data_ptr(), _stream()))
    return w8


def trellis_gemm_fp8(layer: TrellisLinear, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x fp16 [M, in] -> y fp16 [M, out] on the FP8 matrix cores (layer.cb must be 2)."""
    _req(x, torch.float16, "x", layer.code.device)
    if x.dim() != 2 or x.shape[1] != layer.in_features:
        raise ValueError(f"x must be [M, {layer.in_features}]")
    M = x.shape[0]
    out = _out(out, (M, layer.out_features), x.device)
    ws = _ws_arg(ws, layer.workspace_bytes(TRELLIS_OP_GEMM_FP8, M), x.device)
    _check(lib().trellis_gemm_fp8(ctypes.byref(layer.c()), x.data_ptr(), M, out.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream()))
    return out


def trellis_encode_tiles(targets: torch.Tensor, K: int, cb: int = 1, want_states: bool = False,
                         ws: Optional[torch.Tensor] = None):
    """targets f32 [T, 16, 16] -> (code int16 [T, 16K], states uint16-as-int16 [T, 256] or None)."""
    _req(targets, torch.float32, "targets")
    if targets.dim() != 3 or tuple(targets.shape[1:]) != (16, 16):
        raise ValueError("targets must be [T, 16, 16]")
    T = targets.shape[0]
    code = torch.empty((T, 16 * K), dtype=torch.int16, device=targets.device)
    st = torch.empty((T, 256), dtype=torch.int16, device=targets.device) if want_states else None
    nb = lib().trellis_encode_workspace_bytes(T)
    if ws is None:
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=targets.device)
    elif ws.numel() < nb:
        raise ValueError(f"workspace of {ws.numel()} bytes < {nb}")
    _check(lib().trellis_encode_tiles(targets.data_ptr(), T, K, cb, code.data_ptr(), _ptr(st), ws.data_ptr(),
                                      ws.numel(), _stream()))
    return code, st


class ExpertTable:
    """A device-resident table of trellis_linear descriptors (uniform in/out, per-entry K)."""

    def __init__(self, layers: Sequence[TrellisLinear], shared_side: int = -1, device="cuda"):
        self.layers = list(layers)  # keeps the tensors alive
        self.in_features = self.layers[0].in_features
        self.out_features = self.layers[0].out_features
        host = (CLinear * len(self.layers))(*[l.c() for l in self.layers])
        for i, l in enumerate(self.layers):
            if shared_side == 0:
                host[i].rin, host[i].s_in = None, None
            if shared_side == 1:
                host[i].rout, host[i].s_out = None, None
        _check(lib().trellis_validate_table(host, len(self.layers), self.in_features, self.out_features, shared_side))
        raw = bytes(host)
        self.table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(device)
        self.E = len(self.layers)
        self._ws_bytes = {}

    def workspace_bytes(self, n: int) -> int:
        nb = self._ws_bytes.get(n)
        if nb is None:
            probe = CLinear(None, None, None, None, None, 2, self.in_features, self.out_features, 1)
            nb = lib().trellis_workspace_bytes(TRELLIS_OP_MOE_GEMV, ctypes.byref(probe), 1, n)
            self._ws_bytes[n] = nb
        return nb


def trellis_moe_gemv(table: ExpertTable, routed: torch.Tensor, x: torch.Tensor, x_per_expert: bool,
                     shared_r: Optional[torch.Tensor] = None, shared_s: Optional[torch.Tensor] = None,
                     shared_side: int = -1, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """routed int32 [n] (device); x fp16 [in] or [n, in]; returns y fp16 [n, out]."""
    _req(routed, torch.int32, "routed")
    dev = routed.device
    _req(x, torch.float16, "x", dev)
    n = routed.numel()
    if x.numel() != (n if x_per_expert else 1) * table.in_features:
        raise ValueError(f"x must have {'n*' if x_per_expert else ''}in = "
                         f"{(n if x_per_expert else 1) * table.in_features} elements")
    for name, v, dt in (("shared_r", shared_r, torch.float16), ("shared_s", shared_s, torch.float32)):
        if v is not None:
            _req(v, dt, name, dev)
            side_n = table.in_features if shared_side == 0 else table.out_features
            if v.numel() != side_n:
                raise ValueError(f"{name} must have {side_n} elements")
    out = _out(out, (n, table.out_features), dev)
    ws = _ws_arg(ws, table.workspace_bytes(n), dev)
    _check(lib().trellis_moe_gemv(table.table.data_ptr(), table.E, routed.data_ptr(), n, table.in_features,
                                  table.out_features, x.data_ptr(), int(x_per_expert), _ptr(shared_r),
                                  _ptr(shared_s), shared_side, out.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return out


def error_word(ws: Optional[torch.Tensor] = None, device="cuda") -> int:
    """The error word of a workspace (default: the current stream's shared one); it is
    sticky (bit 1: a bad routed id or table entry was skipped; bit 2: a bounded wait ran
    out).  Synchronises."""
    if ws is None:
        ws = _ws.get((torch.device(device).index or 0, _stream()))
    return 0 if ws is None else int(ws[:4].view(torch.int32).item())


def clear_error_word(ws: Optional[torch.Tensor] = None, device="cuda") -> None:
    """Clear a workspace's error word (a fill on the current stream; graph-safe)."""
    if ws is None:
        ws = _ws.get((torch.device(device).index or 0, _stream()))
    if ws is not None:
        ws[:4].zero_()


class MoEMLPTables:
    """Device tables of a routed-expert MLP layer: gate/up slices [E][2H] (entry e*2H + h is
    slice h of gate_e, e*2H + H + h slice h of up_e) and down [E]."""

    def __init__(self, gate: Sequence[Sequence[TrellisLinear]], up: Sequence[Sequence[TrellisLinear]],
                 down: Sequence[TrellisLinear], device="cuda"):
        self.E = len(down)
        self.halves = len(gate[0])
        entries = []
        for e in range(self.E):
            if len(gate[e]) != self.halves or len(up[e]) != self.halves:
                raise ValueError(f"expert {e}: every expert needs {self.halves} gate and up slices")
            entries += list(gate[e]) + list(up[e])
        self.gate_up = ExpertTable(entries, shared_side=0, device=device)
        self.down = ExpertTable(down, shared_side=1, device=device)
        self.hidden = self.gate_up.in_features
        self.inter = self.gate_up.out_features * self.halves
        if self.down.in_features != self.inter or self.down.out_features != self.hidden:
            raise ValueError("down must map inter -> hidden")

    @classmethod
    def from_host(cls, layer, device="cuda") -> "MoEMLPTables":
        """From a ``synth.MoEMLPLayer``; the shared hidden-side arrays are uploaded once and
        every descriptor points at that one copy."""
        t = lambda a: torch.from_numpy(a).to(device)
        r_hi, s_hi = t(layer.r_hidden_in), t(layer.s_hidden_in)
        r_ho, s_ho = t(layer.r_hidden_out), t(layer.s_hidden_out)
        dev = lambda l, rin, s_in, rout, s_out: TrellisLinear(t(l.code), rin, rout, s_in, s_out, l.K,
                                                              getattr(l, "cb", 1))
        E = len(layer.down)
        gate = [[dev(l, r_hi, s_hi, t(l.rout), t(l.s_out)) for l in layer.gate[e]] for e in range(E)]
        up = [[dev(l, r_hi, s_hi, t(l.rout), t(l.s_out)) for l in layer.up[e]] for e in range(E)]
        down = [dev(layer.down[e], t(layer.down[e].rin), t(layer.down[e].s_in), r_ho, s_ho) for e in range(E)]
        obj = cls(gate, up, down, device=device)
        obj.r_hidden_in, obj.s_hidden_in, obj.r_hidden_out, obj.s_hidden_out = r_hi, s_hi, r_ho, s_ho
        return obj

    def workspace_bytes(self, n: int) -> int:
        nb = lib().trellis_moe_mlp_workspace_bytes(self.hidden, self.inter, self.halves, n)
        if nb == 0:
            raise ValueError(f"invalid MLP sizes for n={n}")
        return nb


def trellis_moe_mlp(tables: MoEMLPTables, routed: torch.Tensor, router_w: torch.Tensor, x: torch.Tensor,
                    r_hidden_in: torch.Tensor, s_hidden_in: Optional[torch.Tensor],
                    r_hidden_out: torch.Tensor, s_hidden_out: Optional[torch.Tensor],
                    out: Optional[torch.Tensor] = None, act: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """routed int32 [n], router_w f32 [n], x fp16 [hidden] -> y fp16 [hidden].
    ``act``: optional fp16 [n, inter] receiving silu(gate x) * up x."""
    _req(routed, torch.int32, "routed")
    dev = routed.device
    _req(router_w, torch.float32, "router_w", dev)
    _req(x, torch.float16, "x", dev)
    n = routed.numel()
    if router_w.numel() != n:
        raise ValueError("router_w must have one weight per routed expert")
    if x.numel() != tables.hidden:
        raise ValueError(f"x must have {tables.hidden} elements")
    for name, v, dt in (("r_hidden_in", r_hidden_in, torch.float16), ("r_hidden_out", r_hidden_out, torch.float16),
                        ("s_hidden_in", s_hidden_in, torch.float32), ("s_hidden_out", s_hidden_out, torch.float32)):
        if v is not None:
            _req(v, dt, name, dev)
            if v.numel() != tables.hidden:
                raise ValueError(f"{name} must have {tables.hidden} elements")
    out = _out(out, (tables.hidden,), dev)
    if act is not None:
        _req(act, torch.float16, "act", dev)
        if act.numel() != n * tables.inter:
            raise ValueError(f"act must have n*inter = {n * tables.inter} elements")
    ws = _ws_arg(ws, tables.workspace_bytes(n), dev)
    _check(lib().trellis_moe_mlp(tables.gate_up.table.data_ptr(), tables.down.table.data_ptr(), tables.E,
                                 tables.halves, routed.data_ptr(), router_w.data_ptr(), n, tables.hidden,
                                 tables.inter, x.data_ptr(), _ptr(r_hidden_in), _ptr(s_hidden_in),
                                 _ptr(r_hidden_out), _ptr(s_hidden_out), _ptr(act), out.data_ptr(),
                                 ws.data_ptr(), ws.numel(), _stream()))
    return out


# ---------------------------------------------------------------------------------------
# Microbenchmarks (include/trellis_micro.h): the machine's ceilings, not the method
# ---------------------------------------------------------------------------------------

MICRO_VALU = {"v_add_u32": 0, "v_mul_lo_u32": 1, "v_mul_u32_u24": 2, "v_mad_u32_u24": 3, "v_mad_u32_u16": 4,
              "v_mul_lo_u16_sdwa": 5, "v_pk_mul_lo_u16": 6, "v_bfe_u32": 7, "v_alignbit_b32": 8,
              "v_perm_b32": 9, "v_bitop3_b32": 10, "v_lshrrev_b32": 11, "v_add_f16_sdwa": 12,
              "v_mul_u32_u24_sdwa": 13, "v_fma_f32": 14}
MICRO_DECODE = {"decode_tile": 100, "decode_tile_mfma": 101, "decode_tile_u24": 102}
MICRO_MFMA = {"f16_16x16x32": (0, 16 * 16 * 32), "f16_32x32x16": (1, 32 * 32 * 16),
              "f8_16x16x128": (2, 16 * 16 * 128), "f8_32x32x64": (3, 32 * 32 * 64)}


def micro_cus() -> int:
    return int(lib().trellis_micro_cus())


def micro_stream_read(buf: torch.Tensor, blocks: int = 0) -> torch.Tensor:
    """Enqueue one stream read of ``buf`` (any dtype, 16-byte aligned, size a multiple of 16)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nb = buf.numel() * buf.element_size()
    grid = blocks if blocks > 0 else 8 * micro_cus()
    sink = torch.empty(grid * 256, dtype=torch.int32, device=buf.device)
    _check(lib().trellis_micro_stream_read(buf.data_ptr(), nb, blocks, sink.data_ptr(), _stream()))
    return sink


def micro_clock_kernel(kind: str, name: str, iters: int, waves_per_simd: int, device="cuda"):
    """Run one VALU / decode / MFMA micro kernel; returns (cycles, ticks, ms): int64 tensors
    with one entry per workgroup, and the launch's wall time from events (synchronises)."""
    nblk = micro_cus() * waves_per_simd
    cycles = torch.zeros(nblk, dtype=torch.int64, device=device)
    ticks = torch.zeros(nblk, dtype=torch.int64, device=device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if kind == "mfma":
        sink = torch.empty(nblk * 256, dtype=torch.float32, device=device)
        e0.record()
        st = lib().trellis_micro_mfma(MICRO_MFMA[name][0], iters, waves_per_simd, cycles.data_ptr(),
                                      ticks.data_ptr(), sink.data_ptr(), _stream())
    else:
        op = MICRO_VALU.get(name, MICRO_DECODE.get(name))
        sink = torch.empty(nblk * 256, dtype=torch.int32, device=device)
        e0.record()
        st = lib().trellis_micro_valu(op, iters, waves_per_simd, cycles.data_ptr(), ticks.data_ptr(),
                                      sink.data_ptr(), _stream())
    e1.record()
    if st < 0:
        _check(st)
    torch.cuda.synchronize()
    return cycles, ticks, e0.elapsed_time(e1)
