"""ctypes binding of libtwell.so — argument marshalling only.

Every step of the forward runs in the library's HIP kernels; this module only
checks tensor shapes/dtypes/devices, passes raw device pointers and the current
HIP stream, and turns status codes into exceptions. It never computes a
result itself and has no fallback: if libtwell.so is missing it raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libtwell.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "twell.h")

TWELL_OK = 0
OP_GATE_PACK, OP_FFN_FORWARD, OP_DENSE_FFN, OP_DENSE_FALLBACK, OP_SLICED_UPDOWN, OP_COLUMN_ACTIVITY = 0, 1, 2, 3, 4, 5
OP_FFN_FORWARD_GATEUP = 6


class TwellError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class _Packed(ctypes.Structure):
    _fields_ = [
        ("vals", ctypes.c_void_p),
        ("idx", ctypes.c_void_p),
        ("counts", ctypes.c_void_p),
        ("ovf_rows", ctypes.c_void_p),
        ("n_ovf", ctypes.c_void_p),
    ]


class _Hybrid(ctypes.Structure):
    _fields_ = [
        ("idx", ctypes.c_void_p),
        ("vals", ctypes.c_void_p),
        ("count", ctypes.c_void_p),
        ("res_rows", ctypes.c_void_p),
        ("res_vals", ctypes.c_void_p),
        ("n_res", ctypes.c_void_p),
    ]


class _Spill(ctypes.Structure):
    _fields_ = [
        ("z", ctypes.c_void_p),
        ("slot", ctypes.c_void_p),
        ("n_spill", ctypes.c_void_p),
        ("cap", ctypes.c_int64),
    ]


_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_PK = ctypes.POINTER(_Packed)
_PH = ctypes.POINTER(_Hybrid)
_PS = ctypes.POINTER(_Spill)
_SIGNATURES = {
    "twell_gate_pack": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I32, _I32, _PK, _P, _P, _SZ, _P]),
    "twell_fused_updown": (ctypes.c_int, [_P, _P, _P, _PK, _I64, _I64, _I64, _I32, _I32, _P, _P]),
    "twell_sliced_updown": (ctypes.c_int, [_P, _P, _P, _PK, _I64, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P]),
    "twell_dense_fallback": (ctypes.c_int, [_P, _P, _P, _P, _PK, _I64, _I64, _I64, _P, _P, _SZ, _P, _SZ, _P]),
    "twell_ffn_forward": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P, _SZ, _P]),
    "twell_ffn_forward_timed": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P, _SZ,
                                               _P, _P, _P]),
    "twell_ffn_forward_static": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P]),
    "twell_gateup_pack": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I32, _I32, _PK, _P, _P, _P, _SZ, _P]),
    "twell_hidden_down": (ctypes.c_int, [_P, _PK, _I64, _I64, _I64, _I32, _I32, _P, _P]),
    "twell_ffn_forward_gateup": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P, _SZ,
                                                _P]),
    "twell_dense_ffn_forward": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "twell_column_activity": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _SZ, _P, _SZ, _P]),
    "twell_live_layout": (ctypes.c_int, [_P, _I64, _I32, _P, _I64, ctypes.POINTER(_I64)]),
    "twell_gather_rows": (ctypes.c_int, [_P, _I64, _I64, _P, _I64, _P, _P]),
    "twell_hybrid_pack": (ctypes.c_int, [_PK, _PS, _I64, _I64, _I32, _I32, _I32, _I64, _PH, _P]),
    "twell_gate_pack_spill": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _I32, _I32, _PK, _PS, _P, _P, _SZ, _P]),
    "twell_backward_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32, _I64]),
    "twell_ffn_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _PH, _I64, _I64, _I64, _I32, _I64, _P, _P, _P, _P,
                                          _P, _SZ, _P]),
    "twell_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I64, _I32, _I32]),
    "twell_ctrl_bytes": (_SZ, [_I64]),
    "twell_packed_view": (ctypes.c_int, [_P, _SZ, _I64, _I64, _I64, _I32, _I32, _PK]),
    "twell_status_string": (ctypes.c_char_p, [_I32]),
    "twell_abi_version": (ctypes.c_int32, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtwell.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m activation_sparse_ffn_gate_amd._build` "
                "(there is no CPU fallback)"
            )
        # torch ships its own HIP runtime under the same soname as the system
        # one that libtwell.so links to; the first one loaded serves the whole
        # process, and torch's streams are only valid in torch's. So torch is
        # loaded first, and libtwell.so then binds to the same runtime.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/twell.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(twell_[a-z_0-9]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().twell_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != TWELL_OK:
        raise TwellError(status, where)


def workspace_bytes(op: int, M: int, d: int, F: int, T: int = 0, C: int = 0) -> int:
    return int(lib().twell_workspace_bytes(op, M, d, F, T, C))


def ctrl_bytes(M: int) -> int:
    return int(lib().twell_ctrl_bytes(M))


# --------------------------------------------------------------- torch-facing API
def _torch():
    import torch

    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _bf16(t, name, shape):
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bf16 (or its 16-bit bit pattern), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _dptr(t)


def _f32_out(t, name, shape, device):
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32 of shape {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    return t


@dataclass
class Packed:
    """Device tensors of one TwELL packing (see twell_packed in include/twell.h)."""

    vals: "object"  # float32 [M, F/T, C]
    idx: "object"  # uint8   [M, F/T, C]
    counts: "object"  # int16 storage of uint16 [M, F/T]
    ovf_rows: "object"  # int32 [M]
    n_ovf: "object"  # int32 [1]
    T: int
    C: int

    @classmethod
    def empty(cls, M, F, T, C, device):
        torch = _torch()
        nT = F // T
        return cls(
            torch.empty((M, nT, C), dtype=torch.float32, device=device),
            torch.empty((M, nT, C), dtype=torch.uint8, device=device),
            torch.empty((M, nT), dtype=torch.int16, device=device),
            torch.empty((M,), dtype=torch.int32, device=device),
            torch.empty((1,), dtype=torch.int32, device=device),
            T,
            C,
        )

    def _c(self) -> _Packed:
        return _Packed(*(_dptr(t).value or 0 for t in (self.vals, self.idx, self.counts, self.ovf_rows, self.n_ovf)))


class Workspace:
    """256-byte aligned device scratch, grown on demand and reused.

    zeroed=True makes a control block: zero-filled whenever it is (re)allocated;
    the library leaves it zero-filled after every call, and it is used for
    nothing else.
    """

    def __init__(self, device=None, zeroed=False):
        self.device = device
        self.zeroed = zeroed
        self.buf = None

    def get(self, nbytes: int):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes + 256:
            make = torch.zeros if self.zeroed else torch.empty
            self.buf = make(max(nbytes, 256) + 256, dtype=torch.uint8, device=self.device)
        base = self.buf.data_ptr()
        off = (-base) % 256
        return ctypes.c_void_p(base + off), self.buf.numel() - off


_WS: dict = {}


def _workspace(ws, device, zeroed=False):
    if ws is None:
        key = (device.type, device.index, zeroed)
        if key not in _WS:
            _WS[key] = Workspace(device, zeroed=zeroed)
        ws = _WS[key]
    elif ws.zeroed != zeroed:
        raise ValueError("a control block must be a Workspace(zeroed=True) used for nothing else")
    return ws


def _dptr(t):
    """Device pointer of a tensor, NULL for an empty one."""
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0)


def gate_pack(x, Wg, T: int, C: int, out: Packed | None = None, z_debug=None, ctrl=None) -> Packed:
    """twell_gate_pack. z_debug: None, or a float32 [M, F] tensor to receive z.
    ctrl: a Workspace(zeroed=True) control block (a per-device one by default)."""
    M, d = x.shape
    F = Wg.shape[0]
    px, pw = _bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d))
    out = out or Packed.empty(M, F, T, C, x.device)
    pz = ctypes.c_void_p(0)
    if z_debug is not None:
        _f32_out(z_debug, "z_debug", (M, F), x.device)
        pz = _dptr(z_debug)
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    pk = out._c()
    _check(lib().twell_gate_pack(px, pw, M, d, F, T, C, ctypes.byref(pk), pz, cp, cn, _stream(x)), "twell_gate_pack")
    return out


def fused_updown(x, WuT, Wd, packed: Packed, y=None):
    M, d = x.shape
    F = WuT.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    pk = packed._c()
    _check(lib().twell_fused_updown(*args, ctypes.byref(pk), M, d, F, packed.T, packed.C, _dptr(y), _stream(x)),
           "twell_fused_updown")
    return y


def sliced_updown(x, WuT, Wd, packed: Packed, y=None, workspace=None):
    M, d = x.shape
    F = WuT.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(workspace_bytes(OP_SLICED_UPDOWN, M, d, F, packed.T, packed.C))
    pk = packed._c()
    _check(lib().twell_sliced_updown(*args, ctypes.byref(pk), M, d, F, packed.T, packed.C, _dptr(y), wp, wn,
                                     _stream(x)), "twell_sliced_updown")
    return y


def dense_fallback(x, Wg, WuT, Wd, packed: Packed, y, workspace=None, ctrl=None):
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(workspace_bytes(OP_DENSE_FALLBACK, M, d, F))
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    pk = packed._c()
    _check(lib().twell_dense_fallback(*args, ctypes.byref(pk), M, d, F, _dptr(y), cp, cn, wp, wn, _stream(x)),
           "twell_dense_fallback")
    return y


def ffn_forward(x, Wg, WuT, Wd, T: int, C: int, y=None, workspace=None, ctrl=None):
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(workspace_bytes(OP_FFN_FORWARD, M, d, F, T, C))
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    _check(lib().twell_ffn_forward(*args, M, d, F, T, C, _dptr(y), cp, cn, wp, wn, _stream(x)), "twell_ffn_forward")
    return y


def ffn_forward_timed(x, Wg, WuT, Wd, T: int, C: int, gate_begin, gate_end, y=None, workspace=None, ctrl=None):
    """twell_ffn_forward_timed: the forward, with two torch.cuda.Event
    (enable_timing=True) recorded on the current stream around the gate's
    launches; gate_begin.elapsed_time(gate_end) is then the gate's time."""
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(workspace_bytes(OP_FFN_FORWARD, M, d, F, T, C))
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    evs = []
    for ev in (gate_begin, gate_end):
        if ev.cuda_event == 0:  # torch creates the event on its first record
            ev.record()
        evs.append(ctypes.c_void_p(ev.cuda_event))
    _check(lib().twell_ffn_forward_timed(*args, M, d, F, T, C, _dptr(y), cp, cn, wp, wn, *evs, _stream(x)),
           "twell_ffn_forward_timed")
    return y


def gateup_pack(x, Wg, WuT, T: int, C: int, out: Packed | None = None, z_debug=None, h_debug=None,
                ctrl=None) -> Packed:
    """twell_gateup_pack: dense gate and up products, h packed in TwELL.
    z_debug / h_debug: both None or both float32 [M, F] tensors."""
    M, d = x.shape
    F = Wg.shape[0]
    px, pg, pu = _bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d))
    out = out or Packed.empty(M, F, T, C, x.device)
    pz = ph = ctypes.c_void_p(0)
    if z_debug is not None or h_debug is not None:
        _f32_out(z_debug, "z_debug", (M, F), x.device)
        _f32_out(h_debug, "h_debug", (M, F), x.device)
        pz, ph = _dptr(z_debug), _dptr(h_debug)
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    pk = out._c()
    _check(lib().twell_gateup_pack(px, pg, pu, M, d, F, T, C, ctypes.byref(pk), pz, ph, cp, cn, _stream(x)),
           "twell_gateup_pack")
    return out


def hidden_down(Wd, packed: Packed, y):
    """twell_hidden_down: y rows of non-overflow rows from a packing of h."""
    M, d = y.shape
    F = Wd.shape[0]
    pw = _bf16(Wd, "Wd", (F, d))
    y = _f32_out(y, "y", (M, d), Wd.device)
    pk = packed._c()
    _check(lib().twell_hidden_down(pw, ctypes.byref(pk), M, d, F, packed.T, packed.C, _dptr(y), _stream(Wd)),
           "twell_hidden_down")
    return y


def ffn_forward_gateup(x, Wg, WuT, Wd, T: int, C: int, y=None, workspace=None, ctrl=None):
    """twell_ffn_forward_gateup: the gate-only variant of the forward."""
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    ws = _workspace(workspace, x.device)
    need = max(workspace_bytes(OP_FFN_FORWARD_GATEUP, M, d, F, T, C), workspace_bytes(OP_FFN_FORWARD, M, d, F, T, C))
    wp, wn = ws.get(need)  # also large enough for packed_view
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    _check(lib().twell_ffn_forward_gateup(*args, M, d, F, T, C, _dptr(y), cp, cn, wp, wn, _stream(x)),
           "twell_ffn_forward_gateup")
    return y


def ffn_forward_static(x, Wg, WuT, Wd, T: int, C: int, y=None):
    """twell_ffn_forward_static: the forward for up to 256 rows with the
    library's static scratch buffer (nothing allocated by the library; y is
    allocated here only when not given)."""
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    _check(lib().twell_ffn_forward_static(*args, M, d, F, T, C, _dptr(y), _stream(x)), "twell_ffn_forward_static")
    return y


def dense_ffn_forward(x, Wg, WuT, Wd, y=None, workspace=None):
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)))
    y = _f32_out(y, "y", (M, d), x.device)
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(workspace_bytes(OP_DENSE_FFN, M, d, F))
    _check(lib().twell_dense_ffn_forward(*args, M, d, F, _dptr(y), wp, wn, _stream(x)), "twell_dense_ffn_forward")
    return y


def column_activity(x, Wg, T: int, C: int, bits=None, workspace=None, ctrl=None):
    """twell_column_activity: ORs this batch's unit activity into `bits`
    (int32 [ceil(F / 32)] on x's device; a zeroed one when None) and returns it."""
    torch = _torch()
    M, d = x.shape
    F = Wg.shape[0]
    px, pw = _bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d))
    nwords = -(-F // 32)
    if bits is None:
        bits = torch.zeros(nwords, dtype=torch.int32, device=x.device)
    elif bits.dtype != torch.int32 or tuple(bits.shape) != (nwords,) or not bits.is_contiguous() or not bits.is_cuda:
        raise ValueError(f"bits must be a contiguous int32 device tensor of shape ({nwords},)")
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(workspace_bytes(OP_COLUMN_ACTIVITY, M, d, F, T, C))
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    _check(lib().twell_column_activity(px, pw, M, d, F, T, C, _dptr(bits), cp, cn, wp, wn, _stream(x)),
           "twell_column_activity")
    return bits


def live_layout(bits, F: int, T: int):
    """twell_live_layout (host): numpy int32 source unit of each compacted unit
    (-1 = zero row). bits: host uint32/int32 array or tensor of ceil(F / 32) words."""
    import numpy as np

    b = bits.cpu().numpy() if hasattr(bits, "cpu") else np.asarray(bits)
    b = np.ascontiguousarray(b).view(np.uint32)
    if b.shape != (-(-F // 32),):
        raise ValueError(f"bits must hold {-(-F // 32)} words")
    width = ctypes.c_int64(0)
    _check(lib().twell_live_layout(b.ctypes.data_as(ctypes.c_void_p), F, T, None, 0, ctypes.byref(width)),
           "twell_live_layout")
    src = np.empty(width.value, dtype=np.int32)
    _check(lib().twell_live_layout(b.ctypes.data_as(ctypes.c_void_p), F, T, src.ctypes.data_as(ctypes.c_void_p),
                                   len(src), ctypes.byref(width)), "twell_live_layout")
    return src


def gather_rows(W, src, out=None):
    """twell_gather_rows: out[i] = W[src[i]], a zero row for src[i] < 0.
    src: int32 device tensor [n]."""
    torch = _torch()
    F, d = W.shape
    pw = _bf16(W, "W", (F, d))
    if src.dtype != torch.int32 or src.dim() != 1 or not src.is_contiguous() or not src.is_cuda:
        raise ValueError("src must be a contiguous 1-D int32 device tensor")
    n = src.shape[0]
    if out is None:
        out = torch.empty((n, d), dtype=W.dtype, device=W.device)
    po = _bf16(out, "out", (n, d))
    _check(lib().twell_gather_rows(pw, F, d, _dptr(src), n, po, _stream(W)), "twell_gather_rows")
    return out


def compact_layer(Wg, WuT, Wd, bits, T: int):
    """The layer without its never-active units: (Wg_c, WuT_c, Wd_c, src),
    src the int32 device tensor of source units (-1 = zero padding row)."""
    torch = _torch()
    src = torch.from_numpy(live_layout(bits, Wg.shape[0], T)).to(Wg.device)
    return gather_rows(Wg, src), gather_rows(WuT, src), gather_rows(Wd, src), src


@dataclass
class Hybrid:
    """Device tensors of the hybrid training format (see twell_hybrid in include/twell.h)."""

    idx: "object"  # int32 [M, K]
    vals: "object"  # float32 [M, K]
    count: "object"  # int32 [M]
    res_rows: "object"  # int32 [R]
    res_vals: "object"  # float32 [R, F]
    n_res: "object"  # int32 [1]
    K: int
    R: int

    @classmethod
    def empty(cls, M, F, K, R, device):
        torch = _torch()
        return cls(
            torch.empty((M, K), dtype=torch.int32, device=device),
            torch.empty((M, K), dtype=torch.float32, device=device),
            torch.empty((M,), dtype=torch.int32, device=device),
            torch.empty((R,), dtype=torch.int32, device=device),
            torch.empty((R, F), dtype=torch.float32, device=device),
            torch.empty((1,), dtype=torch.int32, device=device),
            K,
            R,
        )

    def _c(self) -> _Hybrid:
        return _Hybrid(*(_dptr(t).value or 0 for t in (self.idx, self.vals, self.count, self.res_rows,
                                                        self.res_vals, self.n_res)))


@dataclass
class Spill:
    """Device tensors of a training gate's spill list (see twell_spill in include/twell.h)."""

    z: "object"  # float32 [cap, T]
    slot: "object"  # int32 [M, F/T]
    n_spill: "object"  # int32 [1]

    @classmethod
    def empty(cls, M, F, T, cap, device):
        torch = _torch()
        return cls(torch.empty((max(cap, 1), T), dtype=torch.float32, device=device),
                   torch.empty((M, F // T), dtype=torch.int32, device=device),
                   torch.empty((1,), dtype=torch.int32, device=device))

    @property
    def cap(self) -> int:
        return int(self.z.shape[0])

    def _c(self) -> _Spill:
        return _Spill(_dptr(self.z).value or 0, _dptr(self.slot).value or 0, _dptr(self.n_spill).value or 0,
                      self.cap)


def gate_pack_spill(x, Wg, T: int, C: int, cap: int, out: Packed | None = None, spill: Spill | None = None,
                    z_debug=None, ctrl=None):
    """twell_gate_pack_spill: the training gate (packing of capacity C plus the
    spill list of tiles over C, `cap` records). Returns (Packed, Spill)."""
    M, d = x.shape
    F = Wg.shape[0]
    px, pw = _bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d))
    out = out or Packed.empty(M, F, T, C, x.device)
    spill = spill or Spill.empty(M, F, T, cap, x.device)
    pz = ctypes.c_void_p(0)
    if z_debug is not None:
        _f32_out(z_debug, "z_debug", (M, F), x.device)
        pz = _dptr(z_debug)
    cb = _workspace(ctrl, x.device, zeroed=True)
    cp, cn = cb.get(ctrl_bytes(M))
    pk, sp = out._c(), spill._c()
    _check(lib().twell_gate_pack_spill(px, pw, M, d, F, T, C, ctypes.byref(pk), ctypes.byref(sp), pz, cp, cn,
                                       _stream(x)), "twell_gate_pack_spill")
    return out, spill


def hybrid_pack(packed: Packed, F: int, K: int, R: int, out: Hybrid | None = None,
                spill: Spill | None = None) -> Hybrid:
    """twell_hybrid_pack: the hybrid format from a packing (C == T), or from a
    packing of smaller C and the spill list of the same training gate."""
    M = packed.counts.shape[0]
    out = out or Hybrid.empty(M, F, K, R, packed.counts.device)
    pk, ph = packed._c(), out._c()
    sp = ctypes.byref(spill._c()) if spill is not None else None
    _check(lib().twell_hybrid_pack(ctypes.byref(pk), sp, M, F, packed.T, packed.C, K, R, ctypes.byref(ph),
                                   _stream(packed.counts)), "twell_hybrid_pack")
    return out


def backward_workspace_bytes(M: int, d: int, F: int, K: int, R: int) -> int:
    return int(lib().twell_backward_workspace_bytes(M, d, F, K, R))


def ffn_backward(x, Wg, WuT, Wd, dy, hy: Hybrid, workspace=None, out=None):
    """twell_ffn_backward: (dx, dWg, dWuT, dWd), fp32. out: optional tuple of
    the four output tensors to overwrite."""
    torch = _torch()
    M, d = x.shape
    F = Wg.shape[0]
    args = (_bf16(x, "x", (M, d)), _bf16(Wg, "Wg", (F, d)), _bf16(WuT, "WuT", (F, d)), _bf16(Wd, "Wd", (F, d)),
            _bf16(dy, "dy", (M, d)))
    if out is None:
        out = (torch.empty((M, d), dtype=torch.float32, device=x.device),
               *(torch.empty((F, d), dtype=torch.float32, device=x.device) for _ in range(3)))
    shapes = ((M, d), (F, d), (F, d), (F, d))
    ptrs = [_dptr(_f32_out(t, n, sh, x.device)) for t, n, sh in zip(out, ("dx", "dWg", "dWuT", "dWd"), shapes)]
    ws = _workspace(workspace, x.device)
    wp, wn = ws.get(backward_workspace_bytes(M, d, F, hy.K, hy.R))
    ph = hy._c()
    _check(lib().twell_ffn_backward(*args, ctypes.byref(ph), M, d, F, hy.K, hy.R, *ptrs, wp, wn, _stream(x)),
           "twell_ffn_backward")
    return out


def packed_view(M: int, d: int, F: int, T: int, C: int, workspace=None, device=None) -> Packed:
    """Tensor views of the packing twell_ffn_forward keeps in the workspace."""
    torch = _torch()
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    ws = _workspace(workspace, device)
    wp, wn = ws.get(workspace_bytes(OP_FFN_FORWARD, M, d, F, T, C))
    pk = _Packed()
    _check(lib().twell_packed_view(wp, wn, M, d, F, T, C, ctypes.byref(pk)), "twell_packed_view")
    base = ws.buf.data_ptr()
    nT = F // T

    def view(addr, n, dtype, shape):
        off = addr - base
        return ws.buf[off:off + n * torch.tensor([], dtype=dtype).element_size()].view(dtype).view(shape)

    return Packed(
        view(pk.vals, M * nT * C, torch.float32, (M, nT, C)),
        view(pk.idx, M * nT * C, torch.uint8, (M, nT, C)),
        view(pk.counts, M * nT, torch.int16, (M, nT)),
        view(pk.ovf_rows, M, torch.int32, (M,)),
        view(pk.n_ovf, 1, torch.int32, (1,)),
        T,
        C,
    )
