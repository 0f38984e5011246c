"""Tensor-level entry points over the C ABI (same names as the exported calls).

Each function checks its torch tensors (device, dtype, shape, contiguity),
allocates outputs and the workspace with torch (device memory only), and
enqueues the library call on torch's current HIP stream. All computation
happens in the library's gfx950 kernels.

Shapes (row-major): X [m][k], NF4 weight [n][k] (codes uint8 [n][k/2],
absmax float32 [n][k/64]), LoRA A [r][k], B [n][r]; MLP: X [m][d],
gate/up [h][d], down [d][h], A_gate/A_up [r][d], B_gate/B_up [h][r],
A_down [r][h], B_down [d][r]. bf16 everywhere except U/T (fp32) and absmax.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib

_WS = {}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace(nbytes: int, device) -> torch.Tensor:
    """A cached uint8 device buffer of at least nbytes (256-byte aligned by torch)."""
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


@dataclasses.dataclass
class AbsmaxDQ:
    """Double-quantized absmax of nb = n*k/64 blocks: q int8 [nb], scale and
    offset float32 [ceil(nb/256)]."""
    q: torch.Tensor
    scale: torch.Tensor
    offset: torch.Tensor

    def to(self, device):
        return AbsmaxDQ(self.q.to(device), self.scale.to(device), self.offset.to(device))


@dataclasses.dataclass
class NF4Weight:
    """NF4 weight of shape [n][k]: codes uint8 [n][k/2] and either absmax
    float32 [n][k/64] or its double-quantized form `dq` (absmax None)."""
    codes: torch.Tensor
    absmax: Optional[torch.Tensor]
    dq: Optional[AbsmaxDQ] = None

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1] * 2

    def c_struct(self) -> _lib.Nf4:
        _need(self.codes, "codes", torch.uint8, (self.n, self.k // 2))
        if self.absmax is not None:
            _need(self.absmax, "absmax", torch.float32, (self.n, self.k // 64))
            return _lib.Nf4(self.codes.data_ptr(), self.absmax.data_ptr(), self.n, self.k)
        if self.dq is None:
            raise ValueError("NF4Weight needs absmax or its double-quantized form")
        nb = self.n * (self.k // 64)
        ng = (nb + 255) // 256
        _need(self.dq.q, "dq.q", torch.int8, (nb,))
        _need(self.dq.scale, "dq.scale", torch.float32, (ng,))
        _need(self.dq.offset, "dq.offset", torch.float32, (ng,))
        return _lib.Nf4(self.codes.data_ptr(), None, self.n, self.k, self.dq.q.data_ptr(),
                        self.dq.scale.data_ptr(), self.dq.offset.data_ptr())

    def to(self, device):
        return NF4Weight(self.codes.to(device), None if self.absmax is None else self.absmax.to(device),
                         None if self.dq is None else self.dq.to(device))


def absmax_dq_quantize(absmax: torch.Tensor) -> AbsmaxDQ:
    """Double quantization of an fp32 absmax array (read flattened)."""
    if absmax.dtype != torch.float32 or not absmax.is_contiguous():
        raise ValueError("absmax must be a contiguous float32 tensor")
    nb = absmax.numel()
    ng = (nb + 255) // 256
    dev = absmax.device
    out = AbsmaxDQ(torch.empty(nb, dtype=torch.int8, device=dev),
                   torch.empty(ng, dtype=torch.float32, device=dev),
                   torch.empty(ng, dtype=torch.float32, device=dev))
    _lib.check(_lib.lib().qlora_absmax_dq_quantize(_ptr(absmax), nb, _ptr(out.q), _ptr(out.scale),
                                                   _ptr(out.offset), _stream()),
               "qlora_absmax_dq_quantize")
    return out


def absmax_dq_dequant(dq: AbsmaxDQ) -> torch.Tensor:
    """The reconstructed fp32 absmax [nb] of a double-quantized array."""
    nb = dq.q.numel()
    out = torch.empty(nb, dtype=torch.float32, device=dq.q.device)
    _lib.check(_lib.lib().qlora_absmax_dq_dequant(_ptr(dq.q), _ptr(dq.scale), _ptr(dq.offset), nb,
                                                  _ptr(out), _stream()),
               "qlora_absmax_dq_dequant")
    return out


def nf4_double_quantize(w: NF4Weight) -> NF4Weight:
    """The same weight with its absmax double-quantized (absmax dropped)."""
    return NF4Weight(w.codes, None, absmax_dq_quantize(w.absmax))


def version() -> str:
    return _lib.lib().qlora_version().decode()


def trace_enable(on: bool = True) -> None:
    """Start (clearing old records) or stop timing every base-GEMM launch."""
    _lib.check(_lib.lib().qlora_trace_enable(1 if on else 0), "qlora_trace_enable")


def trace_read():
    """(launches, total GPU ms, total algorithmic FLOPs) of the recorded GEMMs."""
    n, ms, fl = _lib.c_i64(0), ctypes.c_double(0), ctypes.c_double(0)
    _lib.check(_lib.lib().qlora_trace_read(ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl)),
               "qlora_trace_read")
    return n.value, ms.value, fl.value


def probe_mfma_peak(iters: int = 20000):
    """(sustained dense bf16 MFMA TFLOP/s, shader clock GHz) of the current GPU."""
    tf, ghz = ctypes.c_double(0), ctypes.c_double(0)
    _lib.check(_lib.lib().qlora_probe_mfma_peak(int(iters), ctypes.byref(tf), ctypes.byref(ghz), _stream()),
               "qlora_probe_mfma_peak")
    return tf.value, ghz.value


def nf4_levels() -> torch.Tensor:
    buf = (ctypes.c_float * 16)()
    _lib.lib().qlora_nf4_levels(buf)
    return torch.tensor(list(buf), dtype=torch.float32)


def gemm_split_count(m: int, n: int, k: int) -> int:
    """K splits of a store-epilogue base GEMM [m][n] of depth k on a bf16 B operand."""
    return int(_lib.lib().qlora_gemm_split_count(m, n, k))


def nf4_dequant(w: NF4Weight) -> torch.Tensor:
    out = torch.empty((w.n, w.k), dtype=torch.bfloat16, device=w.codes.device)
    _lib.check(_lib.lib().qlora_nf4_dequant(w.c_struct(), _ptr(out), _stream()), "qlora_nf4_dequant")
    return out


def nf4_quantize(W: torch.Tensor, out: Optional[NF4Weight] = None) -> NF4Weight:
    """bf16 W [n][k] (k % 64 == 0) -> NF4Weight (codes, absmax) on W's device
    (written into `out` if given)."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    n, k = W.shape
    _need(W, "W", torch.bfloat16, (n, k))
    if out is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=W.device)
        absmax = torch.empty((n, k // 64), dtype=torch.float32, device=W.device)
    else:
        codes, absmax = out.codes, out.absmax
        _need(codes, "codes", torch.uint8, (n, k // 2))
        _need(absmax, "absmax", torch.float32, (n, k // 64))
    _lib.check(_lib.lib().qlora_nf4_quantize(_ptr(W), n, k, _ptr(codes), _ptr(absmax), _stream()),
               "qlora_nf4_quantize")
    return NF4Weight(codes, absmax)


# ------------------------------------------------------------- linear layer --
def linear_workspace_bytes(m, k, n, r, mode="auto") -> int:
    return int(_lib.lib().qlora_linear_workspace_bytes(m, k, n, r, _lib.MODE[mode]))


def linear_fwd(X, w: NF4Weight, A, B, s: float, mode="auto", ws=None):
    """Returns (Y [m][n] bf16, U [m][r] fp32)."""
    m, k, n, r = X.shape[0], w.k, w.n, A.shape[0]
    _need(X, "X", torch.bfloat16, (m, k))
    _need(A, "A", torch.bfloat16, (r, k))
    _need(B, "B", torch.bfloat16, (n, r))
    Y = torch.empty((m, n), dtype=torch.bfloat16, device=X.device)
    U = torch.empty((m, r), dtype=torch.float32, device=X.device)
    nb = linear_workspace_bytes(m, k, n, r, mode)
    ws = workspace(nb, X.device) if ws is None else ws
    st = _lib.lib().qlora_linear_fwd(_ptr(X), m, w.c_struct(), _ptr(A), _ptr(B), r, float(s),
                                     _ptr(Y), _ptr(U), _lib.MODE[mode], _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_linear_fwd")
    return Y, U


def linear_fwd_noalloc(X, w: NF4Weight, A, B, s: float, mode="auto", out=None):
    """The linear forward on the library's own per-device scratch (no
    workspace, nothing allocated by the call itself). out: optional (Y, U)
    to write into; returns (Y [m][n] bf16, U [m][r] fp32)."""
    m, k, n, r = X.shape[0], w.k, w.n, A.shape[0]
    _need(X, "X", torch.bfloat16, (m, k))
    _need(A, "A", torch.bfloat16, (r, k))
    _need(B, "B", torch.bfloat16, (n, r))
    if out is None:
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=X.device)
        U = torch.empty((m, r), dtype=torch.float32, device=X.device)
    else:
        Y, U = out
        _need(Y, "Y", torch.bfloat16, (m, n))
        _need(U, "U", torch.float32, (m, r))
    st = _lib.lib().qlora_linear_fwd_noalloc(_ptr(X), m, w.c_struct(), _ptr(A), _ptr(B), r, float(s),
                                             _ptr(Y), _ptr(U), _lib.MODE[mode], _stream())
    if st == -3:
        raise RuntimeError("qlora_linear_fwd_noalloc: " + _lib.lib().qlora_last_error().decode())
    _lib.check(st, "qlora_linear_fwd_noalloc")
    return Y, U


def linear_fwd_noalloc_max_bytes() -> int:
    return int(_lib.lib().qlora_linear_fwd_noalloc_max_bytes())


def linear_bwd(dY, X, U, w: NF4Weight, A, B, s: float, need_dx=True, mode="auto", ws=None):
    """Returns (dX [m][k] or None, dA [r][k], dB [n][r]), all bf16."""
    m, k, n, r = X.shape[0], w.k, w.n, A.shape[0]
    _need(dY, "dY", torch.bfloat16, (m, n))
    _need(X, "X", torch.bfloat16, (m, k))
    _need(U, "U", torch.float32, (m, r))
    _need(A, "A", torch.bfloat16, (r, k))
    _need(B, "B", torch.bfloat16, (n, r))
    dX = torch.empty((m, k), dtype=torch.bfloat16, device=X.device) if need_dx else None
    dA = torch.empty((r, k), dtype=torch.bfloat16, device=X.device)
    dB = torch.empty((n, r), dtype=torch.bfloat16, device=X.device)
    nb = linear_workspace_bytes(m, k, n, r, mode)
    ws = workspace(nb, X.device) if ws is None else ws
    st = _lib.lib().qlora_linear_bwd(_ptr(dY), _ptr(X), _ptr(U), m, w.c_struct(), _ptr(A), _ptr(B),
                                     r, float(s), _ptr(dX), _ptr(dA), _ptr(dB), _lib.MODE[mode],
                                     _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_linear_bwd")
    return dX, dA, dB


# ---------------------------------------------------------------- gated MLP --
@dataclasses.dataclass
class MlpWeights:
    gate: NF4Weight
    up: NF4Weight
    down: NF4Weight
    a_gate: torch.Tensor
    b_gate: torch.Tensor
    a_up: torch.Tensor
    b_up: torch.Tensor
    a_down: torch.Tensor
    b_down: torch.Tensor
    s: float
    act: str = "swiglu"

    @property
    def d(self):
        return self.gate.k

    @property
    def h(self):
        return self.gate.n

    @property
    def r(self):
        return self.a_gate.shape[0]

    def c_struct(self) -> _lib.MlpWeights:
        d, h, r = self.d, self.h, self.r
        for name, t, shape in (("a_gate", self.a_gate, (r, d)), ("a_up", self.a_up, (r, d)),
                               ("a_down", self.a_down, (r, h)), ("b_gate", self.b_gate, (h, r)),
                               ("b_up", self.b_up, (h, r)), ("b_down", self.b_down, (d, r))):
            _need(t, name, torch.bfloat16, shape)
        return _lib.MlpWeights(self.gate.c_struct(), self.up.c_struct(), self.down.c_struct(),
                               self.a_gate.data_ptr(), self.b_gate.data_ptr(), self.a_up.data_ptr(),
                               self.b_up.data_ptr(), self.a_down.data_ptr(), self.b_down.data_ptr(),
                               d, h, r, float(self.s), _lib.ACT[self.act])


def mlp_workspace_bytes(m, d, h, r, mode="auto") -> int:
    return int(_lib.lib().qlora_mlp_workspace_bytes(m, d, h, r, _lib.MODE[mode]))


def mlp_fwd(X, w: MlpWeights, mode="auto", ws=None):
    """Returns (Y [m][d] bf16, saved) with saved = dict(g, u, Ug, Uu, Ud)."""
    m, d, h, r = X.shape[0], w.d, w.h, w.r
    _need(X, "X", torch.bfloat16, (m, d))
    dev = X.device
    Y = torch.empty((m, d), dtype=torch.bfloat16, device=dev)
    saved = dict(g=torch.empty((m, h), dtype=torch.bfloat16, device=dev),
                 u=torch.empty((m, h), dtype=torch.bfloat16, device=dev),
                 Ug=torch.empty((m, r), dtype=torch.float32, device=dev),
                 Uu=torch.empty((m, r), dtype=torch.float32, device=dev),
                 Ud=torch.empty((m, r), dtype=torch.float32, device=dev))
    nb = mlp_workspace_bytes(m, d, h, r, mode)
    ws = workspace(nb, dev) if ws is None else ws
    cw = w.c_struct()
    st = _lib.lib().qlora_mlp_fwd(_ptr(X), m, ctypes.byref(cw), _ptr(Y), _ptr(saved["g"]),
                                  _ptr(saved["u"]), _ptr(saved["Ug"]), _ptr(saved["Uu"]),
                                  _ptr(saved["Ud"]), _lib.MODE[mode], _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_mlp_fwd")
    return Y, saved


def mlp_bwd(dY, X, saved, w: MlpWeights, need_dx=True, mode="auto", ws=None):
    """Returns dict(dX, dAg, dBg, dAu, dBu, dAd, dBd), all bf16."""
    m, d, h, r = X.shape[0], w.d, w.h, w.r
    _need(dY, "dY", torch.bfloat16, (m, d))
    _need(X, "X", torch.bfloat16, (m, d))
    for k_, sh, dt in (("g", (m, h), torch.bfloat16), ("u", (m, h), torch.bfloat16),
                       ("Ug", (m, r), torch.float32), ("Uu", (m, r), torch.float32),
                       ("Ud", (m, r), torch.float32)):
        _need(saved[k_], k_, dt, sh)
    dev = X.device
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    out = dict(dX=e(m, d) if need_dx else None, dAg=e(r, d), dBg=e(h, r), dAu=e(r, d),
               dBu=e(h, r), dAd=e(r, h), dBd=e(d, r))
    grads = _lib.MlpGrads(out["dAg"].data_ptr(), out["dBg"].data_ptr(), out["dAu"].data_ptr(),
                          out["dBu"].data_ptr(), out["dAd"].data_ptr(), out["dBd"].data_ptr())
    nb = mlp_workspace_bytes(m, d, h, r, mode)
    ws = workspace(nb, dev) if ws is None else ws
    cw = w.c_struct()
    st = _lib.lib().qlora_mlp_bwd(_ptr(dY), _ptr(X), _ptr(saved["g"]), _ptr(saved["u"]),
                                  _ptr(saved["Ug"]), _ptr(saved["Uu"]), _ptr(saved["Ud"]), m,
                                  ctypes.byref(cw), _ptr(out["dX"]), ctypes.byref(grads),
                                  _lib.MODE[mode], _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_mlp_bwd")
    return out


# ------------------------------------------------------ 16-bit base weights --
def linear16_workspace_bytes(m, k, n, r) -> int:
    return int(_lib.lib().qlora_linear16_workspace_bytes(m, k, n, r))


def linear16_fwd(X, W, A, B, s: float, ws=None):
    """bf16 base weight W [n][k]. Returns (Y [m][n] bf16, U [m][r] fp32)."""
    m, k, n, r = X.shape[0], W.shape[1], W.shape[0], A.shape[0]
    _need(X, "X", torch.bfloat16, (m, k))
    _need(W, "W", torch.bfloat16, (n, k))
    _need(A, "A", torch.bfloat16, (r, k))
    _need(B, "B", torch.bfloat16, (n, r))
    Y = torch.empty((m, n), dtype=torch.bfloat16, device=X.device)
    U = torch.empty((m, r), dtype=torch.float32, device=X.device)
    nb = linear16_workspace_bytes(m, k, n, r)
    ws = workspace(nb, X.device) if ws is None else ws
    st = _lib.lib().qlora_linear16_fwd(_ptr(X), m, _ptr(W), n, k, _ptr(A), _ptr(B), r, float(s),
                                       _ptr(Y), _ptr(U), _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_linear16_fwd")
    return Y, U


def linear16_bwd(dY, X, U, W, A, B, s: float, need_dx=True, ws=None):
    """Returns (dX [m][k] or None, dA [r][k], dB [n][r]), all bf16."""
    m, k, n, r = X.shape[0], W.shape[1], W.shape[0], A.shape[0]
    _need(dY, "dY", torch.bfloat16, (m, n))
    _need(X, "X", torch.bfloat16, (m, k))
    _need(U, "U", torch.float32, (m, r))
    _need(W, "W", torch.bfloat16, (n, k))
    _need(A, "A", torch.bfloat16, (r, k))
    _need(B, "B", torch.bfloat16, (n, r))
    dX = torch.empty((m, k), dtype=torch.bfloat16, device=X.device) if need_dx else None
    dA = torch.empty((r, k), dtype=torch.bfloat16, device=X.device)
    dB = torch.empty((n, r), dtype=torch.bfloat16, device=X.device)
    nb = linear16_workspace_bytes(m, k, n, r)
    ws = workspace(nb, X.device) if ws is None else ws
    st = _lib.lib().qlora_linear16_bwd(_ptr(dY), _ptr(X), _ptr(U), m, _ptr(W), n, k, _ptr(A),
                                       _ptr(B), r, float(s), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws),
                                       ws.numel(), _stream())
    _lib.check(st, "qlora_linear16_bwd")
    return dX, dA, dB


@dataclasses.dataclass
class Mlp16Weights:
    """Gated MLP with bf16 base weights: gate, up [h][d], down [d][h]."""
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    a_gate: torch.Tensor
    b_gate: torch.Tensor
    a_up: torch.Tensor
    b_up: torch.Tensor
    a_down: torch.Tensor
    b_down: torch.Tensor
    s: float
    act: str = "swiglu"

    @property
    def d(self):
        return self.gate.shape[1]

    @property
    def h(self):
        return self.gate.shape[0]

    @property
    def r(self):
        return self.a_gate.shape[0]

    def c_struct(self) -> _lib.Mlp16Weights:
        d, h, r = self.d, self.h, self.r
        for name, t, shape in (("gate", self.gate, (h, d)), ("up", self.up, (h, d)),
                               ("down", self.down, (d, h)),
                               ("a_gate", self.a_gate, (r, d)), ("a_up", self.a_up, (r, d)),
                               ("a_down", self.a_down, (r, h)), ("b_gate", self.b_gate, (h, r)),
                               ("b_up", self.b_up, (h, r)), ("b_down", self.b_down, (d, r))):
            _need(t, name, torch.bfloat16, shape)
        return _lib.Mlp16Weights(self.gate.data_ptr(), self.up.data_ptr(), self.down.data_ptr(),
                                 self.a_gate.data_ptr(), self.b_gate.data_ptr(), self.a_up.data_ptr(),
                                 self.b_up.data_ptr(), self.a_down.data_ptr(), self.b_down.data_ptr(),
                                 d, h, r, float(self.s), _lib.ACT[self.act])


def mlp16_workspace_bytes(m, d, h, r) -> int:
    return int(_lib.lib().qlora_mlp16_workspace_bytes(m, d, h, r))


def mlp16_fwd(X, w: Mlp16Weights, ws=None):
    """Returns (Y [m][d] bf16, saved) with saved = dict(g, u, Ug, Uu, Ud)."""
    m, d, h, r = X.shape[0], w.d, w.h, w.r
    _need(X, "X", torch.bfloat16, (m, d))
    dev = X.device
    Y = torch.empty((m, d), dtype=torch.bfloat16, device=dev)
    saved = dict(g=torch.empty((m, h), dtype=torch.bfloat16, device=dev),
                 u=torch.empty((m, h), dtype=torch.bfloat16, device=dev),
                 Ug=torch.empty((m, r), dtype=torch.float32, device=dev),
                 Uu=torch.empty((m, r), dtype=torch.float32, device=dev),
                 Ud=torch.empty((m, r), dtype=torch.float32, device=dev))
    nb = mlp16_workspace_bytes(m, d, h, r)
    ws = workspace(nb, dev) if ws is None else ws
    cw = w.c_struct()
    st = _lib.lib().qlora_mlp16_fwd(_ptr(X), m, ctypes.byref(cw), _ptr(Y), _ptr(saved["g"]),
                                    _ptr(saved["u"]), _ptr(saved["Ug"]), _ptr(saved["Uu"]),
                                    _ptr(saved["Ud"]), _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_mlp16_fwd")
    return Y, saved


def mlp16_bwd(dY, X, saved, w: Mlp16Weights, need_dx=True, ws=None):
    """Returns dict(dX, dAg, dBg, dAu, dBu, dAd, dBd), all bf16."""
    m, d, h, r = X.shape[0], w.d, w.h, w.r
    _need(dY, "dY", torch.bfloat16, (m, d))
    _need(X, "X", torch.bfloat16, (m, d))
    for k_, sh, dt in (("g", (m, h), torch.bfloat16), ("u", (m, h), torch.bfloat16),
                       ("Ug", (m, r), torch.float32), ("Uu", (m, r), torch.float32),
                       ("Ud", (m, r), torch.float32)):
        _need(saved[k_], k_, dt, sh)
    dev = X.device
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    out = dict(dX=e(m, d) if need_dx else None, dAg=e(r, d), dBg=e(h, r), dAu=e(r, d),
               dBu=e(h, r), dAd=e(r, h), dBd=e(d, r))
    grads = _lib.MlpGrads(out["dAg"].data_ptr(), out["dBg"].data_ptr(), out["dAu"].data_ptr(),
                          out["dBu"].data_ptr(), out["dAd"].data_ptr(), out["dBd"].data_ptr())
    nb = mlp16_workspace_bytes(m, d, h, r)
    ws = workspace(nb, dev) if ws is None else ws
    cw = w.c_struct()
    st = _lib.lib().qlora_mlp16_bwd(_ptr(dY), _ptr(X), _ptr(saved["g"]), _ptr(saved["u"]),
                                    _ptr(saved["Ug"]), _ptr(saved["Uu"]), _ptr(saved["Ud"]), m,
                                    ctypes.byref(cw), _ptr(out["dX"]), ctypes.byref(grads),
                                    _ptr(ws), ws.numel(), _stream())
    _lib.check(st, "qlora_mlp16_bwd")
    return out


# ---------------------------------------------- q, k, v on one shared input --
def _need_rows(t: torch.Tensor, name: str, shape):
    """A bf16 [rows][cols] tensor whose rows may be strided (a column slice of
    a wider buffer); returns its row pitch in elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a bf16 GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if shape[0] > 1 else max(t.stride(0), shape[1])


@dataclasses.dataclass
class QkvWeights:
    """q, k, v projections of one input: NF4 base weights W_p [n_p][d],
    LoRA A_p [r][d], B_p [n_p][r]."""
    q: NF4Weight
    k: NF4Weight
    v: NF4Weight
    a_q: torch.Tensor
    b_q: torch.Tensor
    a_k: torch.Tensor
    b_k: torch.Tensor
    a_v: torch.Tensor
    b_v: torch.Tensor
    s: float

    @property
    def d(self):
        return self.q.k

    @property
    def ns(self):
        return (self.q.n, self.k.n, self.v.n)

    @property
    def r(self):
        return self.a_q.shape[0]

    def _lora_check(self):
        d, r = self.d, self.r
        for name, t, shape in (("a_q", self.a_q, (r, d)), ("a_k", self.a_k, (r, d)),
                               ("a_v", self.a_v, (r, d)), ("b_q", self.b_q, (self.ns[0], r)),
                               ("b_k", self.b_k, (self.ns[1], r)), ("b_v", self.b_v, (self.ns[2], r))):
            _need(t, name, torch.bfloat16, shape)
        return [t.data_ptr() for t in (self.a_q, self.b_q, self.a_k, self.b_k, self.a_v, self.b_v)]

    def c_struct(self):
        return _lib.QkvWeights(self.q.c_struct(), self.k.c_struct(), self.v.c_struct(),
                               *self._lora_check(), self.r, float(self.s))


@dataclasses.dataclass
class Qkv16Weights(QkvWeights):
    """The same with bf16 base weights q, k, v [n_p][d] (16-bit LoRA)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor

    @property
    def d(self):
        return self.q.shape[1]

    @property
    def ns(self):
        return (self.q.shape[0], self.k.shape[0], self.v.shape[0])

    def c_struct(self):
        d = self.d
        for name, t, n in (("q", self.q, self.ns[0]), ("k", self.k, self.ns[1]),
                           ("v", self.v, self.ns[2])):
            _need(t, name, torch.bfloat16, (n, d))
        return _lib.Qkv16Weights(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), d,
                                 *self.ns, *self._lora_check(), self.r, float(self.s))


def qkv_workspace_bytes(m, d, n_q, n_k, n_v, r) -> int:
    return int(_lib.lib().qlora_qkv_workspace_bytes(m, d, n_q, n_k, n_v, r))


def _qkv_fwd(fn, X, w, out, ws):
    m, d, r, ns = X.shape[0], w.d, w.r, w.ns
    _need(X, "X", torch.bfloat16, (m, d))
    dev = X.device
    if out is None:
        out = tuple(torch.empty((m, n), dtype=torch.bfloat16, device=dev) for n in ns)
    lds = [_need_rows(t, nm, (m, n)) for t, nm, n in zip(out, ("Q", "K", "V"), ns)]
    U = torch.empty((m, 3 * r), dtype=torch.float32, device=dev)
    nb = qkv_workspace_bytes(m, d, *ns, r)
    ws = workspace(nb, dev) if ws is None else ws
    cw = w.c_struct()
    st = getattr(_lib.lib(), fn)(_ptr(X), m, ctypes.byref(cw), _ptr(out[0]), lds[0], _ptr(out[1]),
                                 lds[1], _ptr(out[2]), lds[2], _ptr(U), _ptr(ws), ws.numel(),
                                 _stream())
    _lib.check(st, fn)
    return out[0], out[1], out[2], U


def _qkv_bwd(fn, dQ, dK, dV, X, U, w, need_dx, ws):
    m, d, r, ns = X.shape[0], w.d, w.r, w.ns
    _need(X, "X", torch.bfloat16, (m, d))
    _need(U, "U", torch.float32, (m, 3 * r))
    lds = [_need_rows(t, nm, (m, n)) for t, nm, n in zip((dQ, dK, dV), ("dQ", "dK", "dV"), ns)]
    dev = X.device
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)  # noqa: E731
    out = dict(dX=e(m, d) if need_dx else None, dAq=e(r, d), dBq=e(ns[0], r), dAk=e(r, d),
               dBk=e(ns[1], r), dAv=e(r, d), dBv=e(ns[2], r))
    grads = _lib.QkvGrads(*[out[k].data_ptr() for k in ("dAq", "dBq", "dAk", "dBk", "dAv", "dBv")])
    nb = qkv_workspace_bytes(m, d, *ns, r)
    ws = workspace(nb, dev) if ws is None else ws
    cw = w.c_struct()
    st = getattr(_lib.lib(), fn)(_ptr(dQ), lds[0], _ptr(dK), lds[1], _ptr(dV), lds[2], _ptr(X),
                                 _ptr(U), m, ctypes.byref(cw), _ptr(out["dX"]),
                                 ctypes.byref(grads), _ptr(ws), ws.numel(), _stream())
    _lib.check(st, fn)
    return out


def qkv_fwd(X, w: QkvWeights, out=None, ws=None):
    """Returns (Q, K, V, U): Q/K/V bf16 [m][n_p] (into `out`, three tensors
    that may be column slices of one buffer, if given), U fp32 [m][3r]."""
    return _qkv_fwd("qlora_qkv_fwd", X, w, out, ws)


def qkv_bwd(dQ, dK, dV, X, U, w: QkvWeights, need_dx=True, ws=None):
    """Returns dict(dX, dAq, dBq, dAk, dBk, dAv, dBv), all bf16."""
    return _qkv_bwd("qlora_qkv_bwd", dQ, dK, dV, X, U, w, need_dx, ws)


def qkv16_fwd(X, w: Qkv16Weights, out=None, ws=None):
    return _qkv_fwd("qlora_qkv16_fwd", X, w, out, ws)


def qkv16_bwd(dQ, dK, dV, X, U, w: Qkv16Weights, need_dx=True, ws=None):
    return _qkv_bwd("qlora_qkv16_bwd", dQ, dK, dV, X, U, w, need_dx, ws)


# -------------------------------------------- RMS layernorm, RoPE, cross entropy --
def rmsnorm_fwd(X, w, eps: float, gemma: bool = False):
    """Returns (Y [m][d] bf16, rstd [m] fp32); Gemma scales by 1 + w."""
    m, d = X.shape
    _need(X, "X", torch.bfloat16, (m, d))
    _need(w, "w", torch.bfloat16, (d,))
    Y = torch.empty_like(X)
    rstd = torch.empty((m,), dtype=torch.float32, device=X.device)
    _lib.check(_lib.lib().qlora_rmsnorm_fwd(_ptr(X), m, d, _ptr(w), float(eps), int(gemma), _ptr(Y),
                                            _ptr(rstd), _stream()), "qlora_rmsnorm_fwd")
    return Y, rstd


def rmsnorm_bwd(dY, X, rstd, w, gemma: bool = False):
    """dX [m][d] bf16 of the RMS layernorm (the norm weight is frozen)."""
    m, d = X.shape
    _need(dY, "dY", torch.bfloat16, (m, d))
    _need(X, "X", torch.bfloat16, (m, d))
    _need(rstd, "rstd", torch.float32, (m,))
    _need(w, "w", torch.bfloat16, (d,))
    dX = torch.empty_like(X)
    _lib.check(_lib.lib().qlora_rmsnorm_bwd(_ptr(dY), _ptr(X), _ptr(rstd), m, d, _ptr(w), int(gemma),
                                            _ptr(dX), _stream()), "qlora_rmsnorm_bwd")
    return dX


def _heads_view(t, name):
    """A bf16 [m][heads][head_dim] tensor whose rows may be strided; returns its row pitch."""
    if not isinstance(t, torch.Tensor) or t.dim() != 3 or t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise ValueError(f"{name} must be a bf16 GPU tensor [m][heads][head_dim]")
    m, h, hd = t.shape
    if t.stride(2) != 1 or t.stride(1) != hd:
        raise ValueError(f"{name}: heads must be dense within a row")
    return t.stride(0) if m > 1 else max(t.stride(0), h * hd)


def _rope(fn, X, pos, base, out, inplace):
    m, heads, hd = X.shape
    ldx = _heads_view(X, "X")
    _need(pos, "pos", torch.int64, (m,))
    Y = X if inplace else (torch.empty_like(X) if out is None else out)
    ldy = _heads_view(Y, "out")
    _lib.check(getattr(_lib.lib(), fn)(_ptr(X), ldx, m, heads, hd, _ptr(pos), float(base), _ptr(Y), ldy,
                                       _stream()), fn)
    return Y


def rope_fwd(X, pos, base: float = 10000.0, out=None, inplace=False):
    """RoPE of X [m][heads][head_dim] at positions pos [m] (int64)."""
    return _rope("qlora_rope_fwd", X, pos, base, out, inplace)


def rope_bwd(dY, pos, base: float = 10000.0, out=None, inplace=False):
    """Transposed rotation: dX from dY [m][heads][head_dim]."""
    return _rope("qlora_rope_bwd", dY, pos, base, out, inplace)


def _logit_rows(t, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise ValueError(f"{name} must be a bf16 GPU tensor [m][V]")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def cross_entropy_fwd(logits, labels):
    """Returns dict(loss [1] fp32, n_valid [1] int32, lse [m] fp32, ce [m] fp32); labels
    int64 [m], a label outside [0, V) (e.g. -100) marks a row without a target."""
    m, V = logits.shape
    ld = _logit_rows(logits, "logits")
    _need(labels, "labels", torch.int64, (m,))
    dev = logits.device
    out = dict(loss=torch.empty((1,), dtype=torch.float32, device=dev),
               n_valid=torch.empty((1,), dtype=torch.int32, device=dev),
               lse=torch.empty((m,), dtype=torch.float32, device=dev),
               ce=torch.empty((m,), dtype=torch.float32, device=dev))
    _lib.check(_lib.lib().qlora_cross_entropy_fwd(_ptr(logits), ld, m, V, _ptr(labels), _ptr(out["lse"]),
                                                  _ptr(out["ce"]), _ptr(out["loss"]), _ptr(out["n_valid"]),
                                                  _stream()), "qlora_cross_entropy_fwd")
    return out


def cross_entropy_bwd(logits, labels, fwd, dloss=None, inplace=False):
    """dlogits [m][V] bf16 of the mean loss; dloss: optional fp32 device scalar."""
    m, V = logits.shape
    ld = _logit_rows(logits, "logits")
    _need(labels, "labels", torch.int64, (m,))
    _need(fwd["lse"], "lse", torch.float32, (m,))
    _need(fwd["n_valid"], "n_valid", torch.int32, (1,))
    if dloss is not None:
        _need(dloss, "dloss", torch.float32, (1,))
    if inplace:
        dX = logits
    else:   # rows padded to a multiple of 8 elements (16 bytes)
        dX = torch.empty((m, (V + 7) // 8 * 8), dtype=torch.bfloat16, device=logits.device)[:, :V]
    ldd = _logit_rows(dX, "dlogits")
    _lib.check(_lib.lib().qlora_cross_entropy_bwd(_ptr(logits), ld, m, V, _ptr(labels), _ptr(fwd["lse"]),
                                                  _ptr(dloss), _ptr(fwd["n_valid"]), _ptr(dX), ldd,
                                                  _stream()), "qlora_cross_entropy_bwd")
    return dX


def cross_entropy_fused(logits, labels, dloss: float = 1.0, inplace=False):
    """Forward and backward in one call (dloss known up front): the outputs of
    cross_entropy_fwd plus "dlogits" for the mean loss scaled by dloss."""
    m, V = logits.shape
    ld = _logit_rows(logits, "logits")
    _need(labels, "labels", torch.int64, (m,))
    dev = logits.device
    out = dict(loss=torch.empty((1,), dtype=torch.float32, device=dev),
               n_valid=torch.empty((1,), dtype=torch.int32, device=dev),
               lse=torch.empty((m,), dtype=torch.float32, device=dev),
               ce=torch.empty((m,), dtype=torch.float32, device=dev))
    if inplace:
        dX = logits
    else:
        dX = torch.empty((m, (V + 7) // 8 * 8), dtype=torch.bfloat16, device=dev)[:, :V]
    ldd = _logit_rows(dX, "dlogits")
    _lib.check(_lib.lib().qlora_cross_entropy_fused(_ptr(logits), ld, m, V, _ptr(labels), float(dloss),
                                                    _ptr(out["lse"]), _ptr(out["ce"]), _ptr(out["loss"]),
                                                    _ptr(out["n_valid"]), _ptr(dX), ldd, _stream()),
               "qlora_cross_entropy_fused")
    out["dlogits"] = dX
    return out
