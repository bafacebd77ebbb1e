"""Thin ctypes binding of libqmm (include/qmm.h).

Argument marshalling only: every step of the matmul runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  If the
library has not been built this module raises on first use -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmm.so")

QMM_OK, QMM_ERR_INVALID_ARG, QMM_ERR_UNSUPPORTED = 0, -1, -2
QMM_ERR_HIP, QMM_ERR_WORKSPACE, QMM_ERR_NO_DEVICE = -3, -4, -5
QMM_F32, QMM_BF16 = 0, 1
QMM_FLAG_F32_OUT = 1
(VARIANT_AUTO, VARIANT_GEMV, VARIANT_MFMA, VARIANT_STREAM, VARIANT_RESIDENT, VARIANT_SLAB,
 VARIANT_GENERIC, VARIANT_WIDE) = (0, 1, 2, 3, 4, 5, 6, 7)
VARIANTS = {"auto": VARIANT_AUTO, "gemv": VARIANT_GEMV, "mfma": VARIANT_MFMA,
            "stream": VARIANT_STREAM, "resident": VARIANT_RESIDENT, "slab": VARIANT_SLAB,
            "generic": VARIANT_GENERIC, "wide": VARIANT_WIDE}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
_DTYPES = {"f32": QMM_F32, "bf16": QMM_BF16}

# Every entry point of include/qmm.h with its ctypes signature.
_c = ctypes
_P = _c.c_void_p
SIGNATURES = {
    "qmm_create": (_c.c_int, [_P, _P]),
    "qmm_destroy": (None, [_P]),
    "qmm_packed_bytes": (_c.c_int, [_P, _P, _P]),
    "qmm_prepack": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "qmm_workspace_bytes": (_c.c_size_t, [_P, _c.c_int32]),
    "qmm_workspace_bytes_ex": (_c.c_size_t, [_P, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32,
                                              _c.c_int32]),
    "qmm_attention_workspace_bytes": (_c.c_size_t, [_c.c_int32, _c.c_int64, _c.c_int32]),
    "qmm_decode_attention": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _c.c_int32, _c.c_int32,
                                        _c.c_int64, _c.c_int32, _c.c_int32, _c.c_int32, _P,
                                        _c.c_size_t, _P]),
    "qmm_run": (_c.c_int, [_P, _P, _P, _P, _P, _c.c_int32, _P, _c.c_size_t, _P]),
    "qmm_run_ex": (_c.c_int, [_P, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_int32, _P, _P, _P,
                              _P, _c.c_int32, _P, _c.c_size_t, _P]),
    "qmm_run_noalloc": (_c.c_int, [_P, _P, _P, _P, _P, _c.c_int32, _P]),
    "qmm_run_sums": (_c.c_int, [_P, _P, _P, _c.c_int32, _P, _P, _P, _c.c_int32, _P, _c.c_size_t,
                                _P]),
    "qmm_sum_group": (_c.c_int32, [_P]),
    "qmm_run_gate_up": (_c.c_int, [_P, _P, _P, _P, _P, _P, _P, _c.c_int32, _c.c_int32, _P]),
    "qmm_residual_rms_norm": (_c.c_int, [_P, _P, _P, _P, _P, _c.c_int32, _c.c_int64, _c.c_float,
                                         _c.c_int32, _P]),
    "qmm_residual_rms_norm_ex": (_c.c_int, [_P, _P, _P, _P, _P, _P, _c.c_int32, _c.c_int32,
                                            _c.c_int32, _c.c_int64, _c.c_float, _c.c_int32, _P]),
    "qmm_debug_unpack": (_c.c_int, [_P, _P, _P, _P]),
    "qmm_get_stats": (_c.c_int, [_P, _P]),
    "qmm_last_error": (_c.c_char_p, []),
    "qmm_hbm_probe": (_c.c_int, [_P, _c.c_size_t, _P, _c.c_int32, _P]),
}


class QmmDesc(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("max_rows", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("sb_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class QmmStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_uint64 * 8), ("last_variant", ctypes.c_int32),
                ("last_ntw", ctypes.c_int32), ("last_splitk", ctypes.c_int32),
                ("last_grid", ctypes.c_int32)]


class QmmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("qmm status %d: %s" % (status, msg))
        self.status = status


_lock = threading.Lock()
_lib = None


def lib():
    """Load libqmm.so (raises if it was not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libqmm.so is not built (run __graft_entry__.build()): " + LIB_PATH)
            # torch owns device memory and streams here: load it (and the HIP
            # runtime it ships) before the library, so that both resolve to the
            # one runtime torch brings
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def _check(status: int) -> None:
    if status != QMM_OK:
        raise QmmError(status, lib().qmm_last_error().decode())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def to_device(a: np.ndarray, device="cuda"):
    """numpy array -> torch tensor on `device`; uint16 arrays are taken as bf16
    bit patterns and come back as torch.bfloat16."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    return torch.from_numpy(a).to(device)


def to_numpy_bits(t) -> np.ndarray:
    """torch tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


class Plan:
    """One projection shape: qmm_create / qmm_destroy plus the calls on it."""

    def __init__(self, bits: int, K: int, N: int, max_rows: int, x_dtype: str = "bf16",
                 sb_dtype: str | None = None, group_size: int = 64, f32_out: bool = False):
        self.bits, self.K, self.N, self.max_rows = bits, K, N, max_rows
        self.x_dtype = x_dtype
        self.sb_dtype = sb_dtype or x_dtype
        self.f32_out = bool(f32_out)
        d = QmmDesc(bits, group_size, K, N, max_rows, _DTYPES[x_dtype],
                    _DTYPES[self.sb_dtype], QMM_FLAG_F32_OUT if f32_out else 0)
        h = ctypes.c_void_p()
        _check(lib().qmm_create(ctypes.byref(d), ctypes.byref(h)))
        self._h = h
        self._ws = {}        # (device, stream) -> zero-filled workspace
        self._retired = []   # replaced workspaces: a captured graph may still use them

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.qmm_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def packed_bytes(self):
        cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().qmm_packed_bytes(self._h, ctypes.byref(cb), ctypes.byref(sb)))
        return cb.value, sb.value

    def prepack(self, w, scales, biases, stream=None):
        """MLX-layout device tensors -> (codes, sb) native-layout tensors."""
        import torch
        cb, sbb = self.packed_bytes()
        codes = torch.empty(cb // 4, dtype=torch.int32, device=w.device)
        sb = torch.empty(sbb // (4 if self.sb_dtype == "f32" else 2),
                         dtype=torch.float32 if self.sb_dtype == "f32" else torch.bfloat16,
                         device=w.device)
        _check(lib().qmm_prepack(self._h, _ptr(w), _ptr(scales), _ptr(biases), _ptr(codes),
                                 _ptr(sb), _stream(stream)))
        return codes, sb

    def workspace_bytes(self, rows: int, variant: int = 0, ntw: int = 0, kwaves: int = 0,
                        splitk: int = 0) -> int:
        if variant or ntw or kwaves or splitk:
            return lib().qmm_workspace_bytes_ex(self._h, variant, ntw, kwaves, splitk, rows)
        return lib().qmm_workspace_bytes(self._h, rows)

    def workspace(self, nbytes: int, device, stream=None):
        """A zero-filled workspace of at least nbytes, one per (device,
        stream): calls on different streams may overlap in time, so they never
        share one.  It is zero-filled on that stream (ordered before the calls
        that use it), and a replaced, smaller one is kept alive, since a
        captured graph may still hold its address."""
        import torch
        if nbytes == 0:
            return None
        st = stream if stream is not None else torch.cuda.current_stream(device)
        key = (str(device), int(st.cuda_stream))
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            if ws is not None:
                self._retired.append(ws)
            with torch.cuda.stream(st):
                ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._ws[key] = ws
        return ws

    def run(self, x, codes, sb, out=None, variant="auto", ntw: int = 0, kwaves: int = 0,
            splitk: int = 0, stream=None, workspace=None):
        """y = x . W^T; x is [..., K] on the device, y is [..., N] in x's dtype."""
        import torch
        rows = x.numel() // self.K
        if out is None:
            out = torch.empty(*x.shape[:-1], self.N,
                              dtype=torch.float32 if self.f32_out else x.dtype, device=x.device)
        v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
        if workspace is None:
            workspace = self.workspace(self.workspace_bytes(rows, v, ntw, kwaves, splitk), x.device,
                                       stream)
        wsb = workspace.numel() if workspace is not None else 0
        _check(lib().qmm_run_ex(self._h, v, ntw, kwaves, splitk, _ptr(x), _ptr(codes), _ptr(sb),
                                _ptr(out), rows, _ptr(workspace), wsb, _stream(stream)))
        return out

    def sum_group(self) -> int:
        """Values per group of the group sums run_sums takes (qmm_sum_group)."""
        return int(lib().qmm_sum_group(self._h))

    def run_sums(self, x, x_sums, codes, sb, out=None, stream=None, workspace=None):
        """y = x . W^T through qmm_run_sums: x_sums f32 [K / sum_group(), ld]
        (ld a multiple of 16, >= rows rounded up to 16), as
        residual_rms_norm(..., group_size=sum_group()) writes them."""
        import torch
        rows = x.numel() // self.K
        if out is None:
            out = torch.empty(*x.shape[:-1], self.N,
                              dtype=torch.float32 if self.f32_out else x.dtype, device=x.device)
        if x_sums.dtype != torch.float32 or x_sums.dim() != 2 or not x_sums.is_contiguous():
            raise ValueError("x_sums must be a contiguous f32 [groups, ld] tensor")
        if x_sums.shape[0] < self.K // self.sum_group():
            raise ValueError("x_sums holds %d groups; K / sum_group() = %d"
                             % (x_sums.shape[0], self.K // self.sum_group()))
        if workspace is None:
            workspace = self.workspace(self.workspace_bytes(rows), x.device, stream)
        wsb = workspace.numel() if workspace is not None else 0
        _check(lib().qmm_run_sums(self._h, _ptr(x), _ptr(x_sums), x_sums.shape[1], _ptr(codes),
                                  _ptr(sb), _ptr(out), rows, _ptr(workspace), wsb,
                                  _stream(stream)))
        return out

    def run_noalloc(self, x, codes, sb, out=None, stream=None):
        """y = x . W^T through qmm_run_noalloc (the library's own device
        workspace; nothing is allocated by the library)."""
        import torch
        rows = x.numel() // self.K
        if out is None:
            out = torch.empty(*x.shape[:-1], self.N,
                              dtype=torch.float32 if self.f32_out else x.dtype, device=x.device)
        _check(lib().qmm_run_noalloc(self._h, _ptr(x), _ptr(codes), _ptr(sb), _ptr(out), rows,
                                     _stream(stream)))
        return out

    def run_gate_up(self, x, gate_codes, gate_sb, up_codes, up_sb, out=None, tile_pairs: int = 0,
                    stream=None):
        """h = silu(x . Wg^T) * (x . Wu^T) with bf16 roundings (qmm_run_gate_up)."""
        import torch
        rows = x.numel() // self.K
        if out is None:
            out = torch.empty(*x.shape[:-1], self.N, dtype=x.dtype, device=x.device)
        _check(lib().qmm_run_gate_up(self._h, _ptr(x), _ptr(gate_codes), _ptr(gate_sb),
                                     _ptr(up_codes), _ptr(up_sb), _ptr(out), rows, tile_pairs,
                                     _stream(stream)))
        return out

    def debug_unpack(self, codes, stream=None):
        import torch
        out = torch.empty(self.N, self.K, dtype=torch.uint8, device=codes.device)
        _check(lib().qmm_debug_unpack(self._h, _ptr(codes), _ptr(out), _stream(stream)))
        return out

    def stats(self) -> dict:
        s = QmmStats()
        _check(lib().qmm_get_stats(self._h, ctypes.byref(s)))
        return {"launches": {VARIANT_NAMES[i]: s.launches[i] for i in (1, 2, 3, 4, 5, 6, 7)},
                "last_variant": VARIANT_NAMES.get(s.last_variant, "none"),
                "last_ntw": s.last_ntw, "last_splitk": s.last_splitk, "last_grid": s.last_grid}


def residual_rms_norm(x, update, weight, eps: float, residual=None, normalized=None,
                      stream=None, group_sums=None, group_size: int = 64):
    """(residual, normalized) of qmm_residual_rms_norm for [..., D] tensors;
    with group_sums (f32 [D / group_size, ld], ld >= rows) also the sum of
    every group of group_size stored normalized values (qmm_residual_rms_norm_ex)."""
    import torch
    D = x.shape[-1]
    rows = x.numel() // D
    if update.shape != x.shape or weight.numel() != D:
        raise ValueError("update must have x's shape and weight D=%d values" % D)
    if update.dtype != x.dtype or weight.dtype != x.dtype:
        raise ValueError("x, update and weight must share one dtype")
    for t in (x, update, weight):
        if not t.is_contiguous():
            raise ValueError("x, update and weight must be contiguous")
    if residual is None:
        residual = torch.empty_like(x)
    if normalized is None:
        normalized = torch.empty_like(x)
    dt = {torch.bfloat16: QMM_BF16, torch.float32: QMM_F32}.get(x.dtype, -1)
    if group_sums is None:
        _check(lib().qmm_residual_rms_norm(_ptr(x), _ptr(update), _ptr(weight), _ptr(residual),
                                           _ptr(normalized), rows, D, float(eps), dt,
                                           _stream(stream)))
    else:
        if (group_sums.dtype != torch.float32 or group_sums.dim() != 2 or
                not group_sums.is_contiguous()):
            raise ValueError("group_sums must be a contiguous f32 [groups, ld] tensor")
        if group_size > 0 and group_sums.shape[0] < D // group_size:
            raise ValueError("group_sums holds %d groups; D / group_size = %d"
                             % (group_sums.shape[0], D // group_size))
        _check(lib().qmm_residual_rms_norm_ex(_ptr(x), _ptr(update), _ptr(weight), _ptr(residual),
                                              _ptr(normalized), _ptr(group_sums), group_size,
                                              group_sums.shape[1], rows, D, float(eps), dt,
                                              _stream(stream)))
    return residual, normalized


def decode_attention(q, k_cache, v_cache, bits: int, group_size: int, out=None,
                     workspace=None, stream=None):
    """out [H, D] of qmm_decode_attention; q bf16 [H, D]; k_cache and v_cache
    are (words int32 [KV, N, D*bits/32], scales bf16 [KV, N, D/gs], biases)."""
    import torch
    H, D = q.shape
    kw, ks, kb = k_cache
    vw, vs, vb = v_cache
    KV, N = kw.shape[0], kw.shape[1]
    for t in (q, kw, ks, kb, vw, vs, vb):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    if q.dtype != torch.bfloat16 or ks.dtype != torch.bfloat16 or vs.dtype != torch.bfloat16:
        raise ValueError("q, scales and biases must be bfloat16")
    if out is None:
        out = torch.empty_like(q)
    need = lib().qmm_attention_workspace_bytes(H, N, D)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().qmm_decode_attention(_ptr(q), _ptr(kw), _ptr(ks), _ptr(kb), _ptr(vw), _ptr(vs),
                                      _ptr(vb), _ptr(out), H, KV, N, D, bits, group_size,
                                      _ptr(workspace), wsb, _stream(stream)))
    return out


def hbm_probe(buf, grid: int = 0, stream=None):
    """Stream-read a device buffer (measurement hook)."""
    import torch
    g = grid or 4096
    sink = torch.empty(g, dtype=torch.int32, device=buf.device)
    _check(lib().qmm_hbm_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), g,
                               _stream(stream)))
    return sink


class QuantizedLinear:
    """A projection ready to run: plan + weights in the native layout."""

    def __init__(self, problem_or_shape, w=None, scales=None, biases=None, max_rows=None,
                 device="cuda", f32_out: bool = False):
        p = problem_or_shape
        self.plan = Plan(p.bits, p.K, p.N, max_rows or max(p.M, 1), p.x_dtype, p.sb_dtype,
                         group_size=getattr(p, "group_size", 64), f32_out=f32_out)
        wd = to_device(p.w if w is None else w, device)
        sd = to_device(p.scales if scales is None else scales, device)
        bd = to_device(p.biases if biases is None else biases, device)
        self.codes, self.sb = self.plan.prepack(wd, sd, bd)

    def __call__(self, x, **kw):
        return self.plan.run(x, self.codes, self.sb, **kw)
