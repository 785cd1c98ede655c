"""Online rotation + W4A4 linear for MI355X (gfx950): Python binding.

A thin ctypes layer over librq.so (the C ABI in include/rq.h).  It only
marshals arguments: torch supplies device memory and the current HIP stream,
every computation runs in the library's HIP kernels.  There is no fallback:
if librq.so is missing or a tensor is not on the GPU, the call raises.

Entry points carry the C names of every function include/rq.h declares
(EXPORTS below): the quantizer, weight prep and linear layers, the fused
decode forms, the 8-bit (QUIK-8B) path, the KV-cache quantizer and the clip
search.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librq.so")

RQ_OK, RQ_EINVAL, RQ_ESHAPE, RQ_EALIGN, RQ_EHIP = range(5)
ROT_KINDS = {"none": 0, "hadamard": 1, "gsr": 2, "kron": 3}

__all__ = ["RqError", "Rotation", "lib", "rq_rotate_quant", "rq_prepare_weights",
           "rq_w4a4_linear", "rq_mixed_outlier_linear", "rq_quant_decode_linear", "rq_kv_rotate_quant",
           "rq_kv_cache_quant", "rq_w8a8_linear", "rq_w8a8_gemm_i32", "rq_search_weight_clip", "rq_w4a4_gemm_i32",
           "rq_prepare_weights_noalloc", "rq_rotate_quant_decode_linear", "rq_status_string", "rq_last_error",
           "rq_abi_version", "EXPORTS"]

# Every symbol include/rq.h declares.
EXPORTS = ("rq_rotate_quant", "rq_prepare_weights_workspace_bytes", "rq_prepare_weights",
           "rq_w4a4_linear", "rq_mixed_outlier_linear", "rq_quant_decode_linear", "rq_kv_rotate_quant",
           "rq_kv_cache_quant", "rq_w8a8_linear", "rq_w8a8_gemm_i32", "rq_search_weight_clip", "rq_w4a4_gemm_i32",
           "rq_prepare_weights_noalloc", "rq_rotate_quant_decode_linear", "rq_status_string", "rq_last_error",
           "rq_abi_version")


class RqError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class _RotDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("block", ctypes.c_int32), ("n1", ctypes.c_int32),
                ("n2", ctypes.c_int32), ("p1", ctypes.c_void_p), ("p2", ctypes.c_void_p),
                ("chan_scale", ctypes.c_void_p)]


class _KvTensor(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("rotate", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("zero", ctypes.c_void_p)]


class _QuantDesc(ctypes.Structure):
    _fields_ = [("asymmetric", ctypes.c_int32), ("clip_ratio", ctypes.c_float),
                ("outlier_idx", ctypes.c_void_p), ("n_out", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("row_clip", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m online_rotation_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.rq_rotate_quant.argtypes = [vp, i64, i64, i64, ctypes.POINTER(_RotDesc),
                                      ctypes.POINTER(_QuantDesc), vp, vp, vp, vp, vp, vp]
        L.rq_prepare_weights_workspace_bytes.argtypes = [ctypes.POINTER(_RotDesc)]
        L.rq_prepare_weights_workspace_bytes.restype = i64
        L.rq_prepare_weights.argtypes = [vp, i64, i64, i64, ctypes.POINTER(_RotDesc),
                                         ctypes.POINTER(_QuantDesc), vp, vp, vp, vp, vp, i64, vp]
        L.rq_prepare_weights_noalloc.argtypes = [vp, i64, i64, i64, ctypes.POINTER(_RotDesc),
                                                 ctypes.POINTER(_QuantDesc), vp, vp, vp, vp, vp]
        L.rq_w4a4_linear.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i64, vp]
        L.rq_mixed_outlier_linear.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, i64, vp, vp,
                                              i32, vp, i64, vp]
        L.rq_w4a4_gemm_i32.argtypes = [vp, i32, i64, i64, vp, i64, vp, i64, vp]
        L.rq_quant_decode_linear.argtypes = [vp, i64, i64, i64, ctypes.POINTER(_QuantDesc), vp, vp,
                                             vp, i64, vp, vp, i64, vp]
        L.rq_kv_rotate_quant.argtypes = [vp, i64, i64, i64, i32, i32, vp, vp, vp, vp]
        L.rq_kv_cache_quant.argtypes = [ctypes.POINTER(_KvTensor), ctypes.POINTER(_KvTensor), i64, i64, i32, vp]
        L.rq_rotate_quant_decode_linear.argtypes = [vp, i64, i64, i64, ctypes.POINTER(_RotDesc),
                                                    ctypes.POINTER(_QuantDesc), vp, vp, vp, i64, vp, vp, i64, vp]
        L.rq_w8a8_linear.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, i64, vp, vp, i32, vp, i64, vp]
        L.rq_w8a8_gemm_i32.argtypes = [vp, i32, i64, i64, vp, vp, i64, vp, i64, vp]
        L.rq_search_weight_clip.argtypes = [vp, i64, i64, i64, ctypes.POINTER(_QuantDesc), i32, vp, vp]
        for fn in ("rq_rotate_quant", "rq_prepare_weights", "rq_prepare_weights_noalloc", "rq_w4a4_linear",
                   "rq_mixed_outlier_linear", "rq_rotate_quant_decode_linear",
                   "rq_w4a4_gemm_i32", "rq_quant_decode_linear", "rq_kv_rotate_quant", "rq_kv_cache_quant",
                   "rq_w8a8_linear",
                   "rq_w8a8_gemm_i32", "rq_search_weight_clip"):
            getattr(L, fn).restype = ctypes.c_int
        L.rq_status_string.argtypes = [ctypes.c_int]
        L.rq_status_string.restype = ctypes.c_char_p
        L.rq_last_error.restype = ctypes.c_char_p
        L.rq_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def rq_status_string(s: int) -> str:
    return lib().rq_status_string(s).decode()


def rq_last_error() -> str:
    return lib().rq_last_error().decode()


def rq_abi_version() -> int:
    return lib().rq_abi_version()


def _check(status: int, fn: str):
    if status != RQ_OK:
        raise RqError(status, fn, rq_last_error() or rq_status_string(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("rq: tensors must live on the GPU (no CPU path exists)")


def _want(t, name, dtype, shape=None, dense=True):
    """Check what the C ABI will read through t: dtype, shape, and either
    dense rows (the ABI takes no stride) or unit inner stride (it takes a
    leading dimension)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"rq: {name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"rq: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dense and not t.is_contiguous():
        raise ValueError(f"rq: {name} must be contiguous")
    if not dense and t.dim() == 2 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"rq: {name} needs unit stride along its rows")


@dataclass
class Rotation:
    """Online transform descriptor (tensors are kept alive by this object)."""
    kind: str = "none"
    block: int = 0
    p1: object = None          # fp32 [n1, n1] device tensor (kron)
    p2: object = None          # fp32 [n2, n2] device tensor (kron)
    chan_scale: object = None  # fp32 [K] device tensor or None (kron)

    def check(self, K: int):
        import torch
        if self.kind not in ROT_KINDS:
            raise ValueError(f"rq: unknown rotation kind {self.kind!r}")
        if self.kind == "kron":
            if self.p1 is None or self.p2 is None:
                raise ValueError("rq: kron needs p1 and p2")
            n1, n2 = int(self.p1.shape[0]), int(self.p2.shape[0])
            _want(self.p1, "p1", torch.float32, (n1, n1))
            _want(self.p2, "p2", torch.float32, (n2, n2))
            _want(self.chan_scale, "chan_scale", torch.float32, (K,))

    def desc(self) -> _RotDesc:
        n1 = int(self.p1.shape[0]) if self.p1 is not None else 0
        n2 = int(self.p2.shape[0]) if self.p2 is not None else 0
        return _RotDesc(ROT_KINDS[self.kind], int(self.block), n1, n2, _ptr(self.p1),
                        _ptr(self.p2), _ptr(self.chan_scale))


def _qdesc(asym: bool, clip: float, outlier_idx, bits: int = 4, row_clip=None):
    n_out = 0 if outlier_idx is None else int(outlier_idx.numel())
    return _QuantDesc(1 if asym else 0, float(clip), _ptr(outlier_idx), n_out, int(bits), _ptr(row_clip)), n_out


def rq_rotate_quant(x, rot: Rotation, clip: float = 1.0, asym: bool = False,
                    outlier_idx=None, code_sum: bool = False, out: dict | None = None,
                    bits: int = 4) -> dict:
    """x fp16 [T, K] (row stride x.stride(0)) -> dict(q, scale, zero, code_sum, x_out).
    bits = 8: one byte per code (rotation none only)."""
    import torch
    _gpu(x, outlier_idx, rot.p1, rot.p2, rot.chan_scale)
    T, K = x.shape
    _want(x, "x", torch.float16, dense=False)
    _want(outlier_idx, "outlier_idx", torch.int32)
    rot.check(K)
    qd, n_out = _qdesc(asym, clip, outlier_idx, bits)
    dev = x.device
    qb = (K - n_out) if bits == 8 else (K - n_out) // 2
    o = dict(out or {})
    o.setdefault("q", torch.empty((T, qb), dtype=torch.uint8, device=dev))
    o.setdefault("scale", torch.empty((T,), dtype=torch.float32, device=dev))
    o.setdefault("zero", torch.empty((T,), dtype=torch.int32, device=dev) if asym else None)
    o.setdefault("code_sum", torch.empty((T,), dtype=torch.int32, device=dev) if code_sum else None)
    o.setdefault("x_out", torch.empty((T, n_out), dtype=torch.float16, device=dev) if n_out else None)
    _want(o["q"], "q", torch.uint8, (T, qb))
    _want(o["scale"], "scale", torch.float32, (T,))
    _want(o["zero"], "zero", torch.int32, (T,))
    _want(o["code_sum"], "code_sum", torch.int32, (T,))
    _want(o["x_out"], "x_out", torch.float16, (T, n_out))
    _gpu(*o.values())
    rd = rot.desc()
    st = lib().rq_rotate_quant(_ptr(x), T, K, x.stride(0), ctypes.byref(rd), ctypes.byref(qd),
                               _ptr(o["q"]), _ptr(o["scale"]), _ptr(o["zero"]),
                               _ptr(o["code_sum"]), _ptr(o["x_out"]), _stream(dev))
    _check(st, "rq_rotate_quant")
    return o


def rq_prepare_weights(w, rot: Rotation, clip: float = 1.0, outlier_idx=None, bits: int = 4,
                       row_clip=None) -> dict:
    """w fp16 [N, K] -> dict(q, scale, rowsum, w_out): rotated, per-channel INT4
    (bits = 8: INT8, one byte per code, rotation none only).  row_clip: fp32
    [N] per-row clip ratios (rotation none), e.g. from rq_search_weight_clip."""
    import torch
    _gpu(w, outlier_idx, rot.p1, rot.p2, rot.chan_scale, row_clip)
    N, K = w.shape
    _want(w, "w", torch.float16, dense=False)
    _want(outlier_idx, "outlier_idx", torch.int32)
    _want(row_clip, "row_clip", torch.float32, (N,))
    rot.check(K)
    qd, n_out = _qdesc(False, clip, outlier_idx, bits, row_clip)
    dev = w.device
    rd = rot.desc()
    ws_bytes = lib().rq_prepare_weights_workspace_bytes(ctypes.byref(rd))
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev) if ws_bytes else None
    o = {"q": torch.empty((N, (K - n_out) if bits == 8 else (K - n_out) // 2), dtype=torch.uint8, device=dev),
         "scale": torch.empty((N,), dtype=torch.float32, device=dev),
         "rowsum": torch.empty((N,), dtype=torch.int32, device=dev),
         "w_out": torch.empty((N, n_out), dtype=torch.float16, device=dev) if n_out else None}
    st = lib().rq_prepare_weights(_ptr(w), N, K, w.stride(0), ctypes.byref(rd), ctypes.byref(qd),
                                  _ptr(o["q"]), _ptr(o["scale"]), _ptr(o["rowsum"]),
                                  _ptr(o["w_out"]), _ptr(ws), ws_bytes, _stream(dev))
    _check(st, "rq_prepare_weights")
    o["_workspace"] = ws   # keep alive until the stream has consumed it
    return o


def rq_prepare_weights_noalloc(w, rot: Rotation, qw, sw, rowsum, w_out=None, clip: float = 1.0,
                               outlier_idx=None, bits: int = 4, row_clip=None) -> None:
    """rq_prepare_weights into caller-given outputs, with no workspace: the
    library's per-GPU scratch array holds the KRON factors' inverses."""
    import torch
    _gpu(w, qw, sw, rowsum, w_out, outlier_idx, rot.p1, rot.p2, rot.chan_scale, row_clip)
    N, K = w.shape
    _want(w, "w", torch.float16, dense=False)
    _want(outlier_idx, "outlier_idx", torch.int32)
    _want(row_clip, "row_clip", torch.float32, (N,))
    rot.check(K)
    qd, n_out = _qdesc(False, clip, outlier_idx, bits, row_clip)
    _want(qw, "qw", torch.uint8, (N, (K - n_out) if bits == 8 else (K - n_out) // 2))
    _want(sw, "sw", torch.float32, (N,))
    _want(rowsum, "rowsum", torch.int32, (N,))
    _want(w_out, "w_out", torch.float16, (N, n_out))
    rd = rot.desc()
    st = lib().rq_prepare_weights_noalloc(_ptr(w), N, K, w.stride(0), ctypes.byref(rd), ctypes.byref(qd),
                                          _ptr(qw), _ptr(sw), _ptr(rowsum), _ptr(w_out), _stream(w.device))
    _check(st, "rq_prepare_weights_noalloc")


def rq_search_weight_clip(w, outlier_idx=None, bits: int = 4, steps: int = 100, out=None):
    """QUIK's per-channel clip ratio by linear search: w fp16 [N, K] -> fp32 [N]."""
    import torch
    _gpu(w, outlier_idx, out)
    N, K = w.shape
    _want(w, "w", torch.float16, dense=False)
    _want(outlier_idx, "outlier_idx", torch.int32)
    clip = out if out is not None else torch.empty((N,), dtype=torch.float32, device=w.device)
    _want(clip, "out", torch.float32, (N,))
    qd, _ = _qdesc(False, 1.0, outlier_idx, bits)
    st = lib().rq_search_weight_clip(_ptr(w), N, K, w.stride(0), ctypes.byref(qd), int(steps), _ptr(clip),
                                     _stream(w.device))
    _check(st, "rq_search_weight_clip")
    return clip


def rq_w4a4_linear(qx, sx, qw, sw, out=None):
    """fp16 y [T, N] = acc * sx[t] * sw[n] from packed symmetric codes."""
    import torch
    _gpu(qx, sx, qw, sw, out)
    T, Kb = qx.shape
    N = qw.shape[0]
    _want(qx, "qx", torch.uint8)
    _want(qw, "qw", torch.uint8, (N, Kb))
    _want(sx, "sx", torch.float32, (T,))
    _want(sw, "sw", torch.float32, (N,))
    y = out if out is not None else torch.empty((T, N), dtype=torch.float16, device=qx.device)
    _want(y, "out", torch.float16, (T, N), dense=False)
    st = lib().rq_w4a4_linear(_ptr(qx), _ptr(sx), T, 2 * Kb, _ptr(qw), _ptr(sw), N, _ptr(y),
                              y.stride(0), _stream(qx.device))
    _check(st, "rq_w4a4_linear")
    return y


def rq_mixed_outlier_linear(qx, sx, zx, qw, sw, w_rowsum, x_out=None, w_out=None, out=None):
    """QUIK mixed linear: dequantized INT4 part + fp16 outlier product."""
    import torch
    _gpu(qx, sx, zx, qw, sw, w_rowsum, x_out, w_out, out)
    T, Kb = qx.shape
    N = qw.shape[0]
    n_out = 0 if x_out is None else int(x_out.shape[1])
    _want(qx, "qx", torch.uint8)
    _want(qw, "qw", torch.uint8, (N, Kb))
    _want(sx, "sx", torch.float32, (T,))
    _want(zx, "zx", torch.int32, (T,))
    _want(sw, "sw", torch.float32, (N,))
    _want(w_rowsum, "w_rowsum", torch.int32, (N,))
    _want(x_out, "x_out", torch.float16, (T, n_out))
    if (x_out is None) != (w_out is None):
        raise ValueError("rq: x_out and w_out come together")
    _want(w_out, "w_out", torch.float16, (N, n_out))
    y = out if out is not None else torch.empty((T, N), dtype=torch.float16, device=qx.device)
    _want(y, "out", torch.float16, (T, N), dense=False)
    st = lib().rq_mixed_outlier_linear(_ptr(qx), _ptr(sx), _ptr(zx), T, 2 * Kb, _ptr(qw),
                                       _ptr(sw), _ptr(w_rowsum), N, _ptr(x_out), _ptr(w_out),
                                       n_out, _ptr(y), y.stride(0), _stream(qx.device))
    _check(st, "rq_mixed_outlier_linear")
    return y


def rq_quant_decode_linear(x, qw, sw, w_rowsum=None, w_out=None, asym: bool = False,
                           clip: float = 1.0, outlier_idx=None, out=None):
    """Unrotated quantizer + linear layer in one launch for T <= 16 rows:
    x fp16 [T, K] -> y fp16 [T, N], equal to rq_rotate_quant(x, none, ...)
    followed by rq_mixed_outlier_linear (asym or outliers) or rq_w4a4_linear."""
    import torch
    _gpu(x, qw, sw, w_rowsum, w_out, outlier_idx, out)
    T, K = x.shape
    N = qw.shape[0]
    _want(x, "x", torch.float16, dense=False)
    _want(outlier_idx, "outlier_idx", torch.int32)
    qd, n_out = _qdesc(asym, clip, outlier_idx)
    _want(qw, "qw", torch.uint8, (N, (K - n_out) // 2))
    _want(sw, "sw", torch.float32, (N,))
    _want(w_rowsum, "w_rowsum", torch.int32, (N,))
    _want(w_out, "w_out", torch.float16, (N, n_out))
    y = out if out is not None else torch.empty((T, N), dtype=torch.float16, device=x.device)
    _want(y, "out", torch.float16, (T, N), dense=False)
    st = lib().rq_quant_decode_linear(_ptr(x), T, K, x.stride(0), ctypes.byref(qd), _ptr(qw), _ptr(sw),
                                      _ptr(w_rowsum), N, _ptr(w_out), _ptr(y), y.stride(0),
                                      _stream(x.device))
    _check(st, "rq_quant_decode_linear")
    return y


def rq_rotate_quant_decode_linear(x, rot: Rotation, qw, sw, w_rowsum=None, w_out=None, asym: bool = False,
                                  clip: float = 1.0, outlier_idx=None, out=None):
    """rq_rotate_quant (with its online transform) + the linear layer in one
    launch for T <= 16 rows: x fp16 [T, K] -> y fp16 [T, N]."""
    import torch
    _gpu(x, qw, sw, w_rowsum, w_out, outlier_idx, out, rot.p1, rot.p2, rot.chan_scale)
    T, K = x.shape
    N = qw.shape[0]
    _want(x, "x", torch.float16, dense=False)
    _want(outlier_idx, "outlier_idx", torch.int32)
    rot.check(K)
    qd, n_out = _qdesc(asym, clip, outlier_idx)
    _want(qw, "qw", torch.uint8, (N, (K - n_out) // 2))
    _want(sw, "sw", torch.float32, (N,))
    _want(w_rowsum, "w_rowsum", torch.int32, (N,))
    _want(w_out, "w_out", torch.float16, (N, n_out))
    y = out if out is not None else torch.empty((T, N), dtype=torch.float16, device=x.device)
    _want(y, "out", torch.float16, (T, N), dense=False)
    rd = rot.desc()
    st = lib().rq_rotate_quant_decode_linear(_ptr(x), T, K, x.stride(0), ctypes.byref(rd), ctypes.byref(qd),
                                             _ptr(qw), _ptr(sw), _ptr(w_rowsum), N, _ptr(w_out), _ptr(y),
                                             y.stride(0), _stream(x.device))
    _check(st, "rq_rotate_quant_decode_linear")
    return y


def rq_kv_rotate_quant(x, group: int = 128, rotate: bool = True, out=None):
    """KV-cache quantizer: per-group normalized Walsh-Hadamard (rotate) and
    group-wise asymmetric INT4.  x fp16 [T, K] -> (q uint8 [T, K/2],
    scale fp32 [T, K/group], zero int32 [T, K/group])."""
    import torch
    _gpu(x, *(out or ()))
    T, K = x.shape
    _want(x, "x", torch.float16, dense=False)
    q, sc, zp = _kv_outputs(x, group, out, "")
    st = lib().rq_kv_rotate_quant(_ptr(x), T, K, x.stride(0), int(group), 1 if rotate else 0,
                                  _ptr(q), _ptr(sc), _ptr(zp), _stream(x.device))
    _check(st, "rq_kv_rotate_quant")
    return q, sc, zp


def _kv_outputs(x, group, out, name):
    import torch
    T, K = x.shape
    if out is None:
        G = K // group if group > 0 else 0
        out = (torch.empty((T, K // 2), dtype=torch.uint8, device=x.device),
               torch.empty((T, G), dtype=torch.float32, device=x.device),
               torch.empty((T, G), dtype=torch.int32, device=x.device))
    q, sc, zp = out
    _want(q, name + "q", torch.uint8, (T, K // 2))
    _want(sc, name + "scale", torch.float32)
    _want(zp, name + "zero", torch.int32, tuple(sc.shape))
    if group > 0 and K % group == 0 and tuple(sc.shape) != (T, K // group):
        raise ValueError(f"rq: {name}scale must have shape {(T, K // group)}")
    return out


def rq_kv_cache_quant(k, v, group: int = 128, rotate_k: bool = True, rotate_v: bool = False,
                      out_k=None, out_v=None):
    """Keys and values of the same tokens through the KV-cache quantizer in
    one launch: k, v fp16 [T, K] -> ((q, scale, zero) of k, (q, scale, zero)
    of v), each as rq_kv_rotate_quant would return it."""
    import torch
    _gpu(k, v, *(out_k or ()), *(out_v or ()))
    _want(k, "k", torch.float16, dense=False)
    _want(v, "v", torch.float16, dense=False)
    if tuple(k.shape) != tuple(v.shape):
        raise ValueError(f"rq: keys {tuple(k.shape)} and values {tuple(v.shape)} differ in shape")
    T, K = k.shape
    out_k = _kv_outputs(k, group, out_k, "keys ")
    out_v = _kv_outputs(v, group, out_v, "values ")
    dk = _KvTensor(_ptr(k), k.stride(0), 1 if rotate_k else 0, *(_ptr(t) for t in out_k))
    dv = _KvTensor(_ptr(v), v.stride(0), 1 if rotate_v else 0, *(_ptr(t) for t in out_v))
    st = lib().rq_kv_cache_quant(ctypes.byref(dk), ctypes.byref(dv), T, K, int(group), _stream(k.device))
    _check(st, "rq_kv_cache_quant")
    return out_k, out_v


def rq_w8a8_linear(qx, sx, zx, qw, sw, w_rowsum, x_out=None, w_out=None, out=None):
    """8-bit mixed linear (QUIK-8B): one-byte codes, dequantized INT8 part +
    fp16 outlier product.  zx None: signed activation codes."""
    import torch
    _gpu(qx, sx, zx, qw, sw, w_rowsum, x_out, w_out, out)
    T, K = qx.shape
    N = qw.shape[0]
    n_out = 0 if x_out is None else int(x_out.shape[1])
    _want(qx, "qx", torch.uint8)
    _want(qw, "qw", torch.uint8, (N, K))
    _want(sx, "sx", torch.float32, (T,))
    _want(zx, "zx", torch.int32, (T,))
    _want(sw, "sw", torch.float32, (N,))
    _want(w_rowsum, "w_rowsum", torch.int32, (N,))
    _want(x_out, "x_out", torch.float16, (T, n_out))
    if (x_out is None) != (w_out is None):
        raise ValueError("rq: x_out and w_out come together")
    _want(w_out, "w_out", torch.float16, (N, n_out))
    y = out if out is not None else torch.empty((T, N), dtype=torch.float16, device=qx.device)
    _want(y, "out", torch.float16, (T, N), dense=False)
    st = lib().rq_w8a8_linear(_ptr(qx), _ptr(sx), _ptr(zx), T, K, _ptr(qw), _ptr(sw), _ptr(w_rowsum), N,
                              _ptr(x_out), _ptr(w_out), n_out, _ptr(y), y.stride(0), _stream(qx.device))
    _check(st, "rq_w8a8_linear")
    return y


def rq_w8a8_gemm_i32(qx, qw, x_unsigned: bool = False, w_rowsum=None, out=None):
    """Raw INT32 accumulator [T, N] of one-byte codes (for bit-exact tests)."""
    import torch
    _gpu(qx, qw, w_rowsum, out)
    T, K = qx.shape
    N = qw.shape[0]
    _want(qx, "qx", torch.uint8)
    _want(qw, "qw", torch.uint8, (N, K))
    _want(w_rowsum, "w_rowsum", torch.int32, (N,))
    acc = out if out is not None else torch.empty((T, N), dtype=torch.int32, device=qx.device)
    _want(acc, "out", torch.int32, (T, N), dense=False)
    st = lib().rq_w8a8_gemm_i32(_ptr(qx), 1 if x_unsigned else 0, T, K, _ptr(qw), _ptr(w_rowsum), N,
                                _ptr(acc), acc.stride(0), _stream(qx.device))
    _check(st, "rq_w8a8_gemm_i32")
    return acc


def rq_w4a4_gemm_i32(qx, qw, x_unsigned: bool = False, out=None):
    """Raw INT32 accumulator [T, N] (for bit-exact tests)."""
    import torch
    _gpu(qx, qw, out)
    T, Kb = qx.shape
    N = qw.shape[0]
    _want(qx, "qx", torch.uint8)
    _want(qw, "qw", torch.uint8, (N, Kb))
    acc = out if out is not None else torch.empty((T, N), dtype=torch.int32, device=qx.device)
    _want(acc, "out", torch.int32, (T, N), dense=False)
    st = lib().rq_w4a4_gemm_i32(_ptr(qx), 1 if x_unsigned else 0, T, 2 * Kb, _ptr(qw), N,
                                _ptr(acc), acc.stride(0), _stream(qx.device))
    _check(st, "rq_w4a4_gemm_i32")
    return acc
