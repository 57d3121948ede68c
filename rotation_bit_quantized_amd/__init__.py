"""Python binding of libqr, the gfx950 HIP library of QuaRot's 4-bit
linear-layer hot path (include/qr.h).

Argument marshalling only: every step of the path runs in the library's
kernels.  PyTorch supplies device memory and the current HIP stream.  If the
library has not been built, importing works but every call raises
LibraryNotBuilt - there is no fallback implementation.

    rot = Rotation.hadamard(4096, signs)            # R = D H / sqrt(n)
    rot = Rotation.kronecker(64, dense, signs=None)  # R = D (H_64/8 kron O)
    codes, scales = rotate_quant(x, rot, group=0)
    y = int4_gemm(codes, scales, w_codes, w_scales, group=0)
    kc, ks, kz = kv_quant(k)                         # k [T, H, 128] or [T, H*128] view
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "QRError", "LibraryNotBuilt", "Rotation", "library", "library_path", "rotate_quant", "int4_gemm",
    "int4_gemm_i32", "kv_quant", "kv_attn_decode", "kv_attn_decode_workspace", "rotate_quant_i8",
    "int8_gemm", "int8_gemm_i32", "swiglu_rotate_quant", "status_str", "version", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqr.so")
_lib = None

QR_OK, QR_EINVAL, QR_ESHAPE, QR_EALIGN, QR_EDEVICE = 0, 1, 2, 3, 4
EXPORTS = ("qr_rotate_quant", "qr_int4_gemm", "qr_kv_quant", "qr_int4_gemm_i32", "qr_kv_attn_decode",
           "qr_kv_attn_decode_workspace", "qr_rotate_quant_i8", "qr_int8_gemm", "qr_int8_gemm_i32",
           "qr_swiglu_rotate_quant", "qr_status_str", "qr_version")


class QRError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")
        self.status = status


class LibraryNotBuilt(RuntimeError):
    pass


class _Rot(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("had_n", ctypes.c_int64), ("dense_m", ctypes.c_int64),
                ("dense", ctypes.c_void_p), ("signs", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libqr.so (raises LibraryNotBuilt when it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise LibraryNotBuilt(f"{_LIB_PATH} is missing: run `python -m rotation_bit_quantized_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, st = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.qr_rotate_quant.argtypes = [vp, i64, i64, ctypes.POINTER(_Rot), i64, vp, vp, vp]
    lib.qr_rotate_quant.restype = st
    lib.qr_int4_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp]
    lib.qr_int4_gemm.restype = st
    lib.qr_int4_gemm_i32.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp]
    lib.qr_int4_gemm_i32.restype = st
    lib.qr_kv_quant.argtypes = [vp, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.qr_kv_quant.restype = st
    lib.qr_kv_attn_decode.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_float, vp, i64, vp, vp]
    lib.qr_kv_attn_decode.restype = st
    lib.qr_kv_attn_decode_workspace.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.qr_kv_attn_decode_workspace.restype = st
    lib.qr_rotate_quant_i8.argtypes = [vp, i64, i64, ctypes.POINTER(_Rot), i64, i64, vp, vp, vp]
    lib.qr_rotate_quant_i8.restype = st
    lib.qr_int8_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp]
    lib.qr_int8_gemm.restype = st
    lib.qr_int8_gemm_i32.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp]
    lib.qr_int8_gemm_i32.restype = st
    lib.qr_swiglu_rotate_quant.argtypes = [vp, vp, i64, i64, ctypes.POINTER(_Rot), i64, vp, vp, vp]
    lib.qr_swiglu_rotate_quant.restype = st
    lib.qr_status_str.argtypes = [st]
    lib.qr_status_str.restype = ctypes.c_char_p
    lib.qr_version.argtypes = []
    lib.qr_version.restype = st
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return library().qr_status_str(int(status)).decode()


def version() -> int:
    return int(library().qr_version())


def _check(fn: str, status: int) -> None:
    if status != QR_OK:
        raise QRError(fn, status)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")


class Rotation:
    """Device-side description of R (see qr_rotation in include/qr.h)."""

    def __init__(self, n: int, had_n: int, dense=None, signs=None, device="cuda"):
        self.n, self.had_n = int(n), int(had_n)
        self.dense = None if dense is None else torch.as_tensor(dense, dtype=torch.float32).to(device).contiguous()
        self.dense_m = 1 if dense is None else int(self.dense.shape[0])
        self.signs = None if signs is None else torch.as_tensor(signs, dtype=torch.int8).to(device).contiguous()
        self._c = _Rot(self.n, self.had_n, self.dense_m, _ptr(self.dense), _ptr(self.signs))

    @classmethod
    def hadamard(cls, n: int, signs=None, device="cuda"):
        return cls(n, n, None, signs, device)

    @classmethod
    def kronecker(cls, had_n: int, dense, signs=None, device="cuda"):
        m = int(len(dense))
        return cls(had_n * m, had_n, dense, signs, device)


def rotate_quant(x: torch.Tensor, rot: Rotation, group: int = 0, codes=None, scales=None, stream=None):
    """qr_rotate_quant on the rows of x (fp16 [rows, >= n], unit column stride).
    Returns (codes uint8 [rows, n/2], scales fp32 [rows] or [rows, n/group])."""
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows = x.shape[0]
    if codes is None:
        codes = torch.empty((rows, rot.n // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows,) if group == 0 else (rows, rot.n // group), dtype=torch.float32,
                             device=x.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float32, "scales")
    ld = x.stride(0) if rows > 1 else max(x.stride(0), rot.n + (-rot.n) % 8)
    st = library().qr_rotate_quant(_ptr(x), rows, ld, ctypes.byref(rot._c), int(group), _ptr(codes),
                                   _ptr(scales), _stream(stream))
    _check("qr_rotate_quant", st)
    return codes, scales


def int4_gemm(a_codes, a_scales, w_codes, w_scales, group: int = 0, y=None, stream=None):
    """qr_int4_gemm: a_codes [M, K/2], w_codes [N, K/2] -> y fp16 [M, N]."""
    for t, dt, nm in ((a_codes, torch.uint8, "a_codes"), (w_codes, torch.uint8, "w_codes"),
                      (a_scales, torch.float32, "a_scales"), (w_scales, torch.float32, "w_scales")):
        _need(t, dt, nm)
    M, kb = a_codes.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != kb:
        raise ValueError("K mismatch between a_codes and w_codes")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=a_codes.device)
    _need(y, torch.float16, "y")
    ld = y.stride(0) if M > 1 else max(y.stride(0), N)
    st = library().qr_int4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, 2 * kb,
                                int(group), _ptr(y), ld, _stream(stream))
    _check("qr_int4_gemm", st)
    return y


def int4_gemm_i32(a_codes, w_codes, group: int = 0, acc=None, stream=None):
    """qr_int4_gemm_i32: exact integer sums, int32 [M, N] or [K/group, M, N]."""
    _need(a_codes, torch.uint8, "a_codes")
    _need(w_codes, torch.uint8, "w_codes")
    M, kb = a_codes.shape
    N = w_codes.shape[0]
    K = 2 * kb
    if acc is None:
        shape = (M, N) if group == 0 else (K // group, M, N)
        acc = torch.empty(shape, dtype=torch.int32, device=a_codes.device)
    _need(acc, torch.int32, "acc")
    st = library().qr_int4_gemm_i32(_ptr(a_codes), _ptr(w_codes), M, N, K, int(group), _ptr(acc),
                                    _stream(stream))
    _check("qr_int4_gemm_i32", st)
    return acc


def kv_quant(kv: torch.Tensor, signs=None, codes=None, scales=None, zeros=None, head_dim: int = 128,
             stream=None):
    """qr_kv_quant on kv fp16 [T, H, 128] (contiguous heads) or a 2-D view
    [T, H*128] with any row stride (e.g. the K slice of a fused QKV output).
    Returns (codes uint8 [T, H, 64], scales fp32 [T, H], zeros uint8 [T, H])."""
    _need(kv, torch.float16, "kv")
    if kv.dim() == 3:
        T, H, D = kv.shape
        if D != head_dim or kv.stride(2) != 1 or kv.stride(1) != head_dim:
            raise ValueError("kv [T, H, D] must have contiguous heads of head_dim")
        ld = kv.stride(0) if T > 1 else H * head_dim
    elif kv.dim() == 2:
        T, HD = kv.shape
        if HD % head_dim or kv.stride(1) != 1:
            raise ValueError("kv [T, H*D] must have unit column stride")
        H = HD // head_dim
        ld = kv.stride(0) if T > 1 else HD
    else:
        raise ValueError("kv must be 2-D or 3-D")
    dev = kv.device
    if codes is None:
        codes = torch.empty((T, H, head_dim // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((T, H), dtype=torch.float32, device=dev)
    if zeros is None:
        zeros = torch.empty((T, H), dtype=torch.uint8, device=dev)
    sg = None
    if signs is not None:
        sg = torch.as_tensor(signs, dtype=torch.int8).to(dev).contiguous()
    st = library().qr_kv_quant(_ptr(kv), T, H, head_dim, ld, _ptr(sg), _ptr(codes), _ptr(scales),
                               _ptr(zeros), _stream(stream))
    _check("qr_kv_quant", st)
    return codes, scales, zeros


def kv_attn_decode_workspace(B: int, Hq: int, Hkv: int, T: int, head_dim: int = 128) -> int:
    """Bytes of workspace qr_kv_attn_decode needs for this shape (host only)."""
    out = ctypes.c_int64(0)
    _check("qr_kv_attn_decode_workspace",
           library().qr_kv_attn_decode_workspace(int(B), int(Hq), int(Hkv), int(T), int(head_dim),
                                                 ctypes.byref(out)))
    return int(out.value)


def kv_attn_decode(q, k_codes, k_scales, k_zeros, v_codes, v_scales, v_zeros, lens=None, signs=None,
                   sm_scale=None, out=None, workspace=None, stream=None):
    """qr_kv_attn_decode: one decode step of attention over the rotated 4-bit
    KV cache.  q fp16 [B, Hq, 128]; k_codes/v_codes uint8 [B, T, Hkv, 64]
    (or [B*T, Hkv, 64] with B taken from q); scales fp32 and zeros uint8
    [B, T, Hkv]; lens int32 [B] or None.  A workspace of the size
    kv_attn_decode_workspace reports is allocated here when not given
    (pass workspace=False to run without one).  Returns out fp16 [B, Hq, 128]."""
    _need(q, torch.float16, "q")
    for t, dt, name in ((k_codes, torch.uint8, "k_codes"), (v_codes, torch.uint8, "v_codes"),
                        (k_scales, torch.float32, "k_scales"), (v_scales, torch.float32, "v_scales"),
                        (k_zeros, torch.uint8, "k_zeros"), (v_zeros, torch.uint8, "v_zeros")):
        _need(t, dt, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, D = q.shape
    if k_codes.dim() == 4:
        T, Hkv = k_codes.shape[1], k_codes.shape[2]
    elif k_codes.dim() == 3:
        T, Hkv = k_codes.shape[0] // max(B, 1), k_codes.shape[1]
    else:
        raise ValueError("k_codes must be [B, T, Hkv, 64] or [B*T, Hkv, 64]")
    dev = q.device
    if sm_scale is None:
        sm_scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    ln = None
    if lens is not None:
        ln = torch.as_tensor(lens, dtype=torch.int32).to(dev).contiguous()
    sg = None
    if signs is not None:
        sg = torch.as_tensor(signs, dtype=torch.int8).to(dev).contiguous()
    if workspace is False:
        ws, ws_bytes = None, 0
    else:
        if workspace is None:
            need = kv_attn_decode_workspace(B, Hq, Hkv, T, D)
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    st = library().qr_kv_attn_decode(_ptr(q), B, Hq, Hkv, T, D, _ptr(k_codes), _ptr(k_scales), _ptr(k_zeros),
                                     _ptr(v_codes), _ptr(v_scales), _ptr(v_zeros), _ptr(ln), _ptr(sg),
                                     float(sm_scale), _ptr(ws), ws_bytes, _ptr(out), _stream(stream))
    _check("qr_kv_attn_decode", st)
    return out


def rotate_quant_i8(x: torch.Tensor, rot: Rotation, bits: int, group: int = 0, codes=None, scales=None,
                    stream=None):
    """qr_rotate_quant_i8 (6- or 8-bit RTN) on the rows of x (fp16 [rows, >= n],
    unit column stride).  Returns (codes int8 [rows, n], scales fp32 [rows] or
    [rows, n/group])."""
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    rows = x.shape[0]
    if codes is None:
        codes = torch.empty((rows, rot.n), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((rows,) if group == 0 else (rows, rot.n // group), dtype=torch.float32,
                             device=x.device)
    _need(codes, torch.int8, "codes")
    _need(scales, torch.float32, "scales")
    ld = x.stride(0) if rows > 1 else max(x.stride(0), rot.n + (-rot.n) % 8)
    st = library().qr_rotate_quant_i8(_ptr(x), rows, ld, ctypes.byref(rot._c), int(group), int(bits),
                                      _ptr(codes), _ptr(scales), _stream(stream))
    _check("qr_rotate_quant_i8", st)
    return codes, scales


def int8_gemm(a_codes, a_scales, w_codes, w_scales, group: int = 0, y=None, stream=None):
    """qr_int8_gemm: a_codes int8 [M, K], w_codes int8 [N, K] -> y fp16 [M, N]."""
    for t, dt, nm in ((a_codes, torch.int8, "a_codes"), (w_codes, torch.int8, "w_codes"),
                      (a_scales, torch.float32, "a_scales"), (w_scales, torch.float32, "w_scales")):
        _need(t, dt, nm)
    M, K = a_codes.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != K:
        raise ValueError("K mismatch between a_codes and w_codes")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=a_codes.device)
    _need(y, torch.float16, "y")
    ld = y.stride(0) if M > 1 else max(y.stride(0), N)
    st = library().qr_int8_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K,
                                int(group), _ptr(y), ld, _stream(stream))
    _check("qr_int8_gemm", st)
    return y


def int8_gemm_i32(a_codes, w_codes, group: int = 0, acc=None, stream=None):
    """qr_int8_gemm_i32: exact integer sums of int8 codes, int32 [M, N] or
    [K/group, M, N]."""
    _need(a_codes, torch.int8, "a_codes")
    _need(w_codes, torch.int8, "w_codes")
    M, K = a_codes.shape
    N = w_codes.shape[0]
    if acc is None:
        shape = (M, N) if group == 0 else (K // group, M, N)
        acc = torch.empty(shape, dtype=torch.int32, device=a_codes.device)
    _need(acc, torch.int32, "acc")
    st = library().qr_int8_gemm_i32(_ptr(a_codes), _ptr(w_codes), M, N, K, int(group), _ptr(acc),
                                    _stream(stream))
    _check("qr_int8_gemm_i32", st)
    return acc


def swiglu_rotate_quant(gate: torch.Tensor, up: torch.Tensor, rot: Rotation, group: int = 0, codes=None,
                        scales=None, stream=None):
    """qr_swiglu_rotate_quant: rotate and quantize x = fp16(silu(gate) * up)
    without forming x.  gate and up fp16 [rows, >= n] with unit column stride
    and the same row stride (e.g. two column halves of one [rows, 2n] tensor).
    Returns (codes uint8 [rows, n/2], scales fp32 [rows] or [rows, n/group])."""
    _need(gate, torch.float16, "gate")
    _need(up, torch.float16, "up")
    if gate.dim() != 2 or up.dim() != 2 or gate.stride(1) != 1 or up.stride(1) != 1 or gate.shape != up.shape:
        raise ValueError("gate and up must be 2-D, equal in shape, with unit column stride")
    rows = gate.shape[0]
    ld = gate.stride(0) if rows > 1 else max(gate.stride(0), rot.n + (-rot.n) % 8)
    if rows > 1 and up.stride(0) != ld:
        raise ValueError("gate and up must share one row stride")
    if codes is None:
        codes = torch.empty((rows, rot.n // 2), dtype=torch.uint8, device=gate.device)
    if scales is None:
        scales = torch.empty((rows,) if group == 0 else (rows, rot.n // group), dtype=torch.float32,
                             device=gate.device)
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float32, "scales")
    st = library().qr_swiglu_rotate_quant(_ptr(gate), _ptr(up), rows, ld, ctypes.byref(rot._c), int(group),
                                          _ptr(codes), _ptr(scales), _stream(stream))
    _check("qr_swiglu_rotate_quant", st)
    return codes, scales
