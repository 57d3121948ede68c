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
    "peak_copy", "peak_mfma", "peak_mfma_codes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqr.so")
_lib = None

QR_OK, QR_EINVAL, QR_ESHAPE, QR_EALIGN, QR_EDEVICE, QR_ESCRATCH = 0, 1, 2, 3, 4, 5
EXPORTS = ("qr_rotate_quant", "qr_int4_gemm", "qr_kv_quant", "qr_int4_gemm_i32", "qr_kv_attn_decode",
           "qr_kv_attn_decode_workspace", "qr_kv_attn_decode_noalloc", "qr_rotate_quant_i8", "qr_int8_gemm",
           "qr_int8_gemm_i32", "qr_swiglu_rotate_quant", "qr_status_str", "qr_version",
           # measurement probes (include/qr_peaks.h)
           "qr_peak_copy", "qr_peak_mfma", "qr_peak_mfma_waves", "qr_peak_mfma_codes")


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
    lib.qr_kv_attn_decode_noalloc.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_float, vp, vp]
    lib.qr_kv_attn_decode_noalloc.restype = st
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
    lib.qr_peak_copy.argtypes = [vp, vp, i64, vp]
    lib.qr_peak_copy.restype = st
    lib.qr_peak_mfma.argtypes = [i64, i64, vp, vp]
    lib.qr_peak_mfma.restype = st
    lib.qr_peak_mfma_waves.argtypes = []
    lib.qr_peak_mfma_waves.restype = i64
    lib.qr_peak_mfma_codes.argtypes = [vp, i64, vp, i64, i64, vp, vp]
    lib.qr_peak_mfma_codes.restype = st
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


def _need(t: torch.Tensor, dtype, name: str, shape=None, contiguous: bool = False) -> None:
    """Type and layout checks of one tensor argument, before any launch: a
    wrong shape or a strided view would otherwise make a kernel read or write
    outside the tensor.  Where the tensors live is checked last, for all of a
    call's tensors at once (_on_gpu)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors) -> None:
    """Every tensor argument of a call lives on one GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _scale_shape(rows: int, n: int, group: int):
    if group < 0 or (group and n % group):
        raise ValueError(f"group {group} must be 0 or divide {n}")
    return (rows,) if group == 0 else (rows, n // group)


def _rows_view(x: torch.Tensor, n: int, name: str) -> int:
    """Row stride (elements) of a 2-D fp16 row-major view [rows, n]."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit column stride")
    if x.shape[1] != n:
        raise ValueError(f"{name} must have {n} columns, got {x.shape[1]}")
    rows = x.shape[0]
    return x.stride(0) if rows > 1 else max(x.stride(0), n + (-n) % 8)


def _check_rotation(rot) -> None:
    if not isinstance(rot, Rotation):
        raise TypeError("rot must be a Rotation")


class Rotation:
    """Device-side description of R (see qr_rotation in include/qr.h)."""

    def __init__(self, n: int, had_n: int, dense=None, signs=None, device="cuda"):
        self.n, self.had_n = int(n), int(had_n)
        self.dense = None if dense is None else torch.as_tensor(dense, dtype=torch.float32).to(device).contiguous()
        if self.dense is not None and (self.dense.dim() != 2 or self.dense.shape[0] != self.dense.shape[1]):
            raise ValueError(f"dense must be a square matrix, got shape {tuple(self.dense.shape)}")
        self.dense_m = 1 if dense is None else int(self.dense.shape[0])
        if self.had_n * self.dense_m != self.n:
            raise ValueError(f"n = {self.n} must equal had_n * dense_m = {self.had_n} * {self.dense_m}")
        self.signs = None if signs is None else torch.as_tensor(signs, dtype=torch.int8).to(device).contiguous()
        if self.signs is not None and self.signs.numel() != self.n:
            raise ValueError(f"signs must hold n = {self.n} entries, got {self.signs.numel()}")
        self._c = _Rot(self.n, self.had_n, self.dense_m, _ptr(self.dense), _ptr(self.signs))

    @classmethod
    def hadamard(cls, n: int, signs=None, device="cuda"):
        return cls(n, n, None, signs, device)

    @classmethod
    def kronecker(cls, had_n: int, dense, signs=None, device="cuda"):
        m = int(len(dense))
        return cls(had_n * m, had_n, dense, signs, device)


def rotate_quant(x: torch.Tensor, rot: Rotation, group: int = 0, codes=None, scales=None, stream=None):
    """qr_rotate_quant on the rows of x (fp16 [rows, n], unit column stride,
    any row stride that is a multiple of 8).  Returns (codes uint8
    [rows, n/2], scales fp32 [rows] or [rows, n/group])."""
    _need(x, torch.float16, "x")
    _check_rotation(rot)
    ld = _rows_view(x, rot.n, "x")
    rows = x.shape[0]
    sshape = _scale_shape(rows, rot.n, group)
    if codes is None:
        codes = torch.empty((rows, rot.n // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _need(codes, torch.uint8, "codes", (rows, rot.n // 2), True)
    _need(scales, torch.float32, "scales", sshape, True)
    _on_gpu(x=x, codes=codes, scales=scales, signs=rot.signs, dense=rot.dense)
    st = library().qr_rotate_quant(_ptr(x), rows, ld, ctypes.byref(rot._c), int(group), _ptr(codes),
                                   _ptr(scales), _stream(stream))
    _check("qr_rotate_quant", st)
    return codes, scales


def _gemm_operands(a_codes, a_scales, w_codes, w_scales, group, dtype, per_byte):
    """Shape checks shared by the GEMM wrappers; returns (M, N, K)."""
    _need(a_codes, dtype, "a_codes")
    _need(w_codes, dtype, "w_codes")
    if a_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("a_codes and w_codes must be 2-D")
    M, kb = a_codes.shape
    N = w_codes.shape[0]
    if w_codes.shape[1] != kb:
        raise ValueError("K mismatch between a_codes and w_codes")
    if not a_codes.is_contiguous() or not w_codes.is_contiguous():
        raise ValueError("a_codes and w_codes must be contiguous (row stride = K codes)")
    K = kb * per_byte
    if a_scales is not None:
        _need(a_scales, torch.float32, "a_scales", contiguous=True)
        _need(w_scales, torch.float32, "w_scales", contiguous=True)
        G = 1 if group == 0 else (K // group if group > 0 and K % group == 0 else -1)
        if G < 0:
            raise ValueError(f"group {group} must be 0 or divide K = {K}")
        if a_scales.numel() != M * G or w_scales.numel() != N * G:
            raise ValueError(f"scales must hold {M}*{G} and {N}*{G} values, got {a_scales.numel()} "
                             f"and {w_scales.numel()}")
    return M, N, K


def _gemm_out(y, M, N, dev):
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
    _need(y, torch.float16, "y", (M, N))
    if y.dim() != 2 or (M > 0 and N > 1 and y.stride(1) != 1):
        raise ValueError("y must be 2-D with unit column stride")
    ld = y.stride(0) if M > 1 else max(y.stride(0), N)
    return y, ld


def _acc_out(acc, M, N, K, group, dev):
    shape = (M, N) if group == 0 else (K // group, M, N)
    if acc is None:
        acc = torch.empty(shape, dtype=torch.int32, device=dev)
    _need(acc, torch.int32, "acc", shape, True)
    return acc


def int4_gemm(a_codes, a_scales, w_codes, w_scales, group: int = 0, y=None, stream=None):
    """qr_int4_gemm: a_codes [M, K/2], w_codes [N, K/2] -> y fp16 [M, N]."""
    M, N, K = _gemm_operands(a_codes, a_scales, w_codes, w_scales, group, torch.uint8, 2)
    y, ld = _gemm_out(y, M, N, a_codes.device)
    _on_gpu(a_codes=a_codes, a_scales=a_scales, w_codes=w_codes, w_scales=w_scales, y=y)
    st = library().qr_int4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K,
                                int(group), _ptr(y), ld, _stream(stream))
    _check("qr_int4_gemm", st)
    return y


def int4_gemm_i32(a_codes, w_codes, group: int = 0, acc=None, stream=None):
    """qr_int4_gemm_i32: exact integer sums, int32 [M, N] or [K/group, M, N]."""
    M, N, K = _gemm_operands(a_codes, None, w_codes, None, group, torch.uint8, 2)
    acc = _acc_out(acc, M, N, K, group, a_codes.device)
    _on_gpu(a_codes=a_codes, w_codes=w_codes, acc=acc)
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
        if D != head_dim or kv.stride(2) != 1 or (H > 1 and kv.stride(1) != head_dim):
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
    _need(codes, torch.uint8, "codes", contiguous=True)
    _need(scales, torch.float32, "scales", contiguous=True)
    _need(zeros, torch.uint8, "zeros", contiguous=True)
    if codes.numel() != T * H * (head_dim // 2) or scales.numel() != T * H or zeros.numel() != T * H:
        raise ValueError(f"codes, scales and zeros must hold {T}*{H}*{head_dim // 2}, {T}*{H} and {T}*{H} values")
    sg = None
    if signs is not None:
        sg = torch.as_tensor(signs, dtype=torch.int8).to(dev).contiguous()
        if sg.numel() != head_dim:
            raise ValueError(f"signs must hold head_dim = {head_dim} entries")
    _on_gpu(kv=kv, codes=codes, scales=scales, zeros=zeros, signs=sg)
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
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, D = q.shape
    dev = q.device
    if k_codes.dim() == 4:
        T, Hkv = k_codes.shape[1], k_codes.shape[2]
        if k_codes.shape[0] != B:
            raise ValueError("k_codes [B, T, Hkv, 64] must match the batch of q")
    elif k_codes.dim() == 3:
        T, Hkv = k_codes.shape[0] // max(B, 1), k_codes.shape[1]
        if k_codes.shape[0] != B * T:
            raise ValueError("k_codes [B*T, Hkv, 64] must hold B whole sequences")
    else:
        raise ValueError("k_codes must be [B, T, Hkv, 64] or [B*T, Hkv, 64]")
    if k_codes.shape[-1] != D // 2:
        raise ValueError(f"k_codes must have {D // 2} code bytes per head")
    for t, dt, name, numel in ((k_codes, torch.uint8, "k_codes", B * T * Hkv * (D // 2)),
                               (v_codes, torch.uint8, "v_codes", B * T * Hkv * (D // 2)),
                               (k_scales, torch.float32, "k_scales", B * T * Hkv),
                               (v_scales, torch.float32, "v_scales", B * T * Hkv),
                               (k_zeros, torch.uint8, "k_zeros", B * T * Hkv),
                               (v_zeros, torch.uint8, "v_zeros", B * T * Hkv)):
        _need(t, dt, name, contiguous=True)
        if t.numel() != numel:
            raise ValueError(f"{name} must hold {numel} values, got {t.numel()}")
    if sm_scale is None:
        sm_scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    _need(out, torch.float16, "out", (B, Hq, D), True)
    ln = None
    if lens is not None:
        ln = torch.as_tensor(lens, dtype=torch.int32).to(dev).contiguous()
        if ln.numel() != B:
            raise ValueError(f"lens must hold B = {B} lengths")
    sg = None
    if signs is not None:
        sg = torch.as_tensor(signs, dtype=torch.int8).to(dev).contiguous()
        if sg.numel() != D:
            raise ValueError(f"signs must hold head_dim = {D} entries")
    if workspace is False:
        ws, ws_bytes = None, 0
    else:
        if workspace is None:
            need = kv_attn_decode_workspace(B, Hq, Hkv, T, D)
            workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
        _need(workspace, workspace.dtype, "workspace", contiguous=True)
        ws, ws_bytes = workspace, workspace.numel() * workspace.element_size()
    _on_gpu(q=q, k_codes=k_codes, k_scales=k_scales, k_zeros=k_zeros, v_codes=v_codes, v_scales=v_scales,
            v_zeros=v_zeros, out=out, lens=ln, signs=sg, workspace=ws)
    st = library().qr_kv_attn_decode(_ptr(q), B, Hq, Hkv, T, D, _ptr(k_codes), _ptr(k_scales), _ptr(k_zeros),
                                     _ptr(v_codes), _ptr(v_scales), _ptr(v_zeros), _ptr(ln), _ptr(sg),
                                     float(sm_scale), _ptr(ws), ws_bytes, _ptr(out), _stream(stream))
    _check("qr_kv_attn_decode", st)
    return out


def rotate_quant_i8(x: torch.Tensor, rot: Rotation, bits: int, group: int = 0, codes=None, scales=None,
                    stream=None):
    """qr_rotate_quant_i8 (6- or 8-bit RTN) on the rows of x (fp16 [rows, n],
    unit column stride).  Returns (codes int8 [rows, n], scales fp32 [rows] or
    [rows, n/group])."""
    _need(x, torch.float16, "x")
    _check_rotation(rot)
    ld = _rows_view(x, rot.n, "x")
    rows = x.shape[0]
    sshape = _scale_shape(rows, rot.n, group)
    if codes is None:
        codes = torch.empty((rows, rot.n), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _need(codes, torch.int8, "codes", (rows, rot.n), True)
    _need(scales, torch.float32, "scales", sshape, True)
    _on_gpu(x=x, codes=codes, scales=scales, signs=rot.signs, dense=rot.dense)
    st = library().qr_rotate_quant_i8(_ptr(x), rows, ld, ctypes.byref(rot._c), int(group), int(bits),
                                      _ptr(codes), _ptr(scales), _stream(stream))
    _check("qr_rotate_quant_i8", st)
    return codes, scales


def int8_gemm(a_codes, a_scales, w_codes, w_scales, group: int = 0, y=None, stream=None):
    """qr_int8_gemm: a_codes int8 [M, K], w_codes int8 [N, K] -> y fp16 [M, N]."""
    M, N, K = _gemm_operands(a_codes, a_scales, w_codes, w_scales, group, torch.int8, 1)
    y, ld = _gemm_out(y, M, N, a_codes.device)
    _on_gpu(a_codes=a_codes, a_scales=a_scales, w_codes=w_codes, w_scales=w_scales, y=y)
    st = library().qr_int8_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales), M, N, K,
                                int(group), _ptr(y), ld, _stream(stream))
    _check("qr_int8_gemm", st)
    return y


def int8_gemm_i32(a_codes, w_codes, group: int = 0, acc=None, stream=None):
    """qr_int8_gemm_i32: exact integer sums of int8 codes, int32 [M, N] or
    [K/group, M, N]."""
    M, N, K = _gemm_operands(a_codes, None, w_codes, None, group, torch.int8, 1)
    acc = _acc_out(acc, M, N, K, group, a_codes.device)
    _on_gpu(a_codes=a_codes, w_codes=w_codes, acc=acc)
    st = library().qr_int8_gemm_i32(_ptr(a_codes), _ptr(w_codes), M, N, K, int(group), _ptr(acc),
                                    _stream(stream))
    _check("qr_int8_gemm_i32", st)
    return acc


def swiglu_rotate_quant(gate: torch.Tensor, up: torch.Tensor, rot: Rotation, group: int = 0, codes=None,
                        scales=None, stream=None):
    """qr_swiglu_rotate_quant: rotate and quantize x = fp16(silu(gate) * up)
    without forming x.  gate and up fp16 [rows, n] with unit column stride
    and the same row stride (e.g. two column halves of one [rows, 2n] tensor).
    Returns (codes uint8 [rows, n/2], scales fp32 [rows] or [rows, n/group])."""
    _need(gate, torch.float16, "gate")
    _need(up, torch.float16, "up", tuple(gate.shape))
    _check_rotation(rot)
    ld = _rows_view(gate, rot.n, "gate")
    ld_up = _rows_view(up, rot.n, "up")
    rows = gate.shape[0]
    if rows > 1 and ld_up != ld:
        raise ValueError("gate and up must share one row stride")
    sshape = _scale_shape(rows, rot.n, group)
    if codes is None:
        codes = torch.empty((rows, rot.n // 2), dtype=torch.uint8, device=gate.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=gate.device)
    _need(codes, torch.uint8, "codes", (rows, rot.n // 2), True)
    _need(scales, torch.float32, "scales", sshape, True)
    _on_gpu(gate=gate, up=up, codes=codes, scales=scales, signs=rot.signs, dense=rot.dense)
    st = library().qr_swiglu_rotate_quant(_ptr(gate), _ptr(up), rows, ld, ctypes.byref(rot._c), int(group),
                                          _ptr(codes), _ptr(scales), _stream(stream))
    _check("qr_swiglu_rotate_quant", st)
    return codes, scales


# ---- measurement probes (include/qr_peaks.h): attainable copy and MFMA rates

def peak_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """qr_peak_copy: stream src into dst (equal byte sizes, contiguous, GPU)."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_contiguous() and dst.is_contiguous()) or dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must be contiguous and of equal byte size")
    _on_gpu(src=src, dst=dst)
    _check("qr_peak_copy", library().qr_peak_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def peak_mfma(kind: int, iters: int, out=None, stream=None):
    """qr_peak_mfma: kind 0 = int8 32x32x32, 1 = fp16 16x16x32, 2 = fp16
    32x32x16, 3 = int8 16x16x64.  Returns (out, ops per call)."""
    waves = int(library().qr_peak_mfma_waves())
    if out is None:
        out = torch.empty((waves * 64,), dtype=torch.int32, device="cuda")
    _need(out, torch.int32, "out", (waves * 64,), True)
    _on_gpu(out=out)
    _check("qr_peak_mfma", library().qr_peak_mfma(int(kind), int(iters), _ptr(out), _stream(stream)))
    per = {0: 65536, 1: 16384, 2: 32768, 3: 32768}[int(kind)]
    return out, waves * int(iters) * 4 * per


def peak_mfma_codes(a_codes: torch.Tensor, w_codes: torch.Tensor, iters: int, out=None, stream=None):
    """qr_peak_mfma_codes: the int8 32x32x32 MFMA loop on operands widened from
    the packed int4 codes a_codes (A side) and w_codes (W side), contiguous
    uint8 GPU tensors of a multiple of 16 bytes.  Returns (out, ops per call)."""
    waves = int(library().qr_peak_mfma_waves())
    for name, t in (("a_codes", a_codes), ("w_codes", w_codes)):
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 tensor")
    if out is None:
        out = torch.empty((waves * 64,), dtype=torch.int32, device="cuda")
    _need(out, torch.int32, "out", (waves * 64,), True)
    _on_gpu(a_codes=a_codes, w_codes=w_codes, out=out)
    _check("qr_peak_mfma_codes", library().qr_peak_mfma_codes(
        _ptr(a_codes), a_codes.numel(), _ptr(w_codes), w_codes.numel(), int(iters), _ptr(out), _stream(stream)))
    return out, waves * int(iters) * 32 * 65536
