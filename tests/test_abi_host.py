"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/qr.h declares, and
reject bad arguments on the host with the documented status before anything
is launched (these calls never reach the device, so they run on the CPU).
"""
import ctypes
import os
import re

import pytest

import rotation_bit_quantized_amd as qr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("qr.h", "qr_peaks.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(qr.library_path()), reason="libqr.so not built")


def declared_functions():
    src = "".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qr_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(qr.EXPORTS)
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(os.path.basename(h) for h in HEADERS)


def test_peak_probes_reject_bad_arguments():
    lib = qr.library()
    assert lib.qr_peak_copy(A16, A16, 100, None) == qr.QR_ESHAPE
    assert lib.qr_peak_copy(MIS, A16, 1024, None) == qr.QR_EALIGN
    assert lib.qr_peak_copy(None, A16, 1024, None) == qr.QR_EINVAL
    assert lib.qr_peak_copy(None, None, 0, None) == qr.QR_OK
    assert lib.qr_peak_mfma(4, 10, A16, None) == qr.QR_EINVAL
    assert lib.qr_peak_mfma(-1, 10, A16, None) == qr.QR_EINVAL
    assert lib.qr_peak_mfma(0, 0, A16, None) == qr.QR_ESHAPE
    assert lib.qr_peak_mfma(0, 10, None, None) == qr.QR_EINVAL
    assert lib.qr_peak_mfma_codes(None, 16, A16, 16, 10, A16, None) == qr.QR_EINVAL
    assert lib.qr_peak_mfma_codes(A16, 16, A16, 16, 10, None, None) == qr.QR_EINVAL
    assert lib.qr_peak_mfma_codes(A16, 24, A16, 16, 10, A16, None) == qr.QR_ESHAPE
    assert lib.qr_peak_mfma_codes(A16, 16, A16, 0, 10, A16, None) == qr.QR_ESHAPE
    assert lib.qr_peak_mfma_codes(A16, 16, A16, 16, 0, A16, None) == qr.QR_ESHAPE
    assert lib.qr_peak_mfma_codes(A16, 16, A16, 16, (1 << 24) + 1, A16, None) == qr.QR_ESHAPE
    assert lib.qr_peak_mfma_codes(MIS, 16, A16, 16, 10, A16, None) == qr.QR_EALIGN


def test_library_exports_every_declared_symbol():
    lib = qr.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {qr.library_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings_and_version():
    for s in range(6):
        assert qr.status_str(s)
    assert qr.status_str(99) == "unknown status"
    assert qr.version() >= 100


def rot(n=4096, had=4096, m=1, dense=None, signs=None):
    return qr._Rot(n, had, m, dense, signs)


A16 = 0x10000      # a fake, 16-byte-aligned device address: never dereferenced, the calls below fail validation
MIS = 0x10001


@pytest.mark.parametrize("args,expect", [
    (dict(x=None), qr.QR_EINVAL),
    (dict(rows=-1), qr.QR_EINVAL),
    (dict(ld=4095), qr.QR_ESHAPE),
    (dict(ld=4100), qr.QR_EALIGN),
    (dict(group=100), qr.QR_ESHAPE),
    (dict(group=16), qr.QR_ESHAPE),
    (dict(group=8192), qr.QR_ESHAPE),
    (dict(x=MIS), qr.QR_EALIGN),
    (dict(codes=MIS), qr.QR_EALIGN),
    (dict(r=rot(n=4096, had=2048)), qr.QR_ESHAPE),
    (dict(r=rot(n=12, had=12)), qr.QR_ESHAPE),
    (dict(r=rot(n=65536, had=65536)), qr.QR_ESHAPE),                    # wider than 32768
    (dict(r=rot(n=32768, had=1024, m=32, dense=A16)), qr.QR_ESHAPE),     # > 16384 needs dense_m <= 16
    (dict(r=rot(n=64 * 172, had=64, m=172, dense=None)), qr.QR_EINVAL),
    (dict(r=rot(n=4096, had=4096, m=1, dense=A16)), qr.QR_EINVAL),
    (dict(r=rot(n=3, had=1, m=3, dense=A16)), qr.QR_ESHAPE),
    (dict(r=None), qr.QR_EINVAL),
    (dict(r=rot(signs=MIS)), qr.QR_EALIGN),
])
def test_rotate_quant_rejects(args, expect):
    lib = qr.library()
    r = args.get("r", rot())
    rp = None if r is None else ctypes.byref(r)
    st = lib.qr_rotate_quant(args.get("x", A16), args.get("rows", 4), args.get("ld", 4096), rp,
                             args.get("group", 0), args.get("codes", A16), args.get("scales", A16), None)
    assert st == expect


def test_rotate_quant_zero_rows_is_noop():
    assert qr.library().qr_rotate_quant(None, 0, 4096, ctypes.byref(rot()), 0, None, None, None) == qr.QR_OK


@pytest.mark.parametrize("args,expect", [
    (dict(K=4000), qr.QR_ESHAPE),
    (dict(K=0), qr.QR_EINVAL),
    (dict(M=-1), qr.QR_EINVAL),
    (dict(group=64), qr.QR_ESHAPE),
    (dict(group=384), qr.QR_ESHAPE),
    (dict(a=None), qr.QR_EINVAL),
    (dict(a=MIS), qr.QR_EALIGN),
    (dict(ld=100), qr.QR_ESHAPE),
    (dict(y=None), qr.QR_EINVAL),
])
def test_gemm_rejects(args, expect):
    lib = qr.library()
    st = lib.qr_int4_gemm(args.get("a", A16), A16, A16, A16, args.get("M", 128), 256, args.get("K", 4096),
                          args.get("group", 0), args.get("y", A16), args.get("ld", 256), None)
    assert st == expect


def test_gemm_empty_is_noop():
    lib = qr.library()
    assert lib.qr_int4_gemm(None, None, None, None, 0, 256, 4096, 0, None, 256, None) == qr.QR_OK
    assert lib.qr_int4_gemm_i32(None, None, 5, 0, 4096, 0, None, None) == qr.QR_OK


def test_gemm_i32_rejects():
    lib = qr.library()
    assert lib.qr_int4_gemm_i32(A16, A16, 4, 4, 4096, 0, None, None) == qr.QR_EINVAL
    assert lib.qr_int4_gemm_i32(A16, A16, 4, 4, 4096, 0, MIS + 1, None) == qr.QR_EALIGN
    assert lib.qr_int4_gemm_i32(A16, A16, 4, 4, 4097, 0, A16, None) == qr.QR_ESHAPE


@pytest.mark.parametrize("args,expect", [
    (dict(D=64), qr.QR_ESHAPE),
    (dict(T=-1), qr.QR_EINVAL),
    (dict(ld=4000), qr.QR_ESHAPE),
    (dict(ld=4100), qr.QR_EALIGN),
    (dict(kv=MIS), qr.QR_EALIGN),
    (dict(kv=None), qr.QR_EINVAL),
    (dict(zeros=None), qr.QR_EINVAL),
    (dict(signs=MIS), qr.QR_EALIGN),
])
def test_kv_rejects(args, expect):
    lib = qr.library()
    st = lib.qr_kv_quant(args.get("kv", A16), args.get("T", 4), 32, args.get("D", 128), args.get("ld", 4096),
                         args.get("signs", None), A16, A16, args.get("zeros", A16), None)
    assert st == expect


def test_kv_empty_is_noop():
    assert qr.library().qr_kv_quant(None, 0, 32, 128, 4096, None, None, None, None, None) == qr.QR_OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 4096, dtype=torch.float16)
    with pytest.raises(ValueError, match="live on the GPU"):
        qr.rotate_quant(x, qr.Rotation.hadamard(4096, device="cpu"))


def _attn(lib, **a):
    f32 = ctypes.c_float
    return lib.qr_kv_attn_decode(a.get("q", A16), a.get("B", 1), a.get("Hq", 32), a.get("Hkv", 32),
                                 a.get("T", 4096), a.get("D", 128), a.get("kc", A16), A16, A16,
                                 a.get("vc", A16), A16, a.get("vz", A16), a.get("lens", None), None,
                                 f32(a.get("sm", 0.088)), a.get("ws", None), a.get("wsb", 0),
                                 a.get("out", A16), None)


@pytest.mark.parametrize("args,expect", [
    (dict(D=64), qr.QR_ESHAPE),
    (dict(Hkv=3), qr.QR_ESHAPE),
    (dict(Hkv=0), qr.QR_ESHAPE),
    (dict(B=-1), qr.QR_EINVAL),
    (dict(T=-5), qr.QR_EINVAL),
    (dict(q=None), qr.QR_EINVAL),
    (dict(out=None), qr.QR_EINVAL),
    (dict(vz=None), qr.QR_EINVAL),
    (dict(kc=MIS), qr.QR_EALIGN),
    (dict(vc=MIS), qr.QR_EALIGN),
    (dict(lens=MIS), qr.QR_EALIGN),
    (dict(sm=float("nan")), qr.QR_EINVAL),
    (dict(ws=A16, wsb=16), qr.QR_EINVAL),        # a workspace smaller than the split needs
    (dict(ws=None, wsb=1 << 20), qr.QR_EINVAL),  # a size without a buffer
    (dict(ws=MIS, wsb=1 << 30), qr.QR_EALIGN),
    (dict(wsb=-1), qr.QR_EINVAL),
    (dict(T=1 << 25, Hq=1, Hkv=1), qr.QR_ESHAPE),   # one sequence's codes past 2^31 bytes
    (dict(T=1 << 21), qr.QR_ESHAPE),
])
def test_attn_rejects(args, expect):
    assert _attn(qr.library(), **args) == expect


def test_attn_empty_batch_is_noop():
    assert _attn(qr.library(), B=0, q=None, out=None, kc=None, vc=None) == qr.QR_OK
    assert _attn(qr.library(), Hq=0, Hkv=0, q=None, out=None) == qr.QR_OK


def test_attn_workspace_size():
    """A sequence is split into chunks of at least 64 tokens so that the
    blocks fill whole rounds of the 768 that are resident at once; each
    chunk leaves a partial of 132 floats per query head.  One query per head
    over 4096 tokens: 4 blocks of eight KV heads -> 64 chunks.  64 sequences
    x 2048 tokens, 32 heads: 256 blocks -> 3 chunks (one round of 768).
    With 8 query heads per KV head: 512 (sequence, KV head) blocks -> 3
    chunks (two rounds).  64 tokens or fewer are never split."""
    assert qr.kv_attn_decode_workspace(1, 32, 32, 4096) == 32 * 64 * 132 * 4
    assert qr.kv_attn_decode_workspace(64, 32, 32, 2048) == 64 * 32 * 3 * 132 * 4
    assert qr.kv_attn_decode_workspace(64, 64, 8, 2048) == 64 * 64 * 3 * 132 * 4
    assert qr.kv_attn_decode_workspace(4, 32, 32, 64) == 0
    with pytest.raises(qr.QRError):
        qr.kv_attn_decode_workspace(1, 32, 32, 4096, head_dim=64)
    with pytest.raises(qr.QRError):
        qr.kv_attn_decode_workspace(1, 32, 5, 4096)
    out = ctypes.c_int64(0)
    assert qr.library().qr_kv_attn_decode_workspace(1, 32, 32, -1, 128, ctypes.byref(out)) == qr.QR_EINVAL
    assert qr.library().qr_kv_attn_decode_workspace(1, 32, 32, 1, 128, None) == qr.QR_EINVAL


def test_i8_rejects():
    lib = qr.library()
    rot = qr._Rot(4096, 4096, 1, None, None)
    args = lambda bits=8, codes=A16: (A16, 4, 4096, ctypes.byref(rot), 0, bits, codes, A16, None)
    assert lib.qr_rotate_quant_i8(*args(bits=5)) == qr.QR_EINVAL
    assert lib.qr_rotate_quant_i8(*args(bits=4)) == qr.QR_EINVAL
    assert lib.qr_rotate_quant_i8(*args(codes=MIS)) == qr.QR_EALIGN
    assert lib.qr_rotate_quant_i8(*args(codes=None)) == qr.QR_EINVAL
    assert lib.qr_rotate_quant_i8(A16, 0, 4096, ctypes.byref(rot), 0, 8, None, None, None) == qr.QR_OK
    gemm = lambda M=128, N=128, K=512, g=0, a=A16: lib.qr_int8_gemm(a, A16, A16, A16, M, N, K, g, A16, N, None)
    assert gemm(K=500) == qr.QR_ESHAPE
    assert gemm(K=(1 << 17) + 128) == qr.QR_ESHAPE        # int32 sums would not stay exact
    assert gemm(g=64) == qr.QR_ESHAPE
    assert gemm(a=MIS) == qr.QR_EALIGN
    assert gemm(a=None) == qr.QR_EINVAL
    assert gemm(M=0) == qr.QR_OK
    assert lib.qr_int8_gemm_i32(A16, A16, 128, 128, 512, 0, None, None) == qr.QR_EINVAL
    assert lib.qr_int8_gemm_i32(A16, A16, 128, 128, 512, 0, MIS, None) == qr.QR_EALIGN


def test_swiglu_rejects():
    lib = qr.library()
    rot = qr._Rot(28672, 4096, 7, A16, None)
    call = lambda g=A16, u=A16, ld=57344, rows=4: lib.qr_swiglu_rotate_quant(g, u, rows, ld, ctypes.byref(rot), 0,
                                                                            A16, A16, None)
    assert call(u=None) == qr.QR_EINVAL
    assert call(g=None) == qr.QR_EINVAL
    assert call(u=MIS) == qr.QR_EALIGN
    assert call(ld=57340) == qr.QR_EALIGN
    assert call(ld=28000) == qr.QR_ESHAPE
    assert call(rows=-1) == qr.QR_EINVAL
    assert call(rows=0, g=None, u=None) == qr.QR_OK


def test_gemm_k_bound_is_exclusive():
    """Products of widened codes reach 2^14 (q = -8 on both sides, or int8
    codes of -128): K = 2^17 would sum to exactly 2^31 and wrap, so the
    largest K accepted is 2^17 - 128 (validated on the host; the accepted
    sizes are not launched here)."""
    lib = qr.library()
    K = 1 << 17
    assert lib.qr_int4_gemm(A16, A16, A16, A16, 128, 128, K, 0, A16, 128, None) == qr.QR_ESHAPE
    assert lib.qr_int4_gemm_i32(A16, A16, 128, 128, K, 0, A16, None) == qr.QR_ESHAPE
    assert lib.qr_int8_gemm(A16, A16, A16, A16, 128, 128, K, 0, A16, 128, None) == qr.QR_ESHAPE
    assert lib.qr_int8_gemm_i32(A16, A16, 128, 128, K, 0, A16, None) == qr.QR_ESHAPE
    assert lib.qr_int4_gemm(A16, A16, A16, A16, 16, 128, K, 0, A16, 128, None) == qr.QR_ESHAPE   # decode size


# ---- the Python binding validates shapes and layouts before any launch.
# These run on CPU tensors: every shape check comes before the check that the
# tensors live on the GPU, so a wrong shape is reported as such.

def _cpu(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_binding_rotation_checks():
    import torch
    with pytest.raises(ValueError, match="signs must hold"):
        qr.Rotation(4096, 4096, signs=torch.ones(4095, dtype=torch.int8), device="cpu")
    with pytest.raises(ValueError, match="square"):
        qr.Rotation(64 * 6, 64, dense=torch.zeros(6, 5), device="cpu")
    with pytest.raises(ValueError, match="had_n"):
        qr.Rotation(4096, 2048, device="cpu")


def test_binding_rotate_quant_checks():
    import torch
    rot = qr.Rotation(512, 512, device="cpu")
    x = _cpu((4, 512), torch.float16)
    with pytest.raises(ValueError, match="columns"):
        qr.rotate_quant(_cpu((4, 520), torch.float16), rot)
    with pytest.raises(ValueError, match="unit column stride"):
        qr.rotate_quant(_cpu((512, 4), torch.float16).t(), rot)
    with pytest.raises(ValueError, match="codes must have shape"):
        qr.rotate_quant(x, rot, codes=_cpu((4, 255), torch.uint8))
    with pytest.raises(ValueError, match="codes must be contiguous"):
        qr.rotate_quant(x, rot, codes=_cpu((4, 512), torch.uint8)[:, ::2])
    with pytest.raises(ValueError, match="scales must have shape"):
        qr.rotate_quant(x, rot, group=128, scales=_cpu((4,), torch.float32))
    with pytest.raises(ValueError, match="group"):
        qr.rotate_quant(x, rot, group=100)
    with pytest.raises(TypeError, match="Rotation"):
        qr.rotate_quant(x, object())
    with pytest.raises(ValueError, match="live on the GPU"):
        qr.rotate_quant(x, rot)
    with pytest.raises(ValueError, match="codes must have shape"):
        qr.rotate_quant_i8(x, rot, 8, codes=_cpu((4, 256), torch.int8))


def test_binding_gemm_checks():
    import torch
    a, w = _cpu((130, 256), torch.uint8), _cpu((70, 256), torch.uint8)
    sa, sw = _cpu((130,), torch.float32), _cpu((70,), torch.float32)
    with pytest.raises(ValueError, match="K mismatch"):
        qr.int4_gemm(a, sa, _cpu((70, 128), torch.uint8), sw)
    with pytest.raises(ValueError, match="contiguous"):
        qr.int4_gemm(_cpu((130, 512), torch.uint8)[:, :256], sa, w, sw)
    with pytest.raises(ValueError, match="scales must hold"):
        qr.int4_gemm(a, _cpu((129,), torch.float32), w, sw)
    with pytest.raises(ValueError, match="scales must hold"):
        qr.int4_gemm(a, sa, w, sw, group=128)                 # group scales are [M][K/128]
    with pytest.raises(ValueError, match="group"):
        qr.int4_gemm(a, sa, w, sw, group=384)
    with pytest.raises(ValueError, match="y must have shape"):
        qr.int4_gemm(a, sa, w, sw, y=_cpu((130, 69), torch.float16))
    with pytest.raises(ValueError, match="acc must have shape"):
        qr.int4_gemm_i32(a, w, group=128, acc=_cpu((130, 70), torch.int32))
    with pytest.raises(ValueError, match="live on the GPU"):
        qr.int4_gemm(a, sa, w, sw)
    with pytest.raises(TypeError, match="int8"):
        qr.int8_gemm(a, sa, w, sw)


def test_binding_kv_and_attention_checks():
    import torch
    kv = _cpu((4, 2, 128), torch.float16)
    with pytest.raises(ValueError, match="hold"):
        qr.kv_quant(kv, codes=_cpu((4, 2, 63), torch.uint8))
    with pytest.raises(ValueError, match="signs must hold"):
        qr.kv_quant(kv, signs=torch.ones(64, dtype=torch.int8))
    with pytest.raises(ValueError, match="contiguous heads"):
        qr.kv_quant(_cpu((4, 128, 2), torch.float16).transpose(1, 2))
    B, T, Hq, Hkv = 2, 8, 4, 2
    q = _cpu((B, Hq, 128), torch.float16)
    kc, vc = _cpu((B, T, Hkv, 64), torch.uint8), _cpu((B, T, Hkv, 64), torch.uint8)
    ks, vs = _cpu((B, T, Hkv), torch.float32), _cpu((B, T, Hkv), torch.float32)
    kz, vz = _cpu((B, T, Hkv), torch.uint8), _cpu((B, T, Hkv), torch.uint8)
    with pytest.raises(ValueError, match="v_scales must hold"):
        qr.kv_attn_decode(q, kc, ks, kz, vc, _cpu((B, T - 1, Hkv), torch.float32), vz, workspace=False)
    with pytest.raises(ValueError, match="lens must hold"):
        qr.kv_attn_decode(q, kc, ks, kz, vc, vs, vz, lens=[1, 2, 3], workspace=False)
    with pytest.raises(ValueError, match="out must have shape"):
        qr.kv_attn_decode(q, kc, ks, kz, vc, vs, vz, out=_cpu((B, Hq, 64), torch.float16), workspace=False)
    with pytest.raises(ValueError, match="batch"):
        qr.kv_attn_decode(_cpu((3, Hq, 128), torch.float16), kc, ks, kz, vc, vs, vz, workspace=False)
    with pytest.raises(ValueError, match="live on the GPU"):
        qr.kv_attn_decode(q, kc, ks, kz, vc, vs, vz, workspace=False)


def test_binding_swiglu_checks():
    import torch
    rot = qr.Rotation(512, 512, device="cpu")
    g = _cpu((4, 512), torch.float16)
    with pytest.raises(ValueError, match="up must have shape"):
        qr.swiglu_rotate_quant(g, _cpu((3, 512), torch.float16), rot)
    both = _cpu((4, 1536), torch.float16)
    with pytest.raises(ValueError, match="one row stride"):
        qr.swiglu_rotate_quant(both[:, :512], _cpu((4, 512), torch.float16), rot)


def test_attn_noalloc_host_checks():
    """The allocation-free decode attention validates like qr_kv_attn_decode
    and rejects, before any launch, a shape whose split partials would not
    fit its 16 MiB static scratch array."""
    lib = qr.library()
    f32 = ctypes.c_float

    def call(B=1, Hq=32, Hkv=32, T=4096, D=128, q=A16, out=A16, kc=A16):
        return lib.qr_kv_attn_decode_noalloc(q, B, Hq, Hkv, T, D, kc, A16, A16, A16, A16, A16, None, None,
                                             f32(0.088), out, None)

    assert qr.kv_attn_decode_workspace(512, 64, 64, 4096) > 16 << 20
    assert call(B=512, Hq=64, Hkv=64) == qr.QR_ESCRATCH
    assert call(D=64) == qr.QR_ESHAPE
    assert call(Hkv=3) == qr.QR_ESHAPE
    assert call(q=None) == qr.QR_EINVAL
    assert call(kc=MIS) == qr.QR_EALIGN
    assert call(B=0, q=None, out=None) == qr.QR_OK
    assert "scratch" in qr.status_str(qr.QR_ESCRATCH)
