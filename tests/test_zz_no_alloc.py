"""GPU test of qr_kv_attn_decode_noalloc, the allocation-free decode attention
(split partials in the library's static scratch array): called through the
C ABI, its output must equal that of qr_kv_attn_decode with a caller-owned
workspace (the same plan and kernels, so bit-identical fp16), on two calls in
a row, the second with a smaller input, and match the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.parity import check_attn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    import rotation_bit_quantized_amd as m
    m.library()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_both(qr, B, T, Hq, Hkv, seed, lens=None):
    lib = qr.library()
    cache = [dev(a) for a in W.make_attn_cache(B, T, Hkv, seed=seed)]
    q = dev(W.make_attn_query(B, Hq, seed=seed + 1))
    ln = None if lens is None else dev(np.asarray(lens, np.int32))
    kc, ks, kz, vc, vs, vz = cache
    sm = ctypes.c_float(1.0 / np.sqrt(128.0))
    stream = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()

    need = qr.kv_attn_decode_workspace(B, Hq, Hkv, T)
    assert 0 < need <= 16 << 20, need             # a split plan that fits the static scratch
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    ref_out = torch.empty((B, Hq, 128), dtype=torch.float16, device="cuda")
    st = lib.qr_kv_attn_decode(ptr(q), B, Hq, Hkv, T, 128, ptr(kc), ptr(ks), ptr(kz), ptr(vc), ptr(vs), ptr(vz),
                               ptr(ln), None, sm, ptr(ws), need, ptr(ref_out), stream)
    assert st == qr.QR_OK
    out = torch.full((B, Hq, 128), 7.0, dtype=torch.float16, device="cuda")
    st = lib.qr_kv_attn_decode_noalloc(ptr(q), B, Hq, Hkv, T, 128, ptr(kc), ptr(ks), ptr(kz), ptr(vc), ptr(vs),
                                       ptr(vz), ptr(ln), None, sm, ptr(out), stream)
    assert st == qr.QR_OK
    torch.cuda.synchronize()
    got, ref = out.cpu().numpy(), ref_out.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), "no-alloc output differs from the workspace call"
    return got, [a.cpu().numpy() for a in cache], q.cpu().numpy()


def test_noalloc_matches_workspace_call_twice(qr):
    # first call: 64 sequences x 2048 tokens, 32 heads (split into chunks)
    run_both(qr, 64, 2048, 32, 32, seed=40)
    # second call, smaller: grouped heads, ragged lengths; also against the oracle
    lens = [1000, 0, 513, 999]
    got, cache, q = run_both(qr, 4, 1000, 16, 4, seed=50, lens=lens)
    kc, ks, kz, vc, vs, vz = cache
    ref = O.kv_attention_decode(q, O.unpack_uint4(kc), ks, kz, O.unpack_uint4(vc), vs, vz, lens=np.asarray(lens))
    check_attn(got, ref, "no-alloc attention")
