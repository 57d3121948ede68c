"""GPU parity of decode attention over the rotated 4-bit KV cache: the HIP
library (through its C ABI) against the CPU oracle.  Caches are seeded
random codes, steps and zero points (workloads.make_attn_cache) or the
oracle's own quantization of seeded K/V; expected values come only from the
oracle.  Tolerance: tests/parity.py (check_attn)."""
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


def run(qr, q, cache, lens=None, signs=None, sm_scale=None, workspace=None):
    kc, ks, kz, vc, vs, vz = (dev(a) for a in cache)
    out = qr.kv_attn_decode(dev(q), kc, ks, kz, vc, vs, vz, lens=lens, signs=signs, sm_scale=sm_scale,
                            workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle(q, cache, lens=None, signs=None, sm_scale=None):
    kc, ks, kz, vc, vs, vz = cache
    return O.kv_attention_decode(q, O.unpack_uint4(kc), ks, kz, O.unpack_uint4(vc), vs, vz, lens=lens,
                                 signs=signs, sm_scale=sm_scale)


@pytest.mark.parametrize("B,T,Hq,Hkv", [(2, 300, 4, 4), (1, 1, 8, 8), (3, 64, 2, 2), (1, 4100, 32, 32),
                                        (2, 777, 16, 2)])
def test_attn_shapes(qr, B, T, Hq, Hkv):
    """Split and unsplit sequences, a single token, a ragged last chunk,
    grouped query heads (8 per KV head)."""
    cache = W.make_attn_cache(B, T, Hkv, seed=B * 1000 + T)
    q = W.make_attn_query(B, Hq, seed=T)
    check_attn(run(qr, q, cache), oracle(q, cache))


def test_attn_lens_signs_scale(qr):
    """Ragged lengths including an empty and a one-token sequence, signs, a
    non-default softmax scale; with and without a workspace (split chunks vs
    one chunk per sequence)."""
    B, T, Hq, Hkv = 5, 1500, 8, 4
    cache = W.make_attn_cache(B, T, Hkv, seed=11)
    q = W.make_attn_query(B, Hq, seed=12)
    lens = np.array([0, 1, 257, 1499, 1500], np.int32)
    signs = np.where(np.random.default_rng(13).random(128) < 0.5, -1, 1).astype(np.int8)
    want = oracle(q, cache, lens=lens, signs=signs, sm_scale=0.15)
    assert qr.kv_attn_decode_workspace(B, Hq, Hkv, T) > 0
    got = run(qr, q, cache, lens=lens, signs=signs, sm_scale=0.15)
    check_attn(got, want)
    assert np.all(got[0] == 0)
    got1 = run(qr, q, cache, lens=lens, signs=signs, sm_scale=0.15, workspace=False)
    check_attn(got1, want)


def test_attn_quantized_kv_chain(qr):
    """Cache made by the oracle's KV quantizer from seeded K/V with outlier
    head dims (the decode recipe), with signs."""
    B, T, H = 2, 400, 8
    signs = np.where(np.random.default_rng(21).random(128) < 0.5, -1, 1).astype(np.int8)
    parts = []
    for stream in (0, 1):
        kv = W.make_kv_large(B * T, H, seed=30 + stream)
        c, step, z, _, _ = O.kv_quantize(kv, signs=signs)
        parts += [O.pack_int4(c.reshape(-1, 128)).reshape(B, T, H, 64), step.reshape(B, T, H).astype(np.float32),
                  z.reshape(B, T, H).astype(np.uint8)]
    q = W.make_attn_query(B, H, seed=22)
    check_attn(run(qr, q, tuple(parts), signs=signs), oracle(q, tuple(parts), signs=signs))


def test_attn_full_size_sampled(qr):
    """The measured shape (64 sequences x 2048 tokens x 32 heads) in the
    launch configuration the bench times; three sequences checked against
    the oracle."""
    B, T, H = 64, 2048, 32
    cache = W.make_attn_cache(B, T, H, seed=1)
    q = W.make_attn_query(B, H, seed=2)
    got = run(qr, q, cache)
    for b in (0, 37, 63):
        sub = tuple(a[b:b + 1] for a in cache)
        check_attn(got[b:b + 1], oracle(q[b:b + 1], sub), what=f"sequence {b}")


@pytest.mark.parametrize("B,T,Hq,Hkv,lens", [(2, 300, 16, 4, None), (3, 130, 32, 2, [0, 1, 129]),
                                             (1, 1000, 16, 1, None), (2, 64, 40, 5, None)])
def test_attn_grouped_heads(qr, B, T, Hq, Hkv, lens):
    """4 to 16 query heads per KV head (the MFMA kernel that serves a KV
    head's query heads together): split and unsplit, ragged and empty
    sequences, a single KV head, a head count that is not a power of two."""
    cache = W.make_attn_cache(B, T, Hkv, seed=T + Hq)
    q = W.make_attn_query(B, Hq, seed=Hq + Hkv)
    signs = np.where(np.random.default_rng(B).random(128) < 0.5, -1, 1).astype(np.int8)
    ln = None if lens is None else np.array(lens, np.int32)
    want = oracle(q, cache, lens=ln, signs=signs)
    check_attn(run(qr, q, cache, lens=ln, signs=signs), want)
    check_attn(run(qr, q, cache, lens=ln, signs=signs, workspace=False), want)


def test_attn_grouped_full_size_sampled(qr):
    """LLaMA-2-70B decode shape: 64 sequences x 2048 tokens, 64 query heads
    over 8 KV heads; three sequences checked against the oracle."""
    B, T, Hq, Hkv = 64, 2048, 64, 8
    cache = W.make_attn_cache(B, T, Hkv, seed=8)
    q = W.make_attn_query(B, Hq, seed=9)
    got = run(qr, q, cache)
    for b in (0, 31, 63):
        sub = tuple(a[b:b + 1] for a in cache)
        check_attn(got[b:b + 1], oracle(q[b:b + 1], sub), what=f"sequence {b}")
