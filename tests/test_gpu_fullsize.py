"""GPU parity at the full sizes, in the launch configurations the benchmark
times, where the persistent kernels give each wave (or block) several rows or
tiles: the multi-row loops, their vmcnt bookkeeping and buffer refills, are
compared with the oracle on sampled outputs.

* rotate + quant, n = 8192, group 128: all 16384 rows of the LLaMA-2-70B
  MLP input in one call (about 8 rows per wave), at 4, 6 and 8 bits;
* rotate + quant, n = 4096: the 12288 rows of W^T of the fused QKV layer
  (the offline weight preparation that feeds the timed GEMM; 6 rows per wave);
* rotate + quant, Kronecker 64 x 172: all 131072 rows of the LLaMA-2-7B
  down_proj input (256 rows per block);
* KV quant: the K and V heads of a fused QKV output read in place
  (2048 tokens x 64 heads, two tiles per wave) and 131072 tokens x 32 heads
  (64 tiles per wave), with and without signs;
* integer GEMM: exact int32 sums on sampled outputs at 2048 x 12288 x 4096 and
  131072 x 4096 x 11008 (the fp16 outputs at full size are checked in
  test_gpu_parity.py), and a ragged shape with more tiles than resident
  blocks (4000 x 9000 x 1152: ~3 tiles per persistent block, partial tiles
  on both edges, a half K-tile at the end), int32 and fp16.

Samples always hold the first rows (first iteration of every wave), bands in
the middle and the last rows (last iterations), and random rows in between,
so they do not depend on the grid size the library picks.  The power-of-two
rotations are formed with the oracle's fwht, which its own tests pin to the
explicit Sylvester product.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.parity import (check_kv, check_output, check_scales, check_symmetric_codes, check_symmetric_int8,
                          epilogue_bound)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    import rotation_bit_quantized_amd as m
    m.library()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sample(n, seed, head=256, band=128, tail=256, rand=768):
    """Sorted distinct row indices: the first `head`, a band around n/2 and
    n/4, the last `tail`, and `rand` random ones."""
    rng = np.random.default_rng(seed)
    idx = set(range(min(head, n)))
    for c in (n // 4, n // 2, 3 * n // 4):
        idx.update(range(max(0, c - band // 2), min(n, c + band // 2)))
    idx.update(range(max(0, n - tail), n))
    idx.update(rng.integers(0, n, size=rand).tolist())
    return np.array(sorted(idx))


def oracle_pow2(x, signs, group, bits=4):
    """y = (x d) H / sqrt(n) per row with the oracle's pinned fwht, then its RTN."""
    n = x.shape[1]
    d = np.ones(n) if signs is None else np.asarray(signs, np.float64)
    y = O.fwht(np.asarray(x, np.float64) * d) / np.sqrt(n)
    return O.quantize_symmetric(y, group, bits)


# ------------------------------------------------------------------ rotate + quant

@pytest.mark.parametrize("bits", [4, 6, 8])
def test_rq_c4_all_rows_one_call(qr, bits):
    """16384 x 8192, group 128, one launch; sampled rows against the oracle."""
    c = W.CONFIGS["c4"]
    x = W.make_x(c)
    signs = W.make_signs(c)
    rot = qr.Rotation.hadamard(c.K, signs)
    xt = dev(x)
    if bits == 4:
        codes, scales = qr.rotate_quant(xt, rot, 128)
    else:
        codes, scales = qr.rotate_quant_i8(xt, rot, bits, 128)
    pick = sample(c.M, seed=bits)
    got_c = host(codes)[pick]
    got_s = host(scales)[pick]
    q, s, t = oracle_pow2(x[pick], signs, 128, bits)
    if bits == 4:
        check_symmetric_codes(got_c, q, t, f"c4 codes ({len(pick)} sampled rows)")
    else:
        check_symmetric_int8(got_c, q, t, f"c4 {bits}-bit codes")
    check_scales(got_s, s, "c4 group scales")


def test_weight_prep_c2_all_channels_one_call(qr):
    """The 12288 rows of W^T (fused QKV, 4096 wide) in one launch, as the
    benchmark prepares its weights; sampled channels against the oracle's
    offline preparation R^T W quantized per output channel."""
    c = W.CONFIGS["c2"]
    w = W.make_w(c)
    signs = W.make_signs(c)
    codes, scales = qr.rotate_quant(dev(w.T), qr.Rotation.hadamard(c.K, signs), 0)
    pick = sample(c.N, seed=22, rand=512)
    wr = O.rotate_weights(w[:, pick], O.rotation_matrix(c.K, signs=signs))
    q, s = O.quantize_weights(wr, 0)
    _, _, t = O.quantize_symmetric(wr.T, 0)
    check_symmetric_codes(host(codes)[pick], q, t, "c2 weight codes")
    check_scales(host(scales)[pick], s, "c2 weight scales")


def test_rq_c3_all_rows_one_call(qr):
    """131072 x 11008 (64 x 172 Kronecker), one launch as the benchmark times
    it; sampled rows against the oracle's Kronecker rotation."""
    c = W.CONFIGS["c3"]
    x = W.make_x(c)
    o = W.make_dense(c)
    codes, scales = qr.rotate_quant(dev(x), qr.Rotation.kronecker(64, o), 0)
    pick = sample(c.M, seed=3, head=128, band=64, tail=128, rand=256)
    y = O.rotate_kron(x[pick], 64, o.astype(np.float64))
    q, s, t = O.quantize_symmetric(y, 0)
    check_symmetric_codes(host(codes)[pick], q, t, "c3 codes")
    check_scales(host(scales)[pick], s, "c3 scales")


# ------------------------------------------------------------------ KV quant

def test_kv_bench_step_slice(qr):
    """K and V of a fused QKV output [2048, 3 x 4096] quantized in one launch
    through the row stride (2048 tokens x 64 heads), as in the benchmark."""
    T, H = 2048, 32
    rng = np.random.default_rng(44)
    qkv = (rng.standard_normal((T, 3 * H * 128)) * 2).astype(np.float16)
    t = dev(qkv)
    codes, step, zero = qr.kv_quant(t[:, H * 128:3 * H * 128])
    ref = np.ascontiguousarray(qkv[:, H * 128:]).reshape(T, 2 * H, 128)
    check_kv(host(codes), host(step), host(zero), ref)


@pytest.mark.parametrize("with_signs", [False, True])
def test_kv_prefill_scale(qr, with_signs):
    """131072 tokens x 32 heads in one launch; sampled tokens (all their heads)."""
    T, H = 131072, 32
    kv = W.make_kv_large(T, H)
    signs = np.where(np.random.default_rng(9).random(128) < 0.5, -1, 1).astype(np.int8) if with_signs else None
    codes, step, zero = qr.kv_quant(dev(kv), signs=signs)
    pick = sample(T, seed=11, head=64, band=32, tail=64, rand=256)
    check_kv(host(codes)[pick], host(step)[pick], host(zero)[pick], kv[pick], signs)


# ------------------------------------------------------------------ integer GEMM at full size

@pytest.mark.parametrize("cfg", ["c2", "c3"])
def test_gemm_i32_full_size_sampled_exact(qr, cfg):
    """The exact int32 sums of the full-size GEMM (random packed codes), on
    sampled rows and columns: bit-exact against the oracle's int64 product."""
    c = W.CONFIGS[cfg]
    M, N, K = c.M, c.N, c.K
    a = W.make_random_packed(M, K // 2, seed=21)
    w = W.make_random_packed(N, K // 2, seed=22)
    acc = qr.int4_gemm_i32(dev(a), dev(w))
    rows = sample(M, seed=5, head=70, band=40, tail=70, rand=60)
    cols = sample(N, seed=6, head=200, band=64, tail=200, rand=100)
    got = host(acc[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(cols, device="cuda")])
    ref = O.int_gemm(O.unpack_int4(a[rows]), O.unpack_int4(w[cols]))
    assert np.array_equal(got.astype(np.int64), ref)


def test_gemm_persistent_ragged_sampled(qr):
    """4000 x 9000 x 1152: the 256 x 192 tiles (16 x 47 of them, partial on
    both edges) run on the persistent grid, about three per block, K ends in
    a half tile.  Exact int32 sums and the fp16 output (per-element epilogue
    bound) on sampled rows, all columns."""
    M, N, K = 4000, 9000, 1152
    a = W.make_random_packed(M, K // 2, seed=31)
    w = W.make_random_packed(N, K // 2, seed=32)
    rng = np.random.default_rng(33)
    sa = (rng.random(M) * 0.1 + 0.01).astype(np.float32)
    sw = (rng.random(N) * 0.01 + 0.001).astype(np.float32)
    acc = qr.int4_gemm_i32(dev(a), dev(w))
    y = qr.int4_gemm(dev(a), dev(sa), dev(w), dev(sw))
    rows = sample(M, seed=7, head=40, band=40, tail=40, rand=40)
    ridx = torch.as_tensor(rows, device="cuda")
    ref = O.int_gemm(O.unpack_int4(a[rows]), O.unpack_int4(w))
    assert np.array_equal(host(acc[ridx]).astype(np.int64), ref)
    yref = O.dequantize_output(ref, sa[rows], sw)
    yg = host(y[ridx])
    check_output(yg, yref)
    assert np.all(np.abs(yg.astype(np.float64) - yref) <= epilogue_bound(ref, sa[rows], sw))
