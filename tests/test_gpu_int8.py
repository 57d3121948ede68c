"""GPU parity of the 6- and 8-bit variants (qr_rotate_quant_i8, qr_int8_gemm,
qr_int8_gemm_i32) against the CPU oracle: integer sums bit-exact, codes
under the boundary rule of tests/parity.py, fp16 outputs within its bounds."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.parity import check_output, check_scales, check_symmetric_int8

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


# ------------------------------------------------------------ integer GEMM on int8 codes

@pytest.mark.parametrize("M,N,K,group", [
    (64, 512, 512, 0),        # decode kernel
    (17, 100, 4096, 0),       # decode, ragged
    (48, 96, 1024, 128),      # decode, group-wise
    (65, 70, 128, 0),         # smallest prefill M, one K-tile
    (320, 640, 4096, 0),      # several prefill tiles
    (257, 130, 512, 0),       # ragged M and N
    (513, 384, 11008, 0),     # K of the down_proj
    (192, 256, 1024, 128),    # group-wise: a group is one K-tile
    (150, 160, 1152, 384),    # groups of three K-tiles
    (300, 200, 640, 0),       # K an odd multiple of 128
    (33, 4100, 11008, 0),     # decode: three token tiles, eleven K chunks (the last a partial one)
    (16, 48, 130944, 0),      # decode at the largest K: the -128 rows reach 2^31 - 2^21
])
def test_int8_gemm_i32_exact(qr, M, N, K, group):
    qa = W.make_random_codes(M, K, seed=7 * M + K, lo=-128, hi=127)
    qw = W.make_random_codes(N, K, seed=11 * N + K, lo=-128, hi=127)
    qa[0, :] = -128                    # extreme codes: |acc| up to 2^14 K
    qw[0, :] = -128
    qw[-1, :] = 127
    acc = host(qr.int8_gemm_i32(dev(qa), dev(qw), group))
    ref = O.int_gemm(qa, qw, group)
    assert acc.shape == ref.shape
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("M,N,K,group", [(64, 512, 512, 0), (320, 640, 4096, 0), (257, 130, 1024, 128),
                                         (40, 300, 1024, 128), (130, 96, 11008, 0), (17, 100, 4096, 0),
                                         (33, 4100, 11008, 0)])
def test_int8_gemm_epilogue(qr, M, N, K, group):
    rng = np.random.default_rng(M + N)
    qa = W.make_random_codes(M, K, seed=M, lo=-127, hi=127)
    qw = W.make_random_codes(N, K, seed=N + 1, lo=-127, hi=127)
    G = 1 if group == 0 else K // group
    sa = (rng.random((M, G)) * 0.01 + 0.001).astype(np.float32)
    sw = (rng.random((N, G)) * 0.001 + 0.0001).astype(np.float32)
    if group == 0:
        sa, sw = sa[:, 0].copy(), sw[:, 0].copy()
    y = host(qr.int8_gemm(dev(qa), dev(sa), dev(qw), dev(sw), group))
    ref = O.dequantize_output(O.int_gemm(qa, qw, group), sa, sw, group)
    check_output(y, ref)
    assert np.all(np.abs(y.astype(np.float64) - ref) <= np.abs(ref) * 2 ** -10 + 1e-6)


# ------------------------------------------------------------ 6- and 8-bit rotate + quant

def check_rq8(qr, x, n, bits, had_n=None, dense=None, signs=None, group=0):
    had_n = n if had_n is None else had_n
    rot = qr.Rotation(n, had_n, dense, signs)
    codes, scales = qr.rotate_quant_i8(dev(x), rot, bits, group)
    r = O.rotation_matrix(n, had_n, dense=None if dense is None else np.asarray(dense, np.float64), signs=signs)
    q, s, t = O.quantize_symmetric(O.rotate(x, r), group, bits)
    check_symmetric_int8(host(codes), q, t)
    check_scales(host(scales), s)


@pytest.mark.parametrize("bits", [6, 8])
def test_rq_i8_c2_rows(qr, bits):
    """n = 4096 with signs (the MFMA kernel)."""
    c = W.CONFIGS["c2"]
    x = W.make_x(c, rows=np.arange(300))
    check_rq8(qr, x, c.K, bits, signs=W.make_signs(c))


@pytest.mark.parametrize("bits", [6, 8])
def test_rq_i8_c4_group128(qr, bits):
    """n = 8192, group 128 (the MFMA kernel, two runs per lane)."""
    c = W.CONFIGS["c4"]
    x = W.make_x(c, rows=np.r_[np.arange(130), np.arange(c.M - 3, c.M)])
    check_rq8(qr, x, c.K, bits, signs=W.make_signs(c), group=128)


@pytest.mark.parametrize("n,had,m,group", [(512, 512, 1, 0), (1024, 1024, 1, 64), (64 * 172, 64, 172, 0),
                                           (4096 * 7, 4096, 7, 0), (96, 32, 3, 32)])
def test_rq_i8_other_rotations(qr, n, had, m, group):
    """Widths and Kronecker factors outside the MFMA kernel (reference-shape
    kernel), 8 bits; zero and one-hot rows."""
    x = W.make_random_rows(5, n, seed=n + m, scale=2.0)
    x[1] = 0
    x[2] = 0
    x[2, n // 3] = 4.0
    dense = None if m == 1 else np.linalg.qr(np.random.default_rng(m).standard_normal((m, m)))[0].astype(np.float32)
    check_rq8(qr, x, n, 8, had_n=had, dense=dense, group=group)


def test_layer_8bit_end_to_end_c1(qr):
    """The c1 layer at 8 bits: activations rotated and quantized on the GPU,
    weights by the oracle offline, the int8 GEMM; against the oracle's layer
    (the codes may differ only on rounding boundaries)."""
    c = W.CONFIGS["c1"]
    x, w, signs = W.make_x(c), W.make_w(c), W.make_signs(c)
    r = O.rotation_matrix(c.K, signs=signs)
    lay = O.linear_w4a4(x, w, r, bits=8)
    codes, scales = qr.rotate_quant_i8(dev(x), qr.Rotation(c.K, c.K, None, signs), 8)
    y = host(qr.int8_gemm(codes, scales, dev(lay["qw"]), dev(lay["sw"].astype(np.float32))))
    check_output(y, lay["out"])
