"""CPU checks of the parity helpers themselves (no GPU): the per-element
epilogue bound holds for an fp32 epilogue simulated in numpy, and is tight
enough to catch a lost K-tile."""
import numpy as np

import oracle as O
import workloads as W
from tests.parity import epilogue_bound


def fp32_epilogue(acc, sx, sw, group):
    """The dequantizing epilogue as the kernels evaluate it: fp32 terms
    float(acc) * (s_x * s_w), summed over groups in increasing order in
    fp32, rounded once to fp16."""
    f = np.float32
    sx = np.asarray(sx, f)
    sw = np.asarray(sw, f)
    if group == 0:
        v = acc.astype(f) * (sx[:, None] * sw[None, :])
    else:
        v = np.zeros(acc.shape[1:], f)
        for j in range(acc.shape[0]):
            v = v + acc[j].astype(f) * (sx[:, j, None] * sw[None, :, j])
    return v.astype(np.float16).astype(np.float64)


def case(M, N, K, group, seed):
    qa = W.make_random_codes(M, K, seed=seed)
    qw = W.make_random_codes(N, K, seed=seed + 1)
    G = 1 if group == 0 else K // group
    sx = W.make_random_scales(M * G, seed + 2).reshape(M, G)
    sw = W.make_random_scales(N * G, seed + 3).reshape(N, G)
    if group == 0:
        sx, sw = sx[:, 0].copy(), sw[:, 0].copy()
    return qa, qw, sx, sw


def test_bound_holds_for_fp32_epilogue():
    for M, N, K, group, seed in [(40, 50, 11008, 0, 1), (30, 40, 8192, 128, 2), (20, 30, 1024, 256, 3)]:
        qa, qw, sx, sw = case(M, N, K, group, seed)
        acc = O.int_gemm(qa, qw, group)
        ref = O.dequantize_output(acc, sx, sw, group)
        got = fp32_epilogue(acc, sx, sw, group)
        assert np.all(np.abs(got - ref) <= epilogue_bound(acc, sx, sw, group))


def test_bound_catches_a_missing_k_tile():
    """Drop one 256-code K-tile from the sums: nearly every element moves by
    more than the bound."""
    qa, qw, sx, sw = case(24, 32, 11008, 0, 7)
    acc = O.int_gemm(qa, qw)
    short = O.int_gemm(qa[:, 256:], qw[:, 256:])
    ref = O.dequantize_output(acc, sx, sw)
    bad = O.dequantize_output(short, sx, sw)
    frac = np.mean(np.abs(bad - ref) > epilogue_bound(acc, sx, sw))
    assert frac > 0.9
