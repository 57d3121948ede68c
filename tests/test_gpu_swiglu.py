"""GPU parity of the fused feed-forward activation + rotation + quantization
(qr_swiglu_rotate_quant) against the oracle: x = fp16(silu(gate) * up)
(oracle.swiglu_fp16), then the oracle's rotation and RTN.  gate is seeded
N(0, 1.5^2) (or wider); up is the layer input recipe of the config.

Rounding x to fp16 is a decision the GPU takes in fp32 (relative error of
silu(g) u below 2^-21: one ulp each for the exponential and the reciprocal,
half an ulp per rounding) and the oracle in fp64.  Where the exact product
lies within 2^-20 of an fp16 rounding midpoint both neighbours are valid.
y is linear in x, so a different choice at such elements k moves output j by
at most B_j = sum_k ulp_k |R[k, j]|: a code may then differ where the
pre-rounding value y_j / s lies within B_j / s of a .5 boundary (besides the
usual window), and the scale max|y| / 7 by at most max_j B_j / 7.  Mismatches
that this does not explain (inside the usual window only) are capped at the
usual fraction of the elements."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests.parity import MAX_MISMATCH_FRAC, SCALE_RTOL, check_symmetric_codes, near_half

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    import rotation_bit_quantized_amd as m
    m.library()
    return m


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ambiguous_ulps(gate, up):
    """Per element: the fp16 ulp of x where silu(g) u lies within 2^-20 of an
    fp16 rounding midpoint, else 0."""
    exact = O.silu(gate) * np.asarray(up, np.float64)
    x = exact.astype(np.float16).astype(np.float64)
    ulp = np.abs(np.spacing(np.abs(x).astype(np.float16)).astype(np.float64))
    side = np.sign(exact - x)
    other = x + side * ulp                      # the fp16 neighbour on the other side of the exact value
    mid = (x + other) / 2
    amb = (side != 0) & (np.abs(exact - mid) <= 2.0 ** -20 * np.maximum(np.abs(exact), 2.0 ** -24))
    return np.where(amb, ulp, 0.0)


def run_and_check(qr, gate, up, n, had_n, dense=None, signs=None, group=0):
    both = torch.from_numpy(np.ascontiguousarray(np.concatenate([gate, up], axis=1))).cuda()   # [rows, 2n]
    rot = qr.Rotation(n, had_n, dense, signs)
    codes, scales = qr.swiglu_rotate_quant(both[:, :n], both[:, n:], rot, group)
    x = O.swiglu_fp16(gate, up)
    amb = ambiguous_ulps(gate, up)
    if dense is not None and n > 4096:
        y = O.rotate_kron(x, had_n, np.asarray(dense, np.float64), signs)
        m = len(dense)
        # |R| = (1/sqrt(p)) (ones kron |O|): B at column (i, b) = sum_k amb_k |O[a_k, b]| / sqrt(p)
        ab = np.abs(np.asarray(dense, np.float64))
        bound = np.tile((amb.reshape(len(x), -1, m).sum(axis=1) @ ab) / np.sqrt(had_n), (1, n // m))
    else:
        r = O.rotation_matrix(n, had_n, dense=None if dense is None else np.asarray(dense, np.float64), signs=signs)
        y = O.rotate(x, r)
        bound = amb @ np.abs(r)
    q, s, t = O.quantize_symmetric(y, group)
    g = n if group == 0 else group
    sb = np.repeat(np.asarray(s, np.float64).reshape(len(x), -1), g, axis=1)
    shift = np.where(sb > 0, bound / np.where(sb > 0, sb, 1.0), 0.0)
    gq = O.unpack_int4(host(codes))
    mism = gq != q
    frac = np.abs(np.abs(t - np.floor(t)) - 0.5)
    explained_by_x = frac <= shift
    unexplained = mism & ~near_half(t) & ~explained_by_x
    assert not unexplained.any(), f"{int(unexplained.sum())} code mismatches beyond the boundary and rounding bounds"
    # the rotated-value roundings: boundary mismatches that the fp16 choice
    # of x does not explain are capped as for every other code
    boundary_only = mism & ~explained_by_x
    assert boundary_only.sum() <= MAX_MISMATCH_FRAC * mism.size, \
        f"{int(boundary_only.sum())} boundary mismatches of {mism.size}"
    assert np.all(np.abs(gq.astype(np.int64) - q) <= 1)
    gs = host(scales).astype(np.float64).reshape(np.asarray(s).shape)
    sref = np.asarray(s, np.float64)
    bmax = bound.reshape(len(x), -1, g).max(axis=2).reshape(sref.shape)
    assert np.all(np.abs(gs - sref) <= SCALE_RTOL * sref + bmax / 7 + 1e-30)
    return int(mism.sum()), int((amb > 0).sum())


def test_swiglu_d70_rows(qr):
    """28672 = 4096 x 7 (LLaMA-2-70B down_proj input): the MFMA kernel, rows
    spread over the persistent blocks (first 600 and last 33 rows)."""
    c = W.CONFIGS["d70"]
    rows = np.r_[np.arange(600), np.arange(c.M - 33, c.M)]
    up = W.make_x(c, rows=rows)
    gate = W.make_random_rows(len(rows), c.K, seed=70, scale=1.5)
    run_and_check(qr, gate, up, c.K, c.had_n, dense=W.make_dense(c))


@pytest.mark.parametrize("m,rows", [(2, 3), (5, 40)])
def test_swiglu_kron4096_small_m(qr, m, rows):
    o = np.linalg.qr(np.random.default_rng(m).standard_normal((m, m)))[0].astype(np.float32)
    up = W.make_random_rows(rows, 4096 * m, seed=m, scale=2.0)
    gate = W.make_random_rows(rows, 4096 * m, seed=m + 100, scale=1.5)
    gate[0] = 0          # silu(0) = 0: an all-zero row
    run_and_check(qr, gate, up, 4096 * m, 4096, dense=o)


def test_swiglu_c3_rows(qr):
    """11008 = 64 x 172 (LLaMA-2-7B down_proj input): reference-shape kernel."""
    c = W.CONFIGS["c3"]
    up = W.make_x(c, rows=np.arange(40))
    gate = W.make_random_rows(40, c.K, seed=3, scale=1.5)
    run_and_check(qr, gate, up, c.K, 64, dense=W.make_dense(c))


@pytest.mark.parametrize("group", [0, 128])
def test_swiglu_pow2_signs(qr, group):
    """A power-of-two width with signs and groups (reference-shape kernel);
    large |gate| exercises both tails of silu."""
    up = W.make_random_rows(33, 1024, seed=5)
    gate = W.make_random_rows(33, 1024, seed=6, scale=8.0)
    signs = np.where(np.random.default_rng(7).random(1024) < 0.5, -1, 1).astype(np.int8)
    run_and_check(qr, gate, up, 1024, 1024, signs=signs, group=group)
