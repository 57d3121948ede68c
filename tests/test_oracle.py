"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed
forms, hand-derived worked examples (tests/golden), invariants, brute force on
tiny inputs, or an independent formulation of the same quantity.  A plausible
slip in the oracle (a dropped term, a wrong sign, an index swap, a transposed
operand, the wrong rounding mode) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


# ---------------------------------------------------------------- Hadamard

def test_hadamard_4_matches_hand_derived():
    assert np.array_equal(O.sylvester_hadamard(4), np.array(GOLD["hadamard_4"]["H"]))


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 512, 1024])
def test_hadamard_orthogonality_exact(n):
    h = O.sylvester_hadamard(n)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [2, 16, 128, 1024])
def test_hadamard_recursion_equals_popcount_formula(n):
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    assert np.array_equal(O.sylvester_hadamard(n), O.hadamard_entry(i, j))


def test_hadamard_symmetric_and_first_row_ones():
    h = O.sylvester_hadamard(256)
    assert np.array_equal(h, h.T)
    assert np.all(h[0] == 1) and np.all(h[:, 0] == 1)


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.sylvester_hadamard(12)


@pytest.mark.parametrize("n", [2, 4, 8, 32, 256, 1024])
def test_fwht_equals_explicit_product(n):
    x = np.random.default_rng(n).standard_normal((7, n))
    ref = x @ O.sylvester_hadamard(n).astype(np.float64)
    got = O.fwht(x)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- rotations

@pytest.mark.parametrize("p,m,use_signs", [(4, 3, False), (16, 12, True), (64, 7, True), (8, 172, False),
                                           (2, 5, True)])
def test_rotate_kron_equals_explicit_product(p, m, use_signs):
    """The factored Kronecker rotation (used where the n x n matrix does not
    fit) is the explicit product x @ R: pinned against np.kron built R."""
    rng = np.random.default_rng(p * 1000 + m)
    n = p * m
    o = np.linalg.qr(rng.standard_normal((m, m)))[0]
    signs = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8) if use_signs else None
    x = rng.standard_normal((5, n)).astype(np.float16)
    ref = O.rotate(x, O.rotation_matrix(n, p, dense=o, signs=signs))
    got = O.rotate_kron(x, p, o, signs)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("n", [4, 512, 4096])
def test_rotation_orthogonal(n):
    r = O.rotation_matrix(n, signs=W.make_signs("c2", n))
    assert np.max(np.abs(r @ r.T - np.eye(n))) < 1e-12


def test_kron_rotation_orthogonal_and_structure():
    o = W.make_dense("c3", dtype=np.float64)
    assert o.shape == (172, 172)
    assert np.max(np.abs(o @ o.T - np.eye(172))) < 1e-12
    r = O.rotation_matrix(64 * 172, 64, dense=o)
    # orthogonality of the 11008-point rotation on a sampled block of rows
    rows = r[::97]
    assert np.max(np.abs(rows @ rows.T - np.eye(rows.shape[0]))) < 1e-12
    # Kronecker index convention k = i*m + a, a fastest: element [i*m+a, j*m+b] = H[i,j]/8 * O[a,b]
    h = O.sylvester_hadamard(64)
    for (i, a, j, b) in [(0, 0, 0, 0), (3, 5, 7, 11), (63, 171, 1, 170), (10, 100, 33, 2)]:
        assert r[i * 172 + a, j * 172 + b] == pytest.approx(h[i, j] / 8.0 * o[a, b], abs=0, rel=1e-15)


def test_kron_rotation_equals_two_sided_matrix_form():
    """x . (A kron B) with x viewed as X[p, m] (m fastest) equals A^T X B."""
    rng = np.random.default_rng(5)
    p, m = 8, 6
    o = np.linalg.qr(rng.standard_normal((m, m)))[0]
    x = rng.standard_normal((3, p * m))
    r = O.rotation_matrix(p * m, p, dense=o)
    hn = O.sylvester_hadamard(p) / np.sqrt(p)
    two_sided = np.stack([(hn.T @ xi.reshape(p, m) @ o).reshape(-1) for xi in x])
    assert np.max(np.abs(O.rotate(x, r) - two_sided)) < 1e-13


@pytest.mark.parametrize("cfg", ["c1", "c2", "c4"])
def test_computational_invariance(cfg):
    """(x R)(R^T W) = x W: DuQuant Knowl 1 identity with G = R orthogonal; QuaRot
    abstract: rotations that leave the layer output unchanged."""
    c = W.CONFIGS[cfg]
    x = W.make_x(c, rows=np.arange(16))
    w = W.make_w(c)[:, :64] if c.N > 64 else W.make_w(c)
    r = O.rotation_matrix(c.K, signs=W.make_signs(c))
    ref = x.astype(np.float64) @ w.astype(np.float64)
    got = O.rotate(x, r) @ O.rotate_weights(w, r)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-13


def test_computational_invariance_kron():
    c = W.CONFIGS["c3"]
    x = W.make_x(c, rows=np.arange(4))
    w = W.make_w(c, cols=np.arange(16))
    r = O.rotation_matrix(c.K, 64, dense=W.make_dense(c, dtype=np.float64))
    ref = x.astype(np.float64) @ w.astype(np.float64)
    got = O.rotate(x, r) @ O.rotate_weights(w, r)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-13


def test_signs_go_on_the_input_side():
    n = 8
    d = np.array([1, -1, -1, 1, 1, 1, -1, 1])
    r = O.rotation_matrix(n, signs=d)
    e3 = np.zeros(n)
    e3[3] = 1.0
    # row 3 of R is d_3 * H[3, :] / sqrt(n)
    assert np.allclose(O.rotate(e3[None], r)[0], d[3] * O.sylvester_hadamard(n)[3] / np.sqrt(n), atol=0)


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("ex", GOLD["rotate_quant"], ids=lambda e: e["name"])
def test_rotate_quant_worked_examples(ex):
    x = np.array([ex["x"]], dtype=np.float16)
    r = O.rotation_matrix(4, signs=ex["signs"])
    y = O.rotate(x, r)
    assert np.allclose(y[0], ex["y"], atol=1e-15)
    q, s, _ = O.quantize_symmetric(y)
    assert s[0] == pytest.approx(ex["scale"], rel=1e-15)
    assert q[0].tolist() == ex["codes"]
    assert O.pack_int4(q)[0].tolist() == ex["packed"]


def test_group_worked_example():
    g = GOLD["quantize_groups"]
    q, s, _ = O.quantize_symmetric(np.array([g["y"]], dtype=np.float64), g["group"])
    assert q[0].tolist() == g["codes"]
    assert np.allclose(s[0], g["scales"], rtol=1e-15, atol=0)


@pytest.mark.parametrize("ex", GOLD["kv"], ids=lambda e: e["name"])
def test_kv_worked_examples(ex):
    v = np.array(ex["v"], dtype=np.float16).reshape(1, 1, 4)
    q, step, z, _, _ = O.kv_quantize(v)
    assert step[0, 0] == pytest.approx(ex["step"], rel=1e-15)
    assert int(z[0, 0]) == ex["zero"]
    assert q[0, 0].tolist() == ex["codes"]
    assert O.pack_int4(q[0])[0].tolist() == ex["packed"]


def test_gemm_worked_example():
    g = GOLD["gemm"]
    acc = O.int_gemm(np.array(g["qa"]), np.array(g["qw"]))
    assert acc.tolist() == g["acc"]
    y = O.dequantize_output(acc, np.array(g["sx"]), np.array(g["sw"]))
    assert y.tolist() == g["y"]


# ---------------------------------------------------------------- closed forms of the rotate+quant path

@pytest.mark.parametrize("n,k,c", [(16, 3, 2.5), (512, 100, -7.0), (4096, 4095, 1000.0)])
def test_one_hot_row_closed_form(n, k, c):
    """x = c e_k: every |y_i| = |c|/sqrt(n), s = |c|/(7 sqrt(n)), codes are
    +-7 with sign d_k H[k, i] sign(c)."""
    d = np.where(np.random.default_rng(n).random(n) < 0.5, -1, 1)
    x = np.zeros((1, n), dtype=np.float16)
    x[0, k] = c
    cf = float(np.float16(c))
    r = O.rotation_matrix(n, signs=d)
    y = O.rotate(x, r)
    assert np.allclose(np.abs(y), abs(cf) / np.sqrt(n), rtol=1e-14)
    q, s, _ = O.quantize_symmetric(y)
    assert s[0] == pytest.approx(abs(cf) / (7 * np.sqrt(n)), rel=1e-14)
    h = O.sylvester_hadamard(n)
    assert np.array_equal(q[0], (7 * d[k] * h[k] * np.sign(cf)).astype(np.int8))


@pytest.mark.parametrize("n,c", [(8, 3.0), (1024, -0.25)])
def test_constant_row_closed_form(n, c):
    """x = c 1, no signs: y = c sqrt(n) e_0, code 7 sign(c) at index 0, zeros elsewhere."""
    x = np.full((1, n), c, dtype=np.float16)
    y = O.rotate(x, O.rotation_matrix(n))
    e = np.zeros(n)
    e[0] = c * np.sqrt(n)
    assert np.allclose(y[0], e, atol=1e-12)
    q, _, _ = O.quantize_symmetric(y)
    expect = np.zeros(n, dtype=np.int8)
    expect[0] = 7 * np.sign(c)
    assert np.array_equal(q[0], expect)


# ---------------------------------------------------------------- RTN invariants

@pytest.mark.parametrize("group", [0, 128])
def test_rtn_invariants(group):
    y = np.random.default_rng(1).laplace(size=(64, 512)) * np.where(np.arange(512) % 97 == 0, 50, 1)
    q, s, t = O.quantize_symmetric(y, group)
    assert q.min() >= -7 and q.max() <= 7          # range [-8, 7], in fact [-7, 7]
    g = 512 if group == 0 else group
    qg = np.abs(q.reshape(64, -1, g))
    assert np.all(qg.max(axis=2) == 7)             # the absmax element maps to +-7
    deq = O.dequantize_symmetric(q, s, group)
    sb = np.repeat(s.reshape(64, -1), g, axis=1)
    assert np.all(np.abs(y - deq) <= sb / 2 * (1 + 1e-12))   # |y - s q| <= s/2
    assert np.allclose(t * sb, y, rtol=1e-12)     # pre-rounding values are y/s


def test_rtn_scale_invariance():
    """Scaling R by c > 0 scales s by c and leaves codes unchanged (up to .5 ties)."""
    y = np.random.default_rng(2).standard_normal((32, 256))
    q1, s1, t1 = O.quantize_symmetric(y)
    q2, s2, _ = O.quantize_symmetric(y * 3.0)
    assert np.allclose(s2, 3 * s1, rtol=1e-14)
    safe = np.abs(np.abs(t1 - np.floor(t1)) - 0.5) > 1e-9
    assert np.array_equal(q1[safe], q2[safe])


def test_group_equal_to_row_width_is_per_token():
    y = np.random.default_rng(3).standard_normal((16, 256))
    q0, s0, _ = O.quantize_symmetric(y, 0)
    q1, s1, _ = O.quantize_symmetric(y, 256)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1[:, 0])


def test_all_zero_row_and_group():
    y = np.zeros((2, 256))
    y[1, 128:] = np.linspace(-1, 1, 128)
    q, s, _ = O.quantize_symmetric(y, 128)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0 and s[1, 1] > 0
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)


def test_rint_is_half_even():
    y = np.array([[7.0, 2.5, -0.5, 1.5, -2.5, 3.5, 0.49999999999, -6.5]])
    q, s, _ = O.quantize_symmetric(y)
    assert s[0] == 1.0
    assert q[0].tolist() == [7, 2, 0, 2, -2, 4, 0, -6]


# ---------------------------------------------------------------- packing

def test_pack_unpack_roundtrip_and_order():
    q = np.array([[0, 1, -1, 7, -8, -7, 3, -3]], dtype=np.int8)
    b = O.pack_int4(q)
    # low nibble = even index, two's complement
    assert b[0].tolist() == [0x10, 0x7F, 0x98, 0xD3]
    assert np.array_equal(O.unpack_int4(b), q)
    allq = np.array([list(itertools.product(range(-8, 8), repeat=2))], dtype=np.int8).reshape(1, -1)
    assert np.array_equal(O.unpack_int4(O.pack_int4(allq)), allq)
    u = np.arange(16, dtype=np.uint8).reshape(1, 16)
    assert np.array_equal(O.unpack_uint4(O.pack_int4(u)), u)


# ---------------------------------------------------------------- GEMM

def test_int_gemm_brute_force():
    qa = W.make_random_codes(5, 12, 1)
    qw = W.make_random_codes(3, 12, 2)
    acc = O.int_gemm(qa, qw)
    for t in range(5):
        for n in range(3):
            assert acc[t, n] == sum(int(qa[t, k]) * int(qw[n, k]) for k in range(12))


def test_int_gemm_matches_float_blas_when_exact():
    qa = W.make_random_codes(64, 4096, 3)
    qw = W.make_random_codes(48, 4096, 4)
    acc = O.int_gemm(qa, qw)
    ref = qa.astype(np.float64) @ qw.astype(np.float64).T     # exact: |acc| < 2^53
    assert np.array_equal(acc, ref.astype(np.int64))
    assert np.abs(acc).max() <= 64 * 4096


def test_group_gemm_sums_to_per_channel():
    qa = W.make_random_codes(16, 512, 5)
    qw = W.make_random_codes(8, 512, 6)
    accg = O.int_gemm(qa, qw, 128)
    assert accg.shape == (4, 16, 8)
    assert np.array_equal(accg.sum(axis=0), O.int_gemm(qa, qw))
    assert np.array_equal(accg[2], O.int_gemm(qa[:, 256:384], qw[:, 256:384]))


@pytest.mark.parametrize("group", [0, 128])
def test_dequant_equals_matmul_of_dequantized_operands(group):
    """dequant(acc) == (s_x q_x)(s_w q_w)^T, the same number formed another way."""
    rng = np.random.default_rng(7)
    qa = W.make_random_codes(12, 256, 8)
    qw = W.make_random_codes(10, 256, 9)
    if group:
        sx = rng.random((12, 2)) + 0.1
        sw = rng.random((10, 2)) + 0.1
    else:
        sx = rng.random(12) + 0.1
        sw = rng.random(10) + 0.1
    y = O.dequantize_output(O.int_gemm(qa, qw, group), sx, sw, group)
    ref = O.dequantize_symmetric(qa, sx, group) @ O.dequantize_symmetric(qw, sw, group).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_weight_quant_is_per_output_channel():
    """W' = R^T W then one scale per column of W' (output channel): a transposed
    operand would give scales per input feature instead."""
    c = W.CONFIGS["c1"]
    w = W.make_w(c).astype(np.float64)
    w[:, 5] *= 100.0                                   # one loud output channel
    r = O.rotation_matrix(c.K, signs=W.make_signs(c))
    q, s = O.quantize_weights(O.rotate_weights(w, r))
    assert q.shape == (c.N, c.K) and s.shape == (c.N,)
    col5 = (r.T @ w)[:, 5]
    assert s[5] == pytest.approx(np.abs(col5).max() / 7, rel=1e-14)
    assert s[5] > 50 * np.median(s)


# ---------------------------------------------------------------- the method's claims on planted outliers

def _rel_err(out, ref):
    return np.linalg.norm(out - ref) / np.linalg.norm(ref)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rotation_lowers_int4_error_c1(seed):
    """QuaRot abstract / summary: rotating removes outliers and makes 4-bit
    quantization easier.  c1 shape with 4 planted outlier channels x50."""
    base = W.CONFIGS["c1"]
    c = W.Config(**{**base.__dict__, "index": 100 + seed})
    x = W.make_x(c)
    w = W.make_w(c)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    rot = O.linear_w4a4(x, w, O.rotation_matrix(c.K, signs=W.make_signs(c)))["out"]
    plain = O.linear_w4a4(x, w, np.eye(c.K))["out"]
    e_rot, e_plain = _rel_err(rot, ref), _rel_err(plain, ref)
    assert e_rot < e_plain
    assert e_rot < 0.2 and e_plain > 0.22


def test_rotation_lowers_int4_error_c2_subset():
    c = W.CONFIGS["c2"]
    x = W.make_x(c, rows=np.arange(256))
    w = W.make_w(c)[:, :512]
    ref = x.astype(np.float64) @ w.astype(np.float64)
    r = O.rotation_matrix(c.K, signs=W.make_signs(c))
    rot = O.linear_w4a4(x, w, r)["out"]
    plain = O.linear_w4a4(x, w, np.eye(c.K))["out"]
    assert _rel_err(rot, ref) < _rel_err(plain, ref)


def test_kron_rotation_lowers_int4_error_c3_subset():
    c = W.CONFIGS["c3"]
    x = W.make_x(c, rows=np.arange(64))
    w = W.make_w(c, cols=np.arange(256))
    ref = x.astype(np.float64) @ w.astype(np.float64)
    r = O.rotation_matrix(c.K, 64, dense=W.make_dense(c, dtype=np.float64))
    rot = O.linear_w4a4(x, w, r)["out"]
    plain = O.linear_w4a4(x, w, np.eye(c.K))["out"]
    assert _rel_err(rot, ref) < _rel_err(plain, ref)


def test_group128_lowers_error_vs_per_token_c4_shape():
    """QuaRot summary, Key points: group size 128 reduces the loss."""
    c = W.CONFIGS["c4"]
    x = W.make_x(c, rows=np.arange(32))
    w = W.make_w(c, cols=np.arange(128))
    ref = x.astype(np.float64) @ w.astype(np.float64)
    r = O.rotation_matrix(c.K, signs=W.make_signs(c))
    g128 = O.linear_w4a4(x, w, r, 128)["out"]
    tok = O.linear_w4a4(x, w, r, 0)["out"]
    plain = O.linear_w4a4(x, w, np.eye(c.K), 0)["out"]
    assert _rel_err(g128, ref) < _rel_err(tok, ref) < _rel_err(plain, ref)


# ---------------------------------------------------------------- KV quantizer

def test_kv_invariants():
    k, v = W.make_kv("c5")
    for t in (k, v):
        q, step, z, _, _ = O.kv_quantize(t)
        assert q.min() >= 0 and q.max() <= 15 and z.min() >= 0 and z.max() <= 15
        y = t.astype(np.float64) @ O.rotation_matrix(128)
        err = np.abs(y - O.kv_dequantize(q, step, z))
        assert np.all(err <= step[..., None] / 2 * (1 + 1e-9))


def test_kv_zero_maps_to_zero_point():
    """A rotated value of exactly 0 is stored as the zero point."""
    v = np.zeros((1, 1, 8), dtype=np.float16)
    v[0, 0, :4] = [1, 2, 3, 4]
    v[0, 0, 4:] = [1, 2, 3, 4]
    # y = v . H_8/sqrt(8): y[j] = 0 for j >= 4 since the two halves are equal
    q, step, z, _, _ = O.kv_quantize(v)
    y = v.astype(np.float64)[0, 0] @ O.rotation_matrix(8)
    assert np.allclose(y[4:], 0, atol=1e-15)
    assert np.all(q[0, 0, 4:] == z[0, 0])


def test_kv_all_zero_head():
    q, step, z, _, _ = O.kv_quantize(np.zeros((2, 3, 128), dtype=np.float16))
    assert np.all(q == 0) and np.all(step == 0) and np.all(z == 0)


def test_kv_rotation_lowers_error():
    """QuaRot abstract: the rotation applied to the KV cache; rotated 4-bit KV
    reconstruction beats unrotated on heads with outlier dims."""
    k, _ = W.make_kv("c5")
    x = k.astype(np.float64)
    r = O.rotation_matrix(128)
    q, step, z, _, _ = O.kv_quantize(k)
    rec_rot = O.kv_dequantize(q, step, z) @ r.T
    # unrotated: same asymmetric quantizer on the raw vectors
    lo = np.minimum(x.min(2), 0)
    hi = np.maximum(x.max(2), 0)
    st = (hi - lo) / 15
    zz = np.rint(-lo / st)
    qq = np.clip(np.rint(x / st[..., None]) + zz[..., None], 0, 15)
    rec_plain = (qq - zz[..., None]) * st[..., None]
    assert _rel_err(rec_rot, x) < 0.5 * _rel_err(rec_plain, x)


# ---------------------------------------------------------------- generators

def test_generators_are_seeded_and_row_subsets_consistent():
    c = W.CONFIGS["c2"]
    a = W.make_x(c, rows=np.array([5, 2047, 0]))
    b = W.make_x(c)
    assert np.array_equal(a, b[[5, 2047, 0]])
    cols = W.outlier_columns(c)
    assert cols.size == 8
    assert np.abs(b[:, cols].astype(np.float64)).mean() > 50 * np.abs(b.astype(np.float64)).mean(axis=0).min()
    assert np.array_equal(W.make_signs(c), W.make_signs(c))


# ------------------------------------------------------------ decode attention

def _attn_inputs(b, t, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 16, size=(b, t, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 16, size=(b, t, hkv, d)).astype(np.uint8)
    ks = rng.uniform(0.02, 0.3, size=(b, t, hkv))
    vs = rng.uniform(0.02, 0.3, size=(b, t, hkv))
    kz = rng.integers(0, 16, size=(b, t, hkv))
    vz = rng.integers(0, 16, size=(b, t, hkv))
    q = rng.standard_normal((b, hq, d)).astype(np.float16)
    return q, kc, ks, kz, vc, vs, vz


def test_attn_worked_example():
    """D = 2, R = H_2 / sqrt(2), unit steps, zero points 0, sm_scale 1.
    Rotated keys (0, 0) and (1, 1) reconstruct to K0 = 0, K1 = (sqrt2, 0);
    q = (ln 3 / sqrt2, 0) scores them 0 and ln 3, so p = (1/4, 3/4).  Rotated
    values (2, 0) and (0, 2) reconstruct to (sqrt2, sqrt2) and (sqrt2, -sqrt2):
    out = (sqrt2, -sqrt2 / 2)."""
    one = np.ones((1, 2, 1))
    zero = np.zeros((1, 2, 1), np.int64)
    kc = np.array([[[[0, 0]], [[1, 1]]]], np.uint8)
    vc = np.array([[[[2, 0]], [[0, 2]]]], np.uint8)
    q = np.array([[[np.log(3) / np.sqrt(2), 0.0]]])
    out = O.kv_attention_decode(q, kc, one, zero, vc, one, zero, sm_scale=1.0)
    assert out[0, 0] == pytest.approx([np.sqrt(2), -np.sqrt(2) / 2], abs=1e-14)


def test_attn_brute_force_tiny():
    """Pure-Python loops from the definition: unpack, dequantize, undo the
    rotation entry by entry (signs and popcount Hadamard), score, softmax with
    math.exp, weighted sum; ragged lengths and grouped query heads."""
    import math
    b_, t_, hq, hkv, d = 2, 3, 4, 2, 8
    q, kc, ks, kz, vc, vs, vz = _attn_inputs(b_, t_, hq, hkv, d, 5)
    signs = [1, -1, -1, 1, 1, 1, -1, 1]
    lens = [3, 2]
    sm = 0.7

    def orig(codes, step, zero, b, t, h):
        rot = [(int(codes[b, t, h, j]) - int(zero[b, t, h])) * float(step[b, t, h]) for j in range(d)]
        # rotated = v R with R[i][j] = signs[i] H[i][j] / sqrt(d); v = rotated R^T
        return [sum(rot[j] * signs[i] * (-1) ** bin(i & j).count("1") for j in range(d)) / math.sqrt(d)
                for i in range(d)]

    got = O.kv_attention_decode(q, kc, ks, kz, vc, vs, vz, lens=lens, signs=np.array(signs), sm_scale=sm)
    for b in range(b_):
        for h in range(hq):
            g = h // (hq // hkv)
            sc = [sm * sum(float(q[b, h, i]) * k for i, k in enumerate(orig(kc, ks, kz, b, t, g)))
                  for t in range(lens[b])]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            want = [sum(e[t] * orig(vc, vs, vz, b, t, g)[i] for t in range(lens[b])) / sum(e) for i in range(d)]
            assert got[b, h] == pytest.approx(want, rel=1e-12, abs=1e-12)


def test_attn_single_token_and_uniform_cases():
    q, kc, ks, kz, vc, vs, vz = _attn_inputs(2, 5, 4, 4, 128, 6)
    r = O.rotation_matrix(128)
    vrec = O.kv_dequantize(vc, vs, vz) @ r.T
    # one token: softmax of a single score is 1 -> out = that token's value
    out = O.kv_attention_decode(q, kc, ks, kz, vc, vs, vz, lens=[1, 1])
    assert np.allclose(out, vrec[:, 0], rtol=0, atol=1e-12)
    # identical keys (or sm_scale 0): uniform weights -> mean of the values
    kc2 = np.repeat(kc[:, :1], 5, axis=1)
    ks2 = np.repeat(ks[:, :1], 5, axis=1)
    kz2 = np.repeat(kz[:, :1], 5, axis=1)
    out = O.kv_attention_decode(q, kc2, ks2, kz2, vc, vs, vz)
    assert np.allclose(out, vrec.mean(axis=1), rtol=0, atol=1e-12)
    out = O.kv_attention_decode(q, kc, ks, kz, vc, vs, vz, sm_scale=0.0)
    assert np.allclose(out, vrec.mean(axis=1), rtol=0, atol=1e-12)
    # empty sequence -> zeros
    out = O.kv_attention_decode(q, kc, ks, kz, vc, vs, vz, lens=[0, 3])
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


def test_attn_rotated_domain_identity():
    """R is orthogonal, so attention in the rotated basis - query rotated by R,
    cache used as stored, output rotated back by R^T - equals the oracle's
    original-basis attention (the identity the GPU kernel uses)."""
    signs = np.where(np.random.default_rng(3).random(128) < 0.5, -1, 1)
    q, kc, ks, kz, vc, vs, vz = _attn_inputs(1, 7, 8, 2, 128, 7)
    r = O.rotation_matrix(128, signs=signs)
    krot = O.kv_dequantize(kc, ks, kz)
    vrot = O.kv_dequantize(vc, vs, vz)
    qr_ = q.astype(np.float64) @ r
    want = np.zeros((1, 8, 128))
    for h in range(8):
        s = krot[0, :, h // 4] @ qr_[0, h] / np.sqrt(128)
        p = np.exp(s - s.max())
        want[0, h] = (p / p.sum()) @ vrot[0, :, h // 4] @ r.T
    got = O.kv_attention_decode(q, kc, ks, kz, vc, vs, vz, signs=signs)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------- 6- and 8-bit RTN variants

@pytest.mark.parametrize("bits,codes", [(8, [127, -64, 32, 13]), (6, [31, -16, 8, 3]), (4, [7, -4, 2, 1])])
def test_rtn_bits_worked_example(bits, codes):
    """y = (1, -0.5, 0.25, 0.1): s = 1/qmax, y/s = qmax * y.  8 bits: 127,
    -63.5 (a tie, to even: -64), 31.75, 12.7.  6 bits: 31, -15.5 (-16), 7.75,
    3.1.  4 bits: 7, -3.5 (-4), 1.75, 0.7."""
    qmax = 2 ** (bits - 1) - 1
    q, s, t = O.quantize_symmetric(np.array([[1.0, -0.5, 0.25, 0.1]]), bits=bits)
    assert q[0].tolist() == codes
    assert s[0] == pytest.approx(1.0 / qmax, rel=1e-15)


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("group", [0, 128])
def test_rtn_bits_invariants(bits, group):
    qmax = 2 ** (bits - 1) - 1
    y = np.random.default_rng(9).laplace(size=(32, 512)) * np.where(np.arange(512) % 89 == 0, 40, 1)
    q, s, t = O.quantize_symmetric(y, group, bits)
    assert q.min() >= -qmax and q.max() <= qmax
    g = 512 if group == 0 else group
    assert np.all(np.abs(q.reshape(32, -1, g)).max(axis=2) == qmax)
    deq = O.dequantize_symmetric(q, s, group)
    sb = np.repeat(s.reshape(32, -1), g, axis=1)
    assert np.all(np.abs(y - deq) <= sb / 2 * (1 + 1e-12))


def test_rtn_bits_one_hot_closed_form():
    """x = c e_k under D H / sqrt(n): every |y_i| = |c| / sqrt(n), so every code
    is +-qmax with the sign of d_k H[k, i] c."""
    n, k, c = 512, 37, -3.0
    d = np.where(np.random.default_rng(4).random(n) < 0.5, -1, 1)
    x = np.zeros((1, n))
    x[0, k] = c
    y = O.rotate(x, O.rotation_matrix(n, signs=d))
    for bits in (6, 8):
        qmax = 2 ** (bits - 1) - 1
        q, s, _ = O.quantize_symmetric(y, bits=bits)
        expect = qmax * np.sign(c) * d[k] * np.array([O.hadamard_entry(k, i) for i in range(n)])
        assert np.array_equal(q[0], expect.astype(np.int8))
        assert s[0] == pytest.approx(abs(c) / np.sqrt(n) / qmax, rel=1e-12)


def test_rtn_6_8_bits_near_lossless():
    """QuaRot abstract: plain RTN at 6 and 8 bits is (near) lossless.  On the
    c1 layer with planted outliers the rotated output error falls about 4x
    per two bits: ~16% (4 bits), ~3.6% (6), ~0.9% (8), and rotation still
    beats no rotation at every width."""
    c = W.CONFIGS["c1"]
    x, w = W.make_x(c), W.make_w(c)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    r = O.rotation_matrix(c.K, signs=W.make_signs(c))
    err = {b: _rel_err(O.linear_w4a4(x, w, r, bits=b)["out"], ref) for b in (4, 6, 8)}
    plain = {b: _rel_err(O.linear_w4a4(x, w, np.eye(c.K), bits=b)["out"], ref) for b in (4, 6, 8)}
    assert err[8] < 0.015 and err[6] < 0.05 and err[4] > 0.1
    assert 2.5 < err[4] / err[6] < 6 and 2.5 < err[6] / err[8] < 6
    assert all(err[b] < plain[b] for b in (4, 6, 8))


# ------------------------------------------------- fused feed-forward activation

def test_silu_closed_forms():
    """silu(0) = 0; silu(g) - silu(-g) = g (since sigma(g) + sigma(-g) = 1);
    silu(ln 3) = (3/4) ln 3; silu -> g for large g, -> 0 for very negative g."""
    g = np.linspace(-9, 9, 37)
    assert O.silu(0.0) == 0.0
    assert np.allclose(O.silu(g) - O.silu(-g), g, rtol=0, atol=1e-14)
    assert O.silu(np.log(3)) == pytest.approx(0.75 * np.log(3), rel=1e-15)
    assert O.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(-40.0)) < 1e-15


def test_swiglu_fp16_rounding():
    """The product is rounded once, to the nearest fp16: exact cases stay
    exact (silu(ln 3) * 4 / ln 3 = 3, silu(0) * 7 = 0); 30 (1 + 2^-11) =
    30.0146... lies 0.00098 below the fp16 neighbour 30.015625 (fp16 spacing
    at 30 is 2^-6) and 0.0146 above 30, so it rounds up."""
    g = np.array([np.log(3), 0.0, 40.0])
    u = np.array([4 / np.log(3), 7.0, 0.75 * (1.0 + 2 ** -11)])   # silu(40) = 40 in fp64
    x = O.swiglu_fp16(g, u)
    assert x.dtype == np.float16
    assert x[0] == np.float16(3.0) and x[1] == 0
    assert float(x[2]) == 30.015625
