"""CPU oracle for QuaRot's per-linear-layer inference hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
cpu_baseline leg may import this package.  It shares no code with the GPU
library (rotation_bit_quantized_amd) and imports nothing from it; the two
meet only in the seeded input generators (package ``workloads``).

Everything here is the plain definition, written for a reader to check by eye:
explicit Sylvester / Kronecker matrices in fp64, the quantizers step by step,
an int64 matrix product and an fp64 dequantization.  The one fast routine,
``fwht``, exists only for speed on large row subsets and is pinned against the
explicit matrix product in the tests.

Sources (pages as titled):
  [QuaRot-abs]  "QuaRot: Outlier-free 4-bit inference in rotated LLMs", ISTA
                Research Explorer record, abstract.
  [QuaRot-sum]  "QuaRot: Outlier-Free 4-Bit Inference in Rotated LLMs",
                Elamur Research summary: "Summary", "Key points".
  [DuQuant]     "DuQuant: Distributing Outliers via Dual Transformation Makes
                Stronger Quantized LLMs" (ChapterPal): Knowl 1 (linear-layer
                identity Y = XW = (XG)(G^-1 W)), Knowl 12 (fixed Hadamard
                rotations normalised by 1/sqrt(2^n) before per-head asymmetric
                quantization; the asymmetric step (gamma max - beta min)/(2^b-1)).
  [QuIP]        "QuIP: 2-Bit Quantization of Large Language Models With
                Guarantees" (Uptrust): abstract (random orthogonal
                pre-/post-processing), citing-paper quote from QuIP# (two-factor
                Kronecker incoherence).

Readings where the pages are silent (each repeated where it is used):
  R1 Sylvester construction, natural order, normalised by 1/sqrt(n).
  R2 The random signs D act on the input side: R = D . H / sqrt(n).
  R3 Non-power-of-two widths n = p*m use R = (H_p / sqrt(p)) kron O_m, with
     the m-index fastest in memory (k = i*m + a).
  R4 Symmetric scale s = max|y| / 7, code = clip(rint(y / s), -8, 7).
  R5 Rounding is round-half-to-even (numpy.rint).
  R6 An all-zero row or group gets s = 0 and all-zero codes.
  R7 Scales are fp32 in storage; the oracle keeps them in fp64.
  R9 A group is a contiguous block of the rotated K index, for activations
     (per token) and weights (per output channel).
  R10 Two codes per byte, low nibble = even index; two's complement for the
     symmetric codes, unsigned for the KV codes.
  R12 KV: per (token, head) y = v . H_D / sqrt(D) (no signs unless given),
     lo = min(min y, 0), hi = max(max y, 0), step = (hi - lo)/15,
     z = rint(-lo / step), q = clip(rint(y / step) + z, 0, 15); step 0 gives
     step = 0, z = 0, q = 0.
  R13 Output dequantization in fp64: y = acc * s_x * s_w, or for groups the sum
     over groups of acc_g * s_x[g] * s_w[g].
  R19 Decode attention over the 4-bit KV cache: the query stays in full
     precision, keys and values are the dequantized cache rotated back to the
     original basis, softmax is unquantized; out = softmax(c q K^T) V over the
     first len tokens of the sequence, query head h reading KV head
     h // (Hq / Hkv); an empty sequence gives zeros.
  R20 6- and 8-bit variants: the same symmetric RTN with qmax = 2^(b-1) - 1
     (31, 127) in place of 7; codes stored one per byte (int8) and multiplied
     as int8, no packing.
  R21 The activation feeding down_proj, fused before the rotation: LLaMA-2's
     gated FFN activation x = silu(gate) * up, silu(g) = g / (1 + e^-g),
     rounded to fp16 (the value an unfused pipeline would hand on), then
     rotated and quantized as any activation row.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "sylvester_hadamard", "hadamard_entry", "fwht", "rotation_matrix", "rotate", "rotate_kron",
    "quantize_symmetric", "pack_int4", "unpack_int4", "unpack_uint4",
    "rotate_weights", "quantize_weights", "int_gemm", "dequantize_output",
    "dequantize_symmetric", "linear_w4a4", "kv_quantize", "kv_dequantize",
    "kv_attention_decode", "silu", "swiglu_fp16",
]


# --------------------------------------------------------------------------
# Hadamard matrices and rotations
# --------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_n (int64), natural order (R1).

    H_1 = [1];  H_2k = [[H_k, H_k], [H_k, -H_k]].  [QuaRot-sum] Summary
    (random orthogonal Hadamard matrices); [DuQuant] Knowl 12 (entries
    +-1/sqrt(2^n) after normalisation)."""
    if n < 1 or n & (n - 1):
        raise ValueError(f"Hadamard size must be a power of two, got {n}")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_entry(i, j):
    """Closed form of the Sylvester entry: (-1)^popcount(i & j)."""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    v = i & j
    parity = np.zeros(np.broadcast(i, j).shape, dtype=np.int64)
    while np.any(v):
        parity ^= v & 1
        v = v >> 1
    return 1 - 2 * parity


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis, fp64:
    returns x @ H_n.  Only a speed-up of ``x @ sylvester_hadamard(n)`` for big
    row subsets; the tests pin it to the explicit product."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    if n & (n - 1):
        raise ValueError("fwht needs a power-of-two length")
    lead = y.shape[:-1]
    h = 1
    while h < n:
        y = y.reshape(*lead, n // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :]
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*lead, n)
        h *= 2
    return y


def rotation_matrix(n: int, had_n: int | None = None, dense=None, signs=None) -> np.ndarray:
    """The orthogonal rotation R (fp64 [n, n]) with rotated activations y = x @ R.

    Power of two (dense is None):  R = D . H_n / sqrt(n)            (R1, R2)
    Kronecker (n = had_n * m):     R = D . ((H_p / sqrt(p)) kron O)  (R3)
    with D = diag(signs) (identity when signs is None).

    [QuaRot-abs]: rotations that leave the output unchanged; [QuaRot-sum]
    Summary: random orthogonal Hadamard matrices, a few applied online;
    [QuIP] abstract: multiplication by random orthogonal matrices; QuIP# quote
    on the same page: two-factor Kronecker construction."""
    had_n = n if had_n is None else had_n
    h = sylvester_hadamard(had_n).astype(np.float64) / np.sqrt(had_n)
    if dense is None:
        if had_n != n:
            raise ValueError("without a dense factor had_n must equal n")
        r = h
    else:
        o = np.asarray(dense, dtype=np.float64)
        if o.shape != (n // had_n, n // had_n) or had_n * o.shape[0] != n:
            raise ValueError("dense factor shape does not match n / had_n")
        r = np.kron(h, o)
    if signs is not None:
        d = np.asarray(signs, dtype=np.float64)
        if d.shape != (n,) or not np.all(np.abs(d) == 1):
            raise ValueError("signs must be a +-1 vector of length n")
        r = d[:, None] * r
    return r


def rotate(x, r: np.ndarray) -> np.ndarray:
    """Rotated activations y = x @ R in fp64 (fp16 input converted exactly)."""
    return np.asarray(x).astype(np.float64) @ r


def rotate_kron(x, had_n: int, dense, signs=None) -> np.ndarray:
    """y = x @ rotation_matrix(n, had_n, dense, signs), n = had_n * m, without
    forming the n x n matrix (for widths where it does not fit in memory).

    With the m-index fastest (k = i*m + a, R3) the Kronecker entry is
    R[i*m + a, j*m + b] = H[i, j] / sqrt(p) * O[a, b], so x viewed as X[i, a]
    gives Y = H_p^T X O / sqrt(p) (H_p is symmetric); the signs scale x first
    (R2).  The tests pin it to the explicit product."""
    x = np.asarray(x).astype(np.float64)
    o = np.asarray(dense, dtype=np.float64)
    m = o.shape[0]
    n = had_n * m
    if x.shape[-1] != n:
        raise ValueError("row width does not match had_n * m")
    if signs is not None:
        x = x * np.asarray(signs, dtype=np.float64)
    z = x.reshape(x.shape[0], had_n, m) @ o          # X[i] O for every i
    y = fwht(np.swapaxes(z, 1, 2)) / np.sqrt(had_n)  # over i, for every column b
    return np.swapaxes(y, 1, 2).reshape(x.shape[0], n)


# --------------------------------------------------------------------------
# Symmetric round-to-nearest 4-bit quantization and nibble packing
# --------------------------------------------------------------------------

def quantize_symmetric(y: np.ndarray, group: int = 0, bits: int = 4):
    """Symmetric b-bit RTN of each row of y (group 0) or of each contiguous
    ``group``-block of a row.  [QuaRot-sum] Key points: activations quantized
    on the fly with round-to-nearest; group size 128 as the group-wise option.
    [QuaRot-abs]: plain round-to-nearest at 6 and 8 bits as well (R20).

    Returns (codes int8 [rows, n], scales fp64 [rows] or [rows, n/group],
    pre-rounding values y/s as fp64 [rows, n]).  With qmax = 2^(b-1) - 1:
      s = max|y| / qmax                     (R4; the group maximum maps to +-qmax)
      q = clip(rint(y / s), -qmax-1, qmax)  (R5)
      max|y| = 0  ->  s = 0, q = 0          (R6)
    """
    if bits not in (4, 6, 8):
        raise ValueError("bits must be 4, 6 or 8")
    qmax = 2 ** (bits - 1) - 1
    y = np.asarray(y, dtype=np.float64)
    rows, n = y.shape
    g = n if group == 0 else group
    if n % g:
        raise ValueError("group must divide the row width")
    yg = y.reshape(rows, n // g, g)
    amax = np.abs(yg).max(axis=2)
    s = amax / qmax
    t = np.zeros_like(yg)
    nz = s > 0
    t[nz] = yg[nz] / s[nz][:, None]
    q = np.clip(np.rint(t), -qmax - 1, qmax).astype(np.int8)
    scales = s[:, 0] if group == 0 else s
    return q.reshape(rows, n), scales, t.reshape(rows, n)


def dequantize_symmetric(q: np.ndarray, s: np.ndarray, group: int = 0) -> np.ndarray:
    """q * s per row or per group (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    rows, n = q.shape
    if group == 0:
        return q * np.asarray(s, dtype=np.float64)[:, None]
    return (q.reshape(rows, n // group, group) * np.asarray(s, np.float64)[:, :, None]).reshape(rows, n)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, low nibble = even index (R10)."""
    q = np.asarray(q).astype(np.int64)
    if q.shape[-1] % 2:
        raise ValueError("row width must be even")
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4 for two's-complement codes: int8 in [-8, 7]."""
    b = np.asarray(b, dtype=np.int64)
    nib = np.stack([b & 0xF, b >> 4], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


def unpack_uint4(b: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4 for unsigned codes: uint8 in [0, 15]."""
    b = np.asarray(b, dtype=np.int64)
    return np.stack([b & 0xF, b >> 4], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2).astype(np.uint8)


def silu(g) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in fp64 (the gate nonlinearity of LLaMA-2's
    feed-forward block; R21)."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def swiglu_fp16(gate, up) -> np.ndarray:
    """x = fp16(silu(gate) * up): the feed-forward activation whose rotation
    and quantization the fused call performs (R21; [QuaRot-abs]: the
    activations of the feed-forward components are rotated as well).  fp16
    round to nearest even of the fp64 product."""
    return (silu(gate) * np.asarray(up, dtype=np.float64)).astype(np.float16)


# --------------------------------------------------------------------------
# Offline weight preparation
# --------------------------------------------------------------------------

def rotate_weights(w, r: np.ndarray) -> np.ndarray:
    """W' = R^T . W (fp64 [K, N]).  [DuQuant] Knowl 1: with Y = XW = (XG)(G^-1 W)
    the inverse transform is folded into W offline; R orthogonal gives
    G^-1 = R^T."""
    return r.T @ np.asarray(w).astype(np.float64)


def quantize_weights(w_rot: np.ndarray, group: int = 0, bits: int = 4):
    """Symmetric RTN of each output channel (column of W'), or of each
    ``group``-block of it along K (R4, R9).  [QuaRot-sum] Key points: RTN as the
    4-bit weight quantizer next to GPTQ (the RTN-GPTQ gap); [QuaRot-abs]: RTN
    at 6 and 8 bits (R20).

    Returns (codes int8 [N, K], scales fp64 [N] or [N, K/group]) in the
    output-channel-major layout the GEMM consumes."""
    q, s, _ = quantize_symmetric(np.asarray(w_rot, dtype=np.float64).T, group, bits)
    return q, s


# --------------------------------------------------------------------------
# Integer GEMM and dequantization
# --------------------------------------------------------------------------

def int_gemm(qa: np.ndarray, qw: np.ndarray, group: int = 0) -> np.ndarray:
    """Exact integer products (int64).  [QuaRot-abs]: all matrix multiplications
    in 4 bits.  qa [M, K] int codes, qw [N, K] int codes.

    group 0: acc[t, n] = sum_k qa[t, k] * qw[n, k]            -> [M, N]
    group g: acc[j, t, n] = the same sum over k in block j     -> [K/g, M, N]
    """
    a = np.asarray(qa, dtype=np.int64)
    w = np.asarray(qw, dtype=np.int64)
    if a.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    if group == 0:
        return a @ w.T
    k = a.shape[1]
    return np.stack([a[:, j:j + group] @ w[:, j:j + group].T for j in range(0, k, group)])


def dequantize_output(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, group: int = 0) -> np.ndarray:
    """fp64 output from integer sums (R13):
    group 0: y = acc * s_x[:, None] * s_w[None, :]
    group g: y = sum_j acc[j] * s_x[:, j, None] * s_w[None, :, j]"""
    sx = np.asarray(sx, dtype=np.float64)
    sw = np.asarray(sw, dtype=np.float64)
    if group == 0:
        return np.asarray(acc, dtype=np.float64) * sx[:, None] * sw[None, :]
    y = np.zeros(acc.shape[1:], dtype=np.float64)
    for j in range(acc.shape[0]):
        y += acc[j].astype(np.float64) * sx[:, j, None] * sw[None, :, j]
    return y


def linear_w4a4(x, w, r: np.ndarray, group: int = 0, bits: int = 4):
    """The whole layer as the oracle computes it: rotate x, quantize it, rotate
    and quantize W offline, integer GEMM, fp64 dequantization (4-bit by
    default; ``bits`` 6 or 8 for the R20 variants).  Returns a dict with every
    intermediate."""
    y = rotate(x, r)
    qx, sx, tx = quantize_symmetric(y, group, bits)
    qw, sw = quantize_weights(rotate_weights(w, r), group, bits)
    acc = int_gemm(qx, qw, group)
    out = dequantize_output(acc, sx, sw, group)
    return dict(y=y, qx=qx, sx=sx, tx=tx, qw=qw, sw=sw, acc=acc, out=out)


# --------------------------------------------------------------------------
# KV-cache quantizer
# --------------------------------------------------------------------------

def kv_quantize(kv, signs=None):
    """Head-wise rotated asymmetric 4-bit KV quantization (R12).

    kv fp16 [T, H, D].  Per (token, head): y = v . H_D / sqrt(D) (D-point
    Sylvester Hadamard, optional signs first); [DuQuant] Knowl 12: fixed
    Hadamard rotation (+-1/sqrt(2^n)) and per-token / per-head asymmetric
    quantization; step = (gamma max - beta min)/(2^b - 1) with gamma = beta = 1
    and b = 4, after widening the range to include 0.  [QuaRot-abs]: the KV
    cache in 4 bits.

    Returns (codes uint8 [T, H, D], step fp64 [T, H], zero int [T, H],
    pre-rounding y/step fp64 [T, H, D], pre-rounding -lo/step fp64 [T, H])."""
    v = np.asarray(kv).astype(np.float64)
    t_, h_, d = v.shape
    r = rotation_matrix(d, d, signs=signs)
    y = v @ r
    lo = np.minimum(y.min(axis=2), 0.0)
    hi = np.maximum(y.max(axis=2), 0.0)
    step = (hi - lo) / 15.0
    nz = step > 0
    zt = np.zeros_like(step)
    zt[nz] = -lo[nz] / step[nz]
    z = np.rint(zt)
    t = np.zeros_like(y)
    t[nz] = y[nz] / step[nz][:, None]
    q = np.clip(np.rint(t) + z[..., None], 0, 15)
    q[~nz] = 0
    z[~nz] = 0
    return q.astype(np.uint8), step, z.astype(np.int64), t, zt


def kv_dequantize(q, step, z) -> np.ndarray:
    """(q - z) * step, the rotated-domain reconstruction."""
    return (np.asarray(q, np.float64) - np.asarray(z, np.float64)[..., None]) * np.asarray(step, np.float64)[..., None]


# --------------------------------------------------------------------------
# Decode attention over the 4-bit KV cache
# --------------------------------------------------------------------------

def kv_attention_decode(q, k_codes, k_step, k_zero, v_codes, v_step, v_zero, lens=None, signs=None,
                        sm_scale=None):
    """One decode step of attention reading the rotated 4-bit KV cache (R19).

    [QuaRot-abs]: computational invariance applied to the attention mechanism
    and the KV cache, the cache held in 4 bits.  [DuQuant] Knowl 12: the
    Query x Key and attention-output x Value products pass through fixed
    head-wise Hadamard rotations, with the softmax output left unquantized.

    q       fp16/fp64 [B, Hq, D]
    k_codes uint8 [B, T, Hkv, D] unsigned codes (unpacked), k_step fp [B, T, Hkv],
            k_zero int [B, T, Hkv]; likewise v_*.
    lens    int [B] tokens per sequence (default all T).
    signs   the +-1 vector the cache was rotated with (R12), or None.
    Returns fp64 [B, Hq, D].

    Keys and values are reconstructed in the original basis:
    K = ((q - z) * step) @ R^T with R = diag(signs) H_D / sqrt(D)."""
    qf = np.asarray(q, np.float64)
    b_, hq, d = qf.shape
    t_, hkv = np.asarray(k_codes).shape[1:3]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    lens = np.full(b_, t_, dtype=np.int64) if lens is None else np.asarray(lens, np.int64)
    r = rotation_matrix(d, d, signs=signs)
    k = kv_dequantize(k_codes, k_step, k_zero) @ r.T     # [B, T, Hkv, D]
    v = kv_dequantize(v_codes, v_step, v_zero) @ r.T
    group = hq // hkv
    out = np.zeros((b_, hq, d))
    for b in range(b_):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(hq):
            kh = k[b, :n, h // group, :]                   # [n, D]
            vh = v[b, :n, h // group, :]
            s = sm_scale * (kh @ qf[b, h])                  # [n]
            e = np.exp(s - s.max())
            out[b, h] = (e / e.sum()) @ vh
    return out
