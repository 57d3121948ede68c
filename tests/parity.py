"""Parity helpers shared by the GPU tests: compare library results with the
CPU oracle under the stated tolerances.

* Quantized codes: identical, except where the oracle's pre-rounding value
  lies within BOUNDARY_WINDOW of a .5 rounding boundary; such mismatches are
  counted and must not exceed MAX_MISMATCH_FRAC of the elements.  (The GPU
  forms the rotated value in fp32, the oracle in fp64; only values that sit
  on a rounding boundary to within fp32 error can round differently.)
* Integer GEMM sums: bit-exact.
* fp16 outputs: relative Frobenius error <= OUT_REL_FRO against the oracle's
  fp64 dequantized output from the oracle's codes; where both sides are fed
  the same codes, every element within epilogue_bound (one fp16 rounding
  plus the fp32 roundings of the epilogue).
* Scales: relative error <= SCALE_RTOL (fp32 transform vs fp64).
* Decode attention outputs (fp16): per (sequence, head) relative Frobenius
  error <= ATTN_REL_FRO and every element within ATTN_ABS_FRAC of that head's
  largest |output|.  The output's own fp16 rounding is at most 2^-12 relative;
  fp32 scores, exponentials and sums over up to 10^5 tokens add well under
  1e-5; the bound leaves a factor of ~2 over fp16 rounding.
"""
from __future__ import annotations

import numpy as np

import oracle as O

BOUNDARY_WINDOW = 1e-3
MAX_MISMATCH_FRAC = 1e-4
OUT_REL_FRO = 2e-3
SCALE_RTOL = 1e-5
ATTN_REL_FRO = 1e-3
ATTN_ABS_FRAC = 1e-3


def near_half(t: np.ndarray) -> np.ndarray:
    """Pre-rounding values within BOUNDARY_WINDOW of a .5 boundary."""
    return np.abs(np.abs(t - np.floor(t)) - 0.5) < BOUNDARY_WINDOW


def check_symmetric_codes(gpu_packed: np.ndarray, q_or: np.ndarray, t_or: np.ndarray, what: str = "codes",
                          cap_count: bool = True):
    """cap_count=False for hand-built inputs full of exact .5 ties (e.g. a
    constant row under random signs), where every tie is a legitimate
    boundary case and the workload-level count cap does not apply."""
    g = O.unpack_int4(gpu_packed)
    assert g.shape == q_or.shape, (g.shape, q_or.shape)
    mism = g != q_or
    bad = mism & ~near_half(t_or)
    nm, nb = int(mism.sum()), int(bad.sum())
    assert nb == 0, f"{what}: {nb} mismatches away from a rounding boundary (first at {np.argwhere(bad)[:5].tolist()})"
    if cap_count:
        assert nm <= MAX_MISMATCH_FRAC * mism.size, f"{what}: {nm} boundary mismatches of {mism.size}"
    # a boundary mismatch can only be off by one
    if nm:
        assert np.abs(g[mism].astype(int) - q_or[mism].astype(int)).max() == 1
    return nm


def check_scales(gpu: np.ndarray, ref: np.ndarray, what: str = "scales"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    zero = ref == 0
    assert np.all(gpu[zero] == 0), f"{what}: nonzero scale for an all-zero row/group"
    rel = np.abs(gpu[~zero] - ref[~zero]) / ref[~zero]
    assert rel.size == 0 or rel.max() <= SCALE_RTOL, f"{what}: max rel err {rel.max():.3e}"


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a))


def check_output(gpu_fp16: np.ndarray, ref: np.ndarray, what: str = "output"):
    e = rel_fro(gpu_fp16.astype(np.float64), ref)
    assert e <= OUT_REL_FRO, f"{what}: relative Frobenius error {e:.3e}"
    return e


def epilogue_bound(acc, sx, sw, group: int = 0) -> np.ndarray:
    """Largest |y_gpu - y_oracle| per element of a GEMM output computed from
    the same integer sums.  The epilogue forms each term acc_j * s_x * s_w in
    fp32 (the integer converted to fp32, the scale product and the term: at
    most three roundings of 2^-24), adds the G terms of a grouped output in
    fp32 (G - 1 more), and rounds the result to fp16 (half an ulp: 2^-11
    relative, or 2^-25 absolute below the normal range).  With T the sum of
    the terms' magnitudes, the fp32 value v is within e32 = (G + 3) 2^-24 T of
    the exact y, and |fp16(v) - y| <= 2^-11 (|y| + e32) + e32 + 2^-25."""
    acc = np.asarray(acc, np.float64)
    sx = np.asarray(sx, np.float64)
    sw = np.asarray(sw, np.float64)
    if group == 0:
        exact = acc * sx[:, None] * sw[None, :]
        terms = np.abs(exact)
        g = 1
    else:
        parts = acc * np.transpose(sx)[:, :, None] * np.transpose(sw)[:, None, :]   # [G, M, N]
        exact = parts.sum(axis=0)
        terms = np.abs(parts).sum(axis=0)
        g = acc.shape[0]
    e32 = (g + 3) * 2.0 ** -24 * terms
    return 2.0 ** -11 * (np.abs(exact) + e32) + e32 + 2.0 ** -25


def check_kv(gpu_codes, gpu_step, gpu_zero, kv, signs=None):
    """KV parity: steps to SCALE_RTOL, zero points exact except where -lo/step
    is on a .5 boundary, codes exact except on a boundary; vectors whose zero
    point legitimately differs are checked by the reconstruction bound."""
    q_or, st_or, z_or, t_or, zt_or = O.kv_quantize(kv, signs)
    T, H, D = kv.shape
    g = O.unpack_uint4(gpu_codes.reshape(T, H, D // 2))
    check_scales(gpu_step, st_or, "kv step")
    zg = gpu_zero.astype(np.int64)
    zmis = zg != z_or
    assert np.all(near_half(zt_or)[zmis]), "kv zero point differs away from a rounding boundary"
    assert zmis.sum() <= max(1, MAX_MISMATCH_FRAC * zmis.size)
    same = ~zmis
    mism = (g != q_or) & same[..., None]
    bad = mism & ~near_half(t_or)
    assert int(bad.sum()) == 0, f"kv codes: {int(bad.sum())} mismatches away from a boundary"
    assert int(mism.sum()) <= MAX_MISMATCH_FRAC * mism.size
    if zmis.any():
        y = kv.astype(np.float64) @ O.rotation_matrix(D, D, signs=signs)
        rec = (g.astype(np.float64) - zg[..., None]) * np.asarray(gpu_step, np.float64)[..., None]
        err = np.abs(rec - y)[zmis]
        assert np.all(err <= (np.asarray(gpu_step, np.float64)[zmis][:, None] * (1.0 + 1e-4)))
    return int(mism.sum()), int(zmis.sum())


def check_attn(gpu_fp16: np.ndarray, ref: np.ndarray, what: str = "attention"):
    g = np.asarray(gpu_fp16, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.sqrt(((g - ref) ** 2).sum(-1))
    nrm = np.sqrt((ref ** 2).sum(-1))
    zero = nrm == 0
    assert np.all(err[zero] == 0), f"{what}: non-zero output where the oracle gives zeros"
    rel = err[~zero] / nrm[~zero]
    assert rel.size == 0 or rel.max() <= ATTN_REL_FRO, f"{what}: worst per-head rel fro {rel.max():.3e}"
    peak = np.abs(ref).max(-1, keepdims=True)
    assert np.all(np.abs(g - ref) <= ATTN_ABS_FRAC * peak + 1e-30), \
        f"{what}: max element error {np.abs(g - ref).max():.3e}"
    return float(rel.max()) if rel.size else 0.0


def check_symmetric_int8(gpu: np.ndarray, q_or: np.ndarray, t_or: np.ndarray, what: str = "int8 codes"):
    """The 6- and 8-bit codes (int8, unpacked) under the same boundary rule
    as check_symmetric_codes."""
    g = np.asarray(gpu).astype(np.int8)
    assert g.shape == q_or.shape, (g.shape, q_or.shape)
    mism = g != q_or
    bad = mism & ~near_half(t_or)
    nm, nb = int(mism.sum()), int(bad.sum())
    assert nb == 0, f"{what}: {nb} mismatches away from a rounding boundary"
    assert nm <= max(1, MAX_MISMATCH_FRAC * g.size), f"{what}: {nm} boundary mismatches"
    assert np.all(np.abs(g.astype(np.int64) - q_or) <= 1), f"{what}: a mismatch larger than one step"
    return nm
