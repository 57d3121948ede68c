"""Seeded synthetic inputs for the QuaRot linear-layer hot path.

This module only draws random numbers and casts them to the storage types the
hot path consumes (fp16 activations, weights and KV rows; +-1 sign vectors; a
seeded orthogonal factor).  It holds none of the method's arithmetic: no
rotation is applied, nothing is quantized.  Both the CPU oracle and the GPU
tests/bench take their inputs from here, and nothing else is shared between
them.

Shapes follow the LLaMA-2 7B/70B layers the QuaRot summary (Elamur Research,
"Key points") measures on: one transformer block at batch 64, sequence 2048.
The outlier structure follows DuQuant (ChapterPal), Knowl 4 "Normal Outliers
versus Massive Outliers": normal outliers are whole channels that stay large
for every token; massive outliers are isolated entries of very large
magnitude at the down_proj input.  The random orthogonal factor follows the
incoherence-processing idea of the QuIP summary (Uptrust), abstract: a random
orthogonal matrix drawn as the Q factor of a Gaussian matrix.

RNG: numpy.random.default_rng([cfg_index, stream]) with streams
  0 = x values, 1 = outlier selection, 2 = W, 3 = signs, 4 = dense factor,
  5 = K rows, 6 = V rows.
Large activations are drawn in blocks of BLOCK_ROWS rows, block b from
default_rng([cfg_index, stream, b]), so any row subset can be regenerated
without drawing the whole matrix.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 4096


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    desc: str
    M: int                 # tokens (activation rows)
    K: int                 # input features (row width n of the rotation)
    N: int                 # output features
    had_n: int             # power-of-two Hadamard size
    dense_m: int           # 1, or size of the dense orthogonal factor
    group: int             # 0 = per token / per output channel, else group size along K
    use_signs: bool        # randomized (D . H) or plain Hadamard
    x_dist: str            # "normal" | "laplace"
    outlier_cols: int      # normal outliers: number of whole columns scaled
    outlier_scale: float
    outlier_frac: float    # massive outliers: Bernoulli fraction of entries scaled
    w_std: float
    kv: dict = field(default_factory=dict)


CONFIGS: dict[str, Config] = {
    "c1": Config("c1", 1, "tiny layer 64x512 -> 512", 64, 512, 512, 512, 1, 0, True,
                 "normal", 4, 50.0, 0.0, 0.02),
    "c2": Config("c2", 2, "LLaMA-2-7B fused QKV prefill 2048x4096 -> 12288", 2048, 4096, 12288,
                 4096, 1, 0, True, "normal", 8, 100.0, 0.0, 0.02),
    "c3": Config("c3", 3, "LLaMA-2-7B down_proj at batch 64 x seq 2048: 131072x11008 -> 4096",
                 131072, 11008, 4096, 64, 172, 0, False, "laplace", 0, 200.0, 0.001, 0.02),
    "c4": Config("c4", 4, "LLaMA-2-70B MLP up/gate, group 128: 16384x8192 -> 28672",
                 16384, 8192, 28672, 8192, 1, 128, True, "normal", 16, 100.0, 0.0, 0.01),
    "c5": Config("c5", 5, "decode step at batch 64: 64x4096 -> 4096, plus KV rows 64x32x128",
                 64, 4096, 4096, 4096, 1, 0, True, "normal", 8, 100.0, 0.0, 0.02,
                 kv=dict(T=64, H=32, D=128, outlier_dims=2, outlier_scale=30.0)),
    # the second non-power-of-two width: LLaMA-2-70B down_proj input,
    # 28672 = 4096 * 7, drawn like c3's down_proj input
    "d70": Config("d70", 6, "LLaMA-2-70B down_proj at 16384 tokens: 16384x28672 -> 8192",
                  16384, 28672, 8192, 4096, 7, 0, False, "laplace", 0, 200.0, 0.001, 0.01),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def outlier_columns(cfg: Config) -> np.ndarray:
    """Channels that carry normal outliers (sorted, without replacement)."""
    if cfg.outlier_cols == 0:
        return np.zeros(0, dtype=np.int64)
    r = _rng(cfg.index, 1)
    return np.sort(r.choice(cfg.K, size=cfg.outlier_cols, replace=False))


def _x_block(cfg: Config, b: int, cols: np.ndarray) -> np.ndarray:
    rows = min(BLOCK_ROWS, cfg.M - b * BLOCK_ROWS)
    r = _rng(cfg.index, 0, b)
    if cfg.x_dist == "normal":
        v = r.standard_normal((rows, cfg.K))
    elif cfg.x_dist == "laplace":
        v = r.laplace(0.0, 1.0, (rows, cfg.K))
    else:  # pragma: no cover
        raise ValueError(cfg.x_dist)
    if cols.size:
        v[:, cols] *= cfg.outlier_scale
    if cfg.outlier_frac > 0:
        m = _rng(cfg.index, 1, b).random((rows, cfg.K)) < cfg.outlier_frac
        v[m] *= cfg.outlier_scale
    return v.astype(np.float16)


def make_x(cfg: Config | str, rows: np.ndarray | slice | None = None) -> np.ndarray:
    """Activations x, fp16 [M, K] (or the requested row subset, in order)."""
    cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    cols = outlier_columns(cfg)
    if rows is None:
        idx = None
        blocks = range((cfg.M + BLOCK_ROWS - 1) // BLOCK_ROWS)
    else:
        idx = np.arange(cfg.M)[rows] if isinstance(rows, slice) else np.asarray(rows, dtype=np.int64)
        blocks = sorted(set((idx // BLOCK_ROWS).tolist()))
    out_rows = cfg.M if idx is None else idx.size
    out = np.empty((out_rows, cfg.K), dtype=np.float16)

    def fill(b):
        blk = _x_block(cfg, b, cols)
        if idx is None:
            out[b * BLOCK_ROWS: b * BLOCK_ROWS + blk.shape[0]] = blk
        else:
            sel = np.nonzero(idx // BLOCK_ROWS == b)[0]
            out[sel] = blk[idx[sel] - b * BLOCK_ROWS]

    blocks = list(blocks)
    if len(blocks) == 1:
        fill(blocks[0])
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
    return out


def make_w(cfg: Config | str, cols: np.ndarray | None = None) -> np.ndarray:
    """Weights W, fp16 [K, N] with y = x @ W (or a subset of output columns)."""
    cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    out = np.empty((cfg.K, cfg.N), dtype=np.float16)
    step = max(1, (1 << 22) // cfg.N)   # row blocks of ~4M elements, one stream per block

    def fill(b):
        r0 = b * step
        r1 = min(cfg.K, r0 + step)
        out[r0:r1] = (_rng(cfg.index, 2, b).standard_normal((r1 - r0, cfg.N)) * cfg.w_std).astype(np.float16)

    nb = (cfg.K + step - 1) // step
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nb)))
    return out if cols is None else np.ascontiguousarray(out[:, cols])


def make_signs(cfg: Config | str, n: int | None = None) -> np.ndarray | None:
    """Random +-1 diagonal (int8 [n]) of the randomized Hadamard, or None."""
    cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    if not cfg.use_signs:
        return None
    n = cfg.K if n is None else n
    return np.where(_rng(cfg.index, 3).random(n) < 0.5, -1, 1).astype(np.int8)


def make_dense(cfg: Config | str, m: int | None = None, dtype=np.float32) -> np.ndarray | None:
    """Seeded m x m orthogonal factor: Q of a QR of a Gaussian matrix, with the
    column signs fixed so that R of the QR has a positive diagonal (a Haar
    draw).  Returned in fp64 (for identities) or rounded to fp32, the type the
    library takes."""
    cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    m = cfg.dense_m if m is None else m
    if m == 1:
        return None
    g = _rng(cfg.index, 4).standard_normal((m, m))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(dtype)


def make_kv(cfg: Config | str = "c5", T: int | None = None):
    """New K and V rows, fp16 [T, H, D], N(0,1) with a few seeded head dims
    scaled (normal outliers per head)."""
    cfg = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    kv = cfg.kv
    T = kv["T"] if T is None else T
    H, D = kv["H"], kv["D"]
    sel = _rng(cfg.index, 1, 99)
    dims = np.stack([np.sort(sel.choice(D, kv["outlier_dims"], replace=False)) for _ in range(H)])
    out = []
    for stream in (5, 6):
        v = _rng(cfg.index, stream).standard_normal((T, H, D))
        for h in range(H):
            v[:, h, dims[h]] *= kv["outlier_scale"]
        out.append(v.astype(np.float16))
    return out[0], out[1]


def make_kv_large(T: int, H: int = 32, D: int = 128, seed: int = 7, outlier_dims: int = 2,
                  outlier_scale: float = 30.0) -> np.ndarray:
    """A prefill-scale K (or V) tensor [T, H, D] fp16 with the decode recipe,
    drawn in blocks of BLOCK_ROWS tokens (stream key [5, seed, block])."""
    sel = _rng(5, seed, 99)
    dims = np.stack([np.sort(sel.choice(D, outlier_dims, replace=False)) for _ in range(H)])
    out = np.empty((T, H, D), dtype=np.float16)

    def fill(b):
        t0 = b * BLOCK_ROWS
        t1 = min(T, t0 + BLOCK_ROWS)
        v = _rng(5, seed, b).standard_normal((t1 - t0, H, D))
        for h in range(H):
            v[:, h, dims[h]] *= outlier_scale
        out[t0:t1] = v.astype(np.float16)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range((T + BLOCK_ROWS - 1) // BLOCK_ROWS)))
    return out


def make_random_rows(rows: int, n: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Generic fp16 N(0, scale) rows for edge-case tests of any width."""
    return (_rng(900, seed).standard_normal((rows, n)) * scale).astype(np.float16)


def make_random_codes(rows: int, k: int, seed: int, lo: int = -8, hi: int = 7) -> np.ndarray:
    """Uniform integer codes in [lo, hi] (int8 [rows, k]) for integer-GEMM tests."""
    return _rng(901, seed).integers(lo, hi + 1, size=(rows, k)).astype(np.int8)


def make_random_packed(rows: int, nbytes: int, seed: int) -> np.ndarray:
    """Uniform random bytes (uint8 [rows, nbytes]): two independent uniform
    4-bit codes per byte, for full-size integer-GEMM inputs."""
    out = np.empty((rows, nbytes), np.uint8)
    step = 8192

    def fill(b):
        r = _rng(902, seed, b)
        out[b * step:(b + 1) * step] = r.integers(0, 256, size=(min(step, rows - b * step), nbytes), dtype=np.uint8)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range((rows + step - 1) // step)))
    return out


def make_random_scales(n: int, seed: int, lo: float = 0.001, hi: float = 0.05) -> np.ndarray:
    """Uniform positive float32 scales in [lo, hi)."""
    return (_rng(903, seed).random(n) * (hi - lo) + lo).astype(np.float32)



def make_attn_cache(B: int, T: int, Hkv: int, seed: int, D: int = 128):
    """A synthetic 4-bit KV cache as the KV quantizer lays it out, for decode
    attention: codes uint8 [B, T, Hkv, D/2] (uniform bytes: two uniform 4-bit
    codes each), steps fp32 [B, T, Hkv] uniform in [0.02, 0.3), zero points
    uint8 [B, T, Hkv] uniform in [0, 15], for K (stream 0) and V (stream 1),
    drawn in blocks of 1024 tokens keyed [904, seed, stream, block].
    Returns (kc, ks, kz, vc, vs, vz)."""
    out = []
    for stream in (0, 1):
        c = np.empty((B, T, Hkv, D // 2), np.uint8)
        s = np.empty((B, T, Hkv), np.float32)
        z = np.empty((B, T, Hkv), np.uint8)
        for b0 in range(0, max(T, 1), 1024):
            b1 = min(b0 + 1024, T)
            if b1 <= b0:
                break
            r = _rng(904, seed, stream, b0 // 1024)
            c[:, b0:b1] = r.integers(0, 256, size=(B, b1 - b0, Hkv, D // 2), dtype=np.uint8)
            s[:, b0:b1] = (r.random((B, b1 - b0, Hkv)) * 0.28 + 0.02).astype(np.float32)
            z[:, b0:b1] = r.integers(0, 16, size=(B, b1 - b0, Hkv), dtype=np.uint8)
        out += [c, s, z]
    return tuple(out)


def make_attn_query(B: int, Hq: int, seed: int, D: int = 128) -> np.ndarray:
    """Decode queries, fp16 [B, Hq, D] N(0, 1) (key [905, seed])."""
    return _rng(905, seed).standard_normal((B, Hq, D)).astype(np.float16)
