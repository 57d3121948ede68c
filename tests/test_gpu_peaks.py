"""GPU checks of the measurement probes (include/qr_peaks.h).

qr_peak_mfma_codes must multiply the codes it is given, widened as the int4
GEMM widens them.  Every accumulator element appears once over a wave's lanes
and registers, so the sum of all lane checksums of a call is

    iters * sum over the round's MFMAs of  sum_k colsum(A)[k] * rowsum(W)[k],

and colsum / rowsum over the 32 rows of a fragment only need which half of
the wave (lanes 0-31 or 32-63) a lane is in: both operands keep k along
their bytes in the same order.  The host computes that sum exactly from the
codes; any other operand (a constant, a wrong piece, no widening) changes it.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    import rotation_bit_quantized_amd as m
    m.library()
    return m


def widen(raw):
    """[..., 16] uint8 packed codes -> [..., 2, 16] int8 operands of the two
    k-steps: per dword w, (w << 4) & 0xF0F0F0F0 then w & 0xF0F0F0F0."""
    w = np.ascontiguousarray(raw).view(np.uint32).astype(np.uint64)
    lo = ((w << 4) & 0xF0F0F0F0).astype(np.uint32)
    hi = (w & 0xF0F0F0F0).astype(np.uint32)
    op0 = np.stack([lo[..., 0], hi[..., 0], lo[..., 1], hi[..., 1]], -1)
    op1 = np.stack([lo[..., 2], hi[..., 2], lo[..., 3], hi[..., 3]], -1)
    return np.ascontiguousarray(np.stack([op0, op1], -2)).view(np.int8)


def half_sums(codes, waves):
    """Per wave, half and fragment f: the byte-wise sums over the half's 32
    lanes of the widened operands, int64 [waves, 2, 8, 2, 16]."""
    pieces = codes.reshape(-1, 16)
    idx = ((np.arange(waves)[:, None, None] * 64 + np.arange(64)[None, :, None]) * 8
           + np.arange(8)[None, None, :]) % pieces.shape[0]
    ops = widen(pieces[idx]).astype(np.int64)            # [waves, 64, 8, 2, 16]
    return ops.reshape(waves, 2, 32, 8, 2, 16).sum(axis=2)


@pytest.mark.parametrize("a_bytes,w_bytes,iters", [(65536, 49152, 3), (16, 48, 1)])
def test_peak_mfma_codes_multiplies_the_given_codes(qr, a_bytes, w_bytes, iters):
    rng = np.random.default_rng(a_bytes + w_bytes)
    a = rng.integers(0, 256, a_bytes, dtype=np.uint8)
    w = rng.integers(0, 256, w_bytes, dtype=np.uint8)
    out, ops = qr.peak_mfma_codes(torch.from_numpy(a).cuda(), torch.from_numpy(w).cuda(), iters)
    torch.cuda.synchronize()
    waves = int(qr.library().qr_peak_mfma_waves())
    assert ops == waves * iters * 32 * 65536
    sa, sw = half_sums(a, waves), half_sums(w, waves)
    total = 0
    for f in range(8):
        for j in range(2):
            total += int((sa[:, :, f] * sw[:, :, (f + 4 * j) % 8]).sum())
    total *= iters
    got = int(out.cpu().numpy().astype(np.int64).sum())
    assert got % (1 << 32) == total % (1 << 32)
