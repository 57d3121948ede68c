"""The decode and prefill steps (rotate-quant, int4 GEMM, KV quant) captured in a HIP graph
and replayed, as bench.py --graph 1 runs it.

Every replay must reproduce the eager results bit for bit.  Before each replay
the outputs are cleared by eager fill kernels and unrelated eager work runs on
other buffers, with synchronizations between, so a replay that skipped a
kernel, read stale state or depended on memory the capture did not own would
show up as a mismatch."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    import rotation_bit_quantized_amd as m
    m.library()
    return m


def test_decode_step_graph_replays_match_eager(qr):
    cfg = W.CONFIGS["c5"]
    M, N, K = cfg.M, cfg.N, cfg.K
    assert cfg.group == 0 and cfg.dense_m == 1
    dev = torch.device("cuda:0")
    signs = W.make_signs(cfg)
    rot = qr.Rotation.hadamard(K, signs)
    wc, ws = qr.rotate_quant(torch.from_numpy(np.ascontiguousarray(W.make_w(cfg).T)).to(dev), rot, 0)
    x = torch.from_numpy(W.make_x(cfg)).to(dev)
    k_host, v_host = W.make_kv(cfg)
    kv_in = torch.from_numpy(np.ascontiguousarray(np.concatenate([k_host, v_host], axis=1))).to(dev)
    T, H = kv_in.shape[0], kv_in.shape[1]

    def outputs():
        return dict(xc=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                    xs=torch.empty((M,), dtype=torch.float32, device=dev),
                    y=torch.empty((M, N), dtype=torch.float16, device=dev),
                    kc=torch.empty((T, H, 64), dtype=torch.uint8, device=dev),
                    ks=torch.empty((T, H), dtype=torch.float32, device=dev),
                    kz=torch.empty((T, H), dtype=torch.uint8, device=dev))

    def run(o, st=None):
        qr.rotate_quant(x, rot, 0, codes=o["xc"], scales=o["xs"], stream=st)
        qr.int4_gemm(o["xc"], o["xs"], wc, ws, 0, y=o["y"], stream=st)
        qr.kv_quant(kv_in, codes=o["kc"], scales=o["ks"], zeros=o["kz"], stream=st)

    ref = outputs()
    run(ref)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}

    out = outputs()
    run(out)                      # eager pass first: the library's per-process state is set up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out, torch.cuda.current_stream())
    torch.cuda.synchronize()

    other = outputs()
    x2 = torch.flip(x, [0]).contiguous()
    for rep in range(4):
        for t in out.values():
            t.zero_()
        qr.rotate_quant(x2, rot, 0, codes=other["xc"], scales=other["xs"])   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs from the eager result"
        torch.cuda.synchronize()


def test_prefill_step_graph_replays_match_eager(qr):
    """The c2 step (2048 x 4096 rotate-quant on the persistent grid, the
    persistent 256 x 192 GEMM against 12288 channels, KV quant of the K and V
    heads read in place from the GEMM output) captured once and replayed."""
    cfg = W.CONFIGS["c2"]
    M, N, K = cfg.M, cfg.N, cfg.K
    assert cfg.group == 0 and cfg.dense_m == 1 and N == 3 * K
    dev = torch.device("cuda:0")
    rot = qr.Rotation.hadamard(K, W.make_signs(cfg))
    wc, ws = qr.rotate_quant(torch.from_numpy(np.ascontiguousarray(W.make_w(cfg).T)).to(dev), rot, 0)
    x = torch.from_numpy(W.make_x(cfg)).to(dev)
    H = 2 * K // 128

    def outputs():
        return dict(xc=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                    xs=torch.empty((M,), dtype=torch.float32, device=dev),
                    y=torch.empty((M, N), dtype=torch.float16, device=dev),
                    kc=torch.empty((M, H, 64), dtype=torch.uint8, device=dev),
                    ks=torch.empty((M, H), dtype=torch.float32, device=dev),
                    kz=torch.empty((M, H), dtype=torch.uint8, device=dev))

    def run(o, st=None):
        qr.rotate_quant(x, rot, 0, codes=o["xc"], scales=o["xs"], stream=st)
        qr.int4_gemm(o["xc"], o["xs"], wc, ws, 0, y=o["y"], stream=st)
        qr.kv_quant(o["y"][:, K:3 * K], codes=o["kc"], scales=o["ks"], zeros=o["kz"], stream=st)

    ref = outputs()
    run(ref)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}

    out = outputs()
    run(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out, torch.cuda.current_stream())
    torch.cuda.synchronize()

    other = outputs()
    x2 = torch.flip(x, [0]).contiguous()
    for rep in range(3):
        for t in out.values():
            t.zero_()
        qr.rotate_quant(x2, rot, 0, codes=other["xc"], scales=other["xs"])   # unrelated eager work
        qr.int4_gemm(other["xc"], other["xs"], wc, ws, 0, y=other["y"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t in out.items():
            assert torch.equal(t, ref[name]), f"replay {rep}: {name} differs from the eager result"
