"""The entry points allocate nothing and synchronize nothing, so they can be
captured in a HIP graph: every replay (with eager work and synchronizations
between replays) must give exactly the eager result."""
import numpy as np
import pytest

from microscaling_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxgpu
    import microscaling_quantized_linear_amd as mx
    return torch, mx, mxgpu


def _replays_match(torch, run, out, eager_work):
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    out.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="thread_local"):
        run()
    for _ in range(4):
        out.zero_()
        eager_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)


def test_graph_linear_w8a8_quant_in_call(env):
    torch, mx, g = env
    M, N, K = 16, 512, 1568
    d = wl.linear_inputs(2, M=M, N=N, K=K)
    wp, cp = g.pack(0, 1, 1, N, K, d["w"], d["codes"])
    x = g.dev(d["x"])
    y = torch.empty((M, N), dtype=torch.int16, device=g.DEV)
    need = mx.mx_linear_workspace(0, 1, N, K, M, 1, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)
    other = torch.randn(1024, 1024, device=g.DEV)

    def run():
        mx.mx_linear(0, 1, N, K, wp, cp, M, 1, 0, x, K, None, 0, None, 0, None, y, N, ws, need)

    _replays_match(torch, run, y, lambda: other.mul_(1.0001))


def test_graph_gemm(env):
    torch, mx, g = env
    M, N, K = 300, 512, 384
    d = wl.linear_inputs(5, M=M, N=N, K=K)
    wp, cp = g.pack(0, 1, 1, N, K, d["w"], d["codes"])
    x = g.dev(d["x"])
    y = torch.empty((M, N), dtype=torch.int16, device=g.DEV)
    need = mx.mx_linear_workspace(0, 1, N, K, M, 1, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)

    def run():
        mx.mx_linear(0, 1, N, K, wp, cp, M, 1, 0, x, K, None, 0, None, 0, None, y, N, ws, need)

    _replays_match(torch, run, y, lambda: ws[16384:].fill_(7))


def test_graph_moe_combined(env):
    torch, mx, g = env
    d = wl.moe_inputs(4, E=8, N=64, K=512, T=6, topk=3)
    E, N, K, T, topk = d["E"], d["N"], d["K"], d["T"], d["topk"]
    wp, cp = g.pack(1, 0, E, N, K, d["w"], d["codes"])
    x, ids, wts = g.dev(d["x"]), g.dev(d["ids"]), g.dev(d["weights"])
    y = torch.empty((T, N), dtype=torch.int16, device=g.DEV)
    need = mx.mx_moe_workspace(1, E, N, K, T, topk, 1)
    ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)

    def run():
        mx.mx_moe_linear(1, E, N, K, wp, cp, T, topk, x, K, ids, wts, y, ws, need)

    _replays_match(torch, run, y, lambda: ws[16384:].fill_(3))


def test_graph_moe_block(env):
    """Up-gate with the SiLU product, then the combined down projection,
    captured as one graph."""
    torch, mx, g = env
    E, inter, H, T, topk = 8, 64, 96, 5, 2
    d13 = wl.moe_inputs(4, E=E, N=2 * inter, K=H, T=T, topk=topk)
    d2 = wl.moe_inputs(4, E=E, N=H, K=inter, T=T, topk=topk, seed=1)
    w13p, c13p = g.pack(1, 0, E, 2 * inter, H, d13["w"], d13["codes"])
    w2p, c2p = g.pack(1, 0, E, H, inter, d2["w"], d2["codes"])
    x, ids, wts = g.dev(d13["x"]), g.dev(d13["ids"]), g.dev(d13["weights"])
    h = torch.empty((T * topk, inter), dtype=torch.int16, device=g.DEV)
    y = torch.empty((T, H), dtype=torch.int16, device=g.DEV)
    need = mx.mx_moe_workspace(1, E, H, inter, T, topk, 1)
    ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)

    def run():
        mx.mx_moe_gate_up(1, E, inter, H, w13p, c13p, T, topk, x, H, ids, h, inter)
        mx.mx_moe_down(1, E, H, inter, w2p, c2p, T, topk, h, inter, ids, wts, y, ws, need)

    def other():
        h.fill_(5)
        ws.fill_(9)

    _replays_match(torch, run, y, other)
