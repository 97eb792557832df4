"""mx_moe_linear_noalloc (the entry point that allocates nothing) against
mx_moe_linear, the entry point with a caller workspace that it is a variant
of: the same outputs bit for bit, and the oracle's bar, on two calls in a
row, the second with a smaller input (the library's buffer keeps the first
call's contents)."""
import numpy as np
import pytest

import oracle
from microscaling_quantized_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxgpu
    return mxgpu


def _noalloc(g, elem, E, N, K, wp, cp, x, ids, weights):
    import torch
    import microscaling_quantized_linear_amd as mx
    T, topk = ids.shape
    combine = weights is not None
    y = torch.full((T, N) if combine else (T, topk, N), 0x7FC0, dtype=torch.int16, device=g.DEV)
    mx.mx_moe_linear_noalloc(elem, E, N, K, wp, cp, T, topk, g.dev(x), K, g.dev(ids),
                             g.dev(weights) if combine else None, y)
    torch.cuda.synchronize()
    return g.host_u16(y)


# the MoE decode shape (E = 32, N = K = 3072, 16 tokens, top-8), then a smaller one
CASES = [dict(E=32, N=3072, K=3072, T=16, topk=8, seed=0),
         dict(E=6, N=256, K=512, T=5, topk=2, seed=1)]


def test_noalloc_moe_matches_workspace_path_twice(g):
    for c in CASES:
        d = wl.moe_inputs(4, E=c["E"], N=c["N"], K=c["K"], T=c["T"], topk=c["topk"],
                          seed=c["seed"])
        E, N, K = c["E"], c["N"], c["K"]
        wp, cp = g.pack(1, 0, E, N, K, d["w"], d["codes"])
        for wts in (d["weights"], None):
            y_ws = g.moe(1, E, N, K, wp, cp, d["x"], d["ids"], wts)
            y_na = _noalloc(g, 1, E, N, K, wp, cp, d["x"], d["ids"], wts)
            assert np.array_equal(y_ws, y_na), f"noalloc differs from the workspace path: {c}"
            ref = oracle.moe_linear(1, E, N, K, d["w"], d["codes"], d["x"], d["ids"], wts)
            g.assert_close(y_na, ref, f"noalloc {c}")


def test_noalloc_moe_graph_replays(g):
    """The callers it is for capture it in a HIP graph: every replay gives the
    eager result bit for bit, also when an eager call with another input used
    the library's buffer in between (calls ordered on one stream)."""
    import torch
    import microscaling_quantized_linear_amd as mx
    a = wl.moe_inputs(4, E=8, N=256, K=512, T=6, topk=3, seed=2)
    b = wl.moe_inputs(4, E=8, N=256, K=512, T=9, topk=2, seed=3)
    E, N, K = 8, 256, 512
    wp, cp = g.pack(1, 0, E, N, K, a["w"], a["codes"])
    x, ids, wts = g.dev(a["x"]), g.dev(a["ids"]), g.dev(a["weights"])
    xb, idsb, wtsb = g.dev(b["x"]), g.dev(b["ids"]), g.dev(b["weights"])
    y = torch.empty((6, N), dtype=torch.int16, device=g.DEV)
    yb = torch.empty((9, N), dtype=torch.int16, device=g.DEV)

    def run():
        mx.mx_moe_linear_noalloc(1, E, N, K, wp, cp, 6, 3, x, K, ids, wts, y)

    def other():
        mx.mx_moe_linear_noalloc(1, E, N, K, wp, cp, 9, 2, xb, K, idsb, wtsb, yb)

    run()
    torch.cuda.synchronize()
    ref = y.clone()
    ref_np = g.host_u16(y)
    g.assert_close(ref_np, oracle.moe_linear(1, E, N, K, a["w"], a["codes"], a["x"], a["ids"],
                                             a["weights"]), "noalloc eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="thread_local"):
        run()
    for _ in range(4):
        y.zero_()
        other()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), "a replay differs from the eager call"
