"""The hot path captured in a HIP graph: every replay must equal the eager
result on the same inputs, also with other eager work and fresh inputs in
between (the decode benchmark times graph replays).  Covers the vector path,
the weight-streaming path (also with its k range split over blocks) and the
tiled GEMM with its split-K workspace (partial sums stored per split and added
by a finish kernel: nothing is cleared, so the graph holds no memset node)."""
import numpy as np
import pytest
import torch

from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

CASES = [  # (m, n, k, path); the first case goes through bitlinear_quantize_forward
    (1, 300, 2560, bl.BL_PATH_GEMV),
    (8, 1000, 512, bl.BL_PATH_SKINNY),
    (64, 128, 4096, bl.BL_PATH_MFMA),     # few tiles: k range split, workspace used
    (40, 700, 384, bl.BL_PATH_MFMA),
    (13, 6150, 8192, bl.BL_PATH_SKINNY),  # 97 row blocks: k split two ways, workspace used
    (130, 5000, 2000, bl.BL_PATH_MFMA_WIDE),  # wide tiles, k split in two, workspace used
]


def test_graph_replays_match_eager():
    torch.cuda.synchronize()
    bufs = []
    for i, (m, n, k, path) in enumerate(CASES):
        w, x = inputs.random_case(30_000 + i, m, n, k, bf16=True)
        packed, gamma = bl.quantize_weights(dev(w))
        xd = dev(x)
        xq, scale, rowsum = bl.quantize_act(xd)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        bufs.append(dict(m=m, n=n, k=k, path=path, packed=packed, gamma=gamma, x=xd, xq=xq,
                         scale=scale, rowsum=rowsum, y=y))
    # the split-K case needs the workspace: the eager pass allocates the
    # binding's shared workspace before capture
    assert bl.forward_workspace_bytes(64, 128, 4096) > 0
    assert bl.forward_workspace_bytes(13, 6150, 8192) > 0

    lib = bl.load()

    def step():
        for i, b in enumerate(bufs):
            if i == 0:
                bl.quantize_forward(b["x"], b["packed"], b["gamma"], b["n"], path=b["path"],
                                    y=b["y"], xq=b["xq"], scale=b["scale"], rowsum=b["rowsum"])
                continue
            st = lib.bitlinear_quantize_act(
                bl._ptr(b["x"]), bl.BL_BF16, b["m"], b["k"], bl._ptr(b["xq"]), bl._ptr(b["scale"]),
                bl._ptr(b["rowsum"]), bl._stream(None))
            assert st == 0
            bl.forward(b["xq"], b["scale"], b["rowsum"], b["packed"], b["gamma"], b["n"], b["k"],
                       path=b["path"], y=b["y"])

    def eager_results():
        step()
        torch.cuda.synchronize()
        return [host(b["y"]).copy() for b in bufs]

    ref = eager_results()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()

    for replay in range(4):
        for b in bufs:
            b["y"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for b, r in zip(bufs, ref):
            np.testing.assert_array_equal(host(b["y"]).view(np.uint32), r.view(np.uint32),
                                          err_msg=f"replay {replay} case {b['m']},{b['n']},{b['k']}")
        # unrelated eager work between replays
        bl.quantize_act(torch.randn(3, 256, device="cuda"))
        torch.cuda.synchronize()

    # new inputs in the captured buffers: replay == eager on the new inputs
    for i, b in enumerate(bufs):
        _, x2 = inputs.random_case(31_000 + i, b["m"], 1, b["k"], bf16=True)
        b["x"].copy_(dev(x2))
    graph.replay()
    torch.cuda.synchronize()
    got = [host(b["y"]).copy() for b in bufs]
    ref2 = eager_results()
    for b, g_, r in zip(bufs, got, ref2):
        np.testing.assert_array_equal(g_.view(np.uint32), r.view(np.uint32),
                                      err_msg=f"fresh inputs, case {b['m']},{b['n']},{b['k']}")
    assert any(not np.array_equal(a, b_) for a, b_ in zip(ref, ref2))
