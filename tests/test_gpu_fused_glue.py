"""A BitLinear product followed by the next layer's input glue in one call
(bitlinear_forward_*_rmsnorm_quantize) gives, bit for bit, what the product
and the glue give as separate calls: the glue kernel finishes the GEMM's split
partial sums with the split-k finish's own arithmetic.  The separate calls are
themselves checked against the oracle in test_gpu_stack.py and
test_gpu_parity.py, so equality here carries that parity over.
"""
import numpy as np
import pytest
import torch

from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import stack as st

from gpu_helpers import host

pytestmark = pytest.mark.gpu


def bits(t):
    a = host(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def product_inputs(m, n, k, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    w = (torch.randn((n, k), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    packed, gamma = bl.quantize_weights(w)
    x = torch.randn((m, k), generator=gen, device="cuda")
    xq, scale, rowsum = bl.quantize_act(x)
    return packed, gamma, xq, scale, rowsum, gen


# (M, N, K): split k on the GEMM (finished in the glue), no split, the
# weight-streaming and vector paths (product output through the workspace)
SHAPES = [(37, 200, 2048), (130, 200, 4096), (64, 2560, 6912), (200, 640, 512), (17, 200, 2048),
          (1, 200, 2048)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_fused_residual_matches_separate_calls(m, n, k):
    packed, gamma, xq, scale, rowsum, gen = product_inputs(m, n, k, 100 + m)
    x0 = torch.randn((m, n), generator=gen, device="cuda")
    y = bl.forward(xq, scale, rowsum, packed, gamma, n, k)
    x_ref = x0.clone()
    ref = bl.residual_rmsnorm_quantize(x_ref, y)
    x = x0.clone()
    got = bl.forward_residual_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n, x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(x), bits(x_ref))
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(bits(a), bits(b))


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_fused_gqa_and_relu2_match_separate_calls(m, n, k):
    packed, gamma, xq, scale, rowsum, _ = product_inputs(m, n, k, 200 + m)
    y = bl.forward(xq, scale, rowsum, packed, gamma, n, k)
    # 4 query heads over 2 key-value heads of 40, value columns from 120
    ref = bl.gqa_rmsnorm_quantize(y, 120, 4, 2, 40)
    got = bl.forward_gqa_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n, 120, 4, 2, 40)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(bits(a), bits(b))
    f = n // 2 - 3
    ref = bl.relu2_rmsnorm_quantize(y, f)
    got = bl.forward_relu2_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n, f)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(bits(a), bits(b))


def test_fused_outputs_may_overwrite_the_inputs():
    m, n, k = 64, 2560, 6912          # the layer stack's down projection: k split four ways
    packed, gamma, xq, scale, rowsum, gen = product_inputs(m, n, k, 7)
    x0 = torch.randn((m, n), generator=gen, device="cuda")
    x_ref = x0.clone()
    ref = bl.forward_residual_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n, x_ref)
    buf = torch.zeros((m * k,), dtype=torch.int8, device="cuda")
    buf[: m * k].view(m, k).copy_(xq)
    xq_in = buf.view(m, k)
    s, r = scale.clone(), rowsum.clone()
    x = x0.clone()
    bl.forward_residual_rmsnorm_quantize(xq_in, s, r, packed, gamma, n, x,
                                         xq_out=buf[: m * n].view(m, n), scale_out=s,
                                         rowsum_out=r)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(x), bits(x_ref))
    np.testing.assert_array_equal(host(buf[: m * n].view(m, n)), host(ref[0]))
    np.testing.assert_array_equal(bits(s), bits(ref[1]))
    np.testing.assert_array_equal(host(r), host(ref[2]))


@pytest.mark.parametrize("m", [64, 130, 40, 17, 1])
def test_fused_stack_matches_unfused_stack(m):
    gen = torch.Generator(device="cuda")

    def weights(layer):
        gen.manual_seed(5000 + layer)
        return {nm: (torch.randn(st.SHAPES[nm], generator=gen, device="cuda") * 0.02)
                .to(torch.bfloat16) for nm in st.MATRICES}

    stack = st.DecoderStack(weights, 2, m, fused=False)
    gen.manual_seed(5999)
    x0 = torch.randn((m, st.HIDDEN), device="cuda", generator=gen)
    stack.x.copy_(x0)
    stack.step()
    torch.cuda.synchronize()
    ref = [bits(stack.x).copy(), host(stack.xq).copy(), bits(stack.scale).copy(),
           host(stack.rowsum).copy()]
    stack.fused = True
    stack.x.copy_(x0)
    stack.step()
    torch.cuda.synchronize()
    got = [bits(stack.x), host(stack.xq), bits(stack.scale), host(stack.rowsum)]
    np.testing.assert_array_equal(got[0], ref[0])
    # xq: the final quantised RMSNorm of the stream occupies the first M x 2560 bytes
    np.testing.assert_array_equal(got[1].reshape(-1)[: m * st.HIDDEN],
                                  ref[1].reshape(-1)[: m * st.HIDDEN])
    np.testing.assert_array_equal(got[2], ref[2])
    np.testing.assert_array_equal(got[3], ref[3])
