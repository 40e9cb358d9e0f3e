"""A BitLinear product followed by the next layer's input glue in one call
(bitlinear_forward_*_rmsnorm_quantize): against the oracle chain
matmul_i32 -> rescale -> add_f32 / gqa_expand / relu2_mul -> rmsnorm_quantize,
and bit for bit against the product and the glue as separate calls (the glue
kernel finishes the GEMM's split partial sums with the split-k finish's own
arithmetic).

Two oracle checks per call:
  - per step: the oracle's glue is fed the product output y (itself within
    1e-5 of the oracle's rescale of the exact int32 product, which the GPU
    matches bit for bit); the residual stream must then match bit for bit and
    the codes within the glue's rounding-edge allowance (assert_quant_close);
  - end to end from the oracle's own float64 y: y rounded to float (as the
    GPU's epilogue does, within two roundings) moves the residual by at most
    2^-21 (|x| + |y|) per element and the codes by one in rare positions.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs
from ternary_weight_linear_absmax_amd import stack as st

from gpu_helpers import assert_quant_close, assert_y_close, dev, host, oracle_matmul_rows

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


# ---- against the oracle -----------------------------------------------------------------------

def _oracle_product(m, n, k, seed):
    """Seeded bf16 weights and activations on both sides; returns the GPU
    operands and the oracle's trits, gamma, int32 product and float64 y."""
    w, x = inputs.random_case(seed, m, n, k, bf16=True)
    t, g = oracle.quantize_weights(w)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    np.testing.assert_array_equal(host(xq), q_ref)
    acc_ref = oracle_matmul_rows(q_ref, t)
    np.testing.assert_array_equal(host(bl.matmul_i32(xq, rowsum, packed, n, k)), acc_ref)
    y_ref = oracle.rescale(acc_ref, s_ref, g)
    y_gpu = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k))
    assert_y_close(y_gpu, y_ref, acc_ref)
    return (xq, scale, rowsum, packed, gamma), y_ref, y_gpu


def _quant_loose(got, want, max_frac=1e-4):
    """Codes from slightly different float inputs: equal up to one in a small
    fraction of positions; scales within 1e-6; row sums consistent."""
    q, s, r = got
    q_ref, s_ref, _ = want
    diff = q.astype(np.int32) - q_ref.astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert np.count_nonzero(diff) <= max(4, int(max_frac * q.size)), np.count_nonzero(diff)
    np.testing.assert_allclose(s, s_ref, rtol=1e-6)
    assert np.array_equal(r, q.astype(np.int64).sum(axis=1))


# (M, N, K) of the layer stack (64 tokens) and of the split-k / no-split /
# weight-streaming / vector paths
RESIDUAL_SHAPES = [(64, 2560, 2560), (64, 2560, 6912), (37, 200, 2048), (130, 200, 4096),
                   (17, 200, 2048), (1, 200, 2048), (1, 2560, 6912)]


@pytest.mark.parametrize("m,n,k", RESIDUAL_SHAPES)
def test_fused_residual_against_oracle(m, n, k):
    ops, y_ref, y_gpu = _oracle_product(m, n, k, 110_000 + m + n + k)
    rng = np.random.default_rng(111_000 + m + n + k)
    x0 = rng.standard_normal((m, n)).astype(np.float32)
    x = dev(x0)
    got = [host(a) for a in bl.forward_residual_rmsnorm_quantize(*ops, n, x)]
    xg = host(x)
    # per step: the oracle's residual and glue on the product output
    x1 = oracle.add_f32(x0, y_gpu)
    np.testing.assert_array_equal(xg.view(np.uint32), x1.view(np.uint32))
    assert_quant_close(got, oracle.rmsnorm_quantize(x1))
    # end to end from the oracle's float64 y
    x1e = oracle.add_f32(x0, y_ref.astype(np.float32))
    bound = 2.0 ** -21 * (np.abs(x1e) + np.abs(y_ref))
    assert np.all(np.abs(xg.astype(np.float64) - x1e) <= bound)
    _quant_loose(got, oracle.rmsnorm_quantize(x1e))


# (M, N, K, v_col, heads, kv_heads, head_dim): the stack's QKV product and
# small grouped-query layouts on the split-k and vector paths
GQA_SHAPES = [(64, st.QKV, st.HIDDEN, st.V_COL, st.HEADS, st.KV_HEADS, st.HEAD_DIM),
              (37, 200, 2048, 120, 4, 2, 40), (130, 200, 4096, 120, 4, 2, 40),
              (1, st.QKV, st.HIDDEN, st.V_COL, st.HEADS, st.KV_HEADS, st.HEAD_DIM)]


@pytest.mark.parametrize("m,n,k,v_col,heads,kv,hd", GQA_SHAPES)
def test_fused_gqa_against_oracle(m, n, k, v_col, heads, kv, hd):
    ops, y_ref, y_gpu = _oracle_product(m, n, k, 120_000 + m + n + k)
    got = [host(a) for a in bl.forward_gqa_rmsnorm_quantize(*ops, n, v_col, heads, kv, hd)]
    v = y_gpu[:, v_col:v_col + kv * hd]
    assert_quant_close(got, oracle.rmsnorm_quantize(oracle.gqa_expand(v, heads, kv)))
    ve = y_ref[:, v_col:v_col + kv * hd].astype(np.float32)
    _quant_loose(got, oracle.rmsnorm_quantize(oracle.gqa_expand(ve, heads, kv)))


RELU2_SHAPES = [(64, 2 * st.FFN, st.HIDDEN, st.FFN), (37, 200, 2048, 97),
                (130, 200, 4096, 100), (17, 200, 2048, 97), (1, 2 * st.FFN, st.HIDDEN, st.FFN)]


@pytest.mark.parametrize("m,n,k,f", RELU2_SHAPES)
def test_fused_relu2_against_oracle(m, n, k, f):
    ops, y_ref, y_gpu = _oracle_product(m, n, k, 130_000 + m + n + k)
    got = [host(a) for a in bl.forward_relu2_rmsnorm_quantize(*ops, n, f)]
    v = oracle.relu2_mul(y_gpu[:, :f], y_gpu[:, f:2 * f])
    assert_quant_close(got, oracle.rmsnorm_quantize(v))
    ye = y_ref.astype(np.float32)
    _quant_loose(got, oracle.rmsnorm_quantize(oracle.relu2_mul(ye[:, :f], ye[:, f:2 * f])))
