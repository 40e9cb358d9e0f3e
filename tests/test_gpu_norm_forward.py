"""One token through bitlinear_norm_forward: the decoder block's input glue
(residual addition, first-token grouped-query attention, or a double input),
RMSNorm, the absmax quantiser and the 2-bit product in one launch, with the
squared-ReLU gate as an optional epilogue, against the oracle.

Per step, as in the layer-stack tests: the quantised token is compared with
the oracle's RMSNorm + quantiser of the same pre-norm values (codes may differ
by one at rounding edges of the double sum, reduced in another order), the
int32 product is required exact for the codes the GPU used (recomputed here
with bitlinear_matmul_i32 from the returned token) and the outputs within
1e-5 of the oracle's rescale of it; the squared-ReLU output is compared with
the oracle's relu2_mul of the float products.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs
from ternary_weight_linear_absmax_amd import stack as st

from gpu_helpers import assert_quant_close, assert_y_close, dev, host

pytestmark = pytest.mark.gpu


def _weights(seed, n, k):
    w, _ = inputs.random_case(seed, 1, n, k, bf16=True)
    t, g = oracle.quantize_weights(w)
    packed, gamma = bl.quantize_weights(dev(w))
    return t, g, packed, gamma


def _outs(k):
    return (torch.empty((1, k), dtype=torch.int8, device="cuda"),
            torch.empty((1,), dtype=torch.float32, device="cuda"),
            torch.empty((1,), dtype=torch.int32, device="cuda"))


def _check_product(q, s, t, g, y):
    """y of the product on the token (q, s) the GPU used."""
    acc_ref = oracle.matmul_i32(q, t)
    assert_y_close(y.reshape(1, -1), oracle.rescale(acc_ref, s, g), acc_ref)
    return acc_ref


@pytest.mark.parametrize("n,k,with_add", [(2560, 2560, True), (3840, 2560, False),
                                          (2560, 6912, True), (1000, 100, True),
                                          (777, 8192, True), (129, 16, False)])
def test_norm_forward_residual(n, k, with_add):
    t, g, packed, gamma = _weights(140_000 + n + k, n, k)
    rng = np.random.default_rng(141_000 + n + k)
    x = rng.standard_normal((1, k)).astype(np.float32)
    add = (rng.standard_normal((1, k)) * 2).astype(np.float32)
    xq, scale, rowsum = _outs(k)
    x_out = torch.full((1, k), float("nan"), dtype=torch.float32, device="cuda")
    y = bl.norm_forward(dev(x), packed, gamma, n, bl.BL_NORM_RESIDUAL,
                        add=dev(add) if with_add else None, x_out=x_out if with_add else None,
                        xq=xq, scale=scale, rowsum=rowsum)
    v = oracle.add_f32(x, add) if with_add else x
    if with_add:
        np.testing.assert_array_equal(host(x_out).view(np.uint32), v.view(np.uint32))
    got = (host(xq), host(scale), host(rowsum))
    assert_quant_close(got, oracle.rmsnorm_quantize(v))
    _check_product(got[0], got[1], t, g, host(y))


@pytest.mark.parametrize("heads,kv,hd,k_in", [(20, 5, 128, 2560), (4, 2, 40, 512),
                                              (8, 8, 64, 1000)])
def test_norm_forward_gqa(heads, kv, hd, k_in):
    kk = heads * hd
    n = 300 + kk
    t, g, packed, gamma = _weights(142_000 + kk, n, kk)
    rng = np.random.default_rng(143_000 + kk)
    v_col = 7 + kv * hd
    qkv = rng.standard_normal((1, v_col + kv * hd + 3)).astype(np.float32)
    xq, scale, rowsum = _outs(kk)
    y = bl.norm_forward(dev(qkv), packed, gamma, n, bl.BL_NORM_GQA, v_col=v_col, heads=heads,
                        kv_heads=kv, head_dim=hd, xq=xq, scale=scale, rowsum=rowsum)
    got = (host(xq), host(scale), host(rowsum))
    v = oracle.gqa_expand(qkv[:, v_col:v_col + kv * hd], heads, kv)
    assert_quant_close(got, oracle.rmsnorm_quantize(v))
    _check_product(got[0], got[1], t, g, host(y))


@pytest.mark.parametrize("f,k", [(6912, 2560), (500, 640), (33, 16)])
def test_norm_forward_relu2_epilogue_and_f64_input(f, k):
    """up/gate with the squared-ReLU gate in the epilogue, then its double
    output as the next product's input (the feed-forward block of one token)."""
    n = 2 * f
    t, g, packed, gamma = _weights(144_000 + f + k, n, k)
    rng = np.random.default_rng(145_000 + f + k)
    x = rng.standard_normal((1, k)).astype(np.float32)
    xq, scale, rowsum = _outs(k)
    v = bl.norm_forward(dev(x), packed, gamma, n, bl.BL_NORM_RESIDUAL, relu2=True, xq=xq,
                        scale=scale, rowsum=rowsum)
    q, s, r = host(xq), host(scale), host(rowsum)
    assert_quant_close((q, s, r), oracle.rmsnorm_quantize(x))
    acc = oracle.matmul_i32(q, t)
    # the product outputs as the GPU rounds them (double product, one rounding)
    y32 = oracle.rescale(acc, s, g).astype(np.float32)
    v_ref = oracle.relu2_mul(y32[:, :f], y32[:, f:])
    np.testing.assert_allclose(host(v).reshape(1, -1), v_ref, rtol=3e-7, atol=0)
    # next product: the double values as input (RMSNorm of relu2(...))
    k2, n2 = f, 640
    t2, g2, packed2, gamma2 = _weights(146_000 + f, n2, k2)
    xq2, scale2, rowsum2 = _outs(k2)
    y2 = bl.norm_forward(v, packed2, gamma2, n2, bl.BL_NORM_F64, xq=xq2, scale=scale2,
                         rowsum=rowsum2)
    got = (host(xq2), host(scale2), host(rowsum2))
    assert_quant_close(got, oracle.rmsnorm_quantize(host(v).reshape(1, -1)))
    _check_product(got[0], got[1], t2, g2, host(y2))


def test_norm_forward_end_to_end_from_the_oracle_chain():
    """The residual form against the oracle chain alone (no GPU intermediate):
    y within 1e-5 of rescale(matmul(rmsnorm_quantize(x + add))) where the codes
    agree, which is every position but rounding edges."""
    n, k = 3840, 2560
    t, g, packed, gamma = _weights(147_000, n, k)
    rng = np.random.default_rng(147_001)
    x = rng.standard_normal((1, k)).astype(np.float32)
    add = rng.standard_normal((1, k)).astype(np.float32)
    x_out = torch.empty((1, k), dtype=torch.float32, device="cuda")
    y = host(bl.norm_forward(dev(x), packed, gamma, n, add=dev(add), x_out=x_out))
    q, s, _ = oracle.rmsnorm_quantize(oracle.add_f32(x, add))
    acc = oracle.matmul_i32(q, t)
    y_ref = oracle.rescale(acc, s, g)
    rel = np.abs(y.astype(np.float64) - y_ref[0]) / np.maximum(np.abs(y_ref[0]), 1e-30)
    assert np.mean(rel <= 1e-5) > 0.999, float(np.mean(rel <= 1e-5))
