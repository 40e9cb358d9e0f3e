"""GPU parity of the variants: b-bit activations (bitlinear_quantize_act_bits)
and sign-binarised weights (bitlinear_quantize_weights_binary), each through
every product path, against the CPU oracle on the same seeded inputs.

Bar as for the main path: bit-exact quantiser outputs, packed bytes and int32
accumulators; fp32 outputs within 1e-5 relative (exact zeros where acc = 0).
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import assert_y_close, dev, host

pytestmark = pytest.mark.gpu

PATHS2 = (bl.BL_PATH_AUTO, bl.BL_PATH_GEMV, bl.BL_PATH_MFMA, bl.BL_PATH_SKINNY,
          bl.BL_PATH_MFMA_WIDE)


def _products(xq, scale, rowsum, packed, gamma, n, k, layout, q_ref, s_ref, t, g, m):
    acc_ref = oracle.matmul_i32(q_ref, t)
    y_ref = oracle.rescale(acc_ref, s_ref, g)
    paths = PATHS2 if layout == bl.BL_PACK2 else (bl.BL_PATH_AUTO,)
    for path in paths:
        if path == bl.BL_PATH_SKINNY and not (m <= 64 and k % 256 == 0):
            continue
        if path == bl.BL_PATH_MFMA_WIDE and k % 16 != 0:
            continue
        acc = host(bl.matmul_i32(xq, rowsum, packed, n, k, layout, path=path))
        np.testing.assert_array_equal(acc, acc_ref, err_msg=f"path {path}")
        y = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k, layout, path=path))
        assert_y_close(y, y_ref, acc_ref)


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("m,n,k,bf16", [(5, 130, 320, True), (1, 300, 2560, True),
                                         (40, 257, 512, False), (3, 77, 100, True)])
def test_act_bits_all_paths(bits, m, n, k, bf16):
    w, x = inputs.random_case(60_000 + 97 * bits + m + n + k, m, n, k, bf16=bf16)
    if m >= 3:
        x[2] = 0                                           # an all-zero token
    t, g = oracle.quantize_weights(w)
    q_ref, s_ref, r_ref = oracle.quantize_act_bits(x, bits)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x), bits=bits)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale), s_ref)
    np.testing.assert_array_equal(host(rowsum), r_ref)
    assert np.abs(host(xq)).max() <= 2 ** (bits - 1) - 1
    _products(xq, scale, rowsum, packed, gamma, n, k, bl.BL_PACK2, q_ref, s_ref, t, g, m)


@pytest.mark.parametrize("layout", [bl.BL_PACK2, bl.BL_PACK3])
@pytest.mark.parametrize("m,n,k,bf16", [(1, 300, 2560, True), (8, 1000, 512, True),
                                         (64, 200, 384, False), (4, 129, 65, True),
                                         (16, 12352, 1024, True)])
def test_binary_weights_all_paths(layout, m, n, k, bf16):
    w, x = inputs.random_case(61_000 + m + n + k, m, n, k, bf16=bf16)
    if bf16:
        w[0, :5] = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001], dtype=np.uint16)
    else:
        w[0, :4] = np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32)
    t, beta = oracle.quantize_weights_binary(w)
    packed_ref = oracle.pack2(t) if layout == bl.BL_PACK2 else oracle.pack3(t)
    packed, gamma = bl.quantize_weights(dev(w), layout, binary=True)
    assert host(gamma)[0] == beta
    np.testing.assert_array_equal(host(packed), packed_ref)
    np.testing.assert_array_equal(host(bl.unpack_weights(packed, n, k, layout)), t)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    xq, scale, rowsum = bl.quantize_act(dev(x))
    np.testing.assert_array_equal(host(xq), q_ref)
    _products(xq, scale, rowsum, packed, gamma, n, k, layout, q_ref, s_ref, t, beta, m)


def test_binary_weights_with_four_bit_activations():
    """Both variants together (the original-BitNet-style 1-bit weights against
    4-bit tokens), on the tiled and the vector path."""
    m, n, k = 33, 500, 768
    w, x = inputs.random_case(62_000, m, n, k, bf16=True)
    t, beta = oracle.quantize_weights_binary(w)
    q_ref, s_ref, _ = oracle.quantize_act_bits(x, 4)
    packed, gamma = bl.quantize_weights(dev(w), binary=True)
    xq, scale, rowsum = bl.quantize_act(dev(x), bits=4)
    _products(xq, scale, rowsum, packed, gamma, n, k, bl.BL_PACK2, q_ref, s_ref, t, beta, m)


# ---- group quantisation of the sign-binarised weights ---------------------------------

@pytest.mark.parametrize("layout", [bl.BL_PACK2, bl.BL_PACK3])
@pytest.mark.parametrize("m,n,k,groups", [(1, 300, 2560, 4), (8, 1000, 512, 8), (64, 200, 384, 2),
                                          (4, 128, 64, 128), (40, 2560, 1024, 1),
                                          (16, 12352, 1024, 16), (130, 640, 2048, 5)])
def test_binary_weight_groups_all_paths(layout, m, n, k, groups):
    """beta_g bit-exact per group, packed bytes and int32 accumulators exact on
    every path, y within 1e-5 of the oracle's per-group rescale."""
    w, x = inputs.random_case(63_000 + m + n + k + groups, m, n, k, bf16=True)
    wf = inputs.bf16_bits_to_f32(w)
    wf[: n // groups] *= np.float32(8.0)                  # groups of different scale
    w = inputs.f32_to_bf16_bits(wf)
    t, beta_ref = oracle.quantize_weights_binary_groups(w, groups)
    packed_ref = oracle.pack2(t) if layout == bl.BL_PACK2 else oracle.pack3(t)
    packed, beta = bl.quantize_weights_binary_groups(dev(w), groups, layout)
    np.testing.assert_array_equal(host(beta), beta_ref)
    np.testing.assert_array_equal(host(packed), packed_ref)
    q_ref, s_ref, _ = oracle.quantize_act(x)
    xq, scale, rowsum = bl.quantize_act(dev(x))
    acc_ref = oracle.matmul_i32(q_ref, t)
    y_ref = oracle.rescale_groups(acc_ref, s_ref, beta_ref)
    paths = PATHS2 if layout == bl.BL_PACK2 else (bl.BL_PATH_AUTO,)
    for path in paths:
        if path == bl.BL_PATH_SKINNY and not (m <= 64 and k % 256 == 0):
            continue
        if path == bl.BL_PATH_MFMA_WIDE and k % 16 != 0:
            continue
        y = host(bl.forward_groups(xq, scale, rowsum, packed, beta, n, k, layout, path=path))
        assert_y_close(y, y_ref, acc_ref)


def test_binary_weight_groups_argument_checks():
    w = torch.zeros((12, 64), dtype=torch.bfloat16, device="cuda")
    for groups in (0, 5, 13):
        with pytest.raises(bl.BitLinearError):
            bl.quantize_weights_binary_groups(w, groups)
