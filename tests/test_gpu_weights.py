"""GPU parity of the weight quantiser: gamma bit for bit and packed bytes
exactly, through the C ABI, on inputs chosen to reach every branch of the
exact summation (window accumulators, per-exponent bins, the tail that is not
a whole 16-byte vector, subnormals, non-finite values) and both packers'
vector and element-wise paths.

Sources: cheatsheet.md BitNet b1.58 summary, "What is BitNet b1.58?", weight
bullet (absmean scale, round, clip to {-1, 0, 1}); asi.tokyo 2B4T article
(four trits per byte); news.hada.io 20406 packing comment (five per byte).
"""
import numpy as np
import pytest

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import dev, host, oracle_weights

pytestmark = pytest.mark.gpu


def _bits_f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def check(w: np.ndarray, layouts=(bl.BL_PACK2, bl.BL_PACK3)):
    g_ref = oracle.absmean_gamma(w)
    for layout in layouts:
        packed, gamma = bl.quantize_weights(dev(w), layout)
        g = host(gamma)[0]
        if np.isnan(g_ref):
            assert np.isnan(g)
            continue
        assert g == g_ref, (g, g_ref)
        if np.isfinite(g_ref):
            _, _, packed_ref = oracle_weights(w, layout)
            np.testing.assert_array_equal(host(packed), packed_ref)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (5, 100), (64, 320), (40, 2560), (257, 1000)])
def test_gaussian_shapes(bf16, shape):
    rng = np.random.default_rng(shape[0] * 7919 + shape[1])
    w = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    check(inputs.f32_to_bf16_bits(w) if bf16 else w)


@pytest.mark.parametrize("bf16", [True, False])
def test_magnitudes_over_all_binades(bf16):
    # every element in its own binade: most fall outside a lane's window
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((96, 512)) * np.exp2(rng.integers(-140, 120, (96, 512)))).astype(np.float32)
    check(inputs.f32_to_bf16_bits(w) if bf16 else w, layouts=(bl.BL_PACK2,))


@pytest.mark.parametrize("bf16", [True, False])
def test_window_opened_on_small_values_then_large_ones(bf16):
    # rows of tiny weights first, then rows 2^40 larger: lanes open their
    # window on the tiny ones and must bin the later large ones exactly
    rng = np.random.default_rng(22)
    w = rng.standard_normal((512, 256), dtype=np.float32)
    w[:256] *= np.float32(2.0**-60)
    w[256:] *= np.float32(2.0**-20)
    check(inputs.f32_to_bf16_bits(w) if bf16 else w, layouts=(bl.BL_PACK2,))


@pytest.mark.parametrize("bf16", [True, False])
def test_sparse_rows_and_zero_vectors(bf16):
    rng = np.random.default_rng(23)
    w = rng.standard_normal((300, 640), dtype=np.float32) * np.float32(0.02)
    w[rng.random((300, 640)) < 0.97] = 0.0
    w[:100] = 0.0
    check(inputs.f32_to_bf16_bits(w) if bf16 else w)


def test_subnormals_and_near_max():
    rng = np.random.default_rng(24)
    sub = _bits_f32(rng.integers(1, 0x00800000, (16, 64)))
    big = _bits_f32(rng.integers(0x7E000000, 0x7F000000, (16, 64)))
    check(sub)
    check(big)
    check(np.concatenate([sub, big]))


def test_ties_and_tail_elements():
    # 2^60 + 2^7 is a tie between two doubles; the odd element count leaves a
    # tail that is not a whole 16-byte vector
    w = np.zeros((3, 7), np.float32)
    w[0, 0] = 2.0**60
    w[2, 6] = 2.0**7
    check(w, layouts=(bl.BL_PACK2,))
    w[1, 3] = 2.0**8
    check(w, layouts=(bl.BL_PACK2,))
    w[2, 5] = 2.0**-149
    check(w, layouts=(bl.BL_PACK2,))


def test_zero_matrix():
    check(np.zeros((33, 65), np.float32))


@pytest.mark.parametrize("value", [np.inf, -np.inf, np.nan])
@pytest.mark.parametrize("pos", [(0, 0), (31, 100), (63, 127)])
def test_nonfinite(value, pos):
    w = np.full((64, 128), 0.01, np.float32)
    w[pos] = value
    check(w, layouts=(bl.BL_PACK2,))


def test_binary_variant_scale_matches_oracle():
    rng = np.random.default_rng(25)
    w = inputs.f32_to_bf16_bits(rng.standard_normal((64, 1000), dtype=np.float32))
    packed, beta = bl.quantize_weights(dev(w), bl.BL_PACK2, binary=True)
    t_ref, b_ref = oracle.quantize_weights_binary(w)
    assert host(beta)[0] == b_ref
    np.testing.assert_array_equal(host(packed), oracle.pack2(t_ref))


@pytest.mark.parametrize("shape_index", [0, 1])
def test_70b_class_matrix_gamma_and_sampled_rows(shape_index):
    # full-size 70B-class matrices: gamma over all N*K elements (2048 blocks),
    # packed rows compared on a sample
    n, k = [(28672, 8192), (8192, 28672)][shape_index]
    w = inputs.normal_bf16(np.random.default_rng(26 + shape_index), (n, k), 0.02)
    g_ref = oracle.absmean_gamma(w)
    rows = np.random.default_rng(7).choice(n, 12, replace=False)
    for layout in (bl.BL_PACK2, bl.BL_PACK3):
        packed, gamma = bl.quantize_weights(dev(w), layout)
        assert host(gamma)[0] == g_ref
        t = oracle.absmean_trits(w[rows], g_ref)
        ref = oracle.pack2(t) if layout == bl.BL_PACK2 else oracle.pack3(t)
        np.testing.assert_array_equal(host(packed.view(n, -1)[rows]), ref)
