"""The per-token absmax quantiser alone, bit for bit against the oracle, over
every kernel branch (bf16 / fp32 rows held in registers, rows too long for
them, lengths that are not a multiple of the vector width) and the edge
rows the definition has: an all-zero row (s = 1, q = 0), exact ties of x * s
(rounded to even), a negative maximum at the last position, tiny and
outlier magnitudes."""
import numpy as np
import pytest

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import dev, host

pytestmark = pytest.mark.gpu

# register kernel up to 32768 bf16 / 16384 fp32 values a row when the row is a
# whole number of 16-byte vectors; the streaming kernel otherwise
WIDTHS = [1, 7, 8, 12, 64, 800, 2560, 6912, 8200, 16384, 16388, 32768, 32776, 40000]


def rows(k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((7, k)).astype(np.float32)
    x[0] = 0.0
    # max |x| = 254 gives s = 0.5: 1, 3, -5 land on exact ties (0, 2, -2)
    ties = np.array([254.0, 1.0, 3.0, -5.0, 7.0, -9.0, 0.5, -253.0], dtype=np.float32)
    x[1] = np.resize(ties, k) if k >= 8 else ties[:k]
    x[2] = -np.abs(x[2]) * 0.5
    x[2, -1] = -10.0                                  # negative maximum, last position
    x[3] *= 1e-30                                     # tiny but normal magnitudes
    x[4, rng.integers(0, k, size=max(1, k // 100))] *= 20.0   # outlier channels
    x[5] = 1.0                                        # constant row: every q = 127
    x[6] *= 1e4
    return x


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("k", WIDTHS)
def test_quantiser_branches_bit_exact(k, bf16):
    x = rows(k, 600 + k)
    xin = inputs.f32_to_bf16_bits(x) if bf16 else x
    q_ref, s_ref, r_ref = oracle.quantize_act(xin)
    xq, scale, rowsum = bl.quantize_act(dev(xin))
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(rowsum), r_ref)
    assert host(scale)[0] == 1.0 and not host(xq)[0].any()
    if k >= 8:
        assert list(q_ref[1, :4]) == [127, 0, 2, -2]


def test_quantiser_many_tokens():
    rng = np.random.default_rng(611)
    x = inputs.f32_to_bf16_bits(rng.standard_normal((3001, 2560)).astype(np.float32))
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    xq, scale, rowsum = bl.quantize_act(dev(x))
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale).view(np.uint32), s_ref.view(np.uint32))
    np.testing.assert_array_equal(host(rowsum), r_ref)
