"""GPU parity of the backward input gradient (straight-through estimators):
grad_x = gamma * grad_y @ t over the packed 2-bit weights, against the
float64 oracle.

Bar: the kernel sums N exact products g * t (t in {-1, 0, 1}) in fp32 and
scales by gamma once, so each element is within the recursive-summation bound
gamma (N + 1) 2^-24 sum_n |g t| + 2^-24 |ref| of the exact value, whatever the
order; the relative L2 error over a whole case must also stay below 1e-6.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import dev, host, oracle_backward_rows

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _check(gx, g_bits_or_f32, t, gamma):
    ref = oracle_backward_rows(g_bits_or_f32, t, gamma)
    g = g_bits_or_f32
    gf = oracle.bf16_to_f32(g) if g.dtype == np.uint16 else g
    n = t.shape[0]
    mag = np.abs(gf.astype(np.float64)) @ np.abs(t.astype(np.float64))
    bound = float(np.float32(gamma)) * (n + 1) * U * mag + U * np.abs(ref) + 1e-37
    err = np.abs(gx.astype(np.float64) - ref)
    assert np.all(err <= bound), f"worst excess {float((err - bound).max()):.3e}"
    l2 = np.linalg.norm(gx.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    assert l2 <= 1e-6, f"relative L2 error {l2:.3e}"


def _grad(rng, m, n, bf16):
    g = (rng.standard_normal((m, n)) * 1e-3).astype(np.float32)
    return inputs.f32_to_bf16_bits(g) if bf16 else g


@pytest.mark.parametrize("m,n,k,bf16", [
    (1, 300, 2560, True), (5, 130, 320, False), (64, 1000, 512, True), (3, 77, 100, False),
    (2, 77, 100, True), (130, 257, 200, False), (65, 64, 129, True), (1, 1, 1, False),
    (7, 4099, 64, False),
    # long rows of grad_x (171 k tiles), ragged M and K
    (130, 64, 21800, True),
])
def test_backward_input_shapes(m, n, k, bf16):
    rng = np.random.default_rng(80_000 + m + n + k)
    w, _ = inputs.random_case(81_000 + m + n + k, 1, n, k, bf16=True)
    t, g = oracle.quantize_weights(w)
    packed, gamma = bl.quantize_weights(dev(w))
    assert host(gamma)[0] == g
    gy = _grad(rng, m, n, bf16)
    gx = host(bl.backward_input(dev(gy), packed, gamma, k))
    _check(gx, gy, t, g)


def test_backward_input_no_rows_gives_zero():
    gy = torch.zeros((3, 0), dtype=torch.float32, device="cuda")
    gamma = torch.ones((1,), dtype=torch.float32, device="cuda")
    packed = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    gx = bl.backward_input(gy, packed, gamma, 40)
    assert not host(gx).any()


@pytest.mark.parametrize("shape", range(len(inputs.PREFILL_SHAPES)))
def test_backward_input_prefill_shapes_all_rows(shape):
    """The 3B-class prefill matrices at M = 512, every element against the oracle."""
    _, w, _ = inputs.prefill(shape)
    n, k = w.shape
    print(f"backward prefill shape {shape}: M=512 N={n} K={k}", flush=True)
    t, g = oracle.quantize_weights(w)
    packed, gamma = bl.quantize_weights(dev(w))
    rng = np.random.default_rng(82_000 + shape)
    gy = _grad(rng, 512, n, True)
    gx = host(bl.backward_input(dev(gy), packed, gamma, k))
    _check(gx, gy, t, g)
