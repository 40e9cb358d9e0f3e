"""Helpers shared by the GPU tests: moving seeded inputs to the device and
running the oracle on the same bytes."""
import numpy as np
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def oracle_weights(w: np.ndarray, layout: int):
    t, g = oracle.quantize_weights(w)
    packed = oracle.pack2(t) if layout == bl.BL_PACK2 else oracle.pack3(t)
    return t, g, packed


def assert_y_close(y: np.ndarray, y_ref: np.ndarray, acc_ref: np.ndarray, rtol: float = 1e-5):
    """fp32 outputs within rtol of the fp64 oracle, elementwise; exact zeros
    where the integer accumulator is zero."""
    y = y.astype(np.float64)
    zero = acc_ref == 0
    assert np.all(y[zero] == 0.0)
    rel = np.abs(y[~zero] - y_ref[~zero]) / np.abs(y_ref[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= rtol, f"max relative error {worst:.3e} > {rtol}"


def assert_quant_close(got, want):
    """xq / scale / rowsum of the glue against the oracle's: codes may differ
    by one in at most 1 in 10^5 positions (rounding edges of the RMSNorm's
    double sum, reduced in another order), scales by 1e-6."""
    q, s, r = got
    q_ref, s_ref, r_ref = want
    diff = q.astype(np.int32) - q_ref.astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert np.count_nonzero(diff) <= max(1, q.size // 100_000), np.count_nonzero(diff)
    np.testing.assert_allclose(s, s_ref, rtol=1e-6)
    np.testing.assert_array_equal(r - r_ref, diff.sum(axis=1))
    assert np.array_equal(r, q.astype(np.int64).sum(axis=1))
