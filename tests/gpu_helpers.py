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


SUBNORMAL_ULP = 2.0 ** -149     # spacing of float32 below the normal range


def assert_y_close(y: np.ndarray, y_ref: np.ndarray, acc_ref: np.ndarray, rtol: float = 1e-5):
    """fp32 outputs within rtol of the fp64 oracle, elementwise; exact zeros
    where the integer accumulator is zero.  An output below the float32
    normal range cannot be nearer than half a subnormal spacing, so one
    subnormal spacing of absolute slack is allowed (it matters only for
    tokens with a near-zero scale)."""
    y = y.astype(np.float64)
    zero = acc_ref == 0
    assert np.all(y[zero] == 0.0)
    err = np.abs(y[~zero] - y_ref[~zero])
    excess = err - (rtol * np.abs(y_ref[~zero]) + SUBNORMAL_ULP)
    worst = float((err / np.abs(y_ref[~zero])).max()) if err.size else 0.0
    assert not np.any(excess > 0), f"max relative error {worst:.3e} > {rtol}"


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


def oracle_threads() -> int:
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_matmul_rows(q: np.ndarray, t: np.ndarray, threads: int = 0) -> np.ndarray:
    """oracle.matmul_i32 over row blocks of q on several host threads (the
    oracle's own function on each block; its ctypes call releases the GIL)."""
    import concurrent.futures
    threads = threads or oracle_threads()
    m = q.shape[0]
    if m < 2 * threads:
        return oracle.matmul_i32(q, t)
    bounds = np.linspace(0, m, threads + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: oracle.matmul_i32(q[bounds[i]:bounds[i + 1]], t),
                            range(threads)))
    return np.concatenate(parts, axis=0)


def oracle_backward_rows(g: np.ndarray, t: np.ndarray, gamma, threads: int = 0) -> np.ndarray:
    """oracle.backward_input over row blocks of grad_y on several host threads."""
    import concurrent.futures
    threads = threads or oracle_threads()
    m = g.shape[0]
    if m < 2 * threads:
        return oracle.backward_input(g, t, gamma)
    bounds = np.linspace(0, m, threads + 1).astype(int)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda i: oracle.backward_input(g[bounds[i]:bounds[i + 1]], t, gamma),
                            range(threads)))
    return np.concatenate(parts, axis=0)
