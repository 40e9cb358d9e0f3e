"""bitlinear_forward_noalloc (the forward with the library's static scratch
array instead of a caller's workspace) against bitlinear_forward_ex on the
same inputs: two calls in a row, the second on a smaller product, so the
second call meets the first call's partial sums in the shared scratch.  Also
checks one case against the oracle and the rejection of a product whose
split-k partial sums do not fit the scratch.
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import assert_y_close, dev, host, oracle_weights

pytestmark = pytest.mark.gpu


def _prepared(seed, m, n, k):
    w, x = inputs.random_case(seed, m, n, k, bf16=True)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    return w, x, packed, gamma, xq, scale, rowsum


def _bits(a):
    return host(a).view(np.uint32)


# (first, second) products and the path both take; the first of each pair
# splits its k range, so it leaves partial sums in the scratch
PAIRS = [
    (((70, 3000, 4000), (37, 200, 2048)), bl.BL_PATH_AUTO),     # tiled GEMM, 2 splits each
    (((13, 6150, 8192), (9, 6144, 8192)), bl.BL_PATH_SKINNY),   # weight streaming, 4 splits
    (((64, 2560, 6912), (64, 640, 2560)), bl.BL_PATH_AUTO),     # layer-stack shapes
    (((5, 130, 320), (3, 77, 100)), bl.BL_PATH_AUTO),           # no scratch needed
]


@pytest.mark.parametrize("pair,path", PAIRS)
def test_noalloc_matches_forward_ex_twice(pair, path):
    print(f"noalloc pair {pair} path {path}", flush=True)
    for i, (m, n, k) in enumerate(pair):
        if i == 0 and m > 5:
            assert bl.forward_workspace_bytes(m, n, k) > 0
        _, _, packed, gamma, xq, scale, rowsum = _prepared(90_000 + m + n + k, m, n, k)
        y_ref = bl.forward(xq, scale, rowsum, packed, gamma, n, k, path=path)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        bl.forward_noalloc(xq, scale, rowsum, packed, gamma, n, k, path=path, y=y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y), _bits(y_ref), err_msg=f"call {i} {(m, n, k)}")


def test_noalloc_against_oracle():
    m, n, k = 70, 3000, 4000
    w, x, packed, gamma, xq, scale, rowsum = _prepared(91_000, m, n, k)
    t, g, _ = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, _ = oracle.quantize_act(x)
    acc_ref = oracle.matmul_i32(q_ref, t)
    y = bl.forward_noalloc(xq, scale, rowsum, packed, gamma, n, k)
    assert_y_close(host(y), oracle.rescale(acc_ref, s_ref, g), acc_ref)


def test_noalloc_rejects_products_beyond_the_scratch():
    m, n, k = 512, 2048, 8192
    assert bl.forward_workspace_bytes(m, n, k) > bl.NOALLOC_SCRATCH_BYTES
    xq = torch.zeros((m, k), dtype=torch.int8, device="cuda")
    scale = torch.ones((m,), dtype=torch.float32, device="cuda")
    rowsum = torch.zeros((m,), dtype=torch.int32, device="cuda")
    packed = torch.zeros((n, bl.packed_row_bytes(k)), dtype=torch.uint8, device="cuda")
    gamma = torch.ones((1,), dtype=torch.float32, device="cuda")
    y = torch.zeros((m, n), dtype=torch.float32, device="cuda")
    with pytest.raises(bl.BitLinearError) as err:
        bl.forward_noalloc(xq, scale, rowsum, packed, gamma, n, k, y=y)
    assert err.value.status == -9
    torch.cuda.synchronize()
    assert not host(y).any()                 # nothing was launched
