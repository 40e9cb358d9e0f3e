"""GPU parity: every HIP kernel against the CPU oracle on the same seeded
inputs, through the C ABI.

Bar: bit-exact for gamma, packed bytes, int8 activations, scales, row sums and
int32 accumulators; fp32 outputs within 1e-5 relative error of the oracle's
double-precision rescale (exact zeros where the accumulator is zero).
"""
import numpy as np
import pytest
import torch

import oracle
from ternary_weight_linear_absmax_amd import bitlinear as bl
from ternary_weight_linear_absmax_amd import inputs

from gpu_helpers import assert_y_close, dev, host, oracle_matmul_rows, oracle_weights

pytestmark = pytest.mark.gpu

LAYOUTS = [bl.BL_PACK2, bl.BL_PACK3]


def run_case(w: np.ndarray, x: np.ndarray, layout: int, paths=(bl.BL_PATH_AUTO,)):
    """Full chain on both sides; returns nothing, asserts parity at every step."""
    n, k = w.shape
    t, g, packed_ref = oracle_weights(w, layout)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    acc_ref = oracle.matmul_i32(q_ref, t)
    y_ref = oracle.rescale(acc_ref, s_ref, g)

    packed, gamma = bl.quantize_weights(dev(w), layout)
    xq, scale, rowsum = bl.quantize_act(dev(x))
    assert host(gamma)[0] == g
    np.testing.assert_array_equal(host(packed), packed_ref)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale), s_ref)
    np.testing.assert_array_equal(host(rowsum), r_ref)
    np.testing.assert_array_equal(host(bl.unpack_weights(packed, n, k, layout)), t)
    m = x.shape[0]
    for path in paths:
        if path == bl.BL_PATH_SKINNY and not skinny_ok(m, k):
            continue
        if path == bl.BL_PATH_MFMA_WIDE and k % 16 != 0:
            continue
        acc = bl.matmul_i32(xq, rowsum, packed, n, k, layout, path=path)
        np.testing.assert_array_equal(host(acc), acc_ref, err_msg=f"path {path}")
        y = bl.forward(xq, scale, rowsum, packed, gamma, n, k, layout, path=path)
        assert_y_close(host(y), y_ref, acc_ref)


def skinny_ok(m, k):
    return 1 <= m <= 64 and k % 256 == 0


def all_paths(layout):
    if layout == bl.BL_PACK2:
        return (bl.BL_PATH_AUTO, bl.BL_PATH_GEMV, bl.BL_PATH_MFMA, bl.BL_PATH_SKINNY,
                bl.BL_PATH_MFMA_WIDE)
    return (bl.BL_PATH_AUTO, bl.BL_PATH_GEMV)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_tiny_layer_fp32(layout):
    w, x = inputs.tiny()
    run_case(w, x, layout, all_paths(layout))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("m,n,k", [
    (1, 1, 1), (1, 7, 15), (3, 77, 100), (2, 33, 64), (4, 129, 65), (5, 130, 320),
    (1, 300, 2560), (9, 64, 1000), (130, 257, 200), (17, 300, 384), (64, 128, 256),
    (129, 129, 129), (200, 513, 1040),
])
def test_ragged_shapes_bf16(layout, m, n, k):
    w, x = inputs.random_case(10_000 + m * 7 + n * 13 + k, m, n, k, bf16=True)
    run_case(w, x, layout, all_paths(layout))


@pytest.mark.parametrize("m,n,k", [
    (5, 130, 256), (16, 1000, 2560), (12, 17, 512), (1, 33, 256), (8, 2560, 6912),
    (16, 4099, 8192), (7, 3840, 2560), (17, 300, 512), (32, 1000, 2560), (33, 130, 256),
    (64, 2560, 6912), (50, 4099, 1024),
    # up to 16 tokens on at least 192 blocks of 64 rows: activations shared
    # through LDS, ragged last row block and token slots
    (13, 12300, 512), (16, 13824, 2560), (1, 12289, 256), (5, 12352, 1024),
    # 96..191 row blocks with long rows: the k range split over blocks (two
    # splits), partial sums added by the finish kernel; ragged and aligned N
    (13, 6150, 8192), (16, 6144, 12288),
    # 128-row blocks: >= 160 of them unsplit (ragged last block), 34 of them
    # with 32 stages of 512 k split four ways, and stages of 256 k where
    # K % 512 != 0
    (13, 20483, 4096), (16, 4229, 16384), (16, 20480, 4352),
    # 64-row blocks with stages of 512 k (K % 512 = 0), ragged N and M
    (5, 12300, 1536), (13, 12352, 1024),
])
def test_skinny_shapes(m, n, k):
    """Weight-streaming matrix-core path: ragged N and M, every row-block /
    wave split and token-group count."""
    w, x = inputs.random_case(20_000 + m * 7 + n * 13 + k, m, n, k, bf16=True)
    run_case(w, x, bl.BL_PACK2, (bl.BL_PATH_SKINNY, bl.BL_PATH_MFMA, bl.BL_PATH_MFMA_WIDE))
    if m <= 16:
        assert bl.forward_path(m, n, k) == (bl.BL_PATH_GEMV if m <= 2 else bl.BL_PATH_SKINNY)


@pytest.mark.parametrize("n", [13824, 6144])
def test_skinny_output_not_16_byte_aligned(n):
    """The skinny epilogue stores rows of four as 16-byte vectors only where
    the output stays aligned; an output offset by one float takes the
    element-wise stores (unsplit and split k range)."""
    m, k = 9, 8192
    w, x = inputs.random_case(20_500 + n, m, n, k, bf16=True)
    t, g, _ = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    acc_ref = oracle.matmul_i32(q_ref, t)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    buf = torch.empty(m * n + 1, dtype=torch.float32, device="cuda")
    y = buf[1:].view(m, n)
    bl.forward(xq, scale, rowsum, packed, gamma, n, k, y=y, path=bl.BL_PATH_SKINNY)
    assert_y_close(host(y), oracle.rescale(acc_ref, s_ref, g), acc_ref)


@pytest.mark.parametrize("n,k", [(129, 16), (77, 1040), (1000, 8000), (33, 80), (2049, 5120)])
def test_base3_one_token_shapes(n, k):
    """Table-decoded base-3 GEMV (one token, K a multiple of 16): ragged N,
    chunks of 80 trits that run past K, one and two chunks per lane."""
    w, x = inputs.random_case(50_000 + n + k, 1, n, k, bf16=True)
    run_case(w, x, bl.BL_PACK3, (bl.BL_PATH_AUTO,))


@pytest.mark.parametrize("n,k", [(4097, 12801), (5000, 2561), (4100, 1283), (6001, 6401)])
def test_base3_partial_sum_tables(n, k):
    """Base-3 GEMV for one token on matrices of many rows with K not a
    multiple of 16: per-group tables of partial sums, the k range in slices
    of 256 packed bytes (a short last slice, K not a multiple of 5), slices
    added by the split-k finish."""
    w, x = inputs.random_case(51_000 + n + k, 1, n, k, bf16=True)
    x[0, :7] = 0
    run_case(w, x, bl.BL_PACK3, (bl.BL_PATH_AUTO,))
    assert bl.forward_workspace_bytes(1, n, k, bl.BL_PACK3) == (
        4 * n * ((bl.packed_row_bytes(k, bl.BL_PACK3) + 255) // 256)
        if bl.packed_row_bytes(k, bl.BL_PACK3) > 256 else 0)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_ragged_shapes_fp32_unaligned_k(layout):
    w, x = inputs.random_case(555, 6, 150, 201, bf16=False)
    run_case(w, x, layout, all_paths(layout))


def test_zero_token_and_zero_weight_rows():
    w, x = inputs.random_case(31, 4, 96, 320, bf16=True)
    x[2] = 0
    w[5] = 0
    for layout in LAYOUTS:
        run_case(w, x, layout, all_paths(layout))


def test_hadamard_weights_give_integer_walsh_hadamard():
    import scipy.linalg
    h = scipy.linalg.hadamard(512).astype(np.float32)
    _, x = inputs.random_case(32, 8, 1, 512, bf16=False)
    for layout in LAYOUTS:
        run_case(h, x, layout, all_paths(layout))


def test_max_k():
    k = bl.MAX_K
    w, x = inputs.random_case(33, 2, 3, k, bf16=True)
    run_case(w, x, bl.BL_PACK2, all_paths(bl.BL_PACK2))
    run_case(w, x, bl.BL_PACK3, all_paths(bl.BL_PACK3))


def test_empty_products_are_noops():
    w, x = inputs.random_case(34, 2, 16, 64, bf16=True)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    y = bl.forward(xq[:0], scale[:0], rowsum[:0], packed, gamma, 16, 64)
    assert y.shape == (0, 16)
    y = bl.forward(xq, scale, rowsum, packed[:0], gamma, 0, 64)
    assert y.shape == (2, 0)
    torch.cuda.synchronize()


def test_repeated_calls_are_bit_identical():
    _, w, x = inputs.decode(3, m=3)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    n, k = w.shape
    for path in (bl.BL_PATH_GEMV, bl.BL_PATH_MFMA, bl.BL_PATH_SKINNY, bl.BL_PATH_MFMA_WIDE):
        ys = [host(bl.forward(xq, scale, rowsum, packed, gamma, n, k, path=path)) for _ in range(3)]
        assert all(np.array_equal(ys[0].view(np.uint32), v.view(np.uint32)) for v in ys[1:])


# ---- decode shapes of the 2B-class model, M = 1 (full parity) ---------------------------

@pytest.mark.parametrize("shape", range(len(inputs.DECODE_SHAPES)))
def test_decode_shapes_m1(shape):
    _, w, x = inputs.decode(shape, m=1)
    run_case(w, x, bl.BL_PACK2, all_paths(bl.BL_PACK2))


@pytest.mark.parametrize("shape", range(len(inputs.DECODE_SHAPES)))
def test_decode_shapes_m1_base3(shape):
    _, w, x = inputs.decode(shape, m=1)
    run_case(w, x, bl.BL_PACK3)


# ---- prefill shapes of the 3B-class model, M = 512 (every output) ---------------------------

@pytest.mark.parametrize("shape", range(len(inputs.PREFILL_SHAPES)))
def test_prefill_shapes_m512_all_rows(shape):
    _, w, x = inputs.prefill(shape)
    n, k = w.shape
    print(f"prefill shape {shape}: M=512 N={n} K={k}", flush=True)
    t, g, packed_ref = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    assert host(gamma)[0] == g
    np.testing.assert_array_equal(host(packed), packed_ref)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale), s_ref)
    np.testing.assert_array_equal(host(rowsum), r_ref)
    acc = host(bl.matmul_i32(xq, rowsum, packed, n, k))
    y = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k))
    acc_ref = oracle_matmul_rows(q_ref, t)
    np.testing.assert_array_equal(acc, acc_ref)
    assert_y_close(y, oracle.rescale(acc_ref, s_ref, g), acc_ref)
    # the zero fraction the generator produces (30% forced near zero)
    zero_frac = float(np.mean(t == 0))
    assert 0.40 < zero_frac < 0.50


# ---- tiled GEMM block shapes with ragged edges ------------------------------------------------

@pytest.mark.parametrize("m,n,k", [
    (260, 12850, 272),    # 64 x 128 tiles (about 300 tiles of 128 x 128), K = 2 BK + 16
    (200, 14083, 400),    # 128 x 128 tiles, one round of the CUs, K = 3 BK + 16
    (129, 5121, 2000),    # 128 x 128 tiles, k range split three ways, K = 15 BK + 80
    (70, 3000, 4000),     # 64 x 64 tiles, k range split in two
])
def test_tiled_gemm_block_shapes(m, n, k):
    """Every block tile and split-K choice of the tiled path, each with a
    partial last tile in M, in N and in K (sampled tokens, every row)."""
    w, x = inputs.random_case(70_000 + m + n + k, m, n, k, bf16=True)
    t, g, packed_ref = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, _ = oracle.quantize_act(x)
    packed, gamma = bl.quantize_weights(dev(w))
    np.testing.assert_array_equal(host(packed), packed_ref)
    xq, scale, rowsum = bl.quantize_act(dev(x))
    assert bl.forward_path(m, n, k) in (bl.BL_PATH_MFMA, bl.BL_PATH_MFMA_WIDE)
    rows = np.array(sorted(r for r in {0, 1, 63, 64, 127, 128, m // 2, m - 2, m - 1} if r < m))
    acc_ref = oracle.matmul_i32(q_ref[rows], t)
    for path in (bl.BL_PATH_MFMA, bl.BL_PATH_MFMA_WIDE):
        acc = host(bl.matmul_i32(xq, rowsum, packed, n, k, path=path))
        y = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k, path=path))
        np.testing.assert_array_equal(acc[rows], acc_ref, err_msg=f"path {path}")
        assert_y_close(y[rows], oracle.rescale(acc_ref, s_ref[rows], g), acc_ref)


@pytest.mark.parametrize("m,n,k,cfg", [
    (256, 12288, 256, "128 x 128 tiles, one round of the CUs"),
    (256, 16640, 256, "64 x 128 tiles"),
    (256, 6144, 1024, "128 x 128 tiles, k range split in two"),
    (300, 12400, 272, "128 x 128 tiles, ragged M, N and K"),
    (500, 3100, 8688, "64 x 128 tiles in one round, stages of 256 k, ragged, partial last stage"),
    (384, 4000, 2000, "64 x 128 tiles in one round, stages of 256 k, K % 256 = 208"),
    (200, 4000, 8240, "128 x 128 tiles, stages of 256 k, k split four ways, ragged"),
    (130, 6000, 16, "128 x 128 tiles, one 16-value stage of the 256-k kernel"),
    (100, 12300, 272, "64 x 128 tiles, a whole and a 16-value stage of 256 k"),
])
def test_tiled_gemm_configs_every_output(m, n, k, cfg):
    """Every output of each tile configuration of the tiled GEMM (every
    accumulator register row of every tile), against the oracle."""
    w, x = inputs.random_case(71_000 + m + n + k, m, n, k, bf16=True)
    t, g, _ = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, _ = oracle.quantize_act(x)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    acc_ref = oracle_matmul_rows(q_ref, t)
    for path in (bl.BL_PATH_MFMA, bl.BL_PATH_MFMA_WIDE):
        acc = host(bl.matmul_i32(xq, rowsum, packed, n, k, path=path))
        np.testing.assert_array_equal(acc, acc_ref, err_msg=f"{cfg}, path {path}")
        y = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k, path=path))
        assert_y_close(y, oracle.rescale(acc_ref, s_ref, g), acc_ref)


@pytest.mark.parametrize("m,n,k", [
    (300, 1100, 272),      # three stages (below the unrolled loop), ragged everything
    (130, 5000, 2000),     # k range split in two, sixteen stages
    (64, 513, 4096),       # two tiles, k range split four ways, one valid column
    (200, 700, 16),        # one 16-value stage
    (150, 777, 512),       # rows of an odd number of floats (element-wise stores)
    (1, 600, 640), (33, 2049, 1040), (512, 8640, 3200),
])
def test_wide_gemm_every_output(m, n, k):
    """The wide-tile GEMM (64 x 512 block tiles) on every output: partial
    token, column and k tiles, split k slices, stage counts inside and outside
    the unrolled loop."""
    w, x = inputs.random_case(74_000 + m + n + k, m, n, k, bf16=True)
    t, g, _ = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, _ = oracle.quantize_act(x)
    packed, gamma = bl.quantize_weights(dev(w))
    xq, scale, rowsum = bl.quantize_act(dev(x))
    acc_ref = oracle_matmul_rows(q_ref, t)
    acc = host(bl.matmul_i32(xq, rowsum, packed, n, k, path=bl.BL_PATH_MFMA_WIDE))
    np.testing.assert_array_equal(acc, acc_ref)
    y = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k, path=bl.BL_PATH_MFMA_WIDE))
    assert_y_close(y, oracle.rescale(acc_ref, s_ref, g), acc_ref)


def test_tiled_gemm_operands_beyond_32_bit_offsets():
    """M * K >= 2^31 bytes of activations: the GEMM runs in blocks of rows
    whose per-lane offsets fit 32 bits.  Activations drawn on the GPU (4 GB of
    bf16) and quantised there; rows around the block boundary and a sample of
    others are checked against the oracle on the int8 rows the GPU produced
    (whose quantisation is itself pinned elsewhere)."""
    m, n, k = (1 << 20) + 300, 72, 2048
    assert m * k >= 1 << 31
    w, _ = inputs.random_case(72_000, 1, n, k, bf16=True)
    t, g, _ = oracle_weights(w, bl.BL_PACK2)
    packed, gamma = bl.quantize_weights(dev(w))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(72_001)
    x = torch.randn((m, k), generator=gen, device="cuda", dtype=torch.bfloat16)
    xq, scale, rowsum = bl.quantize_act(x)
    del x
    boundary = ((1 << 31) - 1) // k // 128 * 128          # first row of the second block
    rows = np.unique(np.concatenate([
        np.arange(0, 130), np.arange(boundary - 200, boundary + 200), np.arange(m - 130, m),
        np.random.default_rng(5).choice(m, size=400, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    q_rows = host(xq[ridx])
    acc_ref = oracle.matmul_i32(q_rows, t)
    np.testing.assert_array_equal(host(rowsum[ridx]), q_rows.astype(np.int64).sum(axis=1))
    for path in (bl.BL_PATH_MFMA, bl.BL_PATH_MFMA_WIDE):
        print(f"beyond 32-bit offsets: path {path}", flush=True)
        y = bl.forward(xq, scale, rowsum, packed, gamma, n, k, path=path)
        acc = bl.matmul_i32(xq, rowsum, packed, n, k, path=path)
        np.testing.assert_array_equal(host(acc[ridx]), acc_ref)
        assert_y_close(host(y[ridx]), oracle.rescale(acc_ref, host(scale[ridx]), g), acc_ref)
        del y, acc


@pytest.mark.parametrize("bf16", [True, False])
def test_scale_overflow_tokens(bf16):
    """Tokens whose max |x| is below 127 / FLT_MAX: s is the largest finite
    float (not infinity), zeros stay 0, y stays finite; quantiser, b-bit
    quantiser and the one-token fused GEMV against the oracle."""
    m, n, k = 3, 200, 512
    w, x = inputs.random_case(73_000 + int(bf16), m, n, k, bf16=False)
    x = x * np.float32(1e-38)
    x[:, ::7] = 0.0
    x[1, 5] = np.float32(3e-37)
    x[2] = x[2] * np.float32(1e-2)                 # subnormal magnitudes (bf16 too)
    x[2, 3] = np.float32(2e-40)
    if bf16:
        x = inputs.f32_to_bf16_bits(x)
    t, g, _ = oracle_weights(w, bl.BL_PACK2)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    assert np.all(s_ref == np.finfo(np.float32).max)
    packed, gamma = bl.quantize_weights(dev(w))
    xd = dev(x)
    xq, scale, rowsum = bl.quantize_act(xd)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale), s_ref)
    np.testing.assert_array_equal(host(rowsum), r_ref)
    acc_ref = oracle.matmul_i32(q_ref, t)
    y = host(bl.forward(xq, scale, rowsum, packed, gamma, n, k))
    assert np.isfinite(y).all()
    assert_y_close(y, oracle.rescale(acc_ref, s_ref, g), acc_ref)
    q4, s4, r4 = oracle.quantize_act_bits(x, 4)
    got = bl.quantize_act(xd, bits=4)
    for a, b in zip(got, (q4, s4, r4)):
        np.testing.assert_array_equal(host(a), b)
    y1, xq1, s1, r1 = bl.quantize_forward(dev(x[:1]), packed, gamma, n)
    np.testing.assert_array_equal(host(xq1), q_ref[:1])
    np.testing.assert_array_equal(host(s1), s_ref[:1])
    assert_y_close(host(y1), oracle.rescale(acc_ref[:1], s_ref[:1], g), acc_ref[:1])


# ---- 70B-class layer (single GPU), M in {1, 16, 128}; base-3 at M = 1 -------------------------

@pytest.mark.parametrize("shape", range(len(inputs.XL_SHAPES)))
def test_xl_layer(shape):
    _, w, x = inputs.xl(shape, m=128)
    n, k = w.shape
    t, g = oracle.quantize_weights(w)
    p2_ref = oracle.pack2(t)
    wd = dev(w)
    packed, gamma = bl.quantize_weights(wd)
    packed3, gamma3 = bl.quantize_weights(wd, bl.BL_PACK3)
    del wd
    assert host(gamma)[0] == g and host(gamma3)[0] == g
    np.testing.assert_array_equal(host(packed), p2_ref)
    del p2_ref
    np.testing.assert_array_equal(host(packed3), oracle.pack3(t))
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    xq, scale, rowsum = bl.quantize_act(dev(x))
    np.testing.assert_array_equal(host(xq), q_ref)
    acc_all = oracle_matmul_rows(q_ref, t)        # every row of every M below
    for m in inputs.XL_MS:
        print(f"xl shape {shape}: M={m}", flush=True)
        acc = host(bl.matmul_i32(xq[:m], rowsum[:m], packed, n, k))
        acc_ref = acc_all[:m]
        np.testing.assert_array_equal(acc, acc_ref, err_msg=f"M={m}")
        y = host(bl.forward(xq[:m], scale[:m], rowsum[:m], packed, gamma, n, k))
        assert_y_close(y, oracle.rescale(acc_ref, s_ref[:m], g), acc_ref)
        if m == 1:
            acc3 = host(bl.matmul_i32(xq[:1], rowsum[:1], packed3, n, k, bl.BL_PACK3))
            np.testing.assert_array_equal(acc3, acc)      # base-3 == 2-bit, bit for bit


# ---- quantise + multiply in one call -------------------------------------------------------

@pytest.mark.parametrize("m,n,k,bf16,layout,path", [
    (1, 300, 2560, True, bl.BL_PACK2, bl.BL_PATH_AUTO),
    (2, 77, 1040, False, bl.BL_PACK2, bl.BL_PATH_AUTO),      # fp32, K % 64 != 0
    (4, 129, 528, True, bl.BL_PACK2, bl.BL_PATH_GEMV),       # four tokens on the vector path
    (3, 50, 100, True, bl.BL_PACK2, bl.BL_PATH_AUTO),        # K % 16 != 0
    (5, 130, 320, True, bl.BL_PACK2, bl.BL_PATH_GEMV),       # two groups of tokens
    (1, 1000, 4096, False, bl.BL_PACK2, bl.BL_PATH_AUTO),
    (8, 1000, 512, True, bl.BL_PACK2, bl.BL_PATH_AUTO),      # skinny
    (64, 200, 384, True, bl.BL_PACK2, bl.BL_PATH_AUTO),      # tiled GEMM
    (1, 100, 640, True, bl.BL_PACK3, bl.BL_PATH_AUTO),       # base-3
    (1, 2560, 6912, True, bl.BL_PACK2, bl.BL_PATH_AUTO),     # decode "down" shape
    # one token, quantised inside the vector kernel: two chunks per lane,
    # four waves per row, partial last chunk, both input types
    (1, 5000, 8192, True, bl.BL_PACK2, bl.BL_PATH_AUTO),
    (1, 300, 28672, False, bl.BL_PACK2, bl.BL_PATH_AUTO),    # too long: two launches
    (1, 100, 8192, False, bl.BL_PACK2, bl.BL_PATH_AUTO),     # 16 input vectors per thread
    (1, 77, 1040, True, bl.BL_PACK2, bl.BL_PATH_GEMV),
    (1, 129, 1040, False, bl.BL_PACK2, bl.BL_PATH_AUTO),
    (1, 40, 16, True, bl.BL_PACK2, bl.BL_PATH_AUTO),
])
def test_quantize_forward(m, n, k, bf16, layout, path):
    w, x = inputs.random_case(40_000 + m * 7 + n * 13 + k, m, n, k, bf16=bf16)
    if m >= 2:
        x[1] = 0                                              # an all-zero token
    t, g, _ = oracle_weights(w, layout)
    q_ref, s_ref, r_ref = oracle.quantize_act(x)
    acc_ref = oracle.matmul_i32(q_ref, t)
    y_ref = oracle.rescale(acc_ref, s_ref, g)
    packed, gamma = bl.quantize_weights(dev(w), layout)
    xd = dev(x)
    y, xq, scale, rowsum = bl.quantize_forward(xd, packed, gamma, n, layout, path=path)
    np.testing.assert_array_equal(host(xq), q_ref)
    np.testing.assert_array_equal(host(scale), s_ref)
    np.testing.assert_array_equal(host(rowsum), r_ref)
    assert_y_close(host(y), y_ref, acc_ref)
    # the workspace contents do not matter: garbage in it gives the same y
    torch.cuda.synchronize()
    for ws in bl._workspaces.values():
        ws.fill_(0xA5)
    y3, _, _, _ = bl.quantize_forward(xd, packed, gamma, n, layout, path=path)
    assert np.array_equal(host(y).view(np.uint32), host(y3).view(np.uint32))
    # bit-identical to the two separate calls
    xq2, s2, r2 = bl.quantize_act(xd)
    y2 = bl.forward(xq2, s2, r2, packed, gamma, n, k, layout, path=path)
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


@pytest.mark.parametrize("bf16", [True, False])
def test_quantize_forward_zero_token(bf16):
    """One all-zero token through the fused one-token kernel: s = 1, q = 0,
    row sum 0, y = 0 exactly."""
    n, k = 333, 2560
    w, x = inputs.random_case(41_000 + int(bf16), 1, n, k, bf16=bf16)
    x[:] = 0
    packed, gamma = bl.quantize_weights(dev(w))
    y, xq, scale, rowsum = bl.quantize_forward(dev(x), packed, gamma, n)
    assert host(scale)[0] == 1.0 and host(rowsum)[0] == 0
    assert not host(xq).any()
    assert np.array_equal(host(y), np.zeros((1, n), dtype=np.float32))
