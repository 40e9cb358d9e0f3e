"""Python binding of libbitlinear (ctypes).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
The names mirror the C ABI in include/bitlinear.h.  If the library has not
been built this module raises at first use: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbitlinear.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "bitlinear.h")

# enums of bitlinear.h
BL_OK = 0
BL_F32, BL_BF16 = 0, 1
BL_PACK2, BL_PACK3 = 0, 1
BL_PATH_AUTO, BL_PATH_GEMV, BL_PATH_MFMA, BL_PATH_SKINNY, BL_PATH_MFMA_WIDE = 0, 1, 2, 3, 4
BL_NORM_RESIDUAL, BL_NORM_GQA, BL_NORM_F64 = 0, 1, 2
MAX_K = 1 << 20

_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def header_functions() -> list[str]:
    """Names of the functions that include/bitlinear.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def load():
    """Load libbitlinear.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "bitlinear_packed_row_bytes": (i64, [i64, i32]),
        "bitlinear_packed_bytes": (i64, [i64, i64, i32]),
        "bitlinear_quantize_weights_workspace_bytes": (i64, [i64, i64]),
        "bitlinear_forward_workspace_bytes": (i64, [i64, i64, i64, i32]),
        "bitlinear_forward_path": (i32, [i64, i64, i64, i32]),
        "bitlinear_status_string": (ctypes.c_char_p, [i32]),
        "bitlinear_quantize_weights": (i32, [p, i32, i64, i64, i32, p, p, p, i64, p]),
        "bitlinear_quantize_act": (i32, [p, i32, i64, i64, p, p, p, p]),
        "bitlinear_quantize_weights_binary": (i32, [p, i32, i64, i64, i32, p, p, p, i64, p]),
        "bitlinear_quantize_act_bits": (i32, [p, i32, i64, i64, i32, p, p, p, p]),
        "bitlinear_quantize_weights_binary_groups": (i32, [p, i32, i64, i64, i64, i32, p, p, p,
                                                           i64, p]),
        "bitlinear_forward_groups": (i32, [p, p, p, i64, p, i32, p, i64, i64, i64, p, p, i64,
                                           i32, p]),
        "bitlinear_backward_input": (i32, [p, i32, i64, i64, p, i32, p, i64, p, p]),
        "bitlinear_forward": (i32, [p, p, p, i64, p, i32, p, i64, i64, p, p, i64, p]),
        "bitlinear_forward_ex": (i32, [p, p, p, i64, p, i32, p, i64, i64, p, p, i64, i32, p]),
        "bitlinear_forward_noalloc": (i32, [p, p, p, i64, p, i32, p, i64, i64, p, i32, p]),
        "bitlinear_matmul_i32": (i32, [p, p, i64, p, i32, i64, i64, p, p, i64, i32, p]),
        "bitlinear_unpack_weights": (i32, [p, i32, i64, i64, p, p]),
        "bitlinear_residual_rmsnorm_quantize": (i32, [p, p, i64, i64, ctypes.c_float, p, p, p, p]),
        "bitlinear_gqa_rmsnorm_quantize": (i32, [p, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                                 p, p, p, p]),
        "bitlinear_relu2_rmsnorm_quantize": (i32, [p, i64, i64, i64, ctypes.c_float, p, p, p, p]),
        "bitlinear_quantize_forward": (i32, [p, i32, i64, i64, p, p, p, p, i32, p, i64, p, p, i64,
                                             i32, p]),
        "bitlinear_forward_glue_workspace_bytes": (i64, [i64, i64, i64]),
        "bitlinear_norm_forward": (i32, [i32, p, p, p, i64, i64, i64, i64, i64, ctypes.c_float, p,
                                         p, i64, i32, p, p, p, p, p]),
        "bitlinear_forward_residual_rmsnorm_quantize": (
            i32, [p, p, p, i64, i64, p, p, i64, p, ctypes.c_float, p, p, p, p, i64, p]),
        "bitlinear_forward_gqa_rmsnorm_quantize": (
            i32, [p, p, p, i64, i64, p, p, i64, i64, i64, i64, i64, ctypes.c_float, p, p, p, p,
                  i64, p]),
        "bitlinear_forward_relu2_rmsnorm_quantize": (
            i32, [p, p, p, i64, i64, p, p, i64, i64, ctypes.c_float, p, p, p, p, i64, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != BL_OK:
        raise BitLinearError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BL_BF16
    if t.dtype == torch.float32:
        return BL_F32
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


# ---- host queries ----------------------------------------------------------------

def status_string(status: int) -> str:
    return load().bitlinear_status_string(status).decode()


def packed_row_bytes(k: int, layout: int = BL_PACK2) -> int:
    return int(load().bitlinear_packed_row_bytes(k, layout))


def packed_bytes(n: int, k: int, layout: int = BL_PACK2) -> int:
    return int(load().bitlinear_packed_bytes(n, k, layout))


def quantize_weights_workspace_bytes(n: int, k: int) -> int:
    return int(load().bitlinear_quantize_weights_workspace_bytes(n, k))


def forward_workspace_bytes(m: int, n: int, k: int, layout: int = BL_PACK2) -> int:
    return int(load().bitlinear_forward_workspace_bytes(m, n, k, layout))


def forward_path(m: int, n: int, k: int, layout: int = BL_PACK2) -> int:
    return int(load().bitlinear_forward_path(m, n, k, layout))


# ---- device calls -------------------------------------------------------------------

_workspaces = {}


def _zero_workspace(nbytes: int, device):
    """A per-device workspace, grown on demand and reused (the library needs no
    initial contents in it).  Calls on different streams that share it must not
    overlap; pass your own workspace for that."""
    key = torch.device(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros((nbytes,), dtype=torch.uint8, device=key)
        _workspaces[key] = ws
    return ws


def quantize_weights(w: torch.Tensor, layout: int = BL_PACK2, stream=None, binary: bool = False,
                     out=None, workspace: torch.Tensor = None):
    """w [N, K] (float32/bfloat16, on the GPU) -> (packed uint8 [N, row_bytes], gamma float32 [1]).
    binary: the sign binariser (bitlinear_quantize_weights_binary); gamma is then its scale.
    out: optional (packed, gamma) to write into; workspace: optional uint8 scratch of at
    least quantize_weights_workspace_bytes(N, K) bytes (no initial contents needed)."""
    lib = load()
    assert w.dim() == 2 and w.is_contiguous()
    n, k = w.shape
    if out is None:
        packed = torch.empty((n, packed_row_bytes(k, layout)), dtype=torch.uint8, device=w.device)
        gamma = torch.empty((1,), dtype=torch.float32, device=w.device)
    else:
        packed, gamma = out
    ws = workspace
    if ws is None:
        ws_bytes = quantize_weights_workspace_bytes(n, k)
        ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=w.device)
    name = "bitlinear_quantize_weights_binary" if binary else "bitlinear_quantize_weights"
    _check(getattr(lib, name)(_ptr(w), _dtype_code(w), n, k, layout, _ptr(packed), _ptr(gamma),
                              _ptr(ws), ws.numel(), _stream(stream)), name)
    return packed, gamma


def quantize_weights_binary_groups(w: torch.Tensor, groups: int, layout: int = BL_PACK2,
                                   stream=None, out=None, workspace: torch.Tensor = None):
    """Sign binariser with one scale per group of N / groups rows:
    w [N, K] -> (packed uint8 [N, row_bytes], beta float32 [groups])."""
    lib = load()
    assert w.dim() == 2 and w.is_contiguous()
    n, k = w.shape
    if out is None:
        packed = torch.empty((n, packed_row_bytes(k, layout)), dtype=torch.uint8, device=w.device)
        beta = torch.empty((groups,), dtype=torch.float32, device=w.device)
    else:
        packed, beta = out
    ws = workspace
    if ws is None:
        ws = torch.empty((max(quantize_weights_workspace_bytes(n, k), 16),), dtype=torch.uint8,
                         device=w.device)
    _check(lib.bitlinear_quantize_weights_binary_groups(
        _ptr(w), _dtype_code(w), n, k, groups, layout, _ptr(packed), _ptr(beta), _ptr(ws),
        ws.numel(), _stream(stream)), "bitlinear_quantize_weights_binary_groups")
    return packed, beta


def forward_groups(xq, scale, rowsum, packed, beta, n: int, k: int, layout: int = BL_PACK2,
                   path: int = BL_PATH_AUTO, y=None, workspace=None, stream=None):
    """y [M, N] float32 = (xq . t^T) * beta[group of n] / scale."""
    lib = load()
    m = xq.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    ws_bytes = forward_workspace_bytes(m, n, k, layout)
    if workspace is None and ws_bytes > 0:
        workspace = _zero_workspace(ws_bytes, xq.device)
    _check(lib.bitlinear_forward_groups(_ptr(xq), _ptr(scale), _ptr(rowsum), m, _ptr(packed),
                                        layout, _ptr(beta), beta.numel(), n, k, _ptr(y),
                                        _ptr(workspace),
                                        0 if workspace is None else workspace.numel(), path,
                                        _stream(stream)),
           "bitlinear_forward_groups")
    return y


def quantize_act(x: torch.Tensor, stream=None, bits: int = 8):
    """x [M, K] -> (xq int8 [M, K], scale float32 [M], rowsum int32 [M]).
    bits < 8: bitlinear_quantize_act_bits (range +-(2^(bits-1) - 1))."""
    lib = load()
    assert x.dim() == 2 and x.is_contiguous()
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    scale = torch.empty((m,), dtype=torch.float32, device=x.device)
    rowsum = torch.empty((m,), dtype=torch.int32, device=x.device)
    if bits == 8:
        _check(lib.bitlinear_quantize_act(_ptr(x), _dtype_code(x), m, k, _ptr(xq), _ptr(scale),
                                          _ptr(rowsum), _stream(stream)),
               "bitlinear_quantize_act")
    else:
        _check(lib.bitlinear_quantize_act_bits(_ptr(x), _dtype_code(x), m, k, bits, _ptr(xq),
                                               _ptr(scale), _ptr(rowsum), _stream(stream)),
               "bitlinear_quantize_act_bits")
    return xq, scale, rowsum


def backward_input(grad_y: torch.Tensor, packed, gamma, k: int, grad_x=None, stream=None):
    """grad_x [M, K] float32 = gamma * grad_y [M, N] @ t [N, K] (straight-through estimators)."""
    lib = load()
    assert grad_y.dim() == 2 and grad_y.is_contiguous()
    m, n = grad_y.shape
    if grad_x is None:
        grad_x = torch.empty((m, k), dtype=torch.float32, device=grad_y.device)
    _check(lib.bitlinear_backward_input(_ptr(grad_y), _dtype_code(grad_y), m, n, _ptr(packed),
                                        BL_PACK2, _ptr(gamma), k, _ptr(grad_x), _stream(stream)),
           "bitlinear_backward_input")
    return grad_x


def forward(xq, scale, rowsum, packed, gamma, n: int, k: int, layout: int = BL_PACK2,
            path: int = BL_PATH_AUTO, y=None, workspace=None, stream=None):
    """y [M, N] float32 = (xq . t^T) * gamma / scale."""
    lib = load()
    m = xq.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    ws_bytes = forward_workspace_bytes(m, n, k, layout)
    if workspace is None and ws_bytes > 0:
        workspace = _zero_workspace(ws_bytes, xq.device)
    _check(lib.bitlinear_forward_ex(_ptr(xq), _ptr(scale), _ptr(rowsum), m, _ptr(packed), layout,
                                    _ptr(gamma), n, k, _ptr(y), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), path,
                                    _stream(stream)),
           "bitlinear_forward_ex")
    return y


NOALLOC_SCRATCH_BYTES = 14 << 20


def forward_noalloc(xq, scale, rowsum, packed, gamma, n: int, k: int, layout: int = BL_PACK2,
                    path: int = BL_PATH_AUTO, y=None, stream=None):
    """bitlinear_forward_noalloc: the forward with the library's static scratch
    instead of a workspace (y must be passed in to allocate nothing here)."""
    lib = load()
    m = xq.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _check(lib.bitlinear_forward_noalloc(_ptr(xq), _ptr(scale), _ptr(rowsum), m, _ptr(packed),
                                         layout, _ptr(gamma), n, k, _ptr(y), path,
                                         _stream(stream)),
           "bitlinear_forward_noalloc")
    return y


def matmul_i32(xq, rowsum, packed, n: int, k: int, layout: int = BL_PACK2,
               path: int = BL_PATH_AUTO, acc=None, workspace=None, stream=None):
    """acc [M, N] int32 = xq . t^T exactly."""
    lib = load()
    m = xq.shape[0]
    if acc is None:
        acc = torch.empty((m, n), dtype=torch.int32, device=xq.device)
    ws_bytes = forward_workspace_bytes(m, n, k, layout)
    if workspace is None and ws_bytes > 0:
        workspace = _zero_workspace(ws_bytes, xq.device)
    _check(lib.bitlinear_matmul_i32(_ptr(xq), _ptr(rowsum), m, _ptr(packed), layout, n, k,
                                    _ptr(acc), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), path,
                                    _stream(stream)),
           "bitlinear_matmul_i32")
    return acc


def quantize_forward(x: torch.Tensor, packed, gamma, n: int, layout: int = BL_PACK2,
                     path: int = BL_PATH_AUTO, y=None, xq=None, scale=None, rowsum=None,
                     workspace=None, stream=None):
    """Per-token quantisation of x [M, K] followed by the product, in one call.
    Returns (y, xq, scale, rowsum)."""
    lib = load()
    assert x.dim() == 2 and x.is_contiguous()
    m, k = x.shape
    dev_ = x.device
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=dev_)
    if scale is None:
        scale = torch.empty((m,), dtype=torch.float32, device=dev_)
    if rowsum is None:
        rowsum = torch.empty((m,), dtype=torch.int32, device=dev_)
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=dev_)
    ws_bytes = forward_workspace_bytes(m, n, k, layout)
    if workspace is None and ws_bytes > 0:
        workspace = _zero_workspace(ws_bytes, dev_)
    _check(lib.bitlinear_quantize_forward(
        _ptr(x), _dtype_code(x), m, k, _ptr(xq), _ptr(scale), _ptr(rowsum), _ptr(packed), layout,
        _ptr(gamma), n, _ptr(y), _ptr(workspace), 0 if workspace is None else workspace.numel(),
        path, _stream(stream)), "bitlinear_quantize_forward")
    return y, xq, scale, rowsum


def _glue_outputs(m, k, device, xq, scale, rowsum):
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=device)
    if scale is None:
        scale = torch.empty((m,), dtype=torch.float32, device=device)
    if rowsum is None:
        rowsum = torch.empty((m,), dtype=torch.int32, device=device)
    return xq, scale, rowsum


def residual_rmsnorm_quantize(x: torch.Tensor, add=None, eps: float = 1e-5, xq=None, scale=None,
                              rowsum=None, stream=None):
    """x += add (in place, float32), then RMSNorm + per-token quantisation.
    Returns (xq, scale, rowsum)."""
    assert x.dtype == torch.float32 and x.dim() == 2 and x.is_contiguous()
    m, k = x.shape
    xq, scale, rowsum = _glue_outputs(m, k, x.device, xq, scale, rowsum)
    _check(load().bitlinear_residual_rmsnorm_quantize(_ptr(x), _ptr(add), m, k, eps, _ptr(xq),
                                                      _ptr(scale), _ptr(rowsum), _stream(stream)),
           "bitlinear_residual_rmsnorm_quantize")
    return xq, scale, rowsum


def gqa_rmsnorm_quantize(qkv: torch.Tensor, v_col: int, heads: int, kv_heads: int,
                         head_dim: int, eps: float = 1e-5, xq=None, scale=None, rowsum=None,
                         stream=None):
    """First-token GQA attention output from the QKV product, then RMSNorm +
    quantisation.  Returns (xq, scale, rowsum)."""
    assert qkv.dtype == torch.float32 and qkv.dim() == 2 and qkv.is_contiguous()
    m, ld = qkv.shape
    k = heads * head_dim
    xq, scale, rowsum = _glue_outputs(m, k, qkv.device, xq, scale, rowsum)
    _check(load().bitlinear_gqa_rmsnorm_quantize(_ptr(qkv), m, ld, v_col, heads, kv_heads,
                                                 head_dim, eps, _ptr(xq), _ptr(scale),
                                                 _ptr(rowsum), _stream(stream)),
           "bitlinear_gqa_rmsnorm_quantize")
    return xq, scale, rowsum


def relu2_rmsnorm_quantize(gate_up: torch.Tensor, f: int, eps: float = 1e-5, xq=None,
                           scale=None, rowsum=None, stream=None):
    """relu(gate)^2 * up from the fused up/gate product, then RMSNorm +
    quantisation.  Returns (xq, scale, rowsum)."""
    assert gate_up.dtype == torch.float32 and gate_up.dim() == 2 and gate_up.is_contiguous()
    m, ld = gate_up.shape
    xq, scale, rowsum = _glue_outputs(m, f, gate_up.device, xq, scale, rowsum)
    _check(load().bitlinear_relu2_rmsnorm_quantize(_ptr(gate_up), m, ld, f, eps, _ptr(xq),
                                                   _ptr(scale), _ptr(rowsum), _stream(stream)),
           "bitlinear_relu2_rmsnorm_quantize")
    return xq, scale, rowsum


def forward_glue_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(load().bitlinear_forward_glue_workspace_bytes(m, n, k))


def _fused_args(xq, n, workspace):
    m, k = xq.shape
    need = forward_glue_workspace_bytes(m, n, k)
    if workspace is None and m > 0:
        workspace = _zero_workspace(need, xq.device)
    nbytes = 0 if workspace is None else workspace.numel()
    return m, k, workspace, nbytes


def forward_residual_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n: int, x: torch.Tensor,
                                      eps: float = 1e-5, xq_out=None, scale_out=None,
                                      rowsum_out=None, workspace=None, stream=None):
    """x += BitLinear(xq) (in place), then RMSNorm + per-token quantisation of
    x into (xq_out, scale_out, rowsum_out), which may be xq, scale, rowsum."""
    assert x.dtype == torch.float32 and x.is_contiguous() and tuple(x.shape) == (xq.shape[0], n)
    m, k, ws, nbytes = _fused_args(xq, n, workspace)
    xq_out, scale_out, rowsum_out = _glue_outputs(m, n, xq.device, xq_out, scale_out, rowsum_out)
    _check(load().bitlinear_forward_residual_rmsnorm_quantize(
        _ptr(xq), _ptr(scale), _ptr(rowsum), m, k, _ptr(packed), _ptr(gamma), n, _ptr(x), eps,
        _ptr(xq_out), _ptr(scale_out), _ptr(rowsum_out), _ptr(ws), nbytes, _stream(stream)),
        "bitlinear_forward_residual_rmsnorm_quantize")
    return xq_out, scale_out, rowsum_out


def forward_gqa_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n: int, v_col: int, heads: int,
                                 kv_heads: int, head_dim: int, eps: float = 1e-5, xq_out=None,
                                 scale_out=None, rowsum_out=None, workspace=None, stream=None):
    """QKV = BitLinear(xq) [M, n], then the first-token GQA glue on it."""
    m, k, ws, nbytes = _fused_args(xq, n, workspace)
    xq_out, scale_out, rowsum_out = _glue_outputs(m, heads * head_dim, xq.device, xq_out,
                                                  scale_out, rowsum_out)
    _check(load().bitlinear_forward_gqa_rmsnorm_quantize(
        _ptr(xq), _ptr(scale), _ptr(rowsum), m, k, _ptr(packed), _ptr(gamma), n, v_col, heads,
        kv_heads, head_dim, eps, _ptr(xq_out), _ptr(scale_out), _ptr(rowsum_out), _ptr(ws),
        nbytes, _stream(stream)), "bitlinear_forward_gqa_rmsnorm_quantize")
    return xq_out, scale_out, rowsum_out


def forward_relu2_rmsnorm_quantize(xq, scale, rowsum, packed, gamma, n: int, f: int,
                                   eps: float = 1e-5, xq_out=None, scale_out=None,
                                   rowsum_out=None, workspace=None, stream=None):
    """gate_up = BitLinear(xq) [M, n], then the squared-ReLU glue on it."""
    m, k, ws, nbytes = _fused_args(xq, n, workspace)
    xq_out, scale_out, rowsum_out = _glue_outputs(m, f, xq.device, xq_out, scale_out, rowsum_out)
    _check(load().bitlinear_forward_relu2_rmsnorm_quantize(
        _ptr(xq), _ptr(scale), _ptr(rowsum), m, k, _ptr(packed), _ptr(gamma), n, f, eps,
        _ptr(xq_out), _ptr(scale_out), _ptr(rowsum_out), _ptr(ws), nbytes, _stream(stream)),
        "bitlinear_forward_relu2_rmsnorm_quantize")
    return xq_out, scale_out, rowsum_out


def norm_forward(src: torch.Tensor, packed, gamma, n: int, input: int = BL_NORM_RESIDUAL,
                 add=None, x_out=None, v_col: int = 0, heads: int = 1, kv_heads: int = 1,
                 head_dim: int = 1, k: int = None, eps: float = 1e-5, relu2: bool = False,
                 out=None, xq=None, scale=None, rowsum=None, stream=None):
    """One token: the input glue (residual / first-token GQA / double input),
    RMSNorm and quantisation, then the 2-bit product, in one launch
    (bitlinear_norm_forward).  Returns out: float [N], or with relu2 double
    [N/2] = relu(gate)^2 * up."""
    if k is None:
        k = heads * head_dim if input == BL_NORM_GQA else src.numel()
    dev_ = src.device
    if out is None:
        out = torch.empty((n // 2,) if relu2 else (n,), dtype=torch.float64 if relu2 else
                          torch.float32, device=dev_)
    _check(load().bitlinear_norm_forward(
        input, _ptr(src), _ptr(add), _ptr(x_out), v_col, heads, kv_heads, head_dim, k, eps,
        _ptr(packed), _ptr(gamma), n, int(relu2), _ptr(out), _ptr(xq), _ptr(scale), _ptr(rowsum),
        _stream(stream)), "bitlinear_norm_forward")
    return out


def unpack_weights(packed, n: int, k: int, layout: int = BL_PACK2, stream=None):
    lib = load()
    trits = torch.empty((n, k), dtype=torch.int8, device=packed.device)
    _check(lib.bitlinear_unpack_weights(_ptr(packed), layout, n, k, _ptr(trits), _stream(stream)),
           "bitlinear_unpack_weights")
    return trits


# names of the C ABI
bitlinear_quantize_weights = quantize_weights
bitlinear_quantize_act = quantize_act
bitlinear_forward = forward
bitlinear_forward_noalloc = forward_noalloc
bitlinear_quantize_weights_binary_groups = quantize_weights_binary_groups
bitlinear_forward_groups = forward_groups
bitlinear_norm_forward = norm_forward
bitlinear_matmul_i32 = matmul_i32
bitlinear_unpack_weights = unpack_weights
bitlinear_quantize_forward = quantize_forward
bitlinear_residual_rmsnorm_quantize = residual_rmsnorm_quantize
bitlinear_gqa_rmsnorm_quantize = gqa_rmsnorm_quantize
bitlinear_relu2_rmsnorm_quantize = relu2_rmsnorm_quantize
bitlinear_packed_bytes = packed_bytes
bitlinear_packed_row_bytes = packed_row_bytes
bitlinear_status_string = status_string
bitlinear_forward_glue_workspace_bytes = forward_glue_workspace_bytes
bitlinear_forward_residual_rmsnorm_quantize = forward_residual_rmsnorm_quantize
bitlinear_forward_gqa_rmsnorm_quantize = forward_gqa_rmsnorm_quantize
bitlinear_forward_relu2_rmsnorm_quantize = forward_relu2_rmsnorm_quantize
