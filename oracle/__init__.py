"""CPU oracle for the BitNet b1.58 BitLinear layer (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline import this package; the product path never does.  The arithmetic
lives in ``bitlinear_oracle.c`` (plain scalar C, double precision where the
method is floating point); this module only builds that file with gcc, loads
it with ctypes and marshals numpy arrays.  It shares no code with the HIP
library.

Sources followed (see the C file for the per-function citations):
  * "1-bit LLM era: Microsoft introduces BitNet b1.58" (cheatsheet.md),
    section "What is BitNet b1.58?": absmean weight quantiser, per-token
    activation scaling, BitLinear in place of nn.Linear, no bias.
  * asi.tokyo article on BitNet b1.58 2B4T: 8-bit activations, four trits
    packed per byte and multiplied with the 8-bit values.
  * news.hada.io topic 20406, ternary-packing comment: five trits per byte.

Every function here is pinned against something other than itself by the
CPU tests (closed forms, brute force, library routines, invariants); none is
marked "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build() -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no fast-math, no FMA
    contraction, no excess precision) and return the library path."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
        "-o", _LIB_PATH + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    f64 = ctypes.c_double
    sig = {
        "orc_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "orc_absmean_gamma": (f32, [p, i32, i64, i64]),
        "orc_abs_sum": (f64, [p, i32, i64, p]),
        "orc_absmean_trits": (None, [p, i32, i64, i64, f32, p]),
        "orc_pack2_pitch": (i64, [i64]),
        "orc_pack2": (None, [p, i64, i64, p]),
        "orc_unpack2": (None, [p, i64, i64, p]),
        "orc_pack3_pitch": (i64, [i64]),
        "orc_pack3": (None, [p, i64, i64, p]),
        "orc_unpack3": (None, [p, i64, i64, p]),
        "orc_quantize_act": (None, [p, i32, i64, i64, p, p, p]),
        "orc_quantize_act_bits": (None, [p, i32, i64, i64, i32, p, p, p]),
        "orc_sign_trits": (None, [p, i32, i64, i64, p]),
        "orc_group_absmean": (None, [p, i32, i64, i64, i64, p]),
        "orc_rescale_groups": (None, [p, p, p, i64, i64, i64, p]),
        "orc_backward_input": (None, [p, i32, i64, i64, p, i64, f32, p]),
        "orc_matmul_i32": (None, [p, i64, p, i64, i64, p]),
        "orc_rescale": (None, [p, p, f32, i64, i64, p]),
        "orc_rmsnorm": (None, [p, i64, i64, ctypes.c_double, p]),
        "orc_relu2_mul": (None, [p, p, i64, p]),
        "orc_add_f32": (None, [p, p, i64]),
        "orc_gqa_expand": (None, [p, i64, i64, i64, i64, i64, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(a: np.ndarray):
    """Return (contiguous array, dtype code).  bf16 data travels as uint16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle input must be float32 or bf16 bits (uint16), got {a.dtype}")


# ---- scalar helpers ---------------------------------------------------------

def bf16_to_f32(bits) -> np.ndarray:
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.orc_bf16_to_f32(int(b)) for b in flat], dtype=np.float32)
    return out.reshape(np.shape(bits))


def pack2_pitch(k: int) -> int:
    return int(_load().orc_pack2_pitch(k))


def pack3_pitch(k: int) -> int:
    return int(_load().orc_pack3_pitch(k))


# ---- weights ----------------------------------------------------------------

def absmean_gamma(w: np.ndarray) -> np.float32:
    w, dt = _as_input(w)
    n, k = w.shape
    return np.float32(_load().orc_absmean_gamma(_ptr(w), dt, n, k))


def abs_sum(w: np.ndarray):
    """(sum of |w| rounded once to double, nonfinite flag: 0, 1 = inf, 2 = NaN)."""
    w, dt = _as_input(w)
    flag = np.zeros(1, dtype=np.int32)
    total = float(_load().orc_abs_sum(_ptr(w), dt, w.size, _ptr(flag)))
    return total, int(flag[0])


def absmean_trits(w: np.ndarray, gamma) -> np.ndarray:
    w, dt = _as_input(w)
    n, k = w.shape
    t = np.empty((n, k), dtype=np.int8)
    _load().orc_absmean_trits(_ptr(w), dt, n, k, float(np.float32(gamma)), _ptr(t))
    return t


def quantize_weights(w: np.ndarray):
    """W -> (trits int8 [N,K], gamma float32)."""
    g = absmean_gamma(w)
    return absmean_trits(w, g), g


def sign_trits(w: np.ndarray) -> np.ndarray:
    """1-bit variant [LUMEN]: -1 for w < 0, +1 otherwise."""
    w, dt = _as_input(w)
    n, k = w.shape
    t = np.empty((n, k), dtype=np.int8)
    _load().orc_sign_trits(_ptr(w), dt, n, k, _ptr(t))
    return t


def quantize_weights_binary(w: np.ndarray):
    """W -> (binary trits int8 [N,K] in {-1, +1}, beta = mean|W| float32)."""
    return sign_trits(w), absmean_gamma(w)


def group_absmean(w: np.ndarray, groups: int) -> np.ndarray:
    """Group quantisation [LUMEN]: beta[g] = mean |w| over rows
    g * N/groups .. (g+1) * N/groups - 1 (groups must divide N), float32 [groups]."""
    w, dt = _as_input(w)
    n, k = w.shape
    assert groups >= 1 and n % groups == 0
    beta = np.empty((groups,), dtype=np.float32)
    _load().orc_group_absmean(_ptr(w), dt, n, k, groups, _ptr(beta))
    return beta


def quantize_weights_binary_groups(w: np.ndarray, groups: int):
    """W -> (binary trits int8 [N,K] in {-1, +1}, beta float32 [groups])."""
    return sign_trits(w), group_absmean(w, groups)


def pack2(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.int8)
    n, k = t.shape
    out = np.empty((n, pack2_pitch(k)), dtype=np.uint8)
    _load().orc_pack2(_ptr(t), n, k, _ptr(out))
    return out


def unpack2(packed: np.ndarray, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    assert packed.shape[1] == pack2_pitch(k)
    t = np.empty((n, k), dtype=np.int8)
    _load().orc_unpack2(_ptr(packed), n, k, _ptr(t))
    return t


def pack3(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.int8)
    n, k = t.shape
    out = np.empty((n, pack3_pitch(k)), dtype=np.uint8)
    _load().orc_pack3(_ptr(t), n, k, _ptr(out))
    return out


def unpack3(packed: np.ndarray, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    assert packed.shape[1] == pack3_pitch(k)
    t = np.empty((n, k), dtype=np.int8)
    _load().orc_unpack3(_ptr(packed), n, k, _ptr(t))
    return t


# ---- activations ------------------------------------------------------------

def quantize_act(x: np.ndarray):
    """x [M,K] -> (q int8 [M,K], s float32 [M], rowsum int32 [M])."""
    x, dt = _as_input(x)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty((m,), dtype=np.float32)
    r = np.empty((m,), dtype=np.int32)
    _load().orc_quantize_act(_ptr(x), dt, m, k, _ptr(q), _ptr(s), _ptr(r))
    return q, s, r


def quantize_act_bits(x: np.ndarray, bits: int):
    """b-bit activations [CS, outlook]: Q = 2^(bits-1) - 1 in place of 127."""
    x, dt = _as_input(x)
    m, k = x.shape
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty((m,), dtype=np.float32)
    r = np.empty((m,), dtype=np.int32)
    _load().orc_quantize_act_bits(_ptr(x), dt, m, k, int(bits), _ptr(q), _ptr(s), _ptr(r))
    return q, s, r


# ---- backward (straight-through estimators) -----------------------------------

def backward_input(grad_y: np.ndarray, t: np.ndarray, gamma) -> np.ndarray:
    """grad_x [M,K] = gamma * grad_y [M,N] @ t [N,K], in float64."""
    g, dt = _as_input(grad_y)
    t = np.ascontiguousarray(t, dtype=np.int8)
    m, n = g.shape
    n2, k = t.shape
    assert n == n2
    out = np.empty((m, k), dtype=np.float64)
    _load().orc_backward_input(_ptr(g), dt, m, n, _ptr(t), k, float(np.float32(gamma)), _ptr(out))
    return out


# ---- contraction and rescale ------------------------------------------------

def matmul_i32(q: np.ndarray, t: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    t = np.ascontiguousarray(t, dtype=np.int8)
    m, k = q.shape
    n, k2 = t.shape
    assert k == k2
    acc = np.empty((m, n), dtype=np.int32)
    _load().orc_matmul_i32(_ptr(q), m, _ptr(t), n, k, _ptr(acc))
    return acc


def rescale(acc: np.ndarray, s: np.ndarray, gamma) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float64)
    _load().orc_rescale(_ptr(acc), _ptr(s), float(np.float32(gamma)), m, n, _ptr(y))
    return y


def rescale_groups(acc: np.ndarray, s: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """y[m, n] = acc[m, n] * beta[n // (N / groups)] / s[m] in float64."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    m, n = acc.shape
    groups = beta.shape[0]
    assert n % groups == 0
    y = np.empty((m, n), dtype=np.float64)
    _load().orc_rescale_groups(_ptr(acc), _ptr(s), _ptr(beta), groups, m, n, _ptr(y))
    return y


def forward(x: np.ndarray, t: np.ndarray, gamma):
    """Whole BitLinear forward from unquantised x and trits: returns
    (q, s, rowsum, acc, y) with y in float64."""
    q, s, r = quantize_act(x)
    acc = matmul_i32(q, t)
    return q, s, r, acc, rescale(acc, s, gamma)


# ---- decoder-block glue (layer-stack workload only) -------------------------

def rmsnorm(x: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    m, k = x.shape
    out = np.empty_like(x)
    _load().orc_rmsnorm(_ptr(x), m, k, float(eps), _ptr(out))
    return out


def relu2_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    gate = np.ascontiguousarray(gate, dtype=np.float64)
    up = np.ascontiguousarray(up, dtype=np.float64)
    assert gate.shape == up.shape
    out = np.empty_like(gate)
    _load().orc_relu2_mul(_ptr(gate), _ptr(up), gate.size, _ptr(out))
    return out


def add_f32(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """x + y in float32 (the residual stream); returns a new array."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    y = np.ascontiguousarray(y, dtype=np.float32)
    assert out.shape == y.shape
    _load().orc_add_f32(_ptr(out), _ptr(y), out.size)
    return out


def gqa_expand(v: np.ndarray, heads: int, kv_heads: int) -> np.ndarray:
    """v [M, kv_heads * head_dim] float32 -> [M, heads * head_dim] float64."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    m, width = v.shape
    head_dim = width // kv_heads
    assert head_dim * kv_heads == width and heads % kv_heads == 0
    out = np.empty((m, heads * head_dim), dtype=np.float64)
    _load().orc_gqa_expand(_ptr(v), m, width, heads, kv_heads, head_dim, _ptr(out))
    return out


def rmsnorm_quantize(v: np.ndarray, eps: float = 1e-5):
    """The input of a BitLinear in the decoder block: RMSNorm (unit gain, in
    double precision), rounded to float32, then the per-token absmax
    quantiser.  Returns (q, s, rowsum)."""
    h = rmsnorm(v, eps).astype(np.float32)
    return quantize_act(h)
