"""The 2B-class decoder layer stack of the layer-stack workload, driven through
the C ABI (argument marshalling only; every step runs in the library's
kernels).

Model shape (asi.tokyo BitNet b1.58 2B4T article; cheatsheet.md summary,
"What is BitNet b1.58?"): hidden 2560, 20 query heads and 5 key-value heads of
128, feed-forward 6912 with squared ReLU, RMSNorm in front of every BitLinear,
no bias.  The workload decodes the first token of M independent sequences
(sequence position 0), so attention reduces to the value vector of each
token's key-value head, expanded over its query-head group.

Per layer (x is the float residual stream, [M, 2560]):

    xq = quant(RMSNorm(x))                      bitlinear_residual_rmsnorm_quantize
    qkv = BitLinear_qkv(xq)                     [M, 3840]: Q 0..2559, K 2560..3199, V 3200..3839
    xq = quant(RMSNorm(GQA-expand(V)))          bitlinear_gqa_rmsnorm_quantize
    o = BitLinear_o(xq)
    x += o; xq = quant(RMSNorm(x))              bitlinear_residual_rmsnorm_quantize
    gu = BitLinear_up_gate(xq)                  [M, 13824]: gate 0..6911, up 6912..13823
    xq = quant(RMSNorm(relu(gate)^2 * up))      bitlinear_relu2_rmsnorm_quantize
    d = BitLinear_down(xq)
    x += d                                      (folded into the next layer's first call)

With `fused` set (the default) every product and the glue after it are one
call (bitlinear_forward_*_rmsnorm_quantize): where the GEMM splits its k
range, the glue kernel finishes the split partial sums itself, so the product
output is never stored and the finishing launch disappears.  The results are
bit for bit those of the unfused sequence.

With one token (M = 1) and `norm` set, each BitLinear takes its input glue as
a prologue instead (bitlinear_norm_forward: residual / GQA / double input,
RMSNorm and quantisation inside the product's blocks) and the up/gate product
applies relu(gate)^2 * up as its epilogue, so a layer is four launches:

    qkv = BitLinear_qkv(quant(RMSNorm(x += d)))            residual prologue
    o   = BitLinear_o(quant(RMSNorm(GQA-expand(V))))        GQA prologue
    v   = relu2(BitLinear_up_gate(quant(RMSNorm(x += o))))  residual prologue, relu2 epilogue
    d   = BitLinear_down(quant(RMSNorm(v)))                 double-input prologue

The residual stream alternates between two buffers (a launch reads the one
and writes the sum to the other).  The RMSNorm sums are reduced in another
order than the glue kernel's, so the result matches the glue sequence up to
rounding edges of the norm, not bit for bit.
"""
from __future__ import annotations

import torch

from . import bitlinear as bl

HIDDEN, HEADS, KV_HEADS, HEAD_DIM, FFN = 2560, 20, 5, 128, 6912
QKV = HIDDEN + 2 * KV_HEADS * HEAD_DIM
V_COL = HIDDEN + KV_HEADS * HEAD_DIM
EPS = 1e-5
MATRICES = ("qkv", "o", "up_gate", "down")
SHAPES = {"qkv": (QKV, HIDDEN), "o": (HIDDEN, HIDDEN), "up_gate": (2 * FFN, HIDDEN),
          "down": (HIDDEN, FFN)}


class DecoderStack:
    """Packed weights of `layers` layers plus the activation buffers of M
    tokens, all resident on the GPU."""

    def __init__(self, layer_weights, layers: int, m: int, device="cuda", fused: bool = True,
                 norm: bool = False):
        """layer_weights(l) -> dict name -> [N, K] bf16/fp32 tensor on the GPU
        (quantised and packed here, then released).  norm: one token, glue as
        the products' prologue (M = 1 only)."""
        assert not norm or m == 1, "the prologue form takes one token"
        self.layers, self.m, self.fused, self.norm = layers, m, fused, norm
        self.packed, self.gamma = [], []
        for layer in range(layers):
            w = layer_weights(layer)
            p, g = {}, {}
            for name in MATRICES:
                assert tuple(w[name].shape) == SHAPES[name], (name, w[name].shape)
                p[name], g[name] = bl.quantize_weights(w[name])
            self.packed.append(p)
            self.gamma.append(g)
            del w
        f32 = dict(dtype=torch.float32, device=device)
        self.x = torch.zeros((m, HIDDEN), **f32)
        self.y = {name: torch.empty((m, SHAPES[name][0]), **f32) for name in MATRICES}
        self.xq = torch.empty((m, FFN), dtype=torch.int8, device=device)
        self.scale = torch.empty((m,), **f32)
        self.rowsum = torch.empty((m,), dtype=torch.int32, device=device)
        if norm:
            self.x_alt = torch.zeros((m, HIDDEN), **f32)
            self.v64 = torch.empty((FFN,), dtype=torch.float64, device=device)

    def packed_bytes(self) -> int:
        return sum(p.numel() for layer in self.packed for p in layer.values())

    def _q(self, k: int):
        """Quantiser outputs for an input of width k (views of one buffer)."""
        return dict(xq=self.xq.view(-1)[: self.m * k].view(self.m, k), scale=self.scale,
                    rowsum=self.rowsum)

    def _linear(self, layer: int, name: str, k: int):
        n = SHAPES[name][0]
        q = self._q(k)
        bl.forward(q["xq"], self.scale, self.rowsum, self.packed[layer][name],
                   self.gamma[layer][name], n, k, y=self.y[name])

    def _fused_layer(self, layer: int, note):
        """One layer as four product + glue calls; expects the quantised
        attention input in xq / scale / rowsum and leaves the next layer's
        there (after x += down)."""
        p, g = self.packed[layer], self.gamma[layer]
        qh, qf = self._q(HIDDEN), self._q(FFN)

        def args(q, name, n):
            return (q["xq"], q["scale"], q["rowsum"], p[name], g[name], n)

        def outs(q):
            return dict(xq_out=q["xq"], scale_out=q["scale"], rowsum_out=q["rowsum"])

        bl.forward_gqa_rmsnorm_quantize(*args(qh, "qkv", QKV), V_COL, HEADS, KV_HEADS, HEAD_DIM,
                                        EPS, **outs(qh))
        note("qkv+attn_norm")
        bl.forward_residual_rmsnorm_quantize(*args(qh, "o", HIDDEN), self.x, EPS, **outs(qh))
        note("o+norm_ffn")
        bl.forward_relu2_rmsnorm_quantize(*args(qh, "up_gate", 2 * FFN), FFN, EPS, **outs(qf))
        note("up_gate+ffn_norm")
        bl.forward_residual_rmsnorm_quantize(*args(qf, "down", HIDDEN), self.x, EPS, **outs(qh))
        note("down+norm_attn")

    def layer(self, layer: int, trace=None):
        """One decoder layer on the resident buffers.  trace: optional callback
        trace(op_name) called after every step (for tests).  Fused: the layer
        starts from the quantised attention input that the previous call left
        (step() makes the first one) and ends with the next one."""
        note = trace or (lambda op: None)
        if self.fused:
            return self._fused_layer(layer, note)
        add = self.y["down"] if layer > 0 else None
        bl.residual_rmsnorm_quantize(self.x, add, EPS, **self._q(HIDDEN))
        note("norm_attn")
        self._linear(layer, "qkv", HIDDEN)
        note("qkv")
        bl.gqa_rmsnorm_quantize(self.y["qkv"], V_COL, HEADS, KV_HEADS, HEAD_DIM, EPS,
                                **self._q(HIDDEN))
        note("attn_norm")
        self._linear(layer, "o", HIDDEN)
        note("o")
        bl.residual_rmsnorm_quantize(self.x, self.y["o"], EPS, **self._q(HIDDEN))
        note("norm_ffn")
        self._linear(layer, "up_gate", HIDDEN)
        note("up_gate")
        bl.relu2_rmsnorm_quantize(self.y["up_gate"], FFN, EPS, **self._q(FFN))
        note("ffn_norm")
        self._linear(layer, "down", FFN)
        note("down")

    def _norm_step(self):
        """One token, four launches per layer (prologue / epilogue forms)."""
        cur, alt = self.x, self.x_alt
        add = None
        for layer in range(self.layers):
            p, g = self.packed[layer], self.gamma[layer]
            if add is None:
                bl.norm_forward(cur, p["qkv"], g["qkv"], QKV, out=self.y["qkv"])
            else:
                bl.norm_forward(cur, p["qkv"], g["qkv"], QKV, add=add, x_out=alt,
                                out=self.y["qkv"])
                cur, alt = alt, cur
            bl.norm_forward(self.y["qkv"], p["o"], g["o"], HIDDEN, bl.BL_NORM_GQA, v_col=V_COL,
                            heads=HEADS, kv_heads=KV_HEADS, head_dim=HEAD_DIM, out=self.y["o"])
            bl.norm_forward(cur, p["up_gate"], g["up_gate"], 2 * FFN, add=self.y["o"], x_out=alt,
                            relu2=True, out=self.v64)
            cur, alt = alt, cur
            bl.norm_forward(self.v64, p["down"], g["down"], HIDDEN, bl.BL_NORM_F64,
                            out=self.y["down"])
            add = self.y["down"]
        # last residual addition (and the quantised RMSNorm of the output)
        bl.residual_rmsnorm_quantize(cur, add, EPS, **self._q(HIDDEN))
        if cur.data_ptr() != self.x.data_ptr():
            self.x.copy_(cur)

    def step(self):
        """All layers on the current residual stream self.x, then the last
        residual addition; self.x holds the stack's output (and xq / scale /
        rowsum its quantised RMSNorm)."""
        if self.norm:
            return self._norm_step()
        if self.fused:
            bl.residual_rmsnorm_quantize(self.x, None, EPS, **self._q(HIDDEN))
        for layer in range(self.layers):
            self.layer(layer)
        if not self.fused:
            bl.residual_rmsnorm_quantize(self.x, self.y["down"], EPS, **self._q(HIDDEN))
