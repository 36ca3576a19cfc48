"""The BitLinear sub-graph of one transformer layer as a chain of library calls.

Attention itself (RoPE, the softmax, the KV cache) is not part of this library: the layer
takes the attention output as an input.  Everything else between the layer's input x and its
output runs in the library's kernels (BitDistill article, "Stage 1": SubLN before the
attention output projection and before the FFN output projection; SLM750-Edge card: RMSNorm
with epsilon 1e-6 and a ReLU^2 FFN with gate, up and down matrices; the Distillix and
Qwen3-shaped layer sets use SwiGLU):

  A1  codes of x with the input RMSNorm (g_attn)       } one activation call
      codes of the attention output with SubLN (g_o)    }
  P1  q, k, v from x's codes; o from the attention codes, plus the residual x -> x1
                                                          (one product call)
  A2  codes of x1 with the FFN RMSNorm (g_ffn)
  P2  gate and up (or up alone) from those codes
  A3  codes of act(gate, up) with SubLN (g_down): the FFN activation in front of the
      quantization (SwiGLU, gated ReLU^2, or ReLU^2 of up)
  P3  down from those codes, plus the residual x1 -> out

Six launches per layer, no host synchronization; the call sequence can be captured into a
HIP graph.  Argument marshalling only: the tables of device pointers are built once per
(weights, buffers) pair and each call hands them to the C entry points.

At decode sizes (every input of the layer fits the fused form: M <= 4 tokens and M * K
within the LDS budget) the same sub-graph takes three launches of the fused layer call, each
product quantizing its own input rows:

  L1  q, k, v from x (input RMSNorm); o from the attention output (SubLN) + residual -> x1
  L2  gate and up from x1 (FFN RMSNorm) as one gated pair: h = act(gate, up) in the epilogue
      (ReLU^2 of up alone for the ungated kind)
  L3  down from h (SubLN) + residual x1 -> out

Every intermediate value is the one the six-launch form computes (the same codes, scales,
fp32 products and activation), so the two forms agree element for element up to the fixed
order of the norms' sums of squares.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

from . import (ACT_NONE, ACT_RELU2, ACT_RELU2_GLU, ACT_SWIGLU, DECODE_MAX_M, _check, _stream,
               act_ex_table, forward_ex_table, lib, linear_ex_table, linear_fused, pack_quad_rows)

ATTN_IN = ("q", "k", "v", "qkv")


@dataclass
class LayerWeights:
    """Packed ternary weights (int32 storage of uint32 words, [N, K/16]) and gamma ([1] fp32)
    per projection, and the four norm weights ([K] fp32, or None for g = 1 omitted)."""
    packed: Dict[str, torch.Tensor]
    gamma: Dict[str, torch.Tensor]
    norms: Dict[str, Optional[torch.Tensor]] = field(default_factory=dict)
    act: int = ACT_SWIGLU
    _quad: Dict[str, torch.Tensor] = field(default_factory=dict, repr=False)

    def quad_rows(self, name: str) -> torch.Tensor:
        """The projection's words in the quad-row layout (packed once, on first use)."""
        if name not in self._quad:
            self._quad[name] = pack_quad_rows(self.packed[name])
        return self._quad[name]

    def fits_quad_rows(self) -> bool:
        """Whether every projection fits the quad-row layout (N % 4 == 0, K % 128 == 0)."""
        return all(self.N(n) % 4 == 0 and self.K(n) % 128 == 0 for n in self.packed)

    def K(self, name: str) -> int:
        return self.packed[name].shape[1] * 16

    def N(self, name: str) -> int:
        return self.packed[name].shape[0]

    @property
    def attn_in(self) -> List[str]:
        return [n for n in ATTN_IN if n in self.packed]

    @property
    def hidden(self) -> int:
        return self.N("down")


class LayerChain:
    """Buffers and call tables for one layer at M tokens."""

    def __init__(self, w: LayerWeights, M: int, eps: float = 1e-6, device: str = "cuda",
                 like: Optional["LayerChain"] = None, fused: Optional[bool] = None,
                 keep_codes: bool = False):
        """`like`: another chain of the same shapes whose buffers this one shares (layers run
        one after another, so a stack of layers needs one set of activation buffers).
        `fused`: the three-launch decode form (default: whenever every input fits it).
        `keep_codes`: in the fused form, also write the codes and scales each product used
        (xq/xs, aq/as_, fq/fs, hq/hs; the six-launch form always has them)."""
        if "o" not in w.packed or "up" not in w.packed or "down" not in w.packed:
            raise ValueError("a layer needs o, up and down projections")
        glu = w.act in (ACT_SWIGLU, ACT_RELU2_GLU)
        if glu != ("gate" in w.packed):
            raise ValueError("gated activations need a gate projection, ReLU^2 of up none")
        d = w.hidden
        if w.N("o") != d or w.K("down") != w.N("up") or any(w.K(n) != d for n in w.attn_in) \
                or w.K("up") != d or (glu and (w.K("gate") != d or w.N("gate") != w.N("up"))):
            raise ValueError("inconsistent layer shapes")
        self.w, self.M, self.eps = w, M, eps
        fits = all(linear_fused(M, k) for k in (d, w.K("o"), w.K("down")))
        self.fused = fits if fused is None else fused
        if self.fused and not fits:
            raise ValueError("the fused form needs M <= 4 and M * K within its LDS budget")
        f32, i8 = torch.float32, torch.int8
        pool = {} if like is None else like._pool
        self._pool = pool
        counter = iter(range(1 << 30))

        def t(*shape, dt=f32):
            key = (next(counter), shape, dt)
            if key not in pool:
                pool[key] = torch.empty(shape, dtype=dt, device=device)
            return pool[key]

        self.x = t(M, d)                       # layer input (caller fills)
        self.attn = t(M, w.K("o"))             # attention output (caller fills)
        self.xq, self.xs = t(M, d, dt=i8), t(M)
        self.aq, self.as_ = t(M, w.K("o"), dt=i8), t(M)
        self.y = {n: t(M, w.N(n)) for n in w.attn_in}
        self.x1 = t(M, d)
        self.fq, self.fs = t(M, d, dt=i8), t(M)
        if self.fused:
            self.gate = self.up = None
            self.h = t(M, w.N("up"))           # FFN hidden state act(gate, up)
        else:
            self.gate = t(M, w.N("gate")) if glu else None
            self.up = t(M, w.N("up"))
            self.h = None
        self.hq, self.hs = t(M, w.K("down"), dt=i8), t(M)
        self.out = t(M, d)
        nrm = w.norms.get
        L = lib()
        self.quad = False
        if self.fused:
            self._build_fused(nrm, glu, keep_codes, L)
            return
        self._a1 = [dict(X=self.x, X_q=self.xq, x_scale=self.xs, norm_weight=nrm("attn"), eps=eps),
                    dict(X=self.attn, X_q=self.aq, x_scale=self.as_, norm_weight=nrm("o"), eps=eps)]
        if not w.attn_in:
            self._a1 = self._a1[1:]
        # Prefill-sized products read the quad-row layout where every projection fits it (whole
        # 128-byte lines per weight load; the same results as on rows).
        self.quad = M > DECODE_MAX_M and w.fits_quad_rows()
        W = w.quad_rows if self.quad else w.packed.__getitem__
        fwd = L.bitlinear_forward_ex_quad_rows_grouped if self.quad else L.bitlinear_forward_ex_grouped
        p1 = [dict(X_q=self.xq, x_scale=self.xs, W_packed=W(n), gamma=w.gamma[n], Y=self.y[n])
              for n in w.attn_in]
        p1.append(dict(X_q=self.aq, x_scale=self.as_, W_packed=W("o"), gamma=w.gamma["o"],
                       Y=self.x1, residual=self.x))
        a2 = [dict(X=self.x1, X_q=self.fq, x_scale=self.fs, norm_weight=nrm("ffn"), eps=eps)]
        p2 = [dict(X_q=self.fq, x_scale=self.fs, W_packed=W("up"), gamma=w.gamma["up"], Y=self.up)]
        if glu:
            p2.insert(0, dict(X_q=self.fq, x_scale=self.fs, W_packed=W("gate"),
                              gamma=w.gamma["gate"], Y=self.gate))
        a3 = [dict(X=self.gate if glu else self.up, X2=self.up if glu else None, act=w.act,
                   X_q=self.hq, x_scale=self.hs, norm_weight=nrm("down"), eps=eps)]
        p3 = [dict(X_q=self.hq, x_scale=self.hs, W_packed=W("down"), gamma=w.gamma["down"],
                   Y=self.out, residual=self.x1)]
        self._calls = [
            (L.bitlinear_quantize_acts_ex_grouped, act_ex_table(self._a1), len(self._a1)),
            (fwd, forward_ex_table(p1), len(p1)),
            (L.bitlinear_quantize_acts_ex_grouped, act_ex_table(a2), 1),
            (fwd, forward_ex_table(p2), len(p2)),
            (L.bitlinear_quantize_acts_ex_grouped, act_ex_table(a3), 1),
            (fwd, forward_ex_table(p3), 1),
        ]
        self._addr = [ctypes.addressof(arr) for _, arr, _ in self._calls]

    def _build_fused(self, nrm, glu, keep, L):
        w, eps = self.w, self.eps

        def codes(q, s):
            return dict(X_q=q, x_scale=s) if keep else {}

        l1 = [dict(X=self.x, norm_weight=nrm("attn"), eps=eps, W_packed=w.packed[n], gamma=w.gamma[n],
                   Y=self.y[n], **(codes(self.xq, self.xs) if i == 0 else {}))
              for i, n in enumerate(w.attn_in)]
        l1.append(dict(X=self.attn, norm_weight=nrm("o"), eps=eps, W_packed=w.packed["o"],
                       gamma=w.gamma["o"], Y=self.x1, residual=self.x, **codes(self.aq, self.as_)))
        if glu:
            l2 = [dict(X=self.x1, norm_weight=nrm("ffn"), eps=eps, W_packed=w.packed["gate"],
                       gamma=w.gamma["gate"], W2_packed=w.packed["up"], gamma2=w.gamma["up"],
                       act=w.act, Y=self.h, **codes(self.fq, self.fs))]
        else:
            l2 = [dict(X=self.x1, norm_weight=nrm("ffn"), eps=eps, W_packed=w.packed["up"],
                       gamma=w.gamma["up"], act=w.act, Y=self.h, **codes(self.fq, self.fs))]
        l3 = [dict(X=self.h, norm_weight=nrm("down"), eps=eps, W_packed=w.packed["down"],
                   gamma=w.gamma["down"], Y=self.out, residual=self.x1, **codes(self.hq, self.hs))]
        self._calls = [(L.bitlinear_linear_ex_grouped, linear_ex_table(c), len(c)) for c in (l1, l2, l3)]
        self._addr = [ctypes.addressof(arr) for _, arr, _ in self._calls]

    def __call__(self, stream=None) -> torch.Tensor:
        """Run the chain on self.x / self.attn; returns self.out (written in place)."""
        st = _stream(stream)
        for (fn, _, n), a in zip(self._calls, self._addr):
            _check(fn.__name__, fn(a, n, st))
        return self.out

    def ops(self) -> int:
        """Integer operations of the layer's products (2 M N K summed)."""
        w = self.w
        names = w.attn_in + ["o", "up", "down"] + (["gate"] if "gate" in w.packed else [])
        return sum(2 * self.M * w.N(n) * w.K(n) for n in names)

    def weight_bytes(self) -> int:
        w = self.w
        return sum(p.numel() * 4 for p in w.packed.values())


def activation_name(act: int) -> str:
    return {ACT_NONE: "none", ACT_SWIGLU: "swiglu", ACT_RELU2_GLU: "relu2_glu",
            ACT_RELU2: "relu2"}[act]
