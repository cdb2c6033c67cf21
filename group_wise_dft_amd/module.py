"""torch drop-in for a naive EQ-Linear layer, running on libeqlinear.so.

``EQLinear(in_features, out_features, group_order=T)`` holds the weight
Wt [D_T, C_T, T] and applies the equivariant linear layer to the last axis of
its input (flat channel index c*T + g, group axis contiguous), i.e. the
block-circulant matrix of the pages' §3.1 eq. (1) in the convolution reading
([pchao] §3.1 eq. (3)).  It caches the frequency-domain weight planes
([paperpeel] App. A.3 "weight caching") and recomputes them when the weight
changes: a new tensor, new storage, or an in-place update (torch's version
counter).

The autograd function calls the C ABI only, on the current stream: forward
-> eqlinear_forward (with the group-shared bias of [pchao] §3.2.1 eq. (7)
when the layer has one), backward -> eqlinear_backward_weight,
eqlinear_backward_input and eqlinear_backward_bias, each only when its
gradient is needed (the eqlinear_octic_* calls for the octic group; its bias
gradient is the same group sum).  (Running the weight gradient on a second
stream beside the input gradient was measured slower at ViT-B FFN size on
MI355X: the two kernels contend for the same LDS and L2.)
"""
from __future__ import annotations

import math

import torch

from . import eqlinear as E


class _Spectrum:
    """Weight-plane cache keyed on the weight tensor's identity and version.

    When the key changes the planes go to a newly allocated buffer: an
    autograd graph recorded before the change keeps the spectrum of the
    weight it saw (its backward reads it), so that buffer is never
    overwritten."""

    def __init__(self, octic: bool = False):
        self.key = None
        self.spec = None
        self.octic = octic

    def get(self, w: torch.Tensor) -> E.WeightSpectrum:
        key = (w.data_ptr(), w._version, tuple(w.shape), w.dtype, w.device)
        if self.key != key or self.spec is None:
            D_T, C_T, T = w.shape
            if self.octic:
                spec = E.new_octic_weight_spectrum(C_T, D_T, w.dtype, w.device)
                E.eqlinear_octic_weight_spectrum(w.detach().contiguous(), spec)
            else:
                spec = E.new_weight_spectrum(C_T, D_T, T, w.dtype, w.device)
                E.eqlinear_weight_spectrum(w.detach().contiguous(), spec)
            self.spec, self.key = spec, key
        return self.spec


class EQLinearFunction(torch.autograd.Function):
    """y = EQ-Linear(x; Wt) on [N, C_T, T] -> [N, D_T, T] (optionally + bias)."""

    @staticmethod
    def forward(ctx, x, w, bias, spec):
        if spec.octic:
            y = E.eqlinear_octic_forward(x, spec, bias=bias)
        else:
            y = E.eqlinear_forward(x, spec, bias=bias)
        ctx.save_for_backward(x, w)
        ctx.spec = spec
        ctx.has_bias = bias is not None
        return y

    @staticmethod
    def backward(ctx, dy):
        x, _ = ctx.saved_tensors
        dy = dy.contiguous()
        dx = dw = db = None
        # cyclic: the weight gradient first -- it reads dY while it is cold
        # and leaves it in the Infinity Cache for the input gradient, which
        # loses more to a cold read; the octic layer measured faster the
        # other way round
        if ctx.spec.octic:
            if ctx.needs_input_grad[0]:
                dx = E.eqlinear_octic_backward_input(dy, ctx.spec)
            if ctx.needs_input_grad[1]:
                dw = E.eqlinear_octic_backward_weight(x, dy)
        else:
            if ctx.needs_input_grad[1]:
                dw = E.eqlinear_backward_weight(x, dy)
            if ctx.needs_input_grad[0]:
                dx = E.eqlinear_backward_input(dy, ctx.spec)
        if ctx.has_bias and ctx.needs_input_grad[2]:
            db = E.eqlinear_backward_bias(dy)
        return dx, dw, db, None


class EQLinear(torch.nn.Module):
    """Equivariant linear layer over the cyclic group of order T, or with
    group="octic" over the octic group D8 (quarter turns and reflections,
    T = 8 components per tuple, element a + 4 b = r^a s^b; the regular-
    representation layer Y[g] = sum_h Wt[h^-1 g] X[h] of the library's octic
    entry points).

    Input [..., in_features] with the group axis innermost (channel index
    c*T + g), output [..., out_features].  The layer works on C_T =
    ceil(in_features / T) input and D_T = ceil(out_features / T) output
    channel tuples.  When T does not divide a feature count, the pages'
    channel padding applies ([paperpeel] §3 "Formulation setup": an
    indivisible width is padded with zero channels): the input is extended
    with zero channels to C_T * T features, and the layer's last
    D_T * T - out_features outputs are dropped (their gradients are zero).
    The layer is equivariant on whole tuples.  Weight init:
    N(0, 1/in_features) (unit-variance outputs for unit-variance inputs).
    """

    def __init__(self, in_features: int, out_features: int, group_order: int | None = None,
                 bias: bool = False, device=None, dtype=None, group: str = "cyclic"):
        super().__init__()
        if group not in ("cyclic", "octic"):
            raise ValueError("group must be 'cyclic' or 'octic'")
        if group == "octic":
            if group_order not in (None, 8):
                raise ValueError("the octic group has order 8")
            T = 8
        else:
            T = 4 if group_order is None else int(group_order)
        if in_features < 1 or out_features < 1 or T < 2:
            raise ValueError("feature counts must be >= 1 and the group order >= 2")
        self.T = T
        self.group = group
        self.C_T, self.D_T = -(-in_features // T), -(-out_features // T)
        self.in_features, self.out_features = in_features, out_features
        w = torch.empty((self.D_T, self.C_T, T), device=device, dtype=dtype)
        self.weight = torch.nn.Parameter(w)
        self.bias = torch.nn.Parameter(torch.empty(self.D_T, device=device, dtype=dtype)) if bias else None
        self._cache = _Spectrum(octic=group == "octic")
        self.reset_parameters()

    def reset_parameters(self):
        with torch.no_grad():
            self.weight.normal_(0.0, 1.0 / math.sqrt(self.in_features))
            if self.bias is not None:
                self.bias.zero_()

    def spectrum(self) -> E.WeightSpectrum:
        return self._cache.get(self.weight)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError("last axis must be in_features=%d" % self.in_features)
        lead = x.shape[:-1]
        pad_in = self.C_T * self.T - self.in_features
        if pad_in:
            x = torch.nn.functional.pad(x, (0, pad_in))
        x3 = x.reshape(-1, self.C_T, self.T).contiguous()
        y = EQLinearFunction.apply(x3, self.weight, self.bias, self.spectrum())
        y = y.reshape(*lead, self.D_T * self.T)
        if self.D_T * self.T != self.out_features:
            y = y[..., : self.out_features]
        return y

    def extra_repr(self) -> str:
        return "in_features=%d, out_features=%d, group=%s, group_order=%d, bias=%s" % (
            self.in_features, self.out_features, self.group, self.T, self.bias is not None)
