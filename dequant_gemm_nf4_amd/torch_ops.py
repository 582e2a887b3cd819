"""PyTorch custom ops and modules over the C ABI: the 4-bit linear layer as
``torch.ops.bnbx.linear4bit`` and a ``Linear4bit`` module that quantizes its
weight on load; the same layer with a LoRA adapter as
``torch.ops.bnbx.linear4bit_lora`` and ``Linear4bitLoRA``.

The pomoai.com overview (module list) has ``Linear4bit`` replacing
``torch.nn.Linear`` and the mlqm.cn article (section 4) loads a model in
4 bits with a quant type (nf4 / fp4), double quantization and a compute
dtype (bf16 / fp16); its section 1 credits 4-bit inference under
``torch.compile(fullgraph=True)``.  The op is an opaque custom op with a
fake (shape-only) implementation, so it traces into a full graph; the
arithmetic runs in the library's kernels (GEMV for at most 16 rows of X,
GEMM otherwise) on the current stream.  Its backward is
``torch.ops.bnbx.linear4bit_dx`` (dX = dY . W_hat, the input gradient; the
4-bit weights are frozen, as the base layer under QLoRA in the pomoai.com
overview, and get none).  The second-level map of double quantization
follows the dtype of ``absmax``: int8 codes are the linear map, uint8 codes
the dynamic 8-bit map.  Nothing here computes.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import tensors as T

_DTYPES = (torch.bfloat16, torch.float16)


def _dq_map(absmax: torch.Tensor) -> str:
    return "dynamic" if absmax.dtype == torch.uint8 else "linear"


def _state(x: torch.Tensor, packed, absmax, absmax2, absmax_mean, out_features: int,
           quant_type: str) -> T.QuantizedWeight:
    K = x.shape[-1]
    return T.QuantizedWeight(n=out_features * K, shape=(out_features, K),
                             double_quant=absmax2 is not None, packed=packed, absmax=absmax,
                             absmax2=absmax2, absmax_mean=absmax_mean, quant_type=quant_type,
                             dtype=x.dtype, dq_map=_dq_map(absmax))


@torch.library.custom_op("bnbx::linear4bit", mutates_args=())
def linear4bit(x: torch.Tensor, packed: torch.Tensor, absmax: torch.Tensor,
               absmax2: Optional[torch.Tensor], absmax_mean: Optional[torch.Tensor],
               out_features: int, quant_type: str) -> torch.Tensor:
    """Y[..., N] = X[..., K] . W_hat[N, K]^T with W_hat the dequantized 4-bit
    weight; X, Y and W_hat in X's dtype (bf16 or fp16)."""
    if x.dtype not in _DTYPES:
        raise TypeError(f"linear4bit: x must be bfloat16 or float16, not {x.dtype}")
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    if x2.stride(-1) != 1 or x2.stride(0) % 8 != 0 or x2.data_ptr() % 16 != 0:
        x2 = x2.contiguous()
    M = x2.shape[0]
    y = torch.empty(M, out_features, dtype=x.dtype, device=x.device)
    if M > 0:
        q = _state(x, packed, absmax, absmax2, absmax_mean, out_features, quant_type)
        (T.gemv if M <= 16 else T.gemm)(x2, q, out=y)
    return y.reshape(*x.shape[:-1], out_features)


@linear4bit.register_fake
def _(x, packed, absmax, absmax2, absmax_mean, out_features, quant_type):
    return x.new_empty(*x.shape[:-1], out_features)


@torch.library.custom_op("bnbx::linear4bit_dx", mutates_args=())
def linear4bit_dx(dy: torch.Tensor, packed: torch.Tensor, absmax: torch.Tensor,
                  absmax2: Optional[torch.Tensor], absmax_mean: Optional[torch.Tensor],
                  in_features: int, quant_type: str) -> torch.Tensor:
    """dX[..., K] = dY[..., N] . W_hat[N, K] in dY's dtype (N % 64 == 0)."""
    if dy.dtype not in _DTYPES:
        raise TypeError(f"linear4bit_dx: dy must be bfloat16 or float16, not {dy.dtype}")
    N = dy.shape[-1]
    dy2 = dy.reshape(-1, N)
    if dy2.stride(-1) != 1 or dy2.stride(0) % 8 != 0 or dy2.data_ptr() % 16 != 0:
        dy2 = dy2.contiguous()
    M = dy2.shape[0]
    dx = torch.empty(M, in_features, dtype=dy.dtype, device=dy.device)
    if M > 0:
        q = T.QuantizedWeight(n=N * in_features, shape=(N, in_features),
                              double_quant=absmax2 is not None, packed=packed, absmax=absmax,
                              absmax2=absmax2, absmax_mean=absmax_mean, quant_type=quant_type,
                              dtype=dy.dtype, dq_map=_dq_map(absmax))
        T.gemm_dx(dy2, q, out=dx)
    return dx.reshape(*dy.shape[:-1], in_features)


@linear4bit_dx.register_fake
def _(dy, packed, absmax, absmax2, absmax_mean, in_features, quant_type):
    return dy.new_empty(*dy.shape[:-1], in_features)


def _setup_context(ctx, inputs, output):
    x, packed, absmax, absmax2, absmax_mean, out_features, quant_type = inputs
    ctx.save_for_backward(packed, absmax, absmax2, absmax_mean)
    ctx.in_features = x.shape[-1]
    ctx.quant_type = quant_type


def _backward(ctx, grad):
    packed, absmax, absmax2, absmax_mean = ctx.saved_tensors
    dx = None
    if ctx.needs_input_grad[0]:
        dx = torch.ops.bnbx.linear4bit_dx(grad, packed, absmax, absmax2, absmax_mean,
                                          ctx.in_features, ctx.quant_type)
    return dx, None, None, None, None, None, None


linear4bit.register_autograd(_backward, setup_context=_setup_context)


@torch.library.custom_op("bnbx::linear4bit_lora", mutates_args=())
def linear4bit_lora(x: torch.Tensor, packed: torch.Tensor, absmax: torch.Tensor,
                    absmax2: Optional[torch.Tensor], absmax_mean: Optional[torch.Tensor],
                    lora_a: torch.Tensor, lora_b: torch.Tensor, scale: float,
                    out_features: int, quant_type: str) -> torch.Tensor:
    """Y[..., N] = X . W_hat^T + rnd(s . X . A^T) . B^T: the frozen 4-bit base
    layer with a LoRA adapter (A [r, K], B [N, r], r a multiple of 16 up to
    256), as the library's down-projection followed by the GEMM with the
    low-rank term fused in (the decode GEMV forms for up to 16 rows).
    Inference only: no autograd is registered, so a backward through it
    raises."""
    if x.dtype not in _DTYPES:
        raise TypeError(f"linear4bit_lora: x must be bfloat16 or float16, not {x.dtype}")
    if lora_a.dtype != x.dtype or lora_b.dtype != x.dtype:
        raise TypeError("linear4bit_lora: the adapter must have the dtype of x")
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    if x2.stride(-1) != 1 or x2.stride(0) % 8 != 0 or x2.data_ptr() % 16 != 0:
        x2 = x2.contiguous()
    M = x2.shape[0]
    y = torch.empty(M, out_features, dtype=x.dtype, device=x.device)
    if M > 0:
        q = _state(x, packed, absmax, absmax2, absmax_mean, out_features, quant_type)
        T.linear_lora(x2, q, lora_a.contiguous(), lora_b.contiguous(), scale, out=y)
    return y.reshape(*x.shape[:-1], out_features)


@linear4bit_lora.register_fake
def _(x, packed, absmax, absmax2, absmax_mean, lora_a, lora_b, scale, out_features, quant_type):
    return x.new_empty(*x.shape[:-1], out_features)


class Linear4bit(torch.nn.Module):
    """A bias-free ``nn.Linear(in_features, out_features)`` whose weight is
    held as 4-bit codes (NF4 or FP4, blocks of 64, optional double quant
    with the linear or the dynamic second-level map) and whose forward runs
    ``torch.ops.bnbx.linear4bit`` in ``compute_dtype``.
    ``load_weight`` quantizes a bf16 [out, in] weight on the device.  The
    input gradient (backward) needs out_features % 64 == 0."""

    def __init__(self, in_features: int, out_features: int, quant_type: str = "nf4",
                 double_quant: bool = True, compute_dtype: torch.dtype = torch.bfloat16,
                 device="cuda", dq_map: str = "linear"):
        super().__init__()
        if quant_type not in T.QUANT_TYPES:
            raise ValueError(f"quant_type must be one of {sorted(T.QUANT_TYPES)}")
        if dq_map not in T.DQ_MAPS:
            raise ValueError(f"dq_map must be one of {sorted(T.DQ_MAPS)}")
        if compute_dtype not in _DTYPES:
            raise ValueError("compute_dtype must be torch.bfloat16 or torch.float16")
        if in_features % 64 != 0:
            raise ValueError("in_features must be a multiple of 64 (one block per row step)")
        self.in_features, self.out_features = in_features, out_features
        self.quant_type, self.double_quant, self.compute_dtype = quant_type, double_quant, \
            compute_dtype
        self.dq_map = dq_map if double_quant else "linear"
        q = T.empty_quantized((out_features, in_features), double_quant, device, quant_type,
                              compute_dtype, self.dq_map)
        self.register_buffer("packed", q.packed)
        self.register_buffer("absmax", q.absmax)
        self.register_buffer("absmax2", q.absmax2)
        self.register_buffer("absmax_mean", q.absmax_mean)

    def quantized(self) -> T.QuantizedWeight:
        return T.QuantizedWeight(self.in_features * self.out_features,
                                 (self.out_features, self.in_features), self.double_quant,
                                 self.packed, self.absmax, self.absmax2, self.absmax_mean,
                                 self.quant_type, self.compute_dtype, self.dq_map)

    @torch.no_grad()
    def load_weight(self, w: torch.Tensor) -> "Linear4bit":
        """Quantize-on-load of a bf16 weight [out_features, in_features]."""
        if tuple(w.shape) != (self.out_features, self.in_features):
            raise ValueError(f"weight shape {tuple(w.shape)} != "
                             f"{(self.out_features, self.in_features)}")
        w = w.to(device=self.packed.device, dtype=torch.bfloat16).contiguous()
        T.quantize(w, self.double_quant, out=self.quantized())
        return self

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, **kw) -> "Linear4bit":
        if linear.bias is not None:
            raise ValueError("Linear4bit has no bias")
        m = cls(linear.in_features, linear.out_features, device=linear.weight.device, **kw)
        return m.load_weight(linear.weight)

    def dequantize(self) -> torch.Tensor:
        return T.dequantize(self.quantized())

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dtype != self.compute_dtype:
            raise TypeError(f"input dtype {x.dtype} != compute dtype {self.compute_dtype}")
        return torch.ops.bnbx.linear4bit(x, self.packed, self.absmax, self.absmax2,
                                         self.absmax_mean, self.out_features, self.quant_type)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"quant_type={self.quant_type}, double_quant={self.double_quant}, "
                f"dq_map={self.dq_map}, "
                f"compute_dtype={self.compute_dtype}")


class Linear4bitLoRA(Linear4bit):
    """``Linear4bit`` with a LoRA adapter beside the frozen 4-bit weight (the
    pomoai.com overview, QLoRA): Y = X . W_hat^T + s . (X . A^T) . B^T with
    A [rank, in_features], B [out_features, rank] in ``compute_dtype`` and
    s = ``scale``; forward runs ``torch.ops.bnbx.linear4bit_lora``.  The
    adapter starts at zero (the layer then equals ``Linear4bit``) and is set
    with ``load_adapter``; training it is not supported here."""

    def __init__(self, in_features: int, out_features: int, rank: int = 16,
                 scale: float = 1.0, **kw):
        super().__init__(in_features, out_features, **kw)
        if rank < 16 or rank > 256 or rank % 16 != 0:
            raise ValueError("rank must be a multiple of 16 between 16 and 256")
        self.rank, self.scale = rank, float(scale)
        dev = self.packed.device
        self.register_buffer("lora_a", torch.zeros(rank, in_features, dtype=self.compute_dtype,
                                                   device=dev))
        self.register_buffer("lora_b", torch.zeros(out_features, rank, dtype=self.compute_dtype,
                                                   device=dev))

    @torch.no_grad()
    def load_adapter(self, a: torch.Tensor, b: torch.Tensor,
                     scale: Optional[float] = None) -> "Linear4bitLoRA":
        if tuple(a.shape) != tuple(self.lora_a.shape) or tuple(b.shape) != tuple(self.lora_b.shape):
            raise ValueError(f"adapter shapes {tuple(a.shape)}, {tuple(b.shape)} != "
                             f"{tuple(self.lora_a.shape)}, {tuple(self.lora_b.shape)}")
        self.lora_a.copy_(a)
        self.lora_b.copy_(b)
        if scale is not None:
            self.scale = float(scale)
        return self

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dtype != self.compute_dtype:
            raise TypeError(f"input dtype {x.dtype} != compute dtype {self.compute_dtype}")
        return torch.ops.bnbx.linear4bit_lora(x, self.packed, self.absmax, self.absmax2,
                                              self.absmax_mean, self.lora_a, self.lora_b,
                                              self.scale, self.out_features, self.quant_type)

    def extra_repr(self) -> str:
        return super().extra_repr() + f", rank={self.rank}, scale={self.scale}"
