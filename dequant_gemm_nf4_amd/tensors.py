"""Torch-tensor convenience layer over the C ABI: allocates device buffers
with PyTorch (plumbing only) and calls the bnbx_* entry points.  Nothing is
computed here."""

from __future__ import annotations

import dataclasses

import torch

from . import (Nf4State, bnbx_dequantize_nf4, bnbx_gemm_nf4, bnbx_gemm_nf4_dx, bnbx_gemm_nf4_lora,
               bnbx_gemm_nf4_workspace_bytes, bnbx_gemv_nf4, bnbx_gemv_nf4_grouped, bnbx_lora_down,
               bnbx_quantize_nf4, bnbx_quantize_nf4_grouped,
               bnbx_quantize_nf4_grouped_workspace_bytes, bnbx_quantize_nf4_workspace_bytes)

BLOCKSIZE = 64
GROUP = 256
QUANT_TYPES = {"nf4": 0, "fp4": 1}
# second-level maps of the block scales (bnbx_nf4_state.double_quant)
DQ_MAPS = {"linear": 1, "dynamic": 2}
DTYPES = {torch.bfloat16: 0, torch.float16: 1}


@dataclasses.dataclass
class QuantizedWeight:
    """Device buffers of one 4-bit tensor plus its C descriptor.  ``dtype``
    is the compute dtype (bf16 or fp16) of its dequantized values and of the
    activations it multiplies; ``dq_map`` the second-level map of the block
    scales with double quant ("linear": int8 codes, "dynamic": uint8 codes
    into the dynamic 8-bit map)."""

    n: int
    shape: tuple
    double_quant: bool
    packed: torch.Tensor          # uint8 [n/2]
    absmax: torch.Tensor          # float32 [nb] or int8 [nb]
    absmax2: torch.Tensor | None  # float32 [ng]
    absmax_mean: torch.Tensor | None  # float32 [1]
    quant_type: str = "nf4"
    dtype: torch.dtype = torch.bfloat16
    dq_map: str = "linear"

    @property
    def state(self) -> Nf4State:
        return Nf4State(
            n=self.n, blocksize=BLOCKSIZE,
            double_quant=DQ_MAPS[self.dq_map] if self.double_quant else 0,
            quant_type=QUANT_TYPES[self.quant_type], compute_dtype=DTYPES[self.dtype],
            absmax=self.absmax.data_ptr(),
            absmax2=self.absmax2.data_ptr() if self.absmax2 is not None else None,
            absmax_mean=self.absmax_mean.data_ptr() if self.absmax_mean is not None else None)


def empty_quantized(shape, double_quant: bool, device="cuda", quant_type: str = "nf4",
                    dtype: torch.dtype = torch.bfloat16, dq_map: str = "linear") -> QuantizedWeight:
    n = 1
    for s in shape:
        n *= int(s)
    nb = -(-n // BLOCKSIZE)
    ng = -(-nb // GROUP)
    packed = torch.empty(n // 2, dtype=torch.uint8, device=device)
    if double_quant:
        absmax = torch.empty(nb, dtype=torch.uint8 if dq_map == "dynamic" else torch.int8,
                             device=device)
        absmax2 = torch.empty(ng, dtype=torch.float32, device=device)
        mean = torch.empty(1, dtype=torch.float32, device=device)
    else:
        absmax = torch.empty(nb, dtype=torch.float32, device=device)
        absmax2 = mean = None
    if dq_map not in DQ_MAPS:
        raise ValueError(f"unknown second-level map {dq_map!r}")
    return QuantizedWeight(n, tuple(shape), double_quant, packed, absmax, absmax2, mean,
                           quant_type, dtype, dq_map)


def workspace_for(n: int, double_quant: bool, device="cuda") -> torch.Tensor | None:
    nbytes = bnbx_quantize_nf4_workspace_bytes(n, BLOCKSIZE, int(double_quant))
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def quantize(w: torch.Tensor, double_quant: bool, out: QuantizedWeight | None = None,
             workspace: torch.Tensor | None = None, stream=None, quant_type: str = "nf4",
             dtype: torch.dtype = torch.bfloat16, dq_map: str = "linear") -> QuantizedWeight:
    """bnbx_quantize_nf4 on a bf16 tensor (any shape, contiguous); ``dtype``
    is the compute dtype recorded for later dequantize / matmul calls,
    ``dq_map`` the second-level map with double quant (ignored with ``out``,
    which carries its own)."""
    assert w.dtype == torch.bfloat16 and w.is_contiguous()
    q = out if out is not None else empty_quantized(w.shape, double_quant, w.device, quant_type,
                                                    dtype, dq_map)
    ws = workspace if workspace is not None else workspace_for(q.n, double_quant, w.device)
    bnbx_quantize_nf4(w, q.packed, q.state, ws, 0 if ws is None else ws.numel(), stream)
    return q


def grouped_workspace_for(ns, double_quant: bool, device="cuda") -> torch.Tensor | None:
    nbytes = bnbx_quantize_nf4_grouped_workspace_bytes(ns, BLOCKSIZE, int(double_quant))
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def quantize_grouped(ws: list, double_quant: bool, outs: list | None = None,
                     workspace: torch.Tensor | None = None, stream=None, quant_type: str = "nf4",
                     dtype: torch.dtype = torch.bfloat16,
                     dq_map: str = "linear") -> list:
    """bnbx_quantize_nf4_grouped on up to eight bf16 tensors (a layer's
    weights) in one call; each result equals quantize() on that tensor."""
    assert all(w.dtype == torch.bfloat16 and w.is_contiguous() for w in ws)
    qs = outs if outs is not None else [
        empty_quantized(w.shape, double_quant, w.device, quant_type, dtype, dq_map) for w in ws]
    wsp = workspace if workspace is not None else grouped_workspace_for(
        [q.n for q in qs], double_quant, ws[0].device)
    bnbx_quantize_nf4_grouped([(w, q.packed, q.state) for w, q in zip(ws, qs)], wsp,
                              0 if wsp is None else wsp.numel(), stream)
    return qs


def dequantize(q: QuantizedWeight, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    o = out if out is not None else torch.empty(q.shape, dtype=q.dtype, device=q.packed.device)
    assert o.dtype == q.dtype
    bnbx_dequantize_nf4(q.packed, q.state, o, stream)
    return o


def gemv(x: torch.Tensor, q: QuantizedWeight, out: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """Y = X . W_hat^T for X [M, K] (M <= 16), W [N, K]."""
    M, K = x.shape
    N = q.shape[0]
    assert x.dtype == q.dtype
    y = out if out is not None else torch.empty(M, N, dtype=q.dtype, device=x.device)
    bnbx_gemv_nf4(x, x.stride(0), q.packed, q.state, M, N, K, y, y.stride(0), stream)
    return y


def gemv_grouped(x: torch.Tensor, qs: list, outs: list | None = None, stream=None) -> list:
    """Y_i = X . W_hat_i^T for up to four weights sharing X [M, K] (M <= 16),
    in one call (bnbx_gemv_nf4_grouped)."""
    M, K = x.shape
    ys = outs if outs is not None else [
        torch.empty(M, q.shape[0], dtype=q.dtype, device=x.device) for q in qs]
    for q in qs:
        assert x.dtype == q.dtype and q.shape[1] == K
    bnbx_gemv_nf4_grouped(x, x.stride(0),
                          [(q.packed, q.state, q.shape[0], y, y.stride(0)) for q, y in zip(qs, ys)],
                          M, K, stream)
    return ys


def gemm(x: torch.Tensor, q: QuantizedWeight, out: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """Y = X . W_hat^T for X [M, K], W [N, K], any M."""
    M, K = x.shape
    N = q.shape[0]
    assert x.dtype == q.dtype
    y = out if out is not None else torch.empty(M, N, dtype=q.dtype, device=x.device)
    nbytes = bnbx_gemm_nf4_workspace_bytes(M, N, K)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if nbytes else None
    bnbx_gemm_nf4(x, x.stride(0), q.packed, q.state, M, N, K, y, y.stride(0), ws, nbytes, stream)
    return y


def gemm_dx(dy: torch.Tensor, q: QuantizedWeight, out: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    """dX = dY . W_hat for dY [M, N], W [N, K] (the input gradient of gemm)."""
    M, N = dy.shape
    K = q.shape[1]
    assert dy.dtype == q.dtype and N == q.shape[0]
    dx = out if out is not None else torch.empty(M, K, dtype=q.dtype, device=dy.device)
    bnbx_gemm_nf4_dx(dy, dy.stride(0), q.packed, q.state, M, N, K, dx, dx.stride(0), stream)
    return dx


def gemm_lora(x: torch.Tensor, q: QuantizedWeight, xa: torch.Tensor, lora_b: torch.Tensor,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X . W_hat^T + XA . B^T for X [M, K], XA [M, r] (= s X A^T), B [N, r]."""
    M, K = x.shape
    N = q.shape[0]
    r = xa.shape[1]
    assert x.dtype == q.dtype == xa.dtype == lora_b.dtype and lora_b.shape == (N, r)
    y = out if out is not None else torch.empty(M, N, dtype=q.dtype, device=x.device)
    bnbx_gemm_nf4_lora(x, x.stride(0), q.packed, q.state, M, N, K, xa, xa.stride(0), lora_b,
                       lora_b.stride(0), r, y, y.stride(0), stream)
    return y


def lora_down(x: torch.Tensor, lora_a: torch.Tensor, scale: float,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """XA = s . X . A^T for X [M, K] and the adapter weight A [r, K]."""
    M, K = x.shape
    r = lora_a.shape[0]
    assert x.dtype == lora_a.dtype and lora_a.shape[1] == K
    xa = out if out is not None else torch.empty(M, r, dtype=x.dtype, device=x.device)
    bnbx_lora_down(x, x.stride(0), lora_a, lora_a.stride(0), M, K, r, scale, DTYPES[x.dtype], xa,
                   xa.stride(0), stream)
    return xa


def linear_lora(x: torch.Tensor, q: QuantizedWeight, lora_a: torch.Tensor, lora_b: torch.Tensor,
                scale: float, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X . W_hat^T + s . (X . A^T) . B^T: the down-projection, then the GEMM
    with the low-rank term fused in (both in the library)."""
    xa = lora_down(x, lora_a, scale, stream=stream)
    return gemm_lora(x, q, xa, lora_b, out=out, stream=stream)

