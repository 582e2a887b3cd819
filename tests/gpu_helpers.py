"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its C ABI (dequant_gemm_nf4_amd), bring results back as
NumPy arrays in the oracle's formats."""

from __future__ import annotations

import numpy as np
import torch

from dequant_gemm_nf4_amd import tensors as T


TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16}


def dev_bf16(bits: np.ndarray, shape=None, dtype: str = "bf16") -> torch.Tensor:
    """16-bit patterns (bf16, or binary16 with dtype="f16") to a device tensor."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    t = torch.from_numpy(a.view(np.int16).copy()).view(TORCH_DTYPE[dtype])
    if shape is not None:
        t = t.reshape(shape)
    return t.cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def gpu_quantize(w_bits: np.ndarray, shape, dq: bool, quant_type: str = "nf4",
                 dtype: str = "bf16", dq_map: str = "linear") -> dict:
    w = dev_bf16(w_bits, shape)
    q = T.quantize(w, dq, quant_type=quant_type, dtype=TORCH_DTYPE[dtype], dq_map=dq_map)
    torch.cuda.synchronize()
    out = {"packed": q.packed.cpu().numpy(), "double_quant": dq, "n": q.n, "blocksize": 64}
    if dq:
        out["dq_map"] = dq_map
    if dq:
        out["absmax"] = q.absmax.cpu().numpy()
        out["absmax2"] = q.absmax2.cpu().numpy()
        out["absmax_mean"] = np.float32(q.absmax_mean.cpu().numpy()[0])
    else:
        out["absmax"] = q.absmax.cpu().numpy()
    out["_device"] = q
    return out


def upload_state(ostate: dict, shape, dtype: str = "bf16") -> T.QuantizedWeight:
    """Device copy of a quant state the oracle produced (its quant type; the
    given compute dtype)."""
    dq = ostate["double_quant"]
    dq_map = ostate.get("dq_map", "linear") if dq else "linear"
    q = T.empty_quantized(shape, dq, quant_type=ostate.get("quant_type", "nf4"),
                          dtype=TORCH_DTYPE[dtype], dq_map=dq_map)
    q.packed.copy_(torch.from_numpy(np.ascontiguousarray(ostate["packed"])))
    if dq:
        code_type = np.uint8 if dq_map == "dynamic" else np.int8
        q.absmax.copy_(torch.from_numpy(np.ascontiguousarray(ostate["absmax"], code_type)))
        q.absmax2.copy_(torch.from_numpy(np.ascontiguousarray(ostate["absmax2"], np.float32)))
        q.absmax_mean.copy_(torch.tensor([float(ostate["absmax_mean"])], dtype=torch.float32))
    else:
        q.absmax.copy_(torch.from_numpy(np.ascontiguousarray(ostate["absmax"], np.float32)))
    return q


def same_f32_bits(a, b) -> bool:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


def assert_state_equal(gpu: dict, ref: dict) -> None:
    assert np.array_equal(gpu["packed"], ref["packed"]), \
        f"packed differs at {np.flatnonzero(gpu['packed'] != ref['packed'])[:10]}"
    if ref["double_quant"]:
        assert np.array_equal(gpu["absmax"], ref["absmax"]), \
            f"q differs at {np.flatnonzero(gpu['absmax'] != ref['absmax'])[:10]}"
        assert same_f32_bits(gpu["absmax2"], ref["absmax2"])
        assert same_f32_bits([gpu["absmax_mean"]], [ref["absmax_mean"]]), \
            (gpu["absmax_mean"], ref["absmax_mean"])
    else:
        assert same_f32_bits(gpu["absmax"], ref["absmax"]), \
            f"absmax differs at {np.flatnonzero(gpu['absmax'] != ref['absmax'])[:10]}"


def product_error(y, ref, tile: int = 32) -> float:
    """Worst relative Frobenius error of a product against its reference over
    the whole matrix, every row, and every tile x tile block of the output
    (the last row and column blocks may be short): a single wrong MFMA
    sub-tile, row group or output element shows up in its row and its tile
    even when the matrix-wide figure hides it.  Where a row's or tile's
    reference is all zero the absolute error is used."""
    r = np.asarray(ref, dtype=np.float64)
    r = r.reshape(-1, r.shape[-1])
    d = np.asarray(y, dtype=np.float64).reshape(r.shape) - r

    def ratio(num2, den2):
        num, den = np.sqrt(num2), np.sqrt(den2)
        return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)

    worst = float(ratio((d * d).sum(), (r * r).sum()))
    worst = max(worst, float(ratio((d * d).sum(axis=1), (r * r).sum(axis=1)).max()))
    M, N = r.shape
    tm, tn = -(-M // tile), -(-N // tile)
    pd = np.zeros((tm * tile, tn * tile))
    pr = np.zeros((tm * tile, tn * tile))
    pd[:M, :N] = d * d
    pr[:M, :N] = r * r
    td = pd.reshape(tm, tile, tn, tile).sum(axis=(1, 3))
    tr = pr.reshape(tm, tile, tn, tile).sum(axis=(1, 3))
    return max(worst, float(ratio(td, tr).max()))
