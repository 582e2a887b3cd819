"""Seeded synthetic inputs for the NF4 path (shared by the tests, the smoke
check and the benchmark).

This module only draws random numbers and rounds them to bfloat16 (or, for
FP16-compute activations, IEEE binary16) for storage; it holds none of the quantization arithmetic, and neither the oracle
nor the HIP library imports the other through it.

Recipe (NumPy PCG64 ``default_rng(seed)``, ``standard_normal`` in binary32,
scaled by sigma, optional outlier scaling, then one round-to-nearest-even to
bfloat16 done by PyTorch's CPU conversion):

=========  =============================================================  ======
workload   tensors                                                        seeds
=========  =============================================================  ======
tiny       W 256x512 N(0, 0.02); X 1x512 N(0, 1); no double quant          1, 2
decode s   W NxK N(0, 0.02) for (4096,4096), (11008,4096), (4096,11008);  1001+10s
           X 1xK N(0, 1); double quant                                    1002+10s
batched    W 14336x4096 N(0, 0.02), 0.1% of entries (without replacement) 2001
           scaled x20; X 16x4096 N(0, 1); double quant                    2002, 2003
prefill    W 8192x8192 N(0, 0.015); X 2048x8192 N(0, 1) with 4 of the     3001
           8192 feature columns scaled x50; double quant                  3002, 3003
=========  =============================================================  ======

FP16 compute dtype: the activations X are drawn with the same seeds and
rounded to binary16 instead (``x_dtype="f16"``); weights stay bfloat16, the
quantize input type.

The bulk quantize-on-load stack (32 layers of Llama-7B-shaped linears) is
drawn on the device by the benchmark, because 6.5e9 host draws would take
minutes; its shapes are listed in ``BULK_LAYER_SHAPES``.  ``bulk_layer(l)``
draws one such layer on the host (W N(0, 0.02), seeds 4000 + 10 l + i for
linear i), for CPU timings of the oracle on a sample of the stack.
"""

from __future__ import annotations

import numpy as np

DECODE_SHAPES = ((4096, 4096), (11008, 4096), (4096, 11008))   # (N, K)
BATCHED_SHAPE = (16, 14336, 4096)                                # (M, N, K)
PREFILL_SHAPE = (2048, 8192, 8192)                               # (M, N, K)
TINY_SHAPE = (1, 256, 512)                                       # (M, N, K)
# per layer: q, k, v, o (4096x4096), gate, up (11008x4096), down (4096x11008)
BULK_LAYER_SHAPES = ((4096, 4096),) * 4 + ((11008, 4096),) * 2 + ((4096, 11008),)
BULK_LAYERS = 32


def to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round binary32 samples to bfloat16 storage (PyTorch CPU, nearest-even)
    and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_f16_bits(f: np.ndarray) -> np.ndarray:
    """Round binary32 samples to IEEE binary16 storage (PyTorch CPU,
    nearest-even) and return the uint16 bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32))
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_16(shape, sigma: float, seed: int, dtype: str = "bf16", **kw) -> np.ndarray:
    """``normal_bf16`` rounded to bfloat16 ("bf16") or binary16 ("f16")."""
    if dtype == "bf16":
        return normal_bf16(shape, sigma, seed, **kw)
    if dtype == "f16":
        return normal_bf16(shape, sigma, seed, _round=to_f16_bits, **kw)
    raise ValueError(dtype)


def normal_bf16(shape, sigma: float, seed: int, outlier_frac: float = 0.0,
                outlier_scale: float = 1.0, outlier_seed: int | None = None,
                outlier_cols: int = 0, _round=None) -> np.ndarray:
    """bfloat16 bit patterns of N(0, sigma^2) samples.

    ``outlier_frac``: that fraction of all entries (chosen without
    replacement with ``outlier_seed``) is multiplied by ``outlier_scale``.
    ``outlier_cols``: that many whole columns (last axis) are multiplied by
    ``outlier_scale`` instead.  Scaling happens before the bf16 rounding."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    f = rng.standard_normal(n, dtype=np.float32)
    f *= np.float32(sigma)
    f = f.reshape(shape)
    if outlier_frac > 0:
        k = int(round(outlier_frac * n))
        idx = np.random.default_rng(outlier_seed).choice(n, size=k, replace=False)
        flat = f.reshape(-1)
        flat[idx] *= np.float32(outlier_scale)
    if outlier_cols > 0:
        cols = np.random.default_rng(outlier_seed).choice(shape[-1], size=outlier_cols,
                                                          replace=False)
        f[..., cols] *= np.float32(outlier_scale)
    return (_round or to_bf16_bits)(f)


def tiny(x_dtype: str = "bf16"):
    M, N, K = TINY_SHAPE
    return normal_bf16((N, K), 0.02, 1), normal_16((M, K), 1.0, 2, x_dtype)


def decode(s: int, x_dtype: str = "bf16"):
    N, K = DECODE_SHAPES[s]
    return (normal_bf16((N, K), 0.02, 1001 + 10 * s),
            normal_16((1, K), 1.0, 1002 + 10 * s, x_dtype))


def batched(x_dtype: str = "bf16"):
    M, N, K = BATCHED_SHAPE
    w = normal_bf16((N, K), 0.02, 2001, outlier_frac=0.001, outlier_scale=20.0,
                    outlier_seed=2003)
    return w, normal_16((M, K), 1.0, 2002, x_dtype)


def prefill(x_dtype: str = "bf16"):
    M, N, K = PREFILL_SHAPE
    w = normal_bf16((N, K), 0.015, 3001)
    x = normal_16((M, K), 1.0, 3002, x_dtype, outlier_scale=50.0, outlier_seed=3003,
                  outlier_cols=4)
    return w, x


def bulk_layer(l: int):
    """The seven linears of layer l of the bulk stack (q, k, v, o, gate, up,
    down), bf16 bit patterns."""
    return [normal_bf16(shape, 0.02, 4000 + 10 * l + i) for i, shape in enumerate(BULK_LAYER_SHAPES)]
