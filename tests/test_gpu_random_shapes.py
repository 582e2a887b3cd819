"""Seeded sweep of random shapes over every product entry point (GEMV, GEMM,
GEMM with a LoRA term, dX), quant type, compute dtype and double quant,
against the oracle: relative Frobenius error <= 5e-3.  The shapes (fixed by
the seed) are ragged in M, N and K within each entry point's limits."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import dev_bf16, host_bits, upload_state, product_error

pytestmark = pytest.mark.gpu

TOL = 5e-3


def cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    kinds = ["gemv", "gemm", "lora", "dx"]
    for i in range(n):
        kind = kinds[i % 4]
        qt = ["nf4", "fp4"][rng.integers(2)]
        dt = ["bf16", "f16"][rng.integers(2)]
        dq = bool(rng.integers(2))
        K = 64 * int(rng.integers(1, 41))
        if kind == "gemv":
            M = int(rng.integers(1, 17))
        else:
            M = int(rng.integers(1, 601))
        N = 64 * int(rng.integers(1, 11)) if kind == "dx" else int(rng.integers(1, 701))
        r = 16 * int(rng.integers(1, 5))
        out.append((i, kind, qt, dt, dq, M, N, K, r))
    return out


@pytest.mark.parametrize("i,kind,qt,dt,dq,M,N,K,r", cases())
def test_random_shape(i, kind, qt, dt, dq, M, N, K, r):
    w = synth.normal_bf16((N, K), 0.03, 12000 + i)
    ref = oracle.quantize(w, dq, quant_type=qt)
    q = upload_state(ref, (N, K), dt)
    if kind == "dx":
        dy = synth.normal_16((M, N), 1.0, 12100 + i, dt)
        got = T.gemm_dx(dev_bf16(dy, (M, N), dt), q)
        want = oracle.dequant_matmul_dx_ref(dy, ref["packed"], ref, N, K, dt)
        shape = (M, K)
    else:
        x = synth.normal_16((M, K), 1.0, 12200 + i, dt)
        xd = dev_bf16(x, (M, K), dt)
        if kind == "lora":
            xa = synth.normal_16((M, r), 0.5, 12300 + i, dt)
            b = synth.normal_16((N, r), 0.05, 12400 + i, dt)
            got = T.gemm_lora(xd, q, dev_bf16(xa, (M, r), dt), dev_bf16(b, (N, r), dt))
            want = oracle.lora_matmul_ref(x, ref["packed"], ref, N, K, xa, b, dt)
        else:
            got = (T.gemv if kind == "gemv" else T.gemm)(xd, q)
            want = oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt)
        shape = (M, N)
    torch.cuda.synchronize()
    y = oracle.bits_to_f32(host_bits(got), dt).astype(np.float64).reshape(shape)
    err = product_error(y, want)
    assert err <= TOL, (kind, qt, dt, dq, M, N, K, err)


def qcases(n=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        size = 2 * int(rng.integers(1, 150001))
        sigma = float(10.0 ** rng.uniform(-4, 2))
        out.append((i, size, sigma, ["nf4", "fp4"][i % 2], bool((i // 2) % 2),
                    ["bf16", "f16"][(i // 4) % 2]))
    return out


@pytest.mark.parametrize("i,size,sigma,qt,dq,dt", qcases())
def test_random_size_quantize_dequantize_bit_exact(i, size, sigma, qt, dq, dt):
    """Quantize on the GPU equals the oracle's codes and scales, and the GPU
    dequantize of the oracle's state equals the oracle's, bit for bit."""
    from tests.gpu_helpers import assert_state_equal, gpu_quantize
    bits = synth.normal_bf16((size,), sigma, 13000 + i)
    ref = oracle.quantize(bits, dq, quant_type=qt)
    got = gpu_quantize(bits, (size,), dq, quant_type=qt, dtype=dt)
    assert_state_equal(got, ref)
    q = upload_state(ref, (size,), dt)
    out = host_bits(T.dequantize(q))
    assert np.array_equal(out, oracle.dequantize(ref["packed"], ref, dtype=dt))


def tall_cases(n=8, seed=20261204):
    """M=1 with more than 8192 rows and K <= 4096: rows chained three or four
    deep per wave (two 8-wave workgroups per CU) or, past 16384 rows, more
    than one pass of 16-wave workgroups."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        qt = ["nf4", "fp4"][i % 2]
        dt = ["bf16", "f16"][rng.integers(2)]
        dq = ["none", "linear", "dynamic"][rng.integers(3)]
        N = int(rng.integers(8193, 20001))
        K = 64 * int(rng.integers(1, 1 + min(64, 40_000_000 // (64 * N))))
        out.append((i, qt, dt, dq, N, K))
    return out


@pytest.mark.parametrize("i,qt,dt,dq,N,K", tall_cases())
def test_random_tall_gemv_m1(i, qt, dt, dq, N, K):
    w = synth.normal_bf16((N, K), 0.03, 12500 + i)
    ref = oracle.quantize(w, dq != "none", quant_type=qt,
                          dq_map="dynamic" if dq == "dynamic" else "linear")
    q = upload_state(ref, (N, K), dt)
    x = synth.normal_16((1, K), 1.0, 12600 + i, dt)
    got = T.gemv(dev_bf16(x, (1, K), dt), q)
    torch.cuda.synchronize()
    want = oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt)
    g = oracle.bits_to_f32(host_bits(got), dt).astype(np.float64).reshape(1, N)
    err = product_error(g, want)
    assert err <= TOL, (i, qt, dt, dq, N, K, err)


def down_cases(n=8, seed=20261205):
    """The LoRA down-projection at random M (both row counts per workgroup),
    K and rank."""
    rng = np.random.default_rng(seed)
    return [(i, ["bf16", "f16"][rng.integers(2)], int(rng.integers(1, 5001)),
             32 * int(rng.integers(1, 97)), 16 * int(rng.integers(1, 17))) for i in range(n)]


@pytest.mark.parametrize("i,dt,M,K,r", down_cases())
def test_random_lora_down(i, dt, M, K, r):
    x = synth.normal_16((M, K), 1.0, 12700 + i, dt)
    a = synth.normal_16((r, K), 0.02, 12800 + i, dt)
    got = T.lora_down(dev_bf16(x, (M, K), dt), dev_bf16(a, (r, K), dt), 0.25)
    torch.cuda.synchronize()
    g = oracle.bits_to_f32(host_bits(got), dt).astype(np.float64).reshape(M, r)
    err = product_error(g, oracle.lora_down_ref(x, a, 0.25, M, K, dt))
    assert err <= TOL, (i, dt, M, K, r, err)
