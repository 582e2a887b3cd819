"""GPU parity of bnbx_gemm_nf4_dx, dX = dY . W_hat (the input gradient of the
4-bit linear layer, weights frozen), against the oracle's binary64 product
with its dequantized weight: relative Frobenius error <= 5e-3 (the kernel
multiplies exactly the dequantized weights and accumulates in fp32, so the
error is the rounding of dX into the compute type).  Called through the C
ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import dev_bf16, host_bits, upload_state, product_error

pytestmark = pytest.mark.gpu

TOL = 5e-3
COMBOS = [("nf4", "bf16"), ("fp4", "bf16"), ("nf4", "f16"), ("fp4", "f16")]


def run_dx(dy_bits, M, N, K, ref, dt):
    q = upload_state(ref, (N, K), dt)
    dy = dev_bf16(dy_bits, (M, N), dt)
    dx = T.gemm_dx(dy, q)
    torch.cuda.synchronize()
    return oracle.bits_to_f32(host_bits(dx), dt).astype(np.float64).reshape(M, K)


@pytest.mark.parametrize("qt,dt", COMBOS)
@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("M,N,K", [(7, 64, 64), (300, 128, 320), (64, 192, 11008),
                                   (513, 1024, 512), (1, 4096, 4096)])
def test_dx_shapes(M, N, K, dq, qt, dt):
    w = synth.normal_bf16((N, K), 0.02, 9500 + N + K)
    dy = synth.normal_16((M, N), 1.0, 9600 + M, dt)
    ref = oracle.quantize(w, dq, quant_type=qt)
    got = run_dx(dy, M, N, K, ref, dt)
    err = product_error(got, oracle.dequant_matmul_dx_ref(dy, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
def test_dx_one_hot_rows_are_weight_rows(qt, dt):
    """dY = rows of the identity: dX is W_hat itself, exactly (one product
    by 1.0 per output, no rounding)."""
    N, K = 128, 512
    w = synth.normal_bf16((N, K), 0.02, 9700)
    ref = oracle.quantize(w, True, quant_type=qt)
    one = 0x3F80 if dt == "bf16" else 0x3C00
    eye = np.zeros((N, N), np.uint16)
    eye[np.arange(N), np.arange(N)] = one
    q = upload_state(ref, (N, K), dt)
    dx = T.gemm_dx(dev_bf16(eye, (N, N), dt), q)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dx), oracle.dequantize(ref["packed"], ref, dtype=dt))


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
def test_dx_prefill_shape_every_row(qt, dt):
    """M=2048, N=K=8192 (the prefill layer's input gradient), double quant:
    the full product runs and all of dX is checked (whole matrix, every row,
    every 32x32 tile)."""
    M, N, K = synth.PREFILL_SHAPE
    w, _ = synth.prefill()
    dy = synth.normal_16((M, N), 1.0, 9800, dt)
    ref = oracle.quantize(w, True, quant_type=qt)
    got = run_dx(dy, M, N, K, ref, dt)
    assert np.all(np.isfinite(got))
    want = oracle.dequant_matmul_dx_ref(dy.reshape(M, N), ref["packed"], ref, N, K, dt)
    err = product_error(got, want)
    assert err <= TOL, err
