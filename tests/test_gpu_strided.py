"""GPU parity with strided buffers: X, Y, dY and dX whose leading dimensions
exceed their logical widths (ldx > K, ldy > N, lddy > N, lddx > K), through
the C ABI.  Products within 5e-3 relative Frobenius of the oracle, and the
padding columns of the outputs left untouched."""

import numpy as np
import pytest
import torch

import dequant_gemm_nf4_amd as B
import oracle
import synth
from tests.gpu_helpers import TORCH_DTYPE, dev_bf16, host_bits, upload_state, product_error

pytestmark = pytest.mark.gpu

TOL = 5e-3
SENTINEL = 0x7E7E   # a NaN pattern in bf16 and binary16: never a product


def strided(bits, rows, cols, ld, dt):
    full = np.full((rows, ld), SENTINEL, np.uint16)
    full[:, :cols] = np.asarray(bits).reshape(rows, cols)
    return dev_bf16(full, (rows, ld), dt)


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("kind,M", [("gemv", 1), ("gemv", 3), ("gemv", 16), ("gemm", 40),
                                    ("gemm", 300)])
def test_forward_strided(kind, M, qt, dt):
    N, K = 384, 1024
    ldx, ldy = K + 64, N + 8
    w = synth.normal_bf16((N, K), 0.02, 9990)
    xb = synth.normal_16((M, K), 1.0, 9991 + M, dt)
    ref = oracle.quantize(w, True, quant_type=qt)
    q = upload_state(ref, (N, K), dt)
    x = strided(xb, M, K, ldx, dt)
    y = torch.full((M, ldy), 0, dtype=TORCH_DTYPE[dt], device="cuda")
    y.view(torch.int16).fill_(SENTINEL)
    fn = B.bnbx_gemv_nf4 if kind == "gemv" else B.bnbx_gemm_nf4
    fn(x, ldx, q.packed, q.state, M, N, K, y, ldy)
    torch.cuda.synchronize()
    yb = host_bits(y).reshape(M, ldy)
    assert np.all(yb[:, N:] == SENTINEL)
    got = oracle.bits_to_f32(yb[:, :N], dt).astype(np.float64)
    err = product_error(got, oracle.dequant_matmul_ref(xb, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("M", [5, 300])
def test_dx_strided(M, qt, dt):
    N, K = 256, 640
    lddy, lddx = N + 16, K + 8
    w = synth.normal_bf16((N, K), 0.02, 9995)
    dyb = synth.normal_16((M, N), 1.0, 9996 + M, dt)
    ref = oracle.quantize(w, True, quant_type=qt)
    q = upload_state(ref, (N, K), dt)
    dy = strided(dyb, M, N, lddy, dt)
    dx = torch.zeros((M, lddx), dtype=TORCH_DTYPE[dt], device="cuda")
    dx.view(torch.int16).fill_(SENTINEL)
    B.bnbx_gemm_nf4_dx(dy, lddy, q.packed, q.state, M, N, K, dx, lddx)
    torch.cuda.synchronize()
    xb = host_bits(dx).reshape(M, lddx)
    assert np.all(xb[:, K:] == SENTINEL)
    got = oracle.bits_to_f32(xb[:, :K], dt).astype(np.float64)
    err = product_error(got, oracle.dequant_matmul_dx_ref(dyb, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err
