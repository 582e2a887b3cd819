"""GPU parity of bnbx_gemm_nf4_lora, Y = X . W_hat^T + XA . B^T (a LoRA term
fused into the 4-bit GEMM's epilogue), against the oracle's binary64 result:
relative Frobenius error <= 5e-3.  Called through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import dev_bf16, host_bits, upload_state, product_error

pytestmark = pytest.mark.gpu

TOL = 5e-3


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("M,N,K,r", [(7, 200, 512, 16), (300, 260, 1024, 64), (513, 384, 256, 32),
                                     (2048, 1024, 2048, 16)])
def test_lora_shapes(M, N, K, r, qt, dt):
    w = synth.normal_bf16((N, K), 0.02, 9800 + r)
    x = synth.normal_16((M, K), 1.0, 9801 + M, dt)
    xa = synth.normal_16((M, r), 0.5, 9802 + r, dt)
    b = synth.normal_16((N, r), 0.05, 9803 + r, dt)
    ref = oracle.quantize(w, True, quant_type=qt)
    q = upload_state(ref, (N, K), dt)
    y = T.gemm_lora(dev_bf16(x, (M, K), dt), q, dev_bf16(xa, (M, r), dt), dev_bf16(b, (N, r), dt))
    torch.cuda.synchronize()
    got = oracle.bits_to_f32(host_bits(y), dt).astype(np.float64).reshape(M, N)
    want = oracle.lora_matmul_ref(x, ref["packed"], ref, N, K, xa, b, dt)
    err = product_error(got, want)
    assert err <= TOL, err
    # the low-rank term is not lost in the tolerance: it alone is far off
    base = oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt)
    assert oracle.rel_frobenius(base, want) > 10 * TOL


def test_lora_zero_adapter_equals_plain_gemm():
    """B = 0: the fused result equals bnbx_gemm_nf4 bit for bit."""
    M, N, K, r = 300, 512, 1024, 16
    w = synth.normal_bf16((N, K), 0.02, 9810)
    x = dev_bf16(synth.normal_16((M, K), 1.0, 9811), (M, K))
    ref = oracle.quantize(w, True)
    q = upload_state(ref, (N, K))
    xa = dev_bf16(synth.normal_16((M, r), 1.0, 9812), (M, r))
    zb = torch.zeros((N, r), dtype=torch.bfloat16, device="cuda")
    y1 = T.gemm(x, q)
    y2 = T.gemm_lora(x, q, xa, zb)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
