"""GPU parity of bnbx_gemm_nf4_lora, Y = X . W_hat^T + XA . B^T (a LoRA term
fused into the 4-bit GEMM), against the oracle's binary64 result:
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
                                     (2048, 1024, 2048, 16), (260, 300, 512, 48),
                                     (130, 520, 1024, 256), (64, 256, 512, 240)])
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


@pytest.mark.parametrize("qt,dt,dq_map", [("nf4", "bf16", "linear"), ("fp4", "f16", "linear"),
                                          ("nf4", "bf16", "dynamic"), ("nf4", "f16", None)])
@pytest.mark.parametrize("M,N,K,r", [(1, 4096, 4096, 16), (1, 11008, 4096, 64), (2, 300, 11008, 256),
                                     (3, 777, 1024, 48), (4, 1000, 512, 240), (1, 20000, 256, 32),
                                     (5, 4100, 4096, 16), (8, 333, 11008, 80), (16, 14336, 4096, 64),
                                     (13, 999, 512, 256), (16, 64, 64, 32),
                                     # one rank per lane slot up to rank 64, two up to 128, four above
                                     (1, 1030, 8192, 64), (1, 1030, 8192, 80), (3, 257, 4096, 80),
                                     (2, 4096, 4096, 128), (1, 700, 4096, 144),
                                     # two 8-wave workgroups per CU (three rows per wave)
                                     (1, 9000, 512, 128), (1, 9000, 1024, 256), (1, 11008, 4096, 16)])
def test_lora_decode_rows(M, N, K, r, qt, dt, dq_map):
    """Up to 16 rows of X: the decode GEMVs add the low-rank term before
    their reductions (up to 4 rows: ragged N, K = 11008 over two waves per
    row, more rows than one pass holds; 5 to 16 rows: one or several K chunks,
    ragged row groups, ranks past one 32-rank chunk per wave; every scale
    layout)."""
    w = synth.normal_bf16((N, K), 0.02, 9840 + r)
    x = synth.normal_16((M, K), 1.0, 9841 + M, dt)
    xa = synth.normal_16((M, r), 0.5, 9842 + r, dt)
    b = synth.normal_16((N, r), 0.05, 9843 + r, dt)
    ref = oracle.quantize(w, dq_map is not None, quant_type=qt, dq_map=dq_map or "linear")
    q = upload_state(ref, (N, K), dt)
    print(f"lora decode M={M} N={N} K={K} r={r} {qt} {dt} {dq_map}", flush=True)
    y = T.gemm_lora(dev_bf16(x, (M, K), dt), q, dev_bf16(xa, (M, r), dt), dev_bf16(b, (N, r), dt))
    torch.cuda.synchronize()
    got = oracle.bits_to_f32(host_bits(y), dt).astype(np.float64).reshape(M, N)
    want = oracle.lora_matmul_ref(x, ref["packed"], ref, N, K, xa, b, dt)
    err = product_error(got, want)
    assert err <= TOL, err
    base = oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt)
    assert oracle.rel_frobenius(base, want) > 10 * TOL


def test_lora_decode_zero_adapter_equals_plain_gemv():
    """B = 0 at M <= 16: the result equals bnbx_gemv_nf4 bit for bit (the same
    kernels, plus exact zeros)."""
    N, K, r = 1500, 2048, 32
    w = synth.normal_bf16((N, K), 0.02, 9850)
    ref = oracle.quantize(w, True)
    q = upload_state(ref, (N, K))
    for M in (1, 2, 3, 4, 6, 16):
        x = dev_bf16(synth.normal_16((M, K), 1.0, 9851 + M), (M, K))
        xa = dev_bf16(synth.normal_16((M, r), 1.0, 9855 + M), (M, r))
        zb = torch.zeros((N, r), dtype=torch.bfloat16, device="cuda")
        y1 = T.gemv(x, q)
        y2 = T.gemm_lora(x, q, xa, zb)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), M


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


# --------------------------------------------------------------------------
# the adapter's down-projection inside the library (bnbx_lora_down)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,K,r", [(1, 64, 16), (7, 1024, 48), (16, 4096, 64), (300, 512, 256),
                                   (2048, 8192, 16), (33, 8192, 128), (4100, 256, 32),
                                   (4099, 96, 256)])
def test_lora_down_against_oracle(M, K, r, dt):
    x = synth.normal_16((M, K), 1.0, 9900 + M, dt)
    a = synth.normal_16((r, K), 0.02, 9901 + r, dt)
    print(f"lora_down M={M} K={K} r={r} {dt}", flush=True)
    xa = T.lora_down(dev_bf16(x, (M, K), dt), dev_bf16(a, (r, K), dt), 0.75)
    torch.cuda.synchronize()
    got = oracle.bits_to_f32(host_bits(xa), dt).astype(np.float64).reshape(M, r)
    err = product_error(got, oracle.lora_down_ref(x, a, 0.75, M, K, dt))
    assert err <= TOL, err


def test_lora_down_one_hot_rows_are_scaled_adapter_columns():
    """X = unit rows: XA[m] = rnd(0.5 * A[:, k_m]), exactly (one product by
    1.0, sums of zeros, a scale by a power of two)."""
    M, K, r = 40, 1024, 32
    a = synth.normal_16((r, K), 0.02, 9910)
    ks = (np.arange(M) * 37 + 3) % K
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80
    xa = T.lora_down(dev_bf16(x, (M, K)), dev_bf16(a, (r, K)), 0.5)
    torch.cuda.synchronize()
    a64 = oracle.bf16_bits_to_f32(a).astype(np.float64).reshape(r, K)
    want = oracle.f32_to_bits((0.5 * a64[:, ks].T).astype(np.float32), "bf16")
    assert np.array_equal(host_bits(xa).reshape(M, r), want.reshape(M, r))


def test_lora_down_repeats_bit_for_bit_and_writes_only_its_block():
    M, K, r = 300, 2048, 64
    x = dev_bf16(synth.normal_16((M, K), 1.0, 9920), (M, K))
    a = dev_bf16(synth.normal_16((r, K), 0.02, 9921), (r, K))
    big = torch.full((M, r + 32), 7.0, dtype=torch.bfloat16, device="cuda")
    T.lora_down(x, a, 1.0, out=big[:, :r])
    first = big.clone()
    T.lora_down(x, a, 1.0, out=big[:, :r])
    torch.cuda.synchronize()
    assert torch.equal(first, big)
    assert torch.all(big[:, r:] == 7.0)


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
def test_linear_lora_end_to_end(qt, dt):
    """Y = X . W_hat^T + s . (X . A^T) . B^T through the two library calls
    (the down-projection, then the GEMM with the low-rank term)."""
    M, N, K, r = 257, 384, 1024, 32
    w = synth.normal_bf16((N, K), 0.02, 9930)
    x = synth.normal_16((M, K), 1.0, 9931, dt)
    a = synth.normal_16((r, K), 0.02, 9932, dt)
    b = synth.normal_16((N, r), 0.05, 9933, dt)
    ref = oracle.quantize(w, True, quant_type=qt)
    y = T.linear_lora(dev_bf16(x, (M, K), dt), upload_state(ref, (N, K), dt),
                      dev_bf16(a, (r, K), dt), dev_bf16(b, (N, r), dt), 2.0)
    torch.cuda.synchronize()
    got = oracle.bits_to_f32(host_bits(y), dt).astype(np.float64).reshape(M, N)
    xa = oracle.lora_down_ref(x, a, 2.0, M, K, dt)
    b64 = oracle.bits_to_f32(b, dt).astype(np.float64).reshape(N, r)
    want = oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt) + xa @ b64.T
    err = product_error(got, want)
    assert err <= TOL, err
    base = oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt)
    assert oracle.rel_frobenius(base, want) > 10 * TOL

