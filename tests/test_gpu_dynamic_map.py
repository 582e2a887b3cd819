"""GPU parity of double quantization with the dynamic 8-bit map (the block
scales' second level as codes into the 256-value dynamic map instead of
linear int8 steps), called through the C ABI against the oracle:

* quantize: packed codes, the uint8 scale codes, the group scales and the
  mean bit-exact, for both quant types, at ragged and full sizes, with
  constructed exact ties and degenerate groups;
* dequantize: every output bit-exact;
* GEMV (M = 1 .. 16), GEMM, GEMM + LoRA and dX: relative Frobenius error
  <= 5e-3 per matrix, row and 32 x 32 tile against the oracle's binary64
  product with its dequantized weight, and exact where one operand is a unit
  vector (the product then is a dequantized weight itself)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import (assert_state_equal, dev_bf16, gpu_quantize, host_bits,
                               product_error, upload_state)

pytestmark = pytest.mark.gpu

TOL = 5e-3
DYN = "dynamic"


def ref_state(w, qt="nf4"):
    return oracle.quantize(w, True, quant_type=qt, dq_map=DYN)


def check_quantize(bits, shape, qt="nf4"):
    got = gpu_quantize(bits, shape, True, quant_type=qt, dq_map=DYN)
    ref = ref_state(bits, qt)
    assert got["_device"].absmax.dtype == torch.uint8
    assert_state_equal(got, ref)
    return got, ref


# --------------------------------------------------------------------------
# quantize
# --------------------------------------------------------------------------
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("s", [0, 1, 2])
def test_dyn_quantize_decode_shapes(s, qt):
    w, _ = synth.decode(s)
    check_quantize(w, w.shape, qt)


def test_dyn_quantize_batched_outliers():
    w, _ = synth.batched()
    check_quantize(w, w.shape)


@pytest.mark.parametrize("n", [2, 62, 66, 64 * 255 + 2, 64 * 257 + 18, 64 * 256 * 5 + 130])
def test_dyn_quantize_ragged(n):
    w = synth.normal_bf16((n,), 0.02, 12000 + n, outlier_frac=0.01, outlier_scale=30.0,
                          outlier_seed=12001)
    check_quantize(w, w.shape)


def test_dyn_quantize_exact_ties_take_the_lower_code():
    """Six blocks with absmax 0, 32, 23, 9, 18.5 and 13.5: the mean is 16,
    the group scale 16, and (a - 16) / 16 is -1, 1, +-0.4375 and +-0.15625.
    0.4375 is exactly the midpoint of map values 214 and 215, 0.15625 that of
    194 and 195, and their negatives those of 39/40 and 59/60: each tie takes
    the lower code."""
    f = np.zeros(6 * 64, np.float32)
    for b, a in enumerate([0.0, 32.0, 23.0, -9.0, 18.5, -13.5]):
        f[64 * b + 3 * b] = a
    bits = oracle.f32_to_bf16_bits(f)
    got, ref = check_quantize(bits, bits.shape)
    assert ref["absmax_mean"] == np.float32(16.0)
    assert float(ref["absmax2"][0]) == 16.0
    dmap = oracle.dynamic_map().astype(np.float64)
    for lo in (214, 194, 39, 59):
        t = {214: 0.4375, 194: 0.15625, 39: -0.4375, 59: -0.15625}[lo]
        assert (dmap[lo] + dmap[lo + 1]) / 2 == t
    assert ref["absmax"].tolist() == [0, 255, 214, 39, 194, 59]


def test_dyn_quantize_constant_groups_store_the_zero_code():
    """Every block's absmax equal: every centred scale is 0, the group scale
    0, and every code the index of 0.0 (127); the dequantized scale is the
    mean itself."""
    n = 64 * 600
    f = np.where(np.arange(n) % 2 == 0, 0.375, -0.375).astype(np.float32)
    bits = oracle.f32_to_bf16_bits(f)
    got, ref = check_quantize(bits, bits.shape)
    assert np.all(ref["absmax"] == 127) and np.all(ref["absmax2"] == 0.0)
    out = host_bits(T.dequantize(got["_device"]))
    assert np.array_equal(out, oracle.dequantize(ref["packed"], ref))


def test_dyn_and_linear_maps_differ():
    """The two second-level maps store different codes for the same weight
    (the flag reaches the kernel) and dequantize to different weights, each
    equal to the oracle's for its own map."""
    w, _ = synth.decode(0)
    lin = gpu_quantize(w, w.shape, True)
    dyn = gpu_quantize(w, w.shape, True, dq_map=DYN)
    assert np.array_equal(lin["packed"], dyn["packed"])
    assert not np.array_equal(lin["absmax"].view(np.uint8), dyn["absmax"])
    out_lin = host_bits(T.dequantize(lin["_device"]))
    out_dyn = host_bits(T.dequantize(dyn["_device"]))
    assert not np.array_equal(out_lin, out_dyn)
    assert np.array_equal(out_dyn, oracle.dequantize(dyn["packed"], dyn))
    assert np.array_equal(out_lin, oracle.dequantize(lin["packed"], lin))


# --------------------------------------------------------------------------
# dequantize
# --------------------------------------------------------------------------
@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "bf16"), ("nf4", "f16"),
                                   ("fp4", "f16")])
@pytest.mark.parametrize("n", [66, 64 * 257 + 18, 4096 * 4096])
def test_dyn_dequant_bit_exact(n, qt, dt):
    w = synth.normal_bf16((n,), 0.02, 12200 + n % 1000, outlier_frac=0.001, outlier_scale=20.0,
                          outlier_seed=12201)
    ref = ref_state(w, qt)
    q = upload_state(ref, (n,), dt)
    out = host_bits(T.dequantize(q))
    want = oracle.dequantize(ref["packed"], ref, dtype=dt)
    bad = np.flatnonzero(out != want)
    assert bad.size == 0, f"{bad.size} mismatches, first at {bad[:8]}"


# --------------------------------------------------------------------------
# products
# --------------------------------------------------------------------------
def as_f64(bits, dt, shape):
    return oracle.bits_to_f32(bits, dt).astype(np.float64).reshape(shape)


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("N,K", [(4096, 4096), (11008, 4096), (4096, 11008), (300, 4160),
                                 (70, 20480), (40, 32768)])
def test_dyn_gemv(M, N, K, qt, dt):
    w = synth.normal_bf16((N, K), 0.02, 12300 + N + K)
    x = synth.normal_16((M, K), 1.0, 12301 + M, dt)
    ref = ref_state(w, qt)
    q = upload_state(ref, (N, K), dt)
    y = T.gemv(dev_bf16(x, (M, K), dt), q)
    torch.cuda.synchronize()
    err = product_error(as_f64(host_bits(y), dt, (M, N)),
                        oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


@pytest.mark.parametrize("M", [1, 3, 16])
def test_dyn_gemv_unit_vector_pins_every_block_scale(M):
    """X = rows of unit vectors.  The decode kernels multiply X by the levels
    rounded to the compute type and scale each block's partial sum by the
    fp32 block scale, so Y[m, n] is exactly rnd(fl32(rnd(L[c]) * a_hat_b))
    for the weight (n, k_m): one product by 1.0, the rest sums of zeros.
    Every block scale of those columns is checked bit for bit."""
    N, K = 2048, 4096
    w = synth.normal_bf16((N, K), 0.02, 12400)
    ref = ref_state(w)
    ks = (np.arange(M) * 997 + 5) % K
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80
    y = T.gemv(dev_bf16(x, (M, K)), upload_state(ref, (N, K)))
    torch.cuda.synchronize()
    lv16 = oracle.bits_to_f32(oracle.f32_to_bits(oracle.codebook(), "bf16"), "bf16")
    scale = oracle.block_scales(ref)
    j = np.arange(N)[None, :] * K + ks[:, None]          # [M, N] weight indices
    want = oracle.f32_to_bits((lv16[ref["codes"][j]] * scale[j // 64]).astype(np.float32),
                              "bf16")
    assert np.array_equal(host_bits(y).reshape(M, N), want)


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("M,N,K", [(7, 64, 64), (300, 260, 320), (513, 1024, 512),
                                   (256, 512, 64 * 66)])
def test_dyn_gemm(M, N, K, qt, dt):
    w = synth.normal_bf16((N, K), 0.02, 12500 + N + K)
    x = synth.normal_16((M, K), 1.0, 12501 + M, dt)
    ref = ref_state(w, qt)
    y = T.gemm(dev_bf16(x, (M, K), dt), upload_state(ref, (N, K), dt))
    torch.cuda.synchronize()
    err = product_error(as_f64(host_bits(y), dt, (M, N)),
                        oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


def test_dyn_gemm_prefill_shape_every_row():
    """M=2048, N=K=8192 with the dynamic map: the whole product checked."""
    M, N, K = synth.PREFILL_SHAPE
    w, x = synth.prefill()
    ref = ref_state(w)
    y = T.gemm(dev_bf16(x, (M, K)), upload_state(ref, (N, K)))
    torch.cuda.synchronize()
    err = product_error(as_f64(host_bits(y), "bf16", (M, N)),
                        oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K))
    assert err <= TOL, err


def test_dyn_gemm_unit_vectors_are_weight_columns():
    M, N, K = 256, 512, 1024
    w = synth.normal_bf16((N, K), 0.02, 12600)
    ref = ref_state(w)
    ks = (np.arange(M) * 131 + 7) % K
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80
    y = T.gemm(dev_bf16(x, (M, K)), upload_state(ref, (N, K)))
    torch.cuda.synchronize()
    wh = oracle.dequantize(ref["packed"], ref).reshape(N, K)
    assert np.array_equal(host_bits(y).reshape(M, N), wh[:, ks].T)


def test_dyn_gemm_lora():
    M, N, K, r = 300, 260, 1024, 16
    w = synth.normal_bf16((N, K), 0.02, 12700)
    x = synth.normal_16((M, K), 1.0, 12701)
    xa = synth.normal_16((M, r), 0.5, 12702)
    b = synth.normal_16((N, r), 0.05, 12703)
    ref = ref_state(w)
    y = T.gemm_lora(dev_bf16(x, (M, K)), upload_state(ref, (N, K)), dev_bf16(xa, (M, r)),
                    dev_bf16(b, (N, r)))
    torch.cuda.synchronize()
    err = product_error(as_f64(host_bits(y), "bf16", (M, N)),
                        oracle.lora_matmul_ref(x, ref["packed"], ref, N, K, xa, b))
    assert err <= TOL, err


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("M,N,K", [(7, 64, 64), (300, 128, 320), (513, 1024, 512)])
def test_dyn_dx(M, N, K, qt, dt):
    w = synth.normal_bf16((N, K), 0.02, 12800 + N + K)
    dy = synth.normal_16((M, N), 1.0, 12801 + M, dt)
    ref = ref_state(w, qt)
    dx = T.gemm_dx(dev_bf16(dy, (M, N), dt), upload_state(ref, (N, K), dt))
    torch.cuda.synchronize()
    err = product_error(as_f64(host_bits(dx), dt, (M, K)),
                        oracle.dequant_matmul_dx_ref(dy, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


def test_dyn_dx_one_hot_rows_are_weight_rows():
    N, K = 128, 512
    w = synth.normal_bf16((N, K), 0.02, 12900)
    ref = ref_state(w)
    eye = np.zeros((N, N), np.uint16)
    eye[np.arange(N), np.arange(N)] = 0x3F80
    dx = T.gemm_dx(dev_bf16(eye, (N, N)), upload_state(ref, (N, K)))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dx), oracle.dequantize(ref["packed"], ref))
