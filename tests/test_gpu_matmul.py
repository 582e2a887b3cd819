"""GPU parity of bnbx_gemv_nf4 and bnbx_gemm_nf4 against the oracle's fp64
product with the oracle's dequantized bf16 weight.  Bar: relative Frobenius
error <= 5e-3 (the matmul tolerance this path fixes).  The kernels
accumulate in fp32 and round Y to bf16 (about 1.1e-3 rms relative), and use
the bf16-rounded levels times an fp32 block scale instead of the bf16
dequantized weight (about 1.6e-3 rms), so 5e-3 leaves room of 2x over their
sum while a wrong index, sign or scale gives errors of order 1."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import assert_state_equal, dev_bf16, gpu_quantize, host_bits, upload_state, product_error

pytestmark = pytest.mark.gpu

TOL = 5e-3


def y_of(t):
    return oracle.bf16_bits_to_f32(host_bits(t)).astype(np.float64).reshape(t.shape)


def setup(w_bits, shape, dq, check_state=True):
    ref = oracle.quantize(w_bits, dq)
    if check_state:
        got = gpu_quantize(w_bits, shape, dq)
        assert_state_equal(got, ref)
        q = got["_device"]
    else:
        q = upload_state(ref, shape)
    return ref, q


def ref_product(x_bits, ref, N, K, rows=None):
    x = np.asarray(x_bits).reshape(-1, K)
    if rows is not None:
        x = x[rows]
    return oracle.dequant_matmul_ref(x, ref["packed"], ref, N, K)


def run(kind, x_bits, M, K, q):
    x = dev_bf16(x_bits, (M, K))
    y = T.gemv(x, q) if kind == "gemv" else T.gemm(x, q)
    torch.cuda.synchronize()
    return y_of(y)


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_tiny(kind):
    w, x = synth.tiny()
    M, N, K = synth.TINY_SHAPE
    ref, q = setup(w, (N, K), False)
    err = product_error(run(kind, x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("s", [0, 1, 2])
def test_decode_shapes_m1(kind, s):
    w, x = synth.decode(s)
    N, K = synth.DECODE_SHAPES[s]
    ref, q = setup(w, (N, K), True)
    err = product_error(run(kind, x, 1, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_batched_m16_outliers(kind):
    w, x = synth.batched()
    M, N, K = synth.BATCHED_SHAPE
    ref, q = setup(w, (N, K), True)
    err = product_error(run(kind, x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("M", list(range(1, 17)))
def test_every_m_ragged_n(kind, M):
    N, K = 1000, 4096
    w = synth.normal_bf16((N, K), 0.02, 7000 + M)
    x = synth.normal_bf16((M, K), 1.0, 7100 + M)
    ref, q = setup(w, (N, K), True, check_state=False)
    err = product_error(run(kind, x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("M", [5, 8, 16])
@pytest.mark.parametrize("N,K,dq", [(200, 64, True), (200, 1088, True), (130, 4096, False),
                                    (70, 2048, True), (130, 8192, True), (50, 8192, False),
                                    (40, 16384, True), (300, 4160, True), (33, 320, False),
                                    (20000, 512, True)])
def test_gemv_more_than_four_rows(M, N, K, dq):
    """4 < M <= 16 (one launch that streams W once, any K): K from one block
    to 256 blocks, K not a multiple of the 256-k slices, ragged row groups,
    more row groups than one batch per workgroup holds, both scale
    layouts."""
    w = synth.normal_bf16((N, K), 0.05, 8000 + K + M)
    x = synth.normal_bf16((M, K), 1.0, 8100 + K + M)
    ref, q = setup(w, (N, K), dq, check_state=False)
    err = product_error(run("gemv", x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("N,K,dq", [(12289, 4096, True), (9000, 2048, False), (16000, 1024, True),
                                    (8193, 4096, True)])
def test_gemv_m1_two_workgroups_per_cu(N, K, dq):
    """M=1 shapes whose rows chain three or more deep per wave and whose X
    fits an 8 KB stage run 8-wave workgroups, two per CU: a ragged last
    workgroup (rows not a multiple of 24 or 32), one and two chunks per lane,
    per-row and fp32 block scales; 8193 rows is the smallest count at K=4096
    that chains three rows per wave (its last workgroup holds one row)."""
    w = synth.normal_bf16((N, K), 0.02, 8300 + N % 97 + K)
    x = synth.normal_bf16((1, K), 1.0, 8400 + K)
    ref, q = setup(w, (N, K), dq, check_state=False)
    err = product_error(run("gemv", x, 1, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("N,K", [(4096, 11008), (11008, 4096)])
def test_gemv_m16_llama_shapes(N, K):
    """M=16 on the Llama-7B down projection (K = 11008, three chunks of
    slices per wave) and the gate/up shape, double quant: all of Y against
    the oracle (whole matrix, every row, every tile)."""
    M = 16
    w = synth.normal_bf16((N, K), 0.02, 8300 + K)
    x = synth.normal_bf16((M, K), 1.0, 8400 + K)
    ref, q = setup(w, (N, K), True, check_state=False)
    err = product_error(run("gemv", x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
@pytest.mark.parametrize("N,K,dq", [(33, 64, False), (64, 192, True), (300, 11008, True),
                                    (40, 40960, True), (7, 4096 + 64, False)])
def test_k_variants(kind, N, K, dq):
    M = 3
    w = synth.normal_bf16((N, K), 0.05, 7200 + K)
    x = synth.normal_bf16((M, K), 1.0, 7300 + K)
    ref, q = setup(w, (N, K), dq, check_state=False)
    err = product_error(run(kind, x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (7, 200, 512), (128, 128, 64), (300, 260, 1024),
                                   (129, 127, 128), (513, 384, 256)])
def test_gemm_tiles_and_tails(M, N, K):
    w = synth.normal_bf16((N, K), 0.02, 7400 + M)
    x = synth.normal_bf16((M, K), 1.0, 7500 + M)
    ref, q = setup(w, (N, K), True, check_state=False)
    err = product_error(run("gemm", x, M, K, q), ref_product(x, ref, N, K))
    assert err <= TOL, err


def test_prefill_full_size_every_row():
    """M=2048, N=K=8192 (double quant, outlier feature columns): the full GEMM
    runs as the benchmark launches it, and all of Y is checked against the
    oracle's binary64 product, over the whole matrix, per row and per 32x32
    output tile."""
    w, x = synth.prefill()
    M, N, K = synth.PREFILL_SHAPE
    ref, q = setup(w, (N, K), True)
    y = run("gemm", x, M, K, q)
    assert np.all(np.isfinite(y))
    err = product_error(y, ref_product(x, ref, N, K))
    assert err <= TOL, err


@pytest.mark.parametrize("kind", ["gemv", "gemm"])
def test_unit_vector_picks_a_column(kind):
    """X = e_k: Y is column k of W_hat.  The GEMM's operands are the
    dequantized weights themselves (the double-quant block scale formed
    exactly as the stored format defines it), so its Y equals the column
    exactly; the GEMV scales bf16 levels by the fp32 block scale, which is
    within the bf16 rounding of the level and of the product (2^-7
    relative)."""
    N, K = 512, 1024
    w = synth.normal_bf16((N, K), 0.02, 7600)
    ref, q = setup(w, (N, K), True, check_state=False)
    what = oracle.bf16_bits_to_f32(oracle.dequantize(ref["packed"], ref)).reshape(N, K)
    for k in (0, 1, 63, 64, 1023):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80
        y = run(kind, x, 1, K, q)[0]
        col = what[:, k].astype(np.float64)
        assert np.all(np.abs(y - col) <= np.abs(col) * 2.0 ** -7 + 1e-30)
        if kind == "gemm":
            assert np.array_equal(y, col), np.flatnonzero(y != col)[:8]


def test_gemv_equals_gemm_across_m():
    N, K = 768, 2048
    w = synth.normal_bf16((N, K), 0.02, 7700)
    ref, q = setup(w, (N, K), True, check_state=False)
    for M in (1, 4, 5, 16):
        x = synth.normal_bf16((M, K), 1.0, 7800 + M)
        a = run("gemv", x, M, K, q)
        b = run("gemm", x, M, K, q)
        assert product_error(a, b) <= TOL


def test_gemm_x_past_32bit_offsets_sampled_rows():
    """X of more than 2 GiB (M = 131372, K = 8192, N = 300): the GEMM addresses
    X with 32-bit buffer offsets and walks M in slabs that keep them in range.
    Rows at both sides of every slab seam the offsets force (multiples of
    130816 rows here), the ends and random rows are checked against the
    oracle.  X comes from a seeded device generator (2.15 GB would take the
    host generator minutes); the checked rows are copied back as they are."""
    N, K, M = 300, 8192, 131072 + 300
    w = synth.normal_bf16((N, K), 0.02, 7900)
    ref, q = setup(w, (N, K), True, check_state=False)
    g = torch.Generator(device="cuda")
    g.manual_seed(7901)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    torch.cuda.synchronize()
    y = T.gemm(x, q)
    torch.cuda.synchronize()
    seam = (2 ** 31 - 2 * K) // (2 * K) // 256 * 256
    rows = {0, 1, M - 2, M - 1}
    for s in range(seam, M, seam):
        rows.update({s - 2, s - 1, s, s + 1})
    rows.update(np.random.default_rng(7902).choice(M, 24, replace=False).tolist())
    rows = np.array(sorted(rows))
    idx = torch.from_numpy(rows).cuda()
    xs = host_bits(x.index_select(0, idx)).reshape(len(rows), K)
    got = y_of(y.index_select(0, idx))
    del x, y
    torch.cuda.empty_cache()
    err = product_error(got, ref_product(xs, ref, N, K))
    assert err <= TOL, err


def test_gemm_weights_past_32bit_offsets_rejected():
    """Weights of 2^31 packed bytes or more (N*K/2 >= 2^31) are outside what the
    GEMM's 32-bit offsets reach: the call returns BNBX_E_UNSUPPORTED before any
    launch (checked with small buffers, which are never touched)."""
    import dequant_gemm_nf4_amd as B
    N, K = 65536, 65536
    q = T.empty_quantized((64, 64), True)
    st = q.state
    st.n = N * K
    x = torch.zeros((1, K), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((1, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.BnbxError) as e:
        B.bnbx_gemm_nf4(x, K, q.packed, st, 1, N, K, y, N)
    assert e.value.status == B.BNBX_E_UNSUPPORTED
    torch.cuda.synchronize()
