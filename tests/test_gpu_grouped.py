"""GPU parity of bnbx_gemv_nf4_grouped (up to four weights that multiply the
same X, one launch for M <= 4), through the C ABI:

* against the oracle's binary64 product of each weight (relative Frobenius
  <= 5e-3 per matrix, row and 32 x 32 tile);
* bit for bit against one bnbx_gemv_nf4 call per weight where both plan the
  same lanes and chunks (row-wise code reads: every row's arithmetic is the
  same, only the rows' placement on the GPU differs);
* the Llama-7B groupings (q, k, v: 3 x 4096x4096; gate, up: 2 x 11008x4096),
  uneven row counts, both second-level maps and no double quant, both quant
  types and compute types, every M from 1 to 16 on a small group."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import dev_bf16, host_bits, product_error, upload_state

pytestmark = pytest.mark.gpu

TOL = 5e-3


def make_group(Ns, K, seed, dq=True, dq_map="linear", qt="nf4", dt="bf16"):
    refs, qs = [], []
    for i, N in enumerate(Ns):
        w = synth.normal_bf16((N, K), 0.02, seed + 17 * i)
        ref = oracle.quantize(w, dq, quant_type=qt, dq_map=dq_map)
        refs.append(ref)
        qs.append(upload_state(ref, (N, K), dt))
    return refs, qs


def check(Ns, K, M, seed, exact=True, **kw):
    dt = kw.get("dt", "bf16")
    refs, qs = make_group(Ns, K, seed, **kw)
    xb = synth.normal_16((M, K), 1.0, seed + 5, dt)
    x = dev_bf16(xb, (M, K), dt)
    print(f"grouped GEMV Ns={Ns} K={K} M={M} {kw}", flush=True)
    ys = T.gemv_grouped(x, qs)
    singles = [T.gemv(x, q) for q in qs]
    torch.cuda.synchronize()
    for N, ref, y, y1 in zip(Ns, refs, ys, singles):
        got = oracle.bits_to_f32(host_bits(y), dt).astype(np.float64).reshape(M, N)
        err = product_error(got, oracle.dequant_matmul_ref(xb, ref["packed"], ref, N, K, dt))
        assert err <= TOL, (N, err)
        if exact:
            assert np.array_equal(host_bits(y), host_bits(y1)), N


@pytest.mark.parametrize("M", [1, 4])
def test_grouped_qkv(M):
    check([4096, 4096, 4096], 4096, M, 13000)


@pytest.mark.parametrize("M", [1, 2])
def test_grouped_gate_up(M):
    check([11008, 11008], 4096, M, 13100)


def test_grouped_more_rows_than_one_pass():
    """3 x 11008 rows at K = 4096: more rows than one grouped pass takes, so
    the call splits the items (here into single-weight launches)."""
    check([11008, 11008, 11008], 4096, 1, 13050)


@pytest.mark.parametrize("dq,dq_map", [(False, "linear"), (True, "linear"), (True, "dynamic")])
@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
def test_grouped_uneven_rows(dq, dq_map, qt, dt):
    check([300, 17, 1000, 64], 512, 1, 13200, dq=dq, dq_map=dq_map, qt=qt, dt=dt)


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_grouped_every_m(M):
    check([256, 96, 320], 1024, M, 13300 + M)


@pytest.mark.parametrize("count", [1, 2, 3, 4])
def test_grouped_counts(count):
    check([520, 130, 64, 333][:count], 2048, 3, 13400 + count)


def test_grouped_split_into_sub_groups():
    """Items that fit one pass only in part: 4096 + 4096 rows in one launch,
    then 11008 + 300 in another (or alone), all checked."""
    check([4096, 4096, 11008, 300], 4096, 1, 13450)


def test_grouped_per_lane_codes():
    """K/64 not a multiple of 4 (per-lane code reads) and K > 16384 (per-lane
    reads, at most three chunks per lane): checked against the oracle only,
    the plans of the single calls may differ."""
    check([100, 50], 4160, 2, 13500, exact=False)
    check([40, 30], 20480, 1, 13600, exact=False, dq_map="dynamic")
    check([40, 30], 32768, 1, 13700, exact=False)


def test_grouped_strided_outputs():
    """Y of each weight written into a column slice of one wider buffer."""
    K, M = 1024, 3
    Ns = [128, 64]
    refs, qs = make_group(Ns, K, 13800)
    xb = synth.normal_16((M, K), 1.0, 13801)
    x = dev_bf16(xb, (M, K))
    big = torch.zeros(M, 256, dtype=torch.bfloat16, device="cuda")
    outs = [big[:, 0:128], big[:, 128:192]]
    T.gemv_grouped(x, qs, outs=outs)
    torch.cuda.synchronize()
    for N, ref, y in zip(Ns, refs, outs):
        got = oracle.bits_to_f32(host_bits(y), "bf16").astype(np.float64).reshape(M, N)
        assert product_error(got, oracle.dequant_matmul_ref(xb, ref["packed"], ref, N, K)) <= TOL
    assert torch.count_nonzero(big[:, 192:]) == 0
