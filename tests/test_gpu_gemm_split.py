"""GPU parity of the GEMM's split-K path (bnbx_gemm_nf4 with the workspace
bnbx_gemm_nf4_workspace_bytes asks for: when the 256 x 256 output tiles fill
at most half of the compute units, K is split over up to four workgroups
per tile; when they fill more than one round but less than two, the tiles
past the first round are split; the fp32 partial tiles are added in split
order), through the C ABI:

* against the oracle's binary64 product (relative Frobenius <= 5e-3 per
  matrix, row and 32 x 32 tile) at the Llama-7B prefill shapes with N = 4096
  and at ragged shapes (rows and columns past a tile, K with a last split
  that is not a multiple of four blocks, four splits);
* beside the same call without a workspace (the tiles run whole): only the
  order of the fp32 additions differs, so the two agree to the bf16
  rounding of Y;
* both quant types, both compute types, both second-level maps and no
  double quant; results repeat bit for bit."""

import numpy as np
import pytest
import torch

import dequant_gemm_nf4_amd as bnbx
import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import dev_bf16, host_bits, product_error, upload_state

pytestmark = pytest.mark.gpu

TOL = 5e-3


def gemm_with(x, q, ws_bytes):
    M, K = x.shape
    N = q.shape[0]
    y = torch.empty(M, N, dtype=q.dtype, device=x.device)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    bnbx.bnbx_gemm_nf4(x, x.stride(0), q.packed, q.state, M, N, K, y, y.stride(0),
                       ws if ws_bytes else None, ws_bytes)
    return y


def check(M, N, K, seed, qt="nf4", dt="bf16", dq=True, dq_map="linear", splits=None,
          tail=None):
    need = bnbx.bnbx_gemm_nf4_workspace_bytes(M, N, K)
    assert need > 0, "shape does not split"
    tiles = -(-M // 256) * -(-N // 256)
    if splits is not None:
        assert need == splits * (tail if tail is not None else tiles) * 256 * 256 * 4
    w = synth.normal_bf16((N, K), 0.02, seed)
    xb = synth.normal_16((M, K), 1.0, seed + 1, dt)
    ref = oracle.quantize(w, dq, quant_type=qt, dq_map=dq_map)
    q = upload_state(ref, (N, K), dt)
    x = dev_bf16(xb, (M, K), dt)
    print(f"split GEMM {M}x{N}x{K} {qt} {dt} dq={dq} {dq_map} workspace={need}", flush=True)
    y_split = gemm_with(x, q, need)
    y_again = gemm_with(x, q, need)
    y_whole = gemm_with(x, q, 0)
    torch.cuda.synchronize()
    got = oracle.bits_to_f32(host_bits(y_split), dt).astype(np.float64).reshape(M, N)
    want = oracle.dequant_matmul_ref(xb, ref["packed"], ref, N, K, dt)
    err = product_error(got, want)
    assert err <= TOL, err
    assert torch.equal(y_split, y_again)
    whole = oracle.bits_to_f32(host_bits(y_whole), dt).astype(np.float64).reshape(M, N)
    # the two paths round the same fp32 sum computed in a different order:
    # within a few bf16 units of each other, far inside the product bound
    assert oracle.rel_frobenius(got, whole) <= 2e-3


def test_split_llama_attention_shape():
    """q/k/v/o at prefill: 2048 x 4096 x 4096, 128 tiles, two splits."""
    check(2048, 4096, 4096, 15000, splits=2)


def test_split_llama_down_shape():
    """down projection at prefill: 2048 x 4096 x 11008 (172 blocks per row:
    splits of 88 and 84 steps)."""
    check(2048, 4096, 11008, 15010, splits=2)


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16"), ("nf4", "f16")])
@pytest.mark.parametrize("dq,dq_map", [(False, "linear"), (True, "linear"), (True, "dynamic")])
def test_split_ragged(qt, dt, dq, dq_map):
    """300 x 500 x 4096: 4 tiles, four splits of 16 steps; rows and columns
    past the tiles."""
    check(300, 500, 4096, 15020, qt=qt, dt=dt, dq=dq, dq_map=dq_map, splits=4)


def test_split_last_range_not_a_multiple_of_four():
    """K = 2112 (33 blocks, per-step block codes): splits of 20 and 13 steps."""
    check(260, 300, 2112, 15030, splits=2)


def test_split_one_row():
    """M = 1 through the GEMM: one row tile, every split."""
    check(1, 1000, 8192, 15040, splits=4)


def test_split_tail_llama_gate_up_shape():
    """gate/up at prefill: 2048 x 11008 x 4096, 344 tiles: 256 whole, the
    88 past the first round split in two."""
    check(2048, 11008, 4096, 15050, splits=2, tail=88)


@pytest.mark.parametrize("qt,dt,dq_map", [("nf4", "bf16", "linear"), ("fp4", "f16", "dynamic")])
def test_split_tail_ragged(qt, dt, dq_map):
    """2500 x 7400 x 2048: 290 tiles (ragged last row and column of tiles),
    34 tail tiles split in two."""
    check(2500, 7400, 2048, 15060, qt=qt, dt=dt, dq_map=dq_map, splits=2, tail=34)
