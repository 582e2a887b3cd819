"""bnbx_quantize_nf4_noalloc (the quantize entry point that allocates nothing:
its double-quant scratch is a fixed device array of the library) against
bnbx_quantize_nf4 with a caller workspace, through the C ABI: packed codes,
int8 scales, group scales and mean bit for bit, on consecutive calls that
share the array (a large weight, then a smaller one, then the large one
again), for both quant types and both second-level maps, plus the oracle on
the same inputs."""

import numpy as np
import pytest
import torch

import dequant_gemm_nf4_amd as bnbx
import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import assert_state_equal, dev_bf16

pytestmark = pytest.mark.gpu


def noalloc_quantize(w, dq, quant_type, dq_map="linear"):
    q = T.empty_quantized(w.shape, dq, w.device, quant_type, dq_map=dq_map)
    bnbx.bnbx_quantize_nf4_noalloc(w, q.packed, q.state)
    return q


def host_state(q):
    out = {"packed": q.packed.cpu().numpy(), "double_quant": q.double_quant,
           "dq_map": q.dq_map}
    out["absmax"] = q.absmax.cpu().numpy()
    if q.double_quant:
        out["absmax2"] = q.absmax2.cpu().numpy()
        out["absmax_mean"] = np.float32(q.absmax_mean.cpu().numpy()[0])
    return out


@pytest.mark.parametrize("dq_map", ["linear", "dynamic"])
@pytest.mark.parametrize("quant_type", ["nf4", "fp4"])
def test_noalloc_equals_workspace_entry_point(quant_type, dq_map):
    shapes = [(4096, 4096), (1000, 512), (4096, 4096), (3, 2 * 64 * 257 + 10)]
    print(f"noalloc quantize, {quant_type}, {dq_map} map, shapes {shapes}", flush=True)
    for i, shape in enumerate(shapes):
        bits = synth.normal_bf16(shape, 0.02, 9100 + i)
        w = dev_bf16(bits, shape)
        for dq in (True, False):
            ref = T.quantize(w, dq, quant_type=quant_type, dq_map=dq_map)
            got = noalloc_quantize(w, dq, quant_type, dq_map)
            torch.cuda.synchronize()
            a, b = host_state(got), host_state(ref)
            assert_state_equal(a, b)
            if i < 2:
                assert_state_equal(a, oracle.quantize(bits, dq, quant_type=quant_type,
                                                      dq_map=dq_map))


def test_noalloc_rejects_past_its_scratch():
    q = T.empty_quantized((64, 64), True)
    st = q.state
    st.n = bnbx.BNBX_NOALLOC_MAX_WEIGHTS + 64
    w = torch.zeros(64 * 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bnbx.BnbxError) as e:
        bnbx.bnbx_quantize_nf4_noalloc(w, q.packed, st)
    assert e.value.status == bnbx.BNBX_E_WORKSPACE
    torch.cuda.synchronize()
