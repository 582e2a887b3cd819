"""GPU parity of bnbx_quantize_nf4_grouped (up to eight tensors quantized in
one call), through the C ABI: every tensor's packed codes, block codes,
group scales and mean must be bit-identical to the oracle's quantization of
that tensor alone (small ragged tensors, both quant types, no double quant
and both second-level maps), and to one bnbx_quantize_nf4 call per tensor on
the seven linears of a Llama-7B-shaped layer."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import assert_state_equal, dev_bf16

pytestmark = pytest.mark.gpu

RAGGED = [2, 66, 512 * 3 + 2, 64 * 1000 + 6, 4096, 64 * 256 * 5 + 64 * 7, 510, 64 * 256 * 3 + 2]


def state_of(q, dq, dq_map):
    out = {"packed": q.packed.cpu().numpy(), "double_quant": dq, "n": q.n, "blocksize": 64,
           "absmax": q.absmax.cpu().numpy()}
    if dq:
        out["dq_map"] = dq_map
        out["absmax2"] = q.absmax2.cpu().numpy()
        out["absmax_mean"] = np.float32(q.absmax_mean.cpu().numpy()[0])
    return out


@pytest.mark.parametrize("dq,dq_map", [(False, "linear"), (True, "linear"), (True, "dynamic")])
@pytest.mark.parametrize("qt", ["nf4", "fp4"])
@pytest.mark.parametrize("count", [1, 3, 8])
def test_grouped_ragged_against_oracle(count, qt, dq, dq_map):
    ns = RAGGED[:count]
    bits = [synth.normal_bf16((n,), 0.02, 14000 + 7 * i + n) for i, n in enumerate(ns)]
    print(f"grouped quantize ns={ns} {qt} dq={dq} {dq_map}", flush=True)
    qs = T.quantize_grouped([dev_bf16(b, (n,)) for b, n in zip(bits, ns)], dq, quant_type=qt,
                            dq_map=dq_map)
    torch.cuda.synchronize()
    for b, q in zip(bits, qs):
        ref = oracle.quantize(b, dq, quant_type=qt, dq_map=dq_map)
        assert_state_equal(state_of(q, dq, dq_map), ref)


def test_grouped_llama_layer_equals_single_calls():
    """q, k, v, o (4096x4096), gate, up (11008x4096) and down (4096x11008)
    quantized in one grouped call, each bit-identical to its own
    bnbx_quantize_nf4 call; q also against the oracle."""
    shapes = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    g = torch.Generator(device="cuda")
    ws = []
    for i, s in enumerate(shapes):
        g.manual_seed(14500 + i)
        ws.append((torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16))
    print("grouped quantize of a Llama-7B layer", flush=True)
    grouped = T.quantize_grouped(ws, True)
    singles = [T.quantize(w, True) for w in ws]
    torch.cuda.synchronize()
    for qg, qs in zip(grouped, singles):
        assert torch.equal(qg.packed, qs.packed)
        assert torch.equal(qg.absmax, qs.absmax)
        assert torch.equal(qg.absmax2.view(torch.int32), qs.absmax2.view(torch.int32))
        assert torch.equal(qg.absmax_mean.view(torch.int32), qs.absmax_mean.view(torch.int32))
    w0 = ws[0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()
    assert_state_equal(state_of(grouped[0], True, "linear"), oracle.quantize(w0, True))


def test_grouped_workspace_reuse_and_smaller_second_call():
    """One workspace for two grouped calls in a row, the second on fewer and
    smaller tensors: the slots and scales left by the first call must not
    leak into the second."""
    big = [synth.normal_bf16((64 * 256 * 9,), 0.02, 14600 + i) for i in range(4)]
    small = [synth.normal_bf16((n,), 0.02, 14700 + n) for n in (64 * 300, 130)]
    ws_bytes = T.bnbx_quantize_nf4_grouped_workspace_bytes([b.size for b in big], 64, 1)
    wsp = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    T.quantize_grouped([dev_bf16(b, (b.size,)) for b in big], True, workspace=wsp)
    qs = T.quantize_grouped([dev_bf16(b, (b.size,)) for b in small], True, workspace=wsp)
    torch.cuda.synchronize()
    for b, q in zip(small, qs):
        assert_state_equal(state_of(q, True, "linear"), oracle.quantize(b, True))
