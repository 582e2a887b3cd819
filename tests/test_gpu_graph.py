"""The whole path captured in a HIP graph (as the benchmark replays it):
every replay, with eager work and synchronisations in between, must equal
the eager result bit for bit (all kernels are deterministic: integer atomics
only, fixed reduction orders)."""

import pytest
import torch

import synth
from dequant_gemm_nf4_amd import tensors as T
from tests.gpu_helpers import dev_bf16

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    N, K = 4096, 4096
    w = dev_bf16(synth.normal_bf16((N, K), 0.02, 8100), (N, K))
    x1 = dev_bf16(synth.normal_bf16((1, K), 1.0, 8101), (1, K))
    xm = dev_bf16(synth.normal_bf16((160, K), 1.0, 8102), (160, K))
    q = T.empty_quantized((N, K), True)
    ws = T.workspace_for(N * K, True)
    deq = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")
    ym = torch.empty(160, N, dtype=torch.bfloat16, device="cuda")

    def path():
        T.quantize(w, True, out=q, workspace=ws)
        T.dequantize(q, out=deq)
        T.gemv(x1, q, out=y1)
        T.gemm(xm, q, out=ym)

    path()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q.packed, q.absmax, q.absmax2, q.absmax_mean, deq, y1, ym)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        path()
    for rep in range(4):
        for t in (q.packed, q.absmax, q.absmax2, q.absmax_mean, deq, y1, ym):
            t.zero_()
        ws.fill_(0xAB)                      # scratch must not leak between calls
        g.replay()
        torch.cuda.synchronize()
        got = (q.packed, q.absmax, q.absmax2, q.absmax_mean, deq, y1, ym)
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"
        path()                              # eager work between replays
        torch.cuda.synchronize()
