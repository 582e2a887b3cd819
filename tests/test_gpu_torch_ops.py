"""GPU checks of torch.ops.bnbx.linear4bit and Linear4bit: the module's
output against the oracle (rel. Frobenius <= 5e-3), the same output from a
torch.compile(fullgraph=True) graph and from a captured HIP graph, and
torch.library.opcheck of the op."""

import numpy as np
import pytest
import torch

import oracle
import synth
from dequant_gemm_nf4_amd.torch_ops import Linear4bit, Linear4bitLoRA
from tests.gpu_helpers import TORCH_DTYPE, dev_bf16, host_bits, product_error

pytestmark = pytest.mark.gpu

TOL = 5e-3


def make(N, K, qt, dt, dq=True, seed=9900, dq_map="linear"):
    w = synth.normal_bf16((N, K), 0.02, seed)
    m = Linear4bit(K, N, quant_type=qt, double_quant=dq, compute_dtype=TORCH_DTYPE[dt],
                   dq_map=dq_map)
    m.load_weight(dev_bf16(w, (N, K)))
    torch.cuda.synchronize()
    return w, m


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("dq,dq_map", [(False, "linear"), (True, "linear"), (True, "dynamic")])
@pytest.mark.parametrize("lead", [(1,), (5,), (2, 32)])
def test_module_against_oracle(qt, dt, dq, dq_map, lead):
    N, K = 384, 1024
    w, m = make(N, K, qt, dt, dq, dq_map=dq_map)
    ref = oracle.quantize(w, dq, quant_type=qt, dq_map=dq_map)
    assert np.array_equal(m.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(m.absmax.cpu().numpy(), ref["absmax"])
    M = int(np.prod(lead))
    xb = synth.normal_16((M, K), 1.0, 9901 + M, dt)
    x = dev_bf16(xb, (*lead, K), dt)
    y = m(x)
    torch.cuda.synchronize()
    assert y.shape == (*lead, N) and y.dtype == TORCH_DTYPE[dt]
    got = oracle.bits_to_f32(host_bits(y), dt).astype(np.float64).reshape(M, N)
    err = product_error(got, oracle.dequant_matmul_ref(xb, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


def test_module_dequantize_and_from_linear():
    N, K = 128, 256
    lin = torch.nn.Linear(K, N, bias=False, device="cuda", dtype=torch.bfloat16)
    m = Linear4bit.from_linear(lin, quant_type="nf4")
    wb = host_bits(lin.weight)
    ref = oracle.quantize(wb, True)
    assert np.array_equal(host_bits(m.dequantize()), oracle.dequantize(ref["packed"], ref))


class TwoLayers(torch.nn.Module):
    def __init__(self, a, b):
        super().__init__()
        self.a, self.b = a, b

    def forward(self, x):
        return self.b(self.a(x))


@pytest.mark.parametrize("M", [1, 40])
def test_torch_compile_fullgraph_equals_eager(M):
    K, H, N = 512, 256, 192
    _, a = make(H, K, "nf4", "bf16", seed=9910)
    _, b = make(N, H, "nf4", "bf16", seed=9911)
    net = TwoLayers(a, b)
    x = dev_bf16(synth.normal_16((M, K), 1.0, 9912), (M, K))
    eager = net(x)
    compiled = torch.compile(net, fullgraph=True, backend="aot_eager")
    out = compiled(x)
    torch.cuda.synchronize()
    assert torch.equal(out, eager)


def test_opcheck():
    N, K = 64, 256
    _, m = make(N, K, "fp4", "f16", dq=True, seed=9920)
    x = dev_bf16(synth.normal_16((3, K), 1.0, 9921, "f16"), (3, K), "f16")
    torch.library.opcheck(torch.ops.bnbx.linear4bit.default,
                          (x, m.packed, m.absmax, m.absmax2, m.absmax_mean, N, "fp4"))


def test_captured_graph_replays_match_eager():
    N, K = 256, 1024
    _, m = make(N, K, "nf4", "bf16", seed=9930)
    x = dev_bf16(synth.normal_16((4, K), 1.0, 9931), (4, K))
    eager = m(x)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m(x)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y = m(x)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)


@pytest.mark.parametrize("qt,dt,dq_map", [("nf4", "bf16", "linear"), ("fp4", "f16", "linear"),
                                         ("nf4", "bf16", "dynamic")])
def test_backward_against_oracle(qt, dt, dq_map):
    """x.grad of sum(g * Linear4bit(x)) is g . W_hat (the bnbx_gemm_nf4_dx
    kernel through the op's autograd), against the oracle."""
    N, K, M = 256, 512, 48
    w, m = make(N, K, qt, dt, True, seed=9940, dq_map=dq_map)
    ref = oracle.quantize(w, True, quant_type=qt, dq_map=dq_map)
    x = dev_bf16(synth.normal_16((M, K), 1.0, 9941, dt), (M, K), dt).requires_grad_(True)
    gb = synth.normal_16((M, N), 1.0, 9942, dt)
    m(x).backward(dev_bf16(gb, (M, N), dt))
    torch.cuda.synchronize()
    got = oracle.bits_to_f32(host_bits(x.grad), dt).astype(np.float64).reshape(M, K)
    err = product_error(got, oracle.dequant_matmul_dx_ref(gb, ref["packed"], ref, N, K, dt))
    assert err <= TOL, err


def test_compiled_backward_equals_eager():
    K, H, N, M = 512, 256, 192, 40
    _, a = make(H, K, "nf4", "bf16", seed=9950)
    _, b = make(N, H, "nf4", "bf16", seed=9951)
    net = TwoLayers(a, b)
    xb = synth.normal_16((M, K), 1.0, 9952)
    g = dev_bf16(synth.normal_16((M, N), 1.0, 9953), (M, N))
    x1 = dev_bf16(xb, (M, K)).requires_grad_(True)
    net(x1).backward(g)
    x2 = dev_bf16(xb, (M, K)).requires_grad_(True)
    torch.compile(net, fullgraph=True, backend="aot_eager")(x2).backward(g)
    torch.cuda.synchronize()
    assert torch.equal(x1.grad, x2.grad)


def test_opcheck_with_grad():
    N, K = 128, 256
    _, m = make(N, K, "nf4", "bf16", dq=True, seed=9960)
    x = dev_bf16(synth.normal_16((3, K), 1.0, 9961), (3, K)).requires_grad_(True)
    torch.library.opcheck(torch.ops.bnbx.linear4bit.default,
                          (x, m.packed, m.absmax, m.absmax2, m.absmax_mean, N, "nf4"))
    dy = dev_bf16(synth.normal_16((3, N), 1.0, 9962), (3, N))
    torch.library.opcheck(torch.ops.bnbx.linear4bit_dx.default,
                          (dy, m.packed, m.absmax, m.absmax2, m.absmax_mean, K, "nf4"))


@pytest.mark.parametrize("qt,dt", [("nf4", "bf16"), ("fp4", "f16")])
@pytest.mark.parametrize("lead", [(3,), (2, 160)])
def test_lora_module_against_oracle(qt, dt, lead):
    """Linear4bitLoRA: Y = X . W_hat^T + s . rnd(X . A^T) . B^T against the
    oracle; with a zero adapter it equals the plain layer (bit for bit where
    both run the GEMM)."""
    N, K, r, s = 256, 512, 32, 0.5
    w = synth.normal_bf16((N, K), 0.02, 9950)
    m = Linear4bitLoRA(K, N, rank=r, scale=s, quant_type=qt, compute_dtype=TORCH_DTYPE[dt])
    m.load_weight(dev_bf16(w, (N, K)))
    M = int(np.prod(lead))
    xb = synth.normal_16((M, K), 1.0, 9951, dt)
    x = dev_bf16(xb, (*lead, K), dt)
    plain = Linear4bit(K, N, quant_type=qt, compute_dtype=TORCH_DTYPE[dt])
    plain.load_weight(dev_bf16(w, (N, K)))
    y0, yp = m(x), plain(x)
    if M > 16:   # both run the GEMM: a zero adapter adds exact zeros
        assert torch.equal(y0.view(torch.int16), yp.view(torch.int16))
    else:        # the plain layer runs the GEMV at up to 16 rows
        assert product_error(y0.float().cpu().numpy().astype(np.float64).reshape(M, N),
                             yp.float().cpu().numpy().astype(np.float64).reshape(M, N)) <= TOL
    a = synth.normal_16((r, K), 0.02, 9952, dt)
    b = synth.normal_16((N, r), 0.05, 9953, dt)
    m.load_adapter(dev_bf16(a, (r, K), dt), dev_bf16(b, (N, r), dt))
    y = m(x)
    torch.cuda.synchronize()
    assert y.shape == (*lead, N)
    got = oracle.bits_to_f32(host_bits(y), dt).astype(np.float64).reshape(M, N)
    ref = oracle.quantize(w, True, quant_type=qt)
    xa = oracle.lora_down_ref(xb, a, s, M, K, dt)
    b64 = oracle.bits_to_f32(b, dt).astype(np.float64).reshape(N, r)
    base = oracle.dequant_matmul_ref(xb, ref["packed"], ref, N, K, dt)
    want = base + xa @ b64.T
    assert product_error(got, want) <= TOL
    assert oracle.rel_frobenius(base, want) > 10 * TOL


def test_lora_module_compiled_equals_eager():
    N, K, r = 192, 256, 16
    w = synth.normal_bf16((N, K), 0.02, 9960)
    m = Linear4bitLoRA(K, N, rank=r, scale=2.0)
    m.load_weight(dev_bf16(w, (N, K)))
    m.load_adapter(dev_bf16(synth.normal_16((r, K), 0.02, 9961, "bf16"), (r, K)),
                   dev_bf16(synth.normal_16((N, r), 0.05, 9962, "bf16"), (N, r)))
    x = dev_bf16(synth.normal_16((40, K), 1.0, 9963, "bf16"), (40, K))
    eager = m(x)
    compiled = torch.compile(m, fullgraph=True, backend="aot_eager")(x)
    torch.cuda.synchronize()
    assert torch.equal(eager.view(torch.int16), compiled.view(torch.int16))
