"""The torch custom op and Linear4bit module without a GPU: registration,
shape inference through the fake implementation (meta tensors), argument
checks."""

import pytest
import torch

from dequant_gemm_nf4_amd import torch_ops  # noqa: F401  (registers bnbx::linear4bit)
from dequant_gemm_nf4_amd.torch_ops import Linear4bit


def test_op_is_registered():
    assert hasattr(torch.ops.bnbx, "linear4bit")
    schema = str(torch.ops.bnbx.linear4bit.default._schema)
    assert "out_features" in schema and "quant_type" in schema


@pytest.mark.parametrize("dq", [False, True])
@pytest.mark.parametrize("shape", [(1, 128), (5, 128), (2, 3, 128), (0, 128)])
def test_fake_shapes_on_meta(shape, dq):
    m = Linear4bit(128, 96, double_quant=dq, device="meta")
    assert m.packed.shape == (96 * 128 // 2,) and m.packed.dtype == torch.uint8
    assert m.absmax.dtype == (torch.int8 if dq else torch.float32)
    assert (m.absmax2 is None) == (not dq)
    x = torch.empty(*shape, dtype=torch.bfloat16, device="meta")
    y = m(x)
    assert y.shape == (*shape[:-1], 96) and y.dtype == torch.bfloat16


def test_fake_shapes_under_fake_tensor_mode():
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode():
        x = torch.empty(4, 256, dtype=torch.float16)
        p = torch.empty(64 * 256 // 2, dtype=torch.uint8)
        a = torch.empty(64 * 256 // 64, dtype=torch.float32)
        y = torch.ops.bnbx.linear4bit(x, p, a, None, None, 64, "fp4")
        assert y.shape == (4, 64) and y.dtype == torch.float16


def test_argument_checks():
    with pytest.raises(ValueError):
        Linear4bit(100, 32, device="meta")                 # in_features % 64
    with pytest.raises(ValueError):
        Linear4bit(128, 32, quant_type="int4", device="meta")
    with pytest.raises(ValueError):
        Linear4bit(128, 32, compute_dtype=torch.float32, device="meta")
    m = Linear4bit(128, 32, compute_dtype=torch.float16, device="meta")
    with pytest.raises(TypeError):
        m(torch.empty(1, 128, dtype=torch.bfloat16, device="meta"))
    with pytest.raises(ValueError):
        m.load_weight(torch.empty(32, 64, dtype=torch.bfloat16, device="meta"))
    assert "quant_type=nf4" in repr(m)


def test_backward_op_fake_shapes():
    assert hasattr(torch.ops.bnbx, "linear4bit_dx")
    dy = torch.empty(2, 3, 64, dtype=torch.bfloat16, device="meta")
    p = torch.empty(64 * 128 // 2, dtype=torch.uint8, device="meta")
    a = torch.empty(64 * 128 // 64, dtype=torch.float32, device="meta")
    dx = torch.ops.bnbx.linear4bit_dx(dy, p, a, None, None, 128, "nf4")
    assert dx.shape == (2, 3, 128)


def test_autograd_shapes_on_meta():
    m = Linear4bit(128, 64, device="meta")
    x = torch.empty(5, 128, dtype=torch.bfloat16, device="meta", requires_grad=True)
    y = m(x)
    (g,) = torch.autograd.grad(y, x, torch.empty_like(y))
    assert g.shape == x.shape and g.dtype == x.dtype


def test_lora_op_and_module_on_meta():
    from dequant_gemm_nf4_amd.torch_ops import Linear4bitLoRA
    assert hasattr(torch.ops.bnbx, "linear4bit_lora")
    schema = str(torch.ops.bnbx.linear4bit_lora.default._schema)
    assert "lora_a" in schema and "lora_b" in schema and "float scale" in schema
    m = Linear4bitLoRA(128, 96, rank=32, scale=2.0, device="meta")
    assert m.lora_a.shape == (32, 128) and m.lora_b.shape == (96, 32)
    y = m(torch.empty(2, 3, 128, dtype=torch.bfloat16, device="meta"))
    assert y.shape == (2, 3, 96) and y.dtype == torch.bfloat16
    assert "rank=32" in repr(m)


def test_lora_module_checks_and_no_backward():
    from dequant_gemm_nf4_amd.torch_ops import Linear4bitLoRA
    for r in (0, 8, 24, 272):
        with pytest.raises(ValueError):
            Linear4bitLoRA(128, 64, rank=r, device="meta")
    m = Linear4bitLoRA(128, 64, rank=16, device="meta")
    with pytest.raises(ValueError):
        m.load_adapter(torch.empty(16, 64, dtype=torch.bfloat16, device="meta"),
                       torch.empty(64, 16, dtype=torch.bfloat16, device="meta"))
    with pytest.raises(TypeError):
        m(torch.empty(1, 128, dtype=torch.float16, device="meta"))
    # inference only: a backward through the adapter layer fails loudly
    x = torch.empty(3, 128, dtype=torch.bfloat16, device="meta", requires_grad=True)
    with pytest.raises(RuntimeError, match="autograd"):
        m(x).sum().backward()
