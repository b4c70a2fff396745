"""The PyTorch integration on the CPU: the FX pass rewrites the chains the
kernel can run (linear -> tanh-GELU / SiLU / ReLU -> * alpha -> + residual)
into torch.ops.lingemm.scaled_linear and leaves the rest alone, and the
operator's fake implementation gives shapes and dtypes without memory."""
import operator

import pytest
import torch
import torch.nn as nn
import torch.nn.functional as F

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
import epilogue_scaled_gemm_amd.torch_ops as tops  # noqa: E402

OP = torch.ops.lingemm.scaled_linear.default


class Block(nn.Module):
    """Decoder-block shaped MLP: up-projection + tanh-GELU, down-projection
    scaled by 0.5 plus the residual, a SiLU branch, an erf-GELU branch (not
    fusable), and a linear whose output has two users (not fusable)."""

    def __init__(self, d=64, h=128):
        super().__init__()
        self.up = nn.Linear(d, h)
        self.act = nn.GELU(approximate="tanh")
        self.down = nn.Linear(h, d)
        self.gate = nn.Linear(d, d, bias=False)
        self.erf = nn.Linear(d, d)
        self.shared = nn.Linear(d, d)
        self.w = nn.Parameter(torch.randn(d, d))

    def forward(self, x):
        y = self.down(self.act(self.up(x))) * 0.5 + x
        g = F.silu(self.gate(y))
        e = F.gelu(self.erf(y))                      # erf form: not the kernel's GELU
        s = self.shared(y)
        t = torch.relu(F.linear(g, self.w)) + s       # functional linear + relu + residual
        return e + s + t


def traced(dtype=torch.bfloat16):
    m = Block().to(dtype)
    return m, torch.fx.symbolic_trace(m)


def ops_in(gm):
    return [n for n in gm.graph.nodes if n.op == "call_function" and n.target is OP]


def test_pass_fuses_the_kernel_chains_and_keeps_the_rest():
    _, gm = traced()
    n = tops.fuse_linear_epilogues(gm)
    fused = ops_in(gm)
    assert n == len(fused) == 4
    by_act = {f.kwargs["act"]: f for f in fused}
    assert set(by_act) == {"gelu_tanh", "none", "silu", "relu"}
    # up -> tanh-GELU (no alpha, no residual)
    assert by_act["gelu_tanh"].kwargs["alpha"] == 1.0 and by_act["gelu_tanh"].kwargs["residual"] is None
    # down -> * 0.5 -> + x (no activation)
    assert by_act["none"].kwargs["alpha"] == 0.5 and by_act["none"].kwargs["residual"].name == "x"
    # gate -> SiLU (no bias)
    assert by_act["silu"].kwargs["bias"] is None
    # functional linear -> relu -> + s (the residual is the other operand)
    assert by_act["relu"].kwargs["residual"] is not None
    mods = {n.target for n in gm.graph.nodes if n.op == "call_module"}
    assert "erf" in mods and "shared" in mods        # erf GELU and two-user linear stay
    assert not {"up", "act", "down", "gate"} & mods
    erf_users = [n for n in gm.graph.nodes if n.op == "call_function" and n.target is F.gelu]
    assert len(erf_users) == 1


def test_pass_fuses_scale_and_residual_without_activation():
    class Down(nn.Module):
        def __init__(self):
            super().__init__()
            self.down = nn.Linear(32, 16)

        def forward(self, h, x):
            return self.down(h) * 0.5 + x

    gm = torch.fx.symbolic_trace(Down().to(torch.bfloat16))
    assert tops.fuse_linear_epilogues(gm) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["act"] == "none" and f.kwargs["alpha"] == 0.5
    assert f.kwargs["residual"].name == "x"
    assert not [n for n in gm.graph.nodes if n.op == "call_function" and n.target in
                (operator.mul, operator.add)]


def test_pass_skips_fp32_weights_and_plain_linears():
    _, gm = traced(torch.float32)
    assert tops.fuse_linear_epilogues(gm) == 0      # the kernel takes bf16 / fp16 weights

    class Plain(nn.Module):
        def __init__(self):
            super().__init__()
            self.l = nn.Linear(16, 16)

        def forward(self, x):
            return self.l(x)

    gm = torch.fx.symbolic_trace(Plain().to(torch.bfloat16))
    assert tops.fuse_linear_epilogues(gm) == 0


def test_fake_implementation_gives_shape_and_dtype():
    x = torch.empty(3, 5, 64, dtype=torch.bfloat16, device="meta")
    w = torch.empty(96, 64, dtype=torch.bfloat16, device="meta")
    y = torch.ops.lingemm.scaled_linear(x, w, quant="bf16", act="gelu_tanh")
    assert y.shape == (3, 5, 96) and y.dtype == torch.bfloat16 and y.device.type == "meta"
    y = torch.ops.lingemm.scaled_linear(x.half(), w.half(), quant="fp16")
    assert y.dtype == torch.float16
    xq = torch.empty(7, 64, dtype=torch.float8_e4m3fn, device="meta")
    wq = torch.empty(32, 64, dtype=torch.float8_e4m3fn, device="meta")
    s = torch.empty(7, device="meta")
    y = torch.ops.lingemm.scaled_linear(xq, wq, scale_a=s, scale_b=torch.empty(32, device="meta"),
                                        quant="fp8_dynamic")
    assert y.shape == (7, 32) and y.dtype == torch.bfloat16
    y = torch.ops.lingemm.scaled_linear_dynamic(x, wq, torch.empty(96, device="meta"))
    assert y.shape == (3, 5, 32) and y.dtype == torch.bfloat16
    with pytest.raises(Exception):
        torch.ops.lingemm.scaled_linear(x, torch.empty(96, 63, dtype=torch.bfloat16, device="meta"))


def test_grouped_fake_implementation():
    x = torch.empty(40, 64, dtype=torch.bfloat16, device="meta")
    w = torch.empty(8, 96, 64, dtype=torch.bfloat16, device="meta")
    off = torch.empty(9, dtype=torch.int32, device="meta")
    y = torch.ops.lingemm.scaled_linear_grouped(x, w, off, quant="bf16", act="silu")
    assert y.shape == (40, 96) and y.dtype == torch.bfloat16 and y.device.type == "meta"
    with pytest.raises(Exception):
        torch.ops.lingemm.scaled_linear_grouped(x, w, torch.empty(8, dtype=torch.int32,
                                                                  device="meta"))


def test_grouped_dynamic_fake_implementation():
    x = torch.empty(40, 256, dtype=torch.bfloat16, device="meta")
    w = torch.empty(4, 96, 256, dtype=torch.float8_e4m3fn, device="meta")
    off = torch.empty(5, dtype=torch.int32, device="meta")
    y = torch.ops.lingemm.scaled_linear_grouped_dynamic(x, w, off, torch.empty(4, 96, device="meta"))
    assert y.shape == (40, 96) and y.dtype == torch.bfloat16


def test_grouped_dynamic_rejects_unquantised_modes():
    # The mode check comes before any device work, so CPU tensors suffice.
    x = torch.empty(4, 256, dtype=torch.bfloat16)
    w = torch.empty(2, 8, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tops.scaled_linear_grouped_dynamic(x, w, torch.zeros(3, dtype=torch.int32),
                                           torch.ones(2, 8), quant="bf16")
