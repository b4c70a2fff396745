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


def x_like(dtype=torch.bfloat16, *shape):
    return torch.zeros(*(shape or (2, 3, 64)), dtype=dtype)


def ops_in(gm):
    return [n for n in gm.graph.nodes if n.op == "call_function" and n.target is OP]


def test_pass_fuses_the_kernel_chains_and_keeps_the_rest():
    _, gm = traced()
    n = tops.fuse_linear_epilogues(gm, (x_like(),))
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
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 4, 32),
                                           x_like(torch.bfloat16, 4, 16))) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["act"] == "none" and f.kwargs["alpha"] == 0.5
    assert f.kwargs["residual"].name == "x"
    assert not [n for n in gm.graph.nodes if n.op == "call_function" and n.target in
                (operator.mul, operator.add)]


def test_pass_skips_fp32_weights_and_plain_linears():
    _, gm = traced(torch.float32)
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.float32),)) == 0  # bf16 / fp16 weights only

    class Plain(nn.Module):
        def __init__(self):
            super().__init__()
            self.l = nn.Linear(16, 16)

        def forward(self, x):
            return self.l(x)

    gm = torch.fx.symbolic_trace(Plain().to(torch.bfloat16))
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 2, 16),)) == 0


class AfterAct(nn.Module):
    """A [N] vector added after the activation is not a residual: the kernel
    would read M x N values from it."""

    def __init__(self):
        super().__init__()
        self.fc = nn.Linear(32, 16)
        self.b2 = nn.Parameter(torch.zeros(16))

    def forward(self, x, r):
        return F.gelu(self.fc(x), approximate="tanh") + self.b2 + r


def test_pass_skips_broadcast_residual():
    gm = torch.fx.symbolic_trace(AfterAct().to(torch.bfloat16))
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 4, 32),
                                           x_like(torch.bfloat16, 4, 16))) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["act"] == "gelu_tanh" and f.kwargs["residual"] is None
    adds = [n for n in gm.graph.nodes if n.op == "call_function" and n.target is operator.add]
    assert len(adds) == 2                        # + b2 and + r stay in the graph


def test_pass_skips_residual_of_another_dtype_or_unknown_shape():
    class Down(nn.Module):
        def __init__(self):
            super().__init__()
            self.down = nn.Linear(32, 16)

        def forward(self, h, x):
            return self.down(h) * 0.5 + x

    m = Down().to(torch.bfloat16)
    gm = torch.fx.symbolic_trace(m)
    # fp32 residual: the add promotes to fp32; the kernel reads bf16.
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 4, 32),
                                           x_like(torch.float32, 4, 16))) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["residual"] is None and f.kwargs["alpha"] == 0.5
    # No example inputs and no metadata: the residual's shape is unknown.
    gm = torch.fx.symbolic_trace(m)
    assert tops.fuse_linear_epilogues(gm) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["residual"] is None
    # A residual that broadcasts over the tokens ([1, 16] against [4, 16]).
    gm = torch.fx.symbolic_trace(m)
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 4, 32),
                                           x_like(torch.bfloat16, 1, 16))) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["residual"] is None


class PagesBlock(nn.Module):
    """The forward pass the pages fuse: gelu(matmul(x, w) + b) with the tanh
    GELU, w a [K, N] weight ("Совместная работа Helion и TorchInductor",
    sections on the TorchInductor integration and on checking the fusion)."""

    def __init__(self, K=64, N=48, op="matmul"):
        super().__init__()
        self.w = nn.Parameter(torch.randn(K, N))
        self.b = nn.Parameter(torch.randn(N))
        self.op = op

    def forward(self, x):
        if self.op == "matmul":
            y = torch.matmul(x, self.w)
        elif self.op == "at":
            y = x @ self.w
        else:
            y = torch.mm(x, self.w)
        return F.gelu(y + self.b, approximate="tanh")


@pytest.mark.parametrize("op", ["matmul", "at", "mm"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_pass_fuses_the_pages_matmul_chain(op, dtype):
    m = PagesBlock(op=op).to(dtype)
    gm = torch.fx.symbolic_trace(m)
    assert tops.fuse_linear_epilogues(gm, (x_like(dtype, 5, 64),)) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["act"] == "gelu_tanh" and f.kwargs["alpha"] == 1.0
    assert f.kwargs["quant"] == ("fp16" if dtype == torch.float16 else "bf16")
    w_nk = getattr(gm, f.args[1].target)
    assert w_nk.shape == (48, 64) and torch.equal(w_nk, m.w.detach().t())
    assert f.kwargs["bias"].target == "b"
    left = {n.target for n in gm.graph.nodes if n.op == "call_function"}
    assert not left & {torch.matmul, operator.matmul, torch.mm, operator.add, F.gelu}


def test_pass_fuses_the_aten_pattern_of_make_fx():
    # The same chain as aten.mm -> aten.add -> aten.gelu(approximate="tanh"),
    # the form an Inductor joint-graph pattern sees; make_fx keeps the
    # parameters as attributes and records fake values in the metadata.
    from torch.fx.experimental.proxy_tensor import make_fx
    m = PagesBlock(op="mm").to(torch.bfloat16)
    gm = make_fx(m)(x_like(torch.bfloat16, 5, 64))
    targets = {n.target for n in gm.graph.nodes if n.op == "call_function"}
    assert torch.ops.aten.mm.default in targets and torch.ops.aten.gelu.default in targets
    assert tops.fuse_linear_epilogues(gm) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["act"] == "gelu_tanh" and f.kwargs["bias"] is not None


def test_pass_treats_a_full_shape_addend_as_residual_before_the_activation():
    # matmul(x, w) + R with R of the full output shape is no bias: the kernel
    # adds a residual after its activation, so only matmul + R is fused and
    # the GELU stays a separate op.  A [1, N] addend is neither.
    class Full(PagesBlock):
        def forward(self, x):
            return F.gelu(torch.matmul(x, self.w) + self.rb, approximate="tanh")

    m = Full()
    m.rb = nn.Parameter(torch.randn(5, 48))
    gm = torch.fx.symbolic_trace(m.to(torch.bfloat16))
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 5, 64),)) == 1
    (f,) = ops_in(gm)
    assert f.kwargs["act"] == "none" and f.kwargs["bias"] is None
    assert f.kwargs["residual"].target == "rb"
    assert [n for n in gm.graph.nodes if n.op == "call_function" and n.target is F.gelu]
    m.rb = nn.Parameter(torch.randn(1, 48))
    gm = torch.fx.symbolic_trace(m.to(torch.bfloat16))
    assert tops.fuse_linear_epilogues(gm, (x_like(torch.bfloat16, 5, 64),)) == 0


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
    y = torch.ops.lingemm.scaled_linear_dynamic(x, wq, torch.empty(32, device="meta"))
    assert y.shape == (3, 5, 32) and y.dtype == torch.bfloat16
    with pytest.raises(Exception):
        torch.ops.lingemm.scaled_linear(x, torch.empty(96, 63, dtype=torch.bfloat16, device="meta"))


@pytest.mark.parametrize("bad", ["broadcast_residual", "fp32_residual", "bias_shape",
                                 "bias_dtype", "scale_a_count", "scale_b_dtype", "x_dtype"])
def test_op_rejects_bad_operands_on_meta(bad):
    x = torch.empty(4, 64, dtype=torch.bfloat16, device="meta")
    w = torch.empty(32, 64, dtype=torch.bfloat16, device="meta")
    kw = dict(quant="bf16")
    if bad == "broadcast_residual":
        kw["residual"] = torch.empty(32, dtype=torch.bfloat16, device="meta")
    elif bad == "fp32_residual":
        kw["residual"] = torch.empty(4, 32, dtype=torch.float32, device="meta")
    elif bad == "bias_shape":
        kw["bias"] = torch.empty(1, 32, dtype=torch.bfloat16, device="meta")
    elif bad == "bias_dtype":
        kw["bias"] = torch.empty(32, dtype=torch.float32, device="meta")
    elif bad in ("scale_a_count", "scale_b_dtype"):
        x = torch.empty(4, 64, dtype=torch.float8_e4m3fn, device="meta")
        w = torch.empty(32, 64, dtype=torch.float8_e4m3fn, device="meta")
        kw = dict(quant="fp8_dynamic", scale_a=torch.empty(4, device="meta"),
                  scale_b=torch.empty(32, device="meta"))
        if bad == "scale_a_count":
            kw["scale_a"] = torch.empty(1, device="meta")
        else:
            kw["scale_b"] = torch.empty(32, dtype=torch.float16, device="meta")
    elif bad == "x_dtype":
        x = torch.empty(4, 64, dtype=torch.float16, device="meta")
    with pytest.raises(ValueError):
        torch.ops.lingemm.scaled_linear(x, w, **kw)


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
