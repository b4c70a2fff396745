"""The PyTorch integration on the GPU: the FX-rewritten blocks (a decoder
MLP, and the pages' gelu(matmul(x, w) + b) forward pass) with every fused
call checked against the oracle, torch.library.opcheck of the custom
operators, separate workspaces per stream, and HIP-graph capture of the
decode path replayed several times with eager work in between."""
import numpy as np
import pytest
import torch
import torch.nn as nn
import torch.nn.functional as F

import oracle
import synth
from gpu_util import assert_close, dev, sample_positions

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
import epilogue_scaled_gemm_amd.torch_ops as tops  # noqa: E402

pytestmark = pytest.mark.gpu


class MLP(nn.Module):
    def __init__(self, d=512, h=1024):
        super().__init__()
        self.up = nn.Linear(d, h)
        self.act = nn.GELU(approximate="tanh")
        self.down = nn.Linear(h, d)

    def forward(self, x):
        return self.down(self.act(self.up(x))) * 0.5 + x


def codes16(t):
    """A 16-bit CUDA tensor -> its bit patterns as numpy uint16 (for the oracle)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def fused_outputs(gm, *args):
    """Run gm and keep the output of every fused scaled_linear call, in order."""
    outs = []

    class Rec(torch.fx.Interpreter):
        def run_node(self, n):
            r = super().run_node(n)
            if n.op == "call_function" and n.target is torch.ops.lingemm.scaled_linear.default:
                outs.append(r)
            return r

    with torch.no_grad():
        y = Rec(gm).run(*args)
    torch.cuda.synchronize()
    return y, outs


@pytest.mark.parametrize("tokens", [(1, 1), (2, 16), (4, 300)])
def test_rewritten_block_matches_oracle(tokens):
    # Each fused call against the oracle at the standard bar: the first on x,
    # the second on the first's bf16 output as the GPU stored it (the
    # intermediate the rewritten block really feeds forward).
    torch.manual_seed(0)
    m = MLP().to(torch.bfloat16).cuda()
    x = torch.randn(*tokens, 512, dtype=torch.bfloat16, device="cuda")
    gm = torch.fx.symbolic_trace(m)
    assert tops.fuse_linear_epilogues(gm, (x,)) == 2
    y, (h, y2) = fused_outputs(gm, x)
    assert y.shape == (*tokens, 512) and y.dtype == torch.bfloat16 and torch.equal(y, y2)
    x2 = codes16(x.reshape(-1, 512))
    r1, _ = oracle.linear("bf16", "gelu_tanh", x2, codes16(m.up.weight),
                          bias=codes16(m.up.bias))
    assert_close(h.reshape(-1, 1024).float().cpu().numpy(), r1, f"up+gelu {tokens}")
    r2, _ = oracle.linear("bf16", "none", codes16(h.reshape(-1, 1024)), codes16(m.down.weight),
                          bias=codes16(m.down.bias), residual=x2, alpha=0.5)
    assert_close(y.reshape(-1, 512).float().cpu().numpy(), r2, f"down*0.5+x {tokens}")


class PagesBlock(nn.Module):
    """gelu(matmul(x, w) + b, approximate="tanh") with w [K, N] and b [N]: the
    forward pass of "Совместная работа Helion и TorchInductor", sections
    "Интеграция с TorchInductor через замену шаблонов подграфов" and
    "Проверка эффективности слияния" (fp16, x / w / b standard normal)."""

    def __init__(self, w, b):
        super().__init__()
        self.w = nn.Parameter(w)
        self.b = nn.Parameter(b)

    def forward(self, x):
        return F.gelu(torch.matmul(x, self.w) + self.b, approximate="tanh")


@pytest.mark.parametrize("M,K,N,sampled", [(64, 512, 256, False), (200, 1024, 384, False),
                                           (4096, 4096, 4096, True)])
def test_pages_block_rewritten_matches_oracle(M, K, N, sampled):
    g = torch.Generator().manual_seed(M + K + N)
    x = torch.randn(M, K, generator=g).to(torch.float16).cuda()
    w = torch.randn(K, N, generator=g).to(torch.float16).cuda()
    b = torch.randn(N, generator=g).to(torch.float16).cuda()
    gm = torch.fx.symbolic_trace(PagesBlock(w, b))
    assert tops.fuse_linear_epilogues(gm, (x,)) == 1
    y, (y1,) = fused_outputs(gm, x)
    assert torch.equal(y, y1) and y.dtype == torch.float16
    w_nk = codes16(w.t().contiguous())
    g16 = y.float().cpu().numpy()
    if sampled:
        im, inn = sample_positions(M, N, 6000, seed=3)
        r, _ = oracle.linear_at("fp16", "gelu_tanh", codes16(x), w_nk, im, inn,
                                bias=codes16(b))
        assert_close(g16[im, inn], r, "pages block 4096^3 (sampled)")
    else:
        r, _ = oracle.linear("fp16", "gelu_tanh", codes16(x), w_nk, bias=codes16(b))
        assert_close(g16, r, f"pages block {M}x{K}x{N}")


def test_two_streams_use_separate_workspaces():
    # Two split-K shapes (tile kernels with K split across workgroups) on two
    # streams at once: each stream has its own handle, so the partials do not
    # mix.  Repeated so the launches overlap.
    ps = [synth.make_custom("fp8_dynamic", "silu", 64, 2048, 4096, seed=11, bias=True),
          synth.make_custom("fp8_dynamic", "gelu_tanh", 96, 1024, 4096, seed=12, bias=True)]
    ops = []
    for p in ps:
        ops.append(dict(x=dev(p.A).view(torch.float8_e4m3fn), w=dev(p.B).view(torch.float8_e4m3fn),
                        sa=dev(p.sa), sb=dev(p.sb), bias=dev(p.bias).view(torch.bfloat16)))
    h = tops.handle_for(torch.device("cuda"))
    assert "split=" in h.describe("fp8_dynamic", 64, 2048, 4096)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    torch.cuda.synchronize()
    for _ in range(8):
        for i, (p, o) in enumerate(zip(ps, ops)):
            with torch.cuda.stream(streams[i]):
                outs[i].append(torch.ops.lingemm.scaled_linear(
                    o["x"], o["w"], bias=o["bias"], scale_a=o["sa"], scale_b=o["sb"],
                    quant="fp8_dynamic", act=p.act))
    torch.cuda.synchronize()
    for i, p in enumerate(ps):
        ref, _ = oracle.linear(p.quant, p.act, **p.operands())
        for y in outs[i]:
            assert_close(y.float().cpu().numpy(), ref, f"stream {i}")


def test_opcheck_scaled_linear():
    x = torch.randn(5, 256, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(128, 256, dtype=torch.bfloat16, device="cuda") * 0.05
    b = torch.randn(128, dtype=torch.bfloat16, device="cuda")
    torch.library.opcheck(torch.ops.lingemm.scaled_linear.default, (x, w),
                          dict(bias=b, act="silu", quant="bf16"),
                          test_utils=("test_schema", "test_faketensor"))
    p = synth.make_custom("fp8_dynamic", "none", 3, 256, 512, seed=1, bias=True)
    X = dev(synth.activations16(3, 512, seed=2)).view(torch.bfloat16)
    torch.library.opcheck(torch.ops.lingemm.scaled_linear_dynamic.default,
                          (X, dev(p.B), dev(p.sb)), dict(bias=dev(p.bias).view(torch.bfloat16)),
                          test_utils=("test_schema", "test_faketensor"))


def test_dynamic_op_matches_oracle():
    p = synth.make_custom("w8a8_int8", "silu", 4, 512, 1024, seed=9, bias=True)
    Xh = synth.activations16(4, 1024, seed=10)
    Qr, Sr = oracle.dynamic_quant("int8_token", Xh)
    ref, _ = oracle.linear("w8a8_int8", "silu", Qr, p.B, Sr, p.sb, p.bias)
    y = torch.ops.lingemm.scaled_linear_dynamic(dev(Xh).view(torch.bfloat16), dev(p.B),
                                                dev(p.sb), bias=dev(p.bias).view(torch.bfloat16),
                                                quant="w8a8_int8", act="silu")
    torch.cuda.synchronize()
    assert_close(y.float().cpu().numpy(), ref, "scaled_linear_dynamic int8")


def test_graph_capture_of_decode_path_replays():
    # The FP8 decode shape: capture four layer calls (two weight copies, the
    # op on both its paths) after an eager warm-up, then replay with new
    # inputs copied in between, checking every replay against eager calls.
    p = synth.make(2, 4)
    A, sa = dev(p.A).view(torch.float8_e4m3fn), dev(p.sa)
    Bs = [dev(p.B).view(torch.float8_e4m3fn), dev(p.B).view(torch.float8_e4m3fn).clone()]
    sb, bias = dev(p.sb), dev(p.bias).view(torch.bfloat16)
    X = torch.randn(4, p.K, dtype=torch.bfloat16, device="cuda")

    def step():
        outs = []
        for B in Bs:
            outs.append(torch.ops.lingemm.scaled_linear(A, B, bias=bias, scale_a=sa, scale_b=sb,
                                                        quant="fp8_dynamic"))
            outs.append(torch.ops.lingemm.scaled_linear_dynamic(X, B, sb, bias=bias))
        return outs

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step()
    rng = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(4):
        A.view(torch.uint8).copy_(dev(synth.to_e4m3_codes(
            torch.randn(4, p.K, generator=rng).numpy())))
        X.copy_(torch.randn(4, p.K, generator=rng).to(torch.bfloat16).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = step()
        torch.cuda.synchronize()
        for c, e in zip(captured, eager):
            assert torch.equal(c, e), f"replay {rep} differs from eager"


@pytest.mark.parametrize("sizes", [[3, 0, 1, 2], [40, 9, 0, 70]])
def test_grouped_op_matches_oracle(sizes):
    # Decode-sized and prefill-sized segments through the custom operator.
    g = synth.make_grouped("fp8_dynamic", "silu", sizes, 96, 512, seed=sum(sizes), residual=True)
    y = torch.ops.lingemm.scaled_linear_grouped(
        dev(g["A"]), dev(np.stack(g["Bs"])), dev(g["offsets"]),
        bias=dev(np.stack(g["biases"])).view(torch.bfloat16),
        residual=dev(g["residual"]).view(torch.bfloat16), scale_a=dev(g["sa"]),
        scale_b=dev(np.stack(g["sbs"])), quant="fp8_dynamic", act="silu", alpha=0.5)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_linear("fp8_dynamic", "silu", g["A"], g["Bs"], g["offsets"],
                                   sa=g["sa"], sbs=g["sbs"], biases=g["biases"],
                                   residual=g["residual"], alpha=0.5)
    assert_close(y.float().cpu().numpy(), ref, "scaled_linear_grouped")


def test_opcheck_scaled_linear_grouped():
    g = synth.make_grouped("bf16", "none", [5, 0, 11], 64, 128, seed=3)
    args = (dev(g["A"]).view(torch.bfloat16), dev(np.stack(g["Bs"])).view(torch.bfloat16),
            dev(g["offsets"]))
    torch.library.opcheck(torch.ops.lingemm.scaled_linear_grouped.default, args,
                          dict(bias=dev(np.stack(g["biases"])).view(torch.bfloat16)),
                          test_utils=("test_schema", "test_faketensor"))


@pytest.mark.parametrize("quant,kind", [("fp8_dynamic", "fp8_token"), ("w8a8_int8", "int8_token"),
                                        ("block_fp8", "fp8_block")])
def test_grouped_dynamic_op_matches_oracle(quant, kind):
    # 16-bit activations quantized per token (or 1x128 block) by the oracle,
    # then the oracle's grouped layer; against the op that does both on the GPU.
    sizes = [3, 0, 40, 9]
    g = synth.make_grouped(quant, "silu", sizes, 128, 256, seed=31)
    Xh = synth.activations16(int(sum(sizes)), 256, seed=32)
    Q, S = oracle.dynamic_quant(kind, Xh)
    ref, _ = oracle.grouped_linear(quant, "silu", Q, g["Bs"], g["offsets"], sa=S,
                                   sbs=g["sbs"], biases=g["biases"])
    y = torch.ops.lingemm.scaled_linear_grouped_dynamic(
        dev(Xh).view(torch.bfloat16), dev(np.stack(g["Bs"])), dev(g["offsets"]),
        dev(np.stack(g["sbs"])), bias=dev(np.stack(g["biases"])).view(torch.bfloat16),
        quant=quant, act="silu")
    torch.cuda.synchronize()
    assert_close(y.float().cpu().numpy(), ref, f"scaled_linear_grouped_dynamic {quant}")
