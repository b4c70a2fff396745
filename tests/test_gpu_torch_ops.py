"""The PyTorch integration on the GPU: the FX-rewritten block against the
original block (reference in fp32 on the CPU), torch.library.opcheck of the
custom operators, and HIP-graph capture of the decode path replayed several
times with eager work in between."""
import numpy as np
import pytest
import torch
import torch.nn as nn

import oracle
import synth
from gpu_util import assert_close, dev

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


def _ref_fp32(m, x):
    """The original module in fp32 on the CPU, with each fused layer's output
    rounded to bf16 as the kernel's one store does."""
    m32 = MLP(m.up.in_features, m.up.out_features)
    m32.load_state_dict({k: v.float().cpu() for k, v in m.state_dict().items()})
    x32 = x.float().cpu()
    h = m32.act(m32.up(x32)).to(torch.bfloat16).float()
    return (m32.down(h) * 0.5 + x32).to(torch.bfloat16).float()


@pytest.mark.parametrize("tokens", [(1, 1), (2, 16), (4, 300)])
def test_rewritten_block_matches_reference(tokens):
    torch.manual_seed(0)
    m = MLP().to(torch.bfloat16).cuda()
    gm = torch.fx.symbolic_trace(m)
    assert tops.fuse_linear_epilogues(gm) == 2
    x = torch.randn(*tokens, 512, dtype=torch.bfloat16, device="cuda")
    with torch.no_grad():
        y = gm(x)
        torch.cuda.synchronize()
        ref = _ref_fp32(m, x)
    assert y.shape == (*tokens, 512) and y.dtype == torch.bfloat16
    # Two chained layers with a bf16 intermediate: a one-ulp difference in
    # the intermediate moves sums that nearly cancel, so the relative rule
    # takes its floor at 1% of the output's RMS rather than at 1e-3.
    g, r = y.float().cpu().numpy(), ref.numpy()
    floor = 0.01 * float(np.sqrt(np.mean(r ** 2)))
    bad = np.abs(g - r) > 1e-2 * np.maximum(np.abs(r), floor)
    assert not bad.any(), f"block {tokens}: {bad.sum()} of {g.size} outside the tolerance"


def test_opcheck_scaled_linear():
    x = torch.randn(5, 256, dtype=torch.bfloat16, device="cuda")
    w = torch.randn(128, 256, dtype=torch.bfloat16, device="cuda") * 0.05
    b = torch.randn(128, dtype=torch.bfloat16, device="cuda")
    torch.library.opcheck(torch.ops.lingemm.scaled_linear.default, (x, w),
                          dict(bias=b, act="silu", quant="bf16"),
                          test_utils=("test_schema", "test_faketensor"))
    p = synth.make_custom("fp8_dynamic", "none", 3, 256, 512, seed=1, bias=True)
    X = dev(synth.activations16(3, 512, seed=2))
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
