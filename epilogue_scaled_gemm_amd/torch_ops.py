"""PyTorch integration of the scaled linear layer.

- ``torch.ops.lingemm.scaled_linear``: a custom operator over the C ABI
  (lin_gemm_run on torch's current stream), with a fake implementation that
  gives the output's shape and dtype without touching device memory, so the
  op traces, exports and captures like a built-in one.
- ``torch.ops.lingemm.scaled_linear_dynamic``: the same layer on 16-bit
  activations quantized on the fly (lin_gemm_run_dynamic).
- ``torch.ops.lingemm.scaled_linear_grouped``: the mixture-of-experts form
  (lin_gemm_run_grouped): token-sorted rows, one weight per expert; and
  ``scaled_linear_grouped_dynamic`` for 16-bit activations quantized first.
- ``fuse_linear_epilogues(gm)``: a torch.fx pass that rewrites
  ``linear -> activation [-> * alpha] [-> + residual]`` chains of a traced
  module into single ``scaled_linear`` calls.

This follows the TorchInductor-integration section of "Совместная работа
Helion и TorchInductor: слияние операторов" (gurufy.ru): register the
composite operator with the dispatcher, give it a shape-only implementation
so tracing does not allocate, and replace the matmul + bias + GELU(tanh)
subgraph with it.  The rewrite here is a plain torch.fx pass rather than an
Inductor joint-graph pattern: the rest of the graph runs eagerly on this
stack, and the pass sees nn.Linear modules and functional calls directly.
Only the tanh form of GELU is fused (the kernel's activation); the erf form
is left alone.

Capturing these ops in a HIP graph (torch.cuda.graph) works once each shape
has run eagerly on the same handle: the first call of a shape may grow the
handle's split-K workspace or staging, which must not happen under capture.
"""
import operator
from typing import Optional

import torch
import torch.nn.functional as F

from . import Handle, out_dtype

_handles = {}


def handle_for(device: torch.device) -> Handle:
    """The library handle of a CUDA device (one per device, created lazily)."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    h = _handles.get(idx)
    if h is None:
        with torch.cuda.device(idx):
            h = Handle()
        _handles[idx] = h
    return h


def _flat(t, K):
    return None if t is None else t.reshape(-1, K).contiguous()


@torch.library.custom_op("lingemm::scaled_linear", mutates_args=())
def scaled_linear(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                  residual: Optional[torch.Tensor] = None, scale_a: Optional[torch.Tensor] = None,
                  scale_b: Optional[torch.Tensor] = None, quant: str = "bf16", act: str = "none",
                  alpha: float = 1.0) -> torch.Tensor:
    """act(s * (x @ weight^T) + bias) * alpha + residual in one kernel.

    x [..., K] (leading dimensions are flattened into tokens), weight [N, K]
    (the nn.Linear layout), bias [N], residual [..., N]; scale_a / scale_b as
    the quant mode needs them.  Returns [..., N] in bf16 (fp16 for fp16).
    """
    K = x.shape[-1]
    N, Kw = weight.shape
    if K != Kw:
        raise ValueError(f"inner dimensions differ: x has K={K}, weight has {Kw}")
    lead = x.shape[:-1]
    x2 = _flat(x, K)
    out = torch.empty((x2.shape[0], N), dtype=out_dtype(quant), device=x.device)
    handle_for(x.device).run(x2, weight.contiguous(), out, quant=quant, act=act, sa=scale_a,
                             sb=scale_b, alpha=alpha, bias=bias, residual=_flat(residual, N))
    return out.reshape(*lead, N)


@scaled_linear.register_fake
def _scaled_linear_fake(x, weight, bias=None, residual=None, scale_a=None, scale_b=None,
                        quant="bf16", act="none", alpha=1.0):
    torch._check(x.shape[-1] == weight.shape[1])
    return x.new_empty((*x.shape[:-1], weight.shape[0]), dtype=out_dtype(quant))


@torch.library.custom_op("lingemm::scaled_linear_dynamic", mutates_args=())
def scaled_linear_dynamic(x: torch.Tensor, weight: torch.Tensor, scale_b: torch.Tensor,
                          bias: Optional[torch.Tensor] = None,
                          residual: Optional[torch.Tensor] = None, quant: str = "fp8_dynamic",
                          act: str = "none", alpha: float = 1.0) -> torch.Tensor:
    """The quantised layer on 16-bit activations x [..., K], quantized per
    token (or per 1x128 block) inside the call."""
    K = x.shape[-1]
    N, Kw = weight.shape
    if K != Kw:
        raise ValueError(f"inner dimensions differ: x has K={K}, weight has {Kw}")
    lead = x.shape[:-1]
    x2 = _flat(x, K)
    out = torch.empty((x2.shape[0], N), dtype=torch.bfloat16, device=x.device)
    x_dtype = "fp16" if x.dtype == torch.float16 else "bf16"
    handle_for(x.device).run_dynamic(x2, weight.contiguous(), out, quant=quant, act=act,
                                     sb=scale_b, alpha=alpha, bias=bias,
                                     residual=_flat(residual, N), x_dtype=x_dtype)
    return out.reshape(*lead, N)


@scaled_linear_dynamic.register_fake
def _scaled_linear_dynamic_fake(x, weight, scale_b, bias=None, residual=None,
                                quant="fp8_dynamic", act="none", alpha=1.0):
    torch._check(x.shape[-1] == weight.shape[1])
    return x.new_empty((*x.shape[:-1], weight.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("lingemm::scaled_linear_grouped", mutates_args=())
def scaled_linear_grouped(x: torch.Tensor, weight: torch.Tensor, offsets: torch.Tensor,
                          bias: Optional[torch.Tensor] = None,
                          residual: Optional[torch.Tensor] = None,
                          scale_a: Optional[torch.Tensor] = None,
                          scale_b: Optional[torch.Tensor] = None, quant: str = "bf16",
                          act: str = "none", alpha: float = 1.0, max_rows: int = 0) -> torch.Tensor:
    """Mixture-of-experts layer: x [M, K] rows sorted by expert, weight
    [E, N, K] (E, N, K/2 bytes for mxfp4), offsets int32 [E + 1] from 0 to M
    on the GPU (expert e owns rows offsets[e] .. offsets[e+1]), bias [E, N],
    residual [M, N], scale_b [E, N] (or the mode's per-expert layout).
    Returns [M, N]."""
    M = x.shape[0]
    N = weight.shape[1]
    out = torch.empty((M, N), dtype=out_dtype(quant), device=x.device)
    handle_for(x.device).run_grouped(x.contiguous(), weight.contiguous(), out,
                                     offsets.contiguous(), quant=quant, act=act, sa=scale_a,
                                     sb=scale_b, alpha=alpha, bias=bias, residual=residual,
                                     max_rows=max_rows)
    return out


@scaled_linear_grouped.register_fake
def _scaled_linear_grouped_fake(x, weight, offsets, bias=None, residual=None, scale_a=None,
                                scale_b=None, quant="bf16", act="none", alpha=1.0, max_rows=0):
    torch._check(offsets.shape[0] == weight.shape[0] + 1)
    return x.new_empty((x.shape[0], weight.shape[1]), dtype=out_dtype(quant))


_DQ_OF = {"fp8_dynamic": ("fp8_token", torch.float8_e4m3fn), "w8a8_int8": ("int8_token", torch.int8),
          "block_fp8": ("fp8_block", torch.float8_e4m3fn)}


@torch.library.custom_op("lingemm::scaled_linear_grouped_dynamic", mutates_args=())
def scaled_linear_grouped_dynamic(x: torch.Tensor, weight: torch.Tensor, offsets: torch.Tensor,
                                  scale_b: torch.Tensor, bias: Optional[torch.Tensor] = None,
                                  residual: Optional[torch.Tensor] = None,
                                  quant: str = "fp8_dynamic", act: str = "none",
                                  alpha: float = 1.0, max_rows: int = 0) -> torch.Tensor:
    """The grouped layer on 16-bit activations x [M, K]: per-token (or 1x128
    block) quantization (lin_gemm_quantize), then lin_gemm_run_grouped on the
    codes.  The per-token scales follow their rows, so quantizing before the
    grouping gives the same codes as quantizing each expert's rows."""
    if quant not in _DQ_OF:
        raise ValueError(f"scaled_linear_grouped_dynamic quantizes for {sorted(_DQ_OF)}, "
                         f"not {quant!r}")
    kind, code_dtype = _DQ_OF[quant]
    M, K = x.shape
    h = handle_for(x.device)
    q = torch.empty((M, K), dtype=code_dtype, device=x.device)
    ns = M * (K // 128) if kind == "fp8_block" else M
    sa = torch.empty(ns, dtype=torch.float32, device=x.device)
    xc = x.contiguous()
    h.quantize(xc, q, sa, kind=kind, x_dtype="fp16" if x.dtype == torch.float16 else "bf16")
    out = torch.empty((M, weight.shape[1]), dtype=torch.bfloat16, device=x.device)
    h.run_grouped(q, weight.contiguous(), out, offsets.contiguous(), quant=quant, act=act,
                  sa=sa, sb=scale_b, alpha=alpha, bias=bias, residual=residual,
                  max_rows=max_rows)
    return out


@scaled_linear_grouped_dynamic.register_fake
def _scaled_linear_grouped_dynamic_fake(x, weight, offsets, scale_b, bias=None, residual=None,
                                        quant="fp8_dynamic", act="none", alpha=1.0, max_rows=0):
    torch._check(offsets.shape[0] == weight.shape[0] + 1)
    return x.new_empty((x.shape[0], weight.shape[1]), dtype=torch.bfloat16)


# --------------------------------------------------------------- FX rewrite

_ACT_FUNCS = {F.silu: "silu", F.relu: "relu", torch.relu: "relu"}
_ACT_MODULES = {torch.nn.SiLU: "silu", torch.nn.ReLU: "relu"}


def _single_user(node):
    return len(node.users) == 1


def _linear_parts(gm, node):
    """(x, weight, bias) nodes/values if `node` is a linear call whose weight
    is a bf16 / fp16 parameter of gm, else None."""
    if node.op == "call_module":
        mod = gm.get_submodule(node.target)
        if type(mod) is not torch.nn.Linear:
            return None
        if mod.weight.dtype not in (torch.bfloat16, torch.float16):
            return None
        with gm.graph.inserting_before(node):
            w = gm.graph.get_attr(node.target + ".weight")
            b = gm.graph.get_attr(node.target + ".bias") if mod.bias is not None else None
        return node.args[0], w, b, mod.weight.dtype
    if node.op == "call_function" and node.target is F.linear:
        x = node.args[0]
        w = node.args[1] if len(node.args) > 1 else node.kwargs.get("weight")
        b = node.args[2] if len(node.args) > 2 else node.kwargs.get("bias")
        if not (isinstance(w, torch.fx.Node) and w.op == "get_attr"):
            return None
        wt = gm.get_parameter(w.target) if w.target in dict(gm.named_parameters()) \
            else getattr(gm, w.target, None)
        if not isinstance(wt, torch.Tensor) or wt.dtype not in (torch.bfloat16, torch.float16):
            return None
        return x, w, b, wt.dtype
    return None


def _activation(gm, node):
    """The kernel activation name if `node` applies one the kernel has."""
    if node.op == "call_function":
        if node.target is F.gelu:
            approx = node.kwargs.get("approximate", node.args[1] if len(node.args) > 1 else "none")
            return "gelu_tanh" if approx == "tanh" else None
        return _ACT_FUNCS.get(node.target)
    if node.op == "call_method" and node.target == "relu":
        return "relu"
    if node.op == "call_module":
        mod = gm.get_submodule(node.target)
        if type(mod) is torch.nn.GELU:
            return "gelu_tanh" if mod.approximate == "tanh" else None
        return _ACT_MODULES.get(type(mod))
    return None


def _scalar_mul(node, prev):
    """alpha if node is prev * alpha (or alpha * prev) with a Python number."""
    if node.op != "call_function" or node.target not in (operator.mul, torch.mul):
        return None
    a, b = node.args[0], node.args[1]
    if a is prev and isinstance(b, (int, float)):
        return float(b)
    if b is prev and isinstance(a, (int, float)):
        return float(a)
    return None


def _tensor_add(node, prev):
    """The other operand if node is prev + other with a tensor node."""
    if node.op != "call_function" or node.target not in (operator.add, torch.add):
        return None
    if len(node.args) != 2 or node.kwargs:
        return None
    a, b = node.args
    other = b if a is prev else (a if b is prev else None)
    return other if isinstance(other, torch.fx.Node) else None


def fuse_linear_epilogues(gm: torch.fx.GraphModule) -> int:
    """Rewrite linear -> act [-> * alpha] [-> + residual] chains of gm into
    torch.ops.lingemm.scaled_linear calls, in place.  A chain is taken only
    as far as each intermediate has a single user; a plain linear with no
    epilogue is left alone.  Returns the number of chains rewritten."""
    count = 0
    for node in list(gm.graph.nodes):
        if node.op not in ("call_module", "call_function") or node.graph is not gm.graph:
            continue
        if not (node.op == "call_function" and node.target is F.linear) and not (
                node.op == "call_module" and type(gm.get_submodule(node.target)) is torch.nn.Linear):
            continue
        tail, act, alpha, residual = node, "none", 1.0, None
        if _single_user(tail):
            u = next(iter(tail.users))
            a = _activation(gm, u)
            if a is not None:
                tail, act = u, a
        if _single_user(tail):
            u = next(iter(tail.users))
            m = _scalar_mul(u, tail)
            if m is not None:
                tail, alpha = u, m
        if _single_user(tail):
            u = next(iter(tail.users))
            r = _tensor_add(u, tail)
            if r is not None:
                tail, residual = u, r
        if tail is node:
            continue
        parts = _linear_parts(gm, node)
        if parts is None:
            continue
        x, w, b, wdtype = parts
        quant = "fp16" if wdtype == torch.float16 else "bf16"
        with gm.graph.inserting_after(tail):
            fused = gm.graph.call_function(
                torch.ops.lingemm.scaled_linear.default, (x, w),
                dict(bias=b, residual=residual, quant=quant, act=act, alpha=alpha))
        tail.replace_all_uses_with(fused)
        count += 1
    gm.graph.eliminate_dead_code()
    gm.graph.lint()
    gm.recompile()
    return count
