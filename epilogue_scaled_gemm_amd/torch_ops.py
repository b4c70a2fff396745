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
- ``fuse_linear_epilogues(gm, example_inputs)``: a torch.fx pass that
  rewrites ``linear -> activation [-> * alpha] [-> + residual]`` chains of a
  traced module, and the ``matmul(x, w) -> + bias -> activation ...`` chain
  of the pages (w a [K, N] parameter), into single ``scaled_linear`` calls.

This follows the TorchInductor-integration section of "Совместная работа
Helion и TorchInductor: слияние операторов" (gurufy.ru): register the
composite operator with the dispatcher, give it a shape-only implementation
so tracing does not allocate, and replace the matmul + bias + GELU(tanh)
subgraph with it.  The rewrite here is a plain torch.fx pass rather than an
Inductor joint-graph pattern: the rest of the graph runs eagerly on this
stack, and the pass sees nn.Linear modules and functional calls directly.
Only the tanh form of GELU is fused (the kernel's activation); the erf form
is left alone.

Streams and graphs.  Each (device, stream) pair gets its own library
handle, so calls on different streams never share a split-K workspace; the
quantized codes of the dynamic op are torch tensors allocated on the calling
stream.  A call whose variant splits K across workgroups grows its handle's
workspace the first time its shape runs on that stream, which cannot happen
while the stream is being captured: before capturing such shapes into a HIP
graph, run them once eagerly on the capture stream
(``torch.cuda.graph(g, stream=s)`` after a warm-up under
``torch.cuda.stream(s)``).  Shapes that run without a split (every decode
shape of the built-in table) capture on any stream.
"""
import operator
from typing import Optional

import torch
import torch.nn.functional as F

from . import Handle, out_dtype

_handles = {}


def handle_for(device: torch.device) -> Handle:
    """The library handle for a CUDA device and its current stream (one per
    (device, stream) pair, created lazily): a handle's split-K workspace
    must not be used by two streams at once."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    stream = torch.cuda.current_stream(idx).cuda_stream
    h = _handles.get((idx, stream))
    if h is None:
        with torch.cuda.device(idx):
            h = Handle()
        _handles[(idx, stream)] = h
    return h


_CODE_DTYPES = {"bf16": (torch.bfloat16,), "fp16": (torch.float16,),
                "fp8_dynamic": (torch.float8_e4m3fn, torch.uint8),
                "block_fp8": (torch.float8_e4m3fn, torch.uint8),
                "w8a8_int8": (torch.int8,), "mxfp4": (torch.bfloat16,)}


def _check_operands(x, weight, bias, residual, scale_a, scale_b, quant, x_is_16bit=False):
    """Shapes and dtypes of the layer's operands, checked before any device
    work: the kernels read exactly [M, K], [N, K], [N] and [M, N] elements
    of the documented types, so a broadcastable or differently typed
    operand must be rejected here, not read out of bounds."""
    if quant not in _CODE_DTYPES:
        raise ValueError(f"unknown quant mode {quant!r}")
    K = x.shape[-1]
    N = weight.shape[0]
    kw = K // 2 if quant == "mxfp4" else K
    if weight.dim() != 2 or weight.shape[1] != kw:
        raise ValueError(f"weight must be [N, {kw}] for x [..., {K}], got {tuple(weight.shape)}")
    codes = (torch.bfloat16, torch.float16) if x_is_16bit else _CODE_DTYPES[quant]
    if x.dtype not in codes:
        raise ValueError(f"x must be {codes} for quant {quant!r}, got {x.dtype}")
    wcodes = (torch.uint8,) if quant == "mxfp4" else _CODE_DTYPES[quant]
    if weight.dtype not in wcodes:
        raise ValueError(f"weight must be {wcodes} for quant {quant!r}, got {weight.dtype}")
    od = out_dtype(quant)
    if bias is not None and (tuple(bias.shape) != (N,) or bias.dtype != od):
        raise ValueError(f"bias must be [{N}] {od}, got {tuple(bias.shape)} {bias.dtype}")
    if residual is not None and (tuple(residual.shape) != (*x.shape[:-1], N) or
                                 residual.dtype != od):
        raise ValueError(f"residual must be {(*x.shape[:-1], N)} {od} (no broadcasting), got "
                         f"{tuple(residual.shape)} {residual.dtype}")
    M = 1
    for d in x.shape[:-1]:
        M = M * d
    want_a = {"fp8_dynamic": M, "w8a8_int8": M, "block_fp8": M * (K // 128)}.get(quant)
    want_b = {"fp8_dynamic": N, "w8a8_int8": N, "block_fp8": (N // 128) * (K // 128),
              "mxfp4": N * (K // 32)}.get(quant)
    if want_a is not None and not x_is_16bit:
        if scale_a is None or scale_a.dtype != torch.float32 or scale_a.numel() != want_a:
            raise ValueError(f"scale_a must hold {want_a} fp32 values for quant {quant!r}")
    if want_b is not None:
        sdt = torch.uint8 if quant == "mxfp4" else torch.float32
        if scale_b is None or scale_b.dtype != sdt or scale_b.numel() != want_b:
            raise ValueError(f"scale_b must hold {want_b} {sdt} values for quant {quant!r}")


_DQ_OF = {"fp8_dynamic": ("fp8_token", torch.float8_e4m3fn), "w8a8_int8": ("int8_token", torch.int8),
          "block_fp8": ("fp8_block", torch.float8_e4m3fn)}


_prologue_cache = {}


def _prologue(h, quant, M, N, K):
    """Whether the built-in table asks for the quantization prologue at this
    shape (the variant's "dq=1"); cached, since the table is fixed."""
    key = (quant, M, N, K)
    v = _prologue_cache.get(key)
    if v is None:
        v = _prologue_cache[key] = "dq=1" in h.describe(quant, M, N, K)
    return v


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
    _check_operands(x, weight, bias, residual, scale_a, scale_b, quant)
    K = x.shape[-1]
    N = weight.shape[0]
    lead = x.shape[:-1]
    x2 = _flat(x, K)
    out = torch.empty((x2.shape[0], N), dtype=out_dtype(quant), device=x.device)
    handle_for(x.device).run(x2, weight.contiguous(), out, quant=quant, act=act, sa=scale_a,
                             sb=scale_b, alpha=alpha, bias=bias, residual=_flat(residual, N))
    return out.reshape(*lead, N)


@scaled_linear.register_fake
def _scaled_linear_fake(x, weight, bias=None, residual=None, scale_a=None, scale_b=None,
                        quant="bf16", act="none", alpha=1.0):
    _check_operands(x, weight, bias, residual, scale_a, scale_b, quant)
    return x.new_empty((*x.shape[:-1], weight.shape[0]), dtype=out_dtype(quant))


@torch.library.custom_op("lingemm::scaled_linear_dynamic", mutates_args=())
def scaled_linear_dynamic(x: torch.Tensor, weight: torch.Tensor, scale_b: torch.Tensor,
                          bias: Optional[torch.Tensor] = None,
                          residual: Optional[torch.Tensor] = None, quant: str = "fp8_dynamic",
                          act: str = "none", alpha: float = 1.0) -> torch.Tensor:
    """The quantised layer on 16-bit activations x [..., K], quantized per
    token (or per 1x128 block) inside the call.  When the shape's variant
    quantizes in the kernel's prologue, one library call does both;
    otherwise the codes and scales go to torch tensors allocated on the
    calling stream (so no handle staging is shared between streams or
    grown under graph capture), then the layer runs on them."""
    if quant not in _DQ_OF:
        raise ValueError(f"scaled_linear_dynamic quantizes for {sorted(_DQ_OF)}, not {quant!r}")
    _check_operands(x, weight, bias, residual, None, scale_b, quant, x_is_16bit=True)
    K = x.shape[-1]
    N = weight.shape[0]
    lead = x.shape[:-1]
    x2 = _flat(x, K)
    M = x2.shape[0]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    x_dtype = "fp16" if x.dtype == torch.float16 else "bf16"
    h = handle_for(x.device)
    wc = weight.contiguous()
    res = _flat(residual, N)
    if x_dtype == "bf16" and M <= 16 and _prologue(h, quant, M, N, K):
        h.run_dynamic(x2, wc, out, quant=quant, act=act, sb=scale_b, alpha=alpha, bias=bias,
                      residual=res, x_dtype=x_dtype)
        return out.reshape(*lead, N)
    kind, code_dtype = _DQ_OF[quant]
    q = torch.empty((M, K), dtype=code_dtype, device=x.device)
    sa = torch.empty(M * (K // 128) if kind == "fp8_block" else M, dtype=torch.float32,
                     device=x.device)
    h.quantize(x2, q, sa, kind=kind, x_dtype=x_dtype)
    h.run(q, wc, out, quant=quant, act=act, sa=sa, sb=scale_b, alpha=alpha, bias=bias,
          residual=res)
    return out.reshape(*lead, N)


@scaled_linear_dynamic.register_fake
def _scaled_linear_dynamic_fake(x, weight, scale_b, bias=None, residual=None,
                                quant="fp8_dynamic", act="none", alpha=1.0):
    if quant not in _DQ_OF:
        raise ValueError(f"scaled_linear_dynamic quantizes for {sorted(_DQ_OF)}, not {quant!r}")
    _check_operands(x, weight, bias, residual, None, scale_b, quant, x_is_16bit=True)
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
_MATMULS = (torch.matmul, operator.matmul, torch.mm, torch.ops.aten.mm.default)
_ADDS = (operator.add, torch.add, torch.ops.aten.add.Tensor)
_MULS = (operator.mul, torch.mul, torch.ops.aten.mul.Tensor)


def _single_user(node):
    return len(node.users) == 1


def _attr_tensor(gm, node):
    """The tensor a get_attr node names, else None."""
    if not (isinstance(node, torch.fx.Node) and node.op == "get_attr"):
        return None
    obj = gm
    for part in node.target.split("."):
        obj = getattr(obj, part, None)
        if obj is None:
            return None
    return obj if isinstance(obj, torch.Tensor) else None


def _meta(gm, node):
    """(shape, dtype) of a node's value: a module attribute's own tensor, or
    the metadata left by ShapeProp ("tensor_meta") or by fake-tensor tracing
    ("val").  None when unknown."""
    t = _attr_tensor(gm, node)
    if t is not None:
        return tuple(t.shape), t.dtype
    if not isinstance(node, torch.fx.Node):
        return None
    tm = node.meta.get("tensor_meta")
    if tm is not None and hasattr(tm, "shape"):
        return tuple(tm.shape), tm.dtype
    v = node.meta.get("val")
    if isinstance(v, torch.Tensor):
        return tuple(v.shape), v.dtype
    return None


def _linear_parts(gm, node):
    """(x, weight node [N, K], bias node or None, weight dtype, N) if `node`
    is a linear call whose weight is a bf16 / fp16 attribute of gm, else
    None.  For matmul(x, w) with w a [K, N] attribute, a [N, K] copy of w is
    registered on gm (made once, at rewrite time) and used as the weight."""
    if node.op == "call_module":
        mod = gm.get_submodule(node.target)
        if type(mod) is not torch.nn.Linear:
            return None
        if mod.weight.dtype not in (torch.bfloat16, torch.float16):
            return None
        with gm.graph.inserting_before(node):
            w = gm.graph.get_attr(node.target + ".weight")
            b = gm.graph.get_attr(node.target + ".bias") if mod.bias is not None else None
        return node.args[0], w, b, mod.weight.dtype, mod.weight.shape[0]
    if node.op == "call_function" and node.target is F.linear:
        x = node.args[0]
        w = node.args[1] if len(node.args) > 1 else node.kwargs.get("weight")
        b = node.args[2] if len(node.args) > 2 else node.kwargs.get("bias")
        wt = _attr_tensor(gm, w)
        if wt is None or wt.dim() != 2 or wt.dtype not in (torch.bfloat16, torch.float16):
            return None
        if b is not None and _meta(gm, b) != ((wt.shape[0],), wt.dtype):
            return None
        return x, w, b, wt.dtype, wt.shape[0]
    if node.op == "call_function" and node.target in _MATMULS and len(node.args) == 2 \
            and not node.kwargs:
        x, w = node.args
        wt = _attr_tensor(gm, w)
        if wt is None or wt.dim() != 2 or wt.dtype not in (torch.bfloat16, torch.float16):
            return None
        name = "_lingemm_nk_" + w.target.replace(".", "_")
        if not hasattr(gm, name):
            gm.register_buffer(name, wt.detach().t().contiguous())
        with gm.graph.inserting_before(node):
            wnk = gm.graph.get_attr(name)
        return x, wnk, None, wt.dtype, wt.shape[1]
    return None


def _is_linear(gm, node):
    if node.op == "call_module":
        return type(gm.get_submodule(node.target)) is torch.nn.Linear
    if node.op != "call_function":
        return False
    if node.target is F.linear:
        return True
    if node.target not in _MATMULS or len(node.args) != 2 or node.kwargs:
        return False
    w = _attr_tensor(gm, node.args[1])
    return w is not None and w.dim() == 2


def _activation(gm, node):
    """The kernel activation name if `node` applies one the kernel has."""
    if node.op == "call_function":
        if node.target in (F.gelu, torch.ops.aten.gelu.default):
            approx = node.kwargs.get("approximate", node.args[1] if len(node.args) > 1 else "none")
            return "gelu_tanh" if approx == "tanh" else None
        if node.target is torch.ops.aten.silu.default:
            return "silu"
        if node.target is torch.ops.aten.relu.default:
            return "relu"
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
    if node.op != "call_function" or node.target not in _MULS or node.kwargs:
        return None
    a, b = node.args[0], node.args[1]
    if a is prev and isinstance(b, (int, float)) and not isinstance(b, bool):
        return float(b)
    if b is prev and isinstance(a, (int, float)) and not isinstance(a, bool):
        return float(a)
    return None


def _tensor_add(gm, node, prev, shape, dtype):
    """The other operand if node is prev + other, where other is a tensor
    node whose known shape and dtype are exactly `shape` and `dtype`."""
    if node.op != "call_function" or node.target not in _ADDS:
        return None
    if len(node.args) != 2 or node.kwargs:
        return None
    a, b = node.args
    other = b if a is prev else (a if b is prev else None)
    if not isinstance(other, torch.fx.Node) or other is prev:
        return None
    return other if _meta(gm, other) == (shape, dtype) else None


def fuse_linear_epilogues(gm: torch.fx.GraphModule, example_inputs=None) -> int:
    """Rewrite the kernel's epilogue chains in gm into
    torch.ops.lingemm.scaled_linear calls, in place, and return how many.

    Chains: ``linear(x) -> act [-> * alpha] [-> + residual]`` (nn.Linear or
    F.linear with a bf16 / fp16 weight attribute), and the pages' form
    ``matmul(x, w) [-> + bias] -> act [-> * alpha] [-> + residual]`` (torch
    .matmul, ``@``, torch.mm or aten.mm, w a [K, N] bf16 / fp16 attribute,
    bias a [N] tensor of the same dtype).  The activation is tanh-GELU, SiLU
    or ReLU.  A link is taken only while the intermediate has one user, and
    a tensor operand is fused only when its shape and dtype are known and
    are exactly what the kernel reads: bias [N], residual the layer's full
    output shape, both in the weight's dtype.  Shapes come from the graph's
    metadata; pass ``example_inputs`` (any tensors of the right shapes and
    dtypes; they are turned into fake tensors, nothing runs) to fill it in
    by shape propagation.  Without metadata, chains that need a placeholder
    or intermediate tensor operand stop before it.  A plain linear or matmul
    with nothing to fuse is left alone.

    For a matmul chain, the rewritten module holds a [N, K] copy of w made
    at rewrite time: later in-place updates of w do not reach it.
    """
    if example_inputs is not None:
        from torch._subclasses.fake_tensor import FakeTensorMode
        from torch.fx.passes.shape_prop import ShapeProp
        mode = FakeTensorMode(allow_non_fake_inputs=True)
        fake = [mode.from_tensor(t) if isinstance(t, torch.Tensor) else t for t in example_inputs]
        ShapeProp(gm, fake_mode=mode).propagate(*fake)
    count = 0
    for node in list(gm.graph.nodes):
        if node.graph is not gm.graph or not _is_linear(gm, node):
            continue
        out = _meta(gm, node)
        tail, act, alpha, residual, bias = node, "none", 1.0, None, None
        is_mm = node.op == "call_function" and node.target in _MATMULS
        wt = _attr_tensor(gm, node.args[1]) if is_mm else None
        if is_mm and _single_user(tail):
            u = next(iter(tail.users))
            b = _tensor_add(gm, u, tail, (wt.shape[1],), wt.dtype)
            if b is not None:
                tail, bias = u, b
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
        if _single_user(tail) and out is not None:
            u = next(iter(tail.users))
            r = _tensor_add(gm, u, tail, out[0], out[1])
            if r is not None:
                tail, residual = u, r
        if tail is node:
            continue
        parts = _linear_parts(gm, node)
        if parts is None:
            continue
        x, w, b, wdtype, _ = parts
        if bias is not None:
            b = bias
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
