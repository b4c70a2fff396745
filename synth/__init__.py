"""Seeded synthetic inputs for the scaled linear layer.

This module produces the raw byte arrays (bf16/fp16 bit patterns, e4m3 codes,
int8 values) and fp32 scale arrays that BOTH the HIP library and the CPU oracle
consume.  It holds none of the layer's arithmetic: it only draws values and
quantises them into input codes (absmax scaling, saturating round-to-nearest
casts done by torch's / numpy's CPU casts).

Workloads follow the five problem shapes the library is measured on:

  1  tiny bf16 + GELU          A[64,512]   B[256,512]   bias, GELU(tanh)
  2  FP8 dynamic decode        A[M,4096]   B[6144,4096] per-token x per-channel, bias
  3  W8A8 int8 decode          A[M,4096]   B[24576,4096] per-token x per-channel, SiLU
  4  block-FP8 linear          A[M,12288]  B[4096,12288] 1x128 / 128x128 scales, residual
  5  prefill decoder block     A[4096,4096] B[4096,4096] bias, GELU(tanh)*0.5 + residual
  6  MXFP4-weight decode       A[M,4096] bf16  B[6144,4096] 4-bit E2M1, E8M0 per 32, bias

The (N, K) pairs of 2-4 stand in for the dense-LLM projection shapes that the
vLLM linear-backend write-up tunes on (its Qwen3 weights and ShareGPT traffic
are not available); values are Gaussian or uniform stand-ins.

Seeds: numpy PCG64.  Weight-side draws (B, then bias) use seed 1000*cfg so the
weight is identical across an M sweep; activation-side draws (A, then residual)
use seed 1000*cfg + M.  Values are drawn in fp32, then quantised or rounded.
"""
from dataclasses import dataclass, field
import functools

import numpy as np
import torch

E4M3_MAX = 448.0
INT8_MAX = 127.0

WORKLOADS = {
    1: dict(name="tiny_bf16_gelu", quant="bf16", act="gelu_tanh", N=256, K=512,
            Ms=(64,), bias=True, residual=False, alpha=1.0, dist="uniform"),
    2: dict(name="fp8_dynamic_decode", quant="fp8_dynamic", act="none", N=6144, K=4096,
            Ms=(1, 2, 4, 8, 16, 24, 32), bias=True, residual=False, alpha=1.0, dist="normal"),
    3: dict(name="w8a8_int8_decode", quant="w8a8_int8", act="silu", N=24576, K=4096,
            Ms=(1, 2, 4, 8, 16, 24, 32), bias=False, residual=False, alpha=1.0, dist="normal"),
    4: dict(name="block_fp8", quant="block_fp8", act="none", N=4096, K=12288,
            Ms=(1, 8, 32, 512, 2048), bias=False, residual=True, alpha=1.0, dist="normal"),
    5: dict(name="prefill_bf16_fused", quant="bf16", act="gelu_tanh", N=4096, K=4096,
            Ms=(4096,), bias=True, residual=True, alpha=0.5, dist="normal"),
    6: dict(name="mxfp4_decode", quant="mxfp4", act="none", N=6144, K=4096,
            Ms=(1, 2, 4, 8, 16, 24, 32), bias=True, residual=False, alpha=1.0, dist="normal"),
    7: dict(name="mxfp4_prefill", quant="mxfp4", act="none", N=6144, K=4096,
            Ms=(4096,), bias=True, residual=False, alpha=1.0, dist="normal"),
    8: dict(name="bf16_decode", quant="bf16", act="none", N=6144, K=4096,
            Ms=(1, 2, 4, 8, 16, 24, 32), bias=True, residual=False, alpha=1.0, dist="normal"),
}

# Mixture-of-experts layer: 128 experts, each token routed to 8 distinct
# experts drawn uniformly (seeded), hidden size K = 2048, expert width 768
# with the gate and up projections stacked (N = 1536); FP8 dynamic scaling
# as workload 2; T tokens give 8 T routed rows (decode up to 32 tokens, a
# 512-token prefill chunk).
MOE = dict(name="fp8_moe", quant="fp8_dynamic", act="none", E=128, topk=8, N=1536,
           K=2048, Ts=(1, 4, 16, 32, 512))


def moe_routing(T: int, E: int, topk: int, seed: int) -> np.ndarray:
    """Rows per expert when each of T tokens picks `topk` distinct experts
    uniformly at random."""
    rng = np.random.Generator(np.random.PCG64(seed))
    picks = np.concatenate([rng.permutation(E)[:topk] for _ in range(T)]) if T else \
        np.zeros(0, np.int64)
    return np.bincount(picks, minlength=E).astype(np.int64)


def moe_bytes(quant: str, sizes, N: int, K: int) -> int:
    """Compulsory HBM bytes of one grouped call: each expert with rows
    streams its weight and weight scales once; every routed row reads its
    activation row and scale and writes its output row; the offsets."""
    sizes = np.asarray(sizes)
    M = int(sizes.sum())
    active = int(np.count_nonzero(sizes))
    return (algorithmic_bytes(quant, M, N, K, False, False) - N * K - 4 * N
            + active * (N * K + 4 * N) + 4 * (len(sizes) + 1))


@dataclass
class Problem:
    """One layer call's operands, as raw codes (numpy) plus metadata."""
    quant: str
    act: str
    M: int
    N: int
    K: int
    A: np.ndarray                 # [M,K] uint16 (bf16/fp16) | uint8 (e4m3) | int8
    B: np.ndarray                 # [N,K] same code type
    sa: np.ndarray = None         # fp32 [M] or [M,K/128]
    sb: np.ndarray = None         # fp32 [N] or [N/128,K/128]
    bias: np.ndarray = None       # uint16 [N]
    residual: np.ndarray = None   # uint16 [M,N]
    alpha: float = 1.0
    name: str = ""
    meta: dict = field(default_factory=dict)

    def operands(self):
        return dict(A=self.A, B=self.B, sa=self.sa, sb=self.sb, bias=self.bias,
                    residual=self.residual, alpha=self.alpha)


# ------------------------------------------------------------------ casts
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Saturate to +-448, then round-to-nearest-even to OCP E4M3FN codes."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def to_int8_codes(x: np.ndarray) -> np.ndarray:
    """Round half to even, clamp to [-127, 127] (symmetric)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return torch.round(t).clamp_(-INT8_MAX, INT8_MAX).to(torch.int8).numpy()


def _absmax(x: np.ndarray, dims) -> np.ndarray:
    return torch.from_numpy(x).abs().amax(dim=dims).numpy()


def _safe_scale(absmax: np.ndarray, qmax: float) -> np.ndarray:
    s = (absmax / np.float32(qmax)).astype(np.float32)
    return np.where(absmax > 0, s, np.float32(1.0)).astype(np.float32)


# ------------------------------------------------------------ quantisers
def quant_rows(x: np.ndarray, kind: str):
    """Per-row (per-token / per-channel) symmetric absmax quantisation."""
    qmax = E4M3_MAX if kind == "fp8" else INT8_MAX
    s = _safe_scale(_absmax(x, 1), qmax)
    q = (torch.from_numpy(x) / torch.from_numpy(s)[:, None]).numpy()
    codes = to_e4m3_codes(q) if kind == "fp8" else to_int8_codes(q)
    return codes, s


def quant_blocks_act(x: np.ndarray):
    """1x128 blocks along K: scale[M][K/128]."""
    M, K = x.shape
    xb = x.reshape(M, K // 128, 128)
    s = _safe_scale(_absmax(xb, 2), E4M3_MAX)
    q = (torch.from_numpy(xb) / torch.from_numpy(s)[:, :, None]).numpy()
    return to_e4m3_codes(q.reshape(M, K)), s


def quant_blocks_weight(x: np.ndarray):
    """128x128 blocks: scale[N/128][K/128]."""
    N, K = x.shape
    xb = x.reshape(N // 128, 128, K // 128, 128)
    s = _safe_scale(_absmax(xb, (1, 3)), E4M3_MAX)
    q = (torch.from_numpy(xb) / torch.from_numpy(s)[:, None, :, None]).numpy()
    return to_e4m3_codes(q.reshape(N, K)), s


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def quant_mxfp4(x: np.ndarray):
    """OCP MX quantisation of weights [N,K] to packed E2M1 codes [N,K/2]
    (low nibble first) and E8M0 scales [N,K/32]: per 32 values, the shared
    exponent floor(log2(max|x|)) - 2 (the largest E2M1 exponent), then each
    value rounded to the nearest E2M1 value (ties to the even code),
    saturating at +-6; an all-zero block gets exponent 0."""
    N, K = x.shape
    xb = x.astype(np.float64).reshape(N, K // 32, 32)
    amax = np.abs(xb).max(axis=2)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    e = np.clip(e, -126, 127).astype(np.int64)
    v = np.abs(xb) / np.ldexp(1.0, e)[:, :, None]
    # nearest E2M1 magnitude, ties to the even code (codes 0..7 by magnitude)
    d = np.abs(v[..., None] - E2M1_VALUES)
    best = np.argmin(d, axis=-1)
    dmin = d.min(axis=-1)
    tie = (np.sum(np.isclose(d, dmin[..., None], rtol=0, atol=0), axis=-1) > 1) & (best % 2 == 1)
    code = np.where(tie, best + 1, best)
    code = np.where(v >= 6.0, 7, code).astype(np.uint8)
    code |= np.where(xb < 0, 8, 0).astype(np.uint8)
    code = code.reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def encode(quant: str, x: np.ndarray, side: str):
    """fp32 values -> (codes, scales) for one operand side ('a' or 'b')."""
    if quant == "bf16":
        return to_bf16_bits(x), None
    if quant == "fp16":
        return to_fp16_bits(x), None
    if quant == "fp8_dynamic":
        return quant_rows(x, "fp8")
    if quant == "w8a8_int8":
        return quant_rows(x, "int8")
    if quant == "block_fp8":
        return quant_blocks_act(x) if side == "a" else quant_blocks_weight(x)
    if quant == "mxfp4":
        return (to_bf16_bits(x), None) if side == "a" else quant_mxfp4(x)
    raise ValueError(quant)


def encode16(quant: str, x: np.ndarray) -> np.ndarray:
    """Bias / residual / output codes: fp16 in fp16 mode, else bf16."""
    return to_fp16_bits(x) if quant == "fp16" else to_bf16_bits(x)


# ----------------------------------------------------------------- draws
def _draw(rng, shape, dist, std):
    if dist == "uniform":
        return (rng.random(shape, dtype=np.float32) * 2.0 - 1.0).astype(np.float32)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


@functools.lru_cache(maxsize=4)
def _weight(cfg: int, quant: str):
    c = WORKLOADS[cfg]
    rng = np.random.Generator(np.random.PCG64(1000 * cfg))
    w = _draw(rng, (c["N"], c["K"]), c["dist"], 0.02)
    B, sb = encode(quant, w, "b")
    del w
    bias = None
    if c["bias"]:
        bias = encode16(quant, (rng.random(c["N"], dtype=np.float32) - np.float32(0.5)))
    return B, sb, bias


def make(cfg: int, M: int = None, quant: str = None) -> Problem:
    """The seeded problem of workload ``cfg`` at token count ``M``.

    ``quant`` overrides the workload's quant mode (e.g. fp16 instead of bf16)
    with the same draws.
    """
    c = WORKLOADS[cfg]
    M = c["Ms"][0] if M is None else int(M)
    quant = quant or c["quant"]
    B, sb, bias = _weight(cfg, quant)
    rng = np.random.Generator(np.random.PCG64(1000 * cfg + M))
    a = _draw(rng, (M, c["K"]), c["dist"], 1.0)
    A, sa = encode(quant, a, "a")
    residual = None
    if c["residual"]:
        residual = encode16(quant, rng.standard_normal((M, c["N"]), dtype=np.float32))
    return Problem(quant=quant, act=c["act"], M=M, N=c["N"], K=c["K"], A=A, B=B, sa=sa,
                   sb=sb, bias=bias, residual=residual, alpha=c["alpha"],
                   name=f"{c['name']}_M{M}", meta=dict(cfg=cfg))


def make_custom(quant: str, act: str, M: int, N: int, K: int, seed: int, bias=True,
                residual=False, alpha=1.0, dist="normal", wstd=0.02) -> Problem:
    """A seeded problem of arbitrary shape (edge cases, ragged tails)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = _draw(rng, (N, K), dist, wstd)
    B, sb = encode(quant, w, "b")
    bias_c = encode16(quant, rng.random(N, dtype=np.float32) - np.float32(0.5)) if bias else None
    a = _draw(rng, (M, K), dist, 1.0)
    A, sa = encode(quant, a, "a")
    res_c = encode16(quant, rng.standard_normal((M, N), dtype=np.float32)) if residual else None
    return Problem(quant=quant, act=act, M=M, N=N, K=K, A=A, B=B, sa=sa, sb=sb, bias=bias_c,
                   residual=res_c, alpha=alpha, name=f"{quant}_{act}_{M}x{N}x{K}_s{seed}")


def activations16(M: int, K: int, seed: int, x_dtype: str = "bf16", outliers: bool = True):
    """Seeded 16-bit activations X[M,K] (codes): N(0,1) rows, each scaled by a
    per-row factor drawn log-uniformly in [0.01, 100], with a few large
    outliers per row (up to 20x the row's scale) when ``outliers``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((M, K), dtype=np.float32)
    x *= np.exp(rng.uniform(np.log(0.01), np.log(100.0), (M, 1))).astype(np.float32)
    if outliers and K >= 64:
        for m in range(M):
            idx = rng.integers(0, K, 4)
            x[m, idx] *= rng.uniform(5.0, 20.0, 4).astype(np.float32)
    return to_fp16_bits(x) if x_dtype == "fp16" else to_bf16_bits(x)


def make_grouped(quant: str, act: str, sizes, N: int, K: int, seed: int, bias=True,
                 residual=False):
    """A seeded mixture-of-experts problem: len(sizes) experts, expert e
    receiving sizes[e] tokens (tokens sorted by expert); per-expert weights,
    weight scales and bias.  Returns a dict of codes plus the int32 offsets."""
    rng = np.random.Generator(np.random.PCG64(seed))
    E = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    Bs, sbs, biases = [], [], []
    for _ in range(E):
        B, sb = encode(quant, _draw(rng, (N, K), "normal", 0.02), "b")
        Bs.append(B)
        sbs.append(sb)
        biases.append(encode16(quant, rng.random(N, dtype=np.float32) - np.float32(0.5))
                      if bias else None)
    A, sa = encode(quant, _draw(rng, (max(M, 1), K), "normal", 1.0), "a")
    A = A[:M]
    sa = None if sa is None else sa[:M]
    res = encode16(quant, rng.standard_normal((M, N), dtype=np.float32)) if residual else None
    return dict(quant=quant, act=act, M=M, N=N, K=K, E=E, A=A, Bs=Bs, sa=sa, sbs=sbs,
                biases=biases if bias else None, residual=res, offsets=offsets)


def algorithmic_bytes(quant: str, M: int, N: int, K: int, bias: bool, residual: bool) -> int:
    """Compulsory HBM bytes of one fused call: operands, scales, bias,
    residual and the one output write."""
    e = 2 if quant in ("bf16", "fp16") else 1
    b = M * K * e + N * K * e
    if quant == "mxfp4":  # bf16 activations, 4-bit weights, one E8M0 byte per 32
        b = 2 * M * K + N * K // 2 + N * K // 32
    if quant in ("fp8_dynamic", "w8a8_int8"):
        b += 4 * M + 4 * N
    elif quant == "block_fp8":
        b += 4 * M * (K // 128) + 4 * (N // 128) * (K // 128)
    if bias:
        b += 2 * N
    if residual:
        b += 2 * M * N
    b += 2 * M * N
    return b


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K
