"""Helpers for the GPU parity tests: move a synth.Problem to the device, run
it through the library's C ABI (via the Python binding) and compare with the
oracle under the pass rule |g - r| <= 1e-2 * max(|r|, 1e-3)."""
import numpy as np
import torch

import oracle

RTOL = 1e-2
FLOOR = 1e-3


def dev(a, dtype=None):
    """numpy codes -> CUDA tensor with the same bytes."""
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def upload(p):
    return dict(A=dev(p.A), B=dev(p.B), sa=dev(p.sa), sb=dev(p.sb), bias=dev(p.bias),
                residual=dev(p.residual))


def out_tensor(p, raw=False):
    if raw:
        return torch.empty((p.M, p.N), dtype=torch.int32 if p.quant == "w8a8_int8" else torch.float32,
                           device="cuda")
    return torch.empty((p.M, p.N), dtype=torch.int16, device="cuda")


def run(h, p, d=None, raw=False, C=None):
    d = d or upload(p)
    C = out_tensor(p, raw) if C is None else C
    h.run(d["A"], d["B"], C, quant=p.quant, act="raw_acc" if raw else p.act, sa=d["sa"],
          sb=d["sb"], alpha=p.alpha, bias=d["bias"], residual=d["residual"])
    torch.cuda.synchronize()
    return C


def decode_out(C, quant):
    """Downloaded 16-bit output codes -> float64 (decoded by torch)."""
    c = C.cpu()
    if c.dtype in (torch.int32, torch.float32):
        return c.numpy()
    dt = torch.float16 if quant == "fp16" else torch.bfloat16
    return c.view(dt).to(torch.float64).numpy()


def assert_close(g, r, what=""):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    ok = oracle.within_tolerance(g, r, RTOL, FLOOR)
    if not ok.all():
        bad = np.argwhere(~ok)
        idx = tuple(bad[0]) if g.ndim > 1 else bad[0]
        worst = np.max(np.abs(g - r) / np.maximum(np.abs(r), FLOOR))
        raise AssertionError(f"{what}: {len(bad)} of {g.size} outside the tolerance; first at "
                             f"{idx}: got {g[idx]!r} want {r[idx]!r}; worst rel {worst:.3g}")


def sample_positions(M, N, count, seed=0):
    """Random positions plus the four corners and the last row / column."""
    rng = np.random.default_rng(seed)
    im = rng.integers(0, M, size=count)
    inn = rng.integers(0, N, size=count)
    edge_m = np.array([0, 0, M - 1, M - 1] + [M - 1] * 64 + list(rng.integers(0, M, 64)))
    edge_n = np.array([0, N - 1, 0, N - 1] + list(rng.integers(0, N, 64)) + [N - 1] * 64)
    return np.concatenate([im, edge_m]), np.concatenate([inn, edge_n])


def reference(p, sampled=None):
    """Oracle values: full [M,N] or at sampled (im, inn)."""
    if sampled is None:
        return oracle.linear(p.quant, p.act, **p.operands())
    im, inn = sampled
    return oracle.linear_at(p.quant, p.act, p.A, p.B, im, inn, sa=p.sa, sb=p.sb, bias=p.bias,
                            residual=p.residual, alpha=p.alpha)
