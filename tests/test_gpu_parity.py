"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
seeded workloads at their real sizes and on ragged shapes.

Bar: int8 raw int32 accumulators bit-exact; every floating-point output
within |g - r| <= 1e-2 * max(|r|, 1e-3) of the oracle's fp64 value.  The
largest shapes (block FP8 at M = 2048, the 4096^3 prefill) are checked at
sampled positions (plus corners and the last row / column) in the same
launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import synth
import oracle
from gpu_util import assert_close, decode_out, reference, run, sample_positions, upload

pytestmark = pytest.mark.gpu

lg = pytest.importorskip("epilogue_scaled_gemm_amd")


@pytest.fixture(scope="module")
def handle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h = lg.Handle()
    yield h
    h.close()


CASES = [(1, 64)] + [(2, m) for m in synth.WORKLOADS[2]["Ms"]] + \
        [(3, m) for m in synth.WORKLOADS[3]["Ms"]] + [(4, m) for m in synth.WORKLOADS[4]["Ms"]] + \
        [(5, 4096)]
SAMPLED = {(4, 2048), (5, 4096)}


@pytest.mark.parametrize("cfg,M", CASES, ids=[f"cfg{c}-M{m}" for c, m in CASES])
def test_workload_parity(handle, cfg, M):
    p = synth.make(cfg, M)
    print(f"[parity] {p.name} variant={handle.describe(p.quant, p.M, p.N, p.K)}", flush=True)
    C = run(handle, p)
    g = decode_out(C, p.quant)
    if (cfg, M) in SAMPLED:
        im, inn = sample_positions(p.M, p.N, 6000, seed=cfg)
        r, _ = reference(p, (im, inn))
        assert_close(g[im, inn], r, p.name)
    else:
        r, _ = reference(p)
        assert_close(g, r, p.name)


@pytest.mark.parametrize("M", synth.WORKLOADS[3]["Ms"])
def test_int8_accumulator_bit_exact(handle, M):
    p = synth.make(3, M)
    C = run(handle, p, raw=True)
    _, acc = oracle.linear(p.quant, "none", p.A, p.B, p.sa, p.sb)
    assert np.array_equal(C.cpu().numpy(), acc)


RAGGED = [
    ("bf16", "gelu_tanh", 100, 272, 336, True, True, 0.5),
    ("fp16", "relu", 77, 144, 264, True, True, 1.0),
    ("fp8_dynamic", "silu", 129, 200, 400, True, False, 1.0),
    ("w8a8_int8", "silu", 65, 48, 4112, False, True, 2.0),
    ("block_fp8", "gelu_tanh", 70, 384, 640, True, True, 0.5),
    ("bf16", "none", 33, 40, 8, False, False, 1.0),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"{c[0]}-{c[2]}x{c[3]}x{c[4]}" for c in RAGGED])
def test_ragged_default_variant(handle, case):
    quant, act, M, N, K, bias, res, alpha = case
    p = synth.make_custom(quant, act, M, N, K, seed=M + N + K, bias=bias, residual=res,
                          alpha=alpha)
    C = run(handle, p)
    r, _ = reference(p)
    assert_close(decode_out(C, quant), r, p.name)


def test_zero_m_is_noop(handle):
    p = synth.make_custom("bf16", "none", 4, 32, 64, seed=1)
    d = upload(p)
    C = torch.full((4, 32), 1234, dtype=torch.int16, device="cuda")
    handle.run(d["A"][:0], d["B"], C, quant="bf16", act="none", M=0)
    torch.cuda.synchronize()
    assert bool((C == 1234).all())


@pytest.mark.parametrize("spec", [None, "tile bm=64 bn=128 wm=1 wn=4",
                                  "decode swap=0 split=2 reduce=twopass waves=8 unroll=2"])
def test_e4m3_every_code_through_the_path(handle, spec):
    # A holds every finite e4m3 code; B is the identity (1.0 = 0x38), unit
    # scales, raw accumulator: C must equal the exact decoded codes.
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0, 0], np.uint8)
    K = codes.size  # 256
    M = 1 if spec is None or spec.startswith("decode") else 40
    A = np.tile(codes, (M, 1))
    B = np.zeros((K, K), np.uint8)
    B[np.arange(K), np.arange(K)] = 0x38
    ones_m, ones_k = np.ones(M, np.float32), np.ones(K, np.float32)
    p = synth.Problem(quant="fp8_dynamic", act="none", M=M, N=K, K=K, A=A, B=B, sa=ones_m,
                      sb=ones_k)
    try:
        handle.set_force(spec)
        C = run(handle, p, raw=True)
    finally:
        handle.set_force(None)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(C.cpu().numpy(), np.tile(want, (M, 1)))


KMAX_I8 = 131056  # the largest K (a multiple of 16) the int8 mode accepts


@pytest.mark.parametrize("M,spec", [
    (2, None),
    (2, "decode swap=1 split=4 reduce=atomic waves=8 unroll=2 rows=16"),
    (2, "decode swap=1 split=8 reduce=twopass waves=4 unroll=4 rows=16"),
    (2, "decode swap=0 split=2 reduce=lastwg waves=8 unroll=2"),
    (40, "tile bm=64 bn=128 wm=1 wn=4"),
    (256, "pp group=4"),
])
def test_int8_accumulator_at_maximum_k(handle, M, spec):
    # +-127 codes at the largest K: accumulators reach +-127^2 K = +-2,113,802,224
    # (just inside int32).  Rows 0 / 1 of A and B are all +127 / all -127,
    # the rest random signs; raw int32 accumulators compared exactly, on every
    # output for the small shapes and on sampled outputs for M = 256.
    N, K = (64 if M < 256 else 256), KMAX_I8
    rng = np.random.default_rng(M)
    A = (rng.choice([-127, 127], (M, K))).astype(np.int8)
    B = (rng.choice([-127, 127], (N, K))).astype(np.int8)
    A[0], A[1], B[0], B[1] = 127, -127, 127, -127
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    p = synth.Problem(quant="w8a8_int8", act="none", M=M, N=N, K=K, A=A, B=B, sa=ones_m,
                      sb=ones_n)
    print(f"[kmax] M={M} spec={spec}", flush=True)
    try:
        handle.set_force(spec)
        C = run(handle, p, raw=True).cpu().numpy()
    finally:
        handle.set_force(None)
    top = 127 * 127 * K
    assert C[0, 0] == top and C[1, 1] == top and C[0, 1] == -top
    if M < 256:
        _, acc = oracle.linear("w8a8_int8", "none", A, B, ones_m, ones_n)
        assert np.array_equal(C, acc)
    else:
        im, inn = sample_positions(M, N, 300, seed=3)
        _, acc = oracle.linear_at("w8a8_int8", "none", A, B, im, inn, ones_m, ones_n)
        assert np.array_equal(C[im, inn], acc)


def test_large_m_default_path(handle):
    # 65536 tokens through the default prefill choice (the ping-pong family,
    # 256 row tiles of one column tile): sampled outputs, corners and the last
    # row against the oracle.
    p = synth.make_custom("bf16", "gelu_tanh", 65536, 256, 64, seed=17, bias=True, residual=True)
    print(f"[parity] {p.name} variant={handle.describe(p.quant, p.M, p.N, p.K)}", flush=True)
    C = run(handle, p)
    im, inn = sample_positions(p.M, p.N, 4000, seed=17)
    r, _ = reference(p, (im, inn))
    assert_close(decode_out(C, p.quant)[im, inn], r, p.name)


# Whole output tiles at full size, in the launch configuration the benchmark
# times: the kernel's tile (256 x 256 for the bf16 prefill, 256 x 128 for
# block FP8 at 2048 tokens) is compared element by element at the first, an
# interior and the last tile position (the last one holds the grid's final
# rows and columns).
FULL_TILES = [(5, 4096, 256, 256, [(0, 0), (7, 9), (15, 15)]),
              (4, 2048, 256, 128, [(0, 0), (3, 17), (7, 31)])]


@pytest.mark.parametrize("cfg,M,TM,TN,tiles", FULL_TILES, ids=["prefill-4096", "block_fp8-2048"])
def test_full_tiles_at_full_size(handle, cfg, M, TM, TN, tiles):
    p = synth.make(cfg, M)
    print(f"[tiles] {p.name} variant={handle.describe(p.quant, p.M, p.N, p.K)}", flush=True)
    C = run(handle, p)
    g = decode_out(C, p.quant)
    for tm, tn in tiles:
        m0, n0 = tm * TM, tn * TN
        assert m0 + TM <= p.M and n0 + TN <= p.N
        mm, nn = np.meshgrid(np.arange(m0, m0 + TM), np.arange(n0, n0 + TN), indexing="ij")
        im, inn = mm.ravel(), nn.ravel()
        r, _ = reference(p, (im, inn))
        assert_close(g[im, inn], r, f"{p.name} tile ({tm}, {tn})")
