"""Host logic of the offline sweep: merging consecutive token counts with the
same winner into ranged table entries, and the built-in table (the sweep's
compiled-in output plus the defaults) parsing and answering lookups."""
import pytest

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
from epilogue_scaled_gemm_amd.sweep import merge_lines, merge_ranges  # noqa: E402

A = "decode swap=1 split=1 reduce=twopass waves=8 unroll=1 rows=12"
B = "decode swap=1 split=1 reduce=twopass waves=8 unroll=4 rows=24"


def test_merge_ranges_joins_only_consecutive_equal_winners():
    e = [("fp8_dynamic", 1, 6144, 4096, A, 1e-6), ("fp8_dynamic", 2, 6144, 4096, A, 2e-6),
         ("fp8_dynamic", 3, 6144, 4096, B, 3e-6), ("fp8_dynamic", 4, 6144, 4096, A, 4e-6),
         ("fp8_dynamic", 6, 6144, 4096, A, 6e-6),              # gap at 5: a new range
         ("w8a8_int8", 7, 6144, 4096, A, 7e-6)]                # other quant: a new range
    m = merge_ranges(e)
    assert [(q, lo, hi, spec) for q, lo, hi, N, K, spec, _ in m] == [
        ("fp8_dynamic", 1, 2, A), ("fp8_dynamic", 3, 3, B), ("fp8_dynamic", 4, 4, A),
        ("fp8_dynamic", 6, 6, A), ("w8a8_int8", 7, 7, A)]
    assert m[0][6] == [1e-6, 2e-6]


def test_merge_keeps_the_counts_new_entries_do_not_cover():
    # New entries for 17-32 and for 512 alone: the old 17-23 / 24-32 entries
    # go, the old 257-512 entry keeps 257-511, other shapes are untouched.
    old = ["block_fp8    17    23    4096   12288  " + A + "   # 1 us",
           "block_fp8    24    32    4096   12288  " + B,
           "block_fp8    257   512   4096   12288  pp split=4 group=4   # 75 us",
           "block_fp8    1     32    4096   4096   " + A,
           "fp8_dynamic  24    32    4096   12288  " + B]
    new = ["block_fp8    17    32    4096   12288  " + B,
           "block_fp8    512   512   4096   12288  pp split=4 group=4"]
    got = [" ".join(l.split("#")[0].split()) for l in merge_lines(old, new)]
    assert got == ["block_fp8 257 511 4096 12288 pp split=4 group=4",
                   "block_fp8 1 32 4096 4096 " + A,
                   "fp8_dynamic 24 32 4096 12288 " + B,
                   "block_fp8 17 32 4096 12288 " + B,
                   "block_fp8 512 512 4096 12288 pp split=4 group=4"]
    # a new range inside an old one splits it in two
    got = [" ".join(l.split("#")[0].split()) for l in
           merge_lines(["bf16 1 * 64 64 " + A], ["bf16 5 9 64 64 " + B])]
    assert got == ["bf16 1 4 64 64 " + A, "bf16 10 * 64 64 " + A, "bf16 5 9 64 64 " + B]


@pytest.mark.parametrize("quant,N,K", [("fp8_dynamic", 6144, 4096), ("w8a8_int8", 24576, 4096),
                                       ("block_fp8", 4096, 12288), ("mxfp4", 6144, 4096)])
def test_builtin_table_covers_every_decode_token_count(quant, N, K):
    h = lg.Handle()
    try:
        for M in range(1, 33):
            v = h.describe(quant, M, N, K)
            assert v.startswith("decode swap=1"), (M, v)
    finally:
        h.close()
