"""Host logic of the offline sweep: merging consecutive token counts with the
same winner into ranged table entries, and the built-in table (the sweep's
compiled-in output plus the defaults) parsing and answering lookups."""
import pytest

lg = pytest.importorskip("epilogue_scaled_gemm_amd")
from epilogue_scaled_gemm_amd.sweep import merge_ranges  # noqa: E402

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
