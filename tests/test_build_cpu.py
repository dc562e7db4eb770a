"""CPU tests of the build's check on inline-asm MFMAs (no GPU needed).

The dK/dV pass issues some MFMAs as inline assembly; the compiler inserts no wait states
around those, so a product whose B operand (accumulation registers) was written by a
v_accvgpr_write just before it reads stale values.  build.py scans the device assembly
for that pattern and fails the build; these tests pin what the scan flags."""

from exact_io_aware_19_amd.build import check_inline_mfma_operands

GOOD = """\tv_accvgpr_write_b32 a10, v3
\tv_add_f32 v1, v2, v3
\ts_waitcnt lgkmcnt(1)
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[48:63], v[2:5], a[184:187], 0
\t;;#ASMEND
"""

BAD = """\tv_accvgpr_write_b32 a186, v183
\tv_accvgpr_write_b32 a187, v182
\ts_waitcnt lgkmcnt(1)
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[48:63], v[2:5], a[184:187], v[48:63]
\t;;#ASMEND
"""

COMPILER_MFMA = """\tv_accvgpr_write_b32 a186, v183
\tv_mfma_f32_32x32x16_bf16 v[48:63], v[2:5], a[184:187], v[48:63]
"""


def test_flags_agpr_write_before_inline_mfma():
    assert len(check_inline_mfma_operands(BAD)) == 1


def test_passes_unrelated_agpr_write():
    assert check_inline_mfma_operands(GOOD) == []


def test_ignores_compiler_scheduled_mfma():
    # products the compiler emits itself get their wait states from the compiler
    assert check_inline_mfma_operands(COMPILER_MFMA) == []


def test_window_bounds_the_search():
    far = BAD.replace("\ts_waitcnt lgkmcnt(1)\n", "".join("\tv_add_f32 v1, v2, v3\n" for _ in range(10)))
    assert check_inline_mfma_operands(far, window=8) == []
    assert len(check_inline_mfma_operands(far, window=16)) == 1
