"""CPU tests of the Python binding's argument checks for the FP8 calls: every check runs
on the host before the library is called, so wrong dtypes, shapes, layouts and devices
raise here without a GPU."""

import pytest
import torch

import exact_io_aware_19_amd as fa

B, H, N, d = 1, 2, 100, 64
NB = -(-N // 64)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def test_quantize_qk_rejects_bad_inputs():
    with pytest.raises(TypeError):
        fa.fa_fp8_quantize_qk(f32(B, H, N, d), u8(B, H, N, d), f32(B, H, NB))
    with pytest.raises(ValueError):
        fa.fa_fp8_quantize_qk(bf16(B, H, N), u8(B, H, N, d), f32(B, H, NB))
    with pytest.raises(ValueError):  # not on the GPU
        fa.fa_fp8_quantize_qk(bf16(B, H, N, d), u8(B, H, N, d), f32(B, H, NB))
    with pytest.raises(ValueError):  # transposed view
        fa.fa_fp8_quantize_qk(bf16(B, H, d, N).transpose(2, 3), u8(B, H, N, d), f32(B, H, NB))


def test_quantize_v_and_forward_reject_bad_inputs():
    with pytest.raises(ValueError):
        fa.fa_fp8_quantize_v(bf16(B, H, N, d), u8(B, H, NB, d, 64), f32(B, H, d))
    with pytest.raises(TypeError):
        fa.fa_forward_fp8(u8(B, H, N, d), f32(B, H, NB), u8(B, H, N, d), f32(B, H, NB), u8(B, H, NB, d, 64),
                          f32(B, H, d), f32(B, H, N, d), f32(B, H, N), 0.125, False)
    with pytest.raises(ValueError):
        fa.fa_forward_fp8(u8(B, H, N, d), f32(B, H, NB), u8(B, H, N, d), f32(B, H, NB), u8(B, H, NB, d, 64),
                          f32(B, H, d), bf16(B, H, N, d), f32(B, H, N), 0.125, False)


def test_v8t_to_rows_inverts_the_documented_layout():
    """fp8_v8t_to_rows is index bookkeeping of the documented V^T layout: byte 32*g + p of
    row c of tile t holds key 64 t + 32 (p // 16) + 8 ((p % 16) // 4) + 4 g + p % 4."""
    nb, dd = 2, 8
    v8t = torch.empty((1, 1, nb, dd, 64), dtype=torch.uint8)
    for t in range(nb):
        for c in range(dd):
            for g in range(2):
                for p in range(32):
                    key = 64 * t + 32 * (p // 16) + 8 * ((p % 16) // 4) + 4 * g + p % 4
                    v8t[0, 0, t, c, 32 * g + p] = (key * 7 + c) % 251
    rows = fa.fp8_v8t_to_rows(v8t, 100)
    assert rows.shape == (1, 1, 100, dd)
    for key in range(100):
        for c in range(dd):
            assert int(rows[0, 0, key, c]) == (key * 7 + c) % 251
