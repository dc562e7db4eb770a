"""CPU pins of the FP8 oracle (oracle/fp8.py) against things other than itself.

* E4M3 decode and encode: torch's own float8_e4m3fn conversion (a library routine, run
  here, not copied) on every code and on ties, neighbours of ties, subnormals and
  random values; closed facts of the format (largest finite 448, smallest subnormal
  2^-9, 253 distinct finite values).
* Walsh-Hadamard transform: scipy's Sylvester-Hadamard matrix (library routine), exact
  for integer inputs; H H^T = d I (the transform applied twice returns d x).
* Block / column quantisation: half-ulp error bounds of E4M3, the block maximum mapping
  to +-448 exactly, zero blocks, the rotation leaving Q K^T unchanged up to the factor d
  that goes into Q's scales.
* FP8 attention: the exact attention of the dequantised inputs equals torch's fp64
  scaled-dot-product attention on them; incoherent processing with block scales lowers
  the error against the unquantised inputs on the outlier workload (the direction of
  the pages' FP8 claim, wiki page FA3 (3)).
* Planted mistakes in oracle/fp8.py (a text mutation each) fail at least one pin.
"""

import math
import os
import types

import numpy as np
import pytest
import scipy.linalg
import torch
import torch.nn.functional as F

import oracle
from oracle import fp8 as O
from exact_io_aware_19_amd import workloads as wl

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def encode_probe_values():
    """All finite E4M3 magnitudes, the midpoints between neighbours (ties), one fp32 ulp
    either side of each midpoint, subnormal-range values and log-uniform randoms."""
    vals = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)  # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(0))
    rng = np.random.default_rng(5)
    rnd = np.exp2(rng.uniform(-12, np.log2(448.0), 4000)).astype(np.float32)
    sub = (np.arange(0, 64, dtype=np.float32) * np.float32(2.0 ** -13))
    x = np.concatenate([vals.astype(np.float32), m32, up, dn, rnd, sub])
    x = x[np.abs(x) <= 448]
    return np.concatenate([x, -x]).astype(np.float32)


# ---- pins (each a function so planted mistakes can be run against all of them) ------

def pin_decode_matches_torch(m):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = m.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def pin_format_facts(m):
    v = m.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = v[~np.isnan(v)]
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    assert np.min(fin[fin > 0]) == 2.0 ** -9
    assert len(np.unique(fin)) == 253  # 254 finite codes, +0 and -0 equal
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])


def pin_encode_matches_torch(m):
    x = encode_probe_values()
    assert np.array_equal(m.e4m3_encode(x), torch_encode(x))


def pin_encode_roundtrip(m):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(m.e4m3_encode(m.e4m3_decode(codes).astype(np.float32)), codes)


def pin_fwht_is_hadamard(m):
    rng = np.random.default_rng(11)
    for d in (64, 128):
        Hd = scipy.linalg.hadamard(d)
        signs = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0).astype(np.float32)
        xi = rng.integers(-50, 50, size=(7, d)).astype(np.float32)  # exact in fp32
        assert np.array_equal(m.fwht_fp32(xi, signs), ((xi * signs) @ Hd).astype(np.float32))
        xr = rng.standard_normal((5, d)).astype(np.float32)
        ref = (xr.astype(np.float64) * signs) @ Hd
        assert np.max(np.abs(m.fwht_fp32(xr, signs) - ref)) < 1e-4 * np.max(np.abs(ref))


def pin_fwht_involution(m):
    rng = np.random.default_rng(12)
    for d in (64, 128):
        x = rng.integers(-8, 8, size=(3, d)).astype(np.float32)
        assert np.array_equal(m.fwht_fp32(m.fwht_fp32(x)), d * x)


def pin_block_quant_bounds(m):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, 2, 200, 64)).astype(np.float32) * np.float32(3.0)
    x[0, 1, 64:128] = 0.0  # one all-zero block
    codes, sc = m.quantize_blocks(x)
    assert sc.shape == (1, 2, 4) and sc[0, 1, 1] == 0.0 and not codes[0, 1, 64:128].any()
    deq = m.dequantize_blocks(codes, sc)
    s_rows = np.repeat(sc.astype(np.float64), 64, axis=2)[:, :, :200, None]
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s_rows) * (1 + 1e-6))
    for hh in range(2):
        for b in range(4):
            if sc[0, hh, b] > 0:
                blk = m.e4m3_decode(codes[0, hh, 64 * b:64 * (b + 1)])
                assert np.max(np.abs(blk)) == 448.0
                assert np.isclose(sc[0, hh, b] * 448.0, np.abs(x[0, hh, 64 * b:64 * (b + 1)]).max(), rtol=1e-6)


def pin_column_quant_bounds(m):
    rng = np.random.default_rng(14)
    x = rng.standard_normal((1, 2, 130, 64)).astype(np.float32)
    x[..., 5] *= 100.0  # an outlier column gets its own scale
    codes, sc = m.quantize_columns(x)
    assert sc.shape == (1, 2, 64)
    assert np.allclose(sc * 448.0, np.abs(x).max(axis=2), rtol=1e-6)
    deq = m.dequantize_columns(codes, sc)
    err = np.abs(deq - x)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc[:, :, None, :]) * (1 + 1e-6))


def pin_rotation_preserves_scores(m):
    rng = np.random.default_rng(15)
    d = 128
    signs = wl.fp8_signs(d, 3)
    q = rng.standard_normal((1, 1, 96, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, 96, d)).astype(np.float32)
    qr, kr = m.fwht_fp32(q, signs), m.fwht_fp32(k, signs)
    ref = q[0, 0].astype(np.float64) @ k[0, 0].T.astype(np.float64)
    got = qr[0, 0].astype(np.float64) @ kr[0, 0].T.astype(np.float64) / d
    assert np.max(np.abs(got - ref)) < 1e-4
    # quantised: Q's post scale 1/d makes the dequantised product approximate Q K^T
    q8, sq = m.quantize_blocks(q, signs, post_scale=1.0 / d)
    k8, sk = m.quantize_blocks(k, signs)
    deq = m.dequantize_blocks(q8, sq)[0, 0] @ m.dequantize_blocks(k8, sk)[0, 0].T
    # rigorous bound: each factor is within half an E4M3 ulp (2^-4 relative) of the
    # rotated value or within half a subnormal step (2^-10 code units) of it
    aq = np.abs(qr[0, 0]).astype(np.float64) / d
    ak = np.abs(kr[0, 0]).astype(np.float64)
    eq = 2.0 ** -4 * aq + 2.0 ** -10 * float(sq.max())
    ek = 2.0 ** -4 * ak + 2.0 ** -10 * float(sk.max())
    bound = eq @ ak.T + aq @ ek.T + eq @ ek.T + 1e-4
    assert np.all(np.abs(deq - ref) <= bound)
    assert np.corrcoef(deq.ravel(), ref.ravel())[0, 1] > 0.999


def pin_fp8_attention_is_exact_attention(m):
    rng = np.random.default_rng(16)
    B, H, N, d = 1, 2, 70, 64
    q8 = rng.integers(0, 0x7E, size=(B, H, N, d)).astype(np.uint8) | (rng.integers(0, 2, (B, H, N, d)) << 7).astype(np.uint8)
    k8 = rng.integers(0x20, 0x50, size=(B, H, N, d)).astype(np.uint8)
    v8 = rng.integers(0, 0x7E, size=(B, H, N, d)).astype(np.uint8)
    sq = np.exp2(rng.integers(-8, -4, size=(B, H, 2))).astype(np.float32)
    sk = np.exp2(rng.integers(-6, -3, size=(B, H, 2))).astype(np.float32)
    sv = np.exp2(rng.integers(-9, -5, size=(B, H, d))).astype(np.float32)
    for causal in (False, True):
        o, lse = m.attention_forward_fp8(q8, sq, k8, sk, v8, sv, 0.125, causal=causal)
        qd = torch.from_numpy(m.e4m3_decode(q8) * np.repeat(sq, 64, axis=2)[:, :, :N, None])
        kd = torch.from_numpy(m.e4m3_decode(k8) * np.repeat(sk, 64, axis=2)[:, :, :N, None])
        vd = torch.from_numpy(m.e4m3_decode(v8) * sv[:, :, None, :])
        ref = F.scaled_dot_product_attention(qd, kd, vd, is_causal=causal, scale=0.125)
        assert np.max(np.abs(o - ref.numpy())) < 1e-12
        s = 0.125 * (qd @ kd.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
        assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


PINS = [pin_decode_matches_torch, pin_format_facts, pin_encode_matches_torch, pin_encode_roundtrip,
        pin_fwht_is_hadamard, pin_fwht_involution, pin_block_quant_bounds, pin_column_quant_bounds,
        pin_rotation_preserves_scores, pin_fp8_attention_is_exact_attention]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_fp8_oracle_pin(pin):
    pin(O)


def test_incoherent_processing_lowers_error_on_outliers():
    """Block scales + Hadamard rotation vs. one scale per head and no rotation (the
    baseline FP8), both measured against exact attention of the unquantised inputs."""
    w = wl.get_workload("fp8_outlier")
    inp = wl.generate(w)
    q, k, v = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v"))
    d = w.d
    ref_o, _ = oracle.ref.attention_forward(q[:, :2], k[:, :2], v[:, :2], w.scale)
    signs = wl.fp8_signs(d, w.seed)
    v8, sv = O.quantize_columns(v[:, :2])
    q8, sq = O.quantize_blocks(q[:, :2], signs, post_scale=1.0 / d)
    k8, sk = O.quantize_blocks(k[:, :2], signs)
    o_ip, _ = O.attention_forward_fp8(q8, sq, k8, sk, v8, sv, w.scale)
    # baseline: per-head scales (a block as long as the head), no rotation
    N = w.N
    q8b, sqb = O.quantize_blocks(q[:, :2], block=N)
    k8b, skb = O.quantize_blocks(k[:, :2], block=N)
    qb = O.dequantize_blocks(q8b, sqb, block=N)
    kb = O.dequantize_blocks(k8b, skb, block=N)
    o_base, _ = oracle.ref.attention_forward(qb, kb, O.dequantize_columns(v8, sv), w.scale)
    rmse_ip = np.sqrt(np.mean((o_ip - ref_o) ** 2))
    rmse_base = np.sqrt(np.mean((o_base - ref_o) ** 2))
    print(f"RMSE baseline {rmse_base:.3e}  block+rotation {rmse_ip:.3e}  ratio {rmse_base / rmse_ip:.2f}")
    assert rmse_ip < rmse_base


MUTATIONS = {
    "encode_truncates": ("r = (abits + 0x7FFFF + lsb) & ~np.uint64(0xFFFFF)", "r = abits & ~np.uint64(0xFFFFF)"),
    "encode_bias_8": ("exp = (r >> 23).astype(np.int64) - 127 + 7", "exp = (r >> 23).astype(np.int64) - 127 + 8"),
    "encode_ties_away": ("sub_code = np.rint(a.astype(np.float64) * 512.0)",
                         "sub_code = np.floor(a.astype(np.float64) * 512.0 + 0.5)"),
    "decode_bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "decode_subnormal_scale": ("m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    "fwht_minus_swapped": ("v[..., 1, :] = a - b", "v[..., 1, :] = b - a"),
    "fwht_last_stage_dropped": ("while h < d:", "while h < d // 2:"),
    "signs_ignored": ("y = (y * np.asarray(signs, dtype=np.float32)).astype(np.float32)", "y = y"),
    "scale_inverted": ("scale = np.where(nz, safe / np.float32(E4M3_MAX)", "scale = np.where(nz, np.float32(E4M3_MAX) / safe"),
    "post_scale_dropped": ("scale = (scale * np.float32(post_scale)).astype(np.float32)", "scale = scale"),
    "column_amax_over_columns": ("amax = np.abs(y).max(axis=2)  # [B,H,d]", "amax = np.abs(y).max(axis=3)[:, :, :, None].repeat(y.shape[3], axis=3)[:, :, 0, :]"),
    "v_scales_dropped": ("return e4m3_decode(codes) * np.asarray(scales, np.float64)[:, :, None, :]",
                         "return e4m3_decode(codes)"),
}


def _mutant(name):
    src = open(os.path.join(ORACLE_DIR, "fp8.py")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation {name}: pattern not found exactly once"
    mod = types.ModuleType(f"oracle.fp8_mut_{name}")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), f"fp8_{name}.py", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_fp8_mistake_is_caught(name):
    m = _mutant(name)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
