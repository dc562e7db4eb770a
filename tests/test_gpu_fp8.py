"""GPU parity of the FP8 path (quantisers and forward) against the fp64 oracle.

Quantisers: bit-exact.  The codes are integers decided by fp32 arithmetic that both
sides do in the same order (one multiply by 448/amax; the Walsh-Hadamard butterflies in
a fixed order), so every code and every scale must match oracle/fp8.py exactly.

Forward: the oracle is exact fp64 attention of the dequantised inputs (the oracle's own
codes, which the quantiser test shows equal the GPU's).  The GPU rounds P to E4M3 before
P V; that is the one rounding beyond fp32 accumulation and the bf16 output, so the
tolerance is derived from it, per element:
    |dO_ic| <= 2^-4 sum_j p_ij |v_jc|  +  sum_j min(p_ij, 2^-14 max_k p_ik) |v_jc|
               +  2^-8 |O_ic|  + 1e-5
(half an E4M3 ulp relative for normal P; for subnormal P the rounding error is at most
the value itself and at most half a subnormal step, 2^-10, divided by the row sum L_i of
the biased P -- the largest biased P of a row is at least 2^4 and equals max_k p_ik L_i,
so 2^-10 / L_i <= 2^-14 max_k p_ik; bf16 output rounding).  The subnormal term thus
scales with the row's largest probability, not with N.  The tests also require the
relative Frobenius error of O to stay below 5e-2: E4M3's relative rounding error has an
RMS of about 2^-4 / sqrt(3) ~ 3.6% per P element, and O's error is a p-weighted average of
such errors on random-sign values, of the same relative size as O.
LSE uses the unrounded P and must match to 1e-3 like the bf16 path.

The scores carry one more error: the fp8 matrix product does not sum its 64 products in
full fp32 precision.  Measured on gfx950 (tests/test_gpu_micro.py, which also asserts
it), the sum of one 32x32x64 product is off by at most 2^-11.8 of its largest |term|,
also when that term cancels; fp32 would be within 2^-18.  So each score may be off by
    delta_i = 2^-10 * scale * max_k |q_ik| * max_j,k |k_jk|   (dequantised; 3.6x margin)
which bounds the LSE error by delta_i and moves every P by a factor within e^(+-2 delta_i):
the tests allow |dLSE_i| <= 1e-3 + delta_i, add (e^(2 delta_i) - 1) sum_j p_ij |v_jc|
to the bound on O and widen its subnormal term by the same factor e^(2 delta_i) (the
kernel's own P and row maximum are off from the exact ones by at most that factor).  For inputs of unit size delta is a few 1e-4; it matters where one
product dominates a score of hundreds (tests/test_gpu_rescale.py).
"""

import math

import numpy as np
import pytest
import torch

import exact_io_aware_19_amd as fa
from exact_io_aware_19_amd import workloads as wl
from oracle import fp8 as O
from oracle import ref

pytestmark = pytest.mark.gpu


def _u8(t):
    return t.cpu().numpy()


def _setup(gpu, w, shape=None):
    inp = wl.generate(w, with_do=False, shape_override=shape)
    t = inp.to_torch(gpu)
    B, H, N, d = shape or w.shape
    signs = wl.fp8_signs(d, w.seed)
    return inp, t, (B, H, N, d), signs


def _quantize_gpu(gpu, t, shape, signs):
    B, H, N, d = shape
    nb = -(-N // 64)
    out = {}
    st = torch.from_numpy(signs).to(gpu) if signs is not None else None
    for name, post in (("q", 1.0 / d if signs is not None else 1.0), ("k", 1.0)):
        x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=gpu)
        sc = torch.empty((B, H, nb), dtype=torch.float32, device=gpu)
        fa.fa_fp8_quantize_qk(t[name], x8, sc, st, post)
        out[name] = (x8, sc)
    v8t = torch.full((B, H, nb, d, 64), 0xAB, dtype=torch.uint8, device=gpu)  # padding must be overwritten
    sv = torch.empty((B, H, d), dtype=torch.float32, device=gpu)
    fa.fa_fp8_quantize_v(t["v"], v8t, sv)
    out["v"] = (v8t, sv)
    torch.cuda.synchronize()
    return out


def _quantize_oracle(inp, signs, d):
    q, k, v = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v"))
    q8, sq = O.quantize_blocks(q, signs, post_scale=1.0 / d if signs is not None else 1.0)
    k8, sk = O.quantize_blocks(k, signs)
    v8, sv = O.quantize_columns(v)
    return (q8, sq), (k8, sk), (v8, sv)


CASES = [("fp8_outlier", None, True), ("fp8_outlier", None, False), ("tiny", (1, 2, 200, 64), True),
         ("gpt2", (1, 2, 300, 64), False)]


@pytest.mark.parametrize("name,shape,rotate", CASES)
def test_quantizers_bit_exact(gpu, name, shape, rotate):
    w = wl.get_workload(name)
    inp, t, shp, signs = _setup(gpu, w, shape)
    signs = signs if rotate else None
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, shp[3])
    assert np.array_equal(_u8(g["q"][0]), q8), "Q codes differ"
    assert np.array_equal(g["q"][1].cpu().numpy(), sq), "Q scales differ"
    assert np.array_equal(_u8(g["k"][0]), k8), "K codes differ"
    assert np.array_equal(g["k"][1].cpu().numpy(), sk), "K scales differ"
    rows = fa.fp8_v8t_to_rows(g["v"][0], shp[2])
    assert np.array_equal(_u8(rows), v8), "V codes differ"
    assert np.array_equal(g["v"][1].cpu().numpy(), sv), "V scales differ"
    # keys past N in the last transposed tile hold code 0
    full = fa.fp8_v8t_to_rows(g["v"][0], g["v"][0].shape[2] * 64)
    assert not _u8(full[:, :, shp[2]:]).any()


def _check_forward(o_gpu, lse_gpu, qd, kd, vd, scale, causal, kv_len, rows=None):
    """Compare GPU rows with the oracle on the dequantised inputs, using the bounds of the
    module docstring; returns (max |dO| / bound, O rel. Frobenius error, max |dLSE| /
    (1e-3 + delta)) -- the last is at most 1 when LSE is within its bound."""
    B, H, N, d = qd.shape
    worst, num, den, lerr = 0.0, 0.0, 0.0, 0.0
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            r = np.arange(N) if rows is None else rows
            s = scale * (qd[b, h, r] @ kd[b, h].T)
            ok = ref.admissible(r, N, causal, kl)
            s = np.where(ok, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.where(ok, np.exp(s - m), 0.0)
            lse = m[:, 0] + np.log(e.sum(axis=1))
            p = e / e.sum(axis=1, keepdims=True)
            o = p @ vd[b, h]
            kmax = np.abs(kd[b, h]).max(axis=1)
            kmax_adm = np.where(ok, kmax[None, :], 0.0).max(axis=1) if ok.shape[1] else np.zeros(len(r))
            delta = 2.0 ** -10 * abs(scale) * np.abs(qd[b, h, r]).max(axis=1) * kmax_adm
            pv = p @ np.abs(vd[b, h])
            sub = np.minimum(p, 2.0 ** -14 * p.max(axis=1, keepdims=True)) * np.exp(2 * delta)[:, None]
            bound = 2.0 ** -4 * pv + np.expm1(2 * delta)[:, None] * pv + sub @ np.abs(vd[b, h]) + \
                2.0 ** -8 * np.abs(o) + 1e-5
            og = o_gpu[b, h, r]
            worst = max(worst, float(np.max(np.abs(og - o) / bound)))
            num += float(np.sum((og - o) ** 2))
            den += float(np.sum(o ** 2))
            with np.errstate(invalid="ignore"):
                dl = np.abs(lse_gpu[b, h, r] - lse)
            dl = np.where(np.isneginf(lse) & np.isneginf(lse_gpu[b, h, r]), 0.0, dl)
            lerr = max(lerr, float(np.max(dl / (1e-3 + delta))))
    return worst, math.sqrt(num / den), lerr


def _run_forward(gpu, g, shp, scale, causal, kv_len=None):
    B, H, N, d = shp
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=gpu)
    fa.fa_forward_fp8(g["q"][0], g["q"][1], g["k"][0], g["k"][1], g["v"][0], g["v"][1], o, lse, scale, causal,
                      kv_len=kv_len)
    torch.cuda.synchronize()
    of = o.float().cpu().numpy().astype(np.float64)
    return of, lse.cpu().numpy().astype(np.float64)


FWD_CASES = [("fp8_outlier", None, False, True, False), ("fp8_outlier", None, True, True, False),
             ("tiny", (1, 2, 200, 64), False, False, False), ("gpt2", (1, 2, 300, 64), True, True, False),
             ("bert_large", (2, 2, 200, 64), False, True, True), ("sweep_n2048_full", (1, 2, 700, 128), True, False, True)]


@pytest.mark.parametrize("name,shape,causal,rotate,padded", FWD_CASES)
def test_forward_fp8_parity(gpu, name, shape, causal, rotate, padded):
    w = wl.get_workload(name)
    inp, t, shp, signs = _setup(gpu, w, shape)
    signs = signs if rotate else None
    B, H, N, d = shp
    kv = None
    kvt = None
    if padded:
        kv = np.random.default_rng(77).integers(N // 3, N, size=B, endpoint=True).astype(np.int32)
        kvt = torch.from_numpy(kv).to(gpu)
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, d)
    assert np.array_equal(_u8(g["q"][0]), q8) and np.array_equal(_u8(g["k"][0]), k8)
    of, lg = _run_forward(gpu, g, shp, w.scale, causal, kvt)
    qd, kd, vd = O.dequantize_blocks(q8, sq), O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of, lg, qd, kd, vd, w.scale, causal, kv)
    print(f"{name} {shp} causal={causal} rotate={rotate} padded={padded}: "
          f"max |dO|/bound {worst:.3f}  O rel-Frobenius {rel:.3e}  |dLSE|/bound {lerr:.3f}", flush=True)
    assert worst <= 1.0 and rel <= 5e-2
    assert lerr <= 1.0
    assert np.all(np.isfinite(of))


def test_fp8_rotation_lowers_error_on_outliers(gpu):
    """Block scales + incoherent processing against the baseline FP8 (one scale per head,
    no rotation; codes from the oracle's quantiser), both through the GPU kernel, both
    against exact attention of the unquantised bf16 inputs."""
    w = wl.get_workload("fp8_outlier")
    inp, t, shp, signs = _setup(gpu, w)
    B, H, N, d = shp
    q, k, v = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v"))
    o_exact, _ = ref.attention_forward(q, k, v, w.scale)
    g = _quantize_gpu(gpu, t, shp, signs)
    o_ip, _ = _run_forward(gpu, g, shp, w.scale, False)
    nb = -(-N // 64)
    q8b, sqb = O.quantize_blocks(q, block=N)
    k8b, skb = O.quantize_blocks(k, block=N)
    gb = dict(g)
    gb["q"] = (torch.from_numpy(q8b).to(gpu), torch.from_numpy(np.repeat(sqb, nb, axis=2).copy()).to(gpu))
    gb["k"] = (torch.from_numpy(k8b).to(gpu), torch.from_numpy(np.repeat(skb, nb, axis=2).copy()).to(gpu))
    o_base, _ = _run_forward(gpu, gb, shp, w.scale, False)
    r_ip = math.sqrt(np.mean((o_ip - o_exact) ** 2))
    r_base = math.sqrt(np.mean((o_base - o_exact) ** 2))
    print(f"GPU FP8 RMSE vs exact: baseline {r_base:.3e}, block+rotation {r_ip:.3e}, ratio {r_base / r_ip:.2f}",
          flush=True)
    assert r_ip < r_base


@pytest.mark.parametrize("causal", [False, True])
def test_forward_fp8_full_size_sampled_rows(gpu, causal):
    """The bench configuration (B=2, H=16, N=8192, d=128, incoherent processing), in the
    launch configuration bench.py times: 48 sampled rows per head checked with the bound."""
    w = wl.get_workload("sweep_n8192_full")
    inp, t, shp, signs = _setup(gpu, w)
    B, H, N, d = shp
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, d)
    assert np.array_equal(_u8(g["q"][0]), q8) and np.array_equal(_u8(g["k"][0]), k8)
    assert np.array_equal(_u8(fa.fp8_v8t_to_rows(g["v"][0], N)), v8)
    of, lg = _run_forward(gpu, g, shp, w.scale, causal)
    rows = np.sort(np.random.default_rng(4242).choice(N, size=48, replace=False))
    rows = np.unique(np.concatenate([rows, [0, N - 1]]))
    qd = O.dequantize_blocks(q8, sq)
    kd, vd = O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of, lg, qd, kd, vd, w.scale, causal, None, rows=rows)
    print(f"full size causal={causal}: max |dO|/bound {worst:.3f}  O rel-Frobenius {rel:.3e}  |dLSE|/bound {lerr:.3f}",
          flush=True)
    assert worst <= 1.0 and rel <= 5e-2 and lerr <= 1.0


def test_forward_fp8_deterministic(gpu):
    w = wl.get_workload("fp8_outlier")
    _, t, shp, signs = _setup(gpu, w)
    g = _quantize_gpu(gpu, t, shp, signs)
    a, la = _run_forward(gpu, g, shp, w.scale, True)
    b, lb = _run_forward(gpu, g, shp, w.scale, True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_forward_fp8_long_context_sampled_rows(gpu):
    """The long-context workload (B=1, H=16, N=65536, d=64, causal, 1% of key rows x8:
    large jumps of the running max) through the FP8 path with incoherent processing,
    quantisers bit-exact at full size, the forward checked on the workload's 64 sampled
    rows (plus the first and last) with the bound of the module docstring."""
    w = wl.get_workload("long_64k")
    inp, t, shp, signs = _setup(gpu, w)
    B, H, N, d = shp
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, d)
    assert np.array_equal(_u8(g["q"][0]), q8) and np.array_equal(_u8(g["k"][0]), k8)
    assert np.array_equal(g["q"][1].cpu().numpy(), sq) and np.array_equal(g["k"][1].cpu().numpy(), sk)
    assert np.array_equal(_u8(fa.fp8_v8t_to_rows(g["v"][0], N)), v8)
    of, lg = _run_forward(gpu, g, shp, w.scale, True)
    rows = np.unique(np.concatenate([inp.rows, [0, N - 1]]))
    qd = O.dequantize_blocks(q8, sq)
    kd, vd = O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of, lg, qd, kd, vd, w.scale, True, None, rows=rows)
    print(f"long context: max |dO|/bound {worst:.3f}  O rel-Frobenius {rel:.3e}  |dLSE|/bound {lerr:.3f}", flush=True)
    assert worst <= 1.0 and rel <= 5e-2 and lerr <= 1.0


@pytest.mark.parametrize("N", [1, 17, 64, 65])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_fp8_edge_sizes(gpu, N, d, causal):
    """Degenerate and ragged lengths (one key, less than a tile, exactly one tile, one key
    into a second tile), both head dims, both masks."""
    w = wl.get_workload("fp8_outlier")
    inp, t, shp, signs = _setup(gpu, w, (1, 2, N, d))
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, d)
    assert np.array_equal(_u8(g["q"][0]), q8) and np.array_equal(_u8(g["k"][0]), k8)
    assert np.array_equal(_u8(fa.fp8_v8t_to_rows(g["v"][0], N)), v8)
    of, lg = _run_forward(gpu, g, shp, w.scale, causal)
    qd, kd, vd = O.dequantize_blocks(q8, sq), O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of, lg, qd, kd, vd, w.scale, causal, None)
    assert worst <= 1.0 and lerr <= 1.0
    if N == 1:  # one key: O is that key's value row exactly up to bf16 rounding of O
        assert np.allclose(of[0, :, 0], vd[0, :, 0], rtol=2.0 ** -8, atol=1e-6)


def test_forward_fp8_empty_key_range(gpu):
    """A batch whose key-padding length is 0: every row of it has no admissible key, so O
    is exactly 0 and LSE is -inf (the other batch is checked against the oracle)."""
    w = wl.get_workload("bert_large")
    inp, t, shp, signs = _setup(gpu, w, (2, 2, 130, 64))
    B, H, N, d = shp
    kv = np.array([0, 77], dtype=np.int32)
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, d)
    of, lg = _run_forward(gpu, g, shp, w.scale, False, torch.from_numpy(kv).to(gpu))
    assert not of[0].any() and np.all(lg[0] == -np.inf)
    qd, kd, vd = O.dequantize_blocks(q8, sq), O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of[1:], lg[1:], qd[1:], kd[1:], vd[1:], w.scale, False, kv[1:])
    assert worst <= 1.0 and lerr <= 1.0


def _bf16_tensor(gpu, x):
    bits = wl.f32_to_bf16_bits(x)
    return bits, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(gpu)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantizers_bit_exact_extreme_values(gpu, d, rotate):
    """Adversarial inputs for the quantisers: values spread over 10^-20 .. 10^20 inside one
    block (many subnormal and zero codes), an all-zero block, negative zeros, a single huge
    outlier, and values that land exactly on E4M3 rounding ties after scaling.  Magnitudes
    stay where the rotation's fp32 sums cannot overflow."""
    rng = np.random.default_rng(99)
    B, H, N = 1, 2, 200
    x = rng.standard_normal((B, H, N, d)).astype(np.float32)
    x *= np.exp(rng.uniform(-46, 46, size=x.shape)).astype(np.float32)  # ~1e-20 .. 1e20
    x[0, 0, 64:128] = 0.0                                              # a block of zeros
    x[0, 0, 64:70, :7] = -0.0
    x[0, 1, 130, 5] = 3.0e30                                           # one huge outlier
    # ties: block amax 448 makes inv = 1, so midpoints between E4M3 neighbours stay ties
    vals = O.e4m3_decode(np.arange(1, 0x7E, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    tie_rows = np.resize(mids, (64, d)).astype(np.float32)
    tie_rows[0, 0] = 448.0
    x[0, 1, 0:64] = tie_rows
    x = wl.bf16_bits_to_f64(wl.f32_to_bf16_bits(x)).astype(np.float32)  # what the GPU receives
    bits, xt = _bf16_tensor(gpu, x)
    signs = wl.fp8_signs(d, 5) if rotate else None
    nb = -(-N // 64)
    x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=gpu)
    sc = torch.empty((B, H, nb), dtype=torch.float32, device=gpu)
    fa.fa_fp8_quantize_qk(xt, x8, sc, None if signs is None else torch.from_numpy(signs).to(gpu),
                          1.0 / d if rotate else 1.0)
    v8t = torch.empty((B, H, nb, d, 64), dtype=torch.uint8, device=gpu)
    sv = torch.empty((B, H, d), dtype=torch.float32, device=gpu)
    fa.fa_fp8_quantize_v(xt, v8t, sv)
    torch.cuda.synchronize()
    xr = wl.bf16_bits_to_f64(bits)
    c_ref, s_ref = O.quantize_blocks(xr, signs, post_scale=1.0 / d if rotate else 1.0)
    v_ref, sv_ref = O.quantize_columns(xr)
    assert np.array_equal(_u8(x8), c_ref)
    assert np.array_equal(sc.cpu().numpy(), s_ref)
    assert np.array_equal(_u8(fa.fp8_v8t_to_rows(v8t, N)), v_ref)
    assert np.array_equal(sv.cpu().numpy(), sv_ref)
    if not rotate:  # the zero block: scale 0, every code a zero (+0 or, for -0.0, 0x80)
        assert sc.cpu().numpy()[0, 0, 1] == 0.0
        assert np.all(O.e4m3_decode(_u8(x8)[0, 0, 64:128]) == 0.0)
        assert np.all(_u8(x8)[0, 0, 64:70, :7] == 0x80)


@pytest.mark.parametrize("scale", [0.0, -0.125])
def test_forward_fp8_any_finite_scale(gpu, scale):
    """A zero or negative scale is carried by the Q codes (sign bits flipped or codes
    zeroed), checked with the same per-element bound against the dequantised inputs."""
    w = wl.get_workload("gpt2")
    inp, t, shp, signs = _setup(gpu, w, (1, 2, 300, 64))
    g = _quantize_gpu(gpu, t, shp, signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, shp[3])
    of, lg = _run_forward(gpu, g, shp, scale, True)
    qd, kd, vd = O.dequantize_blocks(q8, sq), O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of, lg, qd, kd, vd, scale, True, None)
    print(f"fp8 scale {scale}: max |dO|/bound {worst:.3f}  O rel-Frobenius {rel:.3e}  |dLSE|/bound {lerr:.3f}", flush=True)
    assert worst <= 1.0 and rel <= 5e-2 and lerr <= 1.0
