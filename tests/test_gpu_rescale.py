"""GPU parity of the forward's conditional rescaling on scores that climb along the keys
(inputs from ``workloads.staircase``): every block of keys raises each row's maximum by
a fixed amount, so the tile loop meets all branches of the rescale decision --
probabilities formed against the current reference that the test keeps (rise below the
threshold tau of 8 log2 units), a reference that moves on every tile (rise above it),
and probabilities that overflow fp32 before the reference moves (rise beyond 2^128) --
in the 8-wave kernel (d = 128, which forms P first and takes the row max only when a
tile's sum exceeds 2^tau) and in the small-grid kernel (d = 64 at this grid, max
first).  O and LSE are checked against the fp64 oracle.  (The backward takes no
rescale decisions -- it recomputes P from the LSE -- and on these inputs dQ is
ill-conditioned by construction: its first column sums dS times key entries of several
hundred over rows of dS that sum to zero, so bf16 dS cannot meet a 2% bound there.)
"""

import pytest

from exact_io_aware_19_amd import workloads as wl
from oracle import ref
from tests import parity as P

pytestmark = pytest.mark.gpu

# rise per 64-key block in natural-log units: 4.5 (6.5 in log2 units, below tau), 14
# (20, above it) and 110 (159: P against the old reference is inf)
RISES = [4.5, 14.0, 110.0]


@pytest.mark.parametrize("rise", RISES)
@pytest.mark.parametrize("d,N", [(128, 640), (128, 700), (64, 700)])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_staircase_scores(gpu, rise, d, N, causal):
    import exact_io_aware_19_amd as fa

    B, H = 1, 2
    P.say(f"staircase rise={rise} d={d} N={N} causal={causal}")
    inp = wl.staircase(B, H, N, d, rise, seed=9900 + d + N, causal=causal)
    t = inp.to_torch(gpu)
    scale = inp.workload.scale
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=causal, scale=scale)
    q, k, v = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v"))
    o_ref, lse_ref = ref.attention_forward(q, k, v, scale, causal=causal)
    P.check_forward(o, lse, o_ref, lse_ref, label=f"rise {rise} d={d} N={N} causal={causal}")


@pytest.mark.parametrize("rise", RISES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("rotate", [False, True], ids=["plain", "rotated"])
def test_staircase_scores_fp8(gpu, rise, d, causal, rotate):
    """The same inputs through the FP8 forward, whose rescale check is gated by the tile's
    sum of probabilities in the same way; checked with the per-element bound of the FP8
    parity tests (oracle: exact attention of the dequantised codes)."""
    from oracle import fp8 as O
    from tests.test_gpu_fp8 import _check_forward, _quantize_gpu, _quantize_oracle, _run_forward

    B, H, N = 1, 2, 700
    P.say(f"fp8 staircase rise={rise} d={d} causal={causal} rotate={rotate}")
    inp = wl.staircase(B, H, N, d, rise, seed=9950 + d, causal=causal)
    t = inp.to_torch(gpu)
    scale = inp.workload.scale
    signs = wl.fp8_signs(d, inp.workload.seed) if rotate else None
    g = _quantize_gpu(gpu, t, (B, H, N, d), signs)
    (q8, sq), (k8, sk), (v8, sv) = _quantize_oracle(inp, signs, d)
    assert (g["q"][0].cpu().numpy() == q8).all() and (g["k"][0].cpu().numpy() == k8).all()
    of, lg = _run_forward(gpu, g, (B, H, N, d), scale, causal)
    qd, kd, vd = O.dequantize_blocks(q8, sq), O.dequantize_blocks(k8, sk), O.dequantize_columns(v8, sv)
    worst, rel, lerr = _check_forward(of, lg, qd, kd, vd, scale, causal, None)
    P.say(f"  max |dO|/bound {worst:.3f}  O rel-Frobenius {rel:.3e}  |dLSE|/bound {lerr:.3f}")
    assert worst <= 1.0 and rel <= 5e-2 and lerr <= 1.0
