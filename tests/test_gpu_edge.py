"""GPU edge cases of the bf16 path against the fp64 oracle (through the C ABI binding):

* a batch whose key range is empty (kv_len = 0): O = 0, LSE = -inf and zero gradients,
  exactly, while the other batch is checked against the oracle;
* padding invariance: keys and values at or past kv_len never reach any output, so
  changing them leaves O, LSE, dQ, dK and dV bit for bit unchanged;
* head dim 64 at grids of 512 or more 8-wave workgroups (the 8-wave forward; smaller
  d = 64 grids run the 4-wave small-grid forward), with and without padding and causal
  masks, and the two forward kernels bit for bit equal on the same heads;
* head dim 128 in both grid forms of the forward and the dQ pass (full-size grids and
  the split form of small grids) on the same heads;
* any finite scale: zero (uniform weights over the admissible keys) and negative scales,
  forward and backward.
"""

import numpy as np
import pytest

from exact_io_aware_19_amd import workloads as wl
from oracle import ref
from tests import parity as P

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy()


def _fwd_bwd(t, causal, scale, kv):
    import exact_io_aware_19_amd as fa

    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=causal, scale=scale, kv_len=kv)
    grads = fa.backward(t["q"], t["k"], t["v"], o, t["do"], lse, causal=causal, scale=scale, kv_len=kv)
    return o, lse, grads


def _oracle(inp, scale, causal, kv_len):
    q, k, v, do = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    o, lse = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv_len)
    return o, lse, ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv_len)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_empty_key_range(gpu, d, causal):
    """kv_len = [0, 300] at N = 333: batch 0 has no admissible key for any query."""
    import torch

    B, H, N = 2, 2, 333
    P.say(f"empty key range: B={B} H={H} N={N} d={d} causal={causal} kv_len=[0, 300]")
    inp = P.custom_inputs(B, H, N, d, seed=9100 + d + int(causal), causal=causal, with_do=True)
    inp.kv_len = np.array([0, 300], dtype=np.int32)
    t = inp.to_torch(gpu)
    scale = d ** -0.5
    o, lse, grads = _fwd_bwd(t, causal, scale, t["kv_len"])
    torch.cuda.synchronize()
    assert (o[0].float() == 0).all(), "O of a row without admissible keys must be 0"
    assert torch.isinf(lse[0]).all() and (lse[0] < 0).all(), "LSE of such a row must be -inf"
    for name, g in zip(("dQ", "dK", "dV"), grads):
        assert (g[0].float() == 0).all(), f"{name} of the empty batch must be exactly 0"
    o_ref, lse_ref, g_ref = _oracle(inp, scale, causal, inp.kv_len)
    P.check_forward(o, lse, o_ref, lse_ref, label=f"kv_len=[0,300] d={d} causal={causal}")
    P.check_grads([g[1:] for g in grads], [r[1:] for r in g_ref], label=f"kv_len=[0,300] d={d} causal={causal}")


@pytest.mark.parametrize("d,N", [(64, 1000), (128, 700)])
@pytest.mark.parametrize("causal", [False, True])
def test_padding_invariance(gpu, d, N, causal):
    """Keys and values at or past kv_len are never read into any result: replacing them
    (by values 5x larger, or by NaN and inf) changes no output bit; padded dK, dV rows
    are +0."""
    import torch

    B, H = 3, 2
    P.say(f"padding invariance: B={B} H={H} N={N} d={d} causal={causal}")
    inp = P.custom_inputs(B, H, N, d, seed=9200 + d + int(causal), causal=causal, kv_range=(1, N - 1), with_do=True)
    t = inp.to_torch(gpu)
    kv = inp.kv_len
    k2, v2 = t["k"].clone(), t["v"].clone()
    g = torch.Generator(device="cpu").manual_seed(9300 + d)
    for b in range(B):
        n = int(kv[b])
        k2[b, :, n:] = (5 * torch.randn(k2[b, :, n:].shape, generator=g)).to(torch.bfloat16).to(gpu)
        v2[b, :, n:] = (5 * torch.randn(v2[b, :, n:].shape, generator=g)).to(torch.bfloat16).to(gpu)
    # whatever padded memory holds: NaN keys and infinite values in the last batch
    n = int(kv[B - 1])
    k2[B - 1, :, n:] = float("nan")
    v2[B - 1, :, n:] = float("inf")
    t2 = dict(t, k=k2, v=v2)
    scale = d ** -0.5
    o1, l1, g1 = _fwd_bwd(t, causal, scale, t["kv_len"])
    o2, l2, g2 = _fwd_bwd(t2, causal, scale, t["kv_len"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o1), _bits(o2)), "O changed"
    assert torch.equal(l1, l2), "LSE changed"
    for name, a, b_ in zip(("dQ", "dK", "dV"), g1, g2):
        assert np.array_equal(_bits(a), _bits(b_)), f"{name} changed"
    for b in range(B):
        n = int(kv[b])
        for gg in (g2[1], g2[2]):
            assert (gg[b, :, n:].contiguous().view(torch.int16) == 0).all(), "padded dK/dV rows must be +0"


# B=4, H=16, N=2048, d=64: 8 blocks of 256 query rows x 64 heads = 512 workgroups of 8
# waves -- the 8-wave forward kernel (grids below 512 run the 4-wave one)
EIGHT_WAVE_CASES = [(False, None), (False, (700, 2048)), (True, (700, 2048)), (True, None)]


@pytest.mark.parametrize("causal,kvr", EIGHT_WAVE_CASES,
                         ids=lambda c: str(c) if not isinstance(c, bool) else ("causal" if c else "full"))
def test_d64_eight_wave_grid(gpu, causal, kvr):
    B, H, N, d = 4, 16, 2048, 64
    P.say(f"d=64 8-wave grid: B={B} H={H} N={N} causal={causal} kv_range={kvr}")
    inp = P.custom_inputs(B, H, N, d, seed=9400 + int(causal) + (0 if kvr is None else 2), causal=causal,
                          kv_range=kvr, with_do=True)
    t = inp.to_torch(gpu)
    scale = 0.125
    o, lse, grads = _fwd_bwd(t, causal, scale, t["kv_len"])
    o_np, lse_np = P.to_np_bf16(o), lse.cpu().numpy().astype(np.float64)
    g_np = [P.to_np_bf16(g) for g in grads]
    rng = np.random.default_rng(9500)
    heads = sorted({(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(6)} | {(B - 1, H - 1)})
    for b, h in heads:
        kl = None if inp.kv_len is None else int(inp.kv_len[b])
        qh, kh, vh, doh = (inp.head64(n, b, h)[None, None] for n in ("q", "k", "v", "do"))
        kvh = None if kl is None else np.array([kl])
        o_ref, lse_ref = ref.attention_forward(qh, kh, vh, scale, causal=causal, kv_len=kvh)
        P.check_forward(o_np[b, h][None, None], lse_np[b, h][None, None], o_ref, lse_ref, label=f"b{b} h{h}")
        g_ref = ref.attention_backward(qh, kh, vh, doh, scale, causal=causal, kv_len=kvh)
        P.check_grads([g[b, h] for g in g_np], [r[0, 0] for r in g_ref], label=f"b{b} h{h}")


@pytest.mark.parametrize("causal", [False, True])
def test_d64_forward_kernels_agree(gpu, causal):
    """At d = 64 a grid of 512 8-wave workgroups (B=1, H=64, N=2048) runs the 8-wave
    forward and one of 504 (H=63) the 4-wave small-grid forward.  Each wave of either
    kernel owns the same 32 query rows and computes them with the same tiles, order and
    arithmetic, so the 63 common heads agree bit for bit."""
    import torch
    import exact_io_aware_19_amd as fa

    N, d = 2048, 64
    g = torch.Generator(device="cpu").manual_seed(9600 + int(causal))
    q, k, v = (torch.randn(1, 64, N, d, generator=g).to(torch.bfloat16).to(gpu) for _ in range(3))
    o8, l8 = fa.forward(q, k, v, causal=causal, scale=0.125)
    o4, l4 = fa.forward(q[:, :63].contiguous(), k[:, :63].contiguous(), v[:, :63].contiguous(), causal=causal,
                        scale=0.125)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o8[:, :63]), _bits(o4))
    assert torch.equal(l8[:, :63], l4)


# d = 128 problems run in two forms by grid size (split_small_grid in the library, for a
# device of 256 CUs): with B*H*ceil(N/256) above 256 the 8-wave forward and the 8-wave
# dQ pass; with few heads the split forms (two wave groups on the two halves of each
# 128-row block's key range, merged in LDS).  N = 900 gives 15 key tiles (8 + 7), 257 and
# 129 a ragged last tile.
D128_FORM_CASES = [(900, True, (300, 900), 40), (900, False, None, 40), (257, True, None, 80), (129, False, (1, 129), 150)]


@pytest.mark.parametrize("N,causal,kvr,H", D128_FORM_CASES,
                         ids=lambda c: str(c) if not isinstance(c, bool) else ("causal" if c else "full"))
def test_d128_split_and_unsplit_forms(gpu, N, causal, kvr, H):
    import torch

    B, d = 2, 128
    P.say(f"d=128 grid forms: B={B} H={H} / 4 N={N} causal={causal} kv_range={kvr}")
    inp = P.custom_inputs(B, H, N, d, seed=9800 + N + int(causal), causal=causal, kv_range=kvr, with_do=True)
    t = inp.to_torch(gpu)
    scale = d ** -0.5
    o_big, lse_big, g_big = _fwd_bwd(t, causal, scale, t["kv_len"])
    ts = {n: (x[:, :4].contiguous() if n != "kv_len" and x is not None else x) for n, x in t.items()}
    o_sm, lse_sm, g_sm = _fwd_bwd(ts, causal, scale, ts["kv_len"])
    torch.cuda.synchronize()
    forms = {"unsplit": (o_big, lse_big, g_big), "split": (o_sm, lse_sm, g_sm)}
    for b, h in [(0, 0), (1, 3), (0, 2)]:
        kl = None if inp.kv_len is None else int(inp.kv_len[b])
        qh, kh, vh, doh = (inp.head64(n, b, h)[None, None] for n in ("q", "k", "v", "do"))
        kvh = None if kl is None else np.array([kl])
        o_ref, lse_ref = ref.attention_forward(qh, kh, vh, scale, causal=causal, kv_len=kvh)
        g_ref = ref.attention_backward(qh, kh, vh, doh, scale, causal=causal, kv_len=kvh)
        for form, (o, lse, grads) in forms.items():
            P.check_forward(P.to_np_bf16(o[b, h])[None, None], lse[b, h].cpu().numpy().astype(np.float64)[None, None],
                            o_ref, lse_ref, label=f"{form} b{b} h{h}")
            P.check_grads([P.to_np_bf16(g[b, h]) for g in grads], [r[0, 0] for r in g_ref], label=f"{form} b{b} h{h}")


SCALE_CASES = [(1, 2, 128, 64, False, None), (2, 2, 300, 128, True, (100, 300)), (2, 2, 777, 64, True, None)]


@pytest.mark.parametrize("scale", [0.0, -0.125, -1.0])
@pytest.mark.parametrize("case", SCALE_CASES, ids=lambda c: "B%dH%dN%dd%d_%s_%s" % (
    c[0], c[1], c[2], c[3], "causal" if c[4] else "full", "pad" if c[5] else "nopad"))
def test_any_finite_scale(gpu, case, scale):
    B, H, N, d, causal, kvr = case
    P.say(f"scale {scale}: case {case}")
    inp = P.custom_inputs(B, H, N, d, seed=9700 + N + d, causal=causal, kv_range=kvr, with_do=True, scale=scale)
    t = inp.to_torch(gpu)
    o, lse, grads = _fwd_bwd(t, causal, scale, t["kv_len"])
    o_ref, lse_ref, g_ref = _oracle(inp, scale, causal, inp.kv_len)
    P.check_forward(o, lse, o_ref, lse_ref, label=f"scale {scale} {case}")
    if scale == 0.0:
        # closed form: LSE_i = ln(number of admissible keys); dQ = dK = 0 exactly
        rows = np.arange(N)
        lse_np = lse.cpu().numpy().astype(np.float64)
        for b in range(B):
            kl = N if inp.kv_len is None else int(inp.kv_len[b])
            n_i = np.minimum(rows + 1, kl) if causal else np.full(N, kl)
            assert np.abs(lse_np[b] - np.log(n_i)[None]).max() <= P.LSE_MAX
        assert (grads[0].float() == 0).all() and (grads[1].float() == 0).all()
    P.check_grads(grads, g_ref, label=f"scale {scale} {case}")
