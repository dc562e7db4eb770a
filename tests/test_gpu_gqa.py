"""GPU parity of grouped-query and multi-query attention (fa_forward_gqa,
fa_backward_gqa) against the fp64 oracle's grouped functions (through the C ABI
binding).  K/V heads are shared by groups of consecutive query heads; dK and dV sum
the gradients of their group."""

import numpy as np
import pytest

from exact_io_aware_19_amd import workloads as wl
from oracle import ref
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, H_kv, N, d, causal, kv_range)
    (1, 4, 2, 128, 64, False, None),
    (1, 2, 1, 1, 128, True, None),
    (2, 4, 1, 300, 128, True, None),
    (2, 6, 3, 257, 64, True, (1, 257)),
    (1, 8, 2, 1000, 128, False, (500, 1000)),
    (2, 4, 2, 700, 64, False, None),
    (1, 8, 1, 520, 128, True, (100, 520)),
]


def _ids(c):
    return "B%dH%dKV%dN%dd%d_%s_%s" % (c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full",
                                       "pad" if c[6] else "nopad")


def _run(inp, device):
    import exact_io_aware_19_amd as fa

    t = inp.to_torch(device)
    w = inp.workload
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, kv_len=t["kv_len"])
    grads = fa.backward(t["q"], t["k"], t["v"], o, t["do"], lse, causal=w.causal, scale=w.scale, kv_len=t["kv_len"])
    return t, o, lse, grads


def _oracle(inp):
    w = inp.workload
    q, k, v, do = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    o, lse = ref.attention_forward_gqa(q, k, v, w.scale, causal=w.causal, kv_len=inp.kv_len)
    grads = ref.attention_backward_gqa(q, k, v, do, w.scale, causal=w.causal, kv_len=inp.kv_len)
    return o, lse, grads


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_gqa_parity(gpu, case):
    B, H, Hkv, N, d, causal, kvr = case
    P.say(f"gqa case {case}")
    inp = P.custom_inputs(B, H, N, d, seed=9100 + N + H, causal=causal, kv_range=kvr, with_do=True, h_kv=Hkv)
    assert inp.k.shape == (B, Hkv, N, d)
    _, o, lse, grads = _run(inp, gpu)
    o_ref, lse_ref, g_ref = _oracle(inp)
    P.check_forward(o, lse, o_ref, lse_ref, label=str(case))
    P.check_grads(grads, g_ref, label=str(case))
    if inp.kv_len is not None:  # keys padded away for every query: exact zeros
        dk, dv = (g.cpu() for g in grads[1:])
        for b, n in enumerate(inp.kv_len):
            assert (dk[b, :, int(n):].float() == 0).all()
            assert (dv[b, :, int(n):].float() == 0).all()


def test_gqa_workload_sampled_rows(gpu):
    """The grouped large-head workload at full size: sampled query rows of O, LSE and
    dQ against the oracle, computed row by row with each query head's own K/V head."""
    import exact_io_aware_19_amd as fa

    inp = wl.generate("gqa_n8192")
    w = inp.workload
    P.say(f"gqa workload {w.name} {w.shape} h_kv={w.kv_heads}")
    t = inp.to_torch(gpu)
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, t["do"], lse, causal=w.causal, scale=w.scale)
    G = w.H // w.kv_heads
    rng = np.random.default_rng(5)
    for b, h in ((0, 0), (1, 7), (1, 15)):
        rows = np.sort(rng.choice(w.N, size=24, replace=False))
        rows[0] = w.N - 1
        q, k, v, do = (inp.head64(n, b, hh) for n, hh in (("q", h), ("k", h // G), ("v", h // G), ("do", h)))
        o_r, l_r = ref.forward_rows(q, k, v, w.scale, rows, causal=w.causal)
        P.check_forward(P.to_np_bf16(o[b, h])[rows], lse[b, h].cpu().numpy().astype(np.float64)[rows], o_r, l_r,
                        label=f"b{b} h{h} rows")
        dq_r = ref.backward_dq_rows(q, k, v, do, w.scale, rows, causal=w.causal)
        err = P.rel_frob(P.to_np_bf16(dq[b, h])[rows], dq_r)
        P.say(f"  b{b} h{h} dQ rows: rel-Frobenius {err:.3e}")
        assert err <= P.GRAD_REL
    import torch

    assert bool(torch.isfinite(dk.float()).all()) and bool(torch.isfinite(dv.float()).all())


def test_gqa_with_all_heads_equals_mha_bitwise(gpu):
    """H_kv = H through the grouped entry points runs the same kernels as fa_forward /
    fa_backward: bitwise identical outputs."""
    import torch
    import exact_io_aware_19_amd as fa

    inp = P.custom_inputs(2, 3, 333, 128, seed=77, causal=True, with_do=True)
    t = inp.to_torch(gpu)
    w = inp.workload
    o1, l1 = fa.forward(t["q"], t["k"], t["v"], causal=True, scale=w.scale)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    fa.fa_forward_gqa(t["q"], t["k"], t["v"], o2, l2, w.scale, True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    g1 = fa.backward(t["q"], t["k"], t["v"], o1, t["do"], l1, causal=True, scale=w.scale)
    g2 = [torch.empty_like(x) for x in g1]
    ws = torch.empty(fa.fa_backward_workspace_size(2, 3, 333, 128), dtype=torch.uint8, device=gpu)
    fa.fa_backward_gqa(t["q"], t["k"], t["v"], o1, t["do"], l1, *g2, w.scale, True, ws)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_gqa_backward_deterministic(gpu):
    import torch

    inp = P.custom_inputs(1, 8, 600, 64, seed=91, causal=True, with_do=True, h_kv=2)
    _, _, _, g1 = _run(inp, gpu)
    _, _, _, g2 = _run(inp, gpu)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["gqa_n8192", "mqa_n4096"])
def test_gqa_full_size_equals_summed_mha_gradients(gpu, name):
    """At the full workload sizes (gqa_n8192: one workgroup per key block and K/V head;
    mqa_n4096: a group's query heads split over 8 workgroups and reduced): dK, dV of the
    grouped call equal the group sums of the ordinary backward on repeated K/V heads (a
    path checked against the oracle elsewhere), and dQ, O, LSE match it."""
    import torch
    import exact_io_aware_19_amd as fa

    inp = wl.generate(name)
    w = inp.workload
    G = w.H // w.kv_heads
    P.say(f"{name}: {w.shape} h_kv={w.kv_heads} causal={w.causal}")
    t = inp.to_torch(gpu)
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, t["do"], lse, causal=w.causal, scale=w.scale)
    kr = t["k"].repeat_interleave(G, dim=1).contiguous()
    vr = t["v"].repeat_interleave(G, dim=1).contiguous()
    o2, lse2 = fa.forward(t["q"], kr, vr, causal=w.causal, scale=w.scale)
    dq2, dk2, dv2 = fa.backward(t["q"], kr, vr, o2, t["do"], lse2, causal=w.causal, scale=w.scale)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    assert torch.equal(dq.view(torch.int16), dq2.view(torch.int16))
    B, H, N, d = w.shape
    for name_, g, g2 in (("dk", dk, dk2), ("dv", dv, dv2)):
        ref_sum = g2.float().view(B, w.kv_heads, G, N, d).sum(dim=2)
        rel = float((g.float() - ref_sum).norm() / ref_sum.norm())
        P.say(f"  {name_}: rel-Frobenius vs summed per-head gradients {rel:.3e}")
        assert rel <= 1e-2


def test_gqa_split_backward_deterministic(gpu):
    import torch

    inp = P.custom_inputs(2, 8, 1500, 128, seed=93, causal=False, with_do=True, h_kv=1, kv_range=(900, 1500))
    _, _, _, g1 = _run(inp, gpu)
    _, _, _, g2 = _run(inp, gpu)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
