"""GPU parity of fa_forward against the fp64 oracle (through the C ABI binding)."""

import numpy as np
import pytest

from exact_io_aware_19_amd import workloads as wl
from oracle import ref
from tests import parity as P

pytestmark = pytest.mark.gpu

SMALL_CASES = [
    # (B, H, N, d, causal, kv_range)
    (1, 2, 128, 64, False, None),
    (1, 1, 1, 64, False, None),
    (1, 1, 1, 128, True, None),
    (2, 3, 17, 64, True, None),
    (2, 2, 100, 128, False, None),
    (1, 2, 129, 64, True, None),
    (2, 2, 300, 128, True, None),
    (3, 2, 513, 64, False, (1, 513)),
    (2, 2, 700, 128, True, (200, 700)),
    (2, 1, 1000, 64, True, (1, 1000)),
    (1, 2, 1100, 128, False, (700, 1100)),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "B%dH%dN%dd%d_%s_%s" % (c[0], c[1], c[2], c[3], "causal" if c[4] else "full", "pad" if c[5] else "nopad"))
def test_forward_small(gpu, case):
    B, H, N, d, causal, kvr = case
    P.say(f"forward small case {case}")
    inp = P.custom_inputs(B, H, N, d, seed=7000 + N + d, causal=causal, kv_range=kvr, with_do=False)
    _, o, lse = P.run_forward(inp, gpu)
    o_ref, lse_ref = P.oracle_forward_full(inp)
    P.check_forward(o, lse, o_ref, lse_ref, label=str(case))


@pytest.mark.parametrize("name", ["tiny", "bert_large", "gpt2", "sweep_n2048_full", "sweep_n2048_causal"])
def test_forward_workload_full(gpu, name):
    w = wl.get_workload(name)
    P.say(f"forward workload {name} {w.shape} causal={w.causal}")
    inp = wl.generate(w, with_do=False)
    _, o, lse = P.run_forward(inp, gpu)
    o_ref, lse_ref = P.oracle_forward_full(inp)
    P.check_forward(o, lse, o_ref, lse_ref, label=name)


def _sampled_heads_rows(w, n_heads, n_rows, seed):
    rng = np.random.default_rng(seed)
    heads = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, n_heads), rng.integers(0, w.H, n_heads))]
    rows = np.sort(rng.choice(w.N, size=min(n_rows, w.N), replace=False))
    rows[-1] = w.N - 1  # always include the last (ragged / causal-longest) row
    rows[0] = 0
    return heads, np.unique(rows)


@pytest.mark.parametrize("name", ["sweep_n4096_full", "sweep_n4096_causal", "sweep_n8192_full", "sweep_n8192_causal",
                                  "sweep_n16384_full", "sweep_n16384_causal"])
def test_forward_workload_sampled(gpu, name):
    w = wl.get_workload(name)
    P.say(f"forward workload {name} {w.shape} causal={w.causal} (sampled rows)")
    inp = wl.generate(w, with_do=False)
    _, o, lse = P.run_forward(inp, gpu)
    heads, rows = _sampled_heads_rows(w, 4, 96, seed=w.seed + 17)
    o_all = P.to_np_bf16(o)
    lse_all = lse.cpu().numpy().astype(np.float64)
    for b, h in heads:
        o_ref, lse_ref = ref.forward_rows(inp.head64("q", b, h), inp.head64("k", b, h), inp.head64("v", b, h),
                                          w.scale, rows, causal=w.causal)
        P.check_forward(o_all[b, h, rows], lse_all[b, h, rows], o_ref, lse_ref, label=f"{name} b{b} h{h}")


def test_forward_long_context_sampled(gpu):
    w = wl.get_workload("long_64k")
    P.say(f"forward workload long_64k {w.shape} (64 sampled rows, 1% keys x8)")
    inp = wl.generate(w)
    _, o, lse = P.run_forward(inp, gpu)
    o_all = P.to_np_bf16(o)
    lse_all = lse.cpu().numpy().astype(np.float64)
    for h in range(w.H):
        o_ref, lse_ref = ref.forward_rows(inp.head64("q", 0, h), inp.head64("k", 0, h), inp.head64("v", 0, h),
                                          w.scale, inp.rows, causal=True)
        P.check_forward(o_all[0, h, inp.rows], lse_all[0, h, inp.rows], o_ref, lse_ref, label=f"long_64k h{h}")


def test_forward_deterministic(gpu):
    inp = P.custom_inputs(2, 2, 777, 128, seed=99, causal=True, with_do=False)
    _, o1, l1 = P.run_forward(inp, gpu)
    _, o2, l2 = P.run_forward(inp, gpu)
    import torch

    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_forward_invariants(gpu):
    """Constant V gives constant O; causal row 0 equals V[0]; LSE rows normalise P."""
    import torch
    import exact_io_aware_19_amd as fa

    inp = P.custom_inputs(1, 2, 333, 64, seed=5, causal=True, with_do=False)
    t = inp.to_torch(gpu)
    vc = t["v"][:, :, :1, :].expand_as(t["v"]).contiguous()
    o, lse = fa.forward(t["q"], t["k"], vc, causal=True, scale=0.125)
    # O = (sum_j p_j) v / (sum_j p_j): equal to v up to fp32 summation order, then bf16 rounding
    assert torch.allclose(o.float(), vc.float(), rtol=2.0 ** -8, atol=0)
    o2, lse2 = fa.forward(t["q"], t["k"], t["v"], causal=True, scale=0.125)
    assert torch.equal(o2[:, :, 0].view(torch.int16), t["v"][:, :, 0].view(torch.int16))
    q64, k64 = inp.head64("q", 0, 1), inp.head64("k", 0, 1)
    s = 0.125 * q64[[0, 100, 332]] @ k64.T
    for idx, i in enumerate([0, 100, 332]):
        tot = np.exp(s[idx, : i + 1] - float(lse2[0, 1, i])).sum()
        assert abs(tot - 1.0) < 2e-3


def test_forward_no_quadratic_memory(gpu):
    """The library allocates nothing: peak device memory stays at inputs + outputs."""
    import torch
    import exact_io_aware_19_amd as fa

    B, H, N, d = 1, 4, 8192, 64
    q = torch.randn(B, H, N, d, device=gpu, dtype=torch.bfloat16)
    k, v = torch.randn_like(q), torch.randn_like(q)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=gpu, dtype=torch.float32)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(gpu)
    base = torch.cuda.memory_allocated(gpu)
    fa.fa_forward(q, k, v, o, lse, 0.125, True)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated(gpu) == base
    assert torch.isfinite(lse).all()
