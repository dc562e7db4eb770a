"""GPU parity of fa_backward against the fp64 oracle (through the C ABI binding).

The backward consumes the GPU forward's own O and LSE, as a training step would; the
gradients are compared with the oracle's exact gradients of the same bf16 inputs.
"""

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


def _run(inp, device):
    import exact_io_aware_19_amd as fa

    t, o, lse = P.run_forward(inp, device)
    w = inp.workload
    dq, dk, dv = fa.backward(t["q"], t["k"], t["v"], o, t["do"], lse, causal=w.causal, scale=w.scale,
                             kv_len=t["kv_len"])
    return t, o, lse, (dq, dk, dv)


def _oracle_grads(inp):
    w = inp.workload
    q, k, v, do = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    return ref.attention_backward(q, k, v, do, w.scale, causal=w.causal, kv_len=inp.kv_len)


def _check_padding_zeros(grads, kv_len):
    if kv_len is None:
        return
    dk, dv = (g.cpu() for g in grads[1:])
    for b, n in enumerate(kv_len):
        assert (dk[b, :, int(n):].float() == 0).all()
        assert (dv[b, :, int(n):].float() == 0).all()


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "B%dH%dN%dd%d_%s_%s" % (c[0], c[1], c[2], c[3], "causal" if c[4] else "full", "pad" if c[5] else "nopad"))
def test_backward_small(gpu, case):
    B, H, N, d, causal, kvr = case
    P.say(f"backward small case {case}")
    inp = P.custom_inputs(B, H, N, d, seed=8000 + N + d, causal=causal, kv_range=kvr, with_do=True)
    _, _, _, grads = _run(inp, gpu)
    P.check_grads(grads, _oracle_grads(inp), label=str(case))
    _check_padding_zeros(grads, inp.kv_len)


@pytest.mark.parametrize("name", ["tiny", "bert_large", "gpt2", "sweep_n2048_full", "sweep_n2048_causal"])
def test_backward_workload_full(gpu, name):
    w = wl.get_workload(name)
    P.say(f"backward workload {name} {w.shape} causal={w.causal}")
    inp = wl.generate(w, with_do=True)
    _, _, _, grads = _run(inp, gpu)
    P.check_grads(grads, _oracle_grads(inp), label=name)
    _check_padding_zeros(grads, inp.kv_len)


@pytest.mark.parametrize("name,n_heads", [("sweep_n4096_full", 2), ("sweep_n4096_causal", 2), ("sweep_n8192_full", 1),
                                          ("sweep_n8192_causal", 1), ("sweep_n16384_full", 1),
                                          ("sweep_n16384_causal", 1)])
def test_backward_workload_sampled_heads(gpu, name, n_heads):
    """Full sizes in the launch configuration the bench times; the oracle computes the
    complete gradients of a few seeded heads, plus dQ rows and dK, dV key rows of three
    more heads."""
    w = wl.get_workload(name)
    P.say(f"backward workload {name} {w.shape} causal={w.causal} (sampled heads)")
    inp = wl.generate(w, with_do=True)
    _, _, _, grads = _run(inp, gpu)
    g_np = [P.to_np_bf16(g) for g in grads]
    rng = np.random.default_rng(w.seed + 29)
    heads = [divmod(int(x), w.H) for x in rng.choice(w.B * w.H, n_heads + 3, replace=False)]  # distinct
    for j, (b, h) in enumerate(heads):
        qh, kh, vh, doh = (inp.head64(n, b, h) for n in ("q", "k", "v", "do"))
        if j < n_heads:
            ref_g = ref.attention_backward(qh[None, None], kh[None, None], vh[None, None], doh[None, None], w.scale,
                                           causal=w.causal)
            P.check_grads([g[b, h] for g in g_np], [r[0, 0] for r in ref_g], label=f"{name} b{b} h{h}")
        else:
            rows = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 64, replace=False)]))
            dq_ref = ref.backward_dq_rows(qh, kh, vh, doh, w.scale, rows, causal=w.causal)
            err = P.rel_frob(g_np[0][b, h, rows], dq_ref)
            cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 64, replace=False)]))
            dk_ref, dv_ref = ref.backward_dkdv_cols(qh, kh, vh, doh, w.scale, cols, causal=w.causal)
            err_k, err_v = P.rel_frob(g_np[1][b, h, cols], dk_ref), P.rel_frob(g_np[2][b, h, cols], dv_ref)
            P.say(f"  {name} b{b} h{h} rel-Frobenius: dQ rows {err:.3e}, dK key rows {err_k:.3e}, "
                  f"dV key rows {err_v:.3e}")
            assert err <= P.GRAD_REL
            assert err_k <= P.GRAD_REL
            assert err_v <= P.GRAD_REL


def test_backward_deterministic(gpu):
    import torch

    inp = P.custom_inputs(2, 2, 777, 128, seed=98, causal=True, with_do=True)
    _, _, _, g1 = _run(inp, gpu)
    _, _, _, g2 = _run(inp, gpu)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_uses_only_the_workspace(gpu):
    import torch
    import exact_io_aware_19_amd as fa

    B, H, N, d = 1, 4, 4096, 128
    q = torch.randn(B, H, N, d, device=gpu, dtype=torch.bfloat16)
    k, v, do = torch.randn_like(q), torch.randn_like(q), torch.randn_like(q)
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=gpu)
    nw = (N + 255) // 256 * 256  # rows per head, padded to the dQ pass's 256-row blocks
    assert ws.numel() == 2 * 4 * B * H * nw  # D_i and LSE_i * log2(e), fp32
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(gpu)
    base = torch.cuda.memory_allocated(gpu)
    fa.fa_backward(q, k, v, o, do, lse, dq, dk, dv, d ** -0.5, True, ws)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated(gpu) == base
    for g in (dq, dk, dv):
        assert torch.isfinite(g.float()).all()


def test_backward_rejects_small_workspace(gpu):
    import torch
    import exact_io_aware_19_amd as fa

    q = torch.randn(1, 1, 64, 64, device=gpu, dtype=torch.bfloat16)
    o, lse = fa.forward(q, q, q)
    ws = torch.empty(16, dtype=torch.uint8, device=gpu)
    with pytest.raises(fa.FAError) as e:
        fa.fa_backward(q, q, q, o, q, lse, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), 0.125,
                       False, ws)
    assert e.value.status == -5


@pytest.mark.parametrize("causal,kvlen", [(False, False), (True, False), (False, True)])
def test_backward_passes_compose_to_backward(gpu, causal, kvlen):
    """fa_backward_dq_pass then fa_backward_dkdv_pass == fa_backward, bit for bit; each
    pass writes only its own outputs."""
    import torch
    import exact_io_aware_19_amd as fa

    B, H, N, d = 2, 2, 333, 128
    g = torch.Generator(device="cpu").manual_seed(4242)
    q, k, v, do = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(gpu) for _ in range(4))
    kv = torch.tensor([200, 333], dtype=torch.int32, device=gpu) if kvlen else None
    o, lse = fa.forward(q, k, v, causal=causal, kv_len=kv)
    ref = fa.backward(q, k, v, o, do, lse, causal=causal, kv_len=kv)
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=gpu)
    sentinel = torch.full_like(q, 7.0)
    dq, dk, dv = sentinel.clone(), sentinel.clone(), sentinel.clone()
    fa.fa_backward_pass("dq", q, k, v, o, do, lse, dq, dk, dv, d ** -0.5, causal, ws, kv_len=kv)
    torch.cuda.synchronize()
    assert torch.equal(dk, sentinel) and torch.equal(dv, sentinel)
    assert torch.equal(dq.view(torch.int16), ref[0].view(torch.int16))
    fa.fa_backward_pass("dkdv", q, k, v, o, do, lse, dq, dk, dv, d ** -0.5, causal, ws, kv_len=kv)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
