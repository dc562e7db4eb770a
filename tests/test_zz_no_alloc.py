"""GPU test of fa_backward_noalloc (the backward without a workspace argument, for
callers that cannot allocate): through the C ABI it must give exactly the gradients of
fa_backward_kvlen, the entry point with a caller-provided workspace, on two calls in a
row (the second smaller, so it reuses the scratch the first one left), and match the
fp64 oracle."""

import numpy as np
import pytest

from exact_io_aware_19_amd import workloads as wl
from oracle import ref
from tests import parity as P

pytestmark = pytest.mark.gpu


def _case(gpu, B, H, N, d, causal, kvr, seed):
    import torch
    import exact_io_aware_19_amd as fa

    P.say(f"no-alloc backward: B={B} H={H} N={N} d={d} causal={causal} kv_range={kvr}")
    inp = P.custom_inputs(B, H, N, d, seed=seed, causal=causal, kv_range=kvr, with_do=True)
    t = inp.to_torch(gpu)
    scale = d ** -0.5
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=causal, scale=scale, kv_len=t["kv_len"])
    ws = torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=gpu)
    want = [torch.empty_like(t["q"]) for _ in range(3)]
    fa.fa_backward(t["q"], t["k"], t["v"], o, t["do"], lse, *want, scale, causal, ws, kv_len=t["kv_len"])
    got = [torch.full_like(t["q"], 3.0) for _ in range(3)]
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(gpu)
    torch.cuda.reset_peak_memory_stats(gpu)
    fa.fa_backward_noalloc(t["q"], t["k"], t["v"], o, t["do"], lse, *got, scale, causal, kv_len=t["kv_len"])
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated(gpu) == base
    for name, a, b in zip(("dQ", "dK", "dV"), got, want):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name} differs from fa_backward_kvlen"
    q, k, v, do = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    g_ref = ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=inp.kv_len)
    P.check_grads(got, g_ref, label=f"no-alloc B={B} H={H} N={N} d={d}")


def test_noalloc_backward_two_calls(gpu):
    _case(gpu, 2, 4, 1000, 128, True, (300, 1000), seed=9900)
    _case(gpu, 1, 2, 333, 64, False, None, seed=9901)


def test_noalloc_backward_rejects_oversize(gpu):
    import torch
    import exact_io_aware_19_amd as fa

    # 33 heads x 65536 rows of statistics exceed the 16 MiB scratch: refused on the host
    q = torch.zeros(1, 33, 65536, 64, dtype=torch.bfloat16, device=gpu)
    lse = torch.zeros(1, 33, 65536, dtype=torch.float32, device=gpu)
    with pytest.raises(fa.FAError) as e:
        fa.fa_backward_noalloc(q, q, q, q, q, lse, q, q, q, 0.125, False)
    assert e.value.status == -5
