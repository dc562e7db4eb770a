"""The library keeps no global mutable state, so calls on different streams may run at
the same time: two independent problems launched together on two streams (default
priority) must give bit for bit what each gives alone on the current stream."""

import pytest

from tests import parity as P

pytestmark = pytest.mark.gpu


def _problem(gpu, B, H, N, d, causal, kv_range, seed):
    import torch
    import exact_io_aware_19_amd as fa

    inp = P.custom_inputs(B, H, N, d, seed=seed, causal=causal, kv_range=kv_range, with_do=True)
    t = inp.to_torch(gpu)
    w = inp.workload
    bufs = {
        "o": torch.empty_like(t["q"]),
        "lse": torch.empty((B, H, N), dtype=torch.float32, device=gpu),
        "dq": torch.empty_like(t["q"]),
        "dk": torch.empty_like(t["q"]),
        "dv": torch.empty_like(t["q"]),
        "ws": torch.empty(fa.fa_backward_workspace_size(B, H, N, d), dtype=torch.uint8, device=gpu),
    }

    def run(stream):
        fa.fa_forward(t["q"], t["k"], t["v"], bufs["o"], bufs["lse"], w.scale, w.causal, kv_len=t["kv_len"],
                      stream=stream)
        fa.fa_backward(t["q"], t["k"], t["v"], bufs["o"], t["do"], bufs["lse"], bufs["dq"], bufs["dk"], bufs["dv"],
                       w.scale, w.causal, bufs["ws"], kv_len=t["kv_len"], stream=stream)

    def snapshot():
        return {k: v.clone() for k, v in bufs.items() if k != "ws"}

    return run, snapshot, bufs


def _equal(a, b):
    import torch

    for k in a:
        x, y = a[k], b[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), k


def test_concurrent_streams_match_serial(gpu):
    import torch

    P.say("two problems on two streams")
    run_a, snap_a, bufs_a = _problem(gpu, 2, 4, 1024, 128, True, None, seed=4242)
    run_b, snap_b, bufs_b = _problem(gpu, 2, 8, 700, 64, False, (200, 700), seed=4243)
    run_a(None)
    run_b(None)
    torch.cuda.synchronize()
    ref_a, ref_b = snap_a(), snap_b()
    for buf in list(bufs_a.values()) + list(bufs_b.values()):
        if buf.dtype != torch.uint8:
            buf.fill_(0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=gpu), torch.cuda.Stream(device=gpu)
    for rep in range(3):
        with torch.cuda.stream(s1):
            run_a(s1)
        with torch.cuda.stream(s2):
            run_b(s2)
        torch.cuda.synchronize()
        _equal(snap_a(), ref_a)
        _equal(snap_b(), ref_b)
