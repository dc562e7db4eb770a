"""GPU parity of fa_forward_offset: Nq query rows at key positions q_offset .. q_offset +
Nq - 1 against Nk keys -- one GPU's share of a forward whose query rows are split over
several GPUs that each hold the keys and values.  The share's O and LSE are, by the
definition, rows [q_offset, q_offset + Nq) of the whole problem's: checked against the
fp64 oracle on those rows of the whole problem, and bit for bit against the GPU's own
whole-problem forward where both calls run the same kernel form (the same per-wave rows,
tiles and arithmetic)."""

import numpy as np
import pytest

from exact_io_aware_19_amd import workloads as wl
from oracle import ref
from tests import parity as P

pytestmark = pytest.mark.gpu


def _offset_forward(gpu, q, k, v, scale, causal, q_offset, kv_len=None):
    import torch

    import exact_io_aware_19_amd as fa

    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=gpu)
    fa.fa_forward_offset(q, k, v, o, lse, scale, causal, q_offset, kv_len=kv_len)
    torch.cuda.synchronize()
    return o, lse


def _bf16(gpu, bits):
    import torch

    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(gpu)


# (B, H, Nq, Nk, q_offset, d, causal, kv_range)
CASES = [
    (1, 2, 300, 1000, 700, 128, True, None),      # the last rows of a causal sequence
    (2, 2, 256, 2048, 512, 64, True, None),       # a middle block
    (1, 3, 100, 777, 0, 128, False, None),        # no mask, fewer queries than keys
    (2, 2, 200, 500, 400, 64, True, (300, 500)),  # padding; rows past the keys
    (1, 2, 64, 4096, 4032, 128, True, None),      # one tile of queries, many keys
    (1, 2, 129, 129, 0, 128, True, None),         # the square problem
    (2, 2, 65, 3000, 1000, 64, False, (1, 3000)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dNq%dNk%doff%dd%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full", "pad" if c[7] else "nopad"))
def test_offset_forward_parity(gpu, case):
    B, H, Nq, Nk, off, d, causal, kvr = case
    P.say(f"offset forward {case}")
    rng = np.random.default_rng(9900 + Nq + Nk + off)
    q = wl.f32_to_bf16_bits(rng.standard_normal((B, H, Nq, d), dtype=np.float32))
    k = wl.f32_to_bf16_bits(rng.standard_normal((B, H, Nk, d), dtype=np.float32))
    v = wl.f32_to_bf16_bits(rng.standard_normal((B, H, Nk, d), dtype=np.float32))
    kv = None if kvr is None else rng.integers(kvr[0], kvr[1], size=B, endpoint=True).astype(np.int32)
    scale = d ** -0.5
    import torch

    kvt = None if kv is None else torch.from_numpy(kv).to(gpu)
    o, lse = _offset_forward(gpu, _bf16(gpu, q), _bf16(gpu, k), _bf16(gpu, v), scale, causal, off, kvt)
    q64, k64, v64 = (wl.bf16_bits_to_f64(x) for x in (q, k, v))
    rows = off + np.arange(Nq)
    o_ref = np.zeros((B, H, Nq, d))
    lse_ref = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            qf = np.zeros((off + Nq, d))  # the share's rows at their positions
            qf[off:] = q64[b, h]
            o_ref[b, h], lse_ref[b, h] = ref.forward_rows(qf, k64[b, h], v64[b, h], scale, rows, causal=causal,
                                                          kv_len_b=None if kv is None else int(kv[b]))
    P.check_forward(o, lse, o_ref, lse_ref, label=str(case))
    if Nq == Nk and off == 0:  # the square problem: exactly fa_forward
        import exact_io_aware_19_amd as fa

        o2, l2 = fa.forward(_bf16(gpu, q), _bf16(gpu, k), _bf16(gpu, v), causal=causal, scale=scale, kv_len=kvt)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


@pytest.mark.parametrize("B,H,N,d,shards", [(1, 4, 8192, 64, 4), (2, 32, 8192, 128, 4)])
def test_offset_shares_equal_whole_forward(gpu, B, H, N, d, shards):
    """A causal forward split into query shards (each against its admissible key prefix)
    reproduces the whole forward's rows bit for bit: grids chosen so that the shares and
    the whole problem run the same kernel form (the 4-wave small-grid forward at d = 64,
    the 8-wave one at d = 128)."""
    import torch

    import exact_io_aware_19_amd as fa

    P.say(f"offset shares: B={B} H={H} N={N} d={d} shards={shards}")
    g = torch.Generator(device="cpu").manual_seed(9950 + d)
    q, k, v = (torch.randn(B, H, N, d, generator=g).to(torch.bfloat16).to(gpu) for _ in range(3))
    scale = d ** -0.5
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    n = N // shards
    for s in range(shards):
        end = (s + 1) * n
        os_, ls_ = _offset_forward(gpu, q[:, :, s * n:end].contiguous(), k[:, :, :end].contiguous(),
                                   v[:, :, :end].contiguous(), scale, True, s * n)
        assert torch.equal(os_.view(torch.int16), o[:, :, s * n:end].view(torch.int16)), f"shard {s}: O"
        assert torch.equal(ls_, lse[:, :, s * n:end]), f"shard {s}: LSE"


def test_long_context_last_share(gpu):
    """The long-context workload (B=1, H=16, N=65536, d=64, causal, 1% of key rows x8)
    split over 8 GPUs by query rows: the last share (8192 rows at offset 57344, all 65536
    keys) equals the whole forward's rows bit for bit (both run the 8-wave kernel), and the
    workload's sampled rows that fall in it match the oracle."""
    import torch

    import exact_io_aware_19_amd as fa

    w = wl.get_workload("long_64k")
    inp = wl.generate(w)
    t = inp.to_torch(gpu)
    B, H, N, d = w.shape
    off, Nq = N - N // 8, N // 8
    P.say(f"long-context last share: rows [{off}, {N})")
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=True, scale=w.scale)
    os_, ls_ = _offset_forward(gpu, t["q"][:, :, off:].contiguous(), t["k"], t["v"], w.scale, True, off)
    assert torch.equal(os_.view(torch.int16), o[:, :, off:].view(torch.int16))
    assert torch.equal(ls_, lse[:, :, off:])
    rows = np.unique(np.concatenate([inp.rows[inp.rows >= off], [off, N - 1]]))
    o_np, l_np = P.to_np_bf16(os_), ls_.cpu().numpy().astype(np.float64)
    for h in (0, 7, 15):
        o_ref, lse_ref = ref.forward_rows(inp.head64("q", 0, h), inp.head64("k", 0, h), inp.head64("v", 0, h),
                                          w.scale, rows, causal=True)
        P.check_forward(o_np[0, h, rows - off], l_np[0, h, rows - off], o_ref, lse_ref, label=f"head {h}")
