"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI binding
and compare with the fp64 oracle on the same seeded inputs.

Tolerances (bf16 inputs, fp32 accumulation):
  O    max |err| <= 2e-2 and mean |err| <= 2e-3
  LSE  max |err| <= 1e-3
  dQ, dK, dV relative Frobenius error <= 2e-2, over the whole tensor and over every
             64-row tile of every head
"""

import sys

import numpy as np

from exact_io_aware_19_amd import workloads as wl
from oracle import ref

O_MAX, O_MEAN, LSE_MAX, GRAD_REL = 2e-2, 2e-3, 1e-3, 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np_bf16(t):
    """bf16 torch tensor -> fp64 numpy (exact)."""
    import torch

    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return wl.bf16_bits_to_f64(bits)


def custom_inputs(B, H, N, d, seed, causal=False, kv_range=None, with_do=True, scale=None, scaled_key_frac=0.0,
                  h_kv=0):
    w = wl.Workload(f"custom_{B}x{H}x{N}x{d}", B, H, N, d, causal, 1.0 / np.sqrt(d) if scale is None else scale, seed,
                    kv_len_range=kv_range, scaled_key_frac=scaled_key_frac, backward=with_do, h_kv=h_kv)
    return wl.generate(w)


def run_forward(inp, device):
    import exact_io_aware_19_amd as fa

    t = inp.to_torch(device)
    w = inp.workload
    o, lse = fa.forward(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale, kv_len=t["kv_len"])
    return t, o, lse


def oracle_forward_full(inp):
    w = inp.workload
    q, k, v = (wl.bf16_bits_to_f64(getattr(inp, n)) for n in ("q", "k", "v"))
    return ref.attention_forward(q, k, v, w.scale, causal=w.causal, kv_len=inp.kv_len)


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, label=""):
    o_g = to_np_bf16(o_gpu) if not isinstance(o_gpu, np.ndarray) else o_gpu
    l_g = lse_gpu.detach().cpu().numpy().astype(np.float64) if not isinstance(lse_gpu, np.ndarray) else lse_gpu
    err = np.abs(o_g - o_ref)
    finite = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l_g), finite), f"{label}: LSE finiteness differs"
    lerr = np.abs(l_g[finite] - lse_ref[finite]).max(initial=0.0)
    stats = dict(o_max=float(err.max(initial=0.0)), o_mean=float(err.mean()) if err.size else 0.0, lse_max=float(lerr))
    say(f"  {label}: O max {stats['o_max']:.3e} mean {stats['o_mean']:.3e}  LSE max {stats['lse_max']:.3e}")
    assert stats["o_max"] <= O_MAX, (label, stats)
    assert stats["o_mean"] <= O_MEAN, (label, stats)
    assert stats["lse_max"] <= LSE_MAX, (label, stats)
    return stats


def rel_frob(g, ref_g):
    den = np.linalg.norm(ref_g)
    num = np.linalg.norm(g - ref_g)
    return float(num / den) if den > 0 else float(num)


TILE_ROWS = 64


def worst_tile(g, ref_g, rows=TILE_ROWS):
    """Largest relative Frobenius error over the 64-row tiles of every head.

    g, ref_g: [..., N, d].  A whole-tensor norm hides a single wrong row (one bad row of
    a 16384-row head moves it by about 1e-2), so the same bound is also applied to every
    tile of `rows` consecutive rows of each head.  A tile whose exact gradient is zero
    (keys no query attends) is measured by its absolute error, which must then be 0 as
    well.  Returns (error, (head index, first row))."""
    n = g.shape[-2]
    g2 = g.reshape(-1, n, g.shape[-1])
    r2 = ref_g.reshape(-1, n, ref_g.shape[-1])
    worst, where = 0.0, None
    for hd in range(g2.shape[0]):
        for r0 in range(0, n, rows):
            e = rel_frob(g2[hd, r0:r0 + rows], r2[hd, r0:r0 + rows])
            if e > worst or where is None:
                worst, where = e, (hd, r0)
    return worst, where


def check_grads(grads_gpu, grads_ref, label=""):
    out, tiles = {}, {}
    for name, g, r in zip(("dq", "dk", "dv"), grads_gpu, grads_ref):
        gn = to_np_bf16(g) if not isinstance(g, np.ndarray) else g
        assert np.isfinite(gn).all(), f"{label}: {name} has non-finite values"
        out[name] = rel_frob(gn, r)
        tiles[name] = worst_tile(gn, r)
    say(f"  {label}: rel-Frobenius dQ {out['dq']:.3e} dK {out['dk']:.3e} dV {out['dv']:.3e}; worst 64-row tile "
        + " ".join(f"{n} {e:.3e}@{w}" for n, (e, w) in tiles.items()))
    for name, e in out.items():
        assert e <= GRAD_REL, (label, name, out)
    for name, (e, w) in tiles.items():
        assert e <= GRAD_REL, (label, name, "64-row tile", w, e)
    return out
