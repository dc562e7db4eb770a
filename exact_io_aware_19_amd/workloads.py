"""Seeded synthetic workloads shaped like the pages' evaluations.

This module only draws inputs; it holds none of the attention arithmetic.  It serves
both the GPU path (bf16 bit patterns) and the fp64 oracle (the exact values of those
same bf16 numbers), so both sides always see identical inputs.

Shapes stand in for the pages' evaluation workloads (singularity-lens FA1 explainer,
evaluation and results paragraphs: BERT-large, GPT-2, long-context up to 64K tokens;
"FlashAttention" wiki page, FA1: Path-256 at 64K).  No dataset or trained weight is
used: every tensor is i.i.d. N(0, 1) drawn in fp32 from numpy's PCG64 and rounded to
bf16 (round to nearest, ties to even).

Draw order per workload (one generator per workload seed): q ([B, H, N, d] float32),
k, v ([B, H_kv, N, d]; H_kv = H unless the workload groups its K/V heads), then dO,
then the key-padding lengths, then the indices of the key rows scaled x8, then the
sampled query rows, then (workloads with outliers) the flat indices of the q entries and
of the k entries multiplied by 16.  The +-1 sign vector of the FP8 path's incoherent
processing comes from its own generator (``fp8_signs``).
"""

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f64",
    "generate",
    "staircase",
    "fp8_signs",
]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    scale: float
    seed: int
    kv_len_range: tuple = None     # (lo, hi) inclusive, per-batch key padding
    scaled_key_frac: float = 0.0   # fraction of key rows multiplied by 8 (same rows in every head)
    sampled_rows: int = 0          # oracle checks only these query rows (0 = all)
    backward: bool = True
    note: str = ""
    h_kv: int = 0                  # K/V heads (grouped-query attention); 0 = H
    outlier_frac: float = 0.0      # fraction of the entries of q and k multiplied by 16 (FP8 workloads)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def kv_heads(self):
        return self.h_kv or self.H

    def fwd_flops(self):
        """4 B H N^2 d, halved when causal (the convention of the throughput metric)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self):
        return 2.5 * self.fwd_flops()


def _sweep(n, causal):
    return Workload(
        name=f"sweep_n{n}_{'causal' if causal else 'full'}", B=2, H=16, N=n, d=128, causal=causal,
        scale=1.0 / math.sqrt(128), seed=1040 + int(math.log2(n)),
        note="large-head throughput sweep; the same inputs for both mask modes")


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 128, 64, False, 1.0 / 8, 1001, note="tiny forward+backward"),
    "bert_large": Workload("bert_large", 8, 16, 512, 64, False, 1.0 / 8, 1002, kv_len_range=(256, 512),
                           note="BERT-large-shaped, per-batch key padding"),
    "gpt2": Workload("gpt2", 8, 12, 1024, 64, True, 1.0 / 8, 1003, note="GPT-2-shaped causal"),
    **{w.name: w for n in (2048, 4096, 8192, 16384) for w in (_sweep(n, False), _sweep(n, True))},
    "long_64k": Workload("long_64k", 1, 16, 65536, 64, True, 1.0 / 8, 1005, scaled_key_frac=0.01,
                         sampled_rows=64, backward=False,
                         note="long-context causal forward; 1% of key rows x8; 64 sampled query rows"),
    "gqa_n8192": Workload("gqa_n8192", 2, 16, 8192, 128, True, 1.0 / math.sqrt(128), 1006, h_kv=4,
                          note="grouped K/V heads (4 query heads per K/V head), causal, large-head shape"),
    "fp8_outlier": Workload("fp8_outlier", 1, 4, 1000, 128, False, 1.0 / math.sqrt(128), 1008, backward=False,
                            outlier_frac=0.001,
                            note="FP8 forward accuracy: N(0,1) with 0.1% of the q and k entries x16, ragged N"),
    "mqa_n4096": Workload("mqa_n4096", 2, 16, 4096, 128, False, 1.0 / math.sqrt(128), 1007, h_kv=1,
                          note="multi-query attention (one K/V head), large-head shape"),
}


def fp8_signs(d, seed):
    """The +-1 vector (float32 [d]) of the FP8 path's incoherent processing, drawn from
    its own PCG64 generator (seed + 7919) so that it does not disturb any input draw."""
    rng = np.random.default_rng(seed + 7919)
    return np.where(rng.integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)


def get_workload(name):
    return WORKLOADS[name]


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(bits):
    """Exact float64 values of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray          # uint16 bf16 bits [B,H,N,d]
    k: np.ndarray          # [B,H_kv,N,d]
    v: np.ndarray
    do: np.ndarray = None
    kv_len: np.ndarray = None        # int32 [B] or None
    scaled_keys: np.ndarray = None   # int64 indices of key rows multiplied by 8
    rows: np.ndarray = None          # sampled query rows (sorted) or None = all
    extra: dict = field(default_factory=dict)

    def head64(self, name, b, h):
        """fp64 values of one head of tensor `name` ('q','k','v','do')."""
        return bf16_bits_to_f64(getattr(self, name)[b, h])

    def to_torch(self, device):
        """bf16 torch tensors (and int32 kv_len) on `device`."""
        import torch

        def t(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)

        out = {"q": t(self.q), "k": t(self.k), "v": t(self.v)}
        if self.do is not None:
            out["do"] = t(self.do)
        out["kv_len"] = None if self.kv_len is None else torch.from_numpy(self.kv_len.astype(np.int32)).to(device)
        return out


def staircase(B, H, N, d, rise, seed, causal=False, block=64):
    """Inputs whose scores climb along the keys: q = (1, e), k = (rise * (j // block) /
    scale, e'), with e, e' ~ 0.1 N(0, 1) in the other d - 1 dimensions and scale =
    1/sqrt(d), so that the scaled score of key j grows by about `rise` (natural-log units)
    per block of keys.  Every block raises the row maximum: by less than the rescaling
    threshold, by more, or (large rises) by more than the fp32 exponent range of
    un-normalised probabilities.  v, dO ~ N(0, 1).  Draw order: e, e', v, dO."""
    scale = 1.0 / math.sqrt(d)
    w = Workload(f"staircase_{B}x{H}x{N}x{d}_{rise:g}", B, H, N, d, causal, scale, seed, backward=True,
                 note="scores rising by a fixed amount per block of keys")
    rng = np.random.default_rng(seed)
    qf = 0.1 * rng.standard_normal((B, H, N, d), dtype=np.float32)
    kf = 0.1 * rng.standard_normal((B, H, N, d), dtype=np.float32)
    vf = rng.standard_normal((B, H, N, d), dtype=np.float32)
    dof = rng.standard_normal((B, H, N, d), dtype=np.float32)
    qf[..., 0] = 1.0
    kf[..., 0] = (rise / scale) * (np.arange(N, dtype=np.float32) // block)
    return Inputs(workload=w, q=f32_to_bf16_bits(qf), k=f32_to_bf16_bits(kf), v=f32_to_bf16_bits(vf),
                  do=f32_to_bf16_bits(dof))


def generate(w, with_do=None, shape_override=None):
    """Draw the inputs of workload `w` (a Workload or its name).

    shape_override=(B,H,N,d) draws a smaller instance with the same recipe (used by
    tests that need several tiles and a ragged tail at oracle-friendly sizes)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    B, H, N, d = shape_override or w.shape
    group = w.H // w.kv_heads  # query heads per K/V head, kept by a shape override
    if H % group:
        raise ValueError(f"{H} query heads do not split into groups of {group}")
    hkv = H // group
    rng = np.random.default_rng(w.seed)
    qf = rng.standard_normal((B, H, N, d), dtype=np.float32)
    kf = rng.standard_normal((B, hkv, N, d), dtype=np.float32)
    vf = rng.standard_normal((B, hkv, N, d), dtype=np.float32)
    if with_do is None:
        with_do = w.backward
    dof = rng.standard_normal((B, H, N, d), dtype=np.float32) if with_do else None
    kv_len = None
    if w.kv_len_range is not None:
        lo, hi = w.kv_len_range
        lo, hi = min(lo, N), min(hi, N)
        kv_len = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    scaled = None
    if w.scaled_key_frac > 0:
        nsc = max(1, int(math.floor(w.scaled_key_frac * N)))
        scaled = np.sort(rng.choice(N, size=nsc, replace=False))
        kf[:, :, scaled, :] *= 8.0  # exact in bf16
    rows = None
    if w.sampled_rows:
        rows = np.sort(rng.choice(N, size=min(w.sampled_rows, N), replace=False))
    if w.outlier_frac > 0:
        for t in (qf, kf):
            idx = rng.choice(t.size, size=max(1, int(w.outlier_frac * t.size)), replace=False)
            t.reshape(-1)[idx] *= 16.0  # exact in bf16
    return Inputs(
        workload=w,
        q=f32_to_bf16_bits(qf),
        k=f32_to_bf16_bits(kf),
        v=f32_to_bf16_bits(vf),
        do=None if dof is None else f32_to_bf16_bits(dof),
        kv_len=kv_len,
        scaled_keys=scaled,
        rows=rows,
    )
