"""fp64 blocked online-softmax recurrence (the algorithm the GPU kernels implement).

TEST INFRASTRUCTURE ONLY: used by the test suite to show that the blocked recurrence
equals the two-pass definition in ``oracle.ref``; never imported by the product path.

The steps follow the pages' description of tiling plus online softmax: keys and values
are visited block by block; for each query row a running maximum and a running sum of
exponentials are kept; when a block brings a larger maximum, the partial sum and the
partial output accumulated so far are rescaled by exp(m_old - m_new) so that the final
result equals the exact softmax ("FlashAttention" concept wiki page, 定義 (1);
singularity-lens FA1 explainer, paragraphs on tiling and on the online softmax).  The
output is normalised once at the end and the per-row log-sum-exp is kept for the
backward pass (the wiki page's FA2 (1), fewer non-matmul operations -- our reading).

Optional conditional rescaling (FlashAttention-4 summary, 提案手法 second optimisation;
wiki page FA4 (2)): the pages give no rule, so we take this reading -- the reference
maximum m_ref used inside exp() is only moved up when the new row maximum exceeds it by
more than ``tau`` (natural-log units).  The result is exact for any m_ref because
O = sum exp(s - m_ref) v / sum exp(s - m_ref) and LSE = m_ref + log(sum exp(s - m_ref));
tau only bounds how large the un-normalised terms may grow (at most exp(tau)).
"""

import numpy as np

__all__ = ["online_forward_head"]


def online_forward_head(q, k, v, scale, block, causal=False, kv_len_b=None, tau=None):
    """Blocked online-softmax forward of one head.

    q,k,v: [N,d]; block: number of keys per step (1..N); tau: None (always rescale to
    the new maximum) or a threshold >= 0 for conditional rescaling.
    Returns (O [N,d], LSE [N], n_rescales) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    m = np.full(n, -np.inf)          # reference maximum per row
    l = np.zeros(n)                  # running sum of exp(s - m)
    acc = np.zeros((n, d))           # running sum of exp(s - m) * v
    rows = np.arange(n)
    n_rescales = 0
    for j0 in range(0, n, block):
        keys = np.arange(j0, min(n, j0 + block))
        s = scale * (q @ k[keys].T)
        ok = np.ones_like(s, dtype=bool)
        if causal:
            ok &= keys[None, :] <= rows[:, None]
        if kv_len_b is not None:
            ok &= keys[None, :] < kv_len_b
        s = np.where(ok, s, -np.inf)
        blk_max = s.max(axis=1)
        cand = np.maximum(m, blk_max)
        if tau is None:
            move = cand > m
        else:
            move = (m == -np.inf) | (cand - m > tau)
        new_m = np.where(move, cand, m)
        # rescale what was accumulated under the old reference maximum
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(new_m), new_m, 0.0)), 0.0)
        alpha = np.where(move, alpha, 1.0)
        n_rescales += int(np.count_nonzero(move & np.isfinite(m)))
        base = np.where(np.isfinite(new_m), new_m, 0.0)
        p = np.where(ok, np.exp(s - base[:, None]), 0.0)
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[keys]
        m = new_m
    any_ok = l > 0
    o = np.where(any_ok[:, None], acc / np.where(any_ok, l, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(any_ok, m + np.log(np.where(any_ok, l, 1.0)), -np.inf)
    return o, lse, n_rescales
