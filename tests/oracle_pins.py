"""Pins that tie the fp64 oracle to something other than itself.

Every pin takes the oracle modules as arguments (``ref`` = oracle.ref, ``online`` =
oracle.online) so that the mutation tests can run the same pins against copies of the
oracle with a planted mistake and check that at least one pin catches it.

Kinds of pin used (no page prints a numeric example, so none is a page value):
  * hand-derived worked example with a closed form (tests/golden/two_key_example.json);
  * brute force: pure-Python loops over tiny inputs, computing the softmax the naive way
    (exp(s) / sum exp(s), no max subtraction, math.fsum);
  * library special case: torch float64 scaled_dot_product_attention with an explicit
    boolean mask, and torch autograd for the gradients;
  * central finite differences of L = sum(O * dO) for the backward;
  * closed forms and invariants: rows of the softmax sum to one, constant V, the first
    causal row, uniform attention at scale 0, two keys, key shift, key padding,
    permutation equivariance, zero column sum of dK, identical query heads of a K/V
    group (grouped heads);
  * library special case for grouped K/V heads: torch scaled_dot_product_attention
    with enable_gqa=True, forward and autograd;
  * the blocked online recurrence equals the two-pass definition for any block size.
"""

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

MASK_MODES = [(False, None), (True, None), (False, "pad"), (True, "pad")]


def _rng(seed):
    return np.random.default_rng(seed)


def _kv_len(rng, B, N):
    return rng.integers(1, N, size=B, endpoint=True)


def _inputs(seed, B, H, N, d, with_do=False):
    rng = _rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    do = rng.standard_normal((B, H, N, d)) if with_do else None
    return rng, q, k, v, do


def _mask_args(mode, rng, B, N):
    causal, pad = mode
    return causal, (_kv_len(rng, B, N) if pad else None)


def _admissible_py(i, j, causal, kl):
    if causal and j > i:
        return False
    if kl is not None and j >= kl:
        return False
    return True


# ----------------------------------------------------------------------------------
def pin_golden_two_key(ref, online):
    with open(os.path.join(GOLDEN, "two_key_example.json")) as f:
        g = json.load(f)
    ln3 = math.log(3.0)
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    do = np.array(g["do"])[None, None]
    lse_vals = {"ln(4)": math.log(4.0), "ln(10)": math.log(10.0), "0": 0.0}
    for key, causal in (("noncausal", False), ("causal", True)):
        e = g[key]
        o, lse = ref.attention_forward(q, k, v, ln3, causal=causal)
        np.testing.assert_allclose(o[0, 0], np.array(e["o"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], [lse_vals[x] for x in e["lse_expr"]], rtol=0, atol=1e-12)
        dq, dk, dv = ref.attention_backward(q, k, v, do, ln3, causal=causal)
        np.testing.assert_allclose(dv[0, 0], np.array(e["dv"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq[0, 0] / ln3, np.array(e["dq_over_ln3"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk[0, 0] / ln3, np.array(e["dk_over_ln3"]), rtol=0, atol=1e-12)


def pin_bruteforce_forward(ref, online):
    for seed, (N, d) in enumerate([(1, 1), (3, 2), (5, 3), (6, 2)]):
        for mode in MASK_MODES:
            rng, q, k, v, _ = _inputs(100 + seed, 2, 1, N, d)
            causal, kv = _mask_args(mode, rng, 2, N)
            scale = 0.7
            o, lse = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv)
            for b in range(2):
                kl = None if kv is None else int(kv[b])
                for i in range(N):
                    w = []
                    for j in range(N):
                        if _admissible_py(i, j, causal, kl):
                            s = scale * sum(q[b, 0, i, t] * k[b, 0, j, t] for t in range(d))
                            w.append((j, math.exp(s)))
                    z = math.fsum(x for _, x in w)
                    for t in range(d):
                        want = math.fsum(x * v[b, 0, j, t] for j, x in w) / z
                        assert abs(o[b, 0, i, t] - want) < 1e-12, ("O", mode, b, i, t)
                    assert abs(lse[b, 0, i] - math.log(z)) < 1e-12, ("LSE", mode, b, i)


def _torch_mask(N, causal, kl):
    import torch

    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    m = torch.ones(N, N, dtype=torch.bool)
    if causal:
        m &= j <= i
    if kl is not None:
        m &= j < int(kl)
    return m


def pin_torch_sdpa_forward(ref, online):
    import torch
    import torch.nn.functional as F

    for seed, (N, d) in enumerate([(7, 4), (33, 16), (40, 8)]):
        for mode in MASK_MODES:
            rng, q, k, v, _ = _inputs(200 + seed, 2, 2, N, d)
            causal, kv = _mask_args(mode, rng, 2, N)
            scale = 1.0 / math.sqrt(d)
            o, lse = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv)
            for b in range(2):
                kl = None if kv is None else kv[b]
                m = _torch_mask(N, causal, kl)
                tq, tk, tv = (torch.from_numpy(x[b]) for x in (q, k, v))
                to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
                np.testing.assert_allclose(o[b], to.numpy(), rtol=0, atol=1e-12)
                s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
                s = s.masked_fill(~m, float("-inf"))
                np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def pin_torch_autograd_backward(ref, online):
    import torch
    import torch.nn.functional as F

    for seed, (N, d) in enumerate([(9, 4), (24, 8)]):
        for mode in MASK_MODES:
            rng, q, k, v, do = _inputs(300 + seed, 2, 2, N, d, with_do=True)
            causal, kv = _mask_args(mode, rng, 2, N)
            scale = 0.37
            dq, dk, dv = ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv)
            for b in range(2):
                kl = None if kv is None else kv[b]
                m = _torch_mask(N, causal, kl)
                tq, tk, tv = (torch.from_numpy(x[b].copy()).requires_grad_(True) for x in (q, k, v))
                to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
                to.backward(torch.from_numpy(do[b]))
                np.testing.assert_allclose(dq[b], tq.grad.numpy(), rtol=0, atol=1e-11)
                np.testing.assert_allclose(dk[b], tk.grad.numpy(), rtol=0, atol=1e-11)
                np.testing.assert_allclose(dv[b], tv.grad.numpy(), rtol=0, atol=1e-11)


def pin_finite_differences(ref, online):
    eps = 1e-6
    for seed, (N, d) in enumerate([(5, 3), (8, 2)]):
        for mode in MASK_MODES:
            rng, q, k, v, do = _inputs(400 + seed, 1, 1, N, d, with_do=True)
            causal, kv = _mask_args(mode, rng, 1, N)
            scale = 0.9
            grads = ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv)

            def loss(qq, kk, vv):
                o, _ = ref.attention_forward(qq, kk, vv, scale, causal=causal, kv_len=kv)
                return float((o * do).sum())

            for which, g in enumerate(grads):
                fd = np.zeros_like(g)
                for idx in np.ndindex(g.shape):
                    args_p = [q.copy(), k.copy(), v.copy()]
                    args_m = [q.copy(), k.copy(), v.copy()]
                    args_p[which][idx] += eps
                    args_m[which][idx] -= eps
                    fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
                err = np.abs(fd - g).max() / max(1e-3, np.abs(g).max())
                assert err < 1e-6, ("finite differences", mode, which, err)


def pin_softmax_rows_sum_to_one(ref, online):
    for mode in MASK_MODES:
        rng, q, k, v, _ = _inputs(500, 2, 3, 29, 8)
        causal, kv = _mask_args(mode, rng, 2, 29)
        scale = 0.5
        _, lse = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv)
        for b in range(2):
            kl = None if kv is None else int(kv[b])
            for h in range(3):
                s = scale * q[b, h] @ k[b, h].T
                for i in range(29):
                    tot = math.fsum(math.exp(s[i, j] - lse[b, h, i]) for j in range(29) if _admissible_py(i, j, causal, kl))
                    assert abs(tot - 1.0) < 1e-12, ("row sum", mode, b, h, i)


def pin_constant_v(ref, online):
    for mode in MASK_MODES:
        rng, q, k, _, _ = _inputs(600, 2, 2, 17, 5)
        causal, kv = _mask_args(mode, rng, 2, 17)
        c = rng.standard_normal(5)
        v = np.broadcast_to(c, q.shape).copy()
        o, _ = ref.attention_forward(q, k, v, 1.3, causal=causal, kv_len=kv)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-12)


def pin_causal_first_row(ref, online):
    rng, q, k, v, _ = _inputs(700, 2, 2, 13, 6)
    scale = 0.8
    o, lse = ref.attention_forward(q, k, v, scale, causal=True)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], scale * (q[:, :, 0] * k[:, :, 0]).sum(-1), rtol=0, atol=1e-13)


def pin_uniform_scale_zero(ref, online):
    N = 11
    for mode in MASK_MODES:
        rng, q, k, v, do = _inputs(800, 2, 2, N, 4, with_do=True)
        causal, kv = _mask_args(mode, rng, 2, N)
        o, lse = ref.attention_forward(q, k, v, 0.0, causal=causal, kv_len=kv)
        dq, dk, dv = ref.attention_backward(q, k, v, do, 0.0, causal=causal, kv_len=kv)
        for b in range(2):
            kl = N if kv is None else int(kv[b])
            for i in range(N):
                n_i = min(i + 1, kl) if causal else kl
                np.testing.assert_allclose(o[b, :, i], v[b, :, :n_i].mean(axis=1), rtol=0, atol=1e-13)
                np.testing.assert_allclose(lse[b, :, i], math.log(n_i), rtol=0, atol=1e-13)
            for j in range(N):
                want = np.zeros((2, 4))
                for i in range(N):
                    n_i = min(i + 1, kl) if causal else kl
                    if _admissible_py(i, j, causal, kl):
                        want += do[b, :, i] / n_i
                np.testing.assert_allclose(dv[b, :, j], want, rtol=0, atol=1e-13)
        assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0


def pin_two_keys(ref, online):
    rng, q, k, v, _ = _inputs(900, 1, 3, 2, 4)
    scale = 1.1
    o, _ = ref.attention_forward(q, k, v, scale)
    for h in range(3):
        for i in range(2):
            s0 = scale * q[0, h, i] @ k[0, h, 0]
            s1 = scale * q[0, h, i] @ k[0, h, 1]
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            np.testing.assert_allclose(o[0, h, i], w0 * v[0, h, 0] + w1 * v[0, h, 1], rtol=0, atol=1e-14)


def pin_key_shift(ref, online):
    for mode in MASK_MODES:
        rng, q, k, v, _ = _inputs(1000, 2, 2, 15, 6)
        causal, kv = _mask_args(mode, rng, 2, 15)
        scale = 0.6
        c = rng.standard_normal(6)
        o1, l1 = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv)
        o2, l2 = ref.attention_forward(q, k + c, v, scale, causal=causal, kv_len=kv)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2, l1 + scale * (q @ c), rtol=0, atol=1e-12)


def pin_padding(ref, online):
    N = 19
    for causal in (False, True):
        rng, q, k, v, do = _inputs(1100, 3, 2, N, 5, with_do=True)
        kv = rng.integers(1, N, size=3, endpoint=True)
        k2, v2 = k.copy(), v.copy()
        for b in range(3):
            k2[b, :, kv[b]:] = rng.standard_normal(k2[b, :, kv[b]:].shape) * 5
            v2[b, :, kv[b]:] = rng.standard_normal(v2[b, :, kv[b]:].shape) * 5
        o1, l1 = ref.attention_forward(q, k, v, 0.7, causal=causal, kv_len=kv)
        o2, l2 = ref.attention_forward(q, k2, v2, 0.7, causal=causal, kv_len=kv)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
        np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)
        g1 = ref.attention_backward(q, k, v, do, 0.7, causal=causal, kv_len=kv)
        g2 = ref.attention_backward(q, k2, v2, do, 0.7, causal=causal, kv_len=kv)
        np.testing.assert_allclose(g2[0], g1[0], rtol=0, atol=1e-13)
        for b in range(3):
            assert np.abs(g2[1][b, :, kv[b]:]).max(initial=0.0) == 0.0
            assert np.abs(g2[2][b, :, kv[b]:]).max(initial=0.0) == 0.0


def pin_permutation(ref, online):
    rng, q, k, v, _ = _inputs(1200, 1, 2, 21, 4)
    perm_k = rng.permutation(21)
    perm_q = rng.permutation(21)
    o, lse = ref.attention_forward(q, k, v, 0.9)
    o2, lse2 = ref.attention_forward(q, k[:, :, perm_k], v[:, :, perm_k], 0.9)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-12)
    o3, lse3 = ref.attention_forward(q[:, :, perm_q], k, v, 0.9)
    np.testing.assert_allclose(o3, o[:, :, perm_q], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse3, lse[:, :, perm_q], rtol=0, atol=1e-12)


def pin_dk_columns_sum_to_zero(ref, online):
    # each softmax row sums to one, so each row of dS sums to zero and sum_j dK_j = 0
    for mode in MASK_MODES:
        rng, q, k, v, do = _inputs(1300, 2, 2, 14, 3, with_do=True)
        causal, kv = _mask_args(mode, rng, 2, 14)
        _, dk, _ = ref.attention_backward(q, k, v, do, 0.8, causal=causal, kv_len=kv)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)


def pin_sampled_rows_match_full(ref, online):
    for mode in MASK_MODES:
        rng, q, k, v, do = _inputs(1400, 2, 1, 23, 4, with_do=True)
        causal, kv = _mask_args(mode, rng, 2, 23)
        o, lse = ref.attention_forward(q, k, v, 0.4, causal=causal, kv_len=kv)
        dq, _, _ = ref.attention_backward(q, k, v, do, 0.4, causal=causal, kv_len=kv)
        rows = np.array([0, 5, 22, 11])
        for b in range(2):
            kl = None if kv is None else int(kv[b])
            orow, lrow = ref.forward_rows(q[b, 0], k[b, 0], v[b, 0], 0.4, rows, causal=causal, kv_len_b=kl)
            np.testing.assert_allclose(orow, o[b, 0, rows], rtol=0, atol=1e-13)
            np.testing.assert_allclose(lrow, lse[b, 0, rows], rtol=0, atol=1e-13)
            dqr = ref.backward_dq_rows(q[b, 0], k[b, 0], v[b, 0], do[b, 0], 0.4, rows, causal=causal, kv_len_b=kl)
            np.testing.assert_allclose(dqr, dq[b, 0, rows], rtol=0, atol=1e-13)


def pin_sampled_key_columns(ref, online):
    """dK, dV of selected key rows (backward_dkdv_cols) against torch float64 autograd
    and against the full oracle backward, whole-row and in chunks of 3 and 7 query rows,
    every mask mode, a positive and a negative scale; the selection includes the first
    and last key and, with padding, keys past kv_len (zero gradients)."""
    import torch
    import torch.nn.functional as F

    saved = ref._ROW_CHUNK
    try:
        for seed, (N, d, scale) in enumerate([(21, 5, 0.55), (34, 6, -0.35)]):
            for mode in MASK_MODES:
                rng, q, k, v, do = _inputs(1470 + seed, 2, 1, N, d, with_do=True)
                causal, kv = _mask_args(mode, rng, 2, N)
                cols = np.array([N - 1, 0, 7, 3, N // 2, N - 2])
                ref._ROW_CHUNK = saved
                _, dk_full, dv_full = ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv)
                for b in range(2):
                    kl = None if kv is None else kv[b]
                    m = _torch_mask(N, causal, kl)
                    tq, tk, tv = (torch.from_numpy(x[b, 0].copy()).requires_grad_(True) for x in (q, k, v))
                    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
                    to.backward(torch.from_numpy(do[b, 0]))
                    for chunk in (saved, 3, 7):
                        ref._ROW_CHUNK = chunk
                        dkc, dvc = ref.backward_dkdv_cols(q[b, 0], k[b, 0], v[b, 0], do[b, 0], scale, cols,
                                                          causal=causal, kv_len_b=None if kl is None else int(kl))
                        np.testing.assert_allclose(dkc, tk.grad.numpy()[cols], rtol=0, atol=1e-11)
                        np.testing.assert_allclose(dvc, tv.grad.numpy()[cols], rtol=0, atol=1e-11)
                        np.testing.assert_allclose(dkc, dk_full[b, 0, cols], rtol=0, atol=1e-12)
                        np.testing.assert_allclose(dvc, dv_full[b, 0, cols], rtol=0, atol=1e-12)
    finally:
        ref._ROW_CHUNK = saved


def pin_row_chunks(ref, online):
    """The oracle's row-chunked path (taken for long sequences) against torch float64
    SDPA and autograd and against the single-chunk result, with chunks of 3 and 7 rows
    over N = 20 and 37 (ragged last chunk), every mask mode, a positive and a negative
    scale.  dK and dV are sums over all query chunks, so a chunk that overwrote instead
    of accumulating, or rows not offset by the chunk start, fail here."""
    import torch
    import torch.nn.functional as F

    saved = ref._ROW_CHUNK
    try:
        for seed, (N, d, scale) in enumerate([(20, 6, 0.45), (37, 5, -0.3)]):
            for mode in MASK_MODES:
                rng, q, k, v, do = _inputs(1450 + seed, 2, 2, N, d, with_do=True)
                causal, kv = _mask_args(mode, rng, 2, N)
                ref._ROW_CHUNK = saved
                o1, l1 = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv)
                g1 = ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv)
                for chunk in (3, 7):
                    ref._ROW_CHUNK = chunk
                    o, lse = ref.attention_forward(q, k, v, scale, causal=causal, kv_len=kv)
                    g = ref.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv)
                    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-13)
                    np.testing.assert_allclose(lse, l1, rtol=0, atol=1e-13)
                    for a, b_ in zip(g, g1):
                        np.testing.assert_allclose(a, b_, rtol=0, atol=1e-12)
                    for b in range(2):
                        kl = None if kv is None else kv[b]
                        m = _torch_mask(N, causal, kl)
                        tq, tk, tv = (torch.from_numpy(x[b].copy()).requires_grad_(True) for x in (q, k, v))
                        to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)
                        to.backward(torch.from_numpy(do[b]))
                        np.testing.assert_allclose(o[b], to.detach().numpy(), rtol=0, atol=1e-12)
                        s = (torch.matmul(tq, tk.transpose(-1, -2)) * scale).masked_fill(~m, float("-inf"))
                        np.testing.assert_allclose(lse[b], torch.logsumexp(s, dim=-1).detach().numpy(), rtol=0,
                                                   atol=1e-12)
                        for a, tg in zip(g, (tq.grad, tk.grad, tv.grad)):
                            np.testing.assert_allclose(a[b], tg.numpy(), rtol=0, atol=1e-11)
    finally:
        ref._ROW_CHUNK = saved


def pin_online_equals_two_pass(ref, online):
    rng = _rng(1500)
    for N, d in [(1, 3), (17, 4), (64, 8)]:
        q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
        k[rng.choice(N, size=max(1, N // 8), replace=False)] *= 8.0  # force large max jumps
        for causal in (False, True):
            for kl in (None, max(1, N // 2)):
                o_ref, l_ref = ref.forward_rows(q, k, v, 0.5, np.arange(N), causal=causal, kv_len_b=kl)
                for block in sorted({1, 2, 5, 16, N}):
                    for tau in (None, 0.0, 3.0, 8.0 * math.log(2.0)):
                        o, l, _ = online.online_forward_head(q, k, v, 0.5, block, causal=causal, kv_len_b=kl, tau=tau)
                        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
                        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


def pin_torch_sdpa_gqa(ref, online):
    """Grouped K/V heads against torch's own grouped-query attention (enable_gqa) in
    float64, forward and autograd backward, under every mask mode; MQA included."""
    import torch
    import torch.nn.functional as F

    for seed, (H, Hkv, N, d) in enumerate([(4, 2, 11, 4), (6, 3, 16, 8), (4, 1, 9, 4)]):
        for mode in MASK_MODES:
            rng, q, _, _, do = _inputs(1600 + seed, 2, H, N, d, with_do=True)
            k = rng.standard_normal((2, Hkv, N, d))
            v = rng.standard_normal((2, Hkv, N, d))
            causal, kv = _mask_args(mode, rng, 2, N)
            scale = 0.45
            o, lse = ref.attention_forward_gqa(q, k, v, scale, causal=causal, kv_len=kv)
            dq, dk, dv = ref.attention_backward_gqa(q, k, v, do, scale, causal=causal, kv_len=kv)
            for b in range(2):
                kl = None if kv is None else kv[b]
                m = _torch_mask(N, causal, kl)
                tq, tk, tv = (torch.from_numpy(x[b].copy()).requires_grad_(True) for x in (q, k, v))
                to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=True)
                to.backward(torch.from_numpy(do[b]))
                np.testing.assert_allclose(o[b], to.detach().numpy(), rtol=0, atol=1e-12)
                np.testing.assert_allclose(dq[b], tq.grad.numpy(), rtol=0, atol=1e-11)
                np.testing.assert_allclose(dk[b], tk.grad.numpy(), rtol=0, atol=1e-11)
                np.testing.assert_allclose(dv[b], tv.grad.numpy(), rtol=0, atol=1e-11)
                # LSE: per query head against its own K/V head (h // G), torch logsumexp
                G = H // Hkv
                for h in range(H):
                    s = torch.from_numpy(q[b, h]) @ torch.from_numpy(k[b, h // G]).T * scale
                    s = s.masked_fill(~m, float("-inf"))
                    np.testing.assert_allclose(lse[b, h], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def pin_gqa_identical_heads(ref, online):
    """Closed form: when all G query heads of a group carry the same Q and dO, every
    query head sees the same attention, so dK and dV are G times the single-head
    gradients and each O head equals the single-head output."""
    rng = _rng(1700)
    for G in (2, 3):
        N, d = 10, 4
        q1 = rng.standard_normal((1, 1, N, d))
        do1 = rng.standard_normal((1, 1, N, d))
        k = rng.standard_normal((1, 1, N, d))
        v = rng.standard_normal((1, 1, N, d))
        for causal in (False, True):
            o1, _ = ref.attention_forward(q1, k, v, 0.6, causal=causal)
            _, dk1, dv1 = ref.attention_backward(q1, k, v, do1, 0.6, causal=causal)
            q = np.repeat(q1, G, axis=1)
            do = np.repeat(do1, G, axis=1)
            o, _ = ref.attention_forward_gqa(q, k, v, 0.6, causal=causal)
            _, dk, dv = ref.attention_backward_gqa(q, k, v, do, 0.6, causal=causal)
            for h in range(G):
                np.testing.assert_allclose(o[0, h], o1[0, 0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(dk, G * dk1, rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv, G * dv1, rtol=0, atol=1e-12)


ALL_PINS = [
    pin_golden_two_key,
    pin_bruteforce_forward,
    pin_torch_sdpa_forward,
    pin_torch_autograd_backward,
    pin_finite_differences,
    pin_softmax_rows_sum_to_one,
    pin_constant_v,
    pin_causal_first_row,
    pin_uniform_scale_zero,
    pin_two_keys,
    pin_key_shift,
    pin_padding,
    pin_permutation,
    pin_dk_columns_sum_to_zero,
    pin_sampled_rows_match_full,
    pin_sampled_key_columns,
    pin_row_chunks,
    pin_online_equals_two_pass,
    pin_torch_sdpa_gqa,
    pin_gqa_identical_heads,
]


def failing_pins(ref, online):
    """Names of the pins that fail for the given oracle modules."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(ref, online)
        except Exception:  # a planted mistake may also raise (shape errors, NaN, ...)
            bad.append(pin.__name__)
    return bad
