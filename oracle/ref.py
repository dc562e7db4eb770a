"""Plain fp64 CPU oracle for exact scaled-dot-product attention (forward and backward).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute
this module: only the test suite, the smoke check and the bench's CPU-baseline leg use
it.  It shares no code with the HIP kernels and never touches a GPU.

What it computes
----------------
The pages define FlashAttention as an *exact* attention algorithm: it produces the same
output as standard attention and only changes how the work is scheduled through the
memory hierarchy ("FlashAttention" concept wiki page, section 定義; singularity-lens
FA1 explainer, paragraphs on tiling and on the online softmax, which stress that the
result is identical to standard attention).  The oracle is therefore the standard
attention pipeline the FA1 explainer describes -- scores, softmax normalisation, value
product, each materialised in full (explainer, paragraph on the memory hierarchy and the
HBM round trips of standard attention) -- written out in fp64 with numpy, one (batch,
head) at a time:

    S   = scale * Q K^T                               (N x N, masked entries = -inf)
    P   = exp(S - rowmax S) / rowsum(exp(S - rowmax S))   (two-pass softmax)
    O   = P V
    LSE = rowmax S + log rowsum exp(S - rowmax S)     (natural log)

The backward pass is the gradient of L = sum(O * dO) for a given upstream gradient dO.
The pages say only that the backward recomputes the attention matrix on chip instead of
storing it (wiki page, 定義 (2); explainer, paragraph on recomputation); the formulas
below follow from the softmax Jacobian and are pinned against finite differences and
torch autograd in the test suite:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij          ( = sum_k dO_ik O_ik )
    dS = P * (dP - D)
    dQ = scale * dS K ,   dK = scale * dS^T Q

Readings where the pages are silent (masks and the log-sum-exp are not on the pages):
  * causal: query i attends keys j <= i (square problem, N_q = N_k);
  * key padding: for batch b only keys j < kv_len[b] are attended, every query row is
    a real output;
  * masks are applied after scaling, as -inf; a query row with no admissible key has
    O = 0, LSE = -inf and contributes nothing to any gradient;
  * LSE is the natural-log log-sum-exp of the scaled, masked scores.

Large N: rows are processed in chunks of complete length-N score rows.  Each chunk still
holds every key of its rows and applies the exact two-pass softmax -- this is the
definition with rows buffered, not a blocked recurrence over keys.
"""

import numpy as np

__all__ = [
    "admissible",
    "attention_forward",
    "attention_backward",
    "forward_rows",
    "backward_dq_rows",
    "backward_dkdv_cols",
]

_ROW_CHUNK = 1024


def admissible(rows, n_keys, causal, kv_len_b):
    """Boolean [len(rows), n_keys] mask of the keys each query row may attend.

    causal: key j admissible for query i iff j <= i.  kv_len_b (int or None): key j
    admissible iff j < kv_len_b.  Both conditions hold together when both are given.
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(n_keys, dtype=np.int64)
    ok = np.ones((rows.shape[0], n_keys), dtype=bool)
    if causal:
        ok &= keys[None, :] <= rows[:, None]
    if kv_len_b is not None:
        ok &= keys[None, :] < int(kv_len_b)
    return ok


def _softmax_rows(s, ok):
    """Two-pass softmax of the score rows s under mask ok.

    Returns (P, LSE) with P = 0 and LSE = -inf on rows with no admissible key.
    """
    s = np.where(ok, s, -np.inf)
    any_ok = ok.any(axis=1)
    m = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(ok, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    safe_l = np.where(any_ok, l, 1.0)
    p = e / safe_l[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(any_ok, m + np.log(safe_l), -np.inf)
    return p, lse


def _head_forward(q, k, v, scale, causal, kv_len_b, rows):
    """O and LSE of the selected query rows of one head (q: [N,d] fp64)."""
    n = k.shape[0]
    s = scale * (q[rows] @ k.T)
    ok = admissible(rows, n, causal, kv_len_b)
    p, lse = _softmax_rows(s, ok)
    return p @ v, lse


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def attention_forward(q, k, v, scale, causal=False, kv_len=None):
    """Exact attention forward.  q,k,v: [B,H,N,d]; kv_len: None or int array [B].

    Returns O [B,H,N,d] fp64 and LSE [B,H,N] fp64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            for r0 in range(0, N, _ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + _ROW_CHUNK))
                o[b, h, rows], lse[b, h, rows] = _head_forward(q[b, h], k[b, h], v[b, h], scale, causal, kl, rows)
    return o, lse


def _head_backward(q, k, v, do, scale, causal, kv_len_b):
    """dQ, dK, dV of one head for the loss L = sum(O * dO)."""
    n, d = q.shape
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    for r0 in range(0, n, _ROW_CHUNK):
        rows = np.arange(r0, min(n, r0 + _ROW_CHUNK))
        s = scale * (q[rows] @ k.T)
        ok = admissible(rows, n, causal, kv_len_b)
        p, _ = _softmax_rows(s, ok)
        dor = do[rows]
        dv += p.T @ dor
        dp = dor @ v.T
        dsum = (p * dp).sum(axis=1)
        ds = p * (dp - dsum[:, None])
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal=False, kv_len=None):
    """Gradients (dQ, dK, dV), each [B,H,N,d] fp64, of L = sum(O * dO)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    for b in range(B):
        kl = None if kv_len is None else int(kv_len[b])
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _head_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, kl)
    return dq, dk, dv


def _kv_group(H, Hkv):
    """Query heads per K/V head; query head h reads K/V head h // G."""
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"K/V heads ({Hkv}) must divide query heads ({H})")
    return H // Hkv


def attention_forward_gqa(q, k, v, scale, causal=False, kv_len=None):
    """Grouped-query / multi-query attention forward.  q: [B,H,N,d]; k, v: [B,Hkv,N,d]
    with Hkv dividing H.

    The "FlashAttention" concept wiki page names GQA/MQA among its open questions
    (section 未解決の問い) without defining it.  Reading: consecutive query heads form
    the groups, query head h uses K/V head h // (H / Hkv), and the result is ordinary
    attention with each K/V head repeated for its group -- written out as that repeat.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    G = _kv_group(q.shape[1], k.shape[1])
    return attention_forward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), scale, causal=causal,
                             kv_len=kv_len)


def attention_backward_gqa(q, k, v, do, scale, causal=False, kv_len=None):
    """Gradients of L = sum(O * dO) for grouped K/V heads: dQ [B,H,N,d]; dK, dV
    [B,Hkv,N,d].  A repeated K/V head receives the sum of the gradients of its copies
    (chain rule through the repeat in attention_forward_gqa)."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = _kv_group(H, Hkv)
    dq, dk, dv = attention_backward(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, scale, causal=causal,
                                    kv_len=kv_len)
    return dq, dk.reshape(B, Hkv, G, N, d).sum(axis=2), dv.reshape(B, Hkv, G, N, d).sum(axis=2)


def forward_rows(q, k, v, scale, rows, causal=False, kv_len_b=None):
    """O and LSE of a few query rows of ONE head (q,k,v: [N,d]); for sampled checks at
    sizes where the full forward would be slow.  Each row is computed independently
    from all N keys, exactly as in attention_forward."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    return _head_forward(q, k, v, scale, causal, kv_len_b, np.asarray(rows, dtype=np.int64))


def backward_dq_rows(q, k, v, do, scale, rows, causal=False, kv_len_b=None):
    """dQ of a few query rows of ONE head.  Row i of dQ needs only row i of P and dP:
    dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j with D_i = sum_j P_ij dP_ij."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    rows = np.asarray(rows, dtype=np.int64)
    n = k.shape[0]
    s = scale * (q[rows] @ k.T)
    ok = admissible(rows, n, causal, kv_len_b)
    p, _ = _softmax_rows(s, ok)
    dp = do[rows] @ v.T
    dsum = (p * dp).sum(axis=1)
    ds = p * (dp - dsum[:, None])
    return scale * (ds @ k)


def backward_dkdv_cols(q, k, v, do, scale, cols, causal=False, kv_len_b=None):
    """dK and dV of a few key rows ("columns" of P) of ONE head.  Key j's gradients sum
    over every query row: dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i dS_ij Q_i with
    dS_ij = P_ij (dP_ij - D_i).  Each P row is normalised over all of its keys and each
    D_i sums over all of its keys, so every query row is still computed in full (in row
    chunks, as attention_backward does); only the selected columns are kept."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    cols = np.asarray(cols, dtype=np.int64)
    n, d = q.shape
    dk = np.zeros((cols.shape[0], d))
    dv = np.zeros((cols.shape[0], d))
    for r0 in range(0, n, _ROW_CHUNK):
        rows = np.arange(r0, min(n, r0 + _ROW_CHUNK))
        s = scale * (q[rows] @ k.T)
        ok = admissible(rows, n, causal, kv_len_b)
        p, _ = _softmax_rows(s, ok)
        dor = do[rows]
        dp = dor @ v.T
        dsum = (p * dp).sum(axis=1)
        p_c = p[:, cols]
        ds_c = p_c * (dp[:, cols] - dsum[:, None])
        dv += p_c.T @ dor
        dk += scale * (ds_c.T @ q[rows])
    return dk, dv
