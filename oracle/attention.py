"""CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in ``oracle/``.  The
product path (the HIP library and its Python binding) never calls it, and this
module imports nothing from the product.

What it computes is the plain definition of softmax attention, written out in
float64 with NumPy, with no tiling, no online rescaling and no fusion:

* "From-scratch CUDA attention kernel reaches 94.4% of FlashAttention-4 on
  NVIDIA B200", section "How the kernel partitions its work": scores are
  S = Q K^T, a softmax turns them into P, and the output is P V; Q, K, V and O
  are laid out as (batch, heads, sequence, head_dim).
* "FlashStieltjes ...", section "The challenge": the softmax is the
  exponentials of the scores divided by their sum; the single-pass running
  max / running sum form is only a faster route to the same number, so the
  oracle uses the direct two-pass form.
* "FlashAttention for Tesla P100", section "What it supports": causal masking
  of the upper triangle, grouped-query heads (Hq a multiple of Hkv), arbitrary
  sequence length.
* Same page, section "Documentation": the backward's score gradient is
  dS = P * (dP - D) and the value gradient is dV = P^T dO.  D (the per-row
  dot product of dO and O) and dQ = scale * dS K, dK = scale * dS^T Q follow
  from the chain rule; finite differences pin them in the tests.

Readings taken where the pages are silent:

* ``scale`` multiplies Q K^T before the softmax; the log-sum-exp (LSE) is the
  natural-log log-sum-exp of the *scaled* scores over the visible keys.
* causal means square, top-left aligned: key j is visible to query i iff j <= i.
* query head ``hq`` reads KV head ``hq // (Hq // Hkv)``; dK and dV of a KV head
  sum the contributions of every query head in its group.

Every function here is pinned against something other than itself in
``tests/test_oracle.py`` (closed forms, invariants, finite differences, a
pure-Python brute force and the worked numbers printed on the pages).  No
function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head",
    "visible_mask",
    "softmax_probs",
    "attention_forward",
    "attention_backward",
    "attention_dq_rows",
]


def kv_head(hq: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head ``hq``: consecutive query heads share one KV head."""
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return hq // (Hq // Hkv)


def visible_mask(rows, cols, causal: bool) -> np.ndarray:
    """Boolean (len(rows), len(cols)) mask: True where query ``rows[r]`` may see key ``cols[c]``.

    ``cols`` may also be an int n, meaning keys 0..n-1.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(cols, dtype=np.int64) if np.isscalar(cols) else np.asarray(cols, dtype=np.int64)
    if causal:
        return cols[None, :] <= rows[:, None]
    return np.ones((rows.shape[0], cols.shape[0]), dtype=bool)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (B, H, N, D)")
    B, Hq, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise ValueError("k and v must be (B, Hkv, N, D) with the same B, N, D as q")
    Hkv = k.shape[1]
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return B, Hq, Hkv, N, D


def softmax_probs(q_rows: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray,
                  causal: bool):
    """Scores, probabilities and LSE for some query rows of one head.

    ``q_rows`` is (R, D) (the query vectors of the rows listed in ``rows``),
    ``k`` is (N, D).  Returns (S, P, LSE): S = scale * q_rows k^T, P the row
    softmax over the visible keys (0 elsewhere), LSE = m + ln(sum exp(S - m))
    with m the row maximum over visible keys.  All float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S = scale * (q_rows @ k.T)
    vis = visible_mask(rows, k.shape[0], causal)
    masked = np.where(vis, S, -np.inf)
    m = masked.max(axis=1)                       # every row has >= 1 visible key
    e = np.where(vis, np.exp(masked - m[:, None]), 0.0)
    lse = m + np.log(e.sum(axis=1))
    P = np.where(vis, np.exp(masked - lse[:, None]), 0.0)
    return S, P, lse


def attention_forward(q, k, v, scale: float, causal: bool, rows=None, block: int = 512):
    """O and LSE of exact softmax attention, float64.

    q: (B, Hq, N, D); k, v: (B, Hkv, N, D); any real dtype (upcast to float64).
    ``rows``: optional 1-D array of query indices; if given, only those rows
    are computed and O is (B, Hq, len(rows), D), LSE (B, Hq, len(rows)).
    ``block`` only bounds memory (query rows per materialised score block).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, N, D = _check_shapes(q, k, v)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, Hq, R, D), dtype=np.float64)
    L = np.zeros((B, Hq, R), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head(hq, Hq, Hkv)
            for r0 in range(0, R, block):
                rr = rows[r0:r0 + block]
                _, P, lse = softmax_probs(q[b, hq, rr], k[b, kv], scale, rr, causal)
                O[b, hq, r0:r0 + block] = P @ v[b, kv]
                L[b, hq, r0:r0 + block] = lse
    return O, L


def attention_backward(q, k, v, do, scale: float, causal: bool, rows=None, keys=None,
                       block: int = 512, return_delta: bool = False):
    """Gradients of L = sum(O * dO) with respect to q, k, v, float64.

    Follows the definition with P recomputed from the LSE:
      D_i   = sum_d dO_id O_id                 (O from this oracle's own forward)
      dP_ij = dO_i . V_j
      dS_ij = P_ij (dP_ij - D_i)
      dQ_i  = scale * sum_j dS_ij K_j
      dK_j  = scale * sum_{hq in group} sum_i dS_ij Q_i
      dV_j  =         sum_{hq in group} sum_i P_ij dO_i
    ``rows`` restricts the returned dQ rows, ``keys`` the returned dK/dV rows
    (the forward statistics always use every row, so sampled outputs equal the
    corresponding rows of the full result).  Returns (dq, dk, dv) and, with
    ``return_delta``, also D of shape (B, Hq, N).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, N, D = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have the shape of q")
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(N, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    allrows = np.arange(N, dtype=np.int64)

    O, lse = attention_forward(q, k, v, scale, causal, block=block)
    delta = np.einsum("bhnd,bhnd->bhn", do, O)

    dq = np.zeros((B, Hq, rows.shape[0], D), dtype=np.float64)
    dk = np.zeros((B, Hkv, keys.shape[0], D), dtype=np.float64)
    dv = np.zeros((B, Hkv, keys.shape[0], D), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head(hq, Hq, Hkv)
            K, V, Q, dO = k[b, kv], v[b, kv], q[b, hq], do[b, hq]
            # dQ for the requested rows: one row block of (P, dP, dS) at a time.
            for r0 in range(0, rows.shape[0], block):
                rr = rows[r0:r0 + block]
                vis = visible_mask(rr, N, causal)
                S = scale * (Q[rr] @ K.T)
                P = np.where(vis, np.exp(np.where(vis, S, 0.0) - lse[b, hq, rr][:, None]), 0.0)
                dP = dO[rr] @ V.T
                dS = P * (dP - delta[b, hq, rr][:, None])
                dq[b, hq, r0:r0 + block] = scale * (dS @ K)
            # dK, dV for the requested keys: one key block of columns at a time.
            for c0 in range(0, keys.shape[0], block):
                kk = keys[c0:c0 + block]
                vis = visible_mask(allrows, kk, causal)
                S = scale * (Q @ K[kk].T)
                P = np.where(vis, np.exp(np.where(vis, S, 0.0) - lse[b, hq][:, None]), 0.0)
                dP = dO @ V[kk].T
                dS = P * (dP - delta[b, hq][:, None])
                dk[b, kv, c0:c0 + block] += scale * (dS.T @ Q)
                dv[b, kv, c0:c0 + block] += P.T @ dO
    if return_delta:
        return dq, dk, dv, delta
    return dq, dk, dv


def attention_dq_rows(q, k, v, do, scale: float, causal: bool, rows):
    """dQ of the listed query rows only, float64, at a cost linear in N per row.

    Row i's gradient needs nothing from other rows (same definition as attention_backward):
      O_i, LSE_i from row i's scores,  D_i = dO_i . O_i,
      dS_i = P_i (dO_i V^T - D_i),      dQ_i = scale * dS_i K.
    Returns (B, Hq, len(rows), D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, N, D = _check_shapes(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((B, Hq, rows.shape[0], D), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            kv = kv_head(hq, Hq, Hkv)
            _, P, _ = softmax_probs(q[b, hq, rows], k[b, kv], scale, rows, causal)
            O = P @ v[b, kv]
            delta = np.einsum("rd,rd->r", do[b, hq, rows], O)
            dS = P * (do[b, hq, rows] @ v[b, kv].T - delta[:, None])
            dq[b, hq] = scale * (dS @ k[b, kv])
    return dq

