"""fp64 attention forward and backward: the plain definition, written out (test infrastructure only).

What the method computes
------------------------
DASH changes only *when* and *in which order* the partial dQ contributions are
added; the gradients themselves are the textbook softmax-attention gradients
(DASH paper, section 2.1: dK and dV are reduced over the query axis, dQ over the
key/value axis). The backward recomputes the probabilities from the saved
output O and the per-row log-sum-exp instead of storing them ("Writing an
Attention Kernel", section "In the real world": the forward keeps O and the
softmax statistics, and the backward costs about 2.5 forward passes).

Conventions (readings of the pages, stated once here)
-----------------------------------------------------
* Layout [B, H, N, d] for q, o, do, dq and [B, Hkv, N, d] for k, v, dk, dv.
* Query head h reads key/value head h // (H // Hkv) (grouped-query attention,
  "Writing an Attention Kernel", Step 2).
* Scores are scaled by `scale` (1/sqrt(d) in every workload; the eager listing of
  Step 1 applies head_dim ** -0.5 to Q K^T).
* Causal mask is top-left aligned with equal query and key lengths: key k is
  visible to query q iff k <= q (Step 1: minus infinity above the diagonal).
* lse is the natural-log log-sum-exp of the *scaled* scores of each query row.
* D = rowsum(dO * O) uses the O that is passed in.

Everything is evaluated in float64 with numpy BLAS on blocks of at most
`ROW_BLOCK` query rows against the full key range, so no online softmax is
needed and each step can be checked by eye against the formulas.

Parity status: pinned by finite differences, closed-form special cases,
column-sum invariants and an independent torch.autograd evaluation
(tests/test_oracle_attention.py).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 1024

__all__ = ["forward", "backward", "flops_bwd", "ROW_BLOCK"]


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, heads, N, d]")
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, N, d] with q's B, N, d")
    Hkv = k.shape[1]
    if Hkv == 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return B, H, Hkv, N, d


def _scores(qb, kg, scale, rows, causal):
    """Scaled scores s * Q K^T of a row block, masked to -inf above the diagonal."""
    s = scale * (qb @ kg.T)
    if causal:
        cols = np.arange(kg.shape[0])
        s[cols[None, :] > rows[:, None]] = -np.inf
    return s


def forward(q, k, v, causal: bool, scale: float):
    """O = softmax(s Q K^T) V and the natural-log LSE of each row, in float64.

    Inputs are converted to float64. Returns (o [B,H,N,d], lse [B,H,N]).
    Follows the eager definition of "Writing an Attention Kernel", Step 1
    (matmul, scale, mask, softmax, matmul); the LSE is the statistic the
    backward recomputes P from (section "In the real world").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Hkv, N, d = _check(q, k, v)
    G = H // Hkv
    o = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            g = h // G
            for r0 in range(0, N, ROW_BLOCK):
                r1 = min(N, r0 + ROW_BLOCK)
                rows = np.arange(r0, r1)
                s = _scores(q[b, h, r0:r1], k[b, g], scale, rows, causal)
                m = s.max(axis=1)
                l_row = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
                p = np.exp(s - l_row[:, None])
                o[b, h, r0:r1] = p @ v[b, g]
                lse[b, h, r0:r1] = l_row
    return o, lse


def backward(q, k, v, o, do, lse, causal: bool, scale: float):
    """dQ, dK, dV of L = sum(dO * O) for O = softmax(s Q K^T) V, recomputed from (O, LSE).

    Steps, per batch b, query head h (key/value head g = h // G) and query row block:
      P  = exp(s Q K^T - LSE)            (masked entries are 0)
      dV_g += P^T dO
      dP = dO V^T
      D  = rowsum(dO * O)
      dS = P * (dP - D)
      dQ = s dS K
      dK_g += s dS^T Q
    dK and dV of a key/value head sum the contributions of all G query heads that
    read it. Returns float64 arrays (dq [B,H,N,d], dk, dv [B,Hkv,N,d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, H, Hkv, N, d = _check(q, k, v)
    if o.shape != q.shape or do.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("o, do must match q; lse must be [B, H, N]")
    G = H // Hkv
    dq = np.zeros((B, H, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    for b in range(B):
        for h in range(H):
            g = h // G
            for r0 in range(0, N, ROW_BLOCK):
                r1 = min(N, r0 + ROW_BLOCK)
                rows = np.arange(r0, r1)
                qb, dob, ob = q[b, h, r0:r1], do[b, h, r0:r1], o[b, h, r0:r1]
                s = _scores(qb, k[b, g], scale, rows, causal)
                p = np.exp(s - lse[b, h, r0:r1, None])  # exp(-inf) = 0 on masked entries
                dv[b, g] += p.T @ dob
                dp = dob @ v[b, g].T
                D = (dob * ob).sum(axis=1)
                ds = p * (dp - D[:, None])
                dq[b, h, r0:r1] = scale * (ds @ k[b, g])
                dk[b, g] += scale * (ds.T @ qb)
    return dq, dk, dv


def flops_bwd(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Conventional backward FLOP count: 2.5 x the forward's 4 N^2 d per (batch, query head), halved if causal.

    Convention of "Writing an Attention Kernel" (FLOP counting paragraph of Step 1
    and the backward factor in "In the real world").
    """
    f = 2.5 * 4.0 * N * N * d * B * H
    return f / 2.0 if causal else f
