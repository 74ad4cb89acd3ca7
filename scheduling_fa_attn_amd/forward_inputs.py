"""Forward statistics (O, LSE) that the backward consumes, computed with plain torch fp32 ops on the GPU.

The backward's inputs include the forward output O and the per-row natural-log
log-sum-exp of the scaled scores ("Writing an Attention Kernel", section "In the
real world": the forward keeps O and the softmax statistics for the backward).
The benchmark needs them at full size on the GPU; this module produces them from
the seeded Q, K, V with torch matmul/logsumexp in float32, row block by row block.
It is input preparation only: the backward library never calls it.
"""
from __future__ import annotations

import math

import torch

ROWS = 2048


def forward_stats(q, k, v, causal: bool, scale: float | None = None):
    """q [B,H,N,d], k/v [B,Hkv,N,d] bf16 CUDA tensors -> (o bf16 [B,H,N,d], lse fp32 [B,H,N])."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    cols = torch.arange(N, device=q.device)
    for b in range(B):
        for g in range(Hkv):
            kf = k[b, g].float()
            ktf = kf.t().contiguous()
            vf = v[b, g].float()
            for h in range(g * G, (g + 1) * G):
                for r0 in range(0, N, ROWS):
                    r1 = min(N, r0 + ROWS)
                    s = torch.matmul(q[b, h, r0:r1].float(), ktf) * scale
                    if causal:
                        rows = torch.arange(r0, r1, device=q.device)
                        s.masked_fill_(cols[None, :] > rows[:, None], float("-inf"))
                    l_row = torch.logsumexp(s, dim=1)
                    p = torch.exp(s - l_row[:, None])
                    o[b, h, r0:r1] = torch.matmul(p, vf).to(torch.bfloat16)
                    lse[b, h, r0:r1] = l_row
    return o, lse
