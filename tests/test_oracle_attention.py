"""Pins of the fp64 attention oracle against facts that do not depend on it.

* finite differences of L = sum(dO * O(Q, K, V)) (the gradient definition),
* closed-form special cases (N = 1, causal row 0, constant V),
* column-sum invariants of dK and dV,
* torch.autograd and torch's fp64 scaled_dot_product_attention on the CPU
  (independent library implementations),
* mutation check: a planted mistake in a copy of the oracle (dropped term, sign,
  transposed operand, wrong head map, wrong mask edge, missing scale) fails at
  least one of the pins above.
"""
import inspect
import types

import numpy as np
import pytest
import torch

from oracle import attention as oa

CASES = [
    (hkv, n, d, causal)
    for hkv in (1, 2)
    for n in (1, 5, 16)
    for d in (4, 8)
    for causal in (False, True)
]


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    q = _rand((B, H, N, d), rng)
    k = _rand((B, Hkv, N, d), rng)
    v = _rand((B, Hkv, N, d), rng)
    do = _rand((B, H, N, d), rng)
    return q, k, v, do


def _fd_error(mod, q, k, v, do, causal, scale, eps=1e-6):
    """max |finite-difference grad - analytic grad| over q, k, v, relative to the largest analytic gradient."""
    o, lse = mod.forward(q, k, v, causal, scale)
    dq, dk, dv = mod.backward(q, k, v, o, do, lse, causal, scale)

    def loss(qq, kk, vv):
        oo, _ = mod.forward(qq, kk, vv, causal, scale)
        return float((do * oo).sum())

    worst = 0.0
    scale_ref = max(np.abs(dq).max(), np.abs(dk).max(), np.abs(dv).max(), 1e-300)
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = {"q": q, "k": k, "v": v}
            plus = {kk: vv.copy() for kk, vv in args.items()}
            minus = {kk: vv.copy() for kk, vv in args.items()}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (loss(plus["q"], plus["k"], plus["v"]) -
                       loss(minus["q"], minus["k"], minus["v"])) / (2 * eps)
        worst = max(worst, np.abs(fd - grad).max() / scale_ref)
    return worst


@pytest.mark.parametrize("hkv,n,d,causal", CASES)
def test_finite_differences(hkv, n, d, causal):
    q, k, v, do = _inputs(1, 2, hkv, n, d, seed=7 + n + d)
    err = _fd_error(oa, q, k, v, do, causal, 1.0 / np.sqrt(d))
    assert err <= 1e-6, err


def _special_case_failures(mod):
    """Closed-form cases; returns a list of failure messages (empty when all hold)."""
    fails = []
    rng = np.random.default_rng(3)
    scale = 0.5
    # N = 1: the only probability is 1, so dV = dO and dQ = dK = 0.
    q, k, v, do = (rng.standard_normal(s) for s in ((1, 2, 1, 4), (1, 1, 1, 4), (1, 1, 1, 4), (1, 2, 1, 4)))
    o, lse = mod.forward(q, k, v, False, scale)
    dq, dk, dv = mod.backward(q, k, v, o, do, lse, False, scale)
    if not (np.allclose(dv[0, 0], do[0].sum(axis=0)) and np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12):
        fails.append("N=1")
    # Causal row 0 sees only key 0: its dQ row is 0.
    q, k, v, do = _inputs(1, 2, 2, 6, 4, seed=11)
    o, lse = mod.forward(q, k, v, True, scale)
    dq, dk, dv = mod.backward(q, k, v, o, do, lse, True, scale)
    if np.abs(dq[:, :, 0]).max() > 1e-12:
        fails.append("causal row 0")
    # Constant V rows: O = v for every row, so dS = 0 and dQ = dK = 0.
    v_const = np.repeat(rng.standard_normal((1, 2, 1, 4)), 6, axis=2)
    for causal in (False, True):
        o, lse = mod.forward(q, k, v_const, causal, scale)
        dq, dk, dv = mod.backward(q, k, v_const, o, do, lse, causal, scale)
        if np.abs(dq).max() > 1e-12 or np.abs(dk).max() > 1e-12:
            fails.append(f"constant V causal={causal}")
    # Column sums with exact O: sum_k dK[k] = 0 and sum_k dV[k] = sum over the group of sum_q dO[q].
    q, k, v, do = _inputs(2, 4, 2, 9, 4, seed=5)
    for causal in (False, True):
        o, lse = mod.forward(q, k, v, causal, scale)
        dq, dk, dv = mod.backward(q, k, v, o, do, lse, causal, scale)
        if np.abs(dk.sum(axis=2)).max() > 1e-10:
            fails.append(f"dK column sum causal={causal}")
        want = do.reshape(2, 2, 2, 9, 4).sum(axis=(2, 3))
        if np.abs(dv.sum(axis=2) - want).max() > 1e-10:
            fails.append(f"dV column sum causal={causal}")
    return fails


def test_special_cases_and_invariants():
    assert _special_case_failures(oa) == []


def _torch_grads(q, k, v, do, causal, scale):
    """Gradients from torch.autograd on an eager fp64 attention (CPU)."""
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = q.shape[1] // k.shape[1]
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(2, 3).contiguous())
    if causal:
        n = q.shape[2]
        mask = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        s = s.masked_fill(mask, float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_autograd_with_row_blocks(causal, monkeypatch):
    q, k, v, do = _inputs(2, 4, 2, 37, 8, seed=21)
    scale = 1.0 / np.sqrt(8)
    monkeypatch.setattr(oa, "ROW_BLOCK", 16)  # several row blocks and a ragged tail
    o, lse = oa.forward(q, k, v, causal, scale)
    dq, dk, dv = oa.backward(q, k, v, o, do, lse, causal, scale)
    to, tdq, tdk, tdv = _torch_grads(q, k, v, do, causal, scale)
    for a, b in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


@pytest.mark.parametrize("causal", [False, True])
def test_forward_against_torch_sdpa(causal):
    q, k, v, _ = _inputs(1, 6, 2, 33, 16, seed=2)
    o, lse = oa.forward(q, k, v, causal, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), is_causal=causal, scale=0.25, enable_gqa=True)
    assert np.abs(o - ref.numpy()).max() < 1e-12
    # Rows of P sum to 1: attention of V = 1 returns 1 everywhere.
    ones, _ = oa.forward(q, k, np.ones_like(v), causal, 0.25)
    assert np.abs(ones - 1.0).max() < 1e-12
    # LSE is log sum exp of the scaled, masked scores.
    s = 0.25 * np.einsum("hqd,hkd->hqk", q[0], np.repeat(k[0], 3, axis=0))
    if causal:
        s = np.where(np.triu(np.ones((33, 33), bool), 1), -np.inf, s)
    assert np.abs(lse[0] - np.log(np.exp(s).sum(-1))).max() < 1e-12


def test_flop_convention():
    # 2.5 x 4 N^2 d per (batch, head), halved for causal.
    assert oa.flops_bwd(8, 16, 2048, 128, False) == pytest.approx(687.19476736e9)
    assert oa.flops_bwd(1, 16, 16384, 128, True) == pytest.approx(2748.77906944e9)


MUTATIONS = [
    ("dropped D term", "ds = p * (dp - D[:, None])", "ds = p * dp"),
    ("sign of D", "ds = p * (dp - D[:, None])", "ds = p * (dp + D[:, None])"),
    ("transposed P in dV", "dv[b, g] += p.T @ dob", "dv[b, g] += p @ dob"),
    ("transposed dS in dK", "dk[b, g] += scale * (ds.T @ qb)", "dk[b, g] += scale * (ds @ qb)"),
    ("missing scale on dQ", "dq[b, h, r0:r1] = scale * (ds @ k[b, g])", "dq[b, h, r0:r1] = ds @ k[b, g]"),
    ("wrong GQA head map", "g = h // G\n            for r0 in range(0, N, ROW_BLOCK):\n                r1 = min(N, r0 + ROW_BLOCK)\n                rows = np.arange(r0, r1)\n                qb, dob",
     "g = h % Hkv\n            for r0 in range(0, N, ROW_BLOCK):\n                r1 = min(N, r0 + ROW_BLOCK)\n                rows = np.arange(r0, r1)\n                qb, dob"),
    ("mask edge off by one", "s[cols[None, :] > rows[:, None]] = -np.inf", "s[cols[None, :] >= rows[:, None] + 1 + (rows[:, None] > 0)] = -np.inf"),
    ("dP from K instead of V", "dp = dob @ v[b, g].T", "dp = dob @ k[b, g].T"),
]


def _mutant(src, old, new):
    assert src.count(old) >= 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _torch_mismatch(mod):
    """True when mod's forward/backward disagree with torch.autograd on a GQA case."""
    q, k, v, do = _inputs(1, 4, 2, 7, 4, seed=31)
    for causal in (False, True):
        o, lse = mod.forward(q, k, v, causal, 0.5)
        got = (o,) + tuple(mod.backward(q, k, v, o, do, lse, causal, 0.5))
        want = _torch_grads(q, k, v, do, causal, 0.5)
        if any(np.abs(a - b).max() > 1e-10 for a, b in zip(got, want)):
            return True
    return False


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    src = inspect.getsource(oa)
    mod = _mutant(src, old, new)
    caught = {"special cases": bool(_special_case_failures(mod)), "finite differences": False,
              "torch autograd": _torch_mismatch(mod)}
    for hkv, n, d, causal in ((1, 5, 4, True), (2, 5, 4, False), (1, 5, 4, False)):
        q, k, v, do = _inputs(1, 2, hkv, n, d, seed=99)
        if not _fd_error(mod, q, k, v, do, causal, 0.5) <= 1e-6:
            caught["finite differences"] = True
    assert any(caught.values()), f"mutation '{name}' passed every pin"
