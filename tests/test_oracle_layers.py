"""Pins of the oracle's building blocks against things other than the oracle itself:
library routines for special cases, closed forms, invariants and finite differences (fp64)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import decoder as D

rng = np.random.default_rng(7)


def fd_check(f, x, dx_analytic, n=12, h=1e-6, rtol=1e-6):
    """Central finite differences of scalar f at n random coordinates of x (fp64)."""
    flat = x.reshape(-1)
    idx = rng.choice(flat.size, size=min(n, flat.size), replace=False)
    for i in idx:
        old = flat[i]
        flat[i] = old + h
        fp = f()
        flat[i] = old - h
        fm = f()
        flat[i] = old
        fd = (fp - fm) / (2 * h)
        a = dx_analytic.reshape(-1)[i]
        assert abs(fd - a) <= rtol * max(1.0, abs(a)) + 1e-8, (i, fd, a)


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_matches_torch_library():
    x = rng.standard_normal((5, 48))
    g = rng.standard_normal(48)
    y, rstd = D.rmsnorm(x, g, 1e-5)
    ref = F.rms_norm(torch.tensor(x), (48,), torch.tensor(g), 1e-5).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd, 1 / np.sqrt(np.mean(x * x, 1) + 1e-5), rtol=1e-14)


def test_rmsnorm_constant_rows_give_signed_gain():
    # a constant row c gives c/sqrt(c^2+eps)*g, i.e. +-g up to eps
    x = np.array([[3.0] * 8, [-0.5] * 8])
    g = np.arange(1.0, 9.0)
    y, _ = D.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(y, np.stack([g, -g]), rtol=1e-15)


def test_rmsnorm_bwd_finite_differences():
    x = rng.standard_normal((3, 16))
    g = rng.standard_normal(16)
    w = rng.standard_normal((3, 16))
    f = lambda: float(np.sum(D.rmsnorm(x, g, 1e-5)[0] * w))
    y, rstd = D.rmsnorm(x, g, 1e-5)
    dx, dg = D.rmsnorm_bwd(w, x, g, rstd)
    fd_check(f, x, dx)
    fd_check(f, g, dg)


# ---------------------------------------------------------------- RoPE
def test_rope_hand_example():
    # d = 4: pairs (0,2) and (1,3); theta_0 = 1, theta_1 = base^(-1/2); base = 100 -> 0.1
    cos, sin = D.rope_tables(3, 4, 100.0, np.float64)
    x = np.zeros((3, 1, 4))
    x[:, 0, 0] = 1.0          # unit vector on the first pair's first component
    x[:, 0, 1] = 2.0
    y = D.rope(x, cos, sin)
    for p in range(3):
        np.testing.assert_allclose(y[p, 0], [math.cos(p), 2 * math.cos(0.1 * p),
                                             math.sin(p), 2 * math.sin(0.1 * p)], rtol=1e-15, atol=1e-15)


def test_rope_identity_at_position_zero_and_norm_preserving():
    cos, sin = D.rope_tables(9, 16, 10000.0, np.float64)
    x = rng.standard_normal((9, 3, 16))
    y = D.rope(x, cos, sin)
    np.testing.assert_allclose(y[0], x[0], rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)


def test_rope_relative_position_invariance():
    cos, sin = D.rope_tables(12, 8, 10000.0, np.float64)
    q = rng.standard_normal(8)
    k = rng.standard_normal(8)
    Q = D.rope(np.tile(q, (12, 1, 1)), cos, sin)[:, 0]
    K = D.rope(np.tile(k, (12, 1, 1)), cos, sin)[:, 0]
    # <q(p), k(p')> depends only on p - p'
    for delta in (0, 1, 5):
        vals = [Q[p + delta] @ K[p] for p in range(12 - delta)]
        np.testing.assert_allclose(vals, vals[0], rtol=1e-12)


def test_rope_bwd_is_adjoint():
    cos, sin = D.rope_tables(7, 16, 10000.0, np.float64)
    x = rng.standard_normal((7, 2, 16))
    y = rng.standard_normal((7, 2, 16))
    np.testing.assert_allclose(np.sum(D.rope(x, cos, sin) * y), np.sum(x * D.rope_bwd(y, cos, sin)),
                               rtol=1e-13)


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("nq,nkv", [(4, 4), (4, 2), (8, 1)])
def test_attention_matches_torch_sdpa(nq, nkv):
    S, d = 11, 8
    q = rng.standard_normal((S, nq, d))
    k = rng.standard_normal((S, nkv, d))
    v = rng.standard_normal((S, nkv, d))
    o, lse = D.attention(q, k, v)
    tq, tk, tv = (torch.tensor(a).transpose(0, 1)[None] for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)[0]
    np.testing.assert_allclose(o, ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-12)
    # lse from the library's logsumexp over the masked score matrix
    g = nq // nkv
    for h in range(nq):
        s = torch.tensor(q[:, h] @ k[:, h // g].T / math.sqrt(d))
        s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), -math.inf)
        np.testing.assert_allclose(lse[h], torch.logsumexp(s, 1).numpy(), rtol=1e-13)


def test_attention_special_cases():
    d = 4
    # S = 1: the only key is itself, o = v
    q = rng.standard_normal((1, 2, d)); k = rng.standard_normal((1, 1, d)); v = rng.standard_normal((1, 1, d))
    o, _ = D.attention(q, k, v)
    np.testing.assert_allclose(o[0, 0], v[0, 0]); np.testing.assert_allclose(o[0, 1], v[0, 0])
    # q = 0: uniform weights over the causal prefix -> running mean of v
    S = 6
    q = np.zeros((S, 2, d)); k = rng.standard_normal((S, 1, d)); v = rng.standard_normal((S, 1, d))
    o, lse = D.attention(q, k, v)
    prefix_mean = np.cumsum(v[:, 0], 0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(o[:, 0], prefix_mean, rtol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(np.arange(1, S + 1)), rtol=1e-14)


def test_gqa_equals_mha_with_duplicated_kv():
    S, nq, nkv, d = 9, 6, 2, 4
    q = rng.standard_normal((S, nq, d)); k = rng.standard_normal((S, nkv, d)); v = rng.standard_normal((S, nkv, d))
    o1, _ = D.attention(q, k, v)
    o2, _ = D.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1))
    np.testing.assert_allclose(o1, o2, rtol=1e-14)


def test_attention_bwd_finite_differences():
    S, nq, nkv, d = 7, 4, 2, 4
    q = rng.standard_normal((S, nq, d)); k = rng.standard_normal((S, nkv, d)); v = rng.standard_normal((S, nkv, d))
    w = rng.standard_normal((S, nq, d))
    f = lambda: float(np.sum(D.attention(q, k, v)[0] * w))
    o, lse = D.attention(q, k, v)
    dq, dk, dv = D.attention_bwd(w, q, k, v, o, lse)
    fd_check(f, q, dq); fd_check(f, k, dk); fd_check(f, v, dv)


# ---------------------------------------------------------------- SwiGLU
def test_swiglu_matches_torch_and_fd():
    g = rng.standard_normal((4, 9)); u = rng.standard_normal((4, 9)); w = rng.standard_normal((4, 9))
    np.testing.assert_allclose(D.swiglu(g, u), (F.silu(torch.tensor(g)) * torch.tensor(u)).numpy(), rtol=1e-14)
    f = lambda: float(np.sum(D.swiglu(g, u) * w))
    dg, du = D.swiglu_bwd(w, g, u)
    fd_check(f, g, dg); fd_check(f, u, du)


# ---------------------------------------------------------------- cross entropy
def test_cross_entropy_matches_torch_and_fd():
    z = rng.standard_normal((10, 13))
    y = rng.integers(0, 13, 10); y[3] = -1; y[7] = -1
    loss, dz = D.cross_entropy(z, y)
    ref = F.cross_entropy(torch.tensor(z), torch.tensor(y), ignore_index=-1)
    assert abs(loss - float(ref)) < 1e-13
    fd_check(lambda: D.cross_entropy(z, y)[0], z, dz)
    assert np.all(dz[3] == 0) and np.all(dz[7] == 0)


def test_cross_entropy_uniform_logits_is_log_vocab():
    z = np.full((5, 256), 0.37)
    y = np.arange(5)
    loss, _ = D.cross_entropy(z, y)
    assert abs(loss - math.log(256)) < 1e-14


def test_next_token_labels():
    t = np.array([[5, 6, 7], [1, 2, 3]])
    np.testing.assert_array_equal(D.next_token_labels(t), [[6, 7, -1], [2, 3, -1]])


# ---------------------------------------------------------------- MoE routing
def test_topk_ties_go_to_lower_index():
    n2 = np.zeros((1, 4))
    Wr = np.zeros((6, 4))          # all logits equal -> all probabilities equal
    probs, ids, w, _ = D.moe_route(n2, Wr, 3)
    np.testing.assert_array_equal(ids, [[0, 1, 2]])
    np.testing.assert_allclose(w, [[1 / 3] * 3], rtol=1e-15)


def test_moe_single_expert_is_dense_swiglu():
    s = D.Shape(1, 8, 2, 2, 4, n_experts=1, top_k=1, expert_ffn=5)
    P = {"l.router": rng.standard_normal((1, 8)), "l.experts.w_gate": rng.standard_normal((1, 5, 8)),
         "l.experts.w_up": rng.standard_normal((1, 5, 8)), "l.experts.w_down": rng.standard_normal((1, 8, 5))}
    x = rng.standard_normal((6, 8))
    out, _ = D.moe_forward(x, P, "l.", s)
    dense = (F.silu(torch.tensor(x @ P["l.experts.w_gate"][0].T)) * torch.tensor(x @ P["l.experts.w_up"][0].T)).numpy() @ P["l.experts.w_down"][0].T
    np.testing.assert_allclose(out, dense, rtol=1e-13)


def test_moe_all_experts_is_softmax_mixture():
    E = 4
    s = D.Shape(1, 8, 2, 2, 4, n_experts=E, top_k=E, expert_ffn=5)
    P = {"l.router": rng.standard_normal((E, 8)), "l.experts.w_gate": rng.standard_normal((E, 5, 8)),
         "l.experts.w_up": rng.standard_normal((E, 5, 8)), "l.experts.w_down": rng.standard_normal((E, 8, 5))}
    x = rng.standard_normal((6, 8))
    out, _ = D.moe_forward(x, P, "l.", s)
    p = F.softmax(torch.tensor(x @ P["l.router"].T), -1).numpy()
    ref = sum(p[:, e:e + 1] * ((F.silu(torch.tensor(x @ P["l.experts.w_gate"][e].T)).numpy()
                                 * (x @ P["l.experts.w_up"][e].T)) @ P["l.experts.w_down"][e].T) for e in range(E))
    np.testing.assert_allclose(out, ref, rtol=1e-12)


def test_moe_bwd_finite_differences():
    E, k = 6, 2
    s = D.Shape(1, 8, 2, 2, 4, n_experts=E, top_k=k, expert_ffn=5)
    P = {"l.router": rng.standard_normal((E, 8)), "l.experts.w_gate": rng.standard_normal((E, 5, 8)),
         "l.experts.w_up": rng.standard_normal((E, 5, 8)), "l.experts.w_down": rng.standard_normal((E, 8, 5))}
    x = rng.standard_normal((7, 8))
    w = rng.standard_normal((7, 8))
    out, cache = D.moe_forward(x, P, "l.", s)
    ids = cache["ids"].copy()
    # derivatives are taken with the routing held fixed (the top-k choice is piecewise constant)
    f = lambda: float(np.sum(D.moe_forward(x, P, "l.", s, forced_ids=ids)[0] * w))
    G = {n: np.zeros_like(v) for n, v in P.items()}
    dx = D.moe_backward(w, x, P, "l.", s, cache, G)
    fd_check(f, x, dx)
    for n in P:
        fd_check(f, P[n], G[n], n=6)


def test_topk_keeps_largest_probabilities():
    """The router keeps the k experts of largest probability (the top-k by value): a hand case and
    random distinct logits against torch.topk, for several token counts, expert counts and k."""
    # one token whose router logits are (0.1, 3, -1, 2, 0.5): the top-2 are experts 1 then 3
    logit_col = np.array([[0.1], [3.0], [-1.0], [2.0], [0.5]])
    probs, ids, w, logits = D.moe_route(np.array([[1.0]]), logit_col, 2)
    np.testing.assert_array_equal(ids, [[1, 3]])
    np.testing.assert_allclose(w[0], np.exp([3.0, 2.0]) / np.exp([3.0, 2.0]).sum(), rtol=1e-14)
    r = np.random.default_rng(11)
    for T, E, k in [(7, 6, 2), (33, 16, 4), (20, 128, 8), (5, 9, 1)]:
        n2 = r.standard_normal((T, 12))
        Wr = r.standard_normal((E, 12))
        probs, ids, w, _ = D.moe_route(n2, Wr, k)
        ref_v, ref_i = torch.topk(torch.tensor(probs), k, dim=1)
        np.testing.assert_array_equal(ids, ref_i.numpy())
        # every kept probability is at least every dropped one
        kept = np.take_along_axis(probs, ids, 1)
        dropped = probs.copy()
        np.put_along_axis(dropped, ids, -np.inf, 1)
        assert np.all(kept.min(1) > dropped.max(1))
