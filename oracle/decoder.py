"""Oracle (test infrastructure only): a plain, slow NumPy decoder with a hand-written backward.

Nothing in the product path may import this module; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP library.

What it computes is ordinary full-batch training of a pre-norm decoder. Streaming, double
buffering, checkpoint-every-K with block recompute and micro-batching are all reorganisations
of that computation (MegaTrain summary page, 核心方法 and 方法步骤详情; RoundPipe user guide,
输入分割与 microbatch 执行), so the plain definition is the oracle:

* the batch is split into ``n_micro`` contiguous groups of sequences, each group runs
  forward, loss and backward, the returned loss is the SUM of the group losses and the
  gradients are the sum of the group gradients (RoundPipe user guide, 输入分割与 microbatch 执行);
* per layer: RMSNorm, q/k/v projections, RoPE, causal grouped-query attention, output
  projection with residual, RMSNorm, SwiGLU MLP (or a top-k routed MoE of SwiGLU experts) with
  residual. The pages name these blocks only ("Attention and MLP blocks", MegaTrain summary page,
  核心方法); the exact formulas below are the standard ones, and each reading of a formula the
  pages leave open is stated in the comment where it is used.

Precision: every array is kept in the dtype of the parameters passed in (float32 for parity,
float64 for finite-difference pins); loss sums are accumulated in Python floats (fp64).

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

Array = np.ndarray


# ------------------------------------------------------------------------------------------
# RMSNorm  (reading: y = x / sqrt(mean(x^2) + eps) * g, eps = 1e-5, gain initialised to 1)
# ------------------------------------------------------------------------------------------
def rmsnorm(x: Array, g: Array, eps: float) -> Tuple[Array, Array]:
    """Row-wise RMSNorm over the last axis. Returns (y, rstd) with rstd = 1/sqrt(mean(x^2)+eps)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    rstd = (1.0 / np.sqrt(ms + x.dtype.type(eps))).astype(x.dtype)
    return x * rstd * g, rstd[..., 0]


def rmsnorm_bwd(dy: Array, x: Array, g: Array, rstd: Array) -> Tuple[Array, Array]:
    """Chain rule of ``rmsnorm``: returns (dx, dg)."""
    r = rstd[..., None]
    xhat = x * r
    dg = np.sum((dy * xhat).reshape(-1, x.shape[-1]), axis=0)
    dxhat = dy * g
    H = x.shape[-1]
    dx = r * (dxhat - xhat * (np.sum(dxhat * xhat, axis=-1, keepdims=True) / x.dtype.type(H)))
    return dx, dg


# ------------------------------------------------------------------------------------------
# RoPE  (reading: rotate-half pairing (j, j + d/2), theta_j = base^(-2j/d), position restarts at 0
# in every sequence; angles in fp64 on the host, cos/sin rounded to the working dtype)
# ------------------------------------------------------------------------------------------
def rope_tables(seq: int, head_dim: int, base: float, dtype) -> Tuple[Array, Array]:
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    theta = base ** (-2.0 * j / head_dim)
    ang = np.arange(seq, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: Array, cos: Array, sin: Array) -> Array:
    """x: [S, heads, d]; rotates the pair (x[j], x[j+d/2]) by angle p*theta_j at position p."""
    half = x.shape[-1] // 2
    c, s = cos[:, None, :], sin[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_bwd(dy: Array, cos: Array, sin: Array) -> Array:
    """Adjoint of ``rope``: rotation by the negative angle."""
    half = dy.shape[-1] // 2
    c, s = cos[:, None, :], sin[:, None, :]
    da, db = dy[..., :half], dy[..., half:]
    return np.concatenate([da * c + db * s, db * c - da * s], axis=-1)


# ------------------------------------------------------------------------------------------
# causal grouped-query attention  (reading: q head h reads kv head h // (nq/nkv), scale 1/sqrt(d))
# ------------------------------------------------------------------------------------------
def attention(q: Array, k: Array, v: Array) -> Tuple[Array, Array]:
    """q: [S, nq, d]; k, v: [S, nkv, d]. Returns (o [S, nq, d], lse [nq, S]) for one sequence."""
    S, nq, d = q.shape
    group = nq // k.shape[1]
    scale = q.dtype.type(1.0 / np.sqrt(d))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    o = np.empty_like(q)
    lse = np.empty((nq, S), q.dtype)
    for h in range(nq):
        kv = h // group
        s = (q[:, h, :] @ k[:, kv, :].T) * scale
        s[mask] = -np.inf
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        l = np.sum(p, axis=1, keepdims=True)
        o[:, h, :] = (p / l) @ v[:, kv, :]
        lse[h] = (m + np.log(l))[:, 0]
    return o, lse


def attention_bwd(do: Array, q: Array, k: Array, v: Array, o: Array, lse: Array
                  ) -> Tuple[Array, Array, Array]:
    """Gradient of ``attention`` w.r.t. q, k, v (softmax Jacobian via rowsum(dO * O))."""
    S, nq, d = q.shape
    group = nq // k.shape[1]
    scale = q.dtype.type(1.0 / np.sqrt(d))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nq):
        kv = h // group
        s = (q[:, h, :] @ k[:, kv, :].T) * scale
        s[mask] = -np.inf
        p = np.exp(s - lse[h][:, None])
        dv[:, kv, :] += p.T @ do[:, h, :]
        dp = do[:, h, :] @ v[:, kv, :].T
        delta = np.sum(do[:, h, :] * o[:, h, :], axis=1, keepdims=True)
        ds = p * (dp - delta) * scale
        dq[:, h, :] = ds @ k[:, kv, :]
        dk[:, kv, :] += ds.T @ q[:, h, :]
    return dq, dk, dv


# ------------------------------------------------------------------------------------------
# SwiGLU  a = silu(g) * u,  silu(x) = x * sigmoid(x)
# ------------------------------------------------------------------------------------------
def sigmoid(x: Array) -> Array:
    return 1.0 / (1.0 + np.exp(-x))


def swiglu(g: Array, u: Array) -> Array:
    return g * sigmoid(g) * u


def swiglu_bwd(da: Array, g: Array, u: Array) -> Tuple[Array, Array]:
    sg = sigmoid(g)
    silu = g * sg
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    du = da * silu
    return dg, du


# ------------------------------------------------------------------------------------------
# model description
# ------------------------------------------------------------------------------------------
@dataclass
class Shape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int = 0
    vocab: int = 0
    n_experts: int = 0
    top_k: int = 0
    expert_ffn: int = 0
    lora_rank: int = 0
    lora_scale: float = 1.0
    rope_base: float = 10000.0
    rms_eps: float = 1e-5

    @classmethod
    def of(cls, s) -> "Shape":
        return cls(**{k: getattr(s, k) for k in cls.__dataclass_fields__})


def trainable_names(shape: Shape, names) -> List[str]:
    """Full fine-tune trains every tensor; with LoRA only the adapter factors train (base frozen)."""
    if shape.lora_rank:
        return [n for n in names if ".lora." in n]
    return list(names)


# ------------------------------------------------------------------------------------------
# linear maps (nn.Linear orientation: y = x W^T, W is [out, in]); optional LoRA branch
# ------------------------------------------------------------------------------------------
def _proj(x: Array, P: Dict[str, Array], w: str, lora: Optional[str], s: Shape) -> Array:
    y = x @ P[w].T
    if lora is not None:
        # reading: y += scale * (x A^T) B^T with A [r, in], B [out, r], scale = 1
        y = y + s.lora_scale * ((x @ P[lora + ".A"].T) @ P[lora + ".B"].T)
    return y


def _proj_bwd(dy: Array, x: Array, P: Dict[str, Array], w: str, lora: Optional[str], s: Shape,
              G: Dict[str, Array]) -> Array:
    """Returns dx; adds dW (and dA, dB) into G for names present in G."""
    dx = dy @ P[w]
    if w in G:
        G[w] += dy.T @ x
    if lora is not None:
        A, B = P[lora + ".A"], P[lora + ".B"]
        sc = x.dtype.type(s.lora_scale)
        xa = x @ A.T                   # [T, r]
        dyb = dy @ B                   # [T, r]
        dx = dx + sc * (dyb @ A)
        if lora + ".B" in G:
            G[lora + ".B"] += sc * (dy.T @ xa)
        if lora + ".A" in G:
            G[lora + ".A"] += sc * (dyb.T @ x)
    return dx


# ------------------------------------------------------------------------------------------
# MoE MLP (reading: softmax router over E experts, top-k by probability with ties toward the
# lower expert index, weights renormalised over the kept k, no capacity limit / aux loss)
# ------------------------------------------------------------------------------------------
def moe_route(n2: Array, Wr: Array, top_k: int, forced_ids: Optional[Array] = None):
    """Returns (probs [T,E], ids [T,k], weights [T,k], logits [T,E])."""
    logits = n2 @ Wr.T
    m = np.max(logits, axis=1, keepdims=True)
    e = np.exp(logits - m)
    probs = e / np.sum(e, axis=1, keepdims=True)
    if forced_ids is None:
        # stable sort of -p: among equal probabilities the lower index comes first
        ids = np.argsort(-probs, axis=1, kind="stable")[:, :top_k]
    else:
        ids = forced_ids
    kept = np.take_along_axis(probs, ids, axis=1)
    w = kept / np.sum(kept, axis=1, keepdims=True)
    return probs, ids, w, logits


def moe_forward(n2: Array, P: Dict[str, Array], pre: str, s: Shape, forced_ids=None):
    probs, ids, w, logits = moe_route(n2, P[pre + "router"], s.top_k, forced_ids)
    Wg, Wu, Wd = P[pre + "experts.w_gate"], P[pre + "experts.w_up"], P[pre + "experts.w_down"]
    out = np.zeros_like(n2)
    cache = {"probs": probs, "ids": ids, "w": w, "logits": logits, "experts": {}}
    for e in range(s.n_experts):
        rows, slots = np.nonzero(ids == e)
        if rows.size == 0:
            continue
        x = n2[rows]
        g = x @ Wg[e].T
        u = x @ Wu[e].T
        a = swiglu(g, u)
        y = a @ Wd[e].T
        out[rows] += w[rows, slots][:, None] * y
        cache["experts"][e] = (rows, slots, g, u, a, y)
    return out, cache


def moe_backward(dout: Array, n2: Array, P: Dict[str, Array], pre: str, s: Shape, cache,
                 G: Dict[str, Array]) -> Array:
    Wg, Wu, Wd = P[pre + "experts.w_gate"], P[pre + "experts.w_up"], P[pre + "experts.w_down"]
    ids, w, probs = cache["ids"], cache["w"], cache["probs"]
    dn2 = np.zeros_like(n2)
    dw = np.zeros_like(w)
    for e, (rows, slots, g, u, a, y) in cache["experts"].items():
        x = n2[rows]
        dw[rows, slots] = np.sum(dout[rows] * y, axis=1)
        dy = w[rows, slots][:, None] * dout[rows]
        da = dy @ Wd[e]
        dg, du = swiglu_bwd(da, g, u)
        dn2[rows] += dg @ Wg[e] + du @ Wu[e]
        if pre + "experts.w_down" in G:
            G[pre + "experts.w_down"][e] += dy.T @ a
            G[pre + "experts.w_gate"][e] += dg.T @ x
            G[pre + "experts.w_up"][e] += du.T @ x
    # renormalisation w_i = p_i / sum_kept p  ->  dp_i = (dw_i - sum_j dw_j w_j) / sum_kept p
    kept = np.take_along_axis(probs, ids, axis=1)
    ssum = np.sum(kept, axis=1, keepdims=True)
    dkept = (dw - np.sum(dw * w, axis=1, keepdims=True)) / ssum
    dprobs = np.zeros_like(probs)
    np.put_along_axis(dprobs, ids, dkept, axis=1)
    # softmax Jacobian
    dlogits = probs * (dprobs - np.sum(dprobs * probs, axis=1, keepdims=True))
    dn2 += dlogits @ P[pre + "router"]
    if pre + "router" in G:
        G[pre + "router"] += dlogits.T @ n2
    return dn2


# ------------------------------------------------------------------------------------------
# one decoder layer over the tokens of one micro-batch (several sequences of equal length)
# ------------------------------------------------------------------------------------------
def layer_forward(P: Dict[str, Array], i: int, h: Array, s: Shape, n_seq: int,
                  cos: Array, sin: Array, forced_ids=None):
    """h: [T, H] with T = n_seq * S. Returns (h_out, cache)."""
    pre = f"layers.{i}."
    T, H = h.shape
    S = T // n_seq
    d, nq, nkv = s.head_dim, s.n_q_heads, s.n_kv_heads
    lo = (lambda t: pre + "lora." + t) if s.lora_rank else (lambda t: None)
    n1, r1 = rmsnorm(h, P[pre + "attn_norm"], s.rms_eps)
    q = _proj(n1, P, pre + "wq", lo("q"), s).reshape(n_seq, S, nq, d)
    k = _proj(n1, P, pre + "wk", lo("k"), s).reshape(n_seq, S, nkv, d)
    v = _proj(n1, P, pre + "wv", lo("v"), s).reshape(n_seq, S, nkv, d)
    qr = np.stack([rope(q[b], cos, sin) for b in range(n_seq)])
    kr = np.stack([rope(k[b], cos, sin) for b in range(n_seq)])
    o = np.empty_like(qr)
    lse = np.empty((n_seq, nq, S), h.dtype)
    for b in range(n_seq):
        o[b], lse[b] = attention(qr[b], kr[b], v[b])
    o2 = o.reshape(T, nq * d)
    h1 = h + _proj(o2, P, pre + "wo", lo("o"), s)
    n2, r2 = rmsnorm(h1, P[pre + "mlp_norm"], s.rms_eps)
    cache = dict(h=h, n1=n1, r1=r1, qr=qr, kr=kr, v=v, o=o, lse=lse, h1=h1, n2=n2, r2=r2)
    if s.n_experts:
        m, mc = moe_forward(n2, P, pre, s, None if forced_ids is None else forced_ids[i])
        cache["moe"] = mc
        h2 = h1 + m
    else:
        g = n2 @ P[pre + "w_gate"].T
        u = n2 @ P[pre + "w_up"].T
        a = swiglu(g, u)
        cache.update(g=g, u=u, a=a)
        h2 = h1 + a @ P[pre + "w_down"].T
    return h2, cache


def layer_backward(P: Dict[str, Array], i: int, c, dh2: Array, s: Shape, n_seq: int,
                   cos: Array, sin: Array, G: Dict[str, Array]) -> Array:
    """Backward of ``layer_forward``; adds parameter gradients into G; returns dh (layer input)."""
    pre = f"layers.{i}."
    T, H = dh2.shape
    S = T // n_seq
    d, nq, nkv = s.head_dim, s.n_q_heads, s.n_kv_heads
    lo = (lambda t: pre + "lora." + t) if s.lora_rank else (lambda t: None)
    # MLP
    if s.n_experts:
        dn2 = moe_backward(dh2, c["n2"], P, pre, s, c["moe"], G)
    else:
        da = dh2 @ P[pre + "w_down"]
        if pre + "w_down" in G:
            G[pre + "w_down"] += dh2.T @ c["a"]
        dg, du = swiglu_bwd(da, c["g"], c["u"])
        dn2 = dg @ P[pre + "w_gate"] + du @ P[pre + "w_up"]
        if pre + "w_gate" in G:
            G[pre + "w_gate"] += dg.T @ c["n2"]
            G[pre + "w_up"] += du.T @ c["n2"]
    dh1x, dg2 = rmsnorm_bwd(dn2, c["h1"], P[pre + "mlp_norm"], c["r2"])
    if pre + "mlp_norm" in G:
        G[pre + "mlp_norm"] += dg2
    dh1 = dh2 + dh1x
    # attention
    o2 = c["o"].reshape(T, nq * d)
    do2 = _proj_bwd(dh1, o2, P, pre + "wo", lo("o"), s, G)
    do = do2.reshape(n_seq, S, nq, d)
    dq = np.empty_like(c["qr"])
    dk = np.empty_like(c["kr"])
    dv = np.empty_like(c["v"])
    for b in range(n_seq):
        dqr, dkr, dv[b] = attention_bwd(do[b], c["qr"][b], c["kr"][b], c["v"][b], c["o"][b],
                                        c["lse"][b])
        dq[b] = rope_bwd(dqr, cos, sin)
        dk[b] = rope_bwd(dkr, cos, sin)
    n1 = c["n1"]
    dn1 = (_proj_bwd(dq.reshape(T, nq * d), n1, P, pre + "wq", lo("q"), s, G)
           + _proj_bwd(dk.reshape(T, nkv * d), n1, P, pre + "wk", lo("k"), s, G)
           + _proj_bwd(dv.reshape(T, nkv * d), n1, P, pre + "wv", lo("v"), s, G))
    dhx, dg1 = rmsnorm_bwd(dn1, c["h"], P[pre + "attn_norm"], c["r1"])
    if pre + "attn_norm" in G:
        G[pre + "attn_norm"] += dg1
    return dh1 + dhx


# ------------------------------------------------------------------------------------------
# losses
# ------------------------------------------------------------------------------------------
def cross_entropy(logits: Array, labels: Array) -> Tuple[float, Array]:
    """Mean over positions with label >= 0 of (logsumexp(z) - z[y]); returns (loss, dlogits).

    Reading: the mean is the usual criterion default; the user guide leaves ``loss_fn`` to the
    user and sums it across micro-batches (RoundPipe user guide, 输入分割与 microbatch 执行).
    """
    valid = labels >= 0
    count = int(np.sum(valid))
    m = np.max(logits, axis=1, keepdims=True)
    e = np.exp(logits - m)
    ssum = np.sum(e, axis=1, keepdims=True)
    lse = (m + np.log(ssum))[:, 0]
    idx = np.where(valid, labels, 0)
    zy = logits[np.arange(logits.shape[0]), idx]
    per = np.where(valid, lse - zy, 0.0)
    if count == 0:
        return 0.0, np.zeros_like(logits)
    loss = float(np.sum(per.astype(np.float64)) / count)
    d = e / ssum
    d[np.arange(logits.shape[0]), idx] -= 1.0
    d *= (valid.astype(logits.dtype) / logits.dtype.type(count))[:, None]
    return loss, d


def next_token_labels(tokens: Array) -> Array:
    """labels[b, t] = tokens[b, t+1]; the last position of every sequence is ignored (-1)."""
    lab = np.full(tokens.shape, -1, np.int64)
    lab[:, :-1] = tokens[:, 1:]
    return lab


# ------------------------------------------------------------------------------------------
# full forward_backward over micro-batches
# ------------------------------------------------------------------------------------------
def split_microbatches(n_seq: int, n_micro: int) -> List[Tuple[int, int]]:
    """Contiguous equal groups of sequences (RoundPipe user guide, 输入分割与 microbatch 执行:
    batch 12 into 3 micro-batches gives samples 0-3, 4-7, 8-11). Unequal split is an error."""
    if n_micro <= 0 or n_seq % n_micro != 0:
        raise ValueError("batch must be a positive multiple of n_micro")
    b = n_seq // n_micro
    return [(m * b, (m + 1) * b) for m in range(n_micro)]


def microbatch_forward_backward(P: Dict[str, Array], s: Shape, G: Dict[str, Array],
                                tokens: Optional[Array] = None, labels: Optional[Array] = None,
                                hidden: Optional[Array] = None, loss: str = "ce",
                                forced_ids=None, record_ids: Optional[list] = None) -> float:
    """One micro-batch: forward, loss, backward; adds gradients into G; returns its loss.

    Layer inputs are kept and each layer is recomputed from its input during the backward
    (the full per-layer recompute of the RoundPipe user guide, 激活重计算); this only bounds the
    oracle's memory and does not change the arithmetic.
    """
    dt = next(iter(P.values())).dtype if P else hidden.dtype
    if hidden is not None:
        n_seq, S = hidden.shape[0], hidden.shape[1]
        h = hidden.reshape(n_seq * S, s.hidden).astype(dt)
    else:
        n_seq, S = tokens.shape
        h = P["embed"][tokens.reshape(-1)].astype(dt)
    cos, sin = rope_tables(S, s.head_dim, s.rope_base, dt)
    inputs = []
    for i in range(s.n_layers):
        inputs.append(h)
        h, c = layer_forward(P, i, h, s, n_seq, cos, sin, forced_ids)
        if record_ids is not None and s.n_experts:
            record_ids.append(c["moe"]["ids"])
        del c
    # loss anchor (MegaTrain summary page, 方法步骤详情 phase 2)
    if loss == "ce":
        z, rz = rmsnorm(h, P["final_norm"], s.rms_eps)
        logits = z @ P["lm_head"].T
        if labels is None:
            labels = next_token_labels(tokens)
        lval, dlogits = cross_entropy(logits, labels.reshape(-1))
        dz = dlogits @ P["lm_head"]
        if "lm_head" in G:
            G["lm_head"] += dlogits.T @ z
        dh, dgf = rmsnorm_bwd(dz, h, P["final_norm"], rz)
        if "final_norm" in G:
            G["final_norm"] += dgf
    elif loss == "sumsq":
        # reading: loss = sum of squares of the last hidden state, no 1/2 and no mean
        lval = float(np.sum((h * h).astype(np.float64)))
        dh = 2.0 * h
    else:
        raise ValueError(loss)
    # block-free backward: recompute each layer from its stored input, then its backward
    for i in reversed(range(s.n_layers)):
        _, c = layer_forward(P, i, inputs[i], s, n_seq, cos, sin, forced_ids)
        dh = layer_backward(P, i, c, dh, s, n_seq, cos, sin, G)
        del c
    if "embed" in G and tokens is not None:
        np.add.at(G["embed"], tokens.reshape(-1), dh)
    return lval


def forward_backward(P: Dict[str, Array], s: Shape, G: Dict[str, Array], n_micro: int,
                     tokens: Optional[Array] = None, labels: Optional[Array] = None,
                     hidden: Optional[Array] = None, loss: str = "ce", forced_ids=None,
                     record_ids: Optional[list] = None) -> float:
    """Sum of micro-batch losses; gradients of every micro-batch are added into G.

    G maps trainable parameter names to accumulators (zeros after ``step``); passing the same G
    to several calls accumulates, exactly as calling ``forward_backward`` repeatedly before
    ``step`` does (RoundPipe user guide, 核心概念: forward_backward then step).
    """
    n_seq = tokens.shape[0] if tokens is not None else hidden.shape[0]
    S = tokens.shape[1] if tokens is not None else hidden.shape[1]
    total = 0.0
    for lo, hi in split_microbatches(n_seq, n_micro):
        fid = None if forced_ids is None else [f[lo * S:hi * S] for f in forced_ids]
        total += microbatch_forward_backward(
            P, s, G,
            tokens=None if tokens is None else tokens[lo:hi],
            labels=None if labels is None else labels[lo:hi],
            hidden=None if hidden is None else hidden[lo:hi],
            loss=loss, forced_ids=fid, record_ids=record_ids)
    return total


def zero_grads(P: Dict[str, Array], s: Shape) -> Dict[str, Array]:
    return {n: np.zeros_like(P[n]) for n in trainable_names(s, P.keys())}
