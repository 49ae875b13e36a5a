"""A second, independent statement of the decoder, built from torch library routines.

Used only to pin the NumPy oracle: forward values come from ``torch.nn.functional`` routines
(``linear``, ``rms_norm``, ``scaled_dot_product_attention``, ``silu``, ``cross_entropy``,
``softmax``) and gradients from torch autograd, so a dropped term, a wrong sign or a transposed
operand in the oracle's hand-written forward or backward shows up as a mismatch. RoPE has no
library routine; it is pinned by its own invariants in ``test_oracle_layers.py``.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
import torch
import torch.nn.functional as F


def _rope(x: torch.Tensor, base: float) -> torch.Tensor:
    # x: [S, heads, d]; rotate-half with theta_j = base^(-2j/d) (angles in fp64)
    S, _, d = x.shape
    half = d // 2
    j = torch.arange(half, dtype=torch.float64)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * (base ** (-2.0 * j / d))[None, :]
    c = torch.cos(ang).to(x.dtype)[:, None, :]
    s = torch.sin(ang).to(x.dtype)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def _lin(x, P, w, lora, shape):
    y = F.linear(x, P[w])
    if lora is not None:
        y = y + shape.lora_scale * F.linear(F.linear(x, P[lora + ".A"]), P[lora + ".B"])
    return y


def _moe(n2, P, pre, shape, forced):
    logits = F.linear(n2, P[pre + "router"])
    probs = F.softmax(logits, dim=-1)
    if forced is None:
        _, ids = torch.topk(probs, shape.top_k, dim=-1)
    else:
        ids = torch.as_tensor(forced)
    kept = torch.gather(probs, 1, ids)
    w = kept / kept.sum(dim=1, keepdim=True)
    out = torch.zeros_like(n2)
    for slot in range(shape.top_k):
        for e in range(shape.n_experts):
            rows = (ids[:, slot] == e).nonzero()[:, 0]
            if rows.numel() == 0:
                continue
            x = n2[rows]
            a = F.silu(F.linear(x, P[pre + "experts.w_gate"][e])) * F.linear(x, P[pre + "experts.w_up"][e])
            y = F.linear(a, P[pre + "experts.w_down"][e])
            out = out.index_add(0, rows, w[rows, slot][:, None] * y)
    return out


def loss_and_grads(params: Dict[str, np.ndarray], shape, n_micro: int, tokens=None, hidden=None,
                   loss: str = "ce", trainable: Optional[List[str]] = None, forced_ids=None):
    """fp64 torch autograd over the same definition; returns (loss_sum, grads dict)."""
    P = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(trainable is None or k in trainable))
         for k, v in params.items()}
    n_seq = tokens.shape[0] if tokens is not None else hidden.shape[0]
    S = tokens.shape[1] if tokens is not None else hidden.shape[1]
    per = n_seq // n_micro
    total = 0.0
    d, nq, nkv = shape.head_dim, shape.n_q_heads, shape.n_kv_heads
    lo = (lambda p, t: p + "lora." + t) if shape.lora_rank else (lambda p, t: None)
    for m in range(n_micro):
        if tokens is not None:
            tk = torch.as_tensor(tokens[m * per:(m + 1) * per].astype(np.int64))
            h = F.embedding(tk.reshape(-1), P["embed"])
        else:
            h = torch.tensor(hidden[m * per:(m + 1) * per].reshape(-1, shape.hidden), dtype=torch.float64)
        for i in range(shape.n_layers):
            pre = f"layers.{i}."
            n1 = F.rms_norm(h, (shape.hidden,), P[pre + "attn_norm"], shape.rms_eps)
            q = _lin(n1, P, pre + "wq", lo(pre, "q"), shape).reshape(per, S, nq, d)
            k = _lin(n1, P, pre + "wk", lo(pre, "k"), shape).reshape(per, S, nkv, d)
            v = _lin(n1, P, pre + "wv", lo(pre, "v"), shape).reshape(per, S, nkv, d)
            outs = []
            for b in range(per):
                qb = _rope(q[b], shape.rope_base).transpose(0, 1)       # [nq, S, d]
                kb = _rope(k[b], shape.rope_base).transpose(0, 1)
                vb = v[b].transpose(0, 1)
                ob = F.scaled_dot_product_attention(qb[None], kb[None], vb[None], is_causal=True,
                                                    enable_gqa=True)[0]
                outs.append(ob.transpose(0, 1).reshape(S, nq * d))
            o = torch.cat(outs, 0)
            h = h + _lin(o, P, pre + "wo", lo(pre, "o"), shape)
            n2 = F.rms_norm(h, (shape.hidden,), P[pre + "mlp_norm"], shape.rms_eps)
            if shape.n_experts:
                fid = None if forced_ids is None else forced_ids[i][m * per * S:(m + 1) * per * S]
                h = h + _moe(n2, P, pre, shape, fid)
            else:
                a = F.silu(F.linear(n2, P[pre + "w_gate"])) * F.linear(n2, P[pre + "w_up"])
                h = h + F.linear(a, P[pre + "w_down"])
        if loss == "ce":
            z = F.rms_norm(h, (shape.hidden,), P["final_norm"], shape.rms_eps)
            logits = F.linear(z, P["lm_head"])
            lab = torch.full((per, S), -1, dtype=torch.int64)
            lab[:, :-1] = tk.reshape(per, S)[:, 1:]
            lm = F.cross_entropy(logits, lab.reshape(-1), ignore_index=-1)
        else:
            lm = (h * h).sum()
        lm.backward()
        total += float(lm)
    grads = {k: (v.grad.numpy() if v.grad is not None else np.zeros(v.shape)) for k, v in P.items()
             if v.requires_grad}
    return total, grads
