"""Shared helpers of the GPU tests: build a library model and an oracle run from one workload."""
from __future__ import annotations

import numpy as np

import host_offloaded_layer_amd as hol
import workloads as W
from oracle import decoder as D


def lib_model(w: W.Workload, params, k=None, slots=0, gbufs=0, async_opt=0, pinned_budget=0) -> hol.Model:
    s = w.shape
    cfg = hol.make_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                          n_experts=s.n_experts, top_k=s.top_k, expert_ffn=s.expert_ffn,
                          lora_rank=s.lora_rank, lora_scale=s.lora_scale, rope_base=s.rope_base,
                          rms_eps=s.rms_eps, ckpt_every_k=k or w.ckpt_every_k,
                          compute_dtype=hol.BF16 if w.compute == "bf16" else hol.F32,
                          max_tokens=w.batch * w.seq, max_seq=w.seq, lr=w.lr, beta1=w.beta1,
                          beta2=w.beta2, adam_eps=w.adam_eps, weight_slots=slots, grad_buffers=gbufs,
                          async_optimizer=async_opt, pinned_budget_bytes=pinned_budget)
    m = hol.Model(cfg)
    m.set_params(params)
    return m


def lib_fb(m: hol.Model, w: W.Workload, batch) -> float:
    if "tokens" in batch:
        return m.forward_backward(w.n_micro, tokens=batch["tokens"], loss=hol.LOSS_CE)
    return m.forward_backward(w.n_micro, hidden=batch["hidden"], loss=hol.LOSS_SUMSQ)


def oracle_fb(w: W.Workload, params, batch, dtype=np.float64):
    s = D.Shape.of(w.shape)
    P = {k: v.astype(dtype) for k, v in params.items()}
    G = D.zero_grads(P, s)
    if "tokens" in batch:
        loss = D.forward_backward(P, s, G, w.n_micro, tokens=batch["tokens"], loss="ce")
    else:
        loss = D.forward_backward(P, s, G, w.n_micro, hidden=batch["hidden"].astype(dtype), loss="sumsq")
    return loss, G


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
