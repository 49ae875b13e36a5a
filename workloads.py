"""Seeded synthetic workloads shared by the oracle tests, the library tests and the benchmark.

This module holds shapes, parameter names and random number generation only. It contains none of
the method's arithmetic (no layer math, no loss, no optimiser), so that the oracle under ``oracle/``
and the HIP library stay independent of each other while being fed identical inputs.

Five workload shapes follow the decoder families the RoundPipe and MegaTrain pages train (a tiny
decoder for parity, Qwen3-1.7B-, LLaMA-3.1-8B- and Qwen3-235B-A22B-shaped stacks). The pages
fine-tune on real text (MegaTrain summary page, 复现评估: MetaMathQA); that dataset is not used here:
uniform random token ids and N(0,1) hidden states of the same shapes stand in for it.

Generation recipe (all float32):
  * every matrix (and every LoRA factor) ~ N(0, 0.02^2); every RMSNorm gain = 1;
  * tensor number ``i`` in the canonical order below, row chunk ``c`` draws from
    ``Generator(PCG64(SeedSequence([seed, i, c])))`` so large tensors can be filled by threads;
  * tokens ~ uniform integers in [0, vocab) from ``PCG64(SeedSequence([seed]))``;
  * hidden-state inputs ~ N(0, 1) from ``PCG64(SeedSequence([seed]))``.
"""
from __future__ import annotations

import os
import threading
from dataclasses import dataclass, field, replace
from typing import Dict, List, Tuple

import numpy as np


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int = 0                 # dense SwiGLU width (0 when MoE)
    vocab: int = 0               # 0: hidden-state input, no embedding and no head
    n_experts: int = 0           # 0: dense MLP
    top_k: int = 0
    expert_ffn: int = 0
    lora_rank: int = 0           # >0: base frozen, rank-r adapters on q, k, v, o
    lora_scale: float = 1.0
    rope_base: float = 10000.0
    rms_eps: float = 1e-5


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    batch: int                   # sequences per forward_backward call
    seq: int
    n_micro: int
    ckpt_every_k: int
    compute: str                 # "f32" or "bf16"
    loss: str                    # "ce" (next-token cross entropy) or "sumsq"
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    adam_eps: float = 1e-8
    weight_seed: int = 1000
    token_seed: int = 2000
    hidden_seed: int = 3000

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def with_shape(self, **kw) -> "Workload":
        return replace(self, shape=replace(self.shape, **kw))


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 decoder: parity with the tightest tolerance.
    "tiny": Workload("tiny", ModelShape(4, 64, 4, 4, 16, ffn=172, vocab=256),
                     batch=2, seq=32, n_micro=2, ckpt_every_k=2, compute="f32", loss="ce",
                     weight_seed=1001, token_seed=2001, hidden_seed=3001),
    # Qwen3-1.7B-shaped dense decoder.
    "qwen3_1p7b": Workload("qwen3_1p7b", ModelShape(28, 2048, 16, 8, 128, ffn=6144, vocab=151936),
                           batch=4, seq=4096, n_micro=4, ckpt_every_k=4, compute="bf16", loss="ce",
                           weight_seed=1002, token_seed=2002, hidden_seed=3002),
    # LLaMA-3.1-8B-shaped dense decoder at 4K context (the headline workload).
    "llama8b": Workload("llama8b", ModelShape(32, 4096, 32, 8, 128, ffn=14336, vocab=128256),
                        batch=4, seq=4096, n_micro=4, ckpt_every_k=4, compute="bf16", loss="ce",
                        weight_seed=1003, token_seed=2003, hidden_seed=3003),
    # Same shape at 16K context.
    "llama8b_16k": Workload("llama8b_16k", ModelShape(32, 4096, 32, 8, 128, ffn=14336, vocab=128256),
                            batch=2, seq=16384, n_micro=2, ckpt_every_k=8, compute="bf16", loss="ce",
                            weight_seed=1004, token_seed=2004, hidden_seed=3004),
    # Qwen3-235B-A22B-shaped MoE slice with LoRA on q, k, v, o; hidden-state input, sum of squares.
    "qwen3_235b_slice": Workload("qwen3_235b_slice",
                                 ModelShape(8, 4096, 64, 4, 128, vocab=0, n_experts=128, top_k=8,
                                            expert_ffn=1536, lora_rank=16),
                                 batch=1, seq=8192, n_micro=1, ckpt_every_k=4, compute="bf16",
                                 loss="sumsq", weight_seed=1005, token_seed=2005, hidden_seed=3005),
}


# --------------------------------------------------------------------------------------------
# canonical parameter list
# --------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class ParamSpec:
    name: str
    shape: Tuple[int, ...]
    kind: str          # "matrix", "norm" or "lora"
    trainable: bool


def param_specs(s: ModelShape) -> List[ParamSpec]:
    """Canonical order of every parameter tensor (row-major, nn.Linear ``[out, in]`` orientation)."""
    H, d = s.hidden, s.head_dim
    qd, kd = s.n_q_heads * d, s.n_kv_heads * d
    full = s.lora_rank == 0
    out: List[ParamSpec] = []
    if s.vocab:
        out.append(ParamSpec("embed", (s.vocab, H), "matrix", full))
    for i in range(s.n_layers):
        p = f"layers.{i}."
        out += [ParamSpec(p + "attn_norm", (H,), "norm", full),
                ParamSpec(p + "wq", (qd, H), "matrix", full),
                ParamSpec(p + "wk", (kd, H), "matrix", full),
                ParamSpec(p + "wv", (kd, H), "matrix", full),
                ParamSpec(p + "wo", (H, qd), "matrix", full),
                ParamSpec(p + "mlp_norm", (H,), "norm", full)]
        if s.n_experts:
            E, Fe = s.n_experts, s.expert_ffn
            out += [ParamSpec(p + "router", (E, H), "matrix", full),
                    ParamSpec(p + "experts.w_gate", (E, Fe, H), "matrix", full),
                    ParamSpec(p + "experts.w_up", (E, Fe, H), "matrix", full),
                    ParamSpec(p + "experts.w_down", (E, H, Fe), "matrix", full)]
        else:
            F = s.ffn
            out += [ParamSpec(p + "w_gate", (F, H), "matrix", full),
                    ParamSpec(p + "w_up", (F, H), "matrix", full),
                    ParamSpec(p + "w_down", (H, F), "matrix", full)]
        if s.lora_rank:
            r = s.lora_rank
            for t, o, ii in (("q", qd, H), ("k", kd, H), ("v", kd, H), ("o", H, qd)):
                out += [ParamSpec(p + f"lora.{t}.A", (r, ii), "lora", True),
                        ParamSpec(p + f"lora.{t}.B", (o, r), "lora", True)]
    if s.vocab:
        out += [ParamSpec("final_norm", (H,), "norm", full),
                ParamSpec("lm_head", (s.vocab, H), "matrix", full)]
    return out


def n_params(s: ModelShape) -> int:
    return int(sum(int(np.prod(p.shape)) for p in param_specs(s)))


# --------------------------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------------------------
_CHUNK = 1 << 22   # elements per independently seeded chunk


def _fill_normal(out: np.ndarray, seed: int, tensor_index: int, scale: float) -> None:
    flat = out.reshape(-1)
    for c, lo in enumerate(range(0, flat.size, _CHUNK)):
        hi = min(flat.size, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_index, c])))
        g.standard_normal(out=flat[lo:hi], dtype=np.float32)
    if scale != 1.0:
        np.multiply(flat, np.float32(scale), out=flat)


def make_params(w: Workload, threads: int | None = None, std: float = 0.02) -> Dict[str, np.ndarray]:
    """All parameters of workload ``w`` as float32 arrays, keyed by canonical name."""
    specs = param_specs(w.shape)
    params: Dict[str, np.ndarray] = {}
    jobs = []
    for i, p in enumerate(specs):
        a = np.empty(p.shape, np.float32)
        params[p.name] = a
        if p.kind == "norm":
            a.fill(1.0)
        else:
            jobs.append((a, i))
    # split work by chunks across threads (numpy's generators release the GIL)
    tasks = []
    for a, i in jobs:
        flat = a.reshape(-1)
        for c, lo in enumerate(range(0, flat.size, _CHUNK)):
            tasks.append((flat, lo, min(flat.size, lo + _CHUNK), i, c))
    nthr = threads or min(16, os.cpu_count() or 1)
    lock = threading.Lock()
    cursor = [0]

    def worker():
        while True:
            with lock:
                k = cursor[0]
                cursor[0] += 1
            if k >= len(tasks):
                return
            flat, lo, hi, i, c = tasks[k]
            g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.weight_seed, i, c])))
            g.standard_normal(out=flat[lo:hi], dtype=np.float32)
            np.multiply(flat[lo:hi], np.float32(std), out=flat[lo:hi])

    ths = [threading.Thread(target=worker) for _ in range(nthr)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    return params


def make_tokens(w: Workload) -> np.ndarray:
    """Uniform token ids, int32 ``[batch, seq]``."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.token_seed])))
    return g.integers(0, w.shape.vocab, size=(w.batch, w.seq), dtype=np.int32)


def make_hidden(w: Workload) -> np.ndarray:
    """N(0,1) hidden-state input, float32 ``[batch, seq, hidden]``."""
    out = np.empty((w.batch, w.seq, w.shape.hidden), np.float32)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.hidden_seed])))
    g.standard_normal(out=out.reshape(-1), dtype=np.float32)
    return out


def make_batch(w: Workload) -> Dict[str, np.ndarray]:
    """The inputs of one ``forward_backward`` call: ``tokens`` or ``hidden``."""
    if w.shape.vocab:
        return {"tokens": make_tokens(w)}
    return {"hidden": make_hidden(w)}
