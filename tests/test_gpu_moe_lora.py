"""Mixture-of-experts and LoRA layers on the GPU against the oracle.

Routing is a discrete decision taken on rounded values, so where two experts' router logits lie
within rounding distance of each other the library and the oracle may legitimately keep different
experts. The comparison is therefore margin aware:
  1. The oracle is run with the library's routing forced (the ids read back through
     hol_get_routing). It still computes its own top-k from its own router logits. Every token
     whose expert set differs from the library's must have an oracle gap between the k-th and
     (k+1)-th largest logit below `delta`.
  2. Loss and gradients are compared with that forced-routing oracle, to the path's tolerance
     (fp32: 1e-4; bf16: 1e-2 on the loss, 2e-2 per gradient tensor).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import host_offloaded_layer_amd as hol  # noqa: E402
import workloads as W  # noqa: E402
from oracle import adam as OA  # noqa: E402
from oracle import decoder as D  # noqa: E402
from tests.gpu_helpers import lib_fb, lib_model, rel_l2  # noqa: E402

MOE_LORA_TINY = W.Workload("moe_lora_tiny",
                           W.ModelShape(2, 64, 4, 2, 16, vocab=0, n_experts=8, top_k=2, expert_ffn=32, lora_rank=4),
                           batch=2, seq=24, n_micro=1, ckpt_every_k=1, compute="f32", loss="sumsq",
                           weight_seed=61, token_seed=62, hidden_seed=63)
MOE_FULL_TINY = W.Workload("moe_full_tiny",
                           W.ModelShape(2, 64, 4, 4, 16, vocab=128, n_experts=6, top_k=3, expert_ffn=24),
                           batch=4, seq=16, n_micro=2, ckpt_every_k=2, compute="f32", loss="ce",
                           weight_seed=64, token_seed=65)
LORA_DENSE_TINY = W.Workload("lora_dense_tiny",
                             W.ModelShape(3, 64, 4, 2, 16, ffn=96, vocab=128, lora_rank=4),
                             batch=2, seq=20, n_micro=2, ckpt_every_k=2, compute="f32", loss="ce",
                             weight_seed=66, token_seed=67)
MOE_LORA_BF16 = W.Workload("moe_lora_bf16",
                           W.ModelShape(2, 256, 4, 2, 64, vocab=0, n_experts=16, top_k=4, expert_ffn=128,
                                        lora_rank=8),
                           batch=1, seq=256, n_micro=1, ckpt_every_k=2, compute="bf16", loss="sumsq",
                           weight_seed=68, token_seed=69, hidden_seed=70)

MOE_FULL_BF16 = W.Workload("moe_full_bf16",
                           W.ModelShape(2, 256, 4, 2, 64, vocab=512, n_experts=16, top_k=4, expert_ffn=128),
                           batch=2, seq=128, n_micro=2, ckpt_every_k=2, compute="bf16", loss="ce",
                           weight_seed=71, token_seed=72)


def bf16_weights(params):
    """The low-precision copy the bf16 path computes with: base matrices rounded to bf16 (RNE);
    norm gains, the embedding rows and the fp32 LoRA factors unchanged."""
    def keep(n, v):
        return v.ndim < 2 or n == "embed" or ".lora." in n
    return {n: (v if keep(n, v) else OA.bf16_to_f32(OA.bf16_round(v)).reshape(v.shape)) for n, v in params.items()}


def oracle_forced(w, params, batch, ids, dtype):
    """Oracle loss and gradients with the given routing forced, plus, per layer, the oracle's own
    top-k choice and the gap between its k-th and (k+1)-th router logits."""
    s = D.Shape.of(w.shape)
    P = {k: v.astype(dtype) for k, v in params.items()}
    G = D.zero_grads(P, s)
    kw = dict(tokens=batch["tokens"], loss="ce") if "tokens" in batch else \
        dict(hidden=batch["hidden"].astype(dtype), loss="sumsq")
    loss = D.forward_backward(P, s, G, w.n_micro, forced_ids=ids, **kw)
    own, gap = [], []
    if s.n_experts:
        # replay the forward with the forced routing to read each layer's own router decision
        n_seq, S = w.batch, w.seq
        if "tokens" in batch:
            h = P["embed"][batch["tokens"].reshape(-1)]
        else:
            h = batch["hidden"].reshape(n_seq * S, -1).astype(dtype)
        cos, sin = D.rope_tables(S, s.head_dim, s.rope_base, dtype)
        for i in range(s.n_layers):
            h, c = D.layer_forward(P, i, h, s, n_seq, cos, sin, ids)
            lg = np.sort(c["moe"]["logits"], axis=1)[:, ::-1]
            gap.append(lg[:, s.top_k - 1] - lg[:, s.top_k])
            own.append(np.argsort(-c["moe"]["probs"], axis=1, kind="stable")[:, :s.top_k])
    return loss, G, own, gap


def check_routing(lib_ids, own, gap, delta):
    flips = 0
    for l, (a, b, g) in enumerate(zip(lib_ids, own, gap)):
        differ = np.any(np.sort(a, axis=1) != np.sort(b, axis=1), axis=1)
        flips += int(differ.sum())
        assert np.all(g[differ] < delta), (l, g[differ].max())
        # ids are distinct experts in range
        assert np.all(np.sort(a, axis=1)[:, 1:] != np.sort(a, axis=1)[:, :-1])
    return flips


def run_parity(w, tol_loss, tol_grad, delta, ref_weights=lambda p: p, bounds=None):
    params = W.make_params(w, threads=16)
    batch = W.make_batch(w)
    s = w.shape
    T = w.batch * w.seq
    with lib_model(w, params) as m:
        loss = lib_fb(m, w, batch)
        ids = [m.get_routing(l, T, s.top_k) for l in range(s.n_layers)] if s.n_experts else None
        grads = {n: m.get_grad(n) for n in m.index if m.trainable[n]}
        stats = m.stats()
    ref_loss, ref_G, own, gap = oracle_forced(w, ref_weights(params), batch, ids, np.float32 if tol_grad > 1e-3 else np.float64)
    flips = check_routing(ids, own, gap, delta) if ids is not None else 0
    errs = {n: rel_l2(grads[n], g) for n, g in ref_G.items()}
    worst = sorted(errs.items(), key=lambda x: -x[1])[:6]
    print(w.name, "loss", loss, ref_loss, "routing flips", flips, "worst", worst, "stream", stats["n_weight_streams"])
    assert set(grads) == set(ref_G)
    assert abs(loss - ref_loss) <= tol_loss * abs(ref_loss)
    for n, e in errs.items():
        assert e <= (bounds(n) if bounds else tol_grad), (n, e)


def test_moe_lora_tiny_fp32_matches_oracle():
    run_parity(MOE_LORA_TINY, 1e-4, 1e-4, 1e-3)


def test_moe_full_finetune_tiny_fp32_matches_oracle():
    run_parity(MOE_FULL_TINY, 1e-4, 1e-4, 1e-3)


def test_lora_dense_tiny_fp32_matches_oracle():
    run_parity(LORA_DENSE_TINY, 1e-4, 1e-4, 1e-3)


def test_moe_lora_bf16_small_matches_oracle():
    run_parity(MOE_LORA_BF16, 1e-2, 2e-2, 0.05, ref_weights=bf16_weights)


def test_moe_full_finetune_bf16_matches_oracle():
    """bf16 full fine-tune: grouped expert products for the data gradients, per-expert launches
    for the expert weight gradients."""
    run_parity(MOE_FULL_BF16, 1e-2, 2e-2, 0.05, ref_weights=bf16_weights)


def test_moe_lora_real_layer_shapes_matches_oracle():
    """The 235B-A22B layer (64/4 heads, 128 experts x 1536, top-8, LoRA r=16) with 2 layers and 256
    tokens: every kernel in the launch shape of the full slice."""
    w = W.WORKLOADS["qwen3_235b_slice"].with_(seq=256).with_shape(n_layers=2)
    run_parity(w, 1e-2, 2e-2, 0.05, ref_weights=bf16_weights)


@pytest.mark.parametrize("w", [MOE_LORA_TINY, MOE_FULL_TINY, MOE_LORA_BF16, MOE_FULL_BF16], ids=lambda w: w.name)
def test_moe_results_independent_of_k_bitwise(w):
    """The recompute permutes routed rows in a different order (atomics); every result must be
    bitwise the same for any checkpoint interval."""
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    with lib_model(w, params, k=w.shape.n_layers) as m:
        out = {}
        for k in range(1, w.shape.n_layers + 1):
            m.set_ckpt_every_k(k)
            m.zero_grad()
            loss = lib_fb(m, w, batch)
            out[k] = (loss, {n: m.get_grad(n) for n in m.index if m.trainable[n]})
        for k in out:
            assert out[k][0] == out[1][0]
            for n in out[1][1]:
                assert np.array_equal(out[k][1][n], out[1][1][n]), (k, n)


def test_lora_fused_step_and_frozen_tensors():
    """LoRA: only the adapters train; the fused call equals forward_backward + step bit for bit;
    frozen tensors keep their values (bf16 image values read back through get_tensor)."""
    w = MOE_LORA_BF16
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    with lib_model(w, params) as a, lib_model(w, params) as b:
        assert {n for n in a.index if a.trainable[n]} == {n for n in params if ".lora." in n}
        for _ in range(2):
            la = lib_fb(a, w, batch)
            a.step()
            lb = b.forward_backward(w.n_micro, hidden=batch["hidden"], loss=hol.LOSS_SUMSQ, and_step=True)
            assert la == lb
        for n in a.index:
            x, y = a.get_tensor(n), b.get_tensor(n)
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n
            if not a.trainable[n]:
                ref = params[n] if params[n].ndim < 2 else OA.bf16_to_f32(OA.bf16_round(params[n])).reshape(params[n].shape)
                assert np.array_equal(x, ref), n
            else:
                assert not np.array_equal(x, params[n]), n   # adapters moved
