"""Pins of the whole oracle (decoder + loss + backward + micro-batch summation, fp64)."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import decoder as D
from tests import torch_ref

TINY = W.WORKLOADS["tiny"]


def tiny_case(dtype=np.float64, **shape_kw):
    w = TINY.with_shape(**shape_kw) if shape_kw else TINY
    P = {k: v.astype(dtype) for k, v in W.make_params(w, threads=2).items()}
    return w, P, W.make_tokens(w)


def moe_lora_case(dtype=np.float64, n_layers=2, seq=12, batch=2, n_micro=2, std=0.3):
    shape = W.ModelShape(n_layers, 16, 4, 2, 4, vocab=0, n_experts=6, top_k=2, expert_ffn=8,
                         lora_rank=3)
    w = W.Workload("moe_lora_tiny", shape, batch=batch, seq=seq, n_micro=n_micro, ckpt_every_k=1,
                   compute="f32", loss="sumsq", weight_seed=77, hidden_seed=78)
    P = {k: v.astype(dtype) for k, v in W.make_params(w, threads=2, std=std).items()}
    return w, P, W.make_hidden(w).astype(dtype) * 0.5


def run(w, P, tokens=None, hidden=None, n_micro=None, forced=None, record=None):
    s = D.Shape.of(w.shape)
    G = D.zero_grads(P, s)
    loss = D.forward_backward(P, s, G, n_micro or w.n_micro, tokens=tokens, hidden=hidden,
                              loss=w.loss if hidden is not None else "ce", forced_ids=forced,
                              record_ids=record)
    return loss, G


def test_oracle_matches_torch_autograd_dense():
    w, P, tok = tiny_case()
    loss, G = run(w, P, tokens=tok)
    ref_loss, ref_G = torch_ref.loss_and_grads(P, w.shape, w.n_micro, tokens=tok)
    assert abs(loss - ref_loss) <= 1e-12 * abs(ref_loss)
    for n, g in G.items():
        r = ref_G[n]
        assert np.linalg.norm(g - r) <= 1e-10 * max(np.linalg.norm(r), 1e-30), n


def test_oracle_matches_torch_autograd_gqa():
    w, P, tok = tiny_case(n_kv_heads=2, n_layers=2)
    loss, G = run(w, P, tokens=tok)
    ref_loss, ref_G = torch_ref.loss_and_grads(P, w.shape, w.n_micro, tokens=tok)
    assert abs(loss - ref_loss) <= 1e-12 * abs(ref_loss)
    for n, g in G.items():
        assert np.linalg.norm(g - ref_G[n]) <= 1e-10 * max(np.linalg.norm(ref_G[n]), 1e-30), n


def test_oracle_matches_torch_autograd_moe_lora():
    w, P, hid = moe_lora_case()
    rec = []
    loss, G = run(w, P, hidden=hid, record=rec)
    s = D.Shape.of(w.shape)
    # forced routing = the oracle's own ids, so both sides take the same top-k choice
    per_layer = [np.concatenate([rec[m * w.shape.n_layers + i] for m in range(w.n_micro)])
                 for i in range(w.shape.n_layers)]
    ref_loss, ref_G = torch_ref.loss_and_grads(P, w.shape, w.n_micro, hidden=hid, loss="sumsq",
                                               trainable=D.trainable_names(s, P), forced_ids=per_layer)
    assert abs(loss - ref_loss) <= 1e-11 * abs(ref_loss)
    assert set(G) == {n for n in P if ".lora." in n}
    for n, g in G.items():
        assert np.linalg.norm(g - ref_G[n]) <= 1e-9 * max(np.linalg.norm(ref_G[n]), 1e-30), n


def _directional_fd(w, P, G, f, h=1e-5, per_tensor=1, seed=3):
    r = np.random.default_rng(seed)
    for n, g in G.items():
        for _ in range(per_tensor):
            v = r.standard_normal(g.shape)
            old = P[n].copy()
            P[n][...] = old + h * v
            fp = f()
            P[n][...] = old - h * v
            fm = f()
            P[n][...] = old
            fd = (fp - fm) / (2 * h)
            an = float(np.sum(g * v))
            assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (n, fd, an)


def test_oracle_finite_differences_dense():
    w, P, tok = tiny_case(n_layers=2)
    loss, G = run(w, P, tokens=tok)
    f = lambda: run(w, P, tokens=tok)[0]
    _directional_fd(w, P, G, f)


def test_oracle_finite_differences_moe_lora():
    w, P, hid = moe_lora_case(n_layers=1, seq=6, batch=1, n_micro=1)
    rec = []
    loss, G = run(w, P, hidden=hid, record=rec)
    forced = [rec[0]]
    f = lambda: run(w, P, hidden=hid, forced=forced)[0]
    _directional_fd(w, P, G, f)


def test_microbatch_sum_invariant():
    """The returned loss is the sum of micro-batch losses and the gradient the sum of micro-batch
    gradients; with equal label counts that is n_micro times the full-batch mean
    (RoundPipe user guide, 输入分割与 microbatch 执行)."""
    w, P, tok = tiny_case(n_layers=2)
    l2, G2 = run(w, P, tokens=tok, n_micro=2)
    la, Ga = run(w, P, tokens=tok[:1], n_micro=1)
    lb, Gb = run(w, P, tokens=tok[1:], n_micro=1)
    l1, G1 = run(w, P, tokens=tok, n_micro=1)
    assert abs(l2 - (la + lb)) <= 1e-13 * l2
    assert abs(l2 - 2 * l1) <= 1e-13 * l2
    for n in G2:
        np.testing.assert_allclose(G2[n], Ga[n] + Gb[n], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(G2[n], 2 * G1[n], rtol=1e-10, atol=1e-15)


def test_accumulation_over_calls_equals_one_call():
    w, P, tok = tiny_case(n_layers=1)
    s = D.Shape.of(w.shape)
    G = D.zero_grads(P, s)
    D.forward_backward(P, s, G, 1, tokens=tok[:1])
    D.forward_backward(P, s, G, 1, tokens=tok[1:])
    _, G2 = run(w, P, tokens=tok, n_micro=2)
    for n in G:
        np.testing.assert_allclose(G[n], G2[n], rtol=1e-12, atol=1e-15)


def test_zero_head_gives_exact_log_vocab():
    """lm_head = 0 makes every logit 0: each micro-batch loss is exactly ln V."""
    w, P, tok = tiny_case(n_layers=2)
    P["lm_head"][:] = 0
    loss, G = run(w, P, tokens=tok)
    assert abs(loss - w.n_micro * math.log(w.shape.vocab)) < 1e-12
    # and the head gradient is (1/V - onehot)/count summed -> row sums of dW_head are zero
    np.testing.assert_allclose(G["lm_head"].sum(0), 0, atol=1e-14)


def test_small_init_loss_near_log_vocab():
    w, P, tok = tiny_case()
    loss, _ = run(w, P, tokens=tok)
    assert abs(loss / (w.n_micro * math.log(w.shape.vocab)) - 1) < 0.03


def test_identity_layers_when_output_maps_are_zero():
    """wo = w_down = 0 turns every layer into the identity (pure residual)."""
    w, P, tok = tiny_case(n_layers=3)
    s = D.Shape.of(w.shape)
    for i in range(3):
        P[f"layers.{i}.wo"][:] = 0
        P[f"layers.{i}.w_down"][:] = 0
    h = P["embed"][tok[0]]
    cos, sin = D.rope_tables(w.seq, s.head_dim, s.rope_base, np.float64)
    out = h
    for i in range(3):
        out, _ = D.layer_forward(P, i, out, s, 1, cos, sin)
    np.testing.assert_array_equal(out, h)


def test_lora_zero_B_is_base_and_merged_weights_match():
    w, P, hid = moe_lora_case(n_layers=1, seq=6, batch=1, n_micro=1)
    s = D.Shape.of(w.shape)
    cos, sin = D.rope_tables(6, s.head_dim, s.rope_base, np.float64)
    x = hid.reshape(6, -1)
    # merged base: W + s B A equals the LoRA forward
    Pm = {k: v.copy() for k, v in P.items()}
    for t, wname in (("q", "wq"), ("k", "wk"), ("v", "wv"), ("o", "wo")):
        Pm[f"layers.0.{wname}"] += s.lora_scale * P[f"layers.0.lora.{t}.B"] @ P[f"layers.0.lora.{t}.A"]
        Pm[f"layers.0.lora.{t}.B"][:] = 0
    y1, c1 = D.layer_forward(P, 0, x, s, 1, cos, sin)
    y2, _ = D.layer_forward(Pm, 0, x, s, 1, cos, sin, forced_ids=[c1["moe"]["ids"]])
    np.testing.assert_allclose(y1, y2, rtol=1e-11, atol=1e-12)
    # B = 0: the A gradients vanish
    G = {n: np.zeros_like(P[n]) for n in P if ".lora." in n}
    Pz = {k: v.copy() for k, v in P.items()}
    for t in "qkvo":
        Pz[f"layers.0.lora.{t}.B"][:] = 0
    y, c = D.layer_forward(Pz, 0, x, s, 1, cos, sin)
    D.layer_backward(Pz, 0, c, np.ones_like(y), s, 1, cos, sin, G)
    for t in "qkvo":
        assert np.all(G[f"layers.0.lora.{t}.A"] == 0)
        assert np.any(G[f"layers.0.lora.{t}.B"] != 0)


def test_sumsq_gradient_is_twice_output():
    w, P, hid = moe_lora_case(n_layers=0, seq=5, batch=1, n_micro=1)
    s = D.Shape.of(w.shape)
    G = {}
    loss = D.forward_backward(P, s, G, 1, hidden=hid, loss="sumsq")
    assert abs(loss - float(np.sum(hid * hid))) < 1e-12


def test_split_rejects_unequal_microbatches_and_matches_guide_example():
    # the user guide's example: batch 12 in 3 micro-batches -> samples 0-3, 4-7, 8-11
    golden = [tuple(int(x) for x in line.split()) for line in
              open(__file__.replace("test_oracle_model.py", "golden/microbatch_split_12x3.txt"))
              if line.strip() and not line.startswith("#")]
    assert D.split_microbatches(12, 3) == golden
    with pytest.raises(ValueError):
        D.split_microbatches(10, 3)


def test_float32_oracle_close_to_float64():
    w, P64, tok = tiny_case()
    P32 = {k: v.astype(np.float32) for k, v in P64.items()}
    l64, G64 = run(w, P64, tokens=tok)
    l32, G32 = run(w, P32, tokens=tok)
    assert abs(l32 - l64) <= 1e-6 * l64
    for n in G64:
        assert np.linalg.norm(G32[n] - G64[n]) <= 1e-4 * np.linalg.norm(G64[n]), n


def test_oracle_matches_torch_autograd_moe_unforced_routing():
    """Both sides choose their own experts (torch.topk on the torch side). The case is checked to
    have clear top-k margins, so a routing rule that kept other experts than the k most probable
    would show up as a loss and gradient mismatch."""
    w, P, hid = moe_lora_case()
    rec = []
    loss, G = run(w, P, hidden=hid, record=rec)
    s = D.Shape.of(w.shape)
    # no routing decision is near a tie: perturbing the input by 1e-6 relative keeps every id
    rec2 = []
    run(w, P, hidden=hid * (1 + 1e-6), record=rec2)
    for a, b in zip(rec, rec2):
        np.testing.assert_array_equal(a, b)
    ref_loss, ref_G = torch_ref.loss_and_grads(P, w.shape, w.n_micro, hidden=hid, loss="sumsq",
                                               trainable=D.trainable_names(s, P))
    assert abs(loss - ref_loss) <= 1e-11 * abs(ref_loss)
    for n, g in G.items():
        assert np.linalg.norm(g - ref_G[n]) <= 1e-9 * max(np.linalg.norm(ref_G[n]), 1e-30), n
