"""How close can any bf16-operand implementation of the layer get to the oracle? (CPU)

The bf16 path's gradients are held to 2e-2 relative L2 per tensor against the oracle run on the
bf16 copy of the weights, except wq, wk and the attention-norm gain, held to 3e-2. This test is the
evidence for that exception. It runs, in fp32 NumPy, an exact model of a bf16-operand pipeline:
the same arithmetic as the oracle, with every value rounded to bf16 (round-to-nearest-even) where
the bf16 path hands it to a matrix product as an operand or stores it in bf16:

  forward   n1, q/k/v after RoPE, the softmax probabilities before the P.V product, o, n2,
            gate and up outputs, the SwiGLU output a, the final-norm output z;
  backward  d logits, dh before each product that reads it, da, dgu, dO, dS (before the dQ and
            dK products), P (before the dV product), dq/dk/dv and their RoPE backward;
  fp32      everything else: accumulation, residual stream, norm statistics, softmax, loss.

Nothing else differs from the oracle, so the errors measured here are what bf16 operands alone
cost, whatever the kernels. At the LLaMA-3.1-8B layer shapes (2 layers, 2 micro-batches of 256
tokens, the shapes of the GPU parity case) the tensors whose gradients flow through the attention
scores (wq, wk) sit above 2e-2, while every other tensor stays below it. With q, k and v kept in
fp32 instead (everything else still rounded) wq and wk drop below 2e-2: the floor comes from the
bf16 rounding of the score operands.

Test infrastructure only: it uses the oracle's functions for the rounding-free steps and shares
nothing with the HIP library.
"""
import numpy as np
import pytest

import workloads as W
from oracle import decoder as D

torch = pytest.importorskip("torch")


def rnd(x):
    """fp32 -> bf16 (round to nearest even) -> fp32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _attention_fwd(q, k, v, round_p=True):
    """One sequence, q [S, nq, d], k/v [S, nkv, d]; P rounded before the P.V product."""
    S, nq, d = q.shape
    grp = nq // k.shape[1]
    scale = np.float32(1.0 / np.sqrt(d))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    o = np.empty_like(q)
    lse = np.empty((nq, S), np.float32)
    for h in range(nq):
        s = (q[:, h] @ k[:, h // grp].T) * scale
        s[mask] = -np.inf
        m = s.max(1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(1, keepdims=True)
        pv = (rnd(p) if round_p else p) @ v[:, h // grp]
        o[:, h] = pv / l
        lse[h] = (m + np.log(l))[:, 0]
    return rnd(o), lse


def _attention_bwd(do, q, k, v, o, lse):
    S, nq, d = q.shape
    grp = nq // k.shape[1]
    scale = np.float32(1.0 / np.sqrt(d))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nq):
        g = h // grp
        s = (q[:, h] @ k[:, g].T) * scale
        s[mask] = -np.inf
        p = np.exp(s - lse[h][:, None])
        dv[:, g] += rnd(p).T @ do[:, h]
        dp = do[:, h] @ v[:, g].T
        delta = np.sum(do[:, h] * o[:, h], axis=1, keepdims=True)
        ds = rnd(p * (dp - delta) * scale)
        dq[:, h] = ds @ k[:, g]
        dk[:, g] += ds.T @ q[:, h]
    return rnd(dq), rnd(dk), rnd(dv)


def emulate_bf16_path(P, s, tokens, n_micro, round_qkv=True):
    """Loss sum and gradients of the dense decoder with the bf16 path's rounding points.
    P holds the bf16-rounded matrices (fp32 values) and fp32 norm gains / embedding rows."""
    G = {n: np.zeros_like(P[n]) for n in D.trainable_names(s, P.keys())}
    rq = rnd if round_qkv else (lambda x: x)
    d, nq, nkv, H = s.head_dim, s.n_q_heads, s.n_kv_heads, s.hidden
    total = 0.0
    for lo, hi in D.split_microbatches(tokens.shape[0], n_micro):
        tok = tokens[lo:hi]
        n_seq, S = tok.shape
        T = n_seq * S
        cos, sin = D.rope_tables(S, d, s.rope_base, np.float32)
        h = P["embed"][tok.reshape(-1)].astype(np.float32)
        caches = []
        for i in range(s.n_layers):
            pre = f"layers.{i}."
            n1f, r1 = D.rmsnorm(h, P[pre + "attn_norm"], s.rms_eps)
            n1 = rnd(n1f)
            q = (n1 @ P[pre + "wq"].T).reshape(n_seq, S, nq, d)
            k = (n1 @ P[pre + "wk"].T).reshape(n_seq, S, nkv, d)
            v = (n1 @ P[pre + "wv"].T).reshape(n_seq, S, nkv, d)
            q = np.stack([rq(D.rope(q[b], cos, sin)) for b in range(n_seq)])
            k = np.stack([rq(D.rope(k[b], cos, sin)) for b in range(n_seq)])
            v = rq(v)
            o = np.empty_like(q)
            lse = np.empty((n_seq, nq, S), np.float32)
            for b in range(n_seq):
                o[b], lse[b] = _attention_fwd(q[b], k[b], v[b])
            o2 = o.reshape(T, nq * d)
            h1 = h + o2 @ P[pre + "wo"].T
            n2f, r2 = D.rmsnorm(h1, P[pre + "mlp_norm"], s.rms_eps)
            n2 = rnd(n2f)
            g = rnd(n2 @ P[pre + "w_gate"].T)
            u = rnd(n2 @ P[pre + "w_up"].T)
            a = rnd(D.swiglu(g, u))
            caches.append(dict(h=h, n1=n1, r1=r1, q=q, k=k, v=v, o=o, lse=lse, h1=h1, n2=n2, r2=r2,
                               g=g, u=u, a=a))
            h = h1 + a @ P[pre + "w_down"].T
        zf, rz = D.rmsnorm(h, P["final_norm"], s.rms_eps)
        z = rnd(zf)
        logits = z @ P["lm_head"].T
        lval, dlog = D.cross_entropy(logits, D.next_token_labels(tok).reshape(-1))
        total += lval
        dlog = rnd(dlog)
        G["lm_head"] += dlog.T @ z
        dh, dgf = D.rmsnorm_bwd(dlog @ P["lm_head"], h, P["final_norm"], rz)
        G["final_norm"] += dgf
        for i in reversed(range(s.n_layers)):
            pre = f"layers.{i}."
            c = caches[i]
            dhb = rnd(dh)
            da = rnd(dhb @ P[pre + "w_down"])
            G[pre + "w_down"] += dhb.T @ c["a"]
            dg, du = D.swiglu_bwd(da, c["g"], c["u"])
            dg, du = rnd(dg), rnd(du)
            dn2 = dg @ P[pre + "w_gate"] + du @ P[pre + "w_up"]
            G[pre + "w_gate"] += dg.T @ c["n2"]
            G[pre + "w_up"] += du.T @ c["n2"]
            dx, dg2 = D.rmsnorm_bwd(dn2, c["h1"], P[pre + "mlp_norm"], c["r2"])
            G[pre + "mlp_norm"] += dg2
            dh = dh + dx
            dhb = rnd(dh)
            do = rnd(dhb @ P[pre + "wo"]).reshape(n_seq, S, nq, d)
            G[pre + "wo"] += dhb.T @ c["o"].reshape(T, nq * d)
            dq = np.empty_like(c["q"])
            dk = np.empty_like(c["k"])
            dv = np.empty_like(c["v"])
            for b in range(n_seq):
                dqr, dkr, dv[b] = _attention_bwd(do[b], c["q"][b], c["k"][b], c["v"][b], c["o"][b], c["lse"][b])
                dq[b] = rnd(D.rope_bwd(dqr, cos, sin))
                dk[b] = rnd(D.rope_bwd(dkr, cos, sin))
            dq, dk, dv = dq.reshape(T, -1), dk.reshape(T, -1), dv.reshape(T, -1)
            dn1 = dq @ P[pre + "wq"] + dk @ P[pre + "wk"] + dv @ P[pre + "wv"]
            G[pre + "wq"] += dq.T @ c["n1"]
            G[pre + "wk"] += dk.T @ c["n1"]
            G[pre + "wv"] += dv.T @ c["n1"]
            dx, dg1 = D.rmsnorm_bwd(dn1, c["h"], P[pre + "attn_norm"], c["r1"])
            G[pre + "attn_norm"] += dg1
            dh = dh + dx
        np.add.at(G["embed"], tok.reshape(-1), dh)
    return total, G


def _bf16_weights(params):
    """The bf16 copy the path computes with: matrices rounded, gains and embedding rows fp32."""
    return {n: (rnd(v) if v.ndim >= 2 and n != "embed" else v) for n, v in params.items()}


def _rel(a, b):
    return float(np.linalg.norm((a - b).astype(np.float64)) / max(np.linalg.norm(b.astype(np.float64)), 1e-30))


SCORE_INPUTS = ("wq", "wk", "attn_norm")


@pytest.fixture(scope="module")
def llama8b_case():
    w = W.WORKLOADS["llama8b"].with_(batch=2, seq=256, n_micro=2).with_shape(n_layers=2)
    P = _bf16_weights(W.make_params(w, threads=8))
    tokens = W.make_batch(w)["tokens"]
    s = D.Shape.of(w.shape)
    G = D.zero_grads(P, s)
    ref_loss = D.forward_backward(P, s, G, w.n_micro, tokens=tokens)
    return w, P, tokens, s, ref_loss, G


def test_bf16_operands_alone_put_score_weight_gradients_above_2e2(llama8b_case):
    w, P, tokens, s, ref_loss, ref_G = llama8b_case
    loss, G = emulate_bf16_path(P, s, tokens, w.n_micro)
    errs = {n: _rel(G[n], ref_G[n]) for n in ref_G}
    print("loss", loss, ref_loss, "errors", sorted(errs.items(), key=lambda x: -x[1]))
    assert abs(loss - ref_loss) <= 1e-2 * abs(ref_loss)
    score = {n: e for n, e in errs.items() if n.split(".")[-1] in SCORE_INPUTS}
    other = {n: e for n, e in errs.items() if n not in score}
    # the floor: some score-input gradient is above the 2e-2 bar for any bf16-operand pipeline
    assert max(errs[f"layers.{i}.{t}"] for i in range(2) for t in ("wq", "wk")) > 2e-2, score
    # and all of them within the 3e-2 the GPU parity test allows these tensors
    assert max(score.values()) <= 3e-2, score
    # every other tensor meets the 2e-2 bar
    assert max(other.values()) < 2e-2, other


def test_fp32_score_operands_remove_the_floor(llama8b_case):
    w, P, tokens, s, ref_loss, ref_G = llama8b_case
    loss, G = emulate_bf16_path(P, s, tokens, w.n_micro, round_qkv=False)
    errs = {n: _rel(G[n], ref_G[n]) for n in ref_G}
    print("q/k/v in fp32: errors", sorted(errs.items(), key=lambda x: -x[1])[:8])
    for i in range(2):
        for t in ("wq", "wk"):
            assert errs[f"layers.{i}.{t}"] < 2e-2, (i, t, errs[f"layers.{i}.{t}"])
