"""End-to-end parity on the GPU: hol_forward_backward / hol_step through the C ABI against the
oracle on identical seeded inputs (tolerances: fp32 path 1e-4 relative on loss and per-tensor
relative L2 on gradients; bf16 path 1e-2 on loss and 2e-2 per gradient tensor), plus the
invariants the method fixes exactly (independence of K, micro-batch summation, accumulation over
calls, the host Adam step)."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import host_offloaded_layer_amd as hol  # noqa: E402
import workloads as W  # noqa: E402
from oracle import adam as OA  # noqa: E402
from oracle import decoder as D  # noqa: E402
from tests.gpu_helpers import lib_fb, lib_model, oracle_fb, rel_l2  # noqa: E402

TINY = W.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny():
    params = W.make_params(TINY, threads=4)
    batch = W.make_batch(TINY)
    ref_loss, ref_G = oracle_fb(TINY, params, batch)
    return params, batch, ref_loss, ref_G


def test_tiny_fp32_matches_oracle(tiny):
    params, batch, ref_loss, ref_G = tiny
    with lib_model(TINY, params) as m:
        loss = lib_fb(m, TINY, batch)
        print("tiny loss", loss, ref_loss, m.stats())
        assert abs(loss - ref_loss) <= 1e-4 * abs(ref_loss)
        for n, g in ref_G.items():
            assert rel_l2(m.get_grad(n), g) <= 1e-4, n


def test_tiny_results_independent_of_k_bitwise(tiny):
    params, batch, _, _ = tiny
    with lib_model(TINY, params, k=4) as m:
        out = {}
        for k in (1, 2, 3, 4):
            m.set_ckpt_every_k(k)
            m.zero_grad()
            loss = lib_fb(m, TINY, batch)
            out[k] = (loss, {n: m.get_grad(n) for n in m.index})
        for k in (2, 3, 4):
            assert out[k][0] == out[1][0]
            for n in out[1][1]:
                assert np.array_equal(out[k][1][n], out[1][1][n]), (k, n)


def test_tiny_accumulation_and_microbatch_sum(tiny):
    params, batch, ref_loss, ref_G = tiny
    tok = batch["tokens"]
    with lib_model(TINY, params) as m:
        la = m.forward_backward(1, tokens=tok[:1])
        lb = m.forward_backward(1, tokens=tok[1:])    # second call accumulates on the host
        assert abs((la + lb) - ref_loss) <= 1e-4 * ref_loss
        for n, g in ref_G.items():
            assert rel_l2(m.get_grad(n), g) <= 1e-4, n
        # n_micro = 1 over the whole batch: the mean over twice the labels -> half of the sum
        m.zero_grad()
        l1 = m.forward_backward(1, tokens=tok)
        assert abs(2 * l1 - ref_loss) <= 1e-4 * ref_loss


def test_tiny_step_is_host_adam_on_library_gradients(tiny):
    params, batch, _, _ = tiny
    with lib_model(TINY, params) as m:
        lib_fb(m, TINY, batch)
        grads = {n: m.get_grad(n) for n in m.index}
        m.step()
        for n in m.index:
            th = params[n].astype(np.float32).copy()
            m1 = np.zeros_like(th); m2 = np.zeros_like(th)
            OA.adam_update(th, grads[n], m1, m2, 1, lr=TINY.lr)
            got = m.get_tensor(n)
            a, b, st = m.get_adam_state(n)
            assert st == 1
            assert np.array_equal(got.view(np.uint32), th.view(np.uint32)), n
            assert np.array_equal(a.view(np.uint32), m1.view(np.uint32)), n
            assert np.array_equal(b.view(np.uint32), m2.view(np.uint32)), n
            assert not np.any(m.get_grad(n)), n   # step zeroes the gradients
        # the next forward_backward streams the refreshed weights
        new_params = {n: m.get_tensor(n) for n in m.index}
        loss2 = lib_fb(m, TINY, batch)
        ref2, _ = oracle_fb(TINY, new_params, batch)
        assert abs(loss2 - ref2) <= 1e-4 * ref2


def test_poison_free_validation_errors(tiny):
    params, batch, _, _ = tiny
    with lib_model(TINY, params) as m:
        with pytest.raises(hol.HolError) as e:
            m.forward_backward(3, tokens=batch["tokens"])        # 2 sequences into 3 micro-batches
        assert e.value.status == hol.HOL_EINVAL
        bad = batch["tokens"].copy(); bad[0, 0] = TINY.shape.vocab
        with pytest.raises(hol.HolError):
            m.forward_backward(2, tokens=bad)
        with pytest.raises(hol.HolError):
            m.set_ckpt_every_k(3)   # above the K planned at create
        # still usable
        assert math.isfinite(lib_fb(m, TINY, batch))


BF16_SMALL = W.Workload("bf16_small", W.ModelShape(3, 256, 4, 2, 64, ffn=512, vocab=1000),
                        batch=4, seq=160, n_micro=2, ckpt_every_k=2, compute="bf16", loss="ce",
                        weight_seed=51, token_seed=52)


# Tensors whose gradients flow through the attention scores. Rounding the attention inputs to
# bf16 perturbs the scores, and dq / dk sum cancelling terms. tests/test_bf16_rounding_floor.py
# runs an exact bf16-operand model of the layer on the CPU (fp32 arithmetic, bf16 rounding at the
# path's points) at the LLaMA-8B layer shapes of test_bf16_real_layer_shapes_matches_oracle: it
# puts wq / wk at 2.35 % against this reference while every other tensor stays below 2 %, and
# below 2 % too once q, k and v are kept in fp32. These tensors are held to 3e-2; every other
# tensor keeps 2e-2.
SCORE_INPUTS = ("wq", "wk", "attn_norm")


def bf16_weights(params):
    """The low-precision copy the bf16 path computes with: matrices rounded to bf16 (RNE), norm
    gains and the embedding rows (gathered from the fp32 masters) unchanged."""
    return {n: (OA.bf16_to_f32(OA.bf16_round(v)).reshape(v.shape) if v.ndim >= 2 and n != "embed" else v)
            for n, v in params.items()}


def _bf16_parity(w, k=None, std=0.02):
    params = W.make_params(w, threads=16, std=std)
    batch = W.make_batch(w)
    ref_loss, ref_G = oracle_fb(w, bf16_weights(params), batch, dtype=np.float32)
    full_loss, _ = oracle_fb(w, params, batch, dtype=np.float32) if w.shape.n_layers <= 3 else (ref_loss, None)
    with lib_model(w, params, k=k) as m:
        loss = lib_fb(m, w, batch)
        st = m.stats()
        errs = {n: rel_l2(m.get_grad(n), g) for n, g in ref_G.items()}
    worst = sorted(errs.items(), key=lambda x: -x[1])[:6]
    print(w.name, "loss", loss, ref_loss, "fp32-weight oracle loss", full_loss, "worst grads", worst, st)
    assert abs(loss - ref_loss) <= 1e-2 * abs(ref_loss)
    assert abs(loss - full_loss) <= 1e-2 * abs(full_loss)
    for n, e in errs.items():
        bound = 3e-2 if n.split(".")[-1] in SCORE_INPUTS else 2e-2
        assert e <= bound, (n, e)


def test_bf16_small_matches_oracle():
    _bf16_parity(BF16_SMALL)


@pytest.mark.parametrize("name", ["qwen3_1p7b", "llama8b"])
def test_bf16_real_layer_shapes_matches_oracle(name):
    """The real layer, head and vocabulary shapes with 2 layers and 2 x 256 tokens (the oracle
    must finish in seconds); every kernel runs in the tile configuration of the full workload."""
    w = W.WORKLOADS[name].with_(batch=2, seq=256, n_micro=2).with_shape(n_layers=2)
    _bf16_parity(w, k=1)


def _state(m):
    return {n: (m.get_tensor(n), *m.get_adam_state(n)[:2]) for n in m.index}


@pytest.mark.parametrize("wname", ["tiny", "bf16_small"])
def test_fused_forward_backward_step_is_bitwise_fb_then_step(wname):
    w = TINY if wname == "tiny" else BF16_SMALL
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    with lib_model(w, params) as a, lib_model(w, params) as b:
        for it in range(2):
            la = lib_fb(a, w, batch)
            a.step()
            lb = b.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
            assert la == lb, (it, la, lb)
        sa, sb = _state(a), _state(b)
        for n in sa:
            for x, y in zip(sa[n], sb[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n
        # with gradients already accumulated the fused call is the plain sequence
        lib_fb(a, w, batch); lib_fb(a, w, batch); a.step()
        lib_fb(b, w, batch); b.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        sa, sb = _state(a), _state(b)
        for n in sa:
            for x, y in zip(sa[n], sb[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n
            assert not np.any(b.get_grad(n))


@pytest.mark.parametrize("wname", ["tiny", "bf16_small"])
def test_results_independent_of_weight_slots_and_grad_buffers_bitwise(wname):
    """The weight ring depth and the number of gradient buffers only change when copies run:
    two fused steps give the same loss, weights and Adam moments bit for bit."""
    w = TINY if wname == "tiny" else BF16_SMALL
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    runs = []
    for slots, gbufs in ((2, 2), (3, 4), (8, 3), (0, 0)):
        with lib_model(w, params, slots=slots, gbufs=gbufs) as m:
            losses = [m.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True) for _ in range(2)]
            st = m.stats()
            runs.append((losses, _state(m), st["n_weight_streams"]))
    print(wname, "weight streams per call by ring depth", [r[2] for r in runs])
    for losses, state, _ in runs[1:]:
        assert losses == runs[0][0]
        for n in state:
            for x, y in zip(state[n], runs[0][1][n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n


@pytest.mark.parametrize("wname", ["tiny", "bf16_small", "bf16_big_head"])
def test_pinned_ring_gives_identical_results_bitwise(wname):
    """A pinned budget below the image size keeps the image pageable and stages every weight copy
    through a ring of pinned segments of one layer block each (the LM head in pieces): two fused
    steps and a plain forward_backward + step give the same losses, weights and Adam moments bit
    for bit as the fully pinned image, and every streamed weight byte went through the ring."""
    # (bf16_big_head: a vocabulary of 8000 makes the LM-head block larger than a layer block, so
    # the head goes through the ring in pieces)
    w = {"tiny": TINY, "bf16_small": BF16_SMALL, "bf16_big_head": BF16_SMALL.with_shape(vocab=8000)}[wname]
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)

    def run(budget):
        with lib_model(w, params, pinned_budget=budget) as m:
            losses, stats = [], []
            for _ in range(2):
                losses.append(m.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True))
                stats.append(m.stats())
            losses.append(lib_fb(m, w, batch))
            stats.append(m.stats())
            m.step()
            return losses, _state(m), stats

    ref_losses, ref_state, st0 = run(0)
    assert all(st["ring_segments"] == 0 and st["staged_bytes"] == 0 for st in st0)
    seg = -(-st0[0]["layer_image_bytes"] // 4096) * 4096
    print(wname, "layer block", st0[0]["layer_image_bytes"], "head block", st0[0]["head_image_bytes"], "segment", seg)
    if wname == "bf16_big_head":
        assert st0[0]["head_image_bytes"] > 2 * seg
    for nseg, budget in ((2, 2 * seg), (3, 3 * seg + 4095)):
        losses, state, stats = run(budget)
        assert all(st["ring_segments"] == nseg and st["ring_segment_bytes"] == seg for st in stats)
        # every layer copy a call queues is staged (a fused call also stages the next call's head
        # and first layers, which that call then does not copy again)
        for st in stats:
            assert st["staged_bytes"] >= st["n_weight_streams"] * st["layer_image_bytes"], st
        assert stats[0]["staged_bytes"] > 0
        assert losses == ref_losses
        for n in state:
            for x, y in zip(state[n], ref_state[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n


def test_pinned_budget_rejections():
    """A budget below two ring segments, or the ring together with the asynchronous optimiser's
    second image, is HOL_EINVAL at create time."""
    w = TINY
    params = W.make_params(w, threads=8)
    with lib_model(w, params) as m:
        m.forward_backward(w.n_micro, tokens=W.make_batch(w)["tokens"])
        seg = -(-m.stats()["layer_image_bytes"] // 4096) * 4096
    for kw in (dict(pinned_budget=seg + 4096), dict(pinned_budget=2 * seg, async_opt=1)):
        with pytest.raises(hol.HolError) as e:
            lib_model(w, params, **kw)
        assert e.value.status == hol.HOL_EINVAL, kw


@pytest.mark.parametrize("wname", ["tiny", "bf16_small"])
def test_plain_step_after_fused_step_sees_zero_gradients(wname):
    """After a fused step the gradient blocks read as zero: a following plain step() is Adam on
    zero gradients, bit for bit the same as on a model whose gradients were zeroed explicitly."""
    w = TINY if wname == "tiny" else BF16_SMALL
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    with lib_model(w, params) as a, lib_model(w, params) as b:
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        lib_fb(b, w, batch)
        b.step()
        b.zero_grad()
        for n in a.index:
            assert not np.any(a.get_grad(n)), n
        a.step()
        b.step()
        sa, sb = _state(a), _state(b)
        for n in sa:
            for x, y in zip(sa[n], sb[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n
        # and a plain forward_backward after a fused step accumulates from zero
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        b.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        la = lib_fb(a, w, batch)
        lb = lib_fb(b, w, batch)
        assert la == lb
        for n in a.index:
            assert np.array_equal(a.get_grad(n).view(np.uint32), b.get_grad(n).view(np.uint32)), n


@pytest.mark.parametrize("wname", ["tiny", "bf16_small"])
def test_head_weights_sent_ahead_by_a_fused_step_follow_later_writes(wname):
    """A fused step sends the next call's LM-head weights to the device during its own backward.
    A later write of the head (hol_set_tensor, or a plain hol_step) must be what the next call
    computes with: bit for bit the same as a model that never had the weights sent ahead."""
    w = TINY if wname == "tiny" else BF16_SMALL
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    with lib_model(w, params) as a, lib_model(w, params) as b:
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)   # sends the head ahead
        lib_fb(b, w, batch)
        b.step()
        new_head = a.get_tensor("lm_head") * np.float32(1.5)
        a.set_tensor("lm_head", new_head)
        b.set_tensor("lm_head", new_head)
        assert lib_fb(a, w, batch) == lib_fb(b, w, batch)
        for n in a.index:
            assert np.array_equal(a.get_grad(n).view(np.uint32), b.get_grad(n).view(np.uint32)), n
        a.zero_grad()
        b.zero_grad()
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)   # sends the head ahead
        a.step()                                                               # then changes it
        lib_fb(b, w, batch)
        b.step()
        b.step()
        assert lib_fb(a, w, batch) == lib_fb(b, w, batch)
        sa, sb = _state(a), _state(b)
        for n in sa:
            for x, y in zip(sa[n], sb[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n


@pytest.mark.parametrize("wname", ["tiny", "bf16_small"])
def test_first_layers_sent_ahead_by_a_fused_step_follow_later_writes(wname):
    """A fused step sends the next call's first layers (the backward's last, updated last) into
    weight slots before it returns. A later write of them (hol_set_tensor, a plain hol_step)
    must be what the next call computes with, and a staleness-1 call after a fused step computes
    with the image it finds: bit for bit the same as a model that never sent the layer ahead."""
    w = TINY if wname == "tiny" else BF16_SMALL
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    with lib_model(w, params) as a, lib_model(w, params) as b:
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)   # sends layer 0 ahead
        lib_fb(b, w, batch)
        b.step()
        for n in ("layers.0.wq", "layers.0.attn_norm", "layers.1.wo", "layers.2.mlp_norm"):
            new = a.get_tensor(n) * np.float32(1.25)
            a.set_tensor(n, new)
            b.set_tensor(n, new)
        assert lib_fb(a, w, batch) == lib_fb(b, w, batch)
        for n in a.index:
            assert np.array_equal(a.get_grad(n).view(np.uint32), b.get_grad(n).view(np.uint32)), n
        a.zero_grad()
        b.zero_grad()
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)   # sends layer 0 ahead
        a.step()                                                               # then changes it
        lib_fb(b, w, batch)
        b.step()
        b.step()
        assert lib_fb(a, w, batch) == lib_fb(b, w, batch)
        sa, sb = _state(a), _state(b)
        for n in sa:
            for x, y in zip(sa[n], sb[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n
    with lib_model(w, params, async_opt=1) as a, lib_model(w, params, async_opt=1) as b:
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)   # sends layer 0 ahead
        lib_fb(b, w, batch)
        b.step()
        for _ in range(2):   # the second call finds the other image buffer
            assert (a.forward_backward(w.n_micro, tokens=batch["tokens"], stale_step=True) ==
                    b.forward_backward(w.n_micro, tokens=batch["tokens"], stale_step=True))
        a.step()
        b.step()
        assert (a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True) ==
                b.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True))
        sa, sb = _state(a), _state(b)
        for n in sa:
            for x, y in zip(sa[n], sb[n]):
                assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), n


@pytest.mark.parametrize("slots", [0, 2])
@pytest.mark.parametrize("wname", ["tiny", "bf16_small"])
def test_first_layers_sent_ahead_are_not_copied_again(wname, slots):
    """The copies a fused step sends ahead are really used: the next call streams fewer layers
    (h2d_span_bytes counts the copies a call makes for itself), by whole layer images; once those
    layers are written (hol_set_tensor, or a plain hol_step) the next call copies them again.
    Also with the two-slot ring."""
    w = TINY if wname == "tiny" else BF16_SMALL
    params = W.make_params(w, threads=8)
    batch = W.make_batch(w)
    L = w.shape.n_layers
    with lib_model(w, params, slots=slots) as a, lib_model(w, params, slots=slots) as b:
        lib_fb(b, w, batch)
        fresh = b.stats()
        lb, hb = fresh["layer_image_bytes"], fresh["head_image_bytes"]

        def kept_layers(st, head_kept=True):
            diff = fresh["h2d_span_bytes"] - st["h2d_span_bytes"]
            n, rest = divmod(diff - (hb if head_kept else 0), lb)   # the head weights are sent ahead too
            assert rest == 0 and n >= 0, (diff, lb, hb)
            assert fresh["n_weight_streams"] - st["n_weight_streams"] == n
            return n

        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        lib_fb(a, w, batch)
        n = kept_layers(a.stats())
        print(wname, "slots", slots, "layers kept from the previous call", n)
        assert 1 <= n <= L
        # a write of layer 0 (the last layer the fused step updates, always among those sent): that
        # one layer is copied again
        a.zero_grad()
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        a.set_tensor("layers.0.wq", a.get_tensor("layers.0.wq"))
        lib_fb(a, w, batch)
        assert kept_layers(a.stats()) == n - 1
        # writes of every layer: none is kept
        a.zero_grad()
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        for l in range(L):
            a.set_tensor(f"layers.{l}.mlp_norm", a.get_tensor(f"layers.{l}.mlp_norm"))
        lib_fb(a, w, batch)
        assert kept_layers(a.stats()) == 0
        # a plain step after the fused one rewrites every layer image
        a.zero_grad()
        a.forward_backward(w.n_micro, tokens=batch["tokens"], and_step=True)
        a.step()
        lib_fb(a, w, batch)
        assert kept_layers(a.stats(), head_kept=False) == 0
