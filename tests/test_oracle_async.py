"""Pins of the staleness-1 schedule oracle (oracle/async_opt.py) to facts outside it.

* Delayed gradient descent on f(x) = a x^2 / 2: the schedule must reproduce the closed-form
  solution of x_t = x_{t-1} - c x_{t-2} (c = eta a, x_{-1} = x_0), real and complex roots,
  including a step size where the synchronous iteration converges and the delayed one diverges.
* Gradients that do not depend on the parameters: staleness changes nothing, so after the final
  step the state equals the synchronous sequence bit for bit (no gradient dropped, repeated or
  reordered).
* The decoder binding: the first two calls both see theta_0, the third sees the parameters after
  exactly one Adam step on the first call's gradient (and not on the second's).
"""
import numpy as np
import pytest

import workloads as W
from oracle import adam as OA
from oracle import async_opt as AO
from oracle import decoder as D


def _closed_form(c: float, n: int) -> np.ndarray:
    """y_k = x_{k-1} for k = 0..n with y_0 = y_1 = 1 and y_k = y_{k-1} - c y_{k-2}."""
    disc = np.sqrt(complex(1.0 - 4.0 * c))
    r1, r2 = (1 + disc) / 2, (1 - disc) / 2
    alpha, beta = (1 - r2) / (r1 - r2), (r1 - 1) / (r1 - r2)
    k = np.arange(n + 1)
    y = alpha * r1 ** k + beta * r2 ** k
    assert np.max(np.abs(y.imag)) < 1e-9
    return y.real


@pytest.mark.parametrize("a,eta", [(2.0, 0.05), (1.0, 0.5), (3.0, 0.5)])
def test_delayed_gradient_descent_closed_form(a, eta):
    n = 24
    st = {"x": 1.0, "trace": []}

    def grad_fn(t, s):
        return 0.5 * a * s["x"] ** 2, a * s["x"]

    def update_fn(s, g):
        s["x"] = s["x"] - eta * g
        s["trace"].append(s["x"])

    losses, grads = AO.run_stale1(st, grad_fn, update_fn, n)
    y = _closed_form(eta * a, n + 1)
    # call t evaluates at x_{t-1} (x_{-1} = x_0): its gradient is a y_t
    assert np.allclose(grads, a * y[:n], rtol=1e-12, atol=1e-12)
    # parameters after update t: x_t = y_{t+1}, the last one from the final step
    assert np.allclose(st["trace"], y[2:n + 2], rtol=1e-12, atol=1e-12)
    if eta * a == 1.5:
        # synchronous descent contracts by |1 - c| = 0.5 per step; the delayed one grows by
        # sqrt(c) > 1 in modulus
        assert abs(st["x"]) > 10.0 and abs((1 - eta * a) ** n) < 1e-6


def test_without_final_step_one_update_is_pending():
    st = {"x": 1.0, "n": 0}
    AO.run_stale1(st, lambda t, s: (0.0, 1.0), lambda s, g: s.update(x=s["x"] - g, n=s["n"] + 1), 5,
                  flush=False)
    assert st["n"] == 4 and st["x"] == -3.0


def test_parameter_free_gradients_equal_the_synchronous_sequence():
    rng = np.random.default_rng(7)
    gs = [rng.standard_normal(33).astype(np.float32) for _ in range(6)]
    theta0 = rng.standard_normal(33).astype(np.float32)

    def fresh():
        return {"th": theta0.copy(), "m": np.zeros(33, np.float32), "v": np.zeros(33, np.float32), "t": 0}

    def update_fn(s, g):
        s["t"] += 1
        OA.adam_update(s["th"], g, s["m"], s["v"], s["t"], lr=1e-2)

    a = fresh()
    AO.run_stale1(a, lambda t, s: (0.0, gs[t]), update_fn, len(gs))
    b = fresh()
    for g in gs:
        update_fn(b, g)
    assert a["t"] == b["t"] == len(gs)
    for k in ("th", "m", "v"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


def test_decoder_binding_sees_parameters_one_update_behind():
    w = W.WORKLOADS["tiny"].with_shape(n_layers=2)
    s = D.Shape.of(w.shape)
    params = W.make_params(w, threads=2)
    batches = [W.make_batch(w.with_(token_seed=w.token_seed + i)) for i in range(3)]
    lr = 1e-2
    losses, grads, st = AO.decoder_stale1(params, s, batches, w.n_micro, lr, 0.9, 0.999, 1e-8)

    def fb(P, b):
        Pd = {n: v.astype(np.float64) for n, v in P.items()}
        G = D.zero_grads(Pd, s)
        loss = D.forward_backward(Pd, s, G, w.n_micro, tokens=b["tokens"], loss="ce")
        return loss, G

    l0, g0 = fb(params, batches[0])
    l1, _ = fb(params, batches[1])
    assert losses[0] == l0 and losses[1] == l1            # both at theta_0
    theta1 = {n: v.astype(np.float32).copy() for n, v in params.items()}
    m = {n: np.zeros_like(v) for n, v in theta1.items()}
    v = {n: np.zeros_like(x) for n, x in theta1.items()}
    for n in g0:
        OA.adam_update(theta1[n], g0[n].astype(np.float32), m[n], v[n], 1, lr=lr)
    l2, _ = fb(theta1, batches[2])
    assert losses[2] == l2                               # one step, on call 0's gradient
    assert st["t"] == 3
    assert losses[2] != fb(params, batches[2])[0]         # the step changed what call 2 sees
