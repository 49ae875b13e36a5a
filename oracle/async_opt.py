"""Oracle (test infrastructure only): training with the staleness-1 asynchronous optimiser.

Nothing in the product path may import this module; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP library.

RoundPipe paper summary, 异步优化器 (Asynchronous Optimizer) and 方法步骤详情 step 6: the host
optimiser step for one iteration's gradients runs while the GPU already computes the next
iteration, which does not wait for that step; the next iteration therefore sees the parameters
from before the step ("staleness 1", one update behind).

Reading (the pages give no formula). With theta_0 the parameters before the first call, g_t the
gradient of call t's batch (t = 1, 2, ...) and Update the synchronous optimiser step:

    g_t     = grad L_t(theta_{t-2})          (theta_{-1} = theta_0)
    theta_t = Update(theta_{t-1}, g_t)       (run while call t + 1 computes, or by a final
                                              synchronous step)

so every call evaluates its gradient at the parameters as they stand when the call starts and
applies the previous call's gradient while it runs; the first call applies nothing. For
f(x) = a x^2 / 2 with plain gradient descent this is the delayed recursion
x_t = x_{t-1} - eta a x_{t-2}, whose closed form pins ``run_stale1`` in
``tests/test_oracle_async.py``.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Tuple

import numpy as np

from . import adam as A
from . import decoder as D


def run_stale1(state, grad_fn: Callable, update_fn: Callable, n_calls: int, flush: bool = True):
    """Generic staleness-1 schedule.

    ``grad_fn(t, state) -> (loss, g)`` evaluates call t (0-based) at the current parameters held in
    ``state``; ``update_fn(state, g)`` applies one optimiser step to ``state`` in place. Returns the
    per-call losses and gradients; with ``flush`` the last call's gradient is applied at the end
    (the synchronous step that completes the sequence).
    """
    losses: List[float] = []
    grads: List[object] = []
    pending = None
    for t in range(n_calls):
        loss, g = grad_fn(t, state)          # at the parameters as the call finds them
        if pending is not None:
            update_fn(state, pending)        # the previous call's step, overlapped with this call
        pending = g
        losses.append(loss)
        grads.append(g)
    if flush and pending is not None:
        update_fn(state, pending)
    return losses, grads


def decoder_stale1(P: Dict[str, np.ndarray], s: D.Shape, batches: List[dict], n_micro: int,
                   lr: float, b1: float, b2: float, eps: float, fb_dtype=np.float64,
                   flush: bool = True) -> Tuple[List[float], List[Dict[str, np.ndarray]], dict]:
    """The decoder trained with Adam under the staleness-1 schedule.

    ``P`` holds float32 masters (copied, not modified). Each call's forward and backward run in
    ``fb_dtype`` on the masters as the call finds them; the Adam step is the float32 host update
    of ``oracle.adam``. ``batches[t]`` holds ``tokens`` (cross entropy) or ``hidden`` (sum of
    squares). Returns (losses, gradients per call, final state dict with ``P``, ``m``, ``v``,
    ``t``).
    """
    names = D.trainable_names(s, P.keys())
    st = {"P": {n: np.array(v, np.float32, copy=True) for n, v in P.items()},
          "m": {n: np.zeros_like(P[n], np.float32) for n in names},
          "v": {n: np.zeros_like(P[n], np.float32) for n in names},
          "t": 0}

    def grad_fn(t, state):
        Pw = {n: v.astype(fb_dtype) for n, v in state["P"].items()}
        G = D.zero_grads(Pw, s)
        b = batches[t]
        if "tokens" in b:
            loss = D.forward_backward(Pw, s, G, n_micro, tokens=b["tokens"], loss="ce")
        else:
            loss = D.forward_backward(Pw, s, G, n_micro, hidden=b["hidden"].astype(fb_dtype), loss="sumsq")
        return loss, {n: g.astype(np.float32) for n, g in G.items()}

    def update_fn(state, g):
        state["t"] += 1
        for n in names:
            A.adam_update(state["P"][n], g[n], state["m"][n], state["v"][n], state["t"], lr=lr, b1=b1, b2=b2,
                          eps=eps)

    losses, grads = run_stale1(st, grad_fn, update_fn, len(batches), flush=flush)
    return losses, grads, st
