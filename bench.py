"""Benchmark: layer-streamed training throughput on one MI355X.

One step = hol_forward_backward_step over one batch: every row of the hot path (weight streaming,
template kernels, checkpoint/recompute, gradient offload) and the host Adam step with the bf16
refresh, each layer's Adam overlapped with the remaining backward (same result as
hol_forward_backward followed by hol_step). Default workload: LLaMA-3.1-8B-shaped decoder, 4 micro-batches of one 4096-token
sequence, K = 4, bf16 compute with fp32 host masters; seeded synthetic weights N(0, 0.02) and
uniform random tokens.

Prints ONE JSON line. Extra fields: fb-only throughput, host step time, H2D/D2H rates against the
measured pinned-copy peak, per-kernel-class rates, the end-to-end per-layer roofline, and the
oracle's CPU baseline on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
METRIC = "train tokens/sec on 1 MI355X (8B-shape, seq 4K); MFMA util; H2D GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def link_peak_gbs(torch, nbytes=1 << 30, reps=4):
    """Pinned hipMemcpyAsync H2D and D2H peak (GB/s) through torch's copy engine path."""
    h = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(reps):
        d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    h2d = reps * nbytes / (time.perf_counter() - t) / 1e9
    t = time.perf_counter()
    for _ in range(reps):
        h.copy_(d, non_blocking=True)
    torch.cuda.synchronize()
    d2h = reps * nbytes / (time.perf_counter() - t) / 1e9
    del h, d
    return h2d, d2h


def link_sweep(torch, sizes_mb=(4, 16, 64, 256, 1024), budget_s=0.15):
    """Pinned hipMemcpyAsync rates (GB/s) by copy size: H2D alone, D2H alone, and both directions
    at once on two streams (each direction's rate and their sum)."""
    out = {"sizes_mb": list(sizes_mb), "h2d": [], "d2h": [], "bidir_h2d": [], "bidir_d2h": [], "bidir_total": []}
    big = max(sizes_mb) << 20
    h_up = torch.empty(big, dtype=torch.uint8).pin_memory()
    h_dn = torch.empty(big, dtype=torch.uint8).pin_memory()
    d_up = torch.empty(big, dtype=torch.uint8, device="cuda")
    d_dn = torch.empty(big, dtype=torch.uint8, device="cuda")
    s_up, s_dn = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps

    for mb in sizes_mb:
        n = mb << 20
        reps = max(2, int(budget_s * 50e9 / n))
        up = lambda: d_up[:n].copy_(h_up[:n], non_blocking=True)
        dn = lambda: h_dn[:n].copy_(d_dn[:n], non_blocking=True)

        def both():
            with torch.cuda.stream(s_up):
                d_up[:n].copy_(h_up[:n], non_blocking=True)
            with torch.cuda.stream(s_dn):
                h_dn[:n].copy_(d_dn[:n], non_blocking=True)

        t_up, t_dn = timed(up, reps), timed(dn, reps)
        # both directions at once: each stream's own span from events
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        both()
        torch.cuda.synchronize()
        e[0].record(s_up); e[2].record(s_dn)
        for _ in range(reps):
            both()
        e[1].record(s_up); e[3].record(s_dn)
        torch.cuda.synchronize()
        tb_up, tb_dn = e[0].elapsed_time(e[1]) / 1e3 / reps, e[2].elapsed_time(e[3]) / 1e3 / reps
        out["h2d"].append(round(n / t_up / 1e9, 1))
        out["d2h"].append(round(n / t_dn / 1e9, 1))
        out["bidir_h2d"].append(round(n / tb_up / 1e9, 1))
        out["bidir_d2h"].append(round(n / tb_dn / 1e9, 1))
        out["bidir_total"].append(round(2 * n / max(tb_up, tb_dn) / 1e9, 1))
    del h_up, h_dn, d_up, d_dn
    return out


def gemm_roles(w: W.Workload):
    """Names of the decoder GEMM shapes (M, N, K) of one call by the step they belong to."""
    s = w.shape
    T, H, d = w.tokens, s.hidden, s.head_dim
    nqd, QKV, F = s.n_q_heads * d, (s.n_q_heads + 2 * s.n_kv_heads) * d, s.ffn
    roles = {}

    def add(shape, name):
        roles[shape] = roles[shape] + " = " + name if shape in roles else name

    if not s.n_experts:
        add((T, QKV, H), "a4 qkv fwd"); add((T, H, nqd), "a7 o fwd"); add((T, 2 * F, H), "a9 gate/up fwd")
        add((T, H, F), "a10 down fwd")
        add((T, H, QKV), "a4 qkv dX"); add((T, nqd, H), "a7 o dX"); add((T, H, 2 * F), "a9 gate/up dX")
        add((T, F, H), "a10 down dX")
        add((QKV, H, T), "a4 qkv dW"); add((H, nqd, T), "a7 o dW"); add((2 * F, H, T), "a9 gate/up dW")
        add((H, F, T), "a10 down dW")
    return roles


def gemm_table(w: W.Workload, st_list, steps):
    """Per-shape GEMM rates of the timed steps, labelled by row of the hot path."""
    roles = gemm_roles(w)
    V = w.shape.vocab
    acc = {}
    for st in st_list:
        for M, N, K, n, ms, fl in st.get("gemm_shapes", []):
            a = acc.setdefault((M, N, K), [0, 0.0, 0.0])
            a[0] += n; a[1] += ms; a[2] += fl
    rows = []
    for (M, N, K), (n, ms, fl) in sorted(acc.items(), key=lambda kv: -kv[1][1]):
        if (M, N, K) in roles:
            name = roles[(M, N, K)]
        elif V and N == V:
            name = "a13 head fwd"
        elif V and K == V:
            name = "a13 head dX"
        elif V and M == V:
            name = "a13 head dW"
        else:
            name = "other"
        rows.append({"gemm": name, "M": M, "N": N, "K": K, "launches_per_step": n // steps,
                     "avg_us": round(1e3 * ms / n, 1), "tflops": round(fl / ms / 1e9, 1),
                     "frac": round(fl / ms / 1e9 / BF16_PEAK_TFLOPS, 4)})
    return rows


def gemm_shapes_alone(torch, hol, w: W.Workload, reps: int):
    """The workload's decoder GEMMs one shape at a time, as the step launches them: fp32 out;
    bf16 out for the down-projection and o data gradients; residual epilogue for the o and down
    projections; the q/k/v forward with its RoPE epilogue (hol_op_gemm_rope, bf16 out); the
    gate/up forward with its SwiGLU epilogue (hol_op_gemm_swiglu); the weight gradients with the
    split-tail workspace (hol_op_gemm_ws), the o and q/k/v ones reading both operands K-major as
    the step does (the others over transposed copies, NT). In the order listed, `reps` launches
    each after one warm-up launch; before the first shape, half a second of its launches brings
    the device clocks to their loaded steady state (timed from an idle device, the first shape
    read 15-20 % slow)."""
    s = w.shape
    T, H, d = w.tokens, s.hidden, s.head_dim
    nqd, QKV, F = s.n_q_heads * d, (s.n_q_heads + 2 * s.n_kv_heads) * d, s.ffn
    # (name, M, N, K, epilogue, bf16 output)
    shapes = [("a4 qkv fwd", T, QKV, H, 0, False), ("a7 o fwd", T, H, nqd, 2, False),
              ("a9 gate/up fwd", T, 2 * F, H, 0, True), ("a10 down fwd", T, H, F, 2, False),
              ("a10 down dX", T, F, H, 0, True), ("a9 gate/up dX", T, H, 2 * F, 0, False),
              ("a7 o dX", T, nqd, H, 0, True), ("a4 qkv dX", T, H, QKV, 0, False),
              ("a10 down dW", H, F, T, 0, False), ("a9 gate/up dW", 2 * F, H, T, 0, False),
              ("a7 o dW", H, nqd, T, 0, False), ("a4 qkv dW", QKV, H, T, 0, False)]
    stream = torch.cuda.current_stream()
    wsn = hol.lib.hol_op_gemm_workspace_floats()
    ws = torch.empty((wsn,), device="cuda")
    S, n_rot = w.seq, (s.n_q_heads + s.n_kv_heads) * d
    cos_t = torch.rand((S, d // 2), device="cuda")
    sin_t = torch.rand((S, d // 2), device="cuda")
    rows = []
    for name, M, N, K, epi, bf in shapes:
        km = name in ("a7 o dW", "a4 qkv dW")  # both operands K-major ([K][M], [K][N])
        dw = name.endswith("dW")
        # (the step's NT weight gradients read transposed copies whose rows are padded: K rounded
        # up to 8, plus 64)
        lda = ldb = (K + 7) // 8 * 8 + 64 if dw else K
        if km:
            lda, ldb = M, N
        a = torch.randn((K, M) if km else (M, lda), device="cuda").to(torch.bfloat16)
        b = torch.randn((K, N) if km else (N, ldb), device="cuda").to(torch.bfloat16)
        rope = name == "a4 qkv fwd" and d == 128
        c = torch.empty((M, N), device="cuda", dtype=torch.bfloat16 if (bf or rope) else torch.float32)
        r = torch.randn((M, N), device="cuda") if epi == 2 else None
        act = torch.empty((M, N // 2), device="cuda", dtype=torch.bfloat16) if name.startswith("a9 gate/up fwd") else None

        def launch():
            if act is not None:
                hol.check(hol.lib.hol_op_gemm_swiglu(M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N,
                                                     act.data_ptr(), N // 2, hol.BF16, stream.cuda_stream))
                return
            if rope:
                hol.check(hol.lib.hol_op_gemm_rope(M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N, n_rot, S,
                                                   cos_t.data_ptr(), sin_t.data_ptr(), stream.cuda_stream))
                return
            hol.check(hol.lib.hol_op_gemm_ws(M, N, K, a.data_ptr(), lda, int(km), b.data_ptr(), ldb, int(km),
                                             c.data_ptr(), N, r.data_ptr() if r is not None else None, N, hol.BF16,
                                             hol.BF16 if bf else hol.F32, epi, 1.0,
                                             ws.data_ptr() if dw else None, wsn if dw else 0, stream.cuda_stream))

        launch()
        if not rows:
            t_end = time.perf_counter() + 0.5
            while time.perf_counter() < t_end:
                for _ in range(5):
                    launch()
                torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record(stream)
            launch()
            ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        us = 1e3 * float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)]))
        tf = 2.0 * M * N * K / us / 1e6
        rows.append({"gemm": name, "M": M, "N": N, "K": K, "avg_us": round(us, 1), "tflops": round(tf, 1),
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        log(f"[bench] {name:16s} {M:6d} x {N:6d} x {K:6d}: {us:8.1f} us {tf:7.1f} TFLOP/s")
        del a, b, c, r, act
    return {"workload": w.name, "gemm_shapes_alone": rows, "launches_per_shape": reps}


def algorithmic(w: W.Workload, n_streams: int, layer_bytes: int, head_bytes: int):
    """Algorithmic FLOPs and streamed bytes of one forward_backward (recompute included)."""
    s = w.shape
    H, d, nq, nkv, F, V = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads, s.ffn, s.vocab
    T, S, M = w.tokens, w.seq, w.batch
    p_attn = H * (nq * d) * 2 + H * (nkv * d) * 2
    # parameters a token passes through: dense MLP, or the router plus its top_k experts
    p_mlp = s.n_experts * H + s.top_k * 3 * H * s.expert_ffn if s.n_experts else 3 * H * F
    p_layer = p_attn + p_mlp
    attn_fwd = 2.0 * d * nq * S * (S + 1) * M
    L, K = s.n_layers, w.ckpt_every_k
    n_recomp = L - (L - ((L + K - 1) // K - 1) * K)          # every block but the last is recomputed
    f_fwd = 2.0 * p_layer * T + attn_fwd
    # backward: dX, plus dW unless the base is frozen (LoRA adapters are negligible); attention 2.5x
    f_bwd = (1 if s.lora_rank else 2) * (2.0 * p_layer * T) + 2.5 * attn_fwd
    # a recomputed block's last layer skips the product that forms its output (dense: the down
    # projection; the next block restarts from its stored checkpoint)
    n_blocks_recomp = (L + K - 1) // K - 1
    f_skip = 0.0 if s.n_experts else n_blocks_recomp * 2.0 * H * F * T
    f_layers = L * (f_fwd + f_bwd) + n_recomp * f_fwd - f_skip
    f_head = 3 * 2.0 * H * V * T
    return dict(p_layer=p_layer, f_layer=f_layers / L, f_head=f_head, n_recomp=n_recomp,
                flops=f_layers + f_head,
                h2d=n_streams * layer_bytes + head_bytes + 4.0 * T * H)


def profiled_traffic(workload: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, or None when
    there is none for this workload or the GEMM source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and " " not in l.strip())
    src = os.path.join(ROOT, "host_offloaded_layer_amd", "csrc", "k_gemm.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != kv.get("k_gemm_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_baseline(w: W.Workload):
    """The oracle (NumPy fp32) on a bounded sample of the same workload: one decoder layer's
    forward, recompute and backward on one 4096-token sequence, the loss anchor on 512 tokens, and
    Adam on 2^24 parameters; scaled to one step of the full workload."""
    from oracle import adam as OA
    from oracle import decoder as D
    s = D.Shape.of(w.shape)
    # one sequence of at most 4096 tokens (2048 with experts); the layer time is scaled by tokens
    S = min(w.seq, 2048 if s.n_experts else 4096)
    one = w.with_shape(n_layers=1).with_(batch=1, seq=S, n_micro=1)
    P = W.make_params(one)
    cos, sin = D.rope_tables(S, s.head_dim, s.rope_base, np.float32)
    if s.vocab:
        tok = W.make_tokens(one)
        h = P["embed"][tok.reshape(-1)]
    else:
        h = W.make_hidden(one).reshape(S, -1)
    G = D.zero_grads(P, s)
    t0 = time.perf_counter()
    out, _ = D.layer_forward(P, 0, h, s, 1, cos, sin)
    _, c = D.layer_forward(P, 0, h, s, 1, cos, sin)
    D.layer_backward(P, 0, c, np.ones_like(out) * 1e-3, s, 1, cos, sin, G)
    t_layer = time.perf_counter() - t0
    del c
    n_head, t_head = min(512, S - 1), 0.0
    if s.vocab:
        z = h[:n_head]
        t0 = time.perf_counter()
        zz, rz = D.rmsnorm(z, P["final_norm"], s.rms_eps)
        logits = zz @ P["lm_head"].T
        lab = tok.reshape(-1)[1:n_head + 1]
        _, dl = D.cross_entropy(logits, lab)
        dz = dl @ P["lm_head"]
        if "lm_head" in G:
            G["lm_head"] += dl.T @ zz
        D.rmsnorm_bwd(dz, z, P["final_norm"], rz)
        t_head = time.perf_counter() - t0
    n_adam = 1 << 24
    th = np.random.default_rng(0).standard_normal(n_adam, dtype=np.float32)
    g = th * 1e-3
    mm = np.zeros_like(th)
    vv = np.zeros_like(th)
    t0 = time.perf_counter()
    OA.adam_update(th, g, mm, vv, 1)
    t_adam = time.perf_counter() - t0
    total_params = sum(int(np.prod(p.shape)) for p in W.param_specs(w.shape) if p.trainable)
    t_step = (w.tokens / S * s.n_layers * t_layer + (w.tokens / n_head * t_head if s.vocab else 0.0)
              + total_params / n_adam * t_adam)
    try:
        import threadpoolctl
        cores = max(x.get("num_threads", 1) for x in threadpoolctl.threadpool_info())
    except Exception:
        cores = os.cpu_count()
    return {"value": w.tokens / t_step, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"NumPy fp32 oracle: 1 layer fwd+recompute+bwd on 1x{S} tokens ({t_layer:.2f} s), "
                       + (f"loss anchor on {n_head} tokens ({t_head:.2f} s), " if s.vocab else "")
                       + f"Adam on 2^24 params ({t_adam:.2f} s); scaled linearly to {w.tokens} tokens x "
                       f"{s.n_layers} layers" + (f", {w.tokens} head tokens" if s.vocab else "")
                       + f", {total_params} trainable params: {t_step:.1f} s/step")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "qwen3_1p7b", "llama8b_16k", "qwen3_235b_slice", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--optimizer", choices=["sync", "async"], default="sync",
                    help="sync: hol_forward_backward_step (the default, the synchronous step); async: "
                         "hol_forward_backward_async, the staleness-1 optimiser (each call applies the "
                         "previous call's update on host threads while it computes)")
    ap.add_argument("--pinned-budget-gb", type=float, default=0.0,
                    help="pinned host memory the weight image may use (GB); below the image size the "
                         "image stays pageable and every weight copy is staged through the pinned ring. "
                         "0 (default): the whole image is pinned")
    ap.add_argument("--stats-out", default=None,
                    help="write the library's statistics of the last timed step (device timeline included) "
                         "to this JSON file")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes)")
    ap.add_argument("--gemm-shapes", action="store_true",
                    help="instead of training steps: each decoder GEMM shape of the workload alone "
                         "(hol_op_gemm on random bf16 operands, the step's epilogue and output type), "
                         "timed with HIP events; one JSON line per-shape")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU dispatch is not implemented)"}))
        sys.exit(2)
    import torch
    import host_offloaded_layer_amd as hol
    w = W.WORKLOADS[args.workload]
    if args.gemm_shapes:
        print(json.dumps(gemm_shapes_alone(torch, hol, w, args.steps)), flush=True)
        return
    s = w.shape
    log(f"[bench] workload {w.name}: L={s.n_layers} H={s.hidden} tokens={w.tokens} K={w.ckpt_every_k}")
    t0 = time.perf_counter()
    params = W.make_params(w)
    batch = W.make_batch(w)
    log(f"[bench] params generated in {time.perf_counter() - t0:.1f} s")
    cfg = hol.make_config(s.n_layers, s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                          n_experts=s.n_experts, top_k=s.top_k, expert_ffn=s.expert_ffn,
                          lora_rank=s.lora_rank, lora_scale=s.lora_scale, rope_base=s.rope_base,
                          rms_eps=s.rms_eps, ckpt_every_k=w.ckpt_every_k,
                          compute_dtype=hol.BF16 if w.compute == "bf16" else hol.F32,
                          max_tokens=w.tokens, max_seq=w.seq, lr=w.lr,
                          async_optimizer=int(args.optimizer == "async"),
                          pinned_budget_bytes=int(args.pinned_budget_gb * 1e9))
    t0 = time.perf_counter()
    m = hol.Model(cfg)
    m.set_params(params)
    del params
    log(f"[bench] model created and loaded in {time.perf_counter() - t0:.1f} s")
    if args.traffic_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    h2d_peak, d2h_peak = link_peak_gbs(torch)
    log(f"[bench] pinned copy peak: H2D {h2d_peak:.1f} GB/s, D2H {d2h_peak:.1f} GB/s")


    mode = {"and_step": True} if args.optimizer == "sync" else {"stale_step": True}

    def one_step():
        # sync: forward_backward + step, with each layer's host Adam overlapped with the rest of
        # the backward (bitwise the same as the two calls); async: forward_backward at the
        # parameters from before the previous call's update, which runs meanwhile (after the
        # warmup every timed call applies exactly one update)
        if s.vocab:
            loss = m.forward_backward(w.n_micro, tokens=batch["tokens"], **mode)
        else:
            loss = m.forward_backward(w.n_micro, hidden=batch["hidden"], loss=hol.LOSS_SUMSQ, **mode)
        st = m.stats()
        return loss, st, st["step_ms"]

    if args.optimizer == "async" and args.warmup < 1:
        raise SystemExit("--optimizer async needs --warmup >= 1 (the first call applies no update)")
    for i in range(args.warmup):
        loss, fb, step_ms = one_step()
        log(f"[bench] warmup {i}: loss {loss:.4f} fb {fb['fb_ms']:.0f} ms step {step_ms:.0f} ms")
    m.set_kernel_timing(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    recs = []
    for i in range(args.steps):
        loss, fb, step_ms = one_step()
        recs.append((loss, fb, step_ms))
        log(f"[bench] step {i}: loss {loss:.4f} fb {fb['fb_ms']:.0f} ms step {step_ms:.0f} ms "
            f"h2d busy {fb['h2d_busy_ms']:.0f} ms compute busy {fb['compute_busy_ms']:.0f} ms"
            + (f" overlapped step {fb['worker_busy_ms']:.0f} ms, copies waited {fb['async_wait_ms']:.0f} ms"
               if args.optimizer == "async" else ""))
        u = fb.get("units") or []
        if u:
            lag = [e - a for _, a, e in u]
            log(f"[bench]   device: compute from {fb['first_compute_ms']:.1f} to {fb['last_compute_end_ms']:.1f} ms after the "
                f"first weight copy, busy {fb['compute_busy_ms']:.0f} ms")
            log(f"[bench]   host: gpu done at {fb['gpu_done_ms']:.0f} ms, scatter done {fb['scatter_done_ms']:.0f} ms, "
                f"optimiser busy {fb['worker_busy_ms']:.0f} ms over {len(u)} units (first start {u[0][1]:.0f}, "
                f"last end {u[-1][2]:.0f}, max unit {max(lag):.0f} ms); starts "
                + " ".join(f"{int(x)}:{a:.0f}" for x, a, _ in u[::4]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    m.set_kernel_timing(False)
    ms_step = 1e3 * elapsed / args.steps
    value = w.tokens * args.steps / elapsed
    fb_ms = float(np.mean([r[1]["fb_ms"] for r in recs]))
    step_ms = float(np.mean([r[2] for r in recs]))
    fb0 = recs[-1][1]
    if args.stats_out:
        with open(args.stats_out, "w") as f:
            json.dump(fb0, f)
    kern = {}
    for c in fb0["kernels"]:
        ms = sum(r[1]["kernels"][c]["ms"] for r in recs)
        fl = sum(r[1]["kernels"][c]["flops"] for r in recs)
        by = sum(r[1]["kernels"][c]["bytes"] for r in recs)
        n = sum(r[1]["kernels"][c]["launches"] for r in recs)
        if n:
            kern[c] = {"launches_per_step": n // args.steps, "ms_per_step": ms / args.steps,
                       "tflops": fl / ms / 1e9 if ms else 0.0, "gbs": by / ms / 1e6 if ms else 0.0}
    g = kern.get("gemm", {"ms_per_step": 0, "tflops": 0, "launches_per_step": 0})
    alg = algorithmic(w, fb0["n_weight_streams"], fb0["layer_image_bytes"], fb0["head_image_bytes"])
    # per-layer roofline: every layer pass bounded by max(MFMA time, streamed bytes / link peak)
    link = h2d_peak * 1e9
    per_stream_layer = fb0["n_weight_streams"] / s.n_layers
    t_layer = max(alg["f_layer"] / (BF16_PEAK_TFLOPS * 1e12), per_stream_layer * fb0["layer_image_bytes"] / link)
    t_head = max(alg["f_head"] / (BF16_PEAK_TFLOPS * 1e12), fb0["head_image_bytes"] / link)
    t_roof = s.n_layers * t_layer + t_head
    # the rate of the copies the busy time covers (copies sent ahead for the next call have no span)
    h2d_gbs_busy = fb0.get("h2d_span_bytes", fb0["h2d_bytes"]) / (fb0["h2d_busy_ms"] * 1e6) if fb0["h2d_busy_ms"] else 0.0
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.compute == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {s.n_layers} layers, hidden {s.hidden}, {s.n_q_heads}q/{s.n_kv_heads}kv x {s.head_dim}, "
                               + (f"{s.n_experts} experts x {s.expert_ffn} top-{s.top_k}" if s.n_experts else f"ffn {s.ffn}")
                               + (f", LoRA r={s.lora_rank} on a frozen base" if s.lora_rank else "")
                               + f", vocab {s.vocab}; {w.n_micro} micro-batches x {w.batch // w.n_micro} x {w.seq} tokens; K={w.ckpt_every_k}",
                   "global_batch": w.batch, "seq_len": w.seq, "parallelism": "none (1 GPU, layer streaming)",
                   "optimizer": ("synchronous step (hol_forward_backward_step)" if args.optimizer == "sync" else
                                 "staleness-1 asynchronous step (hol_forward_backward_async)"),
                   "weight_image": ("pinned" if not args.pinned_budget_gb else
                                    f"pageable, staged through the pinned ring ({args.pinned_budget_gb:g} GB budget)")},
        "roofline": {"bound": "mfma", "kernel": "gemm_mfma (all decoder and head GEMMs)",
                     "achieved": round(g["tflops"], 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g["tflops"] / BF16_PEAK_TFLOPS, 4), "traffic": profiled_traffic(w.name),
                     "launches_per_step": g["launches_per_step"],
                     "avg_launch_us": round(1e3 * g["ms_per_step"] / max(g["launches_per_step"], 1), 1)},
        "fb_tokens_per_s": round(w.tokens / (fb_ms / 1e3), 1), "fb_ms": round(fb_ms, 1),
        "step_tail_ms": round(step_ms, 1),
        "loss": recs[-1][0],
        "e2e_roofline": {"tokens_per_s": round(w.tokens / t_roof, 1), "frac_fb": round(t_roof / (fb_ms / 1e3), 4),
                         "model": "sum over layers of max(layer FLOPs / bf16 peak, streamed layer bytes / measured H2D peak) + head"},
        "link": {"h2d_peak_gbs": round(h2d_peak, 1), "d2h_peak_gbs": round(d2h_peak, 1),
                 "h2d_gbs_busy": round(h2d_gbs_busy, 1), "h2d_gbs_wall": round(fb0["h2d_bytes"] / (fb0["fb_ms"] * 1e6), 1),
                 "h2d_bytes": fb0["h2d_bytes"], "d2h_bytes": fb0["d2h_bytes"], "weight_streams": fb0["n_weight_streams"],
                 **({"ring_segments": fb0["ring_segments"], "staged_bytes": fb0["staged_bytes"],
                     "staging_ms": round(fb0["staging_ms"], 1)} if fb0.get("ring_segments") else {})},
        "gemm_shapes": gemm_table(w, [r[1] for r in recs], args.steps),
        "model_tflops": round(alg["flops"] / (fb_ms / 1e3) / 1e12, 1),
        "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()} for k, v in kern.items()},
    }
    m.close()
    del m
    # after the timed steps: the sweep's two extra streams stay in the process once created
    out["link_sweep"] = link_sweep(torch)
    log(f"[bench] pinned copy sweep: {out['link_sweep']}")
    if not args.no_cpu_baseline and w.name != "tiny":
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(w)
        log(f"[bench] cpu baseline in {time.perf_counter() - t0:.1f} s")
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
