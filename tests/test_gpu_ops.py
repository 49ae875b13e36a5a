"""Kernel parity on the GPU: every layer-template kernel, called through the C ABI
(include/hol_ops.h), against the oracle's function on identical seeded inputs.

Inputs of bf16 kernels are rounded to bf16 first and the oracle runs in fp64 on those rounded
values, so the only differences left are the kernel's fp32 accumulation order and its output
rounding. Shapes span several tiles plus a ragged tail."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import host_offloaded_layer_amd as hol  # noqa: E402
from oracle import adam as OA  # noqa: E402
from oracle import decoder as D  # noqa: E402

DEV = "cuda"


def dev(a, dtype=torch.float32):
    return torch.as_tensor(np.ascontiguousarray(a)).to(DEV).to(dtype).contiguous()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def bf(a):
    """Round to bf16 and back (fp64 copy of the rounded values)."""
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def sync():
    hol.check(hol.lib.hol_op_sync(None))


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


# ------------------------------------------------------------------ GEMM
def gemm_case(M, N, K, a_km, b_kn, dt, epi, seed=0, out_bf16=False):
    r = np.random.default_rng(seed)
    A = r.standard_normal((K, M) if a_km else (M, K)).astype(np.float32)
    B = r.standard_normal((K, N) if b_kn else (N, K)).astype(np.float32)
    Rm = r.standard_normal((M, N)).astype(np.float32)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    if dt == hol.BF16:
        A64, B64 = bf(A), bf(B)
    else:
        A64, B64 = A.astype(np.float64), B.astype(np.float64)
    Am = A64.T if a_km else A64
    Bm = B64 if b_kn else B64.T
    ref = Am @ Bm
    # leading dimensions padded to a multiple of 8 (16-byte rows for the bf16 kernel)
    lda = -(-A.shape[1] // 8) * 8
    ldb = -(-B.shape[1] // 8) * 8
    Ap = np.zeros((A.shape[0], lda), np.float32); Ap[:, :A.shape[1]] = A
    Bp = np.zeros((B.shape[0], ldb), np.float32); Bp[:, :B.shape[1]] = B
    a, b = dev(Ap, tdt), dev(Bp, tdt)
    cdt = torch.bfloat16 if out_bf16 else torch.float32
    c = dev(Rm, cdt) if epi == 1 else torch.zeros((M, N), dtype=cdt, device=DEV)
    rr = dev(Rm) if epi == 2 else None
    hol.check(hol.lib.hol_op_gemm(M, N, K, a.data_ptr(), lda, int(a_km), b.data_ptr(), ldb,
                                  int(b_kn), c.data_ptr(), N, rr.data_ptr() if rr is not None else None, N,
                                  dt, hol.BF16 if out_bf16 else hol.F32, epi, 1.0, None))
    sync()
    if epi in (1, 2):
        ref = ref + Rm
    return host(c), ref


@pytest.mark.parametrize("a_km,b_kn", [(0, 0), (0, 1), (1, 1), (1, 0)])
@pytest.mark.parametrize("M,N,K", [(300, 200, 136), (512, 384, 256), (37, 129, 8), (300, 520, 96), (600, 520, 320)])
def test_gemm_bf16_mfma_layouts(M, N, K, a_km, b_kn):
    got, ref = gemm_case(M, N, K, a_km, b_kn, hol.BF16, 0)
    # fp32 accumulation of exact bf16 products: error well below 1e-5 of the typical magnitude
    assert np.max(np.abs(got - ref) / (np.abs(ref) + math.sqrt(K))) < 1e-5


@pytest.mark.parametrize("epi", [1, 2])
def test_gemm_bf16_epilogues(epi):
    got, ref = gemm_case(260, 140, 64, 1, 1, hol.BF16, epi, seed=3)
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 8)) < 1e-5


# the NT kernels (K a multiple of 64: 64-deep stages; of 32: 32-deep) with every epilogue, ragged
# M and N over several 256 x 256 tiles
# (N = 300: 16-byte epilogue stores; N = 302: row stride not a multiple of 4, element stores)
@pytest.mark.parametrize("K", [192, 96])
@pytest.mark.parametrize("N", [300, 302])
@pytest.mark.parametrize("epi,out_bf16", [(0, False), (0, True), (1, False), (2, False)])
def test_gemm_bf16_nt_epilogues(K, N, epi, out_bf16):
    got, ref = gemm_case(530, N, K, 0, 0, hol.BF16, epi, seed=K + epi, out_bf16=out_bf16)
    tol = 2 ** -8 if out_bf16 else 1e-5
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 8)) < tol


# the TN kernel (both operands K-major: the weight-gradient layout) with every epilogue, M and N
# ragged over several 256 x 256 tiles
@pytest.mark.parametrize("K", [64, 192])
@pytest.mark.parametrize("M,N", [(520, 304), (264, 776)])
@pytest.mark.parametrize("epi,out_bf16", [(0, False), (0, True), (1, False), (2, False)])
def test_gemm_bf16_tn_epilogues(K, M, N, epi, out_bf16):
    got, ref = gemm_case(M, N, K, 1, 1, hol.BF16, epi, seed=K + M + epi, out_bf16=out_bf16)
    tol = 2 ** -8 if out_bf16 else 1e-5
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 8)) < tol


def test_gemm_bf16_output_rounding():
    got, ref = gemm_case(256, 128, 128, 0, 0, hol.BF16, 0, seed=4, out_bf16=True)
    np.testing.assert_allclose(got, ref, rtol=2 ** -8, atol=1e-3)


@pytest.mark.parametrize("a_km,b_kn", [(0, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_gemm_f32_tiled(a_km, b_kn, epi):
    got, ref = gemm_case(130, 70, 50, a_km, b_kn, hol.F32, epi, seed=5)
    assert np.max(np.abs(got - ref) / (np.abs(ref) + 8)) < 1e-6


# Split tail (hol_op_gemm_ws): 384 tiles = one full round of the 256-block persistent grid plus
# 16 tiles an XCD left, cut in 2 K parts; 320 tiles leave 8 an XCD, cut in 4. Ragged edges, alpha.
@pytest.mark.parametrize("M,N,K", [(6100, 4000, 256), (5000, 4000, 256)])
def test_gemm_split_tail(M, N, K):
    r = np.random.default_rng(M + N)
    A = r.standard_normal((M, K)).astype(np.float32)
    B = r.standard_normal((N, K)).astype(np.float32)
    a, b = dev(A, torch.bfloat16), dev(B, torch.bfloat16)
    wsn = hol.lib.hol_op_gemm_workspace_floats()
    ws = torch.full((wsn,), float("nan"), device=DEV)  # every slot read is written first
    outs = []
    for _ in range(2):
        c = torch.full((M, N), 7.0, device=DEV)
        hol.check(hol.lib.hol_op_gemm_ws(M, N, K, a.data_ptr(), K, 0, b.data_ptr(), K, 0, c.data_ptr(), N, None, 0,
                                         hol.BF16, hol.F32, 0, 0.5, ws.data_ptr(), wsn, None))
        outs.append(c)
    plain = torch.zeros((M, N), device=DEV)
    hol.check(hol.lib.hol_op_gemm(M, N, K, a.data_ptr(), K, 0, b.data_ptr(), K, 0, plain.data_ptr(), N, None, 0,
                                  hol.BF16, hol.F32, 0, 0.5, None))
    sync()
    assert torch.equal(outs[0], outs[1])  # deterministic
    got = host(outs[0])
    assert np.isfinite(got).all()
    rows = np.arange(0, M, 7)
    ref = 0.5 * (bf(A)[rows] @ bf(B).T)
    assert np.max(np.abs(got[rows] - ref) / (np.abs(ref) + math.sqrt(K))) < 1e-5
    assert np.max(np.abs(got - host(plain)) / (np.abs(host(plain)) + math.sqrt(K))) < 1e-5


def test_gemm_ws_leaves_other_epilogues_unsplit():
    """With a workspace, products that are not an fp32 store run exactly as without one."""
    M, N, K = 6100, 4000, 256
    r = np.random.default_rng(5)
    a = dev(r.standard_normal((M, K)), torch.bfloat16)
    b = dev(r.standard_normal((N, K)), torch.bfloat16)
    c0 = dev(r.standard_normal((M, N)))
    wsn = hol.lib.hol_op_gemm_workspace_floats()
    ws = torch.zeros((wsn,), device=DEV)
    c1, c2 = c0.clone(), c0.clone()
    hol.check(hol.lib.hol_op_gemm_ws(M, N, K, a.data_ptr(), K, 0, b.data_ptr(), K, 0, c1.data_ptr(), N, None, 0,
                                     hol.BF16, hol.F32, 1, 1.0, ws.data_ptr(), wsn, None))
    hol.check(hol.lib.hol_op_gemm(M, N, K, a.data_ptr(), K, 0, b.data_ptr(), K, 0, c2.data_ptr(), N, None, 0,
                                  hol.BF16, hol.F32, 1, 1.0, None))
    sync()
    assert torch.equal(c1, c2)


def test_gemm_rejects_misaligned_bf16():
    a = torch.zeros(64, 12, dtype=torch.bfloat16, device=DEV)
    c = torch.zeros(64, 64, device=DEV)
    st = hol.lib.hol_op_gemm(64, 64, 12, a.data_ptr(), 12, 0, a.data_ptr(), 12, 0, c.data_ptr(), 64, None, 0,
                             hol.BF16, hol.F32, 0, 1.0, None)
    assert st == hol.HOL_EINVAL


# ------------------------------------------------------------------ gate/up product with SwiGLU
# hol_op_gemm_swiglu is bit for bit hol_op_gemm (bf16 or fp32 store) followed by hol_op_swiglu_fwd;
# those two are held to the oracle above and below, and the fused result to the oracle here too.
@pytest.mark.parametrize("M,F,K,pad,dt", [
    (300, 96, 128, 0, hol.BF16),     # one partial 256-column tile, ragged rows: fused kernel
    (530, 160, 192, 8, hol.BF16),    # padded row strides of gu and a: fused kernel
    (4352, 2176, 192, 0, hol.BF16),  # 17 x 17 = 289 tiles over 256 blocks: the persistent path
    (260, 100, 128, 0, hol.BF16),    # F % 32 != 0: the product and the element-wise kernel
    (300, 96, 72, 0, hol.BF16),      # K % 64 != 0: likewise
    (130, 48, 64, 0, hol.F32),       # fp32: likewise
])
def test_gemm_swiglu_matches_gemm_then_swiglu(M, F, K, pad, dt):
    N = 2 * F
    r = np.random.default_rng(M + F + K)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    x = dev(r.standard_normal((M, K)) * 0.5, tdt)
    w = dev(r.standard_normal((N, K)) / math.sqrt(K), tdt)
    ldgu, lda = N + pad, F + pad // 2
    gu = torch.full((M, ldgu), 3.0, dtype=tdt, device=DEV)
    act = torch.full((M, lda), 3.0, dtype=tdt, device=DEV)
    hol.check(hol.lib.hol_op_gemm_swiglu(M, N, K, x.data_ptr(), K, w.data_ptr(), K, gu.data_ptr(), ldgu,
                                         act.data_ptr(), lda, dt, None))
    gu_ref = torch.zeros((M, N), dtype=tdt, device=DEV)
    a_ref = torch.zeros((M, F), dtype=tdt, device=DEV)
    hol.check(hol.lib.hol_op_gemm(M, N, K, x.data_ptr(), K, 0, w.data_ptr(), K, 0, gu_ref.data_ptr(), N, None, 0,
                                  dt, dt, 0, 1.0, None))
    hol.check(hol.lib.hol_op_swiglu_fwd(gu_ref.data_ptr(), a_ref.data_ptr(), dt, M, F, None))
    sync()
    assert torch.equal(gu[:, :N], gu_ref) and torch.equal(act[:, :F], a_ref)
    if pad:  # the padding columns are not written
        assert bool((gu[:, N:] == 3.0).all()) and bool((act[:, F:] == 3.0).all())
    # and the oracle: x W^T on the (rounded) inputs in fp64, then SwiGLU of the stored gate / up
    rows = np.arange(0, M, max(1, M // 64))
    ref = host(x)[rows] @ host(w).T
    got_gu = host(gu[:, :N])[rows]
    tol = 2 ** -8 if dt == hol.BF16 else 1e-5
    assert np.max(np.abs(got_gu - ref) / (np.abs(ref) + 1)) < tol
    np.testing.assert_allclose(host(act[:, :F])[rows], D.swiglu(got_gu[:, :F], got_gu[:, F:]), rtol=tol, atol=tol)


# q/k/v product with RoPE in the epilogue: bit for bit the fp32 product then hol_op_rope_qkv
@pytest.mark.parametrize("T,S,nq,nkv,K", [
    (300, 100, 4, 2, 128),     # ragged rows, 3 sequences
    (260, 260, 2, 1, 64),      # N = 512 + 128: a last tile with one head of v
    (4352, 1088, 32, 8, 192),  # 17 x 24 tiles over 256 blocks: the persistent path
])
def test_gemm_rope_matches_gemm_then_rope(T, S, nq, nkv, K):
    d = 128
    N = (nq + 2 * nkv) * d
    r = np.random.default_rng(T + N)
    x = dev(r.standard_normal((T, K)) * 0.5, torch.bfloat16)
    w = dev(r.standard_normal((N, K)) / math.sqrt(K), torch.bfloat16)
    cs, sn = D.rope_tables(S, d, 10000.0, np.float32)
    csd, snd = dev(cs), dev(sn)
    out = torch.full((T, N), 3.0, dtype=torch.bfloat16, device=DEV)
    hol.check(hol.lib.hol_op_gemm_rope(T, N, K, x.data_ptr(), K, w.data_ptr(), K, out.data_ptr(), N, (nq + nkv) * d, S,
                                       csd.data_ptr(), snd.data_ptr(), None))
    f32 = torch.zeros((T, N), device=DEV)
    hol.check(hol.lib.hol_op_gemm(T, N, K, x.data_ptr(), K, 0, w.data_ptr(), K, 0, f32.data_ptr(), N, None, 0,
                                  hol.BF16, hol.F32, 0, 1.0, None))
    ref = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    hol.check(hol.lib.hol_op_rope_qkv(f32.data_ptr(), N, ref.data_ptr(), N, T, nq, nkv, d, S, csd.data_ptr(),
                                      snd.data_ptr(), None))
    sync()
    assert torch.equal(out, ref)
    # and the oracle on sampled rows: x W^T in fp64, RoPE on q and k at position t mod S
    rows = np.arange(0, T, max(1, T // 48))
    y = host(x)[rows] @ host(w).T
    heads = y.reshape(len(rows), nq + 2 * nkv, d)  # (the oracle's rope takes one position per row)
    rot = D.rope(heads[:, :nq + nkv, :], cs[rows % S].astype(np.float64), sn[rows % S].astype(np.float64))
    want = np.concatenate([rot.reshape(len(rows), -1), y[:, (nq + nkv) * d:]], 1)
    got = host(out)[rows]
    assert np.max(np.abs(got - want) / (np.abs(want) + 1)) < 2 ** -7


def test_gemm_rope_rejects_unsupported():
    z = torch.zeros(256 * 256, dtype=torch.bfloat16, device=DEV)
    t = torch.zeros(64, device=DEV)
    # N not a multiple of 128; rotated columns not a multiple of 128; missing tables
    for N, nrot, tab in ((200, 128, t.data_ptr()), (256, 100, t.data_ptr()), (256, 128, None)):
        st = hol.lib.hol_op_gemm_rope(8, N, 64, z.data_ptr(), 64, z.data_ptr(), 64, z.data_ptr(), N, nrot, 1, tab, tab,
                                      None)
        assert st == hol.HOL_EINVAL


def test_gemm_swiglu_rejects_odd_n_and_unpacked_fallback():
    x = torch.zeros(64, 64, dtype=torch.bfloat16, device=DEV)
    gu = torch.zeros(64, 208, dtype=torch.bfloat16, device=DEV)
    a = torch.zeros(64, 104, dtype=torch.bfloat16, device=DEV)
    st = hol.lib.hol_op_gemm_swiglu(64, 199, 64, x.data_ptr(), 64, gu.data_ptr(), 64, gu.data_ptr(), 208,
                                    a.data_ptr(), 104, hol.BF16, None)
    assert st == hol.HOL_EINVAL
    # F = 100 takes the two-kernel path, which needs packed gu and a
    st = hol.lib.hol_op_gemm_swiglu(64, 200, 64, x.data_ptr(), 64, gu.data_ptr(), 64, gu.data_ptr(), 208,
                                    a.data_ptr(), 104, hol.BF16, None)
    assert st == hol.HOL_EINVAL


# ------------------------------------------------------------------ transpose (pure data movement: bit-exact)
@pytest.mark.parametrize("R,C,ldi,ldo", [(256, 384, 384, 256), (300, 136, 136, 304), (1000, 2056, 2064, 1008),
                                         (8, 8, 8, 8), (129, 127, 128, 136)])
def test_transpose_bf16_bitexact(R, C, ldi, ldo):
    g = torch.Generator().manual_seed(R * 7 + C)
    x = torch.randn(R, ldi, generator=g).to(torch.bfloat16).to(DEV)
    out = torch.full((C, ldo), 7.0, dtype=torch.bfloat16, device=DEV)
    hol.check(hol.lib.hol_op_transpose_bf16(x.data_ptr(), ldi, out.data_ptr(), ldo, R, C, None))
    sync()
    xv = x.cpu().view(torch.int16).numpy()
    ov = out.cpu().view(torch.int16).numpy()
    assert np.array_equal(ov[:, :R], xv[:, :C].T)
    pad = torch.tensor(7.0, dtype=torch.bfloat16).view(torch.int16).item()
    assert np.all(ov[:, R:] == pad)      # nothing written past the R columns of each output row


def test_transpose_rejects_misaligned():
    x = torch.zeros(16, 12, dtype=torch.bfloat16, device=DEV)
    assert hol.lib.hol_op_transpose_bf16(x.data_ptr(), 12, x.data_ptr(), 16, 16, 12, None) == hol.HOL_EINVAL


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("H,T,yt,acc", [(64, 37, hol.F32, 1), (4096, 300, hol.BF16, 1), (2048, 1100, hol.F32, 1),
                                        (1540, 2500, hol.F32, 0), (3072, 5000, hol.BF16, 1), (5000, 70, hol.BF16, 1)])
def test_rmsnorm_fwd_bwd(H, T, yt, acc):
    r = np.random.default_rng(H + T)
    x = r.standard_normal((T, H)).astype(np.float32) * 3
    g = (1 + 0.1 * r.standard_normal(H)).astype(np.float32)
    dy = r.standard_normal((T, H)).astype(np.float32)
    dx0 = r.standard_normal((T, H)).astype(np.float32)
    xd, gd, dyd = dev(x), dev(g), dev(dy)
    y = torch.empty((T, H), dtype=torch.bfloat16 if yt == hol.BF16 else torch.float32, device=DEV)
    rs = torch.empty(T, device=DEV)
    hol.check(hol.lib.hol_op_rmsnorm_fwd(xd.data_ptr(), gd.data_ptr(), 1e-5, y.data_ptr(), yt, rs.data_ptr(), T, H, None))
    dx = dev(dx0)
    dgam = torch.full((H,), 0.5, device=DEV)
    ws = torch.empty(hol.lib.hol_op_rmsnorm_bwd_workspace(T, H), device=DEV)
    ry, rr = D.rmsnorm(x.astype(np.float64), g.astype(np.float64), 1e-5)
    tol = 2 ** -8 if yt == hol.BF16 else 1e-6
    if H > 4096:   # forward only (two-pass path); the backward kernel is for rows up to 4096 wide
        assert hol.lib.hol_op_rmsnorm_bwd(dyd.data_ptr(), xd.data_ptr(), gd.data_ptr(), rs.data_ptr(), dx.data_ptr(),
                                          1, dgam.data_ptr(), ws.data_ptr(), T, H, None) == hol.HOL_EINVAL
        sync()
        np.testing.assert_allclose(host(rs), rr, rtol=1e-6)
        np.testing.assert_allclose(host(y), ry, rtol=tol, atol=tol)
        return
    hol.check(hol.lib.hol_op_rmsnorm_bwd(dyd.data_ptr(), xd.data_ptr(), gd.data_ptr(), rs.data_ptr(), dx.data_ptr(), acc,
                                         dgam.data_ptr(), ws.data_ptr(), T, H, None))
    sync()
    rdx, rdg = D.rmsnorm_bwd(dy.astype(np.float64), x.astype(np.float64), g.astype(np.float64), rr)
    np.testing.assert_allclose(host(rs), rr, rtol=1e-6)
    np.testing.assert_allclose(host(y), ry, rtol=tol, atol=tol)
    np.testing.assert_allclose(host(dx), rdx + (dx0 if acc else 0), rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(host(dgam), rdg + 0.5, rtol=1e-5, atol=1e-4)


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("dt", [hol.F32, hol.BF16])
def test_rope_fwd_and_inverse(dt):
    S, nseq, heads, d, ld = 70, 2, 3, 128, 3 * 128 + 64
    r = np.random.default_rng(9)
    x = r.standard_normal((nseq * S, ld)).astype(np.float32)
    cos, sin = D.rope_tables(S, d, 10000.0, np.float32)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    xd = dev(x, tdt)
    xin = host(xd)
    cd, sd = dev(cos), dev(sin)   # keep references: the kernel runs after the call returns
    hol.check(hol.lib.hol_op_rope(xd.data_ptr(), dt, ld, nseq * S, heads, d, S, cd.data_ptr(),
                                  sd.data_ptr(), 0, None))
    sync()
    out = host(xd)
    for b in range(nseq):
        blk = xin[b * S:(b + 1) * S, :heads * d].reshape(S, heads, d)
        ref = D.rope(blk, cos.astype(np.float64), sin.astype(np.float64)).reshape(S, heads * d)
        tol = 2 ** -7 if dt == hol.BF16 else 1e-6
        np.testing.assert_allclose(out[b * S:(b + 1) * S, :heads * d], ref, rtol=tol, atol=tol)
    np.testing.assert_array_equal(out[:, heads * d:], xin[:, heads * d:])  # untouched columns
    if dt == hol.F32:
        hol.check(hol.lib.hol_op_rope(xd.data_ptr(), dt, ld, nseq * S, heads, d, S, cd.data_ptr(), sd.data_ptr(), 1, None))
        sync()
        np.testing.assert_allclose(host(xd), xin, atol=1e-5)



@pytest.mark.parametrize("d,ldx", [(128, 0), (64, 8), (20, 4)])   # 4-pair kernel / one-pair kernel
def test_rope_qkv_fused(d, ldx):
    """q and k rotated, v copied, all rounded to bf16 once; with an input shifted by one float (not
    16-byte aligned) the one-pair kernel runs and must give the same bits."""
    S, nseq, nq, nkv = 37, 3, 4, 2
    W_ = (nq + 2 * nkv) * d
    ldi = W_ + ldx
    T = nseq * S
    r = np.random.default_rng(d)
    x = (r.standard_normal((T, ldi)) * 2).astype(np.float32)
    cos, sin = D.rope_tables(S, d, 10000.0, np.float32)
    cd, sd = dev(cos), dev(sin)
    outs = []
    for shift in (0, 1):
        buf = torch.zeros(T * ldi + 1, device=DEV)
        buf[shift:shift + T * ldi].copy_(torch.as_tensor(x.reshape(-1)))
        out = torch.zeros((T, W_), dtype=torch.bfloat16, device=DEV)
        hol.check(hol.lib.hol_op_rope_qkv(buf[shift:].data_ptr(), ldi, out.data_ptr(), W_, T, nq, nkv, d, S,
                                          cd.data_ptr(), sd.data_ptr(), None))
        sync()
        outs.append(out.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    got = OA.bf16_to_f32(outs[0].view(np.uint16)).reshape(T, W_).astype(np.float64)
    for b in range(nseq):
        blk = x[b * S:(b + 1) * S, :W_].astype(np.float64)
        qk = blk[:, :(nq + nkv) * d].reshape(S, nq + nkv, d)
        ref = D.rope(qk, cos.astype(np.float64), sin.astype(np.float64)).reshape(S, -1)
        np.testing.assert_allclose(got[b * S:(b + 1) * S, :(nq + nkv) * d], ref, rtol=2 ** -8, atol=2 ** -8)
        np.testing.assert_array_equal(got[b * S:(b + 1) * S, (nq + nkv) * d:],
                                      OA.bf16_to_f32(OA.bf16_round(blk[:, (nq + nkv) * d:].astype(np.float32))).reshape(S, -1))

# ------------------------------------------------------------------ SwiGLU
@pytest.mark.parametrize("F", [344, 342])   # 8-wide kernel / one-element kernel
@pytest.mark.parametrize("dt", [hol.F32, hol.BF16])
def test_swiglu_fwd_bwd(dt, F):
    T = 77
    r = np.random.default_rng(2)
    gu = r.standard_normal((T, 2 * F)).astype(np.float32) * 2
    da = r.standard_normal((T, F)).astype(np.float32)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    gud, dad = dev(gu, tdt), dev(da, tdt)
    a = torch.empty((T, F), dtype=tdt, device=DEV)
    dgu = torch.empty((T, 2 * F), dtype=tdt, device=DEV)
    hol.check(hol.lib.hol_op_swiglu_fwd(gud.data_ptr(), a.data_ptr(), dt, T, F, None))
    hol.check(hol.lib.hol_op_swiglu_bwd(dad.data_ptr(), gud.data_ptr(), dgu.data_ptr(), dt, T, F, None))
    sync()
    g64, u64, da64 = host(gud)[:, :F], host(gud)[:, F:], host(dad)
    tol = 2 ** -7 if dt == hol.BF16 else 2e-6
    np.testing.assert_allclose(host(a), D.swiglu(g64, u64), rtol=tol, atol=tol)
    dg, du = D.swiglu_bwd(da64, g64, u64)
    np.testing.assert_allclose(host(dgu), np.concatenate([dg, du], 1), rtol=tol, atol=tol)



@pytest.mark.parametrize("dt", [hol.F32, hol.BF16])
def test_swiglu_vector_and_scalar_kernels_agree_bitwise(dt):
    """Buffers shifted by one element are not 16-byte aligned, which routes the call to the
    one-element kernels; both kernels must give the same bits."""
    T, F = 45, 96
    r = np.random.default_rng(3)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    gu0 = dev(r.standard_normal((T * 2 * F,)).astype(np.float32) * 3, tdt)
    da0 = dev(r.standard_normal((T * F,)).astype(np.float32), tdt)
    outs = []
    for off in (0, 1):
        gu = torch.zeros(T * 2 * F + 1, dtype=tdt, device=DEV)
        da = torch.zeros(T * F + 1, dtype=tdt, device=DEV)
        g, d = gu[off:off + T * 2 * F], da[off:off + T * F]
        g.copy_(gu0)
        d.copy_(da0)
        a = torch.zeros(T * F + 1, dtype=tdt, device=DEV)
        dgu = torch.zeros(T * 2 * F + 1, dtype=tdt, device=DEV)
        hol.check(hol.lib.hol_op_swiglu_fwd(g.data_ptr(), a[off:].data_ptr(), dt, T, F, None))
        hol.check(hol.lib.hol_op_swiglu_bwd(d.data_ptr(), g.data_ptr(), dgu[off:].data_ptr(), dt, T, F, None))
        sync()
        outs.append((host(a[off:off + T * F]), host(dgu[off:off + T * 2 * F])))
    for x, y in zip(outs[0], outs[1]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))

@pytest.mark.parametrize("T,F,ldt", [(200, 128, 200), (1000, 640, 1008), (128, 64, 136), (8, 64, 8)])
def test_swiglu_bwd_with_transpose_bitwise(T, F, ldt):
    """The fused SwiGLU backward writes dgu exactly as hol_op_swiglu_bwd does and dgu^T exactly as
    hol_op_transpose_bf16 transposes it (ragged token tiles, a padded output stride, one tile row
    of 8 tokens); nothing is written past column T of the transposed rows."""
    r = np.random.default_rng(5)
    gud = dev(r.standard_normal((T, 2 * F)).astype(np.float32) * 2, torch.bfloat16)
    dad = dev(r.standard_normal((T, F)).astype(np.float32), torch.bfloat16)
    ref = torch.empty((T, 2 * F), dtype=torch.bfloat16, device=DEV)
    ref_t = torch.empty((2 * F, T), dtype=torch.bfloat16, device=DEV)
    hol.check(hol.lib.hol_op_swiglu_bwd(dad.data_ptr(), gud.data_ptr(), ref.data_ptr(), hol.BF16, T, F, None))
    hol.check(hol.lib.hol_op_transpose_bf16(ref.data_ptr(), 2 * F, ref_t.data_ptr(), T, T, 2 * F, None))
    dgu = torch.zeros((T, 2 * F), dtype=torch.bfloat16, device=DEV)
    dgut = torch.full((2 * F, ldt), 7.0, dtype=torch.bfloat16, device=DEV)
    hol.check(hol.lib.hol_op_swiglu_bwd_t(dad.data_ptr(), gud.data_ptr(), dgu.data_ptr(), dgut.data_ptr(), ldt, T, F,
                                          None))
    sync()
    assert torch.equal(dgu, ref)
    assert torch.equal(dgut[:, :T], ref_t)
    assert torch.all(dgut[:, T:] == 7.0)


def test_swiglu_bwd_with_transpose_rejects_unsupported_shapes():
    x = torch.zeros(4096, dtype=torch.bfloat16, device=DEV)
    p = x.data_ptr()
    assert hol.lib.hol_op_swiglu_bwd_t(p, p, p, p, 16, 16, 48, None) == hol.HOL_EINVAL   # F % 64
    assert hol.lib.hol_op_swiglu_bwd_t(p, p, p, p, 16, 12, 64, None) == hol.HOL_EINVAL   # T % 8
    assert hol.lib.hol_op_swiglu_bwd_t(p, p, p, p, 8, 16, 64, None) == hol.HOL_EINVAL    # ldt < T

# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("dt,S,nseq,nq,nkv,d", [
    (hol.F32, 32, 2, 4, 4, 16),
    (hol.F32, 100, 2, 4, 2, 64),
    (hol.BF16, 200, 1, 8, 2, 128),
    (hol.BF16, 130, 2, 4, 1, 128),
    (hol.BF16, 260, 2, 16, 4, 128),   # 8 (sequence, kv head) pairs: whole pairs dealt to each XCD
    (hol.BF16, 192, 8, 8, 1, 64),
    (hol.BF16, 40, 3, 8, 2, 128),     # shorter than one 64-query tile: whole halves past the end
    (hol.BF16, 97, 1, 32, 8, 128),    # the LLaMA-8B head layout, one ragged tile
])
def test_attention_fwd_bwd(dt, S, nseq, nq, nkv, d):
    r = np.random.default_rng(S + nq)
    T = nseq * S
    q = r.standard_normal((T, nq * d)).astype(np.float32)
    k = r.standard_normal((T, nkv * d)).astype(np.float32)
    v = r.standard_normal((T, nkv * d)).astype(np.float32)
    do = r.standard_normal((T, nq * d)).astype(np.float32)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    qd, kd, vd, dod = dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(do, tdt)
    o = torch.empty((T, nq * d), dtype=tdt, device=DEV)
    lse = torch.empty((nseq, nq, S), device=DEV)
    hol.check(hol.lib.hol_op_attention_fwd(nseq, S, nq, nkv, d, dt, qd.data_ptr(), nq * d, kd.data_ptr(), nkv * d,
                                           vd.data_ptr(), nkv * d, o.data_ptr(), nq * d, lse.data_ptr(), None))
    dq = torch.empty_like(qd); dk = torch.empty_like(kd); dv = torch.empty_like(vd)
    delta = torch.empty((nseq, nq, S), device=DEV)
    hol.check(hol.lib.hol_op_attention_bwd(nseq, S, nq, nkv, d, dt, qd.data_ptr(), nq * d, kd.data_ptr(), nkv * d,
                                           vd.data_ptr(), nkv * d, o.data_ptr(), nq * d, lse.data_ptr(),
                                           dod.data_ptr(), nq * d, dq.data_ptr(), nq * d, dk.data_ptr(), nkv * d,
                                           dv.data_ptr(), nkv * d, delta.data_ptr(), None))
    sync()
    q64, k64, v64, do64 = host(qd), host(kd), host(vd), host(dod)
    o_h = host(o)
    for b in range(nseq):
        sl = slice(b * S, (b + 1) * S)
        ro, rl = D.attention(q64[sl].reshape(S, nq, d), k64[sl].reshape(S, nkv, d), v64[sl].reshape(S, nkv, d))
        # the backward is checked against the oracle given the kernel's own (rounded) output
        rdq, rdk, rdv = D.attention_bwd(do64[sl].reshape(S, nq, d), q64[sl].reshape(S, nq, d),
                                        k64[sl].reshape(S, nkv, d), v64[sl].reshape(S, nkv, d),
                                        o_h[sl].reshape(S, nq, d), rl)
        if dt == hol.BF16:
            assert rel(o_h[sl], ro.reshape(S, -1)) < 6e-3
            assert rel(host(dq)[sl], rdq.reshape(S, -1)) < 1e-2
            assert rel(host(dk)[sl], rdk.reshape(S, -1)) < 1e-2
            assert rel(host(dv)[sl], rdv.reshape(S, -1)) < 1e-2
        else:
            np.testing.assert_allclose(o_h[sl], ro.reshape(S, -1), rtol=1e-5, atol=1e-5)
            np.testing.assert_allclose(host(dq)[sl], rdq.reshape(S, -1), rtol=1e-4, atol=1e-4)
            np.testing.assert_allclose(host(dk)[sl], rdk.reshape(S, -1), rtol=1e-4, atol=1e-4)
            np.testing.assert_allclose(host(dv)[sl], rdv.reshape(S, -1), rtol=1e-4, atol=1e-4)
        np.testing.assert_allclose(host(lse)[b], rl, rtol=1e-5, atol=1e-5)


# the backward with the RoPE backward of dq and dk: head width 128 applies it in the kernels'
# epilogues (one rounding), width 64 through hol_op_rope afterwards; both against the oracle's
# attention_bwd then rope_bwd, and dv exactly as hol_op_attention_bwd writes it
@pytest.mark.parametrize("S,nseq,nq,nkv,d", [(260, 2, 8, 2, 128), (300, 1, 4, 4, 64)])
def test_attention_bwd_rope(S, nseq, nq, nkv, d):
    r = np.random.default_rng(S + d)
    T = nseq * S
    tdt = torch.bfloat16
    qd, kd, vd, dod = (dev(r.standard_normal((T, n * d)), tdt) for n in (nq, nkv, nkv, nq))
    o = torch.empty((T, nq * d), dtype=tdt, device=DEV)
    lse = torch.empty((nseq, nq, S), device=DEV)
    hol.check(hol.lib.hol_op_attention_fwd(nseq, S, nq, nkv, d, hol.BF16, qd.data_ptr(), nq * d, kd.data_ptr(),
                                           nkv * d, vd.data_ptr(), nkv * d, o.data_ptr(), nq * d, lse.data_ptr(), None))
    cs, sn = D.rope_tables(S, d, 10000.0, np.float32)
    csd, snd = dev(cs), dev(sn)
    outs = []
    for fn in ("hol_op_attention_bwd_rope", "hol_op_attention_bwd"):
        dq = torch.empty_like(qd); dk = torch.empty_like(kd); dv = torch.empty_like(vd)
        delta = torch.empty((nseq, nq, S), device=DEV)
        args = [nseq, S, nq, nkv, d, hol.BF16, qd.data_ptr(), nq * d, kd.data_ptr(), nkv * d, vd.data_ptr(), nkv * d,
                o.data_ptr(), nq * d, lse.data_ptr(), dod.data_ptr(), nq * d, dq.data_ptr(), nq * d, dk.data_ptr(),
                nkv * d, dv.data_ptr(), nkv * d, delta.data_ptr()]
        if fn.endswith("rope"):
            args += [csd.data_ptr(), snd.data_ptr()]
        hol.check(getattr(hol.lib, fn)(*args, None))
        outs.append((dq, dk, dv))
    sync()
    (dq, dk, dv), (_, _, dv0) = outs
    assert torch.equal(dv, dv0)
    q64, k64, v64, do64, o64 = host(qd), host(kd), host(vd), host(dod), host(o)
    c64, s64 = cs.astype(np.float64), sn.astype(np.float64)
    for b in range(nseq):
        sl = slice(b * S, (b + 1) * S)
        _, rl = D.attention(q64[sl].reshape(S, nq, d), k64[sl].reshape(S, nkv, d), v64[sl].reshape(S, nkv, d))
        rdq, rdk, _ = D.attention_bwd(do64[sl].reshape(S, nq, d), q64[sl].reshape(S, nq, d), k64[sl].reshape(S, nkv, d),
                                      v64[sl].reshape(S, nkv, d), o64[sl].reshape(S, nq, d), rl)
        assert rel(host(dq)[sl], D.rope_bwd(rdq, c64, s64).reshape(S, -1)) < 1e-2
        assert rel(host(dk)[sl], D.rope_bwd(rdk, c64, s64).reshape(S, -1)) < 1e-2


def test_attention_bwd_rope_rejects_missing_tables():
    z = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    st = hol.lib.hol_op_attention_bwd_rope(1, 4, 1, 1, 16, hol.BF16, *([z.data_ptr(), 16] * 4), z.data_ptr(),
                                           z.data_ptr(), 16, z.data_ptr(), 16, z.data_ptr(), 16, z.data_ptr(), 16,
                                           z.data_ptr(), None, None, None)
    assert st == hol.HOL_EINVAL


def test_attention_single_position():
    """S = 1: the softmax is the single key, so o = v of the head's kv head, dv sums dO over the
    heads of the group, and dq = dk = 0 (dS = P (dP - rowsum(dO o)) vanishes up to the rounding of
    the two sums, hence an absolute bound)."""
    nseq, S, nq, nkv, d = 3, 1, 8, 2, 128
    r = np.random.default_rng(11)
    T, g = nseq * S, nq // nkv
    q, k, v, do = (r.standard_normal((T, n * d)).astype(np.float32) for n in (nq, nkv, nkv, nq))
    qd, kd, vd, dod = (dev(x, torch.bfloat16) for x in (q, k, v, do))
    o = torch.empty((T, nq * d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((nseq, nq, S), device=DEV)
    hol.check(hol.lib.hol_op_attention_fwd(nseq, S, nq, nkv, d, hol.BF16, qd.data_ptr(), nq * d, kd.data_ptr(), nkv * d,
                                           vd.data_ptr(), nkv * d, o.data_ptr(), nq * d, lse.data_ptr(), None))
    dq = torch.empty_like(qd); dk = torch.empty_like(kd); dv = torch.empty_like(vd)
    delta = torch.empty((nseq, nq, S), device=DEV)
    hol.check(hol.lib.hol_op_attention_bwd(nseq, S, nq, nkv, d, hol.BF16, qd.data_ptr(), nq * d, kd.data_ptr(), nkv * d,
                                           vd.data_ptr(), nkv * d, o.data_ptr(), nq * d, lse.data_ptr(),
                                           dod.data_ptr(), nq * d, dq.data_ptr(), nq * d, dk.data_ptr(), nkv * d,
                                           dv.data_ptr(), nkv * d, delta.data_ptr(), None))
    sync()
    q64, k64, v64, do64 = host(qd), host(kd), host(vd), host(dod)
    o_h = host(o).reshape(T, nq, d)
    for h in range(nq):
        np.testing.assert_array_equal(o_h[:, h], v64.reshape(T, nkv, d)[:, h // g])
        qk = np.einsum("td,td->t", q64.reshape(T, nq, d)[:, h], k64.reshape(T, nkv, d)[:, h // g]) / np.sqrt(d)
        np.testing.assert_allclose(host(lse)[:, h, 0], qk, rtol=1e-5, atol=1e-5)
    want_dv = do64.reshape(T, nkv, g, d).sum(axis=2).reshape(T, nkv * d)
    assert rel(host(dv), want_dv) < 1e-2
    assert np.abs(host(dq)).max() < 1e-3 and np.abs(host(dk)).max() < 1e-3


# ------------------------------------------------------------------ cross entropy
@pytest.mark.parametrize("dt,V", [(hol.F32, 256), (hol.BF16, 5000), (hol.BF16, 4999), (hol.F32, 1003)])  # V % 8 != 0: the scalar kernel
def test_cross_entropy_rows(dt, V):
    Tc = 40
    r = np.random.default_rng(V)
    z = (r.standard_normal((Tc, V)) * 2).astype(np.float32)
    lab = r.integers(0, V, Tc).astype(np.int32)
    lab[[3, 17]] = -1
    w = np.where(lab >= 0, 1.0 / np.sum(lab >= 0), 0.0).astype(np.float32)
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    zd, ld, wd = dev(z), torch.as_tensor(lab).to(DEV), dev(w)
    rl = torch.empty(Tc, device=DEV)
    dz = torch.empty((Tc, V), dtype=tdt, device=DEV)
    hol.check(hol.lib.hol_op_cross_entropy(zd.data_ptr(), V, ld.data_ptr(), wd.data_ptr(), rl.data_ptr(),
                                           dz.data_ptr(), dt, V, Tc, V, None))
    sync()
    loss, dref = D.cross_entropy(z.astype(np.float64), lab)
    assert abs(host(rl).sum() - loss) < 1e-5 * loss
    tol = 2 ** -8 if dt == hol.BF16 else 1e-6
    np.testing.assert_allclose(host(dz), dref, rtol=tol, atol=tol * np.abs(dref).max())
