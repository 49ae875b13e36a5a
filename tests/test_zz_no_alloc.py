"""The allocation-free attention backward (hol_op_attention_bwd_noalloc) against the entry point it
is a variant of (hol_op_attention_bwd, with a caller workspace): the same kernels on the same
inputs, so the results must agree bit for bit, on two calls in a row (the second smaller, so it
reads a scratch array still holding the first call's row sums), in both head widths and in fp32,
and a size over the scratch's limit is rejected before any launch."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import host_offloaded_layer_amd as hol  # noqa: E402

DEV = "cuda"
LIMIT = 4 << 20   # row sums the static scratch holds


def _inputs(nseq, S, nq, nkv, d, dt, seed):
    g = torch.Generator().manual_seed(seed)
    T = nseq * S
    tdt = torch.bfloat16 if dt == hol.BF16 else torch.float32
    q, k, v, do = (torch.randn(T, n * d, generator=g).to(tdt).to(DEV) for n in (nq, nkv, nkv, nq))
    o = torch.empty((T, nq * d), dtype=tdt, device=DEV)
    lse = torch.empty((nseq, nq, S), device=DEV)
    hol.check(hol.lib.hol_op_attention_fwd(nseq, S, nq, nkv, d, dt, q.data_ptr(), nq * d, k.data_ptr(), nkv * d,
                                           v.data_ptr(), nkv * d, o.data_ptr(), nq * d, lse.data_ptr(), None))
    return q, k, v, o, lse, do


def _bwd(args, nseq, S, nq, nkv, d, dt, noalloc):
    q, k, v, o, lse, do = args
    dq = torch.full_like(q, 3.0); dk = torch.full_like(k, 3.0); dv = torch.full_like(v, 3.0)
    common = (nseq, S, nq, nkv, d, dt, q.data_ptr(), nq * d, k.data_ptr(), nkv * d, v.data_ptr(), nkv * d,
              o.data_ptr(), nq * d, lse.data_ptr(), do.data_ptr(), nq * d, dq.data_ptr(), nq * d,
              dk.data_ptr(), nkv * d, dv.data_ptr(), nkv * d)
    if noalloc:
        hol.check(hol.lib.hol_op_attention_bwd_noalloc(*common, None))
    else:
        delta = torch.empty((nseq, nq, S), device=DEV)
        hol.check(hol.lib.hol_op_attention_bwd(*common, delta.data_ptr(), None))
    hol.check(hol.lib.hol_op_sync(None))
    return dq, dk, dv


@pytest.mark.parametrize("dt,d", [(hol.BF16, 128), (hol.BF16, 64), (hol.F32, 64)])
def test_noalloc_attention_bwd_matches_workspace_entry_point(dt, d):
    for shape, seed in (((2, 300, 8, 2), 1), ((1, 100, 4, 1), 2)):   # second call smaller
        nseq, S, nq, nkv = shape
        print("noalloc attention bwd", dt, d, shape, flush=True)
        args = _inputs(nseq, S, nq, nkv, d, dt, seed)
        ref = _bwd(args, nseq, S, nq, nkv, d, dt, noalloc=False)
        got = _bwd(args, nseq, S, nq, nkv, d, dt, noalloc=True)
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
            assert torch.isfinite(a.float()).all()


def test_noalloc_attention_bwd_rejects_sizes_over_the_scratch():
    x = torch.zeros(8, dtype=torch.bfloat16, device=DEV)
    p = x.data_ptr()
    S = LIMIT // 4 + 1                    # n_seq * nq * S = LIMIT + 4
    st = hol.lib.hol_op_attention_bwd_noalloc(1, S, 4, 1, 128, hol.BF16, p, 512, p, 128, p, 128, p, 512, p, p, 512,
                                              p, 512, p, 128, p, 128, None)
    assert st == hol.HOL_EINVAL
    assert b"static scratch" in hol.lib.hol_last_error()
