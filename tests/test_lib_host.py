"""Host-side checks of libhol.so that need no GPU: the library loads, exports every symbol the
public headers declare, and its host logic (partitioner, Adam, bf16 refresh, argument checking)
matches the oracle."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import host_offloaded_layer_amd as hol
from oracle import adam as OA
from oracle import partition as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    for h in ("hol.h", "hol_ops.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names |= set(re.findall(r"\b(hol_\w+)\s*\(", txt))
    return names


def test_library_exports_every_declared_symbol():
    decl = declared_symbols()
    assert len(decl) >= 25
    for n in decl:
        assert hasattr(hol.lib, n), n
    assert set(hol.EXPORTED) == decl
    assert "gfx950" in hol.version()


def test_partition_user_guide_example():
    t_f, t_b = [1] * 12, [3] * 12
    for n_gpus in (1, 2, 8):
        fb, bb, tmax, J = hol.partition(t_f, t_b, [1] * 12, [1] * 12, 100, n_gpus, 4)
        assert fb == [0, 3, 6, 9]
        assert bb == list(range(11, -1, -1))
        assert tmax == 3 and J == (4 * 16 + n_gpus * (n_gpus - 1)) * 3


@pytest.mark.parametrize("seed", range(40))
def test_partition_bit_exact_against_brute_force(seed):
    r = np.random.default_rng(seed)
    L = int(r.integers(1, 9))
    big = seed % 3 == 0
    hi = 10 ** 12 if big else 20
    t_f = r.integers(0 if seed % 5 == 0 else 1, hi, L)
    t_b = r.integers(1, 3 * hi, L)
    m_f = r.integers(1, 10, L)
    m_b = r.integers(1, 10, L)
    cap = int(r.integers(9, 40))
    n_gpus = int(r.integers(1, 9))
    n_micro = int(r.integers(1, 17))
    ref = OP.partition_bruteforce(t_f.tolist(), t_b.tolist(), m_f.tolist(), m_b.tolist(), cap, n_gpus, n_micro)
    fb, bb, tmax, J = hol.partition(t_f, t_b, m_f, m_b, cap, n_gpus, n_micro)
    lf, lb, rt, rJ = ref
    assert fb == OP.stage_bounds(lf, L, False)
    assert bb == OP.stage_bounds(lb, L, True)
    assert tmax == rt
    assert J == min(rJ, 2 ** 63 - 1)


def test_partition_rejects_layer_over_cap():
    with pytest.raises(hol.HolError) as e:
        hol.partition([1, 1], [1, 1], [5, 50], [5, 5], 10, 1, 1)
    assert e.value.status == hol.HOL_EINVAL


def test_host_adam_bit_exact_against_oracle():
    r = np.random.default_rng(5)
    n = 100_003
    th = r.standard_normal(n).astype(np.float32)
    m = np.zeros(n, np.float32); v = np.zeros(n, np.float32)
    th2, m2, v2 = th.copy(), m.copy(), v.copy()
    for t in range(1, 5):
        g = (r.standard_normal(n) * 10.0 ** r.uniform(-8, 2, n)).astype(np.float32)
        g[::97] = 0.0
        hol.host_adam(th, g, m, v, t, lr=1e-3)
        OA.adam_update(th2, g, m2, v2, t, lr=1e-3)
        assert np.array_equal(th.view(np.uint32), th2.view(np.uint32))
        assert np.array_equal(m.view(np.uint32), m2.view(np.uint32))
        assert np.array_equal(v.view(np.uint32), v2.view(np.uint32))


def test_host_bf16_round_bit_exact_against_oracle():
    r = np.random.default_rng(6)
    x = np.concatenate([r.standard_normal(50_000).astype(np.float32) * 10.0 ** r.integers(-30, 30, 50_000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-45, 1.00390625], np.float32)])
    np.testing.assert_array_equal(hol.host_bf16_round(x), OA.bf16_round(x))
    assert np.isnan(OA.bf16_to_f32(hol.host_bf16_round(np.array([np.nan], np.float32))))[0]


def _tiny_cfg(**kw):
    base = dict(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=4, head_dim=16, ffn=172, vocab=256,
                max_tokens=64, max_seq=32)
    base.update(kw)
    return hol.make_config(**base)


@pytest.mark.parametrize("bad", [dict(n_q_heads=3, n_kv_heads=2), dict(head_dim=15), dict(hidden=60),
                                 dict(ffn=170, compute_dtype=hol.BF16), dict(ckpt_every_k=0),
                                 dict(max_seq=100), dict(vocab=250, compute_dtype=hol.BF16), dict(ffn=0),
                                 dict(weight_slots=1), dict(weight_slots=9), dict(grad_buffers=1),
                                 dict(grad_buffers=5), dict(async_optimizer=2), dict(async_optimizer=-1)])
def test_create_rejects_bad_config_before_touching_device(bad):
    h = C.c_void_p()
    cfg = _tiny_cfg(**bad)
    st = hol.lib.hol_create(C.byref(cfg), C.byref(h))
    assert st == hol.HOL_EINVAL, hol.lib.hol_last_error()
    assert not h.value


@pytest.mark.parametrize("bad", [dict(n_experts=4, top_k=5, expert_ffn=16, ffn=0),      # top_k > experts
                                 dict(n_experts=600, top_k=2, expert_ffn=16, ffn=0),    # too many experts
                                 dict(n_experts=40, top_k=17, expert_ffn=16, ffn=0),    # top_k above 16
                                 dict(n_experts=4, top_k=0, expert_ffn=16, ffn=0),
                                 dict(n_experts=4, top_k=2, expert_ffn=0, ffn=0),
                                 dict(n_experts=4, top_k=2, expert_ffn=20, ffn=0, compute_dtype=hol.BF16,
                                      vocab=0),
                                 dict(lora_rank=65), dict(lora_rank=-1)])
def test_create_rejects_bad_moe_lora_config(bad):
    h = C.c_void_p()
    cfg = _tiny_cfg(**bad)
    assert hol.lib.hol_create(C.byref(cfg), C.byref(h)) == hol.HOL_EINVAL, hol.lib.hol_last_error()
    assert not h.value


def test_null_arguments_are_einval():
    assert hol.lib.hol_forward_backward(None, None, 0, None) == hol.HOL_EINVAL
    assert hol.lib.hol_forward_backward_async(None, None, 0, None) == hol.HOL_EINVAL
    assert hol.lib.hol_step(None) == hol.HOL_EINVAL
    assert hol.lib.hol_zero_grad(None) == hol.HOL_EINVAL
    assert b"null" in hol.lib.hol_last_error()
