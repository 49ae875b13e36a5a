"""Python binding of ``libhol.so`` (layer-streamed training with host-resident state on MI355X).

Argument marshalling only: every step of the hot path runs in the library's HIP kernels and C++
engine. Importing this package loads the built library; if it is missing the import fails with a
message saying how to build it (there is no fallback implementation).
"""
from __future__ import annotations

import ctypes as C
import json
import os
from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhol.so")

HOL_OK, HOL_EINVAL, HOL_ENOMEM_HOST, HOL_ENOMEM_DEVICE, HOL_EDEVICE, HOL_ESTATE, HOL_EUNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
LOSS_CE, LOSS_SUMSQ = 0, 1

_STATUS = {HOL_EINVAL: "EINVAL", HOL_ENOMEM_HOST: "ENOMEM_HOST", HOL_ENOMEM_DEVICE: "ENOMEM_DEVICE",
           HOL_EDEVICE: "EDEVICE", HOL_ESTATE: "ESTATE", HOL_EUNSUPPORTED: "EUNSUPPORTED"}


class HolError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hol {_STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("expert_ffn", C.c_int32), ("lora_rank", C.c_int32), ("lora_scale", C.c_float),
                ("rope_base", C.c_float), ("rms_eps", C.c_float), ("ckpt_every_k", C.c_int32),
                ("compute_dtype", C.c_int32), ("lr", C.c_float), ("beta1", C.c_float),
                ("beta2", C.c_float), ("adam_eps", C.c_float), ("weight_decay", C.c_float),
                ("device", C.c_int32), ("max_tokens", C.c_int32), ("max_seq", C.c_int32),
                ("weight_slots", C.c_int32), ("grad_buffers", C.c_int32), ("async_optimizer", C.c_int32),
                ("pinned_budget_bytes", C.c_uint64)]


class Batch(C.Structure):
    _fields_ = [("tokens", C.POINTER(C.c_int32)), ("labels", C.POINTER(C.c_int32)),
                ("hidden_in", C.POINTER(C.c_float)), ("batch", C.c_int32), ("seq", C.c_int32),
                ("n_micro", C.c_int32)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python host_offloaded_layer_amd/build.py`")
    lib = C.CDLL(LIB_PATH)
    P, I32, I64, F, D = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_double
    sigs = {
        "hol_create": [C.POINTER(Config), C.POINTER(P)],
        "hol_num_tensors": [P, C.POINTER(I32)],
        "hol_tensor_info": [P, I32, C.c_char_p, C.c_size_t, C.POINTER(I64), C.POINTER(I32), C.POINTER(I32)],
        "hol_set_tensor": [P, I32, P, I64],
        "hol_get_tensor": [P, I32, P, I64],
        "hol_get_grad": [P, I32, P, I64],
        "hol_get_routing": [P, I32, P, I64],
        "hol_get_adam_state": [P, I32, P, P, I64, C.POINTER(I64)],
        "hol_set_adam_state": [P, I32, P, P, I64, I64],
        "hol_zero_grad": [P],
        "hol_set_ckpt_every_k": [P, I32],
        "hol_set_kernel_timing": [P, I32],
        "hol_forward_backward": [P, C.POINTER(Batch), I32, C.POINTER(D)],
        "hol_forward_backward_step": [P, C.POINTER(Batch), I32, C.POINTER(D)],
        "hol_forward_backward_async": [P, C.POINTER(Batch), I32, C.POINTER(D)],
        "hol_step": [P],
        "hol_last_stats": [P, C.c_char_p, C.c_size_t],
        "hol_partition": [P, P, P, P, I32, I64, I32, I32, P, C.POINTER(I32), P, C.POINTER(I32),
                          C.POINTER(I64), C.POINTER(I64)],
        "hol_host_adam": [P, P, P, P, I64, I64, F, F, F, F],
        "hol_host_bf16_round": [P, P, I64],
        "hol_op_gemm": [I32, I32, I32, P, I64, I32, P, I64, I32, P, I64, P, I64, I32, I32, I32, F, P],
        "hol_op_gemm_swiglu": [I32, I32, I32, P, I64, P, I64, P, I64, P, I64, I32, P],
        "hol_op_gemm_rope": [I32, I32, I32, P, I64, P, I64, P, I64, I32, I32, P, P, P],
        "hol_op_gemm_ws": [I32, I32, I32, P, I64, I32, P, I64, I32, P, I64, P, I64, I32, I32, I32, F, P, I64, P],
        "hol_op_gemm_workspace_floats": [],
        "hol_op_rmsnorm_fwd": [P, P, F, P, I32, P, I32, I32, P],
        "hol_op_rmsnorm_bwd": [P, P, P, P, P, I32, P, P, I32, I32, P],
        "hol_op_rope": [P, I32, I64, I32, I32, I32, I32, P, P, I32, P],
        "hol_op_rope_qkv": [P, I64, P, I64, I32, I32, I32, I32, I32, P, P, P],
        "hol_op_swiglu_fwd": [P, P, I32, I32, I32, P],
        "hol_op_swiglu_bwd": [P, P, P, I32, I32, I32, P],
        "hol_op_swiglu_bwd_t": [P, P, P, P, I64, I32, I32, P],
        "hol_op_transpose_bf16": [P, I64, P, I64, I32, I32, P],
        "hol_op_attention_fwd": [I32, I32, I32, I32, I32, I32, P, I64, P, I64, P, I64, P, I64, P, P],
        "hol_op_attention_bwd": [I32, I32, I32, I32, I32, I32, P, I64, P, I64, P, I64, P, I64, P, P, I64,
                                 P, I64, P, I64, P, I64, P, P],
        "hol_op_attention_bwd_rope": [I32, I32, I32, I32, I32, I32, P, I64, P, I64, P, I64, P, I64, P, P, I64,
                                      P, I64, P, I64, P, I64, P, P, P, P],
        "hol_op_attention_bwd_noalloc": [I32, I32, I32, I32, I32, I32, P, I64, P, I64, P, I64, P, I64, P, P,
                                         I64, P, I64, P, I64, P, I64, P],
        "hol_op_cross_entropy": [P, I64, P, P, P, P, I32, I64, I32, I32, P],
        "hol_op_sync": [P],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = C.c_int
    lib.hol_destroy.argtypes = [P]
    lib.hol_destroy.restype = None
    lib.hol_last_error.restype = C.c_char_p
    lib.hol_version.restype = C.c_char_p
    lib.hol_op_rmsnorm_bwd_workspace.argtypes = [I32, I32]
    lib.hol_op_rmsnorm_bwd_workspace.restype = I64
    lib.hol_op_gemm_workspace_floats.restype = I64
    return lib


lib = _load()

# every symbol include/hol.h and include/hol_ops.h declare
EXPORTED = ["hol_create", "hol_destroy", "hol_num_tensors", "hol_tensor_info", "hol_set_tensor",
            "hol_get_tensor", "hol_get_grad", "hol_get_routing", "hol_get_adam_state", "hol_set_adam_state",
            "hol_zero_grad", "hol_set_ckpt_every_k", "hol_set_kernel_timing",
            "hol_forward_backward", "hol_forward_backward_step", "hol_forward_backward_async", "hol_step", "hol_last_stats", "hol_partition",
            "hol_host_adam", "hol_host_bf16_round", "hol_last_error", "hol_version",
            "hol_op_gemm", "hol_op_gemm_rope", "hol_op_gemm_ws", "hol_op_gemm_workspace_floats", "hol_op_gemm_swiglu", "hol_op_rmsnorm_fwd", "hol_op_rmsnorm_bwd_workspace", "hol_op_rmsnorm_bwd",
            "hol_op_rope", "hol_op_rope_qkv", "hol_op_swiglu_fwd", "hol_op_swiglu_bwd", "hol_op_swiglu_bwd_t", "hol_op_transpose_bf16", "hol_op_attention_fwd",
            "hol_op_attention_bwd", "hol_op_attention_bwd_rope", "hol_op_attention_bwd_noalloc", "hol_op_cross_entropy", "hol_op_sync"]


def check(status: int) -> None:
    if status != HOL_OK:
        raise HolError(status, (lib.hol_last_error() or b"").decode(errors="replace"))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ------------------------------------------------------------------------------------------
# model
# ------------------------------------------------------------------------------------------
class Model:
    """One host-resident model driven through the C ABI."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        h = C.c_void_p()
        check(lib.hol_create(C.byref(cfg), C.byref(h)))
        self._h = h
        n = C.c_int32()
        check(lib.hol_num_tensors(h, C.byref(n)))
        self.tensors: List[Tuple[str, Tuple[int, ...], bool]] = []
        name = C.create_string_buffer(256)
        shape = (C.c_int64 * 4)()
        nd, tr = C.c_int32(), C.c_int32()
        for i in range(n.value):
            check(lib.hol_tensor_info(h, i, name, 256, shape, C.byref(nd), C.byref(tr)))
            self.tensors.append((name.value.decode(), tuple(shape[k] for k in range(nd.value)), bool(tr.value)))
        self.index = {t[0]: i for i, t in enumerate(self.tensors)}
        self.trainable = {t[0]: t[2] for t in self.tensors}

    def close(self):
        if getattr(self, "_h", None):
            lib.hol_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def set_tensor(self, name: str, value: np.ndarray) -> None:
        i = self.index[name]
        a = np.ascontiguousarray(value, dtype=np.float32)
        check(lib.hol_set_tensor(self._h, i, _ptr(a), a.size))

    def set_params(self, params: Dict[str, np.ndarray]) -> None:
        for n in self.index:
            self.set_tensor(n, params[n])

    def get_tensor(self, name: str) -> np.ndarray:
        i = self.index[name]
        out = np.empty(self.tensors[i][1], np.float32)
        check(lib.hol_get_tensor(self._h, i, _ptr(out), out.size))
        return out

    def get_routing(self, layer: int, n_tokens: int, top_k: int) -> np.ndarray:
        """Expert ids [n_tokens, top_k] chosen in `layer` by the last forward_backward."""
        out = np.empty((n_tokens, top_k), np.int32)
        check(lib.hol_get_routing(self._h, layer, _ptr(out), out.size))
        return out

    def get_grad(self, name: str) -> np.ndarray:
        i = self.index[name]
        out = np.empty(self.tensors[i][1], np.float32)
        check(lib.hol_get_grad(self._h, i, _ptr(out), out.size))
        return out

    def get_adam_state(self, name: str):
        i = self.index[name]
        m1 = np.empty(self.tensors[i][1], np.float32)
        m2 = np.empty_like(m1)
        st = C.c_int64()
        check(lib.hol_get_adam_state(self._h, i, _ptr(m1), _ptr(m2), m1.size, C.byref(st)))
        return m1, m2, st.value

    def set_adam_state(self, name: str, m1: np.ndarray, m2: np.ndarray, step: int) -> None:
        i = self.index[name]
        a = np.ascontiguousarray(m1, np.float32)
        b = np.ascontiguousarray(m2, np.float32)
        check(lib.hol_set_adam_state(self._h, i, _ptr(a), _ptr(b), a.size, step))

    def zero_grad(self) -> None:
        check(lib.hol_zero_grad(self._h))

    def set_ckpt_every_k(self, k: int) -> None:
        check(lib.hol_set_ckpt_every_k(self._h, k))

    def set_kernel_timing(self, on: bool) -> None:
        check(lib.hol_set_kernel_timing(self._h, int(on)))

    def forward_backward(self, n_micro: int, tokens: Optional[np.ndarray] = None,
                         labels: Optional[np.ndarray] = None, hidden: Optional[np.ndarray] = None,
                         loss: int = LOSS_CE, and_step: bool = False, stale_step: bool = False) -> float:
        """hol_forward_backward; with ``and_step`` hol_forward_backward_step; with ``stale_step``
        hol_forward_backward_async (the accumulated gradient's step overlapped, this call's
        gradient taken at the parameters from before it)."""
        if and_step and stale_step:
            raise ValueError("and_step and stale_step are exclusive")
        b = Batch()
        keep = []
        if tokens is not None:
            t = np.ascontiguousarray(tokens, np.int32)
            keep.append(t)
            b.tokens = t.ctypes.data_as(C.POINTER(C.c_int32))
            b.batch, b.seq = t.shape
        if labels is not None:
            lb = np.ascontiguousarray(labels, np.int32)
            keep.append(lb)
            b.labels = lb.ctypes.data_as(C.POINTER(C.c_int32))
        if hidden is not None:
            hd = np.ascontiguousarray(hidden, np.float32)
            keep.append(hd)
            b.hidden_in = hd.ctypes.data_as(C.POINTER(C.c_float))
            b.batch, b.seq = hd.shape[0], hd.shape[1]
        b.n_micro = n_micro
        out = C.c_double()
        fn = (lib.hol_forward_backward_step if and_step else
              lib.hol_forward_backward_async if stale_step else lib.hol_forward_backward)
        check(fn(self._h, C.byref(b), loss, C.byref(out)))
        return out.value

    def step(self) -> None:
        check(lib.hol_step(self._h))

    def stats(self) -> dict:
        buf = C.create_string_buffer(1 << 20)
        check(lib.hol_last_stats(self._h, buf, 1 << 20))
        return json.loads(buf.value.decode())


def make_config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, *, ckpt_every_k=1,
                compute_dtype=F32, max_tokens, max_seq, n_experts=0, top_k=0, expert_ffn=0,
                lora_rank=0, lora_scale=1.0, rope_base=10000.0, rms_eps=1e-5, lr=1e-3, beta1=0.9,
                beta2=0.999, adam_eps=1e-8, device=0, weight_slots=0, grad_buffers=0,
                async_optimizer=0, pinned_budget_bytes=0) -> Config:
    return Config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_experts, top_k,
                  expert_ffn, lora_rank, lora_scale, rope_base, rms_eps, ckpt_every_k, compute_dtype,
                  lr, beta1, beta2, adam_eps, 0.0, device, max_tokens, max_seq, weight_slots, grad_buffers,
                  async_optimizer, pinned_budget_bytes)


# ------------------------------------------------------------------------------------------
# host-only helpers
# ------------------------------------------------------------------------------------------
def partition(t_f, t_b, m_f, m_b, mem_cap: int, n_gpus: int, n_micro: int):
    """Returns (forward stage starts, backward stage tops, t_max, J)."""
    arrs = [np.ascontiguousarray(x, np.int64) for x in (t_f, t_b, m_f, m_b)]
    L = arrs[0].size
    fb = np.zeros(L, np.int32)
    bb = np.zeros(L, np.int32)
    nf, nb = C.c_int32(), C.c_int32()
    tmax, J = C.c_int64(), C.c_int64()
    check(lib.hol_partition(*[_ptr(a) for a in arrs], L, mem_cap, n_gpus, n_micro, _ptr(fb), C.byref(nf),
                            _ptr(bb), C.byref(nb), C.byref(tmax), C.byref(J)))
    return fb[:nf.value].tolist(), bb[:nb.value].tolist(), tmax.value, J.value


def host_adam(theta, grad, m, v, step_t, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8):
    for a in (theta, grad, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    check(lib.hol_host_adam(_ptr(theta), _ptr(grad), _ptr(m), _ptr(v), theta.size, step_t, lr, beta1, beta2, eps))


def host_bf16_round(x: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    check(lib.hol_host_bf16_round(_ptr(a), _ptr(out), a.size))
    return out


def version() -> str:
    return lib.hol_version().decode()
