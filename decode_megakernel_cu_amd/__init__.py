"""Python binding of libmk.so, the one-launch MoE decode megakernel for MI355X.

Argument marshalling only: every step of the decode path runs in the library's
HIP kernels. The function names mirror the C ABI in ``include/mk.h``. Importing
this package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MK_LIBRARY: another build of the same library (e.g. one compiled with different options);
# default: the in-tree build
LIB_PATH = os.environ.get("MK_LIBRARY") or os.path.join(_HERE, "libmk.so")

MK_OK, MK_E_INVAL, MK_E_STATE, MK_E_KV_OVERFLOW, MK_E_NOMEM, MK_E_HIP, MK_E_DEVICE, MK_E_UNSUPPORTED = (
    0, -1, -2, -3, -4, -5, -6, -7)
MK_MAX_M, MK_MAX_BATCH, MK_MAX_NEW_TOKENS, MK_DEVICE_NONE = 16, 8, 8, -1
MK_MAX_KV_CAPACITY = 1 << 20

# weight kinds, in the order of mk_weight_kind
KINDS = ["embed", "final_norm", "lm_head", "attn_norm", "wq", "wk", "wv", "wo", "w_dq", "q_norm", "w_uq",
         "w_dkv", "kv_norm", "w_uk", "w_uv", "kda_wq", "kda_wk", "kda_wv", "kda_alpha", "kda_beta", "moe_norm",
         "router", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"]
KIND_ID = {k: i for i, k in enumerate(KINDS)}

TRACE_STAMPS = 16  # MK_TRACE_STAMPS

EXPORTS = ["mk_config_preset", "mk_query_sizes", "mk_create", "mk_load_weights", "mk_decode_step", "mk_decode_step_static",
           "mk_decode_step_greedy", "mk_decode_step_sample", "mk_poll", "mk_set_trace", "mk_read_trace", "mk_set_matrix_cores", "mk_last_error",
           "mk_destroy"]


class MkConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "preset", "n_layers", "hidden", "vocab", "attn_kind", "n_heads", "n_kv_heads", "head_dim", "q_lora", "kv_lora",
        "rope_dim", "nope_dim", "v_dim", "kda_dk", "kda_dv", "hybrid_period", "n_experts", "top_k", "ffn",
        "shared_ffn", "norm_topk", "expert_pool_layers", "max_batch", "max_new_tokens", "kv_capacity")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class MkSizes(ctypes.Structure):
    _fields_ = [("arena_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64),
                ("kv_bytes", ctypes.c_uint64), ("kda_state_bytes", ctypes.c_uint64)]


class MkTensorDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("src_on_device", ctypes.c_int32), ("src", ctypes.c_void_p), ("bytes", ctypes.c_uint64)]


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mk error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64
    L.mk_config_preset.argtypes = [ctypes.c_int, ctypes.POINTER(MkConfig)]
    L.mk_query_sizes.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkSizes)]
    L.mk_create.argtypes = [ctypes.POINTER(MkConfig), i32, vp, u64, vp, u64, ctypes.POINTER(vp)]
    L.mk_load_weights.argtypes = [vp, ctypes.POINTER(MkTensorDesc), i32, vp]
    L.mk_decode_step.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.mk_decode_step_static.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    L.mk_decode_step_greedy.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.mk_decode_step_sample.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float, vp, vp, vp]
    L.mk_poll.argtypes = [vp]
    L.mk_last_error.restype = ctypes.c_char_p
    L.mk_last_error.argtypes = []
    L.mk_destroy.argtypes = [vp]
    L.mk_destroy.restype = None
    L.mk_set_trace.argtypes = [vp, i32]
    L.mk_set_matrix_cores.argtypes = [vp, i32]
    L.mk_read_trace.argtypes = [vp, vp, u64, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    for f in ("mk_config_preset", "mk_query_sizes", "mk_create", "mk_load_weights", "mk_decode_step",
              "mk_decode_step_static", "mk_decode_step_greedy",
              "mk_decode_step_sample", "mk_poll", "mk_set_trace", "mk_read_trace", "mk_set_matrix_cores"):
        getattr(L, f).restype = ctypes.c_int
    return L


lib = _load()


def mk_last_error() -> str:
    return lib.mk_last_error().decode()


def _check(rc: int) -> int:
    if rc != MK_OK:
        raise MkError(rc, mk_last_error())
    return rc


def config(model) -> MkConfig:
    """mk_config from any object carrying the fields of the C struct (e.g. synth.ModelConfig; a
    missing `preset` reads as 0, a custom model)."""
    c = MkConfig()
    for name, _ in MkConfig._fields_:
        setattr(c, name, getattr(model, name, 0) if name == "preset" else getattr(model, name))
    return c


def mk_config_preset(preset_id: int) -> MkConfig:
    """The library's description of a preset workload model (ids 1..6, see include/mk.h)."""
    c = MkConfig()
    _check(lib.mk_config_preset(int(preset_id), ctypes.byref(c)))
    return c


def mk_query_sizes(cfg: MkConfig) -> MkSizes:
    s = MkSizes()
    _check(lib.mk_query_sizes(ctypes.byref(cfg), ctypes.byref(s)))
    return s


def mk_create(cfg: MkConfig, device: int, arena: int, arena_bytes: int, workspace: int, workspace_bytes: int):
    h = ctypes.c_void_p()
    _check(lib.mk_create(ctypes.byref(cfg), device, arena, arena_bytes, workspace, workspace_bytes, ctypes.byref(h)))
    return h


def mk_load_weights(ctx, descs, stream: int = 0) -> None:
    arr = (MkTensorDesc * len(descs))(*descs)
    _check(lib.mk_load_weights(ctx, arr, len(descs), stream))


def mk_decode_step(ctx, batch: int, n_new_tokens: int, kv_len: int, tokens: int, kv: int, kda_state: int,
                   logits: int, route: int = 0, stream: int = 0) -> None:
    _check(lib.mk_decode_step(ctx, batch, n_new_tokens, kv_len, tokens, kv, kda_state or None, logits,
                              route or None, stream))


def mk_decode_step_static(ctx, batch: int, n_new_tokens: int, kv_len: int, tokens: int, kv: int, kda_state: int,
                          logits: int, route: int = 0, stream: int = 0) -> None:
    """mk_decode_step on the library's static per-GPU workspace (allocates nothing)."""
    _check(lib.mk_decode_step_static(ctx, batch, n_new_tokens, kv_len, tokens, kv, kda_state or None, logits,
                                     route or None, stream))


def mk_decode_step_greedy(ctx, batch: int, n_new_tokens: int, kv_len: int, tokens: int, kv: int, kda_state: int,
                          logits: int, argmax: int, accepted: int = 0, stream: int = 0) -> None:
    """The step with greedy selection fused after the LM head (logits and accepted may be 0)."""
    _check(lib.mk_decode_step_greedy(ctx, batch, n_new_tokens, kv_len, tokens, kv, kda_state or None, logits or None,
                                     argmax or None, accepted or None, stream))


def mk_decode_step_sample(ctx, batch: int, n_new_tokens: int, kv_len: int, tokens: int, kv: int, kda_state: int,
                          logits: int, temperature: float, top_p: float, uniform: int, sampled: int,
                          stream: int = 0) -> None:
    """The step with temperature / top-p sampling fused after the LM head (uniform: the caller's numbers)."""
    _check(lib.mk_decode_step_sample(ctx, batch, n_new_tokens, kv_len, tokens, kv, kda_state or None, logits or None,
                                     float(temperature), float(top_p), uniform or None, sampled or None, stream))


def mk_poll(ctx) -> None:
    _check(lib.mk_poll(ctx))


def mk_destroy(ctx) -> None:
    lib.mk_destroy(ctx)


def tensor_desc(kind: str, layer: int, expert: int, src: int, nbytes: int, on_device: bool) -> MkTensorDesc:
    return MkTensorDesc(KIND_ID[kind], layer, expert, int(on_device), src, nbytes)


def mk_set_trace(ctx, enable: bool) -> None:
    _check(lib.mk_set_trace(ctx, int(enable)))


MK_MFMA_MIN_ROWS = 3  # MK_MFMA_MIN_ROWS
MK_MFMA_MIN_ROWS_DENSE = 2  # MK_MFMA_MIN_ROWS_DENSE
MK_MAX_M = 16


def mk_set_matrix_cores(ctx, min_rows: int) -> None:
    """GEMV phases of steps with at least min_rows token rows on the matrix cores (> MK_MAX_M: never)."""
    _check(lib.mk_set_matrix_cores(ctx, int(min_rows)))


def mk_read_trace(ctx):
    """Trace of the last step as a numpy array [n_barriers + 1][n_blocks][TRACE_STAMPS] of wall-clock
    ticks (stamp meanings in include/mk.h)."""
    import numpy as np

    nb, nk = ctypes.c_int(), ctypes.c_int()
    _check(lib.mk_read_trace(ctx, None, 0, ctypes.byref(nb), ctypes.byref(nk)))
    out = np.zeros((nb.value + 1, nk.value, TRACE_STAMPS), dtype=np.uint64)
    _check(lib.mk_read_trace(ctx, out.ctypes.data, out.size, ctypes.byref(nb), ctypes.byref(nk)))
    return out
