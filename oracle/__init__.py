"""ctypes front end of the fp64 CPU oracle (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use this package. The product path never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

import synth

_HERE = os.path.dirname(os.path.abspath(__file__))

# kind strings of synth.tensor_list -> ORC_* enum of oracle.h
KINDS = ["embed", "final_norm", "lm_head", "attn_norm", "wq", "wk", "wv", "wo", "w_dq", "q_norm", "w_uq",
         "w_dkv", "kv_norm", "w_uk", "w_uv", "kda_wq", "kda_wk", "kda_wv", "kda_alpha", "kda_beta", "moe_norm",
         "router", "sh_gate", "sh_up", "sh_down", "exp_gate", "exp_up", "exp_down"]
KIND_ID = {k: i for i, k in enumerate(KINDS)}


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "hidden", "vocab", "attn_kind", "n_heads", "n_kv_heads", "head_dim", "q_lora", "kv_lora",
        "rope_dim", "nope_dim", "v_dim", "kda_dk", "kda_dv", "hybrid_period", "n_experts", "top_k", "ffn",
        "shared_ffn", "norm_topk", "expert_pool_layers", "kv_capacity", "mla_explicit")] + [
        ("rms_eps", ctypes.c_double), ("rope_theta", ctypes.c_double)]


class OrcIO(ctypes.Structure):
    _fields_ = [("kcache", ctypes.c_void_p), ("vcache", ctypes.c_void_p), ("latent", ctypes.c_void_p),
                ("kda_state", ctypes.c_void_p), ("cache_batch", ctypes.c_int32), ("sel", ctypes.c_void_p),
                ("probs", ctypes.c_void_p), ("x_trace", ctypes.c_void_p), ("force_sel", ctypes.c_void_p)]


FILL_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_size_t,
                           ctypes.c_void_p)

_lib = None


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-ffp-contract=off",
           "-o", "liboracle.so.tmp", "oracle.c", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(os.path.join(_HERE, "liboracle.so.tmp"), os.path.join(_HERE, "liboracle.so"))


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        L.orc_decode_step.restype = ctypes.c_int
        L.orc_decode_step.argtypes = [ctypes.POINTER(OrcConfig), FILL_FN, vp, i32, i32, i32, vp,
                                      ctypes.POINTER(OrcIO), vp]
        L.orc_rmsnorm.argtypes = [vp, vp, i32, dbl, vp]
        L.orc_rope.argtypes = [vp, i32, i32, dbl]
        L.orc_softmax.argtypes = [vp, i32, vp]
        L.orc_topk.argtypes = [vp, i32, i32, vp]
        L.orc_silu.restype = dbl
        L.orc_silu.argtypes = [dbl]
        L.orc_round_bf16.restype = ctypes.c_uint16
        L.orc_round_bf16.argtypes = [dbl]
        L.orc_matvec.argtypes = [vp, i32, i32, vp, vp]
        L.orc_kda_head.argtypes = [vp, i32, i32, vp, dbl, vp, vp, vp, vp]
        _lib = L
    return _lib


def to_orc_config(cfg: synth.ModelConfig, mla_explicit: bool = False) -> OrcConfig:
    c = OrcConfig()
    for name, _ in OrcConfig._fields_:
        if name == "mla_explicit":
            c.mla_explicit = int(mla_explicit)
        else:
            setattr(c, name, getattr(cfg, name))
    return c


class Provider:
    """Weight provider for the oracle: synthetic tensors from `spec`, with optional overrides.

    overrides: tensor name -> numpy array (uint16 bf16 patterns, or float32 for alpha/beta).
    """

    def __init__(self, cfg: synth.ModelConfig, spec: synth.Spec, overrides: dict | None = None):
        self.cfg, self.spec = cfg, spec
        self.overrides = overrides or {}
        self.by_key = {}
        for t in synth.tensor_list(cfg):
            self.by_key[(KIND_ID[t.kind], t.layer, t.expert)] = t
        self.fetched = []  # (name, n) log, used by the byte model
        self._cb = FILL_FN(self._fill)

    def _fill(self, _user, kind, layer, expert, n, out):
        t = self.by_key[(kind, layer, expert)]
        self.fetched.append((t.name, int(n)))
        if t.name in self.overrides:
            arr = np.ascontiguousarray(self.overrides[t.name]).reshape(-1)
            assert arr.size == n, (t.name, arr.size, n)
            ctypes.memmove(out, arr.ctypes.data, arr.nbytes)
            return
        L, s = synth.lib(), self.spec
        k = synth.key(s.seed, t.name)
        if t.dist == "normal":
            L.synth_normal_bf16(k, synth.scale(s.sigma_for(t.kind)), 0, n, out)
        elif t.dist == "gain":
            L.synth_gain_bf16(k, synth.scale(s.gain_sigma), n, out)
        else:
            L.synth_sigmoid_normal_f32(k, n, out)

    @property
    def callback(self):
        return self._cb


def decode_step(cfg: synth.ModelConfig, provider: Provider, tokens: np.ndarray, kv_len: int, caches: dict,
                cache_batch: int | None = None, trace: bool = False, x_trace: bool = False,
                force_sel: np.ndarray | None = None, mla_explicit: bool = False) -> dict:
    """Run one decode step. `caches` (from synth.host_caches) is updated in place.

    Returns {"logits": [B][T][V] float64, "sel": [L][M][k], "probs": [L][M][E], "x": [L+1][M][H]}.
    """
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    B, T = tokens.shape
    M = B * T
    c = to_orc_config(cfg, mla_explicit)
    io = OrcIO()
    io.cache_batch = cache_batch or B
    for key, field in (("k", "kcache"), ("v", "vcache"), ("latent", "latent"), ("kda_state", "kda_state")):
        if key in caches:
            assert caches[key].flags.c_contiguous
            setattr(io, field, caches[key].ctypes.data)
    out = {"logits": np.zeros((B, T, cfg.vocab), dtype=np.float64)}
    if trace:
        out["sel"] = np.zeros((cfg.n_layers, M, cfg.top_k), dtype=np.int32)
        out["probs"] = np.zeros((cfg.n_layers, M, cfg.n_experts), dtype=np.float64)
        io.sel, io.probs = out["sel"].ctypes.data, out["probs"].ctypes.data
    if x_trace:
        out["x"] = np.zeros((cfg.n_layers + 1, M, cfg.hidden), dtype=np.float64)
        io.x_trace = out["x"].ctypes.data
    if force_sel is not None:
        fs = np.ascontiguousarray(force_sel, dtype=np.int32)
        assert fs.shape == (cfg.n_layers, M, cfg.top_k)
        io.force_sel = fs.ctypes.data
    rc = lib().orc_decode_step(ctypes.byref(c), provider.callback, None, B, T, kv_len, tokens.ctypes.data,
                               ctypes.byref(io), out["logits"].ctypes.data)
    if rc != 0:
        raise ValueError("orc_decode_step rejected its arguments")
    return out
