"""Seeded synthetic inputs for the decode step: workloads, tensor list, generators.

This package holds no arithmetic of the decode step. It defines the five model
workloads (shapes only), the list of tensors each model has, and the seeded
generator that turns (seed, tensor name, element index) into values. The
oracle and the HIP path are both fed from here and from nowhere else.

The generator is defined in ``synth.h``; ``libsynth.so`` is its host
implementation and ``libsynth_dev.so`` its device implementation (bit-identical).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

ATTN_GQA, ATTN_MLA, ATTN_HYBRID = 0, 1, 2


@dataclass(frozen=True)
class ModelConfig:
    """Shapes of one decoder. Field names follow the C structs of the library and oracle."""

    name: str
    n_layers: int
    hidden: int
    vocab: int
    attn_kind: int
    n_heads: int = 0  # GQA query heads, MLA heads, KDA heads
    n_kv_heads: int = 0  # GQA only
    head_dim: int = 0  # GQA only
    q_lora: int = 0
    kv_lora: int = 0
    rope_dim: int = 0
    nope_dim: int = 0
    v_dim: int = 0
    kda_dk: int = 0
    kda_dv: int = 0
    hybrid_period: int = 0  # layer l is MLA iff l % period == period - 1
    n_experts: int = 0
    top_k: int = 0
    ffn: int = 0
    shared_ffn: int = 0
    norm_topk: int = 0
    expert_pool_layers: int = 0  # 0: one expert set per layer
    max_batch: int = 1
    max_new_tokens: int = 8
    kv_capacity: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e4

    # ---- derived helpers (shapes only) ----
    def layer_kind(self, layer: int) -> str:
        if self.attn_kind == ATTN_GQA:
            return "gqa"
        if self.attn_kind == ATTN_MLA:
            return "mla"
        return "mla" if layer % self.hybrid_period == self.hybrid_period - 1 else "kda"

    def pool_slot(self, layer: int) -> int:
        return layer % self.expert_pool_layers if self.expert_pool_layers else layer

    @property
    def n_pool(self) -> int:
        return self.expert_pool_layers or self.n_layers

    @property
    def latent_dim(self) -> int:
        return self.kv_lora + self.rope_dim

    def attention_layers(self) -> list[int]:
        return [l for l in range(self.n_layers) if self.layer_kind(l) != "kda"]

    def kda_layers(self) -> list[int]:
        return [l for l in range(self.n_layers) if self.layer_kind(l) == "kda"]


@dataclass(frozen=True)
class Workload:
    """One measured or tested configuration: a model plus step shape."""

    name: str
    model: ModelConfig
    batch: int
    new_tokens: int
    kv_len: int
    description: str = ""


# --------------------------------------------------------------------------------------
# The five workloads: a tiny and a mid-size MoE decoder, the K3-scale one-GPU share at batch 1-8,
# its speculative-verify step (1 + 6 draft tokens) and the hybrid delta-rule / MLA variant.
# --------------------------------------------------------------------------------------
TINY = ModelConfig(
    name="tiny-moe", n_layers=2, hidden=256, vocab=1024, attn_kind=ATTN_GQA,
    n_heads=4, n_kv_heads=4, head_dim=64, n_experts=8, top_k=2, ffn=512, shared_ffn=0,
    max_batch=8, max_new_tokens=8, kv_capacity=136)

MID = ModelConfig(
    name="mid-moe", n_layers=8, hidden=2048, vocab=32000, attn_kind=ATTN_GQA,
    n_heads=16, n_kv_heads=4, head_dim=128, n_experts=64, top_k=8, ffn=768, shared_ffn=768,
    max_batch=4, max_new_tokens=8, kv_capacity=2056)

K3 = ModelConfig(
    name="k3-share", n_layers=92, hidden=7168, vocab=40960, attn_kind=ATTN_MLA,
    n_heads=16, q_lora=1536, kv_lora=512, rope_dim=64, nope_dim=128, v_dim=128,
    n_experts=48, top_k=1, ffn=2048, shared_ffn=512, expert_pool_layers=46,
    max_batch=8, max_new_tokens=8, kv_capacity=4104)

K3_HYBRID = replace(
    K3, name="k3-hybrid", attn_kind=ATTN_HYBRID, kda_dk=128, kda_dv=128, hybrid_period=4)

# The dense second model: a MoE-free bf16 GQA decoder of about 27 B parameters, the size of the
# dense decoder the pages serve next to the MoE model. The pages give no dimensions; these are
# synthetic choices. n_experts = 0: the feed-forward block is the one SwiGLU block of width
# shared_ffn. The whole model fits one GPU (about 53 GB of bf16 weights).
DENSE = ModelConfig(
    name="dense-27b", n_layers=64, hidden=5120, vocab=151936, attn_kind=ATTN_GQA,
    n_heads=40, n_kv_heads=8, head_dim=128, n_experts=0, top_k=0, ffn=0, shared_ffn=21504,
    max_batch=8, max_new_tokens=8, kv_capacity=4104, rope_theta=1e6)

WORKLOADS = {
    "c1": Workload("c1", TINY, 1, 1, 128, "tiny MoE decoder, batch 1"),
    "c2": Workload("c2", MID, 1, 1, 2048, "mid-size GQA MoE, batch 1"),
    "c2b4": Workload("c2b4", MID, 4, 1, 2048, "mid-size GQA MoE, batch 4"),
    "c3": Workload("c3", K3, 1, 1, 4096, "K3-scale one-GPU share, batch 1"),
    "c3b2": Workload("c3b2", K3, 2, 1, 4096, "K3-scale one-GPU share, batch 2"),
    "c3b4": Workload("c3b4", K3, 4, 1, 4096, "K3-scale one-GPU share, batch 4"),
    "c3b8": Workload("c3b8", K3, 8, 1, 4096, "K3-scale one-GPU share, batch 8"),
    "c4": Workload("c4", K3, 1, 7, 4096, "speculative verify: 1 + 6 draft tokens"),
    "c5": Workload("c5", K3_HYBRID, 8, 1, 4096, "hybrid delta-rule / MLA, batch 8"),
    "dense": Workload("dense", DENSE, 1, 1, 4096, "dense 27B-class GQA decoder, batch 1"),
}


# --------------------------------------------------------------------------------------
# Tensor list
# --------------------------------------------------------------------------------------
@dataclass(frozen=True)
class TensorSpec:
    name: str  # generator stream name
    kind: str  # weight kind (mapped to the library's and the oracle's enums)
    layer: int  # layer, pool slot for experts, -1 for global tensors
    expert: int  # expert index or -1
    shape: tuple
    dist: str  # "normal" (bf16), "gain" (bf16), "sigmoid" (fp32)


@dataclass
class Spec:
    """Seed and scales of the synthetic inputs."""

    seed: int = 0
    sigma: float = 0.02  # weight matrices
    gain_sigma: float = 0.02  # norm gains are 1 + N(0, gain_sigma)
    cache_sigma: float = 1.0
    state_sigma: float = 1.0
    sigma_by_kind: dict = field(default_factory=dict)  # per-kind overrides (stress variants)

    def sigma_for(self, kind: str) -> float:
        return self.sigma_by_kind.get(kind, self.sigma)


def tensor_list(cfg: ModelConfig) -> list[TensorSpec]:
    H, V = cfg.hidden, cfg.vocab
    out = [
        TensorSpec("embed", "embed", -1, -1, (V, H), "normal"),
        TensorSpec("final_norm", "final_norm", -1, -1, (H,), "gain"),
        TensorSpec("lm_head", "lm_head", -1, -1, (V, H), "normal"),
    ]
    for l in range(cfg.n_layers):
        p = f"L{l}."
        t = lambda k, shape, dist="normal": TensorSpec(p + k, k, l, -1, tuple(shape), dist)
        out.append(t("attn_norm", (H,), "gain"))
        kind = cfg.layer_kind(l)
        if kind == "gqa":
            nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
            out += [t("wq", (nq * d, H)), t("wk", (nkv * d, H)), t("wv", (nkv * d, H)), t("wo", (H, nq * d))]
        elif kind == "mla":
            nh = cfg.n_heads
            out += [
                t("w_dq", (cfg.q_lora, H)),
                t("q_norm", (cfg.q_lora,), "gain"),
                t("w_uq", (nh * (cfg.nope_dim + cfg.rope_dim), cfg.q_lora)),
                t("w_dkv", (cfg.kv_lora + cfg.rope_dim, H)),
                t("kv_norm", (cfg.kv_lora,), "gain"),
                t("w_uk", (nh, cfg.nope_dim, cfg.kv_lora)),
                t("w_uv", (nh, cfg.v_dim, cfg.kv_lora)),
                t("wo", (H, nh * cfg.v_dim)),
            ]
        else:
            nh, dk, dv = cfg.n_heads, cfg.kda_dk, cfg.kda_dv
            out += [
                t("kda_wq", (nh * dk, H)),
                t("kda_wk", (nh * dk, H)),
                t("kda_wv", (nh * dv, H)),
                t("kda_alpha", (nh, dk), "sigmoid"),
                t("kda_beta", (nh,), "sigmoid"),
                t("wo", (H, nh * dv)),
            ]
        out.append(t("moe_norm", (H,), "gain"))
        if cfg.n_experts:
            out.append(t("router", (cfg.n_experts, H)))
        if cfg.shared_ffn:
            out += [t("sh_gate", (cfg.shared_ffn, H)), t("sh_up", (cfg.shared_ffn, H)),
                    t("sh_down", (H, cfg.shared_ffn))]
    for s in range(cfg.n_pool):
        for e in range(cfg.n_experts):
            p = f"X{s}.{e}."
            out += [
                TensorSpec(p + "gate", "exp_gate", s, e, (cfg.ffn, H), "normal"),
                TensorSpec(p + "up", "exp_up", s, e, (cfg.ffn, H), "normal"),
                TensorSpec(p + "down", "exp_down", s, e, (H, cfg.ffn), "normal"),
            ]
    return out


def numel(shape) -> int:
    n = 1
    for s in shape:
        n *= int(s)
    return n


# --------------------------------------------------------------------------------------
# Host generator (ctypes over libsynth.so)
# --------------------------------------------------------------------------------------
_lib = None
_dev = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u64, f32, sz = ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t
        L.synth_mix64.restype = u64
        L.synth_mix64.argtypes = [u64]
        L.synth_fnv1a64.restype = u64
        L.synth_fnv1a64.argtypes = [ctypes.c_char_p]
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, ctypes.c_char_p]
        L.synth_scale.restype = f32
        L.synth_scale.argtypes = [ctypes.c_double]
        L.synth_ih.restype = ctypes.c_int32
        L.synth_ih.argtypes = [u64, u64]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_f32_to_bf16.argtypes = [f32]
        vp = ctypes.c_void_p
        L.synth_normal_bf16.argtypes = [u64, f32, u64, sz, vp]
        L.synth_normal_f32.argtypes = [u64, f32, u64, sz, vp]
        L.synth_gain_bf16.argtypes = [u64, f32, sz, vp]
        L.synth_sigmoid_normal_f32.argtypes = [u64, sz, vp]
        L.synth_tokens.argtypes = [u64, ctypes.c_uint32, sz, vp]
        _lib = L
    return _lib


def key(seed: int, name: str) -> int:
    return lib().synth_key(seed & 0xFFFFFFFFFFFFFFFF, name.encode())


def scale(sigma: float) -> float:
    return lib().synth_scale(sigma)


def normal_bf16(seed: int, name: str, n: int, sigma: float, off: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of the stream `name`, elements off..off+n-1."""
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(key(seed, name), scale(sigma), off, n, out.ctypes.data)
    return out


def normal_f32(seed: int, name: str, n: int, sigma: float, off: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(key(seed, name), scale(sigma), off, n, out.ctypes.data)
    return out


def gain_bf16(seed: int, name: str, n: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_gain_bf16(key(seed, name), scale(sigma), n, out.ctypes.data)
    return out


def sigmoid_normal_f32(seed: int, name: str, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_sigmoid_normal_f32(key(seed, name), n, out.ctypes.data)
    return out


def tokens(seed: int, step: int, vocab: int, batch: int, new_tokens: int) -> np.ndarray:
    out = np.empty(batch * new_tokens, dtype=np.int32)
    lib().synth_tokens(key(seed, f"tokens.step{step}"), vocab, out.size, out.ctypes.data)
    return out.reshape(batch, new_tokens)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


def host_tensor(spec: Spec, t: TensorSpec) -> np.ndarray:
    """Generate tensor t on the host. bf16 tensors come back as uint16 bit patterns."""
    n = numel(t.shape)
    if t.dist == "normal":
        return normal_bf16(spec.seed, t.name, n, spec.sigma_for(t.kind)).reshape(t.shape)
    if t.dist == "gain":
        return gain_bf16(spec.seed, t.name, n, spec.gain_sigma).reshape(t.shape)
    if t.dist == "sigmoid":
        return sigmoid_normal_f32(spec.seed, t.name, n).reshape(t.shape)
    raise ValueError(t.dist)


# ---- caches and recurrent state (stream names and element numbering) ----
GQA_POS_STRIDE = 1 << 20  # element (head, pos, j) of a GQA cache stream is (head * 2^20 + pos) * d + j


def gqa_cache_stream(which: str, layer: int, b: int) -> str:
    return f"cache{which}.L{layer}.b{b}"  # which in {"K", "V"}


def latent_cache_stream(layer: int, b: int) -> str:
    return f"latent.L{layer}.b{b}"  # element (pos, j) is pos * (kv_lora + rope) + j


def kda_state_stream(layer: int, b: int) -> str:
    return f"kda_state.L{layer}.b{b}"  # element (h, i, j) is (h * dk + i) * dv + j


# --------------------------------------------------------------------------------------
# Device generator (ctypes over libsynth_dev.so)
# --------------------------------------------------------------------------------------
def dev():
    global _dev
    if _dev is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        u64, f32, vp = ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p
        for fn in (L.synth_dev_normal_bf16, L.synth_dev_normal_f32):
            fn.restype = ctypes.c_int
            fn.argtypes = [u64, f32, u64, u64, vp, vp]
        _dev = L
    return _dev


def dev_normal_bf16(seed: int, name: str, sigma: float, off: int, n: int, d_ptr: int, stream: int = 0):
    rc = dev().synth_dev_normal_bf16(key(seed, name), scale(sigma), off, n, d_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_bf16 failed: hip error {rc}")


def dev_normal_f32(seed: int, name: str, sigma: float, off: int, n: int, d_ptr: int, stream: int = 0):
    rc = dev().synth_dev_normal_f32(key(seed, name), scale(sigma), off, n, d_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_f32 failed: hip error {rc}")


def build(verbose: bool = False) -> None:
    """Compile libsynth.so (gcc) and libsynth_dev.so (hipcc, gfx950)."""
    import subprocess

    def run(cmd):
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True, cwd=_HERE)

    run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
         "-o", "libsynth.so.tmp", "synth.c", "-lm"])
    os.replace(os.path.join(_HERE, "libsynth.so.tmp"), os.path.join(_HERE, "libsynth.so"))
    run(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", "libsynth_dev.so.tmp", "synth_dev.hip"])
    os.replace(os.path.join(_HERE, "libsynth_dev.so.tmp"), os.path.join(_HERE, "libsynth_dev.so"))


# --------------------------------------------------------------------------------------
# Host-side caches and state in the documented device layouts
#   GQA    K, V    [n_layers][cache_batch][n_kv][kv_capacity][head_dim]  bf16
#   MLA    latent  [n_mla_layers][cache_batch][kv_capacity][kv_lora+rope] bf16
#   KDA    state   [n_kda_layers][cache_batch][n_heads][dk][dv]        fp32
# Positions < kv_len hold generated values, the rest zeros.
# --------------------------------------------------------------------------------------
def host_caches(cfg: ModelConfig, spec: Spec, batch: int, kv_len: int, cache_batch: int | None = None) -> dict:
    cb = cache_batch or batch
    cap = cfg.kv_capacity
    out = {}
    if cfg.attn_kind == ATTN_GQA:
        nkv, d = cfg.n_kv_heads, cfg.head_dim
        for which in ("K", "V"):
            arr = np.zeros((cfg.n_layers, cb, nkv, cap, d), dtype=np.uint16)
            for l in range(cfg.n_layers):
                for b in range(batch):
                    for g in range(nkv):
                        vals = normal_bf16(spec.seed, gqa_cache_stream(which, l, b), kv_len * d,
                                           spec.cache_sigma, off=g * GQA_POS_STRIDE * d)
                        arr[l, b, g, :kv_len, :] = vals.reshape(kv_len, d)
            out["k" if which == "K" else "v"] = arr
    else:
        mla = cfg.attention_layers()
        lat = cfg.latent_dim
        arr = np.zeros((len(mla), cb, cap, lat), dtype=np.uint16)
        for o, l in enumerate(mla):
            for b in range(batch):
                arr[o, b, :kv_len, :] = normal_bf16(spec.seed, latent_cache_stream(l, b), kv_len * lat,
                                                    spec.cache_sigma).reshape(kv_len, lat)
        out["latent"] = arr
        kda = cfg.kda_layers()
        if kda:
            nh, dk, dv = cfg.n_heads, cfg.kda_dk, cfg.kda_dv
            st = np.zeros((len(kda), cb, nh, dk, dv), dtype=np.float32)
            for o, l in enumerate(kda):
                for b in range(batch):
                    st[o, b] = normal_f32(spec.seed, kda_state_stream(l, b), nh * dk * dv,
                                          spec.state_sigma).reshape(nh, dk, dv)
            out["kda_state"] = st
    return out
