"""Independent float64 brute-force reference of one decode step, in numpy (test infrastructure).

A second, separately written definition of the step, used only to pin the C oracle on tiny
shapes. It shares nothing with the oracle but the seeded input generator. It is written in
array form from the plain definitions of each block (the step the pages fuse into one program:
"tpu-megakernels README", FAQ "why build a custom megakernel"; the MLA / delta-rule layers of
the model: German news article, section "Auf dem Papier liegt der GB200 vorn"), and it differs
from the oracle on purpose where two forms are equivalent:

- MLA runs in the explicit form: every head's keys and values are reconstructed from the
  latent cache (K = C W_uk^T, V = C W_uv^T), then plain softmax attention; the oracle (like the
  GPU) uses the absorbed form.
- bf16 rounding is done on the bits of the float64 value (round half to even on the 45
  discarded mantissa bits, then the float32 pattern's top half), not by frexp/nearbyint.
- top-k comes from a stable argsort of the probabilities.
- the delta rule is written as S <- (I - beta k k^T) diag(alpha) S + beta k v^T.
"""
from __future__ import annotations

import numpy as np

import synth


def bf16_round(x) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even), returned as float64. Exact for finite normal
    inputs in bf16 range: rounds the float64 bits to 7 stored mantissa bits in one step."""
    x = np.asarray(x, dtype=np.float64)
    b = x.view(np.uint64).copy()
    drop = np.uint64(52 - 7)
    half = np.uint64(1) << (drop - np.uint64(1))
    keep_lsb = (b >> drop) & np.uint64(1)
    b = b + (half - np.uint64(1)) + keep_lsb
    b = b & ~((np.uint64(1) << drop) - np.uint64(1))
    return b.view(np.float64)


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of values already representable in bf16 (float64 in)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf(u16) -> np.ndarray:
    return synth.bf16_to_f32(np.asarray(u16, dtype=np.uint16)).astype(np.float64)


class Weights:
    """float64 copies of every tensor of a model, with optional overrides (bf16 patterns / fp32)."""

    def __init__(self, cfg, spec, overrides=None):
        self.t = {}
        ov = overrides or {}
        for t in synth.tensor_list(cfg):
            a = ov[t.name] if t.name in ov else synth.host_tensor(spec, t)
            a = np.asarray(a).reshape(t.shape)
            self.t[t.name] = bf(a) if a.dtype == np.uint16 else a.astype(np.float64)

    def __getitem__(self, k):
        return self.t[k]


def rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rotate(x, pos, theta):
    """RoPE on the last axis with pairs (j, j + d/2) at frequency theta^(-2j/d); pos broadcast."""
    d = x.shape[-1]
    h = d // 2
    freq = theta ** (-np.arange(h, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def softmax(s, axis=-1):
    e = np.exp(s - s.max(axis=axis, keepdims=True))
    return e / e.sum(axis=axis, keepdims=True)


def silu(z):
    return z / (1.0 + np.exp(-z))


def step(cfg, spec, tokens, kv_len, caches, overrides=None, cache_batch=None):
    """One decode step. caches: dict from synth.host_caches (updated in place, same layouts as the
    library's). Returns dict(logits [B][T][V], sel [L][M][k], probs [L][M][E])."""
    W = Weights(cfg, spec, overrides)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    M, H = B * T, cfg.hidden
    pos = kv_len + np.arange(T)
    x = W["embed"][tokens.reshape(-1)].copy()  # [M][H]
    sels, probs = [], []
    mla_ord = kda_ord = 0
    for l in range(cfg.n_layers):
        p = f"L{l}."
        h = rms(x, W[p + "attn_norm"], cfg.rms_eps)
        kind = cfg.layer_kind(l)
        if kind == "gqa":
            nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
            q = (h @ W[p + "wq"].T).reshape(B, T, nq, d)
            k = (h @ W[p + "wk"].T).reshape(B, T, nkv, d)
            v = (h @ W[p + "wv"].T).reshape(B, T, nkv, d)
            q = rotate(q, pos[None, :, None], cfg.rope_theta)
            k = rotate(k, pos[None, :, None], cfg.rope_theta)
            Kc, Vc = caches["k"][l], caches["v"][l]  # [cb][nkv][cap][d] bf16
            Kc[:B, :, kv_len:kv_len + T] = bf16_bits(bf16_round(k.transpose(0, 2, 1, 3)))
            Vc[:B, :, kv_len:kv_len + T] = bf16_bits(bf16_round(v.transpose(0, 2, 1, 3)))
            Kf, Vf = bf(Kc[:B, :, :kv_len + T]), bf(Vc[:B, :, :kv_len + T])
            grp = np.arange(nq) * nkv // nq
            s = np.einsum("btid,bipd->btip", q, Kf[:, grp]) / np.sqrt(d)
            mask = np.arange(kv_len + T)[None, :] > pos[:, None]  # [T][P]
            s = np.where(mask[None, :, None, :], -np.inf, s)
            o = np.einsum("btip,bipd->btid", softmax(s), Vf[:, grp]).reshape(M, nq * d)
            x = x + o @ W[p + "wo"].T
        elif kind == "mla":
            nh, nd, rd, vd, kvl = cfg.n_heads, cfg.nope_dim, cfg.rope_dim, cfg.v_dim, cfg.kv_lora
            cq = rms(h @ W[p + "w_dq"].T, W[p + "q_norm"], cfg.rms_eps)
            q = (cq @ W[p + "w_uq"].T).reshape(B, T, nh, nd + rd)
            qn, qp = q[..., :nd], rotate(q[..., nd:], pos[None, :, None], cfg.rope_theta)
            kva = (h @ W[p + "w_dkv"].T).reshape(B, T, kvl + rd)
            c = rms(kva[..., :kvl], W[p + "kv_norm"], cfg.rms_eps)
            kpe = rotate(kva[..., kvl:], pos[None, :], cfg.rope_theta)
            Lc = caches["latent"][mla_ord]  # [cb][cap][lat]
            Lc[:B, kv_len:kv_len + T] = bf16_bits(bf16_round(np.concatenate([c, kpe], axis=-1)))
            Cf = bf(Lc[:B, :kv_len + T])  # [B][P][lat]
            Kn = np.einsum("bpj,hrj->bhpr", Cf[..., :kvl], W[p + "w_uk"])  # explicit per-head keys
            Vh = np.einsum("bpj,hvj->bhpv", Cf[..., :kvl], W[p + "w_uv"])  # and values
            s = (np.einsum("bthr,bhpr->bthp", qn, Kn) + np.einsum("bthr,bpr->bthp", qp, Cf[..., kvl:]))
            s = s / np.sqrt(nd + rd)
            mask = np.arange(kv_len + T)[None, :] > pos[:, None]
            s = np.where(mask[None, :, None, :], -np.inf, s)
            o = np.einsum("bthp,bhpv->bthv", softmax(s), Vh).reshape(M, nh * vd)
            x = x + o @ W[p + "wo"].T
            mla_ord += 1
        else:
            nh, dk, dv = cfg.n_heads, cfg.kda_dk, cfg.kda_dv
            q = (h @ W[p + "kda_wq"].T).reshape(B, T, nh, dk)
            k = (h @ W[p + "kda_wk"].T).reshape(B, T, nh, dk)
            v = (h @ W[p + "kda_wv"].T).reshape(B, T, nh, dv)
            k = k / np.linalg.norm(k, axis=-1, keepdims=True)
            al, be = W[p + "kda_alpha"], W[p + "kda_beta"]  # [nh][dk], [nh]
            S = caches["kda_state"][kda_ord]  # [cb][nh][dk][dv] fp32, in place
            o = np.zeros((B, T, nh, dv))
            for b in range(B):
                for i in range(nh):
                    St = S[b, i].astype(np.float64)
                    for t in range(T):
                        kk = k[b, t, i]
                        P = np.eye(dk) - be[i] * np.outer(kk, kk)
                        St = P @ (al[i][:, None] * St) + be[i] * np.outer(kk, v[b, t, i])
                        o[b, t, i] = St.T @ q[b, t, i]
                        St = St.astype(np.float32).astype(np.float64)
                    S[b, i] = St.astype(np.float32)
            x = x + o.reshape(M, nh * dv) @ W[p + "wo"].T
            kda_ord += 1
        h = rms(x, W[p + "moe_norm"], cfg.rms_eps)
        y = np.zeros_like(x)
        if cfg.n_experts:
            r = (h @ W[p + "router"].T).astype(np.float32).astype(np.float64)
            pr = softmax(r)
            sel = np.argsort(-pr, axis=-1, kind="stable")[:, :cfg.top_k]
            wsel = np.take_along_axis(pr, sel, axis=-1)
            if cfg.norm_topk:
                wsel = wsel / wsel.sum(axis=-1, keepdims=True)
            slot = cfg.pool_slot(l)
            for m in range(M):
                for j in range(cfg.top_k):
                    e = sel[m, j]
                    xp = f"X{slot}.{e}."
                    g = silu(W[xp + "gate"] @ h[m]) * (W[xp + "up"] @ h[m])
                    y[m] += wsel[m, j] * (W[xp + "down"] @ g)
            sels.append(sel)
            probs.append(pr)
        if cfg.shared_ffn:
            g = silu(h @ W[p + "sh_gate"].T) * (h @ W[p + "sh_up"].T)
            y = y + g @ W[p + "sh_down"].T
        x = x + y
    logits = rms(x, W["final_norm"], cfg.rms_eps) @ W["lm_head"].T
    out = {"logits": logits.reshape(B, T, cfg.vocab)}
    if cfg.n_experts:
        out["sel"] = np.stack(sels)
        out["probs"] = np.stack(probs)
    return out
