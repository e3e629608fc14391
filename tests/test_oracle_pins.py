"""Pins of the fp64 oracle against closed forms, invariants and special cases.

Each test fixes a value the mathematics determines independently of the
oracle's code: a closed form on special inputs, an identity the operation must
satisfy, or a reduction to a textbook/library routine. Together they are chosen
so that a dropped term, a wrong sign or index, or a transposed operand in any
block of the oracle fails at least one of them.
"""
import ctypes
import math
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth

L = None


def setup_module(_):
    global L
    L = oracle.lib()


def ptr(a):
    return a.ctypes.data


def bf16_bits(x):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def rb(x):
    """round to bf16 with the oracle's rounding (pinned in test_round_bf16)."""
    return np.array([synth.bf16_to_f32(np.array([L.orc_round_bf16(float(v))], np.uint16))[0] for v in np.ravel(x)],
                    dtype=np.float64).reshape(np.shape(x))


def rmsnorm_ref(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / math.sqrt(np.mean(x * x) + eps)


# --------------------------------------------------------------------------------------
# primitives
# --------------------------------------------------------------------------------------
def test_round_bf16():
    f = lambda v: L.orc_round_bf16(v)
    assert f(1.0) == 0x3F80
    assert f(-2.0) == 0xC000
    assert f(0.0) == 0
    # midpoint between 1 and 1 + 2^-7 ties to even (1.0); next midpoint ties up to the even 1 + 2^-6
    assert f(1.0 + 2.0 ** -8) == 0x3F80
    assert f(1.0 + 3 * 2.0 ** -8) == 0x3F82
    # just above a midpoint rounds up (a single rounding from double, no double rounding)
    assert f(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    # agrees with the generator's fp32 -> bf16 converter on fp32 inputs
    rng = np.random.default_rng(0)
    for v in rng.normal(size=200).astype(np.float32):
        assert f(float(v)) == synth.lib().synth_f32_to_bf16(float(v))


def test_rmsnorm_closed_forms():
    n = 64
    g = bf16_bits(np.ones(n))
    y = np.zeros(n)
    x = np.full(n, 3.0)
    L.orc_rmsnorm(ptr(x), ptr(g), n, 0.0, ptr(y))
    np.testing.assert_allclose(y, np.ones(n), rtol=1e-15)
    # one-hot a*e_5: mean square a^2/n, output sqrt(n) * gain at index 5
    x = np.zeros(n)
    x[5] = 2.0
    g2 = bf16_bits(np.linspace(0.5, 2.0, n).astype(np.float32).astype(np.float64) * 0 + 1.5)
    L.orc_rmsnorm(ptr(x), ptr(g2), n, 0.0, ptr(y))
    expect = np.zeros(n)
    expect[5] = math.sqrt(n) * 1.5
    np.testing.assert_allclose(y, expect, rtol=1e-15)
    # epsilon enters inside the square root
    x = np.zeros(n)
    L.orc_rmsnorm(ptr(x), ptr(g), n, 1e-6, ptr(y))
    assert np.all(y == 0)
    x = np.full(n, 1e-3)
    L.orc_rmsnorm(ptr(x), ptr(g), n, 1e-6, ptr(y))
    np.testing.assert_allclose(y, 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-14)


def rope(x, pos, theta=1e4):
    x = np.array(x, dtype=np.float64)
    L.orc_rope(ptr(x), x.size, pos, theta)
    return x


def test_rope_pairs_and_frequencies():
    # d = 4: pairs (0,2) at frequency 1 and (1,3) at frequency theta^(-1/2)
    pos = 3
    y = rope([1, 0, 0, 0], pos)
    np.testing.assert_allclose(y, [math.cos(3), 0, math.sin(3), 0], atol=1e-15)
    y = rope([0, 1, 0, 0], pos)
    f = 1e4 ** -0.5
    np.testing.assert_allclose(y, [0, math.cos(3 * f), 0, math.sin(3 * f)], atol=1e-15)
    y = rope([0, 0, 1, 0], pos)
    np.testing.assert_allclose(y, [-math.sin(3), 0, math.cos(3), 0], atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=64), rng.normal(size=64)
    np.testing.assert_allclose(rope(q, 0), q, rtol=0, atol=0)
    np.testing.assert_allclose(np.linalg.norm(rope(q, 77)), np.linalg.norm(q), rtol=1e-14)
    # relative position: <R(m)q, R(n)k> depends on m - n only
    a = rope(q, 10) @ rope(k, 4)
    b = rope(q, 1010) @ rope(k, 1004)
    np.testing.assert_allclose(a, b, rtol=1e-10)


def test_softmax():
    s = np.array([0.0, math.log(2.0)])
    p = np.zeros(2)
    L.orc_softmax(ptr(s), 2, ptr(p))
    np.testing.assert_allclose(p, [1 / 3, 2 / 3], rtol=1e-15)
    rng = np.random.default_rng(2)
    s = rng.normal(size=1000) * 30
    p = np.zeros_like(s)
    L.orc_softmax(ptr(s), s.size, ptr(p))
    assert abs(p.sum() - 1.0) <= 1e-12
    p2 = np.zeros_like(s)
    s2 = s + 1234.5
    L.orc_softmax(ptr(s2), s.size, ptr(p2))
    np.testing.assert_allclose(p, p2, rtol=1e-9)


def topk(p, k):
    idx = np.zeros(k, dtype=np.int32)
    p = np.ascontiguousarray(p, dtype=np.float64)
    L.orc_topk(ptr(p), p.size, k, ptr(idx))
    return idx


def test_topk_matches_stable_sort_and_tie_break():
    rng = np.random.default_rng(3)
    for _ in range(50):
        p = rng.random(48)
        p[rng.integers(0, 48, 5)] = p[0]  # plant ties
        k = int(rng.integers(1, 9))
        np.testing.assert_array_equal(topk(p, k), np.argsort(-p, kind="stable")[:k])
    np.testing.assert_array_equal(topk(np.full(8, 0.125), 3), [0, 1, 2])


def test_silu():
    assert L.orc_silu(0.0) == 0.0
    for x in (-5.0, -0.3, 0.7, 4.0):
        # x*sigmoid(x) - (-x)*sigmoid(-x) = x
        assert abs(L.orc_silu(x) - L.orc_silu(-x) - x) < 1e-14
    assert abs(L.orc_silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_matvec_is_a_matmul():
    rng = np.random.default_rng(4)
    W = synth.normal_bf16(7, "pin.matvec", 37 * 300, 0.05).reshape(37, 300)
    x = rng.normal(size=300)
    y = np.zeros(37)
    L.orc_matvec(ptr(W), 37, 300, ptr(x), ptr(y))
    np.testing.assert_allclose(y, synth.bf16_to_f32(W).astype(np.float64) @ x, rtol=1e-12, atol=1e-12)


def kda(S, alpha, beta, k, v, q):
    S = np.array(S, dtype=np.float64)
    o = np.zeros(S.shape[1])
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    k, v, q = (np.ascontiguousarray(a, dtype=np.float64) for a in (k, v, q))
    L.orc_kda_head(ptr(S), S.shape[0], S.shape[1], ptr(alpha), beta, ptr(k), ptr(v), ptr(q), ptr(o))
    return S, o


def test_kda_identities():
    rng = np.random.default_rng(5)
    dk, dv = 16, 12
    S0 = rng.normal(size=(dk, dv))
    q, v = rng.normal(size=dk), rng.normal(size=dv)
    k = rng.normal(size=dk)
    k /= np.linalg.norm(k)
    a = rng.uniform(0.2, 0.9, size=dk).astype(np.float32)
    # alpha = 1, beta = 0: state unchanged, o = S^T q
    S, o = kda(S0, np.ones(dk), 0.0, k, v, q)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, S0.T @ q, rtol=1e-12)
    # beta = 1, |k| = 1: the updated state retrieves v exactly at k, for any decay
    S, _ = kda(S0, a, 1.0, k, v, q)
    np.testing.assert_allclose(S.T @ k, v, rtol=1e-10, atol=1e-12)
    # alpha = 0: S' = beta k v^T, so o = beta v (k.q)
    S, o = kda(S0, np.zeros(dk), 0.3, k, v, q)
    np.testing.assert_allclose(o, 0.3 * v * (k @ q), rtol=1e-12)
    # decay is applied to rows (key channels) before the delta step: beta = 0 gives diag(a) S0
    S, _ = kda(S0, a, 0.0, k, v, q)
    np.testing.assert_allclose(S, a.astype(np.float64)[:, None] * S0, rtol=1e-15)


# --------------------------------------------------------------------------------------
# whole-step special cases on tiny models
# --------------------------------------------------------------------------------------
def tiny_gqa(**kw):
    base = dict(n_layers=1, shared_ffn=0, n_experts=2, top_k=1, ffn=256)
    base.update(kw)
    return replace(synth.TINY, **base)


def ones_gain(n):
    return bf16_bits(np.ones(n))


def eye_bits(rows, cols):
    return bf16_bits(np.eye(rows, cols))


def zeros_bits(*shape):
    return np.zeros(shape, dtype=np.uint16)


def run(cfg, overrides, tokens, kv_len, caches=None, spec=None, **kw):
    spec = spec or synth.Spec(seed=11)
    B = tokens.shape[0]
    if caches is None:
        caches = synth.host_caches(cfg, spec, B, kv_len)
    P = oracle.Provider(cfg, spec, overrides)
    return oracle.decode_step(cfg, P, tokens, kv_len, caches, trace=True, x_trace=True, **kw), caches


def embed_rows(spec, cfg, toks):
    E = synth.bf16_to_f32(synth.normal_bf16(spec.seed, "embed", cfg.vocab * cfg.hidden, spec.sigma))
    return E.reshape(cfg.vocab, cfg.hidden)[toks].astype(np.float64)


def identity_overrides(cfg):
    H = cfg.hidden
    ov = {"final_norm": ones_gain(H), "lm_head": eye_bits(cfg.vocab, H)}
    for l in range(cfg.n_layers):
        p = f"L{l}."
        ov.update({p + "attn_norm": ones_gain(H), p + "moe_norm": ones_gain(H)})
    for s in range(cfg.n_pool):
        for e in range(cfg.n_experts):
            ov[f"X{s}.{e}.down"] = zeros_bits(H, cfg.ffn)
    return ov


def test_identity_pass_closed_form():
    """L = 1, kv_len = 0, T = 1, identity attention weights, zero expert output, W_lm = [I; 0]:
    logits[:H] = RMSNorm(x0 + bf16(RMSNorm(x0))), the remaining logits are zero."""
    cfg = tiny_gqa()
    H = cfg.hidden
    ov = identity_overrides(cfg)
    for k in ("wq", "wk", "wv", "wo"):
        ov["L0." + k] = eye_bits(H, H)
    spec = synth.Spec(seed=11)
    toks = np.array([[17]], dtype=np.int32)
    out, _ = run(cfg, ov, toks, 0, spec=spec)
    x0 = embed_rows(spec, cfg, toks[0])[0]
    expect = rmsnorm_ref(x0 + rb(rmsnorm_ref(x0)))
    lg = out["logits"][0, 0]
    np.testing.assert_allclose(lg[:H], expect, rtol=1e-12, atol=1e-12)
    assert np.all(lg[H:] == 0)


def test_attention_scale_and_self_inclusion():
    """kv_len = 1 with a zero cached key and value; the new token attends to itself with
    weight sigmoid((Wq h).(Wk h)/sqrt(d)) -- RoPE at one position keeps the dot product."""
    cfg = tiny_gqa(n_heads=1, n_kv_heads=1, head_dim=256)
    H = cfg.hidden
    spec = synth.Spec(seed=12)
    ov = identity_overrides(cfg)
    Wq = synth.normal_bf16(3, "pin.wq", H * H, 0.1).reshape(H, H)
    Wk = synth.normal_bf16(3, "pin.wk", H * H, 0.1).reshape(H, H)
    ov.update({"L0.wq": Wq, "L0.wk": Wk, "L0.wv": eye_bits(H, H), "L0.wo": eye_bits(H, H)})
    toks = np.array([[5]], dtype=np.int32)
    caches = synth.host_caches(cfg, spec, 1, 1)
    caches["k"][:] = 0
    caches["v"][:] = 0
    out, _ = run(cfg, ov, toks, 1, caches=caches, spec=spec)
    x0 = embed_rows(spec, cfg, toks[0])[0]
    h = rmsnorm_ref(x0)
    q = synth.bf16_to_f32(Wq).astype(np.float64) @ h
    k = synth.bf16_to_f32(Wk).astype(np.float64) @ h
    # the stored key is rounded to bf16 after RoPE at position 1
    kr = rb(rope(k, 1))
    qr = rope(q, 1)
    a1 = 1.0 / (1.0 + math.exp(-(qr @ kr) / math.sqrt(H)))
    np.testing.assert_allclose(out["x"][1, 0], x0 + a1 * rb(h), rtol=1e-11, atol=1e-12)


def test_equal_keys_give_mean_of_values():
    cfg = tiny_gqa()
    H = cfg.hidden
    spec = synth.Spec(seed=13)
    ov = identity_overrides(cfg)
    ov.update({"L0.wk": zeros_bits(H, H), "L0.wv": eye_bits(H, H), "L0.wo": eye_bits(H, H)})
    kv_len = 9
    caches = synth.host_caches(cfg, spec, 1, kv_len)
    caches["k"][:] = 0
    toks = np.array([[3]], dtype=np.int32)
    out, caches = run(cfg, ov, toks, kv_len, caches=caches, spec=spec)
    x0 = embed_rows(spec, cfg, toks[0])[0]
    V = synth.bf16_to_f32(caches["v"][0, 0, :, : kv_len + 1, :]).astype(np.float64)  # [heads][pos][d]
    o = V.mean(axis=1).reshape(-1)
    np.testing.assert_allclose(out["x"][1, 0], x0 + o, rtol=1e-12, atol=1e-13)


def test_gqa_head_mapping_equals_duplicated_mha():
    """n_kv = 2 of n_q = 4: query head i reads kv head floor(i * n_kv / n_q); duplicating
    the kv heads into a 4-head MHA gives the same step."""
    spec = synth.Spec(seed=14)
    gqa = tiny_gqa(n_kv_heads=2, n_layers=2)
    mha = tiny_gqa(n_kv_heads=4, n_layers=2)
    d = gqa.head_dim
    ov_g, ov_m = {}, {}
    for l in range(2):
        for w in ("wk", "wv"):
            W = synth.normal_bf16(spec.seed, f"L{l}.{w}", 2 * d * gqa.hidden, 0.02).reshape(2, d, gqa.hidden)
            ov_g[f"L{l}.{w}"] = W.reshape(2 * d, -1)
            ov_m[f"L{l}.{w}"] = W[[0, 0, 1, 1]].reshape(4 * d, -1)
    kv_len = 20
    cg = synth.host_caches(gqa, spec, 1, kv_len)
    cm = {"k": np.ascontiguousarray(cg["k"][:, :, [0, 0, 1, 1]]), "v": np.ascontiguousarray(cg["v"][:, :, [0, 0, 1, 1]])}
    toks = np.array([[100, 7]], dtype=np.int32)
    og, _ = run(gqa, ov_g, toks, kv_len, caches=cg, spec=spec)
    om, _ = run(mha, ov_m, toks, kv_len, caches=cm, spec=spec)
    np.testing.assert_array_equal(og["logits"], om["logits"])
    # and it differs from the other plausible mapping (i mod n_kv)
    ov_w = dict(ov_m)
    for l in range(2):
        for w in ("wk", "wv"):
            ov_w[f"L{l}.{w}"] = ov_g[f"L{l}.{w}"].reshape(2, d, -1)[[0, 1, 0, 1]].reshape(4 * d, -1)
    cw = {"k": np.ascontiguousarray(cg["k"][:, :, [0, 1, 0, 1]]), "v": np.ascontiguousarray(cg["v"][:, :, [0, 1, 0, 1]])}
    ow, _ = run(mha, ov_w, toks, kv_len, caches=cw, spec=spec)
    assert not np.allclose(og["logits"], ow["logits"])


def test_router_uniform_and_dense_swiglu():
    """W_r = 0 gives p = 1/E and selects experts 0..k-1. With E = k = 1 and W_g = W_u = W_d = I
    (F = H) the MoE adds silu(h) * h with weight 1."""
    cfg = tiny_gqa(n_experts=1, top_k=1, ffn=256)
    H = cfg.hidden
    spec = synth.Spec(seed=15)
    ov = identity_overrides(cfg)
    ov.update({"L0.wo": zeros_bits(H, H), "L0.router": zeros_bits(1, H),
               "X0.0.gate": eye_bits(H, H), "X0.0.up": eye_bits(H, H), "X0.0.down": eye_bits(H, H)})
    toks = np.array([[9]], dtype=np.int32)
    out, _ = run(cfg, ov, toks, 4, spec=spec)
    x0 = embed_rows(spec, cfg, toks[0])[0]
    h = rmsnorm_ref(x0)
    silu = h / (1.0 + np.exp(-h))
    np.testing.assert_allclose(out["x"][1, 0], x0 + silu * h, rtol=1e-12, atol=1e-14)
    cfg8 = tiny_gqa(n_experts=8, top_k=3)
    ov8 = identity_overrides(cfg8)
    ov8["L0.router"] = zeros_bits(8, H)
    out8, _ = run(cfg8, ov8, toks, 4, spec=spec)
    np.testing.assert_array_equal(out8["sel"][0, 0], [0, 1, 2])
    np.testing.assert_allclose(out8["probs"][0, 0], np.full(8, 1 / 8), rtol=1e-15)


def test_expert_weighting_and_routing_trace():
    """Only the selected experts contribute, each scaled by its router probability."""
    cfg = tiny_gqa(n_experts=4, top_k=2, ffn=256, n_layers=1)
    H = cfg.hidden
    spec = synth.Spec(seed=16)
    ov = identity_overrides(cfg)
    ov["L0.wo"] = zeros_bits(H, H)
    for e in range(4):
        ov[f"X0.{e}.gate"] = eye_bits(H, H)
        ov[f"X0.{e}.up"] = eye_bits(H, H)
        ov[f"X0.{e}.down"] = bf16_bits(np.eye(H) * (e + 1))  # expert e adds (e+1) silu(h) h
    toks = np.array([[2]], dtype=np.int32)
    out, _ = run(cfg, ov, toks, 3, spec=spec)
    x0 = embed_rows(spec, cfg, toks[0])[0]
    h = rmsnorm_ref(x0)
    p = out["probs"][0, 0]
    sel = out["sel"][0, 0]
    np.testing.assert_array_equal(sel, np.argsort(-p, kind="stable")[:2])
    f = h / (1.0 + np.exp(-h)) * h
    expect = x0 + sum(p[e] * (e + 1) * f for e in sel)
    np.testing.assert_allclose(out["x"][1, 0], expect, rtol=1e-12, atol=1e-14)
    # forced routing replaces the choice but keeps the probabilities as weights
    out2, _ = run(cfg, ov, toks, 3, spec=spec, force_sel=np.array([[[3, 0]]], dtype=np.int32))
    np.testing.assert_allclose(out2["x"][1, 0], x0 + p[3] * 4 * f + p[0] * 1 * f, rtol=1e-12, atol=1e-14)


def test_dense_swiglu_closed_form():
    """A dense model (n_experts = 0) has no router: with W_g = W_u = W_d = I (width H) its
    feed-forward block adds silu(h) * h to every token."""
    cfg = tiny_gqa(n_experts=0, top_k=0, ffn=0, shared_ffn=256)
    H = cfg.hidden
    spec = synth.Spec(seed=17)
    ov = identity_overrides(cfg)
    ov.update({"L0.wo": zeros_bits(H, H), "L0.sh_gate": eye_bits(H, H), "L0.sh_up": eye_bits(H, H),
               "L0.sh_down": eye_bits(H, H)})
    toks = np.array([[5], [6]], dtype=np.int32)
    out, _ = run(cfg, ov, toks, 4, spec=spec)
    assert out["sel"].shape[-1] == 0
    for b in range(2):
        x0 = embed_rows(spec, cfg, toks[b])[0]
        h = rmsnorm_ref(x0)
        np.testing.assert_allclose(out["x"][1, b], x0 + h / (1.0 + np.exp(-h)) * h, rtol=1e-12, atol=1e-14)


def test_dense_equals_single_expert_moe():
    """One routed expert chosen with probability 1 (E = k = 1: the softmax of one logit) is the
    dense block: a dense model and a one-expert MoE whose expert holds the dense weights give the
    same logits, whatever the router weights."""
    dense = tiny_gqa(n_experts=0, top_k=0, ffn=0, shared_ffn=384, n_layers=2)
    moe = tiny_gqa(n_experts=1, top_k=1, ffn=384, shared_ffn=0, n_layers=2)
    spec = synth.Spec(seed=18, sigma=0.05)
    H = dense.hidden
    ov = {}
    for l in range(2):
        for a, b in (("sh_gate", "gate"), ("sh_up", "up"), ("sh_down", "down")):
            shape = (384, H) if a != "sh_down" else (H, 384)
            w = synth.normal_bf16(spec.seed, f"L{l}.{a}", shape[0] * shape[1], spec.sigma)
            ov[f"X{l}.0.{b}"] = w
    toks = np.array([[3, 40, 7]], dtype=np.int32)
    a, _ = run(dense, {}, toks, 6, spec=spec)
    b, _ = run(moe, ov, toks, 6, spec=spec)
    np.testing.assert_array_equal(b["sel"], np.zeros((2, 3, 1), dtype=np.int32))
    np.testing.assert_allclose(b["probs"], 1.0, rtol=0, atol=0)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-13, atol=1e-13)


def test_causal_mask_among_new_tokens():
    cfg = replace(synth.TINY, n_layers=2)
    spec = synth.Spec(seed=17)
    a, _ = run(cfg, {}, np.array([[1, 2, 3]], dtype=np.int32), 30, spec=spec)
    b, _ = run(cfg, {}, np.array([[1, 2, 999]], dtype=np.int32), 30, spec=spec)
    np.testing.assert_array_equal(a["logits"][0, :2], b["logits"][0, :2])
    assert not np.array_equal(a["logits"][0, 2], b["logits"][0, 2])


# --------------------------------------------------------------------------------------
# MLA
# --------------------------------------------------------------------------------------
MLA_TINY = replace(
    synth.K3, name="mla-tiny", n_layers=2, hidden=64, vocab=96, n_heads=2, q_lora=32, kv_lora=16, rope_dim=8,
    nope_dim=8, v_dim=16, n_experts=4, top_k=1, ffn=64, shared_ffn=32, expert_pool_layers=0, kv_capacity=40)


def test_mla_absorbed_equals_explicit():
    spec = synth.Spec(seed=21, sigma=0.2)
    toks = np.array([[5, 6, 7], [8, 9, 10]], dtype=np.int32)
    a, ca = run(MLA_TINY, {}, toks, 11, spec=spec)
    b, cb = run(MLA_TINY, {}, toks, 11, spec=spec, mla_explicit=True)
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=1e-9, atol=1e-12)
    np.testing.assert_array_equal(ca["latent"], cb["latent"])


def test_mla_value_path_and_scale_closed_form():
    """kv_len = 1 with a zero cached latent entry and q_nope = 0: the new position gets weight
    sigmoid(q_pe . k_pe / sqrt(nope + rope)), and o_h = W_uv,h u_h = a1 * c_new."""
    cfg = replace(MLA_TINY, n_layers=1)
    H, ql, kvl, rd, nd, nh, vd = 64, 32, 16, 8, 8, 2, 16
    spec = synth.Spec(seed=22)
    ov = identity_overrides(cfg)
    ov["L0.w_dq"] = eye_bits(ql, H)  # qa = h[:32]
    ov["L0.q_norm"] = ones_gain(ql)
    wuq = np.zeros((nh, nd + rd, ql))
    for i in range(nh):
        wuq[i, nd:, :rd] = np.eye(rd)  # q_nope = 0, q_pe = c_q[:8]
    ov["L0.w_uq"] = bf16_bits(wuq.reshape(nh * (nd + rd), ql))
    ov["L0.w_dkv"] = eye_bits(kvl + rd, H)  # c = RMSNorm(h[:16]), k_pe = h[16:24]
    ov["L0.kv_norm"] = ones_gain(kvl)
    ov["L0.w_uk"] = bf16_bits(np.ones((nh, nd, kvl)))
    ov["L0.w_uv"] = bf16_bits(np.stack([np.eye(vd, kvl)] * nh))
    ov["L0.wo"] = eye_bits(H, nh * vd)
    ov["L0.router"] = zeros_bits(cfg.n_experts, H)
    ov["L0.sh_down"] = zeros_bits(H, cfg.shared_ffn)
    caches = synth.host_caches(cfg, spec, 1, 1)
    caches["latent"][:] = 0
    toks = np.array([[4]], dtype=np.int32)
    out, caches = run(cfg, ov, toks, 1, caches=caches, spec=spec)
    x0 = embed_rows(spec, cfg, toks[0])[0]
    h = rmsnorm_ref(x0)
    cq = rmsnorm_ref(h[:ql])
    c_new = rb(rmsnorm_ref(h[:kvl]))
    kpe = rb(rope(h[kvl:kvl + rd], 1))
    np.testing.assert_array_equal(synth.bf16_to_f32(caches["latent"][0, 0, 1]), np.concatenate([c_new, kpe]))
    s1 = rope(cq[:rd], 1) @ kpe / math.sqrt(nd + rd)
    a1 = 1.0 / (1.0 + math.exp(-s1))
    expect = x0.copy()
    expect[:vd] += a1 * c_new
    expect[vd:2 * vd] += a1 * c_new
    np.testing.assert_allclose(out["x"][1, 0], expect, rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------------------
# incremental decoding equals one multi-token step
# --------------------------------------------------------------------------------------
def incremental_vs_oneshot(cfg, spec, kv_len, T):
    toks = synth.tokens(spec.seed, 0, cfg.vocab, 2, T)
    c1 = synth.host_caches(cfg, spec, 2, kv_len)
    c2 = {k: v.copy() for k, v in c1.items()}
    P = oracle.Provider(cfg, spec)
    one = oracle.decode_step(cfg, P, toks, kv_len, c1, trace=True)
    for t in range(T):
        step = oracle.decode_step(cfg, P, toks[:, t:t + 1], kv_len + t, c2, trace=True)
        np.testing.assert_allclose(step["logits"][:, 0], one["logits"][:, t], rtol=1e-12, atol=1e-13)
        M = one["sel"].reshape(cfg.n_layers, 2, T, -1)
        np.testing.assert_array_equal(step["sel"].reshape(cfg.n_layers, 2, -1), M[:, :, t])
    for k in c1:
        np.testing.assert_array_equal(c1[k], c2[k])


def test_incremental_equals_oneshot_gqa():
    incremental_vs_oneshot(replace(synth.TINY, n_layers=2), synth.Spec(seed=31), 17, 5)


def test_incremental_equals_oneshot_mla():
    incremental_vs_oneshot(MLA_TINY, synth.Spec(seed=32, sigma=0.1), 9, 7)


def test_incremental_equals_oneshot_hybrid():
    cfg = replace(MLA_TINY, name="hyb-tiny", attn_kind=synth.ATTN_HYBRID, n_layers=4, hybrid_period=4,
                  kda_dk=8, kda_dv=8)
    incremental_vs_oneshot(cfg, synth.Spec(seed=33, sigma=0.1), 6, 4)


def test_rejects_bad_arguments():
    cfg = synth.TINY
    spec = synth.Spec()
    caches = synth.host_caches(cfg, spec, 1, 4)
    P = oracle.Provider(cfg, spec)
    with pytest.raises(ValueError):
        oracle.decode_step(cfg, P, np.array([[cfg.vocab]], np.int32), 4, caches)
    with pytest.raises(ValueError):
        oracle.decode_step(cfg, P, np.array([[1]], np.int32), cfg.kv_capacity, caches)
