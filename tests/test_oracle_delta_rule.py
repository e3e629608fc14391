"""Pins of the oracle's delta-rule block, the hybrid layer placement and the renormalised router,
and the oracle against an independent numpy float64 reference (tests/ref_numpy.py) on tiny shapes.

The delta rule of the hybrid model (benchmark configuration 5; the model mixes delta-rule linear
attention with MLA layers: German news article, section "Auf dem Papier liegt der GB200 vorn"):
per head, S <- diag(alpha) S, then S <- S - beta k (k^T S) + beta k v^T, then o = S^T q, with k
L2-normalised; q = W_q h, k = W_k h, v = W_v h; the block adds W_o concat(o). In every group of
four layers the first three are delta-rule layers and the fourth keeps MLA.

Each whole-step pin below is a closed form on special weights (identity output projection, zero
feed-forward), chosen so that a plausible mistake in the block fails one of them: a dropped
normalisation of k, q and k exchanged, the decay applied to the value axis, alpha or beta taken
from the wrong head, S instead of S^T, or the MLA layer at the wrong position of the group.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import ref_numpy
import synth

H, NH, DK, DV = 64, 2, 8, 8
HYB = replace(
    synth.K3, name="hyb-pin", attn_kind=synth.ATTN_HYBRID, n_layers=1, hidden=H, vocab=96, n_heads=NH,
    q_lora=32, kv_lora=16, rope_dim=8, nope_dim=8, v_dim=16, kda_dk=DK, kda_dv=DV, hybrid_period=4,
    n_experts=4, top_k=1, ffn=64, shared_ffn=32, expert_pool_layers=0, kv_capacity=40, max_batch=2)


def bits(x):
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def bfv(u):
    return synth.bf16_to_f32(u).astype(np.float64)


def rms(x):
    return x / np.sqrt(np.mean(x * x) + 1e-6)


def quiet_ffn(cfg):
    """unit norm gains, zero feed-forward output (routed and shared down projections zero)"""
    ov = {"final_norm": bits(np.ones(cfg.hidden))}
    for l in range(cfg.n_layers):
        ov[f"L{l}.attn_norm"] = bits(np.ones(cfg.hidden))
        ov[f"L{l}.moe_norm"] = bits(np.ones(cfg.hidden))
        ov[f"L{l}.sh_down"] = np.zeros((cfg.hidden, cfg.shared_ffn), np.uint16)
    for s in range(cfg.n_pool):
        for e in range(cfg.n_experts):
            ov[f"X{s}.{e}.down"] = np.zeros((cfg.hidden, cfg.ffn), np.uint16)
    return ov


def kda_step(ov, spec, toks, S0=None, cfg=HYB):
    B = toks.shape[0]
    caches = synth.host_caches(cfg, spec, B, 3)
    if S0 is not None:
        caches["kda_state"][0, :B] = S0
    init = caches["kda_state"].copy()
    P = oracle.Provider(cfg, spec, ov)
    out = oracle.decode_step(cfg, P, toks, 3, caches, trace=True, x_trace=True)
    return out, init, caches


def wmat(spec, name, rows, cols, sigma=0.2):
    return synth.normal_bf16(spec.seed, name, rows * cols, sigma).reshape(rows, cols)


def base_overrides(spec, alpha, beta):
    ov = quiet_ffn(HYB)
    ov["L0.kda_wq"] = wmat(spec, "pin.q", NH * DK, H)
    ov["L0.kda_wk"] = wmat(spec, "pin.k", NH * DK, H)
    ov["L0.kda_wv"] = wmat(spec, "pin.v", NH * DV, H)
    ov["L0.kda_alpha"] = np.asarray(alpha, np.float32).reshape(NH, DK)
    ov["L0.kda_beta"] = np.asarray(beta, np.float32).reshape(NH)
    ov["L0.wo"] = bits(np.eye(H, NH * DV))  # x[: NH*DV] += concat(o)
    return ov


def projections(ov, x0):
    h = rms(x0)
    q = (bfv(ov["L0.kda_wq"]) @ h).reshape(NH, DK)
    k = (bfv(ov["L0.kda_wk"]) @ h).reshape(NH, DK)
    v = (bfv(ov["L0.kda_wv"]) @ h).reshape(NH, DV)
    return q, k, v


def embed_row(spec, cfg, tok):
    E = synth.bf16_to_f32(synth.normal_bf16(spec.seed, "embed", cfg.vocab * cfg.hidden, spec.sigma))
    return E.reshape(cfg.vocab, cfg.hidden)[tok].astype(np.float64)


def test_layer_placement_in_groups_of_four():
    """Configuration 5: 'in every 4-layer group, layers 1-3 replace MLA with gated delta-rule linear
    attention ... layer 4 of each group keeps MLA' (1-based), written out literally for 8 layers.
    The oracle must read exactly the delta-rule tensors of layers 0-2, 4-6 and the MLA tensors of
    layers 3 and 7."""
    cfg = replace(HYB, n_layers=8)
    expect = ["kda", "kda", "kda", "mla", "kda", "kda", "kda", "mla"]
    spec = synth.Spec(seed=40)
    P = oracle.Provider(cfg, spec)
    caches = synth.host_caches(cfg, spec, 1, 3)
    oracle.decode_step(cfg, P, np.array([[5]], np.int32), 3, caches)
    got = []
    for l in range(8):
        kinds = {n.split(".", 1)[1] for n, _ in P.fetched if n.startswith(f"L{l}.")}
        got.append("mla" if "w_dq" in kinds else "kda" if "kda_wq" in kinds else "?")
        assert not ({"w_dq", "kda_wq"} <= kinds)
    assert got == expect
    # the MLA layers wrote their latent rows at position 3, the delta-rule states changed
    assert caches["latent"].shape[0] == 2 and np.any(caches["latent"][:, 0, 3] != 0)
    assert caches["kda_state"].shape[0] == 6


def test_no_decay_no_update_reads_S_transpose_q():
    """alpha = 1, beta = 0: the state is unchanged and o_h = S0_h^T q_h, q = W_q h (not W_k h)."""
    spec = synth.Spec(seed=41)
    ov = base_overrides(spec, np.ones(NH * DK), np.zeros(NH))
    toks = np.array([[7]], np.int32)
    out, init, caches = kda_step(ov, spec, toks)
    x0 = embed_row(spec, HYB, 7)
    q, _, _ = projections(ov, x0)
    S0 = init[0, 0].astype(np.float64)  # [NH][DK][DV]
    o = np.concatenate([S0[i].T @ q[i] for i in range(NH)])
    expect = x0.copy()
    expect[: NH * DV] += o
    np.testing.assert_allclose(out["x"][1, 0], expect, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(caches["kda_state"][0, 0], init[0, 0])


def test_decay_on_key_rows_per_head():
    """beta = 0 with a different decay per head and channel: S' = diag(alpha_h) S0 (rounded to
    fp32, as stored) and o_h = S'^T q_h = S0^T (alpha_h * q_h)."""
    spec = synth.Spec(seed=42)
    rng = np.random.default_rng(42)
    alpha = rng.uniform(0.1, 0.95, size=(NH, DK)).astype(np.float32)
    ov = base_overrides(spec, alpha, np.zeros(NH))
    out, init, caches = kda_step(ov, spec, np.array([[9]], np.int32))
    x0 = embed_row(spec, HYB, 9)
    q, _, _ = projections(ov, x0)
    S0 = init[0, 0].astype(np.float64)
    a = alpha.astype(np.float64)
    Sd = a[:, :, None] * S0  # the output reads the state before it is stored in fp32
    np.testing.assert_array_equal(caches["kda_state"][0, 0], Sd.astype(np.float32))
    o = np.concatenate([Sd[i].T @ q[i] for i in range(NH)])
    expect = x0.copy()
    expect[: NH * DV] += o
    np.testing.assert_allclose(out["x"][1, 0], expect, rtol=1e-12, atol=1e-13)


def test_retrieval_at_normalised_key_with_per_head_beta():
    """Head 0 has beta = 1: after the update S'^T k_hat = v whatever the decay, so with W_q = W_k
    (q = k unnormalised) o_0 = |k_0| v_0. Head 1 has beta = 0 and no decay: o_1 = S0_1^T q_1."""
    spec = synth.Spec(seed=43)
    rng = np.random.default_rng(43)
    alpha = np.ones((NH, DK), np.float32)
    alpha[0] = rng.uniform(0.2, 0.9, size=DK)
    ov = base_overrides(spec, alpha, [1.0, 0.0])
    ov["L0.kda_wq"] = ov["L0.kda_wk"]
    out, init, caches = kda_step(ov, spec, np.array([[11]], np.int32))
    x0 = embed_row(spec, HYB, 11)
    q, k, v = projections(ov, x0)
    S0 = init[0, 0].astype(np.float64)
    o0 = np.linalg.norm(k[0]) * v[0]
    o1 = S0[1].T @ q[1]
    expect = x0.copy()
    expect[:DV] += o0
    expect[DV:2 * DV] += o1
    np.testing.assert_allclose(out["x"][1, 0], expect, rtol=1e-12, atol=1e-13)
    # the stored state of head 0 retrieves v_0 at the normalised key (to fp32 storage precision)
    S1 = caches["kda_state"][0, 0, 0].astype(np.float64)
    kh = k[0] / np.linalg.norm(k[0])
    np.testing.assert_allclose(S1.T @ kh, v[0], rtol=1e-5, atol=1e-6)


def test_key_scale_does_not_matter():
    """k is L2-normalised: W_k and 4 W_k (exact in bf16) give bitwise the same step, with random
    decay and beta; W_q and 4 W_q do not."""
    spec = synth.Spec(seed=44)
    rng = np.random.default_rng(44)
    ov = base_overrides(spec, rng.uniform(0.3, 0.99, size=NH * DK), rng.uniform(0.2, 0.9, size=NH))
    toks = np.array([[3, 4]], np.int32)
    a, _, ca = kda_step(ov, spec, toks)
    ov4 = dict(ov)
    ov4["L0.kda_wk"] = bits(bfv(ov["L0.kda_wk"]) * 4.0)
    b, _, cb = kda_step(ov4, spec, toks)
    np.testing.assert_array_equal(a["logits"], b["logits"])
    np.testing.assert_array_equal(ca["kda_state"], cb["kda_state"])
    ovq = dict(ov)
    ovq["L0.kda_wq"] = bits(bfv(ov["L0.kda_wq"]) * 4.0)
    c, _, _ = kda_step(ovq, spec, toks)
    assert not np.allclose(a["x"][1], c["x"][1])


def test_norm_topk_renormalises_over_chosen():
    """norm_topk = 1: the chosen experts' weights are their probabilities divided by the chosen
    probabilities' sum; identity experts make expert e add (e+1) silu(h) h."""
    cfg = replace(synth.TINY, n_layers=1, n_experts=4, top_k=2, ffn=256, shared_ffn=0, norm_topk=1)
    Hh = cfg.hidden
    spec = synth.Spec(seed=45)
    ov = {"final_norm": bits(np.ones(Hh)), "L0.attn_norm": bits(np.ones(Hh)), "L0.moe_norm": bits(np.ones(Hh)),
          "L0.wo": np.zeros((Hh, Hh), np.uint16)}
    for e in range(4):
        ov[f"X0.{e}.gate"] = bits(np.eye(Hh))
        ov[f"X0.{e}.up"] = bits(np.eye(Hh))
        ov[f"X0.{e}.down"] = bits(np.eye(Hh) * (e + 1))
    caches = synth.host_caches(cfg, spec, 1, 3)
    out = oracle.decode_step(cfg, oracle.Provider(cfg, spec, ov), np.array([[2]], np.int32), 3, caches,
                             trace=True, x_trace=True)
    x0 = embed_row(spec, cfg, 2)
    h = rms(x0)
    p, sel = out["probs"][0, 0], out["sel"][0, 0]
    f = h / (1.0 + np.exp(-h)) * h
    wsum = p[sel].sum()
    expect = x0 + sum(p[e] / wsum * (e + 1) * f for e in sel)
    np.testing.assert_allclose(out["x"][1, 0], expect, rtol=1e-12, atol=1e-14)
    assert abs(sum(p[e] / wsum for e in sel) - 1.0) < 1e-15


# ------------------------------------------------------------------------------------------
# the oracle against the independent numpy reference (explicit MLA, matrix-form delta rule)
# ------------------------------------------------------------------------------------------
MLA_TINY = replace(
    synth.K3, name="mla-tiny", n_layers=2, hidden=64, vocab=96, n_heads=2, q_lora=32, kv_lora=16, rope_dim=8,
    nope_dim=8, v_dim=16, n_experts=4, top_k=2, ffn=64, shared_ffn=32, expert_pool_layers=0, kv_capacity=40,
    max_batch=2)
CASES = {
    "gqa": (replace(synth.TINY, n_layers=2, n_kv_heads=2, max_batch=2), 2, 3, 21, 0.05),
    "mla": (MLA_TINY, 2, 3, 11, 0.2),
    "hybrid": (replace(MLA_TINY, name="hyb-tiny", attn_kind=synth.ATTN_HYBRID, n_layers=5, hybrid_period=4,
                       kda_dk=8, kda_dv=8), 2, 2, 6, 0.2),
    "dense": (replace(synth.TINY, n_layers=2, n_experts=0, top_k=0, ffn=0, shared_ffn=384, max_batch=2), 2, 2, 9, 0.05),
    "norm_topk_pool": (replace(MLA_TINY, norm_topk=1, n_layers=3, expert_pool_layers=2), 1, 4, 5, 0.2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_oracle_equals_numpy_reference(case):
    cfg, B, T, kv_len, sigma = CASES[case]
    spec = synth.Spec(seed=50, sigma=sigma)
    toks = synth.tokens(spec.seed, 0, cfg.vocab, B, T)
    c_orc = synth.host_caches(cfg, spec, B, kv_len, cache_batch=cfg.max_batch)
    c_ref = {k: v.copy() for k, v in c_orc.items()}
    a = oracle.decode_step(cfg, oracle.Provider(cfg, spec), toks, kv_len, c_orc, cache_batch=cfg.max_batch,
                           trace=True)
    b = ref_numpy.step(cfg, spec, toks, kv_len, c_ref)
    scale = np.abs(b["logits"]).max()
    np.testing.assert_allclose(a["logits"], b["logits"], rtol=0, atol=1e-10 * scale)
    if cfg.n_experts:
        np.testing.assert_array_equal(a["sel"], b["sel"])
        np.testing.assert_allclose(a["probs"], b["probs"], rtol=1e-10, atol=1e-15)
    for k in c_orc:
        if k == "kda_state":
            np.testing.assert_allclose(c_orc[k], c_ref[k], rtol=1e-6, atol=1e-6)
        else:
            np.testing.assert_array_equal(c_orc[k], c_ref[k])


def test_numpy_reference_rounding():
    """The reference's bf16 rounding: ties to even, a single rounding from float64."""
    r = ref_numpy.bf16_round
    assert r(1.0 + 2.0 ** -8) == 1.0
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert r(-3.0) == -3.0
    x = np.random.default_rng(0).normal(size=1000).astype(np.float32).astype(np.float64)
    lib = synth.lib()
    want = synth.bf16_to_f32(np.array([lib.synth_f32_to_bf16(float(v)) for v in x], np.uint16))
    np.testing.assert_array_equal(r(x), want.astype(np.float64))
