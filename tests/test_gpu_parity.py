"""GPU parity: the HIP megakernel (through the C ABI) against the fp64 oracle.

Bar (per workload): per (b, t) row max|logit_gpu - logit_oracle| <= 2e-2 * max|logit_oracle|,
identical argmax, identical expert selection in every layer, appended cache entries within
one bf16 rounding of the oracle's, untouched cache entries bitwise unchanged, and the
delta-rule state within fp32 accumulation error.
"""
import gc
import math
from dataclasses import replace

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-2
VECTOR_ONLY = 17  # matrix-core row threshold above the largest step: vector units only

_models = {}


def device_model(cfg, spec):
    """One resident model at a time (the K3-scale arenas take ~200 GB each)."""
    from synth.device_inputs import DeviceModel

    key = (cfg, spec.seed, spec.sigma, spec.gain_sigma, spec.cache_sigma, spec.state_sigma,
           tuple(sorted(spec.sigma_by_kind.items())))
    if key not in _models:
        for k in list(_models):
            _models.pop(k).close()
        gc.collect()
        torch.cuda.empty_cache()
        _models[key] = DeviceModel(cfg, spec, device=0)
    return _models[key]


def teardown_module(_):
    for k in list(_models):
        _models.pop(k).close()


def run_pair(cfg, spec, B, T, kv_len, step=0, mfma_min_rows=3):
    import oracle

    print(f"[case] {cfg.name} L={cfg.n_layers} B={B} T={T} kv_len={kv_len} seed={spec.seed} "
          f"mfma_min_rows={mfma_min_rows}", flush=True)
    toks = synth.tokens(spec.seed, step, cfg.vocab, B, T)
    dm = device_model(cfg, spec)
    dm.set_matrix_cores(mfma_min_rows)
    dm.fill_caches(B, kv_len)
    logits, route = dm.step(toks, kv_len)
    torch.cuda.synchronize()
    dm.poll()
    caches = synth.host_caches(cfg, spec, B, kv_len, cache_batch=cfg.max_batch)
    init = {k: v.copy() for k, v in caches.items()}
    ref = oracle.decode_step(cfg, oracle.Provider(cfg, spec), toks, kv_len, caches, cache_batch=cfg.max_batch,
                             trace=True)
    return dm, logits.cpu().numpy(), route.cpu().numpy(), ref, caches, init


def check_logits(got, ref):
    exp = ref["logits"]
    got = got.astype(np.float64)
    scale = np.abs(exp).max(axis=-1)
    err = np.abs(got - exp).max(axis=-1) / scale
    assert np.all(err <= TOL), f"per-row relative logit error {err.max():.3e} > {TOL}"
    ga, ea = got.argmax(-1), exp.astype(np.float32).argmax(-1)
    if not np.array_equal(ga, ea):
        srt = np.sort(exp, axis=-1)
        margin = (srt[..., -1] - srt[..., -2]) / scale
        pytest.fail(f"argmax differs: gpu {ga.ravel()} oracle {ea.ravel()}, oracle top-2 margin {margin.ravel()}")
    return err.max()


def check_route(route, ref):
    sel = ref["sel"]
    if not np.array_equal(route, sel):
        bad = np.argwhere((route != sel).any(-1))
        l, m = bad[0]
        p = np.sort(ref["probs"][l, m])[::-1]
        pytest.fail(f"expert selection differs at layer {l} row {m}: gpu {route[l, m]} oracle {sel[l, m]}, "
                    f"oracle probability margin {p[ref['sel'].shape[-1] - 1] - p[ref['sel'].shape[-1]]:.3e} "
                    f"({len(bad)} rows differ)")


def bf(u):
    return synth.bf16_to_f32(u).astype(np.float64)


def check_rounded(a_bits, b_bits, what, H):
    """a, b: bf16 patterns of the same quantity computed in fp32 (GPU) and fp64 (oracle) and
    rounded once to bf16. They may differ by one bf16 step of the larger magnitude, plus the
    difference of the two values before the rounding, which is the GPU's fp32 error. The entry is
    a projection of the normalised hidden state (width H), so that error is bounded, to first
    order, by gamma_H = H * 2^-24 of the entry vector's scale: Higham's bound for a sum of H
    products in fp32 (unit roundoff 2^-24), which covers the projection itself and, with room to
    spare, what reaches it from earlier layers (after 90 layers of the K3-scale share at batch 8
    the observed difference is 1.1e-4 of the vector's scale, against gamma_7168 = 4.3e-4). It
    matters only for entries close to zero. The last axis is the entry vector."""
    a, b = bf(a_bits), bf(b_bits)
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-30))) - 7)
    scale = np.abs(b).max(axis=-1, keepdims=True)
    gamma = H * 2.0 ** -24
    bad = np.abs(a - b) > step * 1.0001 + gamma * scale
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = ", ".join(f"{tuple(i)}: gpu {a[tuple(i)]:.6g} oracle {b[tuple(i)]:.6g}" for i in idx)
        pytest.fail(f"{what}: {bad.sum()} of {bad.size} new entries differ by more than one bf16 step: {rows}")


def check_cache(cfg, dm, caches, init, B, T, kv_len):
    new = slice(kv_len, kv_len + T)
    if cfg.attn_kind == synth.ATTN_GQA:
        gk, gv = dm.gqa_cache()
        pairs = [(gk, caches["k"], init["k"]), (gv, caches["v"], init["v"])]
        for g, o, i0 in pairs:
            # untouched entries bitwise equal, new entries within one bf16 rounding
            assert np.array_equal(g[:, :B, :, :kv_len], i0[:, :B, :, :kv_len])
            check_rounded(g[:, :B, :, new], o[:, :B, :, new], "GQA cache", cfg.hidden)
    else:
        g = dm.latent_cache()
        o, i0 = caches["latent"], init["latent"]
        assert np.array_equal(g[:, :B, :kv_len], i0[:, :B, :kv_len])
        check_rounded(g[:, :B, new], o[:, :B, new], "latent cache", cfg.hidden)
        if "kda_state" in caches:
            s = dm.kda_state()[:, :B]
            r = caches["kda_state"][:, :B]
            err = np.abs(s - r).max() / np.abs(r).max()
            assert err < 1e-4, f"delta-rule state error {err:.3e}"


def parity(cfg, spec, B, T, kv_len, mfma_min_rows=3):
    dm, got, route, ref, caches, init = run_pair(cfg, spec, B, T, kv_len, mfma_min_rows=mfma_min_rows)
    err = check_logits(got, ref)
    check_route(route, ref)
    check_cache(cfg, dm, caches, init, B, T, kv_len)
    print(f"[ok] {cfg.name} B={B} T={T}: max rel logit err {err:.2e}", flush=True)


# --------------------------------------------------------------------------------------------
# small models: several tiles, ragged tails, every seed
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_batch1(seed):
    w = synth.WORKLOADS["c1"]
    parity(w.model, synth.Spec(seed=seed), w.batch, w.new_tokens, w.kv_len)


@pytest.mark.parametrize("B,T,kv_len", [(2, 3, 37), (4, 4, 0), (8, 2, 129), (1, 8, 5)])
def test_tiny_shapes(B, T, kv_len):
    parity(synth.TINY, synth.Spec(seed=5), B, T, kv_len)


@pytest.mark.parametrize("B,T,kv_len", [(2, 1, 50), (1, 3, 7), (4, 1, 129)])
def test_tiny_shapes_matrix_cores_small(B, T, kv_len):
    # the matrix-core executor below its default threshold (2..4 token rows)
    parity(synth.TINY, synth.Spec(seed=8), B, T, kv_len, mfma_min_rows=2)


@pytest.mark.parametrize("B,T,kv_len", [(8, 2, 129), (1, 8, 5)])
def test_tiny_shapes_vector_units(B, T, kv_len):
    # the vector-unit GEMV executor at 5..16 rows (the matrix cores are the default there)
    parity(synth.TINY, synth.Spec(seed=5), B, T, kv_len, mfma_min_rows=VECTOR_ONLY)


# row lengths that are not whole 32-column units: 5..16 rows fall back to the vector units
TINY_RAGGED = replace(synth.TINY, name="tiny-ragged", hidden=264, ffn=520, vocab=1000)


@pytest.mark.parametrize("B,T,kv_len", [(8, 1, 40), (2, 4, 3)])
def test_tiny_ragged_rows(B, T, kv_len):
    parity(TINY_RAGGED, synth.Spec(seed=7), B, T, kv_len)


# head dims the host admits besides 64 and 128: one and three 32-column steps per score multiply,
# two and six 16-column value tiles
@pytest.mark.parametrize("head_dim", [32, 96])
def test_tiny_head_dims(head_dim):
    cfg = replace(synth.TINY, name=f"tiny-hd{head_dim}", head_dim=head_dim)
    parity(cfg, synth.Spec(seed=10), 2, 3, 70)


def test_tiny_peaked_attention():
    # larger query/key weights make attention sharply peaked, so attention errors reach the logits
    spec = synth.Spec(seed=6, sigma_by_kind={"wq": 0.25, "wk": 0.25, "wv": 0.1, "wo": 0.1})
    parity(synth.TINY, spec, 2, 3, 64)


def test_mid_batch1():
    w = synth.WORKLOADS["c2"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


def test_mid_batch4():
    w = synth.WORKLOADS["c2b4"]
    parity(w.model, synth.Spec(seed=1), w.batch, w.new_tokens, w.kv_len)


MID_SMALL = replace(synth.MID, name="mid-2layer", n_layers=2)


# 4 query heads per KV head: T = 4 fills one 16-row attention tile exactly, T = 5 spills 4 rows into
# a second; peaked attention so that score errors reach the logits
@pytest.mark.parametrize("B,T,kv_len", [(2, 4, 300), (2, 5, 300)])
def test_mid_attention_row_tiles(B, T, kv_len):
    spec = synth.Spec(seed=8, sigma_by_kind={"wq": 0.1, "wk": 0.1})
    parity(MID_SMALL, spec, B, T, kv_len)


K3_SMALL = replace(synth.K3, name="k3-2layer", n_layers=2, expert_pool_layers=0)
HYB_SMALL = replace(synth.K3_HYBRID, name="hybrid-4layer", n_layers=4, expert_pool_layers=0)


# (2, 8, 4096): 16 token rows over 65 splits of 64 positions; the split-KV merge gives each
# workgroup 16 (row, head, 32-value) tasks, more than one LDS batch holds (15)
@pytest.mark.parametrize("B,T,kv_len", [(1, 1, 4096), (3, 2, 1000), (1, 7, 4096), (8, 1, 33), (2, 8, 4096)])
def test_k3_two_layers(B, T, kv_len):
    parity(K3_SMALL, synth.Spec(seed=2), B, T, kv_len)


# The router folded onto the attention output projection (1-2 rows on the vector executor, up to 8
# on the matrix cores) against the separate router phase (MK_NO_ROUTER_FUSION): both match the oracle,
# select the same experts, and their logits agree to fp32 summation-order differences.
@pytest.mark.parametrize("B,T,kv_len,rows", [(1, 1, 4096, 3), (2, 1, 500, 3), (8, 1, 33, 3), (1, 7, 300, 3),
                                              (2, 1, 77, 2), (4, 1, 300, 3), (1, 3, 64, 3)])
def test_router_fusion_against_router_phase(B, T, kv_len, rows, monkeypatch):
    runs = {}
    for fused in (True, False):
        if fused:
            monkeypatch.delenv("MK_NO_ROUTER_FUSION", raising=False)
        else:
            monkeypatch.setenv("MK_NO_ROUTER_FUSION", "1")
        dm, got, route, ref, caches, init = run_pair(K3_SMALL, synth.Spec(seed=4), B, T, kv_len, mfma_min_rows=rows)
        check_logits(got, ref)
        check_route(route, ref)
        check_cache(K3_SMALL, dm, caches, init, B, T, kv_len)
        runs[fused] = (got, route)
    assert np.array_equal(runs[True][1], runs[False][1])
    diff = np.abs(runs[True][0] - runs[False][0]).max() / np.abs(runs[False][0]).max()
    assert diff < 1e-4, f"fused and separate router phases differ by {diff:.3e} of the logit scale"


# The split-KV merge and W_uv in one phase (1 and 2 token rows of MLA layers on the vector executor,
# where 4 or 2 workgroups split each head's latent values and the last adds their partials, and 3
# to 8 rows on the matrix cores, whole heads per workgroup)
# against the separate merge phase (MK_NO_MERGE_FUSION): both match the oracle, select the same
# experts, and their logits agree to fp32 summation-order differences. 1 row over 5 positions has a
# single split.
@pytest.mark.parametrize("B,T,kv_len", [(2, 1, 4096), (1, 2, 300), (1, 1, 4096), (1, 1, 5), (4, 1, 4096),
                                         (1, 4, 300), (8, 1, 4096), (2, 4, 300), (1, 7, 4096), (3, 1, 500)])
def test_merge_fusion_against_merge_phase(B, T, kv_len, monkeypatch):
    runs = {}
    for fused in (True, False):
        if fused:
            monkeypatch.delenv("MK_NO_MERGE_FUSION", raising=False)
        else:
            monkeypatch.setenv("MK_NO_MERGE_FUSION", "1")
        dm, got, route, ref, caches, init = run_pair(K3_SMALL, synth.Spec(seed=9), B, T, kv_len)
        check_logits(got, ref)
        check_route(route, ref)
        check_cache(K3_SMALL, dm, caches, init, B, T, kv_len)
        runs[fused] = (got, route)
    assert np.array_equal(runs[True][1], runs[False][1])
    diff = np.abs(runs[True][0] - runs[False][0]).max() / np.abs(runs[False][0]).max()
    assert diff < 1e-4, f"fused and separate merge phases differ by {diff:.3e} of the logit scale"


# 2-row and 1-row steps in turn on one context (the model's single MLA layer fuses the merge with
# 2 latent blocks at 2 rows and 4 at 1 row): each step's counters start at zero whatever the
# previous step's row count
def test_merge_fusion_row_counts_alternate():
    for B in (2, 1, 2, 1):
        parity(HYB_SMALL, synth.Spec(seed=3), B, 1, 300)


# renormalised router weights (norm_topk) with a shared expert: the folded router at 1 row (vector
# units) and 4 rows (matrix cores), and the separate router phase at 16 rows
@pytest.mark.parametrize("B,T,kv_len", [(1, 1, 40), (4, 1, 40), (2, 8, 30)])
def test_tiny_norm_topk_shared(B, T, kv_len):
    cfg = replace(synth.TINY, name="tiny-normtopk", norm_topk=1, shared_ffn=256)
    parity(cfg, synth.Spec(seed=8), B, T, kv_len)


# more experts than half the grid: each workgroup takes whole folded router rows (no column parts)
@pytest.mark.parametrize("B,T", [(1, 1), (4, 1), (1, 5)])
def test_router_fusion_whole_rows(B, T):
    cfg = replace(synth.TINY, name="tiny-200experts", n_experts=200, top_k=2)
    parity(cfg, synth.Spec(seed=6), B, T, 40)


# a share of the same model over twice the tensor-parallel ranks: 8 heads, padded to the 16 rows of
# the attention tiles (the absorbed query, the merge and W_uv keep 8)
@pytest.mark.parametrize("B,T,kv_len", [(1, 1, 4096), (8, 1, 700), (1, 7, 2000), (2, 1, 700)])
def test_k3_two_layers_eight_heads(B, T, kv_len):
    parity(replace(K3_SMALL, name="k3-2layer-8heads", n_heads=8), synth.Spec(seed=5), B, T, kv_len)


def test_hybrid_four_layers_eight_heads():
    parity(replace(HYB_SMALL, name="hybrid-4layer-8heads", n_heads=8), synth.Spec(seed=6), 2, 1, 300)


def test_k3_two_layers_widest_rope():
    # rope_dim 128, the widest the host admits: 640-wide latent rows fill the register prefetch of
    # the next 32-position sub-tile exactly (2560 units of 16 bytes); batch 4 over 4097 positions
    # gives splits of 96 positions (three sub-tiles), so later sub-tiles go through it
    cfg = replace(K3_SMALL, name="k3-2layer-rope128", rope_dim=128)
    parity(cfg, synth.Spec(seed=9), 4, 1, 4096)


@pytest.mark.parametrize("B,T,kv_len", [(1, 1, 4096), (1, 7, 600)])
def test_k3_two_layers_rope128_on_hybrid_kernels(B, T, kv_len):
    # an MLA model whose rope dimension is not 64 runs on the hybrid family's kernels: the 1-row
    # instance and the matrix-core verify instance of that family
    cfg = replace(K3_SMALL, name="k3-2layer-rope128", rope_dim=128)
    parity(cfg, synth.Spec(seed=10), B, T, kv_len)


# contexts longer than 921 chunks of 16 positions: the chunks grow with the context (one per
# workgroup at most), so the merge sees at most 256 splits. 20000 positions at batch 1: 209 splits
# of 96 positions; 30000 at batch 2: 118 splits of 256; 131072 at batch 1: 241 splits of 544
# (17 sub-tiles each); the 7-token verify over 50000 positions: 224 splits of 224
@pytest.mark.parametrize("B,T,kv_len", [(1, 1, 20000), (2, 1, 30000), (1, 1, 131072), (1, 7, 50000)])
def test_k3_two_layers_long_context(B, T, kv_len):
    cfg = replace(K3_SMALL, name="k3-2layer-long", max_batch=2, kv_capacity=131080)
    parity(cfg, synth.Spec(seed=31), B, T, kv_len)


def test_k3_two_layers_batch8_vector_units():
    parity(K3_SMALL, synth.Spec(seed=2), 8, 1, 33, mfma_min_rows=VECTOR_ONLY)


def test_k3_two_layers_peaked_mla():
    spec = synth.Spec(seed=3, sigma_by_kind={"w_uq": 0.1, "w_uk": 0.1, "w_dkv": 0.05, "w_uv": 0.1, "wo": 0.05})
    parity(K3_SMALL, spec, 2, 3, 300)


# (1, 1): the 1-row instance of the hybrid family (its MLA layer with the rope dimension read from
# the parameters, one token row as a compile-time constant)
@pytest.mark.parametrize("B,T", [(8, 1), (2, 3), (1, 1)])
def test_hybrid_four_layers(B, T):
    parity(HYB_SMALL, synth.Spec(seed=4), B, T, 517)


# --------------------------------------------------------------------------------------------
# temperature / top-p sampling fused after the LM head
# --------------------------------------------------------------------------------------------
SAMPLE_LOGIT_TOL = 2e-3  # logit error (relative to the row's largest logit) the sampling check allows for


def sample_check(cfg, spec, B, T, kv_len, temperature, top_p, useed, exact_all=False):
    """Every sampled token must be the oracle's draw, or differ from it only where the draw sits
    on a decision boundary within what the logits' error (and fp32 sums over the vocabulary) can
    move: the oracle's running kept mass around the token must straddle u * mass within that
    slack, and the token must be kept or within the slack of the threshold. Most positions (all,
    for sharp distributions) must match exactly."""
    import oracle
    from oracle import sampling

    toks = synth.tokens(spec.seed, 4, cfg.vocab, B, T)
    u = np.random.default_rng(useed).random((B, T))  # the caller's uniform numbers (seeded)
    print(f"[case] sample {cfg.name} B={B} T={T} kv_len={kv_len} temperature={temperature} top_p={top_p}",
          flush=True)
    dm = device_model(cfg, spec)
    dm.set_matrix_cores(3)
    dm.fill_caches(B, kv_len)
    got, logits = dm.step_sample(toks, kv_len, temperature, top_p, u)
    torch.cuda.synchronize()
    dm.poll()
    got = got.cpu().numpy()
    caches = synth.host_caches(cfg, spec, B, kv_len, cache_batch=cfg.max_batch)
    ref = oracle.decode_step(cfg, oracle.Provider(cfg, spec), toks, kv_len, caches, cache_batch=cfg.max_batch)
    check_logits(logits.cpu().numpy(), ref)
    exact = 0
    for b in range(B):
        for t in range(T):
            lg = ref["logits"][b, t]
            r = sampling.sample(lg, temperature, top_p, u[b, t])
            s = int(got[b, t])
            assert 0 <= s < cfg.vocab
            if s == r["token"]:
                exact += 1
                continue
            # p moves by up to a factor exp(+-2 eps / temperature) when each logit moves by eps
            rel = math.expm1(2 * SAMPLE_LOGIT_TOL * np.abs(lg).max() / temperature) + 1e-4
            p, tau = r["p"], r["tau"]
            near = np.abs(p - tau) <= rel * tau
            slack = rel * r["mass"] + p[near].sum()
            kp = np.where(r["kept"] | near, p, 0.0)
            before, after = kp[:s].sum(), kp[:s + 1].sum()
            assert r["kept"][s] or near[s], f"({b},{t}): token {s} outside the nucleus (p {p[s]:.3e}, tau {tau:.3e})"
            assert before - slack <= r["target"] <= after + slack, (
                f"({b},{t}): token {s} covers [{before:.6f}, {after:.6f}], the draw is {r['target']:.6f} "
                f"(oracle token {r['token']}, slack {slack:.2e})")
    need = B * T if exact_all else int(0.75 * B * T)
    assert exact >= need, f"only {exact} of {B * T} draws equal the oracle's"
    print(f"[ok] sample {cfg.name}: {exact}/{B * T} draws equal the oracle's", flush=True)


@pytest.mark.parametrize("temperature,top_p,exact_all", [(1.0, 0.9, False), (0.7, 0.5, False), (1.5, 1.0, False),
                                                         (0.01, 0.9, True), (0.03, 0.3, True)])
def test_sample_tiny(temperature, top_p, exact_all):
    sample_check(synth.TINY, synth.Spec(seed=21, sigma=0.05), 4, 2, 30, temperature, top_p, 5, exact_all)


@pytest.mark.parametrize("temperature,top_p,exact_all", [(1.0, 0.95, False), (0.005, 0.8, True)])
def test_sample_k3_two_layers(temperature, top_p, exact_all):
    # a vocabulary slice of exactly one register tile (40960 = 512 threads x 80)
    sample_check(K3_SMALL, synth.Spec(seed=22), 1, 7, 4096, temperature, top_p, 6, exact_all)


def test_sample_dense_two_layers():
    # a vocabulary of several tiles (151936 logits)
    sample_check(DENSE_SMALL, synth.Spec(seed=23), 2, 2, 1000, 0.02, 0.9, 7, False)


# dense decoders (n_experts = 0): no router, the SwiGLU block alone, one phase fewer per layer
TINY_DENSE = replace(synth.TINY, name="tiny-dense", n_experts=0, top_k=0, ffn=0, shared_ffn=512)
DENSE_SMALL = replace(synth.DENSE, name="dense-2layer", n_layers=2)


@pytest.mark.parametrize("B,T,kv_len,rows", [(1, 1, 64, 3), (2, 3, 37, 3), (8, 2, 100, 3), (8, 2, 100, VECTOR_ONLY),
                                             (1, 8, 5, 3)])
def test_tiny_dense(B, T, kv_len, rows):
    parity(TINY_DENSE, synth.Spec(seed=19), B, T, kv_len, mfma_min_rows=rows)


def test_tiny_dense_ragged_rows():
    # a dense width that is not whole 32-column units: every step on the vector units
    parity(replace(TINY_DENSE, name="tiny-dense-ragged", shared_ffn=520), synth.Spec(seed=19), 4, 2, 21)


@pytest.mark.parametrize("B,T", [(1, 1), (8, 1), (1, 7)])
def test_dense_two_layers(B, T):
    parity(DENSE_SMALL, synth.Spec(seed=20), B, T, 4096)


# two token rows of the dense model on the matrix cores (its default from two rows)
def test_dense_two_layers_two_rows_matrix_cores():
    parity(DENSE_SMALL, synth.Spec(seed=21), 2, 1, 4096, mfma_min_rows=2)


# GQA over 40000 positions: 8 kv heads, 32 splits of 1264 positions per (sequence, kv head); and
# batch 2 over 60000 (16 splits of 3760)
@pytest.mark.parametrize("B,kv_len", [(1, 40000), (2, 60000)])
def test_dense_two_layers_long_context(B, kv_len):
    cfg = replace(DENSE_SMALL, name="dense-2layer-long", max_batch=2, kv_capacity=60008)
    parity(cfg, synth.Spec(seed=32), B, 1, kv_len)


# --------------------------------------------------------------------------------------------
# full sizes, the launch configuration the benchmark times
# --------------------------------------------------------------------------------------------
def test_k3_full_batch1():
    w = synth.WORKLOADS["c3"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


def test_k3_full_verify_t7():
    w = synth.WORKLOADS["c4"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


def test_k3_full_batch8():
    w = synth.WORKLOADS["c3b8"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


def test_hybrid_full_batch8():
    w = synth.WORKLOADS["c5"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


def test_dense_full_batch1():
    w = synth.WORKLOADS["dense"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


# --------------------------------------------------------------------------------------------
# greedy steps: argmax fused after the LM head, draft acceptance on the device
# --------------------------------------------------------------------------------------------
def oracle_greedy(cfg, spec, toks, kv_len):
    import oracle

    from greedy_ref import greedy_tokens

    caches = synth.host_caches(cfg, spec, toks.shape[0], kv_len, cache_batch=cfg.max_batch)
    ref = oracle.decode_step(cfg, oracle.Provider(cfg, spec), toks, kv_len, caches, cache_batch=cfg.max_batch)
    return greedy_tokens(ref["logits"])


def greedy_check(cfg, spec, toks, kv_len, expect_accepted=None):
    from greedy_ref import accepted_drafts, greedy_tokens

    B, T = toks.shape
    print(f"[case] greedy {cfg.name} B={B} T={T} kv_len={kv_len} seed={spec.seed}", flush=True)
    dm = device_model(cfg, spec)
    dm.set_matrix_cores(3)
    dm.fill_caches(B, kv_len)
    logits = torch.empty((B, T, cfg.vocab), dtype=torch.float32, device="cuda")
    am, acc = dm.step_greedy(toks, kv_len, logits=logits)
    torch.cuda.synchronize()
    dm.poll()
    am, acc = am.cpu().numpy(), acc.cpu().numpy()
    # the fused selection agrees with the logits the same step wrote, and with the oracle's
    assert np.array_equal(am, greedy_tokens(logits.cpu().numpy())), "fused argmax differs from the step's logits"
    ref = oracle_greedy(cfg, spec, toks, kv_len)
    assert np.array_equal(am, ref), f"greedy tokens differ: gpu {am.ravel()} oracle {ref.ravel()}"
    assert np.array_equal(acc, accepted_drafts(toks, ref)), f"accepted {acc} vs {accepted_drafts(toks, ref)}"
    if expect_accepted is not None:
        assert acc.tolist() == list(expect_accepted)
    # the same step without writing logits gives the same selection
    am2, acc2 = dm.step_greedy(toks, kv_len)
    torch.cuda.synchronize()
    dm.poll()
    assert np.array_equal(am2.cpu().numpy(), am) and np.array_equal(acc2.cpu().numpy(), acc)
    print(f"[ok] greedy {cfg.name} B={B} T={T}: accepted {acc.tolist()}", flush=True)


@pytest.mark.parametrize("B,T,kv_len", [(1, 1, 64), (2, 4, 37), (8, 2, 100)])
def test_greedy_tiny(B, T, kv_len):
    spec = synth.Spec(seed=9)
    greedy_check(synth.TINY, spec, synth.tokens(spec.seed, 0, synth.TINY.vocab, B, T), kv_len)


def test_greedy_acceptance_tiny():
    """Drafts built from the oracle's own greedy continuation are accepted up to the first planted
    mismatch."""
    cfg, spec, B, T, kv_len = synth.TINY, synth.Spec(seed=10), 3, 5, 40
    toks = synth.tokens(spec.seed, 0, cfg.vocab, B, 1)
    for _ in range(T - 1):  # extend every sequence by the oracle's greedy token for its prefix
        toks = np.concatenate([toks, oracle_greedy(cfg, spec, toks, kv_len)[:, -1:]], axis=1)
    toks[0, 3] = (toks[0, 3] + 1) % cfg.vocab  # sequence 0: drafts 1 and 2 accepted
    toks[1, 1] = (toks[1, 1] + 1) % cfg.vocab  # sequence 1: none
    greedy_check(cfg, spec, toks, kv_len, expect_accepted=[2, 0, 4])


def test_greedy_k3_two_layers_verify():
    spec = synth.Spec(seed=2)
    greedy_check(K3_SMALL, spec, synth.tokens(spec.seed, 3, K3_SMALL.vocab, 1, 7), 4096)


# --------------------------------------------------------------------------------------------
# speculative decoding loop: verify steps with fused acceptance, kv_len rolled back to the
# accepted prefix between rounds
# --------------------------------------------------------------------------------------------
MLA_SMALL = replace(synth.K3, name="mla-small", n_layers=2, hidden=1024, vocab=4096, q_lora=512, n_experts=8,
                    ffn=512, shared_ffn=256, expert_pool_layers=0, max_batch=1, kv_capacity=160)


def oracle_greedy_continuation(cfg, spec, first, kv_len, n):
    """The target's plain greedy decode: n tokens after `first`, one oracle step per token, the
    oracle's cache growing by one row per step. Returns the tokens, the oracle's caches and the
    smallest top-2 logit margin (relative to the row's largest logit)."""
    import oracle

    from greedy_ref import greedy_tokens

    caches = synth.host_caches(cfg, spec, 1, kv_len, cache_batch=cfg.max_batch)
    prov = oracle.Provider(cfg, spec)
    seq, margin = [first], np.inf
    for j in range(n):
        ref = oracle.decode_step(cfg, prov, np.array([[seq[-1]]], dtype=np.int32), kv_len + j, caches,
                                 cache_batch=cfg.max_batch)
        lg = ref["logits"][0, 0]
        top = np.sort(lg)[-2:]
        margin = min(margin, (top[1] - top[0]) / np.abs(lg).max())
        seq.append(int(greedy_tokens(lg)))
    return np.array(seq, dtype=np.int32), caches, margin


def speculative_loop(cfg, spec, T, kv_len, keep):
    """Round r verifies the last yielded token followed by T-1 drafts: the target's own greedy
    continuation with draft keep[r]+1 changed, so exactly keep[r] drafts are accepted (the drafts
    after the changed one are right again: acceptance stops at the first mismatch). The round
    yields the accepted drafts and the target's token after them, and the next round starts at
    kv_len + the tokens yielded so far, overwriting the cache rows of the rejected drafts. The
    yielded tokens must be the plain greedy continuation, and the cache rows of the yielded
    positions those of the plain decode."""
    n = sum(k + 1 for k in keep)
    assert kv_len + n + T <= cfg.kv_capacity
    first = int(synth.tokens(spec.seed, 11, cfg.vocab, 1, 1)[0, 0])
    seq, caches, margin = oracle_greedy_continuation(cfg, spec, first, kv_len, n + T - 1)
    print(f"[case] speculative {cfg.name} T={T} kv_len={kv_len} keep={keep} seed={spec.seed} "
          f"oracle top-2 margin {margin:.2e}", flush=True)
    dm = device_model(cfg, spec)
    dm.set_matrix_cores(3)
    dm.fill_caches(1, kv_len)
    pos = 0
    for r, k in enumerate(keep):
        toks = seq[pos:pos + T].copy()
        if k + 1 < T:
            toks[k + 1] = (toks[k + 1] + 1) % cfg.vocab
        am, acc = dm.step_greedy(toks[None, :], kv_len + pos)
        torch.cuda.synchronize()
        dm.poll()
        am, acc = am.cpu().numpy()[0], int(acc.cpu().numpy()[0])
        assert acc == k, f"round {r}: {acc} drafts accepted, expected {k} (gpu tokens {am}, drafts {toks})"
        want = seq[pos + 1:pos + acc + 2]
        assert np.array_equal(am[:acc + 1], want), f"round {r}: yielded {am[:acc + 1]}, greedy decode {want}"
        pos += acc + 1
    assert pos == n
    rows = slice(kv_len, kv_len + pos)
    if cfg.attn_kind == synth.ATTN_GQA:
        gk, gv = dm.gqa_cache()
        pairs = [(gk[:, :1, :, rows], caches["k"][:, :1, :, rows]), (gv[:, :1, :, rows], caches["v"][:, :1, :, rows])]
    else:
        pairs = [(dm.latent_cache()[:, :1, rows], caches["latent"][:, :1, rows])]
    for g, o in pairs:  # a row left from a rejected draft would differ at O(1)
        a, b = bf(g), bf(o)
        err = (np.abs(a - b).max(axis=-1) / np.abs(b).max(axis=-1)).max()
        assert err < 2e-2, f"cache rows of the yielded tokens differ from the greedy decode's: {err:.3e}"
    print(f"[ok] speculative {cfg.name}: {len(keep)} rounds yielded {pos} tokens", flush=True)


def test_speculative_loop_tiny_t8():
    # one anchor + 7 drafts per round
    # weights at sigma 0.05: a greedy continuation that does not settle into a repeated token
    speculative_loop(synth.TINY, synth.Spec(seed=12, sigma=0.05), 8, 40, [7, 0, 3, 1, 6, 2])


def test_speculative_loop_mla_t7():
    # the verify workload's shape: one anchor + 6 drafts, latent cache
    speculative_loop(MLA_SMALL, synth.Spec(seed=15, sigma=0.05), 7, 64, [6, 2, 0, 5, 3])


# --------------------------------------------------------------------------------------------
# the vector-unit instances built for 2 and 4 token rows (batch 2 runs on them by default)
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,B,kv_len,rows", [
    (K3_SMALL, 2, 4096, 3), (synth.TINY, 2, 50, 3), (DENSE_SMALL, 2, 4096, 3),
    (K3_SMALL, 4, 4096, VECTOR_ONLY), (synth.TINY, 4, 77, VECTOR_ONLY)], ids=lambda v: getattr(v, "name", v))
def test_vector_instances_two_and_four_rows(cfg, B, kv_len, rows):
    parity(cfg, synth.Spec(seed=24), B, 1, kv_len, mfma_min_rows=rows)


# --------------------------------------------------------------------------------------------
# seeds 1 and 2 on every workload's shape (2- and 4-layer versions of the large models)
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("wl", ["c2", "c3", "c4", "c5"])
def test_workload_seeds(wl, seed):
    w = synth.WORKLOADS[wl]
    cfg = {"c2": w.model, "c3": K3_SMALL, "c4": K3_SMALL, "c5": HYB_SMALL}[wl]
    parity(cfg, synth.Spec(seed=seed), w.batch, w.new_tokens, w.kv_len)


def test_k3_full_batch2():
    w = synth.WORKLOADS["c3b2"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


def test_k3_full_batch4():
    w = synth.WORKLOADS["c3b4"]
    parity(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


# --------------------------------------------------------------------------------------------
# run-to-run reproducibility: every output element is owned by one lane and every sum runs in a
# fixed order, so the same step on the same inputs gives the same bits
# --------------------------------------------------------------------------------------------
def bitwise_repeat(cfg, spec, B, T, kv_len, mfma_min_rows=3):
    print(f"[case] repeat {cfg.name} B={B} T={T} kv_len={kv_len} seed={spec.seed}", flush=True)
    dm = device_model(cfg, spec)
    dm.set_matrix_cores(mfma_min_rows)
    dm.fill_caches(B, kv_len)
    kv0 = dm.kv.clone()
    st0 = dm.state.clone() if dm.state is not None else None
    toks = synth.tokens(spec.seed, 6, cfg.vocab, B, T)
    l1, r1 = dm.step(toks, kv_len)
    torch.cuda.synchronize()
    dm.poll()
    kv1 = dm.kv.clone()
    st1 = dm.state.clone() if st0 is not None else None
    # snapshot restore: the cache rows past kv_len and the delta-rule state go back to the snapshot
    dm.kv.copy_(kv0)
    if st0 is not None:
        dm.state.copy_(st0)
    l2, r2 = dm.step(toks, kv_len)
    torch.cuda.synchronize()
    dm.poll()
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "logits differ between two runs of one step"
    assert torch.equal(r1, r2), "routes differ between two runs of one step"
    assert torch.equal(dm.kv, kv1), "appended cache rows differ between two runs"
    if st0 is not None:
        assert torch.equal(dm.state.view(torch.int32), st1.view(torch.int32)), "delta-rule state differs"
    print(f"[ok] repeat {cfg.name} B={B} T={T}: bitwise equal", flush=True)


@pytest.mark.parametrize("cfg,B,T,kv_len,rows", [
    (K3_SMALL, 8, 1, 4096, 3), (K3_SMALL, 1, 1, 4096, 3), (HYB_SMALL, 8, 1, 517, 3), (MID_SMALL, 4, 1, 2048, 3),
    (MID_SMALL, 2, 1, 2048, 3), (synth.TINY, 8, 2, 100, VECTOR_ONLY)], ids=lambda v: getattr(v, "name", v))
def test_bitwise_run_to_run(cfg, B, T, kv_len, rows):
    bitwise_repeat(cfg, synth.Spec(seed=25), B, T, kv_len, rows)


def test_bitwise_run_to_run_full_verify():
    w = synth.WORKLOADS["c4"]
    bitwise_repeat(w.model, synth.Spec(seed=0), w.batch, w.new_tokens, w.kv_len)


# --------------------------------------------------------------------------------------------
# device-side errors: a token outside the vocabulary is reported by mk_poll, which poisons the
# context; the step itself completes (the token is read as token 0), so nothing faults or hangs
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("bad", ["vocab", "negative"])
def test_out_of_vocabulary_token_poisons_context(bad):
    import decode_megakernel_cu_amd as mk
    from synth.device_inputs import DeviceModel

    cfg, spec = synth.TINY, synth.Spec(seed=26)
    for k in list(_models):  # a context of its own: this one ends poisoned
        _models.pop(k).close()
    print(f"[case] bad token ({bad}) {cfg.name}", flush=True)
    dm = DeviceModel(cfg, spec, device=0)
    try:
        dm.fill_caches(2, 10)
        toks = np.array([[5], [cfg.vocab if bad == "vocab" else -3]], dtype=np.int32)
        dm.step(toks, 10)
        torch.cuda.synchronize()
        with pytest.raises(mk.MkError) as e:
            dm.poll()
        assert e.value.code == mk.MK_E_DEVICE
        assert "token 1 of the step" in str(e.value)
        with pytest.raises(mk.MkError) as e:  # the context stays poisoned
            dm.poll()
        assert e.value.code == mk.MK_E_DEVICE
        with pytest.raises(mk.MkError) as e:
            dm.step(np.array([[5], [6]], dtype=np.int32), 10)
        assert e.value.code == mk.MK_E_STATE
        assert "poisoned" in mk.mk_last_error()
    finally:
        dm.close()
    print(f"[ok] bad token ({bad}): MK_E_DEVICE, then MK_E_STATE", flush=True)
