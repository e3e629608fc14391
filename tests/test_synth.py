"""The seeded input generator: published SplitMix64 outputs, rounding, distribution, layouts."""
import numpy as np

import synth


def test_splitmix64_published_outputs():
    # SplitMix64 from state 0 (Steele, Lea and Flood 2014; Vigna's splitmix64.c):
    # outputs are mix64(k * golden) for k = 1, 2, 3
    L = synth.lib()
    g = 0x9E3779B97F4A7C15
    outs = [L.synth_mix64((k * g) & 0xFFFFFFFFFFFFFFFF) for k in (1, 2, 3)]
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_bf16_round_to_nearest_even():
    f = synth.lib().synth_f32_to_bf16
    assert f(1.0) == 0x3F80
    assert f(np.float32(1.0 + 2 ** -8)) == 0x3F80  # tie -> even
    assert f(np.float32(1.0 + 3 * 2 ** -8)) == 0x3F82  # tie -> even (up)
    assert f(np.float32(1.0 + 2 ** -8 + 2 ** -20)) == 0x3F81
    assert f(-0.0) == 0x8000


def test_irwin_hall_stream():
    L = synth.lib()
    key = synth.key(5, "x")
    z = np.array([L.synth_ih(key, i) for i in range(2000)])
    assert np.all(np.abs(z) <= 131070)
    v = synth.normal_f32(5, "x", 2000, 1.0)
    np.testing.assert_array_equal(v, (z.astype(np.float32) * np.float32(synth.scale(1.0))))


def test_normal_statistics_and_determinism():
    a = synth.normal_f32(1, "stats", 1 << 20, 0.02)
    assert abs(a.mean()) < 1e-4
    assert abs(a.std() - 0.02) < 2e-4
    assert np.abs(a).max() <= 0.02 * 3.47
    # kurtosis of a sum of four uniforms is 3 - 1.2/4 = 2.7
    k = np.mean((a / a.std()) ** 4)
    assert abs(k - 2.7) < 0.03
    np.testing.assert_array_equal(a, synth.normal_f32(1, "stats", 1 << 20, 0.02))
    assert not np.array_equal(a[:100], synth.normal_f32(2, "stats", 100, 0.02))
    assert not np.array_equal(a[:100], synth.normal_f32(1, "stats2", 100, 0.02))
    # offsets address the same stream
    np.testing.assert_array_equal(a[1000:1100], synth.normal_f32(1, "stats", 100, 0.02, off=1000))


def test_bf16_stream_is_rounded_fp32_stream():
    f = synth.normal_f32(3, "w", 4096, 0.02)
    b = synth.normal_bf16(3, "w", 4096, 0.02)
    L = synth.lib()
    np.testing.assert_array_equal(b, np.array([L.synth_f32_to_bf16(float(x)) for x in f], dtype=np.uint16))


def test_tokens_uniform_in_range():
    t = synth.tokens(0, 0, 1000, 400, 25)
    assert t.shape == (400, 25)
    assert t.min() >= 0 and t.max() < 1000
    counts = np.bincount(t.ravel(), minlength=1000)
    assert counts.min() > 0


def test_tensor_list_shapes():
    tl = synth.tensor_list(synth.K3)
    names = [t.name for t in tl]
    assert len(names) == len(set(names))
    # 46 pool slots x 48 experts x 3 matrices
    assert sum(t.kind.startswith("exp_") for t in tl) == 46 * 48 * 3
    hyb = synth.tensor_list(synth.K3_HYBRID)
    assert sum(t.kind == "kda_wq" for t in hyb) == 69
    assert sum(t.kind == "w_dq" for t in hyb) == 23


def test_host_cache_layout():
    cfg = synth.TINY
    c = synth.host_caches(cfg, synth.Spec(seed=4), 2, 10, cache_batch=3)
    assert c["k"].shape == (2, 3, 4, cfg.kv_capacity, 64)
    assert np.all(c["k"][:, :, :, 10:] == 0) and np.all(c["k"][:, 2] == 0)
    d = 64
    expect = synth.normal_bf16(4, synth.gqa_cache_stream("K", 1, 1), 10 * d, 1.0, off=3 * synth.GQA_POS_STRIDE * d)
    np.testing.assert_array_equal(c["k"][1, 1, 3, :10].ravel(), expect)
