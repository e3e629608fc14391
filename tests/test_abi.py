"""The C ABI on the host: exports, size queries, and every argument error (no GPU needed)."""
import ctypes
import os
import re
import subprocess
from dataclasses import replace

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mk():
    import decode_megakernel_cu_amd as mk

    return mk


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(mk_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(mk):
    names = declared_functions()
    assert names == sorted(mk.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", mk.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(l.split()[-1] for l in out.stdout.splitlines() if " T " in l)
    for n in names:
        assert n in exported, n
        assert hasattr(mk.lib, n)


def test_traced_build_exports_the_same_symbols(mk):
    # libmk_trace.so: the same sources with the per-phase stamp code compiled in
    path = os.path.join(ROOT, "decode_megakernel_cu_amd", "libmk_trace.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    exported = set(l.split()[-1] for l in out.stdout.splitlines() if " T " in l)
    for n in declared_functions():
        assert n in exported, n


def test_default_build_refuses_tracing(mk, host_ctx):
    # the default library carries no stamp code: enabling tracing is refused, disabling is fine
    _, ctx = host_ctx
    if os.path.basename(mk.LIB_PATH) != "libmk.so":
        pytest.skip("another build of the library is loaded")
    with pytest.raises(mk.MkError) as e:
        mk.mk_set_trace(ctx, True)
    assert e.value.code == mk.MK_E_UNSUPPORTED
    assert "MK_DEVICE_TRACE" in mk.mk_last_error()
    mk.mk_set_trace(ctx, False)


def test_library_is_gfx950():
    import decode_megakernel_cu_amd as mk

    out = subprocess.run(["strings", mk.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "gfx950" in out


def test_struct_sizes_match_header(mk):
    # mk_config: 25 int32 (preset first) + 2 float; mk_tensor_desc: 4 int32 + pointer + uint64
    assert ctypes.sizeof(mk.MkConfig) == 27 * 4
    assert mk.MkConfig._fields_[0][0] == "preset"
    assert ctypes.sizeof(mk.MkTensorDesc) == 32
    assert ctypes.sizeof(mk.MkSizes) == 32


def sizes(mk, cfg):
    return mk.mk_query_sizes(mk.config(cfg))


def test_query_sizes_match_documented_layouts(mk):
    s = sizes(mk, synth.K3)
    c = synth.K3
    assert s.kv_bytes == c.n_layers * c.max_batch * c.kv_capacity * c.latent_dim * 2
    assert s.kda_state_bytes == 0
    # every weight tensor is in the arena once, plus each MoE layer's router folded onto its
    # attention output projection (fp32 [n_experts][hidden + n_heads * v_dim], derived at load
    # time), the layer table and 256-byte padding
    total = sum(synth.numel(t.shape) * (4 if t.dist == "sigmoid" else 2) for t in synth.tensor_list(c))
    total += c.n_layers * c.n_experts * (c.hidden + c.n_heads * c.v_dim) * 4
    assert total <= s.arena_bytes <= total + 256 * (len(synth.tensor_list(c)) + 1) + 2 * c.n_layers * 256
    assert s.arena_bytes < 288e9  # fits one MI355X
    h = sizes(mk, synth.K3_HYBRID)
    nk = len(synth.K3_HYBRID.kda_layers())
    assert h.kda_state_bytes == nk * 8 * 16 * 128 * 128 * 4
    assert h.kv_bytes == 23 * 8 * c.kv_capacity * c.latent_dim * 2
    t = sizes(mk, synth.TINY)
    tc = synth.TINY
    assert t.kv_bytes == 2 * tc.n_layers * tc.max_batch * tc.n_kv_heads * tc.kv_capacity * tc.head_dim * 2


@pytest.mark.parametrize("field,value,code", [
    ("n_layers", 0, -1), ("attn_kind", 7, -1), ("top_k", 9, -1), ("max_batch", 9, -1),
    ("max_new_tokens", 0, -1), ("hidden", 100, -7), ("n_kv_heads", 3, -1), ("head_dim", 256, -7),
])
def test_bad_configs(mk, field, value, code):
    cfg = replace(synth.TINY, **{field: value})
    with pytest.raises(mk.MkError) as e:
        sizes(mk, cfg)
    assert e.value.code == code
    assert mk.mk_last_error()


@pytest.fixture
def host_ctx(mk):
    cfg = synth.TINY
    s = sizes(mk, cfg)
    ctx = mk.mk_create(mk.config(cfg), mk.MK_DEVICE_NONE, 0, s.arena_bytes, 0, s.workspace_bytes)
    yield cfg, ctx
    mk.mk_destroy(ctx)


def load_all(mk, cfg, ctx):
    descs = []
    for t in synth.tensor_list(cfg):
        nbytes = synth.numel(t.shape) * (4 if t.dist == "sigmoid" else 2)
        descs.append(mk.tensor_desc(t.kind, t.layer, t.expert, 1, nbytes, False))
    mk.mk_load_weights(ctx, descs)


@pytest.mark.parametrize("kw", [dict(top_k=1), dict(shared_ffn=0), dict(shared_ffn=12)])
def test_bad_dense_configs(mk, kw):
    # n_experts = 0 is a dense model: top_k 0 and a shared (dense) block of a multiple of 8
    base = dict(n_experts=0, top_k=0, ffn=0, shared_ffn=512)
    base.update(kw)
    with pytest.raises(mk.MkError) as e:
        sizes(mk, replace(synth.TINY, **base))
    assert e.value.code == mk.MK_E_INVAL


@pytest.mark.parametrize("head_dim", [8, 48, 160])
def test_gqa_head_dim_limits(mk, head_dim):
    # GQA attention runs on the matrix cores in 32-column steps, with at most 128 columns per head
    with pytest.raises(mk.MkError) as e:
        sizes(mk, replace(synth.TINY, head_dim=head_dim))
    assert e.value.code == mk.MK_E_UNSUPPORTED
    for ok in (32, 64, 96, 128):
        sizes(mk, replace(synth.TINY, head_dim=ok))


@pytest.mark.parametrize("n_heads,ok", [(16, True), (8, True), (12, True), (2, True), (7, False), (18, False),
                                         (32, False)])
def test_mla_head_counts(mk, n_heads, ok):
    # MLA attention puts the heads in the rows of one 16-row matrix-core tile: an even number of heads
    # up to 16 (a share of the same model over more tensor-parallel ranks has fewer heads)
    for base in (synth.K3, synth.K3_HYBRID):
        cfg = replace(base, n_heads=n_heads)
        if ok:
            sizes(mk, cfg)
        else:
            with pytest.raises(mk.MkError) as e:
                sizes(mk, cfg)
            assert e.value.code == mk.MK_E_UNSUPPORTED


def test_kv_capacity_limit(mk):
    # a step has at most one split-KV chunk per workgroup of the grid (256), so the merge's LDS and
    # the workspace do not grow with the capacity: up to 2^20 positions are admitted, and the
    # workspace of a 2^20-position context equals that of a 4104-position one
    for c in (synth.TINY, synth.K3, synth.DENSE):
        big = sizes(mk, replace(c, kv_capacity=mk.MK_MAX_KV_CAPACITY))
        assert big.kv_bytes == sizes(mk, c).kv_bytes * mk.MK_MAX_KV_CAPACITY // c.kv_capacity
        with pytest.raises(mk.MkError) as e:
            sizes(mk, replace(c, kv_capacity=mk.MK_MAX_KV_CAPACITY + 1))
        assert e.value.code == mk.MK_E_UNSUPPORTED
    assert (sizes(mk, replace(synth.K3, kv_capacity=mk.MK_MAX_KV_CAPACITY)).workspace_bytes
            == sizes(mk, replace(synth.K3, kv_capacity=4104)).workspace_bytes)


def test_dense_layout_and_loading(mk):
    """A dense model's arena holds exactly its tensors (no router, no expert pool); a step is
    refused until every one of them is loaded, and a router tensor is rejected."""
    for c in (synth.DENSE, replace(synth.TINY, n_experts=0, top_k=0, ffn=0, shared_ffn=512)):
        s = sizes(mk, c)
        tl = synth.tensor_list(c)
        assert not any(t.kind in ("router", "exp_gate", "exp_up", "exp_down") for t in tl)
        total = sum(synth.numel(t.shape) * 2 for t in tl)
        assert total <= s.arena_bytes <= total + 256 * (len(tl) + 1) + c.n_layers * 256
    assert sizes(mk, synth.DENSE).arena_bytes < 60e9
    cfg = replace(synth.TINY, n_experts=0, top_k=0, ffn=0, shared_ffn=512)
    s = sizes(mk, cfg)
    ctx = mk.mk_create(mk.config(cfg), mk.MK_DEVICE_NONE, 0, s.arena_bytes, 0, s.workspace_bytes)
    try:
        with pytest.raises(mk.MkError) as e:
            mk.mk_load_weights(ctx, [mk.tensor_desc("router", 0, -1, 1, cfg.hidden * 2, False)])
        assert e.value.code == mk.MK_E_INVAL
        load_all(mk, cfg, ctx)
        with pytest.raises(mk.MkError) as e:  # loaded, but a host-only context cannot launch
            mk.mk_decode_step(ctx, 1, 1, 3, 1, 1, 0, 1, 0, 0)
        assert e.value.code == mk.MK_E_STATE and "host-only" in mk.mk_last_error()
    finally:
        mk.mk_destroy(ctx)


def test_create_rejects_small_buffers(mk):
    cfg = synth.TINY
    s = sizes(mk, cfg)
    with pytest.raises(mk.MkError) as e:
        mk.mk_create(mk.config(cfg), mk.MK_DEVICE_NONE, 0, s.arena_bytes - 1, 0, s.workspace_bytes)
    assert e.value.code == mk.MK_E_NOMEM
    with pytest.raises(mk.MkError) as e:
        mk.mk_create(mk.config(cfg), mk.MK_DEVICE_NONE, 0, s.arena_bytes, 0, s.workspace_bytes - 1)
    assert e.value.code == mk.MK_E_NOMEM


def test_load_weights_validates_descriptors(mk, host_ctx):
    cfg, ctx = host_ctx
    H = cfg.hidden
    bad = [
        mk.tensor_desc("wq", 0, -1, 1, 3, False),  # wrong size
        mk.tensor_desc("wq", cfg.n_layers, -1, 1, H * H * 2, False),  # no such layer
        mk.tensor_desc("w_dq", 0, -1, 1, 1536 * H * 2, False),  # not in a GQA model
        mk.tensor_desc("exp_gate", 0, cfg.n_experts, 1, cfg.ffn * H * 2, False),  # no such expert
        mk.tensor_desc("wq", 0, -1, 0, H * H * 2, False),  # NULL source
    ]
    for d in bad:
        with pytest.raises(mk.MkError) as e:
            mk.mk_load_weights(ctx, [d])
        assert e.value.code == mk.MK_E_INVAL


def test_decode_step_argument_errors(mk, host_ctx):
    cfg, ctx = host_ctx
    ok = dict(batch=1, n_new_tokens=1, kv_len=10, tokens=1, kv=1, kda_state=0, logits=1)

    def step(**kw):
        a = dict(ok)
        a.update(kw)
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step(ctx, **a)
        return e.value.code

    assert step(batch=0) == mk.MK_E_INVAL
    assert step(batch=cfg.max_batch + 1) == mk.MK_E_INVAL
    assert step(n_new_tokens=0) == mk.MK_E_INVAL
    assert step(n_new_tokens=9) == mk.MK_E_INVAL
    assert step(batch=4, n_new_tokens=5) == mk.MK_E_UNSUPPORTED  # 20 rows > 16
    assert step(kv_len=-1) == mk.MK_E_INVAL
    assert step(kv_len=cfg.kv_capacity) == mk.MK_E_KV_OVERFLOW
    assert step(kv_len=cfg.kv_capacity - 2, n_new_tokens=3) == mk.MK_E_KV_OVERFLOW
    assert step(tokens=0) == mk.MK_E_INVAL
    assert step(logits=0) == mk.MK_E_INVAL
    # arguments valid, weights missing
    assert step() == mk.MK_E_STATE
    assert "weight tensors loaded" in mk.mk_last_error()
    load_all(mk, cfg, ctx)
    # all loaded; a host-only context never launches
    assert step() == mk.MK_E_STATE
    assert "host-only" in mk.mk_last_error()


def test_hybrid_needs_state(mk):
    cfg = replace(synth.K3_HYBRID, n_layers=4, expert_pool_layers=0)
    s = sizes(mk, cfg)
    ctx = mk.mk_create(mk.config(cfg), mk.MK_DEVICE_NONE, 0, s.arena_bytes, 0, s.workspace_bytes)
    try:
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step(ctx, 1, 1, 10, 1, 1, 0, 1)
        assert e.value.code == mk.MK_E_INVAL
    finally:
        mk.mk_destroy(ctx)


def test_null_context(mk):
    for fn, args in ((mk.lib.mk_poll, (None,)), (mk.lib.mk_load_weights, (None, None, 0, None))):
        assert fn(*args) == mk.MK_E_INVAL


def test_matrix_core_threshold_arguments(mk, host_ctx):
    _, ctx = host_ctx
    mk.mk_set_matrix_cores(ctx, 2)
    mk.mk_set_matrix_cores(ctx, mk.MK_MFMA_MIN_ROWS)
    mk.mk_set_matrix_cores(ctx, mk.MK_MAX_M + 1)  # vector units only
    for bad in (1, 0, -3):
        with pytest.raises(mk.MkError) as e:
            mk.mk_set_matrix_cores(ctx, bad)
        assert e.value.code == mk.MK_E_INVAL
    with pytest.raises(mk.MkError):
        mk.mk_set_matrix_cores(None, 5)


def test_greedy_step_argument_errors(mk, host_ctx):
    cfg, ctx = host_ctx
    ok = dict(batch=2, n_new_tokens=3, kv_len=10, tokens=1, kv=1, kda_state=0, logits=0, argmax=1, accepted=0)

    def step(**kw):
        a = dict(ok)
        a.update(kw)
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step_greedy(ctx, **a)
        return e.value.code

    assert step(argmax=0) == mk.MK_E_INVAL
    assert step(batch=0) == mk.MK_E_INVAL
    assert step(n_new_tokens=cfg.max_new_tokens + 1) == mk.MK_E_INVAL
    assert step(tokens=0) == mk.MK_E_INVAL
    assert step(kv=0) == mk.MK_E_INVAL
    assert step(kv_len=cfg.kv_capacity - 1) == mk.MK_E_KV_OVERFLOW
    # logits and accepted are optional: the arguments are valid, the weights are missing
    assert step() == mk.MK_E_STATE
    assert step(logits=1, accepted=1) == mk.MK_E_STATE
    with pytest.raises(mk.MkError) as e:
        mk.mk_decode_step_greedy(None, 1, 1, 0, 1, 1, 0, 0, 1)
    assert e.value.code == mk.MK_E_INVAL


def test_sample_step_argument_errors(mk, host_ctx):
    _, ctx = host_ctx
    ok = dict(batch=1, n_new_tokens=1, kv_len=10, tokens=1, kv=1, kda_state=0, logits=1, temperature=0.8, top_p=0.9,
              uniform=1, sampled=1)

    def step(**kw):
        a = dict(ok)
        a.update(kw)
        mk.mk_decode_step_sample(ctx, **a)

    for kw in (dict(temperature=0.0), dict(temperature=-1.0), dict(temperature=float("inf")),
               dict(temperature=float("nan")), dict(top_p=0.0), dict(top_p=1.5), dict(uniform=0), dict(sampled=0),
               dict(logits=0)):
        with pytest.raises(mk.MkError) as e:
            step(**kw)
        assert e.value.code == mk.MK_E_INVAL, kw
    with pytest.raises(mk.MkError) as e:  # valid arguments: the weights are not loaded yet
        step(top_p=1.0)
    assert e.value.code == mk.MK_E_STATE


PRESETS = {1: "c1", 2: "c2", 3: "c3", 4: "c4", 5: "c5", 6: "dense"}


@pytest.mark.parametrize("pid", sorted(PRESETS))
def test_presets_equal_the_workload_models(mk, pid):
    """mk_config_preset(id) describes the same model as the workload the tests and the benchmark
    build from synth (every field), and the library accepts it."""
    c = mk.mk_config_preset(pid)
    model = synth.WORKLOADS[PRESETS[pid]].model
    assert c.preset == pid
    for name, _ in mk.MkConfig._fields_:
        if name == "preset":
            continue
        got, want = getattr(c, name), getattr(model, name)
        if isinstance(want, float):
            assert got == pytest.approx(want, rel=1e-7), name
        else:
            assert got == want, name
    w = synth.WORKLOADS[PRESETS[pid]]
    assert c.kv_capacity == w.kv_len + 8
    s = mk.mk_query_sizes(c)
    assert s.arena_bytes == sizes(mk, model).arena_bytes


@pytest.mark.parametrize("pid", [0, 7, -1])
def test_unknown_preset(mk, pid):
    with pytest.raises(mk.MkError) as e:
        mk.mk_config_preset(pid)
    assert e.value.code == mk.MK_E_INVAL
    assert "preset" in mk.mk_last_error()


def test_preset_field_is_validated(mk):
    c = mk.config(synth.TINY)
    assert c.preset == 0
    mk.mk_query_sizes(c)
    c.preset = 9
    with pytest.raises(mk.MkError) as e:
        mk.mk_query_sizes(c)
    assert e.value.code == mk.MK_E_INVAL


def test_static_step_limits_on_host(mk):
    """mk_decode_step_static refuses, before any launch, a step whose workspace exceeds the static
    array (here 8 new tokens over 9000 positions of latent cache: split-KV partials of ~135 MB on a
    host-only context, which splits into 16-position chunks); a step that fits reaches the
    host-only check."""
    cfg = replace(synth.K3, n_layers=2, expert_pool_layers=0, kv_capacity=9008)
    s = sizes(mk, cfg)
    ctx = mk.mk_create(mk.config(cfg), mk.MK_DEVICE_NONE, 0, s.arena_bytes, 0, s.workspace_bytes)
    try:
        load_all(mk, cfg, ctx)
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step_static(ctx, 1, 8, 9000, 1, 1, 0, 1)
        assert e.value.code == mk.MK_E_UNSUPPORTED
        assert "static scratch" in mk.mk_last_error()
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step_static(ctx, 1, 1, 100, 1, 1, 0, 1)
        assert e.value.code == mk.MK_E_STATE
        with pytest.raises(mk.MkError) as e:
            mk.mk_decode_step_static(ctx, 1, 1, 9008, 1, 1, 0, 1)
        assert e.value.code == mk.MK_E_KV_OVERFLOW
    finally:
        mk.mk_destroy(ctx)


def test_stream_probe_exports_and_arguments():
    """libmkstream.so (the benchmark's read-bandwidth probe) exports what include/mk_stream.h declares,
    and refuses bad arguments before launching anything."""
    import ctypes

    text = open(os.path.join(ROOT, "include", "mk_stream.h")).read()
    declared = sorted(set(re.findall(r"^\s*int\s+(mk_\w+)\s*\(", text, re.M)))
    path = os.path.join(ROOT, "decode_megakernel_cu_amd", "libmkstream.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True)
    exported = sorted(l.split()[-1] for l in out.stdout.splitlines() if " T " in l and l.split()[-1].startswith("mk_"))
    assert declared == exported == ["mk_stream_read"]
    L = ctypes.CDLL(path)
    L.mk_stream_read.restype = ctypes.c_int
    L.mk_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    ok_ptr = 1 << 20  # 256-byte aligned; never dereferenced, every call below fails validation
    for args in [(None, 16384, 0, ok_ptr), (ok_ptr, 16384, 0, None), (ok_ptr + 16, 16384, 0, ok_ptr),
                 (ok_ptr, 0, 0, ok_ptr), (ok_ptr, 16385, 0, ok_ptr), (ok_ptr, 16384, 4, ok_ptr),
                 (ok_ptr, 16384, -1, ok_ptr), (ok_ptr, (1 << 40) + 16384, 0, ok_ptr)]:
        assert L.mk_stream_read(*args, None) == -1, args
