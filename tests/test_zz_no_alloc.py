"""The allocation-free step (mk_decode_step_static) against mk_decode_step, through the C ABI.

mk_decode_step_static runs the same kernels as mk_decode_step on the same split of the work; only
the workspace differs (the library's static per-GPU array instead of the context's). Two calls in
a row on each model, the second with a smaller input (fewer rows, a shorter cache): the logits,
the routes, the appended cache rows and the delta-rule state must equal mk_decode_step's on the
same inputs bit for bit -- stricter than the 2e-2 logit bar against the oracle, which
mk_decode_step meets in the parity tests. A context created without a workspace steps through the
static entry point only.
"""
import gc
from dataclasses import replace

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

K3_SMALL = replace(synth.K3, name="k3-2layer", n_layers=2, expert_pool_layers=0)
HYB_SMALL = replace(synth.K3_HYBRID, name="hybrid-4layer", n_layers=4, expert_pool_layers=0)

# (model, [(batch, new tokens, kv_len), ...]): the second call of each pair is smaller
CASES = [
    (K3_SMALL, [(4, 2, 3000), (1, 1, 700)]),
    (synth.TINY, [(8, 2, 100), (2, 1, 20)]),
    (HYB_SMALL, [(8, 1, 517), (2, 1, 100)]),
]


def free_gpu():
    gc.collect()
    torch.cuda.empty_cache()


def equal_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@pytest.mark.parametrize("cfg,calls", CASES, ids=[c[0].name for c in CASES])
def test_static_step_equals_workspace_step(cfg, calls):
    from synth.device_inputs import DeviceModel

    free_gpu()
    spec = synth.Spec(seed=27)
    dm = DeviceModel(cfg, spec, device=0)
    try:
        for i, (B, T, kv_len) in enumerate(calls):
            print(f"[case] static step {cfg.name} call {i}: B={B} T={T} kv_len={kv_len}", flush=True)
            dm.set_matrix_cores(3)
            dm.fill_caches(B, kv_len)
            kv0 = dm.kv.clone()
            st0 = dm.state.clone() if dm.state is not None else None
            toks = synth.tokens(spec.seed, 10 + i, cfg.vocab, B, T)
            la, ra = dm.step(toks, kv_len)
            torch.cuda.synchronize()
            dm.poll()
            kva = dm.kv.clone()
            sta = dm.state.clone() if st0 is not None else None
            dm.kv.copy_(kv0)
            if st0 is not None:
                dm.state.copy_(st0)
            lb, rb = dm.step_static(toks, kv_len)
            torch.cuda.synchronize()
            dm.poll()
            assert equal_bits(la, lb), f"logits differ (max |d| {(la - lb).abs().max().item():.3e})"
            assert torch.equal(ra, rb), "routes differ"
            assert torch.equal(dm.kv, kva), "appended cache rows differ"
            if st0 is not None:
                assert equal_bits(dm.state, sta), "delta-rule state differs"
            print(f"[ok] static step {cfg.name} call {i}: bitwise equal to mk_decode_step", flush=True)
    finally:
        dm.close()


def test_context_without_workspace():
    import decode_megakernel_cu_amd as mk
    from synth.device_inputs import DeviceModel

    free_gpu()
    cfg, spec = synth.TINY, synth.Spec(seed=28)
    print("[case] context without a workspace", flush=True)
    ref = DeviceModel(cfg, spec, device=0)
    bare = DeviceModel(cfg, spec, device=0, workspace=False)
    try:
        for i, (B, T, kv_len) in enumerate([(4, 3, 60), (1, 1, 10)]):
            toks = synth.tokens(spec.seed, 20 + i, cfg.vocab, B, T)
            ref.fill_caches(B, kv_len)
            bare.fill_caches(B, kv_len)
            la, ra = ref.step(toks, kv_len)
            torch.cuda.synchronize()
            ref.poll()
            with pytest.raises(mk.MkError) as e:
                bare.step(toks, kv_len)
            assert e.value.code == mk.MK_E_STATE
            lb, rb = bare.step_static(toks, kv_len)
            torch.cuda.synchronize()
            bare.poll()
            assert equal_bits(la, lb) and torch.equal(ra, rb)
            assert torch.equal(ref.kv, bare.kv)
        print("[ok] context without a workspace: static steps equal the workspace steps", flush=True)
    finally:
        ref.close()
        bare.close()
