"""Host-side pieces of the benchmark (no GPU): the bench line's refusal of several GPUs, and the byte
model its roofline divides by, checked against the K3-scale share's sizes written out by hand."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    # one GPU's share of the step, no collectives: --gpus 2 exits with a message, before any GPU work
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_k3_share_bytes_at_batch1_by_hand():
    # 92 layers, hidden 7168, MLA (q_lora 1536, kv_lora 512, rope 64, nope 128, v 128, 16 heads),
    # 48 experts of ffn 2048 with top-1 routing (one expert per layer at batch 1), a shared expert of
    # ffn 512, vocab slice 40960, a 4096-long latent cache; bf16 weights and cache, fp32 logits
    L, H, V, kv = 92, 7168, 40960, 4096
    mla = (1536 * H + 1536 + 16 * 192 * 1536 + 576 * H + 512 + 2 * 16 * 128 * 512 + H * 2048)
    moe = 48 * H + 3 * 512 * H
    norms = 2 * H
    per_layer = 2 * (mla + moe + norms)
    expert = 2 * 3 * 2048 * H
    head = 2 * (V * H + H)
    embed = 2 * H
    cache = L * kv * 576 * 2 + L * 576 * 2
    logits = V * 4
    total = L * (per_layer + expert) + head + embed + cache + logits
    cfg = synth.WORKLOADS["c3"].model
    route = np.zeros((cfg.n_layers, 1, 1), dtype=np.int64)  # every layer routes its token to expert 0
    got = bench.algorithmic_bytes(cfg, 1, 1, kv, route)
    assert got["total"] == total
    assert abs(total / 1e9 - 17.958) < 5e-4
    # a second token routed to another expert adds one expert's rows per layer and its cache, logits
    route2 = np.zeros((cfg.n_layers, 2, 1), dtype=np.int64)
    route2[:, 1, 0] = 1
    got2 = bench.algorithmic_bytes(cfg, 2, 1, kv, route2)
    assert got2["experts"] == 2 * got["experts"]
    assert got2["cache_read"] == 2 * got["cache_read"] and got2["logits"] == 2 * got["logits"]
    # the same expert chosen twice is read once
    got_same = bench.algorithmic_bytes(cfg, 2, 1, kv, np.zeros((cfg.n_layers, 2, 1), dtype=np.int64))
    assert got_same["experts"] == got["experts"]
