"""Benchmark: one-launch MoE decode step on the K3-scale one-GPU share (MI355X).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--batches 1,2,4,8] [--no-cpu-baseline]
                [--no-others] [--no-verify] [--no-read-probe] [--trace [--trace-out F]]
python bench.py --calib                      (one pass of the copy and read probes, for counters)
python bench.py --ingest-pmc FETCH.csv WRITE.csv   (turn two rocprofv3 --pmc runs into traffic)

Prints ONE JSON line. `value` is decode tokens/s at batch 1 (the headline configuration:
92 layers, hidden 7168, MLA with a 4096-long latent cache, 48 local experts top-1 plus a
shared expert, LM-head slice 7168 x 40960); the other batch sizes are under "batches", the
7-token verify step under "verify", the other workloads under "workloads". Inputs are
synthetic and seeded and already resident in HBM when the timed region starts. "roofline"
divides the step's algorithmic bytes (the weights the step must read given its routing, the
cache read and written, and the logits) by the megakernel's average duration, measured with
HIP events on the launch stream, against 8 TB/s; "read_probe" is the rate a plain streaming
read of 4 GiB reaches with each of the megakernel's load kinds on the same GPU, and
"roofline_measured_read" states the megakernel against the fastest of them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
WORKLOAD = "c3"


# ------------------------------------------------------------------------------------------
# algorithmic bytes of one step (what the step must move, given its routing)
# ------------------------------------------------------------------------------------------
def algorithmic_bytes(cfg: synth.ModelConfig, B: int, T: int, kv_len: int, route: np.ndarray) -> dict:
    """route: [n_layers][B*T][top_k] selected experts. Returns a byte breakdown."""
    H, V, M = cfg.hidden, cfg.vocab, B * T
    per_layer_fixed = {}
    for t in synth.tensor_list(cfg):
        if t.layer < 0 or t.kind.startswith("exp_"):
            continue
        nb = synth.numel(t.shape) * (4 if t.dist == "sigmoid" else 2)
        per_layer_fixed[t.layer] = per_layer_fixed.get(t.layer, 0) + nb
    expert_bytes = 3 * cfg.ffn * H * 2
    weights = sum(per_layer_fixed.values())
    experts = 0
    for l in range(cfg.n_layers):
        experts += len(np.unique(route[l])) * expert_bytes
    head = V * H * 2 + H * 2  # LM head + final norm
    embed = M * H * 2
    lat = cfg.latent_dim
    n_attn = len(cfg.attention_layers())
    if cfg.attn_kind == synth.ATTN_GQA:
        entry = 2 * cfg.n_kv_heads * cfg.head_dim * 2
    else:
        entry = lat * 2
    cache_read = n_attn * B * kv_len * entry
    cache_write = n_attn * M * entry
    state = 0
    if cfg.attn_kind == synth.ATTN_HYBRID:
        state = 2 * len(cfg.kda_layers()) * B * cfg.n_heads * cfg.kda_dk * cfg.kda_dv * 4
    logits = M * V * 4
    total = weights + experts + head + embed + cache_read + cache_write + state + logits
    return {"total": total, "weights": weights, "experts": experts, "lm_head": head, "embed": embed,
            "cache_read": cache_read, "cache_write": cache_write, "state": state, "logits": logits}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("mk_kernel.hip", "mk_api.cpp", "mk_internal.h"):
        with open(os.path.join(ROOT, "decode_megakernel_cu_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PMC_FILES = {"c3": "megakernel_k3_pmc_traffic.json", "dense": "megakernel_dense_pmc_traffic.json"}


def traffic_from_profiles(B: int, workload: str = WORKLOAD):
    """HBM bytes per launch from the committed PMC summary, if it was taken on this kernel."""
    path = os.path.join(ROOT, "profiles", PMC_FILES[workload])
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_hash") != kernel_source_hash():
        return None
    return d.get("per_launch_bytes", {}).get(str(B))


CALIB_BYTES = 1 << 30  # bytes the elementwise copy reads and writes (the WRITE_SIZE calibration)
STREAM_BYTES = 4 << 30  # bytes the read probe reads per load kind (the FETCH_SIZE calibration)
STREAM_KINDS = {0: "weights (16-byte non-temporal global loads)", 1: "activations (16-byte coherent buffer loads)",
                2: "staging (16-byte memory-to-LDS copies)"}


def stream_probe():
    """ctypes handle of libmkstream.so (include/mk_stream.h)."""
    import ctypes

    path = os.path.join(ROOT, "decode_megakernel_cu_amd", "libmkstream.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(path)
    L.mk_stream_read.restype = ctypes.c_int
    L.mk_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L


def measure_read_bandwidth(reps: int = 10) -> dict:
    """GB/s of one read pass over STREAM_BYTES with each of the megakernel's load kinds (median of
    reps passes, HIP events on the launch stream)."""
    import torch

    L = stream_probe()
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    out = {}
    for kind, what in STREAM_KINDS.items():
        ms = []
        for i in range(reps + 2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            rc = L.mk_stream_read(buf.data_ptr(), STREAM_BYTES, kind, sink.data_ptr(), st.cuda_stream)
            b.record(st)
            if rc != 0:
                raise RuntimeError(f"mk_stream_read failed: {rc}")
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(a.elapsed_time(b))
        t = float(np.median(ms))
        out[str(kind)] = {"what": what, "ms": round(t, 4), "gbs": round(STREAM_BYTES / (t * 1e-3) / 1e9, 1)}
        print(f"# read probe, {what}: {out[str(kind)]['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    del buf
    torch.cuda.empty_cache()
    return {"bytes": STREAM_BYTES, "kinds": out}


def ingest_pmc(fetch_csv: str, write_csv: str, workload: str = WORKLOAD) -> None:
    """HBM traffic of the megakernel from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch).
    FETCH_SIZE is scaled by what the counter reads for the read probe's pass over STREAM_BYTES with
    the weight-stream load kind (the megakernel's reads are almost all weight and cache rows read
    that way; the factors of the other two kinds are recorded beside it); WRITE_SIZE by what it reads
    for the elementwise copy of CALIB_BYTES. Written to profiles/ with the kernel's source hash."""
    import csv

    def per_kernel(path: str, counter: str) -> tuple[dict, float | None, list[float]]:
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        by = {}
        for r in rows:
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
        probe = {}
        for (d, n), v in by.items():
            for k in STREAM_KINDS:
                if f"stream_read<{k}>" in n:
                    probe.setdefault(k, []).append(v)
        # the calibration multiply (x * 1.0 -> y), not the fills torch runs around it
        copy = [v for (d, n), v in by.items() if "elementwise" in n and "Fill" not in n and
                ("AUnaryFunctor" in n or "Mul" in n)]
        mk = [v for (d, n), v in sorted(by.items(), key=lambda kv: int(kv[0][0])) if "mk_decode_kernel" in n]
        if not mk:
            raise SystemExit(f"{path}: no megakernel dispatches for {counter}")
        return ({k: float(np.median(v)) for k, v in probe.items()}, max(copy) if copy else None, mk)

    f_probe, _, f_mk = per_kernel(fetch_csv, "FETCH_SIZE")
    _, w_copy, w_mk = per_kernel(write_csv, "WRITE_SIZE")
    if 0 not in f_probe or w_copy is None:
        raise SystemExit("need the read probe's weight-kind dispatch (FETCH_SIZE) and the copy (WRITE_SIZE)")
    f_scale = {k: STREAM_BYTES / (v * 1024.0) for k, v in f_probe.items()}
    w_scale = CALIB_BYTES / (w_copy * 1024.0)
    fetch = float(np.median(f_mk)) * 1024.0 * f_scale[0]
    write = float(np.median(w_mk)) * 1024.0 * w_scale
    out = {"kernel_hash": kernel_source_hash(), "workload": workload, "batch": 1,
           "calibration": {"fetch": {"bytes": STREAM_BYTES, "probe_kib": {str(k): v for k, v in f_probe.items()},
                                     "scale_by_kind": {str(k): v for k, v in f_scale.items()}, "applied_kind": 0},
                           "write": {"bytes": CALIB_BYTES, "copy_kib": w_copy, "scale": w_scale}},
           "megakernel": {"dispatches": len(f_mk), "fetch_kib_median": float(np.median(f_mk)),
                          "write_kib_median": float(np.median(w_mk)), "fetch_bytes": fetch, "write_bytes": write},
           "per_launch_bytes": {"1": fetch + write}}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", PMC_FILES[workload]), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


# ------------------------------------------------------------------------------------------
# CPU baseline: the oracle on the host's cores, on a bounded sample of the same step
# ------------------------------------------------------------------------------------------
def cpu_baseline(sample_layers: int = 8, budget_s: float = 12.0) -> dict:
    from dataclasses import replace

    import oracle

    w = synth.WORKLOADS[WORKLOAD]
    cfg = replace(w.model, n_layers=sample_layers, expert_pool_layers=0)
    spec = synth.Spec(seed=0)
    toks = synth.tokens(spec.seed, 0, cfg.vocab, w.batch, w.new_tokens)
    caches0 = synth.host_caches(cfg, spec, w.batch, w.kv_len)
    # first run records the tensors the step reads, which are then served from memory so the
    # timed runs measure the oracle's arithmetic rather than the input generator
    rec = oracle.Provider(cfg, spec)
    oracle.decode_step(cfg, rec, toks, w.kv_len, {k: v.copy() for k, v in caches0.items()})
    mem = {}
    for t in synth.tensor_list(cfg):
        if any(name == t.name for name, _ in rec.fetched):
            mem[t.name] = synth.host_tensor(spec, t)
    prov = oracle.Provider(cfg, spec, overrides=mem)
    times = []
    t_start = time.perf_counter()
    while True:
        c = {k: v.copy() for k, v in caches0.items()}
        t0 = time.perf_counter()
        oracle.decode_step(cfg, prov, toks, w.kv_len, c)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    t = float(np.median(times))
    # extrapolate the per-layer part to 92 layers; the embedding and LM head are paid once
    head = oracle.Provider(replace(cfg, n_layers=0), spec, overrides=mem)
    c = {k: v.copy() for k, v in caches0.items()}
    t0 = time.perf_counter()
    oracle.decode_step(replace(cfg, n_layers=0), head, toks, w.kv_len, c)
    t_head = time.perf_counter() - t0
    per_layer = max(t - t_head, 0.0) / sample_layers
    step = t_head + per_layer * w.model.n_layers
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(w.batch * w.new_tokens / step, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{sample_layers} of {w.model.n_layers} layers of the batch-1 step (+ embedding and LM head), "
                      f"median of {len(times)} runs, weights served from host memory; per-layer time scaled to "
                      f"{w.model.n_layers} layers (step {step:.2f} s)"}


# ------------------------------------------------------------------------------------------
# per-phase timing from the device trace (mk_set_trace / mk_read_trace)
# ------------------------------------------------------------------------------------------
PHASES = {
    "gqa": ["qkv", "attention", "merge", "w_o"],
    "mla": ["q_a+kv_a", "q_b", "absorb", "attention", "merge", "w_uv", "w_o"],
    # 2-row steps merge the split-KV partials and apply W_uv in one phase
    "mla_mfused": ["q_a+kv_a", "q_b", "absorb", "attention", "merge+w_uv", "w_o"],
    "kda": ["qkv", "delta_rule", "w_o"],
}
MOE_PHASES = ["router+shared_up", "experts_up", "experts_down"]
# 1- and 2-row steps fold the router onto the attention output projection: two MoE phases
MOE_PHASES_FUSED = ["shared+experts_up", "experts_down"]
DENSE_PHASES = ["gate+up", "down"]  # n_experts = 0: the SwiGLU block alone


def phase_names(cfg, fused: bool = False, mfused: bool = False) -> list[str]:
    names = ["embed"]
    for l in range(cfg.n_layers):
        kind = cfg.layer_kind(l)
        attn = PHASES["mla_mfused" if kind == "mla" and mfused else kind]
        if cfg.n_experts:
            moe = MOE_PHASES_FUSED if fused else MOE_PHASES
            names += [f"{kind}:{p}" for p in attn] + [f"moe:{p}" for p in moe]
        else:
            names += [f"{kind}:{p}" for p in attn] + [f"ffn:{p}" for p in DENSE_PHASES]
    return names + ["lm_head"]


def trace_summary(cfg, tr: np.ndarray, tick_ns: float = 10.0) -> dict:
    """tr [n_barriers + 1][blocks][stamps] (stamp meanings in include/mk.h). The phase before barrier
    j runs from the last departure of barrier j-1 to the last arrival at barrier j; the barrier
    itself from the last arrival to the last departure. Segments inside a phase are medians over
    workgroups of the differences between its stamps (a stamp of 0 means the phase has no such
    mark)."""
    # steps with the router folded (one MoE phase fewer per layer) or the merge and W_uv fused (one
    # MLA phase fewer): the longest phase list the trace holds (greedy and sampling steps add a barrier)
    for fused, mfused in ((False, False), (True, False), (True, True), (False, True)):
        names = phase_names(cfg, fused, mfused)
        if len(names) <= tr.shape[0]:
            break
    t = tr.astype(np.int64)
    arr, dep = t[:, :, 0], t[:, :, 1]
    t0 = arr[0].min()
    out = {}
    prev_dep = t0
    us = tick_ns / 1e3

    def seg(j, a, b):  # median over the workgroups that have both stamps of stamp b - stamp a in record j
        ta = a if isinstance(a, np.ndarray) else t[j, :, a]
        tb = b if isinstance(b, np.ndarray) else t[j, :, b]
        ok = (ta > 0) & (tb > 0)
        if not ok.any():
            return 0.0
        return float(np.median((tb - ta)[ok])) * us

    for j, name in enumerate(names):
        a_max = arr[j].max()
        d_max = dep[j].max()
        s = out.setdefault(name, {"count": 0, "work_us": 0.0, "sync_us": 0.0, "enter_us": 0.0, "route_us": 0.0, "issue_us": 0.0,
                                  "stage_us": 0.0, "dot_us": 0.0, "epi_us": 0.0, "tail_us": 0.0, "drain_us": 0.0,
                                  "next_us": 0.0, "desc_us": 0.0, "plan_us": 0.0})
        s["count"] += 1
        s["work_us"] += (a_max - prev_dep) * us
        s["sync_us"] += (d_max - a_max) * us
        if 1 <= j < len(names) - 1:
            r = j - 1  # record of the barrier before this phase
            nxt = arr[j]
            s["enter_us"] += seg(r, 1, 7)
            if (t[r, :, 6] > 0).any():
                s["route_us"] += seg(r, 1, 6)
                s["issue_us"] += seg(r, 6, 4)
            elif not name.endswith("attention"):
                s["issue_us"] += seg(r, 1, 4)
            s["drain_us"] += seg(r, 5 if (t[r, :, 5] > 0).any() else 3, 8)  # stores of this phase
            s["next_us"] += seg(r, 0, 9)    # preparation while waiting (from arrival)
            s["desc_us"] += seg(r, 0, 10)
            s["plan_us"] += seg(r, 10, 11)
            if name.endswith("attention"):  # staged, scores, softmax (4, 5), values accumulated (3)
                s["stage_us"] += seg(r, 1, 2)
                s["dot_us"] += seg(r, 2, 3)
                s["issue_us"] += seg(r, 2, 4)  # scores
                s["epi_us"] += seg(r, 4, 5)    # softmax
                s["tail_us"] += seg(r, t[r, :, 3], nxt)
            elif (t[r, :, 4] > 0).any():
                s["stage_us"] += seg(r, 4, 2)
                s["dot_us"] += seg(r, 2, 3)
                s["epi_us"] += seg(r, 3, 5)
                s["tail_us"] += seg(r, t[r, :, 5], nxt)
        prev_dep = d_max
    total = (dep[-1].max() - t0) * us
    return {"total_us": total, "phases": out}


def print_trace(summary: dict) -> None:
    print(f"# traced step: {summary['total_us']:.1f} us", file=sys.stderr)
    cols = ["enter", "route", "issue", "stage", "dot", "epi", "tail", "drain", "next", "desc", "plan"]
    print(f"# {'phase':24s} {'n':>4s} {'work/n':>8s} {'sync/n':>8s} " + " ".join(f"{c:>7s}" for c in cols),
          file=sys.stderr)
    for name, s in sorted(summary["phases"].items(), key=lambda kv: -(kv[1]["work_us"] + kv[1]["sync_us"])):
        n = s["count"]
        print(f"# {name:24s} {n:4d} {s['work_us'] / n:8.2f} {s['sync_us'] / n:8.2f} " +
              " ".join(f"{s[c + '_us'] / n:7.2f}" for c in cols), file=sys.stderr)


# ------------------------------------------------------------------------------------------
# Speculative decoding around the verify step, with synthetic drafts: the target's own greedy
# continuation (T=1 greedy steps) supplies drafts that are accepted; mismatching drafts after the
# first L-1 make the step yield L tokens (L-1 accepted drafts and the bonus token).
# ------------------------------------------------------------------------------------------
def speculative(dm, cfg, spec, v, steps: int, warmup: int, stream) -> dict:
    import torch

    T, kv_len = v.new_tokens, v.kv_len
    tok = synth.tokens(spec.seed, 7, cfg.vocab, 1, 1)
    cont = [int(tok[0, 0])]
    for j in range(T - 1):  # greedy continuation, one token per step
        am, _ = dm.step_greedy(np.array([[cont[-1]]], dtype=np.int32), kv_len + j)
        torch.cuda.synchronize()
        cont.append(int(am.cpu().numpy()[0, 0]))
    dm.poll()
    out = {"new_tokens_per_step": T, "drafts": "the target's greedy continuation, then mismatching tokens",
           "lengths": {}}
    # plain greedy decode (one token, no logits written) for comparison
    one = np.array([[cont[0]]], dtype=np.int32)
    d_one = torch.from_numpy(one).cuda()
    am1 = torch.empty((1, 1), dtype=torch.int32, device="cuda")
    acc1 = torch.empty((1,), dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        dm.step_greedy(one, kv_len, d_tokens=d_one, argmax=am1, accepted=acc1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dm.step_greedy(one, kv_len, d_tokens=d_one, argmax=am1, accepted=acc1)
    torch.cuda.synchronize()
    ms1 = (time.perf_counter() - t0) * 1e3 / steps
    out["greedy_decode_b1"] = {"ms_per_step": round(ms1, 4), "tokens_per_s": round(1e3 / ms1, 2)}
    # temperature / top-p sampling fused after the LM head (the caller's uniform numbers on the device)
    d_u = torch.full((1, 1), 0.5, dtype=torch.float32, device="cuda")
    smp = torch.empty((1, 1), dtype=torch.int32, device="cuda")
    lg1 = torch.empty((1, 1, cfg.vocab), dtype=torch.float32, device="cuda")
    def sample_step():
        dm.mk.mk_decode_step_sample(dm.ctx, 1, 1, kv_len, d_one.data_ptr(), dm.kv.data_ptr(),
                                    dm.state.data_ptr() if dm.state is not None else 0, lg1.data_ptr(), 1.0, 0.9,
                                    d_u.data_ptr(), smp.data_ptr(), dm.stream)
    for _ in range(warmup):
        sample_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sample_step()
    torch.cuda.synchronize()
    mss = (time.perf_counter() - t0) * 1e3 / steps
    dm.poll()
    out["sampled_decode_b1"] = {"temperature": 1.0, "top_p": 0.9, "ms_per_step": round(mss, 4),
                                "tokens_per_s": round(1e3 / mss, 2)}
    print(f"# sampled decode B=1 (temperature 1, top-p 0.9): {mss:.3f} ms, {1e3 / mss:.1f} tok/s", file=sys.stderr,
          flush=True)
    for L in (3, 6):  # tokens yielded per step
        toks = np.array([cont[:L] + [(c + 1) % cfg.vocab for c in cont[L:T]]], dtype=np.int32)
        d_tok = torch.from_numpy(toks).cuda()
        am = torch.empty((1, T), dtype=torch.int32, device="cuda")
        acc = torch.empty((1,), dtype=torch.int32, device="cuda")
        for _ in range(warmup):
            dm.step_greedy(toks, kv_len, d_tokens=d_tok, argmax=am, accepted=acc)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            dm.step_greedy(toks, kv_len, d_tokens=d_tok, argmax=am, accepted=acc)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        dm.poll()
        yielded = int(acc.cpu().numpy()[0]) + 1
        out["lengths"][str(L)] = {"accepted_drafts": yielded - 1, "tokens_per_step": yielded,
                                  "ms_per_step": round(ms, 4), "accepted_tokens_per_s": round(yielded * 1e3 / ms, 2)}
        print(f"# speculative T={T} length {L}: {yielded} tokens/step, {ms:.3f} ms, "
              f"{yielded * 1e3 / ms:.1f} accepted tok/s", file=sys.stderr, flush=True)
    print(f"# greedy decode B=1: {ms1:.3f} ms, {1e3 / ms1:.1f} tok/s", file=sys.stderr, flush=True)
    return out


# ------------------------------------------------------------------------------------------
# the measured rows: the headline share at batch 1/2/4/8, its verify step, the other workloads
# ------------------------------------------------------------------------------------------
OTHER_ROWS = [("c1", [1]), ("c2", [1, 4]), ("c5", [8]), ("dense", [1, 2, 4, 8])]


def row_of(r: dict, read_gbs: float | None) -> dict:
    out = {"tokens_per_s": round(r["tokens_per_s"], 2), "kernel_ms": round(r["kernel_ms_avg"], 4),
           "kernel_ms_p10": round(r["kernel_ms_p10"], 4), "kernel_ms_p90": round(r["kernel_ms_p90"], 4),
           "gb_per_step": round(r["bytes"] / 1e9, 4), "hbm_gbs": round(r["gbs"], 1),
           "hbm_frac": round(r["gbs"] / HBM_PEAK_GBS, 4)}
    if read_gbs:
        out["read_probe_frac"] = round(r["gbs"] / read_gbs, 4)
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batches", default="1,2,4,8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--trace", action="store_true", help="print per-phase device timings of one step per batch")
    ap.add_argument("--trace-out", default=None, help="with --trace: write the per-phase summary (JSON) here")
    ap.add_argument("--workload", default=WORKLOAD, choices=["c1", "c2", "c3", "c4", "c5", "dense"],
                    help="c3: the K3-scale share (the headline, followed by every other row); any other: that "
                         "workload alone (for profiling one path; --batches applies)")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the 7-token speculative-verify measurement on the K3-scale share")
    ap.add_argument("--no-others", "--no-dense", dest="no_others", action="store_true",
                    help="skip the rows after the K3-scale share (tiny, mid-size, hybrid, dense)")
    ap.add_argument("--no-read-probe", action="store_true", help="skip the read-bandwidth probe")
    ap.add_argument("--mfma-min-rows", type=int, default=None,
                    help="token rows from which GEMV phases use the matrix cores (library default if omitted)")
    ap.add_argument("--calib", action="store_true",
                    help="first run the counter calibration kernels: one elementwise copy of CALIB_BYTES (fp32 "
                         "x*1 -> y) and one read-probe pass of STREAM_BYTES per load kind")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection CSVs (FETCH_SIZE, WRITE_SIZE) of a --calib run "
                         "into profiles/megakernel_{k3,dense}_pmc_traffic.json (by --workload) and exit")
    args = ap.parse_args()
    if args.trace and not os.environ.get("MK_LIBRARY"):  # the build with the stamp code compiled in
        os.environ["MK_LIBRARY"] = os.path.join(ROOT, "decode_megakernel_cu_amd", "libmk_trace.so")
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc, workload="dense" if args.workload == "dense" else "c3")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the decode step; --gpus {args.gpus} is not supported "
              f"(it measures exactly one GPU, with no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch

    from synth.device_inputs import DeviceModel

    spec = synth.Spec(seed=args.seed)
    stream = torch.cuda.current_stream()
    if args.calib:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        L = stream_probe()
        buf = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device="cuda")
        sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
        for kind in STREAM_KINDS:
            assert L.mk_stream_read(buf.data_ptr(), STREAM_BYTES, kind, sink.data_ptr(), stream.cuda_stream) == 0
            torch.cuda.synchronize()
        del buf
        torch.cuda.empty_cache()
    read = None if args.no_read_probe else measure_read_bandwidth()
    read_gbs = read["kinds"]["0"]["gbs"] if read else None

    def measure(dm, cfg, w, B: int, T: int, trace: bool) -> dict:
        toks = synth.tokens(spec.seed, 1, cfg.vocab, B, T)
        d_tok = torch.from_numpy(toks.astype(np.int32)).cuda()
        logits = torch.empty((B, T, cfg.vocab), dtype=torch.float32, device="cuda")
        _, route = dm.step(toks, w.kv_len, route=True, logits=logits, d_tokens=d_tok)
        torch.cuda.synchronize()
        dm.poll()
        route = route.cpu().numpy()
        for _ in range(args.warmup):
            dm.step(toks, w.kv_len, route=False, logits=logits, d_tokens=d_tok)
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        for i in range(args.steps):
            starts[i].record(stream)
            dm.step(toks, w.kv_len, route=False, logits=logits, d_tokens=d_tok)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        dm.poll()
        kms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
        by = algorithmic_bytes(cfg, B, T, w.kv_len, route)
        r = {"ms_per_step": wall * 1e3 / args.steps, "kernel_ms_avg": float(kms.mean()),
             "kernel_ms_p10": float(np.percentile(kms, 10)), "kernel_ms_p90": float(np.percentile(kms, 90)),
             "tokens_per_s": B * T * args.steps / wall, "bytes": by["total"],
             "gbs": by["total"] / (kms.mean() * 1e-3) / 1e9}
        print(f"# {w.name} B={B} T={T}: {r['kernel_ms_avg']:.3f} ms/launch (p10 {r['kernel_ms_p10']:.3f}, p90 "
              f"{r['kernel_ms_p90']:.3f}), {r['tokens_per_s']:.1f} tok/s, {r['gbs']:.0f} GB/s "
              f"({by['total'] / 1e9:.3f} GB/step)", file=sys.stderr, flush=True)
        if trace:
            dm.mk.mk_set_trace(dm.ctx, True)
            dm.step(toks, w.kv_len, route=False, logits=logits, d_tokens=d_tok)
            torch.cuda.synchronize()
            summary = trace_summary(cfg, dm.mk.mk_read_trace(dm.ctx))
            dm.mk.mk_set_trace(dm.ctx, False)
            print(f"# trace {w.name} B={B} T={T}", file=sys.stderr)
            print_trace(summary)
            r["trace"] = summary
        return r

    def load(wname: str, batches: list[int]):
        w = synth.WORKLOADS[wname]
        t0 = time.time()
        dm = DeviceModel(w.model, spec, device=0)
        if args.mfma_min_rows is not None:
            dm.set_matrix_cores(args.mfma_min_rows)
        dm.fill_caches(max(batches), w.kv_len)
        print(f"# {w.name} model loaded in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
        return w, dm

    batches = [int(b) for b in args.batches.split(",")]
    w, dm = load(args.workload, batches)
    cfg = w.model
    results = {B: measure(dm, cfg, w, B, w.new_tokens, args.trace) for B in batches}
    if args.trace and args.trace_out:
        with open(args.trace_out, "w") as fh:
            json.dump({str(B): r["trace"] for B, r in results.items()}, fh, indent=1)
    verify = spec_dec = None
    if args.workload == "c3" and not args.no_verify:
        v = synth.WORKLOADS["c4"]
        verify = measure(dm, cfg, v, v.batch, v.new_tokens, False)
        spec_dec = speculative(dm, cfg, spec, v, args.steps, args.warmup, stream)
    dm.close()
    del dm  # the K3-scale arena (193 GB) must be freed before the next model is loaded
    import gc

    gc.collect()
    torch.cuda.empty_cache()
    others = {}
    if args.workload == "c3" and not args.no_others:  # each model loaded after the previous one is freed
        for wname, bs in OTHER_ROWS:
            wo, dmo = load(wname, bs)
            others[wname] = (wo, {B: measure(dmo, wo.model, wo, B, wo.new_tokens, False) for B in bs})
            dmo.close()
            del dmo
            gc.collect()
            torch.cuda.empty_cache()

    head = results[batches[0]]
    achieved = head["gbs"]
    out = {
        "metric": "decode tokens/s at batch 1/2/4/8 + achieved HBM GB/s as % of peak",
        "value": round(head["tokens_per_s"], 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,0.02) weights, N(0,1) latent cache, uniform tokens)",
        "config": {"workload": "k3-share decode step: 92 layers, hidden 7168, MLA 16 heads (q_lora 1536, kv_lora 512, "
                               "rope 64), latent cache 4096, 48 experts top-1 ffn 2048 + shared 512, vocab slice "
                               "40960", "batch": batches[0], "new_tokens": w.new_tokens, "kv_len": w.kv_len,
                   "launches_per_step": 1},
        "batches": {str(B): row_of(r, read_gbs) for B, r in results.items()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(batches[0])},
    }
    if read is not None:
        out["read_probe"] = read
        out["roofline_measured_read"] = {"achieved": round(achieved, 1), "read_gbs": read_gbs,
                                         "frac": round(achieved / read_gbs, 4)}
    if spec_dec is not None:
        out["speculative"] = spec_dec
    if verify is not None:  # positions verified per second (1 + 6 draft tokens per step)
        vr = row_of(verify, read_gbs)
        vr["positions_per_s"] = vr.pop("tokens_per_s")
        out["verify_t7"] = vr
    if others:
        out["workloads"] = {}
        for wname, (wo, rs) in others.items():
            entry = {"description": wo.description, "kv_len": wo.kv_len,
                     "batches": {str(B): row_of(r, read_gbs) for B, r in rs.items()}}
            if wname == "c1":  # 14.7 MB of weights: resident in the 256 MB last-level cache, latency only
                entry["note"] = "weights fit the last-level cache; tokens/s and latency only, HBM fraction not meaningful"
            out["workloads"][wname] = entry
        if "dense" in others:
            d0 = others["dense"][1][1]
            out["workloads"]["dense"]["roofline"] = {"bound": "hbm", "achieved": round(d0["gbs"], 1),
                                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                     "frac": round(d0["gbs"] / HBM_PEAK_GBS, 4),
                                                     "traffic": traffic_from_profiles(1, "dense")}
    if args.workload != "c3":
        out["config"]["workload"] = f"{args.workload}: {w.description} (profiling run, not the headline)"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
