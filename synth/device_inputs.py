"""Synthetic inputs placed in device memory for the megakernel library.

Generates every weight tensor of a model with the device generator (large
matrices) or the host generator (gains, delta-rule parameters), hands them to
``mk_load_weights``, and fills the KV cache / recurrent state in the layouts
documented in ``include/mk.h``. Values equal those the oracle receives from
``synth.host_tensor`` / ``synth.host_caches`` bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import synth


def _dev_alloc(nbytes: int, device) -> torch.Tensor:
    # 256-byte aligned device buffer (the caching allocator aligns to at least 512 bytes)
    t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


class DeviceModel:
    """Arena, workspace, cache and state of one model on one GPU, filled from `spec`."""

    def __init__(self, cfg: synth.ModelConfig, spec: synth.Spec, device: int = 0, load: bool = True,
                 workspace: bool = True):
        """workspace=False: a context without a workspace, which steps only through
        mk_decode_step_static."""
        import decode_megakernel_cu_amd as mk

        self.mk = mk
        self.cfg, self.spec, self.device = cfg, spec, torch.device("cuda", device)
        self.mcfg = mk.config(cfg)
        self.sizes = mk.mk_query_sizes(self.mcfg)
        s = self.sizes
        self.arena = _dev_alloc(s.arena_bytes, self.device)
        self.ws = _dev_alloc(s.workspace_bytes, self.device) if workspace else None
        self.kv = torch.zeros(max(s.kv_bytes // 2, 128), dtype=torch.int16, device=self.device)
        self.state = (torch.zeros(s.kda_state_bytes // 4, dtype=torch.float32, device=self.device)
                      if s.kda_state_bytes else None)
        self.ctx = mk.mk_create(self.mcfg, device, self.arena.data_ptr(), s.arena_bytes,
                                self.ws.data_ptr() if workspace else 0, s.workspace_bytes if workspace else 0)
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        if load:
            self.load_weights()

    def close(self):
        if getattr(self, "ctx", None) is not None:
            self.mk.mk_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ weights
    def load_weights(self, overrides: dict | None = None):
        overrides = overrides or {}
        tl = synth.tensor_list(self.cfg)
        biggest = max(synth.numel(t.shape) for t in tl if t.dist == "normal")
        tmp = torch.empty(biggest, dtype=torch.int16, device=self.device)
        hold = []
        for t in tl:
            n = synth.numel(t.shape)
            if t.name in overrides:
                arr = np.ascontiguousarray(overrides[t.name]).reshape(-1)
                dt = torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr).to(self.device)
                hold.append(dt)
                desc = self.mk.tensor_desc(t.kind, t.layer, t.expert, dt.data_ptr(), dt.numel() * dt.element_size(),
                                           True)
            elif t.dist == "normal":
                synth.dev_normal_bf16(self.spec.seed, t.name, self.spec.sigma_for(t.kind), 0, n, tmp.data_ptr(),
                                      self.stream)
                desc = self.mk.tensor_desc(t.kind, t.layer, t.expert, tmp.data_ptr(), n * 2, True)
            else:
                arr = synth.host_tensor(self.spec, t)
                dt = torch.from_numpy(arr.view(np.int16) if arr.dtype == np.uint16 else arr).to(self.device)
                hold.append(dt)
                desc = self.mk.tensor_desc(t.kind, t.layer, t.expert, dt.data_ptr(), dt.numel() * dt.element_size(),
                                           True)
            # stream order keeps `tmp` valid until its copy has run
            self.mk.mk_load_weights(self.ctx, [desc], self.stream)
        torch.cuda.synchronize(self.device)
        del hold, tmp

    # ------------------------------------------------------------------ caches
    def fill_caches(self, batch: int, kv_len: int):
        """Positions < kv_len of sequences < batch from the generator; everything else zero."""
        cfg, sp, st = self.cfg, self.spec, self.stream
        self.kv.zero_()
        Bm, cap = cfg.max_batch, cfg.kv_capacity
        base = self.kv.data_ptr()
        if cfg.attn_kind == synth.ATTN_GQA:
            nkv, d = cfg.n_kv_heads, cfg.head_dim
            for w, which in enumerate(("K", "V")):
                for l in range(cfg.n_layers):
                    for b in range(batch):
                        for g in range(nkv):
                            off = ((((w * cfg.n_layers + l) * Bm + b) * nkv + g) * cap) * d
                            synth.dev_normal_bf16(sp.seed, synth.gqa_cache_stream(which, l, b), sp.cache_sigma,
                                                  g * synth.GQA_POS_STRIDE * d, kv_len * d, base + off * 2, st)
        else:
            lat = cfg.latent_dim
            for o, l in enumerate(cfg.attention_layers()):
                for b in range(batch):
                    off = ((o * Bm + b) * cap) * lat
                    synth.dev_normal_bf16(sp.seed, synth.latent_cache_stream(l, b), sp.cache_sigma, 0, kv_len * lat,
                                          base + off * 2, st)
            if self.state is not None:
                self.state.zero_()
                nh, dk, dv = cfg.n_heads, cfg.kda_dk, cfg.kda_dv
                sb = self.state.data_ptr()
                for o, l in enumerate(cfg.kda_layers()):
                    for b in range(batch):
                        off = ((o * Bm + b) * nh) * dk * dv
                        synth.dev_normal_f32(sp.seed, synth.kda_state_stream(l, b), sp.state_sigma, 0, nh * dk * dv,
                                             sb + off * 4, st)
        torch.cuda.synchronize(self.device)

    # ------------------------------------------------------------------ steps
    def step(self, tokens: np.ndarray, kv_len: int, route: bool = True, logits: torch.Tensor | None = None,
             d_tokens: torch.Tensor | None = None):
        B, T = tokens.shape
        cfg = self.cfg
        if d_tokens is None:
            d_tokens = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to(self.device)
        if logits is None:
            logits = torch.empty((B, T, cfg.vocab), dtype=torch.float32, device=self.device)
        rt = torch.full((cfg.n_layers, B * T, cfg.top_k), -1, dtype=torch.int32, device=self.device) if route else None
        self.mk.mk_decode_step(self.ctx, B, T, kv_len, d_tokens.data_ptr(), self.kv.data_ptr(),
                               self.state.data_ptr() if self.state is not None else 0, logits.data_ptr(),
                               rt.data_ptr() if rt is not None else 0, self.stream)
        return logits, rt

    def step_static(self, tokens: np.ndarray, kv_len: int, route: bool = True, logits: torch.Tensor | None = None,
                    d_tokens: torch.Tensor | None = None):
        """mk_decode_step on the library's static per-GPU workspace."""
        B, T = tokens.shape
        cfg = self.cfg
        if d_tokens is None:
            d_tokens = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to(self.device)
        if logits is None:
            logits = torch.empty((B, T, cfg.vocab), dtype=torch.float32, device=self.device)
        rt = torch.full((cfg.n_layers, B * T, cfg.top_k), -1, dtype=torch.int32, device=self.device) if route else None
        self.mk.mk_decode_step_static(self.ctx, B, T, kv_len, d_tokens.data_ptr(), self.kv.data_ptr(),
                                      self.state.data_ptr() if self.state is not None else 0, logits.data_ptr(),
                                      rt.data_ptr() if rt is not None else 0, self.stream)
        self._keep_tok = d_tokens
        return logits, rt

    def step_greedy(self, tokens: np.ndarray, kv_len: int, logits: torch.Tensor | None = None,
                    d_tokens: torch.Tensor | None = None, argmax: torch.Tensor | None = None,
                    accepted: torch.Tensor | None = None):
        """A greedy step: returns (argmax [B][T] int32, accepted [B] int32); logits are written only if given."""
        B, T = tokens.shape
        if d_tokens is None:
            d_tokens = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to(self.device)
        if argmax is None:
            argmax = torch.full((B, T), -1, dtype=torch.int32, device=self.device)
        if accepted is None:
            accepted = torch.full((B,), -1, dtype=torch.int32, device=self.device)
        self.mk.mk_decode_step_greedy(self.ctx, B, T, kv_len, d_tokens.data_ptr(), self.kv.data_ptr(),
                                      self.state.data_ptr() if self.state is not None else 0,
                                      logits.data_ptr() if logits is not None else 0, argmax.data_ptr(),
                                      accepted.data_ptr(), self.stream)
        return argmax, accepted

    def step_sample(self, tokens: np.ndarray, kv_len: int, temperature: float, top_p: float, uniform: np.ndarray,
                    logits: torch.Tensor | None = None, d_tokens: torch.Tensor | None = None):
        """A sampling step: returns (sampled [B][T] int32, logits [B][T][V] fp32)."""
        B, T = tokens.shape
        if d_tokens is None:
            d_tokens = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).to(self.device)
        if logits is None:
            logits = torch.empty((B, T, self.cfg.vocab), dtype=torch.float32, device=self.device)
        d_u = torch.from_numpy(np.ascontiguousarray(uniform, dtype=np.float32).reshape(B, T)).to(self.device)
        sampled = torch.full((B, T), -1, dtype=torch.int32, device=self.device)
        self.mk.mk_decode_step_sample(self.ctx, B, T, kv_len, d_tokens.data_ptr(), self.kv.data_ptr(),
                                      self.state.data_ptr() if self.state is not None else 0, logits.data_ptr(),
                                      temperature, top_p, d_u.data_ptr(), sampled.data_ptr(), self.stream)
        self._keep = d_u  # alive until the caller synchronises
        return sampled, logits

    def set_matrix_cores(self, min_rows: int):
        """Steps with at least min_rows token rows run their GEMV phases on the matrix cores."""
        self.mk.mk_set_matrix_cores(self.ctx, min_rows)

    def poll(self):
        self.mk.mk_poll(self.ctx)

    # ------------------------------------------------------------------ views for comparisons
    def latent_cache(self) -> np.ndarray:
        cfg = self.cfg
        n = len(cfg.attention_layers())
        return self.kv[: n * cfg.max_batch * cfg.kv_capacity * cfg.latent_dim].view(
            n, cfg.max_batch, cfg.kv_capacity, cfg.latent_dim).cpu().numpy().view(np.uint16)

    def gqa_cache(self) -> tuple[np.ndarray, np.ndarray]:
        cfg = self.cfg
        shape = (2, cfg.n_layers, cfg.max_batch, cfg.n_kv_heads, cfg.kv_capacity, cfg.head_dim)
        a = self.kv[: int(np.prod(shape))].view(*shape).cpu().numpy().view(np.uint16)
        return a[0], a[1]

    def kda_state(self) -> np.ndarray:
        cfg = self.cfg
        return self.state.view(len(cfg.kda_layers()), cfg.max_batch, cfg.n_heads, cfg.kda_dk,
                               cfg.kda_dv).cpu().numpy()
