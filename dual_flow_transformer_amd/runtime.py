"""Device-side state of one decode workload and thin calls into the C ABI.

PyTorch is used for device memory and the current stream only; every step of
the decode path runs in the HIP kernels of libdualflow.so. Inputs are the
seeded synthetic tensors of ``synth.workloads`` (filled on the device by the
generator's HIP twin, or drawn on the host and copied, bit-identical).
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from synth import stream_id
from synth import device as synth_dev
from synth.workloads import Config, Inputs
from . import _abi


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


class DecodeModel:
    """Weights, K/V cache, workspace and outputs of one workload on a GPU.

    bf16 projection matrices are generated row-major and then repacked on the
    device into the fragment layout the library reads (df_pack_weights)."""

    def __init__(self, cfg: Config, device: str = "cuda", fill: str = "device", src: Optional[Inputs] = None,
                 max_seq: Optional[int] = None, prefill_rows: int = 0):
        self.cfg = cfg
        self.dev = torch.device(device)
        self.src = src or Inputs(cfg)
        c = cfg
        self.bf16 = c.dtype == "bf16"
        self.wdt = torch.int16 if self.bf16 else torch.float32
        self.S = max_seq or c.S_max
        moe = c.moe
        ffn = c.ffn
        z = lambda *shape, dt=None: torch.zeros(*shape, dtype=dt or self.wdt, device=self.dev)
        self.tok_emb = [z(c.V, c.d), z(c.V, c.d)]
        self.pos_emb = z(self.S, c.d)
        self.ln1 = torch.zeros(c.L, c.d, dtype=torch.float32, device=self.dev)
        self.ln2 = torch.zeros(c.L, c.d, dtype=torch.float32, device=self.dev)
        self.lnf = torch.zeros(c.d, dtype=torch.float32, device=self.dev)
        self.w_qkv = z(c.L, 3 * c.d, c.d)
        self.w_o = z(c.L, c.d, c.d)
        if moe:
            self.w_router = z(c.L, c.E, c.d)
            self.w_eup = z(c.L, c.E, c.Fe, c.d)
            self.w_edown = z(c.L, c.E, c.d, c.Fe)
            self.w_up = self.w_down = None
        else:
            self.w_up = z(c.L, c.F, c.d)
            self.w_down = z(c.L, c.d, c.F)
            self.w_router = self.w_eup = self.w_edown = None
        self.cpl_a = torch.zeros(c.L, c.d, dtype=torch.float32, device=self.dev)
        self.cpl_b = torch.zeros(c.L, ffn, dtype=torch.float32, device=self.dev)
        self.cpl_c = torch.zeros(c.L, c.d, dtype=torch.float32, device=self.dev)
        self.w_out = z(c.V, c.d)
        self.k = z(c.L, c.B, c.H, self.S, c.Dh)
        self.v = z(c.L, c.B, c.H, self.S, c.Dh)
        self.len = torch.full((c.B,), c.ctx, dtype=torch.int32, device=self.dev)
        self._fill(fill)

        self.config = _abi.df_config(c.L, c.d, c.H, c.Dh, 0 if moe else c.F, c.V, c.E if moe else 0,
                                     c.top_k if moe else 0, c.Fe if moe else 0, c.B, self.S,
                                     _abi.DF_BF16 if self.bf16 else _abi.DF_F32, c.eps, c.variant,
                                     c.top_k_aux if moe else 0, prefill_rows)
        w = _abi.df_weights()
        w.tok_emb[0] = self.tok_emb[0].data_ptr()
        w.tok_emb[1] = self.tok_emb[1].data_ptr()
        w.pos_emb = self.pos_emb.data_ptr()
        w.ln1, w.ln2, w.lnf = self.ln1.data_ptr(), self.ln2.data_ptr(), self.lnf.data_ptr()
        w.w_qkv, w.w_o = self.w_qkv.data_ptr(), self.w_o.data_ptr()
        w.w_up, w.w_down = _ptr(self.w_up), _ptr(self.w_down)
        w.w_router, w.w_exp_up, w.w_exp_down = _ptr(self.w_router), _ptr(self.w_eup), _ptr(self.w_edown)
        w.cpl_a, w.cpl_b, w.cpl_c = self.cpl_a.data_ptr(), self.cpl_b.data_ptr(), self.cpl_c.data_ptr()
        w.w_out = self.w_out.data_ptr()
        self.weights = w
        self.kv = _abi.df_kv(self.k.data_ptr(), self.v.data_ptr(), self.len.data_ptr())
        # one workspace for both calls (the prefill one is the larger)
        self.ws_bytes = _abi.df_prefill_workspace_bytes(self.config)
        if self.ws_bytes == 0 or _abi.df_workspace_bytes(self.config) == 0:
            raise ValueError(f"unsupported config {c}")
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=self.dev)
        self.logits = torch.zeros(c.B, 2, c.V, dtype=torch.float32, device=self.dev)
        self.p_mix = torch.zeros(c.B, c.V, dtype=torch.float32, device=self.dev)
        self.alpha = torch.zeros(c.B, dtype=torch.float32, device=self.dev)
        self.next_tok = torch.zeros(c.B, dtype=torch.int32, device=self.dev)
        self.expert_ids = torch.zeros(c.L, c.B, max(c.top_k, c.top_k_aux, 1), dtype=torch.int32, device=self.dev)

    # -- inputs -----------------------------------------------------------------
    def _up(self, dst: torch.Tensor, arr: np.ndarray):
        a = np.ascontiguousarray(arr)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        dst.copy_(torch.from_numpy(a).reshape(dst.shape))

    def _fill(self, mode: str):
        c, s = self.cfg, self.src
        ws = c.sigma_w
        if mode == "device":
            def fill(t, name, idx_list, n_per, pitch, sigma, offset=0):
                synth_dev.normal_streams(t, [stream_id(name, *i) for i in idx_list], n_per, pitch, c.seed, sigma,
                                         self.bf16, offset)
            for f in range(2):
                fe = 0 if (c.tie_emb and f == 1) else f
                fill(self.tok_emb[f], "tok_emb", [(fe,)], c.V * c.d, c.V * c.d, ws)
            fill(self.pos_emb, "pos_emb", [()], self.S * c.d, self.S * c.d, ws)
            L = range(c.L)
            fill(self.w_qkv, "w_qkv", [(l,) for l in L], 3 * c.d * c.d, 3 * c.d * c.d, ws)
            fill(self.w_o, "w_o", [(l,) for l in L], c.d * c.d, c.d * c.d, ws)
            if c.moe:
                fill(self.w_router, "w_router", [(l,) for l in L], c.E * c.d, c.E * c.d, ws)
                ee = [(l, e) for l in L for e in range(c.E)]
                fill(self.w_eup, "w_eup", ee, c.Fe * c.d, c.Fe * c.d, ws)
                fill(self.w_edown, "w_edown", ee, c.Fe * c.d, c.Fe * c.d, ws)
            else:
                fill(self.w_up, "w_up", [(l,) for l in L], c.F * c.d, c.F * c.d, ws)
                fill(self.w_down, "w_down", [(l,) for l in L], c.F * c.d, c.F * c.d, ws)
            fill(self.w_out, "w_out", [()], c.V * c.d, c.V * c.d, ws)
            if c.ctx > 0:
                for which, t in (("kv_k", self.k), ("kv_v", self.v)):
                    for l in L:
                        idx = [(l, b, h) for b in range(c.B) for h in range(c.H)]
                        fill(t, which, idx, c.ctx * c.Dh, self.S * c.Dh, c.sigma_kv,
                             offset=l * c.B * c.H * self.S * c.Dh)
        elif mode == "host":
            for f in range(2):
                self._up(self.tok_emb[f], s.tok_emb(f))
            self._up(self.pos_emb, s.pos_emb(n_rows=self.S))
            for l in range(c.L):
                self._up(self.w_qkv[l], s.w_qkv(l))
                self._up(self.w_o[l], s.w_o(l))
                if c.moe:
                    self._up(self.w_router[l], s.w_router(l))
                    for e in range(c.E):
                        self._up(self.w_eup[l, e], s.w_exp_up(l, e))
                        self._up(self.w_edown[l, e], s.w_exp_down(l, e))
                else:
                    self._up(self.w_up[l], s.w_up(l))
                    self._up(self.w_down[l], s.w_down(l))
                if c.ctx > 0:
                    for b in range(c.B):
                        self._up(self.k[l, b, :, :c.ctx], s.kv_block("k", l, b, c.ctx))
                        self._up(self.v[l, b, :, :c.ctx], s.kv_block("v", l, b, c.ctx))
            self._up(self.w_out, s.w_out())
        else:
            raise ValueError(mode)
        if self.bf16:   # bf16 projection matrices go to the matrix-core fragment layout
            self._pack(self.w_qkv, c.L, 3 * c.d, c.d)
            self._pack(self.w_o, c.L, c.d, c.d)
            if c.moe:
                self._pack(self.w_router, c.L, c.E, c.d)
                self._pack(self.w_eup, c.L * c.E, c.Fe, c.d)
                self._pack(self.w_edown, c.L * c.E, c.d, c.Fe)
            else:
                self._pack(self.w_up, c.L, c.F, c.d)
                self._pack(self.w_down, c.L, c.d, c.F)
            self._pack(self.w_out, 1, c.V, c.d)
        # small fp32 parameters always come from the host generator
        for l in range(c.L):
            self.ln1[l] = torch.from_numpy(s.ln_gain("ln1", l))
            self.ln2[l] = torch.from_numpy(s.ln_gain("ln2", l))
            self.cpl_a[l] = torch.from_numpy(s.coupling("a", l))
            self.cpl_b[l] = torch.from_numpy(s.coupling("b", l))
            self.cpl_c[l] = torch.from_numpy(s.coupling("c", l))
        self.lnf.copy_(torch.from_numpy(s.ln_gain("lnf", 0)))
        torch.cuda.synchronize(self.dev)

    def _pack(self, t: torch.Tensor, n_mats: int, rows: int, cols: int):
        """Row-major bf16 matrices in `t` to the fragment layout, in place
        (through a temporary copy)."""
        src = t.clone()
        _abi.check(_abi.df_pack_weights(_abi.DF_BF16, src.data_ptr(), t.data_ptr(), n_mats, rows, cols, _stream()),
                   "df_pack_weights")
        torch.cuda.synchronize(self.dev)
        del src

    def tokens(self, arr) -> torch.Tensor:
        return torch.as_tensor(np.asarray(arr, dtype=np.int32), device=self.dev)

    def router_logits(self, step: int) -> torch.Tensor:
        c = self.cfg
        a = np.stack([self.src.router_logits(step, l) for l in range(c.L)])
        return torch.from_numpy(a).to(self.dev)

    # -- calls ------------------------------------------------------------------
    def decode_step(self, tokens: torch.Tensor, aux_on: bool = True, router_logits: Optional[torch.Tensor] = None,
                    logits: bool = True, next_tok: bool = True, expert_ids: bool = True):
        c = self.cfg
        rc = _abi.df_decode_step(self.config, self.weights, self.kv, tokens.data_ptr(), 1 if aux_on else 0,
                                 _ptr(router_logits), self.logits.data_ptr() if logits else None,
                                 self.p_mix.data_ptr(), self.alpha.data_ptr(),
                                 self.next_tok.data_ptr() if next_tok else None,
                                 self.expert_ids.data_ptr() if (expert_ids and c.moe) else None,
                                 self.ws.data_ptr(), self.ws_bytes, _stream())
        _abi.check(rc, "df_decode_step")

    def prefill(self, tokens_bt: torch.Tensor):
        T = tokens_bt.shape[1]
        rc = _abi.df_prefill_primary(self.config, self.weights, self.kv, tokens_bt.data_ptr(), T, self.ws.data_ptr(),
                                     self.ws_bytes, _stream())
        _abi.check(rc, "df_prefill_primary")

    def forward(self, tokens_bt: torch.Tensor, logits: bool = True, next_tok: bool = True):
        """Full-sequence dual forward over tokens [B][T]; returns (logits
        [B][T][2][V] or None, p_mix [B][T][V], alpha [B][T], next_tok [B][T]
        or None). Grows the workspace on first use."""
        c = self.cfg
        T = tokens_bt.shape[1]
        need = _abi.df_forward_workspace_bytes(self.config)
        if need > self.ws_bytes:
            ws = torch.zeros(need, dtype=torch.uint8, device=self.dev)
            ws[:256].copy_(self.ws[:256])             # device status word
            self.ws, self.ws_bytes = ws, need
        lg = torch.empty(c.B, T, 2, c.V, dtype=torch.float32, device=self.dev) if logits else None
        pm = torch.empty(c.B, T, c.V, dtype=torch.float32, device=self.dev)
        al = torch.empty(c.B, T, dtype=torch.float32, device=self.dev)
        nt = torch.empty(c.B, T, dtype=torch.int32, device=self.dev) if next_tok else None
        rc = _abi.df_forward_dual(self.config, self.weights, self.kv, tokens_bt.data_ptr(), T, _ptr(lg),
                                  pm.data_ptr(), al.data_ptr(), _ptr(nt), self.ws.data_ptr(), self.ws_bytes,
                                  _stream())
        _abi.check(rc, "df_forward_dual")
        return lg, pm, al, nt

    def status(self) -> int:
        rc, v = _abi.df_device_status(self.ws.data_ptr(), _stream())
        _abi.check(rc, "df_device_status")
        return v

    # -- byte accounting (algorithmic bytes of one step) -----------------------------
    def algorithmic_bytes(self, aux_on: bool = True, touched_experts: Optional[np.ndarray] = None) -> dict:
        """Bytes a step must move at least: each weight once (MoE: touched
        experts only), the K/V cache read once for both flows, the K/V append,
        the embedding and position rows, coupling vectors, norms, and the
        p_mix write."""
        c = self.cfg
        es = 2 if self.bf16 else 4
        lens = self.len.cpu().numpy().astype(np.int64)
        keys = int((lens + 1).sum())
        w = c.L * (3 * c.d * c.d + c.d * c.d) * es + c.V * c.d * es
        if c.moe:
            te = touched_experts if touched_experts is not None else np.full(c.L, c.E)
            w += c.L * c.E * c.d * es + int(np.sum(te)) * 2 * c.Fe * c.d * es
        else:
            w += c.L * 2 * c.F * c.d * es
        kv_read = c.L * c.H * keys * c.Dh * es * 2
        kv_write = c.L * c.B * c.H * c.Dh * es * 2
        rows = (2 if aux_on else 1) * c.B * c.d * es + c.B * c.d * es
        small = c.L * (2 * c.d + c.d + c.ffn + c.d) * 4 + c.d * 4 + c.B * c.V * 4
        return {"weights": w, "kv_read": kv_read, "kv_write": kv_write, "rows": rows, "small": small,
                "total": w + kv_read + kv_write + rows + small}
