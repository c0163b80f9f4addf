"""Workload shapes and the seeded input recipe.

A ``Config`` holds the sizes of one decode workload; ``Inputs`` draws every
input tensor of that workload from the counter-based generator, by name, one
tensor (or one layer) at a time, so that large workloads never have to be held
on the host at once. Nothing here computes any part of the method.

Input recipe (all values seeded; sigma values per tensor kind):
  token embeddings (primary, aux), position table, projection weights,
  router and expert weights, LM head ..... N(0, sigma_w^2), storage dtype
  coupling vectors a, b, c ................ N(0, sigma_cpl^2), fp32
  LayerNorm gains ......................... 1 + N(0, sigma_ln^2), fp32 (ones if 0)
  prefilled K/V cache entries ............. N(0, sigma_kv^2), storage dtype
  decode-step token ids ................... uniform in [0, V)
  primary router logits (override mode) ... each row a seeded permutation of the
                                            E standard-normal quantiles
                                            Phi^-1((i + 1/2) / E): tie-free
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

from . import normal, normal_streams, permutation, stream_id, uniform_int


@dataclass(frozen=True)
class Config:
    name: str
    L: int = 2
    d: int = 128
    H: int = 4
    Dh: int = 32
    F: int = 512
    V: int = 512
    B: int = 1
    ctx: int = 0              # prefilled positions per sequence (random K/V)
    S_max: int = 128          # cache capacity (positions)
    dtype: str = "f32"        # storage dtype of weights, embeddings and K/V
    moe: bool = False
    E: int = 0
    top_k: int = 0
    Fe: int = 0
    router_override: bool = False
    seed: int = 0
    sigma_w: float = 0.02
    sigma_cpl: float = 0.1
    sigma_kv: float = 1.0
    sigma_ln: float = 0.0
    eps: float = 1e-5
    tie_emb: bool = False     # aux token embedding := primary token embedding
    zero_cpl: bool = False    # a = b = c = 0
    prompt_len: int = 0       # tiny config: prompt length (prefill prompt_len-1)
    n_steps: int = 0          # tiny config: dual decode steps after prefill
    variant: int = 0          # ablation switches (VARIANT_* below)
    top_k_aux: int = 0        # MoE: experts of the aux flow from the primary ranking (0: same as top_k)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def ffn(self) -> int:
        return self.Fe if self.moe else self.F


@dataclass(frozen=True)
class AttnConfig:
    """Shared-KV attention kernel alone (two queries per head)."""
    name: str
    B: int = 32
    H: int = 32
    Dh: int = 128
    len_lo: int = 1024
    len_hi: int = 4096        # inclusive
    S_max: int = 4096
    dtype: str = "bf16"
    seed: int = 1


# Ablation switches of a model variant (bit flags).
VARIANT_NO_COUPLING = 1   # a, b, c couplings off
VARIANT_AUX_OUTPUT = 2    # no mixture: the step outputs the aux distribution
VARIANT_ALPHA_HALF = 4    # alpha = (1 + collision probability) / 2


# The five graded workloads.
C1_TINY = Config("tiny_dense_fp32", L=2, d=128, H=4, Dh=32, F=512, V=512, B=1, ctx=0,
                 S_max=80, dtype="f32", seed=0, prompt_len=63, n_steps=16)
C2_ATTN = AttnConfig("shared_kv_attention_b32_h32_len1024_4096")
C3_DENSE = Config("dense_1p3b_b16_ctx2048", L=24, d=2048, H=16, Dh=128, F=8192, V=32000, B=16,
                  ctx=2048, S_max=2048 + 64, dtype="bf16", seed=2)
C4_MOE = Config("moe_16l_e64_top4_b64_ctx1024", L=16, d=2048, H=16, Dh=128, F=0, V=32000, B=64,
                ctx=1024, S_max=1024 + 64, dtype="bf16", moe=True, E=64, top_k=4, Fe=1024,
                router_override=True, seed=3)
C5_LARGE = Config("dense_32l_d4096_b16_ctx8192", L=32, d=4096, H=32, Dh=128, F=16384, V=32000, B=16,
                  ctx=8192, S_max=8192 + 64, dtype="bf16", seed=4)

PRESETS = {"c1": C1_TINY, "c2": C2_ATTN, "c3": C3_DENSE, "c4": C4_MOE, "c5": C5_LARGE}

# Primary prefill of the 1.3B dense model: the 2048-position prompts whose
# cache the dense decode workload starts from (16 sequences, empty cache).
PREFILL_DENSE = C3_DENSE.replace(name="prefill_dense_1p3b_b16_t2048", ctx=0, S_max=2048, prompt_len=2048)
# Full-sequence dual forward of the same model over the same 16 x 2048 tokens.
FORWARD_DENSE = C3_DENSE.replace(name="forward_dual_dense_1p3b_b16_t2048", ctx=0, S_max=2048, prompt_len=2048)


def normal_quantiles(n: int) -> np.ndarray:
    """Phi^-1((i + 1/2) / n), i = 0..n-1, as float32."""
    from scipy.special import ndtri
    return ndtri((np.arange(n, dtype=np.float64) + 0.5) / n).astype(np.float32)


class Inputs:
    """Seeded inputs of one workload, drawn on demand."""

    def __init__(self, cfg: Config):
        self.cfg = cfg

    # -- helpers -------------------------------------------------------------
    def _w(self, shape, name, *idx, sigma=None):
        c = self.cfg
        return normal(shape, c.seed, stream_id(name, *idx), c.sigma_w if sigma is None else sigma, c.dtype)

    def _f32(self, n, name, *idx, sigma):
        return normal((n,), self.cfg.seed, stream_id(name, *idx), sigma, "f32")

    # -- embeddings ------------------------------------------------------------
    def tok_emb(self, flow: int) -> np.ndarray:
        c = self.cfg
        f = 0 if (c.tie_emb and flow == 1) else flow
        return self._w((c.V, c.d), "tok_emb", f)

    def tok_emb_rows(self, flow: int, tokens) -> np.ndarray:
        """Only the rows of the given token ids (for large vocabularies)."""
        c = self.cfg
        f = 0 if (c.tie_emb and flow == 1) else flow
        sid = stream_id("tok_emb", f)
        return np.stack([normal((c.d,), c.seed, sid, c.sigma_w, c.dtype, offset=int(t) * c.d)
                         for t in tokens])

    def pos_emb(self, rows=None, n_rows=None) -> np.ndarray:
        c = self.cfg
        sid = stream_id("pos_emb")
        if rows is None:
            return normal((n_rows or c.S_max, c.d), c.seed, sid, c.sigma_w, c.dtype)
        return np.stack([normal((c.d,), c.seed, sid, c.sigma_w, c.dtype, offset=int(p) * c.d) for p in rows])

    # -- per-layer parameters ---------------------------------------------------
    def ln_gain(self, name: str, layer: int = 0) -> np.ndarray:
        c = self.cfg
        if c.sigma_ln == 0.0:
            return np.ones(c.d, dtype=np.float32)
        return (1.0 + self._f32(c.d, name, layer, sigma=c.sigma_ln)).astype(np.float32)

    def coupling(self, which: str, layer: int) -> np.ndarray:
        c = self.cfg
        n = c.ffn if which == "b" else c.d
        if c.zero_cpl:
            return np.zeros(n, dtype=np.float32)
        return self._f32(n, "cpl_" + which, layer, sigma=c.sigma_cpl)

    def w_qkv(self, layer: int):
        c = self.cfg
        return self._w((3 * c.d, c.d), "w_qkv", layer)

    def w_o(self, layer: int):
        c = self.cfg
        return self._w((c.d, c.d), "w_o", layer)

    def w_up(self, layer: int):
        c = self.cfg
        return self._w((c.F, c.d), "w_up", layer)

    def w_down(self, layer: int):
        c = self.cfg
        return self._w((c.d, c.F), "w_down", layer)

    def w_router(self, layer: int):
        c = self.cfg
        return self._w((c.E, c.d), "w_router", layer)

    def w_exp_up(self, layer: int, e: int):
        c = self.cfg
        return self._w((c.Fe, c.d), "w_eup", layer, e)

    def w_exp_down(self, layer: int, e: int):
        c = self.cfg
        return self._w((c.d, c.Fe), "w_edown", layer, e)

    def w_out(self):
        c = self.cfg
        return self._w((c.V, c.d), "w_out")

    # -- cache, tokens, router logits ------------------------------------------
    def kv_streams(self, which: str, layer: int, b: int):
        c = self.cfg
        return [stream_id("kv_" + which, layer, b, h) for h in range(c.H)]

    def kv_block(self, which: str, layer: int, b: int, n_pos: int) -> np.ndarray:
        """Prefilled cache entries of one sequence in one layer: [H, n_pos, Dh]."""
        c = self.cfg
        a = normal_streams(self.kv_streams(which, layer, b), n_pos * c.Dh, c.seed, c.sigma_kv, c.dtype)
        return a.reshape(c.H, n_pos, c.Dh)

    def step_tokens(self, step: int) -> np.ndarray:
        c = self.cfg
        return uniform_int(c.B, c.seed, stream_id("tok", step), 0, c.V)

    def prompt(self) -> np.ndarray:
        c = self.cfg
        return uniform_int(c.B * c.prompt_len, c.seed, stream_id("prompt"), 0, c.V).reshape(c.B, c.prompt_len)

    def router_logits(self, step: int, layer: int) -> np.ndarray:
        """Tie-free primary router logits [B, E] (float32)."""
        c = self.cfg
        q = normal_quantiles(c.E)
        out = np.empty((c.B, c.E), dtype=np.float32)
        for b in range(c.B):
            out[b] = q[permutation(c.E, c.seed, stream_id("rperm", step, layer, b))]
        return out


class AttnInputs:
    """Seeded inputs of the attention-only workload."""

    def __init__(self, cfg: AttnConfig):
        self.cfg = cfg

    def lengths(self) -> np.ndarray:
        c = self.cfg
        return uniform_int(c.B, c.seed, stream_id("attn_len"), c.len_lo, c.len_hi + 1)

    def kv_block(self, which: str, b: int, n_pos: int) -> np.ndarray:
        c = self.cfg
        st = [stream_id("attn_" + which, b, h) for h in range(c.H)]
        return normal_streams(st, n_pos * c.Dh, c.seed, 1.0, c.dtype).reshape(c.H, n_pos, c.Dh)

    def queries(self):
        """q1, q2raw: [B, H, Dh] float32; a: [H*Dh] float32 (all N(0,1))."""
        c = self.cfg
        q1 = normal((c.B, c.H, c.Dh), c.seed, stream_id("attn_q", 0), 1.0, "f32")
        q2 = normal((c.B, c.H, c.Dh), c.seed, stream_id("attn_q", 1), 1.0, "f32")
        a = normal((c.H * c.Dh,), c.seed, stream_id("attn_a"), 1.0, "f32")
        return q1, q2, a
