"""Float64 CPU oracle of the Dual-Flow Transformer grouped decode step, the
primary prefill and the full-sequence dual forward.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline may use this module. It is deliberately plain: one row at a time,
library matrix-vector products in float64, no blocking or fusion.

Sources (the pages are summaries of arXiv 2608.12385, "Dual-Flow
Transformers: Decoupling the Primary Prefill Path from Additional Decode
Computation"; cited by page and section):
  [ES] gist.science/es/paper/2608.12385, "Resumen Tecnico: Dual-Flow Transformers"
       sections "Arquitectura Central", "Mecanismos Clave",
       "Costes de Inferencia vs. Entrenamiento".
  [ZH] gist.science/zh/paper/2608.12385, the same summary in Chinese
       (sections on core architecture, key mechanisms, costs).
  [RU] aikraft.ru news page, section on architecture details and the
       Traditional vs Dual-Flow comparison table.

What the pages fix: two residual flows share every attention, MLP and output
matrix and differ only in their token embeddings and small coupling vectors
a_l, b_l, c_l ([ES] Arquitectura Central). The primary flow is a standard
causal Transformer that alone writes the persistent K/V cache; the auxiliary
flow is skipped in prefill, runs from the last prompt position on, forms its
own query Q2 coupled to Q1 through a_l and attends the primary K1/V1; b_l and
c_l carry primary information to the aux flow at the MLP intermediate and the
MLP output, one way only; the output is p_mix = alpha_t p_primary +
(1 - alpha_t) p_aux with alpha_t set from the collision probability of the
primary distribution and kept at 0.5 or more; in MoE models the aux flow
reuses the primary's chosen experts with its own gate weights ([ES] Mecanismos
Clave). Prefill is unchanged and decode reads each weight and K/V region once
for both flows ([ES] Costes de Inferencia vs. Entrenamiento). The ablations
name a minimal Dual construction without coupling and without the
probability mixture ([ES] Resultados), and MoE models may set the expert
fan-outs of the two flows independently ([ES] Contribuciones Clave 3,
Significado y Reivindicaciones): the model variant switches of
``synth.workloads`` (couplings off; output p_aux; alpha = (1 + CP) / 2) and
``top_k_aux`` (the aux flow's experts: the first top_k_aux of the primary's
ranking) select them.

Readings taken where the pages are silent (each stated where it is used):
pre-norm GPT block, LayerNorm with gain only (eps 1e-5, shared by both
flows), learned absolute positions shared by both flows, exact-erf GELU, no
linear biases, untied LM head; aux computes a query only; Q2 = Q2raw + a*Q1
before the 1/sqrt(Dh) scale; b_l after the GELU; c_l on the MLP output before
the residual add; alpha = min(1, max(0.5, sum p1^2)); greedy argmax with
ties to the lowest index; top-k ordered by descending logit with ties to the
lower expert index, gates are the softmax over the k selected logits of each
flow. Weights, embeddings and the K/V cache are stored in the storage dtype;
activations are not rounded: the only rounding rho (to the storage dtype,
nearest-even) in a step is that of the appended K/V entries. (Rounding every
projection input to bf16 as well makes full-depth logits move by ~4e-2 under
fp32-level perturbations, so no two implementations could agree to 2e-2.)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
from scipy.special import erf

# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def decode_bf16(u16: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact): the bits are the
    upper half of the float32 with the same value. Converted in blocks to keep
    the temporaries small; `out` (same shape, float64) may be reused."""
    u = np.ascontiguousarray(u16, dtype=np.uint16)
    if out is None or out.shape != u.shape:
        out = np.empty(u.shape, dtype=np.float64)
    uf, of = u.reshape(-1), out.reshape(-1)
    n = 1 << 22
    for i in range(0, uf.size, n):
        of[i:i + n] = (uf[i:i + n].astype(np.uint32) << 16).view(np.float32)
    return out


def to_f64(raw: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Decode a stored tensor (uint16 = bf16 bits, or float32) into float64."""
    if raw.dtype == np.uint16:
        return decode_bf16(raw, out)
    if out is not None and out.shape == raw.shape:
        out[...] = raw
        return out
    return np.asarray(raw, dtype=np.float64)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits),
    ties to even. Exact for the normal bf16 range, which is all the method
    produces here (no subnormal or overflowing values occur)."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """rho: round to the storage dtype ('bf16' or 'f32'), nearest-even."""
    if dtype == "bf16":
        return _round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# Textbook pieces
# --------------------------------------------------------------------------


def layer_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with a gain and no bias, biased variance.
    (Reading: the pages name no norm; NanoGPT-style pre-norm is taken.)"""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def softmax(x: np.ndarray) -> np.ndarray:
    m = np.max(x)
    p = np.exp(x - m)
    return p / p.sum()


def attention_one(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """Softmax attention of one query over n keys: returns (o, lse).
    scores s_j = q.K_j / sqrt(Dh); o = sum_j softmax(s)_j V_j; lse = log sum exp s."""
    s = (K @ q) / math.sqrt(q.shape[0])
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ V) / l, m + math.log(l)


def attention_dual(K: np.ndarray, V: np.ndarray, q1: np.ndarray, q2raw: np.ndarray,
                   lens: np.ndarray, a: Optional[np.ndarray] = None):
    """Asymmetric shared-K/V attention ([ES] Mecanismos Clave, first item):
    both queries of a head attend the same primary keys/values 0..len_b-1.
    K, V: [B, H, S, Dh] (float64 values); q1, q2raw: [B, H, Dh];
    a: [H*Dh] or None -> q2 = q2raw + a * q1 (query-level coupling).
    Returns o [B, 2, H, Dh] and lse [B, 2, H]."""
    B, H, _, Dh = K.shape
    q1 = np.asarray(q1, dtype=np.float64)
    q2 = np.asarray(q2raw, dtype=np.float64)
    if a is not None:
        q2 = q2 + np.asarray(a, dtype=np.float64).reshape(H, Dh)[None] * q1
    o = np.zeros((B, 2, H, Dh))
    lse = np.zeros((B, 2, H))
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            for f, q in enumerate((q1[b, h], q2[b, h])):
                o[b, f, h], lse[b, f, h] = attention_one(q, K[b, h, :n], V[b, h, :n])
    return o, lse


MIX_COLLISION, MIX_AUX, MIX_HALF = "collision", "aux", "half"


def mix_head(l1: np.ndarray, l2: Optional[np.ndarray], mode: str = MIX_COLLISION):
    """Mixture output ([ES] Mecanismos Clave, mixture objective):
    p_mix = alpha p1 + (1 - alpha) p2 with p_f = softmax(l_f) over the whole
    vocabulary (temperature 1). alpha is read as the collision probability
    sum_v p1(v)^2, floored at 0.5 (the primary keeps at least half the
    weight) and capped at 1 against rounding. With no aux logits (aux flow
    off) the step is primary-only: alpha = 1 and p_mix = p1.
    Ablations ([ES] Resultados, ablations: the minimal Dual construction has
    no probability mixture): mode "aux" outputs the aux distribution alone
    (alpha = 0); mode "half" takes the other reading of the floor,
    alpha = (1 + CP) / 2, also in [0.5, 1].
    next token: argmax of p_mix, ties to the lowest index (greedy reading)."""
    p1 = softmax(np.asarray(l1, dtype=np.float64))
    if l2 is None:
        alpha = 1.0
        p = p1
    else:
        p2 = softmax(np.asarray(l2, dtype=np.float64))
        cp = float(np.sum(p1 * p1))
        if mode == MIX_AUX:
            alpha = 0.0
        elif mode == MIX_HALF:
            alpha = min(1.0, 0.5 * (1.0 + cp))
        elif mode == MIX_COLLISION:
            alpha = min(1.0, max(0.5, cp))
        else:
            raise ValueError(mode)
        p = alpha * p1 + (1.0 - alpha) * p2
    return p, alpha, int(np.argmax(p))


def mix_mode(variant: int) -> str:
    """Mixture mode of a model variant (bit flags of synth.workloads)."""
    if variant & 2 and variant & 4:
        raise ValueError("aux output and alpha = (1 + CP) / 2 exclude each other")
    return MIX_AUX if variant & 2 else (MIX_HALF if variant & 4 else MIX_COLLISION)


def topk_ids(r: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest logits, by descending value, ties to the lower index."""
    return np.argsort(-np.asarray(r, dtype=np.float64), kind="stable")[:k].astype(np.int32)


# --------------------------------------------------------------------------
# Parameters and cache
# --------------------------------------------------------------------------


class Model:
    """Float64 view of a workload's parameters, drawn from a ``synth``
    ``Inputs`` source and decoded here. Layers are decoded on demand and
    kept only for small models (``keep_layers``)."""

    def __init__(self, src, keep_layers: Optional[bool] = None):
        self.src = src
        self.cfg = src.cfg
        c = self.cfg
        n_params = c.L * (4 * c.d * c.d + 2 * c.d * (c.E * c.Fe if c.moe else c.F))
        self.keep = keep_layers if keep_layers is not None else n_params < 64_000_000
        self._layers: Dict[int, dict] = {}
        self._scratch: Dict[str, np.ndarray] = {}   # decode buffers reused layer to layer
        self._out = None
        self._lnf = None

    def _dec(self, key: str, raw: np.ndarray) -> np.ndarray:
        if self.keep:
            return to_f64(raw)
        self._scratch[key] = to_f64(raw, self._scratch.get(key))
        return self._scratch[key]

    def emb(self, flow: int, tokens) -> np.ndarray:
        return to_f64(self.src.tok_emb_rows(flow, tokens))

    def pos(self, positions) -> np.ndarray:
        return to_f64(self.src.pos_emb(rows=positions))

    def layer(self, l: int) -> dict:
        if l in self._layers:
            return self._layers[l]
        s, c = self.src, self.cfg
        p = {
            "ln1": s.ln_gain("ln1", l).astype(np.float64),
            "ln2": s.ln_gain("ln2", l).astype(np.float64),
            "w_qkv": self._dec("w_qkv", s.w_qkv(l)),
            "w_o": self._dec("w_o", s.w_o(l)),
            "a": s.coupling("a", l).astype(np.float64),
            "b": s.coupling("b", l).astype(np.float64),
            "c": s.coupling("c", l).astype(np.float64),
        }
        if c.moe:
            p["w_router"] = self._dec("w_router", s.w_router(l))
            p["w_eup"] = [self._dec(f"w_eup{e}", s.w_exp_up(l, e)) for e in range(c.E)]
            p["w_edown"] = [self._dec(f"w_edown{e}", s.w_exp_down(l, e)) for e in range(c.E)]
        else:
            p["w_up"] = self._dec("w_up", s.w_up(l))
            p["w_down"] = self._dec("w_down", s.w_down(l))
        if self.keep:
            self._layers[l] = p
        return p

    def ln_next(self, l: int) -> np.ndarray:
        """Gain of the norm that follows layer l: LN1 of layer l+1, or the final LN."""
        if l + 1 < self.cfg.L:
            return self.src.ln_gain("ln1", l + 1).astype(np.float64)
        return self.lnf()

    def lnf(self) -> np.ndarray:
        if self._lnf is None:
            self._lnf = self.src.ln_gain("lnf", 0).astype(np.float64)
        return self._lnf

    def w_out(self) -> np.ndarray:
        if self._out is None:
            w = to_f64(self.src.w_out())
            if not self.keep:
                return w
            self._out = w
        return self._out


class Cache:
    """The single persistent K/V cache, held for a chosen set of sequences.

    k[l], v[l]: [nb, H, S_max, Dh] float64 (values of the storage dtype);
    lens[i]: number of filled positions of sequence seqs[i]. Layers may be
    drawn lazily from the seeded prefilled blocks (``lazy``) and dropped after
    use, which keeps very large workloads within host memory; the entries
    the steps append are always recorded in ``appended``."""

    def __init__(self, cfg, seqs: List[int], src=None, lazy: bool = False):
        self.cfg = cfg
        self.seqs = list(seqs)
        self.src = src
        self.lazy = lazy
        self.lens = np.full(len(self.seqs), cfg.ctx, dtype=np.int64)
        self._k: Dict[int, np.ndarray] = {}
        self._v: Dict[int, np.ndarray] = {}
        self.appended: Dict[tuple, tuple] = {}   # (l, seq, pos) -> (k [H,Dh], v [H,Dh])
        self._spare = None

    def _fill(self, l: int):
        c = self.cfg
        nb = len(self.seqs)
        if self.lazy and self._spare is not None:
            k, v = self._spare          # buffers of a released layer, reused
            self._spare = None
            k[...] = 0.0
            v[...] = 0.0
        else:
            k = np.zeros((nb, c.H, c.S_max, c.Dh))
            v = np.zeros((nb, c.H, c.S_max, c.Dh))
        if c.ctx > 0:
            for i, b in enumerate(self.seqs):
                k[i, :, :c.ctx] = to_f64(self.src.kv_block("k", l, b, c.ctx))
                v[i, :, :c.ctx] = to_f64(self.src.kv_block("v", l, b, c.ctx))
        for (ll, b, pos), (kk, vv) in self.appended.items():
            if ll == l:
                i = self.seqs.index(b)
                k[i, :, pos] = kk
                v[i, :, pos] = vv
        return k, v

    def layer(self, l: int):
        if l not in self._k:
            self._k[l], self._v[l] = self._fill(l)
        return self._k[l], self._v[l]

    def release(self, l: int):
        if self.lazy and l in self._k:
            self._spare = (self._k.pop(l), self._v.pop(l))

    def write(self, l: int, i: int, pos: int, k_hd: np.ndarray, v_hd: np.ndarray):
        K, V = self.layer(l)
        K[i, :, pos] = k_hd
        V[i, :, pos] = v_hd
        self.appended[(l, self.seqs[i], pos)] = (k_hd.copy(), v_hd.copy())


@dataclass
class StepResult:
    logits: np.ndarray                    # [nb, 2, V] (aux row zero when aux off)
    p_mix: np.ndarray                     # [nb, V]
    alpha: np.ndarray                     # [nb]
    next_tok: np.ndarray                  # [nb]
    ids: Optional[np.ndarray] = None      # [L, nb, k] (MoE)
    gates: Optional[np.ndarray] = None    # [L, nb, 2, k] (MoE)
    trace: Dict[str, np.ndarray] = field(default_factory=dict)


# --------------------------------------------------------------------------
# Decode step
# --------------------------------------------------------------------------


def _matvec(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W x for one row: the same call for every row, whatever the flow count."""
    return W @ np.ascontiguousarray(x)


def couple_query(q2raw: np.ndarray, a: np.ndarray, q1: np.ndarray) -> np.ndarray:
    """Query-level coupling: Q2 = Q2raw + a_l * Q1, per channel, applied to the
    projected queries before the attention scale (the pages couple Q2 to Q1
    through a learned vector; the elementwise form is the reading)."""
    return q2raw + a * q1


def couple_mid(g2: np.ndarray, b: np.ndarray, g1: np.ndarray) -> np.ndarray:
    """MLP-intermediate coupling on the post-GELU activations: g2 + b_l * g1."""
    return g2 + b * g1


def couple_out(y2: np.ndarray, c: np.ndarray, y1: np.ndarray) -> np.ndarray:
    """MLP-output coupling before the residual add: y2 + c_l * y1."""
    return y2 + c * y1


def qkv_rows(p: dict, u: list, cfg, couple: bool = True):
    """Shared Q/K/V projection of the stacked rows. The primary row yields Q1
    and the K1/V1 to append (rounded to the storage dtype); the aux row goes
    through the same matrix but keeps only its query, coupled to Q1 (the aux
    flow never writes the persistent cache, [ES] Arquitectura Central;
    couple=False: the uncoupled ablation, [ES] Resultados)."""
    d = cfg.d
    qkv1 = _matvec(p["w_qkv"], u[0])
    q = [qkv1[:d]]
    if len(u) == 2:
        q2raw = _matvec(p["w_qkv"], u[1])[:d]
        q.append(couple_query(q2raw, p["a"], q[0]) if couple else q2raw)
    k_new = round_to(qkv1[d:2 * d], cfg.dtype).reshape(cfg.H, cfg.Dh)
    v_new = round_to(qkv1[2 * d:], cfg.dtype).reshape(cfg.H, cfg.Dh)
    return q, k_new, v_new


def attend(q: np.ndarray, K_bh: np.ndarray, V_bh: np.ndarray, pos: int) -> np.ndarray:
    """Decode-time attention of one query over cache positions 0..pos, which
    includes the primary entry just appended at pos (causal by construction)."""
    o, _ = attention_one(q, K_bh[:pos + 1], V_bh[:pos + 1])
    return o


def _mlp_dense(p: dict, v: np.ndarray, flows: int, dtype: str, tr: Optional[dict] = None, couple: bool = True):
    """Dense MLP of both flows with the two MLP couplings ([ES] Mecanismos Clave,
    light coupling): g2 = GELU(z2) + b * GELU(z1) (b_l on the post-activation
    intermediate), then y2 = g2 W2^T + c * y1 (c_l on the MLP output, before
    the residual add). Primary rows never read aux values. couple=False: the
    uncoupled ablation ([ES] Resultados)."""
    g = [gelu(_matvec(p["w_up"], v[f])) for f in range(flows)]
    if flows == 2 and couple:
        g[1] = couple_mid(g[1], p["b"], g[0])
    y = [_matvec(p["w_down"], g[f]) for f in range(flows)]
    if flows == 2 and couple:
        y[1] = couple_out(y[1], p["c"], y[0])
    if tr is not None:
        tr["mlp_g"] = np.stack(g)
        tr["mlp_y"] = np.stack(y)
    return y


def _mlp_moe(p: dict, v: np.ndarray, flows: int, dtype: str, k: int,
             r1_given: Optional[np.ndarray], tr: Optional[dict] = None, k_aux: int = 0,
             couple: bool = True):
    """MoE MLP with router replay ([ES] Mecanismos Clave, router replay): the
    primary router picks the top-k experts; the aux flow reuses exactly those
    experts with its own gates. Gates of each flow are the softmax over that
    flow's router logits at the chosen ids. Each chosen expert is a GELU
    MLP with the b_l coupling on its intermediate; the gate-weighted sum over
    the experts (in rank order) forms y, then c_l couples the outputs.

    Independent fan-outs ([ES] Contribuciones Clave 3 and Significado y
    Reivindicaciones: primary and aux expert fan-outs set separately): with
    k_aux > 0 the aux flow takes the first k_aux experts of the primary's
    ranking (k_aux = k is plain replay). The b_l coupling applies where the
    primary has that expert's intermediate (ranks below k); an aux-only
    expert has none to couple to."""
    ka = k if k_aux <= 0 else k_aux
    r = [_matvec(p["w_router"], v[f]) for f in range(flows)]
    r1 = r[0] if r1_given is None else np.asarray(r1_given, dtype=np.float64)
    ranking = topk_ids(r1, max(k, ka))      # reported whatever the flows
    ids = ranking[:k]
    gates = [softmax(r1[ids])]
    if flows == 2:
        gates.append(softmax(r[1][ranking[:ka]]))
    y = [np.zeros(v.shape[-1]) for _ in range(flows)]
    for j, e in enumerate(ranking):
        if j >= k and (flows == 1 or j >= ka):
            continue
        g = [gelu(_matvec(p["w_eup"][e], v[f])) for f in range(flows)]
        if flows == 2 and couple and j < k:
            g[1] = couple_mid(g[1], p["b"], g[0])
        if j < k:
            y[0] = y[0] + gates[0][j] * _matvec(p["w_edown"][e], g[0])
        if flows == 2 and j < ka:
            y[1] = y[1] + gates[1][j] * _matvec(p["w_edown"][e], g[1])
    if flows == 2 and couple:
        y[1] = couple_out(y[1], p["c"], y[0])
    if tr is not None:
        tr["router"] = np.stack(r)
        tr["ranking"] = ranking
    g_out = np.zeros((flows, max(k, ka)))   # gates by rank, zero beyond a flow's fan-out
    g_out[0, :k] = gates[0]
    if flows == 2:
        g_out[1, :ka] = gates[1]
    return y, ranking, g_out


def decode_step(model: Model, cache: Cache, tokens, aux_on: bool = True,
                router_logits: Optional[np.ndarray] = None, trace: bool = False) -> StepResult:
    """One grouped decode step for every sequence held by ``cache``.

    tokens[i]: token id of sequence cache.seqs[i] at position pos = lens[i].
    Per layer: u = LN1(h); primary [Q1 K1 V1] = u1 Wqkv^T; aux Q2 =
    u2 Wq^T + a * Q1 (aux forms a query only and never writes K/V); the cache
    receives rho(K1), rho(V1) at pos; both queries attend positions 0..pos of
    the primary cache; h += O Wo^T; v = LN2(h); MLP (dense or MoE) with b/c
    couplings; h += y. Then the final LN, the shared LM head and the
    mixture head. ([ES] Arquitectura Central and Mecanismos Clave; the aux
    flow joins the primary on the shared weights once per step, [ES] Costes.)

    router_logits: [L, nb, E] primary router logits supplied by the workload
    (tie-free mode) or None (computed from the router weights).
    Afterwards lens[i] += 1."""
    c = model.cfg
    dt = c.dtype
    flows = 2 if aux_on else 1
    couple = not (c.variant & 1)
    mode = mix_mode(c.variant)
    kr = max(c.top_k, c.top_k_aux, 1)
    nb = len(cache.seqs)
    pos = cache.lens.copy()
    if np.any(pos >= c.S_max):
        raise ValueError("cache full")
    tokens = np.asarray(tokens)
    P = model.pos(pos)
    h = np.zeros((nb, flows, c.d))
    for f in range(flows):
        h[:, f] = model.emb(f, tokens) + P
    ids_all = np.zeros((c.L, nb, kr), dtype=np.int32)
    gates_all = np.zeros((c.L, nb, 2, kr))
    tr: Dict[str, list] = {}
    g_prev = None
    for l in range(c.L):
        p = model.layer(l)
        K, V = cache.layer(l)
        g_in = p["ln1"] if g_prev is None else g_prev
        for i in range(nb):
            lt = {} if trace else None
            u = [layer_norm(h[i, f], g_in, c.eps) for f in range(flows)]
            q, k_new, v_new = qkv_rows(p, u, c, couple)
            cache.write(l, i, int(pos[i]), k_new, v_new)
            o = np.zeros((flows, c.d))
            for hh in range(c.H):
                sl = slice(hh * c.Dh, (hh + 1) * c.Dh)
                for f in range(flows):
                    o[f, sl] = attend(q[f][sl], K[i, hh], V[i, hh], int(pos[i]))
            for f in range(flows):
                h[i, f] = h[i, f] + _matvec(p["w_o"], o[f])
            if trace:
                lt["h_mid"] = h[i].copy()
            v = np.stack([layer_norm(h[i, f], p["ln2"], c.eps) for f in range(flows)])
            if c.moe:
                r1 = None if router_logits is None else router_logits[l][i]
                y, ids, gates = _mlp_moe(p, v, flows, dt, c.top_k, r1, lt, c.top_k_aux, couple)
                ids_all[l, i] = ids
                gates_all[l, i, :flows] = gates
            else:
                y = _mlp_dense(p, v, flows, dt, lt, couple)
            for f in range(flows):
                h[i, f] = h[i, f] + y[f]
            if trace:
                lt["q"] = np.stack(q)
                lt["o"] = o
                lt["h"] = h[i].copy()
                for key_, val in lt.items():
                    tr.setdefault(f"{key_}.{l}", []).append(val)
        g_prev = model.ln_next(l)
        cache.release(l)
    W_out = model.w_out()
    logits = np.zeros((nb, 2, c.V))
    p_mix = np.zeros((nb, c.V))
    alpha = np.zeros(nb)
    nxt = np.zeros(nb, dtype=np.int64)
    for i in range(nb):
        for f in range(flows):
            logits[i, f] = _matvec(W_out, layer_norm(h[i, f], model.lnf(), c.eps))
        p_mix[i], alpha[i], nxt[i] = mix_head(logits[i, 0], logits[i, 1] if flows == 2 else None, mode)
    cache.lens = cache.lens + 1
    res = StepResult(logits, p_mix, alpha, nxt,
                     ids_all if c.moe else None, gates_all if c.moe else None)
    res.trace = {k_: np.stack(v_) for k_, v_ in tr.items()}
    return res


# --------------------------------------------------------------------------
# Prefill (primary flow only, whole prompt at once)
# --------------------------------------------------------------------------


def prefill_primary(model: Model, cache: Cache, prompt: np.ndarray):
    """Standard causal Transformer over the prompt, primary flow only; the aux
    flow is skipped in prefill ([ES] Arquitectura Central, activation; [ES]
    Costes: prefill costs exactly a standard Transformer). prompt: [nb, T]
    token ids written at positions lens .. lens+T-1. Writes rho(K1), rho(V1)
    for every prompt position and advances lens by T. Returns the primary
    logits of every prompt position [nb, T, V]."""
    c = model.cfg
    dt = c.dtype
    prompt = np.asarray(prompt)
    nb, T = prompt.shape
    out = np.zeros((nb, T, c.V))
    for i in range(nb):
        p0 = int(cache.lens[i])
        pos = np.arange(p0, p0 + T)
        h = model.emb(0, prompt[i]) + model.pos(pos)
        g_in = None
        for l in range(c.L):
            p = model.layer(l)
            K, V = cache.layer(l)
            g = p["ln1"] if g_in is None else g_in
            u = layer_norm(h, g, c.eps)
            qkv = u @ p["w_qkv"].T
            Q = qkv[:, :c.d]
            K[i, :, p0:p0 + T] = round_to(qkv[:, c.d:2 * c.d], dt).reshape(T, c.H, c.Dh).transpose(1, 0, 2)
            V[i, :, p0:p0 + T] = round_to(qkv[:, 2 * c.d:], dt).reshape(T, c.H, c.Dh).transpose(1, 0, 2)
            for t in range(T):
                cache.appended[(l, cache.seqs[i], p0 + t)] = (K[i, :, p0 + t].copy(), V[i, :, p0 + t].copy())
            O = np.zeros((T, c.d))
            for t in range(T):
                n = p0 + t + 1            # causal: keys 0..p0+t
                for hh in range(c.H):
                    sl = slice(hh * c.Dh, (hh + 1) * c.Dh)
                    O[t, sl], _ = attention_one(Q[t, sl], K[i, hh, :n], V[i, hh, :n])
            h = h + O @ p["w_o"].T
            v = layer_norm(h, p["ln2"], c.eps)
            if c.moe:
                y = np.zeros_like(h)
                for t in range(T):
                    yy, _, _ = _mlp_moe(p, v[t:t + 1], 1, dt, c.top_k, None)
                    y[t] = yy[0]
            else:
                y = gelu(v @ p["w_up"].T) @ p["w_down"].T
            h = h + y
            g_in = model.ln_next(l)
        out[i] = layer_norm(h, model.lnf(), c.eps) @ model.w_out().T
    cache.lens = cache.lens + T
    return out


# --------------------------------------------------------------------------
# Full-sequence dual forward (both flows at every position)
# --------------------------------------------------------------------------


@dataclass
class ForwardResult:
    logits: np.ndarray                    # [nb, T, 2, V]
    p_mix: np.ndarray                     # [nb, T, V]
    alpha: np.ndarray                     # [nb, T]
    next_tok: np.ndarray                  # [nb, T]


def forward_dual(model: Model, cache: Cache, tokens: np.ndarray) -> ForwardResult:
    """Both flows over a whole token sequence, as in training, where both
    flows are evaluated along the full sequence ([ES] Costes de Inferencia
    vs. Entrenamiento, training). tokens: [nb, T], sequence i at positions
    lens[i] .. lens[i] + T - 1. Written per sequence in matrix form over
    the T positions: the primary flow is the causal Transformer of the
    prefill; the aux flow at position t forms its query from its own
    normed row, Q2 = Q2raw + a * Q1, and attends the primary K1/V1 of
    positions 0 .. t (shared K/V, causal); b_l and c_l couple the MLP rows
    position by position; every position gets both flows' logits and the
    mixture output ([ES] Arquitectura Central, Mecanismos Clave). The cache
    receives rho(K1), rho(V1) of every position and lens advances by T.
    Reading: the aux state at position t depends on positions <= t only
    through the primary K/V, so the result is the one of T teacher-forced
    dual steps. MoE layers route each position on its own (router replay
    per row)."""
    c = model.cfg
    dt = c.dtype
    couple = not (c.variant & 1)
    mode = mix_mode(c.variant)
    tokens = np.asarray(tokens)
    nb, T = tokens.shape
    if np.any(cache.lens + T > c.S_max):
        raise ValueError("cache full")
    d = c.d
    h_all = np.zeros((nb, 2, T, d))
    for i in range(nb):
        pos = np.arange(int(cache.lens[i]), int(cache.lens[i]) + T)
        for f in range(2):
            h_all[i, f] = model.emb(f, tokens[i]) + model.pos(pos)
    g_prev = None
    for l in range(c.L):
        p = model.layer(l)
        K, V = cache.layer(l)
        g_in = p["ln1"] if g_prev is None else g_prev
        for i in range(nb):
            p0 = int(cache.lens[i])
            h = h_all[i]
            u = [layer_norm(h[f], g_in, c.eps) for f in range(2)]
            qkv1 = u[0] @ p["w_qkv"].T
            q1 = qkv1[:, :d]
            q2 = u[1] @ p["w_qkv"][:d].T
            if couple:
                q2 = q2 + p["a"][None, :] * q1
            K[i, :, p0:p0 + T] = round_to(qkv1[:, d:2 * d], dt).reshape(T, c.H, c.Dh).transpose(1, 0, 2)
            V[i, :, p0:p0 + T] = round_to(qkv1[:, 2 * d:], dt).reshape(T, c.H, c.Dh).transpose(1, 0, 2)
            for t in range(T):
                cache.appended[(l, cache.seqs[i], p0 + t)] = (K[i, :, p0 + t].copy(), V[i, :, p0 + t].copy())
            for f, qf in enumerate((q1, q2)):
                o = np.zeros((T, d))
                for t in range(T):
                    n = p0 + t + 1
                    for hh in range(c.H):
                        sl = slice(hh * c.Dh, (hh + 1) * c.Dh)
                        o[t, sl], _ = attention_one(qf[t, sl], K[i, hh, :n], V[i, hh, :n])
                h[f] = h[f] + o @ p["w_o"].T
            v = np.stack([layer_norm(h[f], p["ln2"], c.eps) for f in range(2)])   # [2, T, d]
            if c.moe:
                for t in range(T):
                    y, _, _ = _mlp_moe(p, v[:, t], 2, dt, c.top_k, None, None, c.top_k_aux, couple)
                    for f in range(2):
                        h[f, t] = h[f, t] + y[f]
            else:
                g = [gelu(v[f] @ p["w_up"].T) for f in range(2)]
                if couple:
                    g[1] = g[1] + p["b"][None, :] * g[0]
                y = [g[f] @ p["w_down"].T for f in range(2)]
                if couple:
                    y[1] = y[1] + p["c"][None, :] * y[0]
                for f in range(2):
                    h[f] = h[f] + y[f]
        g_prev = model.ln_next(l)
        cache.release(l)
    W_out = model.w_out()
    logits = np.zeros((nb, T, 2, c.V))
    p_mix = np.zeros((nb, T, c.V))
    alpha = np.zeros((nb, T))
    nxt = np.zeros((nb, T), dtype=np.int64)
    for i in range(nb):
        for f in range(2):
            logits[i, :, f] = layer_norm(h_all[i, f], model.lnf(), c.eps) @ W_out.T
        for t in range(T):
            p_mix[i, t], alpha[i, t], nxt[i, t] = mix_head(logits[i, t, 0], logits[i, t, 1], mode)
    cache.lens = cache.lens + T
    return ForwardResult(logits, p_mix, alpha, nxt)


# --------------------------------------------------------------------------
# The tiny end-to-end run: prefill, then dual steps from the last prompt token
# --------------------------------------------------------------------------


def run_tiny(model: Model, n_steps: Optional[int] = None, forced_tokens=None):
    """Prefill prompt[0..T-2] with the primary flow, then run dual steps from
    the final prompt position on: step 0 consumes prompt[T-1] at position
    T-1 and predicts the first continuation token; step s > 0 consumes the
    token chosen at step s-1 (greedy argmax of p_mix, or forced_tokens[s]).
    ([ES] Arquitectura Central: the aux flow activates at the last prompt
    position and at every generated position.) Returns (cache, results)."""
    c = model.cfg
    n_steps = c.n_steps if n_steps is None else n_steps
    prompt = model.src.prompt()
    cache = Cache(c, list(range(c.B)), model.src)
    prefill_primary(model, cache, prompt[:, :-1])
    tok = prompt[:, -1]
    results = []
    for s in range(n_steps):
        if forced_tokens is not None:
            tok = np.asarray(forced_tokens[s])
        r = decode_step(model, cache, tok, aux_on=True)
        results.append(r)
        tok = r.next_tok
    return cache, results
