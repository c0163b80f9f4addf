"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each pin raises AssertionError when the oracle disagrees with a library
routine, a closed form, a brute-force enumeration or a structural invariant
the pages state. ``test_oracle_pins`` runs them on the oracle as it is;
``test_oracle_mutations`` plants plausible mistakes in the oracle (on the
CPU) and checks that some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from oracle import dualflow as odf
from synth.workloads import Config, Inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TINY_F32 = Config("pin_tiny_f32", L=2, d=64, H=2, Dh=32, F=128, V=64, B=2, ctx=6, S_max=24,
                  dtype="f32", seed=11, sigma_w=0.1, sigma_ln=0.1, prompt_len=8)
TINY_BF16 = TINY_F32.replace(name="pin_tiny_bf16", dtype="bf16", seed=12)
TINY_MOE = Config("pin_tiny_moe", L=2, d=64, H=2, Dh=32, F=0, V=64, B=3, ctx=5, S_max=16,
                  dtype="bf16", moe=True, E=4, top_k=2, Fe=96, seed=13, sigma_w=0.1, sigma_ln=0.1,
                  prompt_len=6)


class ArraySource:
    """An ``Inputs`` source with some tensors replaced (methods by name)."""

    def __init__(self, base, **over):
        self.base = base
        self.cfg = base.cfg
        self.over = over

    def __getattr__(self, name):
        if name in self.over:
            return self.over[name]
        return getattr(self.base, name)


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# Number format and textbook pieces
# ----------------------------------------------------------------------------

def pin_round_bf16():
    """rho(bf16) against torch's fp32->bf16 conversion (round-nearest-even) on
    fp32-representable values, plus hand-worked ties and a value where
    rounding through fp32 first would give a different (wrong) answer."""
    x32 = (_rng(0).standard_normal(20000) * np.exp(_rng(1).uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = odf.round_to(x32.astype(np.float64), "bf16")
    assert np.array_equal(got, want), "bf16 rounding disagrees with torch"
    one = 1.0
    cases = [
        (one + 2 ** -8, one),                        # tie -> even (down)
        (one + 3 * 2 ** -8, one + 2 ** -6),          # tie -> even (up)
        (one + 2 ** -8 + 2 ** -40, one + 2 ** -7),   # just above the tie: up
        (-(one + 2 ** -8 + 2 ** -40), -(one + 2 ** -7)),
        (255.5, 256.0), (0.0, 0.0),
    ]
    for x, r in cases:
        assert odf.round_to(np.array([x]), "bf16")[0] == r, (x, r)


def pin_decode_bf16():
    """decode_bf16 against torch's bf16 -> float64 conversion over all 65536
    bit patterns: every finite value exactly (with the sign of zero and the
    subnormals), both infinities, and NaN patterns decoding to NaN."""
    u16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns
        got = odf.decode_bf16(u16)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "finite / infinite values differ"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "sign of zero differs"
    # hand-worked patterns: 1.0, -2.0, the smallest subnormal, the largest finite value
    hand = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,
            0x7F80: np.inf, 0xFF80: -np.inf}
    for bits, val in hand.items():
        assert odf.decode_bf16(np.array([bits], dtype=np.uint16))[0] == val, hex(bits)


def pin_layer_norm():
    """LayerNorm against torch.nn.functional.layer_norm (float64, gain only)."""
    r = _rng(2)
    x = r.standard_normal((7, 96)) * 3 + 1.5
    g = r.standard_normal(96)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), None, 1e-5).numpy()
    got = odf.layer_norm(x, g, 1e-5)
    assert np.max(np.abs(got - want)) < 1e-12


def pin_gelu():
    """Exact GELU against torch's erf GELU and its limits."""
    x = np.linspace(-8, 8, 1001)
    want = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(odf.gelu(x) - want)) < 1e-14
    assert odf.gelu(np.array([0.0]))[0] == 0.0
    assert abs(odf.gelu(np.array([30.0]))[0] - 30.0) < 1e-12


def pin_attention_sdpa():
    """One-query attention against torch scaled_dot_product_attention (float64)."""
    r = _rng(3)
    for n, Dh in [(1, 32), (5, 32), (37, 128), (200, 64)]:
        q = r.standard_normal(Dh)
        K = r.standard_normal((n, Dh))
        V = r.standard_normal((n, Dh))
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None]).numpy().reshape(Dh)
        o, _ = odf.attention_one(q, K, V)
        assert np.max(np.abs(o - want)) < 1e-12, (n, Dh)


def pin_attention_closed_forms():
    """len 1 gives V0 and lse = s0; equal keys give mean(V) and lse = s + log n;
    a zero query gives mean(V) and lse = log n."""
    r = _rng(4)
    Dh = 32
    q = r.standard_normal(Dh)
    K = r.standard_normal((1, Dh))
    V = r.standard_normal((1, Dh))
    o, lse = odf.attention_one(q, K, V)
    assert np.array_equal(o, V[0]) or np.max(np.abs(o - V[0])) < 1e-15
    assert abs(lse - float(q @ K[0]) / math.sqrt(Dh)) < 1e-12
    n = 17
    Ks = np.repeat(K, n, axis=0)
    Vs = r.standard_normal((n, Dh))
    o, lse = odf.attention_one(q, Ks, Vs)
    assert np.max(np.abs(o - Vs.mean(0))) < 1e-12
    assert abs(lse - (float(q @ K[0]) / math.sqrt(Dh) + math.log(n))) < 1e-12
    o, lse = odf.attention_one(np.zeros(Dh), r.standard_normal((n, Dh)), Vs)
    assert np.max(np.abs(o - Vs.mean(0))) < 1e-12 and abs(lse - math.log(n)) < 1e-12


def pin_attention_dual():
    """Dual-query attention: with a = -1 and Q2raw = Q1 the coupled aux query
    is exactly zero, so its output is the plain mean of the values and its lse
    is log(len); with a = 0 and Q2raw = Q1 both flows agree bitwise; the
    primary flow matches the library attention."""
    r = _rng(5)
    B, H, S, Dh = 3, 2, 40, 32
    K = r.standard_normal((B, H, S, Dh))
    V = r.standard_normal((B, H, S, Dh))
    lens = np.array([1, 23, 40])
    q1 = r.standard_normal((B, H, Dh))
    o, lse = odf.attention_dual(K, V, q1, q1.copy(), lens, a=-np.ones(H * Dh))
    for b in range(B):
        for h in range(H):
            assert np.max(np.abs(o[b, 1, h] - V[b, h, :lens[b]].mean(0))) < 1e-12
            assert abs(lse[b, 1, h] - math.log(lens[b])) < 1e-12
            want = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q1[b, h])[None, None, None], torch.from_numpy(K[b, h, :lens[b]])[None, None],
                torch.from_numpy(V[b, h, :lens[b]])[None, None]).numpy().reshape(Dh)
            assert np.max(np.abs(o[b, 0, h] - want)) < 1e-12
    o, lse = odf.attention_dual(K, V, q1, q1.copy(), lens, a=np.zeros(H * Dh))
    assert np.array_equal(o[:, 0], o[:, 1]) and np.array_equal(lse[:, 0], lse[:, 1])


def pin_mix_properties():
    """alpha in [0.5, 1], p_mix a distribution; one-hot primary gives alpha = 1
    and p_mix = p1; uniform primary gives alpha = 0.5."""
    r = _rng(6)
    for _ in range(20):
        V = int(r.integers(2, 3000))
        l1 = r.standard_normal(V) * r.uniform(0.1, 20)
        l2 = r.standard_normal(V) * r.uniform(0.1, 20)
        p, alpha, nt = odf.mix_head(l1, l2)
        assert 0.5 <= alpha <= 1.0
        assert abs(p.sum() - 1.0) < 1e-12 and np.all(p >= 0)
        assert nt == int(np.argmax(p))
    l1 = np.zeros(50)
    l1[7] = 1000.0
    p, alpha, nt = odf.mix_head(l1, r.standard_normal(50))
    assert alpha == 1.0 and nt == 7 and abs(p[7] - 1.0) < 1e-12
    p, alpha, _ = odf.mix_head(np.zeros(50), np.zeros(50))
    assert alpha == 0.5 and np.max(np.abs(p - 1.0 / 50)) < 1e-15
    p, alpha, nt = odf.mix_head(r.standard_normal(50), None)
    assert alpha == 1.0


def pin_mix_golden():
    """Hand-worked mixture cases (tests/golden/mix_crafted.json)."""
    d = json.load(open(os.path.join(GOLDEN, "mix_crafted.json")))
    for c in d["cases"]:
        p, alpha, nt = odf.mix_head(np.array(c["l1"]), np.array(c["l2"]))
        assert abs(alpha - c["alpha"]) < 1e-12, c["note"]
        assert np.max(np.abs(p - np.array(c["p_mix"]))) < 1e-12, c["note"]
        assert nt == c["next_tok"], c["note"]


def pin_topk():
    """top-k against a brute-force full sort keyed (-value, index), with ties."""
    r = _rng(7)
    for _ in range(200):
        E = int(r.integers(1, 70))
        k = int(r.integers(1, E + 1))
        vals = r.integers(-3, 4, E).astype(np.float64)       # many ties
        want = [i for _, i in sorted((-v, i) for i, v in enumerate(vals))][:k]
        assert list(odf.topk_ids(vals, k)) == want


# ----------------------------------------------------------------------------
# Structural invariants of the method
# ----------------------------------------------------------------------------

def _fresh(cfg, src=None):
    src = src or Inputs(cfg)
    return odf.Model(src), odf.Cache(cfg, list(range(cfg.B)), src)


def _two_steps(cfg, aux_on, src=None, override=True):
    m, cache = _fresh(cfg, src)
    outs = []
    for s in range(2):
        outs.append(odf.decode_step(m, cache, Inputs(cfg).step_tokens(s) % cfg.V, aux_on=aux_on,
                                    router_logits=_router(cfg, s) if override else None))
    return cache, outs


def _router(cfg, step):
    if not cfg.moe:
        return None
    src = Inputs(cfg)
    return np.stack([src.router_logits(step, l) for l in range(cfg.L)])


def pin_aux_onoff(cfg):
    """The primary flow is self-contained and only it writes the cache ([ES]
    Arquitectura Central): with the aux flow on or off, the primary logits and
    every cache entry are bitwise identical."""
    ca, ra = _two_steps(cfg, True)
    cb, rb = _two_steps(cfg, False)
    for x, y in zip(ra, rb):
        assert np.array_equal(x.logits[:, 0], y.logits[:, 0])
        if cfg.moe:
            assert np.array_equal(x.ids, y.ids)
    for l in range(cfg.L):
        ka, va = ca.layer(l)
        kb, vb = cb.layer(l)
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def pin_tied_zero_coupling(cfg):
    """With a = b = c = 0 and the aux embedding tied to the primary one, the
    aux flow repeats the primary flow exactly: aux logits equal primary logits
    bitwise and p_mix equals p_primary. (MoE: with the router computed from
    its weights; supplied primary router logits replace the primary's router
    output only, so they break the symmetry by construction.)"""
    c2 = cfg.replace(tie_emb=True, zero_cpl=True)
    _, outs = _two_steps(c2, True, override=False)
    for r in outs:
        assert np.array_equal(r.logits[:, 0], r.logits[:, 1])
        p1 = np.stack([odf.softmax(x) for x in r.logits[:, 0]])
        assert np.max(np.abs(r.p_mix - p1)) < 1e-15
        if cfg.moe:
            assert np.array_equal(r.gates[:, :, 0], r.gates[:, :, 1])


def pin_kv_sentinel(cfg):
    """A step writes exactly the entries (l, b, h, len_b) of the cache and
    nothing else, and advances every len_b by one."""
    m, cache = _fresh(cfg)
    S = 12345.0
    for l in range(cfg.L):
        K, V = cache.layer(l)
        K[:, :, cfg.ctx:] = S
        V[:, :, cfg.ctx:] = S
    before = [tuple(a.copy() for a in cache.layer(l)) for l in range(cfg.L)]
    lens0 = cache.lens.copy()
    odf.decode_step(m, cache, Inputs(cfg).step_tokens(0), aux_on=True, router_logits=_router(cfg, 0))
    assert np.array_equal(cache.lens, lens0 + 1)
    for l in range(cfg.L):
        for which in (0, 1):
            a0, a1 = before[l][which], cache.layer(l)[which]
            changed = np.any(a0 != a1, axis=-1)            # [B, H, S]
            want = np.zeros_like(changed)
            for b in range(cfg.B):
                want[b, :, lens0[b]] = True
            assert np.array_equal(changed, want)


def pin_prefill_equals_decode(cfg):
    """Prefill of a prompt (one batched causal pass) and the same prompt fed
    token by token through primary-only decode steps write the same cache and
    give the same last-position primary logits."""
    c = cfg.replace(ctx=0)
    src = Inputs(c)
    prompt = src.prompt()
    ma, ca = _fresh(c, src)
    logits = odf.prefill_primary(ma, ca, prompt)
    mb, cb = _fresh(c, src)
    for t in range(prompt.shape[1]):
        r = odf.decode_step(mb, cb, prompt[:, t], aux_on=False)
    ulp = 2.0 ** -7 if c.dtype == "bf16" else 2.0 ** -22
    for l in range(c.L):
        for x, y in zip(ca.layer(l), cb.layer(l)):
            assert np.all(np.abs(x - y) <= ulp * np.abs(x) + 1e-30)
    assert np.max(np.abs(logits[:, -1] - r.logits[:, 0])) < 1e-6
    assert np.array_equal(ca.lens, cb.lens)


def pin_causality(cfg):
    """Prefill is causal: changing the last prompt token changes no earlier
    position's logits."""
    c = cfg.replace(ctx=0)
    src = Inputs(c)
    prompt = src.prompt()
    p2 = prompt.copy()
    p2[:, -1] = (p2[:, -1] + 1) % c.V
    ma, ca = _fresh(c, src)
    la = odf.prefill_primary(ma, ca, prompt)
    mb, cb = _fresh(c, src)
    lb = odf.prefill_primary(mb, cb, p2)
    assert np.max(np.abs(la[:, :-1] - lb[:, :-1])) < 1e-12
    assert np.max(np.abs(la[:, -1] - lb[:, -1])) > 1e-6


def _traced(cfg, cpl):
    """One traced dual step with the coupling vectors given as constants."""
    base = Inputs(cfg)

    def coupling(which, l):
        n = cfg.ffn if which == "b" else cfg.d
        return np.full(n, cpl.get(which, 0.0), dtype=np.float32)

    src = ArraySource(base, coupling=coupling)
    m, cache = _fresh(cfg, src)
    return odf.decode_step(m, cache, base.step_tokens(0), aux_on=True, trace=True,
                           router_logits=_router(cfg, 0)), cache


def pin_query_coupling(cfg):
    """Query coupling closed forms with the aux embedding tied: a = -1 makes
    the aux query exactly zero, so its layer-0 attention output is the plain
    mean of the primary values at positions 0..len (including the entry just
    appended); a = 1 doubles the query exactly; and in layer 0 the aux query
    with a = 1 is the a = 0 aux query plus the primary query (superposition,
    untied embeddings)."""
    c = cfg.replace(tie_emb=True)
    r, cache = _traced(c, {"a": -1.0})
    q = r.trace["q.0"]                                  # [nb, 2, d]
    assert np.all(q[:, 1] == 0.0)
    K, V = cache.layer(0)
    for i in range(c.B):
        n = c.ctx + 1
        for h in range(c.H):
            want = V[i, h, :n].mean(0)
            got = r.trace["o.0"][i, 1, h * c.Dh:(h + 1) * c.Dh]
            assert np.max(np.abs(got - want)) < 1e-12
    r, _ = _traced(c, {"a": 1.0})
    q = r.trace["q.0"]
    assert np.array_equal(q[:, 1], 2.0 * q[:, 0])
    r0, _ = _traced(cfg, {"a": 0.0})
    r1, _ = _traced(cfg, {"a": 1.0})
    q0, q1 = r0.trace["q.0"], r1.trace["q.0"]
    assert np.array_equal(q1[:, 0], q0[:, 0])
    assert np.max(np.abs(q1[:, 1] - (q0[:, 1] + q0[:, 0]))) < 1e-13


def pin_mid_coupling(cfg):
    """MLP-intermediate coupling b: in layer 0 (everything before the MLP is
    independent of b) the aux intermediate with b = 1 equals the aux
    intermediate with b = 0 plus the primary intermediate; with the aux
    embedding tied and b = 1 the aux MLP output is exactly twice the primary
    one (b acts after the GELU, on the primary activation as computed)."""
    if cfg.moe:
        return
    r0, _ = _traced(cfg, {})
    r1, _ = _traced(cfg, {"b": 1.0})
    g0, g1 = r0.trace["mlp_g.0"], r1.trace["mlp_g.0"]
    assert np.array_equal(g1[:, 0], g0[:, 0])
    assert np.max(np.abs(g1[:, 1] - (g0[:, 1] + g0[:, 0]))) < 1e-13
    rt, _ = _traced(cfg.replace(tie_emb=True), {"b": 1.0})
    y = rt.trace["mlp_y.0"]
    assert np.array_equal(y[:, 1], 2.0 * y[:, 0])


def pin_out_coupling(cfg):
    """MLP-output coupling c: in layer 0 the aux MLP output with c = 1 is the
    c = 0 aux output plus the primary output; with the embedding tied and
    c = -1 the aux MLP output is exactly zero, so the aux residual after layer
    0 equals its value after attention."""
    key = "mlp_y.0"
    if cfg.moe:
        return
    r0, _ = _traced(cfg, {})
    r1, _ = _traced(cfg, {"c": 1.0})
    y0, y1 = r0.trace[key], r1.trace[key]
    assert np.array_equal(y1[:, 0], y0[:, 0])
    assert np.max(np.abs(y1[:, 1] - (y0[:, 1] + y0[:, 0]))) < 1e-13
    rt, _ = _traced(cfg.replace(tie_emb=True), {"c": -1.0})
    assert np.all(rt.trace[key][:, 1] == 0.0)
    assert np.array_equal(rt.trace["h.0"][:, 1], rt.trace["h_mid.0"][:, 1])


def pin_step_outputs(cfg):
    """Every step's alpha lies in [0.5, 1] and p_mix sums to 1."""
    _, outs = _two_steps(cfg, True)
    for r in outs:
        assert np.all(r.alpha >= 0.5) and np.all(r.alpha <= 1.0)
        assert np.max(np.abs(r.p_mix.sum(-1) - 1.0)) < 1e-12
        assert np.all(r.next_tok == np.argmax(r.p_mix, axis=-1))


# ----------------------------------------------------------------------------
# MoE with router replay
# ----------------------------------------------------------------------------

def pin_moe_single_expert_is_dense():
    """With one expert and top-1 routing every gate is exactly 1, so the MoE
    model equals the dense model with that expert's weights, bitwise."""
    moe = TINY_MOE.replace(E=1, top_k=1, Fe=96)
    dense = Config("pin_dense_eq", L=moe.L, d=moe.d, H=moe.H, Dh=moe.Dh, F=moe.Fe, V=moe.V, B=moe.B,
                   ctx=moe.ctx, S_max=moe.S_max, dtype=moe.dtype, seed=moe.seed, sigma_w=moe.sigma_w,
                   sigma_ln=moe.sigma_ln)
    bm = Inputs(moe)
    src_d = ArraySource(Inputs(dense), w_up=lambda l: bm.w_exp_up(l, 0), w_down=lambda l: bm.w_exp_down(l, 0),
                        coupling=bm.coupling, kv_block=bm.kv_block, tok_emb_rows=bm.tok_emb_rows,
                        pos_emb=bm.pos_emb, w_qkv=bm.w_qkv, w_o=bm.w_o, w_out=bm.w_out, ln_gain=bm.ln_gain)
    ma, ca = _fresh(moe, bm)
    mb, cb = _fresh(dense, src_d)
    tok = bm.step_tokens(0)
    ra = odf.decode_step(ma, ca, tok, aux_on=True)
    rb = odf.decode_step(mb, cb, tok, aux_on=True)
    assert np.array_equal(ra.logits, rb.logits)
    assert np.all(ra.ids == 0) and np.all(ra.gates == 1.0)


def pin_moe_all_experts_is_full_mixture():
    """With k = E the renormalised top-k gates are the full softmax, so each
    flow's MoE output is the softmax-weighted sum over all experts of that
    flow's own router logits (aux gates from aux logits, primary from primary);
    checked per flow by brute force over the experts, b = c = 0."""
    cfg = TINY_MOE.replace(top_k=TINY_MOE.E, zero_cpl=True)
    src = Inputs(cfg)
    m = odf.Model(src)
    p = m.layer(0)
    r = _rng(8)
    v = odf.round_to(r.standard_normal((2, cfg.d)), "bf16")
    y, ids, gates = odf._mlp_moe(p, v, 2, "bf16", cfg.E, None)
    assert sorted(ids.tolist()) == list(range(cfg.E))
    for f in range(2):
        logits = p["w_router"] @ v[f]
        w = np.exp(logits - logits.max())
        w /= w.sum()
        want = sum(w[e] * (p["w_edown"][e] @ odf.gelu(p["w_eup"][e] @ v[f])) for e in range(cfg.E))
        assert np.max(np.abs(y[f] - want)) < 1e-12


def pin_moe_replay():
    """Router replay: the aux flow uses the primary's expert ids (supplied
    tie-free primary logits decide them), its gates sum to one, and the
    selected ids are the top-k of the supplied logits."""
    cfg = TINY_MOE
    m, cache = _fresh(cfg)
    rl = _router(cfg, 0)
    r = odf.decode_step(m, cache, Inputs(cfg).step_tokens(0), aux_on=True, router_logits=rl)
    for l in range(cfg.L):
        for i in range(cfg.B):
            assert list(r.ids[l, i]) == list(odf.topk_ids(rl[l, i], cfg.top_k))
            assert abs(r.gates[l, i, 0].sum() - 1) < 1e-12 and abs(r.gates[l, i, 1].sum() - 1) < 1e-12


# ----------------------------------------------------------------------------
# Ablation switches and independent aux expert fan-out
# ----------------------------------------------------------------------------

def pin_mix_aux_mode():
    """No mixture ([ES] Resultados, minimal Dual): p_mix is the aux
    distribution itself: alpha = 0, ratios p[i] / p[j] = exp(l2[i] - l2[j])
    (brute force on small vocabularies), a distribution, argmax of l2."""
    r = _rng(21)
    for _ in range(20):
        V = int(r.integers(2, 40))
        l1, l2 = r.standard_normal(V) * 3, r.standard_normal(V) * 3
        p, alpha, nt = odf.mix_head(l1, l2, odf.MIX_AUX)
        assert alpha == 0.0 and abs(p.sum() - 1.0) < 1e-12
        for i in range(V):
            for j in range(V):
                assert abs(p[i] / p[j] - math.exp(l2[i] - l2[j])) < 1e-9 * math.exp(abs(l2[i] - l2[j]))
        assert nt == int(np.argmax(l2))


def pin_mix_half_mode():
    """The other reading of the floor, alpha = (1 + CP) / 2: in [0.5, 1];
    uniform primary gives (1 + 1/V) / 2 exactly; one-hot primary gives 1; a
    two-token primary p1 = (0.9, 0.1) (logits ln 9, 0) gives CP = 0.82,
    alpha = 0.91, and p_mix = 0.91 p1 + 0.09 p2 by hand."""
    r = _rng(22)
    for _ in range(20):
        V = int(r.integers(2, 3000))
        p, alpha, _ = odf.mix_head(r.standard_normal(V) * 5, r.standard_normal(V), odf.MIX_HALF)
        assert 0.5 <= alpha <= 1.0 and abs(p.sum() - 1.0) < 1e-12
    p, alpha, _ = odf.mix_head(np.zeros(40), r.standard_normal(40), odf.MIX_HALF)
    assert abs(alpha - 0.5 * (1 + 1 / 40)) < 1e-15
    l1 = np.zeros(30)
    l1[3] = 1000.0
    assert odf.mix_head(l1, np.zeros(30), odf.MIX_HALF)[1] == 1.0
    p, alpha, nt = odf.mix_head(np.array([math.log(9.0), 0.0]), np.array([0.0, 0.0]), odf.MIX_HALF)
    assert abs(alpha - 0.91) < 1e-12
    assert np.max(np.abs(p - np.array([0.91 * 0.9 + 0.09 * 0.5, 0.91 * 0.1 + 0.09 * 0.5]))) < 1e-12 and nt == 0


def pin_no_coupling_tied(cfg):
    """Couplings off ([ES] Resultados, minimal Dual): with the aux embedding
    tied to the primary one the aux flow repeats the primary exactly, however
    large a, b, c are (sigma 0.5 here), bitwise; and the switch equals zero
    coupling vectors, bitwise, with untied embeddings."""
    c1 = cfg.replace(tie_emb=True, variant=1, sigma_cpl=0.5)
    _, outs = _two_steps(c1, True, override=False)
    for r in outs:
        assert np.array_equal(r.logits[:, 0], r.logits[:, 1])
    _, oa = _two_steps(cfg.replace(variant=1), True)
    _, ob = _two_steps(cfg.replace(zero_cpl=True), True)
    for x, y in zip(oa, ob):
        assert np.array_equal(x.logits, y.logits) and np.array_equal(x.p_mix, y.p_mix)


def pin_variant_mix_in_step(cfg):
    """The mixture switches act on the step's output only: with variant "aux
    output" p_mix = softmax(aux logits) and alpha = 0; with "alpha half"
    alpha = (1 + CP) / 2 from the step's primary logits; logits are the same
    as the default variant's, bitwise."""
    _, base = _two_steps(cfg, True)
    _, aux = _two_steps(cfg.replace(variant=2), True)
    _, half = _two_steps(cfg.replace(variant=4), True)
    for r0, ra, rh in zip(base, aux, half):
        assert np.array_equal(r0.logits, ra.logits) and np.array_equal(r0.logits, rh.logits)
        for i in range(cfg.B):
            assert ra.alpha[i] == 0.0
            assert np.max(np.abs(ra.p_mix[i] - odf.softmax(ra.logits[i, 1]))) < 1e-15
            p1 = odf.softmax(rh.logits[i, 0])
            assert abs(rh.alpha[i] - 0.5 * (1 + np.sum(p1 * p1))) < 1e-15


def pin_fanout_replay_and_primary():
    """Independent fan-outs ([ES] Contribuciones Clave 3): k_aux = k is plain
    replay (bitwise); any k_aux leaves the primary logits, the cache and the
    primary ids unchanged (bitwise), and the reported ids are the primary's
    ranking (top-max(k, k_aux) of its logits, ties to the lower id)."""
    cfg = TINY_MOE
    _, o0 = _two_steps(cfg, True)
    _, ok = _two_steps(cfg.replace(top_k_aux=cfg.top_k), True)
    for x, y in zip(o0, ok):
        assert np.array_equal(x.logits, y.logits) and np.array_equal(x.ids, y.ids)
    for ka in (1, 3, cfg.E):
        c2 = cfg.replace(top_k_aux=ka)
        ca, oa = _two_steps(c2, True)
        cb, ob = _two_steps(cfg, True)
        for s, (x, y) in enumerate(zip(oa, ob)):
            assert np.array_equal(x.logits[:, 0], y.logits[:, 0])
            assert np.array_equal(x.ids[:, :, :cfg.top_k], y.ids)
            rl = _router(cfg, s)
            for l in range(cfg.L):
                for i in range(cfg.B):
                    assert list(x.ids[l, i]) == list(odf.topk_ids(rl[l, i], max(cfg.top_k, ka)))
        for l in range(cfg.L):
            assert all(np.array_equal(a, b) for a, b in zip(ca.layer(l), cb.layer(l)))


def pin_fanout_closed_forms():
    """k_aux = E with b = c = 0: the aux MoE output is the full softmax mixture
    of the aux router over all experts; k_aux = 1: the aux uses the primary's
    top expert alone (gate 1) with the b coupling (that expert is the
    primary's too); the primary output is the top-k mixture either way.
    Brute force per expert."""
    cfg = TINY_MOE.replace(zero_cpl=True)
    m = odf.Model(Inputs(cfg))
    p = m.layer(1)
    r = _rng(23)
    v = odf.round_to(r.standard_normal((2, cfg.d)), "bf16")
    expert = lambda e, x: p["w_edown"][e] @ odf.gelu(p["w_eup"][e] @ x)
    y, ranking, gates = odf._mlp_moe(p, v, 2, "bf16", cfg.top_k, None, k_aux=cfg.E)
    l2 = p["w_router"] @ v[1]
    w = np.exp(l2 - l2.max())
    w /= w.sum()
    assert np.max(np.abs(y[1] - sum(w[e] * expert(e, v[1]) for e in range(cfg.E)))) < 1e-12
    l1 = p["w_router"] @ v[0]
    top = odf.topk_ids(l1, cfg.top_k)
    w1 = np.exp(l1[top] - l1[top].max())
    w1 /= w1.sum()
    assert np.max(np.abs(y[0] - sum(w1[j] * expert(e, v[0]) for j, e in enumerate(top)))) < 1e-12
    cb = TINY_MOE
    mb = odf.Model(Inputs(cb))
    pb = mb.layer(0)
    y, ranking, gates = odf._mlp_moe(pb, v, 2, "bf16", cb.top_k, None, k_aux=1)
    e = int(ranking[0])
    g1 = odf.gelu(pb["w_eup"][e] @ v[0])
    g2 = odf.gelu(pb["w_eup"][e] @ v[1]) + pb["b"] * g1
    l1 = pb["w_router"] @ v[0]
    top = odf.topk_ids(l1, cb.top_k)
    w1 = np.exp(l1[top] - l1[top].max())
    w1 /= w1.sum()
    y1 = sum(w1[j] * (pb["w_edown"][ee] @ odf.gelu(pb["w_eup"][ee] @ v[0])) for j, ee in enumerate(top))
    assert np.max(np.abs(y[1] - (pb["w_edown"][e] @ g2 + pb["c"] * y1))) < 1e-12
    assert gates[1, 0] == 1.0 and np.all(gates[1, 1:] == 0.0)
    # k_aux = E with b, c != 0: b couples only the ranks the primary also ran
    y, ranking, gates = odf._mlp_moe(pb, v, 2, "bf16", cb.top_k, None, k_aux=cb.E)
    l2 = pb["w_router"] @ v[1]
    w2 = np.exp(l2[ranking] - l2[ranking].max())
    w2 /= w2.sum()
    want = pb["c"] * y1
    for j, ee in enumerate(ranking):
        g2 = odf.gelu(pb["w_eup"][ee] @ v[1])
        if j < cb.top_k:
            g2 = g2 + pb["b"] * odf.gelu(pb["w_eup"][ee] @ v[0])
        want = want + w2[j] * (pb["w_edown"][ee] @ g2)
    assert np.max(np.abs(y[1] - want)) < 1e-12


def _forward_vs_steps(cfg, T):
    """forward_dual over T tokens and T teacher-forced dual decode steps
    from the same cache: results and caches (oracle, both)."""
    src = Inputs(cfg)
    toks = np.stack([src.step_tokens(s) for s in range(T)], axis=1)      # [B, T]
    ma, ca = _fresh(cfg, src)
    fw = odf.forward_dual(ma, ca, toks)
    mb, cb = _fresh(cfg, src)
    steps = [odf.decode_step(mb, cb, toks[:, t], aux_on=True) for t in range(T)]
    return fw, ca, steps, cb


def pin_forward_equals_steps(cfg):
    """The full-sequence dual forward is the run of teacher-forced dual decode
    steps over the same tokens (the aux state at a position depends on
    earlier positions only through the primary K/V): logits, p_mix, alpha
    and next tokens of every position agree, and so do the caches. Covered
    for the full method and the ablation switches (couplings off, aux
    output, alpha = (1 + CP) / 2) and, in MoE models, the aux fan-out."""
    variants = [cfg] + [cfg.replace(variant=v) for v in (1, 2, 4)]
    if cfg.moe:
        variants.append(cfg.replace(top_k_aux=cfg.E))
    for c in variants:
        T = 4
        fw, ca, steps, cb = _forward_vs_steps(c, T)
        for t, r in enumerate(steps):
            assert np.max(np.abs(fw.logits[:, t] - r.logits)) < 1e-9
            assert np.max(np.abs(fw.p_mix[:, t] - r.p_mix)) < 1e-12
            assert np.max(np.abs(fw.alpha[:, t] - r.alpha)) < 1e-12
            assert np.array_equal(fw.next_tok[:, t], r.next_tok)
        ulp = 2.0 ** -7 if c.dtype == "bf16" else 2.0 ** -22
        for l in range(c.L):
            for x, y in zip(ca.layer(l), cb.layer(l)):
                assert np.all(np.abs(x - y) <= ulp * np.abs(x) + 1e-30)
        assert np.array_equal(ca.lens, cb.lens)


def pin_forward_primary_is_prefill(cfg):
    """The primary half of the dual forward is the prefill: the same primary
    logits at every position and the same cache (the aux flow never feeds
    back, [ES] Arquitectura Central)."""
    c = cfg.replace(ctx=0)
    src = Inputs(c)
    prompt = src.prompt()
    ma, ca = _fresh(c, src)
    fw = odf.forward_dual(ma, ca, prompt)
    mb, cb = _fresh(c, src)
    lp = odf.prefill_primary(mb, cb, prompt)
    assert np.max(np.abs(fw.logits[:, :, 0] - lp)) < 1e-9
    for l in range(c.L):
        for x, y in zip(ca.layer(l), cb.layer(l)):
            assert np.array_equal(x, y)


def pin_forward_causal(cfg):
    """Both flows of the forward are causal: changing the last token changes
    no earlier position's logits in either flow, and changes the last
    position's."""
    c = cfg.replace(ctx=0)
    src = Inputs(c)
    prompt = src.prompt()
    p2 = prompt.copy()
    p2[:, -1] = (p2[:, -1] + 1) % c.V
    ma, ca = _fresh(c, src)
    a = odf.forward_dual(ma, ca, prompt)
    mb, cb = _fresh(c, src)
    b = odf.forward_dual(mb, cb, p2)
    assert np.max(np.abs(a.logits[:, :-1] - b.logits[:, :-1])) < 1e-12
    assert np.min(np.max(np.abs(a.logits[:, -1] - b.logits[:, -1]), axis=-1)) > 1e-6



def pin_run_tiny_schedule(cfg):
    """The end-to-end run's schedule ([ES] Arquitectura Central: the aux flow
    is skipped in prefill and active from the last prompt position on): the
    primary prefill covers positions 0..T-2, step 0 consumes the last prompt
    token at position T-1 with the aux flow on, step s > 0 consumes the token
    step s-1 chose, and len ends at T-1+n with exactly positions 0..T-2+n
    written. Checked against the full-sequence forward over the consumed
    tokens: its position T-1+s holds both flows' logits, since the aux state
    at a position depends on earlier positions only through the primary K/V."""
    n = 3
    c = cfg.replace(ctx=0, n_steps=n)
    src = Inputs(c)
    prompt = src.prompt()
    T = prompt.shape[1]
    cache, res = odf.run_tiny(odf.Model(src))
    assert len(res) == n
    assert np.array_equal(cache.lens, np.full(c.B, T - 1 + n))
    for l in range(c.L):
        for b in range(c.B):
            written = sorted(pos for (ll, bb, pos) in cache.appended if ll == l and bb == b)
            assert written == list(range(T - 1 + n)), (l, b, written)
    seq = np.concatenate([prompt] + [r.next_tok[:, None] for r in res[:-1]], axis=1)
    mf, cf = _fresh(c, src)
    fw = odf.forward_dual(mf, cf, seq)
    for s_, r in enumerate(res):
        t = T - 1 + s_
        assert np.max(np.abs(r.logits[:, 1])) > 0, "aux flow not active"
        assert np.max(np.abs(fw.logits[:, t] - r.logits)) < 1e-9, f"step {s_} is not position {t}"
        assert np.max(np.abs(fw.p_mix[:, t] - r.p_mix)) < 1e-12
        assert np.array_equal(fw.next_tok[:, t], r.next_tok)


# ----------------------------------------------------------------------------
# Where rounding may sit: appended K/V entries only (no rounded projection inputs)
# ----------------------------------------------------------------------------

# The 24-layer, d 2048 dense model of the 1.3B workload, one sequence, a short
# prefilled context; and a small 8-layer model for the quick check.
R16_FULL_DEPTH = Config("r16_dense_1p3b", L=24, d=2048, H=16, Dh=128, F=8192, V=32000, B=1, ctx=16, S_max=32,
                        dtype="bf16", seed=4)
R16_SMALL = Config("r16_small", L=8, d=512, H=4, Dh=128, F=2048, V=4096, B=2, ctx=16, S_max=32,
                   dtype="bf16", seed=4)
R16_NOISE = 2.0 ** -20      # relative, about the fp32 rounding-order difference of a K = 2048 sum


def step_logits_under_noise(cfg, round_inputs: bool, noise: float, seed: int = 1):
    """Logits of one dual step when every projection input is multiplied by
    (1 +- noise) (seeded signs) and, with round_inputs, then rounded to bf16
    (the reading that rounds every projection input). The noise stands for a
    different but equally correct fp32 summation order."""
    orig = odf._matvec
    rng = np.random.default_rng(seed)

    def mv(W, x):
        x = np.asarray(x, dtype=np.float64)
        if noise:
            x = x * (1.0 + noise * rng.choice([-1.0, 1.0], size=x.shape))
        if round_inputs:
            x = odf.round_to(x, "bf16")
        return orig(W, x)

    odf._matvec = mv
    try:
        src = Inputs(cfg)
        m, cache = _fresh(cfg, src)
        return odf.decode_step(m, cache, src.step_tokens(0), aux_on=True).logits
    finally:
        odf._matvec = orig


def pin_unrounded_inputs_are_stable(cfg=R16_SMALL):
    """With activations unrounded (only the appended K/V rounded), noise of
    2^-20 relative on every projection input moves the logits by less than
    1e-3, twenty times below the 2e-2 logits bar."""
    a = step_logits_under_noise(cfg, False, 0.0)
    b = step_logits_under_noise(cfg, False, R16_NOISE)
    move = float(np.max(np.abs(a - b)))
    assert move < 1e-3, f"unrounded oracle moved {move:.3e}"
    return move


ALL_BASIC = [pin_round_bf16, pin_decode_bf16, pin_layer_norm, pin_gelu, pin_attention_sdpa,
             pin_attention_closed_forms, pin_attention_dual, pin_mix_properties, pin_mix_golden, pin_topk,
             pin_mix_aux_mode, pin_mix_half_mode, pin_unrounded_inputs_are_stable]
MODEL_PINS = [pin_aux_onoff, pin_tied_zero_coupling, pin_kv_sentinel, pin_prefill_equals_decode,
              pin_causality, pin_query_coupling, pin_mid_coupling, pin_out_coupling, pin_step_outputs]
MOE_PINS = [pin_moe_single_expert_is_dense, pin_moe_all_experts_is_full_mixture, pin_moe_replay,
            pin_fanout_replay_and_primary, pin_fanout_closed_forms]
VARIANT_PINS = [pin_no_coupling_tied, pin_variant_mix_in_step]
FORWARD_PINS = [pin_forward_equals_steps, pin_forward_primary_is_prefill, pin_forward_causal,
                pin_run_tiny_schedule]
