"""The grouped decode step on the GPU (df_decode_step, df_prefill_primary)
against the oracle, teacher-forced on the same tokens.

Bars (fp32 accumulation on the GPU, float64 in the oracle): logits within
2e-2 max-abs, p_mix within 1e-3 max-abs; K/V write positions bit-exact
(sentinel-filled cache); appended bf16 values within one bf16 ulp; MoE
expert ids bit-exact. Invariants the pages state hold bitwise on the GPU:
the primary flow and the cache do not depend on the aux flow; with a = b =
c = 0 and tied embeddings the aux flow equals the primary flow."""
import numpy as np
import pytest
import torch

from dual_flow_transformer_amd.runtime import DecodeModel
from gpu_util import argmax_agrees, bits_to_f64, max_abs, say
from oracle import dualflow as odf
from synth.workloads import C1_TINY, Config, Inputs

pytestmark = pytest.mark.gpu

SMALL_BF16 = Config("gpu_small_bf16", L=2, d=256, H=2, Dh=128, F=1024, V=512, B=3, ctx=300, S_max=320,
                    dtype="bf16", seed=21, sigma_w=0.05, sigma_ln=0.1)
# d 768: the Q/K/V projection splits K into 3 slices, a count the attention
# pass's slice sums take in a ragged batch
SMALL_BF16_S3 = Config("gpu_small_bf16_s3", L=2, d=768, H=6, Dh=128, F=1536, V=512, B=3, ctx=200, S_max=224,
                       dtype="bf16", seed=24, sigma_w=0.05, sigma_ln=0.1)
# d 2304 with 36 sequences (72 stacked rows): the Q/K/V projection splits K
# into 9 slices of 256, more than the attention pass's slice sums take in
# one round of loads (8), so they take a second round
BF16_S9 = Config("gpu_bf16_s9_b36", L=1, d=2304, H=18, Dh=128, F=9216, V=512, B=36, ctx=40, S_max=64,
                 dtype="bf16", seed=25, sigma_w=0.02, sigma_ln=0.1)
# a context of 65,536 positions: the fused attention pass (Q/K/V slice sums,
# the new key at the end of a long segment) at large key indices
LONG_CTX = Config("gpu_long_ctx", L=2, d=256, H=2, Dh=128, F=1024, V=512, B=3, ctx=65536, S_max=65544,
                  dtype="bf16", seed=26, sigma_w=0.05, sigma_ln=0.1)
SMALL_F32 = Config("gpu_small_f32", L=2, d=128, H=2, Dh=64, F=256, V=300, B=2, ctx=40, S_max=64,
                   dtype="f32", seed=22, sigma_w=0.05, sigma_ln=0.1)
SMALL_MOE = Config("gpu_small_moe", L=2, d=256, H=2, Dh=128, F=0, V=512, B=8, ctx=40, S_max=64, dtype="bf16",
                   moe=True, E=16, top_k=4, Fe=256, router_override=True, seed=23, sigma_w=0.05, sigma_ln=0.1)
LOGIT_TOL, PMIX_TOL = 2e-2, 1e-3
KV_ABS = 5e-4      # fp32 projection error feeding an appended K/V entry (see test_gpu_fullsize)


def _compare_step(cfg, gm: DecodeModel, r: odf.StepResult, aux_on=True):
    lg = gm.logits.cpu().numpy()
    pm = gm.p_mix.cpu().numpy()
    al = gm.alpha.cpu().numpy()
    nt = gm.next_tok.cpu().numpy()
    flows = 2 if aux_on else 1
    el = max_abs(lg[:, :flows], r.logits[:, :flows])
    ep = max_abs(pm, r.p_mix)
    ea = max_abs(al, r.alpha)
    kl = float(np.max(np.sum(r.p_mix * (np.log(np.maximum(r.p_mix, 1e-30)) - np.log(np.maximum(pm, 1e-30))), -1)))
    say(f"  logits max|d|={el:.3e} p_mix max|d|={ep:.3e} alpha max|d|={ea:.3e} KL={kl:.2e}")
    assert el < LOGIT_TOL and ep < PMIX_TOL and ea < PMIX_TOL
    for b in range(cfg.B):
        assert argmax_agrees(pm[b], r.p_mix[b], nt[b], margin=2e-3)
    return el, ep


def _sentinel(gm: DecodeModel, cfg):
    s = 0x4242 if cfg.dtype == "bf16" else 12345.0
    gm.k[:, :, :, cfg.ctx:] = s
    gm.v[:, :, :, cfg.ctx:] = s
    return s


def _check_writes(gm, cfg, lens0, cache: odf.Cache, sentinel):
    for name, t in (("k", gm.k), ("v", gm.v)):
        a = t.cpu().numpy()
        sv = np.int16(sentinel) if cfg.dtype == "bf16" else np.float32(sentinel)
        changed = np.any(a[:, :, :, cfg.ctx:] != sv, axis=-1)
        want = np.zeros_like(changed)
        for b in range(cfg.B):
            want[:, b, :, lens0[b] - cfg.ctx] = True
        assert np.array_equal(changed, want), f"{name} cache write positions differ"
        for l in range(cfg.L):
            for b in range(cfg.B):
                got = bits_to_f64(t[l, b, :, lens0[b]], cfg.dtype)
                ref = cache.appended[(l, b, int(lens0[b]))][0 if name == "k" else 1]
                ulp = 2.0 ** -7 if cfg.dtype == "bf16" else 2.0 ** -20
                assert np.all(np.abs(got - ref) <= ulp * np.abs(ref) + KV_ABS), f"{name} values l={l} b={b}"


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_BF16_S3, BF16_S9, SMALL_F32], ids=lambda c: c.name)
def test_small_dense_steps(cfg):
    say(f"decode case {cfg.name}")
    gm = DecodeModel(cfg, fill="host")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    s = _sentinel(gm, cfg)
    for step in range(2):
        lens0 = gm.len.cpu().numpy().copy()
        tok = src.step_tokens(step)
        gm.decode_step(gm.tokens(tok))
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True)
        say(f" step {step}")
        _compare_step(cfg, gm, r)
        if step == 0:
            _check_writes(gm, cfg, lens0, cache, s)
    assert np.array_equal(gm.len.cpu().numpy(), cache.lens)
    assert gm.status() == 0


def test_long_context_steps():
    """Two dual steps of a small model at a 65,536-position context (the
    prefilled cache from the device generator), against the oracle on every
    sequence, with the appended K/V checked at position len."""
    cfg = LONG_CTX
    say(f"decode case {cfg.name}")
    gm = DecodeModel(cfg, fill="device")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src, lazy=True)
    s = _sentinel(gm, cfg)
    for step in range(2):
        lens0 = gm.len.cpu().numpy().copy()
        tok = src.step_tokens(step)
        gm.decode_step(gm.tokens(tok))
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True)
        say(f" step {step}")
        _compare_step(cfg, gm, r)
        if step == 0:
            _check_writes(gm, cfg, lens0, cache, s)
    assert np.array_equal(gm.len.cpu().numpy(), cache.lens)
    assert gm.status() == 0


def test_device_fill_matches_host_generator():
    for cfg in (SMALL_BF16, SMALL_MOE, SMALL_F32):
        say(f"fill check {cfg.name}")
        a = DecodeModel(cfg, fill="device")
        b = DecodeModel(cfg, fill="host")
        for name in ("tok_emb", "pos_emb", "w_qkv", "w_o", "w_up", "w_down", "w_router", "w_eup", "w_edown",
                     "w_out", "k", "v"):
            x, y = getattr(a, name), getattr(b, name)
            if x is None:
                continue
            if isinstance(x, list):
                assert all(torch.equal(p, q) for p, q in zip(x, y)), name
            else:
                assert torch.equal(x, y), name


def test_tiny_fp32_end_to_end():
    """Prefill 62 prompt tokens (primary only), then 16 dual steps from the
    last prompt position, teacher-forced on the oracle's greedy tokens."""
    cfg = C1_TINY
    say("tiny end-to-end")
    m = odf.Model(Inputs(cfg))
    cache, res = odf.run_tiny(m)
    prompt = Inputs(cfg).prompt()
    gm = DecodeModel(cfg, fill="host")
    gm.len.zero_()
    gm.prefill(gm.tokens(prompt[:, :-1]).contiguous())
    tok = prompt[:, -1]
    for s, r in enumerate(res):
        gm.decode_step(gm.tokens(tok))
        torch.cuda.synchronize()
        say(f" step {s}")
        _compare_step(cfg, gm, r)
        tok = r.next_tok
    assert int(gm.len[0].item()) == cfg.prompt_len + cfg.n_steps - 1
    # the whole cache (prefill and decode entries)
    n = int(cache.lens[0])
    for l in range(cfg.L):
        K, V = cache.layer(l)
        assert max_abs(gm.k[l, :, :, :n].cpu().numpy(), K[:, :, :n]) < 1e-4
        assert max_abs(gm.v[l, :, :, :n].cpu().numpy(), V[:, :, :n]) < 1e-4


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_F32], ids=lambda c: c.name)
def test_cache_edge_positions(cfg):
    """New key in the last cache slot, a full cache and a short sequence in one
    step: the last slot is written, the full sequence's cache is untouched and
    flagged in the status word (bit 0), the short one writes at its length."""
    say(f"cache edges {cfg.name}")
    gm = DecodeModel(cfg, fill="device")
    S = gm.S
    lens = [S - 1, S, 5] + [7] * (cfg.B - 3)
    lens = lens[:cfg.B]
    gm.len.copy_(torch.tensor(lens, dtype=torch.int32))
    k0, v0 = gm.k.clone(), gm.v.clone()
    gm.decode_step(gm.tokens(Inputs(cfg).step_tokens(0)))
    torch.cuda.synchronize()
    assert gm.status() & 1
    assert torch.isfinite(gm.logits).all() and torch.isfinite(gm.p_mix).all()
    for name, t, t0 in (("k", gm.k, k0), ("v", gm.v, v0)):
        changed = (t != t0).any(dim=-1).cpu().numpy()          # [L, B, H, S]
        want = np.zeros_like(changed)
        for b, n in enumerate(lens):
            if 0 <= n < S:
                want[:, b, :, n] = True
        assert np.array_equal(changed, want), f"{name}: cache rows written {np.argwhere(changed != want)[:4]}"
    assert gm.status() == 0          # reading the status word clears it


# Batch sizes whose dual step stacks more rows than a primary-only step
# would plan alone (24 and 64 sequences: 48 / 128 stacked rows against 24 /
# 64), at the d 2048 shapes of the dense 1.3B and MoE workloads, two layers.
DENSE_B24 = Config("gpu_dense_d2048_b24", L=2, d=2048, H=16, Dh=128, F=8192, V=512, B=24, ctx=64, S_max=80,
                   dtype="bf16", seed=26, sigma_w=0.02, sigma_ln=0.1)
DENSE_B64 = DENSE_B24.replace(name="gpu_dense_d2048_b64", B=64)
MOE_B24 = Config("gpu_moe_d2048_e64_b24", L=2, d=2048, H=16, Dh=128, F=0, V=512, B=24, ctx=64, S_max=80,
                 dtype="bf16", moe=True, E=64, top_k=4, Fe=1024, router_override=True, seed=27, sigma_w=0.02,
                 sigma_ln=0.1)
MOE_B64 = MOE_B24.replace(name="gpu_moe_d2048_e64_b64", B=64)


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_MOE, DENSE_B24, DENSE_B64, MOE_B24, MOE_B64],
                         ids=lambda c: c.name)
def test_primary_independent_of_aux(cfg):
    """Primary logits and every cache byte are bitwise the same with the aux
    flow on or off (the aux flow never feeds back and never writes K/V)."""
    say(f"aux on/off {cfg.name}")
    src = Inputs(cfg)
    a = DecodeModel(cfg, fill="device")
    b = DecodeModel(cfg, fill="device")
    for step in range(2):
        tok = src.step_tokens(step)
        rl = a.router_logits(step) if cfg.moe else None
        a.decode_step(a.tokens(tok), aux_on=True, router_logits=rl)
        b.decode_step(b.tokens(tok), aux_on=False, router_logits=rl)
        torch.cuda.synchronize()
        assert torch.equal(a.logits[:, 0], b.logits[:, 0])
        if cfg.moe:
            assert torch.equal(a.expert_ids, b.expert_ids)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert torch.equal(b.alpha, torch.ones_like(b.alpha))


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_MOE], ids=lambda c: c.name)
def test_tied_zero_coupling_aux_equals_primary(cfg):
    say(f"tied + zero coupling {cfg.name}")
    c = cfg.replace(tie_emb=True, zero_cpl=True)
    gm = DecodeModel(c, fill="device")
    gm.decode_step(gm.tokens(Inputs(c).step_tokens(0)), aux_on=True, router_logits=None)
    torch.cuda.synchronize()
    assert torch.equal(gm.logits[:, 0], gm.logits[:, 1])


def test_deterministic():
    cfg = SMALL_BF16
    outs = []
    for _ in range(2):
        gm = DecodeModel(cfg, fill="device")
        gm.decode_step(gm.tokens(Inputs(cfg).step_tokens(0)))
        torch.cuda.synchronize()
        outs.append((gm.logits.clone(), gm.p_mix.clone(), gm.k.clone()))
    assert all(torch.equal(x, y) for x, y in zip(*outs))


def test_small_moe_router_replay():
    cfg = SMALL_MOE
    say("moe small")
    gm = DecodeModel(cfg, fill="host")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    for step in range(2):
        tok = src.step_tokens(step)
        rl = gm.router_logits(step)
        gm.decode_step(gm.tokens(tok), router_logits=rl)
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True, router_logits=rl.cpu().numpy())
        assert np.array_equal(gm.expert_ids.cpu().numpy(), r.ids), "expert ids differ"
        _compare_step(cfg, gm, r)


# Ablation switches and independent aux expert fan-out ([ES] Resultados;
# Contribuciones Clave 3): GPU against the oracle, two steps each.
@pytest.mark.parametrize("variant", [1, 2, 4, 3], ids=["no_coupling", "aux_output", "alpha_half", "minimal_dual"])
def test_variants_dense(variant):
    cfg = SMALL_BF16.replace(variant=variant)
    say(f"variant {variant} dense")
    gm = DecodeModel(cfg, fill="device")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    for step in range(2):
        tok = src.step_tokens(step)
        gm.decode_step(gm.tokens(tok))
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True)
        _compare_step(cfg, gm, r)
        if variant & 2:
            assert torch.equal(gm.alpha, torch.zeros_like(gm.alpha))


def test_no_coupling_tied_aux_equals_primary():
    """Couplings off with tied embeddings: aux = primary bitwise on the GPU too,
    with nonzero coupling vectors present."""
    cfg = SMALL_BF16.replace(variant=1, tie_emb=True, sigma_cpl=0.5)
    gm = DecodeModel(cfg, fill="device")
    gm.decode_step(gm.tokens(Inputs(cfg).step_tokens(0)))
    torch.cuda.synchronize()
    assert torch.equal(gm.logits[:, 0], gm.logits[:, 1])


@pytest.mark.parametrize("ka,variant", [(8, 0), (1, 0), (16, 0), (8, 1)], ids=["ka8", "ka1", "ka16", "ka8_nocpl"])
def test_moe_aux_fanout(ka, variant):
    """The aux flow takes the first ka experts of the primary ranking: logits,
    p_mix and the reported ranking against the oracle (ranking bit-exact)."""
    cfg = SMALL_MOE.replace(top_k_aux=ka, variant=variant)
    say(f"moe aux fan-out ka={ka} variant={variant}")
    gm = DecodeModel(cfg, fill="host")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    for step in range(2):
        tok = src.step_tokens(step)
        rl = gm.router_logits(step)
        gm.decode_step(gm.tokens(tok), router_logits=rl)
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True, router_logits=rl.cpu().numpy())
        assert np.array_equal(gm.expert_ids.cpu().numpy(), r.ids), "expert ranking differs"
        _compare_step(cfg, gm, r)


@pytest.mark.parametrize("base", [SMALL_MOE, MOE_B24, MOE_B64], ids=lambda c: c.name)
def test_moe_aux_fanout_leaves_primary_bitwise(base):
    """Whatever the aux fan-out, the primary logits and the cache are bitwise
    those of a primary-only step."""
    cfg = base.replace(top_k_aux=12)
    say(f"moe fan-out 12 on/off {cfg.name}")
    src = Inputs(cfg)
    a = DecodeModel(cfg, fill="device")
    b = DecodeModel(cfg, fill="device")
    for step in range(2):
        tok = src.step_tokens(step)
        rl = a.router_logits(step)
        a.decode_step(a.tokens(tok), aux_on=True, router_logits=rl)
        b.decode_step(b.tokens(tok), aux_on=False, router_logits=rl)
        torch.cuda.synchronize()
        assert torch.equal(a.logits[:, 0], b.logits[:, 0])
        assert torch.equal(a.expert_ids, b.expert_ids)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)


def test_moe_computed_router_matches_oracle():
    """Primary router logits computed from the router weights (none supplied):
    the ranking bit-exact against the oracle and the outputs within the bars.
    Precondition checked on the oracle: its ranked primary logits (the kr
    chosen and the next one) are at least 1e-4 apart, far above the fp32
    error of the GPU's router products, so both sides must rank alike."""
    cfg = SMALL_MOE.replace(name="gpu_moe_router_computed", top_k_aux=6)
    say("moe computed router")
    kr = max(cfg.top_k, cfg.top_k_aux)
    gm = DecodeModel(cfg, fill="host")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    for step in range(2):
        tok = src.step_tokens(step)
        gm.decode_step(gm.tokens(tok), router_logits=None)
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True, router_logits=None, trace=True)
        for l in range(cfg.L):
            ranked = -np.sort(-r.trace[f"router.{l}"][:, 0], axis=1)[:, :kr + 1]
            assert np.diff(-ranked, axis=1).min() > 1e-4, "seed gives a near-tie: choose another"
        assert np.array_equal(gm.expert_ids.cpu().numpy(), r.ids), "expert ranking differs"
        _compare_step(cfg, gm, r)


@pytest.mark.parametrize("E", [128, 320], ids=["e128", "e320"])
def test_moe_routing_many_experts(E):
    """Routing with more experts than lanes (2 and 5 logits per lane of the
    ranking wave): ranking bit-exact, outputs within the bars."""
    cfg = SMALL_MOE.replace(name=f"gpu_moe_e{E}", E=E, top_k_aux=8)
    say(f"moe routing E={E}")
    gm = DecodeModel(cfg, fill="host")
    src = Inputs(cfg)
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    for step in range(2):
        tok = src.step_tokens(step)
        rl = gm.router_logits(step)
        gm.decode_step(gm.tokens(tok), router_logits=rl)
        torch.cuda.synchronize()
        r = odf.decode_step(m, cache, tok, aux_on=True, router_logits=rl.cpu().numpy())
        assert np.array_equal(gm.expert_ids.cpu().numpy(), r.ids), "expert ranking differs"
        _compare_step(cfg, gm, r)
