"""The full-sequence dual forward on the GPU (df_forward_dual) against the
oracle's forward_dual: both flows at every position of the tokens.

Bars: logits of both flows within 2e-2 max-abs and p_mix / alpha within
1e-3 at every position (the decode-step bars), the argmax of p_mix the
oracle's unless the oracle's top two are within 2e-3; K/V write positions
bit-exact (untouched entries bitwise unchanged) and written values within
one bf16 ulp plus the fp32 projection error, plus from the second layer on
3 D_l, the effect of one-ulp flips of lower-layer cache entries measured on
the oracle itself (as in the prefill tests)."""
import numpy as np
import pytest
import torch

from dual_flow_transformer_amd.runtime import DecodeModel
from gpu_util import argmax_agrees, bits_to_f64, max_abs, say
from oracle import dualflow as odf
from synth.workloads import Config, Inputs
from test_gpu_decode import KV_ABS, LOGIT_TOL, PMIX_TOL
from test_gpu_prefill import _excess

pytestmark = pytest.mark.gpu

FW_ONE = Config("forward_one_chunk", L=2, d=256, H=2, Dh=128, F=1024, V=512, B=3, ctx=40, S_max=200,
                dtype="bf16", seed=41, sigma_w=0.05, sigma_ln=0.1, prompt_len=100)
FW_MULTI = Config("forward_multi_chunk", L=2, d=256, H=2, Dh=128, F=512, V=256, B=4, ctx=30, S_max=200,
                  dtype="bf16", seed=42, sigma_w=0.05, sigma_ln=0.1, prompt_len=150)
FW_F32 = Config("forward_f32", L=2, d=128, H=2, Dh=64, F=256, V=300, B=2, ctx=20, S_max=64, dtype="f32",
                seed=43, sigma_w=0.05, sigma_ln=0.1, prompt_len=12)
FW_MOE = Config("forward_moe", L=2, d=256, H=2, Dh=128, F=0, V=512, B=4, ctx=20, S_max=64, dtype="bf16",
                moe=True, E=16, top_k=4, Fe=256, seed=44, sigma_w=0.05, sigma_ln=0.1, prompt_len=10)
# chunk rows per flow = prefill_rows / 2: 4 sequences x 64 positions
CHUNK_ROWS = {"forward_multi_chunk": 2 * 4 * 64}


def _oracle(cfg, src, lens, toks, perturb):
    m = odf.Model(src)
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    cache.lens = np.asarray(lens, dtype=np.int64).copy()
    if not perturb:
        return odf.forward_dual(m, cache, toks), cache
    rnd, rng = odf.round_to, np.random.default_rng(cfg.seed)
    odf.round_to = lambda x, dt: rnd(x * (1.0 + rng.uniform(-2.0 ** -17, 2.0 ** -17, np.shape(x))), dt)
    try:
        return odf.forward_dual(m, cache, toks), cache
    finally:
        odf.round_to = rnd


def _run(cfg, lens=None):
    src = Inputs(cfg)
    T = cfg.prompt_len
    toks = src.prompt()
    lens = [cfg.ctx] * cfg.B if lens is None else lens
    gm = DecodeModel(cfg, fill="host", prefill_rows=CHUNK_ROWS.get(cfg.name, 0))
    sentinel = 0x4242 if cfg.dtype == "bf16" else 12345.0
    gm.k[:, :, :, cfg.ctx:] = sentinel
    gm.v[:, :, :, cfg.ctx:] = sentinel
    gm.len.copy_(torch.as_tensor(lens, dtype=torch.int32))
    k0, v0 = gm.k.cpu().numpy(), gm.v.cpu().numpy()
    say(f"forward {cfg.name} variant={cfg.variant} lens={list(lens)[:4]} T={T}")
    lg, pm, al, nt = gm.forward(gm.tokens(toks).contiguous())
    torch.cuda.synchronize()
    fw, cache = _oracle(cfg, src, lens, toks, False)
    el = max_abs(lg.cpu().numpy(), fw.logits)
    ep = max_abs(pm.cpu().numpy(), fw.p_mix)
    ea = max_abs(al.cpu().numpy(), fw.alpha)
    say(f"  logits max|d|={el:.3e} p_mix max|d|={ep:.3e} alpha max|d|={ea:.3e}")
    assert el < LOGIT_TOL and ep < PMIX_TOL and ea < PMIX_TOL
    pmc, ntc = pm.cpu().numpy(), nt.cpu().numpy()
    for b in range(cfg.B):
        for t in range(T):
            assert argmax_agrees(pmc[b, t], fw.p_mix[b, t], ntc[b, t], margin=2e-3), (b, t)
    assert np.array_equal(gm.len.cpu().numpy(), cache.lens)
    assert gm.status() == 0
    # cache: written positions exactly [lens, lens + T), values as in the prefill tests
    flips = _oracle(cfg, src, lens, toks, True)[1] if cfg.dtype == "bf16" else None
    for i, (t, before) in enumerate(((gm.k, k0), (gm.v, v0))):
        a = t.cpu().numpy()
        diff = np.any(a != before, axis=-1)
        written = np.zeros_like(diff)
        for b in range(cfg.B):
            written[:, b, :, lens[b]:lens[b] + T] = True
        assert not np.any(diff & ~written), "entries outside the sequence positions changed"
        for l in range(cfg.L):
            ref = cache.layer(l)[i]
            d_l = 0.0
            if l > 0 and flips is not None:
                alt = flips.layer(l)[i]
                d_l = max(_excess(alt[b, :, lens[b]:lens[b] + T], ref[b, :, lens[b]:lens[b] + T]).max()
                          for b in range(cfg.B))
            for b in range(cfg.B):
                got = bits_to_f64(t[l, b, :, lens[b]:lens[b] + T], cfg.dtype)
                want = ref[b, :, lens[b]:lens[b] + T]
                if cfg.dtype == "bf16":
                    err = _excess(got, want) - (KV_ABS + 3 * d_l)
                else:
                    err = np.abs(got - want) - 1e-4
                assert np.all(err <= 0), f"l={l} b={b}: worst excess {err.max():.3e} (D_l {d_l:.2e})"


def test_forward_one_chunk():
    _run(FW_ONE, lens=[40, 7, 0])


def test_forward_multi_chunk():
    _run(FW_MULTI, lens=[30, 0, 17, 5])


@pytest.mark.parametrize("variant", [1, 2, 4])
def test_forward_variants(variant):
    _run(FW_ONE.replace(variant=variant, prompt_len=40))


@pytest.mark.parametrize("cfg", [FW_F32, FW_MOE, FW_MOE.replace(name="forward_moe_fanout", top_k_aux=8)],
                         ids=lambda c: c.name)
def test_forward_per_position_path(cfg):
    """Models outside the chunked path (fp32, MoE) run one dual step per
    position; the results land at their [batch][T] places."""
    _run(cfg)


def test_forward_matches_dual_steps_on_gpu():
    """The chunked forward and T teacher-forced df_decode_step calls on the
    GPU agree (a property that holds at any size), and both equal the oracle."""
    cfg = FW_ONE.replace(prompt_len=6)
    src = Inputs(cfg)
    toks = src.prompt()
    a = DecodeModel(cfg, fill="host")
    lg, pm, al, nt = a.forward(a.tokens(toks).contiguous())
    b = DecodeModel(cfg, fill="host")
    for t in range(cfg.prompt_len):
        b.decode_step(b.tokens(toks[:, t]))
        assert max_abs(b.logits.cpu().numpy(), lg[:, t].cpu().numpy()) < LOGIT_TOL
        assert max_abs(b.p_mix.cpu().numpy(), pm[:, t].cpu().numpy()) < PMIX_TOL
    torch.cuda.synchronize()
    assert torch.equal(a.len, b.len)
