"""The compute-bound primary prefill on the GPU (df_prefill_primary for dense
bf16 models: tiled matrix-core GEMMs over the prompt rows and a causal
attention pass) against the oracle's prefill_primary, then a dual decode
step from the cache it left.

Bars: K/V write positions bit-exact (sentinel-filled cache, untouched
entries bitwise unchanged); written bf16 values within one bf16 ulp plus
the fp32 projection error (as for the decode step's append) plus, from the
second layer on, 3 D_l: an fp32-level difference before a bf16 rounding
can flip a cached K/V value of a lower layer by one ulp, and every later
position attends that entry, so deeper layers carry the flips' effect.
D_l measures it on the oracle itself: the largest excess over one ulp
between the oracle and the oracle with every K/V value perturbed by a
seeded relative +-2^-17 before rounding (the GPU's pre-rounding error is
about 2^-18 relative). The next dual step's logits and p_mix stay within
the decode-step bars."""
import numpy as np
import pytest
import torch

from dual_flow_transformer_amd import _abi
from dual_flow_transformer_amd.runtime import DecodeModel
from gpu_util import bits_to_f64, say
from oracle import dualflow as odf
from synth.workloads import Config, Inputs
from test_gpu_decode import KV_ABS, _compare_step

pytestmark = pytest.mark.gpu

# one chunk (Tc = max_seq): query blocks of 64 with a ragged tail
ONE_CHUNK = Config("prefill_one_chunk", L=2, d=256, H=2, Dh=128, F=1024, V=512, B=3, ctx=70, S_max=400,
                   dtype="bf16", seed=31, sigma_w=0.05, sigma_ln=0.1, prompt_len=150)
# 32 sequences with 2048-row chunks: 64 positions per chunk, the last one ragged
MULTI_CHUNK = Config("prefill_multi_chunk", L=2, d=256, H=2, Dh=128, F=512, V=256, B=32, ctx=40, S_max=256,
                     dtype="bf16", seed=32, sigma_w=0.05, sigma_ln=0.1, prompt_len=150)
CHUNK_ROWS = {"prefill_multi_chunk": 2048}


def _excess(got, want):
    """|got - want| beyond one bf16 ulp of want (2^-7 |want| bounds the ulp)."""
    return np.abs(got - want) - 2.0 ** -7 * np.abs(want)


def _oracle_prefill(cfg, m, src, lens, prompt, perturb):
    cache = odf.Cache(cfg, list(range(cfg.B)), src)
    cache.lens = np.asarray(lens, dtype=np.int64).copy()
    if not perturb:
        odf.prefill_primary(m, cache, prompt)
        return cache
    rnd, rng = odf.round_to, np.random.default_rng(cfg.seed)
    odf.round_to = lambda x, dt: rnd(x * (1.0 + rng.uniform(-2.0 ** -17, 2.0 ** -17, np.shape(x))), dt)
    try:
        odf.prefill_primary(m, cache, prompt)
    finally:
        odf.round_to = rnd
    return cache


def _run(cfg, lens, T):
    src = Inputs(cfg)
    prompt = src.prompt()[:, :T]
    gm = DecodeModel(cfg, fill="host", prefill_rows=CHUNK_ROWS.get(cfg.name, 0))
    sentinel = 0x4242
    gm.k[:, :, :, cfg.ctx:] = sentinel
    gm.v[:, :, :, cfg.ctx:] = sentinel
    gm.len.copy_(torch.as_tensor(lens, dtype=torch.int32))
    k0, v0 = gm.k.cpu().numpy(), gm.v.cpu().numpy()
    say(f"prefill {cfg.name} lens={list(lens)[:4]}.. T={T}")
    gm.prefill(gm.tokens(prompt).contiguous())
    torch.cuda.synchronize()
    m = odf.Model(src)
    cache = _oracle_prefill(cfg, m, src, lens, prompt, perturb=False)
    flips = _oracle_prefill(cfg, m, src, lens, prompt, perturb=True) if cfg.L > 1 else None
    assert np.array_equal(gm.len.cpu().numpy(), cache.lens)
    assert gm.status() == 0
    # written positions exactly [lens, lens + T); everything else bitwise kept
    for name, t, before in (("k", gm.k, k0), ("v", gm.v, v0)):
        a = t.cpu().numpy()
        diff = np.any(a != before, axis=-1)                     # [L, B, H, S]
        written = np.zeros_like(diff)
        for b in range(cfg.B):
            written[:, b, :, lens[b]:lens[b] + T] = True
        assert not np.any(diff & ~written), f"{name}: entries outside the prompt positions changed"
        # ... and every prompt position left the sentinel / old value behind
        # where the new value differs (checked through the values below)
        i = 0 if name == "k" else 1
        for l in range(cfg.L):
            ref = cache.layer(l)[i]
            d_l = 0.0
            if l > 0:
                alt = flips.layer(l)[i]
                d_l = max(_excess(alt[b, :, lens[b]:lens[b] + T], ref[b, :, lens[b]:lens[b] + T]).max()
                          for b in range(cfg.B))
            for b in range(cfg.B):
                got = bits_to_f64(t[l, b, :, lens[b]:lens[b] + T], "bf16")
                err = _excess(got, ref[b, :, lens[b]:lens[b] + T]) - (KV_ABS + 3 * d_l)
                assert np.all(err <= 0), f"{name} l={l} b={b}: worst excess {err.max():.3e} (D_l {d_l:.2e})"
    return gm, m, cache, src


@pytest.mark.parametrize("cfg,lens,T", [
    (ONE_CHUNK, [70, 13, 0], 150),
    (ONE_CHUNK, [70, 70, 70], 1),
    (MULTI_CHUNK, None, 150),
], ids=["one_chunk_ragged", "one_position", "multi_chunk"])
def test_prefill_then_dual_step(cfg, lens, T):
    if lens is None:
        lens = [(37 * b) % (cfg.ctx + 1) for b in range(cfg.B)]   # 0 .. ctx, varied
    gm, m, cache, src = _run(cfg, lens, T)
    tok = src.step_tokens(0)
    gm.decode_step(gm.tokens(tok))
    torch.cuda.synchronize()
    r = odf.decode_step(m, cache, tok, aux_on=True)
    _compare_step(cfg, gm, r)
    assert gm.status() == 0


def test_prefill_zero_tokens_is_a_no_op():
    cfg = ONE_CHUNK
    gm = DecodeModel(cfg, fill="host")
    k0, len0 = gm.k.clone(), gm.len.clone()
    tok = torch.zeros(cfg.B, 4, dtype=torch.int32, device="cuda")
    _abi.check(_abi.df_prefill_primary(gm.config, gm.weights, gm.kv, tok.data_ptr(), 0, gm.ws.data_ptr(),
                                       gm.ws_bytes, 0), "df_prefill_primary")
    torch.cuda.synchronize()
    assert torch.equal(gm.k, k0) and torch.equal(gm.len, len0)


def test_prefill_past_capacity_is_flagged():
    """Positions at or past max_seq are not written and set the status."""
    cfg = ONE_CHUNK
    src = Inputs(cfg)
    gm = DecodeModel(cfg, fill="host")
    gm.len.fill_(cfg.S_max - 5)
    k0 = gm.k.clone()
    gm.prefill(gm.tokens(src.prompt()[:, :8]).contiguous())
    torch.cuda.synchronize()
    assert gm.status() & 1
    assert torch.equal(gm.k[:, :, :, :cfg.S_max - 5], k0[:, :, :, :cfg.S_max - 5])


def test_prefill_workspace_query():
    cfg = ONE_CHUNK
    gm = DecodeModel(cfg, fill="host")
    need = _abi.df_prefill_workspace_bytes(gm.config)
    rows = cfg.B * min(cfg.S_max, 16384 // cfg.B)
    assert need >= _abi.df_workspace_bytes(gm.config) + rows * (3 * cfg.d + cfg.F) * 4
    rc = _abi.df_prefill_primary(gm.config, gm.weights, gm.kv, gm.tokens(np.zeros((cfg.B, 2), np.int64)).data_ptr(),
                                 2, gm.ws.data_ptr(), need - 256, 0)
    assert rc == _abi.DF_ERR_WORKSPACE
