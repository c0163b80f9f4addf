"""Mixture head (df_mix_head) and explicit K/V writes (df_kv_append) on the
GPU against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from dual_flow_transformer_amd import _abi
from gpu_util import argmax_agrees, max_abs, say
from oracle import dualflow as odf

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


MODES = {_abi.DF_MIX_PRIMARY: None, _abi.DF_MIX_COLLISION: odf.MIX_COLLISION, _abi.DF_MIX_AUX: odf.MIX_AUX,
         _abi.DF_MIX_HALF: odf.MIX_HALF}


def _mix(l, aux_on):
    B, _, V = l.shape
    dl = torch.from_numpy(np.ascontiguousarray(l, dtype=np.float32)).cuda()
    p = torch.full((B, V), float("nan"), device="cuda")
    a = torch.full((B,), float("nan"), device="cuda")
    t = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    rc = _abi.df_mix_head(dl.data_ptr(), B, V, aux_on, p.data_ptr(), a.data_ptr(), t.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return p.cpu().numpy(), a.cpu().numpy(), t.cpu().numpy()


# vocabularies across the kernel's register-resident sizes (up to 4, 8, 16 and 32 Ki
# logits per row) and past them (the path that re-reads the row)
@pytest.mark.parametrize("V,scale,aux_on", [(32000, 1.0, 1), (517, 3.0, 1), (1000, 12.0, 1), (32000, 1.0, 0),
                                            (32000, 1.0, 2), (1000, 12.0, 2), (32000, 1.0, 3), (1000, 12.0, 3),
                                            (5000, 2.0, 1), (9000, 1.0, 1), (32768, 1.0, 1), (40000, 1.0, 1),
                                            (40000, 4.0, 0)])
def test_mix_head_random(V, scale, aux_on):
    say(f"mix head V={V} scale={scale} mode={aux_on}")
    B = 4
    l = synth.normal((B, 2, V), 5, synth.stream_id("mixl", V), scale, "f32")
    p, a, t = _mix(l, aux_on)
    for b in range(B):
        mode = MODES[aux_on]
        rp, ra, _ = odf.mix_head(l[b, 0], l[b, 1] if mode else None, mode or odf.MIX_COLLISION)
        assert max_abs(p[b], rp) < 1e-6 + 1e-4 * rp.max()
        assert abs(a[b] - ra) < 1e-5
        assert argmax_agrees(p[b], rp, t[b])
        assert abs(p[b].astype(np.float64).sum() - 1) < 1e-4


def test_mix_head_golden_cases():
    d = json.load(open(os.path.join(GOLDEN, "mix_crafted.json")))
    for c in d["cases"]:
        l = np.array([[c["l1"], c["l2"]]], dtype=np.float32)
        p, a, t = _mix(l, 1)
        say(f"golden: {c['note']} -> alpha {a[0]} p {p[0]}")
        assert abs(a[0] - c["alpha"]) < 1e-6
        assert max_abs(p[0], c["p_mix"]) < 1e-6
        assert t[0] == c["next_tok"]


def test_mix_head_confident_primary():
    """A peaked primary distribution: collision probability above 0.5."""
    V = 4096
    l = np.zeros((1, 2, V), np.float32)
    l[0, 0, 17] = 12.0
    l[0, 1] = synth.normal((V,), 3, synth.stream_id("mixc"), 1.0, "f32")
    p, a, t = _mix(l, 1)
    rp, ra, rt = odf.mix_head(l[0, 0], l[0, 1])
    assert ra > 0.5 and abs(a[0] - ra) < 1e-5 and t[0] == rt == 17
    assert np.all(np.abs(p[0] - rp) <= 1e-6 + 1e-5 * rp)      # fp32 relative error on the large entry


@pytest.mark.parametrize("dtype", [_abi.DF_BF16, _abi.DF_F32])
def test_kv_append_positions_and_values(dtype):
    L, B, H, S, Dh = 2, 3, 2, 16, 128
    say(f"kv append dtype={dtype}")
    cfg = _abi.df_config(L, H * Dh, H, Dh, 256, 512, 0, 0, 0, B, S, dtype, 1e-5)
    tdt = torch.int16 if dtype == _abi.DF_BF16 else torch.float32
    sentinel = 0x4242 if dtype == _abi.DF_BF16 else 12345.0
    K = torch.full((L, B, H, S, Dh), sentinel, dtype=tdt, device="cuda")
    V = torch.full_like(K, sentinel)
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    kv = _abi.df_kv(K.data_ptr(), V.data_ptr(), lens.data_ptr())
    pos = np.array([0, 7, S - 1], np.int32)
    dk = synth.normal((B, H, Dh), 9, synth.stream_id("kva"), 3.0, "f32")
    dv = synth.normal((B, H, Dh), 9, synth.stream_id("kvb"), 3.0, "f32")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    dpos, ddk, ddv = torch.from_numpy(pos).cuda(), torch.from_numpy(dk).cuda(), torch.from_numpy(dv).cuda()
    rc = _abi.df_kv_append(cfg, kv, 1, dpos.data_ptr(), ddk.data_ptr(), ddv.data_ptr(), st.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    dts = "bf16" if dtype == _abi.DF_BF16 else "f32"
    for arr, src in ((K, dk), (V, dv)):
        a = arr.cpu().numpy()
        changed = np.any(a != (np.int16(sentinel) if dtype == _abi.DF_BF16 else np.float32(sentinel)), axis=-1)
        want = np.zeros_like(changed)
        for b in range(B):
            want[1, b, :, pos[b]] = True
        assert np.array_equal(changed, want)          # write positions: bit-exact
        got = np.stack([a[1, b, :, pos[b]] for b in range(B)])
        gotf = odf.decode_bf16(got.view(np.uint16)) if dtype == _abi.DF_BF16 else got.astype(np.float64)
        assert np.array_equal(gotf, odf.round_to(src.astype(np.float64), dts))   # rounded values: exact
    assert int(st.item()) == 0
    # out-of-range positions: nothing written, status flagged
    bad = torch.from_numpy(np.array([S, -1, 3], np.int32)).cuda()
    before = K.clone()
    rc = _abi.df_kv_append(cfg, kv, 0, bad.data_ptr(), ddk.data_ptr(), ddv.data_ptr(), st.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0 and int(st.item()) == 1
    diff = (K != before).any(dim=-1).cpu().numpy()
    assert diff.sum() == H and diff[0, 2, :, 3].all()
