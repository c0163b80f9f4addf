"""Shared-K/V dual attention on the GPU (df_attention_dual) against the
oracle: ragged small cases element by element, edge lengths, and the full
attention-only workload (B=32, H=32, Dh=128, len in [1024, 4096]) on every
(sequence, head) pair.

Tolerance (fp32 accumulation against float64): a score's rounding error is
at most about Dh * 2^-24 * sum|q_i k_i| ~ 6e-5 for N(0,1) inputs, so output
and LSE errors stay below ~4e-4; the tests use 1e-3."""
import numpy as np
import pytest
import torch

import synth
from synth import device as synth_dev
from dual_flow_transformer_amd import _abi
from gpu_util import bits_to_f64, dev_bf16, max_abs, say
from oracle import dualflow as odf
from synth.workloads import C2_ATTN, AttnInputs

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _run(dtype, B, H, Dh, S, lens, seed, with_a=True):
    say(f"attention case dtype={dtype} B={B} H={H} Dh={Dh} S={S} lens={list(lens)}")
    dt = "bf16" if dtype == _abi.DF_BF16 else "f32"
    K = synth.normal((B, H, S, Dh), seed, synth.stream_id("t_k"), 1.0, dt)
    V = synth.normal((B, H, S, Dh), seed, synth.stream_id("t_v"), 1.0, dt)
    q = synth.normal((B, 2, H, Dh), seed, synth.stream_id("t_q"), 1.0, "f32")
    a = synth.normal((H * Dh,), seed, synth.stream_id("t_a"), 1.0, "f32")
    up = dev_bf16 if dt == "bf16" else (lambda x: torch.from_numpy(x).cuda())
    dK, dV = up(K), up(V)
    dq = torch.from_numpy(q).cuda()
    da = torch.from_numpy(a).cuda() if with_a else None
    dl = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    o = torch.full((B, 2, H, Dh), float("nan"), device="cuda")
    lse = torch.full((B, 2, H), float("nan"), device="cuda")
    wsb = _abi.df_attention_workspace_bytes(B, H, S, Dh)
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")   # no initial contents are needed
    rc = _abi.df_attention_dual(dtype, dK.data_ptr(), dV.data_ptr(), B, H, S, Dh, dl.data_ptr(), dq.data_ptr(),
                                None if da is None else da.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                wsb, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _abi.df_status_str(rc)
    torch.cuda.synchronize()
    go, gl = o.cpu().numpy(), lse.cpu().numpy()
    # a sequence with no keys: zero outputs and LSE -inf; the oracle runs on the others
    nz = [b for b, n in enumerate(lens) if n > 0]
    for b in range(B):
        if b not in nz:
            assert np.all(go[b] == 0.0) and np.all(gl[b] == -np.inf), f"sequence {b}"
    Kf = odf.to_f64(K[nz])
    Vf = odf.to_f64(V[nz])
    ro, rl = odf.attention_dual(Kf, Vf, q[nz, 0], q[nz, 1], [lens[b] for b in nz], a if with_a else None)
    go, gl = go[nz], gl[nz]
    eo, el = max_abs(go, ro), max_abs(gl, rl)
    say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    assert eo < TOL and el < TOL


@pytest.mark.parametrize("dtype,Dh", [(_abi.DF_BF16, 128), (_abi.DF_BF16, 64), (_abi.DF_F32, 32),
                                      (_abi.DF_F32, 128)])
def test_ragged_small(dtype, Dh):
    # lengths span several chunks, a ragged tail, exact chunk multiples and 1
    _run(dtype, 5, 3, Dh, 1100, [1, 256, 257, 1100, 613], seed=31)


def test_no_coupling_vector():
    _run(_abi.DF_BF16, 2, 2, 128, 300, [300, 37], seed=32, with_a=False)


def test_long_context():
    """Contexts far beyond the workloads': 131,072 keys and a ragged 77,777, so
    the flattened key offsets, each wave's key range (about 800 keys here,
    in one or two segments) and the slot staircase run at large indices;
    every (sequence, head) against the oracle."""
    _run(_abi.DF_BF16, 2, 4, 128, 131072, [131072, 77777], seed=33)


@pytest.mark.parametrize("B,H,lens", [(3, 6, [131072, 100000, 123457]),
                                      (4, 9, [131072, 0, 1, 120000])])
def test_long_waves_skewed_split(B, H, lens):
    """Enough keys that the waves average 2048 or more (2,127,174 and
    2,259,657 keys over 1,024 waves), so even-workgroup waves take 3 % more
    keys than odd ones: every (sequence, head) against the oracle, across the
    uneven wave ranges and the combine's slot lookup for them, with a
    sequence that has no keys and one with a single key in the same launch."""
    _run(_abi.DF_BF16, B, H, 64, 131072, lens, seed=34)


def test_full_attention_workload_all_pairs():
    """The attention-only workload at full size (32 sequences x 32 heads,
    lengths uniform in [1024, 4096]: 2,594,976 keys, so the launch takes the
    XCD-skewed split): every (sequence, head) pair and both flows against
    the oracle."""
    c = C2_ATTN
    src = AttnInputs(c)
    lens = src.lengths()
    say(f"full attention workload: B={c.B} H={c.H} Dh={c.Dh} S={c.S_max} lens min {lens.min()} max {lens.max()}")
    K = torch.empty((c.B, c.H, c.S_max, c.Dh), dtype=torch.int16, device="cuda")
    V = torch.empty_like(K)
    for which, t in (("k", K), ("v", V)):
        st = [synth.stream_id("attn_" + which, b, h) for b in range(c.B) for h in range(c.H)]
        synth_dev.normal_streams(t, st, c.S_max * c.Dh, c.S_max * c.Dh, c.seed, 1.0, True)
    q1, q2, a = src.queries()
    q = np.stack([q1, q2], axis=1)
    dq, da = torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda()
    dl = torch.from_numpy(lens.astype(np.int32)).cuda()
    o = torch.full((c.B, 2, c.H, c.Dh), float("nan"), device="cuda")
    lse = torch.full((c.B, 2, c.H), float("nan"), device="cuda")
    wsb = _abi.df_attention_workspace_bytes(c.B, c.H, c.S_max, c.Dh)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    rc = _abi.df_attention_dual(_abi.DF_BF16, K.data_ptr(), V.data_ptr(), c.B, c.H, c.S_max, c.Dh, dl.data_ptr(),
                                dq.data_ptr(), da.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), wsb,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    go, gl = o.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl))
    worst = 0.0
    for b in range(c.B):
        Kb = odf.to_f64(src.kv_block("k", b, int(lens[b])))
        Vb = odf.to_f64(src.kv_block("v", b, int(lens[b])))
        for h in range(c.H):
            qq2 = q2[b, h] + a.reshape(c.H, c.Dh)[h] * q1[b, h]
            for f, qq in enumerate((q1[b, h], qq2)):
                ro, rl = odf.attention_one(qq.astype(np.float64), Kb[h], Vb[h])
                worst = max(worst, max_abs(go[b, f, h], ro), abs(gl[b, f, h] - rl))
    say(f"  all pairs max error {worst:.3e}")
    assert worst < TOL


def test_sampled_launch_timing():
    # kernel timing on every third partial-pass launch: 10 calls time calls 0, 3, 6 and 9,
    # and the timed launches produce the same bits as untimed ones
    B, H, S, Dh = 3, 2, 700, 128
    say(f"timing case B={B} H={H} S={S} Dh={Dh} stride 3 over 10 calls")
    K = synth.normal((B, H, S, Dh), 41, synth.stream_id("t_k"), 1.0, "bf16")
    V = synth.normal((B, H, S, Dh), 41, synth.stream_id("t_v"), 1.0, "bf16")
    q = synth.normal((B, 2, H, Dh), 41, synth.stream_id("t_q"), 1.0, "f32")
    a = synth.normal((H * Dh,), 41, synth.stream_id("t_a"), 1.0, "f32")
    dK, dV = dev_bf16(K), dev_bf16(V)
    dq, da = torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda()
    dl = torch.tensor([700, 1, 333], dtype=torch.int32, device="cuda")
    wsb = _abi.df_attention_workspace_bytes(B, H, S, Dh)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    outs = []

    def call():
        o = torch.empty((B, 2, H, Dh), device="cuda")
        lse = torch.empty((B, 2, H), device="cuda")
        rc = _abi.df_attention_dual(_abi.DF_BF16, dK.data_ptr(), dV.data_ptr(), B, H, S, Dh, dl.data_ptr(),
                                    dq.data_ptr(), da.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), wsb,
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0, _abi.df_status_str(rc)
        outs.append((o, lse))

    call()
    assert _abi.df_timing_enable(0, 3) == 0
    for _ in range(10):
        call()
    rc, ms, n = _abi.df_timing_read()
    assert rc == 0 and n == 4 and ms > 0.0
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])
    # reading disables timing
    call()
    rc, ms, n = _abi.df_timing_read()
    assert rc == 0 and n == 0 and ms == 0.0


@pytest.mark.parametrize("lens", [[0, 5, 0, 300, 0], [0, 0]], ids=["mixed", "all_empty"])
def test_sequences_without_keys(lens):
    """A sequence with no keys gets zero outputs and LSE -inf; the others
    match the oracle as usual."""
    B, H, S, Dh = len(lens), 2, 400, 128
    say(f"empty-sequence case lens={lens}")
    K = synth.normal((B, H, S, Dh), 43, synth.stream_id("t_k"), 1.0, "bf16")
    V = synth.normal((B, H, S, Dh), 43, synth.stream_id("t_v"), 1.0, "bf16")
    q = synth.normal((B, 2, H, Dh), 43, synth.stream_id("t_q"), 1.0, "f32")
    dK, dV, dq = dev_bf16(K), dev_bf16(V), torch.from_numpy(q).cuda()
    dl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.full((B, 2, H, Dh), float("nan"), device="cuda")
    lse = torch.full((B, 2, H), float("nan"), device="cuda")
    wsb = _abi.df_attention_workspace_bytes(B, H, S, Dh)
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
    rc = _abi.df_attention_dual(_abi.DF_BF16, dK.data_ptr(), dV.data_ptr(), B, H, S, Dh, dl.data_ptr(),
                                dq.data_ptr(), None, o.data_ptr(), lse.data_ptr(), ws.data_ptr(), wsb,
                                torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _abi.df_status_str(rc)
    torch.cuda.synchronize()
    go, gl = o.cpu().numpy(), lse.cpu().numpy()
    Kf, Vf = odf.to_f64(K), odf.to_f64(V)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(go[b] == 0.0) and np.all(gl[b] == -np.inf), f"sequence {b}"
            continue
        for h in range(H):
            for f in range(2):
                ro, rl = odf.attention_one(q[b, f, h].astype(np.float64), Kf[b, h, :n], Vf[b, h, :n])
                assert max_abs(go[b, f, h], ro) < TOL and abs(gl[b, f, h] - rl) < TOL
