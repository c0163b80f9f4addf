"""df_attention_dual_noalloc (partial results in the library's static device
array) against df_attention_dual (caller workspace): the same kernels, so
the outputs must agree bit for bit, on two calls in a row, the second with
a smaller input (the array keeps the first call's contents). Both are also
held to the attention bar against the oracle."""
import numpy as np
import pytest
import torch

import synth
from dual_flow_transformer_amd import _abi
from gpu_util import dev_bf16, max_abs, say
from oracle import dualflow as odf

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _inputs(B, H, S, Dh, lens, seed):
    K = synth.normal((B, H, S, Dh), seed, synth.stream_id("t_k"), 1.0, "bf16")
    V = synth.normal((B, H, S, Dh), seed, synth.stream_id("t_v"), 1.0, "bf16")
    q = synth.normal((B, 2, H, Dh), seed, synth.stream_id("t_q"), 1.0, "f32")
    a = synth.normal((H * Dh,), seed, synth.stream_id("t_a"), 1.0, "f32")
    return K, V, q, a, np.asarray(lens, dtype=np.int32)


def _call(noalloc, B, H, S, Dh, dK, dV, dl, dq, da):
    o = torch.full((B, 2, H, Dh), float("nan"), device="cuda")
    lse = torch.full((B, 2, H), float("nan"), device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    if noalloc:
        rc = _abi.df_attention_dual_noalloc(_abi.DF_BF16, dK.data_ptr(), dV.data_ptr(), B, H, S, Dh, dl.data_ptr(),
                                            dq.data_ptr(), da.data_ptr(), o.data_ptr(), lse.data_ptr(), st)
    else:
        wsb = _abi.df_attention_workspace_bytes(B, H, S, Dh)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        rc = _abi.df_attention_dual(_abi.DF_BF16, dK.data_ptr(), dV.data_ptr(), B, H, S, Dh, dl.data_ptr(),
                                    dq.data_ptr(), da.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), wsb,
                                    st)
    assert rc == 0, _abi.df_status_str(rc)
    return o, lse


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(8, 4, 700, 128, [700, 1, 257, 256, 513, 64, 699, 3], 51),   # first call
             (3, 2, 300, 64, [5, 300, 129], 52)]                           # second call, smaller
    for B, H, S, Dh, lens, seed in cases:
        say(f"no-alloc attention B={B} H={H} S={S} Dh={Dh} lens={lens}")
        K, V, q, a, ln = _inputs(B, H, S, Dh, lens, seed)
        dK, dV = dev_bf16(K), dev_bf16(V)
        dq, da, dl = torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda(), torch.from_numpy(ln).cuda()
        o_s, lse_s = _call(True, B, H, S, Dh, dK, dV, dl, dq, da)
        o_w, lse_w = _call(False, B, H, S, Dh, dK, dV, dl, dq, da)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_w) and torch.equal(lse_s, lse_w), "no-alloc entry point differs"
        ro, rl = odf.attention_dual(odf.to_f64(K), odf.to_f64(V), q[:, 0], q[:, 1], lens, a)
        eo, el = max_abs(o_s.cpu().numpy(), ro), max_abs(lse_s.cpu().numpy(), rl)
        say(f"  vs oracle: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo < TOL and el < TOL


def test_noalloc_rejects_oversize():
    z = torch.zeros(64, device="cuda")
    p = z.data_ptr()
    rc = _abi.df_attention_dual_noalloc(_abi.DF_BF16, p, p, 65, 2, 16, 128, p, p, None, p, p, 0)
    assert rc == _abi.DF_ERR_SHAPE
    rc = _abi.df_attention_dual_noalloc(_abi.DF_BF16, p, p, 64, 400, 16, 128, p, p, None, p, p, 0)
    assert rc == _abi.DF_ERR_SHAPE
