"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

from dual_flow_transformer_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "dualflow.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(df_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    lib = _abi.lib()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(_abi.EXPORTS)


def good_config(**kw):
    base = dict(n_layers=2, d_model=256, n_heads=2, head_dim=128, ffn=1024, vocab=512, n_experts=0, top_k=0,
                expert_ffn=0, batch=3, max_seq=64, dtype=_abi.DF_BF16, ln_eps=1e-5, variant=0, top_k_aux=0,
                prefill_rows=0)
    base.update(kw)
    return _abi.df_config(*[base[f] for f, _ in _abi.df_config._fields_])


def fake_weights(p=0x10000, moe=False):
    w = _abi.df_weights()
    w.tok_emb[0] = p; w.tok_emb[1] = p + 0x100
    for i, f in enumerate(["pos_emb", "ln1", "ln2", "lnf", "w_qkv", "w_o", "w_up", "w_down", "cpl_a", "cpl_b",
                           "cpl_c", "w_out"]):
        setattr(w, f, p + 0x1000 * (i + 1))
    if moe:
        w.w_router, w.w_exp_up, w.w_exp_down = p + 0x100000, p + 0x200000, p + 0x300000
    return w


def test_workspace_query():
    assert _abi.df_workspace_bytes(good_config()) > 0
    assert _abi.df_workspace_bytes(good_config(head_dim=48, d_model=96)) == 0
    # prefill: one chunk of batch * min(max_seq, rows / batch) rows on top of the decode workspace
    base = _abi.df_workspace_bytes(good_config())
    for rows, tc in ((0, 64), (96, 32), (2, 1)):
        extra = _abi.df_prefill_workspace_bytes(good_config(prefill_rows=rows)) - base
        assert extra >= 3 * tc * (3 * 256 + 1024) * 4
    assert _abi.df_prefill_workspace_bytes(good_config(dtype=_abi.DF_F32, batch=2)) == \
        _abi.df_workspace_bytes(good_config(dtype=_abi.DF_F32, batch=2))            # one position at a time
    assert _abi.df_attention_workspace_bytes(32, 32, 4096, 128) > 0
    assert _abi.df_attention_workspace_bytes(32, 32, 4096, 100) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _abi.DF_ERR_DTYPE),
    (dict(head_dim=48, d_model=96), _abi.DF_ERR_SHAPE),
    (dict(d_model=384, n_heads=3), _abi.DF_ERR_SHAPE),      # not a multiple of 256 in bf16
    (dict(batch=65), _abi.DF_ERR_SHAPE),
    (dict(n_heads=4), _abi.DF_ERR_SHAPE),                    # d != H*Dh
    (dict(ln_eps=0.0), _abi.DF_ERR_ARG),
    (dict(n_experts=16, top_k=17, expert_ffn=256), _abi.DF_ERR_SHAPE),
    (dict(n_experts=16, top_k=4, expert_ffn=256, dtype=_abi.DF_F32, d_model=256), _abi.DF_ERR_DTYPE),
    (dict(variant=8), _abi.DF_ERR_ARG),                                        # unknown switch
    (dict(prefill_rows=-1), _abi.DF_ERR_ARG),
    (dict(variant=_abi.DF_VARIANT_AUX_OUTPUT | _abi.DF_VARIANT_ALPHA_HALF), _abi.DF_ERR_ARG),
    (dict(top_k_aux=2), _abi.DF_ERR_SHAPE),                                    # dense model
    (dict(n_experts=16, top_k=4, expert_ffn=256, top_k_aux=17), _abi.DF_ERR_SHAPE),
])
def test_decode_rejects_bad_config(kw, code):
    cfg = good_config(**kw)
    kv = _abi.df_kv(0x20000, 0x30000, 0x40000)
    rc = _abi.df_decode_step(cfg, fake_weights(), kv, 0x50000, 1, None, None, 0x60000, 0x70000, None, None,
                             0x80000, 1 << 40, 0)
    assert rc == code


def test_decode_rejects_bad_pointers():
    cfg = good_config()
    kv = _abi.df_kv(0x20000, 0x30000, 0x40000)
    ws = 1 << 40
    call = lambda w, kv, tok=0x50000, pm=0x60000, ws_ptr=0x80000, ws_bytes=ws, aux=1: _abi.df_decode_step(
        cfg, w, kv, tok, aux, None, None, pm, 0x70000, None, None, ws_ptr, ws_bytes, 0)
    w = fake_weights()
    w.w_o = None
    assert call(w, kv) == _abi.DF_ERR_NULL
    w = fake_weights()
    w.w_o = 0x12345
    assert call(w, kv) == _abi.DF_ERR_ALIGN
    assert call(fake_weights(), _abi.df_kv(0, 0x30000, 0x40000)) == _abi.DF_ERR_NULL
    assert call(fake_weights(), kv, tok=None) == _abi.DF_ERR_NULL
    assert call(fake_weights(), kv, pm=None) == _abi.DF_ERR_NULL
    assert call(fake_weights(), kv, aux=2) == _abi.DF_ERR_ARG
    assert call(fake_weights(), kv, ws_ptr=0x80010) == _abi.DF_ERR_ALIGN
    assert call(fake_weights(), kv, ws_bytes=_abi.df_workspace_bytes(cfg) - 1) == _abi.DF_ERR_WORKSPACE
    # MoE config without expert weights
    mcfg = good_config(n_experts=16, top_k=4, expert_ffn=256, ffn=0)
    rc = _abi.df_decode_step(mcfg, fake_weights(), kv, 0x50000, 1, None, None, 0x60000, 0x70000, None, None,
                             0x80000, ws, 0)
    assert rc == _abi.DF_ERR_NULL
    # router logits supplied to a dense model
    rc = _abi.df_decode_step(cfg, fake_weights(), kv, 0x50000, 1, 0x90000, None, 0x60000, 0x70000, None, None,
                             0x80000, ws, 0)
    assert rc == _abi.DF_ERR_ARG


def test_other_entry_points_reject_bad_arguments():
    cfg = good_config()
    kv = _abi.df_kv(0x20000, 0x30000, 0x40000)
    assert _abi.df_prefill_primary(cfg, fake_weights(), kv, None, 4, 0x80000, 1 << 40) == _abi.DF_ERR_NULL
    assert _abi.df_prefill_primary(cfg, fake_weights(), kv, 0x50000, 65, 0x80000, 1 << 40) == _abi.DF_ERR_SHAPE
    ws = 0x80000
    pw = _abi.df_prefill_workspace_bytes(cfg)
    assert _abi.df_prefill_primary(cfg, fake_weights(), kv, 0x50000, 4, ws, pw - 256) == _abi.DF_ERR_WORKSPACE
    assert _abi.df_prefill_primary(cfg, fake_weights(), kv, 0x50000, -1, ws, pw) == _abi.DF_ERR_SHAPE
    # full-sequence dual forward: host checks before any launch
    fw = _abi.df_forward_workspace_bytes(cfg)
    assert fw >= _abi.df_workspace_bytes(cfg)
    f = lambda **k: _abi.df_forward_dual(k.get("cfg", cfg), fake_weights(), kv, k.get("tok", 0x50000), k.get("T", 4),
                                         k.get("lg", None), k.get("pm", 0x60000), k.get("al", 0x70000), None,
                                         k.get("ws", ws), k.get("wsb", fw))
    assert f(tok=None) == _abi.DF_ERR_NULL
    assert f(pm=None) == _abi.DF_ERR_NULL
    assert f(al=None) == _abi.DF_ERR_NULL
    assert f(T=65) == _abi.DF_ERR_SHAPE
    assert f(T=-1) == _abi.DF_ERR_SHAPE
    assert f(lg=0x90008) == _abi.DF_ERR_ALIGN
    assert f(pm=0x60008) == _abi.DF_ERR_ALIGN
    assert f(ws=0x80010) == _abi.DF_ERR_ALIGN
    assert f(wsb=fw - 256) == _abi.DF_ERR_WORKSPACE
    assert f(cfg=good_config(dtype=7)) == _abi.DF_ERR_DTYPE
    assert _abi.df_kv_append(cfg, kv, 2, 0x1000, 0x2000, 0x3000) == _abi.DF_ERR_SHAPE
    assert _abi.df_kv_append(cfg, kv, 0, None, 0x2000, 0x3000) == _abi.DF_ERR_NULL
    assert _abi.df_mix_head(None, 1, 10, 1, 0x1000, 0x2000) == _abi.DF_ERR_NULL
    assert _abi.df_mix_head(0x1000, 0, 10, 1, 0x1000, 0x2000) == _abi.DF_ERR_SHAPE
    assert _abi.df_mix_head(0x1000, 1, 10, 4, 0x1000, 0x2000) == _abi.DF_ERR_ARG
    assert _abi.df_mix_head(0x1000, 1, 10, -1, 0x1000, 0x2000) == _abi.DF_ERR_ARG
    a = lambda **kw: _abi.df_attention_dual(kw.get("dt", 1), 0x10000, 0x20000, 2, 2, 64, kw.get("dh", 128),
                                            0x30000, 0x40000, None, 0x50000, 0x60000, kw.get("ws", 0x70000),
                                            kw.get("wsb", 1 << 30))
    assert a(dt=3) == _abi.DF_ERR_DTYPE
    assert a(dh=96) == _abi.DF_ERR_SHAPE
    assert a(ws=0x70010) == _abi.DF_ERR_ALIGN
    assert a(wsb=16) == _abi.DF_ERR_WORKSPACE
    assert _abi.df_timing_enable(5) == _abi.DF_ERR_ARG
    assert _abi.df_timing_enable(0, 0) == _abi.DF_ERR_ARG
    # streaming read: pointer and size checks come before any device query
    assert _abi.df_stream_read(None, 1024, 0x1000) == _abi.DF_ERR_NULL
    assert _abi.df_stream_read(0x1000, 1024, None) == _abi.DF_ERR_NULL
    assert _abi.df_stream_read(0x1008, 1024, 0x2000) == _abi.DF_ERR_ALIGN
    assert _abi.df_stream_read(0x1000, 1000, 0x2000) == _abi.DF_ERR_ALIGN
    assert _abi.df_stream_read(0x1000, 1024, 0x2002) == _abi.DF_ERR_ALIGN


def test_status_strings():
    assert _abi.df_status_str(0) == "ok"
    assert "workspace" in _abi.df_status_str(_abi.DF_ERR_WORKSPACE)
    assert _abi.df_status_str(12345) == "unknown status code"


def test_pack_and_gemv_reject_bad_arguments():
    p = lambda **kw: _abi.df_pack_weights(kw.get("dt", _abi.DF_BF16), kw.get("src", 0x100000),
                                          kw.get("dst", 0x900000), kw.get("n", 2), kw.get("rows", 32),
                                          kw.get("cols", 64))
    assert p(dt=_abi.DF_F32) == _abi.DF_ERR_DTYPE
    assert p(src=None) == _abi.DF_ERR_NULL
    assert p(rows=24) == _abi.DF_ERR_SHAPE
    assert p(cols=48) == _abi.DF_ERR_SHAPE
    assert p(n=0) == _abi.DF_ERR_SHAPE
    assert p(dst=0x900008) == _abi.DF_ERR_ALIGN
    assert p(dst=0x100000 + 2 * 32 * 64 * 2 - 16) == _abi.DF_ERR_ARG     # overlaps the source
    assert _abi.df_stacked_gemv_workspace_bytes(_abi.DF_BF16, 32, 24, 4096) == 0   # N % 16
    assert _abi.df_stacked_gemv_workspace_bytes(_abi.DF_BF16, 32, 4096, 4000) == 0  # K % 256
    assert _abi.df_stacked_gemv_workspace_bytes(_abi.DF_BF16, 3, 4096, 4096) == 0   # odd rows
    assert _abi.df_stacked_gemv_workspace_bytes(_abi.DF_BF16, 333, 4096, 2048) > 0  # tiled GEMM
    assert _abi.df_stacked_gemv_workspace_bytes(_abi.DF_BF16, 333, 4096, 2000) == 0  # K % 32
    assert _abi.df_stacked_gemv_workspace_bytes(_abi.DF_BF16, 32, 4096, 4096) > 0
