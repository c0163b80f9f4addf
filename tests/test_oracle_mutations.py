"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case patches one plausible error into the oracle (a dropped term, a wrong
sign or operand, a wrong index or tie rule, a misplaced rounding) and checks
that at least one pin then fails. CPU only; nothing here touches a GPU.
"""
import math

import numpy as np
import pytest

import pins
from oracle import dualflow as odf


def _gelu_tanh(x):
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _attn_noscale(q, K, V):
    s = K @ q
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum(), m + math.log(p.sum())


def _ln_unbiased(x, g, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - mu) / np.sqrt(var + eps) * g


def _ln_no_eps(x, g, eps):
    mu = x.mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True)) * g


def _mix_no_floor(l1, l2):
    p1 = odf.softmax(np.asarray(l1, float))
    if l2 is None:
        return p1, 1.0, int(np.argmax(p1))
    p2 = odf.softmax(np.asarray(l2, float))
    a = float(np.sum(p1 * p1))
    p = a * p1 + (1 - a) * p2
    return p, a, int(np.argmax(p))


def _mix_swapped(l1, l2):
    p1 = odf.softmax(np.asarray(l1, float))
    if l2 is None:
        return p1, 1.0, int(np.argmax(p1))
    p2 = odf.softmax(np.asarray(l2, float))
    a = min(1.0, max(0.5, float(np.sum(p1 * p1))))
    p = a * p2 + (1 - a) * p1
    return p, a, int(np.argmax(p))


def _mix_alpha_half_plus(l1, l2):
    p1 = odf.softmax(np.asarray(l1, float))
    if l2 is None:
        return p1, 1.0, int(np.argmax(p1))
    p2 = odf.softmax(np.asarray(l2, float))
    a = 0.5 * (1 + float(np.sum(p1 * p1)))
    p = a * p1 + (1 - a) * p2
    return p, a, int(np.argmax(p))


def _topk_upper_ties(r, k):
    r = np.asarray(r, float)
    idx = np.argsort(-r[::-1], kind="stable")
    return (len(r) - 1 - idx)[:k].astype(np.int32)


def _round_via_f32(x, dtype):
    if dtype == "bf16":
        import torch
        x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
        return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _round_truncate(x, dtype):
    if dtype == "bf16":
        m, e = np.frexp(np.asarray(x, dtype=np.float64))
        return np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _qkv_aux_writes(p, u, cfg, couple=True):
    q, k, v = _orig_qkv(p, u, cfg, couple)
    if len(u) == 2:
        qkv2 = odf._matvec(p["w_qkv"], u[1])
        k = odf.round_to(qkv2[cfg.d:2 * cfg.d], cfg.dtype).reshape(cfg.H, cfg.Dh)
        v = odf.round_to(qkv2[2 * cfg.d:], cfg.dtype).reshape(cfg.H, cfg.Dh)
    return q, k, v


def _qkv_no_round(p, u, cfg, couple=True):
    d = cfg.d
    qkv1 = odf._matvec(p["w_qkv"], u[0])
    q = [qkv1[:d]]
    if len(u) == 2:
        q.append(odf.couple_query(odf._matvec(p["w_qkv"], u[1])[:d], p["a"], q[0]))
    return q, qkv1[d:2 * d].reshape(cfg.H, cfg.Dh), qkv1[2 * d:].reshape(cfg.H, cfg.Dh)


_orig_qkv = odf.qkv_rows


def _qkv_ignores_switch(p, u, cfg, couple=True):
    return _orig_qkv(p, u, cfg, True)


_orig_mix = odf.mix_head


def _mix_half_keeps_floor(l1, l2, mode=odf.MIX_COLLISION):
    if mode == odf.MIX_HALF:
        mode = odf.MIX_COLLISION
    return _orig_mix(l1, l2, mode)


def _mix_aux_mode_primary(l1, l2, mode=odf.MIX_COLLISION):
    if mode == odf.MIX_AUX and l2 is not None:
        p1 = odf.softmax(np.asarray(l1, float))
        return p1, 0.0, int(np.argmax(p1))
    return _orig_mix(l1, l2, mode)


_orig_moe = odf._mlp_moe


def _moe_couples_aux_only_experts(p, v, flows, dtype, k, r1_given, tr=None, k_aux=0, couple=True):
    """b coupling also on aux-only experts (ranks k..k_aux-1), reading the
    primary's intermediate there although the primary never ran them."""
    ka = k if k_aux <= 0 else k_aux
    if flows == 1 or ka <= k:
        return _orig_moe(p, v, flows, dtype, k, r1_given, tr, k_aux, couple)
    y, ranking, gates = _orig_moe(p, v, flows, dtype, k, r1_given, tr, k_aux, couple)
    y = [y[0], y[1].copy()]
    for j in range(k, ka):
        e = ranking[j]
        y[1] = y[1] + gates[1][j] * (p["w_edown"][e] @ (p["b"] * odf.gelu(p["w_eup"][e] @ v[0])))
    return y, ranking, gates


def _attend_excl_new(q, K, V, pos):
    n = max(pos, 1)
    o, _ = odf.attention_one(q, K[:n], V[:n])
    return o


def _decode_shift15(u16, out=None):
    u = np.ascontiguousarray(u16, dtype=np.uint16)
    return (u.astype(np.uint32) << 15).view(np.float32).astype(np.float64)


def _decode_byteswap(u16, out=None):
    u = np.ascontiguousarray(u16, dtype=np.uint16).byteswap()
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


_orig_matvec = odf._matvec


def _matvec_rounds_inputs(W, x):
    return _orig_matvec(W, odf.round_to(np.asarray(x, dtype=np.float64), "bf16"))


MUTATIONS = [
    ("gelu_tanh_approx", "gelu", _gelu_tanh, [pins.pin_gelu]),
    ("attention_no_scale", "attention_one", _attn_noscale, [pins.pin_attention_sdpa]),
    ("layernorm_unbiased_var", "layer_norm", _ln_unbiased, [pins.pin_layer_norm]),
    ("layernorm_no_eps", "layer_norm", _ln_no_eps, [pins.pin_layer_norm]),
    ("alpha_without_floor", "mix_head", _mix_no_floor, [pins.pin_mix_properties, pins.pin_mix_golden]),
    ("mixture_weights_swapped", "mix_head", _mix_swapped, [pins.pin_mix_properties, pins.pin_mix_golden]),
    ("alpha_half_one_plus_cp", "mix_head", _mix_alpha_half_plus, [pins.pin_mix_properties, pins.pin_mix_golden]),
    ("topk_ties_to_upper", "topk_ids", _topk_upper_ties, [pins.pin_topk]),
    ("bf16_double_rounding", "round_to", _round_via_f32, [pins.pin_round_bf16]),
    ("bf16_truncation", "round_to", _round_truncate, [pins.pin_round_bf16]),
    ("bf16_decode_wrong_shift", "decode_bf16", _decode_shift15, [pins.pin_decode_bf16]),
    ("bf16_decode_byte_order", "decode_bf16", _decode_byteswap, [pins.pin_decode_bf16]),
    ("projection_inputs_rounded", "_matvec", _matvec_rounds_inputs, [pins.pin_unrounded_inputs_are_stable]),
    ("query_coupling_sign", "couple_query", lambda q2, a, q1: q2 - a * q1,
     [lambda: pins.pin_query_coupling(pins.TINY_BF16)]),
    ("query_coupling_wrong_operand", "couple_query", lambda q2, a, q1: q2 + a * q2,
     [lambda: pins.pin_query_coupling(pins.TINY_BF16)]),
    ("mid_coupling_wrong_operand", "couple_mid", lambda g2, b, g1: g2 + b * g2,
     [lambda: pins.pin_mid_coupling(pins.TINY_BF16)]),
    ("mid_coupling_rounded_primary", "couple_mid", lambda g2, b, g1: g2 + b * odf._round_bf16(g1),
     [lambda: pins.pin_mid_coupling(pins.TINY_BF16)]),
    ("out_coupling_wrong_operand", "couple_out", lambda y2, c, y1: y2 + c * y2,
     [lambda: pins.pin_out_coupling(pins.TINY_BF16)]),
    ("out_coupling_dropped", "couple_out", lambda y2, c, y1: y2,
     [lambda: pins.pin_out_coupling(pins.TINY_F32)]),
    ("aux_writes_kv", "qkv_rows", _qkv_aux_writes, [lambda: pins.pin_aux_onoff(pins.TINY_BF16)]),
    ("kv_not_rounded", "qkv_rows", _qkv_no_round, [lambda: pins.pin_prefill_equals_decode(pins.TINY_BF16),
                                                    lambda: pins.pin_query_coupling(pins.TINY_BF16)]),
    ("no_coupling_switch_ignored", "qkv_rows", _qkv_ignores_switch,
     [lambda: pins.pin_no_coupling_tied(pins.TINY_BF16)]),
    ("alpha_half_keeps_floor", "mix_head", _mix_half_keeps_floor, [pins.pin_mix_half_mode]),
    ("aux_output_mode_gives_primary", "mix_head", _mix_aux_mode_primary, [pins.pin_mix_aux_mode]),
    ("aux_only_experts_coupled", "_mlp_moe", _moe_couples_aux_only_experts, [pins.pin_fanout_closed_forms]),
    ("attend_excludes_new_entry", "attend", _attend_excl_new,
     [lambda: pins.pin_prefill_equals_decode(pins.TINY_F32), lambda: pins.pin_query_coupling(pins.TINY_F32)]),
]


@pytest.mark.parametrize("name,attr,fn,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, attr, fn, checks):
    monkeypatch.setattr(odf, attr, fn)
    caught = False
    for chk in checks:
        try:
            chk()
        except AssertionError:
            caught = True
            break
    assert caught, f"planted mistake '{name}' passed every pin"


def test_moe_aux_gates_from_primary_is_caught(monkeypatch):
    orig = odf._mlp_moe

    def wrong(p, v, flows, dtype, k, r1_given, tr=None, k_aux=0, couple=True):
        y, ids, gates = orig(p, v, 1, dtype, k, r1_given, tr)
        if flows == 1:
            return y, ids, gates
        # aux reuses the primary gates instead of its own
        g = gates[0]
        yy = [y[0], np.zeros_like(y[0])]
        for j, e in enumerate(ids):
            gg = odf.gelu(p["w_eup"][e] @ v[1]) + p["b"] * odf.gelu(p["w_eup"][e] @ v[0])
            yy[1] = yy[1] + g[j] * (p["w_edown"][e] @ gg)
        yy[1] = yy[1] + p["c"] * yy[0]
        return yy, ids, np.stack([g, g])

    monkeypatch.setattr(odf, "_mlp_moe", wrong)
    with pytest.raises(AssertionError):
        pins.pin_moe_all_experts_is_full_mixture()


def _mutated_forward(old, new):
    """forward_dual with one line of its source replaced."""
    import inspect
    src = inspect.getsource(odf.forward_dual)
    assert old in src, old
    ns = dict(vars(odf))
    exec(compile(src.replace(old, new), "<planted mistake>", "exec"), ns)
    return ns["forward_dual"]


FORWARD_MUTATIONS = [
    ("aux_query_uncoupled", 'q2 = q2 + p["a"][None, :] * q1', "q2 = q2"),
    ("aux_query_from_primary_row", 'q2 = u[1] @ p["w_qkv"][:d].T', 'q2 = u[0] @ p["w_qkv"][:d].T'),
    ("attention_sees_next_position", "n = p0 + t + 1", "n = p0 + t + 2"),
    ("mid_coupling_dropped", 'g[1] = g[1] + p["b"][None, :] * g[0]', "g[1] = g[1]"),
    ("out_coupling_from_aux", 'y[1] = y[1] + p["c"][None, :] * y[0]', 'y[1] = y[1] + p["c"][None, :] * y[1]'),
    ("aux_embedding_is_primary", "h_all[i, f] = model.emb(f, tokens[i])", "h_all[i, f] = model.emb(0, tokens[i])"),
    ("kv_not_rounded", "round_to(qkv1[:, d:2 * d], dt)", "qkv1[:, d:2 * d]"),
    ("mixture_swapped", "mix_head(logits[i, t, 0], logits[i, t, 1], mode)",
     "mix_head(logits[i, t, 1], logits[i, t, 0], mode)"),
]


@pytest.mark.parametrize("name,old,new", FORWARD_MUTATIONS, ids=[m[0] for m in FORWARD_MUTATIONS])
def test_forward_mutation_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(odf, "forward_dual", _mutated_forward(old, new))
    with pytest.raises(AssertionError):
        pins.pin_forward_equals_steps(pins.TINY_BF16)


def _mutated(fn, old, new):
    """An oracle function with one line of its source replaced."""
    import inspect
    src = inspect.getsource(fn)
    assert old in src, old
    ns = dict(vars(odf))
    exec(compile(src.replace(old, new), "<planted mistake>", "exec"), ns)
    return ns[fn.__name__]


RUN_TINY_MUTATIONS = [
    ("prefill_takes_last_prompt_token", "prefill_primary(model, cache, prompt[:, :-1])",
     "prefill_primary(model, cache, prompt)"),
    ("first_step_wrong_token", "tok = prompt[:, -1]", "tok = prompt[:, -2]"),
    ("aux_activated_one_position_late", "aux_on=True", "aux_on=(s > 0)"),
    ("chosen_token_not_fed_back", "tok = r.next_tok", "tok = tok"),
]


@pytest.mark.parametrize("name,old,new", RUN_TINY_MUTATIONS, ids=[m[0] for m in RUN_TINY_MUTATIONS])
def test_run_tiny_mutation_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(odf, "run_tiny", _mutated(odf.run_tiny, old, new))
    with pytest.raises(AssertionError):
        pins.pin_run_tiny_schedule(pins.TINY_F32)
