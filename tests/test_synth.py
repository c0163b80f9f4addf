"""The shared seeded input generator: known answers and basic properties."""
import json
import os

import numpy as np
import torch

import synth
from synth.workloads import C1_TINY, C4_MOE, Inputs, normal_quantiles

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_splitmix64_known_answers():
    d = json.load(open(os.path.join(GOLDEN, "splitmix64_kat.json")))
    got = [int(w) for w in synth.words(d["state"], 3)]
    assert got == [int(x, 16) for x in d["outputs_hex"]]


def test_normal_moments_and_bf16():
    x = synth.normal((400000,), 7, synth.stream_id("t"), 0.5, "f32")
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 0.5) < 5e-3
    b = synth.normal((400000,), 7, synth.stream_id("t"), 0.5, "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, want)


def test_offsets_and_streams_consistent():
    sid = synth.stream_id("w", 3)
    full = synth.normal((10, 8), 1, sid, 1.0, "bf16")
    part = synth.normal((8,), 1, sid, 1.0, "bf16", offset=5 * 8)
    assert np.array_equal(full[5], part)
    st = [synth.stream_id("kv", i) for i in range(4)]
    many = synth.normal_streams(st, 16, 1, 1.0, "bf16")
    for i in range(4):
        assert np.array_equal(many[i], synth.normal((16,), 1, st[i], 1.0, "bf16"))
    assert synth.stream_id("a", 1) != synth.stream_id("a", 2) != synth.stream_id("b", 1)


def test_uniform_int_range():
    u = synth.uniform_int(100000, 3, 9, 1024, 4097)
    assert u.min() >= 1024 and u.max() <= 4096 and abs(u.mean() - 2560) < 20


def test_tie_free_router_logits():
    src = Inputs(C4_MOE.replace(B=8))
    r = src.router_logits(0, 0)
    q = normal_quantiles(64)
    for row in r:
        assert np.array_equal(np.sort(row), np.sort(q))
    assert np.min(np.diff(np.sort(q))) > 0.03


def test_embedding_rows_match_table():
    src = Inputs(C1_TINY)
    tab = src.tok_emb(1)
    rows = src.tok_emb_rows(1, [3, 0, 511])
    assert np.array_equal(rows, tab[[3, 0, 511]])
    assert np.array_equal(src.pos_emb(rows=[5, 7]), src.pos_emb()[[5, 7]])
