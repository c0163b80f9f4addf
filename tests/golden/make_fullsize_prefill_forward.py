"""Writes tests/golden/fullsize_prefill_forward_seq0.npz: the oracle's
results for sequence 0 of the 16 x 2048-token prompts through the dense
1.3B model (24 layers, d 2048), the expected values of the full-size prefill
and dual-forward GPU tests. Calls only the oracle and the seeded input
generator; takes tens of minutes on the CPU, so the GPU tests read its
output instead of recomputing it.

    python tests/golden/make_fullsize_prefill_forward.py

Stored:
  kv_pos [P], kv_layers [NL]: sampled cache positions and layers
  k, v [NL, P, H, Dh] uint16: bf16 bits of the cache entries the oracle's
    forward (whose primary half is the prefill) writes there
  kv_bound [L]: per layer, D_l = the largest excess over one bf16 ulp
    (2^-7 |x|) between the oracle's cache and the oracle's cache with every
    K/V value multiplied by a seeded (1 +- u), u uniform in [0, 2^-17],
    before its rounding (the size of the GPU's bf16 hi/lo operand error),
    over the sampled entries: how far a correct implementation's deeper
    entries may drift through one-ulp rounding flips in earlier layers
  fw_pos [Q]: sampled forward positions; fw_ids [Q, NV]: sampled vocabulary
    ids per position (the 32 largest p_mix entries, then seeded ones)
  fw_logits [Q, 2, NV] float64: both flows' logits at those ids
  fw_pmix [Q, NV] float64, fw_alpha [Q], fw_next [Q] int64
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import dualflow as odf                        # noqa: E402
from synth.workloads import FORWARD_DENSE, PREFILL_DENSE, Inputs   # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fullsize_prefill_forward_seq0.npz")
SEQ = 0
KV_POS = [0, 1, 511, 512, 1023, 1024, 1535, 1536, 2047]
KV_LAYERS = [0, 1, 11, 12, 22, 23]
FW_POS = [0, 511, 512, 1023, 1024, 1535, 1536, 2047]
N_IDS = 1024


def _bits(x):
    """bf16 bit patterns of values that are bf16 already."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def main():
    t0 = time.time()
    c = FORWARD_DENSE
    src = Inputs(c)
    toks = src.prompt()[SEQ:SEQ + 1]
    model = odf.Model(src)
    cache = odf.Cache(c, [SEQ], src)
    fw = odf.forward_dual(model, cache, toks)
    print(f"forward done in {time.time() - t0:.0f} s", flush=True)
    k = np.stack([cache.layer(l)[0][0][:, KV_POS].transpose(1, 0, 2) for l in KV_LAYERS])   # [NL, P, H, Dh]
    v = np.stack([cache.layer(l)[1][0][:, KV_POS].transpose(1, 0, 2) for l in KV_LAYERS])
    rng = np.random.default_rng(2048)
    ids = np.zeros((len(FW_POS), N_IDS), dtype=np.int64)
    for i, t in enumerate(FW_POS):
        top = np.argsort(-fw.p_mix[0, t], kind="stable")[:32]
        rest = np.setdiff1d(rng.permutation(c.V), top)[:N_IDS - 32]
        ids[i] = np.concatenate([top, rest])
    fw_logits = np.stack([fw.logits[0, t][:, ids[i]] for i, t in enumerate(FW_POS)])
    fw_pmix = np.stack([fw.p_mix[0, t][ids[i]] for i, t in enumerate(FW_POS)])
    fw_alpha = fw.alpha[0, FW_POS]
    fw_next = fw.next_tok[0, FW_POS]
    ref_all = [tuple(a.copy() for a in cache.layer(l)) for l in range(c.L)]
    del fw, cache

    # the same prompt through the prefill with every K/V value perturbed before its rounding
    t1 = time.time()
    cp = PREFILL_DENSE
    srcp = Inputs(cp)
    assert np.array_equal(srcp.prompt()[SEQ:SEQ + 1], toks)
    prng = np.random.default_rng(17)
    orig = odf.round_to

    def perturbed(x, dtype):
        x = np.asarray(x, dtype=np.float64)
        return orig(x * (1.0 + prng.uniform(-2.0 ** -17, 2.0 ** -17, x.shape)), dtype)

    odf.round_to = perturbed
    try:
        alt = odf.Cache(cp, [SEQ], srcp)
        odf.prefill_primary(odf.Model(srcp), alt, toks)
    finally:
        odf.round_to = orig
    print(f"perturbed prefill done in {time.time() - t1:.0f} s", flush=True)
    bound = np.zeros(c.L)
    for l in range(c.L):
        for x, y in zip(ref_all[l], alt.layer(l)):
            a, b = x[0][:, KV_POS], y[0][:, KV_POS]
            bound[l] = max(bound[l], float(np.max(np.abs(b - a) - 2.0 ** -7 * np.abs(a))))
    np.savez(OUT, kv_pos=np.array(KV_POS), kv_layers=np.array(KV_LAYERS), k=_bits(k), v=_bits(v),
             kv_bound=bound, fw_pos=np.array(FW_POS), fw_ids=ids, fw_logits=fw_logits, fw_pmix=fw_pmix,
             fw_alpha=fw_alpha, fw_next=fw_next)
    print(f"wrote {OUT} ({os.path.getsize(OUT)} bytes); D_l by layer: {np.array2string(bound, precision=2)}")


if __name__ == "__main__":
    main()
