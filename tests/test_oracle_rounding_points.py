"""Evidence for where the oracle rounds: only the appended K/V entries are
rounded to the storage dtype; projection inputs (normed rows, attention
output, GELU output) stay unrounded.

The pages fix no number format. Two readings were open: round every
projection input to bf16 as well, or keep activations in full precision.
On the 24-layer, d 2048 dense model (the 1.3B workload's shape), a relative
2^-20 perturbation of every projection input -- the size of the difference
between two equally correct fp32 summation orders -- moves one step's logits
by more than the 2e-2 logits bar when the inputs are rounded (rounding flips
of one bf16 ulp compound through the depth), and by about 1e-4 when they are
not. With rounded inputs no two correct implementations could be held to
the bar, so the oracle takes the unrounded reading. CPU only."""
import numpy as np

import pins
from gpu_util import say


def test_rounded_projection_inputs_break_the_logits_bar_at_full_depth():
    cfg = pins.R16_FULL_DEPTH
    moves = {}
    for rounded in (True, False):
        clean = pins.step_logits_under_noise(cfg, rounded, 0.0)
        noisy = pins.step_logits_under_noise(cfg, rounded, pins.R16_NOISE)
        moves[rounded] = float(np.max(np.abs(clean - noisy)))
    say(f"logit move under 2^-20 input noise: rounded inputs {moves[True]:.3e}, unrounded {moves[False]:.3e}")
    assert moves[True] > 2e-2, "rounded projection inputs stay within the logits bar"
    assert moves[False] < 1e-3, "unrounded projection inputs moved the logits"
