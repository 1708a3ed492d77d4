"""The sweep tests' comparison with h rounding ties, on the CPU.

rel_err with the oracle's per-row slack must accept an output that differs
from the oracle's only by rounding a reported tie the other way, and must
still catch a planted error in a row without ties, or one in a row with
ties that exceeds what its ties can move."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import TOL, bf16_to_f64, bits, host_experts, oracle_layer, rel_err

torch.set_num_threads(4)

WL = workloads.Workload("slack", T=48, d=128, f=256, E=4, k=2, quant="fp8_block", seed=77)


@pytest.fixture(scope="module")
def layer():
    x, logits = WL.activations("cpu")
    ws = WL.weights("cpu")
    slack = {}
    ref, ids, w = oracle_layer(WL, x, logits, ws, slack=slack)
    return x, ws, ref, ids, w, slack


def _flipped(x, ws, ids, w, t, j, n):
    """The oracle's output row of token t with h element n of its j-th
    assignment rounded to the other bf16 neighbour."""
    w13, w2, s13, s2 = host_experts(WL, ws, sorted(set(ids[t].tolist())))
    _, out = oracle.moe(bits(x), ids, w, w13, w2, s13, s2, quant=WL.quant,
                        tokens=np.array([t], np.int32), h_flip=[j * WL.f + n])
    return bf16_to_f64(out)[0]


def test_slack_accepts_the_other_rounding_of_a_tie(layer):
    x, ws, ref, ids, w, slack = layer
    assert slack, "the seeded layer has rows with rounding ties"
    _, _, ties = oracle.moe(bits(x), ids, w, *host_experts(WL, ws, range(WL.E)), quant=WL.quant,
                            tie_band=2.0 ** -16)
    t, j, n = (int(v) for v in ties[0])
    assert t in slack
    y = ref.copy()
    y[t] = _flipped(x, ws, ids, w, t, j, n)
    assert not np.array_equal(y[t], ref[t])
    assert rel_err(y, ref, slack)[0] <= 2.0 ** -7     # the two bf16 roundings: one step at most
    assert rel_err(y, ref, slack)[0] < rel_err(y, ref)[0]


def test_slack_still_catches_planted_errors(layer):
    x, ws, ref, ids, w, slack = layer
    rms = float(np.sqrt(np.mean(ref ** 2)))
    clean = [r for r in range(WL.T) if r not in slack]
    assert clean, "the seeded layer has rows without ties"
    # a row without ties: no allowance at all
    y = ref.copy()
    y[clean[0], 5] += 2 * TOL[WL.quant] * max(abs(ref[clean[0], 5]), rms)
    assert rel_err(y, ref, slack)[0] > TOL[WL.quant]
    # a row with ties: an error beyond the sum of its ties' effects
    r = next(iter(slack))
    c = int(np.argmin(slack[r]))
    y = ref.copy()
    y[r, c] += slack[r][c] + 2 * TOL[WL.quant] * max(abs(ref[r, c]), rms)
    assert rel_err(y, ref, slack)[0] > TOL[WL.quant]
