"""Pins of the oracle's bf16 rounding ties of h.

The fp32 sums of the gate and up products have no order fixed by the pages,
so an h whose value lies within fp32 rounding noise of the midpoint between
two bf16 values may round either way; when that decides its quantisation
group's scale, every code of the group moves, and when it decides the
element's own code, that code moves. The oracle reports such elements and
can round listed ones the other way. These tests pin both: a flip moves
exactly one h element by exactly one bf16 step toward its unrounded value,
and the report equals a brute-force enumeration (fp64 h, bf16 brackets by
truncation, group scales from their definitions, e4m3 codes from torch's
cast)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_oracle_moe import _bits, _dequant_weights, _layer, _mx_fake_quant, _oracle_moe, _torch_fake_quant

torch.set_num_threads(4)


def _h64(wl, x, ws, t, e):
    """fp64 h = silu(x Wg) * (x Wu) of token t through expert e (the input
    quantised as the layer does)."""
    W13, _ = _dequant_weights(wl, ws)
    X = x[t:t + 1].double()
    if wl.quant == "mxfp4":
        X = _mx_fake_quant(x[t:t + 1].float())
    elif wl.quant == "fp8_token":
        X = _torch_fake_quant(x[t:t + 1].float(), wl.d)
    elif wl.quant == "fp8_block":
        X = _torch_fake_quant(x[t:t + 1].float(), 128)
    g = X @ W13[e, :wl.f].T
    u = X @ W13[e, wl.f:].T
    return (g * torch.sigmoid(g) * u)[0].numpy()


def _bracket(v):
    """The two bf16 values around the fp64 values v: truncation toward zero
    of the fp32 value, and one step of the bf16 mantissa away from zero."""
    f = np.asarray(v, np.float32)
    b = f.view(np.uint32) & np.uint32(0xFFFF0000)
    tz = b.view(np.float32).astype(np.float64)
    away = (b + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    return tz, away


def _bf16(v):
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).double().numpy()


def test_flip_moves_one_h_element_one_bf16_step_toward_its_value():
    wl = workloads.Workload("flip", T=6, d=128, f=128, E=3, k=2, seed=31)
    x, _, ws, ids, w = _layer(wl)
    y0, _ = _oracle_moe(wl, x, ws, ids, w)
    _, W2 = _dequant_weights(wl, ws)
    for (i, j, n) in [(0, 0, 0), (4, 1, 77), (5, 0, 127)]:
        y1, _ = _oracle_moe(wl, x, ws, ids, w, h_flip=[(i * wl.k + j) * wl.f + n])
        others = np.arange(wl.T) != i
        assert np.array_equal(y1[others], y0[others])
        e = int(ids[i, j])
        col = W2[e][:, n].numpy()
        dy = (y1[i].astype(np.float64) - y0[i]) / float(w[i, j])
        delta = float(dy @ col / (col @ col))          # the change of h[n]
        assert np.abs(dy - delta * col).max() < 1e-5 * np.abs(y0[i]).max()
        h = _h64(wl, x, ws, i, e)[n]
        r = _bf16(h)
        ulp = 2.0 ** (np.floor(np.log2(abs(r))) - 7)
        assert abs(abs(delta) - ulp) < 1e-3 * ulp
        assert np.sign(delta) == np.sign(h - r)


def _scale_key(quant, a):
    if quant != "mxfp4":
        return a
    return -127 if a == 0 else max(-127, min(127, int(np.floor(np.log2(a))) - 2))


def _code(quant, v, amax):
    """The code of v in a group whose largest magnitude is amax."""
    if quant == "mxfp4":
        return int(oracle.fp4_encode(np.array([np.ldexp(v, -_scale_key(quant, amax))]))[0])
    s = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448.0)
    q = torch.tensor([np.float32(v) / s], dtype=torch.float32).clamp(-448, 448)
    return int(q.to(torch.float8_e4m3fn).view(torch.uint8)[0])


@pytest.mark.parametrize("wl", [
    workloads.Workload("ties-token", T=10, d=128, f=256, E=4, k=2, quant="fp8_token", seed=9),
    workloads.Workload("ties-block", T=8, d=256, f=256, E=5, k=3, quant="fp8_block", seed=10),
    workloads.Workload("ties-mx", T=8, d=128, f=96, E=4, k=2, quant="mxfp4", seed=11),
], ids=lambda w: w.name)
def test_reported_ties_are_the_scale_or_code_changing_roundings(wl):
    x, _, ws, ids, w = _layer(wl)
    group = {"fp8_token": wl.f, "fp8_block": 128, "mxfp4": 32}[wl.quant]
    # a band of 1 admits every inexact element, leaving the scale rule alone
    _, _, got = _oracle_moe(wl, x, ws, ids, w, tie_band=1.0)
    want = []
    for t in range(wl.T):
        for j in range(wl.k):
            h = _h64(wl, x, ws, t, int(ids[t, j]))
            r = _bf16(h)
            tz, away = _bracket(h)
            other = np.where(r == tz, away, tz)
            for g0 in range(0, wl.f, group):
                blk = np.abs(r[g0:g0 + group])
                key = _scale_key(wl.quant, blk.max())
                for n in range(g0, g0 + group):
                    if h[n] == r[n]:
                        continue
                    alt = blk.copy()
                    alt[n - g0] = abs(other[n])
                    if _scale_key(wl.quant, alt.max()) != key or \
                            _code(wl.quant, r[n], blk.max()) != _code(wl.quant, other[n], blk.max()):
                        want.append((t, j, n))
    assert len(want) > 0
    assert sorted(map(tuple, got.tolist())) == sorted(want)
    # no band, no report; a narrow band reports a subset
    _, _, none = _oracle_moe(wl, x, ws, ids, w, tie_band=1e-30)
    assert none.shape[0] == 0
    _, _, some = _oracle_moe(wl, x, ws, ids, w, tie_band=2.0 ** -10)
    assert set(map(tuple, some.tolist())) <= set(want)


def test_scale_ties_requantise_their_group_and_code_ties_move_one_element():
    """Rounding a group's largest element the other way moves the output
    through many codes of the group (not along one column of the down
    projection); rounding any other reported element moves that element's
    code alone (exactly along its column)."""
    wl = workloads.Workload("ties-effect", T=8, d=256, f=256, E=5, k=3, quant="fp8_block", seed=10)
    x, _, ws, ids, w = _layer(wl)
    y0, _, ties = _oracle_moe(wl, x, ws, ids, w, tie_band=1.0)
    _, W2 = _dequant_weights(wl, ws)
    seen = set()
    for i, j, n in ties.tolist():
        e = int(ids[i, j])
        h = _bf16(_h64(wl, x, ws, i, e))
        g0 = n - n % 128
        is_max = int(np.argmax(np.abs(h[g0:g0 + 128]))) == n - g0
        if is_max in seen:
            continue
        seen.add(is_max)
        y1, _ = _oracle_moe(wl, x, ws, ids, w, h_flip=[(i * wl.k + j) * wl.f + n])
        others = np.arange(wl.T) != i
        assert np.array_equal(y1[others], y0[others])
        dy = (y1[i].astype(np.float64) - y0[i]) / float(w[i, j])
        col = W2[e][:, n].numpy()
        off = np.linalg.norm(dy - (dy @ col / (col @ col)) * col) / np.linalg.norm(dy)
        if is_max:
            assert off > 0.1
        else:
            assert off < 1e-2    # fp32 summation noise of the two runs
        if len(seen) == 2:
            break
    assert seen == {True, False}
