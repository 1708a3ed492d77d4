"""Pins of the oracle's MoE FFN: the dense masked formulation in fp64 (the
form grouped GEMMs replace), special cases and metamorphic relations."""
import numpy as np
import pytest
import torch

import oracle
import workloads

torch.set_num_threads(4)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _layer(wl, device="cpu"):
    x, logits = wl.activations(device)
    ws = wl.weights(device)
    ids, w = oracle.route(logits.numpy(), wl.k, wl.score)
    return x, logits, ws, ids, w


def _oracle_moe(wl, x, ws, ids, w, **kw):
    if wl.quant == "bf16":
        w13 = [_bits(ws["w13"][e]) for e in range(wl.E)]
        w2 = [_bits(ws["w2"][e]) for e in range(wl.E)]
        s13 = s2 = None
    else:
        w13 = [ws["w13"][e].numpy() for e in range(wl.E)]
        w2 = [ws["w2"][e].numpy() for e in range(wl.E)]
        s13 = [ws["w13_scale"][e].numpy() for e in range(wl.E)]
        s2 = [ws["w2_scale"][e].numpy() for e in range(wl.E)]
    return oracle.moe(_bits(x), ids, w, w13, w2, s13, s2, quant=wl.quant, **kw)


def _mx_dequant(codes, scales):
    """fp64 values of an MXFP4 matrix: nibbles through the E2M1 table (pinned
    against the format's field definition) times 2^(E8M0 code - 127)."""
    table = torch.from_numpy(oracle.fp4_decode(np.arange(16)).astype(np.float64))
    lo, hi = (codes & 15).long(), (codes >> 4).long()
    vals = torch.stack([table[lo], table[hi]], dim=-1).reshape(*codes.shape[:-1], -1)
    exp = scales.double() - 127
    return vals * torch.pow(2.0, exp).repeat_interleave(32, -1)


def _mx_fake_quant(v):
    """Quantise-dequantise rows of v in MXFP4 blocks of 32 (the pinned codec)."""
    shp = v.shape
    blocks = v.float().reshape(-1, 32).numpy()
    out = np.stack([oracle.mx_quant_group(b)[2] for b in blocks])
    return torch.from_numpy(out.astype(np.float64)).reshape(shp)


def _dequant_weights(wl, ws):
    """fp64 weights [E, 2f, d], [E, d, f] from the stored values, via torch's
    e4m3 decoding (a library routine independent of the oracle's codec)."""
    if wl.quant == "bf16":
        return ws["w13"].double(), ws["w2"].double()
    if wl.quant == "mxfp4":
        return _mx_dequant(ws["w13"], ws["w13_scale"]), _mx_dequant(ws["w2"], ws["w2_scale"])
    c13 = ws["w13"].view(torch.float8_e4m3fn).double()
    c2 = ws["w2"].view(torch.float8_e4m3fn).double()
    if wl.quant == "fp8_token":
        return c13 * ws["w13_scale"].double()[:, :, None], c2 * ws["w2_scale"].double()[:, :, None]
    s13 = ws["w13_scale"].double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    s2 = ws["w2_scale"].double().repeat_interleave(128, 1).repeat_interleave(128, 2)
    return c13 * s13, c2 * s2


def _torch_fake_quant(v, group):
    """Quantise-dequantise rows of v in groups with torch's e4m3 cast."""
    shp = v.shape
    g = v.reshape(-1, group).float()
    amax = g.abs().amax(1, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (g / s).clamp(-448, 448).to(torch.float8_e4m3fn).float()
    return (q.double() * s.double()).reshape(shp)


def dense_masked_reference(wl, x, ws, ids, w, round_h):
    """y = sum_e M[:, e] * FFN_e(X) over ALL experts, fp64 matmuls, with
    M[t, e] = w[t, j] if e = ids[t, j] else 0."""
    X = x.double()
    W13, W2 = _dequant_weights(wl, ws)
    group = {"fp8_token": None, "fp8_block": 128}.get(wl.quant)
    if wl.quant == "mxfp4":
        X = _mx_fake_quant(x.float())
    elif wl.quant != "bf16":
        X = _torch_fake_quant(x.float(), wl.d if group is None else group)
    M = torch.zeros(wl.T, wl.E, dtype=torch.float64)
    for j in range(wl.k):
        M[torch.arange(wl.T), torch.from_numpy(ids[:, j]).long()] = torch.from_numpy(w[:, j]).double()
    y = torch.zeros(wl.T, wl.d, dtype=torch.float64)
    for e in range(wl.E):
        g = X @ W13[e, :wl.f].T
        u = X @ W13[e, wl.f:].T
        h = g * torch.sigmoid(g) * u
        if round_h:
            h = h.float().to(torch.bfloat16).double()
            if wl.quant == "mxfp4":
                h = _mx_fake_quant(h)
            elif wl.quant != "bf16":
                h = _torch_fake_quant(h, wl.f if group is None else group)
        y += M[:, e:e + 1] * (h @ W2[e].T)
    return y


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / np.linalg.norm(b)


SHAPES = [
    workloads.get("tiny"),
    workloads.Workload("t2", T=9, d=128, f=128, E=3, k=3, seed=7),
    workloads.Workload("t3", T=12, d=256, f=128, E=6, k=2, score="sigmoid", logits="zipf", seed=8),
    workloads.Workload("t4", T=10, d=128, f=256, E=4, k=2, quant="fp8_token", seed=9),
    workloads.Workload("t5", T=8, d=256, f=256, E=5, k=3, quant="fp8_block", score="sigmoid",
                       logits="zipf", seed=10),
    workloads.Workload("t6", T=8, d=128, f=96, E=4, k=2, quant="mxfp4", seed=11),
]


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: w.name)
def test_oracle_matches_dense_masked_fp64_unrounded(wl):
    x, _, ws, ids, w = _layer(wl)
    y, _ = _oracle_moe(wl, x, ws, ids, w, h_exact=True)
    if wl.quant == "bf16":
        ref = dense_masked_reference(wl, x, ws, ids, w, round_h=False).numpy()
        assert _rel(y, ref) < 1e-5
        assert np.max(np.abs(y - ref)) < 1e-5 * np.abs(ref).max() * 4
    else:
        # unrounded h still sees quantised activations and weights
        ref = dense_masked_reference(wl, x, ws, ids, w, round_h=False).numpy()
        assert _rel(y, ref) < 1e-5


@pytest.mark.parametrize("wl", SHAPES, ids=lambda w: w.name)
def test_oracle_matches_dense_masked_fp64_with_h_rounding(wl):
    x, _, ws, ids, w = _layer(wl)
    y, out = _oracle_moe(wl, x, ws, ids, w)
    ref = dense_masked_reference(wl, x, ws, ids, w, round_h=True).numpy()
    y_exact, _ = _oracle_moe(wl, x, ws, ids, w, h_exact=True)
    gap = _rel(y_exact, ref)           # what skipping the h rounding would cost
    assert _rel(y, ref) < 2e-5
    assert gap > 10 * _rel(y, ref)     # so the rounding step is really applied
    # out is y rounded to bf16
    assert np.array_equal(out, oracle.f32_to_bf16_bits(y).reshape(out.shape))


def test_single_expert_is_a_dense_swiglu_ffn():
    wl = workloads.Workload("e1", T=6, d=128, f=128, E=1, k=1, seed=12)
    x, _, ws, ids, w = _layer(wl)
    assert np.all(ids == 0) and np.all(w == 1.0)
    y, _ = _oracle_moe(wl, x, ws, ids, w, h_exact=True)
    X = x.double()
    g = torch.nn.functional.linear(X, ws["w13"][0, :128].double())
    u = torch.nn.functional.linear(X, ws["w13"][0, 128:].double())
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, ws["w2"][0].double())
    assert _rel(y, ref.numpy()) < 1e-5


def test_zero_input_gives_zero_output():
    wl = SHAPES[0]
    x, _, ws, ids, w = _layer(wl)
    y, out = _oracle_moe(wl, torch.zeros_like(x), ws, ids, w)
    assert not y.any() and not (out & 0x7FFF).any()


@pytest.mark.parametrize("wl", [SHAPES[0], SHAPES[3], SHAPES[5]], ids=lambda w: w.name)
def test_metamorphic_down_scale_by_two_is_exact(wl):
    x, _, ws, ids, w = _layer(wl)
    y, _ = _oracle_moe(wl, x, ws, ids, w)
    ws2 = dict(ws)
    if wl.quant == "bf16":
        ws2["w2"] = (ws["w2"].float() * 2).to(torch.bfloat16)
    elif wl.quant == "mxfp4":
        ws2["w2_scale"] = ws["w2_scale"] + 1       # E8M0: one more binade
    else:
        ws2["w2_scale"] = ws["w2_scale"] * 2
    y2, _ = _oracle_moe(wl, x, ws2, ids, w)
    assert np.array_equal(y2, 2 * y)


def test_metamorphic_token_permutation_duplicates_and_expert_relabel():
    wl = SHAPES[0]
    x, logits, ws, ids, w = _layer(wl)
    y, _ = _oracle_moe(wl, x, ws, ids, w)
    rng = np.random.default_rng(4)
    # token permutation with a duplicated row
    perm = rng.permutation(wl.T)
    perm[-1] = perm[0]
    xp = x[torch.from_numpy(perm)]
    idp, wp = oracle.route(logits.numpy()[perm], wl.k, wl.score)
    yp, _ = _oracle_moe(wl, xp, ws, idp, wp)
    assert np.array_equal(yp, y[perm])
    # expert relabelling: permute the experts and the logits' columns together
    sigma = rng.permutation(wl.E)            # new expert i is old expert sigma[i]
    ws_r = {k: (v[torch.from_numpy(sigma)] if v is not None else None) for k, v in ws.items()}
    idr, wr = oracle.route(logits.numpy()[:, sigma], wl.k, wl.score)
    assert np.array_equal(sigma[idr], ids)
    # the softmax denominator is summed in another order: weights agree to ulps
    assert np.allclose(wr, w, rtol=1e-6, atol=0)
    yr, _ = _oracle_moe(wl, x, ws_r, idr, w)
    assert np.array_equal(yr, y)


def test_token_subset_matches_full_run():
    wl = SHAPES[1]
    x, _, ws, ids, w = _layer(wl)
    y, out = _oracle_moe(wl, x, ws, ids, w)
    sub = np.array([4, 0, 8], np.int32)
    ys, outs = _oracle_moe(wl, x, ws, ids, w, tokens=sub)
    assert np.array_equal(ys, y[sub]) and np.array_equal(outs, out[sub])
    # thread count does not change the result
    y1, _ = _oracle_moe(wl, x, ws, ids, w, threads=1)
    assert np.array_equal(y1, y)
