"""Pins of the oracle's scalar formats: bf16 rounding, OCP e4m3 codec and the
amax/448 quantiser, each checked against torch's own casts or brute force."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _torch_e4m3_table():
    """All 256 codes decoded by torch's float8_e4m3fn (an independent library)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties: low half 0x8000 with even and odd upper halves
        (np.array([0x3f808000, 0x3f818000, 0xbf808000, 0x7f7f8000, 0x00008000],
                  dtype=np.uint32)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-45], np.float32),
    ]).astype(np.float32)
    ours = oracle.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes_match_torch():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = _torch_e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0 and ours[0x7E] == 448.0
    assert ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6


def _brute_force_encode(values, table):
    """Nearest finite code; ties go to the code with an even mantissa LSB;
    magnitudes above 448 saturate."""
    finite = [(c, table[c]) for c in range(256) if not np.isnan(table[c])]
    out = []
    for v in values:
        v = float(v)
        if abs(v) >= 448.0:
            out.append(0x7E | (0x80 if v < 0 else 0))
            continue
        best = None
        for c, t in finite:
            if (t < 0) != (np.signbit(v)) and t != 0:
                continue
            dist = abs(float(t) - v)
            key = (dist, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        c = best[1]
        # keep the sign of zero
        if table[c] == 0:
            c = 0x80 if np.signbit(v) else 0x00
        out.append(c)
    return np.array(out, np.uint8)


def test_e4m3_encode_brute_force_midpoints_and_random():
    table = _torch_e4m3_table()
    pos = np.sort(np.unique(table[(~np.isnan(table)) & (table >= 0)]))
    mids = (pos[1:].astype(np.float64) + pos[:-1]) / 2
    vals = []
    for m in mids:
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    rng = np.random.default_rng(1)
    vals += list((rng.standard_normal(3000) * 10.0 ** rng.uniform(-3.5, 2.8, 3000)).astype(np.float32))
    vals += [0.0, 1e-6, 2.0 ** -10, 3 * 2.0 ** -11, 447.9, 448.0, 449.0, 464.0, 470.0, 1e6]
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals])
    ours = oracle.e4m3_encode(vals)
    assert np.array_equal(ours, _brute_force_encode(vals, table))
    # torch's cast rounds to nearest even but does not saturate: clamp first.
    ref = torch.from_numpy(vals).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_nan_and_saturation():
    out = oracle.e4m3_encode(np.array([np.nan, np.inf, -np.inf, 1e30, -1e30], np.float32))
    assert out[0] & 0x7F == 0x7F
    assert list(out[1:]) == [0x7E, 0xFE, 0x7E, 0xFE]


def test_quant_group_scale_rule():
    rng = np.random.default_rng(2)
    for n in (1, 7, 128, 4096):
        v = (rng.standard_normal(n) * 3.0).astype(np.float32)
        q, s, deq = oracle.quant_group(v)
        amax = np.float32(np.abs(v).max())
        assert s == np.float32(amax / np.float32(448.0))
        # the largest magnitude maps to the largest code
        i = int(np.abs(v).argmax())
        assert q[i] & 0x7F == 0x7E
        # the codes are torch's cast of v / s (fp32 division)
        ref = torch.from_numpy(v / s).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
        assert np.array_equal(q, ref.numpy())
        # dequantised error within half a code spacing (relative 2^-4), or the subnormal step
        err = np.abs(deq - v)
        assert np.all(err <= np.maximum(np.abs(v) * 2.0 ** -4, s * 2.0 ** -10) * 1.0001)
    q, s, deq = oracle.quant_group(np.zeros(16, np.float32))
    assert s == 1.0 and not q.any() and not deq.any()


def test_quant_rows_groups():
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((5, 256)).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.quant_rows(bits, group=128)
    assert scales.shape == (5, 2)
    xf = x.float().numpy()
    for r in range(5):
        for b in range(2):
            seg = xf[r, b * 128:(b + 1) * 128]
            q, s, _ = oracle.quant_group(seg)
            assert scales[r, b] == s
            assert np.array_equal(codes[r, b * 128:(b + 1) * 128], q)
    codes_row, scales_row = oracle.quant_rows(bits, group=256)
    assert scales_row.shape == (5, 1)
    assert np.allclose(scales_row[:, 0], np.abs(xf).max(axis=1) / 448.0, rtol=1e-7, atol=0)
