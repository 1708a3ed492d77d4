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


# ---- MXFP4 (E2M1 elements, E8M0 block scales) ---------------------------

def _minifloat_table(ebits: int, mbits: int, bias: int):
    """Every code of a sign / exponent / mantissa float decoded from the field
    definition: exponent 0 is subnormal (m / 2^mbits * 2^(1 - bias)), the
    rest normal ((1 + m / 2^mbits) * 2^(e - bias)); special values ignored."""
    n = 1 << (1 + ebits + mbits)
    out = np.empty(n, np.float64)
    for c in range(n):
        s = c >> (ebits + mbits)
        e = (c >> mbits) & ((1 << ebits) - 1)
        m = c & ((1 << mbits) - 1)
        frac = m / (1 << mbits)
        v = frac * 2.0 ** (1 - bias) if e == 0 else (1 + frac) * 2.0 ** (e - bias)
        out[c] = -v if s else v
    return out


def test_generic_minifloat_decoder_matches_torch_fp8():
    """The field decoder used to pin E2M1 reproduces torch's e4m3fn and e5m2."""
    e4m3 = _torch_e4m3_table()
    gen = _minifloat_table(4, 3, 7)
    ok = ~np.isnan(e4m3)
    assert np.array_equal(gen[ok], e4m3[ok].astype(np.float64))
    e5m2 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    ok = np.isfinite(e5m2)
    assert np.array_equal(_minifloat_table(5, 2, 15)[ok], e5m2[ok])


def test_fp4_decode_all_codes():
    ours = oracle.fp4_decode(np.arange(16)).astype(np.float64)
    assert np.array_equal(ours, _minifloat_table(2, 1, 1))
    assert list(ours[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute_fp4(values):
    """Nearest E2M1 code by exhaustive search; ties go to the even code;
    magnitudes of 6 and above saturate; the sign of zero is kept."""
    table = _minifloat_table(2, 1, 1)
    out = []
    for v in values:
        v = float(v)
        neg = np.signbit(v)
        a = abs(v)
        if a >= 6.0:
            out.append(15 if neg else 7)
            continue
        best = min(range(8), key=lambda c: (abs(table[c] - a), c & 1))
        out.append(best | (8 if neg else 0))
    return np.array(out, np.uint8)


def test_fp4_encode_brute_force_midpoints_and_random():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    mids = [(a + b) / 2 for a, b in zip(mags, mags[1:])]
    vals = []
    for m in mags + mids + [6.5, 7.0, 8.0, 100.0, 1e30]:
        m32 = np.float32(m)
        vals += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(np.inf))]
    vals = np.array(vals, np.float32)
    vals = np.concatenate([vals, -vals, np.random.default_rng(3).uniform(-9, 9, 4000).astype(np.float32)])
    assert np.array_equal(oracle.fp4_encode(vals), _brute_fp4(vals))
    assert oracle.fp4_encode([-0.0])[0] == 8 and oracle.fp4_encode([0.0])[0] == 0


def test_mx_block_scale_rule_and_error_bound():
    """Shared exponent E = floor(log2(amax)) - 2 (numpy frexp), E8M0 code E + 127
    (torch's E8M0 encoding of 2^E), dequantised value = decode(code) * 2^E, and
    every element within half the E2M1 spacing unless it saturates at 6 * 2^E."""
    rng = np.random.default_rng(5)
    blocks = []
    for scale in [1e-30, 1e-6, 0.01, 1.0, 3.0, 1e4, 1e30]:
        blocks.append(rng.standard_normal(32) * scale)
    for p in [-20, 0, 3, 17]:   # amax exactly a power of two, and just below one
        b = rng.uniform(-1, 1, 32) * 2.0 ** p
        b[7] = 2.0 ** p
        blocks.append(b.copy())
        b[7] = np.nextafter(np.float32(2.0 ** p), np.float32(0))
        blocks.append(b)
    blocks.append(np.zeros(32))
    table = _minifloat_table(2, 1, 1)
    for b in blocks:
        b = b.astype(np.float32)
        q, code, deq = oracle.mx_quant_group(b)
        amax = float(np.max(np.abs(b)))
        if amax == 0:
            assert code == 0 and not deq.any()
            continue
        E = int(np.frexp(np.float64(amax))[1]) - 1 - 2
        assert code == E + 127
        ref_code = torch.tensor([2.0 ** E], dtype=torch.float64).to(torch.float8_e8m0fnu).view(torch.uint8)
        assert code == int(ref_code)
        assert np.array_equal(deq.astype(np.float64), table[q] * 2.0 ** E)
        r = np.abs(b.astype(np.float64)) / 2.0 ** E
        spacing = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
        sat = r >= 6
        err = np.abs(deq.astype(np.float64) - b) / 2.0 ** E
        assert np.all(err[~sat] <= spacing[~sat] / 2)
        assert np.all(np.abs(deq[sat]) == np.float32(6.0 * 2.0 ** E))


def test_mx_quant_rows_packs_blocks():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((5, 96)).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.mx_quant_rows(xb)
    assert codes.shape == (5, 48) and scales.shape == (5, 3)
    xf = x.float().numpy()
    for r in range(5):
        for blk in range(3):
            q, c, _ = oracle.mx_quant_group(xf[r, blk * 32:(blk + 1) * 32])
            assert scales[r, blk] == c
            packed = codes[r, blk * 16:(blk + 1) * 16]
            assert np.array_equal(packed & 15, q[0::2]) and np.array_equal(packed >> 4, q[1::2])


def _golden_mx_blocks():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "mx_worked_blocks.json")
    with open(path) as fh:
        doc = json.load(fh)
    out = []
    for b in doc["blocks"]:
        if "bf16_bits" in b:
            bits = np.array(b["bf16_bits"], np.uint16)
        else:
            v = np.array(b["values"], np.float32)
            bits = oracle.f32_to_bf16_bits(v).reshape(v.shape)
            # every value is exact in bf16 (the blocks are meant for a bf16 quantiser too)
            assert np.array_equal(oracle.bf16_bits_to_f32(bits).view(np.uint32), v.view(np.uint32))
        out.append((b["name"], bits, b["scale"], np.array(b["codes"], np.uint8)))
    return out


def test_mx_worked_blocks_golden():
    """Hand-worked MXFP4 blocks (tests/golden/mx_worked_blocks.json, each
    step written out from the OCP MX definition): amax exactly 4 * 2^j and
    6 * 2^j, just below 8 * 2^j and 4 * 2^j, a subnormal amax and an all-zero
    block. The oracle's block rule and its row quantiser reproduce the
    scale codes and every element code."""
    blocks = _golden_mx_blocks()
    for name, bits, scale, codes in blocks:
        q, c, deq = oracle.mx_quant_group(oracle.bf16_bits_to_f32(bits))
        assert c == scale, name
        assert np.array_equal(q, codes), (name, q, codes)
    rows = np.stack([b for _, b, _, _ in blocks])
    packed, scales = oracle.mx_quant_rows(rows)
    assert np.array_equal(scales[:, 0], [s for _, _, s, _ in blocks])
    for r, (_, _, _, codes) in enumerate(blocks):
        assert np.array_equal(packed[r] & 15, codes[0::2]) and np.array_equal(packed[r] >> 4, codes[1::2])
