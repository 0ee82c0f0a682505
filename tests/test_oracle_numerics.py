"""Pins for oracle.numerics: bf16 and e4m3fn rounding / decoding.

Checked against torch's independent bf16 / float8_e4m3fn conversions, brute
force nearest-value search, and format constants of the OCP 8-bit float
definition (largest finite 448, smallest subnormal 2**-9, smallest normal
2**-6, one = 0x38).
"""

import numpy as np
import torch

from oracle import numerics


def _all_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    return codes, numerics.e4m3_decode(codes)


def test_bf16_round_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38], np.float32),
    ])
    # exact ties: midpoints between adjacent bf16 values
    base = rng.standard_normal(5000).astype(np.float32)
    base_bits = (base.view(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, base_bits.view(np.float32)])
    ours = numerics.bf16_bits(numerics.bf16_round(x.astype(np.float64)))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_is_nearest_from_fp64():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(50000) * 3.0
    r = numerics.bf16_round(x)
    # neighbours: truncate toward zero to bf16 and step one ulp outward
    f32 = x.astype(np.float32)
    lo_bits = (f32.view(np.uint32) & 0xFFFF0000)
    lo = lo_bits.view(np.float32).astype(np.float64)
    hi = (lo_bits + 0x10000).view(np.float32).astype(np.float64)
    cand = np.stack([lo, hi, (lo_bits - 0x10000).view(np.float32).astype(np.float64)])
    err = np.abs(cand - x[None, :])
    best = cand[np.argmin(err, axis=0), np.arange(x.size)]
    assert np.all(np.abs(r - x) <= np.abs(best - x))
    # representable
    assert np.array_equal(numerics.bf16_from_bits(numerics.bf16_bits(r)), r)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes, vals = _all_e4m3_values()
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(vals), nan)
    assert np.array_equal(vals[~nan], ref[~nan])
    assert nan.sum() == 2                       # 0x7F and 0xFF only


def test_e4m3_format_constants():
    d = numerics.e4m3_decode
    assert d(np.uint8(0x7E)) == 448.0
    assert d(np.uint8(0x01)) == 2.0 ** -9
    assert d(np.uint8(0x08)) == 2.0 ** -6
    assert d(np.uint8(0x38)) == 1.0
    assert d(np.uint8(0xFE)) == -448.0
    assert d(np.uint8(0x80)) == 0.0


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(100000),
        rng.standard_normal(50000) * 1e-2,
        rng.standard_normal(20000) * 1e-3,
    ]).astype(np.float32)
    # exact midpoints between adjacent finite codes (ties to even)
    _, vals = _all_e4m3_values()
    pos = np.sort(vals[(vals >= 0) & np.isfinite(vals)])
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32)])
    ours = numerics.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_is_nearest_even_by_brute_force():
    codes, vals = _all_e4m3_values()
    finite = np.isfinite(vals)
    fc, fv = codes[finite], vals[finite]
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-500, 500, 3000), rng.standard_normal(3000) * 0.05,
                        [1000.0, -1000.0, 449.0, 464.0, 465.0, 2.0 ** -10, 3 * 2.0 ** -11]])
    enc = numerics.e4m3_encode(x)
    for xi, ci in zip(x, enc):
        xs = np.clip(xi, -448.0, 448.0)             # saturation
        err = np.abs(fv - xs)
        best = np.flatnonzero(err == err.min())
        # among equally near codes, the even mantissa wins; +0 preferred over -0
        cands = [c for c in fc[best]]
        if len(cands) > 1:
            nz = [c for c in cands if (c & 0x7) % 2 == 0 and c != 0x80]
            cands = nz or cands
        dv = numerics.e4m3_decode(np.uint8(ci))
        assert abs(dv - xs) == err.min(), (xi, ci)
        if len(best) > 1 and np.abs(fv[best]).max() > 0:
            assert (int(ci) & 0x1) == 0, (xi, ci)


def test_e4m3_nan_and_saturation():
    enc = numerics.e4m3_encode(np.array([np.nan, 1e9, -1e9, 448.0, 460.0]))
    assert list(enc) == [0x7F, 0x7E, 0xFE, 0x7E, 0x7E]



def test_probability_rounding_bound_holds_for_the_kernels_scaling():
    """The e4m3 error bound the GPU tests allow (helpers.prob_rounding_bound)
    against brute force: probabilities scaled as the e4m3 kernel scales them,
    P' = 2^(x - m + 6) with a running max m anywhere in [M - 2.5, M + 1) (it
    never passes the row's max M by a whole unit, and the overflow guard keeps
    every P' at or below 2^8.5, so m never lies more than 2.5 below a key the
    row has seen), rounded by the oracle's e4m3 encoder and brought
    back to units of p = 2^(x - M): every key's error is within its share of
    the bound (the bound with a one-hot |v| column per key), the worst case
    comes within 10 % of it, and the subnormal range is reached."""
    from helpers import prob_rounding_bound
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0.0, 4.0, 2000), rng.uniform(-20.0, 0.0, 2000), [0.0]])
    p = 2.0 ** (x - x.max())
    e = prob_rounding_bound(p[None, :], np.eye(len(p)))[0] * p.sum()    # per key
    worst = 0.0
    saw_subnormal = False
    for shift in np.linspace(-2.5, 0.999, 36):       # m - M
        scale = 2.0 ** (6.0 - shift)                  # P' = scale * p
        pq = p * scale
        err = np.abs(numerics.e4m3_decode(numerics.e4m3_encode(pq)) / scale - p)
        assert np.all(err <= e * (1 + 1e-12))
        worst = max(worst, float(np.max(err / e)))
        saw_subnormal |= bool(np.any((pq > 0) & (pq < 2.0 ** -6)))
    assert worst > 0.9 and saw_subnormal
