"""Pins for the oracle's NF4 code table, bf16 rounding, quantizer and decoder.

Each test checks the oracle against something other than itself: the defining
property of the levels through the forward normal CDF (math.erf), torch's own
bf16 conversion, brute-force loops on tiny blocks, exact special cases and
invariants of the format.
"""
import math

import numpy as np
import pytest
import torch

from oracle import nf4


def phi(z: float) -> float:
    """Standard normal CDF through math.erf (independent of scipy's ndtri)."""
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def test_table_structure():
    T = nf4.nf4_table()
    assert T.dtype == np.float32 and T.shape == (16,)
    assert np.all(np.diff(T) > 0), "levels must be strictly ascending"
    assert T[0] == -1.0 and T[7] == 0.0 and T[15] == 1.0
    assert int(np.sum(T < 0)) == 7 and int(np.sum(T > 0)) == 8


def test_table_levels_are_normal_quantiles():
    # Level i, scaled back by the quantile of delta, must sit at its defining
    # probability: positive levels split (1/2, delta] into 8 equal steps,
    # negative levels split [1 - delta, 1/2) into 7 equal steps.
    T = nf4.nf4_levels_f64()
    delta = ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0)) / 2.0
    # z_delta from the CDF by bisection (independent inverse)
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if phi(mid) < delta:
            lo = mid
        else:
            hi = mid
    z_delta = 0.5 * (lo + hi)
    for j in range(1, 9):
        p = phi(T[7 + j] * z_delta)
        assert abs(p - (0.5 + j * (delta - 0.5) / 8.0)) < 1e-12, (j, p)
    for j in range(1, 8):
        p = phi(-T[7 - j] * z_delta)
        assert abs(p - (0.5 + j * (delta - 0.5) / 7.0)) < 1e-12, (j, p)
    # fp32 table is the fp64 levels rounded once
    assert np.array_equal(nf4.nf4_table(), T.astype(np.float32))


def test_bf16_rne_matches_torch():
    rs = np.random.default_rng(0)
    vals = np.concatenate([
        rs.standard_normal(20000).astype(np.float32),
        (rs.standard_normal(2000) * 1e-38).astype(np.float32),        # subnormals
        np.clip(rs.standard_normal(2000) * 1e38, -3.3e38, 3.3e38).astype(np.float32),  # near overflow
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1.0, -1.0], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, both parities of the kept lsb
    u = rs.integers(0, 2**31, 4000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([vals, ties[np.isfinite(ties)]])
    ours = nf4.bf16_rne_bits(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nanbits = nf4.bf16_rne_bits(np.array([np.nan], np.float32))
    assert (int(nanbits[0]) & 0x7F80) == 0x7F80 and (int(nanbits[0]) & 0x7F) != 0


def test_pack_nibble_order():
    codes = np.array([[1, 2, 3, 4, 15, 0] + [7] * 58], dtype=np.uint8)
    packed = nf4.pack_codes(codes)
    assert packed.shape == (1, 32)
    assert list(packed[0, :3]) == [0x12, 0x34, 0xF0]
    assert np.array_equal(nf4.unpack_codes(packed), codes)


def _brute_quantize_block(block):
    """Pure-Python loop over one block with fp32 scalars; ties go to the lower index."""
    T = [np.float32(t) for t in nf4.nf4_table()]
    absmax = np.float32(0.0)
    for w in block:
        a = np.float32(abs(np.float32(w)))
        if a > absmax:
            absmax = a
    codes = []
    for w in block:
        if absmax == 0:
            codes.append(7)
            continue
        v = np.float32(np.float32(w) / absmax)
        best, bestd = 0, None
        for i in range(16):
            d = np.float32(abs(np.float32(v - T[i])))
            if bestd is None or d < bestd:
                best, bestd = i, d
        codes.append(best)
    return codes, absmax


def test_quantize_brute_force():
    rs = np.random.default_rng(1)
    w = (rs.standard_normal((3, 128)) * 0.02).astype(np.float32)
    w[1, :64] = 0.0                       # an all-zero block
    w[2, 5] = -0.5                        # a dominant negative element
    # exact midpoints between levels in the normalised domain -> ties
    T = nf4.nf4_table()
    mids = ((T[:-1].astype(np.float64) + T[1:]) / 2).astype(np.float32)
    w[0, :15] = mids
    w[0, 15] = 1.0
    codes, absmax = nf4.quantize_codes(w)
    for b in range(w.size // 64):
        row, col = divmod(b * 64, 128)
        ref_codes, ref_am = _brute_quantize_block(w[row, col:col + 64])
        assert absmax[b] == ref_am
        assert list(codes[row, col:col + 64]) == ref_codes, b


def test_quantize_invariants():
    rs = np.random.default_rng(2)
    w = (rs.standard_normal((16, 256)) * 0.02).astype(np.float32)
    w[3, 64:128] = 0.0
    packed, absmax = nf4.quantize(w)
    codes = nf4.unpack_codes(packed)
    dec = nf4.decode_f32(packed, absmax)
    blocks = w.reshape(-1, 64)
    dblocks = dec.reshape(-1, 64)
    cblocks = codes.reshape(-1, 64)
    for b in range(blocks.shape[0]):
        if absmax[b] == 0:
            assert np.all(cblocks[b] == 7) and np.all(dblocks[b] == 0.0)
            continue
        i = int(np.argmax(np.abs(blocks[b])))
        # the largest element decodes to exactly +-absmax (code 0 or 15)
        assert dblocks[b, i] == np.sign(blocks[b, i]) * absmax[b]
        assert cblocks[b, i] in (0, 15)
    # quantizing the decoded fp32 weight gives the same codes and absmax back
    packed2, absmax2 = nf4.quantize(dec)
    assert np.array_equal(packed2, packed) and np.array_equal(absmax2, absmax)


def test_decode_power_of_two_absmax_is_exact():
    T = nf4.nf4_table()
    codes = np.tile(np.arange(16, dtype=np.uint8), 4).reshape(1, 64)
    packed = nf4.pack_codes(codes)
    for e in (-130, -20, -1, 0, 3, 60):
        am = np.array([np.ldexp(1.0, e)], np.float32)
        got = nf4.decode_f32(packed, am)[0]
        want = np.array([np.ldexp(float(T[c]), e) for c in codes[0]], np.float32)
        if e > -126:  # outside the subnormal range the product is exact
            assert np.array_equal(got, want)
        bits = nf4.decode_bf16_bits(packed, am)[0]
        ref = torch.from_numpy(got).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(bits, ref)


def test_decode_loop_definition():
    rs = np.random.default_rng(3)
    packed = rs.integers(0, 256, (4, 64), dtype=np.uint8)
    absmax = (rs.random(8) * 0.1).astype(np.float32)
    absmax[0] = np.float32(1e-39)   # subnormal absmax
    T = nf4.nf4_table()
    got = nf4.decode_f32(packed, absmax)
    for r in range(4):
        for c in range(128):
            byte = int(packed[r, c // 2])
            code = (byte >> 4) if c % 2 == 0 else (byte & 15)
            prod = np.float32(T[code]) * np.float32(absmax[(r * 128 + c) // 64])
            assert got[r, c] == prod
