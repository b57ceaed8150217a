"""Pins of the oracle's FP8 weight format (OCP E4M3, one float32 scale per
128 x 128 block).  The pages name FP8 weights but no format: the E4M3 value table
is checked against closed forms of its definition, the quantiser against exact
round trips, the rounding bound, ties to the even code and the block maximum."""
import numpy as np
import pytest

import oracle.moe_ref as ref
from synth import f32_to_bf16_bits


def test_e4m3_table_closed_forms():
    v = ref.E4M3_VALUES
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9                     # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                 # largest subnormal
    assert v[0x08] == 2.0 ** -6                     # smallest normal
    assert v[0x38] == 1.0 and v[0x39] == 1.125
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0   # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                 # codes 0..0x7E increase
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])
    # inside binade e (codes 8e .. 8e+7) the step is 2^(e-10); subnormals step 2^-9
    for e in range(1, 16):
        codes = [c for c in range(8 * e, 8 * e + 8) if c <= 0x7E]
        assert np.all(np.diff(v[codes]) == 2.0 ** (e - 10))
    assert np.all(np.diff(v[0:9]) == 2.0 ** -9)


def block_of(values, N=128, K=128):
    w = np.zeros((1, N, K), dtype=np.float32)
    w.reshape(-1)[: len(values)] = values
    return w


def test_representable_values_round_trip_exactly():
    # a block whose maximum is 448 has scale 1, so every E4M3 value is kept exactly
    vals = ref.E4M3_VALUES[[c for c in range(256) if not np.isnan(ref.E4M3_VALUES[c])]].astype(np.float32)
    w = block_of(vals)
    codes, scale = ref.quantize_fp8_blockwise(w)
    assert scale[0, 0, 0] == 1.0
    back = ref.dequantize_fp8_blockwise(codes, scale)
    assert np.array_equal(back.reshape(-1)[: len(vals)], vals.astype(np.float64))


def test_ties_go_to_the_even_code():
    w = block_of(np.array([448.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10], dtype=np.float32))
    codes, scale = ref.quantize_fp8_blockwise(w)
    c = codes.reshape(-1)
    assert c[0] == 0x7E
    assert c[1] == 0x38 and c[2] == 0x3A and c[3] == 0xB8   # 1.0625 -> 1.0, 1.1875 -> 1.25
    assert c[4] == 0x00 and c[5] == 0x02                    # half of the smallest subnormal -> 0; 1.5 ulp -> 2 ulp


def test_rounding_bound_and_block_max():
    r = np.random.default_rng(2)
    w = (r.normal(size=(3, 256, 384)) * np.array([1e-3, 1.0, 50.0])[:, None, None]).astype(np.float32)
    bits = f32_to_bf16_bits(w)
    codes, scale = ref.quantize_fp8_blockwise(bits)
    assert codes.shape == w.shape and scale.shape == (3, 2, 3)
    wv = ref.widen(bits)
    back = ref.dequantize_fp8_blockwise(codes, scale)
    s = np.repeat(np.repeat(scale.astype(np.float64), 128, axis=1), 128, axis=2)
    # normals: within half a spacing (2^-4 relative); subnormal range: within 2^-10 * scale
    err = np.abs(back - wv)
    assert np.all(err <= np.maximum(np.abs(wv) * 2.0 ** -4, s * 2.0 ** -10) * (1 + 1e-6))
    # the largest |w| of every block lands on +-448 x scale
    blk = np.abs(wv).reshape(3, 2, 128, 3, 128).max(axis=(2, 4))
    cb = (codes & 0x7F).reshape(3, 2, 128, 3, 128).max(axis=(2, 4))
    assert np.all(cb == 0x7E)
    assert np.allclose(blk, 448.0 * scale, rtol=1e-6)


def test_zero_block_and_shape_checks():
    codes, scale = ref.quantize_fp8_blockwise(np.zeros((1, 128, 256), dtype=np.float32))
    assert np.all(codes == 0) and np.all(scale == 1.0)
    with pytest.raises(ValueError):
        ref.quantize_fp8_blockwise(np.zeros((1, 100, 128), dtype=np.float32))


def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plausible slips planted in the oracle's quantiser each fail a pin above:
    round-half-up instead of ties to the even code, truncation toward zero, the
    other common E4M3 variant (exponent bias 8: subnormal step 2^-10, largest
    finite 240) and a scale that maps the block maximum to 240 instead of 448."""
    pins = (test_e4m3_table_closed_forms, test_representable_values_round_trip_exactly,
            test_ties_go_to_the_even_code, test_rounding_bound_and_block_max)
    for p in pins:          # the oracle as it stands passes every pin
        p()
    pos = ref._E4M3_POS

    def half_up(q32):
        a = np.abs(q32.astype(np.float64))
        hi = np.clip(np.searchsorted(pos, a, side="left"), 1, 0x7E)
        lo = hi - 1
        code = np.where(a - pos[lo] < pos[hi] - a, lo, hi)
        code = np.where(a >= pos[0x7E], 0x7E, np.where(a == 0, 0, code))
        return (code | np.where(np.signbit(q32), 0x80, 0)).astype(np.uint8)

    def toward_zero(q32):
        a = np.abs(q32.astype(np.float64))
        code = np.clip(np.searchsorted(pos, a, side="right") - 1, 0, 0x7E)
        return (code | np.where(np.signbit(q32), 0x80, 0)).astype(np.uint8)

    def fnuz_value(code):
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 15, code & 7
        if code == 0x80:
            return float("nan")
        return sign * (m / 8.0 * 2.0 ** -7 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 8))
    fnuz = np.array([fnuz_value(c) for c in range(256)])

    def scale_240(w_bits, block=128):
        w = ref.widen(w_bits).astype(np.float32)
        G, N, K = w.shape
        blk = w.reshape(G, N // block, block, K // block, block)
        amax = np.abs(blk).max(axis=(2, 4))
        scale = np.where(amax > 0, amax / np.float32(240.0), np.float32(1.0)).astype(np.float32)
        q = (blk / scale[:, :, None, :, None]).astype(np.float32)
        return ref._nearest_e4m3(q).reshape(G, N, K), scale

    slips = {
        "round half up": {"_nearest_e4m3": half_up},
        "truncate toward zero": {"_nearest_e4m3": toward_zero},
        "bias-8 variant": {"E4M3_VALUES": fnuz, "_E4M3_POS": fnuz[:0x7F]},
        "block max to 240": {"quantize_fp8_blockwise": scale_240},
    }
    for name, patch in slips.items():
        with monkeypatch.context() as m:
            for attr, v in patch.items():
                m.setattr(ref, attr, v)
            caught = [p.__name__ for p in pins if _fails(p)]
        assert caught, f"no pin catches the planted slip: {name}"
