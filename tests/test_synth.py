"""The seeded input generator: determinism and bfloat16 rounding."""
import numpy as np

from synth import (BF16, F32, TINY, WORKLOADS, MoEShape, bf16_bits_to_f32, draw, f32_to_bf16_bits,
                   make_inputs, router_skew_bias)


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0, 1e-40],
                    dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(vals))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... i.e. 1.015625)
    assert list(got[:4]) == [1.0, 1.0, np.float32(1.015625), 1.0]
    assert got[4] == -2.5 and got[5] == 0.0


def test_streams_are_deterministic_and_independent():
    a = draw(7, 2, 3, (5, 6), 0.5, BF16)
    b = draw(7, 2, 3, (5, 6), 0.5, BF16)
    c = draw(7, 2, 4, (5, 6), 0.5, BF16)
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_threads_do_not_change_bits():
    s = MoEShape("t", T=9, H=64, I=64, E=6, k=2, dtype=BF16, cfg_id=77, n_shared=1, I_shared=64)
    a = make_inputs(s, threads=1)
    b = make_inputs(s, threads=4)
    for f in ("x", "w_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_fan_in_scaling_and_skew():
    s = WORKLOADS[TINY]
    inp = make_inputs(s, threads=2)
    assert inp.x.dtype == np.float32 and inp.w_gate.shape == (4, 256, 128)
    assert abs(inp.w_gate.std() * np.sqrt(128) - 1) < 0.02
    assert abs(inp.w_down.std() * np.sqrt(256) - 1) < 0.02
    b = router_skew_bias(64)
    assert b[0] == 0.0 and abs(b[63] - 0.5 * np.log(1 / 64)) < 1e-6
