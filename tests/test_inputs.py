"""The seeded input generator: reproducible, and its bf16/fp16 rounding is
round-to-nearest-even (checked against torch's and numpy's own conversions)."""
import numpy as np
import pytest

import seeded_inputs as si


def test_reproducible_and_ordered():
    a = si.make_inputs(1, 2, 16, 8, "bf16", 1.0, 7, backward=True)
    b = si.make_inputs(1, 2, 16, 8, "bf16", 1.0, 7, backward=True)
    for nm in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a[nm][1], b[nm][1])
    # Q, K, V, dO are consecutive draws of one generator, in that order
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 16, 8), dtype=np.float32)
    k = rng.standard_normal((1, 2, 16, 8), dtype=np.float32)
    np.testing.assert_array_equal(si.round_to(k, "bf16")[1], a["k"][1])
    np.testing.assert_array_equal(si.round_to(q, "bf16")[1], a["q"][1])


def test_bf16_rounding_matches_torch_rne():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  3.4e38, 1e-40], dtype=np.float32)])
    vals, bits = si.round_to(x, "bf16")
    t = torch.from_numpy(x).to(torch.bfloat16)
    np.testing.assert_array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(vals, t.to(torch.float32).numpy())


def test_f16_and_f32_rounding():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1000).astype(np.float32)
    v, h = si.round_to(x, "f16")
    assert h.dtype == np.float16
    np.testing.assert_array_equal(v, x.astype(np.float16).astype(np.float32))
    v, f = si.round_to(x, "f32")
    np.testing.assert_array_equal(v, x)


def test_workload_table():
    w = si.WORKLOADS["C3"]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal, w.seed) == (2, 32, 8192, 128, "bf16", True, 1003)
    assert w.fwd_flop() == 4 * 2 * 32 * 8192 ** 2 * 128 / 2
    assert si.WORKLOADS["C4"].sigma == 0.5
    assert si.WORKLOADS["C5"].backward


# ---------------------------------------------------------------- E4M3 (8-bit) cache rounding

def test_e4m3_codes_round_trip_and_known_values():
    """OCP E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent
    field 0 is subnormal (m/8 * 2^-6); 0x7F/0xFF are NaN; the largest value
    is 1.75 * 2^8 = 448."""
    import numpy as np
    import seeded_inputs as si
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = si.e4m3_to_f32(codes)
    assert np.array_equal(si.round_e4m3(vals)[vals != 0], codes[vals != 0])  # -0 maps to +0
    known = {0x38: 1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9,
             0x40: 2.0, 0xC6: -3.5, 0x3F: 1.875, 0x00: 0.0}
    for c, v in known.items():
        assert si.e4m3_to_f32(np.array([c], np.uint8))[0] == v
        assert si.round_e4m3(np.array([v], np.float32))[0] == c
    assert np.isnan(si.e4m3_to_f32(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_rounding_ties_to_even_and_saturates():
    import numpy as np
    import seeded_inputs as si
    # midpoints: 1.0625 between 1.0 (0x38, even) and 1.125 (0x39); 1.1875 between 0x39 and 1.25 (0x3A)
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 460.0, 1e9, -1e9, 1.06], np.float32)
    assert si.round_e4m3(x).tolist() == [0x38, 0x3A, 0x00, 0x01, 0x7E, 0x7E, 0xFE, 0x38]
    # nearest: every finite value rounds to a code no further than any other code
    rng = np.random.default_rng(3)
    y = (rng.standard_normal(5000) * 50).astype(np.float32)
    q = si.e4m3_to_f32(si.round_e4m3(y))
    tab = si.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    tab = tab[np.isfinite(tab)]
    best = np.abs(y[:, None] - tab[None, :]).min(axis=1)
    assert np.array_equal(np.abs(y - q), np.minimum(best, np.abs(y - q)))
    assert np.allclose(np.abs(y - q), best, rtol=0, atol=0)


def test_fp8_cache_inputs_share_the_16_bit_draws():
    import numpy as np
    import seeded_inputs as si
    a = si.make_kvcache_inputs(2, 3, 2, 50, 64, "bf16", 1.0, 9)
    b = si.make_kvcache_fp8_inputs(2, 3, 2, 50, 64, "bf16", 1.0, 9)
    assert np.array_equal(a["q"][1], b["q"][1]) and np.array_equal(a["seqlens"], b["seqlens"])
    assert np.array_equal(a["k"][1], b["k16"][1])
    for nm in ("k", "v"):
        deq, codes = b[nm]
        assert codes.dtype == np.uint8 and codes.shape == (2, 3, 50, 64)
        sc = float(b[nm + "_scale"])
        assert sc == 2.0 ** round(np.log2(sc))  # a power of two: dequantised values are exact
        assert np.array_equal(deq.astype(np.float64), si.e4m3_to_f32(codes).astype(np.float64) * sc)
        top = np.abs(si.e4m3_to_f32(codes)).max()
        assert 224.0 < top <= 448.0  # max|x| / scale lands in (224, 448]
        # each value is the nearest scaled code to its 16-bit draw
        x = b[nm + "16"][0] / sc
        assert np.all(np.abs(x - si.e4m3_to_f32(codes)) <= np.abs(x) * 2.0 ** -4 + 2.0 ** -10)


def test_scaled_e4m3_blocks():
    """Per-block quantisation: one scale per 128-row block of a head (V: per
    head), amax / 448 each, codes whose dequantised values are within E4M3's
    half step (2^-4 relative for normal values) of the inputs, and blocks
    independent of each other."""
    x = si.make_inputs(2, 3, 300, 16, "bf16", 1.0, 31)["q"][0]
    x[0, 1, 128:256] *= 100.0  # one loud block
    codes, sc, deq = si.quantise_e4m3_scaled(x, "block")
    assert codes.dtype == np.uint8 and sc.shape == (2, 3, 3) and sc.dtype == np.float32
    np.testing.assert_allclose(sc[0, 1, 1], np.abs(x[0, 1, 128:256]).max() / 448.0, rtol=1e-6)
    np.testing.assert_allclose(sc[0, 1, 0], np.abs(x[0, 1, :128]).max() / 448.0, rtol=1e-6)
    # the loud block's scale does not touch its neighbours
    assert sc[0, 1, 1] > 50 * sc[0, 1, 0]
    assert np.abs(deq).max() <= np.abs(x).max() * (1 + 2.0 ** -4)
    big = np.abs(x) >= 2.0 ** -6 * np.repeat(sc, 128, axis=2)[:, :, :300, None]
    rel = np.abs(deq - x) / np.abs(x)
    assert rel[big].max() <= 2.0 ** -4 + 1e-7
    # dequantised = code value times the float32 scale, exactly
    rows = np.repeat(sc, 128, axis=2)[:, :, :300, None].astype(np.float64)
    np.testing.assert_array_equal(deq, si.e4m3_to_f32(codes).astype(np.float64) * rows)
    # per head (V) and per tensor
    _, sh, _ = si.quantise_e4m3_scaled(x, "block", per_head_only=True)
    assert sh.shape == (2, 3)
    np.testing.assert_allclose(sh, np.abs(x).max(axis=(2, 3)) / 448.0, rtol=1e-6)
    _, st, _ = si.quantise_e4m3_scaled(x, "tensor")
    assert st.shape == (1,)
    # an all-zero block gets scale 1 (codes 0)
    z = np.zeros((1, 1, 130, 4), dtype=np.float32)
    cz, sz, dz = si.quantise_e4m3_scaled(z, "block")
    assert (sz == 1.0).all() and (cz == 0).all() and (dz == 0).all()
