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
