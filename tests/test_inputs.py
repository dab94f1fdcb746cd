"""The seeded generators: deterministic, shaped as the workloads, bf16-exact."""
import numpy as np

from selective_state_space_scan_amd import inputs as I


def test_deterministic_and_shaped():
    w = I.WORKLOADS[0]
    a = I.make_inputs(w, I.seed_for(0))
    b = I.make_inputs(w, I.seed_for(0))
    for k in ("x", "delta", "A_log", "B", "C", "D"):
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (2, 256, 64) and a["B"].shape == (2, 256, 16) and a["A_log"].shape == (64, 16)
    assert np.allclose(a["A_log"][3], np.log(np.arange(1, 17)))
    assert a["valid_len"] is None


def test_bf16_rounding_is_exact_and_ties_to_even():
    v = np.array([1.0, 1.00390625, 1.005859375, 1.01171875, -3.3, 0.0, -0.0], np.float32)
    r = I.round_to_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0078125 and r[3] == 1.015625
    assert r[4] == np.float32(-3.296875)
    I.bf16_bits(r)  # all exactly representable
    w = I.small_workload(I.WORKLOADS[2], batch=1, seqlen=64, dim=32)
    inp = I.make_inputs(w, 1)
    for k in ("x", "delta", "B", "C"):
        I.bf16_bits(inp[k])


def test_varlen_recipe():
    w = I.small_workload(I.WORKLOADS[3], batch=16, seqlen=8192, dim=16)
    inp = I.make_inputs(w, I.seed_for(3))
    vl = inp["valid_len"]
    assert vl.dtype == np.int32 and vl.shape == (16,) and vl.min() >= 128 and vl.max() <= 8192


def test_delta_distribution():
    w = I.small_workload(I.WORKLOADS[4], batch=1, seqlen=4096, dim=64)
    d = I.make_inputs(w, 3)["delta"]
    assert abs(float(d.mean()) + 5.0) < 0.02 and abs(float(d.std()) - 0.5) < 0.02
