"""Host-side helpers of the GPU tests (no GPU): the per-output tolerance table
and the channel-split driver of the oracle's backward, which the full-size
backward checks use and which must give what one oracle call over the whole
problem gives."""
import numpy as np
import pytest

from gpu_util import FP32_OUTPUTS, oracle_bwd, tol_for
from selective_state_space_scan_amd import inputs as I


def test_tolerance_table():
    assert tol_for("f32") == 1e-4 and tol_for("bf16") == 2e-2
    for k in ("y", "dx", "ddelta", "dz"):
        assert tol_for("bf16", k) == 2e-2 and tol_for("f32", k) == 1e-4
    for k in FP32_OUTPUTS:
        assert tol_for("bf16", k) == 1e-4


@pytest.mark.parametrize("nb", [1, 2])
def test_channel_split_backward_matches_one_call(oracle_mod, nb):
    w = I.small_workload(I.WORKLOADS[2], batch=nb, seqlen=90, dim=64)
    inp = I.make_inputs(w, 31 + nb)
    inp["valid_len"] = np.array([90, 41][:nb], np.int32)
    rng = np.random.default_rng(nb)
    dy = rng.standard_normal((nb, 90, 64)).astype(np.float32)
    dhl = rng.standard_normal((nb, 64, 16)).astype(np.float32)
    h0 = rng.standard_normal((nb, 64, 16)).astype(np.float32)
    bias = (0.3 * rng.standard_normal(64)).astype(np.float32)
    z = rng.standard_normal((nb, 90, 64)).astype(np.float32)
    clamp = (0.01, 0.03)
    split = oracle_bwd(inp, dy, dhl, delta_clamp=clamp, h0=h0, delta_bias=bias, z=z, nthreads=16)
    one = oracle_mod.selective_scan_bwd(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], dy,
                                        valid_len=inp["valid_len"], h0=h0, delta_bias=bias, z=z, dh_last=dhl,
                                        delta_clamp=clamp, nthreads=1)
    for k, v in one.items():
        assert split[k].shape == v.shape, k
        # per-channel outputs are the same sums in the same order; dB and dC
        # add the groups' partial sums (a different order, fp64)
        np.testing.assert_allclose(split[k], v, rtol=1e-12, atol=1e-12 * np.max(np.abs(v)), err_msg=k)
