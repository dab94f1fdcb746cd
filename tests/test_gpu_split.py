"""The time split across workgroups (fold kernel + per-part rescan) on the GPU:
two parts are bitwise the unsplit scan; more parts match the oracle."""
import numpy as np
import pytest

from conftest import rel_err
from gpu_util import to_device, to_np64, tol_for
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


def _case(io, N, L, nb, nd, seed, varlen=None, extras=True):
    import dataclasses
    base = I.WORKLOADS[0] if io == "f32" else I.WORKLOADS[2]
    w = dataclasses.replace(I.small_workload(base, batch=nb, seqlen=L, dim=nd), dstate=N)
    inp = I.make_inputs(w, seed)
    rng = np.random.default_rng(seed + 1)
    if extras:
        inp["h0"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
        inp["delta_bias"] = (0.5 * rng.standard_normal(nd)).astype(np.float32)
        z = (2.0 * rng.standard_normal((nb, L, nd))).astype(np.float32)
        inp["z"] = I.round_to_bf16(z) if io == "bf16" else z
    if varlen is not None:
        inp["valid_len"] = np.asarray(varlen, dtype=np.int32)
    return w, inp


def _run(inp, io, parts, chunks=True, clamp=None):
    import torch
    import selective_state_space_scan_amd as ssm
    dev = to_device(inp, io)
    kw = {}
    if "h0" in inp:
        kw = dict(h0=torch.from_numpy(inp["h0"]).cuda(), delta_bias=torch.from_numpy(inp["delta_bias"]).cuda(),
                  z=torch.from_numpy(inp["z"]).cuda().to(dev["x"].dtype))
    out = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                 dev["valid_len"], return_chunk_states=chunks, time_parts=parts,
                                 delta_clamp=clamp, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_two_parts_bitwise_equal_unsplit(io, N):
    import selective_state_space_scan_amd as ssm
    T = ssm.chunk_len(N)
    L = 9 * T + 37
    w, inp = _case(io, N, L, 3, 32, seed=11 * N, varlen=[L, 4 * T + 5, 0])
    ref = _run(inp, io, 1)
    got = _run(inp, io, 2)
    for a, b in zip(ref, got):
        assert np.array_equal(_bits(a), _bits(b))


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,parts", [(16, 3), (16, 8), (32, 5), (64, 4), (64, 7)])
def test_parts_against_oracle(io, N, parts):
    import oracle
    import selective_state_space_scan_amd as ssm
    T = ssm.chunk_len(N)
    L = 16 * T + 19
    # rows ending inside the first part, at a part boundary, in the last part, and empty
    w, inp = _case(io, N, L, 4, 32, seed=parts * 100 + N, varlen=[L, 2 * T + 3, 6 * T, 0])
    y, h, cs = _run(inp, io, parts)
    yr, hr, csr = oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"],
                                        valid_len=inp["valid_len"], h0=inp["h0"], delta_bias=inp["delta_bias"],
                                        z=inp["z"], chunk_len=T, nthreads=8)
    ey, eh, ec = rel_err(to_np64(y), yr), rel_err(to_np64(h), hr), rel_err(to_np64(cs), csr)
    print(f"{io} N={N} parts={parts}: y {ey:.2e} h_last {eh:.2e} chunk states {ec:.2e}", flush=True)
    assert ey <= tol_for(io, "y") and eh <= tol_for(io, "h_last") and ec <= tol_for(io, "chunk_states")
    # padding stays exact: y is +0 past each row's length, the empty row keeps h0
    yb = _bits(y)
    assert not yb[1, 2 * T + 3:].any() and not yb[3].any()
    assert np.array_equal(to_np64(h[3]), inp["h0"][3].astype(np.float64))


def test_auto_split_small_batch_long_sequence():
    """A batch of one row with 64 channels: too few workgroups to fill the GPU,
    so the library splits time by itself; the result matches the oracle."""
    import oracle
    import selective_state_space_scan_amd as ssm
    import torch
    w, inp = _case("bf16", 64, 4096, 1, 64, seed=5, extras=False)
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate, dims.io_dtype = 1, 4096, 64, 64, ssm.SSM_IO_BF16
    parts = ssm.auto_time_parts(ssm._binding.handle_for(torch.cuda.current_device()), dims)
    assert parts == 4096 // 512  # as many as parts of at least 512 steps allow
    y, h, cs = _run(inp, "bf16", None, clamp=(1e-3, 0.1))
    yr, hr, csr = oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"],
                                        delta_clamp=(1e-3, 0.1), chunk_len=ssm.chunk_len(64), nthreads=8)
    assert rel_err(to_np64(y), yr) <= tol_for("bf16", "y") and rel_err(to_np64(h), hr) <= tol_for("bf16", "h_last")
    assert rel_err(to_np64(cs), csr) <= tol_for("bf16", "chunk_states")
    # the same call without a split agrees to rounding
    y1, h1, _ = _run(inp, "bf16", 1, clamp=(1e-3, 0.1))
    assert rel_err(to_np64(h), to_np64(h1)) <= 1e-5


def test_headline_shape_is_not_split():
    import selective_state_space_scan_amd as ssm
    import torch
    h = ssm._binding.handle_for(torch.cuda.current_device())
    for wi in (1, 2, 3):
        w = I.WORKLOADS[wi]
        dims = ssm.ssm_scan_dims()
        dims.batch, dims.seqlen, dims.dim, dims.dstate, dims.io_dtype = w.batch, w.seqlen, w.dim, w.dstate, 1
        assert ssm.auto_time_parts(h, dims) == 1
    w = I.WORKLOADS[4]
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate, dims.io_dtype = w.batch, w.seqlen, w.dim, w.dstate, 1
    assert ssm.auto_time_parts(h, dims) == 16


def test_auto_split_only_while_cus_would_idle():
    """The library splits time only when the (row, 16-channel) groups would
    leave CUs idle: at most three quarters as many groups as CUs; and parts
    hold at least 512 steps."""
    import selective_state_space_scan_amd as ssm
    import torch
    h = ssm._binding.handle_for(torch.cuda.current_device())
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    for groups in (cus // 4, cus // 2, (3 * cus) // 4, (3 * cus) // 4 + 1, cus, (3 * cus) // 2, 2 * cus):
        for N in (16, 32, 64):
            dims = ssm.ssm_scan_dims()
            dims.batch, dims.seqlen, dims.dim, dims.dstate, dims.io_dtype = 1, 4096, 16 * groups, N, 1
            parts = ssm.auto_time_parts(h, dims)
            assert (parts > 1) == (4 * groups <= 3 * cus), (groups, cus, N, parts)
            assert parts <= 4096 // 512, (groups, N, parts)
