"""The forward's optional extras on the GPU against the oracle: initial state
h0 (also in place), delta bias, silu output gate and chunk-boundary states."""
import numpy as np
import pytest

from conftest import rel_err
from gpu_util import oracle_full, to_device, to_np64, tol_for
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


def _case(io, N, L=700, nb=3, nd=32, seed=0, varlen=False):
    base = I.WORKLOADS[0] if io == "f32" else I.WORKLOADS[2]
    w = I.small_workload(base, batch=nb, seqlen=L, dim=nd)
    w = type(w)(**{**w.__dict__, "dstate": N})
    inp = I.make_inputs(w, seed)
    rng = np.random.default_rng(seed + 1)
    inp["h0"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
    inp["delta_bias"] = (0.5 * rng.standard_normal(nd)).astype(np.float32)
    z = (2.0 * rng.standard_normal((nb, L, nd))).astype(np.float32)
    inp["z"] = I.round_to_bf16(z) if io == "bf16" else z
    if varlen:
        inp["valid_len"] = np.array([L, L // 3, 0][:nb], dtype=np.int32)
    return w, inp


def _gpu(inp, io, use=("h0", "delta_bias", "z"), chunks=False, **kw):
    import torch
    import selective_state_space_scan_amd as ssm
    dev = to_device(inp, io)
    extra = {}
    if "h0" in use:
        extra["h0"] = torch.from_numpy(inp["h0"]).cuda()
    if "delta_bias" in use:
        extra["delta_bias"] = torch.from_numpy(inp["delta_bias"]).cuda()
    if "z" in use:
        extra["z"] = torch.from_numpy(inp["z"]).cuda().to(dev["x"].dtype)
    out = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                 dev["valid_len"], return_chunk_states=chunks, **extra, **kw)
    torch.cuda.synchronize()
    return out


def _oracle(inp, use=("h0", "delta_bias", "z"), chunk_len=None):
    import oracle
    return oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"],
                                 valid_len=inp.get("valid_len"), h0=inp["h0"] if "h0" in use else None,
                                 delta_bias=inp["delta_bias"] if "delta_bias" in use else None,
                                 z=inp["z"] if "z" in use else None, chunk_len=chunk_len, nthreads=8)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
@pytest.mark.parametrize("use", [("h0",), ("delta_bias",), ("z",), ("h0", "delta_bias", "z")])
def test_extras_against_oracle(io, N, use):
    w, inp = _case(io, N, seed=N + len(use))
    y, h = _gpu(inp, io, use)
    yr, hr = _oracle(inp, use)
    ey, eh = rel_err(to_np64(y), yr), rel_err(to_np64(h), hr)
    print(f"{io} N={N} {use}: y {ey:.2e} h_last {eh:.2e}", flush=True)
    assert ey <= tol_for(io, "y") and eh <= tol_for(io, "h_last")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N,div", [(16, 1), (64, 1), (16, 2), (16, 32), (32, 4), (64, 2), (64, 8)])
def test_chunk_states_against_oracle(io, N, div):
    import selective_state_space_scan_amd as ssm
    w, inp = _case(io, N, L=1000, seed=7 * N + div, varlen=True)
    cl = ssm.chunk_len(N) // div
    y, h, cs = _gpu(inp, io, ("h0", "z"), chunks=True, chunk_len=cl)
    yr, hr, csr = _oracle(inp, ("h0", "z"), chunk_len=cl)
    assert cs.shape == csr.shape
    ecs = rel_err(to_np64(cs), csr)
    print(f"{io} N={N} chunk_len {cl}: chunk states err {ecs:.2e}", flush=True)
    assert ecs <= tol_for(io, "chunk_states")
    assert np.array_equal(_bits(cs[:, -1]), _bits(h))  # the last chunk state is h_last
    # a row with no valid steps keeps h0 in every chunk state
    assert np.array_equal(to_np64(cs[2]), np.broadcast_to(inp["h0"][2].astype(np.float64), cs[2].shape))


@pytest.mark.parametrize("N", [16, 64])
def test_split_at_chunk_boundary_is_bitwise(N):
    """bjdmk.com.cn section 2.4 / pwwt.cn section 4.2: carrying the state into a
    second run continues the sequence.  Split at a multiple of the chunk
    length, the two runs take exactly the same arithmetic as one run (all
    three without the library's own time split)."""
    import torch
    import selective_state_space_scan_amd as ssm
    w, inp = _case("bf16", N, L=1000, seed=3 * N)
    dev = to_device(inp, "bf16")
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                  time_parts=1)
    T = 3 * ssm.chunk_len(N)
    part = lambda t, a, b: t[:, a:b].contiguous()
    y1, h1 = ssm.selective_scan_fwd(part(dev["x"], 0, T), part(dev["delta"], 0, T), dev["A_log"],
                                    part(dev["B"], 0, T), part(dev["C"], 0, T), dev["D"], None, time_parts=1)
    y2, h2 = ssm.selective_scan_fwd(part(dev["x"], T, 1000), part(dev["delta"], T, 1000), dev["A_log"],
                                    part(dev["B"], T, 1000), part(dev["C"], T, 1000), dev["D"], None, h0=h1,
                                    time_parts=1)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(torch.cat([y1, y2], dim=1)), _bits(y))
    assert np.array_equal(_bits(h2), _bits(h))


def test_h0_in_place():
    import torch
    import selective_state_space_scan_amd as ssm
    w, inp = _case("bf16", 16, seed=99)
    dev = to_device(inp, "bf16")
    h0 = torch.from_numpy(inp["h0"]).cuda()
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None, h0=h0)
    state = h0.clone()
    y2, h2 = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                    h0=state, h_last=state)
    torch.cuda.synchronize()
    assert h2 is state
    assert np.array_equal(_bits(y2), _bits(y)) and np.array_equal(_bits(state), _bits(h))


@pytest.mark.parametrize("time_parts", [None, 4])
def test_h0_in_place_at_a_split_shape(time_parts):
    """One row of 256 channels over 4096 steps: a shape the library splits in
    time by itself.  In place (h0 is h_last) the scan runs unsplit, so the
    results are those of the unsplit scan with h0 in its own buffer, and match
    the oracle."""
    import torch
    import selective_state_space_scan_amd as ssm
    w, inp = _case("bf16", 16, L=4096, nb=1, nd=256, seed=123)
    dev = to_device(inp, "bf16")
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate = 1, 4096, 256, 16
    assert ssm.auto_time_parts(ssm._binding.handle_for(0), dims) >= 2
    h0 = torch.from_numpy(inp["h0"]).cuda()
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                  h0=h0, time_parts=1)
    state = h0.clone()
    y2, h2 = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                    h0=state, h_last=state, time_parts=time_parts)
    torch.cuda.synchronize()
    assert h2 is state
    assert np.array_equal(_bits(y2), _bits(y)) and np.array_equal(_bits(state), _bits(h))
    yr, hr = _oracle(inp, ("h0",))
    ey, eh = rel_err(to_np64(y2), yr), rel_err(to_np64(state), hr)
    print(f"in place, time_parts {time_parts}: y {ey:.2e} h_last {eh:.2e}", flush=True)
    assert ey <= tol_for("bf16", "y") and eh <= tol_for("bf16", "h_last")


def test_seqlen_zero_returns_h0():
    import torch
    import selective_state_space_scan_amd as ssm
    dev = torch.device("cuda:0")
    x = torch.empty((2, 0, 32), dtype=torch.bfloat16, device=dev)
    B = torch.empty((2, 0, 16), dtype=torch.bfloat16, device=dev)
    h0 = torch.randn((2, 32, 16), device=dev)
    y, h = ssm.selective_scan_fwd(x, x, torch.zeros((32, 16), device=dev), B, B, None, None, h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(h, h0) and h is not h0


def test_headline_shape_with_extras():
    """The headline workload with all extras, every element of y and h_last
    against the oracle over the whole problem."""
    import torch
    import selective_state_space_scan_amd as ssm
    w = I.WORKLOADS[2]
    inp = I.make_inputs(w, I.seed_for(2))
    rng = np.random.default_rng(5)
    h0 = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32)
    dbias = (0.3 * rng.standard_normal(w.dim)).astype(np.float32)
    z = I.round_to_bf16(rng.standard_normal((w.batch, w.seqlen, w.dim)).astype(np.float32))
    dev = to_device(inp, "bf16")
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                  h0=torch.from_numpy(h0).cuda(), delta_bias=torch.from_numpy(dbias).cuda(),
                                  z=torch.from_numpy(z).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    yr, hr = oracle_full(inp, h0=h0, delta_bias=dbias, z=z, nthreads=16)
    ey, eh = rel_err(to_np64(y), yr), rel_err(to_np64(h), hr)
    print(f"headline with extras: y err {ey:.3e}  h_last err {eh:.3e}", flush=True)
    assert ey <= tol_for("bf16", "y") and eh <= tol_for("bf16", "h_last")
