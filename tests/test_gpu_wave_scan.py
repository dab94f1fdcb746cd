"""The log-depth (Hillis-Steele) wave-scan combine of a tile's sub-chunks,
selected with combine="wave_scan", against the fp64 oracle: every dstate, both
I/O types, padding, the extras, chunk-boundary states at several chunk lengths,
a time split (whose fold kernel walks, and whose parts scan), and the headline
workload over whole tensors."""
import numpy as np
import pytest

from conftest import rel_err
from gpu_util import oracle_full, to_device, to_np64, tol_for
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu


def _case(io, N, L, nb, nd, seed):
    base = I.WORKLOADS[0] if io == "f32" else I.WORKLOADS[2]
    w = type(base)(**{**I.small_workload(base, batch=nb, seqlen=L, dim=nd).__dict__, "dstate": N})
    inp = I.make_inputs(w, seed)
    rng = np.random.default_rng(seed + 1)
    inp["h0"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
    inp["delta_bias"] = (0.5 * rng.standard_normal(nd)).astype(np.float32)
    z = (2.0 * rng.standard_normal((nb, L, nd))).astype(np.float32)
    inp["z"] = I.round_to_bf16(z) if io == "bf16" else z
    inp["valid_len"] = np.array([L, L // 3 + 1, 0, L - 5][:nb], dtype=np.int32)
    return w, inp


def _run(inp, io, **kw):
    import torch
    import selective_state_space_scan_amd as ssm
    dev = to_device(inp, io)
    out = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                 dev["valid_len"], h0=torch.from_numpy(inp["h0"]).cuda(),
                                 delta_bias=torch.from_numpy(inp["delta_bias"]).cuda(),
                                 z=torch.from_numpy(inp["z"]).cuda().to(dev["x"].dtype), **kw)
    torch.cuda.synchronize()
    return out


def _check(inp, io, label, cl=None, **kw):
    import selective_state_space_scan_amd as ssm
    outs = _run(inp, io, combine="wave_scan", return_chunk_states=cl is not None,
                **({"chunk_len": cl} if cl is not None else {}), **kw)
    ref = oracle_full(inp, h0=inp["h0"], delta_bias=inp["delta_bias"], z=inp["z"], chunk_len=cl)
    names = ("y", "h_last", "chunk_states")
    L = inp["x"].shape[1]
    mask = np.broadcast_to(np.arange(L)[None, :, None] < inp["valid_len"][:, None, None], ref[0].shape)
    errs = {}
    for k, got, r in zip(names, outs, ref):
        g = to_np64(got)
        errs[k] = rel_err(g, r, mask if k == "y" else None)
    print(label, " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= tol_for(io, k) for k, v in errs.items()), errs
    assert np.all(to_np64(outs[0])[~mask] == 0.0)  # padded steps of y are +0
    # the empty row keeps h0
    assert np.array_equal(to_np64(outs[1])[2], inp["h0"][2].astype(np.float64))
    return outs, ssm


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_wave_scan_against_oracle(io, N):
    import selective_state_space_scan_amd as ssm
    T = ssm.chunk_len(N)
    L = 5 * T + 37  # several tiles and a ragged tail
    w, inp = _case(io, N, L, 4, 48, seed=40 + N)
    for div in (1, 2, T // 4):  # chunk states at the tile, half of it, every 4-step sub-chunk
        _check(inp, io, f"{io} N={N} chunk_len {T // div}", cl=T // div)


@pytest.mark.parametrize("N", [16, 32, 64])
def test_wave_scan_with_time_split(N):
    import selective_state_space_scan_amd as ssm
    T = ssm.chunk_len(N)
    w, inp = _case("bf16", N, 12 * T + 19, 4, 32, seed=90 + N)
    _check(inp, "bf16", f"split N={N}", cl=T, time_parts=3)


def test_wave_scan_matches_walk_within_rounding():
    """The two combines associate the same products differently: equal to
    within fp32 rounding, and each within tolerance of the oracle."""
    w, inp = _case("f32", 16, 1000, 4, 64, seed=7)
    yw, hw = _run(inp, "f32")
    ys, hs = _run(inp, "f32", combine="wave_scan")
    assert rel_err(to_np64(ys), to_np64(yw)) <= 1e-5 and rel_err(to_np64(hs), to_np64(hw)) <= 1e-5


def test_wave_scan_headline_shape():
    """B8 L4096 D1024 N16 bf16, every element of y and h_last."""
    import torch
    import selective_state_space_scan_amd as ssm
    w = I.WORKLOADS[2]
    inp = I.make_inputs(w, I.seed_for(2))
    dev = to_device(inp, "bf16")
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                  combine="wave_scan")
    torch.cuda.synchronize()
    yr, hr = oracle_full(inp, nthreads=16)
    ey, eh = rel_err(to_np64(y), yr), rel_err(to_np64(h), hr)
    print(f"wave scan headline: y {ey:.2e} h_last {eh:.2e}", flush=True)
    assert ey <= tol_for("bf16", "y") and eh <= tol_for("bf16", "h_last")


def test_bad_combine_is_rejected():
    import torch
    import selective_state_space_scan_amd as ssm
    w, inp = _case("f32", 16, 64, 1, 16, seed=1)
    dev = to_device(inp, "f32")
    with pytest.raises(ValueError):
        ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], None, None,
                               combine="tree")
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate, dims.io_dtype, dims.delta_softplus = 1, 64, 16, 16, 0, 1
    y = torch.empty_like(dev["x"])
    ex = ssm.ssm_scan_fwd_extras(None, None, None, None, 0, 0, None, 0, 2)
    h = ssm._binding.handle_for(0)
    rc = ssm.ssm_selective_scan_fwd_ex(h, dev["x"].data_ptr(), dev["delta"].data_ptr(), dev["A_log"].data_ptr(),
                                       dev["B"].data_ptr(), dev["C"].data_ptr(), None, None, y.data_ptr(), None,
                                       dims, ex, torch.cuda.current_stream().cuda_stream)
    assert rc == ssm.SSM_ERR_INVALID_ARG
