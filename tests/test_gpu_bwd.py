"""The backward on the GPU against the fp64 oracle's backward (which the CPU
suite pins to finite differences and exact identities)."""
import dataclasses

import numpy as np
import pytest

from conftest import rel_err
from gpu_util import oracle_bwd, to_device, to_np64, tol_for
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddelta", "dA_log", "dB", "dC", "dD", "ddelta_bias", "dz", "dh0")


def _case(io, N, L, nb, nd, seed, varlen=None, extras=True, clamp=None):
    base = I.WORKLOADS[0] if io == "f32" else I.WORKLOADS[2]
    w = dataclasses.replace(I.small_workload(base, batch=nb, seqlen=L, dim=nd), dstate=N)
    inp = I.make_inputs(w, seed)
    rng = np.random.default_rng(seed + 1)
    rnd = (lambda a: I.round_to_bf16(a)) if io == "bf16" else (lambda a: a.astype(np.float32))
    inp["dy"] = rnd(rng.standard_normal((nb, L, nd)).astype(np.float32))
    inp["dh_last"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
    if extras:
        inp["h0"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
        inp["delta_bias"] = (0.5 * rng.standard_normal(nd)).astype(np.float32)
        inp["z"] = rnd(2.0 * rng.standard_normal((nb, L, nd)).astype(np.float32))
    if varlen is not None:
        inp["valid_len"] = np.asarray(varlen, dtype=np.int32)
    return w, inp


def _gpu(inp, io, clamp=None, time_parts=None):
    import torch
    import selective_state_space_scan_amd as ssm
    dev = to_device(inp, io)
    dt = dev["x"].dtype
    ex = {}
    if "h0" in inp:
        ex = dict(h0=torch.from_numpy(inp["h0"]).cuda(), delta_bias=torch.from_numpy(inp["delta_bias"]).cuda(),
                  z=torch.from_numpy(inp["z"]).cuda().to(dt))
    N = dev["A_log"].shape[1]
    y, h, cs = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                      dev["valid_len"], delta_clamp=clamp, return_chunk_states=True,
                                      chunk_len=ssm.bwd_chunk_len(N), time_parts=time_parts, **ex)
    dy = torch.from_numpy(inp["dy"]).cuda().to(dt)
    dhl = torch.from_numpy(inp["dh_last"]).cuda()
    g = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], dev["valid_len"],
                               dy, cs, dh_last=dhl, delta_clamp=clamp, **ex)
    torch.cuda.synchronize()
    return g


def _oracle(inp, clamp=None):
    import oracle
    return oracle.selective_scan_bwd(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["dy"],
                                     valid_len=inp.get("valid_len"), h0=inp.get("h0"),
                                     delta_bias=inp.get("delta_bias"), z=inp.get("z"), dh_last=inp["dh_last"],
                                     delta_clamp=clamp, nthreads=8)


def _compare(g, r, io, label):
    """Every gradient against the oracle's, each to its own tolerance: bf16
    outputs of bf16 I/O (dx, ddelta, dz) to 2e-2, every fp32 one to 1e-4."""
    worst = {}
    for k in GRADS:
        if r.get(k) is None or g.get(k) is None:
            continue
        worst[k] = rel_err(to_np64(g[k]), r[k])
    print(label, " ".join(f"{k} {v:.1e}" for k, v in worst.items()), flush=True)
    bad = {k: v for k, v in worst.items() if not v <= tol_for(io, k)}
    assert not bad, bad


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_bwd_against_oracle(io, N):
    import selective_state_space_scan_amd as ssm
    T = ssm.bwd_chunk_len(N)
    L = 7 * T + 13
    w, inp = _case(io, N, L, 3, 32, seed=200 + N, varlen=[L, 3 * T + 5, 0])
    g = _gpu(inp, io)
    r = _oracle(inp)
    _compare(g, r, io, f"{io} N={N}")
    # padding: zero gradients past each row's length, the empty row's state adjoint passes through
    assert np.all(to_np64(g["dx"][1, 3 * T + 5:]) == 0) and np.all(to_np64(g["dB"][2]) == 0)
    assert np.array_equal(to_np64(g["dh0"][2]), inp["dh_last"][2].astype(np.float64))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bwd_plain_and_clamped(io):
    """No extras (zero initial state, no bias, no gate), full rows; then the
    long-workload recipe's clip on delta."""
    w, inp = _case(io, 16, 300, 2, 48, seed=7, extras=False)
    _compare(_gpu(inp, io), _oracle(inp), io, f"{io} plain")
    w, inp = _case(io, 64, 200, 2, 32, seed=9, extras=False)
    shifted = (inp["delta"] - 1.0).astype(np.float32)  # softplus values on both sides of the clip
    inp["delta"] = I.round_to_bf16(shifted) if io == "bf16" else shifted
    clamp = (1e-3, 0.01)
    _compare(_gpu(inp, io, clamp=clamp), _oracle(inp, clamp=clamp), io, f"{io} clamp")


def test_bwd_short_and_single_tile():
    """Lengths below one tile and exactly one tile: no chunk states needed."""
    import selective_state_space_scan_amd as ssm
    for L in (1, 5, ssm.bwd_chunk_len(16)):
        w, inp = _case("f32", 16, L, 2, 16, seed=L)
        _compare(_gpu(inp, "f32"), _oracle(inp), "f32", f"L={L}")


def test_bwd_deterministic():
    w, inp = _case("bf16", 16, 500, 2, 64, seed=3)
    a = _gpu(inp, "bf16")
    b = _gpu(inp, "bf16")
    for k in GRADS:
        if a[k] is not None:
            assert np.array_equal(a[k].cpu().float().numpy(), b[k].cpu().float().numpy()), k


@pytest.mark.parametrize("io,N", [("f32", 16), ("f32", 32), ("f32", 64), ("bf16", 64)])
def test_bwd_many_parts_ragged(io, N):
    """Two rows of 32 channels leave the GPU idle, so the backward splits time
    into nine parts of five tiles, folded over 8-step sub-chunks; the second
    row ends inside the fifth part (a ragged fold) and is padding after it."""
    import selective_state_space_scan_amd as ssm
    T = ssm.bwd_chunk_len(N)
    L = 40 * T + 11
    w, inp = _case(io, N, L, 2, 32, seed=500 + N, varlen=[L, 23 * T + 7])
    _compare(_gpu(inp, io), _oracle(inp), io, f"{io} N={N} nine parts")


def test_bwd_after_time_split_forward():
    """The chunk states of a time-split forward serve the backward equally."""
    w, inp = _case("bf16", 64, 2048, 1, 32, seed=13)
    _compare(_gpu(inp, "bf16", time_parts=4), _oracle(inp), "bf16", "split fwd")


def test_bwd_grid_filling_shape():
    """A grid of 512 (row, channel group) workgroups takes the four-wave
    kernel (smaller grids take the eight-wave one)."""
    w, inp = _case("bf16", 16, 200, 4, 2048, seed=17, varlen=[200, 77, 130, 5])
    _compare(_gpu(inp, "bf16"), _oracle(inp), "bf16", "grid 512")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_bwd_full_size(cfg):
    """Each full-size workload (the headline B8 L4096 D1024 N16 among them, the
    variable-length batch, the long dstate-64 sequence with the clip, whose
    forward the library time-splits) in the benchmark's launch configuration:
    every element of every gradient, dB and dC included, against the oracle's
    backward over the whole problem."""
    import torch
    import selective_state_space_scan_amd as ssm
    w = I.WORKLOADS[cfg]
    inp = I.make_inputs(w, I.seed_for(cfg))
    cot = I.make_cotangents(w, I.seed_for(cfg) + 500)
    dev = to_device(inp, w.io)
    print(f"{w.name}: forward with chunk states, backward", flush=True)
    y, h, cs = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                      dev["valid_len"], delta_clamp=w.delta_clamp, return_chunk_states=True,
                                      chunk_len=ssm.bwd_chunk_len(w.dstate))
    del y, h
    dy = torch.from_numpy(cot["dy"]).cuda().to(dev["x"].dtype)
    g = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], dev["valid_len"],
                               dy, cs, dh_last=torch.from_numpy(cot["dh_last"]).cuda(), delta_clamp=w.delta_clamp)
    torch.cuda.synchronize()
    g = {k: (None if v is None else to_np64(v)) for k, v in g.items()}
    del dev, dy, cs
    r = oracle_bwd(inp, cot["dy"], cot["dh_last"], delta_clamp=w.delta_clamp, nthreads=16)
    _compare(g, r, w.io, w.name)
    if inp.get("valid_len") is not None:
        t = np.arange(w.seqlen)[None, :]
        pad = t >= np.asarray(inp["valid_len"])[:, None]
        for k in ("dx", "ddelta", "dB", "dC"):
            assert np.all(g[k][pad] == 0.0), k


def test_bwd_empty_and_degenerate():
    """seqlen 0: the initial state's gradient is dh_last and every other one is
    zero; batch 0 is a no-op; a single 16-channel group works."""
    import torch
    import selective_state_space_scan_amd as ssm
    dev = torch.device("cuda:0")
    nb, nd, N = 2, 32, 16
    x = torch.empty((nb, 0, nd), dtype=torch.bfloat16, device=dev)
    Bt = torch.empty((nb, 0, N), dtype=torch.bfloat16, device=dev)
    A_log = torch.zeros((nd, N), device=dev)
    D = torch.ones(nd, device=dev)
    dhl = torch.randn((nb, nd, N), device=dev)
    g = ssm.selective_scan_bwd(x, x, A_log, Bt, Bt, D, None, x, None, dh_last=dhl,
                               delta_bias=torch.zeros(nd, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(g["dh0"], dhl)
    assert torch.all(g["dA_log"] == 0) and torch.all(g["dD"] == 0) and torch.all(g["ddelta_bias"] == 0)
    x0 = torch.empty((0, 10, nd), dtype=torch.bfloat16, device=dev)
    B0 = torch.empty((0, 10, N), dtype=torch.bfloat16, device=dev)
    g0 = ssm.selective_scan_bwd(x0, x0, A_log, B0, B0, D, None, x0, None)
    torch.cuda.synchronize()
    assert g0["dx"].shape == (0, 10, nd)
    w, inp = _case("f32", 16, 77, 1, 16, seed=23)
    _compare(_gpu(inp, "f32"), _oracle(inp), "f32", "one group")


def test_bwd_out_of_range_lengths_clamp():
    """valid_len below 0 or above L acts as 0 or L (forward and backward),
    bit for bit."""
    L = 300
    w, inp = _case("bf16", 16, L, 3, 32, seed=41, varlen=[-7, L + 55, 120])
    w, ref = _case("bf16", 16, L, 3, 32, seed=41, varlen=[0, L, 120])
    g, gr = _gpu(inp, "bf16"), _gpu(ref, "bf16")
    for k, v in gr.items():
        if v is not None:
            a = g[k].contiguous().view(_int_view(g[k])).cpu().numpy()
            b = v.contiguous().view(_int_view(v)).cpu().numpy()
            assert np.array_equal(a, b), k


def _int_view(t):
    import torch
    return torch.int16 if t.dtype == torch.bfloat16 else torch.int32


def test_bwd_binding_rejects_bad_arguments():
    """The binding's own checks raise before anything is enqueued."""
    import torch
    import selective_state_space_scan_amd as ssm
    w, inp = _case("bf16", 16, 100, 2, 32, seed=77, extras=False)
    dev = to_device(inp, "bf16")
    dy = torch.from_numpy(inp["dy"]).cuda().to(torch.bfloat16)
    _, _, cs = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                      return_chunk_states=True, chunk_len=ssm.bwd_chunk_len(16))
    args = (dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"])
    with pytest.raises(ValueError):
        ssm.selective_scan_bwd(*args, torch.full((2,), 100, dtype=torch.int64, device="cuda"), dy, cs)
    with pytest.raises(ValueError):
        ssm.selective_scan_bwd(*args, None, dy, cs[:, :1].contiguous())
    with pytest.raises(ValueError):
        ssm.selective_scan_bwd(*args, None, dy, cs, z=dev["x"].float())
    with pytest.raises(ValueError):
        ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A_log"][:, 0].contiguous(), dev["B"], dev["C"],
                               dev["D"], None, dy, cs)
    torch.cuda.synchronize()
    g = ssm.selective_scan_bwd(*args, None, dy, cs)  # and the good call still works
    torch.cuda.synchronize()
    assert torch.isfinite(g["dx"].float()).all()


def test_bwd_outputs_only_4_byte_aligned():
    """dB and dC, or the workspace, only 4-byte (not 16-byte) aligned, through
    the raw entry point: the same bits as the binding's call with its own
    (aligned) buffers."""
    import torch
    import selective_state_space_scan_amd as ssm
    w, inp = _case("bf16", 16, 300, 2, 32, seed=91, varlen=[300, 177], extras=False)
    dev = to_device(inp, "bf16")
    dy = torch.from_numpy(inp["dy"]).cuda().to(torch.bfloat16)
    dhl = torch.from_numpy(inp["dh_last"]).cuda()
    cl = ssm.bwd_chunk_len(16)
    _, _, cs = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                      dev["valid_len"], return_chunk_states=True, chunk_len=cl)
    ref = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                 dev["valid_len"], dy, cs, dh_last=dhl)
    torch.cuda.synchronize()
    nb, L, nd = dev["x"].shape
    n = nb * L * 16
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate = nb, L, nd, 16
    dims.io_dtype, dims.delta_softplus = ssm.SSM_IO_BF16, 1
    nbytes = ssm.bwd_workspace_bytes(dims)
    p = lambda t: None if t is None else t.data_ptr()
    h = ssm._binding.handle_for(torch.cuda.current_device())
    for outs_off, ws_off in ((1, 0), (0, 4)):
        big = torch.full((2 * n + 8,), float("nan"), dtype=torch.float32, device="cuda")
        # dB 4 bytes and dC 8 bytes past a 256-byte boundary, or both aligned
        dB, dC = (big[1:1 + n], big[n + 2:2 * n + 2]) if outs_off else (big[:n], big[n + 4:2 * n + 4])
        out = {k: torch.empty_like(v) for k, v in ref.items() if v is not None and k not in ("dB", "dC")}
        ws = torch.empty(nbytes + 16, dtype=torch.uint8, device="cuda")[ws_off:ws_off + nbytes]
        bio = ssm.ssm_scan_bwd_io(p(dy), p(dhl), p(cs), p(out["dx"]), p(out["ddelta"]), None, p(out["dA_log"]),
                                  p(dB), p(dC), p(out["dD"]), None, p(out["dh0"]), p(ws), nbytes)
        rc = ssm.ssm_selective_scan_bwd(h, p(dev["x"]), p(dev["delta"]), p(dev["A_log"]), p(dev["B"]), p(dev["C"]),
                                        p(dev["D"]), p(dev["valid_len"]), dims, None, bio,
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == ssm.SSM_OK
        torch.cuda.synchronize()
        for k, got in (("dB", dB), ("dC", dC), ("dx", out["dx"]), ("dA_log", out["dA_log"])):
            bits = torch.int16 if got.dtype == torch.bfloat16 else torch.int32
            a = got.contiguous().view(bits).reshape(-1).cpu().numpy()
            b = ref[k].contiguous().view(bits).reshape(-1).cpu().numpy()
            assert np.array_equal(a, b), (k, outs_off, ws_off)


def test_bwd_length_paired_rows_bit_exact():
    """The backward at exactly two (row, channel-group) workgroups per CU with
    rows of their own lengths takes the length-paired row order; without the
    last row (one group short of the pairing, the same four-wave unsplit
    kernel otherwise) it does not.  Every per-row gradient (dx, ddelta, dB,
    dC, dh0) of the other rows is the same bit for bit either way."""
    import torch
    import selective_state_space_scan_amd as ssm
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nd = 512
    nb = 2 * cus // (nd // 16)
    if nb < 3 or nb > 64 or (2 * cus) % (nd // 16) or cus % 8 or (cus // 8) % (nd // 16):
        pytest.skip("the pairing needs whole rows per XCD half on this GPU")
    T = ssm.bwd_chunk_len(16)
    L = 9 * T + 5
    vl = np.random.default_rng(6).integers(1, L + 1, size=nb).astype(np.int32)
    vl[0], vl[1], vl[2] = 0, L, vl[3]
    w, inp = _case("bf16", 16, L, nb, nd, seed=61, varlen=vl, extras=False)
    g = _gpu(inp, "bf16")
    sub = {k: (v[:nb - 1] if k in ("x", "delta", "B", "C", "dy", "dh_last", "valid_len") else v) for k, v in inp.items()}
    gs = _gpu(sub, "bf16")
    for k in ("dx", "ddelta", "dB", "dC", "dh0"):
        a = g[k][:nb - 1].float().cpu().numpy()
        assert np.array_equal(a, gs[k].float().cpu().numpy()), k
