"""A seeded sweep over combinations the targeted tests cover one at a time:
random shapes (ragged lengths, several tiles), dstate 16/32/64, fp32 and bf16
I/O, padded rows, every forward extra, the clip, explicit time splits and
(every fifth case) the wave-scan combine -- forward and backward against the
fp64 oracle, to the same per-tensor tolerances as the targeted tests."""
import dataclasses

import numpy as np
import pytest

from conftest import rel_err
from gpu_util import to_device, to_np64, tol_for
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu

N_CASES = 160


def _draw(case: int):
    rng = np.random.default_rng(7000 + case)
    io = ("f32", "bf16")[case % 2]
    N = (16, 32, 64)[(case // 2) % 3]
    nb = int(rng.integers(1, 4))
    L = int(rng.integers(1, 700))
    nd = 16 * int(rng.integers(1, 4))
    varlen = bool(rng.integers(0, 2))
    use = [k for k in ("h0", "delta_bias", "z") if rng.integers(0, 2)]
    clamp = (1e-3, 0.1) if rng.integers(0, 4) == 0 else None
    parts = int(rng.choice([1, 2, 3, 5]))
    return io, N, nb, L, nd, varlen, use, clamp, parts, rng


def _combine(case: int) -> str:
    return "wave_scan" if case % 5 == 4 else "walk"


def _inputs(io, N, nb, L, nd, varlen, rng, seed):
    base = I.WORKLOADS[0] if io == "f32" else I.WORKLOADS[2]
    w = dataclasses.replace(I.small_workload(base, batch=nb, seqlen=L, dim=nd), dstate=N)
    inp = I.make_inputs(w, seed)
    rnd = (lambda a: I.round_to_bf16(a)) if io == "bf16" else (lambda a: a.astype(np.float32))
    inp["h0"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
    inp["delta_bias"] = (0.5 * rng.standard_normal(nd)).astype(np.float32)
    inp["z"] = rnd(2.0 * rng.standard_normal((nb, L, nd)).astype(np.float32))
    inp["dy"] = rnd(rng.standard_normal((nb, L, nd)).astype(np.float32))
    inp["dh_last"] = rng.standard_normal((nb, nd, N)).astype(np.float32)
    if varlen:
        inp["valid_len"] = rng.integers(0, L + 3, size=nb).astype(np.int32)
    return inp


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_forward_and_backward(case):
    import torch
    import oracle
    import selective_state_space_scan_amd as ssm
    io, N, nb, L, nd, varlen, use, clamp, parts, rng = _draw(case)
    inp = _inputs(io, N, nb, L, nd, varlen, rng, seed=8000 + case)
    print(f"case {case}: io {io} N {N} nb {nb} L {L} nd {nd} varlen {varlen} use {use} clamp {clamp} "
          f"parts {parts} combine {_combine(case)}", flush=True)
    dev = to_device(inp, io)
    dt = dev["x"].dtype
    ex = {}
    if "h0" in use:
        ex["h0"] = torch.from_numpy(inp["h0"]).cuda()
    if "delta_bias" in use:
        ex["delta_bias"] = torch.from_numpy(inp["delta_bias"]).cuda()
    if "z" in use:
        ex["z"] = torch.from_numpy(inp["z"]).cuda().to(dt)
    cl = ssm.bwd_chunk_len(N)
    y, h, cs = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                      dev["valid_len"], delta_clamp=clamp, return_chunk_states=True, chunk_len=cl,
                                      time_parts=parts, combine=_combine(case), **ex)
    dy = torch.from_numpy(inp["dy"]).cuda().to(dt)
    dhl = torch.from_numpy(inp["dh_last"]).cuda()
    g = ssm.selective_scan_bwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                               dev["valid_len"], dy, cs, dh_last=dhl, delta_clamp=clamp, **ex)
    torch.cuda.synchronize()

    kw = {k: inp[k] for k in use}
    yr, hr, csr = oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"],
                                        valid_len=inp.get("valid_len"), delta_clamp=clamp, chunk_len=cl,
                                        nthreads=8, **kw)
    for k, got, ref in (("y", y, yr), ("h_last", h, hr), ("chunk_states", cs, csr)):
        assert rel_err(to_np64(got), ref) <= tol_for(io, k), k
    r = oracle.selective_scan_bwd(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"], inp["dy"],
                                  valid_len=inp.get("valid_len"), dh_last=inp["dh_last"], delta_clamp=clamp,
                                  nthreads=8, **kw)
    for k in ("dx", "ddelta", "dA_log", "dB", "dC", "dD", "ddelta_bias", "dz", "dh0"):
        if r.get(k) is None or g.get(k) is None:
            continue
        assert rel_err(to_np64(g[k]), r[k]) <= tol_for(io, k), k
