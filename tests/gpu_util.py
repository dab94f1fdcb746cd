"""Helpers shared by the GPU tests: moving generated inputs to the device,
running the HIP path through the binding, and running the oracle on the same
inputs."""
from __future__ import annotations

import numpy as np


def to_device(inp: dict, io: str, device="cuda:0"):
    import torch
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for k in ("x", "delta", "B", "C"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(device=device).to(dt).contiguous()
    out["A_log"] = torch.from_numpy(np.ascontiguousarray(inp["A_log"], dtype=np.float32)).to(device)
    out["D"] = None if inp.get("D") is None else torch.from_numpy(np.asarray(inp["D"], np.float32)).to(device)
    vl = inp.get("valid_len")
    out["valid_len"] = None if vl is None else torch.from_numpy(np.asarray(vl, np.int32)).to(device)
    return out


def run_gpu(dev: dict, delta_softplus=True, delta_clamp=None, sync=True, time_parts=None):
    """The forward through the binding; time_parts None lets the library choose
    its time split (the product default), 1 disables it."""
    import torch
    import selective_state_space_scan_amd as ssm
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                  dev["valid_len"], delta_softplus=delta_softplus, delta_clamp=delta_clamp,
                                  time_parts=time_parts)
    if sync:
        torch.cuda.synchronize()
    return y, h


def to_np64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_full(inp: dict, delta_softplus=True, delta_clamp=None, nthreads=8, **extras):
    import oracle
    return oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp.get("D"),
                                 valid_len=inp.get("valid_len"), delta_softplus=delta_softplus,
                                 delta_clamp=delta_clamp, nthreads=nthreads, **extras)


def oracle_rows(inp: dict, rows, delta_softplus=True, delta_clamp=None, nthreads=8):
    import oracle
    return oracle.selective_scan_rows(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], rows,
                                      D=inp.get("D"), valid_len=inp.get("valid_len"),
                                      delta_softplus=delta_softplus, delta_clamp=delta_clamp, nthreads=nthreads)


# Outputs written in fp32 whatever the I/O type: the final and chunk-boundary
# states and the gradients of fp32 parameters and of the [B, L, N] B and C.
FP32_OUTPUTS = frozenset({"h_last", "chunk_states", "dA_log", "dB", "dC", "dD", "ddelta_bias", "dh0"})


def tol_for(io: str, out: str | None = None) -> float:
    """Max relative error allowed for one output tensor: 1e-4 for fp32 I/O and
    for every fp32 output (computed in fp32 from inputs that the bf16 rounding
    left exact, so only fp32 arithmetic separates it from the fp64 oracle);
    2e-2 for the outputs that bf16 I/O rounds to bf16 (y, dx, ddelta, dz), whose
    rounding alone is up to 2^-9 relative."""
    return 1e-4 if io == "f32" or out in FP32_OUTPUTS else 2e-2


def oracle_bwd(inp: dict, dy, dh_last, delta_clamp=None, h0=None, delta_bias=None, z=None, nthreads=16):
    """The oracle's backward over the whole problem.  Its own threads split the
    batch rows; with fewer rows than threads the channels are split too, into
    groups run on parallel Python threads (the C call releases the GIL), and dB
    and dC, which sum over every channel, are added up over the groups in fp64."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    nb, L, nd = inp["x"].shape
    groups = max(1, min(nthreads // max(nb, 1), nd // 16))
    bounds = [nd * g // groups // 16 * 16 for g in range(groups)] + [nd]

    def part(c0, c1):
        sl = slice(c0, c1)
        pick = lambda a, ax: None if a is None else np.take(a, np.arange(c0, c1), axis=ax)
        return oracle.selective_scan_bwd(
            inp["x"][:, :, sl], inp["delta"][:, :, sl], inp["A_log"][sl], inp["B"], inp["C"], pick(inp.get("D"), 0),
            dy[:, :, sl], valid_len=inp.get("valid_len"), h0=pick(h0, 1), delta_bias=pick(delta_bias, 0),
            z=pick(z, 2), dh_last=pick(dh_last, 1), delta_clamp=delta_clamp, nthreads=min(nb, nthreads))

    with ThreadPoolExecutor(groups) as ex:
        parts = list(ex.map(lambda g: part(bounds[g], bounds[g + 1]), range(groups)))
    axis = dict(dx=2, ddelta=2, dz=2, dA_log=0, dD=0, ddelta_bias=0, dh0=1)
    out = {k: (None if parts[0][k] is None else np.concatenate([p[k] for p in parts], axis=ax))
           for k, ax in axis.items()}
    for k in ("dB", "dC"):
        out[k] = np.sum([p[k] for p in parts], axis=0)
    return out
