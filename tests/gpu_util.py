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
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def oracle_full(inp: dict, delta_softplus=True, delta_clamp=None, nthreads=8):
    import oracle
    return oracle.selective_scan(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp.get("D"),
                                 valid_len=inp.get("valid_len"), delta_softplus=delta_softplus,
                                 delta_clamp=delta_clamp, nthreads=nthreads)


def oracle_rows(inp: dict, rows, delta_softplus=True, delta_clamp=None, nthreads=8):
    import oracle
    return oracle.selective_scan_rows(inp["x"], inp["delta"], inp["A_log"], inp["B"], inp["C"], rows,
                                      D=inp.get("D"), valid_len=inp.get("valid_len"),
                                      delta_softplus=delta_softplus, delta_clamp=delta_clamp, nthreads=nthreads)


def tol_for(io: str) -> float:
    """Max relative error allowed (fp32 I/O: 1e-4; bf16 I/O: 2e-2)."""
    return 1e-4 if io == "f32" else 2e-2
