"""At dstate 32 and 64 the two or four lane rows that hold the state groups of
one time sub-chunk share its per-(step, channel) work: each row loads x and
delta and runs softplus, the clip and the gate for some of the sub-chunk's
steps and the rows exchange the results; the readout sums (forward) and the
sums over states (backward) are reduce-scattered so that each row finishes the
steps it stores.  At dstate 16 the forward reads out each sub-chunk's last
step as C.(Abar h) + u (C.B).  Rows whose valid length ends at every step of
a sub-chunk put the boundary between the rows' steps, and the sub-chunk's
last step, in every position; forward and backward are checked against the
fp64 oracle, with the gate, h0, a delta bias, the clip and chunk-boundary
states."""
import numpy as np
import pytest

from conftest import rel_err
from gpu_util import oracle_full, to_device, to_np64, tol_for
from test_gpu_bwd import _case, _compare, _gpu, _oracle

pytestmark = pytest.mark.gpu


def _lengths(T):
    # the last tile's sub-chunks (4 steps each in the forward, 2 in the
    # backward) cut after each of their steps, a whole row, an empty row
    return [2 * T + r for r in range(1, 9)] + [3 * T, 0]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_forward_lengths_ending_at_every_step_of_a_sub_chunk(io, N):
    import torch
    import selective_state_space_scan_amd as ssm
    T = ssm.chunk_len(N)
    lens = _lengths(T)
    w, inp = _case(io, N, 3 * T, len(lens), 32, seed=300 + N, varlen=lens)
    dev = to_device(inp, io)
    cl = T // 2
    clamp = (1e-3, 0.1) if N == 64 else None
    y, h, cs = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"],
                                      dev["valid_len"], h0=torch.from_numpy(inp["h0"]).cuda(),
                                      delta_bias=torch.from_numpy(inp["delta_bias"]).cuda(),
                                      z=torch.from_numpy(inp["z"]).cuda().to(dev["x"].dtype), delta_clamp=clamp,
                                      return_chunk_states=True, chunk_len=cl)
    torch.cuda.synchronize()
    yr, hr, csr = oracle_full(inp, delta_clamp=clamp, h0=inp["h0"], delta_bias=inp["delta_bias"], z=inp["z"],
                              chunk_len=cl)
    L = 3 * T
    mask = np.broadcast_to(np.arange(L)[None, :, None] < np.asarray(lens)[:, None, None], yr.shape)
    ey, eh, ec = rel_err(to_np64(y), yr, mask), rel_err(to_np64(h), hr), rel_err(to_np64(cs), csr)
    print(f"{io} N={N}: y {ey:.2e} h_last {eh:.2e} chunk states {ec:.2e}", flush=True)
    assert ey <= tol_for(io, "y") and eh <= tol_for(io, "h_last") and ec <= tol_for(io, "chunk_states")
    assert np.all(to_np64(y)[~mask] == 0.0)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64])
def test_backward_lengths_ending_at_every_step_of_a_sub_chunk(io, N):
    import selective_state_space_scan_amd as ssm
    T = ssm.bwd_chunk_len(N)
    lens = _lengths(T)
    w, inp = _case(io, N, 3 * T, len(lens), 32, seed=400 + N, varlen=lens)
    clamp = (1e-3, 0.1) if N == 64 else None
    _compare(_gpu(inp, io, clamp=clamp), _oracle(inp, clamp=clamp), io, f"{io} N={N}")
