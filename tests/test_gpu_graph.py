"""The forward and backward captured into a HIP graph (torch.cuda.CUDAGraph)
and replayed several times, with eager work and synchronisations between the
replays: every replay must equal the eager call on the same inputs bit for bit
(the library issues kernels only, no memset or allocation, so a captured call
is the same launches)."""
import dataclasses

import numpy as np
import pytest

from gpu_util import to_device
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.detach().contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _inputs(seed, nb=3, L=1100, nd=64, N=16, varlen=(1100, 517, 0)):
    w = dataclasses.replace(I.small_workload(I.WORKLOADS[2], batch=nb, seqlen=L, dim=nd), dstate=N)
    inp = I.make_inputs(w, seed)
    inp["valid_len"] = np.asarray(varlen, dtype=np.int32)
    return to_device(inp, w.io)


def _fwd(ssm, d, parts, ws, out=None):
    y, h = (None, None) if out is None else out
    return ssm.selective_scan_fwd(d["x"], d["delta"], d["A_log"], d["B"], d["C"], d["D"], d["valid_len"], y=y,
                                  h_last=h, time_parts=parts, workspace=ws)


def _load(static, src):
    for k in ("x", "delta", "B", "C", "A_log", "valid_len"):
        static[k].copy_(src[k])
    static["D"].copy_(src["D"])


@pytest.mark.parametrize("parts", [1, 4])
def test_forward_graph_replays(parts):
    import torch
    import selective_state_space_scan_amd as ssm
    static = _inputs(31)
    other = _inputs(32)
    ws = None
    if parts > 1:
        dims = ssm.ssm_scan_dims()
        dims.batch, dims.seqlen, dims.dim = static["x"].shape
        dims.dstate = static["A_log"].shape[1]
        dims.io_dtype = ssm.SSM_IO_BF16
        ws = torch.empty(ssm.workspace_bytes(dims, parts), dtype=torch.uint8, device="cuda")
    ref_static = [t.clone() for t in _fwd(ssm, static, parts, ws)]
    ref_other = [t.clone() for t in _fwd(ssm, other, parts, ws)]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            y, h = _fwd(ssm, static, parts, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for i in range(4):
        # eager work of the program between replays, on the same workspace
        y.fill_(float("nan"))
        h.fill_(float("nan"))
        _fwd(ssm, other, parts, ws)
        torch.cuda.synchronize()
        if i == 2:
            _load(static, other)
        g.replay()
        torch.cuda.synchronize()
        want = ref_other if i >= 2 else ref_static
        assert np.array_equal(_bits(y), _bits(want[0])), f"replay {i}: y differs"
        assert np.array_equal(_bits(h), _bits(want[1])), f"replay {i}: h_last differs"


def test_backward_graph_replays():
    import torch
    import selective_state_space_scan_amd as ssm
    static = _inputs(41)
    rng = np.random.default_rng(42)
    dy = torch.from_numpy(I.round_to_bf16(rng.standard_normal(static["x"].shape).astype(np.float32))).cuda()
    dy = dy.to(torch.bfloat16)
    nb, _, nd = static["x"].shape
    N = static["A_log"].shape[1]
    dhl = torch.from_numpy(rng.standard_normal((nb, nd, N)).astype(np.float32)).cuda()
    cl = ssm.bwd_chunk_len(N)

    def step():
        y, h, cs = ssm.selective_scan_fwd(static["x"], static["delta"], static["A_log"], static["B"], static["C"],
                                          static["D"], static["valid_len"], return_chunk_states=True, chunk_len=cl,
                                          time_parts=1)
        g = ssm.selective_scan_bwd(static["x"], static["delta"], static["A_log"], static["B"], static["C"],
                                   static["D"], static["valid_len"], dy, cs, dh_last=dhl)
        return y, g

    y_ref, g_ref = step()
    g_ref = {k: v.clone() for k, v in g_ref.items() if v is not None}
    y_ref = y_ref.clone()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            y, g = step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for i in range(3):
        for v in g.values():
            if v is not None:
                v.fill_(float("nan"))
        step()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y), _bits(y_ref)), f"replay {i}: y differs"
        for k, v in g_ref.items():
            assert np.array_equal(_bits(g[k]), _bits(v)), f"replay {i}: {k} differs"


def test_noalloc_forward_graph_replays():
    """The allocation-free forward (the time split's carries in the library's
    static scratch) captured into a graph: each replay equals the eager call,
    also after eager calls on other inputs have overwritten the scratch."""
    import torch
    import selective_state_space_scan_amd as ssm
    static = _inputs(41, nb=1, L=3000, nd=256, varlen=(2999,))
    other = _inputs(42, nb=1, L=3000, nd=256, varlen=(3000,))
    dims = ssm.ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim = static["x"].shape
    dims.dstate = static["A_log"].shape[1]
    dims.io_dtype, dims.delta_softplus = ssm.SSM_IO_BF16, 1
    h = ssm._binding.handle_for(torch.cuda.current_device())
    parts = ssm.auto_time_parts(h, dims)
    assert parts >= 2  # the scratch is in use
    ex = ssm.ssm_scan_fwd_extras(None, None, None, None, 0, 0, None, 0)

    def call(d, y, hl, stream):
        args = [d[k].data_ptr() for k in ("x", "delta", "A_log", "B", "C", "D", "valid_len")]
        rc = ssm.ssm_selective_scan_fwd_noalloc(h, *args, y.data_ptr(), hl.data_ptr(), dims, ex, stream)
        assert rc == ssm.SSM_OK, ssm.error_string(rc)

    cur = torch.cuda.current_stream().cuda_stream
    refs = {}
    for name, d in (("static", static), ("other", other)):
        y, hl = torch.empty_like(d["x"]), torch.empty((1, 256, 16), dtype=torch.float32, device="cuda")
        call(d, y, hl, cur)
        refs[name] = (y, hl)
    torch.cuda.synchronize()
    y = torch.empty_like(static["x"])
    hl = torch.empty((1, 256, 16), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(static, y, hl, s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    y2, h2 = torch.empty_like(y), torch.empty_like(hl)
    for i in range(4):
        y.fill_(float("nan"))
        hl.fill_(float("nan"))
        call(other, y2, h2, cur)  # rewrites the scratch with another problem's carries
        torch.cuda.synchronize()
        if i == 2:
            _load(static, other)
        g.replay()
        torch.cuda.synchronize()
        want = refs["other"] if i >= 2 else refs["static"]
        assert np.array_equal(_bits(y), _bits(want[0])), f"replay {i}: y differs"
        assert np.array_equal(_bits(hl), _bits(want[1])), f"replay {i}: h_last differs"
