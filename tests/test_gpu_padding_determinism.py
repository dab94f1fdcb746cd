"""Bit-exact valid-length handling, determinism and concurrent streams (needs the GPU)."""
import numpy as np
import pytest

from gpu_util import run_gpu, to_device, to_np64
from selective_state_space_scan_amd import inputs as I

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


LENGTHS = [0, 1, 3, 4, 5, 63, 64, 65, 127, 128, 129, 255, 256, 257, 600, 999, 1000]


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("parts", [1, None])
def test_padding_bit_exact(io, N, parts):
    """pwwt.cn section 2.3 / 5.2: padding is the identity and must not touch
    the valid outputs.  y at padded steps is +0.0; garbage (NaN, Inf) in the
    padding changes nothing; valid_len = L matches no valid_len; without a time
    split, a padded row equals the same row run alone with its own length
    (bitwise).  parts None: the library's own time split (7 parts at N = 64)."""
    import functools
    import torch
    run = functools.partial(run_gpu, time_parts=parts)
    L = 1000
    base = I.WORKLOADS[0] if io == "f32" else I.WORKLOADS[3]
    w = I.small_workload(base, batch=len(LENGTHS), seqlen=L, dim=32)
    w = type(w)(**{**w.__dict__, "dstate": N, "varlen_lo": None})
    inp = I.make_inputs(w, 31337 + N)
    inp["valid_len"] = np.array(LENGTHS, np.int32)
    dev = to_device(inp, io)
    y, h = run(dev)
    yb, hb = _bits(y), _bits(h)
    for b, l in enumerate(LENGTHS):
        assert np.all(yb[b, l:] == 0), f"row {b}: padded y must be +0.0 bits"
    # garbage in the padding
    garb = {k: dev[k].clone() for k in ("x", "delta", "B", "C")}
    for b, l in enumerate(LENGTHS):
        garb["x"][b, l:] = float("nan")
        garb["delta"][b, l:] = float("inf")
        garb["B"][b, l:] = float("nan")
        garb["C"][b, l:] = float("-inf")
    y2, h2 = run(dict(dev, **garb))
    assert np.array_equal(_bits(y2), yb) and np.array_equal(_bits(h2), hb)
    # each row alone, truncated to its length (a split depends on the length)
    for b, l in enumerate(LENGTHS):
        if l == 0:
            assert np.all(to_np64(h[b]) == 0.0)
            continue
        if parts != 1:
            continue
        one = {k: dev[k][b:b + 1, :l].contiguous() for k in ("x", "delta", "B", "C")}
        one.update(A_log=dev["A_log"], D=dev["D"], valid_len=None)
        y1, h1 = run(one)
        assert np.array_equal(_bits(y1)[0], yb[b, :l]), f"row {b} (len {l}): y differs from the row run alone"
        assert np.array_equal(_bits(h1)[0], hb[b]), f"row {b} (len {l}): h_last differs"
    # valid_len all = L vs none; and out-of-range lengths clamp
    full = dict(dev, valid_len=torch.full((w.batch,), L, dtype=torch.int32, device=y.device))
    over = dict(dev, valid_len=torch.full((w.batch,), L + 7, dtype=torch.int32, device=y.device))
    none = dict(dev, valid_len=None)
    r_full, r_over, r_none = run(full), run(over), run(none)
    assert np.array_equal(_bits(r_full[0]), _bits(r_none[0])) and np.array_equal(_bits(r_full[1]), _bits(r_none[1]))
    assert np.array_equal(_bits(r_over[0]), _bits(r_none[0])) and np.array_equal(_bits(r_over[1]), _bits(r_none[1]))
    neg = dict(dev, valid_len=torch.full((w.batch,), -5, dtype=torch.int32, device=y.device))
    yn, hn = run(neg)
    assert np.all(_bits(yn) == 0) and np.all(_bits(hn) == 0)


def test_config3_lengths_bit_exact_rows():
    """The variable-length workload recipe (lengths uniform in [128, 8192]) at
    reduced width: each padded row equals that row run alone, bitwise."""
    w = I.small_workload(I.WORKLOADS[3], batch=6, seqlen=8192, dim=16)
    inp = I.make_inputs(w, I.seed_for(3) + 7)
    dev = to_device(inp, w.io)
    y, h = run_gpu(dev, time_parts=1)
    for b in range(w.batch):
        l = int(inp["valid_len"][b])
        one = {k: dev[k][b:b + 1, :l].contiguous() for k in ("x", "delta", "B", "C")}
        one.update(A_log=dev["A_log"], D=dev["D"], valid_len=None)
        y1, h1 = run_gpu(one, time_parts=1)
        assert np.array_equal(_bits(y1)[0], _bits(y)[b, :l]) and np.array_equal(_bits(h1)[0], _bits(h)[b])
        assert np.all(_bits(y)[b, l:] == 0)


@pytest.mark.parametrize("nd", [512, 128])
def test_length_paired_rows_bit_exact(nd):
    """Rows with their own lengths at exactly two (row, 16-channel) workgroups
    per CU take the length-paired row order (the longest row shares its CUs
    with the shortest): each row still equals the row run alone, bitwise,
    with tied lengths and an empty row among them (16 rows of 512 channels,
    and 64 rows of 128, the most rows the pairing ranks)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nb = 2 * cus // (nd // 16)
    if nb < 2 or nb > 64 or (2 * cus) % (nd // 16) or cus % 8 or (cus // 8) % (nd // 16):
        pytest.skip("the pairing needs whole rows per XCD half on this GPU")
    L = 700 if nb <= 16 else 300
    w = I.small_workload(I.WORKLOADS[3], batch=nb, seqlen=L, dim=nd)
    inp = I.make_inputs(w, 4321)
    vl = np.random.default_rng(5).integers(1, L + 1, size=nb).astype(np.int32)
    vl[0], vl[1], vl[2], vl[3] = 0, L, 300, 300
    inp["valid_len"] = vl
    dev = to_device(inp, w.io)
    y, h = run_gpu(dev, time_parts=1)
    for b in range(nb):
        l = int(vl[b])
        if l == 0:
            assert np.all(_bits(y)[b] == 0) and np.all(_bits(h)[b] == 0)
            continue
        one = {k: dev[k][b:b + 1, :l].contiguous() for k in ("x", "delta", "B", "C")}
        one.update(A_log=dev["A_log"], D=dev["D"], valid_len=None)
        y1, h1 = run_gpu(one, time_parts=1)
        assert np.array_equal(_bits(y1)[0], _bits(y)[b, :l]), b
        assert np.array_equal(_bits(h1)[0], _bits(h)[b]), b
        assert np.all(_bits(y)[b, l:] == 0), b


def test_determinism():
    """pwwt.cn section 5.2: the same input twice must give the same bits."""
    w = I.small_workload(I.WORKLOADS[2], batch=4, seqlen=2048, dim=256)
    dev = to_device(I.make_inputs(w, 99), w.io)
    ya, ha = run_gpu(dev)
    ya, ha = ya.clone(), ha.clone()
    for _ in range(3):
        yb, hb = run_gpu(dev)
        assert np.array_equal(_bits(ya), _bits(yb)) and np.array_equal(_bits(ha), _bits(hb))


def test_concurrent_streams():
    """pwwt.cn section 5.2 (sporadic errors under multi-stream concurrency):
    two streams with different inputs give the serial results bitwise."""
    import torch
    import selective_state_space_scan_amd as ssm
    w = I.small_workload(I.WORKLOADS[2], batch=4, seqlen=2048, dim=512)
    d1 = to_device(I.make_inputs(w, 1), w.io)
    d2 = to_device(I.make_inputs(w, 2), w.io)
    r1 = [t.clone() for t in run_gpu(d1)]
    r2 = [t.clone() for t in run_gpu(d2)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            a = ssm.selective_scan_fwd(d1["x"], d1["delta"], d1["A_log"], d1["B"], d1["C"], d1["D"], None)
        with torch.cuda.stream(s2):
            b = ssm.selective_scan_fwd(d2["x"], d2["delta"], d2["A_log"], d2["B"], d2["C"], d2["D"], None)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert np.array_equal(_bits(a[0]), _bits(r1[0])) and np.array_equal(_bits(a[1]), _bits(r1[1]))
        assert np.array_equal(_bits(b[0]), _bits(r2[0])) and np.array_equal(_bits(b[1]), _bits(r2[1]))


def test_explicit_stream_argument():
    """stream= given as a torch stream and as a raw hipStream_t handle (not the
    current stream): the same bits as calls on the current stream, for a
    forward that splits time (its scratch allocated by the binding) and for the
    backward."""
    import torch
    import selective_state_space_scan_amd as ssm
    w = I.small_workload(I.WORKLOADS[2], batch=2, seqlen=3000, dim=64)
    d = to_device(I.make_inputs(w, 5), w.io)
    cot = I.make_cotangents(w, 6)
    dy = torch.from_numpy(cot["dy"]).cuda().to(d["x"].dtype)
    args = (d["x"], d["delta"], d["A_log"], d["B"], d["C"], d["D"], None)
    cl = ssm.bwd_chunk_len(w.dstate)
    ref = [t.clone() for t in ssm.selective_scan_fwd(*args, time_parts=3, return_chunk_states=True, chunk_len=cl)]
    gref = {k: v.clone() for k, v in ssm.selective_scan_bwd(*args, dy, ref[2]).items() if v is not None}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for st in (s, s.cuda_stream):
        y, h, cs = ssm.selective_scan_fwd(*args, time_parts=3, return_chunk_states=True, chunk_len=cl, stream=st)
        g = ssm.selective_scan_bwd(*args, dy, cs, stream=st)
        s.synchronize()
        for a, b in zip((y, h, cs), ref):
            assert np.array_equal(_bits(a), _bits(b))
        for k, v in gref.items():
            assert np.array_equal(_bits(g[k]), _bits(v)), k


def test_h_last_optional_and_outputs_given():
    import torch
    import selective_state_space_scan_amd as ssm
    w = I.small_workload(I.WORKLOADS[2], batch=2, seqlen=500, dim=32)
    dev = to_device(I.make_inputs(w, 5), w.io)
    y_ref, h_ref = run_gpu(dev)
    y_out = torch.full_like(dev["x"], 7.0)
    y, h = ssm.selective_scan_fwd(dev["x"], dev["delta"], dev["A_log"], dev["B"], dev["C"], dev["D"], None,
                                  y=y_out, return_h_last=False)
    torch.cuda.synchronize()
    assert h is None and y is y_out and np.array_equal(_bits(y), _bits(y_ref))


def test_seqlen_zero_writes_zero_state():
    import torch
    import selective_state_space_scan_amd as ssm
    dev = torch.device("cuda:0")
    x = torch.empty((2, 0, 32), dtype=torch.bfloat16, device=dev)
    B = torch.empty((2, 0, 16), dtype=torch.bfloat16, device=dev)
    A_log = torch.zeros((32, 16), device=dev)
    h_last = torch.full((2, 32, 16), 3.0, device=dev)
    y, h = ssm.selective_scan_fwd(x, x, A_log, B, B, None, None, h_last=h_last)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 32) and torch.all(h == 0)
