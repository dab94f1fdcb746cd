"""The C ABI library on the host (no GPU needed): it loads, exports every
function declared in include/ssm_scan.h, and rejects bad arguments with the
documented codes before touching the GPU (argument checks precede the handle
check, so a NULL handle reaches them)."""
import ctypes
import os
import re

import pytest

import selective_state_space_scan_amd as ssm

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(REPO, "include", "ssm_scan.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(ssm.EXPORTED), names
    lib = ctypes.CDLL(ssm.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_error_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99, 5):
        s = ssm.error_string(code)
        assert isinstance(s, str) and s


def _dims(**kw):
    d = ssm.ssm_scan_dims()
    d.batch, d.seqlen, d.dim, d.dstate = kw.get("batch", 2), kw.get("seqlen", 8), kw.get("dim", 16), kw.get("dstate", 16)
    d.io_dtype = kw.get("io", ssm.SSM_IO_BF16)
    d.delta_softplus = kw.get("softplus", 1)
    d.delta_clamp = kw.get("clamp", 0)
    d.delta_min, d.delta_max = kw.get("dmin", 0.0), kw.get("dmax", 0.0)
    return d


MB = 1 << 20
# Fake, non-overlapping, aligned addresses: never dereferenced, since every call
# below fails an argument check (or the NULL-handle check) first.
PTRS = dict(x=1 * MB, delta=2 * MB, A_log=3 * MB, B=4 * MB, C=5 * MB, D=None, valid_len=None, y=6 * MB, h_last=7 * MB)


def call(dims, **over):
    p = dict(PTRS, **over)
    return ssm.ssm_selective_scan_fwd(over.get("handle"), p["x"], p["delta"], p["A_log"], p["B"], p["C"], p["D"],
                                      p["valid_len"], p["y"], p["h_last"], dims, None)


def test_valid_arguments_reach_the_handle_check():
    assert call(_dims()) == ssm.SSM_ERR_INVALID_ARG  # NULL handle


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), ssm.SSM_ERR_INVALID_ARG),
    (dict(seqlen=-1), ssm.SSM_ERR_INVALID_ARG),
    (dict(dim=-16), ssm.SSM_ERR_INVALID_ARG),
    (dict(io=7), ssm.SSM_ERR_INVALID_ARG),
    (dict(softplus=2), ssm.SSM_ERR_INVALID_ARG),
    (dict(clamp=3), ssm.SSM_ERR_INVALID_ARG),
    (dict(clamp=1, dmin=0.5, dmax=0.1), ssm.SSM_ERR_INVALID_ARG),
    (dict(clamp=1, dmin=-1.0, dmax=0.1), ssm.SSM_ERR_INVALID_ARG),
    (dict(dstate=8), ssm.SSM_ERR_UNSUPPORTED),
    (dict(dstate=17), ssm.SSM_ERR_UNSUPPORTED),
    (dict(dim=24), ssm.SSM_ERR_UNSUPPORTED),
    # grid limits: one workgroup per (row, 16 channels), fewer than 2^31 of them
    (dict(batch=2**31, dim=16), ssm.SSM_ERR_UNSUPPORTED),
    (dict(batch=2**20, dim=2**16), ssm.SSM_ERR_UNSUPPORTED),
])
def test_bad_dims(kw, code):
    assert call(_dims(**kw)) == code


TB = 1 << 40
# Fake addresses 1 TiB apart, so that rows of up to 2 GiB never overlap.
FAR = dict(x=1 * TB, delta=2 * TB, A_log=3 * TB, B=4 * TB, C=5 * TB, D=None, valid_len=None, y=6 * TB,
           h_last=7 * TB)


@pytest.mark.parametrize("io,esz,dim,dstate", [(ssm.SSM_IO_BF16, 2, 1024, 16), (ssm.SSM_IO_F32, 4, 1024, 16),
                                               (ssm.SSM_IO_BF16, 2, 16, 64)])
def test_row_size_limit(io, esz, dim, dstate):
    """A batch row of x, delta, y (or of B, C when dstate > dim) must span fewer
    than 2^31 bytes: the longest such sequence passes every argument check (and
    meets the NULL handle), one step more is unsupported -- forward and
    backward."""
    longest = (2**31 - 1) // (max(dim, dstate) * esz)
    ok = _dims(batch=1, seqlen=longest, dim=dim, dstate=dstate, io=io)
    over = _dims(batch=1, seqlen=longest + 1, dim=dim, dstate=dstate, io=io)
    assert call(ok, **FAR) == ssm.SSM_ERR_INVALID_ARG  # the handle
    assert call(over, **FAR) == ssm.SSM_ERR_UNSUPPORTED
    bio = ssm.ssm_scan_bwd_io(dy=8 * TB, chunk_states=9 * TB, dx=10 * TB, ddelta=11 * TB, dA_log=12 * TB,
                              dB=13 * TB, dC=14 * TB, workspace=16 * TB, workspace_bytes=1 << 62)

    def bwd(d):
        return ssm.ssm_selective_scan_bwd(None, FAR["x"], FAR["delta"], FAR["A_log"], FAR["B"], FAR["C"], None,
                                          None, d, None, bio, None)

    assert bwd(ok) == ssm.SSM_ERR_INVALID_ARG  # the handle
    assert bwd(over) == ssm.SSM_ERR_UNSUPPORTED


def test_null_dims():
    lib = ssm.lib()
    assert lib.ssm_selective_scan_fwd(None, 1, 2, 3, 4, 5, None, None, 6, None, None, None) == ssm.SSM_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["x", "delta", "A_log", "B", "C", "y"])
def test_null_required_pointer(name):
    assert call(_dims(), **{name: None}) == ssm.SSM_ERR_INVALID_ARG


def test_misaligned_pointers():
    assert call(_dims(io=ssm.SSM_IO_BF16), x=1 * MB + 1) == ssm.SSM_ERR_UNSUPPORTED
    assert call(_dims(io=ssm.SSM_IO_F32), x=1 * MB + 2) == ssm.SSM_ERR_UNSUPPORTED
    assert call(_dims(), A_log=3 * MB + 2) == ssm.SSM_ERR_UNSUPPORTED
    assert call(_dims(), h_last=7 * MB + 2) == ssm.SSM_ERR_UNSUPPORTED


def test_aliasing():
    assert call(_dims(), y=PTRS["x"]) == ssm.SSM_ERR_ALIAS
    assert call(_dims(), y=PTRS["B"] + 2) == ssm.SSM_ERR_ALIAS
    assert call(_dims(), h_last=PTRS["A_log"]) == ssm.SSM_ERR_ALIAS
    assert call(_dims(), h_last=PTRS["y"]) == ssm.SSM_ERR_ALIAS
    # adjacent but disjoint ranges are fine (y = 2*8*16*2 bytes below h_last)
    assert call(_dims(), y=7 * MB - 2 * 8 * 16 * 2) == ssm.SSM_ERR_INVALID_ARG


def _ex_call(dims, extras, **over):
    p = dict(PTRS, **over)
    return ssm.ssm_selective_scan_fwd_ex(None, p["x"], p["delta"], p["A_log"], p["B"], p["C"], p["D"],
                                         p["valid_len"], p["y"], p["h_last"], dims, extras, None)


def test_extras_checks():
    E = ssm.ssm_scan_fwd_extras
    assert ssm.chunk_len(16) == 128 and ssm.chunk_len(32) == 64 and ssm.chunk_len(64) == 32
    assert ssm.chunk_len(8) == 0
    # NULL extras and all-NULL extras reach the handle check
    assert _ex_call(_dims(), None) == ssm.SSM_ERR_INVALID_ARG
    assert _ex_call(_dims(), E()) == ssm.SSM_ERR_INVALID_ARG
    # chunk states: a multiple of 4 that divides the tile (128 at dstate 16)
    for bad in (0, -4, 2, 6, 12, 256):
        assert _ex_call(_dims(), E(chunk_states=8 * MB, chunk_len=bad)) == ssm.SSM_ERR_INVALID_ARG, bad
    bad_x = dict(x=PTRS["x"] + 1)  # fails the later alignment check when the chunk length is accepted
    for good in (4, 8, 16, 32, 64, 128):
        assert _ex_call(_dims(), E(chunk_states=8 * MB, chunk_len=good), **bad_x) == ssm.SSM_ERR_UNSUPPORTED, good
    assert _ex_call(_dims(dstate=64), E(chunk_states=8 * MB, chunk_len=64), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    # misaligned extras
    assert _ex_call(_dims(), E(h0=8 * MB + 2)) == ssm.SSM_ERR_UNSUPPORTED
    assert _ex_call(_dims(io=ssm.SSM_IO_BF16), E(z=8 * MB + 1)) == ssm.SSM_ERR_UNSUPPORTED
    # outputs must not overlap the extra inputs; h0 may be h_last itself
    assert _ex_call(_dims(), E(z=PTRS["y"])) == ssm.SSM_ERR_ALIAS
    assert _ex_call(_dims(), E(h0=PTRS["h_last"] + 4)) == ssm.SSM_ERR_ALIAS
    assert _ex_call(_dims(), E(h0=PTRS["h_last"])) == ssm.SSM_ERR_INVALID_ARG  # in place: reaches the handle check
    assert _ex_call(_dims(), E(chunk_states=PTRS["x"], chunk_len=128)) == ssm.SSM_ERR_ALIAS
    assert _ex_call(_dims(), E(chunk_states=PTRS["h_last"], chunk_len=128)) == ssm.SSM_ERR_ALIAS
    # the combine: walk (0) or wave scan (1)
    assert _ex_call(_dims(), E(combine=ssm.SSM_COMBINE_WAVE_SCAN)) == ssm.SSM_ERR_INVALID_ARG  # the NULL handle
    assert _ex_call(_dims(), E(combine=ssm.SSM_COMBINE_WAVE_SCAN), x=PTRS["x"] + 1) == ssm.SSM_ERR_UNSUPPORTED
    for bad in (2, -1):
        assert _ex_call(_dims(), E(combine=bad), x=PTRS["x"] + 1) == ssm.SSM_ERR_INVALID_ARG, bad


def test_time_split_checks():
    E = ssm.ssm_scan_fwd_extras
    d = _dims(batch=2, seqlen=1000, dim=32, dstate=16)
    # 8 tiles of 128 steps; 3 parts of 3, 3 and 2 tiles: two state blocks and one delta-sum block
    assert ssm.workspace_bytes(d, 3) == 4 * (2 * 2 * 32 * 16 + 2 * 32)
    assert ssm.workspace_bytes(d, 2) == 4 * (2 * 32 * 16)
    assert ssm.workspace_bytes(d, 1) == 0 and ssm.workspace_bytes(d, 0) == 0
    assert ssm.workspace_bytes(d, 100) == 4 * (7 * 2 * 32 * 16 + 6 * 2 * 32)  # at most one part per tile
    assert ssm.workspace_bytes(d, -1) == -1 and ssm.workspace_bytes(_dims(dstate=8), 2) == -1
    assert ssm.workspace_bytes(_dims(seqlen=100, dstate=16), 4) == 0  # one tile: no split
    assert ssm.auto_time_parts(None, d) == 1
    need = ssm.workspace_bytes(d, 3)
    bad_x = dict(x=PTRS["x"] + 1)  # a misaligned input: fails after the extras checks
    # an explicit split with too small (or no) workspace is rejected before anything else
    assert _ex_call(d, E(time_parts=3, workspace=8 * MB, workspace_bytes=need - 4), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert _ex_call(d, E(time_parts=3), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert _ex_call(d, E(time_parts=3, workspace=8 * MB, workspace_bytes=need), **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    assert _ex_call(d, E(time_parts=-1), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert _ex_call(d, E(workspace_bytes=64), **bad_x) == ssm.SSM_ERR_INVALID_ARG  # bytes without a pointer
    # automatic and no split never need a workspace
    assert _ex_call(d, E(time_parts=0), **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    assert _ex_call(d, E(time_parts=1), **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    # the workspace must be aligned and overlap nothing
    assert _ex_call(d, E(time_parts=3, workspace=8 * MB + 2, workspace_bytes=need)) == ssm.SSM_ERR_UNSUPPORTED
    assert _ex_call(d, E(time_parts=3, workspace=PTRS["B"], workspace_bytes=need)) == ssm.SSM_ERR_ALIAS
    assert _ex_call(d, E(time_parts=3, workspace=PTRS["y"] - 64, workspace_bytes=need)) == ssm.SSM_ERR_ALIAS
    assert _ex_call(d, E(time_parts=3, workspace=PTRS["h_last"], workspace_bytes=need)) == ssm.SSM_ERR_ALIAS
    assert _ex_call(d, E(time_parts=3, workspace=8 * MB, workspace_bytes=need)) == ssm.SSM_ERR_INVALID_ARG  # handle


def _na_call(dims, extras, **over):
    p = dict(PTRS, **over)
    return ssm.ssm_selective_scan_fwd_noalloc(None, p["x"], p["delta"], p["A_log"], p["B"], p["C"], p["D"],
                                              p["valid_len"], p["y"], p["h_last"], dims, extras, None)


def test_noalloc_checks():
    """The allocation-free forward: the checks of the extended entry point, no
    caller workspace, and explicit splits bounded by the static scratch."""
    E = ssm.ssm_scan_fwd_extras
    assert ssm.SSM_SCAN_NOALLOC_SCRATCH_BYTES == 16 << 20
    d = _dims(batch=2, seqlen=1000, dim=32, dstate=16)
    bad_x = dict(x=PTRS["x"] + 1)  # a misaligned input: fails after the extras checks
    assert _na_call(d, None) == ssm.SSM_ERR_INVALID_ARG  # valid: the NULL handle
    assert _na_call(d, E(time_parts=3)) == ssm.SSM_ERR_INVALID_ARG
    assert _na_call(d, E(time_parts=3), **bad_x) == ssm.SSM_ERR_UNSUPPORTED  # no workspace needed
    # a caller workspace is refused
    need = ssm.workspace_bytes(d, 3)
    assert _na_call(d, E(time_parts=3, workspace=8 * MB, workspace_bytes=need), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert _na_call(d, E(workspace=8 * MB), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert _na_call(d, E(workspace_bytes=64), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    # two parts carry one [batch, dim, dstate] block: 64 x 4096 x 16 floats is
    # exactly the scratch, one more row is too much
    at = _dims(batch=64, seqlen=256, dim=4096, dstate=16)
    assert ssm.workspace_bytes(at, 2) == ssm.SSM_SCAN_NOALLOC_SCRATCH_BYTES
    assert _na_call(at, E(time_parts=2), **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    over = _dims(batch=65, seqlen=256, dim=4096, dstate=16)
    assert _na_call(over, E(time_parts=2)) == ssm.SSM_ERR_SCRATCH
    big = _dims(batch=16, seqlen=32768, dim=2048, dstate=64)
    assert ssm.workspace_bytes(big, 16) > ssm.SSM_SCAN_NOALLOC_SCRATCH_BYTES
    assert _na_call(big, E(time_parts=16)) == ssm.SSM_ERR_SCRATCH
    # the automatic split never fails for size: it runs unsplit instead
    assert _na_call(big, E(time_parts=0), **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    assert _na_call(over, None, **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    # the other checks are those of the extended entry point
    assert _na_call(d, E(h0=PTRS["h_last"] + 4)) == ssm.SSM_ERR_ALIAS
    assert _na_call(d, E(chunk_states=8 * MB, chunk_len=6)) == ssm.SSM_ERR_INVALID_ARG
    assert ssm.error_string(ssm.SSM_ERR_SCRATCH) != ssm.error_string(-99)


def test_bwd_checks():
    import ctypes
    BIO = ssm.ssm_scan_bwd_io
    E = ssm.ssm_scan_fwd_extras
    assert ssm.bwd_chunk_len(16) == 32 and ssm.bwd_chunk_len(32) == 16 and ssm.bwd_chunk_len(64) == 8
    assert ssm.bwd_chunk_len(8) == 0
    d = _dims(batch=2, seqlen=100, dim=32, dstate=16)
    need = ssm.bwd_workspace_bytes(d)
    assert need == 4 * (2 * 2 * 2 * 100 * 16 + 31 * 2 * 32 * 16 + 47 * 2 * 32)
    assert ssm.bwd_workspace_bytes(_dims(dstate=8)) == -1 and ssm.bwd_workspace_bytes(_dims(dim=24)) == -1

    def io(**kw):
        base = dict(dy=8 * MB, chunk_states=9 * MB, dx=10 * MB, ddelta=11 * MB, dA_log=12 * MB, dB=13 * MB,
                    dC=14 * MB, workspace=16 * MB, workspace_bytes=need)
        base.update(kw)
        return BIO(**base)

    def call(bio, dims=d, extras=None, **over):
        p = dict(PTRS, **over)
        return ssm.ssm_selective_scan_bwd(None, p["x"], p["delta"], p["A_log"], p["B"], p["C"], p["D"],
                                          p["valid_len"], dims, extras, bio, None)

    assert call(io()) == ssm.SSM_ERR_INVALID_ARG  # everything valid: the NULL handle
    bad_x = dict(x=PTRS["x"] + 1)
    assert call(io(), **bad_x) == ssm.SSM_ERR_UNSUPPORTED  # misaligned input
    assert call(io(workspace_bytes=need - 4), **bad_x) == ssm.SSM_ERR_INVALID_ARG  # workspace too small
    assert call(io(workspace=None), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert call(io(chunk_states=None), **bad_x) == ssm.SSM_ERR_INVALID_ARG  # 100 steps > one 32-step tile
    assert call(io(chunk_states=None), dims=_dims(batch=2, seqlen=32, dim=32, dstate=16), **bad_x) == \
        ssm.SSM_ERR_UNSUPPORTED  # one tile needs no chunk states
    for k in ("dy", "dx", "ddelta", "dA_log", "dB", "dC"):
        assert call(io(**{k: None}), **bad_x) == ssm.SSM_ERR_INVALID_ARG, k
    # the gate needs dz
    assert call(io(), extras=E(z=15 * MB), **bad_x) == ssm.SSM_ERR_INVALID_ARG
    assert call(io(dz=17 * MB), extras=E(z=15 * MB), **bad_x) == ssm.SSM_ERR_UNSUPPORTED
    # outputs may not overlap inputs, each other or the workspace
    assert call(io(dx=PTRS["x"])) == ssm.SSM_ERR_ALIAS
    assert call(io(dB=8 * MB)) == ssm.SSM_ERR_ALIAS  # dy
    assert call(io(dC=13 * MB + 64)) == ssm.SSM_ERR_ALIAS  # dB
    assert call(io(workspace=12 * MB)) == ssm.SSM_ERR_ALIAS  # dA_log
    assert call(io(dh0=9 * MB)) == ssm.SSM_ERR_ALIAS  # chunk states
    # the chunk states read are [row, chunk] = [0..1, 0..3] up to (1, 2): 7 of the
    # 8 [dim, dstate] blocks (2048 bytes each), the last row's included
    assert call(io(dh0=9 * MB + 6 * 2048)) == ssm.SSM_ERR_ALIAS
    assert call(io(dh0=9 * MB + 7 * 2048 - 4)) == ssm.SSM_ERR_ALIAS
    assert call(io(dh0=9 * MB + 7 * 2048)) == ssm.SSM_ERR_INVALID_ARG  # past them: the NULL handle
    assert call(io(dD=11 * MB + 2)) == ssm.SSM_ERR_UNSUPPORTED  # misaligned
    assert ssm.ssm_selective_scan_bwd(None, *[None] * 7, d, None, io(), None) == ssm.SSM_ERR_INVALID_ARG
    assert ssm.ssm_selective_scan_bwd(None, *[None] * 7, _dims(dstate=8), None, io(), None) == \
        ssm.SSM_ERR_UNSUPPORTED


def test_empty_problem_needs_only_the_handle():
    assert call(_dims(batch=0), x=None, delta=None, B=None, C=None, y=None, A_log=None) == ssm.SSM_ERR_INVALID_ARG


def test_create_without_gpu_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(ssm.SsmScanError) as ei:
        ssm.ssm_scan_create(0)
    assert ei.value.code in (ssm.SSM_ERR_NO_DEVICE, ssm.SSM_ERR_HIP)
    lib = ssm.lib()
    assert lib.ssm_scan_create(None, 0) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_scan_destroy(None) == ssm.SSM_OK


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 16)
    with pytest.raises(ValueError):
        ssm.selective_scan_fwd(x, x, torch.zeros(16, 16), torch.zeros(1, 8, 16), torch.zeros(1, 8, 16))


def test_peaks_library_loads_and_checks_arguments():
    """The benchmark's peak-rate microbenchmark library is built beside the
    scan library and rejects bad arguments before touching the GPU."""
    from selective_state_space_scan_amd import build as B
    assert os.path.exists(B.PEAKS_LIB_PATH), "run __graft_entry__.build() first"
    lib = ctypes.CDLL(B.PEAKS_LIB_PATH)
    f = lib.ssm_peak_launch
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(2, None, None, 0, None, 0, 1, None) == -1     # no blocks
    assert f(2, None, None, 0, None, 16, -1, None) == -1   # negative iterations
    assert f(0, None, None, 16, None, 16, 0, None) == -1   # read without buffers
    assert f(1, 8, None, 16, None, 16, 0, None) == -1      # copy without destination
    assert f(7, None, None, 0, 8, 16, 0, None) == -1       # unknown benchmark


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the HIP library every entry point raises: there is no other
    path to fall back to."""
    from selective_state_space_scan_amd import _binding as B
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libssmscan.so"))
    with pytest.raises(ImportError, match="HIP library not built"):
        B.lib()
    for call_ in (lambda: B.chunk_len(16), lambda: B.bwd_chunk_len(16), lambda: B.error_string(0),
                  lambda: B.ssm_scan_create(0)):
        with pytest.raises(ImportError):
            call_()
