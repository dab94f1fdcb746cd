"""ctypes binding of the C ABI in ``include/ssm_scan.h`` (argument marshalling only).

Every step of the scan runs in the HIP library; this module checks tensor
shapes, dtypes and devices, allocates outputs with torch, and passes raw device
pointers and the current HIP stream across the ABI.  There is no fallback: if
the library is missing or no GPU is usable, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

SSM_OK = 0
SSM_ERR_INVALID_ARG = -1
SSM_ERR_UNSUPPORTED = -2
SSM_ERR_ALIAS = -3
SSM_ERR_HIP = -4
SSM_ERR_NO_DEVICE = -5
SSM_ERR_DEVICE_MISMATCH = -6
SSM_ERR_SCRATCH = -7

SSM_SCAN_NOALLOC_SCRATCH_BYTES = 16 << 20

SSM_IO_F32 = 0
SSM_IO_BF16 = 1

SSM_COMBINE_WALK = 0
SSM_COMBINE_WAVE_SCAN = 1

# Names declared in include/ssm_scan.h.
EXPORTED = ("ssm_scan_create", "ssm_selective_scan_fwd", "ssm_selective_scan_fwd_ex", "ssm_scan_chunk_len",
            "ssm_scan_auto_time_parts", "ssm_scan_workspace_bytes", "ssm_scan_bwd_chunk_len",
            "ssm_scan_bwd_workspace_bytes", "ssm_selective_scan_bwd", "ssm_scan_destroy", "ssm_scan_error_string",
            "ssm_selective_scan_fwd_noalloc")


class SsmScanError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {error_string(code)} ({code})")
        self.code = code


class ssm_scan_dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("delta_softplus", ctypes.c_int32),
        ("delta_clamp", ctypes.c_int32),
        ("delta_min", ctypes.c_float),
        ("delta_max", ctypes.c_float),
    ]


class ssm_scan_fwd_extras(ctypes.Structure):
    _fields_ = [
        ("h0", ctypes.c_void_p),
        ("delta_bias", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("chunk_states", ctypes.c_void_p),
        ("chunk_len", ctypes.c_int64),
        ("time_parts", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
        ("combine", ctypes.c_int32),
    ]


class ssm_scan_bwd_io(ctypes.Structure):
    _fields_ = [
        ("dy", ctypes.c_void_p),
        ("dh_last", ctypes.c_void_p),
        ("chunk_states", ctypes.c_void_p),
        ("dx", ctypes.c_void_p),
        ("ddelta", ctypes.c_void_p),
        ("dz", ctypes.c_void_p),
        ("dA_log", ctypes.c_void_p),
        ("dB", ctypes.c_void_p),
        ("dC", ctypes.c_void_p),
        ("dD", ctypes.c_void_p),
        ("ddelta_bias", ctypes.c_void_p),
        ("dh0", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
    ]


_lib = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return LIB_PATH


def lib() -> ctypes.CDLL:
    """Load ``libssmscan.so`` (built in-tree by ``build.build()``); raise if absent."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"HIP library not built: {LIB_PATH} is missing; run "
                "`python -m selective_state_space_scan_amd.build` (or __graft_entry__.build())")
        # torch ships its own HIP runtime under the same soname as the system
        # one the library links against; loading torch first makes the library
        # bind to that copy, so the process holds a single HIP runtime whatever
        # the import order of the caller.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.ssm_scan_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int]
        L.ssm_scan_create.restype = ctypes.c_int
        L.ssm_scan_destroy.argtypes = [vp]
        L.ssm_scan_destroy.restype = ctypes.c_int
        L.ssm_scan_error_string.argtypes = [ctypes.c_int]
        L.ssm_scan_error_string.restype = ctypes.c_char_p
        L.ssm_selective_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.POINTER(ssm_scan_dims), vp]
        L.ssm_selective_scan_fwd.restype = ctypes.c_int
        L.ssm_selective_scan_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.POINTER(ssm_scan_dims), ctypes.POINTER(ssm_scan_fwd_extras), vp]
        L.ssm_selective_scan_fwd_ex.restype = ctypes.c_int
        L.ssm_selective_scan_fwd_noalloc.argtypes = L.ssm_selective_scan_fwd_ex.argtypes
        L.ssm_selective_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_scan_chunk_len.argtypes = [ctypes.c_int64]
        L.ssm_scan_chunk_len.restype = ctypes.c_int64
        L.ssm_scan_auto_time_parts.argtypes = [vp, ctypes.POINTER(ssm_scan_dims)]
        L.ssm_scan_auto_time_parts.restype = ctypes.c_int32
        L.ssm_scan_workspace_bytes.argtypes = [ctypes.POINTER(ssm_scan_dims), ctypes.c_int32]
        L.ssm_scan_workspace_bytes.restype = ctypes.c_int64
        L.ssm_scan_bwd_chunk_len.argtypes = [ctypes.c_int64]
        L.ssm_scan_bwd_chunk_len.restype = ctypes.c_int64
        L.ssm_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(ssm_scan_dims)]
        L.ssm_scan_bwd_workspace_bytes.restype = ctypes.c_int64
        L.ssm_selective_scan_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(ssm_scan_dims),
                                             ctypes.POINTER(ssm_scan_fwd_extras), ctypes.POINTER(ssm_scan_bwd_io), vp]
        L.ssm_selective_scan_bwd.restype = ctypes.c_int
        _lib = L
        return L


def error_string(code: int) -> str:
    return lib().ssm_scan_error_string(int(code)).decode()


# ---- raw C ABI (pointers as ints) ------------------------------------------

def ssm_scan_create(device_ordinal: int) -> int:
    h = ctypes.c_void_p()
    rc = lib().ssm_scan_create(ctypes.byref(h), int(device_ordinal))
    if rc != SSM_OK:
        raise SsmScanError(rc, "ssm_scan_create")
    return h.value


def ssm_scan_destroy(handle: int | None) -> None:
    rc = lib().ssm_scan_destroy(handle)
    if rc != SSM_OK:
        raise SsmScanError(rc, "ssm_scan_destroy")


def ssm_selective_scan_fwd(handle, x, delta, A_log, B, C, D, valid_len, y, h_last, dims: ssm_scan_dims,
                           stream) -> int:
    """Calls the C entry point with raw pointers (ints or None); returns the status code."""
    return lib().ssm_selective_scan_fwd(handle, x, delta, A_log, B, C, D, valid_len, y, h_last,
                                        ctypes.byref(dims), stream)


def ssm_selective_scan_fwd_ex(handle, x, delta, A_log, B, C, D, valid_len, y, h_last, dims: ssm_scan_dims,
                              extras: ssm_scan_fwd_extras | None, stream) -> int:
    """The extended entry point (raw pointers); returns the status code."""
    return lib().ssm_selective_scan_fwd_ex(handle, x, delta, A_log, B, C, D, valid_len, y, h_last,
                                           ctypes.byref(dims), None if extras is None else ctypes.byref(extras),
                                           stream)


def ssm_selective_scan_fwd_noalloc(handle, x, delta, A_log, B, C, D, valid_len, y, h_last, dims: ssm_scan_dims,
                                   extras: ssm_scan_fwd_extras | None, stream) -> int:
    """The allocation-free entry point (raw pointers; the time split's carries
    in the library's static scratch); returns the status code."""
    return lib().ssm_selective_scan_fwd_noalloc(handle, x, delta, A_log, B, C, D, valid_len, y, h_last,
                                                ctypes.byref(dims), None if extras is None else ctypes.byref(extras),
                                                stream)


def chunk_len(dstate: int) -> int:
    """Steps per chunk of the chunk-boundary states for this state count."""
    return int(lib().ssm_scan_chunk_len(int(dstate)))


_default_chunk_len = chunk_len  # the parameter of selective_scan_fwd shadows the name


def bwd_chunk_len(dstate: int) -> int:
    """The chunk length the forward must save chunk states at for the backward."""
    return int(lib().ssm_scan_bwd_chunk_len(int(dstate)))


def bwd_workspace_bytes(dims: ssm_scan_dims) -> int:
    return int(lib().ssm_scan_bwd_workspace_bytes(ctypes.byref(dims)))


def ssm_selective_scan_bwd(handle, x, delta, A_log, B, C, D, valid_len, dims: ssm_scan_dims,
                           extras: ssm_scan_fwd_extras | None, io: ssm_scan_bwd_io, stream) -> int:
    """The backward entry point (raw pointers); returns the status code."""
    return lib().ssm_selective_scan_bwd(handle, x, delta, A_log, B, C, D, valid_len, ctypes.byref(dims),
                                        None if extras is None else ctypes.byref(extras), ctypes.byref(io), stream)


def auto_time_parts(handle, dims: ssm_scan_dims) -> int:
    """The time split the library picks for these dims on the handle's GPU."""
    return int(lib().ssm_scan_auto_time_parts(handle, ctypes.byref(dims)))


def workspace_bytes(dims: ssm_scan_dims, time_parts: int) -> int:
    """Device workspace bytes a split into (at most) time_parts parts needs."""
    return int(lib().ssm_scan_workspace_bytes(ctypes.byref(dims), int(time_parts)))


# ---- torch front end -----------------------------------------------------

_handles: dict[int, int] = {}
_handles_lock = threading.Lock()


def handle_for(device_index: int) -> int:
    with _handles_lock:
        h = _handles.get(device_index)
        if h is None:
            h = ssm_scan_create(device_index)
            _handles[device_index] = h
        return h


def _stream_for(stream, dev):
    """The stream to enqueue on as a torch stream object: the current stream of
    ``dev`` for None, a torch stream as given, and a raw hipStream_t handle
    wrapped as an external stream.  The tensors a call allocates are allocated
    with that stream current, so that the caching allocator orders their reuse
    after the call's kernels."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(dev)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=dev)


def selective_scan_fwd(x, delta, A_log, B, C, D=None, valid_len=None, *, delta_softplus: bool = True,
                       delta_clamp=None, y=None, h_last=None, return_h_last: bool = True, h0=None, delta_bias=None,
                       z=None, return_chunk_states: bool = False, chunk_len=None, time_parts=None, workspace=None,
                       combine: str = "walk", stream=None):
    """Selective-scan forward on the GPU.  Returns ``(y, h_last)``, or
    ``(y, h_last, chunk_states)`` with ``return_chunk_states``.

    x, delta: [batch, L, dim]; B, C: [batch, L, dstate]; all four the same dtype
    (torch.float32 or torch.bfloat16).  A_log: [dim, dstate] float32.  D: [dim]
    float32 or None.  valid_len: [batch] int32 or None.  delta_clamp: None or
    (min, max), applied after softplus.  Outputs are allocated unless given:
    y like x, h_last [batch, dim, dstate] float32 (None if return_h_last is
    False and no h_last is given).  The call is asynchronous on ``stream``
    (default: the current stream of x's device).

    Extras: h0 [batch, dim, dstate] float32 initial state (may be h_last
    itself); delta_bias [dim] float32 added to delta before softplus; z like x,
    output gate y * silu(z); chunk states [batch, ceil(L / chunk_len(dstate)),
    dim, dstate] float32, the state after every chunk (``chunk_len`` steps, a
    multiple of 4 dividing chunk_len(dstate); default chunk_len(dstate)).

    Time split: ``time_parts`` None lets the library choose (it splits only
    batches too small to fill the GPU), 1 never splits, P >= 2 asks for at most
    P parts.  ``workspace`` is an optional contiguous uint8 tensor on x's device
    used as scratch for a split; one is allocated when needed and not given.

    ``combine``: "walk" (default) joins a tile's sub-chunks by a serial carry
    walk, "wave_scan" by a log-depth scan across each wave's sub-chunks and a
    walk over the wave totals (the same result within rounding).
    """
    import torch

    if x.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    dev = x.device
    io = {torch.float32: SSM_IO_F32, torch.bfloat16: SSM_IO_BF16}.get(x.dtype)
    if io is None:
        raise TypeError("x must be float32 or bfloat16")
    if x.dim() != 3:
        raise ValueError("x must be [batch, L, dim]")
    nb, L, nd = x.shape
    if A_log.dim() != 2 or A_log.shape[0] != nd:
        raise ValueError("A_log must be [dim, dstate]")
    N = A_log.shape[1]
    for name, t, shape, dt in (("delta", delta, (nb, L, nd), x.dtype), ("B", B, (nb, L, N), x.dtype),
                               ("C", C, (nb, L, N), x.dtype), ("A_log", A_log, (nd, N), torch.float32)):
        if tuple(t.shape) != shape or t.dtype != dt or t.device != dev:
            raise ValueError(f"{name} must be {shape} {dt} on {dev}, got {tuple(t.shape)} {t.dtype} on {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if D is not None and (tuple(D.shape) != (nd,) or D.dtype != torch.float32 or D.device != dev
                          or not D.is_contiguous()):
        raise ValueError("D must be a contiguous [dim] float32 tensor on x's device")
    if valid_len is not None and (tuple(valid_len.shape) != (nb,) or valid_len.dtype != torch.int32
                                  or valid_len.device != dev or not valid_len.is_contiguous()):
        raise ValueError("valid_len must be a contiguous [batch] int32 tensor on x's device")
    if y is not None and (tuple(y.shape) != (nb, L, nd) or y.dtype != x.dtype or y.device != dev
                          or not y.is_contiguous()):
        raise ValueError("y must be a contiguous tensor like x")
    if h_last is not None and (tuple(h_last.shape) != (nb, nd, N) or h_last.dtype != torch.float32
                               or h_last.device != dev or not h_last.is_contiguous()):
        raise ValueError("h_last must be a contiguous [batch, dim, dstate] float32 tensor")

    for name, t, shape in (("h0", h0, (nb, nd, N)), ("delta_bias", delta_bias, (nd,))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or t.device != dev
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {shape} float32 tensor on x's device")
    if z is not None and (tuple(z.shape) != (nb, L, nd) or z.dtype != x.dtype or z.device != dev
                          or not z.is_contiguous()):
        raise ValueError("z must be a contiguous tensor like x")
    cl = _default_chunk_len(N) if chunk_len is None else int(chunk_len)
    if return_chunk_states and cl <= 0:
        raise ValueError(f"no chunk length for dstate {N} (unsupported) or chunk_len <= 0")
    stream = _stream_for(stream, dev)
    sptr = stream.cuda_stream
    chunk_states = None
    with torch.cuda.stream(stream):
        if y is None:
            y = torch.empty_like(x)
        if h_last is None and return_h_last:
            h_last = torch.empty((nb, nd, N), dtype=torch.float32, device=dev)
        if return_chunk_states:
            chunk_states = torch.empty((nb, (L + cl - 1) // cl, nd, N), dtype=torch.float32, device=dev)
    dims = ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate = nb, L, nd, N
    dims.io_dtype = io
    dims.delta_softplus = 1 if delta_softplus else 0
    if delta_clamp is not None:
        dims.delta_clamp = 1
        dims.delta_min, dims.delta_max = float(delta_clamp[0]), float(delta_clamp[1])

    def ptr(t):
        return None if t is None or t.numel() == 0 else t.data_ptr()

    with torch.cuda.device(dev):
        h = handle_for(dev.index if dev.index is not None else torch.cuda.current_device())
        parts = auto_time_parts(h, dims) if time_parts is None else int(time_parts)
        if parts < 1:
            raise ValueError("time_parts must be None or >= 1")
        ws_bytes = workspace_bytes(dims, parts) if parts >= 2 else 0
        if ws_bytes > 0:
            if workspace is None:
                with torch.cuda.stream(stream):
                    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            elif (workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous()
                  or workspace.numel() < ws_bytes):
                raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {ws_bytes} bytes on {dev}")
        comb = {"walk": SSM_COMBINE_WALK, "wave_scan": SSM_COMBINE_WAVE_SCAN}.get(combine)
        if comb is None:
            raise ValueError('combine must be "walk" or "wave_scan"')
        extras = None
        if (h0 is not None or delta_bias is not None or z is not None or chunk_states is not None
                or ws_bytes > 0 or time_parts is not None or comb != SSM_COMBINE_WALK):
            extras = ssm_scan_fwd_extras(ptr(h0), ptr(delta_bias), ptr(z), ptr(chunk_states),
                                         cl if chunk_states is not None else 0, parts,
                                         ptr(workspace) if ws_bytes > 0 else None, ws_bytes, comb)
        if extras is None:
            rc = ssm_selective_scan_fwd(h, ptr(x), ptr(delta), ptr(A_log), ptr(B), ptr(C), ptr(D), ptr(valid_len),
                                        ptr(y), ptr(h_last), dims, sptr)
        else:
            rc = ssm_selective_scan_fwd_ex(h, ptr(x), ptr(delta), ptr(A_log), ptr(B), ptr(C), ptr(D),
                                           ptr(valid_len), ptr(y), ptr(h_last), dims, extras, sptr)
    if rc != SSM_OK:
        raise SsmScanError(rc, "ssm_selective_scan_fwd")
    if return_chunk_states:
        return y, h_last, chunk_states
    return y, h_last


def selective_scan_bwd(x, delta, A_log, B, C, D, valid_len, dy, chunk_states, *, dh_last=None, h0=None,
                       delta_bias=None, z=None, delta_softplus: bool = True, delta_clamp=None, workspace=None,
                       stream=None) -> dict:
    """Gradients of ``selective_scan_fwd`` for the loss sum(dy * y) + sum(dh_last * h_last).

    The forward inputs and flags must be the ones of the forward call, and
    ``chunk_states`` that call's chunk states saved with
    ``chunk_len=bwd_chunk_len(dstate)`` (None is accepted when L fits one
    chunk).  Returns a dict: dx, ddelta (w.r.t. the raw delta) and dz (None
    without z) like x; dA_log [dim, dstate], dB, dC [batch, L, dstate], dD and
    ddelta_bias [dim] (None when D / delta_bias is None) and dh0 [batch, dim,
    dstate], all float32.  Asynchronous on ``stream``.
    """
    import torch

    if x.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    dev = x.device
    io = {torch.float32: SSM_IO_F32, torch.bfloat16: SSM_IO_BF16}.get(x.dtype)
    if io is None or x.dim() != 3:
        raise ValueError("x must be a [batch, L, dim] float32 or bfloat16 tensor")
    nb, L, nd = x.shape
    if A_log.dim() != 2 or A_log.shape[0] != nd:
        raise ValueError("A_log must be [dim, dstate]")
    N = A_log.shape[1]
    for name, t, shape, dt in (("delta", delta, (nb, L, nd), x.dtype), ("B", B, (nb, L, N), x.dtype),
                               ("C", C, (nb, L, N), x.dtype), ("A_log", A_log, (nd, N), torch.float32),
                               ("dy", dy, (nb, L, nd), x.dtype)):
        if tuple(t.shape) != shape or t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {shape} {dt} tensor on {dev}")
    cl = bwd_chunk_len(N)
    n_chunks = (L + cl - 1) // cl if cl > 0 else 0
    if chunk_states is not None and (tuple(chunk_states.shape) != (nb, n_chunks, nd, N)
                                     or chunk_states.dtype != torch.float32 or chunk_states.device != dev
                                     or not chunk_states.is_contiguous()):
        raise ValueError(f"chunk_states must be [batch, {n_chunks}, dim, dstate] float32 "
                         f"(the forward's, with chunk_len={cl})")
    for name, t, shape in (("dh_last", dh_last, (nb, nd, N)), ("h0", h0, (nb, nd, N)),
                           ("delta_bias", delta_bias, (nd,)), ("D", D, (nd,))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32 or t.device != dev
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {shape} float32 tensor on {dev}")
    if z is not None and (tuple(z.shape) != (nb, L, nd) or z.dtype != x.dtype or z.device != dev
                          or not z.is_contiguous()):
        raise ValueError("z must be a contiguous tensor like x")
    if valid_len is not None and (tuple(valid_len.shape) != (nb,) or valid_len.dtype != torch.int32
                                  or valid_len.device != dev or not valid_len.is_contiguous()):
        raise ValueError("valid_len must be a contiguous [batch] int32 tensor on x's device")
    stream = _stream_for(stream, dev)
    sptr = stream.cuda_stream
    with torch.cuda.stream(stream):
        out = dict(dx=torch.empty_like(x), ddelta=torch.empty_like(x),
                   dz=torch.empty_like(x) if z is not None else None,
                   dA_log=torch.empty((nd, N), dtype=torch.float32, device=dev),
                   dB=torch.empty((nb, L, N), dtype=torch.float32, device=dev),
                   dC=torch.empty((nb, L, N), dtype=torch.float32, device=dev),
                   dD=torch.empty(nd, dtype=torch.float32, device=dev) if D is not None else None,
                   ddelta_bias=torch.empty(nd, dtype=torch.float32, device=dev) if delta_bias is not None else None,
                   dh0=torch.empty((nb, nd, N), dtype=torch.float32, device=dev))
    dims = ssm_scan_dims()
    dims.batch, dims.seqlen, dims.dim, dims.dstate = nb, L, nd, N
    dims.io_dtype = io
    dims.delta_softplus = 1 if delta_softplus else 0
    if delta_clamp is not None:
        dims.delta_clamp = 1
        dims.delta_min, dims.delta_max = float(delta_clamp[0]), float(delta_clamp[1])

    def ptr(t):
        return None if t is None or t.numel() == 0 else t.data_ptr()

    nbytes = bwd_workspace_bytes(dims)
    if nbytes < 0:
        raise ValueError("unsupported dims for the backward")
    if workspace is None:
        with torch.cuda.stream(stream):
            workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
    elif (workspace.dtype != torch.uint8 or workspace.device != dev or workspace.numel() < nbytes
          or not workspace.is_contiguous()):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of at least {nbytes} bytes on {dev}")
    extras = ssm_scan_fwd_extras(ptr(h0), ptr(delta_bias), ptr(z), None, 0, 0, None, 0)
    bio = ssm_scan_bwd_io(ptr(dy), ptr(dh_last), ptr(chunk_states), ptr(out["dx"]), ptr(out["ddelta"]),
                          ptr(out["dz"]), ptr(out["dA_log"]), ptr(out["dB"]), ptr(out["dC"]), ptr(out["dD"]),
                          ptr(out["ddelta_bias"]), ptr(out["dh0"]), ptr(workspace), max(nbytes, 4))
    with torch.cuda.device(dev):
        h = handle_for(dev.index if dev.index is not None else torch.cuda.current_device())
        rc = ssm_selective_scan_bwd(h, ptr(x), ptr(delta), ptr(A_log), ptr(B), ptr(C), ptr(D), ptr(valid_len),
                                    dims, extras, bio, sptr)
    if rc != SSM_OK:
        raise SsmScanError(rc, "ssm_selective_scan_bwd")
    return out
