"""fp64 CPU oracle for the selective state-space scan forward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
``cpu_baseline`` leg are the only callers.  The oracle is a plain serial loop in
C (``ssm_oracle.c``) and shares no code with the HIP library.

What it computes, and the passages it follows, is stated in ``ssm_oracle.c``:
the diagonal selective recurrence h_t = exp(Delta_t*A) h_{t-1} + Delta_t B_t x_t
with y_t = C_t . h_t + D x_t (pwwt.cn article, sections 1.1 and 2.4), padding as
the identity (section 2.3) and a zero initial state (section 4.1).

Inputs may be any float dtype; they are converted to fp64 (exact for fp32, and
for bf16 values that arrive as fp32).  Outputs are fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_lock = threading.Lock()
_libs: dict[int, ctypes.CDLL] = {}


def lib_path(mutation: int = 0) -> str:
    name = "libssm_oracle.so" if mutation == 0 else f"libssm_oracle_mut{mutation}.so"
    return os.path.join(_BUILD_DIR, name)


def build(mutation: int = 0, force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math).  ``mutation`` > 0 plants
    one known mistake (for the tests that show the pins notice it)."""
    out = lib_path(mutation)
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(_SRC):
        return out
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", f"-DORACLE_MUTATION={mutation}",
           "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load(mutation: int = 0) -> ctypes.CDLL:
    with _lock:
        if mutation in _libs:
            return _libs[mutation]
        path = build(mutation)
        lib = ctypes.CDLL(path)
        d = ctypes.POINTER(ctypes.c_double)
        i32 = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.oracle_scan_ab.argtypes = [d, d, ctypes.c_double, i64, d]
        lib.oracle_scan_ab.restype = None
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        common = [d, d, d, d, d, d, i32, d, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                  ctypes.c_double, ctypes.c_double]
        lib.oracle_selective_scan.argtypes = common + [d, d, ctypes.c_int]
        lib.oracle_selective_scan.restype = ctypes.c_int
        lib.oracle_selective_scan_ex.argtypes = common + [d, d, d, i64, d, d, ctypes.c_int]
        lib.oracle_selective_scan_ex.restype = ctypes.c_int
        lib.oracle_selective_scan_rows.argtypes = common + [d, d, i64p, i64p, i64, d, d, ctypes.c_int]
        lib.oracle_selective_scan_rows.restype = ctypes.c_int
        lib.oracle_selective_scan_bwd.argtypes = common + [d, d, d, d] + [d] * 9 + [ctypes.c_int]
        lib.oracle_selective_scan_bwd.restype = ctypes.c_int
        lib.oracle_mutation_id.argtypes = []
        lib.oracle_mutation_id.restype = ctypes.c_int
        _libs[mutation] = lib
        return lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def scan_ab(a, b, h0: float = 0.0, mutation: int = 0) -> np.ndarray:
    """The bare affine recurrence h_t = a_t h_{t-1} + b_t (1-D inputs)."""
    a = _f64(a).reshape(-1)
    b = _f64(b).reshape(-1)
    if a.shape != b.shape:
        raise ValueError("a and b must have the same length")
    h = np.empty_like(a)
    _load(mutation).oracle_scan_ab(_ptr(a), _ptr(b), float(h0), a.shape[0], _ptr(h))
    return h


def softplus(v: float, mutation: int = 0) -> float:
    return _load(mutation).oracle_softplus(float(v))


def silu(v: float, mutation: int = 0) -> float:
    return _load(mutation).oracle_silu(float(v))


def _prep(x, delta, A_log, B, C, D, valid_len, h0):
    x = _f64(x)
    delta = _f64(delta)
    A_log = _f64(A_log)
    B = _f64(B)
    C = _f64(C)
    D = _f64(D)
    h0 = _f64(h0)
    if x.ndim != 3 or delta.shape != x.shape:
        raise ValueError("x and delta must be [B, L, D]")
    nb, L, nd = x.shape
    if A_log.ndim != 2 or A_log.shape[0] != nd:
        raise ValueError("A_log must be [D, N]")
    N = A_log.shape[1]
    if B.shape != (nb, L, N) or C.shape != (nb, L, N):
        raise ValueError("B and C must be [B, L, N]")
    if D is not None and D.shape != (nd,):
        raise ValueError("D must be [D]")
    if h0 is not None and h0.shape != (nb, nd, N):
        raise ValueError("h0 must be [B, D, N]")
    vl = None
    if valid_len is not None:
        vl = np.ascontiguousarray(np.asarray(valid_len, dtype=np.int32).reshape(-1))
        if vl.shape != (nb,):
            raise ValueError("valid_len must be [B]")
    return x, delta, A_log, B, C, D, vl, h0, nb, L, nd, N


def _extras(delta_bias, z, nb, L, nd):
    delta_bias = _f64(delta_bias)
    z = _f64(z)
    if delta_bias is not None and delta_bias.shape != (nd,):
        raise ValueError("delta_bias must be [D]")
    if z is not None and z.shape != (nb, L, nd):
        raise ValueError("z must be [B, L, D]")
    return delta_bias, z


def selective_scan(x, delta, A_log, B, C, D=None, valid_len=None, h0=None, delta_softplus: bool = True,
                   delta_clamp=None, delta_bias=None, z=None, chunk_len=None, nthreads: int = 1, mutation: int = 0):
    """Full forward.  Returns (y [B,L,D], h_last [B,D,N]) in fp64, and with
    ``chunk_len`` also the chunk-boundary states [B, ceil(L/chunk_len), D, N]."""
    x, delta, A_log, B, C, D, vl, h0, nb, L, nd, N = _prep(x, delta, A_log, B, C, D, valid_len, h0)
    delta_bias, z = _extras(delta_bias, z, nb, L, nd)
    clamp = delta_clamp is not None
    dmin, dmax = (float(delta_clamp[0]), float(delta_clamp[1])) if clamp else (0.0, 0.0)
    y = np.empty((nb, L, nd), dtype=np.float64)
    h_last = np.empty((nb, nd, N), dtype=np.float64)
    cs = None
    if chunk_len is not None:
        cs = np.empty((nb, (L + chunk_len - 1) // chunk_len, nd, N), dtype=np.float64)
    rc = _load(mutation).oracle_selective_scan_ex(
        _ptr(x), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(vl, ctypes.c_int32), _ptr(h0),
        nb, L, nd, N, int(bool(delta_softplus)), int(clamp), dmin, dmax, _ptr(delta_bias), _ptr(z), _ptr(cs),
        int(chunk_len or 1), _ptr(y), _ptr(h_last), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan failed ({rc})")
    if chunk_len is not None:
        return y, h_last, cs
    return y, h_last


def selective_scan_rows(x, delta, A_log, B, C, rows, D=None, valid_len=None, h0=None,
                        delta_softplus: bool = True, delta_clamp=None, delta_bias=None, z=None, nthreads: int = 1,
                        mutation: int = 0):
    """Forward for the listed (b, d) rows only.  Returns (y_rows [R, L], h_rows [R, N])."""
    x, delta, A_log, B, C, D, vl, h0, nb, L, nd, N = _prep(x, delta, A_log, B, C, D, valid_len, h0)
    delta_bias, z = _extras(delta_bias, z, nb, L, nd)
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    rb = np.ascontiguousarray(rows[:, 0])
    rd = np.ascontiguousarray(rows[:, 1])
    clamp = delta_clamp is not None
    dmin, dmax = (float(delta_clamp[0]), float(delta_clamp[1])) if clamp else (0.0, 0.0)
    R = rows.shape[0]
    y = np.empty((R, L), dtype=np.float64)
    h = np.empty((R, N), dtype=np.float64)
    rc = _load(mutation).oracle_selective_scan_rows(
        _ptr(x), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(vl, ctypes.c_int32), _ptr(h0),
        nb, L, nd, N, int(bool(delta_softplus)), int(clamp), dmin, dmax, _ptr(delta_bias), _ptr(z),
        _ptr(rb, ctypes.c_int64),
        _ptr(rd, ctypes.c_int64), R, _ptr(y), _ptr(h), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan_rows failed ({rc})")
    return y, h


def selective_scan_bwd(x, delta, A_log, B, C, D=None, dy=None, valid_len=None, h0=None, delta_softplus: bool = True,
                       delta_clamp=None, delta_bias=None, z=None, dh_last=None, nthreads: int = 1,
                       mutation: int = 0) -> dict:
    """Gradients of the forward for the loss sum(dy * y) + sum(dh_last * h_last)
    (reverse-mode differentiation of the serial loop; see ssm_oracle.c).
    Returns a dict of fp64 arrays: dx, ddelta (w.r.t. the raw delta), dA_log,
    dB, dC, dD, ddelta_bias, dz (None without z), dh0."""
    x, delta, A_log, B, C, D, vl, h0, nb, L, nd, N = _prep(x, delta, A_log, B, C, D, valid_len, h0)
    delta_bias, z = _extras(delta_bias, z, nb, L, nd)
    dy = _f64(dy)
    if dy is None or dy.shape != (nb, L, nd):
        raise ValueError("dy must be [B, L, D]")
    dh_last = _f64(dh_last)
    if dh_last is not None and dh_last.shape != (nb, nd, N):
        raise ValueError("dh_last must be [B, D, N]")
    clamp = delta_clamp is not None
    dmin, dmax = (float(delta_clamp[0]), float(delta_clamp[1])) if clamp else (0.0, 0.0)
    out = dict(dx=np.empty((nb, L, nd)), ddelta=np.empty((nb, L, nd)), dA_log=np.empty((nd, N)),
               dB=np.empty((nb, L, N)), dC=np.empty((nb, L, N)), dD=np.empty(nd), ddelta_bias=np.empty(nd),
               dz=np.empty((nb, L, nd)) if z is not None else None, dh0=np.empty((nb, nd, N)))
    rc = _load(mutation).oracle_selective_scan_bwd(
        _ptr(x), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(vl, ctypes.c_int32), _ptr(h0),
        nb, L, nd, N, int(bool(delta_softplus)), int(clamp), dmin, dmax, _ptr(delta_bias), _ptr(z), _ptr(dy),
        _ptr(dh_last), _ptr(out["dx"]), _ptr(out["ddelta"]), _ptr(out["dA_log"]), _ptr(out["dB"]), _ptr(out["dC"]),
        _ptr(out["dD"]), _ptr(out["ddelta_bias"]), _ptr(out["dz"]), _ptr(out["dh0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan_bwd failed ({rc})")
    if D is None:
        out["dD"] = None
    return out
