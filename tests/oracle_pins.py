"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes the oracle module and a mutation id (0 = the real
oracle; >0 = a build with one planted mistake) and raises AssertionError when
the oracle disagrees with the pinned fact.  None of them re-types the oracle's
loop: the expectations come from a printed worked example, exact rational
arithmetic, closed forms, invariants or a library routine (numpy.convolve).
"""
from __future__ import annotations

import itertools
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_closed_form():
    rows = []
    with open(os.path.join(GOLDEN, "closed_form_a05_b1_L8.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t, h = line.split()
            rows.append((int(t), float(h)))
    return rows


# ---- P1: the a = 0.5, b = 1, length-8 worked example -----------------------

def pin_closed_form_scan(orc, mutation=0):
    """pwwt.cn section 2.3 note: a = 0.5, b = 1, L = 8, hand-computed values."""
    rows = load_closed_form()
    h = orc.scan_ab(np.full(8, 0.5), np.ones(8), 0.0, mutation=mutation)
    expect = np.array([v for _, v in rows])
    assert np.array_equal(h, expect), (h, expect)


def pin_closed_form_full_path(orc, mutation=0):
    """The same example through the full method: delta = 1 (no softplus),
    A = -ln 2 so Abar = 1/2, B = x = C = 1, no skip term: y_t = h_t."""
    rows = load_closed_form()
    L = 8
    one = np.ones((1, L, 1))
    A_log = np.array([[math.log(math.log(2.0))]])
    y, h_last = orc.selective_scan(one, one, A_log, one, one, D=None, delta_softplus=False, mutation=mutation)
    expect = np.array([v for _, v in rows])
    assert np.max(np.abs(y[0, :, 0] - expect)) < 1e-14, y[0, :, 0]
    assert abs(h_last[0, 0, 0] - expect[-1]) < 1e-14


# ---- P2: order sensitivity of the combine ---------------------------------

def _exact_scan(a, b, h0=Fraction(0)):
    """h_t = a_t h_{t-1} + b_t in exact rational arithmetic."""
    h = Fraction(h0)
    out = []
    for ai, bi in zip(a, b):
        h = Fraction(ai) * h + Fraction(bi)
        out.append(h)
    return out


def pin_order_sensitivity(orc, mutation=0):
    """pwwt.cn section 2.1: the combine is order sensitive.  A constant
    sequence cannot show a swap, so use a = (1/2, 1/4), b = (1, 2): h_2 = 2.25
    (absorbing the input before the decay would give 0.5*... and 2.0-style
    values instead)."""
    h = orc.scan_ab(np.array([0.5, 0.25]), np.array([1.0, 2.0]), 0.0, mutation=mutation)
    assert np.array_equal(h, np.array([1.0, 2.25])), h
    # a cycling through {1, 1/2, 1/4} with small integer b: exact in fp64 at this length
    a = [Fraction(1), Fraction(1, 2), Fraction(1, 4)] * 4
    b = [3, -1, 2, 5, 0, -4, 1, 1, 2, -3, 7, 1]
    ex = [float(v) for v in _exact_scan(a, b)]
    got = orc.scan_ab(np.array([float(v) for v in a]), np.array(b, dtype=float), 0.0, mutation=mutation)
    assert np.array_equal(got, np.array(ex)), (got, ex)


# ---- P3: brute-force unrolled sums ----------------------------------------

def pin_bruteforce_scan(orc, mutation=0):
    """h_t = sum_{s<=t} (prod_{r=s+1..t} a_r) b_s (the unrolled recurrence),
    evaluated by brute force; exact for dyadic inputs, 1e-13 for real ones."""
    rng = np.random.default_rng(7)
    for L in (1, 2, 5, 12):
        a = [Fraction(int(k), 8) for k in rng.integers(0, 9, size=L)]
        b = [Fraction(int(k), 8) for k in rng.integers(-16, 17, size=L)]
        brute = []
        for t in range(L):
            acc = Fraction(0)
            for s in range(t + 1):
                p = Fraction(1)
                for rr in range(s + 1, t + 1):
                    p *= a[rr]
                acc += p * b[s]
            brute.append(float(acc))
        got = orc.scan_ab(np.array([float(v) for v in a]), np.array([float(v) for v in b]), 0.0, mutation=mutation)
        assert np.array_equal(got, np.array(brute)), (L, got, brute)
    L = 64
    a = rng.uniform(0.0, 1.0, size=L)
    b = rng.standard_normal(L)
    logs = np.concatenate([[0.0], np.cumsum(np.log(a))])
    brute = np.array([sum(math.exp(logs[t + 1] - logs[s + 1]) * b[s] for s in range(t + 1)) for t in range(L)])
    got = orc.scan_ab(a, b, 0.0, mutation=mutation)
    assert np.max(np.abs(got - brute) / np.maximum(np.abs(brute), 1.0)) < 1e-13


# ---- P4: associativity ----------------------------------------------------

def _combine(p, q):
    """(a1, b1) then (a2, b2) = (a1*a2, a2*b1 + b2) (pwwt.cn section 2.1)."""
    return (p[0] * q[0], q[0] * p[1] + q[1])


def _bracketings(items):
    if len(items) == 1:
        yield items[0]
        return
    for k in range(1, len(items)):
        for left in _bracketings(items[:k]):
            for right in _bracketings(items[k:]):
                yield _combine(left, right)


def pin_associativity(orc, mutation=0):
    """pwwt.cn section 2.1: composition of the affine steps is associative, so
    every bracketing of the pairs gives the serial result (bitwise for dyadic
    pairs; the final b component is h_L from h_0 = 0)."""
    rng = np.random.default_rng(11)
    for L in (2, 3, 5, 7):
        a = [float(k) / 4 for k in rng.integers(0, 5, size=L)]
        b = [float(k) / 4 for k in rng.integers(-8, 9, size=L)]
        h = orc.scan_ab(np.array(a), np.array(b), 0.0, mutation=mutation)
        pairs = list(zip(a, b))
        n = 0
        for agg in _bracketings(pairs):
            n += 1
            assert agg[1] == h[-1], (L, agg, h[-1])
        assert n == math.comb(2 * (L - 1), L - 1) // L


# ---- P5: identity element and padding --------------------------------------

def _rand_problem(rng, nb, L, nd, N, bias=-4.0):
    x = rng.standard_normal((nb, L, nd))
    delta = 0.5 * rng.standard_normal((nb, L, nd)) + bias
    A_log = np.log(np.arange(1, N + 1, dtype=float))[None, :].repeat(nd, 0) + 0.1 * rng.standard_normal((nd, N))
    B = rng.standard_normal((nb, L, N))
    C = rng.standard_normal((nb, L, N))
    D = rng.standard_normal(nd)
    return x, delta, A_log, B, C, D


def pin_identity_and_padding(orc, mutation=0):
    """pwwt.cn section 2.3 (padding as the identity (1, 0)) and section 5.2
    (a padded batch must match single-sequence inference)."""
    # (1, 0) is a two-sided identity of the recurrence
    rng = np.random.default_rng(5)
    a = rng.uniform(0, 1, 6)
    b = rng.standard_normal(6)
    base = orc.scan_ab(a, b, 0.0, mutation=mutation)
    padded = orc.scan_ab(np.concatenate([a, np.ones(3)]), np.concatenate([b, np.zeros(3)]), 0.0, mutation=mutation)
    assert np.array_equal(padded[:6], base) and np.all(padded[6:] == base[-1])

    nb, L, nd, N = 3, 40, 16, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    vl = np.array([40, 17, 0], dtype=np.int32)
    # garbage in the padding must not matter
    xg, dg, Bg, Cg = x.copy(), delta.copy(), B.copy(), C.copy()
    for bi, l in enumerate(vl):
        xg[bi, l:] = np.nan
        dg[bi, l:] = np.inf
        Bg[bi, l:] = np.nan
        Cg[bi, l:] = -np.inf
    y, h = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=vl, mutation=mutation)
    yg, hg = orc.selective_scan(xg, dg, A_log, Bg, Cg, D, valid_len=vl, mutation=mutation)
    assert np.array_equal(y, yg) and np.array_equal(h, hg)
    for bi, l in enumerate(vl):
        if l > 0:
            y1, h1 = orc.selective_scan(x[bi:bi + 1, :l], delta[bi:bi + 1, :l], A_log, B[bi:bi + 1, :l],
                                        C[bi:bi + 1, :l], D, mutation=mutation)
            assert np.array_equal(y[bi, :l], y1[0]), bi
            assert np.array_equal(h[bi], h1[0]), bi
        else:
            assert np.all(h[bi] == 0.0)
        tail = y[bi, l:]
        assert np.all(tail == 0.0) and not np.any(np.signbit(tail)), "padded y must be +0.0"
    # out-of-range lengths clamp into [0, L]
    y2, h2 = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=np.array([L + 5, L, L], np.int32),
                                mutation=mutation)
    y3, h3 = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=None, mutation=mutation)
    assert np.array_equal(y2, y3) and np.array_equal(h2, h3)
    y4, h4 = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=np.array([-3, 0, 0], np.int32),
                                mutation=mutation)
    assert np.all(y4 == 0.0) and np.all(h4 == 0.0)


# ---- P6: degenerate cases ----------------------------------------------------

def pin_degenerate(orc, mutation=0):
    """a = 1: h = cumsum(b); b = 0: h = 0; a = 0: h = b; B = 0 or C = 0: y = D*x."""
    rng = np.random.default_rng(3)
    b = rng.integers(-50, 50, size=30).astype(float)
    assert np.array_equal(orc.scan_ab(np.ones(30), b, 0.0, mutation=mutation), np.cumsum(b))
    assert np.array_equal(orc.scan_ab(rng.uniform(0, 1, 30), np.zeros(30), 0.0, mutation=mutation), np.zeros(30))
    assert np.array_equal(orc.scan_ab(np.zeros(30), b, 0.0, mutation=mutation), b)
    nb, L, nd, N = 2, 24, 8, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    y, h = orc.selective_scan(x, delta, A_log, np.zeros_like(B), C, D, mutation=mutation)
    assert np.array_equal(y, D[None, None, :] * x) and np.all(h == 0.0)
    yc, hc = orc.selective_scan(x, delta, A_log, B, np.zeros_like(C), D, mutation=mutation)
    _, href = orc.selective_scan(x, delta, A_log, B, C, D, mutation=mutation)
    assert np.array_equal(yc, D[None, None, :] * x) and np.array_equal(hc, href)


# ---- P7: the time-invariant case is a causal convolution --------------------

def pin_lti_convolution(orc, mutation=0):
    """pwwt.cn section 1.2: with delta, B and C constant over time the SSM is a
    causal convolution of x with K_j = sum_n C_n Abar_n^j delta B_n,
    Abar_n = exp(delta A_n) (checked with numpy.convolve)."""
    rng = np.random.default_rng(13)
    nb, L, nd, N = 2, 64, 8, 4
    x = rng.standard_normal((nb, L, nd))
    draw = 0.5 * rng.standard_normal(nd) - 2.0
    delta = np.broadcast_to(draw[None, None, :], (nb, L, nd)).copy()
    A_log = np.log(np.arange(1, N + 1, dtype=float))[None, :].repeat(nd, 0) + 0.2 * rng.standard_normal((nd, N))
    Bc = rng.standard_normal((nb, N))
    Cc = rng.standard_normal((nb, N))
    B = np.broadcast_to(Bc[:, None, :], (nb, L, N)).copy()
    C = np.broadcast_to(Cc[:, None, :], (nb, L, N)).copy()
    y, _ = orc.selective_scan(x, delta, A_log, B, C, None, mutation=mutation)
    sp = np.log1p(np.exp(draw))  # softplus of a moderate value
    A = -np.exp(A_log)
    j = np.arange(L)
    for bi in range(nb):
        for d in range(nd):
            abar = np.exp(sp[d] * A[d])
            K = np.sum(Cc[bi][None, :] * abar[None, :] ** j[:, None] * sp[d] * Bc[bi][None, :], axis=1)
            ref = np.convolve(x[bi, :, d], K)[:L]
            err = np.max(np.abs(y[bi, :, d] - ref)) / max(np.max(np.abs(ref)), 1e-30)
            assert err < 1e-12, (bi, d, err)


# ---- P8: softplus ------------------------------------------------------------

def pin_softplus(orc, mutation=0):
    """softplus(v) = log(1 + e^v): softplus(0) = ln 2, ~v for large v, ~e^v for
    very negative v (the series e^v - e^2v/2 + e^3v/3 there).  Read through the full path: one step, Abar = 1
    (A_log = -1000 so A = -0), B = x = C = 1, no skip term, so y_0 = delta."""
    cases = [(0.0, math.log(2.0)), (30.0, 30.0 + math.exp(-30.0)), (-30.0, math.exp(-30.0) - math.exp(-60.0) / 2 + math.exp(-90.0) / 3),
             (100.0, 100.0), (-5.0, math.log1p(math.exp(-5.0)))]
    for v, expect in cases:
        assert abs(orc.softplus(v, mutation=mutation) - expect) <= 1e-15 * abs(expect)
        one = np.ones((1, 1, 1))
        y, _ = orc.selective_scan(one, np.full((1, 1, 1), v), np.array([[-1000.0]]), one, one, None,
                                  mutation=mutation)
        assert abs(y[0, 0, 0] - expect) <= 2e-15 * abs(expect), (v, y[0, 0, 0], expect)


# ---- P9: splitting the sequence and carrying the state -----------------------

def pin_split_invariance(orc, mutation=0):
    """bjdmk.com.cn section 4.2 / pwwt.cn section 4.2: running [0, T) and then
    [T, L) from the carried state equals one run over [0, L), bitwise."""
    rng = np.random.default_rng(17)
    nb, L, nd, N, T = 2, 50, 8, 4, 19
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    y, h = orc.selective_scan(x, delta, A_log, B, C, D, mutation=mutation)
    y1, h1 = orc.selective_scan(x[:, :T], delta[:, :T], A_log, B[:, :T], C[:, :T], D, mutation=mutation)
    y2, h2 = orc.selective_scan(x[:, T:], delta[:, T:], A_log, B[:, T:], C[:, T:], D, h0=h1, mutation=mutation)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y) and np.array_equal(h2, h)


# ---- full method against its unrolled closed form -----------------------------

def pin_bruteforce_full(orc, mutation=0):
    """y_t = sum_n C_tn sum_{s<=t} exp(A_n * sum_{r=s+1..t} delta_r) delta_s B_sn x_s
    + D x_t (the unrolled form, with the exponent of a sum instead of a product
    of exponentials), brute force on tiny random inputs, with and without the
    delta clip."""
    rng = np.random.default_rng(19)
    nb, L, nd, N = 2, 9, 3, 3
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N, bias=-1.0)
    for clamp in (None, (0.05, 0.4)):
        y, h = orc.selective_scan(x, delta, A_log, B, C, D, delta_clamp=clamp, mutation=mutation)
        sp = np.logaddexp(0.0, delta)
        if clamp is not None:
            sp = np.clip(sp, clamp[0], clamp[1])
        A = -np.exp(A_log)
        for bi, d in itertools.product(range(nb), range(nd)):
            for t in range(L):
                acc = 0.0
                hs = np.zeros(N)
                for s in range(t + 1):
                    decay = np.exp(A[d] * np.sum(sp[bi, s + 1:t + 1, d]))
                    hs += decay * sp[bi, s, d] * B[bi, s] * x[bi, s, d]
                acc = float(np.dot(C[bi, t], hs)) + D[d] * x[bi, t, d]
                assert abs(y[bi, t, d] - acc) <= 1e-12 * max(1.0, abs(acc)), (bi, t, d, y[bi, t, d], acc)
            assert np.max(np.abs(h[bi, d] - hs)) <= 1e-12 * max(1.0, np.max(np.abs(hs)))


# ---- extras: delta bias, output gate, chunk-boundary states ----------------

def pin_delta_bias(orc, mutation=0):
    """The per-channel bias is added to the raw delta before softplus: a biased
    run equals an unbiased run on delta + bias (bitwise: the same fp64 sum)."""
    rng = np.random.default_rng(23)
    nb, L, nd, N = 2, 20, 8, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    bias = rng.standard_normal(nd)
    y1, h1 = orc.selective_scan(x, delta, A_log, B, C, D, delta_bias=bias, mutation=mutation)
    y2, h2 = orc.selective_scan(x, delta + bias[None, None, :], A_log, B, C, D, mutation=mutation)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def pin_output_gate(orc, mutation=0):
    """y <- y * silu(z) with silu(v) = v / (1 + e^-v), applied to the whole
    readout C.h + D x (nxbn.cn section 3's kernel body ends with the gate): the
    gated output is the ungated one times silu(z), z = 0 gives +-0, and the
    state is untouched."""
    rng = np.random.default_rng(29)
    nb, L, nd, N = 2, 20, 8, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    z = rng.standard_normal((nb, L, nd)) * 3.0
    z[0, 3, :] = 0.0
    yg, hg = orc.selective_scan(x, delta, A_log, B, C, D, z=z, mutation=mutation)
    y, h = orc.selective_scan(x, delta, A_log, B, C, D, mutation=mutation)
    silu = z / (1.0 + np.exp(-z))
    assert np.max(np.abs(yg - y * silu) / np.maximum(np.abs(y * silu), 1e-300)) < 1e-14
    assert np.all(yg[0, 3, :] == 0.0) and np.array_equal(h, hg)
    assert orc.silu(0.0, mutation=mutation) == 0.0
    assert abs(orc.silu(40.0, mutation=mutation) - 40.0) < 1e-12


def pin_chunk_states(orc, mutation=0):
    """The state after each chunk equals the final state of the same run cut
    at the chunk's end (also with padded rows: past the valid length the state
    no longer changes)."""
    rng = np.random.default_rng(31)
    nb, L, nd, N, cl = 3, 23, 8, 4, 5
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    vl = np.array([23, 12, 0], dtype=np.int32)
    y, h, cs = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=vl, chunk_len=cl, mutation=mutation)
    assert cs.shape == (nb, 5, nd, N)
    for k in range(cs.shape[1]):
        end = min((k + 1) * cl, L)
        _, hk = orc.selective_scan(x[:, :end], delta[:, :end], A_log, B[:, :end], C[:, :end], D,
                                   valid_len=np.minimum(vl, end), mutation=mutation)
        assert np.array_equal(cs[:, k], hk), k
    assert np.array_equal(cs[:, -1], h)


# ---- backward -------------------------------------------------------------

def _loss(orc, mutation, x, delta, A_log, B, C, D, vl, h0, bias, z, dy, dhl, clamp=None):
    y, h = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=vl, h0=h0, delta_bias=bias, z=z,
                              delta_clamp=clamp, mutation=mutation)
    return float(np.sum(dy * y) + np.sum(dhl * h))


def _bwd_problem(seed, clamp=False):
    rng = np.random.default_rng(seed)
    nb, L, nd, N = 2, 7, 3, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N, bias=-1.0)
    vl = np.array([L, 4], dtype=np.int32)
    h0 = rng.standard_normal((nb, nd, N))
    bias = 0.3 * rng.standard_normal(nd)
    z = 1.5 * rng.standard_normal((nb, L, nd))
    dy = rng.standard_normal((nb, L, nd))
    dhl = rng.standard_normal((nb, nd, N))
    if clamp:
        # softplus values well inside or well outside [0.25, 0.6]: no kink within the difference step
        sp = np.log1p(np.exp(delta + bias[None, None, :]))
        near = (np.abs(sp - 0.25) < 0.02) | (np.abs(sp - 0.6) < 0.02)
        delta = np.where(near, delta + 0.1, delta)
    return x, delta, A_log, B, C, D, vl, h0, bias, z, dy, dhl


def pin_bwd_finite_differences(orc, mutation=0):
    """Every gradient of the backward against central differences of the
    forward's loss sum(dy*y) + sum(dh_last*h_last), element by element, with
    padding, initial state, delta bias, gate, and (second case) the clip."""
    for seed, clamp in ((41, None), (43, (0.25, 0.6))):
        x, delta, A_log, B, C, D, vl, h0, bias, z, dy, dhl = _bwd_problem(seed, clamp is not None)
        g = orc.selective_scan_bwd(x, delta, A_log, B, C, D, dy, valid_len=vl, h0=h0, delta_bias=bias, z=z,
                                   dh_last=dhl, delta_clamp=clamp, mutation=mutation)
        args = dict(x=x, delta=delta, A_log=A_log, B=B, C=C, D=D, h0=h0, bias=bias, z=z)
        names = dict(x="dx", delta="ddelta", A_log="dA_log", B="dB", C="dC", D="dD", h0="dh0", bias="ddelta_bias",
                     z="dz")
        eps = 1e-6
        for k, arr in args.items():
            fd = np.empty_like(arr)
            for idx in np.ndindex(arr.shape):
                plus, minus = arr.copy(), arr.copy()
                plus[idx] += eps
                minus[idx] -= eps
                ap, am = dict(args, **{k: plus}), dict(args, **{k: minus})
                lp = _loss(orc, mutation, ap["x"], ap["delta"], ap["A_log"], ap["B"], ap["C"], ap["D"], vl, ap["h0"],
                           ap["bias"], ap["z"], dy, dhl, clamp)
                lm = _loss(orc, mutation, am["x"], am["delta"], am["A_log"], am["B"], am["C"], am["D"], vl, am["h0"],
                           am["bias"], am["z"], dy, dhl, clamp)
                fd[idx] = (lp - lm) / (2 * eps)
            got = g[names[k]]
            scale = max(1.0, float(np.max(np.abs(fd))))
            assert np.max(np.abs(got - fd)) <= 1e-6 * scale, (k, clamp, np.max(np.abs(got - fd)))


def pin_bwd_linearity(orc, mutation=0):
    """Exact identities of the linear parts (Euler's theorem for linear maps):
    with delta, A, B, C, D fixed, y and h_last are linear in (x, h0) jointly, so
    <dy, y> + <dh_last, h_last> = <dx, x> + <dh0, h0>; y - D x is linear in C,
    so <dy, y - D x> = <dC, C>; from a zero state it is linear in B too, so
    <dy, y - D x> = <dB, B>; and <dy, D x> = <dD, D>."""
    rng = np.random.default_rng(47)
    nb, L, nd, N = 2, 9, 3, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N, bias=-1.0)
    h0 = rng.standard_normal((nb, nd, N))
    dy = rng.standard_normal((nb, L, nd))
    dhl = rng.standard_normal((nb, nd, N))
    y, h = orc.selective_scan(x, delta, A_log, B, C, D, h0=h0, mutation=mutation)
    g = orc.selective_scan_bwd(x, delta, A_log, B, C, D, dy, h0=h0, dh_last=dhl, mutation=mutation)
    lhs = np.sum(dy * y) + np.sum(dhl * h)
    assert abs(lhs - (np.sum(g["dx"] * x) + np.sum(g["dh0"] * h0))) <= 1e-12 * max(1.0, abs(lhs))
    ydx = y - D[None, None, :] * x
    assert abs(np.sum(dy * ydx) - np.sum(g["dC"] * C)) <= 1e-12 * max(1.0, abs(np.sum(dy * ydx)))
    assert abs(np.sum(dy * D[None, None, :] * x) - np.sum(g["dD"] * D)) <= 1e-12 * max(1.0, float(np.sum(np.abs(D))))
    y0, _ = orc.selective_scan(x, delta, A_log, B, C, D, mutation=mutation)
    g0 = orc.selective_scan_bwd(x, delta, A_log, B, C, D, dy, mutation=mutation)
    y0dx = y0 - D[None, None, :] * x
    assert abs(np.sum(dy * y0dx) - np.sum(g0["dB"] * B)) <= 1e-12 * max(1.0, abs(np.sum(dy * y0dx)))


def pin_bwd_padding(orc, mutation=0):
    """pwwt.cn section 2.3 in reverse: padded steps get zero gradients, garbage
    in the padding changes nothing, and a padded row's gradients equal those of
    the row run alone with its own length."""
    rng = np.random.default_rng(53)
    nb, L, nd, N = 3, 8, 2, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N, bias=-1.0)
    vl = np.array([8, 5, 0], dtype=np.int32)
    dy = rng.standard_normal((nb, L, nd))
    dhl = rng.standard_normal((nb, nd, N))
    g = orc.selective_scan_bwd(x, delta, A_log, B, C, D, dy, valid_len=vl, dh_last=dhl, mutation=mutation)
    for k in ("dx", "ddelta"):
        assert np.all(g[k][1, 5:] == 0.0) and np.all(g[k][2] == 0.0)
    assert np.all(g["dB"][1, 5:] == 0.0) and np.all(g["dC"][2] == 0.0)
    assert np.array_equal(g["dh0"][2], dhl[2])  # nothing happens to an empty row's state
    xg, dg, Bg, Cg = x.copy(), delta.copy(), B.copy(), C.copy()
    xg[1, 5:] = np.nan
    dg[1, 5:] = np.inf
    Bg[2] = np.nan
    Cg[1, 5:] = -np.inf
    g2 = orc.selective_scan_bwd(xg, dg, A_log, Bg, Cg, D, dy, valid_len=vl, dh_last=dhl, mutation=mutation)
    for k in g:
        if g[k] is not None:
            assert np.array_equal(g[k], g2[k]), k
    g1 = orc.selective_scan_bwd(x[1:2, :5], delta[1:2, :5], A_log, B[1:2, :5], C[1:2, :5], D, dy[1:2, :5],
                                dh_last=dhl[1:2], mutation=mutation)
    for k in ("dx", "ddelta", "dB", "dC"):
        assert np.array_equal(g1[k][0], g[k][1, :5]), k
    assert np.array_equal(g1["dh0"][0], g["dh0"][1])


ALL_PINS = {
    "closed_form_scan": pin_closed_form_scan,
    "closed_form_full_path": pin_closed_form_full_path,
    "order_sensitivity": pin_order_sensitivity,
    "bruteforce_scan": pin_bruteforce_scan,
    "associativity": pin_associativity,
    "identity_and_padding": pin_identity_and_padding,
    "degenerate": pin_degenerate,
    "lti_convolution": pin_lti_convolution,
    "softplus": pin_softplus,
    "split_invariance": pin_split_invariance,
    "bruteforce_full": pin_bruteforce_full,
    "delta_bias": pin_delta_bias,
    "output_gate": pin_output_gate,
    "chunk_states": pin_chunk_states,
    "bwd_finite_differences": pin_bwd_finite_differences,
    "bwd_linearity": pin_bwd_linearity,
    "bwd_padding": pin_bwd_padding,
}

def pin_rows_match_full(orc, mutation=0):
    """The row sampler the full-size GPU checks use: the forward restricted to
    listed (b, d) rows equals the matching slices of the full forward bit for
    bit (rows in any order, repeated, all rows of a batch), with padding
    (lengths 0, partial and L), h0, delta bias, output gate and clip, on one
    thread and on several -- every (b, d) row is the same serial loop, so the
    two entry points may differ only in indexing."""
    rng = np.random.default_rng(14)
    nb, L, nd, N = 3, 37, 12, 4
    x, delta, A_log, B, C, D = _rand_problem(rng, nb, L, nd, N)
    vl = np.array([L, 11, 0], dtype=np.int32)
    h0 = rng.standard_normal((nb, nd, N))
    bias = 0.5 * rng.standard_normal(nd)
    z = 2.0 * rng.standard_normal((nb, L, nd))
    rows = [(1, 5), (0, 0), (2, 11), (1, 5), (0, 11)] + [(1, d) for d in range(nd)]
    rows += [(int(rng.integers(nb)), int(rng.integers(nd))) for _ in range(9)]
    rows = np.array(rows, dtype=np.int64)
    for clamp in (None, (0.01, 0.02)):
        y, h = orc.selective_scan(x, delta, A_log, B, C, D, valid_len=vl, h0=h0, delta_bias=bias, z=z,
                                  delta_clamp=clamp, nthreads=2, mutation=mutation)
        for nthreads in (1, 3):
            yr, hr = orc.selective_scan_rows(x, delta, A_log, B, C, rows, D=D, valid_len=vl, h0=h0, delta_bias=bias,
                                             z=z, delta_clamp=clamp, nthreads=nthreads, mutation=mutation)
            assert yr.shape == (len(rows), L) and hr.shape == (len(rows), N)
            for r, (bi, di) in enumerate(rows):
                assert np.array_equal(yr[r], y[bi, :, di]), (clamp, nthreads, r, bi, di)
                assert np.array_equal(hr[r], h[bi, di]), (clamp, nthreads, r, bi, di)


ALL_PINS["rows_match_full"] = pin_rows_match_full

# The planted mistakes (see ssm_oracle.c) and the pins expected to notice each.
MUTATIONS = {
    1: ("input absorbed before the decay", {"closed_form_scan", "order_sensitivity", "bruteforce_scan"}),
    2: ("readout before the state update", {"closed_form_full_path", "bruteforce_full"}),
    3: ("sign of A dropped", {"closed_form_full_path", "lti_convolution", "bruteforce_full"}),
    4: ("skip term dropped", {"degenerate", "bruteforce_full"}),
    5: ("softplus skipped", {"softplus", "lti_convolution", "bruteforce_full"}),
    6: ("delta missing from the input term", {"lti_convolution", "bruteforce_full"}),
    7: ("padding resets the state", {"identity_and_padding"}),
    8: ("B and C swapped in the input term", {"bruteforce_full"}),
    9: ("output gate applied before the skip term", {"output_gate"}),
    10: ("delta bias added after softplus", {"delta_bias"}),
    11: ("backward: adjoint not decayed through the step", {"bwd_finite_differences", "bwd_linearity"}),
    12: ("backward: dA without the delta factor", {"bwd_finite_differences"}),
    13: ("backward: softplus derivative missing", {"bwd_finite_differences"}),
    14: ("row sampler pairs a row's b with the previous row's d", {"rows_match_full"}),
}
