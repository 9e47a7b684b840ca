"""Pins for the fp64 oracle: checks of the oracle against facts the pages and
the mathematics fix, each written independently of the oracle's own code.

Every function takes an oracle instance (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees.  ``tests/test_oracle.py`` runs them
on the real oracle; ``tests/test_oracle_mutants.py`` runs them on copies of
the oracle with a planted mistake and requires at least one to fail.

Page citations (the pages are web articles on Mamba; section names as printed):
  p1  53ai.com explainer, section 3.3 "Parallel Associative Scan"
  p2  gsyq.cn "Mamba 状态空间模型深度解析", sections "连续到离散的转换",
      "选择性的实现细节", "硬件优化并行扫描算法", "计算复杂度分析"
  p3  VMamba reading note, sections "循环结构表示以快速推理",
      "卷积结构表示以并行训练", "mamba：从S4到S6的算法变化流程"
  p5  joto.ai "Mamba：2 状态空间模型", sections on time invariance and
      "离散到连续" (zero-order hold)
  p2 also: "选择性的数学解析" (Delta = Softplus(Linear(x)));
  p3 also: "简化的SSM架构" (the gated block around the SSM)
  p1 also: "一、Motivation" (recurrent inference with a carried state)
"""
from __future__ import annotations

import math
import os

import numpy as np
from scipy.integrate import solve_ivp
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    """Parse ``key: v1 v2 ...`` lines of a golden fixture (``#`` = comment)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = [float(s) for s in v.split()]
    return out


def _rel_close(got, ref, rtol=1e-12, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= rtol * scale, "%s: max abs err %.3e > %.1e * %.3e" % (what, err, rtol, scale)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _random_problem(rng, Bt, L, D, N, lti=False):
    x = rng.standard_normal((Bt, L, D))
    if lti:
        delta = np.broadcast_to(rng.uniform(0.05, 0.5, (Bt, 1, D)), (Bt, L, D)).copy()
        B = np.broadcast_to(rng.standard_normal((Bt, 1, N)), (Bt, L, N)).copy()
        C = np.broadcast_to(rng.standard_normal((Bt, 1, N)), (Bt, L, N)).copy()
    else:
        delta = rng.uniform(0.05, 0.5, (Bt, L, D))
        B = rng.standard_normal((Bt, L, N))
        C = rng.standard_normal((Bt, L, N))
    A = -rng.uniform(0.2, 3.0, (D, N))          # general negative A, rows differ
    Dsk = rng.uniform(0.5, 1.5, D)
    return x, delta, A, B, C, Dsk


def _bbar_factor(delta, A, zoh):
    """Input factor g with Bbar = g * B: Delta, or ZOH (exp(Delta A) - 1) / A
    (p2 "连续到离散的转换": Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B, which
    is elementwise for diagonal A).  delta (..., 1), A (N,) -> (..., N)."""
    if not zoh:
        return np.broadcast_to(delta, np.broadcast_shapes(delta.shape, A.shape))
    return np.expm1(delta * A) / A


# --------------------------------------------------------------------------
# P1: the hand expansion of y_2 and y_3 (p3 "循环结构表示以快速推理" and
#     "卷积结构表示以并行训练")
# --------------------------------------------------------------------------

def pin_hand_expansion_lti(orc):
    """With Delta = ln 2, A = -1 the page's Abar = exp(Delta A) is 1/2; with
    B = 1/ln 2 the simplified Bbar = Delta B is 1; C = 1, D = 0.  The page's
    y_3 = C Abar^3 Bbar x0 + C Abar^2 Bbar x1 + C Abar Bbar x2 + C Bbar x3 then
    has the coefficients stored in golden/lti_hand_expansion_p3.txt."""
    g = read_golden("lti_hand_expansion_p3.txt")
    x = np.array([[[1.5], [-2.0], [0.25], [3.0]]])          # (1, 4, 1)
    delta = np.full((1, 4, 1), math.log(2.0))
    A = np.array([[-1.0]])
    B = np.full((1, 4, 1), 1.0 / math.log(2.0))
    C = np.ones((1, 4, 1))
    y, _ = orc.scan(x, delta, A, B, C, D=np.zeros(1))
    xs = x[0, :, 0]
    y2_ref = np.dot(g["y2_coeffs"], xs[:3])
    y3_ref = np.dot(g["y3_coeffs"], xs)
    _rel_close(y[0, 2, 0], y2_ref, 1e-14, "y2 hand expansion")
    _rel_close(y[0, 3, 0], y3_ref, 1e-14, "y3 hand expansion")


def pin_hand_expansion_selective(orc):
    """The same expansion with time-varying (selective) parameters, N = 3:
    y_2 = C_2 . (Abar_2 Abar_1 Bbar_0 x0 + Abar_2 Bbar_1 x1 + Bbar_2 x2) + D x2,
    where Abar_t = exp(Delta_t A) and Bbar_t = Delta_t B_t (p3 expansion with
    the time indices made explicit; p2 loop h[k] = A_bar[k] h[k-1] + B_bar[k] x[k])."""
    rng = _rng(11)
    N = 3
    x = rng.standard_normal((1, 3, 1))
    delta = rng.uniform(0.1, 0.9, (1, 3, 1))
    A = -rng.uniform(0.3, 2.0, (1, N))
    B = rng.standard_normal((1, 3, N))
    C = rng.standard_normal((1, 3, N))
    Dsk = np.array([0.7])
    for zoh in (False, True):
        y, _ = orc.scan(x, delta, A, B, C, D=Dsk, zoh=zoh)
        ab = [np.exp(delta[0, t, 0] * A[0]) for t in range(3)]
        bb = [_bbar_factor(delta[0, t, 0], A[0], zoh) * B[0, t] for t in range(3)]
        xs = x[0, :, 0]
        h2 = ab[2] * ab[1] * bb[0] * xs[0] + ab[2] * bb[1] * xs[1] + bb[2] * xs[2]
        y2 = float(np.dot(C[0, 2], h2)) + Dsk[0] * xs[2]
        h1 = ab[1] * bb[0] * xs[0] + bb[1] * xs[1]
        y1 = float(np.dot(C[0, 1], h1)) + Dsk[0] * xs[1]
        y0 = float(np.dot(C[0, 0], bb[0] * xs[0])) + Dsk[0] * xs[0]
        _rel_close(y[0, :, 0], [y0, y1, y2], 1e-13, "selective expansion zoh=%s" % zoh)


# --------------------------------------------------------------------------
# P2: LTI closed form y = K * x, K = (C Bbar, C Abar Bbar, ..., C Abar^k Bbar)
#     (p3 "卷积结构表示以并行训练"; time invariance p5)
# --------------------------------------------------------------------------

def pin_lti_kernel(orc):
    rng = _rng(22)
    Bt, L, D, N = 2, 300, 5, 4
    for zoh in (False, True):
        x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N, lti=True)
        y, _ = orc.scan(x, delta, A, B, C, D=Dsk, zoh=zoh)
        k = np.arange(L)
        for b in range(Bt):
            for d in range(D):
                dt = delta[b, 0, d]
                abar = np.exp(dt * A[d])                               # (N,)
                bbar = _bbar_factor(np.array([dt]), A[d], zoh) * B[b, 0]
                K = (C[b, 0] * bbar * abar[None, :] ** k[:, None]).sum(axis=1)   # (L,)
                ref = np.convolve(x[b, :, d], K)[:L] + Dsk[d] * x[b, :, d]
                _rel_close(y[b, :, d], ref, 1e-12, "LTI kernel b=%d d=%d zoh=%s" % (b, d, zoh))


def pin_lti_steady_state(orc):
    """Constant x: the LTI output converges to sum_n C Bbar x / (1 - Abar) + D x."""
    Bt, L, D, N = 1, 4000, 3, 4
    rng = _rng(23)
    x = np.full((Bt, L, D), 0.8)
    delta = np.broadcast_to(rng.uniform(0.05, 0.3, (Bt, 1, D)), (Bt, L, D)).copy()
    A = -rng.uniform(0.5, 2.0, (D, N))
    B = np.broadcast_to(rng.standard_normal((Bt, 1, N)), (Bt, L, N)).copy()
    C = np.broadcast_to(rng.standard_normal((Bt, 1, N)), (Bt, L, N)).copy()
    Dsk = rng.uniform(0.5, 1.5, D)
    for zoh in (False, True):
        y, _ = orc.scan(x, delta, A, B, C, D=Dsk, zoh=zoh)
        for d in range(D):
            dt = delta[0, 0, d]
            abar = np.exp(dt * A[d])
            bbar = _bbar_factor(np.array([dt]), A[d], zoh) * B[0, 0]
            yinf = float(np.sum(C[0, 0] * bbar * 0.8 / (1 - abar))) + Dsk[d] * 0.8
            _rel_close(y[0, -1, d], yinf, 1e-10, "steady state d=%d zoh=%s" % (d, zoh))


# --------------------------------------------------------------------------
# P3: brute-force explicit sum (unrolled recurrence with time-indexed factors;
#     prod_{i=j+1..t} Abar_i = exp(A (S_t - S_j)))
# --------------------------------------------------------------------------

def brute_force(x, delta, A, B, C, Dsk, h0, zoh, u=None):
    """O(L^2 N) explicit sum; u overrides x as the scan input."""
    Bt, L, D = x.shape
    N = A.shape[1]
    u = x if u is None else u
    y = np.zeros((Bt, L, D))
    for b in range(Bt):
        for d in range(D):
            S = np.cumsum(delta[b, :, d])                        # S_t
            g = _bbar_factor(delta[b, :, d][:, None], A[d][None, :], zoh)   # (L, N)
            bu = g * B[b] * u[b, :, d][:, None]                  # (L, N)
            for t in range(L):
                decay = np.exp(A[d][None, :] * (S[t] - S[: t + 1])[:, None])   # (t+1, N)
                h = (decay * bu[: t + 1]).sum(axis=0)
                if h0 is not None:
                    h = h + np.exp(A[d] * S[t]) * h0[b, d]
                y[b, t, d] = float(np.dot(C[b, t], h)) + Dsk[d] * u[b, t, d]
    return y


def pin_brute_force(orc):
    rng = _rng(33)
    Bt, L, D, N = 2, 40, 3, 5
    for zoh in (False, True):
        x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
        h0 = rng.standard_normal((Bt, D, N))
        y, _ = orc.scan(x, delta, A, B, C, D=Dsk, h0=h0, zoh=zoh)
        ref = brute_force(x, delta, A, B, C, Dsk, h0, zoh)
        _rel_close(y, ref, 1e-12, "brute force zoh=%s" % zoh)


# --------------------------------------------------------------------------
# P4: associativity / chunk-split invariance (p1 section 3.3: the result does
#     not depend on how the elements are grouped; p2: associative scan)
# --------------------------------------------------------------------------

def combine(left, right):
    """(a, b) o (a', b') = (a a', a' b + b'), left = earlier elements."""
    a, b = left
    a2, b2 = right
    return a * a2, a2 * b + b2


def pin_split_invariance(orc):
    """scan(L1) then scan(L2, h0 = h_last) equals scan(L1 + L2), for y and
    h_last, with and without the conv prologue (whose halo crosses the cut)."""
    rng = _rng(44)
    Bt, L, D, N = 2, 90, 4, 3
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    h0 = rng.standard_normal((Bt, D, N))
    for zoh in (False, True):
        y_full, h_full = orc.scan(x, delta, A, B, C, D=Dsk, h0=h0, zoh=zoh)
        for cut in (1, 37, 89):
            y1, h1 = orc.scan(x[:, :cut], delta[:, :cut], A, B[:, :cut], C[:, :cut],
                              D=Dsk, h0=h0, zoh=zoh)
            y2, h2 = orc.scan(x[:, cut:], delta[:, cut:], A, B[:, cut:], C[:, cut:],
                              D=Dsk, h0=h1, zoh=zoh)
            _rel_close(np.concatenate([y1, y2], axis=1), y_full, 1e-12, "split y cut=%d" % cut)
            _rel_close(h2, h_full, 1e-12, "split h_last cut=%d" % cut)


def pin_associative_chunks(orc):
    """Evaluate the state with the combine operator over an arbitrary chunking
    and an arbitrary bracketing of the chunk summaries, and compare the
    resulting y and h_last with the oracle's sequential recurrence."""
    rng = _rng(45)
    Bt, L, D, N = 1, 70, 2, 4
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    h0 = rng.standard_normal((Bt, D, N))
    y_seq, h_seq = orc.scan(x, delta, A, B, C, D=Dsk, h0=h0)
    cuts = [0, 5, 6, 23, 40, 41, 64, L]
    for d in range(D):
        a_el = np.exp(delta[0, :, d][:, None] * A[d][None, :])           # (L, N)
        b_el = delta[0, :, d][:, None] * B[0] * x[0, :, d][:, None]     # (L, N)
        # chunk summaries from the identity (1, 0)
        summ = []
        for c0, c1 in zip(cuts[:-1], cuts[1:]):
            acc = (np.ones(N), np.zeros(N))
            for t in range(c0, c1):
                acc = combine(acc, (a_el[t], b_el[t]))
            summ.append(acc)
        # exclusive prefix of summaries with a right-leaning bracketing:
        # carry_c = h0 o (s_0 o (s_1 o (... o s_{c-1})))
        y = np.zeros(L)
        for ci, (c0, c1) in enumerate(zip(cuts[:-1], cuts[1:])):
            if ci == 0:
                carry = h0[0, d]
            else:
                tree = summ[ci - 1]
                for j in range(ci - 2, -1, -1):
                    tree = combine(summ[j], tree)
                carry = tree[0] * h0[0, d] + tree[1]
            h = carry
            for t in range(c0, c1):
                h = a_el[t] * h + b_el[t]
                y[t] = float(np.dot(C[0, t], h)) + Dsk[d] * x[0, t, d]
        _rel_close(y, y_seq[0, :, d], 1e-12, "assoc chunks y d=%d" % d)
        _rel_close(h, h_seq[0, d], 1e-12, "assoc chunks h d=%d" % d)


def pin_operator_associative():
    """(p o q) o r == p o (q o r) for the combine operator on random triples."""
    rng = _rng(46)
    for _ in range(100):
        p, q, r = [(rng.uniform(0, 1, 8), rng.standard_normal(8)) for _ in range(3)]
        l = combine(combine(p, q), r)
        rr = combine(p, combine(q, r))
        _rel_close(l[0], rr[0], 1e-14, "assoc a")
        _rel_close(l[1], rr[1], 1e-14, "assoc b")


# --------------------------------------------------------------------------
# P5: prefix sum (p1 section 3.3 worked example)
# --------------------------------------------------------------------------

def pin_prefix_sum(orc):
    """Delta = 1, A = 0 (Abar = 1; Bbar = Delta B = 1, and the ZOH limit is
    Delta as well), B = C = 1, D = 0: the scan is the inclusive prefix sum, and
    the page's example must come out exactly."""
    g = read_golden("prefix_sum_p1.txt")
    xs = np.array(g["input"])
    L = xs.size
    for zoh in (False, True):
        y, h = orc.scan(xs.reshape(1, L, 1), np.ones((1, L, 1)), np.zeros((1, 1)),
                        np.ones((1, L, 1)), np.ones((1, L, 1)), D=np.zeros(1), zoh=zoh)
        assert list(y[0, :, 0]) == g["output"], (list(y[0, :, 0]), g["output"])
        assert h[0, 0, 0] == g["output"][-1]


# --------------------------------------------------------------------------
# P6: exact ZOH against the ODE h' = a h + b x(t) with sample-and-hold input
#     (p5 zero-order hold as a DAC; p3 ZOH discretization)
# --------------------------------------------------------------------------

def pin_zoh_constant_input(orc):
    """Constant x, Delta, B = 1, h0 = 0, scalar a < 0: after k+1 steps the
    state is (exp(a (k+1) Delta) - 1) / a * x, the exact ODE solution."""
    L, dt, a, xv = 50, 0.07, -1.3, 0.9
    y, h = orc.scan(np.full((1, L, 1), xv), np.full((1, L, 1), dt), np.array([[a]]),
                    np.ones((1, L, 1)), np.ones((1, L, 1)), D=np.zeros(1), zoh=True)
    k = np.arange(1, L + 1)
    ref = np.expm1(a * k * dt) / a * xv
    _rel_close(y[0, :, 0], ref, 1e-12, "zoh constant input")


def pin_zoh_ode(orc):
    """Random piecewise-constant input held for Delta_k; the state sampled at
    the end of each hold interval must equal an independent numerical
    integration of the continuous system (scipy's DOP853)."""
    rng = _rng(66)
    L, N = 12, 3
    a = -rng.uniform(0.3, 2.5, N)
    dts = rng.uniform(0.05, 0.6, L)
    xs = rng.standard_normal(L)
    Bv = rng.standard_normal((L, N))
    Cv = rng.standard_normal((L, N))
    h0 = rng.standard_normal(N)
    y, h_last = orc.scan(xs.reshape(1, L, 1), dts.reshape(1, L, 1), a.reshape(1, N),
                         Bv.reshape(1, L, N), Cv.reshape(1, L, N), D=np.zeros(1),
                         h0=h0.reshape(1, 1, N), zoh=True)
    h = h0.copy()
    for k in range(L):
        sol = solve_ivp(lambda t, s: a * s + Bv[k] * xs[k], (0.0, dts[k]), h,
                        method="DOP853", rtol=1e-12, atol=1e-14)
        h = sol.y[:, -1]
        _rel_close(y[0, k, 0], float(np.dot(Cv[k], h)), 1e-9, "zoh ode y k=%d" % k)
    _rel_close(h_last[0, 0], h, 1e-9, "zoh ode h_last")


# --------------------------------------------------------------------------
# P7: special cases
# --------------------------------------------------------------------------

def pin_special_cases(orc):
    rng = _rng(77)
    Bt, L, D, N = 2, 30, 4, 3
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    h0 = rng.standard_normal((Bt, D, N))
    for zoh in (False, True):
        # Delta = 0: the state never moves, y = C_t . h0 + D x
        y, h = orc.scan(x, np.zeros_like(delta), A, B, C, D=Dsk, h0=h0, zoh=zoh)
        ref = np.einsum("bln,bdn->bld", C, h0) + Dsk[None, None, :] * x
        _rel_close(y, ref, 1e-13, "delta=0 y")
        _rel_close(h, h0, 0.0, "delta=0 h")
        # C = 0: y = D x
        y, _ = orc.scan(x, delta, A, B, np.zeros_like(C), D=Dsk, h0=h0, zoh=zoh)
        _rel_close(y, Dsk[None, None, :] * x, 0.0, "C=0")
        # x = 0: free decay h_t = exp(A S_t) h0
        y, h = orc.scan(np.zeros_like(x), delta, A, B, C, D=Dsk, h0=h0, zoh=zoh)
        S = np.cumsum(delta, axis=1)                                   # (Bt, L, D)
        ht = np.exp(A[None, None] * S[..., None]) * h0[:, None]       # (Bt, L, D, N)
        _rel_close(y, np.einsum("bln,bldn->bld", C, ht), 1e-12, "x=0 y")
        _rel_close(h, ht[:, -1], 1e-12, "x=0 h")
        # D = None means no skip term
        y0, _ = orc.scan(x, delta, A, B, C, D=None, zoh=zoh)
        y1, _ = orc.scan(x, delta, A, B, C, D=np.zeros(D), zoh=zoh)
        _rel_close(y0, y1, 0.0, "D=None")
    # channel permutation: channels are independent SSMs (p3 S4->S6 section)
    perm = rng.permutation(D)
    y, h = orc.scan(x, delta, A, B, C, D=Dsk, h0=h0)
    yp, hp = orc.scan(x[:, :, perm], delta[:, :, perm], A[perm], B, C, D=Dsk[perm],
                      h0=h0[:, perm])
    _rel_close(yp, y[:, :, perm], 0.0, "perm y")
    _rel_close(hp, h[:, perm], 0.0, "perm h")


# --------------------------------------------------------------------------
# P8: decode step == scan (p1 motivation: the recurrent form needs only the
#     previous state and the current input)
# --------------------------------------------------------------------------

def pin_decode_equals_scan(orc):
    rng = _rng(88)
    Bt, L, D, N = 3, 25, 4, 5
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    h0 = rng.standard_normal((Bt, D, N))
    for zoh in (False, True):
        y_scan, h_scan = orc.scan(x, delta, A, B, C, D=Dsk, h0=h0, zoh=zoh)
        h = h0.copy()
        ys = []
        for t in range(L):
            yt, h = orc.step(h, x[:, t], delta[:, t], A, B[:, t], C[:, t], D=Dsk, zoh=zoh)
            ys.append(yt)
        _rel_close(np.stack(ys, axis=1), y_scan, 1e-13, "decode y")
        _rel_close(h, h_scan, 1e-13, "decode h")


# --------------------------------------------------------------------------
# P9: causal depthwise conv1d + SiLU prologue (p2 SelectiveSSM: Conv1d with
#     padding d_conv - 1 and groups = d_model, causal; SiLU z * sigmoid(z))
# --------------------------------------------------------------------------

def _conv_only(orc, x, w, bias):
    """Run the oracle with C = 0 and D = 1 so that y is the scan input u."""
    Bt, L, D = x.shape
    N = 2
    y, _ = orc.scan(x, np.full_like(x, 0.1), -np.ones((D, N)), np.ones((Bt, L, N)),
                    np.zeros((Bt, L, N)), D=np.ones(D), conv_w=w, conv_b=bias)
    return y


def silu_ref(z):
    return z * expit(z)


def pin_conv_identity_tap(orc):
    """Weights e_{K-1} (only the tap on the current input) and zero bias give
    u = silu(x)."""
    rng = _rng(99)
    Bt, L, D, K = 2, 20, 3, 4
    x = rng.standard_normal((Bt, L, D))
    w = np.zeros((D, K))
    w[:, K - 1] = 1.0
    _rel_close(_conv_only(orc, x, w, np.zeros(D)), silu_ref(x), 1e-15, "identity tap")


def pin_conv_numpy(orc):
    """u[t] = silu(bias + (x * w)[t]) with the causal convolution written as
    numpy.convolve(x_d, w_d reversed)[:L] (cross-correlation with K-1 zeros
    of left padding, first L outputs)."""
    rng = _rng(98)
    Bt, L, D = 2, 33, 3
    for K in (1, 2, 3, 4):
        x = rng.standard_normal((Bt, L, D))
        w = rng.standard_normal((D, K))
        bias = rng.standard_normal(D)
        ref = np.zeros((Bt, L, D))
        for b in range(Bt):
            for d in range(D):
                ref[b, :, d] = silu_ref(np.convolve(x[b, :, d], w[d, ::-1])[:L] + bias[d])
        _rel_close(_conv_only(orc, x, w, bias), ref, 1e-13, "conv K=%d" % K)


def pin_conv_scan_brute(orc):
    """Conv prologue feeding the scan and the skip term: brute force on u."""
    rng = _rng(97)
    Bt, L, D, N, K = 1, 30, 2, 3, 4
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    w = rng.standard_normal((D, K))
    bias = rng.standard_normal(D)
    u = np.zeros_like(x)
    for d in range(D):
        u[0, :, d] = silu_ref(np.convolve(x[0, :, d], w[d, ::-1])[:L] + bias[d])
    for zoh in (False, True):
        y, _ = orc.scan(x, delta, A, B, C, D=Dsk, conv_w=w, conv_b=bias, zoh=zoh)
        ref = brute_force(x, delta, A, B, C, Dsk, None, zoh, u=u)
        _rel_close(y, ref, 1e-12, "conv+scan zoh=%s" % zoh)


# --------------------------------------------------------------------------
# P10: step size from its pre-activation, Delta = softplus(v + bias[d])
#      (p2 "选择性的数学解析": Delta = Softplus(Linear(x)); p3 "mamba：从S4到S6
#      的算法变化流程": tau_Delta = softplus)
# --------------------------------------------------------------------------

def pin_softplus_delta(orc):
    """The fused form equals the scan fed with numpy's log(exp(0) + exp(v))
    of the biased pre-activation, for both discretizations, with the conv
    prologue and with pre-activations far into both tails."""
    rng = _rng(110)
    Bt, L, D, N, K = 2, 30, 4, 3, 4
    x, _, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    raw = rng.normal(-2.0, 3.0, (Bt, L, D))
    raw[0, :4, 0] = [-60.0, -35.0, 35.0, 60.0]
    bias = rng.normal(0.0, 1.0, D)
    w = rng.standard_normal((D, K))
    cb = rng.standard_normal(D)
    for zoh in (False, True):
        for conv in (False, True):
            kw = dict(D=Dsk, zoh=zoh, conv_w=w if conv else None, conv_b=cb if conv else None)
            y, h = orc.scan(x, raw, A, B, C, delta_bias=bias, delta_softplus=True, **kw)
            y_ref, h_ref = orc.scan(x, np.logaddexp(0.0, raw + bias), A, B, C, **kw)
            _rel_close(y, y_ref, 1e-13, "softplus y zoh=%s conv=%s" % (zoh, conv))
            _rel_close(h, h_ref, 1e-13, "softplus h zoh=%s conv=%s" % (zoh, conv))
    # a bias without softplus is a plain shift
    y, _ = orc.scan(x, raw + 5.0, A, B, C, D=Dsk, delta_bias=bias)
    y_ref, _ = orc.scan(x, raw + 5.0 + bias, A, B, C, D=Dsk)
    _rel_close(y, y_ref, 1e-13, "bias only")


def pin_softplus_values(orc):
    """With one state, h0 = 0, A = -1, B = C = x = 1 and no skip, a single
    Delta*B step outputs Delta itself.  Closed forms: softplus(0) = ln 2,
    softplus(ln(e - 1)) = 1, softplus(v) = v + log1p(exp(-v)) and
    softplus(-v) = log1p(exp(-v)); each checked to 1e-14 relative, the tiny
    ones included (log(1 + exp(v)) evaluated naively loses them entirely)."""
    v = np.array([0.0, math.log(math.e - 1.0), 40.0, -40.0, -700.0, 2.5])
    ref = np.array([math.log(2.0), 1.0, 40.0 + math.log1p(math.exp(-40.0)),
                    math.log1p(math.exp(-40.0)), math.exp(-700.0),
                    2.5 + math.log1p(math.exp(-2.5))])
    one = np.ones((1, 1, 1))
    got = np.empty(v.size)
    for t in range(v.size):
        yt, _ = orc.scan(one, v[t].reshape(1, 1, 1), -np.ones((1, 1)), one, one,
                         delta_softplus=True)
        got[t] = yt[0, 0, 0]
    rel = np.abs(got - ref) / np.abs(ref)
    assert np.all(rel <= 1e-14), ("softplus values", got, ref)


# --------------------------------------------------------------------------
# P11: output gate out = y * silu(z) (p3 "简化的SSM架构": the Mamba block wraps
#      the SSM in a gated-MLP branch; reading: the gate multiplies the whole
#      SSM output, skip term included)
# --------------------------------------------------------------------------

def pin_gate(orc):
    rng = _rng(111)
    Bt, L, D, N = 2, 25, 5, 4
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    z = rng.normal(0.0, 3.0, (Bt, L, D))
    z[0, 0, :] = [0.0, -50.0, 50.0, 1e-3, -1e-3]
    w = rng.standard_normal((D, 3))
    for zoh in (False, True):
        for conv in (False, True):
            kw = dict(D=Dsk, zoh=zoh, conv_w=w if conv else None)
            y0, h0 = orc.scan(x, delta, A, B, C, **kw)
            y1, h1 = orc.scan(x, delta, A, B, C, z=z, **kw)
            _rel_close(y1, y0 * (z * expit(z)), 1e-14, "gate zoh=%s conv=%s" % (zoh, conv))
            _rel_close(h1, h0, 0.0, "gate leaves the state alone")
    assert np.all(y1[0, 0, 0] == 0.0)


# --------------------------------------------------------------------------
# P12: conv window carried across calls (p1 "一、Motivation": recurrent
#      inference needs only the carried state and the new input)
# --------------------------------------------------------------------------

def pin_conv_state_window(orc):
    """conv_state_out is the last K-1 raw inputs, oldest first, reaching into
    conv_state_in when the call is shorter than the window."""
    rng = _rng(112)
    Bt, D, N, K = 2, 3, 2, 4
    S = K - 1
    w = rng.standard_normal((D, K))
    st = rng.standard_normal((Bt, D, S))
    for L in (0, 1, 2, 3, 7):
        x = rng.standard_normal((Bt, L, D))
        out = np.full((Bt, D, S), np.nan)
        orc.scan(x, np.full_like(x, 0.1), -np.ones((D, N)), np.ones((Bt, L, N)),
                 np.ones((Bt, L, N)), conv_w=w, conv_state_in=st, conv_state_out=out)
        seq = np.concatenate([st, np.transpose(x, (0, 2, 1))], axis=2)   # (Bt, D, S + L)
        _rel_close(out, seq[:, :, L:L + S], 0.0, "window L=%d" % L)


def pin_conv_state_prefix(orc):
    """A conv state acts as K-1 extra inputs before token 0: the scan input u
    with state s equals the u that a zero-state call over [s, x] computes at
    its last L positions (numpy convolution of the concatenated sequence)."""
    rng = _rng(113)
    Bt, L, D = 2, 12, 3
    for K in (2, 3, 4):
        x = rng.standard_normal((Bt, L, D))
        w = rng.standard_normal((D, K))
        bias = rng.standard_normal(D)
        st = rng.standard_normal((Bt, D, K - 1))
        N = 2
        y, _ = orc.scan(x, np.full_like(x, 0.1), -np.ones((D, N)), np.ones((Bt, L, N)),
                        np.zeros((Bt, L, N)), D=np.ones(D), conv_w=w, conv_b=bias,
                        conv_state_in=st)
        ref = np.zeros((Bt, L, D))
        for b in range(Bt):
            for d in range(D):
                full = np.concatenate([st[b, d], x[b, :, d]])
                ref[b, :, d] = silu_ref(np.convolve(full, w[d, ::-1])[K - 1:K - 1 + L] + bias[d])
        _rel_close(y, ref, 1e-13, "state as prefix K=%d" % K)


def pin_conv_split_invariance(orc):
    """scan(x[:cut]) then scan(x[cut:]) with h and the conv window carried
    equals scan(x), including cuts shorter than the window, with softplus
    Delta and the gate on."""
    rng = _rng(114)
    Bt, L, D, N = 2, 40, 3, 4
    x, raw, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    bias = rng.standard_normal(D)
    z = rng.standard_normal((Bt, L, D))
    h0 = rng.standard_normal((Bt, D, N))
    for K in (2, 4):
        w = rng.standard_normal((D, K))
        cb = rng.standard_normal(D)
        st0 = rng.standard_normal((Bt, D, K - 1))
        kw = dict(D=Dsk, conv_w=w, conv_b=cb, delta_bias=bias, delta_softplus=True, zoh=True)
        cs_full = np.zeros((Bt, D, K - 1))
        y_full, h_full = orc.scan(x, raw, A, B, C, h0=h0, z=z, conv_state_in=st0,
                                  conv_state_out=cs_full, **kw)
        for cut in (1, 2, 21, 39):
            sl1, sl2 = slice(0, cut), slice(cut, L)
            cs1 = np.zeros((Bt, D, K - 1))
            y1, h1 = orc.scan(x[:, sl1], raw[:, sl1], A, B[:, sl1], C[:, sl1], h0=h0,
                              z=z[:, sl1], conv_state_in=st0, conv_state_out=cs1, **kw)
            cs2 = np.zeros((Bt, D, K - 1))
            y2, h2 = orc.scan(x[:, sl2], raw[:, sl2], A, B[:, sl2], C[:, sl2], h0=h1,
                              z=z[:, sl2], conv_state_in=cs1, conv_state_out=cs2, **kw)
            what = "K=%d cut=%d" % (K, cut)
            _rel_close(np.concatenate([y1, y2], axis=1), y_full, 1e-12, "split y " + what)
            _rel_close(h2, h_full, 1e-12, "split h " + what)
            _rel_close(cs2, cs_full, 0.0, "split window " + what)


def pin_decode_conv_equals_scan(orc):
    """Decode steps with the conv window, softplus Delta and the gate equal
    one scan over the same tokens, for y, h and the window."""
    rng = _rng(115)
    Bt, L, D, N, K = 2, 9, 3, 4, 4
    x, raw, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    bias = rng.standard_normal(D)
    z = rng.standard_normal((Bt, L, D))
    h0 = rng.standard_normal((Bt, D, N))
    w = rng.standard_normal((D, K))
    cb = rng.standard_normal(D)
    st0 = rng.standard_normal((Bt, D, K - 1))
    for zoh in (False, True):
        cs_scan = np.zeros((Bt, D, K - 1))
        y_scan, h_scan = orc.scan(x, raw, A, B, C, D=Dsk, h0=h0, z=z, conv_w=w, conv_b=cb,
                                  conv_state_in=st0, conv_state_out=cs_scan, zoh=zoh,
                                  delta_bias=bias, delta_softplus=True)
        h, cs = h0.copy(), st0.copy()
        ys = []
        for t in range(L):
            yt, h, cs = orc.step(h, x[:, t], raw[:, t], A, B[:, t], C[:, t], D=Dsk, zoh=zoh,
                                 delta_bias=bias, delta_softplus=True, z=z[:, t], conv_w=w,
                                 conv_b=cb, conv_state=cs)
            ys.append(yt)
        _rel_close(np.stack(ys, axis=1), y_scan, 1e-13, "decode+conv y")
        _rel_close(h, h_scan, 1e-13, "decode+conv h")
        _rel_close(cs, cs_scan, 0.0, "decode+conv window")


# --------------------------------------------------------------------------
# P13: backward pass = derivative of the forward pass (the pages give no
#      gradient formula; the derivative of the defined function is fixed by
#      the mathematics).  Checked against central finite differences of the
#      oracle's forward scan, and against homogeneity identities at sizes
#      where differencing every input would be slow.
# --------------------------------------------------------------------------

_BWD_INPUTS = ("x", "delta", "A", "B", "C", "D", "h0")
_BWD_GRAD = {"x": "dx", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "h0": "dh0"}


def _bwd_problem(rng, Bt, L, D, N):
    x, delta, A, B, C, Dsk = _random_problem(rng, Bt, L, D, N)
    return dict(x=x, delta=delta, A=A, B=B, C=C, D=Dsk, h0=rng.standard_normal((Bt, D, N)))


def _loss(orc, v, dy, dhl, zoh):
    y, hl = orc.scan(v["x"], v["delta"], v["A"], v["B"], v["C"], D=v["D"], h0=v["h0"], zoh=zoh)
    return float((dy * y).sum() + (dhl * hl).sum())


def pin_bwd_finite_differences(orc):
    """Every gradient (dx, dDelta, dA, dB, dC, dD, dh0) equals the central
    difference (eps = 1e-6) of the loss sum(dy y) + sum(dh_last h_last),
    both discretizations, including an A entry exactly 0 for ZOH."""
    rng = _rng(130)
    Bt, L, D, N = 2, 6, 2, 3
    for zoh in (False, True):
        v = _bwd_problem(rng, Bt, L, D, N)
        if zoh:
            v["A"][1, 2] = 0.0
        dy = rng.standard_normal((Bt, L, D))
        dhl = rng.standard_normal((Bt, D, N))
        g = orc.scan_bwd(v["x"], v["delta"], v["A"], v["B"], v["C"], dy, D=v["D"], h0=v["h0"],
                         dh_last=dhl, zoh=zoh)
        eps = 1e-6
        for name in _BWD_INPUTS:
            arr = v[name]
            num = np.zeros_like(arr)
            for i in np.ndindex(arr.shape):
                w = dict(v)
                ap = arr.copy()
                ap[i] += eps
                w[name] = ap
                lp = _loss(orc, w, dy, dhl, zoh)
                am = arr.copy()
                am[i] -= eps
                w[name] = am
                lm = _loss(orc, w, dy, dhl, zoh)
                num[i] = (lp - lm) / (2 * eps)
            got = g[_BWD_GRAD[name]]
            scale = max(1.0, float(np.abs(num).max()))
            err = float(np.abs(got - num).max())
            assert err <= 1e-7 * scale, ("d" + name, zoh, err, scale)


def pin_bwd_homogeneity(orc):
    """Degree-one homogeneity (Euler): the loss is linear in (x, h0) jointly,
    in C apart from the skip and h_last terms, and -- with h0 = 0 -- in B
    apart from the skip term, so L = sum(dx x) + sum(dh0 h0),
    sum(dC C) = L - sum(dy D u) - sum(dh_last h_last) and
    sum(dB B) = L - sum(dy D u).  Also dD = sum over b, t of dy * x."""
    rng = _rng(131)
    Bt, L, D, N = 2, 150, 3, 4
    for zoh in (False, True):
        v = _bwd_problem(rng, Bt, L, D, N)
        dy = rng.standard_normal((Bt, L, D))
        dhl = rng.standard_normal((Bt, D, N))
        g = orc.scan_bwd(v["x"], v["delta"], v["A"], v["B"], v["C"], dy, D=v["D"], h0=v["h0"],
                         dh_last=dhl, zoh=zoh)
        loss = _loss(orc, v, dy, dhl, zoh)
        skip = float((dy * v["D"] * v["x"]).sum())
        _, hl = orc.scan(v["x"], v["delta"], v["A"], v["B"], v["C"], D=v["D"], h0=v["h0"],
                         zoh=zoh)
        last = float((dhl * hl).sum())          # h_last does not depend on C
        tol = 1e-11 * max(1.0, abs(loss))
        assert abs((g["dx"] * v["x"]).sum() + (g["dh0"] * v["h0"]).sum() - loss) <= tol
        assert abs((g["dC"] * v["C"]).sum() - (loss - skip - last)) <= tol
        _rel_close(g["dD"], (dy * v["x"]).sum(axis=(0, 1)), 1e-13, "dD")
        w = dict(v, h0=np.zeros_like(v["h0"]))
        g0 = orc.scan_bwd(w["x"], w["delta"], w["A"], w["B"], w["C"], dy, D=w["D"],
                          h0=w["h0"], dh_last=dhl, zoh=zoh)
        loss0 = _loss(orc, w, dy, dhl, zoh)
        assert abs((g0["dB"] * w["B"]).sum() - (loss0 - skip)) <= 1e-11 * max(1.0, abs(loss0))


def _abs_problem(v, dy, dhl):
    return ({k: np.abs(a) for k, a in v.items()}, np.abs(dy), np.abs(dhl))


def pin_bwd_magnitude_is_abs_problem(orc):
    """The per-entry magnitude of a gradient is its chain-rule sum with every
    quantity replaced by its absolute value.  Where every term of a gradient
    is a product of the inputs, the states and the adjoints with nonnegative
    factors only (dx, dB, dC, dD, dh0 for both discretizations, and dA for
    Delta*B, whose A-factor derivative is 0), that is exactly the gradient of
    the same problem with every input replaced by its absolute value: the
    states and adjoints of that problem are the magnitudes of the signed one.
    The gradients returned beside the magnitudes are the plain ones, bit for
    bit."""
    rng = _rng(132)
    Bt, L, D, N = 2, 40, 3, 4
    for zoh in (False, True):
        v = _bwd_problem(rng, Bt, L, D, N)
        if zoh:
            v["A"][2, 1] = 0.0
        dy = rng.standard_normal((Bt, L, D))
        dhl = rng.standard_normal((Bt, D, N))
        args = (v["x"], v["delta"], v["A"], v["B"], v["C"], dy)
        kw = dict(D=v["D"], h0=v["h0"], dh_last=dhl, zoh=zoh)
        g, m = orc.scan_bwd(*args, mag=True, **kw)
        g_plain = orc.scan_bwd(*args, **kw)
        for k in g:
            assert np.array_equal(g[k], g_plain[k]), k
        a, ady, adhl = _abs_problem(v, dy, dhl)
        a["A"] = v["A"]            # the decay exp(Delta A) keeps its sign
        ga = orc.scan_bwd(a["x"], a["delta"], a["A"], a["B"], a["C"], ady, D=a["D"],
                          h0=a["h0"], dh_last=adhl, zoh=zoh)
        keys = ["dx", "dB", "dC", "dD", "dh0"] + ([] if zoh else ["dA"])
        for k in keys:
            _rel_close(m[k], ga[k], 1e-12, "magnitude %s zoh=%d" % (k, zoh))


def pin_bwd_magnitude_bounds(orc):
    """Every magnitude bounds its gradient from above (triangle inequality),
    for signed inputs in both discretizations; and dDelta's magnitude equals
    |dDelta| when x = 0 and h0, C, dy, dh_last are nonnegative, since every
    term is then A * Abar * h_{t-1} times a nonnegative adjoint (A < 0)."""
    rng = _rng(133)
    Bt, L, D, N = 2, 60, 3, 4
    for zoh in (False, True):
        v = _bwd_problem(rng, Bt, L, D, N)
        dy = rng.standard_normal((Bt, L, D))
        dhl = rng.standard_normal((Bt, D, N))
        g, m = orc.scan_bwd(v["x"], v["delta"], v["A"], v["B"], v["C"], dy, D=v["D"],
                            h0=v["h0"], dh_last=dhl, zoh=zoh, mag=True)
        for k in g:
            assert np.all(np.abs(g[k]) <= m[k] * (1 + 1e-12) + 1e-300), (k, zoh)
            assert np.all(m[k] >= 0.0), (k, zoh)
        w = dict(v, x=np.zeros_like(v["x"]), h0=np.abs(v["h0"]), C=np.abs(v["C"]))
        g, m = orc.scan_bwd(w["x"], w["delta"], w["A"], w["B"], w["C"], np.abs(dy), D=w["D"],
                            h0=w["h0"], dh_last=np.abs(dhl), zoh=zoh, mag=True)
        assert np.all(g["ddelta"] <= 0.0)
        _rel_close(m["ddelta"], np.abs(g["ddelta"]), 1e-12, "magnitude ddelta zoh=%d" % zoh)


ALL_PINS = [
    pin_hand_expansion_lti, pin_hand_expansion_selective, pin_lti_kernel,
    pin_lti_steady_state, pin_brute_force, pin_split_invariance,
    pin_associative_chunks, pin_prefix_sum, pin_zoh_constant_input, pin_zoh_ode,
    pin_special_cases, pin_decode_equals_scan, pin_conv_identity_tap,
    pin_conv_numpy, pin_conv_scan_brute, pin_softplus_delta, pin_softplus_values, pin_gate,
    pin_conv_state_window, pin_conv_state_prefix, pin_conv_split_invariance,
    pin_decode_conv_equals_scan, pin_bwd_finite_differences, pin_bwd_homogeneity,
    pin_bwd_magnitude_is_abs_problem, pin_bwd_magnitude_bounds,
]
