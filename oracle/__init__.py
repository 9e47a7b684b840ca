"""fp64 CPU oracle for the selective state-space scan -- test infrastructure.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and it shares no code with the GPU library.

The arithmetic lives in ``ssm_oracle.cpp`` (the plain sequential recurrence in
double precision); this module only builds that file with g++ and marshals
numpy arrays into it.  See the header of ``ssm_oracle.cpp`` for the passages of
the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "libssm_oracle.so")


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with g++ (plain -O2, no fast-math) into ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one build of the oracle library."""

    GRADS = ("dx", "ddelta", "dA", "dB", "dC", "dD", "dh0")   # order of the C arguments

    def __init__(self, path: str = _LIB_PATH):
        if not os.path.exists(path):
            build(out=path)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.ssm_ref_scan_f64.argtypes = [i64, i64, i64, i64, dp, dp, dp, ci, dp, dp, dp, dp,
                                         dp, dp, dp, dp, i64, dp, ci, dp, dp, dp, ci]
        lib.ssm_ref_scan_f64.restype = ctypes.c_int
        lib.ssm_ref_step_f64.argtypes = [i64, i64, i64, dp, dp, dp, dp, ci, dp, dp, dp, dp,
                                         dp, dp, dp, i64, dp, ci, dp, ci]
        lib.ssm_ref_step_f64.restype = ctypes.c_int
        lib.ssm_ref_scan_bwd_f64.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp,
                                             dp, dp, ci, dp, dp, dp, dp, dp, dp, dp, ci]
        lib.ssm_ref_scan_bwd_f64.restype = ctypes.c_int
        lib.ssm_ref_scan_bwd_mag_f64.argtypes = ([i64, i64, i64, i64] + [dp] * 9 + [ci]
                                                 + [dp] * 14 + [ci])
        lib.ssm_ref_scan_bwd_mag_f64.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    @staticmethod
    def _f64(a):
        if a is None:
            return None
        return np.ascontiguousarray(a, dtype=np.float64)

    @staticmethod
    def _ptr(a):
        if a is None:
            return None
        return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))

    def scan(self, x, delta, A, B, C, D=None, h0=None, conv_w=None, conv_b=None,
             zoh=False, want_h_last=True, nthreads=0, delta_bias=None, delta_softplus=False,
             z=None, conv_state_in=None, conv_state_out=None):
        """Return (y, h_last) in float64.  Shapes: x, delta, z (batch, L, dim);
        A (dim, N); B, C (batch, L, N); D, delta_bias (dim,); h0 (batch, dim,
        N); conv_w (dim, K); conv_b (dim,); conv_state_in (batch, dim, K-1).
        ``conv_state_out``, a float64 array of shape (batch, dim, K-1), is
        filled with the last K-1 inputs when given."""
        x, delta, A, B, C = map(self._f64, (x, delta, A, B, C))
        D, h0, conv_w, conv_b = map(self._f64, (D, h0, conv_w, conv_b))
        delta_bias, z, conv_state_in = map(self._f64, (delta_bias, z, conv_state_in))
        batch, L, dim = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and A.shape == (dim, N)
        assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
        for v, shp in ((D, (dim,)), (delta_bias, (dim,)), (h0, (batch, dim, N)),
                       (z, x.shape)):
            if v is not None:
                assert v.shape == shp, (v.shape, shp)
        K = 0
        if conv_w is not None:
            assert conv_w.ndim == 2 and conv_w.shape[0] == dim
            K = conv_w.shape[1]
            if conv_b is not None:
                assert conv_b.shape == (dim,)
        for v in (conv_state_in, conv_state_out):
            if v is not None:
                assert conv_w is not None and v.shape == (batch, dim, K - 1)
        if conv_state_out is not None:
            assert conv_state_out.dtype == np.float64 and conv_state_out.flags.c_contiguous
        y = np.zeros((batch, L, dim), dtype=np.float64)
        h_last = np.zeros((batch, dim, N), dtype=np.float64) if want_h_last else None
        rc = self.lib.ssm_ref_scan_f64(batch, L, dim, N, self._ptr(x), self._ptr(delta),
                                       self._ptr(delta_bias), int(bool(delta_softplus)),
                                       self._ptr(A), self._ptr(B), self._ptr(C), self._ptr(D),
                                       self._ptr(z), self._ptr(h0), self._ptr(conv_w),
                                       self._ptr(conv_b), K, self._ptr(conv_state_in),
                                       int(bool(zoh)), self._ptr(y), self._ptr(h_last),
                                       self._ptr(conv_state_out), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return y, h_last

    def step(self, h, x, delta, A, B, C, D=None, zoh=False, nthreads=0, delta_bias=None,
             delta_softplus=False, z=None, conv_w=None, conv_b=None, conv_state=None):
        """One decode step.  Returns (y, h_new) in float64, or (y, h_new,
        conv_state_new) when ``conv_w`` is given; the inputs are not modified.
        Shapes: h (batch, dim, N); x, delta, z (batch, dim); B, C (batch, N);
        conv_w (dim, K); conv_state (batch, dim, K-1)."""
        h = np.array(h, dtype=np.float64, copy=True, order="C")
        x, delta, A, B, C, D = map(self._f64, (x, delta, A, B, C, D))
        delta_bias, z, conv_w, conv_b = map(self._f64, (delta_bias, z, conv_w, conv_b))
        batch, dim, N = h.shape
        assert x.shape == (batch, dim) and delta.shape == (batch, dim)
        assert A.shape == (dim, N) and B.shape == (batch, N) and C.shape == (batch, N)
        if z is not None:
            assert z.shape == (batch, dim)
        K = 0
        cs = None
        if conv_w is not None:
            K = conv_w.shape[1]
            assert conv_w.shape == (dim, K)
            cs = (np.zeros((batch, dim, K - 1)) if conv_state is None else
                  np.array(conv_state, dtype=np.float64, copy=True, order="C"))
            assert cs.shape == (batch, dim, K - 1)
        y = np.zeros((batch, dim), dtype=np.float64)
        rc = self.lib.ssm_ref_step_f64(batch, dim, N, self._ptr(h), self._ptr(x),
                                       self._ptr(delta), self._ptr(delta_bias),
                                       int(bool(delta_softplus)), self._ptr(A), self._ptr(B),
                                       self._ptr(C), self._ptr(D), self._ptr(z),
                                       self._ptr(conv_w), self._ptr(conv_b), K, self._ptr(cs),
                                       int(bool(zoh)), self._ptr(y), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return (y, h) if conv_w is None else (y, h, cs)

    def scan_bwd(self, x, delta, A, B, C, dy, D=None, h0=None, dh_last=None, zoh=False,
                 nthreads=0, mag=False):
        """Gradients of sum(dy * y) + sum(dh_last * h_last) for the scan
        without conv prologue.  Returns a dict of float64 arrays: dx, ddelta
        (batch, L, dim), dA (dim, N), dB, dC (batch, L, N), dD (dim,), dh0
        (batch, dim, N).

        With ``mag=True`` returns (gradients, magnitudes): the second dict has
        the same keys and shapes and holds, for every entry, its chain-rule
        sum with every term and every quantity inside a term replaced by its
        absolute value -- the scale against which the rounding error of that
        one entry is bounded, in any evaluation order."""
        x, delta, A, B, C, dy = map(self._f64, (x, delta, A, B, C, dy))
        D, h0, dh_last = map(self._f64, (D, h0, dh_last))
        batch, L, dim = x.shape
        N = A.shape[1]
        assert delta.shape == x.shape and dy.shape == x.shape and A.shape == (dim, N)
        assert B.shape == (batch, L, N) and C.shape == (batch, L, N)
        for v, shp in ((D, (dim,)), (h0, (batch, dim, N)), (dh_last, (batch, dim, N))):
            if v is not None:
                assert v.shape == shp, (v.shape, shp)
        g = {"dx": np.zeros(x.shape), "ddelta": np.zeros(x.shape), "dA": np.zeros((dim, N)),
             "dB": np.zeros(B.shape), "dC": np.zeros(C.shape), "dD": np.zeros(dim),
             "dh0": np.zeros((batch, dim, N))}
        common = [batch, L, dim, N, self._ptr(x), self._ptr(delta), self._ptr(A), self._ptr(B),
                  self._ptr(C), self._ptr(D), self._ptr(h0), self._ptr(dy), self._ptr(dh_last),
                  int(bool(zoh))] + [self._ptr(g[k]) for k in self.GRADS]
        if not mag:
            rc = self.lib.ssm_ref_scan_bwd_f64(*common, int(nthreads))
        else:
            m = {k: np.zeros_like(v) for k, v in g.items()}
            rc = self.lib.ssm_ref_scan_bwd_mag_f64(*common, *[self._ptr(m[k]) for k in self.GRADS],
                                                   int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (rc=%d)" % rc)
        return (g, m) if mag else g


_default = None


def default() -> Oracle:
    """The oracle built from ``ssm_oracle.cpp`` next to this file."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
