"""Seeded synthetic workloads for the selective scan.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random inputs and rounds them to their storage precision; it contains
none of the scan's arithmetic (no discretization, recurrence or readout), so
neither the GPU path nor the oracle depends on the other through it.

Every array is produced on the host with numpy's PCG64 generator in float32;
tensors stored as bfloat16 are rounded to nearest-even on the host before
either side sees them, so both sides consume exactly the same values.

Workloads (shapes: batch Bt, length L, channels D, states N):

  tiny   Bt=2,   L=64,        D=32,   N=16, fp32, Delta*B discretization
  fp32   Bt=8,   L=2048,      D=1536, N=16, fp32, log-uniform Delta in [1e-3, 0.1]
  conv   Bt=4,   L=8192,      D=2560, N=16, bf16, conv1d(k=4)+SiLU prologue, exact ZOH
  long   Bt=1,   L=1,048,576, D=512,  N=16, bf16 (+ an LTI variant)
  decode Bt=256, D=5120, N=16, 512 single-token steps, bf16 tokens, fp32 state

Distributions (as the Mamba pages' selective SSM module parameterizes them):
x, B, C ~ N(0, 1); Delta = softplus(0.5 * N(0, 1) - 4) unless stated;
A = -exp(A_log) with A_log[d, n] = log(n + 1), i.e. A[d, n] = -(n + 1);
D_skip = 1 unless stated; h0 = 0 unless stated; conv weights 0.5 * N(0, 1),
conv bias 0.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEED_BASE = 83_000


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs here are finite, so NaN payloads are not treated specially."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> the exact float32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bf16_to_f32(bf16_bits(a))


def softplus(z: np.ndarray) -> np.ndarray:
    """log(1 + exp(z)) in float32 (input distribution of Delta)."""
    z = np.asarray(z, dtype=np.float32)
    return np.logaddexp(np.float32(0.0), z).astype(np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    batch: int
    seqlen: int
    dim: int
    dstate: int
    in_dtype: str          # "f32" or "bf16": storage of x, delta, B, C
    out_dtype: str         # storage of y
    zoh: bool = False
    conv_k: int = 0        # 0 = no conv prologue
    delta_dist: str = "softplus"   # or "loguniform"
    dskip_dist: str = "one"        # or "uniform"
    steps: int = 0         # decode workloads: number of consecutive steps
    a_dist: str = "log"    # "log": A_log[d, n] = log(n + 1); "random": -U(0.1, 8)

    @property
    def elems(self) -> int:
        L = self.seqlen if self.steps == 0 else self.steps
        return self.batch * L * self.dim * self.dstate

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 32, 16, "f32", "f32"),
    "fp32": Workload("fp32", 2, 8, 2048, 1536, 16, "f32", "f32",
                     delta_dist="loguniform", dskip_dist="uniform"),
    "conv": Workload("conv", 3, 4, 8192, 2560, 16, "bf16", "bf16", zoh=True, conv_k=4),
    "long": Workload("long", 4, 1, 1 << 20, 512, 16, "bf16", "bf16"),
    "decode": Workload("decode", 5, 256, 1, 5120, 16, "bf16", "bf16", steps=512),
    # carries that survive whole chunks: Delta = 1e-4 everywhere
    "longmem": Workload("longmem", 99, 2, 65536, 128, 16, "f32", "f32",
                        delta_dist="const:1e-4"),
}


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _delta(rng, shape, dist):
    if dist == "softplus":
        return softplus(np.float32(0.5) * _normal(rng, shape) - np.float32(4.0))
    if dist == "loguniform":
        lo, hi = math.log(1e-3), math.log(0.1)
        return np.exp(rng.uniform(lo, hi, size=shape).astype(np.float32)).astype(np.float32)
    if dist.startswith("const:"):
        return np.full(shape, float(dist[6:]), dtype=np.float32)
    raise ValueError(dist)


def _store(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def a_matrix(dim: int, dstate: int) -> np.ndarray:
    """A = -exp(A_log), A_log[d, n] = log(n + 1): every row is -(1..N)."""
    a_log = np.log(np.arange(1, dstate + 1, dtype=np.float64))
    return np.broadcast_to(-np.exp(a_log), (dim, dstate)).astype(np.float32).copy()


def a_random(rng, dim: int, dstate: int) -> np.ndarray:
    """A general negative A: -U(0.1, 8), different for every (d, n)."""
    return (-rng.uniform(0.1, 8.0, size=(dim, dstate))).astype(np.float32)


def scan_inputs(w: Workload, seed: Optional[int] = None, lti: bool = False,
                h0: bool = False) -> dict:
    """Inputs of one ssm_scan_fwd call as float32 numpy arrays holding the
    exact stored values (bf16-rounded where the workload stores bf16).

    lti=True draws Delta (per batch and channel), B and C (per batch) once and
    repeats them over t, so the parameters are constant in time.
    h0=True draws an initial state h0 ~ N(0, 1); otherwise h0 is None (zero).
    """
    if seed is None:
        seed = SEED_BASE + w.config_id + (40 if lti else 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    Bt, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    out = {}
    out["x"] = _store(_normal(rng, (Bt, L, D)), w.in_dtype)
    if lti:
        d1 = _store(_delta(rng, (Bt, 1, D), w.delta_dist), w.in_dtype)
        b1 = _store(_normal(rng, (Bt, 1, N)), w.in_dtype)
        c1 = _store(_normal(rng, (Bt, 1, N)), w.in_dtype)
        out["delta"] = np.ascontiguousarray(np.broadcast_to(d1, (Bt, L, D)))
        out["B"] = np.ascontiguousarray(np.broadcast_to(b1, (Bt, L, N)))
        out["C"] = np.ascontiguousarray(np.broadcast_to(c1, (Bt, L, N)))
    else:
        out["delta"] = _store(_delta(rng, (Bt, L, D), w.delta_dist), w.in_dtype)
        out["B"] = _store(_normal(rng, (Bt, L, N)), w.in_dtype)
        out["C"] = _store(_normal(rng, (Bt, L, N)), w.in_dtype)
    out["A"] = a_matrix(D, N) if w.a_dist == "log" else a_random(rng, D, N)
    if w.dskip_dist == "one":
        out["D"] = np.ones(D, dtype=np.float32)
    else:
        out["D"] = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    if w.conv_k:
        out["conv_w"] = (np.float32(0.5) * _normal(rng, (D, w.conv_k))).astype(np.float32)
        out["conv_b"] = np.zeros(D, dtype=np.float32)
    else:
        out["conv_w"] = None
        out["conv_b"] = None
    out["h0"] = _normal(rng, (Bt, D, N)) if h0 else None
    return out


def decode_inputs(w: Workload, steps: Optional[int] = None, seed: Optional[int] = None) -> dict:
    """Inputs of `steps` consecutive ssm_step calls: h (Bt, D, N) ~ N(0, 1)
    fp32, and per step x, delta (steps, Bt, D), B, C (steps, Bt, N) drawn as
    the tiny workload and stored in the workload's dtype."""
    if seed is None:
        seed = SEED_BASE + w.config_id
    if steps is None:
        steps = w.steps
    rng = np.random.Generator(np.random.PCG64(seed))
    Bt, D, N = w.batch, w.dim, w.dstate
    out = {"h": _normal(rng, (Bt, D, N))}
    out["x"] = _store(_normal(rng, (steps, Bt, D)), w.in_dtype)
    out["delta"] = _store(_delta(rng, (steps, Bt, D), w.delta_dist), w.in_dtype)
    out["B"] = _store(_normal(rng, (steps, Bt, N)), w.in_dtype)
    out["C"] = _store(_normal(rng, (steps, Bt, N)), w.in_dtype)
    out["A"] = a_matrix(D, N)
    out["D"] = np.ones(D, dtype=np.float32)
    return out


def fused_inputs(w: Workload, seed: Optional[int] = None, steps: Optional[int] = None) -> dict:
    """Extra inputs of the fused steps around the scan, drawn after the
    workload's own recipe:

      delta_raw   (Bt, L, D)  pre-activation of the step size, 0.5 * N(0, 1),
                              stored in the workload's dtype; with
      delta_bias  (D,)        -4 + U(-0.5, 0.5) fp32, softplus(delta_raw +
                              delta_bias) follows the Delta recipe above;
      z           (Bt, L, D)  gate stream N(0, 1), workload dtype;
      conv_state  (Bt, D, K-1) the inputs before token 0, N(0, 1) rounded to
                              the workload's dtype (like x), fp32 storage;
      conv_w, conv_b          (with a conv) weights 0.5 * N(0, 1) and zero bias.

    With ``steps`` the per-token arrays get a leading (steps,) axis and no L
    axis instead (decode inputs)."""
    if seed is None:
        seed = SEED_BASE + w.config_id + 500
    rng = np.random.Generator(np.random.PCG64(seed))
    Bt, L, D = w.batch, w.seqlen, w.dim
    lead = (steps, Bt, D) if steps is not None else (Bt, L, D)
    K = max(w.conv_k, 1)
    out = {
        "delta_raw": _store(np.float32(0.5) * _normal(rng, lead), w.in_dtype),
        "delta_bias": (np.float32(-4.0) + rng.uniform(-0.5, 0.5, size=D)).astype(np.float32),
        "z": _store(_normal(rng, lead), w.in_dtype),
        "conv_state": _store(_normal(rng, (Bt, D, K - 1)), w.in_dtype),
    }
    if w.conv_k:
        # the conv weights of the workload recipe, for callers (decode) whose
        # scan inputs carry none
        out["conv_w"] = (np.float32(0.5) * _normal(rng, (D, w.conv_k))).astype(np.float32)
        out["conv_b"] = np.zeros(D, dtype=np.float32)
    return out


def grad_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Upstream gradients for the backward scan: dy (Bt, L, D) ~ N(0, 1) in
    the workload's dtype and dh_last (Bt, D, N) ~ N(0, 1) fp32."""
    if seed is None:
        seed = SEED_BASE + w.config_id + 700
    rng = np.random.Generator(np.random.PCG64(seed))
    return {"dy": _store(_normal(rng, (w.batch, w.seqlen, w.dim)), w.in_dtype),
            "dh_last": _normal(rng, (w.batch, w.dim, w.dstate))}
