"""GPU parity of the backward selective scan (ssm_scan_bwd, through the C ABI
via the binding) against the fp64 oracle's reverse-mode derivative.

Tolerance.  Every gradient entry is a sum of chain-rule terms with
cancellation (dA over batch rows and time steps, dB and dC over channels,
dDelta and dx over states and the adjoint's geometric tail).  The oracle
returns, beside each entry, its magnitude: the same sum with every quantity
replaced by its absolute value.  Each entry is compared as
  |gpu - ref| <= rtol * magnitude
with rtol the forward tolerance of the input precision (2e-4 for fp32
inputs, 2e-2 for bf16 inputs): the rounding error of a sum is bounded by a
multiple of the sum of its terms' sizes, whatever the order it is evaluated
in, so an entry that cancels to near zero is held to the size of its own
terms.
"""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as G
import ssm_inputs as SI

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import selective_state_space_83_amd as ssm  # noqa: E402

GRADS = G.GRADS


@pytest.fixture(autouse=True, scope="module")
def _lib():
    ssm.load_library()
    yield


def run_case(Bt, L, D, N, idt, zoh, h0, dhl, skip, super_chunk, seed):
    w = SI.Workload("bwd", 120, Bt, L, D, N, idt, idt, zoh=zoh, a_dist="random",
                    dskip_dist="uniform")
    inp = SI.scan_inputs(w, seed=seed, h0=h0)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    dy = SI._store(rng.standard_normal((Bt, L, D), dtype=np.float32), idt)
    dh_last = rng.standard_normal((Bt, D, N), dtype=np.float32) if dhl else None
    Dv = inp["D"] if skip else None
    g = ssm.scan_bwd(G.dev(inp["x"], idt), G.dev(inp["delta"], idt), G.dev(inp["A"]),
                     G.dev(inp["B"], idt), G.dev(inp["C"], idt), G.dev(dy, idt), D=G.dev(Dv),
                     h0=G.dev(inp.get("h0")), dh_last=G.dev(dh_last), zoh=zoh,
                     super_chunk=super_chunk)
    torch.cuda.synchronize()
    ref, mag = G.oracle_bwd(inp, dy, dh_last=dh_last, D=Dv, h0=inp.get("h0"), zoh=zoh)
    reps = []
    for k in GRADS:
        reps.append(G.compare_grad(g[k].cpu().numpy(), ref[k], mag[k], idt, k))
    return g, reps


# (batch, L, D, N, dtype, zoh, h0, dh_last, skip, super_chunk)
BWD_SMALL = [
    (1, 1, 1, 1, "f32", False, False, False, True, 0),
    (2, 5, 3, 2, "f32", True, True, True, True, 0),
    (2, 16, 64, 4, "f32", False, True, False, True, 0),
    (3, 17, 65, 8, "f32", True, False, True, False, 0),
    (2, 100, 70, 16, "f32", False, True, True, True, 32),
    (1, 257, 130, 16, "f32", True, True, True, True, 64),
    (2, 300, 200, 1, "bf16", False, True, True, True, 16),
    (2, 129, 64, 16, "bf16", True, True, False, True, 0),
    (4, 1000, 128, 16, "f32", False, True, True, True, 0),
    (1, 4097, 64, 4, "bf16", True, False, True, True, 256),
    (2, 33, 129, 2, "f32", True, True, True, True, 16),
]


@pytest.mark.parametrize("case", BWD_SMALL, ids=lambda c: "b%d_L%d_D%d_N%d_%s_zoh%d_h%d_g%d_s%d_sc%d" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], c[8], c[9]))
def test_bwd_small_shapes(case):
    G.say("case", case)
    run_case(*case, seed=3000 + BWD_SMALL.index(case))


@pytest.mark.parametrize("idt", ["f32", "bf16"])
def test_bwd_planned_size(idt):
    """A longer problem in the library's own plan (super-chunks and the
    16-step forward carries both in play)."""
    _, reps = run_case(2, 2048, 256, 16, idt, idt == "bf16", True, True, True, 0, seed=3100)
    G.say(reps)


def test_bwd_planned_short_super_chunks():
    """Many channels and a moderate length: the plan's super-chunks (160
    steps here, from the wave target) are cut to 128 steps because the
    reverse carry walk then still crosses only 16 of them."""
    _, reps = run_case(2, 2048, 9216, 4, "bf16", True, True, True, True, 0, seed=3101)
    G.say(reps)


# (batch, L, D, N, in dtype, zoh, super-chunk): the reverse carry walk over
# more than 64 super-chunks with fewer than 65536 chains runs in groups
GROUPED_WALK = [
    (1, 4096, 64, 16, "f32", False, 16),    # 255 carries: 16 groups of 16
    (2, 2048, 130, 16, "bf16", True, 16),   # 127 carries: 12 groups, the last of 6
    (1, 2100, 33, 4, "f32", False, 32),     # 65 carries: 9 groups, the last of 1
    (1, 2048, 33, 4, "f32", True, 32),      # 63 carries: one sequential walk
]


@pytest.mark.parametrize("case", GROUPED_WALK, ids=lambda c: "b%d_L%d_D%d_N%d_%s_zoh%d_sc%d" % c)
def test_bwd_grouped_reverse_walk(case):
    Bt, L, D, N, idt, zoh, sc = case
    G.say("case", case)
    _, reps = run_case(Bt, L, D, N, idt, zoh, True, True, True, sc,
                       seed=3300 + GROUPED_WALK.index(case))
    G.say(reps)


@pytest.mark.parametrize("idt", ["f32", "bf16"])
@pytest.mark.parametrize("zoh", [False, True])
def test_bwd_large_delta(idt, zoh):
    """Step sizes large enough that exp(Delta A) underflows to 0 (Delta up to
    100 against |A| up to 8) next to ordinary ones, and within waves that also
    hold tiny step sizes (the slow-decay form then runs beside a total
    decay): every gradient against the oracle, from kept states and with the
    states recomputed, for several super-chunk lengths."""
    Bt, L, D, N = 2, 700, 130, 16
    w = SI.Workload("bigbwd", 122, Bt, L, D, N, idt, idt, zoh=zoh, a_dist="random",
                    dskip_dist="uniform")
    inp = SI.scan_inputs(w, seed=3400 + 2 * int(zoh) + (idt == "bf16"), h0=True)
    dl = inp["delta"].copy()
    dl[:, 100:110, :] = 50.0
    dl[:, 300:305, ::3] = 100.0
    dl[:, 500:520, 0::2] = 1e-6
    dl[:, 500:520, 1::2] = 60.0
    inp["delta"] = SI._store(dl, idt)
    gi = SI.grad_inputs(w)
    t = {k: G.dev(inp[k], idt) for k in ("x", "delta", "B", "C")}
    A, Dv, h0 = G.dev(inp["A"]), G.dev(inp["D"]), G.dev(inp["h0"])
    dy, dhl = G.dev(gi["dy"], idt), G.dev(gi["dh_last"])
    hs = torch.empty(ssm.saved_states_shape(Bt, L, D, N), device="cuda")
    ssm.scan(t["x"], t["delta"], A, t["B"], t["C"], Dv, h0=h0, zoh=zoh, h_saved=hs)
    ref, mag = G.oracle_bwd(inp, gi["dy"], dh_last=gi["dh_last"], D=inp["D"], h0=inp["h0"],
                            zoh=zoh)
    for sc in (0, 16, 64):
        for kept in (True, False):
            G.say("large delta bwd", idt, zoh, sc, kept)
            g = ssm.scan_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0,
                             dh_last=dhl, zoh=zoh, super_chunk=sc, h_saved=hs if kept else None)
            torch.cuda.synchronize()
            for k in GRADS:
                G.compare_grad(g[k].cpu().numpy(), ref[k], mag[k], idt,
                               "%s sc=%d kept=%d" % (k, sc, kept))


def test_bwd_deterministic():
    """Two calls give bitwise-identical gradients (partials are summed in a
    fixed order)."""
    Bt, L, D, N = 2, 700, 130, 16
    w = SI.Workload("bwd", 121, Bt, L, D, N, "f32", "f32", a_dist="random")
    inp = SI.scan_inputs(w, seed=3200, h0=True)
    dy = np.random.default_rng(1).standard_normal((Bt, L, D)).astype(np.float32)
    args = [G.dev(inp[k]) for k in ("x", "delta", "A", "B", "C")] + [G.dev(dy)]
    g1 = ssm.scan_bwd(*args, D=G.dev(inp["D"]), h0=G.dev(inp["h0"]))
    g2 = ssm.scan_bwd(*args, D=G.dev(inp["D"]), h0=G.dev(inp["h0"]))
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_empty_sequence():
    """L = 0: dA and dD are zero and dh0 is dh_last."""
    Bt, D, N = 2, 70, 16
    x = torch.empty((Bt, 0, D), device="cuda")
    B = torch.empty((Bt, 0, N), device="cuda")
    A = -torch.ones((D, N), device="cuda")
    dhl = torch.randn((Bt, D, N), device="cuda")
    g = ssm.scan_bwd(x, x, A, B, B, x, D=torch.ones(D, device="cuda"), dh_last=dhl)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dA"]).item() == 0 and torch.count_nonzero(g["dD"]).item() == 0
    assert torch.equal(g["dh0"], dhl)


def test_bwd_workload_fp32_full():
    """The bench's backward at full size (batch 8, L 2048, D 1536, N 16,
    fp32): the same seeded inputs and upstream gradients, the forward keeping
    its states and the backward started from them, and the backward that
    computes the states itself; every gradient of both compared with the
    oracle element by element."""
    w = SI.WORKLOADS["fp32"]
    G.say("workload", w)
    inp = SI.scan_inputs(w, h0=True)
    gi = SI.grad_inputs(w)
    t = {k: G.dev(inp[k]) for k in ("x", "delta", "B", "C")}
    A, Dv, h0 = G.dev(inp["A"]), G.dev(inp["D"]), G.dev(inp["h0"])
    dy, dhl = G.dev(gi["dy"]), G.dev(gi["dh_last"])
    hs = torch.empty(ssm.saved_states_shape(w.batch, w.seqlen, w.dim, w.dstate), device="cuda")
    fwd, _, _ = ssm.prepare_scan(t["x"], t["delta"], A, t["B"], t["C"], Dv, h0=h0, h_saved=hs)
    bwd, g = ssm.prepare_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0,
                             dh_last=dhl, h_saved=hs)
    own, g_own = ssm.prepare_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0,
                                 dh_last=dhl)
    fwd.run()
    bwd.run()
    own.run()
    torch.cuda.synchronize()
    ref, mag = G.oracle_bwd(inp, gi["dy"], dh_last=gi["dh_last"], D=inp["D"], h0=inp["h0"])
    for k in GRADS:
        G.say(G.compare_grad(g[k].cpu().numpy(), ref[k], mag[k], "f32", k))
        G.say(G.compare_grad(g_own[k].cpu().numpy(), ref[k], mag[k], "f32",
                             k + " (states recomputed)"))


def test_bwd_workload_long_full():
    """The long workload's backward (batch 1, L 2^20, D 512, N 16, bf16) from
    kept states, in the bench's launch configuration (512-step super-chunks,
    grouped reverse carry walk): every entry of every gradient compared with
    the oracle, which runs on 32-channel blocks in parallel (dB and dC are
    the sums of the blocks' partials)."""
    w = SI.WORKLOADS["long"]
    G.say("workload", w)
    inp = SI.scan_inputs(w, h0=True)
    gi = SI.grad_inputs(w)
    t = {k: G.dev(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    A, Dv, h0 = G.dev(inp["A"]), G.dev(inp["D"]), G.dev(inp["h0"])
    dy, dhl = G.dev(gi["dy"], "bf16"), G.dev(gi["dh_last"])
    hs = torch.empty(ssm.saved_states_shape(w.batch, w.seqlen, w.dim, w.dstate), device="cuda")
    ssm.scan(t["x"], t["delta"], A, t["B"], t["C"], Dv, h0=h0, h_saved=hs)
    g = ssm.scan_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0, dh_last=dhl,
                     h_saved=hs)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in g.items()}
    del g, hs, t, dy
    torch.cuda.empty_cache()
    G.say("gpu done; oracle on channel blocks")
    ref, mag = G.oracle_bwd_channel_blocks(inp, gi["dy"], gi["dh_last"], inp["D"], inp["h0"])
    for k in GRADS:
        G.say(G.compare_grad(got[k], ref[k], mag[k], "bf16", k))


def test_bwd_workload_conv_shape():
    """The backward the bench times on the conv workload's shape (batch 4,
    L 8192, D 2560, N 16, bf16, exact ZOH; the backward covers the scan, so
    x is the scan input), from kept states in the bench's launch
    configuration; every entry of every gradient compared with the
    oracle."""
    w = SI.WORKLOADS["conv"]
    G.say("workload", w)
    inp = SI.scan_inputs(w, h0=True)
    gi = SI.grad_inputs(w)
    t = {k: G.dev(inp[k], "bf16") for k in ("x", "delta", "B", "C")}
    A, Dv, h0 = G.dev(inp["A"]), G.dev(inp["D"]), G.dev(inp["h0"])
    dy, dhl = G.dev(gi["dy"], "bf16"), G.dev(gi["dh_last"])
    hs = torch.empty(ssm.saved_states_shape(w.batch, w.seqlen, w.dim, w.dstate), device="cuda")
    fwd, _, _ = ssm.prepare_scan(t["x"], t["delta"], A, t["B"], t["C"], Dv, h0=h0, zoh=True,
                                 h_saved=hs)
    bwd, g = ssm.prepare_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0,
                             dh_last=dhl, zoh=True, h_saved=hs)
    fwd.run()
    bwd.run()
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in g.items()}
    ref, mag = G.oracle_bwd(inp, gi["dy"], dh_last=gi["dh_last"], D=inp["D"], h0=inp["h0"],
                            zoh=True)
    for k in GRADS:
        G.say(G.compare_grad(got[k], ref[k], mag[k], "bf16", k))
