"""GPU parity of the states the forward scan keeps for the backward pass
(h_saved: the state entering steps 16, 32, ...) and of the backward scan
started from them.

The kept state entering step 16 k is the final state of the same scan over
the first 16 k steps, so the oracle's reference for it is the h_last of a
prefix scan (the recurrence is causal: the prefix sees the same inputs, conv
window and fused steps).  States are compared at the forward state tolerance
of the input precision; gradients as in test_gpu_bwd.py.
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


@pytest.fixture(autouse=True, scope="module")
def _lib():
    ssm.load_library()
    yield


def prefix_states(inp, ex, use, zoh, L):
    """Oracle states entering steps 16, 32, ... < L (prefix scans)."""
    out = []
    for t in range(16, L, 16):
        sub = dict(inp)
        for k in ("x", "delta", "B", "C"):
            sub[k] = np.ascontiguousarray(inp[k][:, :t])
        sx = dict(ex) if ex is not None else None
        if sx is not None:
            for k in ("delta_raw", "z"):
                if sx.get(k) is not None:
                    sx[k] = np.ascontiguousarray(sx[k][:, :t])
            _, hl, _ = G.oracle_scan_fused(sub, sx, use, zoh=zoh)
        else:
            _, hl = G.oracle_scan(sub, zoh=zoh)
        out.append(hl)
    Bt, D, N = inp["x"].shape[0], inp["x"].shape[2], inp["A"].shape[1]
    return np.stack(out, axis=1) if out else np.zeros((Bt, 0, D, N))


def run_forward_saved(inp, ex, use, idt, zoh, chunk_len):
    """The library's forward with h_saved; returns (y, h_last, h_saved) and
    checks that keeping the states leaves y and h_last bit-identical."""
    Bt, L, D = inp["x"].shape
    N = inp["A"].shape[1]
    t = {k: G.dev(inp[k], idt) for k in ("x", "B", "C")}
    t["delta"] = G.dev(G.step_size_inputs(inp, ex, use)[0] if ex is not None else inp["delta"], idt)
    for k in ("A", "D", "conv_w", "conv_b", "h0"):
        t[k] = G.dev(inp.get(k))
    kw = G.fused_kwargs(inp, ex, use, idt) if ex is not None else {}
    if inp.get("conv_w") is not None and ex is not None and "state" in use:
        kw["conv_state_in"] = G.dev(ex["conv_state"])
    hs = torch.full(ssm.saved_states_shape(Bt, L, D, N), float("nan"), device="cuda")
    outs = []
    for saved in (None, hs):
        y, hl = ssm.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], h0=t["h0"],
                         conv_w=t["conv_w"], conv_b=t["conv_b"], zoh=zoh, chunk_len=chunk_len,
                         h_saved=saved, **kw)
        torch.cuda.synchronize()
        outs.append((y.float().cpu().numpy(), hl.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    return outs[1][0], outs[1][1], hs.cpu().numpy()


# (batch, L, D, N, dtype, zoh, chunk_len, fused steps)
SAVED_FWD = [
    (2, 200, 70, 16, "f32", False, 0, ()),
    (2, 200, 70, 16, "f32", True, 48, ()),
    (1, 257, 130, 8, "bf16", True, 0, ()),
    (3, 33, 65, 4, "f32", False, 1000, ()),       # one chunk, L not a multiple of 4
    (2, 17, 32, 1, "f32", False, 0, ()),
    (1, 16, 32, 2, "f32", False, 0, ()),           # nothing to keep
    (2, 130, 64, 16, "f32", True, 0, ("softplus", "gate", "state")),
    (1, 300, 96, 16, "bf16", False, 64, ("bias", "gate")),
    (2, 101, 33, 16, "f32", False, 4, ()),         # chunks of one block
    (1, 50, 70, 2, "bf16", True, 8, ()),
    (2, 67, 40, 8, "f32", True, 12, ("state",)),   # conv window, chunks of 3 blocks
]


@pytest.mark.parametrize("case", SAVED_FWD, ids=lambda c: "b%d_L%d_D%d_N%d_%s_zoh%d_cl%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "+".join(c[7]) or "plain"))
def test_forward_keeps_states(case):
    Bt, L, D, N, idt, zoh, cl, use = case
    G.say("case", case)
    conv_k = 4 if "state" in use else 0
    w = SI.Workload("saved", 130 + SAVED_FWD.index(case), Bt, L, D, N, idt, idt, zoh=zoh,
                    conv_k=conv_k, a_dist="random")
    inp = SI.scan_inputs(w, h0=True)
    ex = SI.fused_inputs(w) if use else None
    _, _, hs = run_forward_saved(inp, ex, set(use), idt, zoh, cl)
    ref = prefix_states(inp, ex, set(use), zoh, L)
    assert hs.shape == ref.shape == ssm.saved_states_shape(Bt, L, D, N)
    G.compare(hs, ref, G.TOL[idt], "h_saved")


# (batch, L, D, N, dtype, zoh, super_chunk)
SAVED_BWD = [
    (2, 100, 70, 16, "f32", False, 32),
    (1, 257, 130, 16, "f32", True, 64),
    (2, 300, 200, 1, "bf16", False, 16),
    (4, 1000, 128, 16, "f32", False, 0),
    (1, 4097, 64, 4, "bf16", True, 256),
    (2, 2048, 256, 16, "bf16", True, 0),
    (2, 16, 40, 16, "f32", False, 0),               # nothing kept
    (3, 17, 65, 2, "bf16", True, 0),
    (2, 333, 96, 8, "f32", True, 48),
]


@pytest.mark.parametrize("case", SAVED_BWD, ids=lambda c: "b%d_L%d_D%d_N%d_%s_zoh%d_sc%d" % c)
def test_backward_from_kept_states(case):
    """Backward started from the forward's kept states: the oracle's
    gradients, and close to the backward that computes the states itself."""
    Bt, L, D, N, idt, zoh, sc = case
    G.say("case", case)
    w = SI.Workload("savedbwd", 140 + SAVED_BWD.index(case), Bt, L, D, N, idt, idt, zoh=zoh,
                    a_dist="random", dskip_dist="uniform")
    inp = SI.scan_inputs(w, h0=True)
    gi = SI.grad_inputs(w)
    t = {k: G.dev(inp[k], idt) for k in ("x", "delta", "B", "C")}
    A, Dv, h0 = G.dev(inp["A"]), G.dev(inp["D"]), G.dev(inp["h0"])
    dy, dhl = G.dev(gi["dy"], idt), G.dev(gi["dh_last"])
    hs = torch.empty(ssm.saved_states_shape(Bt, L, D, N), device="cuda")
    ssm.scan(t["x"], t["delta"], A, t["B"], t["C"], Dv, h0=h0, zoh=zoh, h_saved=hs)
    g_saved = ssm.scan_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0, dh_last=dhl,
                           zoh=zoh, super_chunk=sc, h_saved=hs)
    g_own = ssm.scan_bwd(t["x"], t["delta"], A, t["B"], t["C"], dy, D=Dv, h0=h0, dh_last=dhl,
                         zoh=zoh, super_chunk=sc)
    torch.cuda.synchronize()
    ref, mag = G.oracle_bwd(inp, gi["dy"], dh_last=gi["dh_last"], D=inp["D"], h0=inp["h0"],
                            zoh=zoh)
    for k in G.GRADS:
        got = g_saved[k].cpu().numpy()
        G.compare_grad(got, ref[k], mag[k], idt, k)
        G.compare_grad(got, g_own[k].cpu().numpy(), mag[k], idt, k + " (vs recomputed states)")


def _in_canary(shape, pad, canary, dtype=torch.float32):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), canary, dtype=dtype, device="cuda")
    return buf, buf[pad:pad + n].view(*shape)


def test_no_writes_outside_kept_states_and_gradients():
    """h_saved, every gradient and the backward workspace sit inside larger
    buffers filled with a canary; after the forward (keeping states, split
    into chunks) and the backward from the kept states, every canary is
    unchanged and the gradients still match the oracle."""
    import ctypes
    Bt, L, D, N = 2, 333, 70, 16
    w = SI.Workload("canary", 150, Bt, L, D, N, "f32", "f32", a_dist="random")
    inp = SI.scan_inputs(w, h0=True)
    gi = SI.grad_inputs(w)
    t = {k: G.dev(inp[k]) for k in ("x", "delta", "B", "C", "A", "D", "h0")}
    dy, dhl = G.dev(gi["dy"]), G.dev(gi["dh_last"])
    pad, canary = 4096, -12345.5
    hs_buf, hs = _in_canary(ssm.saved_states_shape(Bt, L, D, N), pad, canary)
    ssm.scan(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], h0=t["h0"], chunk_len=40,
             h_saved=hs)
    shapes = {"dx": (Bt, L, D), "ddelta": (Bt, L, D), "dA": (D, N), "dB": (Bt, L, N),
              "dC": (Bt, L, N), "dD": (D,), "dh0": (Bt, D, N)}
    bufs, grads = {}, {}
    for k, shp in shapes.items():
        bufs[k], grads[k] = _in_canary(shp, pad, canary)
    args = ssm.make_bwd_args(t["x"], t["delta"], t["A"], t["B"], t["C"], dy, t["D"], t["h0"],
                             dhl, False, grads, 0, hs)
    lib = ssm.load_library()
    need = int(lib.ssm_scan_bwd_workspace_size(ctypes.byref(args)))
    wbuf = torch.full((need + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    args.workspace = wbuf[pad:pad + need].data_ptr()
    args.workspace_bytes = need
    status = lib.ssm_scan_bwd(ctypes.byref(args), torch.cuda.current_stream().cuda_stream)
    assert status == 0, lib.ssm_last_error_message()
    torch.cuda.synchronize()
    for name, buf in [("h_saved", hs_buf)] + list(bufs.items()):
        assert torch.all(buf[:pad] == canary) and torch.all(buf[-pad:] == canary), name
    assert torch.all(wbuf[:pad] == 0xA5) and torch.all(wbuf[-pad:] == 0xA5), "workspace"
    ref, mag = G.oracle_bwd(inp, gi["dy"], dh_last=gi["dh_last"], D=inp["D"], h0=inp["h0"])
    for k in shapes:
        G.compare_grad(grads[k].cpu().numpy(), ref[k], mag[k], "f32", k)
