"""C-ABI contract of libssmscan.so, checked on the CPU: exported symbols versus
include/ssm_scan.h, struct layout, status strings, the workspace/plan query,
and every argument-error path (all of which return before any HIP call, so
these run without a GPU; fake pointers are never dereferenced)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import selective_state_space_83_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.LIB_PATH):
        from selective_state_space_83_amd import _build
        _build.build()
    return ssm.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z_0-9]+)\s*\(", text)))


def test_exports_match_header(lib):
    names = header_functions()
    assert names == sorted(ssm.EXPORTS)
    nm = subprocess.run(["nm", "-D", "--defined-only", ssm.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ssm_\w+)", nm))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


LAYOUT_C = r"""
#include <stdio.h>
#include <stddef.h>
#include "ssm_scan.h"
#define F(T, f) printf("%s %s %zu\n", #T, #f, offsetof(T, f));
int main(void) {
  printf("ssm_scan_args_t sizeof %zu\n", sizeof(ssm_scan_args_t));
  printf("ssm_step_args_t sizeof %zu\n", sizeof(ssm_step_args_t));
  printf("ssm_scan_bwd_args_t sizeof %zu\n", sizeof(ssm_scan_bwd_args_t));
  %FIELDS%
  return 0;
}
"""


STRUCTS = (("ssm_scan_args_t", ssm.ScanArgs), ("ssm_step_args_t", ssm.StepArgs),
           ("ssm_scan_bwd_args_t", ssm.BwdArgs))


def test_struct_layout_matches_header(tmp_path):
    lines = []
    for T, cls in STRUCTS:
        for f, _ in cls._fields_:
            lines.append("F(%s, %s)" % (T, f))
    src = tmp_path / "layout.c"
    src.write_text(LAYOUT_C.replace("%FIELDS%", "\n  ".join(lines)))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for line in out.splitlines():
        T, f, v = line.split()
        got[(T, f)] = int(v)
    assert got[("ssm_scan_args_t", "sizeof")] == ctypes.sizeof(ssm.ScanArgs)
    assert got[("ssm_step_args_t", "sizeof")] == ctypes.sizeof(ssm.StepArgs)
    assert got[("ssm_scan_bwd_args_t", "sizeof")] == ctypes.sizeof(ssm.BwdArgs)
    for T, cls in STRUCTS:
        for f, _ in cls._fields_:
            assert got[(T, f)] == getattr(cls, f).offset, (T, f)


def test_version_and_status_strings(lib):
    assert lib.ssm_abi_version() == 3
    for s in range(0, 8):
        assert lib.ssm_status_string(s)
    assert lib.ssm_status_string(99) == b"unknown status"


# ---------------------------------------------------------------------------
# argument errors (fake, never dereferenced, well-separated addresses)
# ---------------------------------------------------------------------------

GB = 1 << 30


def valid_scan_args(batch=2, L=64, D=32, N=16, dtype=ssm.SSM_F32, chunk_len=0):
    a = ssm.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = batch, L, D, N
    a.in_dtype = a.out_dtype = dtype
    a.disc = ssm.SSM_DISC_DELTA_B
    base = 0x100000000
    for i, f in enumerate(["x", "delta", "A", "Bm", "Cm", "Dskip", "h0", "h_last", "y",
                           "workspace"]):
        setattr(a, f, base + i * GB)
    a.chunk_len = chunk_len
    a.workspace_bytes = 1 << 40
    return a


def call(lib, a):
    return lib.ssm_scan_fwd(ctypes.byref(a), None)


def expect(lib, a, status):
    got = call(lib, a)
    assert got == status, (got, lib.ssm_last_error_message())
    assert lib.ssm_last_error_message()


def test_null_args(lib):
    assert lib.ssm_scan_fwd(None, None) == ssm.SSM_ERR_NULL
    assert lib.ssm_step(None, None) == ssm.SSM_ERR_NULL


@pytest.mark.parametrize("field", ["x", "delta", "A", "Bm", "Cm", "y"])
def test_required_pointer_missing(lib, field):
    a = valid_scan_args()
    setattr(a, field, None)
    expect(lib, a, ssm.SSM_ERR_NULL)


@pytest.mark.parametrize("field,value", [("batch", -1), ("seqlen", -3), ("dim", -1),
                                         ("dstate", 0)])
def test_bad_sizes(lib, field, value):
    a = valid_scan_args()
    setattr(a, field, value)
    expect(lib, a, ssm.SSM_ERR_SHAPE)


def test_overflowing_sizes(lib):
    a = valid_scan_args()
    a.batch, a.seqlen, a.dim = 1 << 30, 1 << 30, 1 << 30
    expect(lib, a, ssm.SSM_ERR_SHAPE)


@pytest.mark.parametrize("n", [3, 5, 32, 64])
def test_unsupported_dstate(lib, n):
    a = valid_scan_args(N=n)
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


@pytest.mark.parametrize("field,value", [("in_dtype", 2), ("out_dtype", -1), ("disc", 5)])
def test_bad_enums(lib, field, value):
    a = valid_scan_args()
    setattr(a, field, value)
    expect(lib, a, ssm.SSM_ERR_DTYPE)


@pytest.mark.parametrize("k", [0, 5, -1])
def test_bad_conv_k(lib, k):
    a = valid_scan_args()
    a.conv_w = 0x100000000 + 20 * GB
    a.conv_k = k
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


def test_reserved_and_chunk_len(lib):
    a = valid_scan_args()
    a.reserved = 1
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)
    a = valid_scan_args(chunk_len=-5)
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


@pytest.mark.parametrize("field", ["x", "Bm", "y", "h0", "workspace"])
def test_misaligned(lib, field):
    a = valid_scan_args()
    setattr(a, field, getattr(a, field) + 2)
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


@pytest.mark.parametrize("inp", ["x", "delta", "A", "Bm", "Cm", "Dskip", "h0"])
def test_y_aliases_input(lib, inp):
    a = valid_scan_args()
    a.y = getattr(a, inp)
    expect(lib, a, ssm.SSM_ERR_ALIAS)


def test_partial_overlaps(lib):
    a = valid_scan_args()
    a.y = a.x + 64            # overlaps the tail of x's range
    expect(lib, a, ssm.SSM_ERR_ALIAS)
    a = valid_scan_args()
    a.h_last = a.h0           # in-place continuation is not allowed
    expect(lib, a, ssm.SSM_ERR_ALIAS)
    a = valid_scan_args()
    a.h_last = a.y + 16
    expect(lib, a, ssm.SSM_ERR_ALIAS)


def test_adjacent_buffers_are_not_aliases(lib, monkeypatch):
    # y placed right after x's last byte must pass the alias check; it then
    # fails only at the workspace check (workspace removed on purpose)
    a = valid_scan_args(batch=1, L=4096, D=64)
    a.y = a.x + 1 * 4096 * 64 * 4
    a.workspace = None
    need = ssm.load_library().ssm_scan_workspace_size(ctypes.byref(a))
    assert need > 0
    expect(lib, a, ssm.SSM_ERR_WORKSPACE)


def test_workspace_checks(lib):
    a = valid_scan_args(batch=1, L=4096, D=64)
    need = lib.ssm_scan_workspace_size(ctypes.byref(a))
    assert need > 0
    a.workspace_bytes = need - 1
    expect(lib, a, ssm.SSM_ERR_WORKSPACE)
    a.workspace = None
    a.workspace_bytes = need
    expect(lib, a, ssm.SSM_ERR_WORKSPACE)
    a = valid_scan_args(batch=1, L=4096, D=64)
    a.workspace = a.x + 256   # overlaps x
    expect(lib, a, ssm.SSM_ERR_ALIAS)


def test_empty_problems_are_noops(lib):
    # seqlen == 0 without h_last, and batch * dim == 0: nothing is enqueued,
    # even with NULL data pointers
    a = ssm.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = 2, 0, 8, 16
    assert call(lib, a) == ssm.SSM_OK
    a.batch, a.seqlen, a.dim = 0, 10, 8
    assert call(lib, a) == ssm.SSM_OK
    a.batch, a.seqlen, a.dim = 3, 10, 0
    assert call(lib, a) == ssm.SSM_OK
    s = ssm.StepArgs()
    s.batch, s.dim, s.dstate = 0, 5, 16
    assert lib.ssm_step(ctypes.byref(s), None) == ssm.SSM_OK


def test_empty_sequence_h_last_alias(lib):
    a = ssm.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = 2, 0, 8, 16
    a.h0 = 0x100000000
    a.h_last = a.h0 + 64
    expect(lib, a, ssm.SSM_ERR_ALIAS)


# ---------------------------------------------------------------------------
# fused steps (softplus step size, gate, conv window)
# ---------------------------------------------------------------------------

def with_conv(a, k=4):
    a.conv_w = 0x100000000 + 20 * GB
    a.conv_k = k
    return a


def test_softplus_flag_and_reserved2(lib):
    a = valid_scan_args()
    a.delta_softplus = 2
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)
    a = valid_scan_args()
    a.reserved2 = 1
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


@pytest.mark.parametrize("field", ["conv_state_in", "conv_state_out"])
def test_conv_state_needs_conv(lib, field):
    a = valid_scan_args()
    setattr(a, field, 0x100000000 + 21 * GB)
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


@pytest.mark.parametrize("inp", ["x", "delta", "conv_w", "conv_state_in", "z", "delta_bias"])
def test_conv_state_out_aliases_input(lib, inp):
    a = with_conv(valid_scan_args())
    a.conv_state_in = 0x100000000 + 21 * GB
    a.z = 0x100000000 + 22 * GB
    a.delta_bias = 0x100000000 + 23 * GB
    a.conv_state_out = getattr(a, inp)
    expect(lib, a, ssm.SSM_ERR_ALIAS)


@pytest.mark.parametrize("out", ["y", "h_last", "workspace"])
def test_conv_state_out_aliases_output(lib, out):
    a = with_conv(valid_scan_args(batch=1, L=4096, D=64))
    a.conv_state_out = getattr(a, out) + 4
    expect(lib, a, ssm.SSM_ERR_ALIAS)


@pytest.mark.parametrize("inp", ["z", "delta_bias"])
def test_y_aliases_fused_input(lib, inp):
    a = valid_scan_args()
    a.z = 0x100000000 + 22 * GB
    a.delta_bias = 0x100000000 + 23 * GB
    a.y = getattr(a, inp)
    expect(lib, a, ssm.SSM_ERR_ALIAS)


def test_fused_misaligned(lib):
    a = valid_scan_args()
    a.z = 0x100000000 + 22 * GB + 2
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)
    a = with_conv(valid_scan_args())
    a.conv_state_out = 0x100000000 + 21 * GB + 2
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


def test_empty_sequence_conv_state_alias(lib):
    a = ssm.ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = 2, 0, 8, 16
    with_conv(a, 3)
    a.conv_state_in = 0x100000000
    a.conv_state_out = a.conv_state_in + 8
    expect(lib, a, ssm.SSM_ERR_ALIAS)


def test_step_fused_errors(lib):
    s = valid_step_args()
    s.delta_softplus = 7
    assert step_call(lib, s) == ssm.SSM_ERR_UNSUPPORTED
    s = valid_step_args()
    s.conv_w, s.conv_k = 0x100000000 + 20 * GB, 5
    assert step_call(lib, s) == ssm.SSM_ERR_UNSUPPORTED
    s = valid_step_args()
    s.conv_w, s.conv_k = 0x100000000 + 20 * GB, 4      # window of 3 needs a state
    assert step_call(lib, s) == ssm.SSM_ERR_NULL
    s.conv_state = s.h + 64
    assert step_call(lib, s) == ssm.SSM_ERR_ALIAS
    s.conv_state = s.x
    assert step_call(lib, s) == ssm.SSM_ERR_ALIAS
    s.conv_state = 0x100000000 + 21 * GB + 2
    assert step_call(lib, s) == ssm.SSM_ERR_UNSUPPORTED
    s = valid_step_args()
    s.z = s.y
    assert step_call(lib, s) == ssm.SSM_ERR_ALIAS


# ---------------------------------------------------------------------------
# states kept for the backward pass (h_saved)
# ---------------------------------------------------------------------------

SAVED = 0x100000000 + 30 * GB


def test_binding_abi_matches_header():
    m = re.search(r"#define SSM_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == ssm.ABI_VERSION


def test_saved_states_shape():
    assert ssm.saved_states_shape(2, 0, 8, 16) == (2, 0, 8, 16)
    assert ssm.saved_states_shape(2, 16, 8, 16) == (2, 0, 8, 16)
    assert ssm.saved_states_shape(2, 17, 8, 16) == (2, 1, 8, 16)
    assert ssm.saved_states_shape(2, 64, 8, 16) == (2, 3, 8, 16)
    assert ssm.saved_states_shape(1, 65, 8, 4) == (1, 4, 8, 4)


@pytest.mark.parametrize("cl", [7, 9, 30])
def test_saved_states_need_chunks_of_four(lib, cl):
    a = valid_scan_args(batch=1, L=256, D=64, chunk_len=cl)
    a.h_saved = SAVED
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


@pytest.mark.parametrize("L,cl", [(256, 0), (256, 8), (256, 100), (255, 1000), (255, 255)])
def test_saved_states_chunk_ok(lib, L, cl):
    # a split scan with chunks of a multiple of 4, or an unsplit one of any
    # length, passes the chunk check and stops at the alias check
    a = valid_scan_args(batch=1, L=L, D=64, chunk_len=cl)
    a.h_saved = a.y + 4
    expect(lib, a, ssm.SSM_ERR_ALIAS)


@pytest.mark.parametrize("other", ["x", "Bm", "h0", "y", "h_last", "workspace"])
def test_saved_states_alias(lib, other):
    a = valid_scan_args(batch=1, L=4096, D=64)
    a.h_saved = getattr(a, other) + 4
    expect(lib, a, ssm.SSM_ERR_ALIAS)


def test_saved_states_misaligned(lib):
    a = valid_scan_args()
    a.h_saved = SAVED + 2
    expect(lib, a, ssm.SSM_ERR_UNSUPPORTED)


def test_bwd_saved_states(lib):
    a = valid_bwd_args(batch=8, L=2048, D=1536, N=16)
    full = lib.ssm_scan_bwd_workspace_size(ctypes.byref(a))
    a.h_saved = SAVED
    saved = lib.ssm_scan_bwd_workspace_size(ctypes.byref(a))
    # the 16-step forward carries (and their Delta sums) are not needed
    assert full - saved >= 8 * 127 * 1536 * (16 + 1) * 4
    a.h_saved = a.dx + 4                   # an input over a gradient
    assert bwd_call(lib, a) == ssm.SSM_ERR_ALIAS
    a.h_saved = SAVED + 2
    assert bwd_call(lib, a) == ssm.SSM_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# plan and workspace
# ---------------------------------------------------------------------------

def plan(lib, **kw):
    a = valid_scan_args(**kw)
    return lib.ssm_scan_plan_chunk_len(ctypes.byref(a)), lib.ssm_scan_workspace_size(ctypes.byref(a))


def expected_ws(batch, L, D, N, T):
    """dsum (Bt, C-1, D) and hsum (Bt, C-1, D, N) fp32, then -- when the
    carry walk is grouped (more than 64 chunk summaries and fewer than 65536
    chains Bt * D * N) -- the group sums
    (Bt, G, D) and group states (Bt, G, D, N), G = ceil(sqrt(C - 1)) groups of
    ceil((C - 1) / G) chunks; each buffer 256-byte aligned."""
    C = -(-L // T)
    if C <= 1:
        return 0
    al = lambda v: (v + 255) // 256 * 256
    ws = al(batch * (C - 1) * D * 4) + al(batch * (C - 1) * D * N * 4)
    nc = C - 1
    if nc > 64 and batch * D * N < 65536:
        G = math.isqrt(nc - 1) + 1
        gsz = -(-nc // G)
        G = -(-nc // gsz)
        ws += al(batch * G * D * 4) + al(batch * G * D * N * 4)
    return ws


@pytest.mark.parametrize("shape", [(2, 64, 32, 16), (8, 2048, 1536, 16), (4, 8192, 2560, 16),
                                   (1, 1 << 20, 512, 16), (3, 1000, 65, 4), (1, 1, 1, 1)])
def test_plan_and_workspace(lib, shape):
    b, L, D, N = shape
    T, ws = plan(lib, batch=b, L=L, D=D, N=N)
    assert 1 <= T <= L
    assert ws == expected_ws(b, L, D, N, T)


@pytest.mark.parametrize("shape,T", [
    ((8, 2048, 1536, 16), 100),      # 192 wave columns x 21 chunks = 4032 waves
    ((4, 8192, 2560, 16), 256),      # 25 chunks of 328 at the wave target: capped at 256 steps
    ((1, 1 << 20, 512, 16), 256),    # 512 chunks of 2048: capped at 256 steps
    ((16, 2048, 2560, 16), 344),     # 6 chunks: too few for the cap
    ((1, 16384, 1024, 16), 64),      # 64-step chunks at four waves per SIMD stay
    ((4, 2048, 768, 16), 32),        # four per SIMD would cut 28-step chunks: three per SIMD
    ((8, 4096, 384, 16), 64),        # 52 -> 64
    ((8, 1024, 512, 16), 24),        # 16 -> 24
    ((2, 64, 32, 16), 64),           # short, few channels: one pass, lanes over time
    ((2, 128, 32, 16), 128),         # two blocks of 64 steps: still one pass
    ((2, 1024, 32, 16), 8),          # too long for one pass: the minimum chunk binds
    ((256, 4096, 5120, 16), 4096),   # enough waves without cutting the sequence
])
def test_auto_plan(lib, shape, T):
    b, L, D, N = shape
    assert plan(lib, batch=b, L=L, D=D, N=N)[0] == T


def test_single_pass_plan_rule(lib):
    """Short sequences of few channels (seqlen <= 512 and batch * dim *
    ceil(seqlen / 64) <= 4096 blocks of 64 steps, fewer below 64 steps) take
    the one-pass lane
    scan: the plan reports seqlen and needs no workspace, with or without
    the conv prologue.  A forced chunk length, a longer sequence or more
    channels keep the chunked passes."""
    assert plan(lib, batch=2, L=64, D=32, N=16) == (64, 0)            # 64 blocks
    assert plan(lib, batch=4, L=64, D=1024, N=16) == (64, 0)          # 4096 blocks
    assert plan(lib, batch=1, L=512, D=512, N=16) == (512, 0)         # 8 x 512
    assert plan(lib, batch=2, L=65, D=1024, N=1) == (65, 0)           # 2 x 2 x 1024
    assert plan(lib, batch=1, L=1, D=1, N=1) == (1, 0)
    T, ws = plan(lib, batch=5, L=64, D=1024, N=16)                    # 5120 blocks
    assert T < 64 and ws > 0
    T, ws = plan(lib, batch=1, L=513, D=32, N=16)                     # past 512 steps
    assert T < 513 and ws > 0
    T, ws = plan(lib, batch=3, L=65, D=1024, N=16)                    # 6144 blocks
    assert T < 65 and ws > 0
    T, ws = plan(lib, batch=2, L=64, D=128, N=16, chunk_len=8)
    assert T == 8 and ws > 0
    # the conv prologue runs inside the lane scan too
    a = valid_scan_args(batch=2, L=64, D=128, N=16)
    a.conv_w, a.conv_k = 0x100000000 + 12 * GB, 4
    assert lib.ssm_scan_plan_chunk_len(ctypes.byref(a)) == 64
    assert lib.ssm_scan_workspace_size(ctypes.byref(a)) == 0
    a = valid_scan_args(batch=2, L=1000, D=128, N=16)
    a.conv_w, a.conv_k = 0x100000000 + 12 * GB, 4
    assert lib.ssm_scan_plan_chunk_len(ctypes.byref(a)) < 1000
    assert lib.ssm_scan_workspace_size(ctypes.byref(a)) > 0


def test_short_sequence_rules(lib):
    """Shorter than a block of 64 steps, at most 64 * seqlen wave-blocks take
    the lane scan (its lanes stand partly idle); sequences of at most 32 steps
    are never cut into chunks."""
    a = lambda **kw: lane_scan(lib, N=16, **kw)
    assert a(batch=1, L=8, D=256) == 1          # 256 <= 512
    assert a(batch=1, L=8, D=2048) == 0         # 2048 > 512
    assert a(batch=1, L=32, D=2048) == 1        # 2048 <= 2048
    assert a(batch=2, L=32, D=2048) == 0
    assert a(batch=1, L=1, D=64) == 1
    assert a(batch=1, L=1, D=65) == 0
    assert plan(lib, batch=1, L=16, D=2048, N=16) == (16, 0)
    assert plan(lib, batch=2, L=32, D=2048, N=16) == (32, 0)
    assert plan(lib, batch=1, L=1, D=65, N=16) == (1, 0)
    T, ws = plan(lib, batch=2, L=33, D=2048, N=16)
    assert T < 33 and ws > 0


def lane_scan(lib, **kw):
    a = valid_scan_args(**kw)
    return lib.ssm_scan_plan_lane_scan(ctypes.byref(a))


def test_lane_scan_query(lib):
    """ssm_scan_plan_lane_scan tells the one-pass lane scan from the chunked
    passes, also where both report seqlen and no workspace (a chunked plan of
    one chunk); a conv prologue keeps the lane scan; it reads 0 for a forced
    chunk length and invalid sizes."""
    assert lane_scan(lib, batch=2, L=64, D=32, N=16) == 1
    assert lane_scan(lib, batch=1, L=512, D=512, N=16) == 1
    assert lane_scan(lib, batch=5, L=64, D=1024, N=16) == 0
    assert lane_scan(lib, batch=1, L=513, D=32, N=16) == 0
    assert lane_scan(lib, batch=2, L=64, D=128, N=16, chunk_len=8) == 0
    # one chunk of the chunked plan: same chunk length and workspace as the lane scan
    assert plan(lib, batch=256, L=4, D=5120, N=16) == (4, 0)
    assert lane_scan(lib, batch=256, L=4, D=5120, N=16) == 0
    a = valid_scan_args(batch=2, L=64, D=128, N=16)
    a.conv_w, a.conv_k = 0x100000000 + 12 * GB, 4
    assert lib.ssm_scan_plan_lane_scan(ctypes.byref(a)) == 1
    a = valid_scan_args(batch=2, L=64, D=32, N=16)
    a.dstate = 0
    assert lib.ssm_scan_plan_lane_scan(ctypes.byref(a)) == 0
    assert lib.ssm_scan_plan_lane_scan(None) == 0


def test_plan_respects_chunk_len(lib):
    for cl in (1, 7, 64, 100, 5000):
        T, ws = plan(lib, batch=2, L=1000, D=64, N=16, chunk_len=cl)
        assert T == min(cl, 1000)
        assert ws == expected_ws(2, 1000, 64, 16, T)


def test_workspace_monotone_in_length(lib):
    prev = 0
    for L in (64, 128, 1024, 4096, 65536):
        _, ws = plan(lib, batch=1, L=L, D=128, N=16, chunk_len=64)
        assert ws >= prev
        prev = ws


def test_big_batch_is_not_chunked(lib):
    T, ws = plan(lib, batch=256, L=4096, D=5120, N=16)
    assert T == 4096 and ws == 0


def test_size_queries_reject_garbage(lib):
    a = valid_scan_args()
    a.seqlen = -1
    assert lib.ssm_scan_workspace_size(ctypes.byref(a)) == 0
    assert lib.ssm_scan_plan_chunk_len(ctypes.byref(a)) == 0
    assert lib.ssm_scan_workspace_size(None) == 0


# ---------------------------------------------------------------------------
# decode step errors
# ---------------------------------------------------------------------------

def valid_step_args():
    s = ssm.StepArgs()
    s.batch, s.dim, s.dstate = 4, 64, 16
    s.in_dtype = s.out_dtype = ssm.SSM_BF16
    base = 0x100000000
    for i, f in enumerate(["x", "delta", "A", "Bm", "Cm", "Dskip", "h", "y"]):
        setattr(s, f, base + i * GB)
    return s


def step_call(lib, s):
    return lib.ssm_step(ctypes.byref(s), None)


@pytest.mark.parametrize("field", ["x", "delta", "A", "Bm", "Cm", "h", "y"])
def test_step_required(lib, field):
    s = valid_step_args()
    setattr(s, field, None)
    assert step_call(lib, s) == ssm.SSM_ERR_NULL


def test_step_errors(lib):
    s = valid_step_args()
    s.y = s.h + 8
    assert step_call(lib, s) == ssm.SSM_ERR_ALIAS
    s = valid_step_args()
    s.h = s.x
    assert step_call(lib, s) == ssm.SSM_ERR_ALIAS
    s = valid_step_args()
    s.dstate = 12
    assert step_call(lib, s) == ssm.SSM_ERR_UNSUPPORTED
    s = valid_step_args()
    s.in_dtype = 9
    assert step_call(lib, s) == ssm.SSM_ERR_DTYPE
    s = valid_step_args()
    s.dim = -2
    assert step_call(lib, s) == ssm.SSM_ERR_SHAPE
    s = valid_step_args()
    s.h += 2
    assert step_call(lib, s) == ssm.SSM_ERR_UNSUPPORTED
    s = valid_step_args()
    s.reserved = 3
    assert step_call(lib, s) == ssm.SSM_ERR_UNSUPPORTED


# ---------------------------------------------------------------------------
# backward errors and workspace
# ---------------------------------------------------------------------------

def valid_bwd_args(batch=2, L=64, D=32, N=16):
    a = ssm.BwdArgs()
    a.batch, a.seqlen, a.dim, a.dstate = batch, L, D, N
    a.in_dtype = ssm.SSM_F32
    base = 0x100000000
    for i, f in enumerate(["x", "delta", "A", "Bm", "Cm", "Dskip", "h0", "dy", "dh_last", "dx",
                           "ddelta", "dA", "dB", "dC", "dD", "dh0", "workspace"]):
        setattr(a, f, base + i * GB)
    a.workspace_bytes = 1 << 40
    return a


def bwd_call(lib, a):
    return lib.ssm_scan_bwd(ctypes.byref(a), None)


@pytest.mark.parametrize("field", ["x", "delta", "A", "Bm", "Cm", "dy", "dx", "ddelta", "dA",
                                   "dB", "dC"])
def test_bwd_required(lib, field):
    a = valid_bwd_args()
    setattr(a, field, None)
    assert bwd_call(lib, a) == ssm.SSM_ERR_NULL


def test_bwd_errors(lib):
    a = valid_bwd_args()
    a.super_chunk = 24                     # not a multiple of 16
    assert bwd_call(lib, a) == ssm.SSM_ERR_UNSUPPORTED
    a = valid_bwd_args(N=12)
    assert bwd_call(lib, a) == ssm.SSM_ERR_UNSUPPORTED
    a = valid_bwd_args()
    a.reserved = 1
    assert bwd_call(lib, a) == ssm.SSM_ERR_UNSUPPORTED
    a = valid_bwd_args()
    a.disc = 7
    assert bwd_call(lib, a) == ssm.SSM_ERR_DTYPE
    a = valid_bwd_args()
    a.dx = a.x                             # gradient over an input
    assert bwd_call(lib, a) == ssm.SSM_ERR_ALIAS
    a = valid_bwd_args()
    a.dB = a.dC + 8                        # two gradients overlap
    assert bwd_call(lib, a) == ssm.SSM_ERR_ALIAS
    a = valid_bwd_args()
    a.workspace = a.dA                     # workspace over an output
    assert bwd_call(lib, a) == ssm.SSM_ERR_ALIAS
    a = valid_bwd_args()
    a.workspace_bytes = 16
    assert bwd_call(lib, a) == ssm.SSM_ERR_WORKSPACE
    a = valid_bwd_args()
    a.dy += 2
    assert bwd_call(lib, a) == ssm.SSM_ERR_UNSUPPORTED


def test_bwd_workspace_size(lib):
    a = valid_bwd_args(batch=8, L=2048, D=1536, N=16)
    need = lib.ssm_scan_bwd_workspace_size(ctypes.byref(a))
    # at least the per-tile dB / dC partials and the 16-step forward carries
    dtiles = 24
    assert need >= 2 * 8 * 2048 * dtiles * 16 * 4 + 8 * 127 * 1536 * 16 * 4
    a.super_chunk = 5
    assert lib.ssm_scan_bwd_workspace_size(ctypes.byref(a)) == 0
    assert lib.ssm_scan_bwd_workspace_size(None) == 0


# ---------------------------------------------------------------------------
# python wrapper: refuses CPU tensors instead of falling back
# ---------------------------------------------------------------------------

def test_wrapper_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 8)
    A = -torch.ones(8, 16)
    B = torch.zeros(1, 4, 16)
    with pytest.raises(ValueError):
        ssm.scan(x, x.clone(), A, B, B.clone(), y=torch.zeros(1, 4, 8), want_h_last=False)
    with pytest.raises(ValueError):
        ssm.make_scan_args(x, x, A, B[:, :, :8], B)


def test_noalloc_refuses_plans_beyond_its_scratch(lib):
    """ssm_scan_fwd_noalloc checks everything on the host before any HIP
    call: bad arguments as ssm_scan_fwd does, and a forced chunk length whose
    summaries exceed the library's scratch array (SSM_ERR_WORKSPACE)."""
    a = valid_scan_args(batch=1, L=1 << 19, D=512, chunk_len=64)
    assert lib.ssm_scan_workspace_size(ctypes.byref(a)) > ssm.NOALLOC_SCRATCH_BYTES
    assert lib.ssm_scan_fwd_noalloc(ctypes.byref(a), None) == ssm.SSM_ERR_WORKSPACE
    assert b"scratch" in lib.ssm_last_error_message()
    assert lib.ssm_scan_fwd_noalloc(None, None) == ssm.SSM_ERR_NULL
    a = valid_scan_args()
    a.x = None
    assert lib.ssm_scan_fwd_noalloc(ctypes.byref(a), None) == ssm.SSM_ERR_NULL
