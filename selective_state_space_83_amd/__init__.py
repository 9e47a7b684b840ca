"""selective_state_space_83_amd -- the selective state-space scan (the core of
Mamba's S6 layer) on AMD Instinct MI355X.

This module is a thin ctypes binding over ``libssmscan.so`` (contract:
``include/ssm_scan.h``).  It only checks tensor placement and marshals
pointers, sizes and the current HIP stream; every step of the computation runs
in the library's HIP kernels.  PyTorch supplies device memory and streams.

    y, h_last = scan(x, delta, A, B, C, D=None, h0=None, ...)
    y = step(h, x, delta, A, B, C, D=None, ...)      # h updated in place

Shapes: x, delta, z (batch, L, dim); A (dim, N); B, C (batch, L, N); D,
delta_bias (dim,); h0, h_last, h (batch, dim, N); conv_w (dim, K <= 4);
conv_b (dim,); conv states (batch, dim, K - 1).  x, delta, B, C, z are
float32 or bfloat16 (all the same); A, D, delta_bias, states and conv weights
are float32.  Optional fused steps: delta_softplus (Delta = softplus(delta +
delta_bias)), the gate z (y * silu(z)) and the conv window carried across
calls (conv_state_in / conv_state_out for the scan, conv_state for step).

If the library is not built, importing works but every call raises: there is
no CPU fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmscan.so")

SSM_OK = 0
SSM_ERR_NULL = 1
SSM_ERR_SHAPE = 2
SSM_ERR_DTYPE = 3
SSM_ERR_UNSUPPORTED = 4
SSM_ERR_ALIAS = 5
SSM_ERR_WORKSPACE = 6
SSM_ERR_HIP = 7

# the version of include/ssm_scan.h these structures mirror; load_library
# refuses a library built from another one (its structs would differ)
ABI_VERSION = 3

# states kept for the backward pass: one every SAVE_STRIDE steps
SAVE_STRIDE = 16

SSM_F32 = 0
SSM_BF16 = 1
SSM_DISC_DELTA_B = 0
SSM_DISC_ZOH = 1


class ScanArgs(ctypes.Structure):
    """Mirror of ssm_scan_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("disc", ctypes.c_int32), ("conv_k", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p), ("Dskip", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("h_last", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("chunk_len", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("ev_main_start", ctypes.c_void_p), ("ev_main_stop", ctypes.c_void_p),
        ("delta_bias", ctypes.c_void_p), ("delta_softplus", ctypes.c_int32),
        ("reserved2", ctypes.c_int32), ("z", ctypes.c_void_p),
        ("conv_state_in", ctypes.c_void_p), ("conv_state_out", ctypes.c_void_p),
        ("h_saved", ctypes.c_void_p),
    ]


class StepArgs(ctypes.Structure):
    """Mirror of ssm_step_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("disc", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p), ("Dskip", ctypes.c_void_p),
        ("h", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("delta_bias", ctypes.c_void_p), ("delta_softplus", ctypes.c_int32),
        ("conv_k", ctypes.c_int32), ("z", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
        ("conv_b", ctypes.c_void_p), ("conv_state", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of ssm_scan_bwd_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("in_dtype", ctypes.c_int32), ("disc", ctypes.c_int32),
        ("super_chunk", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("delta", ctypes.c_void_p), ("A", ctypes.c_void_p),
        ("Bm", ctypes.c_void_p), ("Cm", ctypes.c_void_p), ("Dskip", ctypes.c_void_p),
        ("h0", ctypes.c_void_p), ("dy", ctypes.c_void_p), ("dh_last", ctypes.c_void_p),
        ("dx", ctypes.c_void_p), ("ddelta", ctypes.c_void_p), ("dA", ctypes.c_void_p),
        ("dB", ctypes.c_void_p), ("dC", ctypes.c_void_p), ("dD", ctypes.c_void_p),
        ("dh0", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("ev_main_start", ctypes.c_void_p), ("ev_main_stop", ctypes.c_void_p),
        ("h_saved", ctypes.c_void_p),
    ]


EXPORTS = ["ssm_abi_version", "ssm_scan_workspace_size", "ssm_scan_plan_chunk_len",
           "ssm_scan_plan_lane_scan",
           "ssm_scan_fwd", "ssm_scan_fwd_noalloc", "ssm_step", "ssm_scan_bwd_workspace_size",
           "ssm_scan_bwd", "ssm_status_string", "ssm_last_error_message"]

# bytes of device scratch ssm_scan_fwd_noalloc keeps per GPU (SSM_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libssmscan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run __graft_entry__.build() or "
                           "python -m selective_state_space_83_amd._build" % path)
    # PyTorch first: the library then binds to the HIP runtime PyTorch loads
    # (the same soname); loaded before it, the library would bring in the
    # system runtime, and launches would not see the device PyTorch uses
    _torch()
    lib = ctypes.CDLL(path)
    lib.ssm_abi_version.restype = ctypes.c_int
    lib.ssm_abi_version.argtypes = []
    lib.ssm_scan_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs)]
    lib.ssm_scan_plan_chunk_len.restype = ctypes.c_int64
    lib.ssm_scan_plan_chunk_len.argtypes = [ctypes.POINTER(ScanArgs)]
    lib.ssm_scan_plan_lane_scan.restype = ctypes.c_int32
    lib.ssm_scan_plan_lane_scan.argtypes = [ctypes.POINTER(ScanArgs)]
    lib.ssm_scan_fwd.restype = ctypes.c_int
    lib.ssm_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), ctypes.c_void_p]
    lib.ssm_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssm_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), ctypes.c_void_p]
    lib.ssm_step.restype = ctypes.c_int
    lib.ssm_step.argtypes = [ctypes.POINTER(StepArgs), ctypes.c_void_p]
    lib.ssm_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
    lib.ssm_scan_bwd.restype = ctypes.c_int
    lib.ssm_scan_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p]
    lib.ssm_status_string.restype = ctypes.c_char_p
    lib.ssm_status_string.argtypes = [ctypes.c_int]
    lib.ssm_last_error_message.restype = ctypes.c_char_p
    lib.ssm_last_error_message.argtypes = []
    got = int(lib.ssm_abi_version())
    if got != ABI_VERSION:
        raise RuntimeError("%s has ABI version %d, this binding mirrors version %d; rebuild it"
                           % (path, got, ABI_VERSION))
    if path == LIB_PATH:
        _lib = lib
    return lib


class SSMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("ssm status %d: %s" % (status, detail))


class SSMArgumentError(SSMError, ValueError):
    pass


def _raise_for(lib, status: int):
    if status == SSM_OK:
        return
    detail = lib.ssm_last_error_message().decode() or lib.ssm_status_string(status).decode()
    if status == SSM_ERR_HIP:
        raise SSMError(status, detail)
    raise SSMArgumentError(status, detail)


# ---------------------------------------------------------------------------
# torch-facing wrappers (argument marshalling only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise ValueError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    # the library launches on the current device (its stream): every tensor
    # must live there
    cur = _torch().cuda.current_device()
    if t.device.index is not None and t.device.index != cur:
        raise ValueError("tensor is on cuda:%d but the current device is cuda:%d"
                         % (t.device.index, cur))
    return t.data_ptr()


def _f32(t, name):
    torch = _torch()
    if t is not None and t.dtype != torch.float32:
        raise ValueError("%s must be float32" % name)
    return t


def _stream_handle(stream) -> Optional[int]:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _on_stream(stream):
    """Context in which the outputs and the workspace of a call are
    allocated: the stream the call's kernels run on.  PyTorch's caching
    allocator hands a freed block only to later allocations on the stream
    it was allocated on, so a workspace freed when the call returns cannot
    be given to other work while the call's kernels still use it."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def saved_states_shape(batch: int, seqlen: int, dim: int, dstate: int) -> tuple:
    """Shape of the states a scan keeps for the backward pass (h_saved): the
    state entering steps 16, 32, ... below seqlen."""
    n = (seqlen + SAVE_STRIDE - 1) // SAVE_STRIDE - 1 if seqlen > 0 else 0
    return (batch, n, dim, dstate)


def make_scan_args(x, delta, A, B, C, D=None, h0=None, h_last=None, y=None, conv_w=None,
                   conv_b=None, zoh=False, chunk_len=0, delta_bias=None, delta_softplus=False,
                   z=None, conv_state_in=None, conv_state_out=None, h_saved=None) -> ScanArgs:
    """Fill a ScanArgs from tensors (shape checks are the library's job)."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, dim) and A (dim, N)")
    batch, L, dim = x.shape
    a = ScanArgs()
    a.batch, a.seqlen, a.dim, a.dstate = batch, L, dim, A.shape[1]
    a.in_dtype = _dtype_code(x)
    for name, t in (("delta", delta), ("B", B), ("C", C)):
        if _dtype_code(t) != a.in_dtype:
            raise ValueError("%s must have the dtype of x" % name)
    if tuple(delta.shape) != tuple(x.shape):
        raise ValueError("delta must have the shape of x")
    if tuple(B.shape) != (batch, L, a.dstate) or tuple(C.shape) != (batch, L, a.dstate):
        raise ValueError("B and C must be (batch, L, N)")
    if tuple(A.shape) != (dim, a.dstate):
        raise ValueError("A must be (dim, N)")
    if D is not None and tuple(D.shape) != (dim,):
        raise ValueError("D must be (dim,)")
    for name, t in (("h0", h0), ("h_last", h_last)):
        if t is not None and tuple(t.shape) != (batch, dim, a.dstate):
            raise ValueError("%s must be (batch, dim, N)" % name)
    if y is not None and tuple(y.shape) != tuple(x.shape):
        raise ValueError("y must have the shape of x")
    a.out_dtype = _dtype_code(y) if y is not None else a.in_dtype
    a.disc = SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B
    a.x, a.delta, a.A, a.Bm, a.Cm = _ptr(x), _ptr(delta), _ptr(_f32(A, "A")), _ptr(B), _ptr(C)
    a.Dskip = _ptr(_f32(D, "D"))
    a.h0, a.h_last = _ptr(_f32(h0, "h0")), _ptr(_f32(h_last, "h_last"))
    a.y = _ptr(y)
    if conv_w is not None:
        if conv_w.dim() != 2 or conv_w.shape[0] != dim:
            raise ValueError("conv_w must be (dim, K)")
        if conv_b is not None and tuple(conv_b.shape) != (dim,):
            raise ValueError("conv_b must be (dim,)")
        a.conv_w, a.conv_b = _ptr(_f32(conv_w, "conv_w")), _ptr(_f32(conv_b, "conv_b"))
        a.conv_k = conv_w.shape[1]
        for name, t in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
            if t is not None and tuple(t.shape) != (batch, dim, a.conv_k - 1):
                raise ValueError("%s must be (batch, dim, K - 1)" % name)
    a.conv_state_in = _ptr(_f32(conv_state_in, "conv_state_in"))
    a.conv_state_out = _ptr(_f32(conv_state_out, "conv_state_out"))
    _fill_fused(a, dim, delta_bias, delta_softplus, z, tuple(x.shape))
    a.chunk_len = int(chunk_len)
    a.h_saved = _saved_ptr(h_saved, batch, L, dim, a.dstate)
    return a


def _saved_ptr(h_saved, batch, L, dim, N):
    if h_saved is None:
        return None
    want = saved_states_shape(batch, L, dim, N)
    if tuple(h_saved.shape) != want:
        raise ValueError("h_saved must be %s" % (want,))
    return _ptr(_f32(h_saved, "h_saved"))


def _fill_fused(a, dim, delta_bias, delta_softplus, z, z_shape):
    if delta_bias is not None and tuple(delta_bias.shape) != (dim,):
        raise ValueError("delta_bias must be (dim,)")
    a.delta_bias = _ptr(_f32(delta_bias, "delta_bias"))
    a.delta_softplus = 1 if delta_softplus else 0
    if z is not None:
        if tuple(z.shape) != z_shape:
            raise ValueError("z must have the shape of x")
        if _dtype_code(z) != a.in_dtype:
            raise ValueError("z must have the dtype of x")
    a.z = _ptr(z)


def workspace_size(args: ScanArgs) -> int:
    return int(load_library().ssm_scan_workspace_size(ctypes.byref(args)))


def plan_chunk_len(args: ScanArgs) -> int:
    return int(load_library().ssm_scan_plan_chunk_len(ctypes.byref(args)))


def plan_lane_scan(args: ScanArgs) -> bool:
    """Whether the call runs the one-pass lane scan (k_scan_wave) rather than
    the chunked passes."""
    return bool(load_library().ssm_scan_plan_lane_scan(ctypes.byref(args)))


def abi_version() -> int:
    return int(load_library().ssm_abi_version())


def scan(x, delta, A, B, C, D=None, h0=None, conv_w=None, conv_b=None, zoh=False,
         out_dtype=None, want_h_last=True, y=None, h_last=None, chunk_len=0,
         workspace=None, stream=None, events=None, delta_bias=None, delta_softplus=False,
         z=None, conv_state_in=None, conv_state_out=None,
         h_saved=None) -> Tuple[object, object]:
    """Selective-scan forward on the current (or given) stream.

    Returns (y, h_last); h_last is None when want_h_last is False and no
    h_last tensor is passed.  ``workspace`` (uint8 device tensor) may be
    passed to avoid an allocation per call; ``events`` = (start, stop) raw
    hipEvent_t handles recorded around the output-pass kernel.
    ``conv_state_out`` (float32 (batch, dim, K - 1)) is filled in place, and
    so is ``h_saved`` (float32, ``saved_states_shape(...)``), the states the
    backward pass (``scan_bwd(..., h_saved=...)``) starts from."""
    torch = _torch()
    lib = load_library()
    with _on_stream(stream):
        if y is None:
            odt = out_dtype if out_dtype is not None else x.dtype
            y = torch.empty(x.shape, dtype=odt, device=x.device)
        if h_last is None and want_h_last:
            h_last = torch.empty((x.shape[0], x.shape[2], A.shape[1]), dtype=torch.float32,
                                 device=x.device)
        args = make_scan_args(x, delta, A, B, C, D, h0, h_last, y, conv_w, conv_b, zoh,
                              chunk_len, delta_bias, delta_softplus, z, conv_state_in,
                              conv_state_out, h_saved)
        need = int(lib.ssm_scan_workspace_size(ctypes.byref(args)))
        if need > 0:
            if workspace is None or workspace.numel() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
            args.workspace = _ptr(workspace)
            args.workspace_bytes = workspace.numel()
        if events is not None:
            args.ev_main_start, args.ev_main_stop = events
        status = lib.ssm_scan_fwd(ctypes.byref(args), _stream_handle(stream))
    _raise_for(lib, status)
    return y, h_last


def scan_noalloc(args: ScanArgs, stream=None) -> None:
    """ssm_scan_fwd_noalloc on arguments filled by ``make_scan_args`` (outputs
    included): the forward scan with its chunk summaries in the library's
    per-GPU scratch array, so neither this function nor the library
    allocates.  Calls on one GPU must not overlap in time."""
    lib = load_library()
    _raise_for(lib, lib.ssm_scan_fwd_noalloc(ctypes.byref(args), _stream_handle(stream)))


class PreparedScan:
    """A scan whose arguments are validated and marshalled once, for callers
    that run the same shapes and buffers repeatedly (a decode loop, a
    benchmark, stream capture).  ``run()`` only launches; the tensors passed
    to ``prepare_scan`` must stay alive and unchanged in place/shape.  The
    object keeps the outputs and workspace it allocated alive; when it has
    run on a stream other than the one it was prepared on, synchronize that
    stream before dropping it."""

    def __init__(self, args: ScanArgs, keep: tuple):
        self.args = args
        self._keep = keep          # tensors whose pointers are in args
        self._lib = load_library()

    def run(self, stream=None, events=None):
        if events is not None:
            self.args.ev_main_start, self.args.ev_main_stop = events
        else:
            self.args.ev_main_start = self.args.ev_main_stop = None
        status = self._lib.ssm_scan_fwd(ctypes.byref(self.args), _stream_handle(stream))
        _raise_for(self._lib, status)


def prepare_scan(x, delta, A, B, C, D=None, h0=None, conv_w=None, conv_b=None, zoh=False,
                 y=None, h_last=None, chunk_len=0, workspace=None, out_dtype=None,
                 delta_bias=None, delta_softplus=False, z=None, conv_state_in=None,
                 conv_state_out=None, h_saved=None):
    """Allocate outputs and workspace (if not given), check and marshal the
    arguments once; returns (PreparedScan, y, h_last)."""
    torch = _torch()
    lib = load_library()
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype if out_dtype is not None else x.dtype,
                        device=x.device)
    args = make_scan_args(x, delta, A, B, C, D, h0, h_last, y, conv_w, conv_b, zoh, chunk_len,
                          delta_bias, delta_softplus, z, conv_state_in, conv_state_out, h_saved)
    need = int(lib.ssm_scan_workspace_size(ctypes.byref(args)))
    if need > 0 and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if need > 0:
        args.workspace = _ptr(workspace)
        args.workspace_bytes = workspace.numel()
    keep = (x, delta, A, B, C, D, h0, h_last, y, conv_w, conv_b, workspace, delta_bias, z,
            conv_state_in, conv_state_out, h_saved)
    return PreparedScan(args, keep), y, h_last


def make_step_args(h, x, delta, A, B, C, D=None, y=None, zoh=False, delta_bias=None,
                   delta_softplus=False, z=None, conv_w=None, conv_b=None,
                   conv_state=None) -> StepArgs:
    if h.dim() != 3 or x.dim() != 2:
        raise ValueError("h must be (batch, dim, N) and x (batch, dim)")
    batch, dim, N = h.shape
    a = StepArgs()
    a.batch, a.dim, a.dstate = batch, dim, N
    a.in_dtype = _dtype_code(x)
    for name, t in (("delta", delta), ("B", B), ("C", C)):
        if _dtype_code(t) != a.in_dtype:
            raise ValueError("%s must have the dtype of x" % name)
    if tuple(x.shape) != (batch, dim) or tuple(delta.shape) != (batch, dim):
        raise ValueError("x and delta must be (batch, dim)")
    if tuple(B.shape) != (batch, N) or tuple(C.shape) != (batch, N):
        raise ValueError("B and C must be (batch, N)")
    if tuple(A.shape) != (dim, N):
        raise ValueError("A must be (dim, N)")
    if D is not None and tuple(D.shape) != (dim,):
        raise ValueError("D must be (dim,)")
    if y is not None and tuple(y.shape) != (batch, dim):
        raise ValueError("y must be (batch, dim)")
    a.out_dtype = _dtype_code(y) if y is not None else a.in_dtype
    a.disc = SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B
    a.x, a.delta, a.A, a.Bm, a.Cm = _ptr(x), _ptr(delta), _ptr(_f32(A, "A")), _ptr(B), _ptr(C)
    a.Dskip = _ptr(_f32(D, "D"))
    a.h = _ptr(_f32(h, "h"))
    a.y = _ptr(y)
    _fill_fused(a, dim, delta_bias, delta_softplus, z, (batch, dim))
    if conv_w is not None:
        if conv_w.dim() != 2 or conv_w.shape[0] != dim:
            raise ValueError("conv_w must be (dim, K)")
        if conv_b is not None and tuple(conv_b.shape) != (dim,):
            raise ValueError("conv_b must be (dim,)")
        a.conv_k = conv_w.shape[1]
        if conv_state is not None and tuple(conv_state.shape) != (batch, dim, a.conv_k - 1):
            raise ValueError("conv_state must be (batch, dim, K - 1)")
        a.conv_w, a.conv_b = _ptr(_f32(conv_w, "conv_w")), _ptr(_f32(conv_b, "conv_b"))
        a.conv_state = _ptr(_f32(conv_state, "conv_state"))
    return a


class PreparedStep:
    """A decode step whose arguments are checked and marshalled once (see
    PreparedScan); ``run()`` only launches."""

    def __init__(self, args: StepArgs, keep: tuple):
        self.args = args
        self._keep = keep
        self._lib = load_library()

    def run(self, stream=None):
        status = self._lib.ssm_step(ctypes.byref(self.args), _stream_handle(stream))
        _raise_for(self._lib, status)


def prepare_step(h, x, delta, A, B, C, D=None, zoh=False, y=None, out_dtype=None,
                 delta_bias=None, delta_softplus=False, z=None, conv_w=None, conv_b=None,
                 conv_state=None):
    """Returns (PreparedStep, y) for repeated launches on the same buffers."""
    torch = _torch()
    if y is None:
        y = torch.empty(x.shape, dtype=out_dtype if out_dtype is not None else x.dtype,
                        device=x.device)
    args = make_step_args(h, x, delta, A, B, C, D, y, zoh, delta_bias, delta_softplus, z,
                          conv_w, conv_b, conv_state)
    keep = (h, x, delta, A, B, C, D, y, delta_bias, z, conv_w, conv_b, conv_state)
    return PreparedStep(args, keep), y


def step(h, x, delta, A, B, C, D=None, zoh=False, y=None, out_dtype=None, stream=None,
         delta_bias=None, delta_softplus=False, z=None, conv_w=None, conv_b=None,
         conv_state=None):
    """One decode step; h (float32, (batch, dim, N)) and, with a conv,
    conv_state (float32, (batch, dim, K - 1)) are updated in place.
    Returns y (batch, dim)."""
    torch = _torch()
    lib = load_library()
    with _on_stream(stream):
        if y is None:
            y = torch.empty(x.shape, dtype=out_dtype if out_dtype is not None else x.dtype,
                            device=x.device)
        args = make_step_args(h, x, delta, A, B, C, D, y, zoh, delta_bias, delta_softplus, z,
                              conv_w, conv_b, conv_state)
        status = lib.ssm_step(ctypes.byref(args), _stream_handle(stream))
    _raise_for(lib, status)
    return y


def make_bwd_args(x, delta, A, B, C, dy, D=None, h0=None, dh_last=None, zoh=False, grads=None,
                  super_chunk=0, h_saved=None) -> BwdArgs:
    """Fill a BwdArgs; ``grads`` is the dict of float32 gradient tensors
    (dx, ddelta, dA, dB, dC and optionally dD, dh0); ``h_saved`` the states
    kept by the forward scan of the same inputs, or None."""
    if x.dim() != 3 or A.dim() != 2:
        raise ValueError("x must be (batch, L, dim) and A (dim, N)")
    batch, L, dim = x.shape
    N = A.shape[1]
    a = BwdArgs()
    a.batch, a.seqlen, a.dim, a.dstate = batch, L, dim, N
    a.in_dtype = _dtype_code(x)
    for name, t in (("delta", delta), ("B", B), ("C", C), ("dy", dy)):
        if _dtype_code(t) != a.in_dtype:
            raise ValueError("%s must have the dtype of x" % name)
    if tuple(delta.shape) != tuple(x.shape) or tuple(dy.shape) != tuple(x.shape):
        raise ValueError("delta and dy must have the shape of x")
    if tuple(B.shape) != (batch, L, N) or tuple(C.shape) != (batch, L, N):
        raise ValueError("B and C must be (batch, L, N)")
    if D is not None and tuple(D.shape) != (dim,):
        raise ValueError("D must be (dim,)")
    for name, t in (("h0", h0), ("dh_last", dh_last)):
        if t is not None and tuple(t.shape) != (batch, dim, N):
            raise ValueError("%s must be (batch, dim, N)" % name)
    shapes = {"dx": (batch, L, dim), "ddelta": (batch, L, dim), "dA": (dim, N),
              "dB": (batch, L, N), "dC": (batch, L, N), "dD": (dim,), "dh0": (batch, dim, N)}
    for k, t in grads.items():
        if t is not None and tuple(t.shape) != shapes[k]:
            raise ValueError("%s must be %s" % (k, shapes[k]))
        setattr(a, k, _ptr(_f32(t, k)))
    a.disc = SSM_DISC_ZOH if zoh else SSM_DISC_DELTA_B
    a.super_chunk = int(super_chunk)
    a.x, a.delta, a.A, a.Bm, a.Cm = _ptr(x), _ptr(delta), _ptr(_f32(A, "A")), _ptr(B), _ptr(C)
    a.Dskip = _ptr(_f32(D, "D"))
    a.h0 = _ptr(_f32(h0, "h0"))
    a.dy = _ptr(dy)
    a.dh_last = _ptr(_f32(dh_last, "dh_last"))
    a.h_saved = _saved_ptr(h_saved, batch, L, dim, N)
    return a


class PreparedBwd:
    """A backward scan whose arguments are checked and marshalled once (see
    PreparedScan); ``run()`` only launches."""

    def __init__(self, args: BwdArgs, keep: tuple):
        self.args = args
        self._keep = keep
        self._lib = load_library()

    def run(self, stream=None, events=None):
        if events is not None:
            self.args.ev_main_start, self.args.ev_main_stop = events
        else:
            self.args.ev_main_start = self.args.ev_main_stop = None
        status = self._lib.ssm_scan_bwd(ctypes.byref(self.args), _stream_handle(stream))
        _raise_for(self._lib, status)


def _bwd_outputs(x, A, want_dD, want_dh0):
    torch = _torch()
    batch, L, dim = x.shape
    N = A.shape[1]
    dev = x.device
    f32 = torch.float32
    return {"dx": torch.empty((batch, L, dim), dtype=f32, device=dev),
            "ddelta": torch.empty((batch, L, dim), dtype=f32, device=dev),
            "dA": torch.empty((dim, N), dtype=f32, device=dev),
            "dB": torch.empty((batch, L, N), dtype=f32, device=dev),
            "dC": torch.empty((batch, L, N), dtype=f32, device=dev),
            "dD": torch.empty((dim,), dtype=f32, device=dev) if want_dD else None,
            "dh0": torch.empty((batch, dim, N), dtype=f32, device=dev) if want_dh0 else None}


def prepare_bwd(x, delta, A, B, C, dy, D=None, h0=None, dh_last=None, zoh=False,
                want_dD=True, want_dh0=True, super_chunk=0, workspace=None, h_saved=None):
    """Allocate the gradients and the workspace, check and marshal once;
    returns (PreparedBwd, grads dict)."""
    torch = _torch()
    lib = load_library()
    g = _bwd_outputs(x, A, want_dD, want_dh0)
    args = make_bwd_args(x, delta, A, B, C, dy, D, h0, dh_last, zoh, g, super_chunk, h_saved)
    need = int(lib.ssm_scan_bwd_workspace_size(ctypes.byref(args)))
    if need > 0 and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if need > 0:
        args.workspace = _ptr(workspace)
        args.workspace_bytes = workspace.numel()
    keep = (x, delta, A, B, C, dy, D, h0, dh_last, workspace, h_saved) + tuple(g.values())
    return PreparedBwd(args, keep), {k: v for k, v in g.items() if v is not None}


def scan_bwd(x, delta, A, B, C, dy, D=None, h0=None, dh_last=None, zoh=False, want_dD=True,
             want_dh0=True, super_chunk=0, workspace=None, stream=None, h_saved=None) -> dict:
    """Backward selective scan on the current (or given) stream: the
    gradients of sum(dy * y) + sum(dh_last * h_last) of ``scan`` (no fused
    steps).  Returns a dict of float32 tensors dx, ddelta, dA, dB, dC and,
    when asked, dD and dh0."""
    torch = _torch()
    lib = load_library()
    dev = x.device
    with _on_stream(stream):
        g = _bwd_outputs(x, A, want_dD, want_dh0)
        args = make_bwd_args(x, delta, A, B, C, dy, D, h0, dh_last, zoh, g, super_chunk,
                             h_saved)
        need = int(lib.ssm_scan_bwd_workspace_size(ctypes.byref(args)))
        if need > 0:
            if workspace is None or workspace.numel() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            args.workspace = _ptr(workspace)
            args.workspace_bytes = workspace.numel()
        status = lib.ssm_scan_bwd(ctypes.byref(args), _stream_handle(stream))
    _raise_for(lib, status)
    return {k: v for k, v in g.items() if v is not None}
