"""Thin ctypes binding of ``libvimscan.so`` (C ABI in include/vimscan.h).

Argument marshalling only: shapes, dtypes, devices and contiguity are checked, torch supplies the
device memory (output and workspace) and the current stream, and every step of the scan runs in
the library's HIP kernels. If the library is not built, calls raise; there is no other path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libvimscan.so"
_lock = threading.Lock()
_lib = None

VIMSCAN_F32 = 0
VIMSCAN_BF16 = 1
VIMSCAN_FLAG_GENERAL_DECAY = 1
VIMSCAN_FLAG_AUX_SWAP = 2
VIMSCAN_FLAG_FORWARD_ONLY = 4

class VimscanError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"vimscan status {status}: {text}")
        self.status = status


class _Launch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_inner", ctypes.c_int64),
                ("d_state", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("chunk_len", ctypes.c_int64), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p),
                ("scan_events", ctypes.c_void_p * 2)]


class _Plan(ctypes.Structure):
    _fields_ = [("sequences", ctypes.c_int64), ("seq_tokens", ctypes.c_int64), ("chunk_len", ctypes.c_int64),
                ("chunks", ctypes.c_int64), ("workgroups", ctypes.c_int64), ("kernels", ctypes.c_int32),
                ("park_in_workspace", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


class _Conv(ctypes.Structure):
    _fields_ = [("w_f", ctypes.c_void_p), ("bias_f", ctypes.c_void_p), ("w_b", ctypes.c_void_p),
                ("bias_b", ctypes.c_void_p), ("k", ctypes.c_int64)]


EXPORTED = ("vimscan_bidir_fwd", "vimscan_bidir_conv_fwd", "vimscan_fwd", "vimscan_plan_launch",
            "vimscan_workspace_bytes", "vimscan_status_string", "vimscan_version", "vimscan_ncssd_fwd",
            "vimscan_ncssd_plan", "vimscan_bidir_order_fwd", "vimscan_bidir_fwd_noalloc", "vimscan_wait_timeouts")

# Size of the static scratch array behind vimscan_bidir_fwd_noalloc (VIMSCAN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 96 << 20


def lib_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library():
    """Open libvimscan.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
            lib = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            lib.vimscan_bidir_fwd.restype = ctypes.c_int
            lib.vimscan_bidir_fwd.argtypes = [vp] * 13 + [ctypes.c_int64, vp, ctypes.POINTER(_Launch)]
            lib.vimscan_bidir_fwd_noalloc.restype = ctypes.c_int
            lib.vimscan_bidir_fwd_noalloc.argtypes = [vp] * 13 + [ctypes.c_int64, vp, ctypes.POINTER(_Launch)]
            lib.vimscan_fwd.restype = ctypes.c_int
            lib.vimscan_fwd.argtypes = [vp] * 8 + [ctypes.c_int64, vp, ctypes.POINTER(_Launch)]
            lib.vimscan_bidir_conv_fwd.restype = ctypes.c_int
            lib.vimscan_bidir_conv_fwd.argtypes = ([vp, ctypes.POINTER(_Conv)] + [vp] * 12
                                                   + [ctypes.c_int64, vp, ctypes.POINTER(_Launch)])
            lib.vimscan_plan_launch.restype = ctypes.c_int
            lib.vimscan_plan_launch.argtypes = [ctypes.POINTER(_Launch), ctypes.c_int64, ctypes.POINTER(_Plan)]
            lib.vimscan_workspace_bytes.restype = ctypes.c_int
            lib.vimscan_workspace_bytes.argtypes = [ctypes.POINTER(_Launch), ctypes.c_int64,
                                                    ctypes.POINTER(ctypes.c_size_t)]
            lib.vimscan_status_string.restype = ctypes.c_char_p
            lib.vimscan_status_string.argtypes = [ctypes.c_int]
            lib.vimscan_version.restype = ctypes.c_char_p
            lib.vimscan_version.argtypes = []
            lib.vimscan_bidir_order_fwd.restype = ctypes.c_int
            lib.vimscan_bidir_order_fwd.argtypes = [vp] * 14 + [ctypes.c_int64, vp, ctypes.POINTER(_Launch)]
            lib.vimscan_ncssd_fwd.restype = ctypes.c_int
            lib.vimscan_ncssd_fwd.argtypes = [vp] * 4 + [ctypes.c_int64, vp, ctypes.POINTER(_Launch)]
            lib.vimscan_ncssd_plan.restype = ctypes.c_int
            lib.vimscan_ncssd_plan.argtypes = [ctypes.POINTER(_Launch), ctypes.c_int64, ctypes.POINTER(_Plan)]
            lib.vimscan_wait_timeouts.restype = ctypes.c_int
            lib.vimscan_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().vimscan_status_string(int(status)).decode()


def wait_timeouts() -> int:
    """Waves of the one-kernel chunked scans on the current device whose wait for earlier chunks'
    aggregates gave up after its bound since the library was loaded (vimscan_wait_timeouts; 0
    unless the hardware broke the in-order dispatch the kernel relies on). Synchronous."""
    n = ctypes.c_uint64(0)
    _check(load_library().vimscan_wait_timeouts(ctypes.byref(n)))
    return int(n.value)


def _check(status: int):
    if status != 0:
        raise VimscanError(status, status_string(status))


def _io_code(dtype) -> int:
    if dtype == torch.float32:
        return VIMSCAN_F32
    if dtype == torch.bfloat16:
        return VIMSCAN_BF16
    raise TypeError(f"io dtype must be float32 or bfloat16, got {dtype}")


def make_launch(batch, seqlen, d_inner, d_state=16, io_dtype=VIMSCAN_BF16, chunk_len=0, general_decay=False,
                workspace=0, workspace_bytes=0, stream=0, aux_swap=False, forward_only=False) -> _Launch:
    flags = ((VIMSCAN_FLAG_GENERAL_DECAY if general_decay else 0) | (VIMSCAN_FLAG_AUX_SWAP if aux_swap else 0)
             | (VIMSCAN_FLAG_FORWARD_ONLY if forward_only else 0))
    return _Launch(int(batch), int(seqlen), int(d_inner), int(d_state), int(io_dtype), flags, int(chunk_len),
                   workspace or None, int(workspace_bytes), stream or None)


def launch_info(batch, seqlen, d_inner, d_state=16, seg_len=0, io_dtype="bf16", chunk_len=0, forward_only=False,
                aux_swap=False) -> dict:
    """The library's execution plan for a call with this shape (host only)."""
    code = VIMSCAN_BF16 if io_dtype == "bf16" else VIMSCAN_F32
    launch = make_launch(batch, seqlen, d_inner, d_state, code, chunk_len, aux_swap=aux_swap,
                         forward_only=forward_only)
    plan = _Plan()
    _check(load_library().vimscan_plan_launch(ctypes.byref(launch), int(seg_len), ctypes.byref(plan)))
    return {f: getattr(plan, f) for f, _ in _Plan._fields_}


def workspace_bytes(batch, seqlen, d_inner, d_state=16, seg_len=0, io_dtype="bf16", chunk_len=0,
                    forward_only=False) -> int:
    code = VIMSCAN_BF16 if io_dtype == "bf16" else VIMSCAN_F32
    launch = make_launch(batch, seqlen, d_inner, d_state, code, chunk_len, forward_only=forward_only)
    n = ctypes.c_size_t(0)
    _check(load_library().vimscan_workspace_bytes(ctypes.byref(launch), int(seg_len), ctypes.byref(n)))
    return n.value


class PreparedCall:
    """A validated call of the scan on fixed tensors: ``__call__`` only queues the kernels (one
    ctypes call), for loops that re-run the same shapes. Arguments as ``bidir_fwd``; the stream is
    torch's current stream for x's device at preparation time unless ``stream`` is given."""

    def __init__(self, x, dt, z, B_f, C_f, B_b, C_b, A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b, seg_len: int = 0,
                 out=None, chunk_len: int = 0, general_decay: bool = False, workspace=None, stream=None,
                 conv=None, aux_swap: bool = False, forward_only: bool = False, order=None, noalloc: bool = False):
        lib = load_library()
        if noalloc and (conv is not None or forward_only or order is not None or aux_swap or workspace is not None):
            raise ValueError("the allocation-free call is the plain bidirectional scan (no conv, order, swap, "
                             "forward-only or workspace)")
        if forward_only and conv is not None:
            raise ValueError("the forward-only scan takes no convolution")
        if order is not None and (conv is not None or forward_only):
            raise ValueError("a scan order goes with the plain bidirectional scan only")
        ios = (x, dt, z, B_f, C_f, B_b, C_b)
        params = (A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b)
        if x.dim() != 3:
            raise ValueError("x must be (batch, seqlen, d_inner)")
        Bsz, L, Di = x.shape
        N = B_f.shape[-1] if B_f.dim() == 3 else -1
        dev = x.device
        if dev.type != "cuda":
            raise ValueError("inputs must be on a GPU device")
        io = _io_code(x.dtype)
        shapes = [(Bsz, L, Di)] * 3 + [(Bsz, L, N)] * 4
        for t, shp in zip(ios, shapes):
            if t.device != dev or t.dtype != x.dtype or tuple(t.shape) != shp or not t.is_contiguous():
                raise ValueError("x, dt, z (B,L,Di) and B_*, C_* (B,L,N) must share device and dtype and be "
                                 "contiguous")
        pshapes = [(Di, N), (Di, N), (Di,), (Di,), (Di,), (Di,)]
        for t, shp in zip(params, pshapes):
            if t.device != dev or t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
                raise ValueError("A_* (Di,N) and D_*, dt_bias_* (Di,) must be contiguous float32 on x's device")
        cstruct = None
        if conv is not None:
            w_f, b_f, w_b, b_b = conv
            K = w_f.shape[-1] if w_f.dim() == 2 else -1
            for t, shp in zip((w_f, b_f, w_b, b_b), ((Di, K), (Di,), (Di, K), (Di,))):
                if t.device != dev or t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
                    raise ValueError("conv = (w_f, bias_f, w_b, bias_b): taps (Di,K) and biases (Di,), contiguous "
                                     "float32 on x's device")
            cstruct = _Conv(w_f.data_ptr(), b_f.data_ptr(), w_b.data_ptr(), b_b.data_ptr(), K)
            params = params + tuple(conv)
        if order is not None:
            T = seg_len if seg_len > 0 else L
            if (order.device != dev or order.dtype != torch.int32 or not order.is_contiguous()
                    or tuple(order.shape) != (Bsz * L // max(T, 1), T)):
                raise ValueError("order must be a contiguous int32 (batch * L / T, T) tensor on x's device")
            params = params + (order,)
        if out is None:
            out = torch.empty_like(x)
        elif out.device != dev or out.dtype != x.dtype or out.shape != x.shape or not out.is_contiguous():
            raise ValueError("out must match x")
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        launch = make_launch(Bsz, L, Di, N, io, chunk_len, general_decay, 0, 0, stream, aux_swap=aux_swap,
                             forward_only=forward_only)
        need = ctypes.c_size_t(0)
        _check(lib.vimscan_workspace_bytes(ctypes.byref(launch), int(seg_len), ctypes.byref(need)))
        if need.value > 0 and not noalloc:
            if workspace is None or workspace.numel() * workspace.element_size() < need.value:
                workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
            launch.workspace = workspace.data_ptr()
            launch.workspace_bytes = workspace.numel() * workspace.element_size()
        self.out = out
        self._keep = (ios, params, out, workspace)   # keep every buffer alive while prepared
        self._launch = launch
        self._conv = cstruct
        if noalloc:
            self._fn = lib.vimscan_bidir_fwd_noalloc
            self._args = (tuple(t.data_ptr() for t in ios + params)
                          + (int(seg_len), out.data_ptr(), ctypes.byref(launch)))
        elif forward_only:
            self._fn = lib.vimscan_fwd
            self._args = (tuple(t.data_ptr() for t in (x, dt, z, B_f, C_f, A_f, D_f, dt_bias_f))
                          + (int(seg_len), out.data_ptr(), ctypes.byref(launch)))
        elif order is not None:
            self._fn = lib.vimscan_bidir_order_fwd
            self._args = (tuple(t.data_ptr() for t in ios + params)
                          + (int(seg_len), out.data_ptr(), ctypes.byref(launch)))
        elif cstruct is None:
            self._fn = lib.vimscan_bidir_fwd
            self._args = (tuple(t.data_ptr() for t in ios + params)
                          + (int(seg_len), out.data_ptr(), ctypes.byref(launch)))
        else:
            self._fn = lib.vimscan_bidir_conv_fwd
            self._args = ((x.data_ptr(), ctypes.byref(cstruct)) + tuple(t.data_ptr() for t in ios[1:] + params[:6])
                          + (int(seg_len), out.data_ptr(), ctypes.byref(launch)))

    def set_scan_events(self, ev0: int = 0, ev1: int = 0):
        """hipEvent_t handles (e.g. torch.cuda.Event(...).cuda_event, already created) that the
        following calls record just before and just after the main scan kernel; 0, 0 stops it."""
        self._launch.scan_events[0] = ev0 or None
        self._launch.scan_events[1] = ev1 or None

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def bidir_fwd_noalloc(x, dt, z, B_f, C_f, B_b, C_b, A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b, seg_len: int = 0,
                      out=None, chunk_len: int = 0, general_decay: bool = False):
    """bidir_fwd through vimscan_bidir_fwd_noalloc: the library takes its scratch from its static
    per-GPU array (at most NOALLOC_SCRATCH_BYTES) instead of a workspace. With ``out`` given the
    call allocates no device memory at all. Queued on torch's current stream; does not
    synchronise."""
    return PreparedCall(x, dt, z, B_f, C_f, B_b, C_b, A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b, seg_len, out,
                        chunk_len, general_decay, noalloc=True)()


def bidir_fwd(x, dt, z, B_f, C_f, B_b, C_b, A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b, seg_len: int = 0,
              out=None, chunk_len: int = 0, general_decay: bool = False, workspace=None, conv=None,
              aux_swap: bool = False, order=None):
    """y = silu(z) * (forward selective scan + backward selective scan), on the GPU.

    x, dt, z: (B, L, Di); B_*, C_*: (B, L, 16), all float32 or all bfloat16, contiguous, on one
    CUDA(HIP) device. A_*: (Di, 16); D_*, dt_bias_*: (Di,), float32. seg_len: 0, or the period of
    the state reset (must divide L). conv: None, or (w_f, bias_f, w_b, bias_b) float32 taps (Di, K)
    and biases (Di,) of the directional convolution + SiLU in front of each direction
    (vimscan_bidir_conv_fwd). order: None, or an int32 (B * L / T, T) tensor whose rows list each
    sequence's tokens in the order the forward path visits them (vimscan_bidir_order_fwd; T =
    seg_len or L). Returns y (B, L, Di) in x's dtype (``out`` if given).
    Queued on torch's current stream for x's device; does not synchronise."""
    return PreparedCall(x, dt, z, B_f, C_f, B_b, C_b, A_f, A_b, D_f, D_b, dt_bias_f, dt_bias_b, seg_len, out,
                        chunk_len, general_decay, workspace, conv=conv, aux_swap=aux_swap, order=order)()


def prepare_fwd(x, dt, z, B, C, A, D, dt_bias, seg_len: int = 0, out=None, chunk_len: int = 0,
                general_decay: bool = False, aux_swap: bool = False, workspace=None, stream=None) -> PreparedCall:
    """A prepared forward-only call (vimscan_fwd): x, dt, z (B, L, Di); B, C (B, L, 16); A (Di, 16);
    D, dt_bias (Di,). ``aux_swap`` exchanges each sequence's first and last output after the scan."""
    return PreparedCall(x, dt, z, B, C, B, C, A, A, D, D, dt_bias, dt_bias, seg_len, out, chunk_len, general_decay,
                        workspace, stream, aux_swap=aux_swap, forward_only=True)


def fwd(x, dt, z, B, C, A, D, dt_bias, seg_len: int = 0, out=None, chunk_len: int = 0, general_decay: bool = False,
        aux_swap: bool = False, workspace=None):
    """y = silu(z) * (C.h + D x) of the forward scan alone, on the GPU (vimscan_fwd); arguments as
    ``prepare_fwd``. Queued on torch's current stream; does not synchronise."""
    return prepare_fwd(x, dt, z, B, C, A, D, dt_bias, seg_len, out, chunk_len, general_decay, aux_swap, workspace)()


def ncssd_info(batch, seqlen, d_inner, d_state=16, seg_len=0, io_dtype="bf16", chunk_len=0) -> dict:
    """The library's plan for an NC-SSD call with this shape (host only; vimscan_ncssd_plan)."""
    code = VIMSCAN_BF16 if io_dtype == "bf16" else VIMSCAN_F32
    launch = make_launch(batch, seqlen, d_inner, d_state, code, chunk_len)
    plan = _Plan()
    _check(load_library().vimscan_ncssd_plan(ctypes.byref(launch), int(seg_len), ctypes.byref(plan)))
    return {f: getattr(plan, f) for f, _ in _Plan._fields_}


class PreparedNcssd:
    """A validated NC-SSD call on fixed tensors (vimscan_ncssd_fwd): y = C (B^T (x . m)) per
    sequence. x (B, L, Di); B, C (B, L, N) with N in {16, 32, 64}; x, B, C all float32 or all
    bfloat16, contiguous, on one device; m (B, L) float32. seg_len: 0, or the length of the folded
    sequences (must divide L). ``__call__`` only queues the kernels on the stream (torch's current
    stream for x's device unless given)."""

    def __init__(self, x, B, C, m, seg_len: int = 0, out=None, chunk_len: int = 0, workspace=None, stream=None):
        lib = load_library()
        if x.dim() != 3:
            raise ValueError("x must be (batch, seqlen, d_inner)")
        Bsz, L, Di = x.shape
        N = B.shape[-1] if B.dim() == 3 else -1
        dev = x.device
        if dev.type != "cuda":
            raise ValueError("inputs must be on a GPU device")
        io = _io_code(x.dtype)
        for t, shp in ((x, (Bsz, L, Di)), (B, (Bsz, L, N)), (C, (Bsz, L, N))):
            if t.device != dev or t.dtype != x.dtype or tuple(t.shape) != shp or not t.is_contiguous():
                raise ValueError("x (B,L,Di) and B, C (B,L,N) must share device and dtype and be contiguous")
        if m.device != dev or m.dtype != torch.float32 or tuple(m.shape) != (Bsz, L) or not m.is_contiguous():
            raise ValueError("m must be a contiguous float32 (B, L) tensor on x's device")
        if out is None:
            out = torch.empty_like(x)
        elif out.device != dev or out.dtype != x.dtype or out.shape != x.shape or not out.is_contiguous():
            raise ValueError("out must match x")
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        launch = make_launch(Bsz, L, Di, N, io, chunk_len, False, 0, 0, stream)
        plan = _Plan()
        _check(lib.vimscan_ncssd_plan(ctypes.byref(launch), int(seg_len), ctypes.byref(plan)))
        need = plan.workspace_bytes
        if need > 0:
            if workspace is None or workspace.numel() * workspace.element_size() < need:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            launch.workspace = workspace.data_ptr()
            launch.workspace_bytes = workspace.numel() * workspace.element_size()
        self.out = out
        self.plan = {f: getattr(plan, f) for f, _ in _Plan._fields_}
        self._keep = (x, B, C, m, out, workspace)
        self._launch = launch
        self._fn = lib.vimscan_ncssd_fwd
        self._args = (x.data_ptr(), B.data_ptr(), C.data_ptr(), m.data_ptr(), int(seg_len), out.data_ptr(),
                      ctypes.byref(launch))

    def set_scan_events(self, ev0: int = 0, ev1: int = 0):
        """hipEvent_t handles recorded before the first and after the last kernel of each call."""
        self._launch.scan_events[0] = ev0 or None
        self._launch.scan_events[1] = ev1 or None

    def __call__(self):
        _check(self._fn(*self._args))
        return self.out


def ncssd_fwd(x, B, C, m, seg_len: int = 0, out=None, chunk_len: int = 0, workspace=None):
    """NC-SSD global-state form y = C (B^T (x . m)) on the GPU (vimscan_ncssd_fwd); arguments as
    ``PreparedNcssd``. Queued on torch's current stream; does not synchronise."""
    return PreparedNcssd(x, B, C, m, seg_len, out, chunk_len, workspace)()
