"""MoE token dispatch / combine on one AMD MI355X: Python binding of libep.

The binding only marshals arguments: it checks dtypes, shapes and devices of
torch tensors, passes their device pointers and the current HIP stream to the
C ABI in include/ep.h, and turns a nonzero status into an exception.  Every
step of the computation runs in the HIP kernels of libep.so; there is no
Python or CPU fallback -- if libep.so cannot be loaded, calls raise.

Entry points (same names as the C ABI):
  ep_num_recv_rows(prob)                     -> R
  ep_layout_workspace_bytes(prob)            -> bytes
  ep_layout(prob, topk_idx, layout, workspace, stream=None)
  ep_dispatch(prob, x, layout, recv_x, recv_scales=None, stream=None)
  ep_layout_dispatch(prob, topk_idx, layout, workspace, x, recv_x, recv_scales=None,
                     stream=None)
  ep_layout_dispatch_noalloc(prob, topk_idx, layout, x, recv_x, recv_scales=None,
                             stream=None)   (workspace: the library's device array)
  ep_combine(prob, expert_out, layout, topk_weights, y, stream=None)
  ep_e4m3_encode(inp, out, stream=None)
  ep_strerror(code)

Helpers that allocate with torch (plumbing, outside the computation):
  Problem(...), Layout.empty(prob, device), alloc_workspace, alloc_recv.

Prepared calls (prepare_layout / prepare_dispatch / prepare_combine) check
and marshal the arguments once and return a callable that only issues the C
call, for loops that launch the same problem many times.
"""
import ctypes
import os

__all__ = [
    "Problem", "Layout", "EpError", "ep_num_recv_rows", "ep_layout_workspace_bytes",
    "ep_layout", "ep_dispatch", "ep_combine", "ep_e4m3_encode", "ep_strerror",
    "alloc_workspace", "alloc_recv", "library_path", "load_library",
    "prepare_layout", "prepare_dispatch", "prepare_combine", "ep_layout_dispatch",
    "prepare_layout_dispatch", "ep_layout_dispatch_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libep.so")
_lib = None

EP_OK, EP_ERR_ARG, EP_ERR_UNSUPPORTED, EP_ERR_ALIGN, EP_ERR_HIP = 0, -1, -2, -3, -4


class EpError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed with status {code}: {ep_strerror(code)}")
        self.code = code


class Problem(ctypes.Structure):
    """ep_problem: T, H, k, E, capacity (0 = contiguous), use_fp8 (0 bf16,
    1 E4M3FN + fp32 scales, 2 E4M3FN + UE8M0 scale bytes)."""
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("use_fp8", ctypes.c_int32)]

    def __init__(self, num_tokens, hidden, num_topk, num_experts, capacity=0, use_fp8=0):
        super().__init__(num_tokens, hidden, num_topk, num_experts, capacity, int(use_fp8))

    def __repr__(self):
        return (f"Problem(T={self.num_tokens}, H={self.hidden}, k={self.num_topk}, "
                f"E={self.num_experts}, cap={self.capacity}, fp8={self.use_fp8})")


class _LayoutPtrs(ctypes.Structure):
    _fields_ = [("count", ctypes.c_void_p), ("offset", ctypes.c_void_p),
                ("slot_of", ctypes.c_void_p), ("src_of_slot", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


def library_path():
    return _LIB_PATH


def load_library():
    """Load libep.so, building it first only if no build exists."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    # torch ships its own HIP runtime under the same soname; loading it first
    # makes libep bind to that runtime, so torch's streams and memory are ours.
    _torch()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Problem)
    L = ctypes.POINTER(_LayoutPtrs)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.ep_num_recv_rows.restype = i64
    lib.ep_num_recv_rows.argtypes = [P]
    lib.ep_layout_workspace_bytes.restype = i64
    lib.ep_layout_workspace_bytes.argtypes = [P]
    lib.ep_layout.restype = ctypes.c_int
    lib.ep_layout.argtypes = [P, vp, L, vp, ctypes.c_size_t, vp]
    lib.ep_dispatch.restype = ctypes.c_int
    lib.ep_dispatch.argtypes = [P, vp, L, vp, vp, vp]
    lib.ep_layout_dispatch.restype = ctypes.c_int
    lib.ep_layout_dispatch.argtypes = [P, vp, L, vp, ctypes.c_size_t, vp, vp, vp, vp]
    lib.ep_layout_dispatch_noalloc.restype = ctypes.c_int
    lib.ep_layout_dispatch_noalloc.argtypes = [P, vp, L, vp, vp, vp, vp]
    lib.ep_combine.restype = ctypes.c_int
    lib.ep_combine.argtypes = [P, vp, L, vp, vp, vp]
    lib.ep_e4m3_encode.restype = ctypes.c_int
    lib.ep_e4m3_encode.argtypes = [vp, vp, i64, vp]
    lib.ep_strerror.restype = ctypes.c_char_p
    lib.ep_strerror.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def ep_strerror(code):
    return load_library().ep_strerror(int(code)).decode()


def ep_num_recv_rows(prob):
    return int(load_library().ep_num_recv_rows(ctypes.byref(prob)))


def ep_layout_workspace_bytes(prob):
    return int(load_library().ep_layout_workspace_bytes(ctypes.byref(prob)))


def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be in GPU memory")
    return t.data_ptr() if t.numel() else None


class Layout:
    """Device tensors written by ep_layout (int32): count [E], offset [E+1],
    slot_of [T, k], src_of_slot [R], status [2]."""

    def __init__(self, count, offset, slot_of, src_of_slot, status):
        self.count, self.offset, self.slot_of = count, offset, slot_of
        self.src_of_slot, self.status = src_of_slot, status

    @classmethod
    def empty(cls, prob, device="cuda"):
        torch = _torch()
        i32 = torch.int32
        R = ep_num_recv_rows(prob)
        if R < 0:
            raise ValueError(f"invalid problem {prob!r}")
        return cls(torch.empty(prob.num_experts, dtype=i32, device=device),
                   torch.empty(prob.num_experts + 1, dtype=i32, device=device),
                   torch.empty((prob.num_tokens, prob.num_topk), dtype=i32, device=device),
                   torch.empty(R, dtype=i32, device=device),
                   torch.empty(2, dtype=i32, device=device))

    def _struct(self, prob, check_all=True):
        T, k, E = prob.num_tokens, prob.num_topk, prob.num_experts
        torch = _torch()
        s = _LayoutPtrs()
        s.slot_of = _ptr(self.slot_of, "slot_of", torch.int32, T * k, allow_none=True)
        if check_all:
            s.count = _ptr(self.count, "count", torch.int32, E)
            s.offset = _ptr(self.offset, "offset", torch.int32, E + 1)
            s.src_of_slot = _ptr(self.src_of_slot, "src_of_slot", torch.int32,
                                 ep_num_recv_rows(prob), allow_none=True)
            s.status = _ptr(self.status, "status", torch.int32, 2)
        return s


def alloc_workspace(prob, device="cuda"):
    torch = _torch()
    n = ep_layout_workspace_bytes(prob)
    if n < 0:
        raise ValueError(f"invalid problem {prob!r}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _scale_dtype(prob):
    """Block-scale element type: fp32 (use_fp8 = 1) or UE8M0 bytes (use_fp8 = 2)."""
    return _torch().uint8 if prob.use_fp8 == 2 else _torch().float32


def alloc_recv(prob, device="cuda"):
    """Receive buffers for dispatch: (recv_x, recv_scales or None)."""
    torch = _torch()
    R = ep_num_recv_rows(prob)
    if prob.use_fp8:
        return (torch.empty((R, prob.hidden), dtype=torch.uint8, device=device),
                torch.empty((R, prob.hidden // 128), dtype=_scale_dtype(prob), device=device))
    return torch.empty((R, prob.hidden), dtype=torch.bfloat16, device=device), None


def _check(fn, code):
    if code != EP_OK:
        raise EpError(fn, code)


def ep_layout(prob, topk_idx, layout, workspace, stream=None):
    torch = _torch()
    lib = load_library()
    idx = _ptr(topk_idx, "topk_idx", torch.int32, prob.num_tokens * prob.num_topk,
               allow_none=True)
    s = layout._struct(prob)
    ws = _ptr(workspace, "workspace", allow_none=True)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("ep_layout", lib.ep_layout(ctypes.byref(prob), idx, ctypes.byref(s), ws, nbytes,
                                      _stream_handle(stream)))


def ep_dispatch(prob, x, layout, recv_x, recv_scales=None, stream=None):
    torch = _torch()
    lib = load_library()
    T, H = prob.num_tokens, prob.hidden
    R = ep_num_recv_rows(prob)
    s = layout._struct(prob, check_all=False)
    xp = _ptr(x, "x", torch.bfloat16, T * H, allow_none=True)
    if prob.use_fp8:
        rp = _ptr(recv_x, "recv_x", (torch.uint8, torch.float8_e4m3fn), R * H, allow_none=True)
        sp = _ptr(recv_scales, "recv_scales", _scale_dtype(prob), R * (H // 128), allow_none=True)
    else:
        rp = _ptr(recv_x, "recv_x", torch.bfloat16, R * H, allow_none=True)
        sp = None
    _check("ep_dispatch", lib.ep_dispatch(ctypes.byref(prob), xp, ctypes.byref(s), rp, sp,
                                          _stream_handle(stream)))


def _layout_dispatch_args(prob, topk_idx, layout, workspace, x, recv_x, recv_scales):
    torch = _torch()
    T, H = prob.num_tokens, prob.hidden
    R = ep_num_recv_rows(prob)
    idx = _ptr(topk_idx, "topk_idx", torch.int32, T * prob.num_topk, allow_none=True)
    xp = _ptr(x, "x", torch.bfloat16, T * H, allow_none=True)
    s = layout._struct(prob)
    ws = _ptr(workspace, "workspace", allow_none=True)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if prob.use_fp8:
        rp = _ptr(recv_x, "recv_x", (torch.uint8, torch.float8_e4m3fn), R * H, allow_none=True)
        sp = _ptr(recv_scales, "recv_scales", _scale_dtype(prob), R * (H // 128), allow_none=True)
    else:
        rp = _ptr(recv_x, "recv_x", torch.bfloat16, R * H, allow_none=True)
        sp = None
    return s, (ctypes.byref(prob), idx, ctypes.byref(s), ws, nbytes, xp, rp, sp)


def ep_layout_dispatch(prob, topk_idx, layout, workspace, x, recv_x, recv_scales=None,
                       stream=None):
    lib = load_library()
    _s, args = _layout_dispatch_args(prob, topk_idx, layout, workspace, x, recv_x, recv_scales)
    _check("ep_layout_dispatch", lib.ep_layout_dispatch(*args, _stream_handle(stream)))


def ep_layout_dispatch_noalloc(prob, topk_idx, layout, x, recv_x, recv_scales=None,
                               stream=None):
    """ep_layout_dispatch with the library's own fixed device array as the
    workspace (nothing is allocated; calls that overlap on one GPU race)."""
    lib = load_library()
    _s, args = _layout_dispatch_args(prob, topk_idx, layout, None, x, recv_x, recv_scales)
    pr, idx, s, _ws, _nbytes, xp, rp, sp = args
    _check("ep_layout_dispatch_noalloc",
           lib.ep_layout_dispatch_noalloc(pr, idx, s, xp, rp, sp, _stream_handle(stream)))


def ep_combine(prob, expert_out, layout, topk_weights, y, stream=None):
    torch = _torch()
    lib = load_library()
    T, H, k = prob.num_tokens, prob.hidden, prob.num_topk
    R = ep_num_recv_rows(prob)
    s = layout._struct(prob, check_all=False)
    ep = _ptr(expert_out, "expert_out", torch.bfloat16, R * H, allow_none=True)
    wp = _ptr(topk_weights, "topk_weights", torch.float32, T * k, allow_none=True)
    yp = _ptr(y, "y", torch.bfloat16, T * H, allow_none=True)
    _check("ep_combine", lib.ep_combine(ctypes.byref(prob), ep, ctypes.byref(s), wp, yp,
                                        _stream_handle(stream)))


def ep_e4m3_encode(inp, out, stream=None):
    torch = _torch()
    lib = load_library()
    n = inp.numel()
    ip = _ptr(inp, "inp", torch.float32, allow_none=True)
    op = _ptr(out, "out", (torch.uint8, torch.float8_e4m3fn), n, allow_none=True)
    _check("ep_e4m3_encode", lib.ep_e4m3_encode(ip, op, n, _stream_handle(stream)))


class _Prepared:
    """A C-ABI call with its arguments checked and marshalled once.  Holds
    references to the tensors so their memory stays alive."""

    def __init__(self, name, fn, args, keep):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self, stream=None):
        _check(self.name, self._fn(*self._args, _stream_handle(stream)))


def prepare_layout(prob, topk_idx, layout, workspace):
    torch = _torch()
    lib = load_library()
    idx = _ptr(topk_idx, "topk_idx", torch.int32, prob.num_tokens * prob.num_topk,
               allow_none=True)
    s = layout._struct(prob)
    nbytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(prob), idx, ctypes.byref(s), _ptr(workspace, "workspace"), nbytes)
    return _Prepared("ep_layout", lib.ep_layout, args, (prob, s, topk_idx, layout, workspace))


def prepare_dispatch(prob, x, layout, recv_x, recv_scales=None):
    torch = _torch()
    lib = load_library()
    T, H = prob.num_tokens, prob.hidden
    R = ep_num_recv_rows(prob)
    xp = _ptr(x, "x", torch.bfloat16, T * H, allow_none=True)
    s = layout._struct(prob, check_all=False)
    if prob.use_fp8:
        rp = _ptr(recv_x, "recv_x", (torch.uint8, torch.float8_e4m3fn), R * H, allow_none=True)
        sp = _ptr(recv_scales, "recv_scales", _scale_dtype(prob), R * (H // 128), allow_none=True)
    else:
        rp = _ptr(recv_x, "recv_x", torch.bfloat16, R * H, allow_none=True)
        sp = None
    args = (ctypes.byref(prob), xp, ctypes.byref(s), rp, sp)
    return _Prepared("ep_dispatch", lib.ep_dispatch, args, (prob, s, x, layout, recv_x, recv_scales))


def prepare_combine(prob, expert_out, layout, topk_weights, y):
    torch = _torch()
    lib = load_library()
    T, H, k = prob.num_tokens, prob.hidden, prob.num_topk
    R = ep_num_recv_rows(prob)
    ep = _ptr(expert_out, "expert_out", torch.bfloat16, R * H, allow_none=True)
    wp = _ptr(topk_weights, "topk_weights", torch.float32, T * k, allow_none=True)
    yp = _ptr(y, "y", torch.bfloat16, T * H, allow_none=True)
    s = layout._struct(prob, check_all=False)
    args = (ctypes.byref(prob), ep, ctypes.byref(s), wp, yp)
    return _Prepared("ep_combine", lib.ep_combine, args,
                     (prob, s, expert_out, layout, topk_weights, y))


def prepare_layout_dispatch(prob, topk_idx, layout, workspace, x, recv_x, recv_scales=None):
    lib = load_library()
    s, args = _layout_dispatch_args(prob, topk_idx, layout, workspace, x, recv_x, recv_scales)
    return _Prepared("ep_layout_dispatch", lib.ep_layout_dispatch, args,
                     (prob, s, topk_idx, layout, workspace, x, recv_x, recv_scales))
