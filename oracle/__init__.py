"""Python access to the CPU oracle (liboracle.so, built from ep_oracle.cpp).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports or links it.

All arrays are numpy, C-contiguous:
  bf16 data travels as uint16 bit patterns, E4M3FN data as uint8 codes,
  routing ids / slots as int32, weights / scales as float32.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # compile on first use (g++ only, seconds)
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_bf16_round.restype = ctypes.c_uint16
    lib.orc_bf16_round.argtypes = [ctypes.c_float]
    lib.orc_bf16_to_float.restype = ctypes.c_float
    lib.orc_bf16_to_float.argtypes = [ctypes.c_uint16]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_bf16_round_array.restype = None
    lib.orc_bf16_round_array.argtypes = [_vp, _vp, _i64]
    lib.orc_e4m3_encode_array.restype = None
    lib.orc_e4m3_encode_array.argtypes = [_vp, _vp, _i64]
    lib.orc_layout.restype = ctypes.c_int
    lib.orc_layout.argtypes = [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.orc_dispatch.restype = ctypes.c_int
    lib.orc_dispatch.argtypes = [_i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]
    lib.orc_combine.restype = ctypes.c_int
    lib.orc_combine.argtypes = [_i32, _i32, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _need(a, dtype, shape=None):
    a = np.ascontiguousarray(a, dtype=dtype)
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a


# ---- codecs -----------------------------------------------------------------

def bf16_round(f32):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    f = _need(f32, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().orc_bf16_round_array(_ptr(f), _ptr(out), f.size)
    return out


def bf16_to_float(bits):
    """bf16 bit patterns -> fp32 (exact)."""
    b = _need(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def e4m3_encode(f32):
    """fp32 array -> OCP E4M3FN codes (uint8), RNE, saturating to +-448."""
    f = _need(f32, np.float32)
    out = np.empty(f.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(f), _ptr(out), f.size)
    return out


def e4m3_decode(code: int) -> float:
    return _load().orc_e4m3_decode(code)


def e4m3_decode_table():
    """float64 [256]: value of every code (NaN for 0x7F / 0xFF)."""
    lib = _load()
    return np.array([lib.orc_e4m3_decode(c) for c in range(256)], np.float64)


# ---- the method -------------------------------------------------------------

def num_recv_rows(T, k, E, cap):
    return T * k if cap == 0 else E * cap


def layout(topk_idx, E, cap=0):
    """Returns dict(count[E], offset[E+1], slot_of[T,k], src_of_slot[R], status[2])."""
    idx = _need(topk_idx, np.int32)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [T, k]")
    T, k = idx.shape
    R = num_recv_rows(T, k, E, cap)
    count = np.empty(E, np.int32)
    offset = np.empty(E + 1, np.int32)
    slot_of = np.empty((T, k), np.int32)
    src_of_slot = np.empty(R, np.int32)
    status = np.empty(2, np.int32)
    rc = _load().orc_layout(T, k, E, cap, _ptr(idx), _ptr(count), _ptr(offset), _ptr(slot_of),
                            _ptr(src_of_slot), _ptr(status))
    if rc != 0:
        raise ValueError("orc_layout rejected its arguments")
    return dict(count=count, offset=offset, slot_of=slot_of, src_of_slot=src_of_slot,
                status=status)


def _token_ranges(t0, t1, threads):
    n = t1 - t0
    parts = max(1, min(int(threads), n))
    cuts = [t0 + (n * i) // parts for i in range(parts + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(parts) if cuts[i + 1] > cuts[i]]


def _run_ranges(fn, t0, t1, threads):
    """Call fn(a, b) over a split of [t0, t1) into token ranges, in host
    threads (ctypes releases the GIL during the C call).  Every token is
    handled by exactly one call, and the oracle's per-token work does not
    depend on the split, so the result equals one serial call."""
    ranges = _token_ranges(t0, t1, threads)
    if len(ranges) <= 1:
        return [fn(t0, t1)]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(ranges)) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def dispatch(x_bf16, slot_of, R, use_fp8, recv_x=None, recv_scales=None, t0=0, t1=None,
             threads=1):
    """Scatter (and optionally quantise) token rows into receive rows.

    use_fp8: 0 bf16 rows; 1 E4M3FN rows + fp32 scales [R, H/128]; 2 E4M3FN rows
    + UE8M0 scale bytes [R, H/128].
    x_bf16 uint16 [T, H]; slot_of int32 [T, k].  recv_x / recv_scales may be
    passed pre-filled (rows no entry maps to keep their contents); otherwise
    they are created filled with 0xFF bytes.  Returns (recv_x, recv_scales).
    threads > 1 splits the tokens [t0, t1) over that many host threads (the
    receive rows of different tokens are disjoint, so the result is the same).
    """
    x = _need(x_bf16, np.uint16)
    s = _need(slot_of, np.int32)
    T, H = x.shape
    k = s.shape[1]
    t1 = T if t1 is None else t1
    mode = int(use_fp8)
    if mode not in (0, 1, 2):
        raise ValueError("use_fp8 must be 0 (bf16), 1 (fp32 scales) or 2 (UE8M0 scales)")
    if mode:
        if recv_x is None:
            recv_x = np.full((R, H), 0xFF, np.uint8)
        if recv_scales is None:
            recv_scales = (np.full((R, H // 128), -1, np.int32).view(np.float32) if mode == 1
                           else np.full((R, H // 128), 0xFF, np.uint8))
    else:
        if recv_x is None:
            recv_x = np.full((R, H), 0xFFFF, np.uint16)
    lib = _load()

    def part(a, b):
        return lib.orc_dispatch(T, H, k, R, mode, a, b, _ptr(x), _ptr(s),
                                _ptr(recv_x), _ptr(recv_scales) if mode else None)

    if any(rc != 0 for rc in _run_ranges(part, t0, t1, threads)):
        raise ValueError("orc_dispatch rejected its arguments")
    return recv_x, (recv_scales if use_fp8 else None)


def combine(expert_out_bf16, slot_of, topk_weights, t0=0, t1=None, want_acc=True, threads=1):
    """Weighted gather-reduce.  Returns (y uint16 [T, H], acc float32 [T, H] or None).

    Rows outside [t0, t1) of y / acc are left zero.  threads > 1 splits the
    tokens over that many host threads (each output row is one token's).
    """
    eo = _need(expert_out_bf16, np.uint16)
    s = _need(slot_of, np.int32)
    w = _need(topk_weights, np.float32, s.shape)
    R, H = eo.shape
    T, k = s.shape
    t1 = T if t1 is None else t1
    y = np.zeros((T, H), np.uint16)
    acc = np.zeros((T, H), np.float32) if want_acc else None
    lib = _load()

    def part(a, b):
        return lib.orc_combine(T, H, k, R, a, b, _ptr(eo), _ptr(s), _ptr(w), _ptr(y), _ptr(acc))

    if any(rc != 0 for rc in _run_ranges(part, t0, t1, threads)):
        raise ValueError("orc_combine rejected its arguments")
    return y, acc
