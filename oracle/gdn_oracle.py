"""ctypes wrapper around the sequential C++ oracle (gdn_oracle.cpp).

TEST INFRASTRUCTURE ONLY (see the package docstring). Arrays are numpy, in the
torch-style row-major shapes that equal the pages' innermost-first layouts
(mlx-native 0.4.0 "src/ops/gated_delta_net.rs", module doc "Memory layouts"):

    q, k          (S, T, H_k, D_k)
    v             (S, T, H_v, D_v)
    g, beta       (S, T, H_v)
    state_in      (S, H_v, D_v, D_k)
    output        (S, T, H_v, D_v)
    state_capture (S, T, H_v, D_v, D_k)
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "gdn_oracle.cpp")
HEADER = os.path.join(HERE, "gdn_oracle.h")
LIBRARY = os.path.join(HERE, "liboracle_gdn.so")

HEAD_MAP_MOD = 0  # kh = vh % n_k_heads (capture kernel, mlx-native 0.9.2)
HEAD_MAP_DIV = 1  # kh = vh / (n_v_heads / n_k_heads) (mlx-native 0.4.0 doc)

# Plain IEEE arithmetic: no fused multiply-add, no fast-math reassociation.
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math"]

_lock = threading.Lock()
_libs: dict = {}


class _Shape(ctypes.Structure):
    _fields_ = [(name, ctypes.c_uint32) for name in
                ("d_k", "d_v", "n_k_heads", "n_v_heads", "n_tokens", "n_seqs",
                 "q_scale_bits")]


def build(force: bool = True) -> str:
    """Compile liboracle_gdn.so with g++ and return its path."""
    if force or not os.path.exists(LIBRARY) or (
            os.path.getmtime(LIBRARY) < max(os.path.getmtime(SOURCE),
                                            os.path.getmtime(HEADER))):
        tmp = LIBRARY + f".tmp{os.getpid()}"
        subprocess.run(["g++", *CXXFLAGS, SOURCE, "-o", tmp], check=True)
        os.replace(tmp, LIBRARY)
    return LIBRARY


def _load(path: str | None = None):
    """Load (once) the oracle library at path (default: the built one)."""
    with _lock:
        key = path or LIBRARY
        if key not in _libs:
            if path is None:
                build(force=False)
            lib = ctypes.CDLL(key)
            for name, real in (("oracle_gdn_forward_f32", ctypes.c_float),
                               ("oracle_gdn_forward_f64", ctypes.c_double)):
                fn = getattr(lib, name)
                fp = ctypes.POINTER(ctypes.c_float)
                rp = ctypes.POINTER(real)
                fn.argtypes = [fp] * 6 + [ctypes.POINTER(_Shape), ctypes.c_int,
                                          rp, rp, rp]
                fn.restype = ctypes.c_int
            for name, real in (("oracle_gdn_forward_ex_f32", ctypes.c_float),
                               ("oracle_gdn_forward_ex_f64", ctypes.c_double)):
                if hasattr(lib, name):
                    fn = getattr(lib, name)
                    fp = ctypes.POINTER(ctypes.c_float)
                    rp = ctypes.POINTER(real)
                    fn.argtypes = [fp] * 6 + [ctypes.POINTER(_Shape), ctypes.c_int,
                                              ctypes.c_uint32, rp, rp, rp]
                    fn.restype = ctypes.c_int
            if hasattr(lib, "oracle_gdn_forward_ex_bf16"):
                u16 = ctypes.POINTER(ctypes.c_uint16)
                fn = lib.oracle_gdn_forward_ex_bf16
                fn.argtypes = [u16, u16, u16] + [ctypes.POINTER(ctypes.c_float)] * 3 + [
                    ctypes.POINTER(_Shape), ctypes.c_int, ctypes.c_uint32, u16,
                    ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
                fn.restype = ctypes.c_int
            if hasattr(lib, "oracle_gdn_forward_bf16"):
                u16 = ctypes.POINTER(ctypes.c_uint16)
                fn = lib.oracle_gdn_forward_bf16
                fn.argtypes = [u16, u16, u16] + [ctypes.POINTER(ctypes.c_float)] * 3 + [
                    ctypes.POINTER(_Shape), ctypes.c_int, u16,
                    ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]
                fn.restype = ctypes.c_int
                lib.oracle_f32_to_bf16.argtypes = [ctypes.POINTER(ctypes.c_float), u16,
                                                   ctypes.c_uint64]
                lib.oracle_f32_to_bf16.restype = None
            for name, real in (("oracle_gdn_forward_range_f32", ctypes.c_float),
                               ("oracle_gdn_forward_range_f64", ctypes.c_double)):
                if hasattr(lib, name):
                    fn = getattr(lib, name)
                    fp = ctypes.POINTER(ctypes.c_float)
                    rp = ctypes.POINTER(real)
                    fn.argtypes = [fp] * 6 + [ctypes.POINTER(_Shape), ctypes.c_int,
                                              ctypes.c_uint64, ctypes.c_uint64, rp, rp, rp]
                    fn.restype = ctypes.c_int
            if hasattr(lib, "oracle_gdn_rollback"):
                fn = lib.oracle_gdn_rollback
                fn.argtypes = [ctypes.POINTER(ctypes.c_float),
                               ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(_Shape),
                               ctypes.POINTER(ctypes.c_float)]
                fn.restype = ctypes.c_int
            _libs[key] = lib
    return _libs[key]


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# Option bit of the oracle's _ex entry points: normalise every key row.
OPT_NORMALIZE_K = 2


def reference(q, k, v, g, beta, state_in, *, q_scale_bits: int = 0,
              head_map: int = HEAD_MAP_MOD, capture: bool = False,
              precision: str = "f32", normalize_k: bool = False,
              library: str | None = None):
    """Run the oracle. Returns (output, state_out) or (output, state_out, capture).

    Shapes are taken from the arrays: q is (S, T, H_k, D_k), v is (S, T, H_v, D_v).
    precision="f32" is the oracle proper; "f64" is the binary64 shadow.
    normalize_k replaces every key row by k / sqrt(sum k^2 + 1e-6) first.
    library selects another build of gdn_oracle.cpp (the planted-mistake
    tests use this); None means the regular build.
    """
    q, k, v, g, beta, state_in = (_f32(a) for a in (q, k, v, g, beta, state_in))
    S, T, Hk, Dk = q.shape
    Sv, Tv, Hv, Dv = v.shape
    if k.shape != q.shape or (Sv, Tv) != (S, T):
        raise ValueError("q, k, v disagree on (S, T) or q/k shapes differ")
    if g.shape != (S, T, Hv) or beta.shape != (S, T, Hv):
        raise ValueError("g and beta must be (S, T, H_v)")
    if state_in.shape != (S, Hv, Dv, Dk):
        raise ValueError("state_in must be (S, H_v, D_v, D_k)")

    real, dtype, fname = {
        "f32": (ctypes.c_float, np.float32, "oracle_gdn_forward_f32"),
        "f64": (ctypes.c_double, np.float64, "oracle_gdn_forward_f64"),
    }[precision]
    out = np.empty((S, T, Hv, Dv), dtype=dtype)
    st = np.empty((S, Hv, Dv, Dk), dtype=dtype)
    cap = np.empty((S, T, Hv, Dv, Dk), dtype=dtype) if capture else None
    shape = _Shape(Dk, Dv, Hk, Hv, T, S, q_scale_bits & 0xFFFFFFFF)
    fp = ctypes.c_float
    lib = _load(library)
    common = (_ptr(q, fp), _ptr(k, fp), _ptr(v, fp), _ptr(g, fp), _ptr(beta, fp),
              _ptr(state_in, fp), ctypes.byref(shape), head_map)
    outs = (_ptr(out, real), _ptr(st, real),
            _ptr(cap, real) if cap is not None else ctypes.POINTER(real)())
    if normalize_k:
        fname = fname.replace("oracle_gdn_forward_", "oracle_gdn_forward_ex_")
        rc = getattr(lib, fname)(*common, OPT_NORMALIZE_K, *outs)
    else:
        rc = getattr(lib, fname)(*common, *outs)
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return (out, st, cap) if capture else (out, st)


_pools: dict = {}


def _pool(threads: int):
    """A thread pool of the given size, kept for later calls (creating one per
    call would cost more than a short oracle call)."""
    from concurrent.futures import ThreadPoolExecutor
    with _lock:
        if threads not in _pools:
            _pools[threads] = ThreadPoolExecutor(max_workers=threads)
        return _pools[threads]


def _ranges(n: int, parts: int):
    """[begin, end) bounds of `parts` contiguous, nearly equal slices of n items."""
    parts = max(1, min(parts, n))
    return [(n * i // parts, n * (i + 1) // parts) for i in range(parts)]


def reference_threads(q, k, v, g, beta, state_in, *, threads: int, q_scale_bits: int = 0,
                      head_map: int = HEAD_MAP_MOD, capture: bool = False,
                      precision: str = "f32"):
    """The oracle (or its f64 shadow) with its independent (sequence, value
    head) pairs split into `threads` contiguous ranges that run concurrently
    (each range is one call of the same loop body; ctypes releases the GIL
    during a call). The result is reference(...)'s bit for bit. Used to time
    the oracle on all of a host's cores, and to check large GPU cases."""
    q, k, v, g, beta, state_in = (_f32(a) for a in (q, k, v, g, beta, state_in))
    S, T, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (S, T) or g.shape != (S, T, Hv) or \
            beta.shape != (S, T, Hv) or state_in.shape != (S, Hv, Dv, Dk):
        raise ValueError("inconsistent shapes (see reference)")
    real, dtype = {"f32": (ctypes.c_float, np.float32),
                   "f64": (ctypes.c_double, np.float64)}[precision]
    out = np.empty((S, T, Hv, Dv), dtype)
    st = np.empty((S, Hv, Dv, Dk), dtype)
    cap = np.empty((S, T, Hv, Dv, Dk), dtype) if capture else None
    shape = _Shape(Dk, Dv, Hk, Hv, T, S, q_scale_bits & 0xFFFFFFFF)
    fp = ctypes.c_float
    fn = getattr(_load(), f"oracle_gdn_forward_range_{precision}")
    args = (_ptr(q, fp), _ptr(k, fp), _ptr(v, fp), _ptr(g, fp), _ptr(beta, fp),
            _ptr(state_in, fp), ctypes.byref(shape), head_map)
    outs = (_ptr(out, real), _ptr(st, real), _ptr(cap, real) if cap is not None else
            ctypes.POINTER(real)())
    ranges = _ranges(S * Hv, threads)
    rcs = list(_pool(len(ranges)).map(lambda r: fn(*args, r[0], r[1], *outs), ranges))
    if any(rcs):
        raise ValueError(f"oracle rejected the inputs (codes {rcs})")
    return (out, st, cap) if capture else (out, st)


def rollback_threads(state_capture, accepted, state, *, threads: int):
    """rollback(...) with the sequences split into `threads` contiguous ranges
    copied concurrently; the same result bit for bit."""
    cap = _f32(state_capture)
    S, T, Hv, Dv, Dk = cap.shape
    out = np.array(state, dtype=np.float32, copy=True, order="C")
    acc = np.ascontiguousarray(accepted, dtype=np.uint32)
    if out.shape != (S, Hv, Dv, Dk) or acc.shape != (S,):
        raise ValueError("inconsistent shapes (see rollback)")
    lib = _load()
    u32 = ctypes.POINTER(ctypes.c_uint32)

    def part(r):
        s0, s1 = r
        shape = _Shape(Dk, Dv, 1, Hv, T, s1 - s0, 0)
        return lib.oracle_gdn_rollback(_ptr(cap[s0:s1], ctypes.c_float),
                                       acc[s0:s1].ctypes.data_as(u32), ctypes.byref(shape),
                                       _ptr(out[s0:s1], ctypes.c_float))
    ranges = _ranges(S, threads)
    rcs = list(_pool(len(ranges)).map(part, ranges))
    if any(rcs):
        raise ValueError(f"oracle rejected the inputs (codes {rcs})")
    return out


def rollback(state_capture, accepted, state, *, library: str | None = None):
    """Accepted-prefix rollback: returns a copy of state (S, H_v, D_v, D_k) with
    sequence s replaced by state_capture[s, accepted[s]] when accepted[s] < T.
    state_capture is (S, T, H_v, D_v, D_k)."""
    cap = _f32(state_capture)
    S, T, Hv, Dv, Dk = cap.shape
    out = np.array(state, dtype=np.float32, copy=True, order="C")
    if out.shape != (S, Hv, Dv, Dk):
        raise ValueError("state must be (S, H_v, D_v, D_k) matching the capture")
    acc = np.ascontiguousarray(accepted, dtype=np.uint32)
    if acc.shape != (S,):
        raise ValueError("accepted must hold one index per sequence")
    shape = _Shape(Dk, Dv, 1, Hv, T, S, 0)
    rc = _load(library).oracle_gdn_rollback(
        _ptr(cap, ctypes.c_float), acc.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
        ctypes.byref(shape), _ptr(out, ctypes.c_float))
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return out


def to_bf16(x, *, library: str | None = None):
    """The oracle's f32 -> bf16 rounding: uint16 bit patterns of x's elements."""
    a = _f32(x)
    out = np.empty(a.shape, np.uint16)
    _load(library).oracle_f32_to_bf16(_ptr(a, ctypes.c_float),
                                      out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                      a.size)
    return out


def reference_bf16(q, k, v, g, beta, state_in, *, q_scale_bits: int = 0,
                   head_map: int = HEAD_MAP_MOD, capture: bool = False,
                   normalize_k: bool = False, library: str | None = None):
    """bf16 variant: q, k, v are uint16 bf16 bit patterns (shapes as in
    reference); returns (output as uint16 bf16 bits, state_out f32[, capture])."""
    q16, k16, v16 = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v))
    g, beta, state_in = (_f32(a) for a in (g, beta, state_in))
    S, T, Hk, Dk = q16.shape
    Hv, Dv = v16.shape[2], v16.shape[3]
    out = np.empty((S, T, Hv, Dv), np.uint16)
    st = np.empty((S, Hv, Dv, Dk), np.float32)
    cap = np.empty((S, T, Hv, Dv, Dk), np.float32) if capture else None
    shape = _Shape(Dk, Dv, Hk, Hv, T, S, q_scale_bits & 0xFFFFFFFF)
    u16 = ctypes.POINTER(ctypes.c_uint16)
    fp = ctypes.c_float
    rc = _load(library).oracle_gdn_forward_ex_bf16(
        q16.ctypes.data_as(u16), k16.ctypes.data_as(u16), v16.ctypes.data_as(u16),
        _ptr(g, fp), _ptr(beta, fp), _ptr(state_in, fp), ctypes.byref(shape), head_map,
        OPT_NORMALIZE_K if normalize_k else 0,
        out.ctypes.data_as(u16), _ptr(st, fp),
        _ptr(cap, fp) if cap is not None else ctypes.POINTER(fp)())
    if rc != 0:
        raise ValueError(f"oracle rejected the inputs (code {rc})")
    return (out, st, cap) if capture else (out, st)
