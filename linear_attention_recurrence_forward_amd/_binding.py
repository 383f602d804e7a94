"""ctypes binding of libgdn.so (include/gdn.h).

Argument marshalling only: every step of the forward pass runs in the library's
HIP kernels. torch supplies device memory and the current HIP stream. If the
library is missing the calls raise; there is no other implementation to fall
back to.

The tensor checks here (device, dtype, contiguity, element counts) are the ones
the pages make on their buffers before encoding (mlx-native 0.21.1
src/ops/gated_delta_net_decode.rs, validate and
dispatch_gated_delta_net_decode_with_capture); raw pointers carry no such
information, so they cannot live in the C library.
"""

from __future__ import annotations

import ctypes
import os
import struct
import threading

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libgdn.so")

STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL_POINTER", 2: "GDN_ERR_ZERO_DIM",
    3: "GDN_ERR_ZERO_EXTENT", 4: "GDN_ERR_GQA_RATIO", 5: "GDN_ERR_UNSUPPORTED_DK",
    6: "GDN_ERR_RESERVED_NONZERO", 7: "GDN_ERR_SIZE_OVERFLOW", 8: "GDN_ERR_MISALIGNED",
    9: "GDN_ERR_ALIASING", 10: "GDN_ERR_LAUNCH", 11: "GDN_ERR_OPTION",
}
# Option bits of gdn_forward_ex.
OPT_BF16_IO = 1
OPT_NORMALIZE_K = 2
STATUS_CODE = {v: k for k, v in STATUS.items()}

EXPORTS = ("gdn_check_params", "gdn_forward", "gdn_forward_bf16", "gdn_forward_capture",
           "gdn_forward_ex", "gdn_rollback", "gdn_status_string")
IO_ARRAYS = ("q", "k", "v", "output")  # the arrays gdn_forward_bf16 takes in bf16


class GdnParams(ctypes.Structure):
    """The 9-word params block: d_k, d_v, n_k_heads, n_v_heads, n_tokens,
    n_seqs, two reserved zeros, q_scale_bits."""
    _fields_ = [(n, ctypes.c_uint32) for n in
                ("d_k", "d_v", "n_k_heads", "n_v_heads", "n_tokens", "n_seqs",
                 "reserved6", "reserved7", "q_scale_bits")]

    def counts(self) -> dict:
        """Element count of every array for these params."""
        ts = self.n_tokens * self.n_seqs
        state = self.d_k * self.d_v * self.n_v_heads * self.n_seqs
        return dict(q=self.d_k * self.n_k_heads * ts, k=self.d_k * self.n_k_heads * ts,
                    v=self.d_v * self.n_v_heads * ts, output=self.d_v * self.n_v_heads * ts,
                    g=self.n_v_heads * ts, beta=self.n_v_heads * ts,
                    state_in=state, state_out=state, state_capture=state * self.n_tokens)


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{where}: {self.name}: {gdn_status_string(status)}")


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return LIBRARY


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIBRARY):
                raise RuntimeError(
                    f"{LIBRARY} is not built; build it with "
                    "`python -m linear_attention_recurrence_forward_amd.build` "
                    "(or __graft_entry__.build())")
            lib = ctypes.CDLL(LIBRARY)
            fp, p = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(GdnParams)
            lib.gdn_check_params.argtypes = [p]
            lib.gdn_check_params.restype = ctypes.c_int
            lib.gdn_forward.argtypes = [fp] * 8 + [p, ctypes.c_void_p]
            lib.gdn_forward.restype = ctypes.c_int
            lib.gdn_forward_capture.argtypes = [fp] * 9 + [p, ctypes.c_void_p]
            lib.gdn_forward_capture.restype = ctypes.c_int
            vp = ctypes.c_void_p
            lib.gdn_forward_bf16.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, p, vp]
            lib.gdn_forward_bf16.restype = ctypes.c_int
            lib.gdn_forward_ex.argtypes = [vp, vp, vp, fp, fp, fp, vp, fp, fp, p,
                                           ctypes.c_uint32, vp]
            lib.gdn_forward_ex.restype = ctypes.c_int
            lib.gdn_rollback.argtypes = [fp, ctypes.POINTER(ctypes.c_uint32), fp, p,
                                         ctypes.c_void_p]
            lib.gdn_rollback.restype = ctypes.c_int
            lib.gdn_status_string.argtypes = [ctypes.c_int]
            lib.gdn_status_string.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def make_params(d_k, d_v, n_k_heads, n_v_heads, n_tokens, n_seqs, q_scale_bits=0,
                reserved6=0, reserved7=0) -> GdnParams:
    return GdnParams(d_k, d_v, n_k_heads, n_v_heads, n_tokens, n_seqs,
                     reserved6, reserved7, q_scale_bits & 0xFFFFFFFF)


def params_for(q: torch.Tensor, v: torch.Tensor, q_scale_bits: int = 0) -> GdnParams:
    """Params from torch-shaped q (S, T, H_k, D_k) and v (S, T, H_v, D_v)."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be (S, T, H_k, D_k) and v (S, T, H_v, D_v)")
    S, T, Hk, Dk = q.shape
    Sv, Tv, Hv, Dv = v.shape
    if (Sv, Tv) != (S, T):
        raise ValueError(f"q {tuple(q.shape)} and v {tuple(v.shape)} disagree on (S, T)")
    return make_params(Dk, Dv, Hk, Hv, T, S, q_scale_bits)


def gdn_check_params(params: GdnParams) -> int:
    """Status code of the host-only params check (0 = GDN_OK)."""
    return _load().gdn_check_params(ctypes.byref(params))


def gdn_status_string(status: int) -> str:
    return _load().gdn_status_string(int(status)).decode()


def _ptr(t):
    return ctypes.cast(ctypes.c_void_p(t.data_ptr()), ctypes.POINTER(ctypes.c_float))


def _check_tensors(where: str, params: GdnParams, tensors: dict, io=torch.float32):
    counts = params.counts()
    device = None
    for name, t in tensors.items():
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{where}: {name} must be a torch.Tensor")
        want = io if name in IO_ARRAYS else torch.float32
        if t.dtype != want:
            kind = "bf16" if want == torch.bfloat16 else "f32"
            raise ValueError(f"{where}: {name} must be {kind} (got {t.dtype})")
        if t.device.type != "cuda":
            raise ValueError(f"{where}: {name} must be on the GPU (got {t.device})")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{where}: {name} is on {t.device}, other arrays on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{where}: {name} must be contiguous")
        if name == "state_capture" and params.n_seqs == 1:
            # One sequence: a larger (preallocated) capture buffer is accepted and
            # only its first n_tokens slices are written; with several sequences
            # the per-sequence stride depends on n_tokens, so the size must match
            # (mlx-native 0.21.1, dispatch_gated_delta_net_decode_with_capture).
            if t.numel() < counts[name]:
                raise ValueError(f"{where}: {name} element count {t.numel()} < required "
                                 f"{counts[name]}")
        elif t.numel() != counts[name]:
            raise ValueError(f"{where}: {name} element count {t.numel()} != expected "
                             f"{counts[name]}")
    return device


def _stream_handle(device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def gdn_forward(q, k, v, g, beta, state_in, output, state_out, params: GdnParams,
                stream=None) -> None:
    """Enqueue one forward call (C: gdn_forward). Raises GdnError on a nonzero
    status; the call is asynchronous on `stream` (default: current stream)."""
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in, output=output,
                   state_out=state_out)
    lib = _load()
    st = lib.gdn_check_params(ctypes.byref(params))
    if st != 0:
        raise GdnError(st, "gdn_forward")
    device = _check_tensors("gdn_forward", params, tensors)
    st = lib.gdn_forward(*(_ptr(t) for t in tensors.values()), ctypes.byref(params),
                         _stream_handle(device, stream))
    if st != 0:
        raise GdnError(st, "gdn_forward")


def gdn_forward_capture(q, k, v, g, beta, state_in, output, state_out, state_capture,
                        params: GdnParams, stream=None) -> None:
    """Enqueue one forward call that also writes the per-token state
    (C: gdn_forward_capture). state_capture must hold exactly
    n_tokens * d_k * d_v * n_v_heads * n_seqs floats, or at least that many
    when n_seqs == 1 (only the first n_tokens slices are written)."""
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in, output=output,
                   state_out=state_out, state_capture=state_capture)
    lib = _load()
    st = lib.gdn_check_params(ctypes.byref(params))
    if st != 0:
        raise GdnError(st, "gdn_forward_capture")
    device = _check_tensors("gdn_forward_capture", params, tensors)
    st = lib.gdn_forward_capture(*(_ptr(t) for t in tensors.values()),
                                 ctypes.byref(params), _stream_handle(device, stream))
    if st != 0:
        raise GdnError(st, "gdn_forward_capture")


def gdn_forward_bf16(q, k, v, g, beta, state_in, output, state_out, state_capture,
                     params: GdnParams, stream=None) -> None:
    """Enqueue one forward call with bf16 q, k, v and output (C:
    gdn_forward_bf16); g, beta and the state stay f32. state_capture may be
    None."""
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in, output=output,
                   state_out=state_out)
    if state_capture is not None:
        tensors["state_capture"] = state_capture
    lib = _load()
    st = lib.gdn_check_params(ctypes.byref(params))
    if st != 0:
        raise GdnError(st, "gdn_forward_bf16")
    device = _check_tensors("gdn_forward_bf16", params, tensors, io=torch.bfloat16)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.gdn_forward_bf16(ptr(q), ptr(k), ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                              ptr(output), _ptr(state_out),
                              _ptr(state_capture) if state_capture is not None else None,
                              ctypes.byref(params), _stream_handle(device, stream))
    if st != 0:
        raise GdnError(st, "gdn_forward_bf16")


def gdn_forward_ex(q, k, v, g, beta, state_in, output, state_out, state_capture,
                   params: GdnParams, options: int, stream=None) -> None:
    """Enqueue one forward call with an options word (C: gdn_forward_ex):
    OPT_BF16_IO (q, k, v, output in bf16) and OPT_NORMALIZE_K (every key row
    used as k / sqrt(sum k^2 + 1e-6)). state_capture may be None."""
    tensors = dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in, output=output,
                   state_out=state_out)
    if state_capture is not None:
        tensors["state_capture"] = state_capture
    lib = _load()
    st = lib.gdn_check_params(ctypes.byref(params))
    if st != 0:
        raise GdnError(st, "gdn_forward_ex")
    if options & ~(OPT_BF16_IO | OPT_NORMALIZE_K):
        raise GdnError(STATUS_CODE["GDN_ERR_OPTION"], "gdn_forward_ex")
    io = torch.bfloat16 if options & OPT_BF16_IO else torch.float32
    device = _check_tensors("gdn_forward_ex", params, tensors, io=io)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = lib.gdn_forward_ex(ptr(q), ptr(k), ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
                            ptr(output), _ptr(state_out),
                            _ptr(state_capture) if state_capture is not None else None,
                            ctypes.byref(params), options, _stream_handle(device, stream))
    if st != 0:
        raise GdnError(st, "gdn_forward_ex")


def gdn_rollback(state_capture, accepted, state, params: GdnParams, stream=None) -> None:
    """Enqueue the accepted-prefix rollback (C: gdn_rollback): for each
    sequence s with accepted[s] < n_tokens, state[s] = state_capture[s,
    accepted[s]]. accepted is a device tensor of n_seqs int32/uint32."""
    lib = _load()
    st = lib.gdn_check_params(ctypes.byref(params))
    if st != 0:
        raise GdnError(st, "gdn_rollback")
    device = _check_tensors("gdn_rollback", params,
                            dict(state_capture=state_capture, state_out=state))
    if not isinstance(accepted, torch.Tensor) or accepted.dtype not in (torch.int32,
                                                                         torch.uint32):
        raise ValueError("gdn_rollback: accepted must be an int32 or uint32 tensor")
    if accepted.device != device or not accepted.is_contiguous():
        raise ValueError("gdn_rollback: accepted must be contiguous, on the state's device")
    if accepted.numel() != params.n_seqs:
        raise ValueError(f"gdn_rollback: accepted element count {accepted.numel()} != "
                         f"expected {params.n_seqs}")
    acc = ctypes.cast(ctypes.c_void_p(accepted.data_ptr()), ctypes.POINTER(ctypes.c_uint32))
    st = lib.gdn_rollback(_ptr(state_capture), acc, _ptr(state), ctypes.byref(params),
                          _stream_handle(device, stream))
    if st != 0:
        raise GdnError(st, "gdn_rollback")


def scale_bits(q_scale=None, q_scale_bits=None) -> int:
    """Params word 8 from a q_scale value or its bits (at most one of them):
    None for both means q is pre-scaled (bits 0). A value is stored as its
    binary32 bits; +0.0 has bits 0, which the params block reads as "no
    scale", so it is refused (mlx-native 0.21.1 src/ops/gated_delta_net_decode.rs,
    module doc "Buffer / params contract")."""
    if q_scale is not None and q_scale_bits is not None:
        raise ValueError("pass q_scale or q_scale_bits, not both")
    if q_scale is None:
        return 0 if q_scale_bits is None else int(q_scale_bits) & 0xFFFFFFFF
    bits = f32_bits(float(q_scale))
    if bits == 0:
        raise ValueError("q_scale=+0.0 cannot be expressed: bits 0 mean q is pre-scaled")
    return bits


def forward(q, k, v, g, beta, state_in, *, q_scale=None, q_scale_bits=None,
            capture: bool = False, normalize_k: bool = False, output=None, state_out=None,
            state_capture=None, stream=None):
    """Convenience wrapper on torch-shaped tensors:
    q, k (S, T, H_k, D_k); v (S, T, H_v, D_v); g, beta (S, T, H_v);
    state_in (S, H_v, D_v, D_k). q, k, v in f32, or all three in bf16 (then the
    output is bf16 too; the state is f32 either way). q_scale (a float) or
    q_scale_bits (its binary32 bits) folds a scale into every output; neither
    means q is pre-scaled. normalize_k: use every key row as
    k / sqrt(sum k^2 + 1e-6) (gdn_forward_ex). Allocates missing outputs and
    returns (output, state_out) or (output, state_out, state_capture)."""
    params = params_for(q, v, scale_bits(q_scale, q_scale_bits))
    S, T, Hv, Dv = v.shape
    Dk = q.shape[3]
    bf16 = q.dtype == torch.bfloat16
    if output is None:
        output = torch.empty((S, T, Hv, Dv), dtype=q.dtype if bf16 else torch.float32,
                             device=q.device)
    if state_out is None:
        state_out = torch.empty((S, Hv, Dv, Dk), dtype=torch.float32, device=q.device)
    if capture and state_capture is None:
        state_capture = torch.empty((S, T, Hv, Dv, Dk), dtype=torch.float32,
                                    device=q.device)
    if normalize_k:
        gdn_forward_ex(q, k, v, g, beta, state_in, output, state_out,
                       state_capture if capture else None, params,
                       OPT_NORMALIZE_K | (OPT_BF16_IO if bf16 else 0), stream)
        return (output, state_out, state_capture) if capture else (output, state_out)
    if bf16:
        gdn_forward_bf16(q, k, v, g, beta, state_in, output, state_out,
                         state_capture if capture else None, params, stream)
        return (output, state_out, state_capture) if capture else (output, state_out)
    if capture:
        gdn_forward_capture(q, k, v, g, beta, state_in, output, state_out, state_capture,
                            params, stream)
        return output, state_out, state_capture
    gdn_forward(q, k, v, g, beta, state_in, output, state_out, params, stream)
    return output, state_out
