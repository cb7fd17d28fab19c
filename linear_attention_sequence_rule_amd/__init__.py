"""Gated DeltaNet gated delta rule on AMD Instinct MI355X (gfx950): Python binding of libgdn.so.

The functions here carry the names of the C ABI (``include/gdn.h``) and only marshal arguments:
they check tensor placement and dtypes, allocate outputs with torch (memory only), and pass raw
device pointers and the current HIP stream to the library.  Every step of the computation runs
in the library's HIP kernels; there is no CPU or PyTorch fallback.  If ``libgdn.so`` has not
been built (``__graft_entry__.build()``) every call raises.

    o, final_state = gdn_chunk_fwd(q, k, v, g, beta, initial_state, cu_seqlens)
    o = gdn_recurrent_step(q, k, v, g, beta, state)          # state updated in place
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = ["gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_recurrent_step", "gdn_status_string",
           "gdn_chunk_workspace_size", "GdnError", "lib_path", "load_library", "GDN_OK", "GDN_ERR_INVALID_ARG",
           "GDN_ERR_UNSUPPORTED", "GDN_ERR_WORKSPACE", "GDN_ERR_HIP", "GDN_ERR_SCRATCH", "GDN_F32", "GDN_BF16",
           "GDN_QK_L2NORM", "GDN_SEGMENTS", "GDN_CONV_FUSED", "GDN_NOALLOC_SCRATCH_BYTES"]

GDN_OK, GDN_ERR_INVALID_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP, GDN_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20
GDN_F32, GDN_BF16 = 0, 1
GDN_QK_L2NORM = 1
GDN_CONV_FUSED = 1 << 16


def GDN_SEGMENTS(n: int) -> int:
    """Flag bits requesting n segments per sequence (0 = automatic)."""
    return (int(n) & 0xFF) << 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdn.so")
_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s returned %s" % (where, gdn_status_string(status)))


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdn.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build() first" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, U, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float
    lib.gdn_chunk_fwd.restype = I
    lib.gdn_chunk_fwd.argtypes = [P] * 16 + [I] * 8 + [F, F, U, P]
    lib.gdn_chunk_fwd_noalloc.restype = I
    lib.gdn_chunk_fwd_noalloc.argtypes = [P] * 14 + [I] * 8 + [F, F, U, P]
    lib.gdn_chunk_workspace_size.restype = I
    lib.gdn_chunk_workspace_size.argtypes = [I] * 10 + [U, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdn_recurrent_step.restype = I
    lib.gdn_recurrent_step.argtypes = [P] * 12 + [I] * 6 + [F, F, U, P]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [I]
    _lib = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load_library().gdn_status_string(int(status)).decode()


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _check_dev(name, t, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _check_shape(name, t, shape):
    """Raise ValueError unless tensor t (when given) has exactly this shape: the C ABI cannot see
    device buffer sizes, so a short buffer would be read or written out of bounds."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(int(x) for x in shape), tuple(t.shape)))


def _check_rank(name, t, rank):
    if t.dim() != rank:
        raise ValueError("%s must have %d dimensions, got shape %s" % (name, rank, tuple(t.shape)))


def gdn_chunk_workspace_size(N, T_tot, H, dk, dv, dtype=GDN_BF16, chunk=64, has_cu_seqlens=False, has_conv=False,
                             flags=GDN_QK_L2NORM, Hk=None) -> int:
    n = ctypes.c_size_t(0)
    Hk = H if Hk is None else Hk
    st = load_library().gdn_chunk_workspace_size(N, T_tot, H, Hk, dk, dv, dtype, chunk, int(bool(has_cu_seqlens)),
                                                 int(bool(has_conv)), flags, ctypes.byref(n))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_workspace_size")
    return int(n.value)


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, conv_w=None, *, N=None, o=None,
                  final_state=None, output_final_state=True, scale=1.0, l2norm=True, chunk=64, workspace=None,
                  segments=0, gate_params=None, conv_state=None, out_gate=None, norm_weight=None, norm_eps=1e-3,
                  conv_fused=False, stream=None):
    """Chunked prefill.  q, k [T_tot, Hk, dk]; v [T_tot, H, dv] (bf16 or fp32; H a multiple of Hk, value
    head h reads query/key head h // (H // Hk)); g, beta [T_tot, H] fp32 (the raw a and b when
    gate_params [2, H] = (A_log, dt_bias) is given); initial_state [N, H, dv, dk] fp32 or None;
    cu_seqlens [N+1] int32 or None (N equal sequences, N given or 1); conv_w [C, 4] fp32 or None,
    C = 2*Hk*dk + H*dv; conv_state [N, 3, C] in the dtype of q, read as the conv history and
    updated in place, or None; segments per sequence (0 = automatic); out_gate [T_tot, H, dv] (dtype
    of q) with norm_weight [dv] fp32: the output epilogue o * rsqrt(mean(o^2) + norm_eps) * (1 + w) *
    sigmoid(z) (norm_eps default 1e-3, the value the pages suggest for bf16).
    A workspace (uint8 device tensor) is allocated here when the call needs one and none large
    enough is given.  Returns (o, final_state or None)."""
    import torch
    _check_rank("q", q, 3)
    _check_rank("v", v, 3)
    T_tot, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _check_rank("cu_seqlens", cu_seqlens, 1)
        N = cu_seqlens.shape[0] - 1
    elif N is None:
        N = initial_state.shape[0] if initial_state is not None else 1
    # every shape against the header's, before anything reaches the library
    _check_shape("k", k, (T_tot, Hk, dk))
    _check_shape("v", v, (T_tot, H, dv))
    _check_shape("g", g, (T_tot, H))
    _check_shape("beta", beta, (T_tot, H))
    _check_shape("gate_params", gate_params, (2, H))
    _check_shape("initial_state", initial_state, (N, H, dv, dk))
    _check_shape("final_state", final_state, (N, H, dv, dk))
    _check_shape("o", o, (T_tot, H, dv))
    cc = 2 * Hk * dk + H * dv
    _check_shape("conv_w", conv_w, (cc, 4))
    _check_shape("conv_state", conv_state, (N, 3, cc))
    _check_shape("out_gate", out_gate, (T_tot, H, dv))
    _check_shape("norm_weight", norm_weight, (dv,))
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("conv_state", conv_state), ("out_gate", out_gate)):
        _check_dev(name, t, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("gate_params", gate_params), ("initial_state", initial_state),
                    ("conv_w", conv_w), ("final_state", final_state), ("norm_weight", norm_weight)):
        _check_dev(name, t, torch.float32)
    _check_dev("cu_seqlens", cu_seqlens, torch.int32)
    if o is None:
        o = torch.empty((T_tot, H, dv), dtype=q.dtype, device=q.device)
    _check_dev("o", o, q.dtype)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    flags = (GDN_QK_L2NORM if l2norm else 0) | GDN_SEGMENTS(segments) | (GDN_CONV_FUSED if conv_fused else 0)
    ws_bytes = ctypes.c_size_t(0 if workspace is None else workspace.numel() * workspace.element_size())
    need = gdn_chunk_workspace_size(N, T_tot, H, dk, dv, dt, chunk, cu_seqlens is not None, conv_w is not None, flags,
                                    Hk=Hk)
    if need > ws_bytes.value:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = ctypes.c_size_t(need)
    st = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate_params), _ptr(initial_state),
                           _ptr(cu_seqlens), _ptr(conv_w), _ptr(conv_state), _ptr(out_gate), _ptr(norm_weight),
                           _ptr(o), _ptr(final_state), _ptr(workspace), ctypes.byref(ws_bytes), N, T_tot, H, Hk, dk,
                           dv, dt, chunk, float(scale), float(norm_eps), flags, _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, initial_state, cu_seqlens, conv_w, *, o, final_state, N=None,
                          scale=1.0, l2norm=True, chunk=64, segments=0, gate_params=None, conv_state=None,
                          out_gate=None, norm_weight=None, norm_eps=1e-3, conv_fused=False, stream=None):
    """gdn_chunk_fwd through the entry point that allocates nothing: the workspace is the library's
    static device scratch.  The outputs o [T_tot, H, dv] and final_state [N, H, dv, dk] (or None) are
    the caller's; this wrapper allocates nothing either.  Arguments otherwise as gdn_chunk_fwd."""
    import torch
    _check_rank("q", q, 3)
    _check_rank("v", v, 3)
    T_tot, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    if cu_seqlens is not None:
        _check_rank("cu_seqlens", cu_seqlens, 1)
        N = cu_seqlens.shape[0] - 1
    elif N is None:
        N = initial_state.shape[0] if initial_state is not None else 1
    _check_shape("k", k, (T_tot, Hk, dk))
    _check_shape("v", v, (T_tot, H, dv))
    _check_shape("g", g, (T_tot, H))
    _check_shape("beta", beta, (T_tot, H))
    _check_shape("gate_params", gate_params, (2, H))
    _check_shape("initial_state", initial_state, (N, H, dv, dk))
    _check_shape("final_state", final_state, (N, H, dv, dk))
    _check_shape("o", o, (T_tot, H, dv))
    cc = 2 * Hk * dk + H * dv
    _check_shape("conv_w", conv_w, (cc, 4))
    _check_shape("conv_state", conv_state, (N, 3, cc))
    _check_shape("out_gate", out_gate, (T_tot, H, dv))
    _check_shape("norm_weight", norm_weight, (dv,))
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("conv_state", conv_state), ("out_gate", out_gate), ("o", o)):
        _check_dev(name, t, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("gate_params", gate_params), ("initial_state", initial_state),
                    ("conv_w", conv_w), ("final_state", final_state), ("norm_weight", norm_weight)):
        _check_dev(name, t, torch.float32)
    _check_dev("cu_seqlens", cu_seqlens, torch.int32)
    flags = (GDN_QK_L2NORM if l2norm else 0) | GDN_SEGMENTS(segments) | (GDN_CONV_FUSED if conv_fused else 0)
    st = lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate_params),
                                   _ptr(initial_state), _ptr(cu_seqlens), _ptr(conv_w), _ptr(conv_state),
                                   _ptr(out_gate), _ptr(norm_weight), _ptr(o), _ptr(final_state), N, T_tot, H, Hk,
                                   dk, dv, dt, chunk, float(scale), float(norm_eps), flags, _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_chunk_fwd_noalloc")
    return o, final_state


def gdn_recurrent_step(q, k, v, g, beta, state, *, o=None, scale=1.0, l2norm=True, gate_params=None, conv_w=None,
                       conv_state=None, out_gate=None, norm_weight=None, norm_eps=1e-3, stream=None):
    """One decode token per sequence.  q, k [N, Hk, dk]; v [N, H, dv]; g, beta [N, H] fp32 (the raw a
    and b when gate_params [2, H] is given); state [N, H, dv, dk] fp32, updated in place; conv_w
    [C, 4] fp32 with conv_state [N, 3, C] (C = 2*Hk*dk + H*dv; dtype of q, updated in place), or
    neither; out_gate [N, H, dv] with norm_weight [dv]: the output epilogue, as for gdn_chunk_fwd.
    Returns o [N, H, dv]."""
    import torch
    _check_rank("q", q, 3)
    _check_rank("v", v, 3)
    N, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    _check_shape("k", k, (N, Hk, dk))
    _check_shape("v", v, (N, H, dv))
    _check_shape("g", g, (N, H))
    _check_shape("beta", beta, (N, H))
    _check_shape("gate_params", gate_params, (2, H))
    _check_shape("state", state, (N, H, dv, dk))
    _check_shape("o", o, (N, H, dv))
    cc = 2 * Hk * dk + H * dv
    _check_shape("conv_w", conv_w, (cc, 4))
    _check_shape("conv_state", conv_state, (N, 3, cc))
    _check_shape("out_gate", out_gate, (N, H, dv))
    _check_shape("norm_weight", norm_weight, (dv,))
    lib = load_library()
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("conv_state", conv_state), ("out_gate", out_gate)):
        _check_dev(name, t, q.dtype)
    for name, t in (("g", g), ("beta", beta), ("gate_params", gate_params), ("state", state), ("conv_w", conv_w),
                    ("norm_weight", norm_weight)):
        _check_dev(name, t, torch.float32)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check_dev("o", o, q.dtype)
    st = lib.gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate_params), _ptr(state),
                                _ptr(conv_w), _ptr(conv_state), _ptr(out_gate), _ptr(norm_weight), _ptr(o), N, H, Hk,
                                dk, dv, dt, float(scale), float(norm_eps), GDN_QK_L2NORM if l2norm else 0,
                                _stream(stream))
    if st != GDN_OK:
        raise GdnError(st, "gdn_recurrent_step")
    return o
