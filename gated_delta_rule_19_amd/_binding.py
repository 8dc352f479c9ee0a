"""ctypes binding of ``libgdn2.so`` (argument marshalling only).

Every computation runs in the library's gfx950 kernels; this module checks
tensor shapes/dtypes/devices, allocates outputs and workspace with torch, and
passes raw device pointers plus torch's current HIP stream to the C ABI
declared in ``include/gdn2.h``.  There is no fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn2.so")

ABI_VERSION = 8
GDN2_F32, GDN2_BF16 = 0, 1
FLAG_GATE_LOGITS, FLAG_NEG_EIGVAL, FLAG_QK_L2NORM = 1, 2, 4
CONV_SILU = 1
_STATUS = {0: "GDN2_OK", 1: "GDN2_ERR_NULL", 2: "GDN2_ERR_SHAPE", 3: "GDN2_ERR_DTYPE",
           4: "GDN2_ERR_ALIAS", 5: "GDN2_ERR_WORKSPACE", 6: "GDN2_ERR_DEVICE", 7: "GDN2_ERR_ALIGN"}
EXPORTED = ("gdn2_abi_version", "gdn2_status_str", "gdn2_chunk_fwd_workspace_size",
            "gdn2_chunk_fwd", "gdn2_chunk_prep", "gdn2_chunk_state", "gdn2_recurrent_step",
            "gdn2_gated_rmsnorm", "gdn2_chunk_fwd_varlen_workspace_size", "gdn2_chunk_fwd_varlen",
            "gdn2_recurrent_varlen", "gdn2_chunk_bwd_workspace_size", "gdn2_chunk_bwd",
            "gdn2_short_conv", "gdn2_short_conv_bwd_workspace_size", "gdn2_short_conv_bwd",
            "gdn2_chunk_bwd_varlen_workspace_size", "gdn2_chunk_bwd_varlen", "gdn2_chunk_fwd_noalloc",
            "gdn2_chunk_prep_workspace_size", "gdn2_recurrent_step_gated", "gdn2_chunk_fwd_conv",
            "gdn2_recurrent_step_conv")
NOALLOC_SCRATCH_BYTES = 64 << 20


class Problem(ctypes.Structure):
    """Mirror of ``gdn2_problem`` (include/gdn2.h)."""
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("chunk", ctypes.c_int32),
                ("io_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("Hv", ctypes.c_int64)]

    @property
    def value_heads(self) -> int:
        return self.Hv if self.Hv else self.H


class Conv(ctypes.Structure):
    """Mirror of ``gdn2_conv`` (include/gdn2.h): the short convolution fused into the prologue."""
    _fields_ = [("weight", ctypes.c_void_p), ("state_in", ctypes.c_void_p), ("state_out", ctypes.c_void_p),
                ("K", ctypes.c_int32), ("flags", ctypes.c_int32)]


class Gdn2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None


def lib():
    """Load ``libgdn2.so`` once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, P = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Problem)
        L.gdn2_abi_version.restype = ctypes.c_int
        L.gdn2_abi_version.argtypes = []
        L.gdn2_status_str.restype = ctypes.c_char_p
        L.gdn2_status_str.argtypes = [ctypes.c_int]
        L.gdn2_chunk_fwd_workspace_size.restype = sz
        L.gdn2_chunk_fwd_workspace_size.argtypes = [P]
        L.gdn2_chunk_prep_workspace_size.restype = sz
        L.gdn2_chunk_prep_workspace_size.argtypes = [P]
        L.gdn2_chunk_fwd.restype = ctypes.c_int
        L.gdn2_chunk_fwd.argtypes = [P] + [vp] * 9 + [vp, sz, vp]
        L.gdn2_chunk_fwd_noalloc.restype = ctypes.c_int
        L.gdn2_chunk_fwd_noalloc.argtypes = [P] + [vp] * 9 + [vp]
        L.gdn2_chunk_prep.restype = ctypes.c_int
        L.gdn2_chunk_prep.argtypes = [P] + [vp] * 6 + [vp, sz, vp]
        L.gdn2_chunk_state.restype = ctypes.c_int
        L.gdn2_chunk_state.argtypes = [P, vp, vp, vp, vp, sz, vp]
        L.gdn2_recurrent_step_gated.restype = ctypes.c_int
        L.gdn2_recurrent_step_gated.argtypes = [P] + [vp] * 11 + [vp]
        L.gdn2_recurrent_step.restype = ctypes.c_int
        L.gdn2_recurrent_step.argtypes = [P] + [vp] * 9 + [vp]
        CP = ctypes.POINTER(Conv)
        L.gdn2_chunk_fwd_conv.restype = ctypes.c_int
        L.gdn2_chunk_fwd_conv.argtypes = [P, CP] + [vp] * 9 + [vp, sz, vp]
        L.gdn2_recurrent_step_conv.restype = ctypes.c_int
        L.gdn2_recurrent_step_conv.argtypes = [P, CP] + [vp] * 9 + [vp]
        L.gdn2_gated_rmsnorm.restype = ctypes.c_int
        L.gdn2_gated_rmsnorm.argtypes = [P, vp, vp, vp, vp, vp]
        L.gdn2_chunk_fwd_varlen_workspace_size.restype = sz
        L.gdn2_chunk_fwd_varlen_workspace_size.argtypes = [P]
        L.gdn2_chunk_fwd_varlen.restype = ctypes.c_int
        L.gdn2_chunk_fwd_varlen.argtypes = [P, vp] + [vp] * 9 + [vp, sz, vp]
        L.gdn2_recurrent_varlen.restype = ctypes.c_int
        L.gdn2_recurrent_varlen.argtypes = [P, vp] + [vp] * 9 + [vp]
        L.gdn2_chunk_bwd_workspace_size.restype = sz
        L.gdn2_chunk_bwd_workspace_size.argtypes = [P]
        L.gdn2_chunk_bwd.restype = ctypes.c_int
        L.gdn2_chunk_bwd.argtypes = [P] + [vp] * 16 + [vp, sz, vp]
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.gdn2_short_conv.restype = ctypes.c_int
        L.gdn2_short_conv.argtypes = [i64] * 3 + [i32] * 3 + [vp] * 5 + [vp]
        L.gdn2_short_conv_bwd_workspace_size.restype = sz
        L.gdn2_short_conv_bwd_workspace_size.argtypes = [i64] * 3 + [i32]
        L.gdn2_short_conv_bwd.restype = ctypes.c_int
        L.gdn2_short_conv_bwd.argtypes = [i64] * 3 + [i32] * 3 + [vp] * 8 + [vp, sz, vp]
        L.gdn2_chunk_bwd_varlen_workspace_size.restype = sz
        L.gdn2_chunk_bwd_varlen_workspace_size.argtypes = [P]
        L.gdn2_chunk_bwd_varlen.restype = ctypes.c_int
        L.gdn2_chunk_bwd_varlen.argtypes = [P, vp] + [vp] * 16 + [vp, sz, vp]
        if L.gdn2_abi_version() != ABI_VERSION:   # the Problem mirror must match the library's struct
            raise ImportError(f"{LIB_PATH} has ABI {L.gdn2_abi_version()}, this binding expects {ABI_VERSION}: "
                              "rebuild it")
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().gdn2_abi_version())


def status_str(code: int) -> str:
    return lib().gdn2_status_str(int(code)).decode()


def _check(code: int):
    if code != 0:
        raise Gdn2Error(code, status_str(code))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def problem(B, T, H, dk, dv, io_dtype: torch.dtype, chunk: int = 64, gate_dtype: torch.dtype = torch.float32,
            flags: int = 0, Hv: int = 0) -> Problem:
    """H query/key heads; Hv value heads (0 = H), a multiple of H."""
    code = {torch.float32: GDN2_F32, torch.bfloat16: GDN2_BF16}
    return Problem(B, T, H, dk, dv, chunk, code.get(io_dtype, -1), code.get(gate_dtype, -1), int(flags), int(Hv))


def _problem_from(q, k, v, alpha, b, w, flags: int = 0) -> Tuple[Problem, torch.device]:
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q/k must be [B,T,H,dk], alpha/b [B,T,Hv,dk] and v/w [B,T,Hv,dv]")
    B, T, H, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if H == 0 and Hv != 0 or H != 0 and Hv % H != 0:
        raise ValueError(f"value heads ({Hv}) must be a multiple of query/key heads ({H})")
    for name, x, heads, last in (("k", k, H, dk), ("alpha", alpha, Hv, dk), ("b", b, Hv, dk), ("v", v, Hv, dv),
                                 ("w", w, Hv, dv)):
        if tuple(x.shape) != (B, T, heads, last):
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {(B, T, heads, last)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q, k, v must share one dtype: float32 or bfloat16")
    if not (alpha.dtype == b.dtype == w.dtype) or alpha.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("alpha, b, w must share one dtype: float32 or bfloat16")
    dev = q.device
    for name, x in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("b", b), ("w", w)):
        if x.device != dev or dev.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor on {dev}")
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return problem(B, T, H, dk, dv, q.dtype, gate_dtype=alpha.dtype, flags=flags, Hv=Hv), dev


def _check_state(S, p: Problem, dev, name):
    if S is None:
        return
    if tuple(S.shape) != (p.B, p.value_heads, p.dk, p.dv) or S.dtype != torch.float32:
        raise ValueError(f"{name} must be float32 [{p.B},{p.value_heads},{p.dk},{p.dv}]")
    if S.device != dev or not S.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {dev}")


def chunk_fwd_workspace_size(B, T, H, dk, dv, io_dtype: torch.dtype, Hv: int = 0) -> int:
    # the workspace size does not depend on the gate dtype or the flags
    return int(lib().gdn2_chunk_fwd_workspace_size(ctypes.byref(problem(B, T, H, dk, dv, io_dtype, Hv=Hv))))


def chunk_prep_workspace_size(B, T, H, dk, dv, io_dtype: torch.dtype, Hv: int = 0) -> int:
    """Workspace of the two stages ``chunk_prep`` / ``chunk_state`` (every shape)."""
    return int(lib().gdn2_chunk_prep_workspace_size(ctypes.byref(problem(B, T, H, dk, dv, io_dtype, Hv=Hv))))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def chunk_fwd(q, k, v, alpha, b, w, S0=None, *, out_state: bool = True, o=None, S_out=None,
              workspace=None, flags: int = 0):
    """Chunked forward (``gdn2_chunk_fwd``).  Returns (o, S_final or None).
    ``flags``: FLAG_* prologue options (gate logits, negative-eigenvalue b, q/k L2 norm)."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S0, p, dev, "S0")
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    need = int(lib().gdn2_chunk_fwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().gdn2_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                _ptr(S0), _ptr(o), _ptr(S_out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, S_out


def chunk_fwd_noalloc(q, k, v, alpha, b, w, S0=None, *, o, S_out=None, flags: int = 0):
    """Chunked forward with the library's own fixed workspace (``gdn2_chunk_fwd_noalloc``):
    the call allocates nothing, so the caller passes the outputs ``o`` (and ``S_out`` for
    the final state).  Returns (o, S_out)."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S0, p, dev, "S0")
    _check_state(S_out, p, dev, "S_out")
    if tuple(o.shape) != tuple(v.shape) or o.dtype != v.dtype or o.device != dev or not o.is_contiguous():
        raise ValueError("o must be a contiguous tensor shaped and typed like v")
    _check(lib().gdn2_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b),
                                        _ptr(w), _ptr(S0), _ptr(o), _ptr(S_out), _stream(dev)))
    return o, S_out


def chunk_prep(q, k, v, alpha, b, w, workspace, flags: int = 0):
    """First stage of the chunked forward (``gdn2_chunk_prep``): fills ``workspace``."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check(lib().gdn2_chunk_prep(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(dev)))


def chunk_state(p: Problem, workspace, o, S0=None, S_out=None):
    """Second stage of the chunked forward (``gdn2_chunk_state``): writes o (and S_out)."""
    dev = workspace.device
    _check_state(S0, p, dev, "S0")
    _check_state(S_out, p, dev, "S_out")
    _check(lib().gdn2_chunk_state(ctypes.byref(p), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(dev)))


def recurrent_step(q, k, v, alpha, b, w, S_in=None, *, o=None, S_out=None, out_state: bool = True,
                   inplace: bool = False, flags: int = 0):
    """Fused recurrent forward (``gdn2_recurrent_step``); T == 1 is one decode step.

    ``inplace=True`` writes the final state back into ``S_in``.
    Returns (o, S_final or None).
    """
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S_in, p, dev, "S_in")
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if inplace:
        if S_in is None:
            raise ValueError("inplace needs S_in")
        S_out = S_in
    elif S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    _check(lib().gdn2_recurrent_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                     _ptr(S_in), _ptr(o), _ptr(S_out), _stream(dev)))
    return o, S_out


def _conv_from(p: Problem, dev, weight, state, state_out, K, silu):
    """The fused convolution's descriptor; checks shapes ([C, K] fp32 taps, [B, K-1, C] windows
    in the I/O dtype, C = 2 H dk + Hv dv)."""
    C = 2 * p.H * p.dk + p.value_heads * p.dv
    K = int(weight.shape[1]) if K is None else int(K)
    if tuple(weight.shape) != (C, K) or weight.dtype != torch.float32 or weight.device != dev \
            or not weight.is_contiguous():
        raise ValueError(f"conv weight must be a contiguous float32 [{C}, {K}] tensor on {dev}")
    io = torch.bfloat16 if p.io_dtype == GDN2_BF16 else torch.float32
    for name, t in (("conv state", state), ("conv state_out", state_out)):
        if t is not None and (tuple(t.shape) != (p.B, K - 1, C) or t.dtype != io or t.device != dev
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [{p.B}, {K - 1}, {C}] {io} tensor on {dev}")
    return Conv(_ptr(weight), _ptr(state), _ptr(state_out), K, CONV_SILU if silu else 0)


def chunk_fwd_conv(q, k, v, alpha, b, w, conv_weight, conv_state=None, S0=None, *, conv_silu: bool = False,
                   want_conv_state: bool = True, conv_state_out=None, out_state: bool = True, o=None,
                   S_out=None, workspace=None, flags: int = 0):
    """Chunked forward with the short convolution fused into its prologue
    (``gdn2_chunk_fwd_conv``): equals :func:`short_conv` on the concatenated [q | k | v]
    followed by :func:`chunk_fwd` on the three parts.  ``conv_weight``: [C, K] float32,
    C = 2 H dk + Hv dv; ``conv_state``: [B, K-1, C] window before the first token (None =
    zeros); ``conv_state_out=conv_state`` updates it in place.
    Returns (o, S_final or None, conv window after the last token or None)."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S0, p, dev, "S0")
    K = int(conv_weight.shape[1])
    C = 2 * p.H * p.dk + p.value_heads * p.dv
    if conv_state_out is None and want_conv_state and K > 1:
        conv_state_out = torch.empty((p.B, K - 1, C), dtype=v.dtype, device=dev)
    cv = _conv_from(p, dev, conv_weight, conv_state, conv_state_out, K, conv_silu)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    need = int(lib().gdn2_chunk_fwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().gdn2_chunk_fwd_conv(ctypes.byref(p), ctypes.byref(cv), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                     _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, S_out, (conv_state_out if K > 1 else None)


def recurrent_step_conv(q, k, v, alpha, b, w, conv_weight, conv_state=None, S_in=None, *, conv_silu: bool = False,
                        want_conv_state: bool = True, conv_state_out=None, o=None, S_out=None,
                        out_state: bool = True, inplace: bool = False, flags: int = 0):
    """Recurrent forward with the short convolution fused (``gdn2_recurrent_step_conv``);
    T == 1 is the decode step with its window.  ``conv_state_out`` must be a different
    buffer from ``conv_state``.  Returns (o, S_final or None, window or None)."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S_in, p, dev, "S_in")
    K = int(conv_weight.shape[1])
    C = 2 * p.H * p.dk + p.value_heads * p.dv
    if conv_state_out is None and want_conv_state and K > 1:
        conv_state_out = torch.empty((p.B, K - 1, C), dtype=v.dtype, device=dev)
    cv = _conv_from(p, dev, conv_weight, conv_state, conv_state_out, K, conv_silu)
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if inplace:
        if S_in is None:
            raise ValueError("inplace needs S_in")
        S_out = S_in
    elif S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    _check(lib().gdn2_recurrent_step_conv(ctypes.byref(p), ctypes.byref(cv), _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(alpha), _ptr(b), _ptr(w), _ptr(S_in), _ptr(o), _ptr(S_out),
                                          _stream(dev)))
    return o, S_out, (conv_state_out if K > 1 else None)


def recurrent_step_gated(q, k, v, alpha, b, w, g, norm_weight, S_in=None, *, y=None, S_out=None,
                         out_state: bool = True, inplace: bool = False, flags: int = 0):
    """Recurrent forward with the output step fused (``gdn2_recurrent_step_gated``):
    returns (y, S_final or None), y = o / sqrt(mean(o^2) + 1e-5) * norm_weight * g * sigmoid(g)."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S_in, p, dev, "S_in")
    if tuple(g.shape) != tuple(v.shape) or g.dtype != v.dtype or g.device != dev or not g.is_contiguous():
        raise ValueError("g must be a contiguous tensor shaped and typed like v")
    if (tuple(norm_weight.shape) != (p.dv,) or norm_weight.dtype != torch.float32 or norm_weight.device != dev
            or not norm_weight.is_contiguous()):
        raise ValueError(f"norm_weight must be a contiguous float32 [{p.dv}] tensor on {dev}")
    if y is None:
        y = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if inplace:
        if S_in is None:
            raise ValueError("inplace needs S_in")
        S_out = S_in
    elif S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    _check(lib().gdn2_recurrent_step_gated(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b),
                                           _ptr(w), _ptr(S_in), _ptr(g), _ptr(norm_weight), _ptr(y), _ptr(S_out),
                                           _stream(dev)))
    return y, S_out


def _varlen_problem(q, k, v, alpha, b, w, cu_seqlens, flags):
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    if p.B != 1:
        raise ValueError("a packed batch is passed as [1, T, heads, d] tensors")
    if (not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1
            or cu_seqlens.numel() < 1 or cu_seqlens.device != dev or not cu_seqlens.is_contiguous()):
        raise ValueError(f"cu_seqlens must be a contiguous int32 [N+1] tensor on {dev}")
    p.B = cu_seqlens.numel() - 1
    return p, dev


def chunk_fwd_varlen_workspace_size(N, T, H, dk, dv, io_dtype: torch.dtype, Hv: int = 0) -> int:
    """Workspace bytes of ``chunk_fwd_varlen`` for N sequences of T packed tokens in all."""
    return int(lib().gdn2_chunk_fwd_varlen_workspace_size(ctypes.byref(problem(N, T, H, dk, dv, io_dtype, Hv=Hv))))


def chunk_fwd_varlen(q, k, v, alpha, b, w, cu_seqlens, S0=None, *, out_state: bool = True, o=None, S_out=None,
                     workspace=None, flags: int = 0):
    """Chunked forward over a packed batch (``gdn2_chunk_fwd_varlen``).

    q, k: [1, T, H, dk]; alpha, b: [1, T, Hv, dk]; v, w: [1, T, Hv, dv]; cu_seqlens: int32 [N+1]
    token offsets on the GPU (sequence i = tokens cu_seqlens[i] .. cu_seqlens[i+1]-1); S0:
    [N, Hv, dk, dv] or None.  Returns (o [1, T, Hv, dv], S_final [N, Hv, dk, dv] or None)."""
    p, dev = _varlen_problem(q, k, v, alpha, b, w, cu_seqlens, flags)
    _check_state(S0, p, dev, "S0")
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    need = int(lib().gdn2_chunk_fwd_varlen_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().gdn2_chunk_fwd_varlen(ctypes.byref(p), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(S_out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(dev)))
    return o, S_out


def recurrent_varlen(q, k, v, alpha, b, w, cu_seqlens, S_in=None, *, o=None, S_out=None, out_state: bool = True,
                     inplace: bool = False, flags: int = 0):
    """Fused recurrent forward over a packed batch (``gdn2_recurrent_varlen``); layouts as for
    ``chunk_fwd_varlen``.  ``inplace=True`` writes the final states back into ``S_in``."""
    p, dev = _varlen_problem(q, k, v, alpha, b, w, cu_seqlens, flags)
    _check_state(S_in, p, dev, "S_in")
    if o is None:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if inplace:
        if S_in is None:
            raise ValueError("inplace needs S_in")
        S_out = S_in
    elif S_out is None and out_state:
        S_out = torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
    _check_state(S_out, p, dev, "S_out")
    _check(lib().gdn2_recurrent_varlen(ctypes.byref(p), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(b), _ptr(w), _ptr(S_in), _ptr(o), _ptr(S_out), _stream(dev)))
    return o, S_out


def chunk_bwd_workspace_size(B, T, H, dk, dv, io_dtype: torch.dtype, gate_dtype: torch.dtype = torch.float32,
                             flags: int = 0, Hv: int = 0) -> int:
    p = problem(B, T, H, dk, dv, io_dtype, gate_dtype=gate_dtype, flags=flags, Hv=Hv)
    return int(lib().gdn2_chunk_bwd_workspace_size(ctypes.byref(p)))


def chunk_bwd(q, k, v, alpha, b, w, dO, S0=None, dS_T=None, *, want_dS0: bool = True, workspace=None,
              flags: int = 0):
    """Backward of the chunked forward (``gdn2_chunk_bwd``) with the same ``flags`` and
    head layout: gradients of sum(dO * o) + sum(dS_T * S_T) w.r.t. q, k, v, alpha, b, w
    (same shapes and dtypes as the inputs; of the logits with FLAG_GATE_LOGITS, of the raw
    q/k with FLAG_QK_L2NORM) and S0 (float32, when ``want_dS0``).  Returns a dict dq, dk,
    dv, dalpha, db, dw, dS0."""
    p, dev = _problem_from(q, k, v, alpha, b, w, flags)
    _check_state(S0, p, dev, "S0")
    _check_state(dS_T, p, dev, "dS_T")
    if tuple(dO.shape) != tuple(v.shape) or dO.dtype != v.dtype or dO.device != dev or not dO.is_contiguous():
        raise ValueError("dO must be a contiguous tensor like v")
    g = {n: torch.empty_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b),
                                            ("dw", w))}
    g["dS0"] = (torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
                if want_dS0 else None)
    need = int(lib().gdn2_chunk_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().gdn2_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0),
                                _ptr(dO), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]),
                                _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)))
    return g


def chunk_bwd_varlen_workspace_size(N, T, H, dk, dv, io_dtype: torch.dtype, Hv: int = 0, flags: int = 0,
                                    gate_dtype: torch.dtype = torch.float32) -> int:
    """Workspace bytes of ``chunk_bwd_varlen`` for N sequences of T packed tokens in all."""
    p = problem(N, T, H, dk, dv, io_dtype, gate_dtype=gate_dtype, flags=flags, Hv=Hv)
    return int(lib().gdn2_chunk_bwd_varlen_workspace_size(ctypes.byref(p)))


def chunk_bwd_varlen(q, k, v, alpha, b, w, dO, cu_seqlens, S0=None, dS_T=None, *, want_dS0: bool = True,
                     workspace=None, flags: int = 0):
    """Backward of :func:`chunk_fwd_varlen` (``gdn2_chunk_bwd_varlen``): tensors and the
    int32 [N+1] offsets on the GPU as there ([1, T, heads, d]), states [N, Hv, dk, dv].
    Returns a dict dq, dk, dv, dalpha, db, dw, dS0 as :func:`chunk_bwd`."""
    p, dev = _varlen_problem(q, k, v, alpha, b, w, cu_seqlens, flags)
    _check_state(S0, p, dev, "S0")
    _check_state(dS_T, p, dev, "dS_T")
    if tuple(dO.shape) != tuple(v.shape) or dO.dtype != v.dtype or dO.device != dev or not dO.is_contiguous():
        raise ValueError("dO must be a contiguous tensor like v")
    g = {n: torch.empty_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b),
                                            ("dw", w))}
    g["dS0"] = (torch.empty((p.B, p.value_heads, p.dk, p.dv), dtype=torch.float32, device=dev)
                if want_dS0 else None)
    need = int(lib().gdn2_chunk_bwd_varlen_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().gdn2_chunk_bwd_varlen(ctypes.byref(p), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                       _ptr(b), _ptr(w), _ptr(S0), _ptr(dO), _ptr(dS_T), _ptr(g["dq"]),
                                       _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]), _ptr(g["db"]), _ptr(g["dw"]),
                                       _ptr(g["dS0"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(dev)))
    return g


def gated_rmsnorm(o, g, weight, *, out=None, inplace: bool = False):
    """Output step (``gdn2_gated_rmsnorm``): y = o / sqrt(mean(o^2) + 1e-5) * weight * silu(g)
    per (token, head) row.  o, g: [B,T,H,dv] (float32 or bfloat16); weight: [dv] float32.
    ``inplace=True`` writes y over o.  Returns y."""
    if o.dim() != 4 or tuple(g.shape) != tuple(o.shape) or g.dtype != o.dtype:
        raise ValueError("o and g must be [B,T,H,dv] tensors of one dtype")
    if o.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("o must be float32 or bfloat16")
    B, T, H, dv = o.shape
    if tuple(weight.shape) != (dv,) or weight.dtype != torch.float32:
        raise ValueError(f"weight must be float32 [{dv}]")
    dev = o.device
    for name, x in (("o", o), ("g", g), ("weight", weight)):
        if x.device != dev or dev.type != "cuda" or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor on {dev}")
    y = o if inplace else (torch.empty_like(o) if out is None else out)
    # dk is not used by this call; 16 is any supported value
    p = problem(B, T, H, 16, dv, o.dtype)
    _check(lib().gdn2_gated_rmsnorm(ctypes.byref(p), _ptr(o), _ptr(g), _ptr(weight), _ptr(y), _stream(dev)))
    return y


def _conv_check(x, weight, state, what="x"):
    if x.dim() != 3:
        raise ValueError(f"{what} must be [B,T,C]")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"{what} must be float32 or bfloat16")
    B, T, C = x.shape
    if weight.dim() != 2 or weight.shape[0] != C or weight.dtype != torch.float32:
        raise ValueError(f"weight must be float32 [{C}, K]")
    K = weight.shape[1]
    if state is not None and (tuple(state.shape) != (B, K - 1, C) or state.dtype != x.dtype):
        raise ValueError(f"state must be [{B}, {K - 1}, {C}] of the dtype of {what}")
    dev = x.device
    for name, t in ((what, x), ("weight", weight), ("state", state)):
        if t is not None and (t.device != dev or dev.type != "cuda" or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor on {dev}")
    return B, T, C, K, dev, (GDN2_BF16 if x.dtype == torch.bfloat16 else GDN2_F32)


def short_conv(x, weight, state=None, *, silu: bool = False, want_state: bool = True, out=None,
               state_out=None):
    """Short convolution (``gdn2_short_conv``): causal depthwise over tokens,
    y[t] = sum_i weight[:, i] * xe[t - (K-1) + i] (then z * sigmoid(z) with ``silu``),
    xe reading ``state`` [B, K-1, C] before the first token (None = zeros).
    x: [B, T, C] float32 or bfloat16 (C a multiple of 8); weight: [C, K] float32, K <= 8.
    Returns (y, new state [B, K-1, C] or None); ``state_out=state`` updates it in place."""
    B, T, C, K, dev, code = _conv_check(x, weight, state)
    y = torch.empty_like(x) if out is None else out
    so = None
    if want_state:
        so = state_out if state_out is not None else torch.empty((B, K - 1, C), dtype=x.dtype, device=dev)
    _check(lib().gdn2_short_conv(B, T, C, K, CONV_SILU if silu else 0, code, _ptr(x), _ptr(weight), _ptr(state),
                                 _ptr(y), _ptr(so) if K > 1 else None, _stream(dev)))
    return y, so


def short_conv_bwd_workspace_size(B, T, C, K) -> int:
    return int(lib().gdn2_short_conv_bwd_workspace_size(B, T, C, K))


def short_conv_bwd(x, weight, dy, state=None, *, silu: bool = False, want_dstate: bool = True, workspace=None,
                   dstate_out=None):
    """Gradient of :func:`short_conv` (``gdn2_short_conv_bwd``) given dy = dL/dy and,
    optionally, dstate_out = dL/dstate_out [B, K-1, C] (the gradient of the window after
    the last token, e.g. the next piece's dstate).
    Returns (dx, dweight [C, K] float32, dstate [B, K-1, C] or None)."""
    B, T, C, K, dev, code = _conv_check(x, weight, state)
    if tuple(dy.shape) != (B, T, C) or dy.dtype != x.dtype or dy.device != dev or not dy.is_contiguous():
        raise ValueError("dy must be a contiguous GPU tensor shaped and typed like x")
    if dstate_out is not None and (tuple(dstate_out.shape) != (B, K - 1, C) or dstate_out.dtype != x.dtype
                                   or dstate_out.device != dev or not dstate_out.is_contiguous()):
        raise ValueError("dstate_out must be a contiguous [B, K-1, C] GPU tensor typed like x")
    dx = torch.empty_like(x)
    dw = torch.empty((C, K), dtype=torch.float32, device=dev)
    ds = torch.empty((B, K - 1, C), dtype=x.dtype, device=dev) if want_dstate else None
    need = short_conv_bwd_workspace_size(B, T, C, K)
    if workspace is None:
        workspace = alloc_workspace(need, dev)
    _check(lib().gdn2_short_conv_bwd(B, T, C, K, CONV_SILU if silu else 0, code, _ptr(x), _ptr(weight), _ptr(state),
                                     _ptr(dy), _ptr(dstate_out) if K > 1 else None, _ptr(dx), _ptr(dw),
                                     _ptr(ds) if K > 1 else None,
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev)))
    return dx, dw, ds
