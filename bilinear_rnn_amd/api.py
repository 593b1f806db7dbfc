"""Thin ctypes binding of libcomba.so (the C ABI in include/comba.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
layout, outputs and the workspace are allocated with torch, and the call is
enqueued on torch's current stream. Every step of the computation runs in
the HIP kernels of libcomba.so; there is no fallback path. If the library is
missing, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

# COMBA_LIBRARY names another build of the same library (the host-sanitizer build of
# the CPU checks); by default the in-tree libcomba.so.
_LIB_PATH = os.environ.get("COMBA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcomba.so")
_lib = None

COMBA_OK = 0
COMBA_ERR_INVALID_ARG = -1
COMBA_ERR_UNSUPPORTED = -2
COMBA_ERR_WORKSPACE = -3
COMBA_ERR_HIP = -4
COMBA_BF16 = 0
COMBA_FP32 = 1
COMBA_FUSE_GATE_LOGITS = 1
COMBA_FUSE_QK_L2NORM = 2
COMBA_CHECK_ALPHA_RANGE = 1
COMBA_CHECK_CU_ORDER = 2
COMBA_CHECK_CU_BOUNDS = 4

# COMBA_DEBUG_CHECKS=1: every forward, decode and backward call first checks the
# device-side preconditions (comba_check_inputs), waits for the result and
# raises CombaError when one fails. Off by default: it synchronises the stream.
DEBUG_CHECKS = os.environ.get("COMBA_DEBUG_CHECKS", "") not in ("", "0")

EXPORTED = ("comba_abi_version", "comba_status_string", "comba_last_error",
            "comba_chunk_fwd_workspace_size", "comba_chunk_fwd", "comba_chunk_fwd_fused", "comba_chunk_fwd_ex",
            "comba_recurrent_step", "comba_recurrent_step_fused", "comba_recurrent_step_ex",
            "comba_chunk_fwd_segmented_workspace_size",
            "comba_chunk_fwd_segmented", "comba_chunk_bwd_workspace_size", "comba_chunk_bwd",
            "comba_varlen_order", "comba_mfma_peak_probe", "comba_chunk_states_size", "comba_chunk_fwd_keep_states",
            "comba_chunk_bwd_cached_workspace_size", "comba_chunk_bwd_cached", "comba_chunk_fwd_noalloc",
            "comba_lds_probe", "comba_check_inputs")


class CombaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libcomba.so (built in-tree by ``python -m bilinear_rnn_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m bilinear_rnn_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        i32, sz = ctypes.c_int32, ctypes.c_size_t
        L.comba_abi_version.argtypes = []
        L.comba_abi_version.restype = i32
        L.comba_status_string.argtypes = [i32]
        L.comba_status_string.restype = ctypes.c_char_p
        L.comba_last_error.argtypes = []
        L.comba_last_error.restype = ctypes.c_char_p
        L.comba_chunk_fwd_workspace_size.argtypes = [i32] * 7
        L.comba_chunk_fwd_workspace_size.restype = sz
        L.comba_chunk_fwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32,
                                      i32, i32, vp, fp, vp, sz, vp]
        L.comba_chunk_fwd.restype = i32
        L.comba_chunk_fwd_fused.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32,
                                            i32, i32, vp, fp, vp, sz, ctypes.c_uint32, vp]
        L.comba_chunk_fwd_fused.restype = i32
        L.comba_recurrent_step.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32,
                                           i32, i32, vp, fp, vp]
        L.comba_recurrent_step.restype = i32
        L.comba_recurrent_step_fused.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32,
                                                 i32, i32, i32, vp, fp, ctypes.c_uint32, vp]
        L.comba_recurrent_step_fused.restype = i32
        L.comba_chunk_fwd_segmented_workspace_size.argtypes = [i32] * 6
        L.comba_chunk_fwd_segmented_workspace_size.restype = sz
        L.comba_chunk_fwd_ex.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32,
                                         i32, i32, vp, fp, vp, sz, ctypes.c_uint32, vp]
        L.comba_chunk_fwd_ex.restype = i32
        L.comba_recurrent_step_ex.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32,
                                              i32, i32, vp, fp, ctypes.c_uint32, vp]
        L.comba_recurrent_step_ex.restype = i32
        L.comba_chunk_fwd_segmented.argtypes = [vp, vp, vp, fp, fp, fp, fp, i32, i32, i32, i32, i32, i32, i32, i32,
                                                vp, fp, i32, vp, sz, ctypes.c_uint32, vp]
        L.comba_chunk_fwd_segmented.restype = i32
        L.comba_chunk_bwd_workspace_size.argtypes = [i32] * 6
        L.comba_chunk_bwd_workspace_size.restype = sz
        L.comba_chunk_bwd.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32, vp, fp,
                                      fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
        L.comba_chunk_bwd.restype = i32
        L.comba_varlen_order.argtypes = [ip, i32, ip, vp]
        L.comba_varlen_order.restype = i32
        L.comba_chunk_states_size.argtypes = [i32] * 6
        L.comba_chunk_states_size.restype = sz
        L.comba_chunk_fwd_keep_states.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32,
                                                  i32, i32, vp, fp, vp, sz, fp, sz, vp]
        L.comba_chunk_fwd_keep_states.restype = i32
        L.comba_chunk_bwd_cached_workspace_size.argtypes = [i32] * 6
        L.comba_chunk_bwd_cached_workspace_size.restype = sz
        L.comba_chunk_bwd_cached.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32, i32, vp,
                                             fp, fp, sz, fp, fp, fp, fp, fp, fp, fp, vp, sz, vp]
        L.comba_chunk_bwd_cached.restype = i32
        L.comba_chunk_fwd_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, ip, i32, i32, i32, i32, i32, i32,
                                              i32, i32, vp, fp, vp]
        L.comba_chunk_fwd_noalloc.restype = i32
        L.comba_mfma_peak_probe.argtypes = [fp, i32, i32, vp]
        L.comba_mfma_peak_probe.restype = i32
        L.comba_lds_probe.argtypes = [i32, ip, i32, vp, i32, vp]
        L.comba_lds_probe.restype = i32
        L.comba_check_inputs.argtypes = [fp, ctypes.c_int64, ip, i32, i32, vp, vp]
        L.comba_check_inputs.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().comba_status_string(int(status)).decode()


def last_error() -> str:
    return lib().comba_last_error().decode()


def _check(status: int):
    if status != COMBA_OK:
        raise CombaError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_DT = {torch.bfloat16: COMBA_BF16, torch.float32: COMBA_FP32}


def _require(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _prepare(q, k, v, alpha, beta, d, initial_state, cu_seqlens, out_dtype):
    if q.dtype not in _DT:
        raise ValueError(f"q must be bfloat16 or float32 (got {q.dtype})")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B, T, Hqk, K] and v [B, T, H, V]")
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    if H % Hk != 0:
        raise ValueError(f"the q/k head count {Hk} must divide the value head count {H}")
    _require(q, "q", q.dtype)
    _require(k, "k", q.dtype, (B, T, Hk, K))
    _require(v, "v", q.dtype, (B, T, H, V))
    _require(alpha, "alpha", torch.float32, (B, T, H))
    _require(beta, "beta", torch.float32, (B, T, H))
    _require(d, "d", torch.float32, (H,))
    if cu_seqlens is not None:
        _require(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _require(initial_state, "initial_state", torch.float32, (N, H, V, K))
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("d", d),
                    ("initial_state", initial_state), ("cu_seqlens", cu_seqlens)):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}: all tensors must share one device")
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DT:
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    return B, T, H, Hk, K, V, N, out_dtype


def _fusion(gate_logits: bool, qk_l2norm: bool) -> int:
    return (COMBA_FUSE_GATE_LOGITS if gate_logits else 0) | (COMBA_FUSE_QK_L2NORM if qk_l2norm else 0)


def workspace_size(B: int, T: int, H: int, K: int, V: int, num_seqs: int = 0,
                   dtype: torch.dtype = torch.bfloat16) -> int:
    return int(lib().comba_chunk_fwd_workspace_size(B, T, H, K, V, num_seqs, _DT[dtype]))


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
              beta: torch.Tensor, d: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
              output_final_state: bool = True, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, gate_logits: bool = False,
              qk_l2norm: bool = False,
              segments: Optional[int] = None,
              chunk_states: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunk-wise forward through ``comba_chunk_fwd``. Returns (o, final_state).

    q and k may hold fewer heads than v (a divisor of H): consecutive value
    heads then share one q / k head (``comba_chunk_fwd_ex``).

    ``gate_logits``: alpha and beta hold pre-sigmoid logits; ``qk_l2norm``: q
    and k are L2-normalised per head and token inside the kernel. Either flag
    routes the call through ``comba_chunk_fwd_fused``. ``segments`` (an int,
    0 = automatic; fixed-length batches only) routes it through the
    segment-parallel ``comba_chunk_fwd_segmented``. ``chunk_states`` (fp32,
    at least ``chunk_states_size`` bytes; no fusion, segments or shared q / k)
    routes it through ``comba_chunk_fwd_keep_states``, which also keeps every
    chunk's incoming state there for ``chunk_bwd``."""
    B, T, H, Hk, K, V, N, out_dtype = _prepare(q, k, v, alpha, beta, d, initial_state, cu_seqlens, out_dtype)
    if DEBUG_CHECKS:
        _debug_check(alpha, cu_seqlens, T, check_alpha=not gate_logits)
    L = lib()
    if out is None:
        out = torch.empty((B, T, H, V), dtype=out_dtype, device=q.device)
    _require(out, "out", out_dtype, (B, T, H, V))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _require(final_state, "final_state", torch.float32, (N, H, V, K))
    fusion = _fusion(gate_logits, qk_l2norm)
    if segments is not None:
        if cu_seqlens is not None:
            raise ValueError("segments applies to fixed-length batches (no cu_seqlens)")
        nws = int(L.comba_chunk_fwd_segmented_workspace_size(B, T, H, K, V, int(segments)))
        if nws > 0 and (workspace is None or workspace.numel() < nws):
            workspace = torch.empty((nws,), dtype=torch.uint8, device=q.device)
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            _check(L.comba_chunk_fwd_segmented(
                _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(d), _ptr(initial_state), B, T, H, Hk, K,
                V, _DT[q.dtype], _DT[out_dtype], _ptr(out), _ptr(final_state), int(segments), _ptr(workspace),
                0 if workspace is None else workspace.numel(), fusion, ctypes.c_void_p(stream)))
        return out, final_state
    if chunk_states is not None:
        if fusion or Hk != H:
            raise ValueError("chunk_states goes with the plain forward (no fusion, one q / k head per value head)")
        _require(chunk_states, "chunk_states", torch.float32)
        if chunk_states.device != q.device:
            raise ValueError("chunk_states must be on q's device")
    nws = int(L.comba_chunk_fwd_workspace_size(B, T, H, K, V, N if cu_seqlens is not None else 0, _DT[q.dtype]))
    if nws > 0 and (workspace is None or workspace.numel() < nws):
        workspace = torch.empty((nws,), dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        head = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(d), _ptr(initial_state),
                _ptr(cu_seqlens), N if cu_seqlens is not None else 0, B, T, H)
        tail = (K, V, _DT[q.dtype], _DT[out_dtype], _ptr(out), _ptr(final_state), _ptr(workspace),
                0 if workspace is None else workspace.numel())
        if chunk_states is not None:
            _check(L.comba_chunk_fwd_keep_states(*head, *tail, _ptr(chunk_states), chunk_states.numel() * 4,
                                                 ctypes.c_void_p(stream)))
        elif Hk != H:
            _check(L.comba_chunk_fwd_ex(*head, Hk, *tail, fusion, ctypes.c_void_p(stream)))
        elif fusion:
            _check(L.comba_chunk_fwd_fused(*head, *tail, fusion, ctypes.c_void_p(stream)))
        else:
            _check(L.comba_chunk_fwd(*head, *tail, ctypes.c_void_p(stream)))
    return out, final_state


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                      beta: torch.Tensor, d: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                      output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunk-wise forward through ``comba_chunk_fwd_noalloc``: no workspace; the
    library keeps the packed-sequence order in its own device array (at most
    16384 sequences; calls that overlap in time on one GPU race). Pass ``out``
    and ``final_state`` to keep the call itself free of allocations."""
    B, T, H, Hk, K, V, N, out_dtype = _prepare(q, k, v, alpha, beta, d, initial_state, cu_seqlens, out_dtype)
    if Hk != H:
        raise ValueError("chunk_fwd_noalloc takes one q / k head per value head")
    if DEBUG_CHECKS:
        _debug_check(alpha, cu_seqlens, T)
    L = lib()
    if out is None:
        out = torch.empty((B, T, H, V), dtype=out_dtype, device=q.device)
    _require(out, "out", out_dtype, (B, T, H, V))
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _require(final_state, "final_state", torch.float32, (N, H, V, K))
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        _check(L.comba_chunk_fwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(d), _ptr(initial_state), _ptr(cu_seqlens),
            N if cu_seqlens is not None else 0, B, T, H, K, V, _DT[q.dtype], _DT[out_dtype], _ptr(out),
            _ptr(final_state), ctypes.c_void_p(stream)))
    return out, final_state


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                   beta: torch.Tensor, d: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                   in_place: bool = False, output_final_state: bool = True,
                   out: Optional[torch.Tensor] = None,
                   final_state: Optional[torch.Tensor] = None, gate_logits: bool = False,
                   qk_l2norm: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Token-by-token recurrence through ``comba_recurrent_step`` (T == 1: decode).

    With ``in_place`` the state is updated in ``initial_state`` itself.
    ``gate_logits`` and ``qk_l2norm`` as in ``chunk_fwd`` (through
    ``comba_recurrent_step_fused``)."""
    B, T, H, Hk, K, V, N, out_dtype = _prepare(q, k, v, alpha, beta, d, initial_state, cu_seqlens, out_dtype)
    if DEBUG_CHECKS:
        _debug_check(alpha, cu_seqlens, T, check_alpha=not gate_logits)
    L = lib()
    if out is None:
        out = torch.empty((B, T, H, V), dtype=out_dtype, device=q.device)
    _require(out, "out", out_dtype, (B, T, H, V))
    if in_place:
        if initial_state is None:
            raise ValueError("in_place requires initial_state")
        final_state = initial_state
    elif final_state is None and output_final_state:
        final_state = torch.empty((N, H, V, K), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _require(final_state, "final_state", torch.float32, (N, H, V, K))
    fusion = _fusion(gate_logits, qk_l2norm)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        head = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(d), _ptr(initial_state),
                _ptr(cu_seqlens), N if cu_seqlens is not None else 0, B, T, H)
        tail = (K, V, _DT[q.dtype], _DT[out_dtype], _ptr(out), _ptr(final_state))
        if Hk != H:
            _check(L.comba_recurrent_step_ex(*head, Hk, *tail, fusion, ctypes.c_void_p(stream)))
        elif fusion:
            _check(L.comba_recurrent_step_fused(*head, *tail, fusion, ctypes.c_void_p(stream)))
        else:
            _check(L.comba_recurrent_step(*head, *tail, ctypes.c_void_p(stream)))
    return out, final_state


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
              d: torch.Tensor, do: torch.Tensor, initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, d_final_state: Optional[torch.Tensor] = None,
              need_initial_state_grad: bool = True,
              workspace: Optional[torch.Tensor] = None,
              chunk_states: Optional[torch.Tensor] = None) -> dict:
    """Gradients through ``comba_chunk_bwd`` for dL/do = ``do`` and dL/dS_final =
    ``d_final_state`` (None: 0). Returns a dict of fp32 tensors dq, dk, dv,
    dalpha, dbeta, dd and (unless disabled) dinitial_state. With
    ``chunk_states`` (kept by ``chunk_fwd(..., chunk_states=...)`` on the same
    inputs) the call goes through ``comba_chunk_bwd_cached``, which does not
    recompute them."""
    B, T, H, Hk, K, V, N, _ = _prepare(q, k, v, alpha, beta, d, initial_state, cu_seqlens, None)
    if Hk != H:
        raise ValueError("the backward takes one q / k head per value head")
    _require(do, "do", q.dtype, (B, T, H, V))
    if DEBUG_CHECKS:
        _debug_check(alpha, cu_seqlens, T)
    if d_final_state is not None:
        _require(d_final_state, "d_final_state", torch.float32, (N, H, V, K))
    L = lib()
    f32 = dict(dtype=torch.float32, device=q.device)
    g = dict(dq=torch.empty((B, T, H, K), **f32), dk=torch.empty((B, T, H, K), **f32),
             dv=torch.empty((B, T, H, V), **f32), dalpha=torch.empty((B, T, H), **f32),
             dbeta=torch.empty((B, T, H), **f32), dd=torch.empty((H,), **f32))
    g["dinitial_state"] = torch.empty((N, H, V, K), **f32) if need_initial_state_grad else None
    nseq = N if cu_seqlens is not None else 0
    if chunk_states is not None:
        _require(chunk_states, "chunk_states", torch.float32)
        if chunk_states.device != q.device:
            raise ValueError("chunk_states must be on q's device")
        nws = int(L.comba_chunk_bwd_cached_workspace_size(B, T, H, K, V, nseq))
    else:
        nws = int(L.comba_chunk_bwd_workspace_size(B, T, H, K, V, nseq))
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty((nws,), dtype=torch.uint8, device=q.device)
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(d), _ptr(initial_state), _ptr(cu_seqlens),
            nseq, B, T, H, K, V, _DT[q.dtype], _ptr(do), _ptr(d_final_state))
    grads = (_ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]), _ptr(g["dbeta"]), _ptr(g["dd"]),
             _ptr(g["dinitial_state"]), _ptr(workspace), workspace.numel())
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if chunk_states is not None:
            _check(L.comba_chunk_bwd_cached(*head, _ptr(chunk_states), chunk_states.numel() * 4, *grads,
                                            ctypes.c_void_p(stream)))
        else:
            _check(L.comba_chunk_bwd(*head, *grads, ctypes.c_void_p(stream)))
    return g


def chunk_states_size(B: int, T: int, H: int, K: int, V: int, num_seqs: int = 0) -> int:
    """Bytes of the chunk-state buffer of ``chunk_fwd(..., chunk_states=...)``."""
    return int(lib().comba_chunk_states_size(B, T, H, K, V, num_seqs))


def bwd_cached_workspace_size(B: int, T: int, H: int, K: int, V: int, num_seqs: int = 0) -> int:
    return int(lib().comba_chunk_bwd_cached_workspace_size(B, T, H, K, V, num_seqs))


def bwd_workspace_size(B: int, T: int, H: int, K: int, V: int, num_seqs: int = 0) -> int:
    return int(lib().comba_chunk_bwd_workspace_size(B, T, H, K, V, num_seqs))


def segmented_workspace_size(B: int, T: int, H: int, K: int, V: int, segments: int = 0) -> int:
    return int(lib().comba_chunk_fwd_segmented_workspace_size(B, T, H, K, V, segments))


def varlen_order(cu_seqlens: torch.Tensor) -> torch.Tensor:
    """Longest-first order of packed sequences through ``comba_varlen_order``."""
    _require(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    order = torch.empty((N,), dtype=torch.int32, device=cu_seqlens.device)
    with torch.cuda.device(cu_seqlens.device):
        stream = torch.cuda.current_stream(cu_seqlens.device).cuda_stream
        _check(lib().comba_varlen_order(_ptr(cu_seqlens), N, _ptr(order), ctypes.c_void_p(stream)))
    return order


_CHECK_NAMES = ((COMBA_CHECK_ALPHA_RANGE, "an alpha outside (0, 1] or NaN"),
                (COMBA_CHECK_CU_ORDER, "cu_seqlens decreases"),
                (COMBA_CHECK_CU_BOUNDS, "cu_seqlens does not start at 0 and end at T"))


def check_inputs(alpha: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None, T: Optional[int] = None,
                 check_alpha: bool = True) -> int:
    """Device-side preconditions through ``comba_check_inputs``: returns the OR of
    the COMBA_CHECK_* bits of the violated ones (0: all hold). Waits for the
    stream. ``T`` is the packed length cu_seqlens must end at (default: the
    token axis of alpha)."""
    _require(alpha, "alpha", torch.float32)
    N = 0
    if cu_seqlens is not None:
        _require(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
        if T is None:
            T = alpha.shape[1] if alpha.dim() >= 2 else alpha.numel()
    flags = torch.empty((1,), dtype=torch.int32, device=alpha.device)
    with torch.cuda.device(alpha.device):
        stream = torch.cuda.current_stream(alpha.device).cuda_stream
        _check(lib().comba_check_inputs(_ptr(alpha), alpha.numel() if check_alpha else 0, _ptr(cu_seqlens), N,
                                        0 if T is None else int(T), _ptr(flags), ctypes.c_void_p(stream)))
    return int(flags.item())


def _debug_check(alpha: torch.Tensor, cu_seqlens: Optional[torch.Tensor], T: int, check_alpha: bool = True):
    bad = check_inputs(alpha, cu_seqlens, T, check_alpha)
    if bad:
        raise CombaError(COMBA_ERR_INVALID_ARG, "device-side preconditions violated: " +
                         "; ".join(name for bit, name in _CHECK_NAMES if bad & bit))


PEAK_PROBE_FLOPS_PER_BLOCK_ITER = 4 * 4 * 16384   # wavefronts x MFMAs per iteration x flops per MFMA


LDS_PROBE_KINDS = {"read16": 0, "read8": 1, "read4": 2, "read8_tr": 3,
                   "write16": 4, "write8": 5, "write4": 6, "write2": 7}


def lds_probe(kind: str, lane_offsets, iters: int, sink: torch.Tensor) -> None:
    """One launch of ``comba_lds_probe``: ``sink.numel() // 256`` workgroups
    repeating one LDS access whose 64 per-lane byte offsets are given."""
    if kind not in LDS_PROBE_KINDS:
        raise ValueError(f"kind must be one of {sorted(LDS_PROBE_KINDS)}")
    offs = [int(o) for o in lane_offsets]
    if len(offs) != 64:
        raise ValueError("64 lane offsets")
    if not (isinstance(sink, torch.Tensor) and sink.is_cuda and sink.dtype == torch.int32 and sink.is_contiguous()):
        raise TypeError("sink must be a contiguous int32 CUDA tensor")
    arr = (ctypes.c_int32 * 64)(*offs)
    with torch.cuda.device(sink.device):
        stream = torch.cuda.current_stream(sink.device).cuda_stream
        _check(lib().comba_lds_probe(LDS_PROBE_KINDS[kind], arr, int(iters), ctypes.c_void_p(sink.data_ptr()),
                                     sink.numel() // 256, ctypes.c_void_p(stream)))


def mfma_peak_probe(sink: torch.Tensor, iters: int) -> int:
    """One launch of ``comba_mfma_peak_probe`` over ``sink.numel() // 256``
    workgroups; returns the flops it performs."""
    _require(sink, "sink", torch.float32)
    blocks = sink.numel() // 256
    with torch.cuda.device(sink.device):
        stream = torch.cuda.current_stream(sink.device).cuda_stream
        _check(lib().comba_mfma_peak_probe(_ptr(sink), blocks, int(iters), ctypes.c_void_p(stream)))
    return blocks * iters * PEAK_PROBE_FLOPS_PER_BLOCK_ITER
