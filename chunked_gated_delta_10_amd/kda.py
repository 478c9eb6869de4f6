"""Thin Python binding of libkda.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
checks tensor dtypes/shapes, allocates outputs and workspace with torch (the
only thing torch is used for, together with the current stream) and passes
raw device pointers through the C ABI declared in ``include/kda.h``.

There is no fallback: if ``libkda.so`` is missing every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIB names another build of the same library (e.g. a host-sanitizer build for the CPU tests)
LIB_PATH = os.environ.get("KDA_LIB") or os.path.join(_HERE, "libkda.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kda.h")

KDA_STATE_NONE, KDA_STATE_BF16, KDA_STATE_FP32 = 0, 1, 2
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
          4: "KDA_ERR_STATE_DTYPE_MISMATCH", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_ALIGN", 7: "KDA_ERR_HIP"}

_lib = None


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (STATUS.get(status, str(status)), detail))
        self.status = status
        self.detail = detail


def header_functions():
    """Names of the functions include/kda.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def load():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkda.so is not built (%s); run __graft_entry__.build() first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kda_fwd_workspace_bytes.restype = Z
    lib.kda_fwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.kda_fwd.restype = I
    lib.kda_fwd.argtypes = [P, P, P, P, P, P, F, I, P, I, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.kda_fwd_noalloc.restype = I
    lib.kda_fwd_noalloc.argtypes = [P, P, P, P, P, P, F, I, P, I, P, P, I, I, I, I, I, I, I, P]
    lib.kda_fwd_varlen.restype = I
    lib.kda_fwd_varlen.argtypes = [P, P, P, P, P, P, F, I, P, I, P, P, I, P, I, I, I, I, I, I, P, Z, P]
    lib.kda_decode_step.restype = I
    lib.kda_decode_step.argtypes = [P, P, P, P, P, P, F, I, P, I, P, I, I, I, I, I, P]
    lib.kda_la_fwd.restype = I
    lib.kda_la_fwd.argtypes = [P, P, P, P, P, F, I, P, I, P, P, I, I, I, I, I, I, I, P, Z, P]
    lib.kda_la_fwd_varlen.restype = I
    lib.kda_la_fwd_varlen.argtypes = [P, P, P, P, P, F, I, P, I, P, P, I, P, I, I, I, I, I, I, P, Z, P]
    lib.kda_la_decode_step.restype = I
    lib.kda_la_decode_step.argtypes = [P, P, P, P, P, F, I, P, I, P, I, I, I, I, I, P]
    lib.kda_bwd_workspace_bytes.restype = Z
    lib.kda_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.kda_bwd.restype = I
    lib.kda_bwd.argtypes = [P, P, P, P, P, P, F, I, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P, Z, P]
    lib.kda_bwd_varlen.restype = I
    lib.kda_bwd_varlen.argtypes = [P, P, P, P, P, P, F, I, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P,
                                   Z, P]
    lib.kda_fwd_check.restype = I
    lib.kda_fwd_check.argtypes = [P, P]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [I]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_kernel_timing_enable.restype = None
    lib.kda_kernel_timing_enable.argtypes = [I]
    lib.kda_kernel_timing_read.restype = I
    lib.kda_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), I]
    lib.kda_kernel_name.restype = ctypes.c_char_p
    lib.kda_kernel_name.argtypes = [I]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise KdaError(status, load().kda_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _state_code(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return KDA_STATE_NONE
    if t.dtype == torch.float32:
        return KDA_STATE_FP32
    if t.dtype == torch.bfloat16:
        return KDA_STATE_BF16
    raise TypeError("state must be float32 or bfloat16, got %s" % t.dtype)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype):
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _same_device(first: torch.Tensor, *rest) -> None:
    for t in rest:
        if t is not None and t.device != first.device:
            raise ValueError("inputs are on different devices (%s and %s)" % (first.device, t.device))


def _check_out(out: torch.Tensor, shape, device) -> None:
    """A caller-supplied output must be exactly what the kernels write: the
    library cannot see buffer sizes, so a short or mistyped buffer would be
    written past its end."""
    if out.dtype != torch.bfloat16:
        raise TypeError("out must be bfloat16, got %s" % out.dtype)
    if tuple(out.shape) != tuple(shape):
        raise ValueError("out must have shape %s, got %s" % (tuple(shape), tuple(out.shape)))
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if out.device != device:
        raise ValueError("out is on %s, the inputs on %s" % (out.device, device))


def _check_state(t: Optional[torch.Tensor], name: str, shape, device) -> None:
    if t is None:
        return
    _state_code(t)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.device != device:
        raise ValueError("%s is on %s, the inputs on %s" % (name, t.device, device))


def _check_workspace(ws: torch.Tensor, nbytes: int, device) -> None:
    if ws.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor, got %s" % ws.dtype)
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if ws.device != device:
        raise ValueError("workspace is on %s, the inputs on %s" % (ws.device, device))
    if ws.numel() < nbytes:
        raise ValueError("workspace holds %d bytes, %d needed" % (ws.numel(), nbytes))


def kernel_timing(enable: bool) -> None:
    """Turn per-kernel HIP-event timing of this thread's launches on or off."""
    load().kda_kernel_timing_enable(1 if enable else 0)


def kernel_timing_read() -> dict:
    """{kernel name: (total ms, launches)} since the last read (waits for the events)."""
    lib = load()
    n = 16
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    k = lib.kda_kernel_timing_read(ms, cnt, n)
    if k < 0:
        raise RuntimeError("kda_kernel_timing_read failed")
    return {lib.kda_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(k) if cnt[i] > 0}


def check(workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Waits for the stream and raises KdaError if the last forward call on
    `workspace` (None: the allocation-free scratch) recorded an internal error."""
    _check(load().kda_fwd_check(_ptr(workspace), _stream(stream)))


def workspace_bytes(B: int, T: int, H_qk: int, H: int, N: int = 0) -> int:
    return int(load().kda_fwd_workspace_bytes(B, T, H_qk, H, N))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _prep(q, k, v, g_raw, beta_logits, A_log):
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16)
    _need(v, "v", torch.bfloat16)
    _need(g_raw, "g_raw", torch.bfloat16)
    if beta_logits is not None:
        _need(beta_logits, "beta_logits", torch.float32)
    _need(A_log, "A_log", torch.float32)
    _same_device(q, k, v, g_raw, beta_logits, A_log)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B, T, H_qk, K] and v [B, T, H, V]")
    B, T, H_qk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    if g_raw.shape == (B, T, H, K):
        per_channel = 1
    elif g_raw.shape == (B, T, H):
        per_channel = 0
    else:
        raise ValueError("g_raw must be [B, T, H, K] (per channel) or [B, T, H] (scalar)")
    if (beta_logits is not None and beta_logits.shape != (B, T, H)) or A_log.shape != (H,):
        raise ValueError("beta_logits must be [B, T, H] and A_log [H]")
    return B, T, H_qk, H, K, V, per_channel


def fwd(q, k, v, g_raw, beta_logits, A_log, scale: Optional[float] = None,
        initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
        final_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None,
        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA forward over B rows of T tokens.  Returns (out, final_state)."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, beta_logits, A_log)
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    _check_out(out, (B, T, H, V), dev)
    if final_state is None and output_final_state:
        sd = state_dtype or (initial_state.dtype if initial_state is not None else torch.float32)
        final_state = torch.empty((B, H, V, K), dtype=sd, device=dev)
    _check_state(initial_state, "initial_state", (B, H, V, K), dev)
    _check_state(final_state, "final_state", (B, H, V, K), dev)
    nbytes = workspace_bytes(B, T, H_qk, H, 0)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check_workspace(workspace, nbytes, dev)
    _check(lib.kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log), scale,
                       per_channel, _ptr(initial_state), _state_code(initial_state), _ptr(out),
                       _ptr(final_state), _state_code(final_state), B, T, H_qk, H, K, V, _ptr(workspace),
                       workspace.numel(), _stream(stream)))
    return out, final_state


# Capacity of the static scratch array behind fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES in include/kda.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def fwd_noalloc(q, k, v, g_raw, beta_logits, A_log, out: torch.Tensor, final_state: Optional[torch.Tensor],
                scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_fwd through the allocation-free entry point: the caller passes `out`
    (and `final_state`, or None), and the library's static scratch array holds
    the intermediates, so nothing is allocated, by torch or by the library.
    Sizes beyond the scratch capacity raise KdaError (KDA_ERR_WORKSPACE)."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, beta_logits, A_log)
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    _check_out(out, (B, T, H, V), dev)
    _check_state(initial_state, "initial_state", (B, H, V, K), dev)
    _check_state(final_state, "final_state", (B, H, V, K), dev)
    _check(lib.kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log), scale,
                               per_channel, _ptr(initial_state), _state_code(initial_state), _ptr(out),
                               _ptr(final_state), _state_code(final_state), B, T, H_qk, H, K, V, _stream(stream)))
    return out, final_state


def fwd_varlen(q, k, v, g_raw, beta_logits, A_log, cu_seqlens: torch.Tensor, scale: Optional[float] = None,
               initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
               final_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None,
               stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA forward over packed sequences (B = 1).  Returns (out, final_state [N, H, V, K])."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, beta_logits, A_log)
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    if cu_seqlens.device != dev:
        raise ValueError("cu_seqlens is on %s, the inputs on %s" % (cu_seqlens.device, dev))
    if out is None:
        out = torch.empty((1, T, H, V), dtype=torch.bfloat16, device=dev)
    _check_out(out, (1, T, H, V), dev)
    if final_state is None and output_final_state:
        sd = state_dtype or (initial_state.dtype if initial_state is not None else torch.float32)
        final_state = torch.empty((N, H, V, K), dtype=sd, device=dev)
    _check_state(initial_state, "initial_state", (N, H, V, K), dev)
    _check_state(final_state, "final_state", (N, H, V, K), dev)
    nbytes = workspace_bytes(1, T, H_qk, H, max(N, 0))
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check_workspace(workspace, nbytes, dev)
    _check(lib.kda_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log), scale,
                              per_channel, _ptr(initial_state), _state_code(initial_state), _ptr(out),
                              _ptr(final_state), _state_code(final_state), _ptr(cu_seqlens), N, T, H_qk, H, K, V,
                              _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, final_state


def decode_step(q, k, v, g_raw, beta_logits, A_log, state: torch.Tensor, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step; `state` [B, H, V, K] is updated in place.  Returns out [B, H, V]."""
    lib = load()
    for t, n, dt in ((q, "q", torch.bfloat16), (k, "k", torch.bfloat16), (v, "v", torch.bfloat16),
                     (g_raw, "g_raw", torch.bfloat16), (beta_logits, "beta_logits", torch.float32),
                     (A_log, "A_log", torch.float32)):
        _need(t, n, dt)
    _same_device(q, k, v, g_raw, A_log)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3:
        raise ValueError("q, k must be [B, H_qk, K] and v [B, H, V]")
    B, H_qk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    if g_raw.shape == (B, H, K):
        per_channel = 1
    elif g_raw.shape == (B, H):
        per_channel = 0
    else:
        raise ValueError("g_raw must be [B, H, K] or [B, H]")
    _check_state(state, "state", (B, H, V, K), q.device)
    scale = K ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, V), dtype=torch.bfloat16, device=q.device)
    _check_out(out, (B, H, V), q.device)
    _check(lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log), scale,
                               per_channel, _ptr(state), _state_code(state), _ptr(out), B, H_qk, H, K, V,
                               _stream(stream)))
    return out


# ---- decay-only linear attention ---------------------------------------------
# The same chunked path without the delta rule: S_t = Diag(exp(g_t)) S_{t-1}
# + k_t v_t^T, o_t = scale * S_t^T q_t, q and k used as given.


def _states(initial_state, final_state, output_final_state, state_dtype, C, H, V, K, dev):
    if final_state is None and output_final_state:
        sd = state_dtype or (initial_state.dtype if initial_state is not None else torch.float32)
        final_state = torch.empty((C, H, V, K), dtype=sd, device=dev)
    _check_state(initial_state, "initial_state", (C, H, V, K), dev)
    _check_state(final_state, "final_state", (C, H, V, K), dev)
    return final_state


def la_fwd(q, k, v, g_raw, A_log, scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
           output_final_state: bool = True, final_state: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           state_dtype: Optional[torch.dtype] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked decay-only linear attention over B rows of T tokens.  Returns (out, final_state)."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, None, A_log)
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    _check_out(out, (B, T, H, V), dev)
    final_state = _states(initial_state, final_state, output_final_state, state_dtype, B, H, V, K, dev)
    nbytes = workspace_bytes(B, T, H_qk, H, 0)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check_workspace(workspace, nbytes, dev)
    _check(lib.kda_la_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(A_log), scale, per_channel,
                          _ptr(initial_state), _state_code(initial_state), _ptr(out), _ptr(final_state),
                          _state_code(final_state), B, T, H_qk, H, K, V, _ptr(workspace), workspace.numel(),
                          _stream(stream)))
    return out, final_state


def la_fwd_varlen(q, k, v, g_raw, A_log, cu_seqlens: torch.Tensor, scale: Optional[float] = None,
                  initial_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  final_state: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, state_dtype: Optional[torch.dtype] = None,
                  stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked decay-only linear attention over packed sequences (B = 1).  Returns (out, final_state)."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, None, A_log)
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    if cu_seqlens.device != dev:
        raise ValueError("cu_seqlens is on %s, the inputs on %s" % (cu_seqlens.device, dev))
    if out is None:
        out = torch.empty((1, T, H, V), dtype=torch.bfloat16, device=dev)
    _check_out(out, (1, T, H, V), dev)
    final_state = _states(initial_state, final_state, output_final_state, state_dtype, N, H, V, K, dev)
    nbytes = workspace_bytes(1, T, H_qk, H, max(N, 0))
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check_workspace(workspace, nbytes, dev)
    _check(lib.kda_la_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(A_log), scale, per_channel,
                                 _ptr(initial_state), _state_code(initial_state), _ptr(out), _ptr(final_state),
                                 _state_code(final_state), _ptr(cu_seqlens), N, T, H_qk, H, K, V, _ptr(workspace),
                                 workspace.numel(), _stream(stream)))
    return out, final_state


def la_decode_step(q, k, v, g_raw, A_log, state: torch.Tensor, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decay-only linear-attention decode step; `state` [B, H, V, K] is updated in place."""
    lib = load()
    for t, n, dt in ((q, "q", torch.bfloat16), (k, "k", torch.bfloat16), (v, "v", torch.bfloat16),
                     (g_raw, "g_raw", torch.bfloat16), (A_log, "A_log", torch.float32)):
        _need(t, n, dt)
    _same_device(q, k, v, g_raw, A_log)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3:
        raise ValueError("q, k must be [B, H_qk, K] and v [B, H, V]")
    B, H_qk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    if g_raw.shape == (B, H, K):
        per_channel = 1
    elif g_raw.shape == (B, H):
        per_channel = 0
    else:
        raise ValueError("g_raw must be [B, H, K] or [B, H]")
    _check_state(state, "state", (B, H, V, K), q.device)
    scale = K ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, V), dtype=torch.bfloat16, device=q.device)
    _check_out(out, (B, H, V), q.device)
    _check(lib.kda_la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(A_log), scale, per_channel,
                                  _ptr(state), _state_code(state), _ptr(out), B, H_qk, H, K, V, _stream(stream)))
    return out


# ---- backward (scalar gate) ----------------------------------------------------


def bwd_workspace_bytes(B: int, T: int, H_qk: int, H: int, N: int = 0) -> int:
    return int(load().kda_bwd_workspace_bytes(B, T, H_qk, H, N))


def _grad_buffers(B, T, H_qk, H, K, V, C, dev, want_dinit, per_channel):
    f = dict(dtype=torch.float32, device=dev)
    return dict(dq=torch.empty((B, T, H_qk, K), **f), dk=torch.empty((B, T, H_qk, K), **f),
                dv=torch.empty((B, T, H, V), **f),
                dg_raw=torch.empty((B, T, H, K) if per_channel else (B, T, H), **f),
                dbeta_logits=torch.empty((B, T, H), **f), dA_log=torch.empty((H,), **f),
                dinitial_state=torch.empty((C, H, V, K), **f) if want_dinit else None)


def _bwd_checks(dout, dfinal, initial_state, B, T, H, V, K, C, dev):
    _need(dout, "dout", torch.bfloat16)
    if tuple(dout.shape) != (B, T, H, V) or dout.device != dev:
        raise ValueError("dout must be a bf16 [B, T, H, V] tensor on the inputs' device")
    for t, n in ((dfinal, "dfinal"), (initial_state, "initial_state")):
        if t is None:
            continue
        _need(t, n, torch.float32)
        if tuple(t.shape) != (C, H, V, K) or t.device != dev:
            raise ValueError("%s must be a float32 %s tensor on the inputs' device" % (n, (C, H, V, K)))


def bwd(q, k, v, g_raw, beta_logits, A_log, dout, dfinal: Optional[torch.Tensor] = None,
        scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of sum(dout * out) + sum(dfinal * final_state) through fwd (g_raw [B, T, H] for one decay
    per token-head, [B, T, H, K] for one per key channel).

    Returns {dq, dk, dv, dg_raw, dbeta_logits, dA_log, dinitial_state}, all float32 (dg_raw in g_raw's
    shape)."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, beta_logits, A_log)
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    _bwd_checks(dout, dfinal, initial_state, B, T, H, V, K, B, dev)
    nbytes = bwd_workspace_bytes(B, T, H_qk, H, 0)
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check_workspace(workspace, nbytes, dev)
    g = _grad_buffers(B, T, H_qk, H, K, V, B, dev, True, per_channel)
    _check(lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log), scale, per_channel,
                       _ptr(initial_state), _ptr(dout), _ptr(dfinal), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                       _ptr(g["dg_raw"]), _ptr(g["dbeta_logits"]), _ptr(g["dA_log"]), _ptr(g["dinitial_state"]),
                       B, T, H_qk, H, K, V, _ptr(workspace), workspace.numel(), _stream(stream)))
    return g


def bwd_varlen(q, k, v, g_raw, beta_logits, A_log, dout, cu_seqlens: torch.Tensor,
               dfinal: Optional[torch.Tensor] = None, scale: Optional[float] = None,
               initial_state: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> dict:
    """bwd over packed sequences (B = 1); states and dinitial_state are [N, H, V, K]."""
    lib = load()
    B, T, H_qk, H, K, V, per_channel = _prep(q, k, v, g_raw, beta_logits, A_log)
    if B != 1:
        raise ValueError("packed sequences need B == 1")
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    N = cu_seqlens.numel() - 1
    scale = K ** -0.5 if scale is None else float(scale)
    dev = q.device
    if cu_seqlens.device != dev:
        raise ValueError("cu_seqlens is on %s, the inputs on %s" % (cu_seqlens.device, dev))
    _bwd_checks(dout, dfinal, initial_state, 1, T, H, V, K, N, dev)
    nbytes = bwd_workspace_bytes(1, T, H_qk, H, max(N, 0))
    if workspace is None:
        workspace = _workspace(nbytes, dev)
    _check_workspace(workspace, nbytes, dev)
    g = _grad_buffers(1, T, H_qk, H, K, V, max(N, 0), dev, True, per_channel)
    _check(lib.kda_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log), scale,
                              per_channel,
                              _ptr(initial_state), _ptr(dout), _ptr(dfinal), _ptr(g["dq"]), _ptr(g["dk"]),
                              _ptr(g["dv"]), _ptr(g["dg_raw"]), _ptr(g["dbeta_logits"]), _ptr(g["dA_log"]),
                              _ptr(g["dinitial_state"]), _ptr(cu_seqlens), N, T, H_qk, H, K, V, _ptr(workspace),
                              workspace.numel(), _stream(stream)))
    return g
