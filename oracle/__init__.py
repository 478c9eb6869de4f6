"""fp64 CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links
or calls it, and it shares no code with the GPU path.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, token by token; see
its header for the recurrence and the layouts).  This module only compiles
that file with the host C compiler, widens the caller's arrays to fp64 and
calls it.

bf16 tensors are passed as ``numpy.uint16`` arrays holding the raw bf16 bit
patterns; they are widened exactly (a bf16 value is the upper half of an
fp32 value).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

_lib = None


SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build(force: bool = True, sanitize: bool = False, out: Optional[str] = None) -> str:
    """Compile kda_oracle.c into libkda_oracle.so next to it (gcc, OpenMP).

    sanitize=True builds an AddressSanitizer + UndefinedBehaviorSanitizer
    copy instead (to ``out``); loading it needs gcc's libasan preloaded."""
    lib = out or _LIB
    if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(_SRC):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    opt = SANITIZE_FLAGS if sanitize else ["-O3"]
    cmd = ["gcc"] + opt + ["-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("KDA_ORACLE_LIB")  # another build of kda_oracle.c (e.g. a sanitizer build)
    if not path:
        path = build(force=False)
    lib = ctypes.CDLL(path)
    d = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd.argtypes = [d, d, d, d, d, d, ctypes.c_double, ctypes.c_int, d, d, d,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_uint8), ctypes.c_int]
    lib.kda_oracle_decode.restype = ctypes.c_int
    lib.kda_oracle_decode.argtypes = [d, d, d, d, d, d, ctypes.c_double, ctypes.c_int, d, d,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int]
    _lib = lib
    return lib


def widen(x) -> np.ndarray:
    """Exact fp64 copy of an array: uint16 arrays are read as bf16 bit patterns."""
    x = np.ascontiguousarray(np.asarray(x))
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _threads(nthreads: Optional[int]) -> int:
    if nthreads is not None:
        return int(nthreads)
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0)


def kda_fwd(q, k, v, g_raw, beta_logits, A_log, scale: float, gate_per_channel: bool = True,
            initial_state=None, cu_seqlens=None, chain_mask=None, nthreads: Optional[int] = None):
    """Oracle forward.  Returns (out fp64 [B,T,H,V], final_state fp64 [C,H,V,K]).

    q, k: [B,T,H_qk,K]; v: [B,T,H,V]; g_raw: [B,T,H,K] or [B,T,H];
    beta_logits: [B,T,H]; A_log: [H]; initial_state: [C,H,V,K] or None;
    cu_seqlens: int32 [N+1] (then B == 1, C == N) or None (C == B).
    chain_mask: optional bool [C,H]; unselected chains come back as NaN.
    """
    lib = _load()
    q, k, v, g_raw = widen(q), widen(k), widen(v), widen(g_raw)
    beta_logits, A_log = widen(beta_logits), widen(A_log)
    B, T, H_qk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T)
    assert g_raw.shape == ((B, T, H, K) if gate_per_channel else (B, T, H))
    assert beta_logits.shape == (B, T, H) and A_log.shape == (H,)
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
        C = cu.shape[0] - 1
    else:
        C = B
    init = None
    if initial_state is not None:
        init = widen(initial_state)
        assert init.shape == (C, H, V, K)
    mask = None
    if chain_mask is not None:
        mask = np.ascontiguousarray(np.asarray(chain_mask, dtype=np.uint8).reshape(C, H))
    out = np.full((B, T, H, V), np.nan if mask is not None else 0.0)
    final = np.full((C, H, V, K), np.nan if mask is not None else 0.0)
    rc = lib.kda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log),
                            float(scale), int(bool(gate_per_channel)), _ptr(init), _ptr(out),
                            _ptr(final), B, T, H_qk, H, K, V,
                            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if cu is not None else None,
                            C if cu is not None else 0,
                            mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)) if mask is not None else None,
                            _threads(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_fwd rejected its arguments (code %d)" % rc)
    return out, final


def kda_decode(q, k, v, g_raw, beta_logits, A_log, scale: float, state, gate_per_channel: bool = True,
               nthreads: Optional[int] = None):
    """Oracle single-token decode.  Returns (out fp64 [B,H,V], new_state fp64 [B,H,V,K]).

    q, k: [B,H_qk,K]; v: [B,H,V]; g_raw: [B,H,K] or [B,H]; beta_logits: [B,H];
    state: [B,H,V,K] (not modified; the advanced state is returned).
    """
    lib = _load()
    q, k, v, g_raw = widen(q), widen(k), widen(v), widen(g_raw)
    beta_logits, A_log = widen(beta_logits), widen(A_log)
    B, H_qk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    st = widen(state).copy()
    assert st.shape == (B, H, V, K)
    out = np.zeros((B, H, V))
    rc = lib.kda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_logits), _ptr(A_log),
                               float(scale), int(bool(gate_per_channel)), _ptr(st), _ptr(out),
                               B, H_qk, H, K, V, _threads(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_decode rejected its arguments (code %d)" % rc)
    return out, st


if __name__ == "__main__":  # pragma: no cover - build helper
    print(build(force=True))
    sys.exit(0)
