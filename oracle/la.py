"""fp64 CPU oracle for decay-only linear attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  The GPU library never imports or
calls it, and it shares no code with the GPU path.

What it computes.  The cuLA benchmark page (GB200, CUDA 13.0), in its
lightning-attention section, times a chunked forward ("no_state" and
"varlen" modes) and a single-token decode of decay-only linear attention
without defining the operator.  It is read here as the KDA recurrence with
the delta-rule erase and the write strength removed (the plainest reading,
and the one the KDA chunk form reduces to when the UT transform is the
identity):

    per chain (batch row or packed sequence, value head h), state S in
    R^{K x V}, starting from initial_state (or zeros), for each token t:

      g_t = -exp(A_log[h]) * softplus(g_raw_t)    (one scalar per token-head,
                                                  or one per channel)
      S_t = Diag(exp(g_t)) S_{t-1} + k_t v_t^T
      o_t = scale * S_t^T q_t

q and k are used as given (no normalisation).  Value head h reads q/k head
h / (H / H_qk).  Layouts are those of the KDA oracle: q, k [B,T,H_qk,K],
v [B,T,H,V], g_raw [B,T,H,K] or [B,T,H], state [C,H,V,K] with
state[c,h,v,kk] = S[kk][v].  The state advances one token at a time in fp64,
exactly as the recurrence reads; numpy does the per-token vector arithmetic.
"""

from __future__ import annotations

import numpy as np

from . import widen


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _log_decay(g_raw, a_log):
    """g = -exp(A_log[h]) * softplus(g_raw) for one token-head (a scalar or a K-vector)."""
    return -np.exp(a_log) * _softplus(g_raw)


def la_fwd(q, k, v, g_raw, A_log, scale: float, gate_per_channel: bool = False, initial_state=None,
           cu_seqlens=None, chain_mask=None):
    """Oracle forward.  Returns (out fp64 [B,T,H,V], final_state fp64 [C,H,V,K]).

    cu_seqlens: int32 [N+1] (then B == 1 and C == N) or None (C == B).
    chain_mask: optional bool [C,H]; unselected chains come back as NaN.
    """
    q, k, v, g_raw, A_log = widen(q), widen(k), widen(v), widen(g_raw), widen(A_log)
    B, T, H_qk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    G = H // H_qk
    assert k.shape == q.shape and v.shape[:2] == (B, T) and H % H_qk == 0
    assert g_raw.shape == ((B, T, H, K) if gate_per_channel else (B, T, H)) and A_log.shape == (H,)
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        assert B == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
        spans = [(0, int(cu[n]), int(cu[n + 1])) for n in range(cu.shape[0] - 1)]
    else:
        spans = [(b, 0, T) for b in range(B)]
    C = len(spans)
    init = None if initial_state is None else widen(initial_state)
    assert init is None or init.shape == (C, H, V, K)
    mask = np.ones((C, H), dtype=bool) if chain_mask is None else np.asarray(chain_mask, dtype=bool).reshape(C, H)
    out = np.full((B, T, H, V), np.nan if chain_mask is not None else 0.0)
    final = np.full((C, H, V, K), np.nan if chain_mask is not None else 0.0)
    for c, (b, t0, t1) in enumerate(spans):
        for h in range(H):
            if not mask[c, h]:
                continue
            hq = h // G
            S = np.zeros((K, V)) if init is None else init[c, h].T.copy()   # S[kk, v]
            for t in range(t0, t1):
                g = _log_decay(g_raw[b, t, h], A_log[h])
                decay = np.exp(g) * np.ones(K)
                S = decay[:, None] * S + np.outer(k[b, t, hq], v[b, t, h])
                out[b, t, h] = scale * (S.T @ q[b, t, hq])
            final[c, h] = S.T
    return out, final


def la_decode(q, k, v, g_raw, A_log, scale: float, state, gate_per_channel: bool = False):
    """Oracle single-token step.  Returns (out fp64 [B,H,V], new_state fp64 [B,H,V,K]).

    q, k: [B,H_qk,K]; v: [B,H,V]; g_raw: [B,H,K] or [B,H]; state: [B,H,V,K]
    (not modified; the advanced state is returned).
    """
    q, k, v, g_raw, A_log = widen(q), widen(k), widen(v), widen(g_raw), widen(A_log)
    st = widen(state).copy()
    B, H_qk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    G = H // H_qk
    out = np.zeros((B, H, V))
    for b in range(B):
        for h in range(H):
            hq = h // G
            g = _log_decay(g_raw[b, h], A_log[h])
            S = (np.exp(g) * np.ones(K))[:, None] * st[b, h].T + np.outer(k[b, hq], v[b, h])
            out[b, h] = scale * (S.T @ q[b, hq])
            st[b, h] = S.T
    return out, st
