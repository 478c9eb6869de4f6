"""fp64 CPU oracle for the KDA backward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module; the GPU library never imports or
calls it, and it shares no code with the GPU path.

The FlashQLA H200 results page times a backward pass of the gated delta
rule ("BACKWARD BENCHMARKS", sequences split into 8, 32-64 heads, 16k-256k
tokens) without stating it; the backward of an operator is the gradient of a
scalar loss through it, so this module is reverse-mode differentiation of
the forward recurrence the KDA oracle computes (``kda_oracle.c``):

    qn  = q_t / sqrt(sum(q_t^2) + eps),  kn = k_t / sqrt(sum(k_t^2) + eps)
    g_t = -exp(A_log[h]) * softplus(g_raw_t),   b_t = sigmoid(beta_logit_t)
    S'  = Diag(exp(g_t)) S_{t-1}                 (decay first)
    u_t = b_t (v_t - S'^T kn)                    (delta-rule write)
    S_t = S' + kn u_t^T,    o_t = scale * S_t^T qn

Given the upstream gradients dout (of every o_t) and dfinal (of the final
state), ``kda_bwd`` returns the gradients of
    L = sum(dout * out) + sum(dfinal * final_state)
with respect to q, k, v, g_raw, beta_logits, A_log and initial_state, by
walking each chain's tokens backwards through the steps above in reverse
order, with the states of the forward walk kept (token by token, fp64, no
chunking).  Grouped value heads add the gradients of every value head of a
group into its q/k head; the scalar gate adds the per-channel terms of a
token into its one decay.

``kda_fwd`` here is the same forward, written with array operations that
stay analytic (sum of squares, log(1 + exp)), so the tests can push complex
inputs through it for complex-step derivatives.  It is pinned to the C
oracle's forward; the gradients are pinned to complex-step and central
finite-difference derivatives of it.  Layouts are the C oracle's: q, k
[B,T,H_qk,K]; v, out [B,T,H,V]; g_raw [B,T,H,K] or [B,T,H]; beta_logits
[B,T,H]; A_log [H]; states [C,H,V,K] with state[c,h,v,kk] = S[kk][v].
"""

from __future__ import annotations

import numpy as np

EPS = 1e-6


def _softplus(x):
    if np.iscomplexobj(x):
        return np.log1p(np.exp(x))  # analytic form for complex-step inputs
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _chains(B, T, H, cu_seqlens):
    """(chain slot c, batch row b, first token, last token + 1, value head h) for every chain."""
    out = []
    if cu_seqlens is None:
        for b in range(B):
            for h in range(H):
                out.append((b, b, 0, T, h))
    else:
        cu = np.asarray(cu_seqlens)
        for n in range(len(cu) - 1):
            for h in range(H):
                out.append((n, 0, int(cu[n]), int(cu[n + 1]), h))
    return out


def _token_forward(qt, kt, vt, grt, bt, a_log, S, scale):
    """One token of one chain.  Returns the values the backward walk needs."""
    nq = np.sqrt((qt * qt).sum() + EPS)
    nk = np.sqrt((kt * kt).sum() + EPS)
    qn, kn = qt / nq, kt / nk
    g = -np.exp(a_log) * _softplus(grt)
    D = np.exp(g)
    beta = _sigmoid(bt)
    Sp = (D * np.ones(S.shape[0]))[:, None] * S
    r = vt - Sp.T @ kn
    u = beta * r
    S_new = Sp + np.outer(kn, u)
    o = scale * (S_new.T @ qn)
    return dict(nq=nq, nk=nk, qn=qn, kn=kn, g=g, D=D, beta=beta, Sp=Sp, r=r, u=u, S_prev=S, S=S_new, o=o)


def kda_fwd(q, k, v, g_raw, beta_logits, A_log, scale, gate_per_channel=True, initial_state=None,
            cu_seqlens=None):
    """Forward (token by token).  Works for real or complex inputs.  Returns (out, final_state)."""
    B, T, H_qk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    G = H // H_qk
    dt = np.result_type(q, k, v, g_raw, beta_logits, A_log, 1.0 if initial_state is None else initial_state)
    chains = _chains(B, T, H, cu_seqlens)
    C = B if cu_seqlens is None else len(cu_seqlens) - 1
    out = np.zeros((B, T, H, V), dtype=dt)
    final = np.zeros((C, H, V, K), dtype=dt)
    for c, b, t0, t1, h in chains:
        S = np.zeros((K, V), dtype=dt) if initial_state is None else np.array(initial_state[c, h].T, dtype=dt)
        for t in range(t0, t1):
            st = _token_forward(q[b, t, h // G], k[b, t, h // G], v[b, t, h], g_raw[b, t, h], beta_logits[b, t, h],
                                A_log[h], S, scale)
            out[b, t, h] = st["o"]
            S = st["S"]
        final[c, h] = S.T
    return out, final


def kda_bwd(q, k, v, g_raw, beta_logits, A_log, scale, dout, dfinal, gate_per_channel=True, initial_state=None,
            cu_seqlens=None):
    """Gradients of L = sum(dout * out) + sum(dfinal * final_state).

    Returns a dict with dq, dk, dv, dg_raw, dbeta_logits, dA_log and
    dinitial_state (the last shaped like the states; zeros if there is no
    initial state, which is then the zero state)."""
    q, k, v, g_raw = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g_raw))
    beta_logits, A_log = np.asarray(beta_logits, np.float64), np.asarray(A_log, np.float64)
    B, T, H_qk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    G = H // H_qk
    C = B if cu_seqlens is None else len(cu_seqlens) - 1
    grads = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dg_raw=np.zeros_like(g_raw),
                 dbeta_logits=np.zeros_like(beta_logits), dA_log=np.zeros_like(A_log),
                 dinitial_state=np.zeros((C, H, V, K)))
    for c, b, t0, t1, h in _chains(B, T, H, cu_seqlens):
        hq = h // G
        a_log = A_log[h]
        # forward walk, keeping every token's intermediate values
        S = np.zeros((K, V)) if initial_state is None else np.array(initial_state[c, h].T, dtype=np.float64)
        steps = []
        for t in range(t0, t1):
            steps.append(_token_forward(q[b, t, hq], k[b, t, hq], v[b, t, h], g_raw[b, t, h], beta_logits[b, t, h],
                                        a_log, S, scale))
            S = steps[-1]["S"]
        # backward walk
        dS = np.array(dfinal[c, h].T, dtype=np.float64)   # dL/dS_t, K x V
        for t in range(t1 - 1, t0 - 1, -1):
            st = steps[t - t0]
            do = dout[b, t, h]
            # o = scale S_t^T qn
            dS = dS + scale * np.outer(st["qn"], do)
            dqn = scale * (st["S"] @ do)
            # S_t = S' + kn u^T
            du = dS.T @ st["kn"]
            dkn = dS @ st["u"]
            dSp = dS.copy()
            # u = b (v - S'^T kn)
            dbeta = du @ st["r"]
            grads["dv"][b, t, h] += st["beta"] * du
            dr = st["beta"] * du
            dSp -= np.outer(st["kn"], dr)
            dkn -= st["Sp"] @ dr
            # S' = Diag(D) S_{t-1}
            dD = (dSp * st["S_prev"]).sum(axis=1)
            Dvec = st["D"] * np.ones(K)
            dS = Dvec[:, None] * dSp
            # D = exp(g), g = -exp(A_log) softplus(g_raw)
            dg = dD * Dvec
            if not gate_per_channel:
                dg = dg.sum()
            dsp = dg * (-np.exp(a_log))
            grads["dg_raw"][b, t, h] += dsp * _sigmoid(g_raw[b, t, h])
            grads["dA_log"][h] += np.sum(dg * st["g"])
            # b = sigmoid(beta_logit)
            grads["dbeta_logits"][b, t, h] += dbeta * st["beta"] * (1.0 - st["beta"])
            # qn = q / sqrt(|q|^2 + eps), kn likewise
            qv, kv = q[b, t, hq], k[b, t, hq]
            grads["dq"][b, t, hq] += dqn / st["nq"] - qv * (qv @ dqn) / st["nq"] ** 3
            grads["dk"][b, t, hq] += dkn / st["nk"] - kv * (kv @ dkn) / st["nk"] ** 3
        grads["dinitial_state"][c, h] = dS.T
    return grads
