"""Design check for the backward pass in chunk (UT / WY) form, CPU only.

The backward oracle walks tokens in reverse.  A GPU backward would instead
walk 64-token chunks: recompute the state S_c entering every chunk (a
forward pass of the chunked recurrence), run the adjoint recurrence of the
chunk step in reverse,

    dU   = M^T dO' + Kbar dS'
    dS_c = Qhat^T dO' - W^T dU + Diag(exp(Gamma_L)) dS'      (dO' = scale dO)

and turn the per-chunk adjoints into input gradients through the reverse of
the UT transform (dA = -T^T dT T^T on the strictly lower triangle) and of
the decay factoring.  This file writes that algorithm out in fp64 numpy
(plain exponentials: T <= 40 keeps them in range) and checks it against the
oracle's gradients, for chunk sizes that split the sequence raggedly, both
gate modes, grouped value heads, packed sequences and an initial state.  It
pins the derivation a kernel would follow, not a kernel.
"""

import numpy as np
import pytest

import oracle
from oracle import kda_backward as KB

EPS = 1e-6


def _prologue(q, k, g_raw, beta_logit, a_log, per_channel, K):
    nq = np.sqrt((q * q).sum(-1, keepdims=True) + EPS)
    nk = np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
    sp = np.logaddexp(0.0, g_raw)
    g = -np.exp(a_log) * sp
    if not per_channel:
        g = np.repeat(g[:, None], K, axis=1)
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    return q / nq, k / nk, nq, nk, g, beta


def _chunk_quantities(qn, kn, g, beta, v):
    L = qn.shape[0]
    G = np.cumsum(g, axis=0)
    GL = G[-1]
    Kh, Qh, Kt, Kb = np.exp(G) * kn, np.exp(G) * qn, np.exp(-G) * kn, np.exp(GL - G) * kn
    A = np.tril(beta[:, None] * (Kh @ Kt.T), -1)
    M = np.tril(Qh @ Kt.T)
    T = np.linalg.inv(np.eye(L) + A)
    W = T @ (beta[:, None] * Kh)
    Uv = T @ (beta[:, None] * v)
    return dict(G=G, GL=GL, Kh=Kh, Qh=Qh, Kt=Kt, Kb=Kb, A=A, M=M, T=T, W=W, Uv=Uv)


def chunked_backward_one_chain(q, k, v, g_raw, beta_logit, a_log, scale, dout, dfinal, S0, per_channel, C):
    """One (sequence, value head) chain.  q, k [T,K]; v, dout [T,V]; g_raw [T,K] or [T];
    beta_logit [T]; S0, dfinal [K,V] (S[k][v]).  Returns the gradients as a dict."""
    T_, K = q.shape
    qn, kn, nq, nk, g, beta = _prologue(q, k, g_raw, beta_logit, a_log, per_channel, K)
    bounds = [(s, min(s + C, T_)) for s in range(0, T_, C)]
    # forward over chunks, keeping the state entering each chunk (what a kernel would store or recompute)
    S = S0.copy()
    entering, cache = [], []
    for s, e in bounds:
        cq = _chunk_quantities(qn[s:e], kn[s:e], g[s:e], beta[s:e], v[s:e])
        entering.append(S.copy())
        U = cq["Uv"] - cq["W"] @ S
        cq["U"] = U
        cache.append(cq)
        S = np.exp(cq["GL"])[:, None] * S + cq["Kb"].T @ U
    dqn, dkn, dv = np.zeros_like(qn), np.zeros_like(kn), np.zeros_like(v)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    dS = dfinal.copy()
    for (s, e), cq, Sc in zip(reversed(bounds), reversed(cache), reversed(entering)):
        L = e - s
        dO = scale * dout[s:e]
        U, M, T, W, Kb, Kh, Kt, Qh = (cq[n] for n in ("U", "M", "T", "W", "Kb", "Kh", "Kt", "Qh"))
        b = beta[s:e]
        # adjoint of the chunk step
        dU = M.T @ dO + Kb @ dS
        dQh = dO @ Sc.T
        dM = np.tril(dO @ U.T)
        dKb = U @ dS.T
        dW = -dU @ Sc.T
        dexpGL = (dS * Sc).sum(axis=1)
        dS_prev = Qh.T @ dO - W.T @ dU + np.exp(cq["GL"])[:, None] * dS
        # Uv = T diag(b) V and W = T diag(b) Khat
        Y = T.T @ dU
        dv[s:e] += b[:, None] * Y
        db = (Y * v[s:e]).sum(1)
        Z = T.T @ dW
        dKh = b[:, None] * Z
        db += (Z * Kh).sum(1)
        dT = dU @ (b[:, None] * v[s:e]).T + dW @ (b[:, None] * Kh).T
        # T = (I + A)^-1 and A = strict_lower(diag(b) Khat Ktilde^T)
        dA = np.tril(-T.T @ dT @ T.T, -1)
        Gm = Kh @ Kt.T
        db += (dA * Gm).sum(1)
        dGm = b[:, None] * dA
        dKh += dGm @ Kt
        dKt = dGm.T @ Kh
        # M = lower(Qhat Ktilde^T)
        dQh += dM @ Kt
        dKt += dM.T @ Qh
        # decay factoring back to qn, kn and the cumulative gates
        E, Ei, EL = np.exp(cq["G"]), np.exp(-cq["G"]), np.exp(cq["GL"] - cq["G"])
        dqn[s:e] += E * dQh
        dkn[s:e] += E * dKh + Ei * dKt + EL * dKb
        dGam = Qh * dQh + Kh * dKh - Kt * dKt - Kb * dKb
        dGam[L - 1] += (Kb * dKb).sum(0) + np.exp(cq["GL"]) * dexpGL
        dg[s:e] += np.cumsum(dGam[::-1], axis=0)[::-1]
        dbeta[s:e] += db
        dS = dS_prev
    # prologue
    dq = dqn / nq - q * (q * dqn).sum(-1, keepdims=True) / nq ** 3
    dk = dkn / nk - k * (k * dkn).sum(-1, keepdims=True) / nk ** 3
    if not per_channel:
        dg = dg.sum(1)
    sig = 1.0 / (1.0 + np.exp(-g_raw))
    dg_raw = dg * (-np.exp(a_log)) * sig
    g_tok = -np.exp(a_log) * np.logaddexp(0.0, g_raw)
    dA_log = (dg * g_tok).sum()
    dbl = dbeta * beta * (1 - beta)
    return dict(dq=dq, dk=dk, dv=dv, dg_raw=dg_raw, dbeta_logits=dbl, dA_log=dA_log, dinitial_state=dS)


def chunked_backward(x, dout, dfinal, scale, per_channel, C, cu=None):
    q, k, v, g_raw, bl, A_log, S0 = (x[n] for n in ("q", "k", "v", "g_raw", "beta_logits", "A_log", "initial_state"))
    B, T_, H_qk, K = q.shape
    H = v.shape[2]
    G = H // H_qk
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v), dg_raw=np.zeros_like(g_raw),
               dbeta_logits=np.zeros_like(bl), dA_log=np.zeros_like(A_log),
               dinitial_state=np.zeros_like(S0))
    spans = [(b, b, 0, T_) for b in range(B)] if cu is None else \
        [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    for c, b, t0, t1 in spans:
        for h in range(H):
            hq = h // G
            if t1 == t0:
                out["dinitial_state"][c, h] = dfinal[c, h]
                continue
            r = chunked_backward_one_chain(q[b, t0:t1, hq], k[b, t0:t1, hq], v[b, t0:t1, h], g_raw[b, t0:t1, h],
                                           bl[b, t0:t1, h], A_log[h], scale, dout[b, t0:t1, h], dfinal[c, h].T,
                                           S0[c, h].T, per_channel, C)
            out["dq"][b, t0:t1, hq] += r["dq"]
            out["dk"][b, t0:t1, hq] += r["dk"]
            out["dv"][b, t0:t1, h] = r["dv"]
            out["dg_raw"][b, t0:t1, h] = r["dg_raw"]
            out["dbeta_logits"][b, t0:t1, h] = r["dbeta_logits"]
            out["dA_log"][h] += r["dA_log"]
            out["dinitial_state"][c, h] = r["dinitial_state"].T
    return out


def draw(B=1, T=13, H=2, H_qk=2, K=6, V=5, per_channel=True, lens=None, seed=0):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((B, T, H_qk, K)), k=rng.standard_normal((B, T, H_qk, K)),
             v=rng.standard_normal((B, T, H, V)),
             g_raw=rng.standard_normal((B, T, H, K) if per_channel else (B, T, H)),
             beta_logits=rng.standard_normal((B, T, H)), A_log=rng.uniform(-2.0, 0.0, H))
    Cn = B if lens is None else len(lens)
    x["initial_state"] = 0.3 * rng.standard_normal((Cn, H, V, K))
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, cu, rng.standard_normal((B, T, H, V)), rng.standard_normal((Cn, H, V, K))


CASES = [
    (dict(per_channel=True), 4),
    (dict(per_channel=True), 5),             # ragged last chunk
    (dict(per_channel=True, T=16), 16),      # one chunk
    (dict(per_channel=False, H=4, H_qk=2, seed=1), 4),
    (dict(per_channel=True, H=4, H_qk=1, seed=2), 3),
    (dict(per_channel=True, lens=[5, 0, 8], seed=3), 4),
    (dict(per_channel=True, T=37, K=8, V=8, seed=4), 8),
]


@pytest.mark.parametrize("case,C", CASES)
def test_chunk_form_backward_matches_the_oracle(case, C):
    x, cu, dout, dfinal = draw(**case)
    per_channel = case["per_channel"]
    got = chunked_backward(x, dout, dfinal, 0.5, per_channel, C, cu)
    ref = KB.kda_bwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta_logits"], x["A_log"], 0.5, dout, dfinal,
                     gate_per_channel=per_channel, initial_state=x["initial_state"], cu_seqlens=cu)
    for name, r in ref.items():
        np.testing.assert_allclose(got[name], r, rtol=1e-9, atol=1e-10, err_msg=name)


def test_chunk_form_forward_state_matches_the_c_oracle():
    # the chunk states the backward recomputes are the forward's: same final state as the C oracle
    x, cu, dout, dfinal = draw(T=23, seed=5)
    q, k = x["q"][0, :, 0], x["k"][0, :, 0]
    qn, kn, _, _, g, beta = _prologue(q, k, x["g_raw"][0, :, 0], x["beta_logits"][0, :, 0], x["A_log"][0], True, 6)
    S = x["initial_state"][0, 0].T.copy()
    for s in range(0, 23, 4):
        cq = _chunk_quantities(qn[s:s + 4], kn[s:s + 4], g[s:s + 4], beta[s:s + 4], x["v"][0, s:s + 4, 0])
        S = np.exp(cq["GL"])[:, None] * S + cq["Kb"].T @ (cq["Uv"] - cq["W"] @ S)
    _, fin = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta_logits"], x["A_log"], 0.5,
                            initial_state=x["initial_state"])
    np.testing.assert_allclose(S.T, fin[0, 0], rtol=1e-11, atol=1e-12)


def scalar_gate_chunk_backward(q, k, v, g_raw, bl, a_log, scale, dout, dfinal, S0, C):
    """The scalar-gate (gated delta rule) special case in the form a kernel would use: every decay is a
    scalar per token, so the decay factors reduce to row scalings by e_r = exp(G_r), f_r = exp(G_L - G_r)
    and one 64 x 64 mask Lam[r, i] = exp(G_r - G_i) (r >= i, all <= 1) on the Gram matrices
    P = qn kn^T and Gm = kn kn^T: no exponential of a positive exponent appears anywhere."""
    T_, K = q.shape
    nq = np.sqrt((q * q).sum(-1, keepdims=True) + EPS)
    nk = np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
    qn, kn = q / nq, k / nk
    g = -np.exp(a_log) * np.logaddexp(0.0, g_raw)            # [T]
    beta = 1.0 / (1.0 + np.exp(-bl))
    bounds = [(s, min(s + C, T_)) for s in range(0, T_, C)]
    S = S0.copy()
    fw = []
    for s, e in bounds:
        G = np.cumsum(g[s:e])
        ee, ff, eL = np.exp(G), np.exp(G[-1] - G), np.exp(G[-1])
        Lam = np.tril(np.exp(np.minimum(G[:, None] - G[None, :], 0.0)))
        P, Gm = qn[s:e] @ kn[s:e].T, kn[s:e] @ kn[s:e].T
        M = P * Lam
        A = np.tril(beta[s:e, None] * Gm * Lam, -1)
        T = np.linalg.inv(np.eye(e - s) + A)
        R = v[s:e] - ee[:, None] * (kn[s:e] @ S)
        U = T @ (beta[s:e, None] * R)
        fw.append(dict(G=G, ee=ee, ff=ff, eL=eL, Lam=Lam, P=P, Gm=Gm, M=M, T=T, R=R, U=U, S=S.copy()))
        S = eL * S + kn[s:e].T @ (ff[:, None] * U)
    dqn, dkn, dv = np.zeros_like(qn), np.zeros_like(kn), np.zeros_like(v)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    dS = dfinal.copy()
    for (s, e), c in zip(reversed(bounds), reversed(fw)):
        dO = scale * dout[s:e]
        qc, kc, b, Sc = qn[s:e], kn[s:e], beta[s:e], c["S"]
        # adjoint chunk step (what the sequential kernel computes per value-column tile)
        dU = c["M"].T @ dO + c["ff"][:, None] * (kc @ dS)
        dS_prev = qc.T @ (c["ee"][:, None] * dO) - kc.T @ ((b * c["ee"])[:, None] * (c["T"].T @ dU)) + c["eL"] * dS
        # chunk-parallel gradients
        SdO = dO @ Sc.T                                        # [L, K]
        dqn[s:e] += c["ee"][:, None] * SdO
        de = (qc * SdO).sum(1)
        UdS = c["U"] @ dS.T                                    # [L, K]
        dkn[s:e] += c["ff"][:, None] * UdS
        df = (kc * UdS).sum(1)
        deL = (dS * Sc).sum()
        dM = np.tril(dO @ c["U"].T)
        Y = c["T"].T @ dU
        dR = b[:, None] * Y
        db = (Y * c["R"]).sum(1)
        dv[s:e] += dR
        kS = kc @ Sc
        dkn[s:e] -= c["ee"][:, None] * (dR @ Sc.T)
        de -= (dR * kS).sum(1)
        dT = dU @ (b[:, None] * c["R"]).T
        dA = np.tril(-c["T"].T @ dT @ c["T"].T, -1)
        db += (dA * c["Gm"] * c["Lam"]).sum(1)
        dGm = b[:, None] * dA * c["Lam"]
        dLam = b[:, None] * dA * c["Gm"] + dM * c["P"]
        dP = dM * c["Lam"]
        dkn[s:e] += (dGm + dGm.T) @ kc + dP.T @ qc
        dqn[s:e] += dP @ kc
        W = dLam * c["Lam"]
        dG = W.sum(1) - W.sum(0) + de * c["ee"] - df * c["ff"]
        dG[-1] += (df * c["ff"]).sum() + deL * c["eL"]
        dg[s:e] += np.cumsum(dG[::-1])[::-1]
        dbeta[s:e] += db
        dS = dS_prev
    dq = dqn / nq - q * (q * dqn).sum(-1, keepdims=True) / nq ** 3
    dk = dkn / nk - k * (k * dkn).sum(-1, keepdims=True) / nk ** 3
    sig = 1.0 / (1.0 + np.exp(-g_raw))
    return dict(dq=dq, dk=dk, dv=dv, dg_raw=dg * (-np.exp(a_log)) * sig, dbeta_logits=dbeta * beta * (1 - beta),
                dA_log=(dg * g).sum(), dinitial_state=dS)


@pytest.mark.parametrize("T,C,A_log", [(13, 4, -1.0), (40, 16, 0.5), (37, 8, 3.0)])
def test_scalar_gate_chunk_form_backward_matches_the_oracle(T, C, A_log):
    rng = np.random.default_rng(T + C)
    K = V = 6
    q, k, v = rng.standard_normal((T, K)), rng.standard_normal((T, K)), rng.standard_normal((T, V))
    g_raw, bl = rng.standard_normal(T), rng.standard_normal(T)
    S0, dout, dfinal = 0.3 * rng.standard_normal((K, V)), rng.standard_normal((T, V)), rng.standard_normal((K, V))
    got = scalar_gate_chunk_backward(q, k, v, g_raw, bl, A_log, 0.5, dout, dfinal, S0, C)
    ref = KB.kda_bwd(q[None, :, None], k[None, :, None], v[None, :, None], g_raw[None, :, None], bl[None, :, None],
                     np.array([A_log]), 0.5, dout[None, :, None], dfinal.T[None, None], gate_per_channel=False,
                     initial_state=S0.T[None, None])
    squeeze = dict(dq=lambda a: a[0, :, 0], dk=lambda a: a[0, :, 0], dv=lambda a: a[0, :, 0],
                   dg_raw=lambda a: a[0, :, 0], dbeta_logits=lambda a: a[0, :, 0], dA_log=lambda a: a[0],
                   dinitial_state=lambda a: a[0, 0].T)
    for name, r in ref.items():
        np.testing.assert_allclose(got[name], squeeze[name](r), rtol=1e-9, atol=1e-10, err_msg=name)
