"""Pins of the backward oracle (oracle/kda_backward.py), CPU only.

Its forward is tied to the C oracle's; its gradients are tied to
derivatives taken from that forward by two independent methods:
complex-step differentiation (exact to rounding: Im f(x + i h d) / h with
h = 1e-30 is the directional derivative, with no cancellation) and central
finite differences; plus a closed form at T = 1.  Every input is covered
(q, k, v, g_raw, beta_logits, A_log, initial_state), in both gate modes,
with grouped value heads and with packed sequences, so a dropped term, a
wrong sign or a transposed operand in any step of the reverse walk fails.
"""

import numpy as np
import pytest

import oracle
from oracle import kda_backward as KB

NAMES = ("q", "k", "v", "g_raw", "beta_logits", "A_log", "initial_state")


def draw(B=1, T=9, H=2, H_qk=2, K=4, V=4, per_channel=True, lens=None, seed=0, with_state=True):
    rng = np.random.default_rng(seed)
    x = dict(
        q=rng.standard_normal((B, T, H_qk, K)), k=rng.standard_normal((B, T, H_qk, K)),
        v=rng.standard_normal((B, T, H, V)),
        g_raw=rng.standard_normal((B, T, H, K) if per_channel else (B, T, H)),
        beta_logits=rng.standard_normal((B, T, H)), A_log=rng.uniform(-2.0, 0.5, H),
    )
    C = B if lens is None else len(lens)
    x["initial_state"] = rng.standard_normal((C, H, V, K)) * 0.3 if with_state else None
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    up = dict(dout=rng.standard_normal((B, T, H, V)), dfinal=rng.standard_normal((C, H, V, K)))
    return x, cu, up


def loss(x, cu, up, per_channel, scale=0.5):
    out, fin = KB.kda_fwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta_logits"], x["A_log"], scale,
                          gate_per_channel=per_channel, initial_state=x["initial_state"], cu_seqlens=cu)
    return np.sum(up["dout"] * out) + np.sum(up["dfinal"] * fin)


def grads(x, cu, up, per_channel, scale=0.5):
    return KB.kda_bwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta_logits"], x["A_log"], scale, up["dout"],
                      up["dfinal"], gate_per_channel=per_channel, initial_state=x["initial_state"], cu_seqlens=cu)


CASES = [
    dict(per_channel=True),
    dict(per_channel=False),
    dict(per_channel=True, H=4, H_qk=2, seed=1),            # grouped value heads
    dict(per_channel=False, H=4, H_qk=1, seed=2),
    dict(per_channel=True, lens=[4, 0, 5], seed=3),        # packed sequences, one empty
    dict(per_channel=True, K=8, V=4, T=12, seed=4),
    dict(per_channel=True, with_state=False, seed=5),
]


@pytest.mark.parametrize("case", CASES)
def test_forward_matches_the_c_oracle(case):
    x, cu, _ = draw(**case)
    out, fin = KB.kda_fwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta_logits"], x["A_log"], 0.5,
                          gate_per_channel=case["per_channel"], initial_state=x["initial_state"], cu_seqlens=cu)
    ro, rf = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g_raw"], x["beta_logits"], x["A_log"], 0.5,
                            gate_per_channel=case["per_channel"], initial_state=x["initial_state"], cu_seqlens=cu)
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fin, rf, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("case", CASES)
def test_gradients_match_complex_step(case):
    x, cu, up = draw(**case)
    g = grads(x, cu, up, case["per_channel"])
    rng = np.random.default_rng(100)
    h = 1e-30
    for name in NAMES:
        if x[name] is None:
            continue
        for _ in range(2):
            d = rng.standard_normal(x[name].shape)
            xc = {n: (None if a is None else a.astype(np.complex128)) for n, a in x.items()}
            xc[name] = xc[name] + 1j * h * d
            ref = loss(xc, cu, up, case["per_channel"]).imag / h
            got = np.sum(g["d" + name] * d)
            assert abs(got - ref) <= 1e-10 * max(1.0, abs(ref)), (name, got, ref)


def test_gradients_match_central_differences_elementwise():
    x, cu, up = draw(per_channel=True, H=4, H_qk=2, T=7, seed=6)
    g = grads(x, cu, up, True)
    eps = 1e-6
    rng = np.random.default_rng(7)
    for name in NAMES:
        for _ in range(3):
            idx = tuple(rng.integers(0, s) for s in x[name].shape)
            xp = {n: (None if a is None else a.copy()) for n, a in x.items()}
            xm = {n: (None if a is None else a.copy()) for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd = (loss(xp, cu, up, True) - loss(xm, cu, up, True)) / (2 * eps)
            assert abs(g["d" + name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, g["d" + name][idx], fd)


def test_single_token_from_zero_state_closed_form():
    # T = 1, S0 = 0:  o = scale * b (qn . kn) v, so dL/dv = scale * b (qn . kn) dout
    # and dL/dbeta_logit = scale * (qn . kn) (v . dout) * b (1 - b) (no final-state term)
    x, cu, up = draw(T=1, H=1, H_qk=1, K=4, V=4, with_state=False, seed=8)
    up["dfinal"][:] = 0.0
    g = grads(x, cu, up, True, scale=0.5)
    q, k = x["q"][0, 0, 0], x["k"][0, 0, 0]
    qn = q / np.sqrt(q @ q + 1e-6)
    kn = k / np.sqrt(k @ k + 1e-6)
    b = 1 / (1 + np.exp(-x["beta_logits"][0, 0, 0]))
    do = up["dout"][0, 0, 0]
    np.testing.assert_allclose(g["dv"][0, 0, 0], 0.5 * b * (qn @ kn) * do, rtol=1e-13)
    np.testing.assert_allclose(g["dbeta_logits"][0, 0, 0], 0.5 * (qn @ kn) * (x["v"][0, 0, 0] @ do) * b * (1 - b),
                               rtol=1e-12)
    # with no state and one token the decay multiplies a zero state: no gate gradient
    assert not np.any(g["dg_raw"]) and not np.any(g["dA_log"])


def test_a_wrong_sign_in_the_erase_term_is_caught():
    # mutation check of the pins themselves: flipping the erase term's sign in
    # the forward changes the loss's derivative, which the complex step sees
    x, cu, up = draw(seed=9)
    g = grads(x, cu, up, True)
    orig = KB._token_forward

    def flipped(qt, kt, vt, grt, bt, a_log, S, scale):
        st = orig(qt, kt, vt, grt, bt, a_log, S, scale)
        r = vt + st["Sp"].T @ st["kn"]
        u = st["beta"] * r
        S_new = st["Sp"] + np.outer(st["kn"], u)
        st.update(r=r, u=u, S=S_new, o=scale * (S_new.T @ st["qn"]))
        return st

    d = np.random.default_rng(10).standard_normal(x["k"].shape)
    KB._token_forward = flipped
    try:
        xc = {n: (None if a is None else a.astype(np.complex128)) for n, a in x.items()}
        xc["k"] = xc["k"] + 1j * 1e-30 * d
        ref = loss(xc, cu, up, True).imag / 1e-30
    finally:
        KB._token_forward = orig
    assert abs(np.sum(g["dk"] * d) - ref) > 1e-3 * abs(ref)
