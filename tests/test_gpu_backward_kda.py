"""GPU parity of the backward pass with one decay per key channel (KDA: g_raw
[B, T, H, 128]; kda.bwd / kda.bwd_varlen with gate_per_channel = 1 through the
C ABI) against the fp64 backward oracle, with the bars and helpers of the
scalar-gate tests (test_gpu_backward.py).

The per-channel decays enter through the masked Gram matrices: across 16-token
blocks they are folded into fp16 matrix-core operands (every factor <= 1),
inside a block each exp(Gamma_r - Gamma_i) is evaluated exactly in fp32, so
harsh gates (decays far below fp16's range inside one block) are covered.
"""

import numpy as np
import pytest

from chunked_gated_delta_10_amd.inputs import make_inputs

from test_gpu_backward import NAMES, compare, run_gpu_bwd, run_oracle_bwd, upstream

pytestmark = pytest.mark.gpu

CASES = [
    # (label, make_inputs kwargs, dfinal std or None)
    ("kda dense B=1 T=64 H=1 no state", dict(B=1, T=64, H=1, H_qk=1, seed=171), None),
    ("kda dense B=2 T=200 H=2 state", dict(B=2, T=200, H=2, H_qk=2, state_std=0.05, seed=172), 0.1),
    ("kda dense B=1 T=1 H=2", dict(B=1, T=1, H=2, H_qk=2, state_std=0.05, seed=173), 0.1),
    ("kda grouped B=1 T=130 H=4 H_qk=2", dict(B=1, T=130, H=4, H_qk=2, state_std=0.05, seed=174), 0.1),
    ("kda grouped B=1 T=97 H=6 H_qk=1", dict(B=1, T=97, H=6, H_qk=1, seed=175), 0.1),
    ("kda harsh decay A_log=1.5", dict(B=1, T=150, H=2, H_qk=2, A_log=1.5, state_std=0.05, seed=176), 0.1),
    ("kda weak decay A_log=-4", dict(B=1, T=150, H=2, H_qk=2, A_log=-4.0, state_std=0.05, seed=177), 0.1),
    ("kda varlen N=5 with empty and 1-token",
     dict(B=1, T=230, H=2, H_qk=2, N=5, lengths=[64, 0, 1, 100, 65], state_std=0.05, seed=178), 0.1),
    ("kda correlated keys, strong writes, no decay",
     dict(B=1, T=192, H=2, H_qk=2, A_log=-8.0, k_noise=0.5, b_shift=4.6, seed=179), 0.1),
]


@pytest.mark.parametrize("label,kw,dstd", CASES, ids=[c[0] for c in CASES])
def test_kda_backward_matches_the_oracle(label, kw, dstd):
    inp = make_inputs(gate_per_channel=True, **{"A_log": (-1.0, 1.0), **kw})
    dout, dfinal = upstream(inp, kw["seed"] + 500, dstd)
    got = run_gpu_bwd(inp, dout, dfinal)
    ref = run_oracle_bwd(inp, dout, dfinal)
    compare(got, ref, label, inp["g_raw"], inp.get("cu_seqlens"))


def test_kda_backward_extreme_decay():
    # per-token decays of e^-60 and below (A_log = 3, g_raw ~ N(3, 1)): every cross-block factor and most
    # in-block ones underflow and the gate gradients are tiny, formed from products that are not.  The
    # token gradients are held to the usual bars; dinitial_state (about e^-60 per token of the sequence in
    # the fp64 oracle, zero in fp32) to an absolute 1e-6 of dfinal's scale; dA_log, a sum of 19,200 tiny
    # terms of both signs, to 0.1 of its condition (measured 0.063: the terms' small relative errors add
    # up against a sum they nearly cancel in).
    from test_gpu_backward import dA_log_condition, rel_l2
    inp = make_inputs(1, 150, 2, 2, gate_per_channel=True, A_log=3.0, g_shift=3.0, state_std=0.05, seed=180)
    dout, dfinal = upstream(inp, 680)
    got, ref = run_gpu_bwd(inp, dout, dfinal), run_oracle_bwd(inp, dout, dfinal)
    for n in ("dq", "dk", "dv", "dg_raw", "dbeta_logits"):
        rel = rel_l2(got[n], ref[n])
        print("kda extreme decay", n, "%.1e" % rel, flush=True)
        assert rel <= 5e-3, (n, rel)
    assert np.max(np.abs(got["dinitial_state"] - ref["dinitial_state"])) <= 1e-6 * np.max(np.abs(dfinal))
    cond = dA_log_condition(ref, inp["g_raw"])
    assert np.max(np.abs(got["dA_log"] - ref["dA_log"]) / cond) <= 0.1


def test_kda_backward_grouped_heads_long_sequence():
    # 64 chunks, two value heads on each q/k head
    inp = make_inputs(1, 4096, 8, 4, gate_per_channel=True, A_log=(-1.0, 1.0), state_std=0.05, seed=181)
    dout, dfinal = upstream(inp, 681)
    compare(run_gpu_bwd(inp, dout, dfinal), run_oracle_bwd(inp, dout, dfinal), "kda grouped T=4096 H=8 H_qk=4",
            inp["g_raw"])


def test_kda_backward_benchmark_shape_sampled_heads():
    # the KDA backward benchmark shape (B=2, T=16384, H=16, fp32 initial state): 8192 (chunk, head) jobs and
    # chains of 256 chunks; heads 0 and 15 of both rows against the oracle
    from chunked_gated_delta_10_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["kda_bwd"]
    inp = workload_inputs("kda_bwd")
    dout, dfinal = upstream(inp, w.seed + 500)
    got = run_gpu_bwd(inp, dout, dfinal)
    heads = [0, 15]
    ref = run_oracle_bwd(inp, dout, dfinal, heads=heads)
    sub = {n: (got[n][heads] if n == "dA_log" else got[n][:, heads] if n == "dinitial_state"
               else got[n][:, :, heads]) for n in NAMES}
    compare(sub, ref, "kda_bwd shape B=2 T=16384 H=16, heads 0 and 15", inp["g_raw"][:, :, heads])


# ---- seeded random configurations -----------------------------------------------------------------
REGIMES = {
    "workload": dict(A_log=(-1.0, 1.0)),
    "slow decay": dict(A_log=(-6.0, -4.0)),
    "harsh decay": dict(A_log=(2.0, 3.0)),
    "correlated keys": dict(A_log=-8.0, k_noise=0.5, b_shift=4.6),
}


def draw_kda_bwd_case(i):
    """Case i: q/k heads and grouping, dense rows or packed sequences (empty ones allowed), lengths rarely a
    multiple of 64, initial state and dfinal present or not, and a gate regime, all from seed 5100 + i."""
    rng = np.random.default_rng(5100 + i)
    H_qk = int(rng.choice([1, 2, 4]))
    H = H_qk * int(rng.choice([1, 2, 3]))
    regime = str(rng.choice(sorted(REGIMES)))
    kw = dict(REGIMES[regime], gate_per_channel=True, seed=6100 + i)
    if rng.integers(0, 2):
        kw["state_std"] = 0.05
    dstd = 0.1 if rng.integers(0, 2) else None
    if rng.integers(0, 2):
        N = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 300, N)]
        if sum(lens) == 0:
            lens[0] = 1
        inp = make_inputs(1, sum(lens), H, H_qk, N=N, lengths=lens, **kw)
        shape = "packed %s" % lens
    else:
        B, T = int(rng.integers(1, 3)), int(rng.integers(1, 400))
        inp = make_inputs(B, T, H, H_qk, **kw)
        shape = "B=%d T=%d" % (B, T)
    what = "kda bwd case %d: %s H=%d H_qk=%d, %s, state %s, dfinal %s" % (
        i, shape, H, H_qk, regime, "none" if inp["initial_state"] is None else "fp32", dstd)
    return inp, dstd, what


@pytest.mark.parametrize("i", range(16))
def test_kda_backward_random_configuration(i):
    inp, dstd, what = draw_kda_bwd_case(i)
    print(what, flush=True)
    dout, dfinal = upstream(inp, 7100 + i, dstd)
    compare(run_gpu_bwd(inp, dout, dfinal), run_oracle_bwd(inp, dout, dfinal), what, inp["g_raw"],
            inp.get("cu_seqlens"))


def test_kda_backward_zero_tokens():
    # T = 0 with the per-channel gate: no token gradients; dinitial_state = dfinal, dA_log = 0
    import torch
    from chunked_gated_delta_10_amd import kda
    H = 2
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    df = torch.randn(3, H, 128, 128, device="cuda")
    g = kda.bwd_varlen(z(1, 0, H, 128), z(1, 0, H, 128), z(1, 0, H, 128), z(1, 0, H, 128),
                       torch.zeros(1, 0, H, device="cuda"), torch.zeros(H, device="cuda"), z(1, 0, H, 128),
                       torch.zeros(4, dtype=torch.int32, device="cuda"), dfinal=df)
    torch.cuda.synchronize()
    assert g["dg_raw"].shape == (1, 0, H, 128)
    assert torch.equal(g["dinitial_state"], df)
    assert torch.count_nonzero(g["dA_log"]) == 0
