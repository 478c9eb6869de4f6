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
    compare(got, ref, label, inp["g_raw"])
