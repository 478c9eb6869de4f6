"""GPU parity on seeded random configurations of medium size (a deterministic list).

The small random cases (tests/test_gpu_random_shapes.py) keep every chain on a
workgroup of its own.  These draw up to 12 packed sequences of up to 2500
tokens, or up to 4 rows, over up to 64 value heads grouped on up to 16 q/k
heads, so that chains outnumber the CUs' one-tile slots (two-tile recurrence,
grids in rounds) and the grouped kernel shares q/k records; states fp32 or
bf16, four gate regimes, both gate modes.  A few backward cases of moderate
size go with them.  Every case is checked against the oracle with the pooled
and the per-(chain, head) bars.
"""

import numpy as np
import pytest
import torch

from chunked_gated_delta_10_amd.inputs import make_inputs
import kda_util as U
from test_gpu_backward import compare, run_gpu_bwd, run_oracle_bwd, upstream

pytestmark = pytest.mark.gpu

REGIMES = {
    "workload": dict(A_log=(-1.0, 1.0)),
    "slow decay": dict(A_log=(-6.0, -4.0)),
    "harsh decay": dict(A_log=(2.0, 3.0)),
    "correlated keys": dict(A_log=-8.0, k_noise=0.5, b_shift=4.6),
}


def draw(i, big):
    rng = np.random.default_rng(50000 + i)
    per_channel = bool(rng.integers(0, 2))
    H_qk = int(rng.choice([1, 2, 4, 8, 16] if big else [1, 2, 4]))
    H = H_qk * int(rng.choice([1, 2, 4] if big else [1, 2, 3]))
    if not per_channel and H > H_qk and big:
        H = min(H, 32)
    regime = str(rng.choice(sorted(REGIMES)))
    kw = dict(REGIMES[regime], gate_per_channel=per_channel, seed=60000 + i)
    if rng.integers(0, 2):
        kw["state_std"] = 0.05
    tmax = 2500 if big else 700
    if rng.integers(0, 2):
        N = int(rng.integers(1, 13 if big else 6))
        lens = [int(x) for x in rng.integers(0, tmax, N)]
        if sum(lens) == 0:
            lens[0] = 64
        inp = make_inputs(1, sum(lens), H, H_qk, N=N, lengths=lens, **kw)
        shape = "packed %s" % lens
    else:
        B, T = int(rng.integers(1, 5 if big else 3)), int(rng.integers(1, tmax))
        inp = make_inputs(B, T, H, H_qk, **kw)
        shape = "B=%d T=%d" % (B, T)
    what = "medium case %d: %s H=%d H_qk=%d %s gate, %s, state %s" % (
        i, shape, H, H_qk, "per-channel" if per_channel else "scalar", regime,
        "none" if inp["initial_state"] is None else "fp32")
    return inp, what


@pytest.mark.parametrize("i", range(10))
def test_medium_forward_configuration(i):
    inp, what = draw(i, True)
    sdt = torch.bfloat16 if (i % 3 == 0 and inp["initial_state"] is not None) else torch.float32
    print(what, "bf16 state" if sdt == torch.bfloat16 else "", flush=True)
    out, fin = U.run_gpu(inp, sdt)
    ref_out, ref_fin = U.run_oracle(U.state_as_stored(inp, sdt))
    U.assert_parity(out, fin, ref_out, ref_fin, sdt, what, cu_seqlens=inp.get("cu_seqlens"))


@pytest.mark.parametrize("i", [0, 3, 6, 8])  # two per-channel and two scalar-gate draws
def test_medium_backward_configuration(i):
    inp, what = draw(1000 + i, False)
    print(what, flush=True)
    dout, dfinal = upstream(inp, 70000 + i, 0.1 if i % 2 else None)
    compare(run_gpu_bwd(inp, dout, dfinal), run_oracle_bwd(inp, dout, dfinal), what, inp["g_raw"],
            inp.get("cu_seqlens"))
