"""GPU parity on seeded random configurations (a deterministic list, the same on every run).

Each case draws, from its own seed: the gate mode (per key channel or one per
token-head), q/k heads and the value heads grouped on them, dense rows or
packed sequences (empty ones allowed), lengths that are rarely a multiple of
64, the state (none, fp32, bf16), a gate regime (the workloads', slow decay,
decay spans that need the exact fallback, or correlated keys with strong
writes and no decay) and, for per-channel gates, the precise path.  Two more
cases are large enough (>= 256 (chunk, q/k head) jobs) for the grouped
kernel's shared records.  Every case is checked against the oracle with the
pooled and the per-(chain, head) bars.
"""

import numpy as np
import pytest
import torch

from chunked_gated_delta_10_amd.inputs import make_inputs
import kda_util as U

pytestmark = pytest.mark.gpu

REGIMES = {
    "workload": dict(A_log=(-1.0, 1.0)),
    "slow decay": dict(A_log=(-6.0, -4.0)),
    "harsh decay": dict(A_log=(2.0, 3.0)),
    "correlated keys": dict(A_log=-8.0, k_noise=0.5, b_shift=4.6),
}


def draw_case(i):
    rng = np.random.default_rng(900 + i)
    per_channel = bool(rng.integers(0, 2))
    H_qk = int(rng.choice([1, 2, 4]))
    H = H_qk * int(rng.choice([1, 2, 3]))
    regime = str(rng.choice(sorted(REGIMES)))
    state = str(rng.choice(["none", "fp32", "bf16"]))
    precise = per_channel and bool(rng.integers(0, 3) == 0)
    kw = dict(REGIMES[regime], gate_per_channel=per_channel, seed=1000 + i)
    if state != "none":
        kw["state_std"] = 0.05
    if rng.integers(0, 2):
        N = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.integers(0, 400, N)]
        if sum(lens) == 0:
            lens[0] = 1
        inp = make_inputs(1, sum(lens), H, H_qk, N=N, lengths=lens, **kw)
        shape = "packed %s" % lens
    else:
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 600))
        inp = make_inputs(B, T, H, H_qk, **kw)
        shape = "B=%d T=%d" % (B, T)
    what = "case %d: %s H=%d H_qk=%d %s gate, %s, state %s%s" % (
        i, shape, H, H_qk, "per-channel" if per_channel else "scalar", regime, state, ", precise" if precise else "")
    sdt = torch.bfloat16 if state == "bf16" else torch.float32
    return inp, sdt, precise, what


@pytest.mark.parametrize("i", range(24))
def test_random_configuration(i, monkeypatch):
    inp, sdt, precise, what = draw_case(i)
    if precise:
        monkeypatch.setenv("KDA_PRECISE", "1")
    print(what, flush=True)
    out, fin = U.run_gpu(inp, sdt)
    ref_out, ref_fin = U.run_oracle(U.state_as_stored(inp, sdt))
    U.assert_parity(out, fin, ref_out, ref_fin, sdt, what, cu_seqlens=inp.get("cu_seqlens"))


@pytest.mark.parametrize("regime", ["workload", "harsh decay"])
def test_random_grouped_kernel_configuration(regime):
    # B=2, T=4100, H_qk=2: 2 x 65 x 2 = 260 (chunk, q/k head) jobs take the grouped kernel
    rng = np.random.default_rng(77 if regime == "workload" else 78)
    H = 2 * int(rng.choice([2, 3, 4]))
    inp = make_inputs(2, 4100, H, 2, gate_per_channel=False, state_std=0.05, seed=int(rng.integers(1 << 30)),
                      **REGIMES[regime])
    what = "grouped kernel B=2 T=4100 H=%d H_qk=2, %s" % (H, regime)
    print(what, flush=True)
    out, fin = U.run_gpu(inp)
    ref_out, ref_fin = U.run_oracle(inp)
    U.assert_parity(out, fin, ref_out, ref_fin, torch.float32, what)
