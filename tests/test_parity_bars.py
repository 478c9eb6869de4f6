"""The parity bars themselves (CPU only): an error confined to one chain must
fail the per-(chain, head) check even where the pooled norms would pass it,
and an all-zero output must fail."""

import numpy as np
import pytest

from chunked_gated_delta_10_amd.inputs import make_inputs
import kda_util as U


@pytest.fixture(scope="module")
def reference():
    # 8 rows x 4 heads = 32 chains with mild gates, so every chain's output
    # has a similar norm and one chain is 1/32 of the pooled norm
    inp = make_inputs(8, 64, 4, 4, state_std=0.02, seed=31, A_log=(-4.0, -2.0))
    ref_out, ref_fin = U.run_oracle(inp)
    rng = np.random.default_rng(5)
    # rounding-sized relative noise everywhere (the size of a bf16 output rounding)
    out = ref_out * (1.0 + rng.uniform(-2.0 ** -9, 2.0 ** -9, ref_out.shape))
    fin = ref_fin * (1.0 + rng.uniform(-2.0 ** -12, 2.0 ** -12, ref_fin.shape))
    return ref_out, ref_fin, out, fin


def test_clean_result_passes(reference):
    ref_out, ref_fin, out, fin = reference
    U.assert_parity(out, fin, ref_out, ref_fin, what="rounding noise only")


def test_output_error_in_one_chain_fails_only_per_chain(reference):
    ref_out, ref_fin, out, fin = reference
    bad = out.copy()
    bad[3, :, 3] *= 1.02  # row 3, head 3: 2% off
    sel = ~np.isnan(ref_out)
    assert U.rel_l2(bad[sel], ref_out[sel]) <= U.OUT_REL          # the pooled norm hides it
    assert np.max(np.abs(bad - ref_out)) <= U.OUT_MAXABS
    with pytest.raises(AssertionError, match="per-chain output bar"):
        U.assert_parity(bad, fin, ref_out, ref_fin, what="one chain 2% off")


def test_state_error_in_one_chain_fails_only_per_chain(reference):
    ref_out, ref_fin, out, fin = reference
    bad = fin.copy()
    bad[3, 3] *= 1.004
    assert U.rel_l2(bad, ref_fin) <= U.STATE_REL_FP32
    with pytest.raises(AssertionError, match="per-chain final-state bar"):
        U.assert_parity(out, bad, ref_out, ref_fin, what="one state 0.4% off")


def test_packed_chains_are_split_by_cu_seqlens():
    lens = [30, 0, 70, 28]
    inp = make_inputs(1, sum(lens), 2, 2, state_std=0.02, N=len(lens), lengths=lens, seed=32, A_log=(-4.0, -2.0))
    ref_out, ref_fin = U.run_oracle(inp)
    out = ref_out.copy()
    out[0, 30 + 0:30 + 70, 1] *= 1.02  # sequence 2 (the empty one is sequence 1), head 1
    per = {(c, h): (o, f) for c, h, o, f in U.chain_errors(out, ref_fin, ref_out, ref_fin, inp["cu_seqlens"])}
    assert len(per) == 8
    assert abs(per[(2, 1)][0] - 0.02) < 1e-9
    assert all(o == 0.0 for (c, h), (o, f) in per.items() if (c, h) != (2, 1))


def test_zero_output_fails():
    inp = make_inputs(1, 128, 2, 2, seed=33)
    ref_out, ref_fin = U.run_oracle(inp)
    with pytest.raises(AssertionError):
        U.assert_parity(np.zeros_like(ref_out), ref_fin, ref_out, ref_fin, what="zero output")


def test_backward_bars_catch_an_error_confined_to_one_chain():
    # gradients of 8 rows x 4 heads with rounding-sized noise pass; the same with a 2% error in one
    # (row, head) of dv passes the pooled bar but fails the per-chain one
    from test_gpu_backward import compare
    rng = np.random.default_rng(7)
    B, T, H, D = 8, 40, 4, 128
    ref = {"dq": rng.standard_normal((B, T, H, D)), "dk": rng.standard_normal((B, T, H, D)),
           "dv": rng.standard_normal((B, T, H, D)), "dg_raw": rng.standard_normal((B, T, H)),
           "dbeta_logits": rng.standard_normal((B, T, H)), "dA_log": rng.standard_normal(H),
           "dinitial_state": rng.standard_normal((B, H, D, D))}
    g_raw = np.zeros((B, T, H), dtype=np.uint16)  # bf16 zeros: only dA_log's condition reads it
    got = {n: v * (1.0 + rng.uniform(-2.0 ** -11, 2.0 ** -11, np.shape(v))) for n, v in ref.items()}
    ref["dA_log"] = got["dA_log"].copy()
    compare(got, ref, "noise only", g_raw)
    bad = dict(got)
    bad["dv"] = got["dv"].copy()
    bad["dv"][3, :, 2] *= 1.02
    pooled = np.linalg.norm(bad["dv"] - ref["dv"]) / np.linalg.norm(ref["dv"])
    assert pooled < 5e-3
    with pytest.raises(AssertionError, match="per chain"):
        compare(bad, ref, "one chain off by 2%", g_raw)


def test_backward_dinitial_state_absolute_bar():
    # dinitial_state entries all far under fp16's range (harsh decays): zero from the kernel passes against
    # 1e-9-sized reference values; at ordinary magnitudes an error of 1e-3 in one slice still fails
    from test_gpu_backward import compare
    rng = np.random.default_rng(8)
    B, T, H, D = 2, 40, 2, 128
    ref = {"dq": rng.standard_normal((B, T, H, D)), "dk": rng.standard_normal((B, T, H, D)),
           "dv": rng.standard_normal((B, T, H, D)), "dg_raw": rng.standard_normal((B, T, H)),
           "dbeta_logits": rng.standard_normal((B, T, H)), "dA_log": np.zeros(H),
           "dinitial_state": 1e-9 * rng.standard_normal((B, H, D, D))}
    g_raw = np.zeros((B, T, H), dtype=np.uint16)
    got = {n: v.copy() for n, v in ref.items()}
    got["dinitial_state"] = np.zeros_like(ref["dinitial_state"])
    compare(got, ref, "tiny dinitial_state flushed to zero", g_raw)
    ref["dinitial_state"] = 1e-2 * rng.standard_normal((B, H, D, D))
    got["dinitial_state"] = ref["dinitial_state"].copy()
    got["dinitial_state"][1, 0] += 1e-3 * rng.standard_normal((D, D))
    with pytest.raises(AssertionError, match="dinitial_state"):
        compare(got, ref, "one dinitial_state slice off by 1e-3", g_raw)
