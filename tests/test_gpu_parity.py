"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases span several chunks, ragged tails, every sub-chunk boundary and
the special paths (grouped heads, packed sequences, bf16 state, the exact
fallback for very large decay spans).  The full-size workloads run in the
same launch configuration the benchmark times and are compared on sampled
chains, which the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

from chunked_gated_delta_10_amd import kda
from chunked_gated_delta_10_amd.inputs import (SWEEP_HEAD_SHAPES, SWEEP_PATTERNS, WORKLOADS, make_inputs,
                                               sweep_inputs, workload_inputs)
import kda_util as U

pytestmark = pytest.mark.gpu


def check(inp, state_dtype=torch.float32, what="", chain_mask=None):
    print("case:", what, flush=True)
    out, fin = U.run_gpu(inp, state_dtype)
    ref_out, ref_fin = U.run_oracle(U.state_as_stored(inp, state_dtype), chain_mask=chain_mask)
    return U.assert_parity(out, fin, ref_out, ref_fin, state_dtype, what, cu_seqlens=inp.get("cu_seqlens"))


def test_tiny_workload():
    check(workload_inputs("kda_tiny"), what="kda_tiny B=1 T=512 H=4")


@pytest.mark.parametrize("T", [1, 16, 17, 63, 64, 65, 129, 300])
def test_ragged_lengths(T):
    inp = make_inputs(2, T, 3, 3, state_std=0.02, seed=100 + T)
    check(inp, what="ragged T=%d" % T)


def test_mild_gates_long_memory():
    inp = make_inputs(1, 700, 2, 2, state_std=0.02, seed=7, A_log=(-6.0, -4.0))
    check(inp, what="mild gates T=700")


def test_harsh_gates_take_exact_fallback():
    # exp(A_log) ~ 12..20 makes 16-token decay spans far beyond 2^-100
    inp = make_inputs(1, 200, 2, 2, state_std=0.02, seed=8, A_log=(2.5, 3.0))
    check(inp, what="harsh gates")


def test_mixed_gates_some_subchunks_fallback():
    inp = make_inputs(1, 256, 4, 4, state_std=0.02, seed=9, A_log=(-1.0, 2.2), g_shift=0.5)
    check(inp, what="mixed gates")


@pytest.mark.parametrize("H_qk,H,T", [(2, 8, 333), (1, 4, 64), (4, 4, 100)])
def test_scalar_gate_grouped_heads(H_qk, H, T):
    inp = make_inputs(1, T, H, H_qk, gate_per_channel=False, A_log=0.0, seed=11 + T)
    check(inp, what="scalar gate H_qk=%d H=%d T=%d" % (H_qk, H, T))


def test_scalar_gate_with_state():
    inp = make_inputs(2, 150, 4, 2, gate_per_channel=False, A_log=(-3.0, 0.0), state_std=0.05, seed=12)
    check(inp, what="scalar gate with state")


@pytest.mark.parametrize("B,T,H,H_qk,state_dtype", [
    (2, 150, 8, 2, torch.float32),    # 12 (chunk, q/k head) jobs: per-head kernel and records
    (6, 150, 8, 2, torch.bfloat16),   # 36 jobs: per-head path, two column tiles
    (44, 150, 8, 2, torch.float32),   # 264 jobs: grouped kernel, 352 chains in several rounds
    (44, 150, 8, 2, torch.bfloat16),
    (1, 8192, 16, 2, torch.float32),  # 256 jobs: grouped kernel, 16 chains (one tile, L2 touches)
])
def test_scalar_gate_grouped_heads_both_paths(B, T, H, H_qk, state_dtype):
    # With at least 256 (chunk, q/k head) jobs the value heads of a q/k group
    # share one copy of the qn and kn^T record fragments, written by the
    # grouped chunk-local kernel; smaller grids take the per-head kernel.
    inp = make_inputs(B, T, H, H_qk, gate_per_channel=False, A_log=(-3.0, 0.0), state_std=0.05, seed=27 + B + T)
    check(inp, state_dtype=state_dtype, what="scalar gate grouped B=%d T=%d H=%d H_qk=%d %s" % (B, T, H, H_qk,
                                                                                             state_dtype))


@pytest.mark.parametrize("A_log", [(2.5, 3.0), (-8.0, -6.0)])
def test_grouped_kernel_extreme_scalar_decays(A_log):
    # The grouped kernel's records (264 jobs) with decays that underflow within
    # a chunk (exp(A_log) ~ 12..20) or hardly decay at all: the recurrence's
    # residual V - exp(Gamma_r) (kn S) and its row factors at both extremes.
    inp = make_inputs(44, 150, 8, 2, gate_per_channel=False, A_log=A_log, state_std=0.05, seed=71)
    check(inp, what="grouped kernel, scalar decays A_log in %s" % (A_log,))


@pytest.mark.parametrize("lens", [[1, 64, 300, 0, 65, 129], [1, 64, 3000, 0, 65, 129, 700]])
def test_scalar_gate_grouped_heads_packed(lens):
    # three value heads per q/k head, packed sequences with an empty one and a
    # state: 60 jobs (per-head path) and 276 jobs (grouped kernel)
    inp = make_inputs(1, sum(lens), 12, 4, gate_per_channel=False, A_log=(-2.0, 0.0), state_std=0.05,
                      N=len(lens), lengths=lens, seed=28 + len(lens))
    check(inp, what="scalar gate grouped packed %s" % lens)


@pytest.mark.parametrize("per_channel,H,H_qk", [(True, 4, 4), (False, 8, 2)])
def test_correlated_keys_strong_writes_no_decay(per_channel, H, H_qk):
    # Keys along one shared direction plus half as much noise (cosine ~0.9
    # between keys), beta ~ 0.99 and per-token decays ~ 1: the strictly lower
    # block of (I + A) is close to all ones, the regime that stresses the UT
    # inverse and the fp16 state-path operands (the rows of U telescope within
    # a chunk).  Measured worst chain: final-state rel-L2 7.4e-4 here, 1.3e-3 at
    # noise 0.2; the precise mode (test_gpu_precise.py) takes the closer keys.
    inp = make_inputs(2, 300, H, H_qk, gate_per_channel=per_channel, A_log=-8.0, b_shift=4.6, state_std=0.02,
                      k_noise=0.5, seed=40 + H + 50)
    check(inp, what="correlated keys noise=0.5 per_channel=%s H=%d H_qk=%d" % (per_channel, H, H_qk))


def test_grouped_heads_per_channel_gate():
    inp = make_inputs(1, 200, 6, 2, state_std=0.02, seed=13)
    check(inp, what="per-channel gate, grouped heads")


def test_bf16_state():
    inp = make_inputs(2, 190, 2, 2, state_std=0.05, seed=14, A_log=(-5.0, -3.0))
    check(inp, state_dtype=torch.bfloat16, what="bf16 state")


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_many_chains_shallow_pipeline(state_dtype):
    # 40 rows x 8 heads = 320 chains -> 1280 two-tile recurrence workgroups,
    # several rounds of one workgroup per CU
    inp = make_inputs(40, 150, 8, 4, state_std=0.05, seed=24, A_log=(-4.0, -1.0))
    check(inp, state_dtype=state_dtype, what="many chains %s" % state_dtype)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_two_column_tiles_per_workgroup(state_dtype):
    # 6 rows x 8 heads = 48 chains: too many for one 16-column tile per CU,
    # so 32-column workgroups, all resident at once
    inp = make_inputs(6, 150, 8, 4, state_std=0.05, seed=25, A_log=(-4.0, -1.0))
    check(inp, state_dtype=state_dtype, what="two column tiles %s" % state_dtype)


def test_two_column_tiles_packed():
    lens = [1, 64, 300, 65, 0, 129]
    inp = make_inputs(1, sum(lens), 8, 2, state_std=0.05, N=len(lens), lengths=lens, seed=26)
    check(inp, what="two column tiles packed %s" % lens)


@pytest.mark.parametrize("h_qk,h_v", SWEEP_HEAD_SHAPES)
def test_grouped_head_shapes_packed(h_qk, h_v):
    # every head shape of the grouped-head sweep, scalar decay, packed A+B+C
    lens = [150, 41, 64]
    inp = make_inputs(1, sum(lens), h_v, h_qk, gate_per_channel=False, A_log=0.0, N=len(lens), lengths=lens,
                      seed=30 + h_v + h_qk)
    check(inp, what="grouped heads h_qk=%d h_v=%d packed %s" % (h_qk, h_v, lens))


def test_packed_sequences_edge_lengths():
    lens = [19, 64, 1, 130, 0, 77, 65, 63]
    inp = make_inputs(1, sum(lens), 3, 3, state_std=0.02, N=len(lens), lengths=lens, seed=15)
    check(inp, what="packed %s" % lens)


def test_packed_sequences_without_initial_state():
    lens = [5, 200, 33]
    inp = make_inputs(1, sum(lens), 2, 2, N=len(lens), lengths=lens, seed=16)
    check(inp, what="packed no state")


def test_packed_equals_separate_calls_on_gpu():
    lens = [40, 129, 7]
    inp = make_inputs(1, sum(lens), 2, 2, state_std=0.02, N=len(lens), lengths=lens, seed=17)
    out, fin = U.run_gpu(inp)
    cu = inp["cu_seqlens"]
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        one = {x: (inp[x][:, s:e] if x in U.TOKEN_KEYS else inp[x]) for x in inp}
        one["cu_seqlens"] = None
        one["initial_state"] = inp["initial_state"][n:n + 1]
        o1, f1 = U.run_gpu(one)
        np.testing.assert_allclose(o1, out[:, s:e], rtol=0, atol=2e-3)
        np.testing.assert_allclose(f1, fin[n:n + 1], rtol=0, atol=1e-4)


@pytest.mark.parametrize("split", [1, 63, 100])
def test_state_handoff(split):
    T = 260
    inp = make_inputs(1, T, 2, 2, state_std=0.02, seed=18, A_log=(-6.0, -4.0))
    a = {n: (x[:, :split] if n in U.TOKEN_KEYS else x) for n, x in inp.items()}
    b = {n: (x[:, split:] if n in U.TOKEN_KEYS else x) for n, x in inp.items()}
    o1, f1 = U.run_gpu(a)
    b["initial_state"] = f1.astype(np.float32)
    o2, f2 = U.run_gpu(b)
    ref_out, ref_fin = U.run_oracle(inp)
    U.assert_parity(np.concatenate([o1, o2], axis=1), f2, ref_out, ref_fin, what="handoff at %d" % split)


def test_initial_state_aliases_final_state():
    inp = make_inputs(1, 130, 2, 2, state_std=0.05, seed=19)
    d = U.to_device(inp)
    st = d["initial_state"]
    out, fin = kda.fwd(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], scale=inp["scale"],
                       initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    ref_out, ref_fin = U.run_oracle(inp)
    U.assert_parity(out.float().cpu().numpy(), st.cpu().numpy().astype(np.float64), ref_out, ref_fin,
                    what="aliased state")


def test_zero_tokens_copy_state():
    inp = make_inputs(2, 0, 2, 2, state_std=0.05, seed=20)
    out, fin = U.run_gpu(inp)
    assert out.shape[1] == 0
    np.testing.assert_array_equal(fin, inp["initial_state"].astype(np.float64))


def test_zero_tokens_without_state_gives_zero_state():
    inp = make_inputs(2, 0, 2, 2, seed=22)
    out, fin = U.run_gpu(inp)
    assert out.shape[1] == 0 and fin.shape == (2, 2, 128, 128)
    assert not np.any(fin)


def test_packed_all_sequences_empty():
    inp = make_inputs(1, 0, 2, 1, N=3, lengths=[0, 0, 0], state_std=0.05, seed=23)
    out, fin = U.run_gpu(inp)
    assert out.shape[1] == 0
    np.testing.assert_array_equal(fin, inp["initial_state"].astype(np.float64))


def test_run_to_run_bitwise_determinism():
    inp = make_inputs(2, 333, 4, 2, state_std=0.02, seed=21)
    o1, f1 = U.run_gpu(inp)
    o2, f2 = U.run_gpu(inp)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_zero_output_would_fail_the_bar():
    inp = workload_inputs("kda_tiny")
    ref_out, _ = U.run_oracle(inp)
    assert U.rel_l2(np.zeros_like(ref_out), ref_out) > U.OUT_REL


# ---------------------------------------------------------------- decode ----

def run_decode_gpu(q, k, v, g, b, A_log, state, scale, state_dtype=torch.float32):
    dq, dk, dv, dg = (U.bf16_tensor(x) for x in (q, k, v, g))
    st = torch.from_numpy(state).to(device="cuda", dtype=state_dtype)
    out = kda.decode_step(dq, dk, dv, dg, torch.from_numpy(b).cuda(), torch.from_numpy(A_log).cuda(), st,
                          scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("per_channel,H_qk,H,sdt", [(True, 4, 4, torch.float32), (False, 2, 8, torch.float32),
                                                    (True, 4, 4, torch.bfloat16)])
def test_decode_step(per_channel, H_qk, H, sdt):
    import oracle
    inp = make_inputs(5, 1, H, H_qk, gate_per_channel=per_channel, state_std=0.05, seed=22, decode=True)
    s0 = inp["initial_state"]
    if sdt == torch.bfloat16:
        s0 = torch.from_numpy(s0).to(torch.bfloat16).float().numpy()
    out, st = run_decode_gpu(inp["q"], inp["k"], inp["v"], inp["g_raw"], inp["b"], inp["A_log"], s0,
                             inp["scale"], sdt)
    ro, rs = oracle.kda_decode(inp["q"], inp["k"], inp["v"], inp["g_raw"], inp["b"], inp["A_log"], inp["scale"], s0,
                               gate_per_channel=per_channel)
    U.assert_parity(out, st, ro, rs, sdt, what="decode pc=%s H_qk=%d H=%d %s" % (per_channel, H_qk, H, sdt))


def test_decode_steps_match_chunked_forward():
    T = 40
    inp = make_inputs(3, T, 2, 2, state_std=0.05, seed=23, A_log=(-4.0, -2.0))
    out_f, fin_f = U.run_gpu(inp)
    st = inp["initial_state"].copy()
    outs = []
    for t in range(T):
        o, st = run_decode_gpu(inp["q"][:, t], inp["k"][:, t], inp["v"][:, t], inp["g_raw"][:, t], inp["b"][:, t],
                               inp["A_log"], st.astype(np.float32), inp["scale"])
        outs.append(o)
    ref_out, ref_fin = U.run_oracle(inp)
    U.assert_parity(np.stack(outs, axis=1), st, ref_out, ref_fin, what="T decode steps")
    np.testing.assert_allclose(np.stack(outs, axis=1), out_f, rtol=0, atol=5e-3)


# ------------------------------------------------------ full-size workloads --

def sampled_mask(C, H, picks):
    m = np.zeros((C, H), dtype=bool)
    for c, h in picks:
        m[c, h] = True
    return m


@pytest.mark.parametrize("name", ["kda_dense", "kda_varlen", "gdn_gva"])
def test_full_size_workload_sampled_chains(name):
    w = WORKLOADS[name]
    inp = workload_inputs(name)
    C = w.N if w.N else w.B
    if name == "kda_varlen":
        lens = np.diff(inp["cu_seqlens"])
        longest, shortest = int(np.argmax(lens)), int(np.argmin(lens))
        picks = [(longest, 0), (longest, w.H - 1), (shortest, 3), (C // 2, 7)]
    else:
        picks = [(0, 0), (C - 1, w.H - 1), (0, w.H // 2 + 1)]
    check(inp, what=name + " sampled chains", chain_mask=sampled_mask(C, w.H, picks))


@pytest.mark.parametrize("h_qk,h_v,pattern", [(2, 8, "28672+4096"), (16, 64, "8192x4"), (32, 32, "24576+8192")])
def test_full_size_sweep_rows_sampled_chains(h_qk, h_v, pattern):
    # two rows of the grouped-head sweep at their full size, in the launch
    # configuration the sweep times; the oracle checks sampled chains
    lens = SWEEP_PATTERNS[pattern]
    full = sweep_inputs(h_qk, h_v)
    T = sum(lens)
    inp = dict(full)
    for n in ("q", "k", "v", "g_raw", "b"):
        inp[n] = np.ascontiguousarray(full[n][:, :T])
    inp["cu_seqlens"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    picks = [(0, 0), (len(lens) - 1, h_v - 1)]
    check(inp, what="sweep h_qk=%d h_v=%d %s sampled chains" % (h_qk, h_v, pattern),
          chain_mask=sampled_mask(len(lens), h_v, picks))


def test_full_size_decode():
    import oracle
    w = WORKLOADS["kda_decode"]
    inp = workload_inputs("kda_decode")
    out, st = run_decode_gpu(inp["q"], inp["k"], inp["v"], inp["g_raw"], inp["b"], inp["A_log"],
                             inp["initial_state"], inp["scale"])
    ro, rs = oracle.kda_decode(inp["q"], inp["k"], inp["v"], inp["g_raw"], inp["b"], inp["A_log"], inp["scale"],
                               inp["initial_state"])
    U.assert_parity(out, st, ro, rs, what="kda_decode B=%d H=%d" % (w.B, w.H))
