"""GPU parity of the backward pass with one decay per token-head (kda.bwd /
kda.bwd_varlen, C ABI kda_bwd / kda_bwd_varlen) against the fp64 backward
oracle; the helpers serve the per-channel gate's tests as well.

The oracle (oracle/kda_backward.py) is reverse-mode differentiation of the
token-by-token forward, pinned on the CPU to complex-step and finite
differences.  The GPU runs the chunk form of both chains (the forward's chunk
states, then the adjoint) and the chunk-parallel gradients on fp16 matrix
cores with fp32 accumulation and fp16 storage of the chunk states: the
precision of the forward's own chunk path, whose state error the forward
tests hold to 1e-3 rel-L2.  Every gradient is bilinear in those states and the
upstream gradients, so its relative error is of that order times a small
factor: each gradient is held to GRAD_REL rel-L2 and to GRAD_MAXABS of its
own largest magnitude.  dA_log is a sum over every token of a head,
sum_t dg_t g_t, whose terms have both signs: its error is held to GRAD_REL
times sum_t |dg_t g_t| (the sum's condition), computed from the oracle's dg_raw
(dg_t g_t = dg_raw_t softplus(g_raw_t) / sigmoid(g_raw_t)).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import kda_backward as KB
from chunked_gated_delta_10_amd import kda
from chunked_gated_delta_10_amd.inputs import make_inputs, bf16_bits

from kda_util import bf16_tensor, rel_l2

pytestmark = pytest.mark.gpu

GRAD_REL = 5e-3
GRAD_MAXABS = 2e-2  # of max |reference| of the same gradient
# per (sequence, head): the same error measured on each chain's own slice, so that an error confined to one
# chain is not diluted by the others; twice the pooled bar (short chains hold few values)
GRAD_REL_CHAIN = 1e-2
CHAIN_FLOOR = 1e-2  # of a typical slice's norm; see chain_worst
# dinitial_state entries within this absolute distance of the oracle pass whatever their relative error (the
# upstream gradients here are of unit scale): the adjoint chain stores and multiplies fp16 values, whose
# resolution below the normal range (2^-14) is the subnormal spacing 2^-24 ~ 6e-8, so when harsh decays leave
# every entry of every slice under ~1e-6 (the fp64 oracle's values reach 1e-9 and below) relative bars measure
# only that rounding; at ordinary magnitudes (1e-2..1e-1) the bound is far below fp16's relative resolution
DINIT_ABS = 1e-6
NAMES = ("dq", "dk", "dv", "dg_raw", "dbeta_logits", "dA_log", "dinitial_state")


def upstream(inp, seed, dfinal_std=0.1):
    rng = np.random.default_rng(seed)
    B, T, H = inp["v"].shape[:3]
    cu = inp.get("cu_seqlens")
    C = B if cu is None else len(cu) - 1
    dout = bf16_bits(rng.standard_normal((B, T, H, 128), dtype=np.float32))
    dfinal = None if dfinal_std is None else (rng.standard_normal((C, H, 128, 128), dtype=np.float32)
                                              * np.float32(dfinal_std))
    return dout, dfinal


def run_gpu_bwd(inp, dout, dfinal):
    dev = "cuda"
    t = {n: bf16_tensor(inp[n], dev) for n in ("q", "k", "v", "g_raw")}
    b = torch.from_numpy(inp["b"]).to(dev)
    a = torch.from_numpy(inp["A_log"]).to(dev)
    s0 = None if inp["initial_state"] is None else torch.from_numpy(inp["initial_state"]).to(dev)
    do = bf16_tensor(dout, dev)
    df = None if dfinal is None else torch.from_numpy(dfinal).to(dev)
    cu = inp.get("cu_seqlens")
    if cu is None:
        g = kda.bwd(t["q"], t["k"], t["v"], t["g_raw"], b, a, do, dfinal=df, scale=inp["scale"], initial_state=s0)
    else:
        g = kda.bwd_varlen(t["q"], t["k"], t["v"], t["g_raw"], b, a, do, torch.from_numpy(cu).to(dev),
                           dfinal=df, scale=inp["scale"], initial_state=s0)
    torch.cuda.synchronize()
    return {n: g[n].cpu().numpy().astype(np.float64) for n in NAMES}


def run_oracle_bwd(inp, dout, dfinal, heads=None):
    """The oracle on all value heads, or on `heads` only (q/k heads not shared: H == H_qk).  The gate mode
    follows g_raw's rank."""
    w = oracle.widen
    q, k, v, g, b, a = w(inp["q"]), w(inp["k"]), w(inp["v"]), w(inp["g_raw"]), inp["b"], inp["A_log"]
    do = w(dout)
    s0, df = inp["initial_state"], dfinal
    B, T, H = v.shape[:3]
    C = B if inp.get("cu_seqlens") is None else len(inp["cu_seqlens"]) - 1
    if df is None:
        df = np.zeros((C, H, 128, 128))
    if heads is not None:
        hs = list(heads)
        q, k, v, g, b, a, do = q[:, :, hs], k[:, :, hs], v[:, :, hs], g[:, :, hs], b[:, :, hs], a[hs], do[:, :, hs]
        s0 = None if s0 is None else s0[:, hs]
        df = df[:, hs]
    return KB.kda_bwd(q, k, v, g, b, a, inp["scale"], do, df, gate_per_channel=g.ndim == 4, initial_state=s0,
                      cu_seqlens=inp.get("cu_seqlens"))


def dA_log_condition(ref, g_raw_bits):
    """sum over a head's tokens (and key channels) of |dg g| (the magnitude the dA_log sum is formed from)."""
    x = oracle.widen(g_raw_bits)                                   # [B, T, H] or [B, T, H, K]
    sp = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
    sig = 1.0 / (1.0 + np.exp(-x))
    return np.abs(ref["dg_raw"] * sp / sig).sum(axis=(0, 1) if x.ndim == 3 else (0, 1, 3))


def chain_worst(got, ref, cu_seqlens=None):
    """Worst per-(sequence, head) rel-L2 of every gradient with a token axis, and of dinitial_state per
    (sequence, head).  Each slice's error is taken relative to max(its reference norm, CHAIN_FLOOR times a
    typical slice's norm): under harsh decays a chain's dinitial_state is a product of many factors near zero
    (down to 1e-30 and below in the fp64 oracle), and once its entries fall under fp16's normal range
    (2^-14 ~ 6e-5, against typical entries of 1e-2..1e-1) the fp16 chain operands and stored state
    gradients keep only a few significant bits; such a slice is held to an absolute error of CHAIN_FLOOR
    times the typical slice instead of to a relative one."""
    B, T = got["dv"].shape[:2]
    spans = ([(b, 0, T) for b in range(B)] if cu_seqlens is None else
             [(0, int(cu_seqlens[n]), int(cu_seqlens[n + 1])) for n in range(len(cu_seqlens) - 1)])
    slices = {}
    for n in ("dq", "dk", "dv", "dg_raw", "dbeta_logits"):
        slices[n] = [(got[n][b, t0:t1, h], ref[n][b, t0:t1, h])
                     for b, t0, t1 in spans if t1 > t0 for h in range(got[n].shape[2])]
    x, r = got["dinitial_state"], ref["dinitial_state"]
    slices["dinitial_state"] = [(x[c, h], r[c, h]) for c in range(x.shape[0]) for h in range(x.shape[1])]
    worst = {}
    for n, sl in slices.items():
        norms = np.array([np.linalg.norm(rr) for _, rr in sl])
        if len(sl) == 0 or not np.any(norms > 0):
            continue
        floor = CHAIN_FLOOR * np.sqrt(np.mean(norms ** 2))
        worst[n] = max(0.0 if n == "dinitial_state" and np.max(np.abs(xx - rr)) <= DINIT_ABS else
                       float(np.linalg.norm(xx - rr) / max(nr, floor)) for (xx, rr), nr in zip(sl, norms))
    return worst


def compare(got, ref, label, g_raw_bits, cu_seqlens=None):
    errs = {}
    for n in NAMES:
        r, x = ref[n], got[n]
        assert x.shape == r.shape, (label, n, x.shape, r.shape)
        assert np.all(np.isfinite(x)), (label, n)
        if n == "dA_log":  # per head, against the condition of the sum
            rel = float(np.max(np.abs(x - r) / np.maximum(dA_log_condition(ref, g_raw_bits), 1e-30)))
            mx = rel
        else:
            rel = rel_l2(x, r)
            mx = float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30))
        errs[n] = (rel, mx)
    worst = chain_worst(got, ref, cu_seqlens)
    print(label, " ".join("%s %.1e/%.1e" % (n, *errs[n]) for n in NAMES), "| worst chain",
          " ".join("%s %.1e" % kv for kv in worst.items()), flush=True)
    for n, (rel, mx) in errs.items():
        if n == "dinitial_state" and np.max(np.abs(got[n] - ref[n])) <= DINIT_ABS:
            continue
        assert rel <= GRAD_REL and mx <= GRAD_MAXABS, (label, n, rel, mx)
    for n, e in worst.items():
        assert e <= GRAD_REL_CHAIN, (label, n, "per chain", e)


CASES = [
    # (label, make_inputs kwargs, dfinal std or None)
    ("dense B=2 T=200 H=2 state", dict(B=2, T=200, H=2, H_qk=2, state_std=0.05, seed=71), 0.1),
    ("dense B=1 T=64 H=1 no state", dict(B=1, T=64, H=1, H_qk=1, seed=72), None),
    ("dense B=1 T=1 H=2", dict(B=1, T=1, H=2, H_qk=2, state_std=0.05, seed=73), 0.1),
    ("grouped B=1 T=130 H=4 H_qk=2", dict(B=1, T=130, H=4, H_qk=2, state_std=0.05, seed=74), 0.1),
    ("grouped B=1 T=97 H=6 H_qk=1", dict(B=1, T=97, H=6, H_qk=1, seed=75), 0.1),
    ("strong decay A_log=1.5", dict(B=1, T=150, H=2, H_qk=2, A_log=1.5, state_std=0.05, seed=76), 0.1),
    ("weak decay A_log=-4", dict(B=1, T=150, H=2, H_qk=2, A_log=-4.0, state_std=0.05, seed=77), 0.1),
    ("varlen N=5 with empty and 1-token",
     dict(B=1, T=230, H=2, H_qk=2, N=5, lengths=[64, 0, 1, 100, 65], state_std=0.05, seed=78), 0.1),
]


@pytest.mark.parametrize("label,kw,dstd", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_the_oracle(label, kw, dstd):
    inp = make_inputs(gate_per_channel=False, **{"A_log": (-1.0, 1.0), **kw})
    dout, dfinal = upstream(inp, kw["seed"] + 500, dstd)
    got = run_gpu_bwd(inp, dout, dfinal)
    ref = run_oracle_bwd(inp, dout, dfinal)
    compare(got, ref, label, inp["g_raw"], inp.get("cu_seqlens"))


def test_backward_grouped_heads_long_sequence():
    # 64 chunks, two value heads on each q/k head: dq, dk summed over the group across many chunks
    inp = make_inputs(1, 4096, 8, 4, gate_per_channel=False, A_log=(-1.0, 1.0), state_std=0.05, seed=79)
    dout, dfinal = upstream(inp, 579)
    got = run_gpu_bwd(inp, dout, dfinal)
    ref = run_oracle_bwd(inp, dout, dfinal)
    compare(got, ref, "grouped heads T=4096 H=8 H_qk=4", inp["g_raw"])


def test_backward_many_jobs_sampled_heads():
    # 128 chunks x 32 heads = 4096 (chunk, head) jobs, chains on the widest column tiles; heads 0 and 31
    # are checked against the oracle
    inp = make_inputs(1, 8192, 32, 32, gate_per_channel=False, A_log=(-1.0, 1.0), state_std=0.05, seed=80)
    dout, dfinal = upstream(inp, 580)
    got = run_gpu_bwd(inp, dout, dfinal)
    heads = [0, 31]
    ref = run_oracle_bwd(inp, dout, dfinal, heads=heads)
    sub = {n: (got[n][heads] if n == "dA_log" else got[n][:, heads] if n == "dinitial_state"
               else got[n][:, :, heads]) for n in NAMES}
    compare(sub, ref, "T=8192 H=32, heads 0 and 31", inp["g_raw"][:, :, heads])


def test_backward_benchmark_shape_sampled_heads():
    # the scalar-gate backward benchmark configuration (8 packed sequences x 4096 tokens, 32 heads, one
    # bwd_varlen call; 16,640 (chunk, head) jobs, chains on 128-column tiles); heads 0 and 31 against the
    # oracle
    from chunked_gated_delta_10_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["gdn_bwd"]
    inp = workload_inputs("gdn_bwd")
    dout, dfinal = upstream(inp, w.seed + 500)
    got = run_gpu_bwd(inp, dout, dfinal)
    heads = [0, 31]
    ref = run_oracle_bwd(inp, dout, dfinal, heads=heads)
    sub = {n: (got[n][heads] if n == "dA_log" else got[n][:, heads] if n == "dinitial_state"
               else got[n][:, :, heads]) for n in NAMES}
    compare(sub, ref, "gdn_bwd shape 8 x 4096 H=32, heads 0 and 31", inp["g_raw"][:, :, heads], inp["cu_seqlens"])


def test_backward_extreme_decay():
    # per-token decays of e^-60 and below (A_log = 3, g_raw ~ N(3, 1)): the gate gradients are tiny, formed
    # from products that are not.  Token gradients at the usual bars; dinitial_state (about e^-60 per token
    # of the sequence in the fp64 oracle, zero in fp32) to an absolute 1e-6 of dfinal's scale; dA_log, a sum
    # of tiny terms of both signs, to 0.1 of its condition.
    inp = make_inputs(1, 150, 2, 2, gate_per_channel=False, A_log=3.0, g_shift=3.0, state_std=0.05, seed=81)
    dout, dfinal = upstream(inp, 581)
    got, ref = run_gpu_bwd(inp, dout, dfinal), run_oracle_bwd(inp, dout, dfinal)
    for n in ("dq", "dk", "dv", "dg_raw", "dbeta_logits"):
        rel = rel_l2(got[n], ref[n])
        print("extreme decay", n, "%.1e" % rel, flush=True)
        assert rel <= GRAD_REL, (n, rel)
    assert np.max(np.abs(got["dinitial_state"] - ref["dinitial_state"])) <= 1e-6 * np.max(np.abs(dfinal))
    cond = dA_log_condition(ref, inp["g_raw"])
    assert np.max(np.abs(got["dA_log"] - ref["dA_log"]) / cond) <= 0.1


@pytest.mark.parametrize("per_channel", [False, True], ids=["scalar gate", "per-channel gate"])
def test_backward_deterministic(per_channel):
    # two calls on the same inputs: every gradient that is not accumulated with float atomics (dA_log always
    # is; dq, dk only when value heads share q/k heads, not here) is bit for bit the same
    inp = make_inputs(1, 300, 4, 4, gate_per_channel=per_channel, state_std=0.05, seed=82, N=3,
                      lengths=[130, 64, 106])
    dout, dfinal = upstream(inp, 582)
    a, b = run_gpu_bwd(inp, dout, dfinal), run_gpu_bwd(inp, dout, dfinal)
    for n in NAMES:
        if n != "dA_log":
            assert np.array_equal(a[n], b[n]), n
    np.testing.assert_allclose(a["dA_log"], b["dA_log"], rtol=1e-5, atol=1e-7)


def test_backward_zero_tokens():
    # T = 0: no token gradients; dinitial_state = dfinal, dA_log = 0
    H = 2
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    df = torch.randn(3, H, 128, 128, device="cuda")
    g = kda.bwd_varlen(z(1, 0, H, 128), z(1, 0, H, 128), z(1, 0, H, 128), z(1, 0, H),
                       torch.zeros(1, 0, H, device="cuda"), torch.zeros(H, device="cuda"), z(1, 0, H, 128),
                       torch.zeros(4, dtype=torch.int32, device="cuda"), dfinal=df)
    torch.cuda.synchronize()
    assert torch.equal(g["dinitial_state"], df)
    assert torch.count_nonzero(g["dA_log"]) == 0


# ---- seeded random configurations -----------------------------------------------------------------
REGIMES = {
    "workload": dict(A_log=(-1.0, 1.0)),
    "slow decay": dict(A_log=(-6.0, -4.0)),
    "harsh decay": dict(A_log=(2.0, 3.0)),
    "correlated keys": dict(A_log=-8.0, k_noise=0.5, b_shift=4.6),
}


def draw_bwd_case(i):
    """Case i: q/k heads and grouping, dense rows or packed sequences (empty ones allowed), lengths rarely a
    multiple of 64, initial state and dfinal present or not, and a gate regime, all from seed 1900 + i."""
    rng = np.random.default_rng(1900 + i)
    H_qk = int(rng.choice([1, 2, 4]))
    H = H_qk * int(rng.choice([1, 2, 3]))
    regime = str(rng.choice(sorted(REGIMES)))
    kw = dict(REGIMES[regime], gate_per_channel=False, seed=2900 + i)
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
    what = "bwd case %d: %s H=%d H_qk=%d, %s, state %s, dfinal %s" % (
        i, shape, H, H_qk, regime, "none" if inp["initial_state"] is None else "fp32", dstd)
    return inp, dstd, what


@pytest.mark.parametrize("i", range(16))
def test_backward_random_configuration(i):
    inp, dstd, what = draw_bwd_case(i)
    print(what, flush=True)
    dout, dfinal = upstream(inp, 3900 + i, dstd)
    compare(run_gpu_bwd(inp, dout, dfinal), run_oracle_bwd(inp, dout, dfinal), what, inp["g_raw"],
            inp.get("cu_seqlens"))
