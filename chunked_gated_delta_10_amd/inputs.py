"""Seeded synthetic inputs for the KDA forward workloads.

This module draws random numbers and packs them into the storage formats the
operator takes (bf16 bit patterns, fp32, int32 offsets).  It holds none of
the operator's arithmetic, so both the GPU path's tests and the CPU oracle
may consume what it produces.

Recipe (all draws fp32 from ``numpy.random.default_rng(seed)``, in the order
q, k, v, g_raw, A_log, b, S0; tensors stored as bf16 are rounded to nearest
even):

* q, k, v, g_raw ~ N(0, 1), stored bf16.  q and k are normalised inside the
  operator, so raw normal draws are passed.
* A_log ~ U(lo, hi) per value head (fp32) or a constant.
* b (beta logits) ~ N(0, 1), fp32.
* S0 ~ N(0, std^2) fp32 in the [C, H, V, K] state layout, or absent.

Workloads are the shapes of the cuLA KDA tables (fixed-length B x T sweep
and the random-length varlen row with 20 sequences, lengths 19..3147, total
16384), the FlashQLA H200 gated-delta forward row (1 x 32768 tokens,
h_qk = 16, h_v = 64) and the cuLA single-token decode table (batch 256,
64 heads, head dim 128); the decay-only linear-attention workloads take the
shapes of the cuLA lightning-attention tables (packed sequences, decode at
batch 256, 64 heads, head dim 128).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

HEAD_DIM = 128


def bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + (((u >> 16) & 1) + 0x7FFF)) >> 16
    return u.astype(np.uint16)


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    H_qk: int
    gate_per_channel: bool = True
    A_log: Tuple[float, float] = (-1.0, 1.0)   # U(lo, hi); lo == hi means a constant
    state_std: Optional[float] = None          # None: no initial state
    N: int = 0                                  # packed sequences (varlen) when > 0
    decode: bool = False
    seed: int = 0
    delta: bool = True                          # False: decay-only linear attention (no beta)
    lengths: Optional[Tuple[int, ...]] = None   # packed sequence lengths (default: random, see varlen_lengths)
    backward: bool = False                      # the backward pass (upstream gradient from backward_upstream)
    K: int = HEAD_DIM
    V: int = HEAD_DIM
    note: str = ""

    @property
    def tokens(self) -> int:
        return self.B * self.T


# The five workloads; seed = 1000 + index.
WORKLOADS: Dict[str, Workload] = {
    "kda_tiny": Workload("kda_tiny", B=1, T=512, H=4, H_qk=4, seed=1000,
                         note="KDA fwd, B=1 T=512 H=4, zero initial state"),
    "kda_dense": Workload("kda_dense", B=2, T=16384, H=16, H_qk=16, state_std=0.02, seed=1001,
                          note="KDA fwd, B=2 T=16384 H=16, fp32 initial/final state"),
    "kda_varlen": Workload("kda_varlen", B=1, T=16384, H=16, H_qk=16, state_std=0.02, N=20, seed=1002,
                           note="KDA fwd varlen, 20 sequences, lengths 19..3147, total 16384"),
    "gdn_gva": Workload("gdn_gva", B=1, T=32768, H=64, H_qk=16, gate_per_channel=False,
                        A_log=(0.0, 0.0), seed=1003,
                        note="gated delta rule, scalar decay, h_qk=16 h_v=64, T=32768"),
    "kda_decode": Workload("kda_decode", B=256, T=1, H=64, H_qk=64, state_std=0.02, decode=True, seed=1004,
                           note="KDA single-token decode, B=256 H=64, fp32 state in place"),
    # decay-only linear attention (the cuLA page's lightning-attention tables):
    # packed no-state forward over 16 random-length sequences, and the
    # single-token decode at batch 256, 64 heads, head dim 128
    "la_varlen": Workload("la_varlen", B=1, T=16384, H=64, H_qk=64, gate_per_channel=False, A_log=(0.0, 0.0),
                          N=16, seed=1005, delta=False,
                          note="decay-only linear attention, 16 packed sequences (19..3147), H=64, no state"),
    "la_decode": Workload("la_decode", B=256, T=1, H=64, H_qk=64, gate_per_channel=False, A_log=(0.0, 0.0),
                          state_std=0.02, decode=True, seed=1006, delta=False,
                          note="decay-only linear attention decode, B=256 H=64, fp32 state in place"),
    # the backward of the gated delta rule (the FlashQLA H200 page's backward table: sequences split into 8,
    # here its 32-head, 32k-token row)
    "gdn_bwd": Workload("gdn_bwd", B=1, T=32768, H=32, H_qk=32, gate_per_channel=False, A_log=(0.0, 0.0), N=8,
                        lengths=(4096,) * 8, seed=1007, backward=True,
                        note="gated delta rule backward, scalar decay, 8 sequences x 4096 tokens, 32 heads"),
    # the backward of KDA itself (one decay per key channel) on the forward's dense shape
    "kda_bwd": Workload("kda_bwd", B=2, T=16384, H=16, H_qk=16, state_std=0.02, seed=1008, backward=True,
                        note="KDA backward, per-channel decay, B=2 T=16384 H=16, fp32 initial state"),
}


def varlen_lengths(rng: np.random.Generator, N: int = 20, total: int = 16384, lo: int = 19,
                   hi: int = 3147) -> np.ndarray:
    """Random sequence lengths in [lo, hi] summing to total, with lo and hi both present.

    Two sequences take the extreme lengths; the other N-2 get lo plus a
    Dirichlet(1) share of what is left (floored, the remainder handed out one
    token at a time in order); a draw with any length above hi is redrawn.
    The N lengths are then shuffled.
    """
    rest = total - hi - lo - (N - 2) * lo
    assert rest >= 0
    while True:
        share = rng.dirichlet(np.ones(N - 2)) * rest
        extra = np.floor(share).astype(np.int64)
        extra[: rest - int(extra.sum())] += 1
        lens = lo + extra
        if lens.max() <= hi:
            break
    lens = np.concatenate([[lo, hi], lens]).astype(np.int64)
    lens = lens[rng.permutation(N)]
    assert lens.sum() == total and lens.min() >= lo and lens.max() <= hi
    return lens


def cu_seqlens_from_lengths(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def make_inputs(B: int, T: int, H: int, H_qk: int, *, gate_per_channel: bool = True,
                A_log=(-1.0, 1.0), state_std: Optional[float] = None, N: int = 0,
                lengths=None, seed: int = 0, K: int = HEAD_DIM, V: int = HEAD_DIM,
                decode: bool = False, g_shift: float = 0.0, b_shift: float = 0.0,
                k_noise: Optional[float] = None) -> dict:
    """Draw one batch of inputs.

    Returns a dict of numpy arrays: q, k, v, g_raw (uint16 bf16 bits), b, A_log
    (float32), initial_state (float32 or None), cu_seqlens (int32 or None),
    plus the scale 1/sqrt(K).  With decode=True the token axis is dropped
    (q: [B, H_qk, K]).  g_shift / b_shift add a constant to the normal draws
    of g_raw / b before rounding (used by tests that need milder or harsher
    gates).  With k_noise set, keys are nearly parallel: each q/k head draws
    one direction d ~ N(0, I) after every other draw, and its keys become
    d + k_noise * (the normal draw), so the decayed Gram entries sit near 1.
    """
    rng = np.random.default_rng(seed)
    lead = (B,) if decode else (B, T)
    q = rng.standard_normal(lead + (H_qk, K), dtype=np.float32)
    k = rng.standard_normal(lead + (H_qk, K), dtype=np.float32)
    v = rng.standard_normal(lead + (H, V), dtype=np.float32)
    g_shape = lead + ((H, K) if gate_per_channel else (H,))
    g = rng.standard_normal(g_shape, dtype=np.float32) + np.float32(g_shift)
    lo, hi = (float(A_log), float(A_log)) if np.isscalar(A_log) else (float(A_log[0]), float(A_log[1]))
    if lo == hi:
        a_log = np.full((H,), lo, dtype=np.float32)
    else:
        a_log = rng.uniform(lo, hi, size=(H,)).astype(np.float32)
    b = rng.standard_normal(lead + (H,), dtype=np.float32) + np.float32(b_shift)
    cu = None
    if N > 0:
        assert B == 1 and not decode
        if lengths is None:
            lengths = varlen_lengths(rng, N=N, total=T)
        cu = cu_seqlens_from_lengths(lengths)
        assert cu[-1] == T
    C = N if N > 0 else B
    s0 = None
    if state_std is not None:
        s0 = (rng.standard_normal((C, H, V, K), dtype=np.float32) * np.float32(state_std)).astype(np.float32)
    if k_noise is not None:
        d = rng.standard_normal((H_qk, K), dtype=np.float32)
        k = (d + np.float32(k_noise) * k).astype(np.float32)
    return {
        "q": bf16_bits(q), "k": bf16_bits(k), "v": bf16_bits(v), "g_raw": bf16_bits(g),
        "A_log": a_log, "b": b.astype(np.float32), "initial_state": s0, "cu_seqlens": cu,
        "scale": 1.0 / np.sqrt(K), "gate_per_channel": gate_per_channel,
    }


def workload_inputs(name: str) -> dict:
    w = WORKLOADS[name]
    return make_inputs(w.B, w.T, w.H, w.H_qk, gate_per_channel=w.gate_per_channel, A_log=w.A_log,
                       state_std=w.state_std, N=w.N, lengths=w.lengths, seed=w.seed, K=w.K, V=w.V,
                       decode=w.decode)


def backward_upstream(inp: dict, seed: int, dfinal_std: Optional[float] = None):
    """Upstream gradients for a backward call: dout ~ N(0, 1) stored bf16 (bits), shaped like the output,
    and dfinal ~ N(0, dfinal_std^2) fp32 in the state layout (None: no final-state gradient)."""
    rng = np.random.default_rng(seed)
    B, T, H, V = inp["v"].shape
    cu = inp.get("cu_seqlens")
    C = B if cu is None else len(cu) - 1
    K = inp["q"].shape[-1]
    dout = bf16_bits(rng.standard_normal((B, T, H, V), dtype=np.float32))
    dfinal = None
    if dfinal_std is not None:
        dfinal = (rng.standard_normal((C, H, V, K), dtype=np.float32) * np.float32(dfinal_std)).astype(np.float32)
    return dout, dfinal


# Grouped-value-head sweep (the forward table of the FlashQLA H200 benchmark
# results page): head shapes (h_qk, h_v) and packed sequence patterns.  Every
# row uses the scalar per-token decay g = -softplus(N(0,1)) (A_log = 0), no
# initial state, and is drawn once per head shape at 32768 tokens; a pattern
# uses the first sum(lengths) tokens.
SWEEP_HEAD_SHAPES = [(2, 8), (4, 16), (8, 24), (8, 32), (16, 16), (16, 32), (16, 48), (16, 64), (32, 32)]
SWEEP_PATTERNS: Dict[str, Tuple[int, ...]] = {
    "1x2048": (2048,), "1x4096": (4096,), "1x8192": (8192,), "1x16384": (16384,), "1x32768": (32768,),
    "28672+4096": (28672, 4096), "24576+8192": (24576, 8192), "16384+16384": (16384, 16384),
    "8192+24576": (8192, 24576), "4096+28672": (4096, 28672),
    "12288+4096": (12288, 4096), "6144+2048": (6144, 2048), "4096+4096": (4096, 4096), "2048+6144": (2048, 6144),
    "1024+7168": (1024, 7168),
    "8192x4": (8192,) * 4, "4096x8": (4096,) * 8, "2048x4": (2048,) * 4, "1024x8": (1024,) * 8,
}
SWEEP_TOKENS = 32768


def sweep_inputs(h_qk: int, h_v: int, seed: int = 2000) -> dict:
    """Inputs of one head shape of the grouped-head sweep (B=1, T=32768)."""
    return make_inputs(1, SWEEP_TOKENS, h_v, h_qk, gate_per_channel=False, A_log=0.0, seed=seed + 100 * h_qk + h_v)
