"""Shared helpers for the GPU parity tests: move seeded numpy inputs to the
device, run the HIP path through the binding, run the oracle, compare."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from chunked_gated_delta_10_amd import kda

TOKEN_KEYS = ("q", "k", "v", "g_raw", "b")

# Parity bars: out max-abs <= 2e-2 and rel-L2 <= 5e-3; fp32 final state
# rel-L2 <= 1e-3.  bf16 state storage alone costs ~1.7e-3 rel-L2, so a bf16
# final state is held to 8e-3.
OUT_MAXABS = 2e-2
OUT_REL = 5e-3
STATE_REL_FP32 = 1e-3
STATE_REL_BF16 = 8e-3


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device(inp: dict, state_dtype=torch.float32, device="cuda") -> dict:
    d = {n: bf16_tensor(inp[n], device) for n in ("q", "k", "v", "g_raw")}
    d["b"] = torch.from_numpy(inp["b"]).to(device)
    d["A_log"] = torch.from_numpy(inp["A_log"]).to(device)
    s0 = inp.get("initial_state")
    d["initial_state"] = None if s0 is None else torch.from_numpy(s0).to(device=device, dtype=state_dtype)
    cu = inp.get("cu_seqlens")
    d["cu_seqlens"] = None if cu is None else torch.from_numpy(cu).to(device)
    return d


def run_gpu(inp: dict, state_dtype=torch.float32, **kw):
    d = to_device(inp, state_dtype)
    B, T, H_qk = inp["q"].shape[:3]
    H = inp["v"].shape[2]
    cu = inp.get("cu_seqlens")
    N = 0 if cu is None else len(cu) - 1
    ws = torch.empty(max(kda.workspace_bytes(B, T, H_qk, H, N), 256), dtype=torch.uint8, device="cuda")
    if d["cu_seqlens"] is not None:
        out, fin = kda.fwd_varlen(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], d["cu_seqlens"],
                                  scale=inp["scale"], initial_state=d["initial_state"], state_dtype=state_dtype,
                                  workspace=ws, **kw)
    else:
        out, fin = kda.fwd(d["q"], d["k"], d["v"], d["g_raw"], d["b"], d["A_log"], scale=inp["scale"],
                           initial_state=d["initial_state"], state_dtype=state_dtype, workspace=ws, **kw)
    kda.check(ws)  # no internal error (timed-out wait, unexpected placement) in the launch
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), fin.float().cpu().numpy().astype(np.float64)


def state_as_stored(inp: dict, state_dtype) -> dict:
    """The oracle must see the initial state the GPU sees (bf16-rounded if stored bf16)."""
    s0 = inp.get("initial_state")
    if s0 is None or state_dtype == torch.float32:
        return inp
    r = dict(inp)
    r["initial_state"] = torch.from_numpy(s0).to(torch.bfloat16).float().numpy()
    return r


def run_oracle(inp: dict, chain_mask=None):
    return oracle.kda_fwd(inp["q"], inp["k"], inp["v"], inp["g_raw"], inp["b"], inp["A_log"], inp["scale"],
                          gate_per_channel=inp["gate_per_channel"], initial_state=inp.get("initial_state"),
                          cu_seqlens=inp.get("cu_seqlens"), chain_mask=chain_mask)


def rel_l2(x, y):
    n = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / n) if n > 0 else float(np.linalg.norm(x))


def chain_errors(out, fin, ref_out, ref_fin, cu_seqlens=None):
    """Per-(chain, head) rel-L2 of the output and of the final state.

    out / ref_out: [B, T, H, V] (forward) or [B, H, V] (one decode step);
    fin / ref_fin: [C, H, V, K].  A chain is a batch row, or a packed
    sequence when cu_seqlens is given.  Chains the oracle did not compute
    (NaN in the reference) are skipped.  Returns a list of
    (chain, head, out rel-L2, final-state rel-L2).
    """
    if out.ndim == 3:
        out, ref_out = out[:, None], ref_out[:, None]
    B, T, H, _ = ref_out.shape
    if cu_seqlens is None:
        spans = [(b, b, slice(None)) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens)
        spans = [(n, 0, slice(int(cu[n]), int(cu[n + 1]))) for n in range(len(cu) - 1)]
    res = []
    for c, b, sl in spans:
        for h in range(H):
            ro, rf = ref_out[b, sl, h], ref_fin[c, h]
            if np.isnan(rf).any() or np.isnan(ro).any():
                continue
            res.append((c, h, rel_l2(out[b, sl, h], ro), rel_l2(fin[c, h], rf)))
    return res


def assert_parity(out, fin, ref_out, ref_fin, state_dtype=torch.float32, what="", cu_seqlens=None):
    """Pooled bars (out max-abs and rel-L2, final-state rel-L2) over every
    compared element, plus the rel-L2 bars per (chain, head), so an error
    confined to one chain cannot hide in the pooled norm."""
    sel = ~np.isnan(ref_out)
    o, ro = out[sel], ref_out[sel]
    maxabs = float(np.max(np.abs(o - ro))) if o.size else 0.0
    rel = rel_l2(o, ro)
    srel_bar = STATE_REL_FP32 if state_dtype == torch.float32 else STATE_REL_BF16
    fsel = ~np.isnan(ref_fin)
    frel = rel_l2(fin[fsel], ref_fin[fsel])
    per = chain_errors(out, fin, ref_out, ref_fin, cu_seqlens)
    worst_o = max(per, key=lambda r: r[2]) if per else (-1, -1, 0.0, 0.0)
    worst_f = max(per, key=lambda r: r[3]) if per else (-1, -1, 0.0, 0.0)
    msg = ("%s out max-abs %.3e rel-L2 %.3e | final rel-L2 %.3e | %d chains, worst out rel-L2 %.3e (chain %d "
           "head %d), worst final rel-L2 %.3e (chain %d head %d)" % (
               what, maxabs, rel, frel, len(per), worst_o[2], worst_o[0], worst_o[1], worst_f[3], worst_f[0],
               worst_f[1]))
    print(msg, flush=True)
    assert np.all(np.isfinite(out)), "non-finite output " + msg
    assert maxabs <= OUT_MAXABS and rel <= OUT_REL, msg
    assert frel <= srel_bar, msg
    assert worst_o[2] <= OUT_REL, "per-chain output bar: " + msg
    assert worst_f[3] <= srel_bar, "per-chain final-state bar: " + msg
    return maxabs, rel, frel
