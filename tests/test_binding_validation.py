"""The binding's checks of caller-supplied buffers (CPU only).

The C ABI receives bare pointers and cannot see buffer sizes, so the
binding must refuse an output, state or workspace that the kernels would
write past or misread.  The checks are exercised directly on CPU tensors
(the device of the inputs is passed in)."""

import pytest
import torch

from chunked_gated_delta_10_amd import kda

CPU = torch.device("cpu")


def test_out_accepts_exact_buffer():
    kda._check_out(torch.empty((2, 5, 3, 128), dtype=torch.bfloat16), (2, 5, 3, 128), CPU)


@pytest.mark.parametrize("out,exc", [
    (torch.empty((2, 5, 3, 128), dtype=torch.float32), TypeError),       # wrong dtype
    (torch.empty((2, 4, 3, 128), dtype=torch.bfloat16), ValueError),     # short
    (torch.empty((2, 5, 3, 129), dtype=torch.bfloat16), ValueError),     # long rows
    (torch.empty((2, 3, 5, 128), dtype=torch.bfloat16).transpose(1, 2), ValueError),  # not contiguous
    (torch.empty((2 * 5 * 3 * 128,), dtype=torch.bfloat16), ValueError),  # right size, wrong shape
])
def test_out_rejected(out, exc):
    with pytest.raises(exc):
        kda._check_out(out, (2, 5, 3, 128), CPU)


def test_out_on_other_device_rejected():
    with pytest.raises(ValueError):
        kda._check_out(torch.empty((1, 1, 1, 128), dtype=torch.bfloat16), (1, 1, 1, 128), torch.device("meta"))


@pytest.mark.parametrize("st,exc", [
    (torch.empty((2, 3, 128, 128), dtype=torch.float16), TypeError),
    (torch.empty((2, 3, 128, 127), dtype=torch.float32), ValueError),
    (torch.empty((2, 3, 128, 128), dtype=torch.float32).transpose(2, 3), ValueError),
])
def test_state_rejected(st, exc):
    with pytest.raises(exc):
        kda._check_state(st, "final_state", (2, 3, 128, 128), CPU)


def test_state_accepts_fp32_bf16_and_none():
    for dt in (torch.float32, torch.bfloat16):
        kda._check_state(torch.empty((2, 3, 128, 128), dtype=dt), "s", (2, 3, 128, 128), CPU)
    kda._check_state(None, "s", (2, 3, 128, 128), CPU)


@pytest.mark.parametrize("ws,exc", [
    (torch.empty(4096, dtype=torch.int32), TypeError),
    (torch.empty(100, dtype=torch.uint8), ValueError),
    (torch.empty((64, 128), dtype=torch.uint8).t(), ValueError),
])
def test_workspace_rejected(ws, exc):
    with pytest.raises(exc):
        kda._check_workspace(ws, 4096, CPU)


def test_workspace_accepts_large_enough_buffer():
    kda._check_workspace(torch.empty(5000, dtype=torch.uint8), 4096, CPU)


def test_inputs_must_share_a_device():
    a = torch.empty(3)
    with pytest.raises(ValueError):
        kda._same_device(a, a, torch.empty(3, device="meta"))
    kda._same_device(a, a, None, a)


def test_host_inputs_rejected_before_the_library_is_called():
    q = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        kda.fwd(q, q, q, q, torch.zeros((1, 4, 1)), torch.zeros(1))


@pytest.mark.parametrize("dout,dfinal,s0,exc", [
    (torch.empty((1, 5, 3, 128), dtype=torch.float32), None, None, TypeError),     # dout must be bf16
    (torch.empty((1, 5, 3, 128), dtype=torch.bfloat16), None, None, ValueError),   # not a device tensor
])
def test_bwd_upstream_rejected(dout, dfinal, s0, exc):
    with pytest.raises(exc):
        kda._bwd_checks(dout, dfinal, s0, 1, 5, 3, 128, 128, 1, CPU)
