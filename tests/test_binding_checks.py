"""Argument checks of the Python binding that guard the kernels' indexing.

The staged backward entry points index LSE and D as fp32 [B, H, N] on the
device of Q, and every workspace as device memory of the size the library
asked for; anything else would make a kernel read or write out of bounds.
The binding rejects such arguments with ValueError before any call into the
library. The CPU tests exercise the checks themselves; the GPU tests confirm
that each staged wrapper applies them (no kernel is launched: the check
comes first)."""
import pytest
import torch

import exact_attention_34_amd as fa


def _ref(B=2, H=3, N=5, d=64):
    return torch.zeros(B, H, N, d, dtype=torch.bfloat16)


@pytest.mark.parametrize("bad", [
    torch.zeros(2, 3, 5, dtype=torch.bfloat16),          # wrong dtype
    torch.zeros(2, 3, 5, dtype=torch.float64),
    torch.zeros(2, 3, 6, dtype=torch.float32),           # wrong N
    torch.zeros(3, 2, 5, dtype=torch.float32),           # B and H swapped
    torch.zeros(2, 3, 5, 1, dtype=torch.float32),        # extra dimension
    torch.zeros(2, 5, 3, dtype=torch.float32).transpose(1, 2),  # not contiguous
    torch.zeros(2, 3, 5, dtype=torch.float32, device="meta"),   # another device
    None,
])
def test_row_vector_check_rejects(bad):
    with pytest.raises(ValueError):
        fa._check_rows(bad, "lse", _ref())


def test_row_vector_check_accepts():
    fa._check_rows(torch.zeros(2, 3, 5, dtype=torch.float32), "lse", _ref())


@pytest.mark.parametrize("bad", [
    torch.zeros(99, dtype=torch.uint8),                  # too small
    torch.zeros(200, dtype=torch.uint8)[::2],            # not contiguous
    torch.zeros(100, dtype=torch.uint8, device="meta"),  # another device
    "not a tensor",
])
def test_workspace_check_rejects(bad):
    with pytest.raises(ValueError):
        fa._workspace(bad, 100, _ref())


def test_workspace_check_accepts_and_allocates():
    ws = torch.zeros(25, dtype=torch.float32)            # 100 bytes
    assert fa._workspace(ws, 100, _ref()) is ws
    new = fa._workspace(None, 300, _ref())
    assert new.numel() == 300 and new.device == _ref().device


@pytest.mark.gpu
def test_staged_wrappers_reject_bad_vectors():
    B, H, N, d = 1, 2, 64, 64
    q = torch.zeros(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    good = torch.zeros(B, H, N, dtype=torch.float32, device="cuda")
    bads = [torch.zeros(B, H, N, dtype=torch.bfloat16, device="cuda"),
            torch.zeros(B, H, N - 1, dtype=torch.float32, device="cuda"),
            torch.zeros(B, H, N, dtype=torch.float32)]        # host memory
    for bad in bads:
        with pytest.raises(ValueError):
            fa.bwd_preprocess(q, q, bad)
        with pytest.raises(ValueError):
            fa.bwd_dkdv(q, q, q, q, bad, good, out, out)
        with pytest.raises(ValueError):
            fa.bwd_dkdv(q, q, q, q, good, bad, out, out)
        with pytest.raises(ValueError):
            fa.bwd_dq(q, q, q, q, bad, good, out)
        with pytest.raises(ValueError):
            fa.bwd_dq_d(q, q, q, q, q, good, bad, out)
        with pytest.raises(ValueError):
            fa.bwd(q, q, q, q, q, bad)
        with pytest.raises(ValueError):
            fa.bwd_dq_ws(q, q, q, q, q, bad, out, torch.zeros(1 << 16, dtype=torch.uint8,
                                                               device="cuda"))
    for ws in (None, torch.zeros(16, dtype=torch.uint8, device="cuda"),
               torch.zeros(1 << 16, dtype=torch.uint8)):
        with pytest.raises(ValueError):
            fa.bwd_dq_ws(q, q, q, q, q, good, out, ws)
        with pytest.raises(ValueError):
            fa.bwd_dkdv_ws(q, q, q, q, out, out, ws)
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, q, good, workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, q, good, workspace=torch.zeros(1 << 16, dtype=torch.uint8))
