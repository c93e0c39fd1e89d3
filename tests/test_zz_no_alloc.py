"""fa_bwd_noalloc (the backward with D in the library's static scratch)
against fa_bwd on the same inputs, through the C ABI: two calls in a row on
one device, the second on a smaller problem, so that the second reuses
scratch the first left filled. The two entry points run the same kernels on
the same inputs, so the gradients must be identical bit for bit (stronger
than the oracle tolerances); the first call is also checked against the
fp64 oracle on two slices."""
import ctypes

import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import check_grads, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


def _noalloc(fa, d, o, lse, w, outs):
    """One fa_bwd_noalloc call through ctypes into preallocated outputs."""
    code = {torch.bfloat16: fa.BF16, torch.float16: fa.F16}[d["q"].dtype]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fa.lib().fa_bwd_noalloc(code, w.B, w.H, w.N, w.d, P(d["q"]), P(d["k"]), P(d["v"]),
                                 P(o), P(d["do"]), P(lse), w.scale, int(w.causal),
                                 P(outs[0]), P(outs[1]), P(outs[2]), st)
    assert rc == 0, fa.lib().fa_status_str(rc)


@pytest.mark.parametrize("first,second", [
    (("big", 4, 8, 1500, 128, "bf16", True), ("small", 1, 3, 333, 128, "bf16", True)),
    (("big64", 2, 16, 2048, 64, "f16", False), ("small64", 1, 1, 70, 64, "f16", False)),
    (("big64c", 2, 8, 2000, 64, "bf16", True), ("small64c", 1, 2, 300, 64, "bf16", True)),
])
def test_noalloc_matches_fa_bwd(fa, oracle_lib, first, second):
    for i, spec in enumerate((first, second)):
        name, B, H, N, dd, dt, causal = spec
        w = ai.custom("noalloc-" + name, B, H, N, dd, dt, causal, seed=600 + i)
        print("noalloc call %d: %s" % (i + 1, w), flush=True)
        inp = ai.make_inputs(w)
        d = {k: v.cuda() for k, v in inp.items()}
        o, lse = fa.fwd(d["q"], d["k"], d["v"], w.scale, w.causal)
        ref = fa.bwd(d["q"], d["k"], d["v"], o, d["do"], lse, w.scale, w.causal)
        outs = tuple(torch.full_like(d["q"], float("nan")) for _ in range(3))
        _noalloc(fa, d, o, lse, w, outs)
        torch.cuda.synchronize()
        for a, b, key in zip(outs, ref, ("dq", "dk", "dv")):
            assert torch.equal(a, b), (w.name, key)
        # the binding's face of the same entry point, allocating its outputs
        got = fa.bwd_noalloc(d["q"], d["k"], d["v"], o, d["do"], lse, w.scale, w.causal)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        if i == 0:
            for b_, h_ in ((0, 0), (B - 1, H - 1)):
                q, k, v, do = (f64(inp[x][b_, h_]) for x in ("q", "k", "v", "do"))
                g = oracle_lib.attention_bwd(q, k, v, do, w.scale, w.causal)
                check_grads(w.dtype, {n: f64(t[b_, h_]) for n, t in zip(("dq", "dk", "dv"), outs)},
                            {n: g[n] for n in ("dq", "dk", "dv")}, what=w.name)


def test_noalloc_refuses_too_many_rows(fa):
    """B*H*N above the scratch size: an error before anything is enqueued."""
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    p = q.data_ptr()
    rc = fa.lib().fa_bwd_noalloc(fa.BF16, 1 << 12, 1 << 10, 2, 64, p, p, p, p, p, p, 0.125, 0,
                                 p, p, p, None)
    assert rc == -5, rc
    assert "scratch" in fa.lib().fa_status_str(rc).decode()
