"""GPU parity of the standard-attention path (S and P stored in device memory)
against the fp64 oracle, through the C ABI.

The path computes the same O, LSE, dQ, dK and dV as the tiled kernels up to
rounding, so the tolerances are the same (parity_utils.TOL). The stored P is
also checked directly: against the oracle's probabilities, its zero padding
and (causal) its zero upper triangle.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import TOL, check_fwd, check_grads, f64, max_abs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


def _run_std(fa, w, inp, backward=True):
    d = {k: v.to("cuda") for k, v in inp.items()}
    o, lse, P = fa.std_fwd(d["q"], d["k"], d["v"], w.scale, w.causal)
    out = {"o": o, "lse": lse, "P": P}
    if backward:
        dq, dk, dv = fa.std_bwd(d["q"], d["k"], d["v"], o, d["do"], P, w.scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def _check_slices(oracle, w, inp, got, slices, backward):
    os_, ors, ls, lrs = [], [], [], []
    g, gr = {k: [] for k in ("dq", "dk", "dv")}, {k: [] for k in ("dq", "dk", "dv")}
    for b, h in slices:
        q, k, v = (f64(inp[x][b, h]) for x in ("q", "k", "v"))
        o_ref, l_ref = oracle.attention_fwd(q, k, v, w.scale, w.causal)
        os_.append(f64(got["o"][b, h])); ors.append(o_ref)
        ls.append(f64(got["lse"][b, h])); lrs.append(l_ref)
        if backward:
            ref = oracle.attention_bwd(q, k, v, f64(inp["do"][b, h]), w.scale, w.causal)
            for n in g:
                g[n].append(f64(got[n][b, h])); gr[n].append(ref[n])
    e = check_fwd(w.dtype, np.stack(os_), np.stack(ls), np.stack(ors), np.stack(lrs),
                  what=w.name)
    r = None
    if backward:
        r = check_grads(w.dtype, {k: np.stack(v) for k, v in g.items()},
                        {k: np.stack(v) for k, v in gr.items()}, what=w.name)
    print("%s O/LSE max-abs %.3g/%.3g grads rel-L2 %s" % (w.name, e[0], e[1], r), flush=True)


SMALL = [(dt, d, causal, N) for dt in ("bf16", "f16") for d in (64, 128)
         for causal in (False, True) for N in (1, 17, 130, 257)]


@pytest.mark.parametrize("dt,d,causal,N", SMALL)
def test_std_small(fa, oracle_lib, dt, d, causal, N):
    """Every slice of small shapes: one partial 128-row tile up to three,
    N = 1, and rows whose stride carries padding."""
    w = ai.custom("std-%s-d%d-%s-N%d" % (dt, d, "c" if causal else "nc", N), 1, 2, N, d, dt,
                  causal, seed=2000 + N + d)
    inp = ai.make_inputs(w)
    got = _run_std(fa, w, inp)
    _check_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1)], True)


@pytest.mark.parametrize("causal", [False, True])
def test_std_stored_p(fa, oracle_lib, causal):
    """P as stored: the oracle's probabilities rounded to bf16 (within one
    rounding step), exact zeros in the padding columns and, under the mask,
    above the diagonal; rows sum to one within the rounding of N values."""
    N, d = 300, 64
    w = ai.custom("std-p-%s" % ("c" if causal else "nc"), 1, 1, N, d, "bf16", causal, seed=31)
    inp = ai.make_inputs(w, with_do=False)
    got = _run_std(fa, w, inp, backward=False)
    P = got["P"][0, 0].float().numpy().astype(np.float64)
    ld = fa.std_row_stride(N)
    assert P.shape == (N, ld)
    assert np.all(P[:, N:] == 0.0)
    q, k, v = (f64(inp[x][0, 0]) for x in ("q", "k", "v"))
    _, _, p_ref = oracle_lib.attention_fwd_rows(q, np.arange(N), k, v, w.scale, causal,
                                                return_p=True)
    err = np.abs(P[:, :N] - p_ref)
    assert np.all(err <= 2.0 ** -8 * p_ref + 1e-7), float(err.max())
    if causal:
        assert np.all(np.triu(P[:, :N], 1) == 0.0)
    assert np.max(np.abs(P.sum(1) - 1.0)) <= 4e-3


@pytest.mark.parametrize("causal", [False, True])
def test_std_medium_matches_oracle_and_tiled_path(fa, oracle_lib, causal):
    """B2 H4 N2048 d128 bf16 (16 column tiles per slice): sampled slices
    against the oracle, and every slice against the tiled kernels."""
    w = ai.custom("std-mid-%s" % ("c" if causal else "nc"), 2, 4, 2048, 128, "bf16", causal,
                  seed=33)
    inp = ai.make_inputs(w)
    got = _run_std(fa, w, inp)
    _check_slices(oracle_lib, w, inp, got, [(0, 0), (1, 3)], True)
    d = {k: v.to("cuda") for k, v in inp.items()}
    o, lse = fa.fwd(d["q"], d["k"], d["v"], w.scale, causal)
    dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], o, d["do"], lse, w.scale, causal)
    torch.cuda.synchronize()
    t = TOL["bf16"]
    assert max_abs(got["o"], o.cpu()) <= t["o_abs"]
    assert max_abs(got["lse"], lse.cpu()) <= t["lse_abs"]
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        a, b = f64(got[name]), f64(ref.cpu())
        assert np.linalg.norm(a - b) <= t["g_rel"] * np.linalg.norm(b), name
