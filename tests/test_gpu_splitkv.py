"""GPU parity of the split-key forward and of the partial-result merge.

* fa_fwd_splitkv against the fp64 oracle (the plain definition over all keys)
  on small shapes, several split counts, ragged tails and the causal mask;
  and against fa_fwd on the under-filled c2 workload with the library's own
  split choice.
* fa_lse_merge against the oracle's merge (the two-block merge of the pages'
  online softmax, folded over the parts) on random parts, with empty parts
  and rows whose parts are all empty.
Tolerances are those of parity_utils.TOL; the merge in fp32 is held to the
fp32 bound (max-abs <= 1e-5).
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import TOL, check_fwd, f64, max_abs, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


CASES = [(dt, d, causal, N, ns) for dt, d in (("bf16", 128), ("f16", 64), ("bf16", 64))
         for causal in (False, True) for N, ns in ((1, 2), (65, 2), (257, 3), (1000, 5),
                                                   (1000, 64))]


@pytest.mark.parametrize("dt,d,causal,N,nsplit", CASES)
def test_splitkv_matches_oracle(fa, oracle_lib, dt, d, causal, N, nsplit):
    w = ai.custom("split-%s-d%d-N%d" % (dt, d, N), 1, 2, N, d, dt, causal, seed=3000 + N + d)
    inp = ai.make_inputs(w, with_do=False)
    dev = {k: v.cuda() for k, v in inp.items()}
    o, lse = fa.fwd_splitkv(dev["q"], dev["k"], dev["v"], w.scale, causal, nsplit)
    torch.cuda.synchronize()
    print(w.name, "causal", causal, "parts", fa.fwd_splitkv_parts(1, 2, N, nsplit, causal),
          flush=True)
    for h in range(2):
        o_ref, l_ref = oracle_lib.attention_fwd(f64(inp["q"][0, h]), f64(inp["k"][0, h]),
                                                f64(inp["v"][0, h]), w.scale, causal)
        check_fwd(dt, f64(o[0, h]), f64(lse[0, h]), o_ref, l_ref, what=w.name)


@pytest.mark.parametrize("nsplit", [0, 2, 4])
def test_splitkv_on_underfilled_grid(fa, oracle_lib, nsplit):
    """c2 (128 query blocks in all): the library's own choice (no split: its
    rows are too short to repay the merge) and explicit splits, against
    fa_fwd within the 16-bit tolerance and the oracle on sampled slices."""
    w = ai.WORKLOADS["c2"]
    inp = ai.make_inputs(w, with_do=False)
    dev = {k: v.cuda() for k, v in inp.items()}
    parts = fa.fwd_splitkv_parts(w.B, w.H, w.N, nsplit, w.causal)
    assert parts == (1 if nsplit == 0 else nsplit), parts
    o, lse = fa.fwd_splitkv(dev["q"], dev["k"], dev["v"], w.scale, w.causal, nsplit)
    o1, lse1 = fa.fwd(dev["q"], dev["k"], dev["v"], w.scale, w.causal)
    torch.cuda.synchronize()
    assert max_abs(o, o1) <= TOL[w.dtype]["o_abs"]
    assert max_abs(lse, lse1) <= TOL[w.dtype]["lse_abs"]
    if parts == 1:  # a single range runs the plain forward
        assert torch.equal(o, o1) and torch.equal(lse, lse1)
    for b, h in ((0, 0), (1, 7)):
        o_ref, l_ref = oracle_lib.attention_fwd(f64(inp["q"][b, h]), f64(inp["k"][b, h]),
                                                f64(inp["v"][b, h]), w.scale, w.causal)
        check_fwd(w.dtype, f64(o[b, h]), f64(lse[b, h]), o_ref, l_ref, what="c2 split")


def test_splitkv_deterministic(fa):
    w = ai.custom("split-det", 2, 3, 777, 128, "bf16", True, seed=9)
    d = {k: v.cuda() for k, v in ai.make_inputs(w, with_do=False).items()}
    a = fa.fwd_splitkv(d["q"], d["k"], d["v"], w.scale, True, 4)
    b = fa.fwd_splitkv(d["q"], d["k"], d["v"], w.scale, True, 4)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _random_parts(P, rows, d, seed, empty_frac=0.2):
    g = torch.Generator().manual_seed(seed)
    o = torch.randn(P, rows, d, generator=g, dtype=torch.float32)
    lse = 3.0 * torch.randn(P, rows, generator=g, dtype=torch.float32)
    drop = torch.rand(P, rows, generator=g) < empty_frac
    lse[drop] = -float("inf")
    o[drop] = 0.0
    lse[:, 5] = -float("inf")   # a row with only empty parts
    o[:, 5] = 0.0
    return o, lse


@pytest.mark.parametrize("P", [1, 2, 7])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_lse_merge_matches_oracle(fa, oracle_lib, P, d, out):
    o_parts, lse_parts = _random_parts(P, 300, d, seed=P * 100 + d)
    o, lse = fa.lse_merge(o_parts.cuda(), lse_parts.cuda(), ai.DTYPES[out])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_lib.lse_merge(f64(o_parts), f64(lse_parts))
    got_o, got_l = f64(o), f64(lse)
    empty = ~np.isfinite(l_ref)
    assert empty[5] and np.all(np.isneginf(got_l[empty])) and np.all(got_o[empty] == 0.0)
    keep = ~empty
    tol = TOL[out]
    assert max_abs(got_l[keep], l_ref[keep]) <= 1e-5
    if out == "f32":
        assert max_abs(got_o[keep], o_ref[keep]) <= tol["o_abs"]
    else:
        check_fwd(out, got_o[keep], got_l[keep], o_ref[keep], l_ref[keep], what="merge")


def test_splitkv_long_rows_small_grid(fa, oracle_lib):
    """B1 H4 N8192 causal (128 paired query-block units, fewer than the
    chip's compute units): the library splits the keys; sampled rows of every
    head against the row-wise oracle, including the first and last rows."""
    w = ai.custom("split-long", 1, 4, 8192, 128, "bf16", True, seed=42)
    inp = ai.make_inputs(w, with_do=False)
    dev = {k: v.cuda() for k, v in inp.items()}
    assert fa.fwd_splitkv_parts(w.B, w.H, w.N, 0, True) > 1
    o, lse = fa.fwd_splitkv(dev["q"], dev["k"], dev["v"], w.scale, True, 0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    for h in range(w.H):
        rows = np.sort(rng.choice(w.N, 16, replace=False))
        rows[0], rows[-1] = 0, w.N - 1
        o_ref, l_ref = oracle_lib.attention_fwd_rows(f64(inp["q"][0, h])[rows], rows,
                                                     f64(inp["k"][0, h]), f64(inp["v"][0, h]),
                                                     w.scale, True)
        check_fwd(w.dtype, f64(o[0, h])[rows], f64(lse[0, h])[rows], o_ref, l_ref,
                  what="split-long head %d" % h)
