"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

* Small shapes (one to a few tiles, ragged tails, N = 1) are compared element
  by element on every slice.
* The five workloads run at full size in the same launch configuration the
  benchmark times; the oracle checks sampled (batch, head) slices in full.
* Invariants that need no oracle run at full size: constant V rows, Q = 0,
  the gradient sums, determinism.
Tolerances are in parity_utils.TOL.
"""
import math

import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import TOL, check_fwd, check_grads, f64, max_abs, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


def _gpu(inp):
    return {k: v.to("cuda") for k, v in inp.items()}


def _run(fa, w, inp, backward=True):
    d = _gpu(inp)
    o, lse = fa.fwd(d["q"], d["k"], d["v"], w.scale, w.causal)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], o, d["do"], lse, w.scale, w.causal)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def _compare_slices(oracle, w, inp, got, slices, backward):
    fwd_o, fwd_o_ref, lse, lse_ref = [], [], [], []
    grads = {k: [] for k in ("dq", "dk", "dv")}
    grads_ref = {k: [] for k in ("dq", "dk", "dv")}
    for b, h in slices:
        q, k, v = (f64(inp[x][b, h]) for x in ("q", "k", "v"))
        o_ref, l_ref = oracle.attention_fwd(q, k, v, w.scale, w.causal)
        fwd_o.append(f64(got["o"][b, h])); fwd_o_ref.append(o_ref)
        lse.append(f64(got["lse"][b, h])); lse_ref.append(l_ref)
        if backward:
            g = oracle.attention_bwd(q, k, v, f64(inp["do"][b, h]), w.scale, w.causal)
            for name in grads:
                grads[name].append(f64(got[name][b, h])); grads_ref[name].append(g[name])
    e = check_fwd(w.dtype, np.stack(fwd_o), np.stack(lse), np.stack(fwd_o_ref),
                  np.stack(lse_ref), what=w.name)
    r = None
    if backward:
        r = check_grads(w.dtype, {k: np.stack(v) for k, v in grads.items()},
                        {k: np.stack(v) for k, v in grads_ref.items()}, what=w.name)
    print("%s slices=%s O/LSE max-abs=%.3g/%.3g grads rel-L2=%s" % (w.name, slices, e[0], e[1], r),
          flush=True)


# ---------------------------------------------------------------------------
# Small shapes: every slice, every element
# ---------------------------------------------------------------------------

SMALL = [(dt, d, causal, N) for dt in ("bf16", "f16") for d in (64, 128)
         for causal in (False, True) for N in (1, 17, 64, 65, 130, 257)]


@pytest.mark.parametrize("dt,d,causal,N", SMALL)
def test_small_fwd_bwd(fa, oracle_lib, dt, d, causal, N):
    w = ai.custom("small-%s-d%d-%s-N%d" % (dt, d, "c" if causal else "nc", N), 1, 2, N, d, dt,
                  causal, seed=1000 + N + d)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1)], True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 129, 300])
def test_small_fwd_f32(fa, oracle_lib, d, causal, N):
    w = ai.Workload("f32-d%d-N%d" % (d, N), 1, 2, N, d, "f32", causal, False, 2000 + N)
    inp = ai.make_inputs(w, with_do=False)
    got = _run(fa, w, inp, backward=False)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1)], False)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 2, 1000), (2, 64, 300)])
def test_fwd_f32_both_paths(fa, oracle_lib, d, causal, B, H, N):
    """fp32 forward on both sides of the launcher's rule. B1 H2 N1000: 16 blocks
    of 128 rows, so each 32-row group runs in one workgroup whose waves split its
    32 key tiles (4 or 8 each) and merge their parts; B2 H64 N300: 384 blocks,
    one workgroup per 128-row block (fwd_f32_kernel)."""
    w = ai.Workload("f32-paths-d%d-B%dH%dN%d" % (d, B, H, N), B, H, N, d, "f32", causal, False,
                    3000 + N + d)
    inp = ai.make_inputs(w, with_do=False)
    got = _run(fa, w, inp, backward=False)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (B - 1, H - 1)], False)


@pytest.mark.parametrize("causal", [False, True])
def test_many_tiles_ragged(fa, oracle_lib, causal):
    """N = 1000: 8 query blocks and 16 key tiles, the last ones partial."""
    w = ai.custom("mid", 2, 2, 1000, 128, "bf16", causal, seed=77)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1), (1, 0), (1, 1)], True)


# ---------------------------------------------------------------------------
# The five workloads at full size; sampled slices checked by the oracle
# ---------------------------------------------------------------------------

def _corners_and_random(B, H, extra, seed):
    """The four corner (batch, head) slices and `extra` others drawn at random."""
    corners = sorted({(0, 0), (0, H - 1), (B - 1, 0), (B - 1, H - 1)})
    rest = [(b, h) for b in range(B) for h in range(H) if (b, h) not in corners]
    rng = np.random.default_rng(seed)
    pick = rng.choice(len(rest), min(extra, len(rest)), replace=False)
    return corners + sorted(rest[i] for i in pick)


SAMPLES = {
    "c1": [(0, 0)],
    "c2": [(0, 0), (0, 5), (1, 2), (1, 7)],
    "c3": _corners_and_random(4, 32, 6, seed=3),
    "c4": [(0, 0), (0, 7), (0, 15)],
    "c5": _corners_and_random(16, 32, 8, seed=5),
}


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_parity(fa, oracle_lib, name):
    w = ai.WORKLOADS[name]
    print("workload", w, flush=True)
    inp = ai.make_inputs(w, with_do=w.backward)
    got = _run(fa, w, inp, backward=w.backward)
    _compare_slices(oracle_lib, w, inp, got, SAMPLES[name], w.backward)


def test_c4_forward_rows_more_slices(fa, oracle_lib):
    """c4 at full size: forward rows sampled from every head (row-wise oracle)."""
    w = ai.WORKLOADS["c4"]
    inp = ai.make_inputs(w, with_do=False)
    got = _run(fa, w, inp, backward=False)
    rng = np.random.default_rng(4)
    for h in range(w.H):
        rows = np.sort(rng.choice(w.N, 24, replace=False))
        rows[0], rows[-1] = 0, w.N - 1
        k, v = f64(inp["k"][0, h]), f64(inp["v"][0, h])
        o_ref, l_ref = oracle_lib.attention_fwd_rows(f64(inp["q"][0, h])[rows], rows, k, v,
                                                     w.scale, True)
        check_fwd(w.dtype, f64(got["o"][0, h])[rows], f64(got["lse"][0, h])[rows], o_ref,
                  l_ref, what="c4 head %d" % h)


@pytest.mark.parametrize("name", ["perf-8k", "perf-8k-causal"])
def test_headline_shape(fa, oracle_lib, name):
    """The N = 8192 throughput shape (B2 H16 d128 bf16) in the launch
    configuration the benchmark times: one slice's forward and backward in
    full against the oracle, and 16 forward rows from every other slice."""
    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, [(1, 7)], True)
    rng = np.random.default_rng(8)
    for b in range(w.B):
        for h in range(w.H):
            if (b, h) == (1, 7):
                continue
            rows = np.sort(rng.choice(w.N, 16, replace=False))
            rows[0], rows[-1] = 0, w.N - 1
            k, v = f64(inp["k"][b, h]), f64(inp["v"][b, h])
            o_ref, l_ref = oracle_lib.attention_fwd_rows(f64(inp["q"][b, h])[rows], rows, k, v,
                                                         w.scale, w.causal)
            check_fwd(w.dtype, f64(got["o"][b, h])[rows], f64(got["lse"][b, h])[rows], o_ref,
                      l_ref, what="%s slice %d,%d" % (name, b, h))


@pytest.mark.parametrize("causal,N", [(False, 4000), (True, 4500)])
def test_eight_wave_blocks_ragged(fa, oracle_lib, causal, N):
    """Shapes on which the forward and the dQ sweep run 256-row workgroups
    (B*H = 64 slices give at least one such unit per CU, and N >= 4096 under
    the mask), with a partial last block and a partial last key tile."""
    w = ai.custom("w8-%s-N%d" % ("c" if causal else "nc", N), 4, 16, N, 128, "bf16", causal,
                  seed=55)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (3, 15)], True)


@pytest.mark.parametrize("causal", [False, True])
def test_block_size_independence(fa, causal):
    """The query-block size is the library's choice (256 rows when the grid
    has enough such units, else 128) and no row's arithmetic depends on it:
    a slice computed inside a B4 H16 N4096 batch (256-row blocks in the
    forward and the dQ sweep) equals the same slice computed alone (128-row
    blocks), O, LSE, dQ, dK and dV bit for bit."""
    assert fa_launch_rule(64, 4096, causal) and not fa_launch_rule(1, 4096, causal)
    w = ai.custom("bs-%s" % ("c" if causal else "nc"), 4, 16, 4096, 128, "bf16", causal, seed=77)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    for b, h in [(0, 0), (3, 15)]:
        one = {k: v[b:b + 1, h:h + 1].contiguous() for k, v in inp.items()}
        w1 = ai.custom("bs-one", 1, 1, 4096, 128, "bf16", causal, seed=77)
        alone = _run(fa, w1, one)
        for k in ("o", "lse", "dq", "dk", "dv"):
            assert torch.equal(alone[k][0, 0], got[k][b, h]), (k, b, h)


def fa_launch_rule(BH, N, causal):
    """The library's rule for 256-row blocks (fa_launch.h, use_256_row_blocks)."""
    nqb = (N + 255) // 256
    units = BH * ((nqb + 1) // 2 if causal else nqb)
    return units >= 256 and (not causal or N >= 4096)


def single_block_rule(d, N, causal):
    """The library's rule for single query blocks in longest-first order
    (fa_launch.h, use_single_block_order), and its slices per group
    (single_block_group)."""
    return causal and d == 64 and N <= 4096


def single_block_group(BH, N, d):
    return max(1, min(BH, (4 << 20) // (4 * N * d)))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_single_block_order_groups(fa, oracle_lib, dt):
    """Causal d = 64, N = 2000: the forward and the dQ sweep take single
    query blocks longest first over groups of 8 slices; B3 H7 gives groups of
    8, 8 and 5 slices, so the last group is short. Slices at the ends of every
    group against the oracle."""
    B, H, N = 3, 7, 2000
    S = single_block_group(B * H, N, 64)
    assert single_block_rule(64, N, True) and S == 8 and (B * H) % S != 0
    w = ai.custom("lpt-groups-%s" % dt, B, H, N, 64, dt, True, seed=31)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    ends = sorted({i for g0 in range(0, B * H, S) for i in (g0, min(g0 + S, B * H) - 1)})
    _compare_slices(oracle_lib, w, inp, got, [divmod(i, H) for i in ends], True)


@pytest.mark.parametrize("N", [4096, 4097])
def test_single_block_rule_boundary(fa, oracle_lib, N):
    """Causal d = 64 on both sides of the single-block rule (N = 4096 single
    blocks in longest-first order, N = 4097 pairs of blocks with a one-row
    last block): two slices against the oracle."""
    assert single_block_rule(64, N, True) == (N == 4096)
    w = ai.custom("lpt-edge-%d" % N, 2, 2, N, 64, "f16", True, seed=47)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (1, 1)], True)


@pytest.mark.parametrize("dt,causal", [("bf16", False), ("f16", True)])
def test_d64_sweep_streams_several_units(fa, oracle_lib, dt, causal):
    """d = 64 with more key-block units than compute units, so that every
    workgroup of the dK/dV sweep walks several units (blocks of different
    slices, the next block's rows and first tile loaded during the previous
    block's last step), N = 2000 leaving a partial last key block and query
    tile: corner slices and two others against the oracle."""
    w = ai.custom("d64-units-%s-%s" % (dt, "c" if causal else "nc"), 4, 16, 2000, 64, dt,
                  causal, seed=64)
    inp = ai.make_inputs(w)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, _corners_and_random(4, 16, 2, seed=9), True)


# ---------------------------------------------------------------------------
# Score ranges that keep moving the running max
# ---------------------------------------------------------------------------

def _scale_keys(inp, factor):
    """Key row j multiplied by factor[j], rounded to the dtype again (the
    oracle sees the same rounded keys)."""
    dt = inp["k"].dtype
    inp["k"] = (inp["k"].double() * factor[:, None]).to(dt).contiguous()
    return inp


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_rising_along_keys(fa, oracle_lib, dt, causal):
    """Key j scaled by 1 + 40 j / N: a row's largest score keeps growing over
    the sweep (to about 40 times the usual spread at the end), so the running
    max m moves in many tiles and O~ and l are rescaled each time."""
    N = 1000
    w = ai.custom("rising-%s-%s" % (dt, "c" if causal else "nc"), 1, 2, N, 128, dt, causal,
                  seed=91)
    inp = _scale_keys(ai.make_inputs(w, with_do=False),
                      1 + 40 * torch.arange(N, dtype=torch.float64) / N)
    got = _run(fa, w, inp, backward=False)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1)], False)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_one_key_far_above_the_rest(fa, oracle_lib, dt, causal):
    """Key 700 scaled by 30: in about half of the rows its score lies tens of
    units above everything before it, so exponentials taken against the
    earlier max would overflow fp16 and fp32; the sweep must move m first."""
    N = 900
    w = ai.custom("spike-%s-%s" % (dt, "c" if causal else "nc"), 1, 2, N, 64, dt, causal,
                  seed=92)
    f = torch.ones(N, dtype=torch.float64)
    f[700] = 30.0
    inp = _scale_keys(ai.make_inputs(w, with_do=False), f)
    got = _run(fa, w, inp, backward=False)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1)], False)


@pytest.mark.parametrize("scale", [1e-3, 4.0])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_scales(fa, oracle_lib, scale, causal):
    """scale = 1e-3 (P nearly uniform: O near the mean of the visible V rows)
    and scale = 4 (scores spread over hundreds of units: P nearly one-hot and
    the reference moves often), forward and backward, bf16 d = 128."""
    import types
    base = ai.custom("scale-%g-%s" % (scale, "c" if causal else "nc"), 1, 2, 700, 128, "bf16",
                     causal, seed=95)
    w = types.SimpleNamespace(name=base.name, scale=scale, causal=causal, dtype=base.dtype)
    inp = ai.make_inputs(base)
    got = _run(fa, w, inp)
    _compare_slices(oracle_lib, w, inp, got, [(0, 0), (0, 1)], True)


# ---------------------------------------------------------------------------
# Invariants at full size (no oracle)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c3", "c5"])
def test_constant_v_rows(fa, name):
    """Rows of P sum to one: V_j = v for every j gives O_i = v."""
    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w, with_do=False)
    v = inp["v"][:, :, :1, :].expand_as(inp["v"]).contiguous()
    inp["v"] = v
    got = _run(fa, w, inp, backward=False)
    err = max_abs(got["o"], v)
    assert err <= 2 * 2.0 ** -8 * float(v.abs().max()), err


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_zero_q_gives_mean(fa, name):
    """Q = 0: O_i is the mean of the visible V rows, LSE_i = ln(count)."""
    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w, with_do=False)
    inp["q"] = torch.zeros_like(inp["q"])
    got = _run(fa, w, inp, backward=False)
    n = torch.arange(1, w.N + 1, dtype=torch.float64) if w.causal else \
        torch.full((w.N,), float(w.N), dtype=torch.float64)
    assert max_abs(got["lse"], torch.log(n).expand(w.B, w.H, w.N)) <= 1e-5
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        vv = inp["v"][b, h].double()
        ref = torch.cumsum(vv, 0) / n[:, None] if w.causal else vv.mean(0).expand_as(vv)
        assert max_abs(got["o"][b, h], ref) <= 2e-2
        assert rel_l2(got["o"][b, h], ref) <= 1e-2


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_gradient_sums_and_determinism(fa, name):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per slice; O, LSE, dQ, dK
    and dV are bitwise reproducible."""
    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w)
    a = _run(fa, w, inp)
    b = _run(fa, w, inp)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key
    dk = a["dk"].double()
    dv = a["dv"].double()
    do = inp["do"].double()
    sk = dk.sum(2).norm(dim=-1) / dk.norm(dim=(2, 3))
    assert float(sk.max()) <= 2e-2, float(sk.max())
    sv = (dv.sum(2) - do.sum(2)).norm(dim=-1) / do.sum(2).norm(dim=-1)
    assert float(sv.max()) <= 2e-2, float(sv.max())


def _coarse(t):
    """Values on the grid of multiples of 1/16 inside (-4, 4): sums of two such
    values stay below 8 in magnitude and are exact in bf16 and fp16."""
    return (torch.round(t.double() * 16).clamp(-63, 63) / 16).to(t.dtype).contiguous()


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_key_shift_invariance(fa, name):
    """K_j -> K_j + c for every key j adds scale q_i . c to every score of
    row i: P, and so O, dV and dK, are unchanged; LSE_i moves by scale q_i . c;
    dQ moves by scale (sum_j dS_ij) c = 0 because the rows of dS sum to zero.
    K and c are taken on a coarse grid so that K + c is exact in the dtype,
    and the two runs differ only in the kernels' rounding."""
    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w)
    inp["k"] = _coarse(inp["k"])
    g = torch.Generator().manual_seed(17)
    c = _coarse(torch.randn(w.B, w.H, 1, w.d, generator=g)).to(inp["k"].dtype)
    shifted = dict(inp, k=(inp["k"].double() + c.double()).to(inp["k"].dtype).contiguous())
    assert torch.equal(shifted["k"].double() - inp["k"].double(), c.double().expand_as(inp["k"]))
    a = _run(fa, w, inp)
    b = _run(fa, w, shifted)
    assert max_abs(b["o"], a["o"]) <= 2e-2
    assert rel_l2(b["o"], a["o"]) <= 4e-3
    qc = w.scale * (inp["q"].double() * c.double()).sum(-1)    # scale q_i . c
    assert max_abs(b["lse"].double() - a["lse"].double(), qc) <= 2e-3
    for key in ("dq", "dk", "dv"):
        r = rel_l2(b[key], a[key])
        assert r <= 1e-2, (key, r)


def test_joint_key_value_permutation(fa):
    """Without the mask, permuting the rows of K and V together permutes the
    terms of every row's sums only: O, LSE and dQ are unchanged, and dK, dV
    come out permuted the same way (c3 at full size)."""
    w = ai.WORKLOADS["c3"]
    inp = ai.make_inputs(w)
    perm = torch.randperm(w.N, generator=torch.Generator().manual_seed(23))
    moved = dict(inp, k=inp["k"][:, :, perm].contiguous(), v=inp["v"][:, :, perm].contiguous())
    a = _run(fa, w, inp)
    b = _run(fa, w, moved)
    assert max_abs(b["o"], a["o"]) <= 2e-2
    assert rel_l2(b["o"], a["o"]) <= 4e-3
    assert max_abs(b["lse"], a["lse"]) <= 1e-4
    assert rel_l2(b["dq"], a["dq"]) <= 1e-2
    for key in ("dk", "dv"):
        r = rel_l2(b[key], a[key][:, :, perm])
        assert r <= 1e-2, (key, r)


@pytest.mark.parametrize("hd,dt", [(128, "bf16"), (64, "f16")])
def test_stages_match_fused_call(fa, hd, dt):
    """fa_bwd equals its three stages called one by one, in either order of
    the two gradient sweeps, equals fa_bwd_dq_d then fa_bwd_dkdv, and equals
    its own two launches called apart (fa_bwd_dq_ws, fa_bwd_dkdv_ws); the D
    that fa_bwd_dq_d forms equals fa_bwd_preprocess's bit for bit. At d = 64
    (causal, N <= 4096) the dQ sweeps are the single-block kernels, both the
    one forming D and the one reading it."""
    if hd == 64:
        assert single_block_rule(64, 700, True)
    w = ai.custom("stages-d%d" % hd, 2, 4, 700, hd, dt, True, seed=11)
    d = _gpu(ai.make_inputs(w))
    o, lse = fa.fwd(d["q"], d["k"], d["v"], w.scale, True)
    dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], o, d["do"], lse, w.scale, True)
    dvec = torch.empty_like(lse)
    dk2, dv2, dq2 = torch.empty_like(dk), torch.empty_like(dv), torch.empty_like(dq)
    fa.bwd_preprocess(o, d["do"], dvec)
    ref_d = (o.float() * d["do"].float()).sum(-1)
    assert torch.allclose(dvec, ref_d, rtol=1e-4, atol=1e-4)
    fa.bwd_dq(d["q"], d["k"], d["v"], d["do"], lse, dvec, dq2, w.scale, True)
    fa.bwd_dkdv(d["q"], d["k"], d["v"], d["do"], lse, dvec, dk2, dv2, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2) and torch.equal(dq, dq2)
    dvec3 = torch.full_like(dvec, float("nan"))
    dk3, dv3, dq3 = torch.empty_like(dk), torch.empty_like(dv), torch.empty_like(dq)
    fa.bwd_dq_d(d["q"], d["k"], d["v"], o, d["do"], lse, dvec3, dq3, w.scale, True)
    fa.bwd_dkdv(d["q"], d["k"], d["v"], d["do"], lse, dvec3, dk3, dv3, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(dvec3, dvec)
    assert torch.equal(dk, dk3) and torch.equal(dv, dv3) and torch.equal(dq, dq3)
    # fa_bwd's two launches as two calls, on a workspace that starts as NaN.
    ws = torch.full((fa.bwd_workspace_bytes(d["q"].dtype, 2, 4, 700, w.d),), 255,
                    dtype=torch.uint8, device="cuda")
    dk4, dv4, dq4 = torch.empty_like(dk), torch.empty_like(dv), torch.empty_like(dq)
    fa.bwd_dq_ws(d["q"], d["k"], d["v"], o, d["do"], lse, dq4, ws, w.scale, True)
    fa.bwd_dkdv_ws(d["q"], d["k"], d["v"], d["do"], dk4, dv4, ws, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk4) and torch.equal(dv, dv4) and torch.equal(dq, dq4)


def test_nan_in_query_row_stays_in_that_row(fa):
    w = ai.custom("nan", 1, 1, 200, 64, "bf16", False, seed=3)
    inp = ai.make_inputs(w)
    inp["q"][0, 0, 37, 5] = float("nan")
    got = _run(fa, w, inp, backward=False)
    o = got["o"][0, 0].float()
    assert torch.isnan(o[37]).all()
    assert torch.isfinite(torch.cat([o[:37], o[38:]])).all()
