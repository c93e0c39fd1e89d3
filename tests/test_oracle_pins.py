"""Pins for the fp64 CPU oracle: checks against what the pages and the
mathematics fix, independent of the oracle's own code.

Each test names the passage it follows. Together they are chosen so that a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
the oracle fails at least one of them:

* worked examples printed on the pages (online normaliser, softmax Jacobian);
* the pages' own algorithms (per-element online softmax, block merge of
  (m, l, O~)) evaluated here in Python, which must reach the oracle's plain
  definition exactly up to rounding;
* brute force with the textbook softmax (no max subtraction, exact sums);
* closed forms (constant V, Q = 0) and invariants;
* central finite differences of the forward for every gradient.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------

def test_online_normaliser_worked_example(oracle_lib):
    """Flash Attention notes, 'Online Softmax' part 6: x = [1,3,2,5].

    With d = 1, every query equal to 1, keys equal to x and scale 1, row i of
    the causal product sees exactly x[0..i], so its LSE is m_i + ln l_i for
    the running (m, l) of the page's table, step by step."""
    ex = _load("online_softmax_worked_example.json")
    x = np.array(ex["x"], dtype=np.float64)
    N = len(x)
    q = np.ones((N, 1))
    k = x.reshape(N, 1)
    v = np.eye(N)[:, :1]  # any V; only LSE is checked here
    half_ulp = 0.5 * 10.0 ** (-ex["printed_decimals"])
    _, lse = oracle_lib.attention_fwd(q, k, v, 1.0, causal=True)
    for i, st in enumerate(ex["steps"]):
        l_oracle = math.exp(lse[i] - st["m"])
        assert abs(l_oracle - st["l"]) <= half_ulp, (i, l_oracle, st)
    # the page's standard (non-causal) computation: m = 5, l = 1.2034
    _, lse_nc = oracle_lib.attention_fwd(q, k, v, 1.0, causal=False)
    assert np.all(np.abs(np.exp(lse_nc - 5.0) - ex["steps"][-1]["l"]) <= half_ulp)
    # the final terms exp(x_j - m) = P_j * l, read off P of the last row
    _, _, P = oracle_lib.attention_fwd_rows(q[-1:], [N - 1], k, v, 1.0, True,
                                            return_p=True)
    terms = P[0] * math.exp(lse[-1] - 5.0)
    assert np.all(np.abs(terms - np.array(ex["final_terms"])) <= half_ulp)


def test_softmax_jacobian_worked_example(oracle_lib):
    """Appendix A, conclusion 2, part 7: s = (1, 2), dp = (1, 0).

    Two queries equal to 1 (d = 1), keys (1, 2), scale 1: both score rows are
    s. V = [[1], [0]] and dO = [[1], [0]] make row 0 of dP = dO V^T equal to
    (1, 0) and row 1 zero, so row 0 of dS is the page's ds, rho is D_0, and
    dK_j = sum_i dS_ij q_i = ds_j, dQ_0 = ds . k, dV_j = P_0j."""
    ex = _load("softmax_jacobian_example.json")
    tol = 0.5 * 10.0 ** (-ex["printed_decimals"])
    q = np.ones((2, 1))
    k = np.array([[1.0], [2.0]])
    v = np.array([[1.0], [0.0]])
    do = np.array([[1.0], [0.0]])
    o, _ = oracle_lib.attention_fwd(q, k, v, 1.0, causal=False)
    g = oracle_lib.attention_bwd(q, k, v, do, 1.0, causal=False, return_ds=True)
    p = o[0, 0], 1.0 - o[0, 0]  # O_0 = P_00 * 1 + P_01 * 0
    assert abs(p[0] - ex["p"][0]) <= tol and abs(p[1] - ex["p"][1]) <= tol
    assert abs(g["D"][0] - ex["rho"]) <= tol
    assert np.all(np.abs(g["dS"][0] - np.array(ex["ds"])) <= tol)
    assert np.all(np.abs(g["dS"][1]) <= 1e-15)
    assert np.all(np.abs(g["dk"][:, 0] - np.array(ex["ds"])) <= tol)
    assert abs(g["dq"][0, 0] - (ex["ds"][0] * 1 + ex["ds"][1] * 2)) <= 3 * tol
    assert np.all(np.abs(g["dv"][:, 0] - np.array(ex["p"])) <= tol)
    # the page's Jacobian J = diag(p) - p p^T, applied to dp
    J = np.array(ex["jacobian"])
    assert np.all(np.abs(J @ np.array(ex["dp"]) - g["dS"][0]) <= 2 * tol)
    # exact values: p_1 = 1/(1+e), ds_1 = p_1 p_2
    p1 = 1.0 / (1.0 + math.e)
    assert abs(g["dS"][0, 0] - p1 * (1 - p1)) <= 1e-15
    assert abs(g["dS"][0, 1] + p1 * (1 - p1)) <= 1e-15


# ---------------------------------------------------------------------------
# The pages' algorithms, evaluated here, against the oracle's definition
# ---------------------------------------------------------------------------

def _online_normaliser(x):
    """Per-element online softmax (Online Softmax part 2, the boxed update):
    l_{i+1} = l_i * e^{m_i - m_{i+1}} + e^{x_{i+1} - m_{i+1}}."""
    m, l = -math.inf, 0.0
    for xi in x:
        m_new = max(m, xi)
        l = l * math.exp(m - m_new) + math.exp(xi - m_new)
        m = m_new
    return m, l


@pytest.mark.parametrize("magnitude", [1.0, 30.0, 1000.0])
def test_online_normaliser_equals_oracle_lse(oracle_lib, magnitude):
    """The 2-pass online normaliser (part 2.2) and the oracle's 3-pass safe
    softmax (part 1.3) give the same LSE, including at |x| ~ 1000 where the
    naive exp overflows (part 1.2)."""
    rng = _rng(1)
    for trial in range(20):
        N = int(rng.integers(1, 200))
        x = rng.standard_normal(N) * magnitude
        m, l = _online_normaliser(x)
        q = np.ones((1, 1))
        _, lse = oracle_lib.attention_fwd_rows(q, [N - 1], x.reshape(N, 1),
                                               np.zeros((N, 1)), 1.0, False)
        ref = m + math.log(l)
        assert abs(lse[0] - ref) <= 1e-15 * max(1.0, abs(ref)) * 8, (trial, lse[0], ref)


def _block_stats(s, v):
    """(m, l, O~) of one key block: Online Softmax parts 3.1 and 4.1."""
    m = s.max()
    if m == -math.inf:
        return -math.inf, 0.0, np.zeros(v.shape[1])
    w = np.exp(s - m)
    return m, w.sum(), w @ v


def _merge(a, b):
    """The boxed merges of parts 3.1 and 4.1:
    m = max(m_A, m_B), l = l_A e^{m_A-m} + l_B e^{m_B-m}, same for O~."""
    (ma, la, oa), (mb, lb, ob) = a, b
    m = max(ma, mb)
    if m == -math.inf:
        return a
    fa, fb = math.exp(ma - m), math.exp(mb - m)
    return m, la * fa + lb * fb, oa * fa + ob * fb


def _blocked_row(s, v, cuts, order):
    blocks = [_block_stats(s[a:b], v[a:b]) for a, b in zip(cuts[:-1], cuts[1:])]
    if order == "left":
        acc = blocks[0]
        for bl in blocks[1:]:
            acc = _merge(acc, bl)
    elif order == "right":
        acc = blocks[-1]
        for bl in reversed(blocks[:-1]):
            acc = _merge(bl, acc)
    else:  # pairwise tree
        while len(blocks) > 1:
            nxt = [_merge(blocks[i], blocks[i + 1]) for i in range(0, len(blocks) - 1, 2)]
            if len(blocks) % 2:
                nxt.append(blocks[-1])
            blocks = nxt
        acc = blocks[0]
    m, l, ot = acc
    return ot / l, m + math.log(l)


@pytest.mark.parametrize("causal", [False, True])
def test_block_merge_any_partition_equals_oracle(oracle_lib, causal):
    """Merging per-block (m, l, O~) in any partition and any association order
    (the merge is associative, Online Softmax part 3.1) reaches the oracle's
    O and LSE to rounding."""
    rng = _rng(2)
    N, d, scale = 97, 8, 0.35
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    o_ref, lse_ref = oracle_lib.attention_fwd(q, k, v, scale, causal)
    for bs in (1, 3, 16, 64, N):
        cuts = list(range(0, N, bs)) + [N]
        for order in ("left", "right", "tree"):
            for i in (0, 1, 40, N - 1):
                s = scale * (k @ q[i])
                if causal:
                    s[i + 1:] = -math.inf
                o, lse = _blocked_row(s, v, cuts, order)
                assert np.allclose(o, o_ref[i], rtol=1e-13, atol=1e-13), (bs, order, i)
                assert abs(lse - lse_ref[i]) <= 1e-13 * max(1, abs(lse_ref[i]))


def test_brute_force_textbook_softmax(oracle_lib):
    """Tiny inputs against the naive definition (Online Softmax part 1.1,
    y_i = e^{x_i} / sum_j e^{x_j}) with exactly rounded sums (math.fsum)."""
    rng = _rng(3)
    for trial in range(30):
        N = int(rng.integers(1, 7)); d = int(rng.integers(1, 5))
        causal = bool(trial % 2)
        scale = float(rng.uniform(0.1, 1.5))
        q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        o, lse = oracle_lib.attention_fwd(q, k, v, scale, causal)
        for i in range(N):
            w = []
            for j in range(N):
                if causal and j > i:
                    w.append(0.0)
                else:
                    w.append(math.exp(scale * math.fsum(q[i, c] * k[j, c] for c in range(d))))
            Z = math.fsum(w)
            for c in range(d):
                ref = math.fsum(w[j] * v[j, c] for j in range(N)) / Z
                assert abs(o[i, c] - ref) <= 1e-14 * max(1.0, abs(ref)), (trial, i, c)
            assert abs(lse[i] - math.log(Z)) <= 1e-14 * max(1.0, abs(math.log(Z)))


# ---------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_rows_reproduce_v(oracle_lib, causal):
    """Rows of P sum to 1, so V_j = v for all j gives O_i = v."""
    rng = _rng(4)
    N, d = 50, 6
    q = rng.standard_normal((N, d)) * 3; k = rng.standard_normal((N, d)) * 3
    vrow = rng.standard_normal(d)
    v = np.tile(vrow, (N, 1))
    o, _ = oracle_lib.attention_fwd(q, k, v, 0.7, causal)
    assert np.allclose(o, vrow[None, :], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_gives_mean_of_v(oracle_lib, causal):
    """Q = 0 makes every score 0: O_i is the mean of the visible V rows and
    LSE_i = ln(count) -- N without the mask, i + 1 with it."""
    rng = _rng(5)
    N, d = 33, 5
    q = np.zeros((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    o, lse = oracle_lib.attention_fwd(q, k, v, 0.9, causal)
    for i in range(N):
        n = i + 1 if causal else N
        assert np.allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - math.log(n)) <= 1e-14


def test_key_shift_and_permutation_invariance(oracle_lib):
    """Adding the same vector c to every key adds q_i.c to a whole score row,
    which softmax ignores; permuting K and V rows together (no mask) permutes
    the terms of each row sum."""
    rng = _rng(6)
    N, d = 40, 7
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    o, lse = oracle_lib.attention_fwd(q, k, v, 0.5, False)
    c = rng.standard_normal(d)
    o2, lse2 = oracle_lib.attention_fwd(q, k + c, v, 0.5, False)
    assert np.allclose(o2, o, rtol=0, atol=1e-13)
    assert np.allclose(lse2 - lse, 0.5 * (q @ c), rtol=0, atol=1e-13)
    perm = rng.permutation(N)
    o3, lse3 = oracle_lib.attention_fwd(q, k[perm], v[perm], 0.5, False)
    assert np.allclose(o3, o, rtol=0, atol=1e-13)
    assert np.allclose(lse3, lse, rtol=0, atol=1e-13)


def test_causal_row_equals_noncausal_prefix(oracle_lib):
    """Row i of the causal product equals the unmasked product over keys 0..i
    (the mask removes exactly the keys j > i)."""
    rng = _rng(7)
    N, d = 30, 4
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    o, lse = oracle_lib.attention_fwd(q, k, v, 0.8, True)
    for i in (0, 5, 17, N - 1):
        oi, li = oracle_lib.attention_fwd_rows(q[i:i + 1], [N], k[:i + 1], v[:i + 1], 0.8, False)
        assert np.allclose(oi[0], o[i], rtol=0, atol=1e-14)
        assert abs(li[0] - lse[i]) <= 1e-14


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(oracle_lib, causal):
    """Central differences of L = sum(dO o O) with respect to every entry of
    Q, K and V agree with the oracle's dQ, dK, dV (backward derivation page,
    parts 3 and 4, with the scale carried through S = scale Q K^T)."""
    rng = _rng(8 + causal)
    for N, d in ((1, 3), (5, 2), (8, 4)):
        scale = 0.7
        q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d)); do = rng.standard_normal((N, d))
        g = oracle_lib.attention_bwd(q, k, v, do, scale, causal)

        def loss(q_, k_, v_):
            o, _ = oracle_lib.attention_fwd(q_, k_, v_, scale, causal)
            return float(np.sum(do * o))

        for name, x, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                h = 1e-6 * max(1.0, abs(x[idx]))
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
                args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
                num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                            loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            err = np.abs(num - grad).max()
            assert err <= 1e-6 * max(1.0, np.abs(num).max()), (name, N, d, err)


@pytest.mark.parametrize("causal", [False, True])
def test_d_identity(oracle_lib, causal):
    """rowsum(dP o P) = rowsum(dO o O) (backward derivation page, part 5)."""
    rng = _rng(10)
    N, d = 64, 16
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d)); do = rng.standard_normal((N, d))
    g = oracle_lib.attention_bwd(q, k, v, do, 0.25, causal)
    assert np.allclose(g["D"], g["Dprime"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_sum_identities(oracle_lib, causal):
    """sum_j dS_ij = 0 (the Jacobian's columns sum to zero, since rows of P
    sum to 1), hence sum_j dK_j = scale * sum_i (sum_j dS_ij) Q_i = 0; and
    sum_j dV_j = sum_j sum_i P_ij dO_i = sum_i dO_i."""
    rng = _rng(11)
    N, d = 48, 6
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d)); do = rng.standard_normal((N, d))
    g = oracle_lib.attention_bwd(q, k, v, do, 0.6, causal, return_ds=True)
    assert np.allclose(g["dS"].sum(axis=1), 0.0, atol=1e-13)
    assert np.allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)
    assert np.allclose(g["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_constant_upstream_dp_gives_zero_ds(oracle_lib):
    """Conclusion 2: a dp constant along the row gives ds = 0. Equal V rows
    make dP_ij = dO_i . v constant in j, so dS, dQ and dK vanish."""
    rng = _rng(12)
    N, d = 20, 3
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = np.tile(rng.standard_normal(d), (N, 1)); do = rng.standard_normal((N, d))
    g = oracle_lib.attention_bwd(q, k, v, do, 1.0, False, return_ds=True)
    assert np.abs(g["dS"]).max() <= 1e-14
    assert np.abs(g["dq"]).max() <= 1e-13 and np.abs(g["dk"]).max() <= 1e-13


def test_cross_entropy_special_case(oracle_lib):
    """Conclusion 2, part 9: with dp = -y / p for a distribution y, the
    general formula reduces to ds = p - y. With d = N and V = I, dP = dO, so
    choosing dO_i = -y_i / P_i (P from a closed-form softmax of the scores)
    must give dS = P - Y."""
    rng = _rng(13)
    N = 6
    q = rng.standard_normal((N, N)); k = rng.standard_normal((N, N))
    v = np.eye(N)
    s = 0.4 * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True)); p /= p.sum(axis=1, keepdims=True)
    y = rng.dirichlet(np.ones(N), size=N)
    do = -y / p
    g = oracle_lib.attention_bwd(q, k, v, do, 0.4, False, return_ds=True)
    assert np.allclose(g["dS"], p - y, rtol=0, atol=1e-12)


def test_thread_count_does_not_change_results(oracle_lib):
    """Each output element is summed by one thread in a fixed order."""
    rng = _rng(14)
    N, d = 70, 8
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d)); do = rng.standard_normal((N, d))
    n0 = oracle_lib.num_threads()
    try:
        oracle_lib.set_num_threads(1)
        a = oracle_lib.attention_bwd(q, k, v, do, 0.3, True)
        oracle_lib.set_num_threads(max(2, n0))
        b = oracle_lib.attention_bwd(q, k, v, do, 0.3, True)
    finally:
        oracle_lib.set_num_threads(n0)
    for key in ("dq", "dk", "dv", "D"):
        assert np.array_equal(a[key], b[key])


# ---------------------------------------------------------------------------
# The merge of partial results (Online Softmax parts 3.1 and 4.1), as used
# by the split-KV forward: pinned against the forward's plain definition.
# ---------------------------------------------------------------------------

def _partials_over_key_sets(oracle_lib, q, k, v, scale, key_sets):
    """Non-causal attention of every query over each key subset, by the
    oracle's plain definition restricted to those keys."""
    qpos = np.arange(q.shape[0])
    o_parts, lse_parts = [], []
    for ks in key_sets:
        o, lse = oracle_lib.attention_fwd_rows(q, qpos, k[ks], v[ks], scale, False)
        o_parts.append(o)
        lse_parts.append(lse)
    return np.stack(o_parts), np.stack(lse_parts)


@pytest.mark.parametrize("split", ["contiguous", "strided", "uneven"])
def test_lse_merge_of_key_subsets_equals_full_attention(oracle_lib, split):
    """Attention over disjoint key subsets, merged, is attention over all
    keys (the merge is exact, not an approximation)."""
    rng = _rng(11)
    N, d, scale = 41, 6, 0.4
    q = rng.standard_normal((N, d)) * 2.0
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    keys = np.arange(N)
    if split == "contiguous":
        sets = [keys[:10], keys[10:30], keys[30:]]
    elif split == "strided":
        sets = [keys[r::4] for r in range(4)]
    else:
        sets = [keys[:1], keys[1:2], keys[2:]]
    o_parts, lse_parts = _partials_over_key_sets(oracle_lib, q, k, v, scale, sets)
    o, lse = oracle_lib.lse_merge(o_parts, lse_parts)
    o_ref, lse_ref = oracle_lib.attention_fwd(q, k, v, scale, False)
    assert np.allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, lse_ref, rtol=1e-13, atol=1e-13)


def test_lse_merge_ignores_empty_parts_and_order(oracle_lib):
    """A part with LSE = -inf (no visible key) contributes nothing, the
    order of the parts does not matter, a single part passes through, and a
    row with only empty parts gets O = 0, LSE = -inf."""
    rng = _rng(12)
    N, d, scale = 17, 5, 0.6
    q = rng.standard_normal((N, d)); k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    keys = np.arange(N)
    o_parts, lse_parts = _partials_over_key_sets(oracle_lib, q, k, v, scale,
                                                 [keys[:7], keys[7:]])
    o2, lse2 = oracle_lib.lse_merge(o_parts, lse_parts)
    junk = rng.standard_normal((1, N, d)) * 1e3
    o3, lse3 = oracle_lib.lse_merge(np.concatenate([o_parts[:1], junk, o_parts[1:]]),
                                    np.concatenate([lse_parts[:1], np.full((1, N), -np.inf),
                                                    lse_parts[1:]]))
    assert np.allclose(o3, o2, rtol=1e-14, atol=1e-14) and np.allclose(lse3, lse2, rtol=1e-14)
    o4, lse4 = oracle_lib.lse_merge(o_parts[::-1], lse_parts[::-1])
    assert np.allclose(o4, o2, rtol=1e-13, atol=1e-13) and np.allclose(lse4, lse2, rtol=1e-13)
    o1, lse1 = oracle_lib.lse_merge(o_parts[:1], lse_parts[:1])
    assert np.allclose(o1, o_parts[0], rtol=1e-14, atol=1e-14)
    assert np.array_equal(lse1, lse_parts[0])
    o0, lse0 = oracle_lib.lse_merge(junk, np.full((1, N), -np.inf))
    assert np.all(o0 == 0.0) and np.all(lse0 == -np.inf)


def test_rows_at_offset_positions_equal_prefix_attention(oracle_lib):
    """Queries appended after a cached prefix (query i at position Nk - Nq + i)
    under the causal mask: each equals unmasked attention over the keys up to
    its position, and the last one sees every key."""
    rng = _rng(31)
    Nq, Nk, d = 5, 23, 4
    q = rng.standard_normal((Nq, d)); k = rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, d))
    pos = np.arange(Nq) + Nk - Nq
    o, lse = oracle_lib.attention_fwd_rows(q, pos, k, v, 0.7, True)
    for i, p in enumerate(pos):
        oi, li = oracle_lib.attention_fwd_rows(q[i:i + 1], [Nk], k[:p + 1], v[:p + 1], 0.7, False)
        assert np.allclose(oi[0], o[i], rtol=0, atol=1e-14)
        assert abs(li[0] - lse[i]) <= 1e-14
    assert pos[-1] == Nk - 1
