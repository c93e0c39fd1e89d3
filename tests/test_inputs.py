"""The seeded input generator: deterministic, correctly shaped and rounded."""
import math

import torch

import attn_inputs as ai


def test_deterministic_and_dtype():
    w = ai.custom("t", 2, 3, 40, 64, "bf16", seed=5)
    a, b = ai.make_inputs(w), ai.make_inputs(w)
    for key in ("q", "k", "v", "do"):
        assert a[key].dtype == torch.bfloat16 and a[key].shape == (2, 3, 40, 64)
        assert torch.equal(a[key], b[key])
    c = ai.make_inputs(ai.custom("t", 2, 3, 40, 64, "bf16", seed=6))
    assert not torch.equal(a["q"], c["q"])


def test_draw_order_and_scaling():
    """Q, K, V, dO are drawn in that order; std scaling multiplies them."""
    w1 = ai.custom("t", 1, 1, 16, 64, "f32", seed=9)
    w2 = ai.custom("t", 1, 1, 16, 64, "f32", seed=9, qkv_std=0.5, do_std=0.1)
    a, b = ai.make_inputs(w1), ai.make_inputs(w2)
    g = torch.Generator().manual_seed(9)
    ref_q = torch.randn((1, 1, 16, 64), generator=g)
    assert torch.equal(a["q"], ref_q)
    assert torch.allclose(b["q"], 0.5 * a["q"]) and torch.allclose(b["v"], 0.5 * a["v"])
    assert torch.allclose(b["do"], 0.1 * a["do"])


def test_rope_rotates_pairs():
    """Rotary embedding keeps |(x_k, x_{k+d/2})| and leaves row 0 unchanged."""
    x = torch.randn(1, 1, 9, 8, dtype=torch.float64)
    y = ai._rope_fp64(x)
    assert torch.allclose(y[..., 0, :], x[..., 0, :])
    nx = x[..., :4] ** 2 + x[..., 4:] ** 2
    ny = y[..., :4] ** 2 + y[..., 4:] ** 2
    assert torch.allclose(nx, ny)
    # row 1, pair 0 turns by exactly 1 radian (theta_0 = 1)
    c, s = math.cos(1.0), math.sin(1.0)
    assert torch.allclose(y[0, 0, 1, 0], x[0, 0, 1, 0] * c - x[0, 0, 1, 4] * s)


def test_workload_table():
    w = ai.WORKLOADS
    assert (w["c1"].B, w["c1"].H, w["c1"].N, w["c1"].d, w["c1"].dtype) == (1, 1, 256, 64, "f32")
    assert w["c4"].causal and w["c4"].qkv_std == 0.5 and w["c4"].dtype == "f16"
    assert w["c5"].rope and w["c5"].causal and abs(w["c5"].do_std - 0.1) < 1e-12
    assert w["perf-8k"].fwd_flops() == 4.0 * 2 * 16 * 8192 ** 2 * 128
    assert w["perf-8k-causal"].bwd_flops() == 5.0 * 2 * 16 * 8192 ** 2 * 128
