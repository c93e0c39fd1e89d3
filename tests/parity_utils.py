"""Tolerances and comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (in the test, against the fp64 oracle on the same rounded inputs):
  fp32 inputs:      O and LSE max-abs error <= 1e-5
  fp16/bf16 inputs: O max-abs <= 2e-2 and rel-L2 <= 1e-2; LSE max-abs <= 1e-3
  gradients:        dQ, dK, dV rel-L2 <= 2e-2 each
rel-L2(x, ref) = ||x - ref||_2 / ||ref||_2 over the compared elements.
"""
import numpy as np
import torch

TOL = {
    "f32": {"o_abs": 1e-5, "lse_abs": 1e-5},
    "f16": {"o_abs": 2e-2, "o_rel": 1e-2, "lse_abs": 1e-3, "g_rel": 2e-2},
    "bf16": {"o_abs": 2e-2, "o_rel": 1e-2, "lse_abs": 1e-3, "g_rel": 2e-2},
}


def f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def rel_l2(x, ref):
    x, ref = f64(x), f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return num / den if den > 0 else num


def max_abs(x, ref):
    x, ref = f64(x), f64(ref)
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def check_fwd(dtype, o, lse, o_ref, lse_ref, what=""):
    t = TOL[dtype]
    e_o, e_l = max_abs(o, o_ref), max_abs(lse, lse_ref)
    assert np.all(np.isfinite(f64(o))) and np.all(np.isfinite(f64(lse))), what
    assert e_o <= t["o_abs"], "%s O max-abs %.3g > %.3g" % (what, e_o, t["o_abs"])
    assert e_l <= t["lse_abs"], "%s LSE max-abs %.3g > %.3g" % (what, e_l, t["lse_abs"])
    if "o_rel" in t:
        r = rel_l2(o, o_ref)
        assert r <= t["o_rel"], "%s O rel-L2 %.3g > %.3g" % (what, r, t["o_rel"])
    return e_o, e_l


def check_grads(dtype, got, ref, what=""):
    t = TOL[dtype]
    out = {}
    for name in ("dq", "dk", "dv"):
        assert np.all(np.isfinite(f64(got[name]))), (what, name)
        r = rel_l2(got[name], ref[name])
        out[name] = r
        assert r <= t["g_rel"], "%s %s rel-L2 %.3g > %.3g" % (what, name, r, t["g_rel"])
    return out
