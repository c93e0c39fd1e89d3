"""Tensors past 2^31 elements: B41 H400 N1024 d128 bf16 and B41 H800 N1024
d64 fp16 hold 2^31 + 2^21 elements per tensor, so the last slices start beyond
element 2^31. Forward and backward run on the whole batch; slices on both
sides of that boundary are compared with the fp64 oracle (parity_utils
tolerances). The causal d = 64 case runs the forward and the dQ sweep as
single query blocks in longest-first order over groups of 16 slices."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import check_fwd, check_grads, f64

pytestmark = pytest.mark.gpu

# (B, H, N, d, dtype) and the (b, h) slices compared, flattened: slice s
# starts at element s * N * d, which is 2^31 for s = 2^31 / (N d).
SHAPES = {"d128": (41, 400, 1024, 128, "bf16", [0, 16383, 16384, 16399]),
          "d64": (41, 800, 1024, 64, "f16", [0, 32767, 32768, 32799])}


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


@pytest.mark.parametrize("shape", ["d128", "d64"])
@pytest.mark.parametrize("causal", [False, True])
def test_tensors_past_4gib(fa, oracle_lib, causal, shape):
    if torch.cuda.get_device_properties(0).total_memory < (96 << 30):
        pytest.skip("needs about 45 GiB of device memory")
    B, H, N, d, dt, SLICES = SHAPES[shape]
    w = ai.custom("large-%s-%s" % (shape, "c" if causal else "nc"), B, H, N, d, dt, causal,
                  seed=4000 + int(causal))
    assert w.B * w.H * w.N * w.d > 2 ** 31
    assert SLICES[1] * N * d < 2 ** 31 <= SLICES[2] * N * d
    inp = ai.make_inputs_device(w)
    o, lse = fa.fwd(inp["q"], inp["k"], inp["v"], w.scale, causal)
    dq, dk, dv = fa.bwd(inp["q"], inp["k"], inp["v"], o, inp["do"], lse, w.scale, causal)
    torch.cuda.synchronize()
    H = w.H
    pick = lambda t: torch.stack([t[s // H, s % H] for s in SLICES]).cpu()
    host = {n: pick(t) for n, t in dict(inp, o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}
    del inp, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    os_, ors, ls, lrs = [], [], [], []
    g, gr = {n: [] for n in ("dq", "dk", "dv")}, {n: [] for n in ("dq", "dk", "dv")}
    for i in range(len(SLICES)):
        q, k, v, do = (f64(host[n][i]) for n in ("q", "k", "v", "do"))
        o_ref, l_ref = oracle_lib.attention_fwd(q, k, v, w.scale, causal)
        ref = oracle_lib.attention_bwd(q, k, v, do, w.scale, causal)
        os_.append(f64(host["o"][i])); ors.append(o_ref)
        ls.append(f64(host["lse"][i])); lrs.append(l_ref)
        for n in g:
            g[n].append(f64(host[n][i])); gr[n].append(ref[n])
    e = check_fwd(w.dtype, np.stack(os_), np.stack(ls), np.stack(ors), np.stack(lrs), what=w.name)
    r = check_grads(w.dtype, {n: np.stack(v) for n, v in g.items()},
                    {n: np.stack(v) for n, v in gr.items()}, what=w.name)
    print("%s slices %s: O/LSE max-abs %.3g/%.3g grads rel-L2 %s" % (w.name, SLICES, e[0], e[1], r),
          flush=True)
