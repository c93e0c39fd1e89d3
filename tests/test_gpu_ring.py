"""Sequence sharding on one GPU: the computation each device does in ring
attention ("Flash Attention" notes, Online Softmax part 7, item 2), with the
shards held on one GPU and the exchange left out.

The sequence is cut into P shards. Forward: query shard r folds, one key
shard at a time, the partial result over key shard s into its running
(O, LSE) with fa_lse_merge; the partials come from fa_fwd_kvcache (key
shard s < r: no mask; s = r: the causal mask on the diagonal block; s > r:
skipped under the causal mask). Backward: for every pair (r, s) the two
gradient sweeps run on the shards with the global LSE and D of shard r, and
dQ_r, dK_s, dV_s are the sums of the pair contributions. Both must give
attention over the whole sequence (the oracle) within the usual tolerances.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import check_fwd, check_grads, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


@pytest.mark.parametrize("causal", [False, True])
def test_sharded_forward_and_backward(fa, oracle_lib, causal):
    B, H, N, d, P = 1, 2, 1024, 128, 4
    w = ai.custom("ring", B, H, N, d, "bf16", causal, seed=66)
    inp = ai.make_inputs(w)
    q, k, v, do = (inp[x].cuda() for x in ("q", "k", "v", "do"))
    n = N // P
    sh = lambda t, r: t[:, :, r * n:(r + 1) * n].contiguous()
    o_parts, l_parts = [], []
    for r in range(P):
        state = None
        for s in range(P):
            if causal and s > r:
                continue
            o, l = fa.fwd_kvcache(sh(q, r), sh(k, s), sh(v, s), w.scale, causal and s == r, 0)
            part = (o.float().reshape(-1, d), l.reshape(-1))
            if state is None:
                state = part
            else:
                state = fa.lse_merge(torch.stack([state[0], part[0]]).contiguous(),
                                     torch.stack([state[1], part[1]]).contiguous())
        o_parts.append(state[0].reshape(B, H, n, d))
        l_parts.append(state[1].reshape(B, H, n))
    o_all = torch.cat(o_parts, 2)
    lse_all = torch.cat(l_parts, 2).contiguous()
    o16 = o_all.to(torch.bfloat16).contiguous()
    # backward: global D = rowsum(dO o O), then the sweeps per shard pair
    dvec = torch.empty_like(lse_all)
    fa.bwd_preprocess(o16, do, dvec)
    dq = torch.zeros(B, H, N, d, dtype=torch.float32, device="cuda")
    dk = torch.zeros_like(dq)
    dv = torch.zeros_like(dq)
    for r in range(P):
        for s in range(P):
            if causal and s > r:
                continue
            qr, dor = sh(q, r), sh(do, r)
            lr, dr = sh(lse_all, r), sh(dvec, r)
            ks, vs = sh(k, s), sh(v, s)
            pdq, pdk, pdv = (torch.empty_like(qr) for _ in range(3))
            diag = causal and s == r
            fa.bwd_dq(qr, ks, vs, dor, lr, dr, pdq, w.scale, diag)
            fa.bwd_dkdv(qr, ks, vs, dor, lr, dr, pdk, pdv, w.scale, diag)
            dq[:, :, r * n:(r + 1) * n] += pdq.float()
            dk[:, :, s * n:(s + 1) * n] += pdk.float()
            dv[:, :, s * n:(s + 1) * n] += pdv.float()
    torch.cuda.synchronize()
    for h in range(H):
        qh, kh, vh, doh = (f64(inp[x][0, h]) for x in ("q", "k", "v", "do"))
        o_ref, l_ref = oracle_lib.attention_fwd(qh, kh, vh, w.scale, causal)
        check_fwd("bf16", f64(o16[0, h]), f64(lse_all[0, h]), o_ref, l_ref, what="ring fwd")
        g = oracle_lib.attention_bwd(qh, kh, vh, doh, w.scale, causal)
        check_grads("bf16", {"dq": f64(dq[0, h]), "dk": f64(dk[0, h]), "dv": f64(dv[0, h])}, g,
                    what="ring bwd")
