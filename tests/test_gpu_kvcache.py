"""GPU parity of attention over a cached prefix (fa_fwd_kvcache).

Nq new queries over Nk keys; under the causal mask query i sits at position
Nk - Nq + i. The oracle is attention_fwd_rows with those positions (the plain
definition, pinned on the CPU to equal unmasked attention over each query's
visible prefix). Also: the pages' incremental use of the online-softmax state
-- the state over a prefix of the keys, updated with the keys that arrive
later through fa_lse_merge, equals attention over all keys at once.
"""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from parity_utils import check_fwd, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


def _qkv(B, H, Nq, Nk, d, dt, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Nq, d, generator=g).to(ai.DTYPES[dt])
    k = torch.randn(B, H, Nk, d, generator=g).to(ai.DTYPES[dt])
    v = torch.randn(B, H, Nk, d, generator=g).to(ai.DTYPES[dt])
    return q, k, v


CASES = [(dt, d, causal, Nq, Nk, ns) for dt, d in (("bf16", 128), ("f16", 64))
         for causal in (False, True)
         for Nq, Nk, ns in ((1, 1, 0), (1, 777, 0), (1, 4096, 8), (7, 300, 2), (128, 1000, 3),
                            (200, 200, 0), (300, 5000, 0))]
# without the mask the query count is free: more new queries than keys
CASES += [(dt, d, False, Nq, Nk, ns) for dt, d in (("bf16", 128), ("f16", 64))
          for Nq, Nk, ns in ((300, 70, 0), (129, 64, 2))]


@pytest.mark.parametrize("dt,d,causal,Nq,Nk,nsplit", CASES)
def test_kvcache_matches_oracle(fa, oracle_lib, dt, d, causal, Nq, Nk, nsplit):
    B, H = 1, 2
    q, k, v = _qkv(B, H, Nq, Nk, d, dt, seed=Nq * 7 + Nk + d)
    o, lse = fa.fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), d ** -0.5, causal, nsplit)
    torch.cuda.synchronize()
    pos = np.arange(Nq) + (Nk - Nq if causal else 0)
    for h in range(H):
        o_ref, l_ref = oracle_lib.attention_fwd_rows(f64(q[0, h]), pos, f64(k[0, h]),
                                                     f64(v[0, h]), d ** -0.5, causal)
        check_fwd(dt, f64(o[0, h]), f64(lse[0, h]), o_ref, l_ref,
                  what="kvcache Nq%d Nk%d" % (Nq, Nk))


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("Nk,nsplit", [(33, 0), (300, 1), (5000, 0), (5000, 7), (20000, 0)])
def test_decode_many_slices(fa, oracle_lib, dt, d, Nk, nsplit):
    """One new query per slice (the vector decoding kernel): 15 slices, key
    ranges from one partial batch to many per wave, against the oracle on
    every slice."""
    B, H = 3, 5
    q, k, v = _qkv(B, H, 1, Nk, d, dt, seed=Nk + nsplit + d)
    o, lse = fa.fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), d ** -0.5, True, nsplit)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            o_ref, l_ref = oracle_lib.attention_fwd_rows(f64(q[b, h]), np.array([Nk - 1]),
                                                         f64(k[b, h]), f64(v[b, h]), d ** -0.5,
                                                         True)
            check_fwd(dt, f64(o[b, h]), f64(lse[b, h]), o_ref, l_ref,
                      what="decode Nk%d nsplit%d" % (Nk, nsplit))


def test_kvcache_equals_fwd_when_nq_equals_nk(fa):
    """Nq = Nk with the causal mask is the ordinary causal forward."""
    w = ai.custom("kv-eq", 2, 3, 650, 128, "bf16", True, seed=5)
    d = {x: t.cuda() for x, t in ai.make_inputs(w, with_do=False).items()}
    o1, l1 = fa.fwd(d["q"], d["k"], d["v"], w.scale, True)
    o2, l2 = fa.fwd_kvcache(d["q"], d["k"], d["v"], w.scale, True, 3)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3


def test_prefix_state_updated_by_new_keys(fa, oracle_lib):
    """The online-softmax state (O, LSE) of queries over a cached prefix of the
    keys, merged with their state over the keys that arrive afterwards, is
    attention over all keys (the merge of the Online Softmax notes, parts 3.1
    and 4.1, applied as the keys stream in)."""
    B, H, Nq, Nk, d = 2, 4, 64, 3000, 128
    q, k, v = _qkv(B, H, Nq, Nk, d, "bf16", seed=21)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    cut = [0, 1100, 2048, 2050, Nk]       # keys arrive in four pieces
    o_parts, l_parts = [], []
    for a, b in zip(cut[:-1], cut[1:]):
        o, l = fa.fwd_kvcache(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(),
                              d ** -0.5, False, 0)
        o_parts.append(o.float().reshape(-1, d))
        l_parts.append(l.reshape(-1))
    # the state after every piece: fold each new piece into the running state
    state_o, state_l = o_parts[0], l_parts[0]
    for po, pl in zip(o_parts[1:], l_parts[1:]):
        state_o, state_l = fa.lse_merge(torch.stack([state_o, po]).contiguous(),
                                        torch.stack([state_l, pl]).contiguous())
    torch.cuda.synchronize()
    o_all = state_o.reshape(B, H, Nq, d)
    l_all = state_l.reshape(B, H, Nq)
    for b, h in ((0, 0), (1, 3)):
        o_ref, l_ref = oracle_lib.attention_fwd_rows(f64(q[b, h]), np.arange(Nq), f64(k[b, h]),
                                                     f64(v[b, h]), d ** -0.5, False)
        check_fwd("bf16", f64(o_all[b, h]), f64(l_all[b, h]), o_ref, l_ref, what="stream")
