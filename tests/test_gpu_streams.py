"""Streams and graph capture. Every entry point enqueues on the stream it is
given and allocates nothing, so the calls can run on a side stream and be
captured into a HIP graph (torch.cuda.CUDAGraph) for replay, as a serving
loop or a training step would. The kernels are deterministic, so results
must match the eager default-stream run bit for bit."""
import pytest
import torch

import attn_inputs as ai

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_34_amd as fa
    fa.lib()
    return fa


def _dev(w):
    return {k: v.cuda() for k, v in ai.make_inputs(w).items()}


def _fwd_bwd(fa, d, w):
    o, lse = fa.fwd(d["q"], d["k"], d["v"], w.scale, w.causal)
    dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], o, d["do"], lse, w.scale, w.causal)
    return [o, lse, dq, dk, dv]


@pytest.mark.parametrize("causal", [False, True])
def test_side_stream_matches_default_stream(fa, causal):
    w = ai.custom("side-stream", 2, 4, 1000, 128, "bf16", causal, seed=71)
    d = _dev(w)
    ref = [t.clone() for t in _fwd_bwd(fa, d, w)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = _fwd_bwd(fa, d, w)
    s.synchronize()  # only the side stream: the work must have been queued there
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


@pytest.mark.parametrize("causal", [False, True])
def test_graph_replays_match_eager(fa, causal):
    """Forward + backward captured once and replayed on new inputs copied
    into the captured buffers; eager runs and synchronisations between the
    replays; every replay is checked against the eager result."""
    w = ai.custom("graph", 2, 4, 777, 64, "bf16", causal, seed=72)
    static = _dev(w)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):  # warm-up outside the capture
            _fwd_bwd(fa, static, w)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _fwd_bwd(fa, static, w)
    for rep in range(4):
        new = _dev(ai.custom("graph", 2, 4, 777, 64, "bf16", causal, seed=100 + rep))
        for k in static:
            static[k].copy_(new[k])
        g.replay()
        torch.cuda.synchronize()
        ref = _fwd_bwd(fa, new, w)
        torch.cuda.synchronize()
        for name, r, o in zip(("o", "lse", "dq", "dk", "dv"), ref, outs):
            assert torch.equal(r, o), (rep, name)


def test_decode_graph_replays_match_eager(fa):
    """One decoding step (one new query per slice over a 4096-key cache, the
    split-key path with its workspace) captured and replayed."""
    B, H, Nk, d = 4, 8, 4096, 128
    gen = torch.Generator(device="cuda").manual_seed(73)
    k = torch.randn(B, H, Nk, d, generator=gen, device="cuda").bfloat16()
    v = torch.randn(B, H, Nk, d, generator=gen, device="cuda").bfloat16()
    q = torch.randn(B, H, 1, d, generator=gen, device="cuda").bfloat16()
    scale = d ** -0.5
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.fwd_kvcache(q, k, v, scale, True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, lse = fa.fwd_kvcache(q, k, v, scale, True)
    for rep in range(4):
        q.copy_(torch.randn(B, H, 1, d, generator=gen, device="cuda").bfloat16())
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = fa.fwd_kvcache(q, k, v, scale, True)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
