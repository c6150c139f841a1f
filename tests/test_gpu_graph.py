"""A whole step (indexer, top-k, attention) captured once in a HIP graph and replayed.

The library's calls launch only kernels on the caller's stream (workspaces are allocated before the
calls, flags and histograms are cleared by kernels, never by memset), so a step prepared on a stream can
be captured on it and replayed.  Every replay, with eager work and synchronizations of the program in
between, must give outputs bit-identical to the eager step's: the top-k indices and every attention
layer's output.
"""
import pytest
import torch

from workloads import CONFIGS, make_inputs
from workloads.step import Step

pytestmark = pytest.mark.gpu

CASES = {
    "full_decode_small": CONFIGS["full_decode_64k"].replace(batch=7, q_tokens=7, context=3001, ragged=True),
    "reindex_small": CONFIGS["reindex_decode_1m"].replace(batch=7, q_tokens=7, context=40001, n_blocks=200,
                                                          ragged=True),
    "lowp_score_free": CONFIGS["lowp_full_decode_1m"].replace(batch=5, q_tokens=5, context=100003, ragged=True),
    "prefill_small": CONFIGS["prefill_4096_at_128k"].replace(q_tokens=300, context=2000, reuse_layers=2),
}


def _snapshot(st):
    return [st.idx.clone()] + [o.clone() for o in st.outs]


def _same(a, b):
    return all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x, y.view(torch.int16)
                           if y.dtype == torch.bfloat16 else y) for x, y in zip(a, b))


@pytest.mark.parametrize("name", list(CASES))
def test_step_graph_replays_equal_eager(name):
    cfg = CASES[name]
    print(f"\n[graph] {name}", flush=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x = make_inputs(cfg, 31, device="cuda")
        st = Step(cfg, x)            # the prepared calls are bound to this stream
        st()
        st()
    s.synchronize()
    want = _snapshot(st)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        st()
    for rep in range(3):
        for t in [st.idx] + st.outs:  # overwrite the outputs eagerly, so each replay must rewrite them
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(st)
        assert _same(got, want), f"replay {rep} differs from the eager step"
        junk = torch.randn(1 << 20, device="cuda").sum()  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
