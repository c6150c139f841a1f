"""The top-k entry point that allocates nothing (csa2_topk_select_noalloc) returns exactly what
csa2_topk_select returns with a workspace of its own, call after call on the same fixed scratch
array: a large wide-row call, then a smaller one (whose select must not read what the first left
behind), then a narrow call that needs no workspace."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _case(rows, width, seed, n_blocks=0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    scores = torch.randn(rows, width, generator=g, device="cuda", dtype=torch.float32)
    # exact ties across columns, -0 / +0, NaN and -inf sprinkled in
    scores[:, 5::97] = scores[:, 3:4]
    scores[:, 11::1013] = float("nan")
    scores[:, 17::389] = -0.0
    scores[:, 19::577] = float("-inf")
    hi = (width // 8 if n_blocks else width) - 1
    pos = torch.randint(0, max(hi, 1), (rows,), generator=g, device="cuda", dtype=torch.int64)
    pos[0] = hi
    if rows > 1:
        pos[1] = 100          # fewer visible columns than k
    cand = None
    if n_blocks:
        cand = torch.sort(torch.randperm(width // 8 // 1, generator=g, device="cuda")[:n_blocks]).values
        cand = cand.to(torch.int32).repeat(rows, 1).contiguous()
        cand[-1, -3:] = -1
    return scores, pos, cand


@pytest.mark.parametrize("order", ["big_then_small", "small_then_big"])
def test_noalloc_equals_workspace_call(order):
    import sparse_latent_attention_amd as csa2
    shapes = [(64, 1 << 20, 512, 0), (8, 100003, 512, 0), (5, 3000, 64, 0), (4, 16384, 512, 2048)]
    if order == "small_then_big":
        shapes = shapes[1:2] + shapes[:1] + shapes[2:]
    for i, (rows, width, k, nb) in enumerate(shapes):
        print(f"[noalloc] call {i}: rows={rows} width={width} k={k} reindex_blocks={nb}", flush=True)
        scores, pos, cand = _case(rows, width, 70 + i, nb)
        ref = torch.full((rows, k), -5, dtype=torch.int32, device="cuda")
        got = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        csa2.topk_select(scores, pos, 1, ref, cand=cand)
        csa2.topk_select_noalloc(scores, pos, 1, got, cand=cand)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy()), f"call {i} differs"
        if nb == 0:
            # the select itself against a host sort of the same scores (NaN as -inf, lower column on ties)
            s = scores[0].cpu().numpy().astype(np.float64)
            nv = int(pos[0]) + 1
            key = np.where(np.isnan(s[:nv]), -np.inf, s[:nv])
            order_ = sorted(range(nv), key=lambda c: (-key[c], c))[:k]
            assert np.array_equal(np.sort(np.array(order_)), got[0, :min(k, nv)].cpu().numpy())


def test_noalloc_refuses_oversized_shapes():
    import sparse_latent_attention_amd as csa2
    scores = torch.zeros(1023, 131072, dtype=torch.float32, device="cuda")
    pos = torch.full((1023,), 131071, dtype=torch.int64, device="cuda")
    out = torch.empty(1023, 512, dtype=torch.int32, device="cuda")
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.topk_select_noalloc(scores, pos, 1, out)
    assert e.value.status == csa2.ERR_WORKSPACE
