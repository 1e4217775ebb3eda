"""moe_dispatch_noalloc (static library scratch, no workspace) against
moe_dispatch (caller workspace): bitwise the same outputs, on two calls in a
row on one device, the second with a smaller input (the shared scratch keeps
the first call's contents)."""
import numpy as np
import pytest
import torch

from top_routing_expert_route_amd import api
from top_routing_expert_route_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"
KEYS = ("seg_offsets", "kept_count", "slot_row", "n_dropped")


def _same(a, b, rows):
    for k in KEYS:
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["row_src"][:rows], b["row_src"][:rows])
    if a["x_perm"] is not None:
        assert torch.equal(a["x_perm"][:rows].view(torch.int16), b["x_perm"][:rows].view(torch.int16))


def _case(T, E, k, d, cf, e0, nle, seed):
    g = np.random.default_rng(seed)
    idx = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(g.standard_normal((T, d), dtype=np.float32)).to(torch.bfloat16).to(DEV)
    return x, torch.from_numpy(idx).to(DEV)


# (T, E, k, d, capacity_factor, expert_begin, num_local_experts): a large
# planner case (chunk counts in the scratch) followed by a smaller one, and a
# small single-block planner case followed by a smaller capped one
SEQUENCES = [
    [(20000, 64, 4, 256, 1.25, 0, 0), (3000, 64, 4, 256, 0.0, 8, 16)],
    [(4096, 8, 2, 512, 0.0, 0, 0), (700, 8, 2, 512, 1.0, 0, 0)],
    [(40000, 256, 8, 64, 0.0, 0, 32), (9000, 128, 2, 64, 2.0, 64, 64)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_dispatch_matches_workspace_dispatch(seq):
    assert api.lib().moe_dispatch_noalloc_scratch_bytes() == 64 * 1024
    for i, (T, E, k, d, cf, e0, nle) in enumerate(SEQUENCES[seq]):
        print("noalloc case", seq, i, (T, E, k, d, cf, e0, nle), flush=True)
        x, idx = _case(T, E, k, d, cf, e0, nle, seed=100 * seq + i)
        ref = api.moe_dispatch(x, idx, E, cf, e0, nle)
        got = api.moe_dispatch(x, idx, E, cf, e0, nle, noalloc=True)
        torch.cuda.synchronize()
        rows = int(ref["seg_offsets"][-1].item())
        assert rows > 0
        _same(got, ref, rows)
