"""moe_route_noalloc (the routing call that takes no workspace and uses the library's fixed
per-GPU scratch array) against moe_route on the same inputs: every output bit for bit, on two
calls in a row, the second with a smaller layer, through the C ABI."""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
from workloads import make_inputs

pytestmark = pytest.mark.gpu

OUTS = ("topk_ids", "topk_w", "counts", "offsets", "perm", "inv_perm")


def _routed(inp, noalloc, fill):
    dm = moe.dims(inp.T, inp.d, inp.f, inp.E, inp.k)
    A, dev = max(inp.T * inp.k, 1), "cuda"
    b = {"topk_ids": torch.full((inp.T, inp.k), fill, dtype=torch.int32, device=dev),
         "topk_w": torch.full((inp.T, inp.k), float(fill), dtype=torch.float32, device=dev),
         "counts": torch.full((inp.E,), fill, dtype=torch.int32, device=dev),
         "offsets": torch.full((inp.E + 1,), fill, dtype=torch.int32, device=dev),
         "perm": torch.full((A,), fill, dtype=torch.int32, device=dev),
         "inv_perm": torch.full((A,), fill, dtype=torch.int32, device=dev)}
    logits = torch.from_numpy(inp.logits).to(dev)
    if noalloc:
        moe.moe_route_noalloc(dm, logits, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["perm"],
                              b["inv_perm"])
    else:
        ws = torch.empty((max(moe.moe_workspace_bytes(dm, moe.MOE_WS_ROUTE), 256),), dtype=torch.uint8, device=dev)
        moe.moe_route(dm, logits, b["topk_ids"], b["topk_w"], b["counts"], b["offsets"], b["perm"], b["inv_perm"],
                      ws)
    torch.cuda.synchronize()
    n = int(b["offsets"][-1].item())
    b["perm"] = b["perm"][:n]              # entries past the routed total are unspecified
    return b


def test_noalloc_route_matches_route_on_two_calls():
    # the Qwen3-30B-A3B-shaped routing (T=16384, E=128, top-8: 128 plan segments), then a smaller
    # layer with more experts than tokens per segment (T=1000, E=300, top-6) on the same scratch
    for T, E, k, seed in ((16384, 128, 8, 2), (1000, 300, 6, 40)):
        print(f"[case] noalloc route T={T} E={E} k={k}", flush=True)
        inp = make_inputs(T, 128, 128, E, k, seed=seed, with_dy=False)
        ref = _routed(inp, noalloc=False, fill=-7)
        got = _routed(inp, noalloc=True, fill=-9)
        for name in OUTS:
            a, b = ref[name], got[name]
            assert a.shape == b.shape and torch.equal(a.view(torch.int32), b.view(torch.int32)), name
        assert int(got["counts"].sum().item()) == T * k
