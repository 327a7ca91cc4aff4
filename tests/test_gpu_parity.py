"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle, element by element,
on seeded inputs small enough for the full oracle but spanning several tiles and ragged tails,
plus the edge cases of a dropless layer.  Routing ids and the plan must be bit-exact."""
import numpy as np
import pytest
import torch

import grouped_gemm_expert_router_amd as moe
import oracle
from workloads import make_config, make_inputs
from moe_testlib import GpuLayer, check_full_parity, oracle_full, to_np, bf16_dev

pytestmark = pytest.mark.gpu


def _inputs(T, d, f, E, k, seed, bias=None):
    return make_inputs(T, d, f, E, k, seed=seed, logits_bias=bias)


def test_tiny_config_forward():
    inp = make_config("tiny")
    print(f"[case] tiny T={inp.T} d={inp.d} f={inp.f} E={inp.E} k={inp.k}", flush=True)
    gl = GpuLayer(inp, backward=False).run(backward=False)
    check_full_parity(gl, oracle_full(inp), backward=False)


CASES = {
    # name: (T, d, f, E, k, seed)
    "tiny_fwd_bwd": (64, 128, 256, 8, 2, 0),
    "ragged_tails": (77, 256, 384, 6, 3, 5),
    "top1": (50, 128, 128, 4, 1, 6),
    "k_equals_E": (40, 128, 128, 8, 8, 7),
    "single_expert": (33, 128, 256, 1, 1, 8),
    "one_token": (1, 128, 128, 4, 2, 11),
    "multi_tile": (300, 256, 256, 4, 2, 12),
    "wide": (200, 512, 384, 8, 4, 13),
    # limits of the ABI: the most experts (most of them empty) and the largest k (= E)
    "max_experts": (96, 128, 128, 1024, 4, 14),
    "max_k": (24, 128, 128, 64, 64, 15),
    # more 256x256 output tiles than compute units in each ragged-M product (288 each), with
    # ragged row tails in every expert
    "tiles_beyond_one_per_cu": (4000, 768, 384, 8, 6, 16),
    # router shapes: 16 lanes per token with k = 16 (every lane keeps a slot), and a row of 100
    # logits that leaves some lanes partly or wholly without experts
    "router_k16_E128": (100, 128, 128, 128, 16, 17),
    "router_E100": (70, 128, 128, 100, 5, 18),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    T, d, f, E, k, seed = CASES[name]
    print(f"[case] {name} T={T} d={d} f={f} E={E} k={k} seed={seed}", flush=True)
    inp = _inputs(T, d, f, E, k, seed)
    gl = GpuLayer(inp).run()
    check_full_parity(gl, oracle_full(inp))


def test_all_tokens_to_one_expert():
    E = 8
    bias = np.zeros(E, np.float32)
    bias[5] = 10.0              # top-1 is expert 5 for every token; the second slot stays
    inp = _inputs(96, 128, 256, E, 2, 20, bias)   # routed, with weights ~e^-10 (bf16-representable)
    print("[case] one hot expert", flush=True)
    gl = GpuLayer(inp).run()
    errs = check_full_parity(gl, oracle_full(inp))
    assert "dW1[5]" in errs


def test_empty_experts_get_zero_weight_gradients():
    E = 16
    bias = np.zeros(E, np.float32)
    bias[::2] = -100.0          # even experts never selected
    inp = _inputs(90, 128, 256, E, 2, 21, bias)
    print("[case] empty experts", flush=True)
    gl = GpuLayer(inp)
    gl.b["dW1"].fill_(7.0)
    gl.b["dW2"].fill_(7.0)
    gl.run()
    ref = oracle_full(inp)
    assert np.all(ref["plan"].counts[::2] == 0)
    check_full_parity(gl, ref)


@pytest.mark.parametrize("E,k", [(32, 4), (128, 8)])
def test_tie_heavy_routing_is_bitexact(E, k):
    inp = _inputs(257, 128, 128, E, k, 22)
    g = np.random.default_rng(0)
    L = g.integers(-2, 3, size=(inp.T, inp.E)).astype(np.float32)
    L[g.random(L.shape) < 0.2] = -0.0
    inp.logits = L
    print(f"[case] tie-heavy routing E={E} k={k}", flush=True)
    gl = GpuLayer(inp).run()
    check_full_parity(gl, oracle_full(inp))


def test_prerouted_plan_with_sentinels():
    inp = _inputs(120, 128, 256, 8, 3, 23)
    g = np.random.default_rng(1)
    ids, w = oracle.route(inp.logits, inp.k)
    ids = ids.copy()
    ids[g.random(ids.shape) < 0.3] = -1          # slots owned by another rank
    inp.topk_ids = ids.astype(np.int32)
    inp.topk_w = w.astype(np.float32)
    inp.logits = None
    print("[case] pre-routed with -1 sentinels", flush=True)
    gl = GpuLayer(inp).run()
    ref = oracle_full(inp)
    check_full_parity(gl, ref)
    assert np.all(to_np(gl.b["d_topk_w"])[ids < 0] == 0)


def test_zero_tokens():
    inp = _inputs(0, 128, 256, 4, 2, 24)
    print("[case] T=0", flush=True)
    gl = GpuLayer(inp)
    gl.b["dW1"].fill_(3.0)
    gl.b["dW2"].fill_(3.0)
    gl.run()
    assert torch.all(gl.b["offsets"] == 0)
    assert torch.all(gl.b["dW1"] == 0) and torch.all(gl.b["dW2"] == 0)


def test_bitwise_run_to_run_determinism():
    inp = _inputs(300, 256, 256, 8, 4, 25)
    print("[case] determinism", flush=True)
    gl = GpuLayer(inp).run()
    first = {k: v.clone() for k, v in gl.b.items() if k not in ("ws_route", "ws_fwd", "ws_bwd")}
    gl.run()
    for k, v in first.items():
        assert torch.equal(v.view(torch.uint8) if v.dtype != torch.uint8 else v,
                           gl.b[k].view(torch.uint8) if gl.b[k].dtype != torch.uint8 else gl.b[k]), k


@pytest.mark.parametrize("k", [2, 8])
def test_permute_then_combine_is_k_times_x_bitexact(k):
    """combine(permute(x)) with unit weights adds k equal bf16 rows: exact when k is 2 or 8."""
    inp = _inputs(130, 256, 128, 16, k, 26)
    print(f"[case] permute/combine k={k}", flush=True)
    gl = GpuLayer(inp, backward=False)
    gl.route()
    b = gl.b
    A = inp.T * k
    xp = torch.empty((A, inp.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_permute(gl.dm, gl.x, b["inv_perm"], xp)
    slot_rows = xp[b["inv_perm"].long()]                 # back to pair order for the combine
    y = torch.empty((inp.T, inp.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(gl.dm, slot_rows.contiguous(), b["inv_perm"], y)
    torch.cuda.synchronize()
    expect = (gl.x.float() * k).to(torch.bfloat16)
    assert torch.equal(y.view(torch.int16), expect.view(torch.int16))
    # the gather itself: sorted row pos holds token perm[pos] // k
    perm = b["perm"][:A].long()
    assert torch.equal(xp.view(torch.int16), gl.x[perm // k].view(torch.int16))


@pytest.mark.parametrize("T,k", [(2600, 2), (5000, 1)])
def test_weight_gradient_split_over_heavy_expert(T, k):
    """One expert receives more rows than one weight-gradient chunk (2048): its dW is summed
    from fp32 chunk partials in chunk order (two and three chunks here)."""
    E = 4
    bias = np.zeros(E, np.float32)
    bias[1] = 10.0
    inp = _inputs(T, 128, 128, E, k, 27, bias)
    print(f"[case] split-K heavy expert T={T} k={k}", flush=True)
    gl = GpuLayer(inp).run()
    ref = oracle_full(inp)
    assert ref["plan"].counts[1] > 2048
    check_full_parity(gl, ref)
