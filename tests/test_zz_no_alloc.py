"""moe_forward_noalloc (the allocation-free entry point, workspace = the library's fixed
device scratch) against moe_forward with a caller's workspace, through the C ABI.

Two calls in a row on the same scratch, the second with a smaller batch: each must give
exactly moe_forward's output and routing (same kernels, bitwise reproducible results)."""
import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_amd as moe
import synth
from devinputs import out_to_f64, to_device
from gpu_common import TOL, compare_outputs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


CASES = [
    # seed, T, d, n, E, k, act, w, shared, bias  (the second call is the smaller one)
    (41, 48, 1024, 512, 32, 4, "bf16", "bf16", 1, True),
    (42, 9, 1024, 512, 32, 4, "bf16", "bf16", 1, True),
]


def test_noalloc_matches_forward_twice_second_smaller():
    assert moe.workspace_size(moe.problem(48, 1024, 512, 32, 4, 1)) <= moe.NOALLOC_SCRATCH_BYTES
    for seed, T, d, n, E, k, act, w, shared, bias in CASES:
        print(f"[noalloc] seed={seed} T={T} d={d} n={n} E={E} k={k} shared={shared}", flush=True)
        inp = synth.make_tiny(seed, T, d, n, E, k, act=act, w=w, shared=shared, bias=bias)
        p, x, wr, b, W = to_device(inp)
        ws = moe.alloc_workspace(p)
        ref, rr = moe.forward(p, x, wr, b, W, ws, route_out=True)
        got, rg = moe.forward_noalloc(p, x, wr, b, W, route_out=True)
        torch.cuda.synchronize()
        assert moe.last_device_error(ws) == 0
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), "output differs from moe_forward"
        for key in ("topk_ids", "topk_weights", "logits", "counts", "offsets", "perm", "inv_perm"):
            assert torch.equal(rg[key], rr[key]), f"{key} differs from moe_forward"
        v = oracle.InputsView(inp)
        ref64, info = oracle.moe_forward_view(v)
        assert np.array_equal(rg["topk_ids"].cpu().numpy(), info["ids"])
        compare_outputs(out_to_f64(got), ref64, TOL[w], f"noalloc T={T}")


def test_noalloc_refuses_problems_beyond_the_scratch():
    p = moe.problem(4096, 2048, 512, 256, 8, layout="packed")
    assert moe.workspace_size(p) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((4096, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as ei:
        moe.forward_noalloc(p, x, x, None, moe.Weights(), out=torch.empty_like(x))
    assert ei.value.code == 3
