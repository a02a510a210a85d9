"""GPU parity at the full size of the large fp8 workload: d=7168, 256 routed experts
(top-8) plus one shared expert, n=2048, e4m3 weights with 128x128 block scales,
bf16 activations, T in {1, 8, 64, 512, 4096}.  Every T uses the same weights and
the first T of the same 4096 token rows.

Routing and permutation are checked exactly on every token; outputs are checked
on sampled tokens, which the oracle computes one by one (the whole layer at
T=4096 is about 3 TFLOP of float64 work)."""
import gc

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_amd as moe
import synth
from devinputs import out_to_f64, to_device
from gpu_common import TOL, check_permutation, check_routing, compare_outputs, oracle_reference, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def large():
    require_gpu()
    print("[large fp8] drawing 257 experts of e4m3 weights", flush=True)
    inp = synth.make_inputs(synth.config("large_fp8"))
    p, x, wr, b, W = to_device(inp)
    yield inp, x, wr, b, W
    del W
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", synth.LARGE_FP8_T)
def test_large_fp8_forward(large, T):
    inp_full, x_full, wr, b, W = large
    print(f"[large fp8] T={T}", flush=True)
    cfg = synth.config("large_fp8", T)
    inp = synth.MoEInputs(cfg=cfg, hidden=inp_full.hidden[:T], w_router=inp_full.w_router, bias=None,
                          w_gate=inp_full.w_gate, w_up=inp_full.w_up, w_down=inp_full.w_down,
                          s_gate=inp_full.s_gate, s_up=inp_full.s_up, s_down=inp_full.s_down,
                          sh_gate=inp_full.sh_gate, sh_up=inp_full.sh_up, sh_down=inp_full.sh_down,
                          sh_s_gate=inp_full.sh_s_gate, sh_s_up=inp_full.sh_s_up, sh_s_down=inp_full.sh_s_down)
    p = moe.problem(T, cfg["d"], cfg["n"], cfg["E"], cfg["k"], 1, "bf16", "fp8", layout="packed")
    x = x_full[:T].contiguous()
    ws = moe.alloc_workspace(p)
    out, r = moe.forward(p, x, wr, b, W, ws, route_out=True)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0
    v = oracle.InputsView(inp)
    L, ids, gids, mism = check_routing(v, r, cfg["k"], cfg["E"])
    check_permutation(r, cfg["k"], cfg["E"])
    rng = np.random.default_rng(T)
    toks = np.arange(T) if T == 1 else np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 2)]))
    ref = oracle_reference(v, L[toks], ids[toks], gids[toks], mism[toks], tokens=toks)
    got = out_to_f64(out)[toks]
    err, worst = compare_outputs(got, ref, TOL["fp8"], f"large_fp8 T={T}")
    print(f"  tokens={toks.tolist()} rel_frob={err:.3e} worst_token={worst:.3e}", flush=True)
    del ws, out, r
