"""GPU parity at the full size of the large fp8 workload: d=7168, 256 routed experts
(top-8) plus one shared expert, n=2048, e4m3 weights with 128x128 block scales,
bf16 activations, T in {1, 8, 64, 512, 4096}.  Every T uses the same weights and
the first T of the same 4096 token rows.

Routing and permutation are checked exactly on every token, and the output of every
token is compared with the oracle's.  The oracle runs once, over all 4096 rows,
expert by expert (each expert's float64 weights decoded once, on worker threads, while
the previous expert multiplies): a token's output depends on no other token, so the
outputs for each T are the first T rows of that run.  Each T reports the m-tile size the
tile table gives it."""
import gc
import os

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_amd as moe
import synth
from devinputs import out_to_f64, to_device
from gpu_common import (TOL, ExpertPrefetch, check_permutation, check_routing, compare_outputs,
                        compare_outputs_requant, oracle_reference, require_gpu)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


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


@pytest.fixture(scope="module")
def oracle_all_rows(large):
    inp = large[0]
    print("[large fp8] oracle over all 4096 rows, expert by expert", flush=True)
    v = oracle.InputsView(inp)
    pf = ExpertPrefetch(v, threads=min(16, len(os.sched_getaffinity(0))), lookahead=24)
    out, info = oracle.moe_forward(v.x, v.w_router, v.bias, v.k, pf, v.E, lambda: pf(v.E))
    pf.pool.shutdown()
    print("[large fp8] oracle done", flush=True)
    return out, info


@pytest.fixture(scope="module")
def oracle_all_rows_aq(large):
    """The oracle in the fp8-activation mode (hidden rows and H quantised), all 4096 rows."""
    inp = large[0]
    print("[large fp8] oracle with fp8 activations over all 4096 rows", flush=True)
    v = oracle.InputsView(inp)
    pf = ExpertPrefetch(v, threads=min(16, len(os.sched_getaffinity(0))), lookahead=24)
    out, info = oracle.moe_forward(v.x, v.w_router, v.bias, v.k, pf, v.E, lambda: pf(v.E), act_quant=True)
    pf.pool.shutdown()
    print("[large fp8] oracle done", flush=True)
    return out, info


@pytest.mark.parametrize("T", synth.LARGE_FP8_T)
def test_large_fp8_forward(large, oracle_all_rows, T):
    inp_full, x_full, wr, b, W = large
    ref_all, info_all = oracle_all_rows
    print(f"[large fp8] T={T}", flush=True)
    cfg = synth.config("large_fp8", T)
    inp = synth.MoEInputs(cfg=cfg, hidden=inp_full.hidden[:T], w_router=inp_full.w_router, bias=None,
                          w_gate=inp_full.w_gate, w_up=inp_full.w_up, w_down=inp_full.w_down,
                          s_gate=inp_full.s_gate, s_up=inp_full.s_up, s_down=inp_full.s_down,
                          sh_gate=inp_full.sh_gate, sh_up=inp_full.sh_up, sh_down=inp_full.sh_down,
                          sh_s_gate=inp_full.sh_s_gate, sh_s_up=inp_full.sh_s_up, sh_s_down=inp_full.sh_s_down)
    p = moe.problem(T, cfg["d"], cfg["n"], cfg["E"], cfg["k"], 1, "bf16", "fp8", layout="packed")
    rows = moe.plan_describe(p)["m_tile_rows"]
    assert rows in (16, 32, 64, 128, 160)  # (the tuned table's choice)
    x = x_full[:T].contiguous()
    ws = moe.alloc_workspace(p)
    out, r = moe.forward(p, x, wr, b, W, ws, route_out=True)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0
    v = oracle.InputsView(inp)
    L, ids, gids, mism = check_routing(v, r, cfg["k"], cfg["E"])
    assert np.array_equal(ids, info_all["ids"][:T])
    check_permutation(r, cfg["k"], cfg["E"])
    ref = oracle_reference(v, L, ids, gids, mism, ref=ref_all[:T])
    got = out_to_f64(out)
    err, worst = compare_outputs(got, ref, TOL["fp8"], f"large_fp8 T={T}")
    print(f"  all {T} tokens ({rows}-row m-tiles): rel_frob={err:.3e} worst_token={worst:.3e} "
          f"near_tie_flips={int(mism.sum())}",
          flush=True)
    del ws, out, r


# The fp8-activation mode at the T whose m-tiles are above 16 rows (where it applies); every
# token compared with the oracle in the same mode (bound 1e-2: both sides quantise alike, see
# the parity tests) and the whole output with the unquantised oracle (6e-2: the E4M3 rounding
# of both GEMM inputs).
@pytest.mark.parametrize("T", [t for t in synth.LARGE_FP8_T if t >= 512])
def test_large_fp8_forward_fp8_activations(large, oracle_all_rows, oracle_all_rows_aq, T):
    inp_full, x_full, wr, b, W = large
    print(f"[large fp8, fp8 activations] T={T}", flush=True)
    cfg = synth.config("large_fp8", T)
    inp = synth.MoEInputs(cfg=cfg, hidden=inp_full.hidden[:T], w_router=inp_full.w_router, bias=None,
                          w_gate=inp_full.w_gate, w_up=inp_full.w_up, w_down=inp_full.w_down,
                          s_gate=inp_full.s_gate, s_up=inp_full.s_up, s_down=inp_full.s_down,
                          sh_gate=inp_full.sh_gate, sh_up=inp_full.sh_up, sh_down=inp_full.sh_down,
                          sh_s_gate=inp_full.sh_s_gate, sh_s_up=inp_full.sh_s_up, sh_s_down=inp_full.sh_s_down)
    p = moe.problem(T, cfg["d"], cfg["n"], cfg["E"], cfg["k"], 1, "bf16", "fp8", layout="packed", act_quant=True)
    plan = moe.plan_describe(p)
    assert plan["fp8_activations"] == 1 and plan["m_tile_rows"] > 16
    x = x_full[:T].contiguous()
    ws = moe.alloc_workspace(p)
    out, r = moe.forward(p, x, wr, b, W, ws, route_out=True)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0
    v = oracle.InputsView(inp)
    L, ids, gids, mism = check_routing(v, r, cfg["k"], cfg["E"])
    check_permutation(r, cfg["k"], cfg["E"])
    got = out_to_f64(out)
    ref = oracle_reference(v, L, ids, gids, mism, ref=oracle_all_rows_aq[0][:T], act_quant=True)
    ids_used = np.where(mism[:, None], gids, ids)
    w_used = oracle.gate_weights(L, ids_used)
    err, worst, n_above = compare_outputs_requant(got, ref, v, ids_used, w_used, 1e-2,
                                                  f"large_fp8 T={T} fp8 activations")
    ref_plain = oracle_reference(v, L, ids, gids, mism, ref=oracle_all_rows[0][:T])
    err_p = oracle.rel_frobenius(got, ref_plain)
    assert err_p <= 6e-2, f"large_fp8 T={T} vs unquantised oracle: rel Frobenius {err_p:.3e}"
    print(f"  all {T} tokens ({plan['m_tile_rows']}-row m-tiles): rel_frob={err:.3e} worst_token={worst:.3e} "
          f"({n_above} above 1e-2, each matched by an alternative requantisation); vs unquantised oracle {err_p:.3e}",
          flush=True)
    del ws, out, r
