"""Shared helpers of the GPU parity tests: run the library, run the oracle, compare."""
import os

import numpy as np
import pytest
import torch

import oracle
import routed_grouped_gemm_amd as moe
from devinputs import out_to_f64, to_device

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 5e-2}   # relative Frobenius bound per weight dtype


class ExpertPrefetch:
    """expert(e) for the oracle's forward, which asks for experts in increasing id order (then
    the shared expert, id E): the float64 views of the next `lookahead` experts are decoded on
    worker threads while the caller multiplies with the current one.  Only the order of work
    changes; every value is the InputsView's own."""

    def __init__(self, v, threads=16, lookahead=24):
        from concurrent.futures import ThreadPoolExecutor
        self.v = v
        self.pool = ThreadPoolExecutor(max(1, threads))
        self.lookahead = lookahead
        self.pending = {}
        self.next_id = 0
        self.decoded = 0

    def _submit_upto(self, last):
        while self.next_id <= min(last, self.v.E):
            self.pending[self.next_id] = self.pool.submit(self.v.expert, self.next_id)
            self.next_id += 1

    def __call__(self, e):
        self._submit_upto(e + self.lookahead)
        fut = self.pending.pop(e, None)
        for old in [q for q in self.pending if q < e]:  # experts the caller skipped (no rows)
            self.pending.pop(old).cancel()
        self.decoded += 1
        return fut.result() if fut is not None else self.v.expert(e)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(moe.LIB_PATH):
        from routed_grouped_gemm_amd import build
        build.build()


def run_forward(inp, layout="packed", **kw):
    p, x, wr, b, W = to_device(inp, layout=layout)
    # a forced m-tile may need a few KB more of m-tile descriptors than the table's tile
    ws = moe.alloc_workspace(p, extra=(4 << 20) if kw.get("m_tile_rows") else 0)
    out, r = moe.forward(p, x, wr, b, W, ws, route_out=True, **kw)
    torch.cuda.synchronize()
    assert moe.last_device_error(ws) == 0, "device-side fault flag set"
    return out, r, dict(p=p, x=x, wr=wr, b=b, W=W, ws=ws)


def check_routing(v, r, k, E, tokens=None):
    """Stage-wise exactness on the GPU's own logits, then the end-to-end near-tie rule.
    Returns (oracle logits, oracle ids, gpu ids, near-tie-mismatch mask)."""
    gL = r["logits"].cpu().numpy().astype(np.float64)
    gids = r["topk_ids"].cpu().numpy()
    gw = r["topk_weights"].cpu().numpy().astype(np.float64)
    if tokens is not None:
        gL, gids, gw = gL[tokens], gids[tokens], gw[tokens]
    # (i) the oracle's selection applied to the GPU's logits is bit-exact
    assert np.array_equal(oracle.select_topk(gL, k), gids)
    # weights: softmax of the GPU's kept logits, float32 arithmetic -> 1e-6 relative
    ref_w = oracle.gate_weights(gL, gids)
    assert np.allclose(gw, ref_w, rtol=1e-6, atol=1e-7)
    # (ii) end to end against the oracle's float64 logits
    x = v.x if tokens is None else v.x[tokens]
    L = oracle.router_logits(x, v.w_router, v.bias)
    delta = float(np.abs(gL - L).max())
    assert delta < 1e-3 * max(1.0, float(np.abs(L).max()))
    ids = oracle.select_topk(L, k)
    mism = np.any(ids != gids, axis=1)
    near = oracle.near_tie_tokens(L, k, delta)
    assert not np.any(mism & ~near), f"routing differs on {int((mism & ~near).sum())} non-tie tokens"
    return L, ids, gids, mism


def check_permutation(r, k, E):
    gids = r["topk_ids"].cpu().numpy()
    counts, offsets, perm, inv = oracle.permute(gids, E)
    assert np.array_equal(r["counts"].cpu().numpy(), counts)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(r["perm"].cpu().numpy(), perm)
    assert np.array_equal(r["inv_perm"].cpu().numpy(), inv)


def compare_outputs(got, ref, tol, what=""):
    """Whole-output relative Frobenius error <= tol, and the same bound per token."""
    err = oracle.rel_frobenius(got, ref)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    worst = float((num / den).max())
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    assert err <= tol, f"{what}: rel Frobenius {err:.3e} > {tol}"
    assert worst <= tol, f"{what}: worst per-token rel error {worst:.3e} > {tol}"
    return err, worst


def oracle_reference(v, L, ids, gids, mism, tokens=None, ref=None):
    """Oracle outputs with the oracle's own routing, except near-tie tokens where the
    GPU legitimately chose differently: those use the GPU's ids (weights from the
    oracle's logits).  ref: the oracle's outputs of these tokens, if already computed."""
    toks = np.arange(v.x.shape[0]) if tokens is None else np.asarray(tokens)
    if ref is not None:
        ref = np.array(ref, np.float64, copy=True)
    elif tokens is None:
        ref, _ = oracle.moe_forward_view(v)
    else:
        ref, _, _ = oracle.moe_forward_tokens(v, toks)
    for r_i in np.nonzero(mism)[0]:
        gi = gids[r_i:r_i + 1]
        w = oracle.gate_weights(L[r_i:r_i + 1], gi)
        o, _, _ = oracle.moe_forward_tokens(v, toks[r_i:r_i + 1], ids=gi, weights=w)
        ref[r_i] = o[0]
    return ref


def full_parity(inp, tol=None, layout="packed", **kw):
    c = inp.cfg
    tol = tol if tol is not None else TOL[c["w"]]
    out, r, ctx = run_forward(inp, layout=layout, **kw)
    v = oracle.InputsView(inp)
    L, ids, gids, mism = check_routing(v, r, c["k"], c["E"])
    check_permutation(r, c["k"], c["E"])
    ref = oracle_reference(v, L, ids, gids, mism)
    got = out_to_f64(out)
    err, worst = compare_outputs(got, ref, tol, c.get("name", ""))
    return dict(err=err, worst=worst, near_tie_flips=int(mism.sum()), out=out, r=r, ctx=ctx)
