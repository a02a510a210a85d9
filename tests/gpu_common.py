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


def run_forward(inp, layout="packed", act_quant=False, **kw):
    p, x, wr, b, W = to_device(inp, layout=layout, act_quant=act_quant)
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


def oracle_reference(v, L, ids, gids, mism, tokens=None, ref=None, act_quant=False):
    """Oracle outputs with the oracle's own routing, except near-tie tokens where the
    GPU legitimately chose differently: those use the GPU's ids (weights from the
    oracle's logits).  ref: the oracle's outputs of these tokens, if already computed.
    act_quant: the oracle's fp8-activation mode (the library used fp8 activations)."""
    toks = np.arange(v.x.shape[0]) if tokens is None else np.asarray(tokens)
    if ref is not None:
        ref = np.array(ref, np.float64, copy=True)
    elif tokens is None:
        ref, _ = oracle.moe_forward_view(v, act_quant=act_quant)
    else:
        ref, _, _ = oracle.moe_forward_tokens(v, toks, act_quant=act_quant)
    for r_i in np.nonzero(mism)[0]:
        gi = gids[r_i:r_i + 1]
        w = oracle.gate_weights(L[r_i:r_i + 1], gi)
        o, _, _ = oracle.moe_forward_tokens(v, toks[r_i:r_i + 1], ids=gi, weights=w, act_quant=act_quant)
        ref[r_i] = o[0]
    return ref


def requant_alternatives(v, t, ids_row, w_row, margin):
    """The H requantisation decisions of token t that sit within `margin` of a boundary, each
    as the change of the token's output if it went the other way.

    The library computes h = silu(g) * u in float32 (the fp8 matrix cores sum the block
    products in float32) and the oracle in float64, so where h lies within the library's
    rounding of an E4M3 rounding midpoint (a distance of `margin` steps of the value's binade)
    both neighbouring codes are correct results, and likewise both scales where a block's
    largest |h| lies within `margin` (relative) of a power-of-two scale boundary.  Returns a
    list of output-space vectors: the weight of the row times W_down applied to the code (or
    block) change."""
    xq = oracle.fp8_quantize_rows(v.x[t:t + 1])[0]
    rows = [(int(e), float(wj)) for e, wj in zip(ids_row, w_row)] + ([(v.E, 1.0)] if v.has_shared else [])
    alts = []
    for e, wt in rows:
        wg, wu, wd = v.expert(e)
        h = (oracle.silu(xq @ wg.T) * (xq @ wu.T))[0]
        hq, kexp = oracle.fp8_quantize_rows(h[None, :])
        hq, kexp = hq[0], kexp[0]
        sc = np.repeat(np.ldexp(1.0, kexp), 128)
        y = np.abs(h) / sc
        _, ex = np.frexp(y)
        step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
        frac = y / step - np.floor(y / step)
        for i in np.nonzero(np.abs(frac - 0.5) < margin)[0]:
            down = np.floor(y[i] / step[i]) * step[i]
            other = down + step[i] if abs(hq[i]) == down * sc[i] else down
            alts.append(wt * (np.copysign(other * sc[i], h[i]) - hq[i]) * wd[:, i])
        amax = np.abs(h).reshape(-1, 128).max(axis=1)
        for b in range(len(amax)):
            if amax[b] <= 0:
                continue
            for k2 in (kexp[b] + 1, kexp[b] - 1):
                edge = np.ldexp(448.0, max(kexp[b], k2) - 1)
                if abs(amax[b] / edge - 1.0) < margin and np.all(np.abs(h[128 * b:128 * b + 128]) <= np.ldexp(448.0, k2)):
                    blk = h[128 * b:128 * b + 128] / np.ldexp(1.0, k2)
                    alt = oracle.e4m3_round(blk) * np.ldexp(1.0, k2)
                    alts.append(wt * wd[:, 128 * b:128 * b + 128] @ (alt - hq[128 * b:128 * b + 128]))
    return alts


def compare_outputs_requant(got, ref, v, ids, weights, tol, what="", margin=1e-3):
    """compare_outputs for the fp8-activation mode: the whole output within tol, and every
    token within tol of the oracle's output or of one of its equally correct alternatives:
    the oracle's output with some of the token's near-boundary H requantisation decisions
    (requant_alternatives) taken the other way, chosen greedily (each step takes the decision
    whose change brings the oracle closest to the library).  Returns (rel Frobenius, worst
    token error against the oracle's own decisions, tokens that needed an alternative)."""
    err = oracle.rel_frobenius(got, ref)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    per = num / den
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    assert err <= tol, f"{what}: rel Frobenius {err:.3e} > {tol}"
    above = np.nonzero(per > tol)[0]
    for t in above:
        alts = requant_alternatives(v, t, ids[t], weights[t], margin)
        assert alts, f"{what}: token {t} at {per[t]:.3e} with no requantisation decision near a boundary"
        cur, left = ref[t].copy(), list(range(len(alts)))
        best = per[t]
        while left:
            trial = [(float(np.linalg.norm(got[t] - cur - alts[q]) / max(np.linalg.norm(cur + alts[q]), 1e-30)), q)
                     for q in left]
            e_q, q = min(trial)
            if e_q >= best:
                break
            best, cur = e_q, cur + alts[q]
            left.remove(q)
        assert best <= tol, f"{what}: token {t} at {per[t]:.3e}, best alternative {best:.3e} > {tol}"
    return err, float(per.max()), len(above)


def full_parity(inp, tol=None, layout="packed", act_quant=False, **kw):
    """act_quant: run the library's fp8-activation mode; the oracle then quantises as the
    library does when the m-tiles are above 16 rows (the mode's scope), else not."""
    c = inp.cfg
    tol = tol if tol is not None else TOL[c["w"]]
    out, r, ctx = run_forward(inp, layout=layout, act_quant=act_quant, **kw)
    rows = kw.get("m_tile_rows") or moe.plan_describe(ctx["p"])["m_tile_rows"]
    fp8_act = bool(act_quant) and rows > 16
    v = oracle.InputsView(inp)
    L, ids, gids, mism = check_routing(v, r, c["k"], c["E"])
    check_permutation(r, c["k"], c["E"])
    ref = oracle_reference(v, L, ids, gids, mism, act_quant=fp8_act)
    got = out_to_f64(out)
    if fp8_act:
        ids_used = np.where(mism[:, None], gids, ids)
        w_used = oracle.gate_weights(L, ids_used)
        err, worst, n_above = compare_outputs_requant(got, ref, v, ids_used, w_used, tol, c.get("name", ""))
    else:
        err, worst = compare_outputs(got, ref, tol, c.get("name", ""))
    return dict(err=err, worst=worst, near_tie_flips=int(mism.sum()), out=out, r=r, ctx=ctx, v=v, fp8_act=fp8_act,
                routing=(L, ids, gids, mism))
