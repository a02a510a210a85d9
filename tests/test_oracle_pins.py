"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each check compares the oracle with brute force on tiny inputs, a closed form,
an invariant, or an independent library routine (torch CPU float64 ops, the
torch fp8/bf16 casts).  The last test plants mistakes into the oracle and
checks that at least one pin catches each of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth


# ----------------------------------------------------------------------------
# brute-force reference written with plain Python loops only
# ----------------------------------------------------------------------------
def bf_logits(x, wr, bias=None):
    T, d = len(x), len(x[0])
    E = len(wr)
    return [[math.fsum(x[t][i] * wr[e][i] for i in range(d)) + (0.0 if bias is None else bias[e])
             for e in range(E)] for t in range(T)]


def bf_topk(Lrow, k):
    """Pairwise-comparison selection: expert a precedes b iff La > Lb or (La == Lb and a < b)."""
    E = len(Lrow)

    def before(a, b):
        return Lrow[a] > Lrow[b] or (Lrow[a] == Lrow[b] and a < b)

    rank = [sum(1 for b in range(E) if b != a and before(b, a)) for a in range(E)]
    out = [None] * E
    for a in range(E):
        out[rank[a]] = a
    return out[:k]


def bf_softmax_kept(vals):
    m = max(vals)
    z = [math.exp(v - m) for v in vals]
    s = math.fsum(z)
    return [q / s for q in z]


def bf_ffn_row(xr, wg, wu, wd):
    n, d = len(wg), len(xr)
    h = []
    for c in range(n):
        g = math.fsum(xr[i] * wg[c][i] for i in range(d))
        u = math.fsum(xr[i] * wu[c][i] for i in range(d))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return [math.fsum(h[c] * wd[o][c] for c in range(n)) for o in range(len(wd))]


def bf_layer(x, wr, bias, k, experts, shared=None):
    """Whole layer with loops: per token, per kept slot, add w * FFN_e(x)."""
    L = bf_logits(x, wr, bias)
    out = []
    for t in range(len(x)):
        ids = bf_topk(L[t], k)
        w = bf_softmax_kept([L[t][e] for e in ids])
        acc = [0.0] * len(x[0])
        for j, e in enumerate(ids):
            y = bf_ffn_row(x[t], *experts[e])
            acc = [a + w[j] * v for a, v in zip(acc, y)]
        if shared is not None:
            y = bf_ffn_row(x[t], *shared)
            acc = [a + v for a, v in zip(acc, y)]
        out.append(acc)
    return out, L


def tolist(a):
    return np.asarray(a, np.float64).tolist()


def rand_problem(seed, T, d, n, E, k, shared=False, bias=False, int_logits=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    if int_logits:  # small integers -> exact ties are common
        x = rng.integers(-2, 3, (T, d)).astype(np.float64)
        wr = rng.integers(-1, 2, (E, d)).astype(np.float64)
    ex = [(rng.standard_normal((n, d)) * 0.5, rng.standard_normal((n, d)) * 0.5,
           rng.standard_normal((d, n)) * 0.5) for _ in range(E)]
    sh = (rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((d, n))) if shared else None
    b = rng.standard_normal(E) if bias else None
    return x, wr, b, ex, sh


def run_oracle(x, wr, b, k, ex, sh):
    return oracle.moe_forward(x, wr, b, k, lambda e: ex[e], len(ex), (lambda: sh) if sh is not None else None)


# ----------------------------------------------------------------------------
# pin checks, as functions returning a list of failure strings (reused by the
# planted-mistake test at the bottom)
# ----------------------------------------------------------------------------
def check_fp8_decode():
    fails = []
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.array_equal(np.isnan(ours), np.isnan(ref)):
        fails.append("fp8 NaN codes differ")
    ok = ~np.isnan(ref)
    if not np.array_equal(ours[ok], ref[ok]):
        fails.append("fp8 decode differs from torch float8_e4m3fn")
    # spec landmarks
    for code, val in [(0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0xB8, -1.0),
                      (0x07, 7 * 2.0 ** -9), (0x3F, 1.875)]:
        if oracle.e4m3_decode(np.array([code], np.uint8))[0] != val:
            fails.append(f"fp8 code {code:#x} != {val}")
    return fails


def check_dequant_blocks():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (256, 384)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10  # no NaN codes
    s = rng.uniform(0.5, 2.0, (2, 3)).astype(np.float32)
    got = oracle.dequant_blocks(q, s)
    dec = oracle.e4m3_decode(q)
    fails = []
    for i in range(0, 256, 37):
        for j in range(0, 384, 41):
            if got[i, j] != dec[i, j] * float(s[i // 128, j // 128]):
                fails.append(f"dequant block index wrong at {i},{j}")
                return fails
    return fails


def check_widen():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000, 0x4049], np.uint16)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fails = []
    if not np.array_equal(oracle.widen(bits, "bf16"), ref):
        fails.append("bf16 widen differs from torch")
    return fails


def check_logits():
    x, wr, b, _, _ = rand_problem(1, 5, 7, 3, 4, 2, bias=True)
    got = oracle.router_logits(x, wr, b)
    ref = np.array(bf_logits(tolist(x), tolist(wr), tolist(b)))
    return [] if np.allclose(got, ref, rtol=1e-12, atol=1e-12) else ["logits differ from fsum dots"]


def check_topk_bruteforce():
    fails = []
    for seed in range(40):
        E = 2 + seed % 7
        k = 1 + seed % E
        x, wr, b, _, _ = rand_problem(seed, 6, 5, 2, E, k, int_logits=(seed % 2 == 0))
        L = oracle.router_logits(x, wr, None)
        ids = oracle.select_topk(L, k)
        for t in range(L.shape[0]):
            if list(ids[t]) != bf_topk(L[t].tolist(), k):
                fails.append(f"topk mismatch seed {seed} token {t}")
                return fails
    return fails


def check_topk_special():
    fails = []
    L = np.zeros((3, 6))
    if not np.array_equal(oracle.select_topk(L, 4), np.tile(np.arange(4), (3, 1))):
        fails.append("all-equal logits must give ids 0..k-1")
    w = oracle.gate_weights(L, oracle.select_topk(L, 4))
    if not np.allclose(w, 0.25, rtol=0, atol=1e-15):
        fails.append("all-equal logits must give w = 1/k")
    # -0.0 ties +0.0 -> lower id first, in both orders
    for row in ([-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]):
        if list(oracle.select_topk(np.array([row]), 2)[0]) != [0, 1]:
            fails.append("-0.0 must tie +0.0")
    # duplicated router rows -> exact ties resolved to the lower id
    rng = np.random.default_rng(7)
    wr = rng.standard_normal((5, 4))
    wr[3] = wr[1]
    x = rng.standard_normal((8, 4))
    ids = oracle.select_topk(oracle.router_logits(x, wr), 5)
    for t in range(8):
        r = list(ids[t])
        if r.index(1) > r.index(3):
            fails.append("duplicated expert rows must order the lower id first")
            break
    # k = E is a full sort by (logit desc, id asc)
    L = rng.standard_normal((4, 7))
    ids = oracle.select_topk(L, 7)
    for t in range(4):
        if list(ids[t]) != sorted(range(7), key=lambda e: (-L[t, e], e)):
            fails.append("k=E must be a full sort")
    return fails


def check_weights():
    fails = []
    rng = np.random.default_rng(11)
    L = rng.standard_normal((10, 6)) * 3
    w1 = oracle.gate_weights(L, oracle.select_topk(L, 1))
    if not np.all(w1 == 1.0):
        fails.append("k=1 weight must be exactly 1")
    ids = oracle.select_topk(L, 2)
    w2 = oracle.gate_weights(L, ids)
    for t in range(10):
        l0, l1 = L[t, ids[t, 0]], L[t, ids[t, 1]]
        if not math.isclose(w2[t, 0], 1.0 / (1.0 + math.exp(l1 - l0)), rel_tol=1e-14):
            fails.append("k=2 weight must be sigmoid(L0-L1)")
            break
    ids = oracle.select_topk(L, 4)
    w4 = oracle.gate_weights(L, ids)
    if not np.allclose(w4.sum(1), 1.0, rtol=0, atol=1e-14):
        fails.append("weights must sum to 1")
    if np.any(np.diff(w4, axis=1) > 0):
        fails.append("weights must be non-increasing over slots")
    for t in range(10):
        ref = bf_softmax_kept([L[t, e] for e in ids[t]])
        if not np.allclose(w4[t], ref, rtol=1e-14, atol=0):
            fails.append("weights differ from brute-force softmax")
            break
    return fails


def check_permute():
    fails = []
    for seed in range(25):
        rng = np.random.default_rng(100 + seed)
        E = 1 + seed % 9
        k = 1 + seed % E
        T = 1 + seed % 13
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        if seed % 5 == 0:  # one hot expert in every token
            ids[:, 0] = 0
            for t in range(T):
                rest = [e for e in rng.permutation(E) if e != 0][: k - 1]
                ids[t, 1:] = rest
        counts, offsets, perm, inv_perm = oracle.permute(ids, E)
        if counts.sum() != T * k or offsets[E] != T * k or np.any(np.diff(offsets) < 0):
            fails.append("counts/offsets invariants")
        if not np.array_equal(inv_perm[perm], np.arange(T * k)):
            fails.append("perm is not a bijection with inv_perm")
        ref = sorted(((int(ids[t, j]), t, j) for t in range(T) for j in range(k)))
        if [t * k + j for (_, t, j) in ref] != perm.tolist():
            fails.append(f"perm differs from sorted (e, t, j), seed {seed}")
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            if np.any(ids.reshape(-1)[seg] != e) or np.any(np.diff(seg // k) <= 0):
                fails.append("segment not one expert / not sorted by token")
        if fails:
            return fails
    return fails


def check_ffn_bruteforce():
    fails = []
    for seed in range(6):
        x, wr, b, ex, sh = rand_problem(seed, 3, 5, 4, 3, 2)
        for e in range(3):
            got = oracle.expert_ffn(x, *ex[e])
            ref = np.array([bf_ffn_row(xr, *map(tolist, ex[e])) for xr in tolist(x)])
            if not np.allclose(got, ref, rtol=1e-12, atol=1e-12):
                fails.append("expert FFN differs from loops")
                return fails
    return fails


def check_layer_bruteforce():
    fails = []
    for seed, (T, d, n, E, k, shared, bias) in enumerate(
            [(4, 6, 5, 4, 2, False, False), (3, 5, 3, 5, 3, True, True), (5, 4, 6, 3, 3, False, True),
             (2, 8, 8, 4, 1, True, False), (4, 4, 4, 6, 4, False, False)]):
        x, wr, b, ex, sh = rand_problem(200 + seed, T, d, n, E, k, shared=shared, bias=bias)
        out, info = run_oracle(x, wr, b, k, ex, sh)
        ref, _ = bf_layer(tolist(x), tolist(wr), None if b is None else tolist(b), k,
                          [tuple(map(tolist, m)) for m in ex], None if sh is None else tuple(map(tolist, sh)))
        if not np.allclose(out, np.array(ref), rtol=1e-11, atol=1e-11):
            fails.append(f"layer differs from brute force (case {seed})")
    return fails


def torch_dense_ffn(x, wg, wu, wd):
    """Dense SwiGLU FFN with torch float64 CPU ops (an independent library path)."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    g = torch.matmul(X, torch.from_numpy(np.ascontiguousarray(wg.T)))
    u = torch.matmul(X, torch.from_numpy(np.ascontiguousarray(wu.T)))
    return torch.matmul(torch.nn.functional.silu(g) * u, torch.from_numpy(np.ascontiguousarray(wd.T))).numpy()


def check_closed_forms():
    fails = []
    rng = np.random.default_rng(5)
    T, d, n, E = 9, 12, 10, 5
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    one = (rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((d, n)))
    dense = torch_dense_ffn(x, *one)
    # k = E with identical experts is the dense FFN (weights sum to 1)
    out, _ = run_oracle(x, wr, None, E, [one] * E, None)
    if not np.allclose(out, dense, rtol=1e-12, atol=1e-12):
        fails.append("k=E identical experts != dense FFN")
    # E = 1, k = 1 is the dense FFN
    out, _ = run_oracle(x, wr[:1], None, 1, [one], None)
    if not np.allclose(out, dense, rtol=1e-12, atol=1e-12):
        fails.append("E=1,k=1 != dense FFN")
    # shared expert alone with identical routed experts adds a second dense FFN
    out, _ = run_oracle(x, wr, None, 2, [one] * E, one)
    if not np.allclose(out, 2 * dense, rtol=1e-12, atol=1e-12):
        fails.append("shared expert must add with weight 1")
    # zero hidden -> zero output
    ex = [(rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((d, n))) for _ in range(E)]
    out, _ = run_oracle(np.zeros((3, d)), wr, None, 2, ex, None)
    if np.any(out != 0):
        fails.append("zero hidden must give zero output")
    # doubling every W_down doubles the output exactly
    o1, _ = run_oracle(x, wr, None, 3, ex, None)
    o2, _ = run_oracle(x, wr, None, 3, [(a, b, 2 * c) for a, b, c in ex], None)
    if not np.array_equal(o2, 2 * o1):
        fails.append("doubling W_down must double the output exactly")
    # relabelling experts (router rows and expert weights together) changes nothing
    pi = rng.permutation(E)
    o3, _ = run_oracle(x, wr[pi], None, 3, [ex[p] for p in pi], None)
    if not np.allclose(o3, o1, rtol=1e-12, atol=1e-12):
        fails.append("expert relabelling changed the output")
    # permuting tokens permutes outputs
    tp = rng.permutation(T)
    o4, _ = run_oracle(x[tp], wr, None, 3, ex, None)
    if not np.allclose(o4, o1[tp], rtol=1e-12, atol=1e-12):
        fails.append("token permutation is not equivariant")
    # silu against torch
    z = np.linspace(-30, 30, 601)
    if not np.allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300):
        fails.append("silu differs from torch")
    return fails


def check_token_subset():
    x, wr, b, ex, sh = rand_problem(9, 7, 6, 5, 4, 2, shared=True, bias=True)
    out, info = run_oracle(x, wr, b, 2, ex, sh)

    class V:
        pass
    v = V()
    v.x, v.w_router, v.bias, v.k, v.E = x, wr, b, 2, 4
    v.expert = lambda e: sh if e == 4 else ex[e]
    v.has_shared = True
    sub, ids, w = oracle.moe_forward_tokens(v, [5, 1])
    if not np.allclose(sub, out[[5, 1]], rtol=1e-12, atol=1e-12):
        return ["token-subset forward differs from the full forward"]
    return []


def check_rel_frobenius():
    """Closed forms of ||got - ref||_F / ||ref||_F: a 3-4-5 triangle, a uniform relative
    scaling, an orthogonal perturbation, a zero output, and a zero reference (whose
    denominator is taken as 1)."""
    fails = []
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])
    cases = [
        (ref, ref, 0.0),
        (ref * 1.25, ref, 0.25),
        (ref + 0.5 * np.array([[0.0, 4.0], [-3.0, 0.0]]), ref, 0.5),   # |perturbation| = 2.5, |ref| = 5
        (np.zeros_like(ref), ref, 1.0),
        (np.array([[0.6, 0.8]]), np.zeros((1, 2)), 1.0),
        (np.array([[1.0, 2.0, 2.0]]), np.array([[1.0, 2.0, 4.0]]), 2.0 / math.sqrt(21.0)),
    ]
    for got, r, want in cases:
        v = oracle.rel_frobenius(got, r)
        if not abs(v - want) <= 1e-15 * max(1.0, want):
            fails.append(f"rel_frobenius {v!r} != {want!r}")
    return fails


# ----------------------------------------------------------------------------
# fp8 activations: E4M3 rounding, block scales, the quantised FFN
# ----------------------------------------------------------------------------
def _e4m3_table():
    """Every finite non-negative E4M3 value with its code, from the decode definition."""
    codes = np.arange(0x7f, dtype=np.uint8)  # 0x00 .. 0x7e (0x7f is NaN)
    return [(float(v), int(c)) for v, c in zip(oracle.e4m3_decode(codes), codes)]


def bf_e4m3_round(v):
    """Nearest E4M3 value by exhaustive search over the code table; a tie goes to the even code."""
    a = abs(v)
    best = None
    for val, code in _e4m3_table():
        key = (abs(val - a), code & 1)
        if best is None or key < best[0]:
            best = (key, val)
    return math.copysign(best[1], v)


def bf_scale_exp(amax):
    """Smallest integer kexp >= -127 with amax <= 448 * 2^kexp, by counting up."""
    kexp = -127
    while amax > 448.0 * 2.0 ** kexp:
        kexp += 1
    return kexp


def bf_quant_row(row, block=128):
    out = []
    for b0 in range(0, len(row), block):
        blk = row[b0:b0 + block]
        kexp = bf_scale_exp(max(abs(q) for q in blk))
        out += [bf_e4m3_round(q / 2.0 ** kexp) * 2.0 ** kexp for q in blk]
    return out


def check_e4m3_round():
    fails = []
    table = _e4m3_table()
    vals = np.array([v for v, _ in table])
    # every E4M3 value rounds to itself, with either sign
    for sgn in (1.0, -1.0):
        if not np.array_equal(oracle.e4m3_round(sgn * vals), sgn * vals):
            fails.append("e4m3_round moves an E4M3 value")
    # ties to the even code (closed forms), saturation-free top end, subnormal ties
    cases = [(1.0625, 1.0), (1.1875, 1.25), (-1.0625, -1.0), (2.0 ** -10, 0.0), (3 * 2.0 ** -10, 2.0 ** -8),
             (432.0, 448.0), (416.0, 416.0), (448.0, 448.0), (0.3, 0.3125), (17.0, 16.0), (19.0, 20.0)]
    for v, want in cases:
        got = float(oracle.e4m3_round(np.array([v]))[0])
        if got != want:
            fails.append(f"e4m3_round({v}) = {got}, want {want}")
    # the torch CPU float8_e4m3fn cast on float32-exact inputs: midpoints between neighbours,
    # quarter steps either side of them, random values over the whole range
    pos = vals
    mids = (pos[:-1] + pos[1:]) / 2
    quart = np.concatenate([mids - (pos[1:] - pos[:-1]) / 4, mids + (pos[1:] - pos[:-1]) / 4])
    rng = np.random.default_rng(11)
    rnd = rng.uniform(-448, 448, 4000) * np.exp2(-rng.integers(0, 14, 4000))
    probe = np.concatenate([mids, -mids, quart, -quart, rnd]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(probe.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.array_equal(oracle.e4m3_round(probe), ref):
        fails.append("e4m3_round differs from the torch float8_e4m3fn cast")
    # brute force on a sample
    for v in probe[::97]:
        if float(oracle.e4m3_round(np.array([v]))[0]) != bf_e4m3_round(float(v)):
            fails.append(f"e4m3_round({v}) differs from exhaustive search")
            break
    return fails


def check_fp8_quantize_rows():
    fails = []
    amax = [448.0, 448.0 * (1 + 2.0 ** -7), 224.0, 224.5, 3.5, 3.5 * (1 + 2.0 ** -7), 1e-3, 0.0, 1e-45, 3e38]
    got = oracle.fp8_block_scale_exponents(np.array(amax))
    want = [bf_scale_exp(a) for a in amax]
    if got.tolist() != want or want[:6] != [0, 1, -1, 0, -7, -6] or want[7] != -127:
        fails.append(f"block scale exponents {got.tolist()} != {want}")
    rng = np.random.default_rng(12)
    # rows with very different block magnitudes, zero blocks, exact E4M3 blocks
    v = rng.standard_normal((3, 512)) * np.array([1.0, 1e-3, 300.0, 1e4])[None, :].repeat(128, 1)
    v[1, 128:256] = 0.0
    v[2, 256:384] = np.array([e for e, _ in _e4m3_table()] + [-448.0]) * 2.0 ** -5
    q, kexp = oracle.fp8_quantize_rows(v)
    ref = np.array([bf_quant_row(r) for r in v.tolist()])
    if not np.array_equal(q, ref):
        fails.append("fp8_quantize_rows differs from the brute-force quantiser")
    if not np.array_equal(q[2, 256:384], v[2, 256:384]):
        fails.append("a block of scaled E4M3 values is not kept exactly")
    # rows and blocks are quantised independently
    if not np.array_equal(oracle.fp8_quantize_rows(v[1:2])[0], q[1:2]):
        fails.append("row quantisation depends on other rows")
    # error bound: half a step of the value's binade, or of the subnormal range
    s = np.repeat(np.ldexp(1.0, kexp), 128, axis=1)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, s * 2.0 ** -10)
    if np.any(np.abs(q - v) > bound * (1 + 1e-12)):
        fails.append("fp8 quantisation error above half a step")
    return fails


def check_act_quant_ffn():
    fails = []
    rng = np.random.default_rng(13)
    d, n = 128, 256
    x = rng.standard_normal((3, d))
    wg, wu = rng.standard_normal((n, d)) / 11, rng.standard_normal((n, d)) / 11
    wd = rng.standard_normal((d, n)) / 16
    got = oracle.expert_ffn(x, wg, wu, wd, act_quant=True)
    Wg, Wu, Wd = tolist(wg), tolist(wu), tolist(wd)
    for t in range(3):
        xq = bf_quant_row(x[t].tolist())
        h = []
        for c in range(n):
            g = math.fsum(xq[i] * Wg[c][i] for i in range(d))
            u = math.fsum(xq[i] * Wu[c][i] for i in range(d))
            h.append(g / (1.0 + math.exp(-g)) * u)
        hq = bf_quant_row(h)
        ref = [math.fsum(hq[c] * Wd[o][c] for c in range(n)) for o in range(d)]
        if not np.allclose(got[t], ref, rtol=1e-11, atol=1e-11):
            fails.append("quantised expert FFN differs from loops")
            break
    plain = oracle.expert_ffn(x, wg, wu, wd)
    rel = np.linalg.norm(got - plain) / np.linalg.norm(plain)
    if not (1e-3 < rel < 6e-2):
        fails.append(f"fp8-activation FFN error {rel:.3g} outside the E4M3 error range")
    return fails


ALL_CHECKS = [check_rel_frobenius, check_fp8_decode, check_dequant_blocks, check_widen, check_logits, check_topk_bruteforce,
              check_topk_special, check_weights, check_permute, check_ffn_bruteforce, check_layer_bruteforce,
              check_closed_forms, check_token_subset, check_e4m3_round, check_fp8_quantize_rows,
              check_act_quant_ffn]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    fails = check()
    assert not fails, fails


# ----------------------------------------------------------------------------
# other properties
# ----------------------------------------------------------------------------
def test_near_tie_detector():
    L = np.array([[3.0, 2.0, 1.0, 0.0], [1.0, 1.0 + 1e-9, 0.0, -1.0], [2.0, 0.0, 0.0 + 1e-9, -5.0]])
    m = oracle.near_tie_tokens(L, 2, 1e-6)
    assert m.tolist() == [False, True, True]


def test_fp8_roundtrip_error_bound():
    """Block quantisation then decode is within half an e4m3 ulp (2^-4 relative)
    of the float32 weights for normal-range codes."""
    w = synth.normal_f32(99, 2, 0, (256, 256), 0.05)
    q, s = synth.fp8_block_quantize(w)
    back = oracle.dequant_blocks(q, s)
    rel = np.abs(back - w) / np.maximum(np.abs(w), 1e-30)
    big = np.abs(w) >= np.repeat(np.repeat(s, 128, 0), 128, 1) * 2.0 ** -6
    assert rel[big].max() <= 2.0 ** -4 + 1e-12
    assert np.abs(back).max() <= np.abs(w).max() * (1 + 1e-7)


def test_generators_deterministic_and_shared():
    a = synth.make_tiny(3, 8, 16, 8, 4, 2, act="bf16", w="bf16")
    b = synth.make_tiny(3, 8, 16, 8, 4, 2, act="bf16", w="bf16")
    assert np.array_equal(a.hidden, b.hidden) and np.array_equal(a.w_gate, b.w_gate)
    dec = synth.config("decode_bf16")
    pre = synth.config("prefill_bf16")
    assert np.array_equal(synth.make_hidden(dec), synth.make_hidden(pre)[:16])
    assert np.array_equal(synth.make_router(dec), synth.make_router(pre))


def test_longer_token_draws_extend_shorter_ones():
    """Workloads draw T_gen rows and take the first T: the rows of a T do not depend on T_gen."""
    a = synth.normal_f32(2, synth.TAG_HIDDEN, 0, (4096, 64), 1.0)
    b = synth.normal_f32(2, synth.TAG_HIDDEN, 0, (32768, 64), 1.0)
    assert np.array_equal(a, b[:4096])
    pre = synth.config("prefill_bf16")
    big = synth.config("prefill_bf16", 32768)
    assert np.array_equal(synth.make_hidden(pre), synth.make_hidden(big)[:4096])


def test_bf16_encoder_matches_torch():
    x = synth.normal_f32(4, 0, 0, (4096,), 3.0)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ----------------------------------------------------------------------------
def _mut_tie_high(L, k):
    L = np.asarray(L, np.float64)
    E = L.shape[1]
    return np.stack([np.lexsort((-np.arange(E), -L[t]))[:k] for t in range(L.shape[0])]).astype(np.int32)


def _mut_softmax_all(L, ids):
    z = np.exp(L - L.max(1, keepdims=True))
    p = z / z.sum(1, keepdims=True)
    return np.take_along_axis(p, ids.astype(np.int64), axis=1)


def _mut_ffn_swap(xr, wg, wu, wd):
    g = xr @ np.asarray(wu).T
    u = xr @ np.asarray(wg).T
    return (g / (1 + np.exp(-g)) * u) @ np.asarray(wd).T


def _mut_ffn_sign(xr, wg, wu, wd):
    g = xr @ np.asarray(wg).T
    u = xr @ np.asarray(wu).T
    return (g / (1 + np.exp(g)) * u) @ np.asarray(wd).T


def _mut_permute_slot_major(ids, E):
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    counts, offsets, _, _ = _orig_permute(ids, E)
    order = sorted(range(T * k), key=lambda q: (ids.reshape(-1)[q], q % k, q // k))
    perm = np.array(order, np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(T * k)
    return counts, offsets, perm, inv


def _mut_decode_bias8(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 7
    sign = np.where(s == 1, -1.0, 1.0)
    return np.where(e == 0, sign * np.ldexp(m / 8.0, -7), sign * np.ldexp(1 + m / 8.0, (e - 8)))


def _mut_dequant_transposed(codes, scales, block=128):
    w = oracle.e4m3_decode(codes)
    R, C = w.shape
    sT = np.asarray(scales, np.float64)
    s = np.repeat(np.repeat(sT, block, axis=0), block, axis=1)
    if sT.shape[0] != sT.shape[1]:
        s = np.repeat(np.repeat(sT.reshape(sT.shape[1], sT.shape[0]), block, axis=0), block, axis=1)
    return w * s


def _mut_combine_no_shared(w, y_slots, y_shared=None):
    return np.einsum("tj,tjd->td", w, y_slots)


def _mut_logits_no_bias(x, w_router, bias=None):
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def _mut_relfrob_squared(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = float((ref * ref).sum())
    return float(((got - ref) ** 2).sum() / (den if den > 0 else 1.0))


def _mut_relfrob_maxabs(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = float(np.abs(ref).max()) if ref.size else 0.0
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def _mut_e4m3_half_up(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    return np.copysign(np.floor(a / step + 0.5) * step, v)


def _mut_e4m3_no_subnormal(v):
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    step = np.ldexp(1.0, ex - 1 - 3)
    return np.copysign(np.rint(a / step) * step, v)


def _mut_scale_exp_floor(amax):
    amax = np.asarray(amax, np.float64)
    pos = amax > 0
    k = np.floor(np.log2(np.where(pos, amax, 1.0) / 448.0))
    return np.maximum(np.where(pos, k, -127), -127).astype(np.int64)


def _mut_ffn_h_not_quantised(xr, wg, wu, wd, act_quant=False):
    xr = np.asarray(xr, np.float64)
    if act_quant:
        xr = oracle.moe.fp8_quantize_rows(xr)[0]
    g = xr @ np.asarray(wg).T
    u = xr @ np.asarray(wu).T
    return (g / (1 + np.exp(-g)) * u) @ np.asarray(wd).T


_orig_permute = oracle.moe.permute

MUTATIONS = {
    "tie_to_higher_id": ("select_topk", _mut_tie_high),
    "softmax_over_all_experts": ("gate_weights", _mut_softmax_all),
    "gate_up_swapped": ("expert_ffn", _mut_ffn_swap),
    "silu_sign": ("expert_ffn", _mut_ffn_sign),
    "perm_slot_major": ("permute", _mut_permute_slot_major),
    "fp8_bias_8": ("e4m3_decode", _mut_decode_bias8),
    "scales_transposed": ("dequant_blocks", _mut_dequant_transposed),
    "shared_dropped": ("combine", _mut_combine_no_shared),
    "bias_dropped": ("router_logits", _mut_logits_no_bias),
    "rel_frobenius_squared": ("rel_frobenius", _mut_relfrob_squared),
    "rel_frobenius_max_abs": ("rel_frobenius", _mut_relfrob_maxabs),
    "e4m3_ties_away": ("e4m3_round", _mut_e4m3_half_up),
    "e4m3_no_subnormals": ("e4m3_round", _mut_e4m3_no_subnormal),
    "fp8_scale_floor": ("fp8_block_scale_exponents", _mut_scale_exp_floor),
    "fp8_h_not_requantised": ("expert_ffn", _mut_ffn_h_not_quantised),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oracle.moe, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for check in ALL_CHECKS:
        try:
            if check():
                caught.append(check.__name__)
        except Exception as ex:  # a crash also counts as caught
            caught.append(f"{check.__name__}:{type(ex).__name__}")
    assert caught, f"planted mistake {name} passed every pin"


def test_zipf_bias_fixture_reproduces():
    """The stored skewed-load bias gives, under the oracle's routing of the
    seeded tokens, the stored Zipf-like counts (hot expert near T, cold ones ~20)."""
    import json
    cfg = synth.config("skewed_bf16")
    with open(synth.ZIPF_BIAS_FILE) as f:
        rec = json.load(f)
    x = oracle.widen(synth.make_hidden(cfg), cfg["act"])
    wr = oracle.widen(synth.make_router(cfg), cfg["act"])
    b = synth.load_zipf_bias(cfg).astype(np.float64)
    ids = oracle.select_topk(oracle.router_logits(x, wr, b), cfg["k"])
    cnt = np.bincount(ids.reshape(-1), minlength=cfg["E"])
    by_rank = cnt[synth.zipf_rank_permutation(cfg)]
    assert by_rank.tolist() == rec["achieved_counts_by_rank"]
    assert 1.0 <= rec["fitted_exponent"] <= 1.2
    assert by_rank[0] > 0.9 * cfg["T"] and by_rank.min() >= 1


def test_prefetched_expert_views_give_the_same_forward():
    """The parity tests of the large fp8 workload feed the oracle's forward an expert view
    that decodes upcoming experts on worker threads; its result must be exactly the plain
    view's."""
    from gpu_common import ExpertPrefetch
    inp = synth.make_tiny(5, 37, 256, 256, 9, 3, act="bf16", w="fp8", shared=1, bias=True)
    v = oracle.InputsView(inp)
    ref, info = oracle.moe_forward_view(v)
    pf = ExpertPrefetch(v, threads=3, lookahead=4)
    out, info2 = oracle.moe_forward(v.x, v.w_router, v.bias, v.k, pf, v.E, lambda: pf(v.E))
    assert np.array_equal(out, ref)
    assert np.array_equal(info["perm"], info2["perm"])
    assert pf.decoded == int((info["counts"] > 0).sum()) + 1
