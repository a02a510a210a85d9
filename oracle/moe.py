"""float64 CPU oracle of one MoE layer's forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests/, the entry module's smoke() and the benchmark's cpu_baseline leg may
import this file.  It is slow on purpose: every step is the plain definition,
with numpy's matmul, sort and exp as the only library steps.

Pages cited (by title; short names used below):
  [vLLM-config]  "MoE 的隐藏加速开关：那些按显卡命名的 config 到底是什么"
                 (syt-nju.github.io, visual reading of the vLLM fused-MoE configs)
  [Weave]        "Weave：MoE大内核细粒度动态SM调度，4×H100实现2.89×层加速"
  [Fusion]       "MoE推理优化：内核融合与分步执行方案对比"
  [FlashMoE]     the FlashMoE principles explainer (71396.com)
  [GC-MoE]       "GC-MoE：用CUDA Green Contexts解耦MoE通信与计算"

What the layer computes ([vLLM-config] section 02, the four-box diagram and the
text around it; [FlashMoE] section 二.1; [Fusion] section 二, scheme B):
  1. a router scores every expert for every token and keeps the top k;
  2. tokens are grouped (permuted) by the expert they go to;
  3. every chosen expert is a small FFN: gate and up projections, SwiGLU, down
     projection;
  4. the k expert outputs of a token are summed, weighted by the gate weights.

Readings where the pages leave a step open (each is listed with its reason in
the design notes of the repository):
  * softmax over the k kept logits (equal in exact arithmetic to a full softmax
    renormalised over the kept experts); selection is on logits, not on
    probabilities;
  * order experts by logit descending, exact ties (IEEE equality, so -0.0 ties
    +0.0) to the lower expert id; slot j = 0..k-1 is that order;
  * the router bias, when present, is added to the logits and so affects both
    selection and weights;
  * SwiGLU is silu(x Wg^T) * (x Wu^T), then times Wd^T, with no biases;
  * the shared expert has weight 1 and is added after the k routed slots;
  * fp8 weights are OCP E4M3 codes times one float32 scale per 128x128 block;
  * the permutation is the stable order of (expert, token, slot);
  * in the fp8-activation mode, a GEMM's activations are E4M3 codes times one
    power-of-two scale per token and 128-element K block, the smallest such
    scale that fits the block, codes rounded to nearest even (fp8_quantize_rows).

Layouts follow the synthetic-input module: w_router [E,d], w_gate/w_up [E,n,d],
w_down [E,d,n] (each row is one output channel).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# storage -> exact float64 values
# ----------------------------------------------------------------------------
def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of an f32 array or of bf16 bit patterns (uint16)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn" variant) -> float64.

    [vLLM-config] section 03 names fp8_w8a8 weights with block_shape [128,128];
    the code format is the OCP E4M3 definition: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits, no infinities, and S.1111.111 is NaN.
    Normal:    (-1)^s * 2^(e-7) * (1 + m/8)
    Subnormal: (-1)^s * 2^(-6) * (m/8)          (e == 0)
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    out = np.where((e == 15) & (m == 7), np.nan, out)
    return out


def dequant_blocks(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """W[i, j] = decode(q[i, j]) * scale[i // block, j // block]  (float64, exact)."""
    # decode through a 256-entry table of the code values (same definition, faster)
    w = e4m3_decode(np.arange(256, dtype=np.uint8))[np.asarray(codes, np.uint8)]
    R, C = w.shape
    s = np.asarray(scales, np.float64)
    assert s.shape == (R // block, C // block) and R % block == 0 and C % block == 0
    w = w.reshape(R // block, block, C // block, block) * s[:, None, :, None]
    return w.reshape(R, C)


# ----------------------------------------------------------------------------
# fp8 activations (the optional fp8-activation mode of the expert GEMMs)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0  # largest finite OCP E4M3 value: 2^8 * 1.75


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest OCP E4M3 value, ties to the even code.

    Needs |v| <= 448 (the callers scale into that range, so no value saturates).
    A value in the binade [2^e, 2^(e+1)) has 3 fraction bits, so the E4M3 values
    there are 2^(e-3) apart; below 2^-6 (the subnormal range) they are 2^-9
    apart.  Rounding to the nearest multiple of that step, with halves going to
    the even multiple (numpy's rint), is round-to-nearest-even on the code; the
    sign is kept, also when the magnitude rounds to zero.
    """
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX):
        raise ValueError("e4m3_round: |v| > 448")
    _, ex = np.frexp(a)                       # a = m * 2^ex with m in [0.5, 1): binade ex - 1
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    return np.copysign(np.rint(a / step) * step, v)


def fp8_block_scale_exponents(amax: np.ndarray) -> np.ndarray:
    """Per block: the smallest integer kexp with amax <= 448 * 2^kexp, at least -127.

    The scale of a block is the power of two 2^kexp (an 8-bit shared exponent, as
    in the MX formats of [GC-MoE], "two MMA implementations"), the smallest one
    that maps the block into the E4M3 range.  An all-zero block gets -127.
    """
    amax = np.asarray(amax, np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    kexp = np.ceil(np.log2(safe / E4M3_MAX))
    # the log is rounded: settle the boundary with exact comparisons
    kexp = np.where(safe > np.ldexp(E4M3_MAX, kexp.astype(np.int64)), kexp + 1, kexp)
    kexp = np.where(safe <= np.ldexp(E4M3_MAX, (kexp - 1).astype(np.int64)), kexp - 1, kexp)
    return np.maximum(np.where(pos, kexp, -127), -127).astype(np.int64)


def fp8_quantize_rows(v: np.ndarray, block: int = 128):
    """Activations as the expert GEMMs read them in the fp8-activation mode.

    Each row (one token) is cut into blocks of `block` consecutive K elements
    (the 128-wide K block of the fp8_w8a8 block_shape [128,128] of
    [vLLM-config] section 03); a block is scaled by 2^-kexp
    (fp8_block_scale_exponents of its largest magnitude), rounded to E4M3 and
    scaled back.  Returns (the float64 values the GEMM multiplies, kexp [rows,
    blocks]).
    """
    v = np.asarray(v, np.float64)
    R, C = v.shape
    assert C % block == 0
    b = v.reshape(R, C // block, block)
    kexp = fp8_block_scale_exponents(np.abs(b).max(axis=2) if C else np.zeros((R, 0)))
    sc = np.ldexp(1.0, kexp)[:, :, None]
    return (e4m3_round(b / sc) * sc).reshape(R, C), kexp


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """L[t, e] = sum_i x[t, i] * W_r[e, i]  (+ b[e]).

    [vLLM-config] section 02: each token goes through a router that picks its
    top-k experts; [FlashMoE] section 二.1: the gate computes routing (top-k) on
    the GPU.  The bias term is the skewed-load workload's per-expert bias.
    """
    L = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """ids[t, j]: the k experts with the largest logits, in descending order.

    Ties (IEEE equality) go to the lower expert id.  [vLLM-config] section 02
    ("256 choose 8").  np.lexsort sorts by the last key first: primarily by -L,
    then by expert id; float comparison treats -0.0 and +0.0 as equal.
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(L)):
        raise ValueError("non-finite logits are outside the contract")
    ids = np.empty((T, k), dtype=np.int32)
    eid = np.arange(E)
    for t in range(T):
        order = np.lexsort((eid, -L[t]))
        ids[t] = order[:k]
    return ids


def gate_weights(L: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w[t, j] = exp(L[t, e_j]) / sum_j' exp(L[t, e_j'])  over the k kept experts.

    [vLLM-config] section 02: the top-k outputs are summed with the gate
    weights; the weights are the softmax of the kept logits (shifted by the
    largest kept logit for range, which does not change the value).
    """
    kept = np.take_along_axis(np.asarray(L, np.float64), ids.astype(np.int64), axis=1)
    z = np.exp(kept - kept[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k):
    """Router logits, top-k ids and gate weights of every token."""
    L = router_logits(x, w_router, bias)
    ids = select_topk(L, k)
    return L, ids, gate_weights(L, ids)


# ----------------------------------------------------------------------------
# permutation
# ----------------------------------------------------------------------------
def permute(ids: np.ndarray, E: int):
    """Group the T*k (token, slot) assignments by expert.

    [vLLM-config] section 02: tokens are sorted and grouped by expert before the
    grouped GEMM; [FlashMoE] section 五.3: no padded payload (segments are
    unpadded here).
      counts[e]   = #{(t, j) : ids[t, j] == e}
      offsets     = exclusive prefix sum of counts, offsets[E] = T*k
      perm[p]     = t*k + j, in the stable order of (expert, token, slot)
      inv_perm[t*k + j] = p
    """
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    # a stable argsort of the expert id keeps (token, slot) order inside a group
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(T * k, dtype=np.int32)
    return counts, offsets, perm, inv_perm


# ----------------------------------------------------------------------------
# expert FFN and combine
# ----------------------------------------------------------------------------
def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(xr: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
               act_quant: bool = False) -> np.ndarray:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T for rows x.

    [vLLM-config] section 02: each chosen expert is a small FFN of three
    matmuls (gate, up, down) and SwiGLU; [Fusion] section 二: two linear layers
    and the SwiGLU activation.  No intermediate rounding, except in the
    fp8-activation mode (act_quant): the gate/up GEMMs read x, and the down GEMM
    reads h = silu(g) * u, as fp8_quantize_rows makes them (the w8a8 kernel of
    [vLLM-config] section 03; the requantisation fused after SwiGLU of [GC-MoE],
    "two MMA implementations").
    """
    xr = np.asarray(xr, np.float64)
    if act_quant:
        xr = fp8_quantize_rows(xr)[0]
    g = xr @ np.asarray(wg, np.float64).T
    u = xr @ np.asarray(wu, np.float64).T
    h = silu(g) * u
    if act_quant:
        h = fp8_quantize_rows(h)[0]
    return h @ np.asarray(wd, np.float64).T


def combine(w: np.ndarray, y_slots: np.ndarray, y_shared=None) -> np.ndarray:
    """out[t] = sum_{j=0..k-1} w[t, j] * y_slots[t, j]  (+ y_shared[t]).

    [vLLM-config] section 02: the top-k outputs are summed with their gate
    weights; [FlashMoE] section 二.1: results are merged with weights.  The
    always-on shared expert ([GC-MoE], "two MMA implementations": fused shared
    experts) has weight 1.
    """
    out = np.einsum("tj,tjd->td", np.asarray(w, np.float64), np.asarray(y_slots, np.float64))
    if y_shared is not None:
        out = out + y_shared
    return out


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------
class InputsView:
    """float64 view of a synthetic input set (decodes storage lazily, per expert)."""

    def __init__(self, inp):
        self.inp = inp
        c = inp.cfg
        self.cfg = c
        self.act, self.wdt = c["act"], c["w"]
        self.k, self.E = c["k"], c["E"]
        self.x = widen(inp.hidden, self.act)
        self.w_router = widen(inp.w_router, self.act)
        self.bias = None if inp.bias is None else np.asarray(inp.bias, np.float32).astype(np.float64)

    def _mat(self, q, s):
        if self.wdt == "fp8":
            return dequant_blocks(q, s)
        return widen(q, self.wdt)

    def expert(self, e: int):
        i = self.inp
        if e == self.E:  # the shared expert
            return (self._mat(i.sh_gate, i.sh_s_gate), self._mat(i.sh_up, i.sh_s_up),
                    self._mat(i.sh_down, i.sh_s_down))
        sg = None if i.s_gate is None else i.s_gate[e]
        su = None if i.s_up is None else i.s_up[e]
        sd = None if i.s_down is None else i.s_down[e]
        return self._mat(i.w_gate[e], sg), self._mat(i.w_up[e], su), self._mat(i.w_down[e], sd)

    @property
    def has_shared(self) -> bool:
        return self.inp.sh_gate is not None


def moe_forward(x, w_router, bias, k, expert, n_experts, shared=None, act_quant=False):
    """The whole layer: route, permute, per-expert FFN on its group, combine.

    expert(e) -> (wg [n,d], wu [n,d], wd [d,n]) float64; shared() likewise or
    None; act_quant: the expert FFNs' fp8-activation mode (expert_ffn).
    Returns (out [T,d], dict of routing results).
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    L, ids, w = route(x, w_router, bias, k)
    counts, offsets, perm, inv_perm = permute(ids, n_experts)
    y_sorted = np.zeros((T * k, d), dtype=np.float64)
    for e in range(n_experts):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        tok = perm[lo:hi] // k
        wg, wu, wd = expert(e)
        y_sorted[lo:hi] = expert_ffn(x[tok], wg, wu, wd, act_quant)
    y_slots = y_sorted[inv_perm].reshape(T, k, d)
    y_sh = None
    if shared is not None:
        wg, wu, wd = shared()
        y_sh = expert_ffn(x, wg, wu, wd, act_quant)
    out = combine(w, y_slots, y_sh)
    return out, dict(logits=L, ids=ids, weights=w, counts=counts, offsets=offsets,
                     perm=perm, inv_perm=inv_perm)


def moe_forward_view(v: InputsView, act_quant=False):
    return moe_forward(v.x, v.w_router, v.bias, v.k, v.expert, v.E,
                       (lambda: v.expert(v.E)) if v.has_shared else None, act_quant)


def moe_forward_tokens(v: InputsView, tokens, ids=None, weights=None, act_quant=False):
    """Outputs of a subset of tokens only (a token's output depends on no other
    token).  ids/weights may be given to use a fixed routing; otherwise the
    oracle's own routing of those tokens is used.  Returns (out [len,d], ids, w).
    """
    tokens = np.asarray(tokens, np.int64)
    xs = v.x[tokens]
    if ids is None:
        _, ids, weights = route(xs, v.w_router, v.bias, v.k)
    out = np.zeros_like(xs)
    cache = {}
    for r in range(len(tokens)):
        for j in range(v.k):
            e = int(ids[r, j])
            if e not in cache:
                cache[e] = v.expert(e)
            wg, wu, wd = cache[e]
            out[r] += weights[r, j] * expert_ffn(xs[r:r + 1], wg, wu, wd, act_quant)[0]
    if v.has_shared:
        wg, wu, wd = v.expert(v.E)
        out += expert_ffn(xs, wg, wu, wd, act_quant)
    return out, ids, weights


# ----------------------------------------------------------------------------
# comparison helpers
# ----------------------------------------------------------------------------
def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def near_tie_tokens(L_ref: np.ndarray, k: int, delta: float) -> np.ndarray:
    """Tokens whose routing could change under a logit perturbation <= delta.

    A token is a near tie when two adjacent ranks among the first k+1 (the
    kept experts and the first one left out) differ by less than 2*delta.
    Returns a boolean mask over tokens.
    """
    L = np.asarray(L_ref, np.float64)
    T, E = L.shape
    ids = select_topk(L, min(E, k + 1))
    v = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    gaps = v[:, :-1] - v[:, 1:]
    if gaps.shape[1] == 0:
        return np.zeros(T, bool)
    return np.any(gaps < 2.0 * delta, axis=1)
